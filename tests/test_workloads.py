"""The seeded input generators and shape lists.

* Philox4x32-10 known-answer vectors of its authors' reference release
  (Random123, kat_vectors: counters/keys all zero, all ones, and the pi
  digits).
* Parameter counts of the standard models: ResNet-50 25,557,032 in 161
  tensors; the 1.3B GPT decoder 1,315,723,264 in 292; Llama-7B 6,738,415,616
  in 291.
"""
import numpy as np

import workloads as W


def test_philox_known_answers():
    def run(c, k):
        out = W.philox4x32_10([c[0]], [c[1]], [c[2]], [c[3]], k[0], k[1])
        return [int(x[0]) for x in out]
    assert run([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    assert run([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6,
                                                       0x6D5451FD]
    assert run([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_shape_totals():
    assert (len(W.resnet50()), sum(p.numel for p in W.resnet50())) == (161, 25_557_032)
    assert (len(W.gpt_decoder()), sum(p.numel for p in W.gpt_decoder())) == (292, 1_315_723_264)
    assert (len(W.llama()), sum(p.numel for p in W.llama())) == (291, 6_738_415_616)
    assert [p.numel for p in W.tiny_linear()] == [1280, 10]


def test_many_small_sizes_are_seeded_and_in_range():
    a = [p.numel for p in W.many_small()]
    b = [p.numel for p in W.many_small()]
    assert a == b and len(a) == 20000
    assert min(a) >= 64 and max(a) <= 65536
    # log-uniform: the median sits near sqrt(64 * 65536) = 2048
    assert 1700 < np.median(a) < 2400


def test_normal_stream_is_offset_consistent_and_has_the_right_moments():
    full = W.normal_f32(3, 9, 1001, 1e-3)
    assert np.array_equal(full[17:400], W.normal_f32(3, 9, 383, 1e-3, offset=17))
    big = W.normal_f32(0, 1, 400_000, 1e-3).astype(np.float64)
    assert abs(big.mean()) < 1e-5 and abs(big.std() - 1e-3) < 1e-5
    assert not np.array_equal(W.normal_f32(0, 1, 64, 1.0), W.normal_f32(1, 1, 64, 1.0))


def test_bf16_inputs_are_bf16_patterns_of_the_f32_draws():
    wl = W.workload("llama7b")
    h = W.host_rank_flat(wl, 0, n=1000)
    assert h.dtype == np.uint16
    f = (h.astype(np.uint32) << np.uint32(16)).view(np.float32)
    x = W.normal_f32(0, wl.stream, 1000, wl.sigma)
    assert np.all(np.abs(f - x) <= np.abs(x) * 2 ** -8)
