// Bandwidth probe for the benchmark: the memory access pattern of the
// reduce (N non-temporal 16-byte loads per lane from N buffers at the same
// offset, one non-temporal 16-byte store, one-wave blocks) with none of its
// arithmetic or indexing, so that the benchmark can report the reduce
// against the ceiling of its own access pattern on the box it runs on, next
// to the nominal 8 TB/s.  Not part of the ABI in ddp.h; built into
// libddp_probe.so.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 64;

struct Ptrs {
    const u32x4 *p[8];
};

template <int N, bool WRITE>
__global__ void __launch_bounds__(kThreads)
stream_probe(Ptrs P, u32x4 *out, int64_t nvec, unsigned *sink)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= nvec) return;
    u32x4 v[N];
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = __builtin_nontemporal_load(P.p[k] + i);
    u32x4 acc = v[0];
#pragma unroll
    for (int k = 1; k < N; ++k) acc ^= v[k];
    if (WRITE)
        __builtin_nontemporal_store(acc, out + i);
    else if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u)
        sink[0] = 1;   // keeps the loads alive; practically never taken
}

template <int N>
int launch(const Ptrs &P, void *out, int64_t nvec, int write, unsigned lds, void *sink,
           hipStream_t st)
{
    const dim3 g((unsigned)((nvec + kThreads - 1) / kThreads)), b(kThreads);
    if (write)
        stream_probe<N, true><<<g, b, lds, st>>>(P, static_cast<u32x4 *>(out), nvec,
                                                 static_cast<unsigned *>(sink));
    else
        stream_probe<N, false><<<g, b, lds, st>>>(P, static_cast<u32x4 *>(out), nvec,
                                                  static_cast<unsigned *>(sink));
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

// n in 1..8 buffers of nvec 16-byte vectors (16-byte aligned); out: nvec
// vectors when write != 0; sink: one device uint32.  blocks_per_cu > 0 caps
// the resident blocks per CU the way the library's kernels are capped (an
// unused dynamic LDS reservation of LDS_per_CU / blocks_per_cu bytes); 0
// leaves occupancy to the registers.  Returns 0 or -1.
extern "C" int ddp_probe_stream(const void *const *ptrs, int n, void *out, int64_t nvec, int write,
                                int blocks_per_cu, void *sink, void *stream)
{
    if (!ptrs || n < 1 || n > 8 || nvec < 1 || !sink || (write && !out)) return -1;
    if ((nvec + kThreads - 1) / kThreads > 0x7fffffff || blocks_per_cu < 0) return -1;
    unsigned lds = 0;
    if (blocks_per_cu > 0) {
        int dev = 0, per_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                                  dev) != hipSuccess ||
            per_cu <= 0)
            return -1;
        lds = (unsigned)(per_cu / blocks_per_cu);
    }
    Ptrs P;
    for (int k = 0; k < 8; ++k) P.p[k] = static_cast<const u32x4 *>(ptrs[k < n ? k : 0]);
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (n) {
    case 1: return launch<1>(P, out, nvec, write, lds, sink, st);
    case 2: return launch<2>(P, out, nvec, write, lds, sink, st);
    case 3: return launch<3>(P, out, nvec, write, lds, sink, st);
    case 4: return launch<4>(P, out, nvec, write, lds, sink, st);
    case 5: return launch<5>(P, out, nvec, write, lds, sink, st);
    case 6: return launch<6>(P, out, nvec, write, lds, sink, st);
    case 7: return launch<7>(P, out, nvec, write, lds, sink, st);
    default: return launch<8>(P, out, nvec, write, lds, sink, st);
    }
}
