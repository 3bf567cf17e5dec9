// The reduce and the fused average + SGD step: kernels, their launches,
// the plan's device tables, and the entry points ddp_bucket_allreduce_avg,
// ddp_sync_allreduce_avg[_bucket], ddp_sync_sgd_update,
// ddp_plan_prepare[_ranks].
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel);
//        [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

// N known at compile time (2..16): all N * kUnroll vector loads in flight,
// the fold done from registers in any rotation.
template <int NR, bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
reduce_fast(RankArgs ra, int64_t total, Buckets bk, float inv, void *out)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (kThreads * kUnroll * VEC);

    // Every rank's vector at the lane's offset, in rank order, in either
    // summation order: the addresses depend on the tile alone, so all
    // NR * kUnroll loads are in flight before the tile's ring segments are
    // looked up below.  A lane whose vector runs past the end reads the first
    // vector of each rank buffer instead (in bounds since total >= VEC) and
    // never uses it.
    u32x4 v[kUnroll][NR];
    int64_t i0[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) i0[u] = tile0 + ((int64_t)threadIdx.x + u * kThreads) * VEC;
    if (total >= VEC) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int k = 0; k < NR; ++k)
                v[u][k] = ld_stream(static_cast<const char *>(ra.p[k]) +
                                    (i0[u] + VEC <= total ? i0[u] * ISZ : 0));
    }

    const Segs sg = tile_segs<RING>(bk, total, NR, tile, tile0);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const bool in_a = i0[u] >= sg.a_lo && i0[u] + VEC <= sg.a_hi;
        const bool in_b = RING && i0[u] >= sg.b_lo && i0[u] + VEC <= sg.b_hi;
        if (in_a || in_b) {
            float acc[VEC];
            if (!RING)
                fold_seq<NR, IN>(v[u], acc);
            else
                fold_ring<NR, IN>(v[u], in_a ? sg.sa : sg.sb, acc);
            store_vec<IN, OUT>(out, i0[u], acc, inv);
        } else if (i0[u] < total) {
            reduce_elems<IN, OUT, RING>(ra, NR, total, bk, first_bucket(bk, tile), inv, out,
                                            i0[u], VEC);
        }
    }
    head_block<IN, OUT, RING>(ra, NR, total, bk, inv, out, tile0);
}

// Fused average + SGD step, N known at compile time (1..8).  Per lane: the N
// gradient vectors and the lane's parameter (and momentum) vectors are loaded
// together, the average is folded and scaled, optionally stored, and the
// parameters updated in place.  Parameters are f32: one 16-byte vector per 4
// elements, so a bf16 lane (8 elements) moves two.
// bf16 gradients, the split lane layout of sgd_vec_split: lane L of a tile
// takes elements [4L, 4L + 4) and [256 + 4L, 256 + 4L + 4), loaded as two
// 8-byte vectors per rank, so that each of its parameter and momentum
// stores is one 16-byte piece of a 1 KiB contiguous wave store.  A lane
// whose two groups do not lie in one ring segment of the tile (a tile that
// holds a ring cut), or reach past the end, folds them element by element.
template <int NR, bool RING, bool MOM>
__device__ __forceinline__ void sgd_tile_bf16(const RankArgs &ra, int64_t total, const Buckets &bk,
                                              float inv, const SgdArgs &sa)
{
    constexpr int H = kThreads * 4;   // the second group, 256 elements on
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (2 * H);
    const int64_t iA = tile0 + 4 * (int64_t)threadIdx.x, iB = iA + H;
    u32x4 v[NR], pv[2], mv[2];
    if (total >= 8) {   // a lane past the end reads the first elements and drops them
        const bool whole = iB + 4 <= total;
        const int64_t a = whole ? iA : 0, b = whole ? iB : 0;
#pragma unroll
        for (int k = 0; k < NR; ++k) v[k] = ld_split(ra.p[k], 2 * a, 2 * b);
        const char *pp = reinterpret_cast<const char *>(sa.param);
        pv[0] = ld_stream(pp + 4 * a);
        pv[1] = ld_stream(pp + 4 * b);
        if (MOM) {
            const char *mp = reinterpret_cast<const char *>(sa.mom);
            mv[0] = ld_stream(mp + 4 * a);
            mv[1] = ld_stream(mp + 4 * b);
        }
    }
    const Segs sg = tile_segs<RING>(bk, total, NR, tile, tile0);
    const bool in_a = iA >= sg.a_lo && iB + 4 <= sg.a_hi;
    const bool in_b = RING && iA >= sg.b_lo && iB + 4 <= sg.b_hi;
    if (in_a || in_b) {
        float y[8];
        if (!RING || NR == 1)
            fold_seq<NR, kBF16>(v, y);
        else
            fold_ring<NR, kBF16>(v, in_a ? sg.sa : sg.sb, y);
        if (NR > 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] * inv;
        }
        sgd_vec_split<MOM>(sa.grad_out, static_cast<void *>(sa.param), static_cast<void *>(sa.mom),
                           iA, iB, y, pv, mv, sa.lr, sa.mu);
    } else {
        const int32_t b0 = first_bucket(bk, tile);
        if (iA < total) sgd_elems<kBF16, kBF16, RING, MOM>(ra, NR, total, bk, b0, inv, sa, iA, 4);
        if (iB < total) sgd_elems<kBF16, kBF16, RING, MOM>(ra, NR, total, bk, b0, inv, sa, iB, 4);
    }
}

template <int NR, bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
reduce_sgd_fast(RankArgs ra, int64_t total, Buckets bk, float inv, SgdArgs sa)
{
    static_assert(kUnroll == 1, "the fused kernel processes one vector per lane");
    if constexpr (IN == kBF16) {
        static_assert(OUT == kBF16, "bf16 gradients average to bf16");
        sgd_tile_bf16<NR, RING, MOM>(ra, total, bk, inv, sa);
        return;
    }
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (kThreads * VEC);
    const int64_t i0 = tile0 + (int64_t)threadIdx.x * VEC;

    // The lane's gradient vectors from every rank in rank order, and its
    // parameter (and momentum) vectors, issued before the ring segments are
    // looked up; a lane past the end reads the first vectors and drops them.
    u32x4 v[NR], pv[PV], mv[PV];
    if (total >= VEC) {
        const bool whole = i0 + VEC <= total;
        const int64_t go = whole ? i0 * ISZ : 0, po = whole ? i0 * 4 : 0;
#pragma unroll
        for (int k = 0; k < NR; ++k) v[k] = ld_stream(static_cast<const char *>(ra.p[k]) + go);
#pragma unroll
        for (int j = 0; j < PV; ++j) {
            pv[j] = ld_stream(reinterpret_cast<const char *>(sa.param) + po + 16 * j);
            if (MOM) mv[j] = ld_stream(reinterpret_cast<const char *>(sa.mom) + po + 16 * j);
        }
    }

    const Segs sg = tile_segs<RING>(bk, total, NR, tile, tile0);
    const bool in_a = i0 >= sg.a_lo && i0 + VEC <= sg.a_hi;
    const bool in_b = RING && i0 >= sg.b_lo && i0 + VEC <= sg.b_hi;
    if (in_a || in_b) {
        float y[VEC];
        if (!RING || NR == 1)
            fold_seq<NR, IN>(v, y);
        else
            fold_ring<NR, IN>(v, in_a ? sg.sa : sg.sb, y);
        if (NR > 1) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = y[e] * inv;
        }
        sgd_vec<IN, OUT, MOM>(sa, i0, y, pv, mv);
    } else if (i0 < total) {
        sgd_elems<IN, OUT, RING, MOM>(ra, NR, total, bk, first_bucket(bk, tile), inv, sa, i0, VEC);
    }
}

// Any N up to DDP_MAX_RANKS (launched for N > 16).  A wave makes one pass per ring segment its
// lanes lie in (usually one), so the rank order of each pass is
// wave-uniform, and folds with fold_looped.
template <bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
reduce_many(RankArgs ra, int N, int64_t total, Buckets bk, float inv, void *out)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    static_assert(kUnroll == 1, "one vector per lane");
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (kThreads * VEC);
    const int64_t i0 = tile0 + (int64_t)threadIdx.x * VEC;
    const Segs sg = tile_segs<RING>(bk, total, N, tile, tile0);
    const bool in_a = i0 >= sg.a_lo && i0 + VEC <= sg.a_hi;
    const bool in_b = RING && i0 >= sg.b_lo && i0 + VEC <= sg.b_hi;
#pragma unroll 1
    for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
        const bool mine = pass == 0 ? in_a : in_b;
        if (!__builtin_amdgcn_ballot_w64(mine)) continue;   // no lane of the wave here
        float acc[VEC];
        fold_looped<IN, RING>(ra.p, N, pass == 0 ? sg.sa : sg.sb, mine ? i0 * ISZ : 0, acc);
        if (mine) store_vec<IN, OUT>(out, i0, acc, inv);
    }
    if (!in_a && !in_b && i0 < total)
        reduce_elems<IN, OUT, RING>(ra, N, total, bk, first_bucket(bk, tile), inv, out, i0, VEC);
    head_block<IN, OUT, RING>(ra, N, total, bk, inv, out, tile0);
}

// reduce_sgd_many for bf16 gradients, in the split lane layout of
// sgd_tile_bf16.
template <bool RING, bool MOM>
__device__ __forceinline__ void sgd_many_bf16(const RankArgs &ra, int N, int64_t total,
                                              const Buckets &bk, float inv, const SgdArgs &sa)
{
    constexpr int H = kThreads * 4;
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (2 * H);
    const int64_t iA = tile0 + 4 * (int64_t)threadIdx.x, iB = iA + H;
    u32x4 pv[2], mv[2];
    if (total >= 8) {   // a lane past the end reads the first elements and drops them
        const bool whole = iB + 4 <= total;
        const int64_t a = whole ? iA : 0, b = whole ? iB : 0;
        const char *pp = reinterpret_cast<const char *>(sa.param);
        pv[0] = ld_stream(pp + 4 * a);
        pv[1] = ld_stream(pp + 4 * b);
        if (MOM) {
            const char *mp = reinterpret_cast<const char *>(sa.mom);
            mv[0] = ld_stream(mp + 4 * a);
            mv[1] = ld_stream(mp + 4 * b);
        }
    }
    const Segs sg = tile_segs<RING>(bk, total, N, tile, tile0);
    const bool in_a = iA >= sg.a_lo && iB + 4 <= sg.a_hi;
    const bool in_b = RING && iA >= sg.b_lo && iB + 4 <= sg.b_hi;
#pragma unroll 1
    for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
        const bool mine = pass == 0 ? in_a : in_b;
        if (!__builtin_amdgcn_ballot_w64(mine)) continue;
        float y[8];
        fold_looped_split<RING>(ra.p, N, pass == 0 ? sg.sa : sg.sb, mine ? 2 * iA : 0,
                                mine ? 2 * iB : 0, y);
        if (mine) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = y[e] * inv;
            sgd_vec_split<MOM>(sa.grad_out, static_cast<void *>(sa.param),
                               static_cast<void *>(sa.mom), iA, iB, y, pv, mv, sa.lr, sa.mu);
        }
    }
    if (!in_a && !in_b) {
        const int32_t b0 = first_bucket(bk, tile);
        if (iA < total) sgd_elems<kBF16, kBF16, RING, MOM>(ra, N, total, bk, b0, inv, sa, iA, 4);
        if (iB < total) sgd_elems<kBF16, kBF16, RING, MOM>(ra, N, total, bk, b0, inv, sa, iB, 4);
    }
}

// The fused average + SGD step for any N up to DDP_MAX_RANKS: the lane's
// parameter (and momentum) vectors are issued first, then the ranks are
// folded as in reduce_many and the epilogue of reduce_sgd_fast applied.
template <bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
reduce_sgd_many(RankArgs ra, int N, int64_t total, Buckets bk, float inv, SgdArgs sa)
{
    if constexpr (IN == kBF16) {
        static_assert(OUT == kBF16, "bf16 gradients average to bf16");
        sgd_many_bf16<RING, MOM>(ra, N, total, bk, inv, sa);
        return;
    }
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    static_assert(kUnroll == 1, "one vector per lane");
    const int64_t tile = tile_of_block(bk);
    const int64_t tile0 = tile * (kThreads * VEC);
    const int64_t i0 = tile0 + (int64_t)threadIdx.x * VEC;
    u32x4 pv[PV], mv[PV];
    if (total >= VEC) {   // a lane past the end reads the first vectors and drops them
        const int64_t po = i0 + VEC <= total ? i0 * 4 : 0;
#pragma unroll
        for (int j = 0; j < PV; ++j) {
            pv[j] = ld_stream(reinterpret_cast<const char *>(sa.param) + po + 16 * j);
            if (MOM) mv[j] = ld_stream(reinterpret_cast<const char *>(sa.mom) + po + 16 * j);
        }
    }
    const Segs sg = tile_segs<RING>(bk, total, N, tile, tile0);
    const bool in_a = i0 >= sg.a_lo && i0 + VEC <= sg.a_hi;
    const bool in_b = RING && i0 >= sg.b_lo && i0 + VEC <= sg.b_hi;
#pragma unroll 1
    for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
        const bool mine = pass == 0 ? in_a : in_b;
        if (!__builtin_amdgcn_ballot_w64(mine)) continue;
        float y[VEC];
        fold_looped<IN, RING>(ra.p, N, pass == 0 ? sg.sa : sg.sb, mine ? i0 * ISZ : 0, y);
        if (mine) {
#pragma unroll
            for (int e = 0; e < VEC; ++e) y[e] = y[e] * inv;
            sgd_vec<IN, OUT, MOM>(sa, i0, y, pv, mv);
        }
    }
    if (!in_a && !in_b && i0 < total)
        sgd_elems<IN, OUT, RING, MOM>(ra, N, total, bk, first_bucket(bk, tile), inv, sa, i0, VEC);
}

// One element per thread, element-aligned buffers: elements [0, total) of
// the single bucket bk.
template <bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
reduce_scalar(RankArgs ra, int N, int64_t total, Buckets bk, float inv, void *out)
{
    const int64_t i = tile_of_block(bk) * kThreads + threadIdx.x;
    if (i >= total) return;
    reduce_elems<IN, OUT, RING>(ra, N, total, bk, 0, inv, out, i, 1);
}

// ---------------------------------------------------------------- launches

template <bool RING, int IN, int OUT>
ddp_status_t launch_typed(const RankArgs &ra, int N, int64_t total, const Buckets &bk, float inv,
                          void *out, hipStream_t st, bool vec_ok)
{
    Buckets lb = bk;
    const dim3 b(kThreads);
    if (vec_ok) {
        const int64_t tiles = (total + tile_elems(IN) - 1) / tile_elems(IN) +
                              (!bk.base && bk.lo < 0 ? 1 : 0);   // + the head block
        const unsigned lds = lds_for_blocks(reduce_blocks_per_cu(N, RING));
        return launch_split(tiles, kThreads, "reduce kernel launch", [&](int64_t b0, unsigned n) {
            lb.first_block = b0;
            const dim3 g(n);
            const bool fixed = with_rank_count<2, 16>(N, [&](auto nr) {
                reduce_fast<decltype(nr)::value, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, lb, inv,
                                                                                  out);
            });
            if (!fixed) reduce_many<RING, IN, OUT><<<g, b, lds, st>>>(ra, N, total, lb, inv, out);
        });
    }
    return launch_split((total + kThreads - 1) / kThreads, kThreads, "reduce kernel launch",
                        [&](int64_t b0, unsigned n) {
                            lb.first_block = b0;
                            reduce_scalar<RING, IN, OUT><<<dim3(n), b, 0, st>>>(ra, N, total, lb,
                                                                               inv, out);
                        });
}

}  // namespace

namespace ddp_detail {

ddp_status_t launch_reduce(const RankArgs &ra, int N, int64_t total, int order, int in, int out_dt,
                           const Buckets &bk, void *out, hipStream_t st, bool vec_ok)
{
    const float inv = 1.0f / (float)N;
    const bool ring = order == DDP_ORDER_RING;
    if (in == DDP_F32 && out_dt == DDP_F32)
        return ring ? launch_typed<true, kF32, kF32>(ra, N, total, bk, inv, out, st, vec_ok)
                    : launch_typed<false, kF32, kF32>(ra, N, total, bk, inv, out, st, vec_ok);
    if (in == DDP_BF16 && out_dt == DDP_BF16)
        return ring ? launch_typed<true, kBF16, kBF16>(ra, N, total, bk, inv, out, st, vec_ok)
                    : launch_typed<false, kBF16, kBF16>(ra, N, total, bk, inv, out, st, vec_ok);
    return ring ? launch_typed<true, kF32, kBF16>(ra, N, total, bk, inv, out, st, vec_ok)
                : launch_typed<false, kF32, kBF16>(ra, N, total, bk, inv, out, st, vec_ok);
}

}  // namespace ddp_detail

namespace {

// One bucket of len elements.  The vector kernel streams best from 128-byte
// aligned tiles (an L2 line: a misaligned 1 KiB wave load touches 9 lines
// instead of 8), and its stores want the output aligned to a lane's store
// width.  It starts h < 64 elements into the bucket and numbers the bucket
// [-h, len - h), so that the ring chunks stay those of the whole bucket; the
// launch's extra head block reduces the first h elements one by one.  h puts
// every rank buffer on a 128-byte (else 16-byte) boundary when they all sit
// at the same offset from one -- a bucket at an unpadded offset into equally
// aligned flat buffers -- and the output can follow; otherwise it puts the
// output on a 128-byte boundary and the rank loads run at whatever element
// alignment they have (the loads accept any).  Only a bucket shorter than
// that head takes the per-element kernel alone.
ddp_status_t launch_one_bucket(const RankArgs &ra, int N, int64_t len, int order, int in,
                               int out_dt, void *out, hipStream_t st)
{
    const int isz = dtype_size(in), osz = dtype_size(out_dt);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(ra.p[0]);
    bool same128 = true, same16 = true;
    for (int r = 1; r < N; ++r) {
        const uintptr_t ar = reinterpret_cast<uintptr_t>(ra.p[r]);
        same128 = same128 && ar % 128 == a0 % 128;
        same16 = same16 && ar % 16 == a0 % 16;
    }
    const int64_t store_bytes = vec_elems(in) * osz;   // one lane's store: 16 or 8 bytes
    const uintptr_t ao = reinterpret_cast<uintptr_t>(out);
    int64_t h = -1;
    for (const uintptr_t line : {uintptr_t(128), uintptr_t(16)}) {
        if (!same16 || (line == 128 && !same128)) continue;
        const int64_t hh = (int64_t)((line - a0 % line) % line) / isz;
        if (hh < len && hh < kThreads && (ao + hh * osz) % store_bytes == 0) {
            h = hh;
            break;
        }
    }
    if (h < 0) {   // the output's 128-byte boundary (out is element-aligned)
        const int64_t hh = (int64_t)((128 - ao % 128) % 128) / osz;
        if (hh < len) h = hh;
    }
    if (h < 0)
        return launch_reduce(ra, N, len, order, in, out_dt, single_bucket(0, len), out, st, false);
    RankArgs rest;
    std::memset(&rest, 0, sizeof(rest));
    for (int r = 0; r < N; ++r) rest.p[r] = static_cast<const char *>(ra.p[r]) + h * isz;
    return launch_reduce(rest, N, len - h, order, in, out_dt, single_bucket(-h, len - h),
                         static_cast<char *>(out) + h * osz, st, true);
}

template <bool RING, int IN, int OUT, bool MOM>
ddp_status_t launch_sgd_typed(const RankArgs &ra, int N, int64_t total, const Buckets &bk,
                              float inv, const SgdArgs &sa, hipStream_t st)
{
    Buckets lb = bk;
    const dim3 b(kThreads);
    const int64_t tiles = (total + tile_elems(IN) - 1) / tile_elems(IN);
    const unsigned lds = lds_for_blocks(sgd_blocks_per_cu(N, MOM));
    return launch_split(tiles, kThreads, "fused SGD kernel launch", [&](int64_t b0, unsigned n) {
        lb.first_block = b0;
        const dim3 g(n);
        const bool fixed = with_rank_count<1, 8>(N, [&](auto nr) {
            reduce_sgd_fast<decltype(nr)::value, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total,
                                                                                       lb, inv, sa);
        });
        if (!fixed) reduce_sgd_many<RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, N, total, lb, inv, sa);
    });
}

template <bool RING, bool MOM>
ddp_status_t launch_sgd_pair(const RankArgs &ra, int N, int64_t total, int in, int out_dt,
                             const Buckets &bk, float inv, const SgdArgs &sa, hipStream_t st)
{
    if (in == DDP_F32 && out_dt == DDP_F32)
        return launch_sgd_typed<RING, kF32, kF32, MOM>(ra, N, total, bk, inv, sa, st);
    if (in == DDP_BF16 && out_dt == DDP_BF16)
        return launch_sgd_typed<RING, kBF16, kBF16, MOM>(ra, N, total, bk, inv, sa, st);
    return launch_sgd_typed<RING, kF32, kBF16, MOM>(ra, N, total, bk, inv, sa, st);
}

ddp_status_t launch_sgd(const RankArgs &ra, int N, int64_t total, int order, int in, int out_dt,
                        const Buckets &bk, const SgdArgs &sa, hipStream_t st)
{
    const float inv = 1.0f / (float)N;
    const bool ring = order == DDP_ORDER_RING, mom = sa.mom != nullptr;
    if (ring)
        return mom ? launch_sgd_pair<true, true>(ra, N, total, in, out_dt, bk, inv, sa, st)
                   : launch_sgd_pair<true, false>(ra, N, total, in, out_dt, bk, inv, sa, st);
    return mom ? launch_sgd_pair<false, true>(ra, N, total, in, out_dt, bk, inv, sa, st)
               : launch_sgd_pair<false, false>(ra, N, total, in, out_dt, bk, inv, sa, st);
}

}  // namespace

namespace ddp_detail {

// Common validation of a reduce call.  Returns OK or an error code.  The
// output may be null only when out_optional is set.
ddp_status_t check_reduce(const void *const *ptrs, int32_t n, int64_t len, int order, int in,
                          int out_dt, const void *out, bool out_optional)
{
    if (n < 1 || len < 0) return DDP_ERR_INVALID_ARG;
    if (order != DDP_ORDER_SEQUENTIAL && order != DDP_ORDER_RING) return DDP_ERR_INVALID_ARG;
    if (!dtype_ok(in) || !dtype_ok(out_dt)) return DDP_ERR_INVALID_ARG;
    if (n > DDP_MAX_RANKS) return DDP_ERR_UNSUPPORTED;
    if (!pair_ok(in, out_dt)) return DDP_ERR_UNSUPPORTED;
    if (n == 1 && in != out_dt) return DDP_ERR_UNSUPPORTED;
    if (len > INT64_MAX / 4) return DDP_ERR_OVERFLOW;
    if (len == 0) return DDP_OK;   // nothing is read or written: pointers may be null
    if (!ptrs || (!out && !out_optional)) return DDP_ERR_INVALID_ARG;
    for (int r = 0; r < n; ++r) {
        if (!ptrs[r]) return DDP_ERR_INVALID_ARG;
        if (!aligned(ptrs[r], dtype_size(in))) return DDP_ERR_INVALID_ARG;
    }
    if (!out) return DDP_OK;
    if (!aligned(out, dtype_size(out_dt))) return DDP_ERR_INVALID_ARG;
    return check_alias(ptrs, n, len, dtype_size(in), out, dtype_size(out_dt));
}

// N == 1: the input is the result ([TR24] 九 skips the collective when
// world_size <= 1).
ddp_status_t copy_single(const void *in, int64_t len, int esize, void *out, hipStream_t st)
{
    if (in == out || len == 0) return DDP_OK;
    const hipError_t e =
        hipMemcpyAsync(out, in, (size_t)(len * esize), hipMemcpyDeviceToDevice, st);
    return e == hipSuccess ? DDP_OK : hip_fail("hipMemcpyAsync (N == 1)", e);
}

}  // namespace ddp_detail

namespace {

// Device tables of `plan` for tiles of `tile` elements on the current device.
ddp_status_t plan_tables(ddp_plan *plan, int64_t tile, const ddp_dev_tables **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    std::lock_guard<std::mutex> lock(plan->mu);
    auto key = std::make_pair(dev, tile);
    auto it = plan->dev.find(key);
    if (it != plan->dev.end()) {
        *out = &it->second;
        return DDP_OK;
    }
    ddp_dev_tables t;
    const int32_t nb = plan->n_buckets();
    t.n_tiles = (plan->total + tile - 1) / tile;
    const int64_t stride = tile << kTileTableShift;   // elements between table entries
    const int64_t entries = (plan->total + stride - 1) / stride;
    std::vector<int32_t> tb;
    try {
        tb.resize((size_t)std::max<int64_t>(entries, 1));
    } catch (...) {
        return DDP_ERR_NOMEM;
    }
    for (int64_t k = 0; k < entries; ++k)
        tb[k] = bucket_holding(plan->bucket_base.data(), nb, k * stride);
    const size_t base_bytes = sizeof(int64_t) * (size_t)(nb + 1);
    const size_t tb_bytes = sizeof(int32_t) * tb.size();
    if ((e = hipMalloc(&t.bucket_base, base_bytes)) != hipSuccess)
        return hip_fail("hipMalloc (bucket table)", e, DDP_ERR_NOMEM);
    if ((e = hipMalloc(&t.tile_bucket, tb_bytes)) != hipSuccess) {
        (void)hipFree(t.bucket_base);
        return hip_fail("hipMalloc (tile table)", e, DDP_ERR_NOMEM);
    }
    if ((e = hipMemcpy(t.bucket_base, plan->bucket_base.data(), base_bytes,
                       hipMemcpyHostToDevice)) != hipSuccess ||
        (e = hipMemcpy(t.tile_bucket, tb.data(), tb_bytes, hipMemcpyHostToDevice)) != hipSuccess) {
        (void)hipFree(t.bucket_base);
        (void)hipFree(t.tile_bucket);
        return hip_fail("hipMemcpy (plan tables)", e);
    }
    auto ins = plan->dev.emplace(key, t);
    *out = &ins.first->second;
    return DDP_OK;
}

// Ring segments of every tile of a plan for n_ranks ranks: one word per tile
// (ring_tile_word), striped by XCD -- tile t at (t % 8) * stride + t / 8 --
// so that each XCD's L2 fetches only lines of its own tiles.  Built on the
// host and uploaded once per device, tile size and rank count.
ddp_status_t ring_tile_desc(ddp_plan *plan, int64_t tile, int n_ranks, const uint32_t **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    std::lock_guard<std::mutex> lock(plan->mu);
    const auto key = std::make_tuple(dev, tile, n_ranks);
    auto it = plan->ring_desc.find(key);
    if (it != plan->ring_desc.end()) {
        *out = it->second;
        return DDP_OK;
    }
    const int64_t n_tiles = (plan->total + tile - 1) / tile;
    const int64_t stride = word_stride(n_tiles);
    std::vector<uint32_t> w;
    try {
        w.assign((size_t)std::max<int64_t>(kXcds * stride, 1), 0u);
    } catch (...) {
        return DDP_ERR_NOMEM;
    }
    const int64_t *base = plan->bucket_base.data();
    const int32_t nb = plan->n_buckets();
    for (int64_t t = 0; t < n_tiles; ++t)
        w[(size_t)((t % kXcds) * stride + t / kXcds)] = ring_tile_word(base, nb, tile, n_ranks, t);
    uint32_t *d = nullptr;
    const size_t bytes = sizeof(uint32_t) * w.size();
    if ((e = hipMalloc(&d, bytes)) != hipSuccess)
        return hip_fail("hipMalloc (ring segment table)", e, DDP_ERR_NOMEM);
    if ((e = hipMemcpy(d, w.data(), bytes, hipMemcpyHostToDevice)) != hipSuccess) {
        (void)hipFree(d);
        return hip_fail("hipMemcpy (ring segment table)", e);
    }
    plan->ring_desc.emplace(key, d);
    *out = d;
    return DDP_OK;
}

// The tables of a RING synchronisation over n_ranks ranks.
ddp_status_t ring_buckets(ddp_plan *plan, int in, int n_ranks, Buckets *bk)
{
    const ddp_dev_tables *t = nullptr;
    ddp_status_t st = plan_tables(plan, tile_elems(in), &t);
    if (st != DDP_OK) return st;
    const uint32_t *desc = nullptr;
    if ((st = ring_tile_desc(plan, tile_elems(in), n_ranks, &desc)) != DDP_OK) return st;
    *bk = {t->bucket_base, t->tile_bucket, desc, word_stride(t->n_tiles), 0, plan->total,
           plan->n_buckets(), 0};
    return DDP_OK;
}

}  // namespace

void ddp_internal_free_plan_tables(ddp_plan *plan)
{
    std::lock_guard<std::mutex> lock(plan->mu);
    if (plan->dev.empty() && plan->ring_desc.empty()) return;
    int cur = -1;
    (void)hipGetDevice(&cur);
    for (auto &kv : plan->dev) {
        (void)hipSetDevice(kv.first.first);
        (void)hipFree(kv.second.bucket_base);
        (void)hipFree(kv.second.tile_bucket);
    }
    for (auto &kv : plan->ring_desc) {
        (void)hipSetDevice(std::get<0>(kv.first));
        (void)hipFree(kv.second);
    }
    plan->dev.clear();
    plan->ring_desc.clear();
    if (cur >= 0) (void)hipSetDevice(cur);
}

extern "C" {

ddp_status_t ddp_bucket_allreduce_avg(const void *const *rank_ptrs, int32_t n_ranks, int64_t len,
                                      ddp_order_t order, ddp_dtype_t in_dtype,
                                      ddp_dtype_t out_dtype, void *out, void *stream)
{
    ddp_status_t stc = check_reduce(rank_ptrs, n_ranks, len, order, in_dtype, out_dtype, out);
    if (stc != DDP_OK) return stc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (len == 0) return DDP_OK;
    if (n_ranks == 1) return copy_single(rank_ptrs[0], len, dtype_size(in_dtype), out, st);
    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    for (int r = 0; r < n_ranks; ++r) ra.p[r] = rank_ptrs[r];
    return launch_one_bucket(ra, n_ranks, len, order, in_dtype, out_dtype, out, st);
}

ddp_status_t ddp_plan_prepare(ddp_plan_t *plan)
{
    if (!plan) return DDP_ERR_INVALID_ARG;
    const ddp_dev_tables *t = nullptr;
    return plan_tables(plan, tile_elems(plan->dtype), &t);
}

ddp_status_t ddp_plan_prepare_ranks(ddp_plan_t *plan, int32_t n_ranks)
{
    if (!plan || n_ranks < 1 || n_ranks > DDP_MAX_RANKS) return DDP_ERR_INVALID_ARG;
    if (n_ranks == 1) return ddp_plan_prepare(plan);
    Buckets bk;
    return ring_buckets(plan, plan->dtype, n_ranks, &bk);
}

ddp_status_t ddp_sync_allreduce_avg(ddp_plan_t *plan, const void *const *rank_flat, int32_t n_ranks,
                                    ddp_order_t order, ddp_dtype_t out_dtype, void *out_flat,
                                    void *stream)
{
    if (!plan) return DDP_ERR_INVALID_ARG;
    const int in = plan->dtype;
    const int64_t total = plan->total;
    ddp_status_t stc = check_reduce(rank_flat, n_ranks, total, order, in, out_dtype, out_flat);
    if (stc != DDP_OK) return stc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (total == 0) return DDP_OK;
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));
    if (n_ranks == 1) return copy_single(rank_flat[0], total, dtype_size(in), out_flat, st);

    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    // the vector stores want the output on a 16-byte boundary; the rank
    // buffers are read at whatever element alignment they have
    const bool vec_ok = aligned(out_flat, 16);
    for (int r = 0; r < n_ranks; ++r) ra.p[r] = rank_flat[r];
    if (!vec_ok) {
        // an output off a 16-byte boundary: one launch per bucket, each
        // aligned to its own part of the output
        const int isz = dtype_size(in), osz = dtype_size(out_dtype);
        for (int32_t b = 0; b < plan->n_buckets(); ++b) {
            const int64_t base = plan->bucket_base[b], len = plan->bucket_base[b + 1] - base;
            if (len == 0) continue;
            RankArgs sub;
            std::memset(&sub, 0, sizeof(sub));
            for (int r = 0; r < n_ranks; ++r)
                sub.p[r] = static_cast<const char *>(rank_flat[r]) + base * isz;
            ddp_status_t s2 = launch_one_bucket(sub, n_ranks, len, order, in, out_dtype,
                                                static_cast<char *>(out_flat) + base * osz, st);
            if (s2 != DDP_OK) return s2;
        }
        return DDP_OK;
    }
    if (order == DDP_ORDER_SEQUENTIAL) {
        // the sequential fold does not depend on bucket boundaries
        return launch_reduce(ra, n_ranks, total, order, in, out_dtype, single_bucket(0, total),
                             out_flat, st, true);
    }
    Buckets bk;
    if ((stc = ring_buckets(plan, in, n_ranks, &bk)) != DDP_OK) return stc;
    return launch_reduce(ra, n_ranks, total, order, in, out_dtype, bk, out_flat, st, true);
}

ddp_status_t ddp_sync_allreduce_avg_bucket(ddp_plan_t *plan, int32_t bucket,
                                           const void *const *rank_flat, int32_t n_ranks,
                                           ddp_order_t order, ddp_dtype_t out_dtype,
                                           void *out_flat, void *stream)
{
    if (!plan || bucket < 0 || bucket >= plan->n_buckets()) return DDP_ERR_INVALID_ARG;
    const int in = plan->dtype;
    // the flat buffers as a whole are checked as by ddp_sync_allreduce_avg
    ddp_status_t stc =
        check_reduce(rank_flat, n_ranks, plan->total, order, in, out_dtype, out_flat);
    if (stc != DDP_OK) return stc;
    const int64_t base = plan->bucket_base[bucket], len = plan->bucket_base[bucket + 1] - base;
    if (len == 0) return DDP_OK;
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int isz = dtype_size(in), osz = dtype_size(out_dtype);
    char *out_b = static_cast<char *>(out_flat) + base * osz;
    if (n_ranks == 1)
        return copy_single(static_cast<const char *>(rank_flat[0]) + base * isz, len, isz, out_b,
                           st);
    RankArgs sub;
    std::memset(&sub, 0, sizeof(sub));
    for (int r = 0; r < n_ranks; ++r) sub.p[r] = static_cast<const char *>(rank_flat[r]) + base * isz;
    return launch_one_bucket(sub, n_ranks, len, order, in, out_dtype, out_b, st);
}

ddp_status_t ddp_sync_sgd_update(ddp_plan_t *plan, const void *const *rank_flat, int32_t n_ranks,
                                 ddp_order_t order, ddp_dtype_t out_dtype, void *grad_out,
                                 float *param_flat, float *momentum_flat, float lr, float momentum,
                                 void *stream)
{
    if (!plan) return DDP_ERR_INVALID_ARG;
    const int in = plan->dtype;
    const int64_t total = plan->total;
    ddp_status_t stc =
        check_reduce(rank_flat, n_ranks, total, order, in, out_dtype, grad_out, true);
    if (stc != DDP_OK) return stc;
    if (total == 0) return DDP_OK;
    if (!param_flat || !aligned(param_flat, 4)) return DDP_ERR_INVALID_ARG;
    if (momentum_flat && !aligned(momentum_flat, 4)) return DDP_ERR_INVALID_ARG;
    const int isz = dtype_size(in), osz = dtype_size(out_dtype);
    // parameters and momentum are written: they may overlap nothing else
    const uintptr_t pa = reinterpret_cast<uintptr_t>(param_flat);
    const uintptr_t ma = reinterpret_cast<uintptr_t>(momentum_flat);
    const uintptr_t ga = reinterpret_cast<uintptr_t>(grad_out);
    for (int r = 0; r < n_ranks; ++r) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(rank_flat[r]);
        if (overlaps(x, total * isz, pa, total * 4)) return DDP_ERR_ALIAS;
        if (momentum_flat && overlaps(x, total * isz, ma, total * 4)) return DDP_ERR_ALIAS;
    }
    if (grad_out && overlaps(ga, total * osz, pa, total * 4)) return DDP_ERR_ALIAS;
    if (momentum_flat && grad_out && overlaps(ga, total * osz, ma, total * 4)) return DDP_ERR_ALIAS;
    if (momentum_flat && overlaps(pa, total * 4, ma, total * 4)) return DDP_ERR_ALIAS;

    hipStream_t st = static_cast<hipStream_t>(stream);
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));
    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    // every buffer is read and written at whatever element alignment it has
    for (int r = 0; r < n_ranks; ++r) ra.p[r] = rank_flat[r];
    const SgdArgs sa = {param_flat, momentum_flat, grad_out, lr, momentum};
    if (order == DDP_ORDER_SEQUENTIAL || n_ranks == 1) {
        // neither depends on bucket boundaries (one rank: the input itself)
        return launch_sgd(ra, n_ranks, total, order, in, out_dtype, single_bucket(0, total), sa, st);
    }
    Buckets bk;
    if ((stc = ring_buckets(plan, in, n_ranks, &bk)) != DDP_OK) return stc;
    return launch_sgd(ra, n_ranks, total, order, in, out_dtype, bk, sa, st);
}

}  // extern "C"
