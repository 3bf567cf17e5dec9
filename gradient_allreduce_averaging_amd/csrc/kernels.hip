// HIP kernels of libddp for gfx950 (MI355X) and the C-ABI entry points that
// launch them.
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel);
//        [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn).
//
// Reduce + scale ([TR24] 一 and 九; [DDP] 2.10-2.11, 4.2).  Every output
// element is owned by exactly one thread, which loads that element from all
// N rank buffers, folds the N values in the fixed order in FP32, multiplies
// by fl(1/N) and stores (optionally rounded to bf16, nearest-even).  There is
// no cross-thread reduction, so the result does not depend on the grid.
//
// Layout and launch.  A block is one wave and owns a tile of 64 16-byte
// vectors (256 f32 or 512 bf16 elements): each wave load is 1 KiB contiguous
// per rank.  A lane issues its N loads (every rank at its own offset, in rank
// order) before anything else, so N * 16 bytes per lane are in flight; loads
// and stores are non-temporal.  Launches cap the resident blocks per CU with
// an unused dynamic-LDS reservation (see "occupancy").  The path is HBM-bound
// (0.22 flop/byte for FP32, N = 8): no LDS traffic, no MFMA, no cross-lane
// work.
//
// Ring order.  Element i of a bucket [base, end) sits in chunk
// c = (i - base) / C with C = ceil((end - base) / N) and starts its fold at
// rank (c + 1) mod N.  While its loads are in flight a tile reads one
// precomputed word naming the chunk segment holding its first element and
// the segment after it (start ranks and in-tile ends); a lane whose vector
// lies wholly inside either folds from registers in that segment's rotated
// order, and a vector straddling a chunk or bucket boundary (at most a few
// per bucket) or the ragged tail takes a per-element path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "internal.h"

namespace {

// Reduce tiles: one wave per block, one 16-byte vector per lane and rank.
// Many short single-wave blocks keep every CU's queue full to the end of the
// grid; measured against 128/256/512-thread blocks and 2-4 vectors per lane,
// this shape streams fastest on gfx950 for every workload shape tried.
constexpr int kThreads = 64;
constexpr int kUnroll = 1;             // 16-byte vectors per lane per rank
constexpr int kTileTableShift = 6;     // one bucket-table entry per 64 tiles
static_assert(kThreads * kUnroll * 8 <= 1023 && DDP_MAX_RANKS <= 64,
              "a ring-segment word holds 10-bit tile offsets and 6-bit ranks");
constexpr int kCopyThreads = 256;      // flatten / unflatten blocks
constexpr int64_t kCopyUnitElems = 4096;    // elements per copy-table entry
constexpr int64_t kCopyBlockElems = 2048;   // elements per copy block: a unit gets
constexpr int kCopyBlocksPerUnit = (int)(kCopyUnitElems / kCopyBlockElems);   // this many blocks
static_assert(kCopyUnitElems % kCopyBlockElems == 0, "a copy unit splits into whole blocks");

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct RankArgs {
    const void *p[DDP_MAX_RANKS];
};

// Bucket boundaries as the kernels see them.  base == nullptr means a single
// bucket [0, total).
struct Buckets {
    const int64_t *base;          // [n_buckets + 1]
    const int32_t *tile_bucket;   // [ceil(n_tiles / 2^kTileTableShift)] bucket of the
                                  // first element of every 2^kTileTableShift-th tile
    const uint32_t *tile_desc;    // ring segments of every tile (encoding at tile_segs,
                                  // layout at ring_tile_desc), or null for a single bucket
    int64_t desc_stride;          // tiles per XCD stripe of tile_desc
    int64_t lo, hi;               // base == nullptr: the one bucket is [lo, hi) in the
                                  // launch's element numbering (lo < 0 when the launch
                                  // starts past the bucket's first elements)
    int32_t n_buckets;
};

// One bucket spanning [lo, hi) of a launch's elements.
__host__ __device__ inline Buckets single_bucket(int64_t lo, int64_t hi)
{
    return {nullptr, nullptr, nullptr, 0, lo, hi, 1};
}

// Workgroups are dealt to the XCDs round-robin, so tile t runs on XCD t % 8.
constexpr int kXcds = 8;

// The chunk segments a tile may meet on the vector path.
struct Segs {
    int64_t a_lo, a_hi, b_lo, b_hi;
    int sa, sb;
};

// Streaming 16-byte accesses of the reduce.  Every byte is touched once, so
// they are non-temporal (the `nt` cache policy): on gfx950 this lifts a pure
// streaming read from ~6.5 to ~7.2 TB/s and the reduce by ~15 %.
__device__ __forceinline__ u32x4 ld_stream(const char *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
template <typename V>
__device__ __forceinline__ void st_stream(void *p, const V &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<V *>(p));
}

__device__ __forceinline__ float widen_bf16(uint32_t h) { return __uint_as_float(h << 16); }

// f32 -> bf16, round to nearest, ties to even; NaN stays NaN (quiet, sign kept).
__device__ __forceinline__ uint32_t bf16_rne(float y)
{
    const uint32_t u = __float_as_uint(y);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Element e of a 16-byte vector, widened to FP32.
template <int IN>
__device__ __forceinline__ float lane(const u32x4 &v, int e)
{
    if (IN == kF32) return __uint_as_float(v[e]);
    const uint32_t w = v[e >> 1];
    return (e & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

template <int IN>
__device__ __forceinline__ float load_elem(const void *p, int64_t i)
{
    if (IN == kF32) return static_cast<const float *>(p)[i];
    return widen_bf16(static_cast<const uint16_t *>(p)[i]);
}

template <int OUT>
__device__ __forceinline__ void store_elem(void *out, int64_t i, float y)
{
    if (OUT == kF32)
        static_cast<float *>(out)[i] = y;
    else
        static_cast<uint16_t *>(out)[i] = (uint16_t)bf16_rne(y);
}

__device__ __forceinline__ int wrap(int r, int n) { return r >= n ? r - n : r; }

// Ring start rank of element i (any bucket at or after b0).
__device__ __forceinline__ int ring_start(const Buckets &bk, int32_t b0, int64_t total, int N,
                                          int64_t i)
{
    int64_t base = bk.lo, end = bk.hi;
    if (bk.base) {
        int32_t b = b0;
        while (bk.base[b + 1] <= i) ++b;
        base = bk.base[b];
        end = bk.base[b + 1];
    }
    const int64_t C = (end - base + N - 1) / N;
    return (int)(((i - base) / C + 1) % N);
}

// The scaled average of element i, one element at a time (N >= 2).
template <int IN, bool RING>
__device__ __forceinline__ float avg_elem(const RankArgs &ra, int N, int64_t total,
                                          const Buckets &bk, int32_t b0, float inv, int64_t i)
{
    int r = RING ? ring_start(bk, b0, total, N, i) : 0;
    float acc = load_elem<IN>(ra.p[r], i);
    if (!RING) acc = 0.0f + acc;
    for (int k = 1; k < N; ++k) {
        r = wrap(r + 1, N);
        acc = acc + load_elem<IN>(ra.p[r], i);
    }
    return acc * inv;
}

// Per-element path: positions [i0, i0 + cnt) clipped to total.
template <int IN, int OUT, bool RING>
__device__ void reduce_elems(const RankArgs &ra, int N, int64_t total, const Buckets &bk,
                             int32_t b0, float inv, void *out, int64_t i0, int cnt)
{
    for (int e = 0; e < cnt; ++e) {
        const int64_t i = i0 + e;
        if (i >= total) break;
        store_elem<OUT>(out, i, avg_elem<IN, RING>(ra, N, total, bk, b0, inv, i));
    }
}

// ---------------------------------------------------------------- SGD epilogue
// The optimizer step the 1/N average can be folded into ([TR24] 九, note on
// removing the separate scale kernel; update rule of [DDP] 5.3):
//   g = the averaged gradient as stored (bf16: rounded, then widened back)
//   momentum (optional): v = mu * m + g; m = v; g = v
//   p = p - lr * g
struct SgdArgs {
    float *param;      // flat f32 parameters, updated in place
    float *mom;        // flat f32 momentum buffer, or null
    void *grad_out;    // flat averaged gradient (OUT elements), or null
    float lr, mu;
};

template <bool MOM>
__device__ __forceinline__ float sgd_elem(float p, float g, float &m, float lr, float mu)
{
    if (MOM) {
        float v = mu * m;
        v = v + g;
        m = v;
        g = v;
    }
    const float step = lr * g;
    return p - step;
}

// Per-element fused path.  N == 1 takes the input as the average, bit for bit.
template <int IN, int OUT, bool RING, bool MOM>
__device__ void sgd_elems(const RankArgs &ra, int N, int64_t total, const Buckets &bk, int32_t b0,
                          float inv, const SgdArgs &sa, int64_t i0, int cnt)
{
    for (int e = 0; e < cnt; ++e) {
        const int64_t i = i0 + e;
        if (i >= total) break;
        const float y = N == 1 ? load_elem<IN>(ra.p[0], i) : avg_elem<IN, RING>(ra, N, total, bk, b0, inv, i);
        float g = y;
        if (OUT == kBF16) {
            const uint32_t h = bf16_rne(y);
            g = widen_bf16(h);
            if (sa.grad_out) static_cast<uint16_t *>(sa.grad_out)[i] = (uint16_t)h;
        } else if (sa.grad_out) {
            static_cast<float *>(sa.grad_out)[i] = y;
        }
        float m = MOM ? sa.mom[i] : 0.0f;
        sa.param[i] = sgd_elem<MOM>(sa.param[i], g, m, sa.lr, sa.mu);
        if (MOM) sa.mom[i] = m;
    }
}

// Tile processed by this block.
__device__ __forceinline__ int64_t tile_of_block() { return blockIdx.x; }

// A single bucket that starts before the launch's element 0 (lo < 0: its
// first -lo elements sit just before the aligned address the vector path
// starts at) gets one extra block at the end of the grid.  Its tile lies past
// the end, so the vector path finds no work there (its loads read the dummy
// vector), and this reduces the head elements one per lane.  The check comes
// after the vector path, so no other block waits on it before its loads.
template <int IN, int OUT, bool RING>
__device__ __forceinline__ void head_block(const RankArgs &ra, int N, int64_t total,
                                           const Buckets &bk, float inv, void *out)
{
    if (bk.base || bk.lo >= 0 || blockIdx.x != gridDim.x - 1) return;
    if (threadIdx.x < -bk.lo)
        reduce_elems<IN, OUT, RING>(ra, N, total, bk, 0, inv, out, bk.lo + threadIdx.x, 1);
}

// Ring segments of tile `tile`, whose first element is tile0 (block-uniform
// values): segment a holds the tile's first element, segment b follows it
// (b_lo == a_hi; b is empty when a reaches the end).  A vector inside one of
// them folds with that segment's start rank; any other takes the per-element
// path.  With a plan the segments come from one precomputed word per tile,
// so a wave makes a single scalar load, issued while its vector loads are in
// flight:
//   bits 0-5 start rank of a, 6-11 start rank of b,
//   12-21 end of a and 22-31 end of b, both relative to tile0.
// A single bucket [lo, hi) is computed here.
template <bool RING>
__device__ __forceinline__ Segs tile_segs(const Buckets &bk, int64_t total, int N, int64_t tile,
                                          int64_t tile0)
{
    Segs s;
    s.a_lo = 0;
    s.a_hi = total;
    s.b_lo = 0;
    s.b_hi = 0;
    s.sa = 0;
    s.sb = 0;
    if (!RING) return s;
    if (bk.tile_desc) {
        const uint32_t d = bk.tile_desc[(tile % kXcds) * bk.desc_stride + tile / kXcds];
        s.sa = (int)(d & 63u);
        s.sb = (int)((d >> 6) & 63u);
        s.a_lo = tile0;
        s.a_hi = tile0 + (int64_t)((d >> 12) & 1023u);
        s.b_lo = s.a_hi;
        s.b_hi = tile0 + (int64_t)(d >> 22);
    } else {
        const int64_t C = (bk.hi - bk.lo + N - 1) / N;
        const int64_t c = (tile0 - bk.lo) / C;
        s.a_lo = bk.lo + c * C;
        s.a_hi = min(s.a_lo + C, bk.hi);
        s.sa = (int)((c + 1) % N);
        s.b_lo = s.b_hi = s.a_hi;
        if (s.a_hi < bk.hi) {
            s.b_hi = min(s.b_lo + C, bk.hi);
            s.sb = (int)((c + 2) % N);
        }
    }
    s.sa = __builtin_amdgcn_readfirstlane(s.sa);
    s.sb = __builtin_amdgcn_readfirstlane(s.sb);
    return s;
}

// A bucket at or before the one holding tile0, where the per-element path
// starts its forward search.
__device__ __forceinline__ int32_t first_bucket(const Buckets &bk, int64_t tile)
{
    return bk.tile_bucket ? bk.tile_bucket[tile >> kTileTableShift] : 0;
}

// The fold of one lane's vectors, v[k] holding rank k's vector at the lane's
// offset.  Ring order starting at rank R:
//   acc = ((x_R + x_{R+1}) + ...) + x_{R-1}   (ranks mod NR)
template <int NR, int IN, int R>
__device__ __forceinline__ void fold_from(const u32x4 *v, float *acc)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
#pragma unroll
    for (int e = 0; e < VEC; ++e) acc[e] = lane<IN>(v[R], e);
#pragma unroll
    for (int k = 1; k < NR; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + lane<IN>(v[(R + k) % NR], e);
}

// Rotation R behind its branch: an empty volatile asm inside the branch
// claims to rewrite the inputs (in place, so no copies stay live), so the adds
// that read them cannot be hoisted above it.  Without this the compiler
// evaluates all NR rotations and selects one: NR times the adds and twice the
// registers.  The values are untouched.
template <int NR, int IN, int R>
__device__ __forceinline__ void fold_from_here(u32x4 *v, float *acc)
{
#pragma unroll
    for (int k = 0; k < NR; ++k) asm volatile("" : "+v"(v[k]));
    fold_from<NR, IN, R>(v, acc);
}

// The same for a start rank s known at run time (one of the tile's two, so
// at most two of the branches run): a branch picks one of the NR
// compile-time rotations.
template <int NR, int IN, int R = 0>
__device__ __forceinline__ void fold_ring(u32x4 *v, int s, float *acc)
{
    if constexpr (R + 1 < NR) {
        if (s == R)
            fold_from_here<NR, IN, R>(v, acc);
        else
            fold_ring<NR, IN, R + 1>(v, s, acc);
    } else {
        fold_from_here<NR, IN, R>(v, acc);
    }
}

// Sequential order: acc = ((+0 + x_0) + x_1) + ... + x_{NR-1}; with one rank
// the input itself.
template <int NR, int IN>
__device__ __forceinline__ void fold_seq(const u32x4 *v, float *acc)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
        const float x = lane<IN>(v[0], e);
        acc[e] = NR == 1 ? x : 0.0f + x;
    }
#pragma unroll
    for (int k = 1; k < NR; ++k)
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[e] = acc[e] + lane<IN>(v[k], e);
}

// Any N up to DDP_MAX_RANKS: the ranks walked in the fold order starting at
// the wave-uniform rank s, eight loads in flight at a time.  Every rank
// pointer is a scalar load, and a short last group is cut by a uniform
// branch rather than dummy loads.  Lanes not taking part pass off = 0 and
// re-read vector 0.
template <int IN, bool RING>
__device__ __forceinline__ void fold_looped(const RankArgs &ra, int N, int s, int64_t off,
                                            float *acc)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int G = 8;
#pragma unroll 1
    for (int k0 = 0; k0 < N; k0 += G) {
        u32x4 v[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (k0 + j < N) {
                int r = s + k0 + j;
                r = r >= N ? r - N : r;
                v[j] = ld_stream(static_cast<const char *>(ra.p[r]) + off);
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (k0 + j < N) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const float x = lane<IN>(v[j], e);
                    acc[e] = k0 + j > 0 ? acc[e] + x : (RING ? x : 0.0f + x);
                }
            }
        }
    }
}

// Convert and store one vector of scaled averages y at element i0; for a
// bf16 output y is replaced by the stored value widened back to f32.
template <int IN, int OUT>
__device__ __forceinline__ void store_y(void *out, int64_t i0, float *y, bool write)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    if (OUT == kF32) {
        u32x4 o;
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(y[e]);
        if (write) st_stream(static_cast<float *>(out) + i0, o);
    } else {
        uint32_t h[VEC];
        for (int e = 0; e < VEC; ++e) {
            h[e] = bf16_rne(y[e]);
            y[e] = widen_bf16(h[e]);
        }
        if (VEC == 4) {
            u32x2 o;
            o[0] = h[0] | (h[1] << 16);
            o[1] = h[2] | (h[3] << 16);
            if (write) st_stream(static_cast<uint16_t *>(out) + i0, o);
        } else {
            u32x4 o;
            for (int w = 0; w < 4; ++w) o[w] = h[2 * w] | (h[2 * w + 1] << 16);
            if (write) st_stream(static_cast<uint16_t *>(out) + i0, o);
        }
    }
}

// Scale, convert and store one vector of accumulators at element i0.
template <int IN, int OUT>
__device__ __forceinline__ void store_vec(void *out, int64_t i0, const float *acc, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    float y[VEC];
    for (int e = 0; e < VEC; ++e) y[e] = acc[e] * inv;
    store_y<IN, OUT>(out, i0, y, true);
}

// N known at compile time (2..8): all N * kUnroll vector loads in flight.
template <int NR, bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
reduce_fast(RankArgs ra, int64_t total, Buckets bk, float inv, void *out)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const int64_t tile = tile_of_block();
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
    head_block<IN, OUT, RING>(ra, NR, total, bk, inv, out);
}

// The vector epilogue of the fused step: store the average y (bf16: y
// becomes the stored value widened back), then update the lane's parameter
// vectors pv (and momentum mv), already loaded, in place.
template <int IN, int OUT, bool MOM>
__device__ __forceinline__ void sgd_vec(const SgdArgs &sa, int64_t i0, float *y, const u32x4 *pv,
                                        const u32x4 *mv)
{
    constexpr int PV = (IN == kF32 ? 4 : 8) / 4;
    store_y<IN, OUT>(sa.grad_out, i0, y, sa.grad_out != nullptr);
#pragma unroll
    for (int j = 0; j < PV; ++j) {
        u32x4 po, mo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float m = MOM ? __uint_as_float(mv[j][w]) : 0.0f;
            po[w] = __float_as_uint(
                sgd_elem<MOM>(__uint_as_float(pv[j][w]), y[4 * j + w], m, sa.lr, sa.mu));
            mo[w] = __float_as_uint(m);
        }
        st_stream(sa.param + i0 + 4 * j, po);
        if (MOM) st_stream(sa.mom + i0 + 4 * j, mo);
    }
}

// Fused average + SGD step, N known at compile time (1..8).  Per lane: the N
// gradient vectors and the lane's parameter (and momentum) vectors are loaded
// together, the average is folded and scaled, optionally stored, and the
// parameters updated in place.  Parameters are f32: one 16-byte vector per 4
// elements, so a bf16 lane (8 elements) moves two.
template <int NR, bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
reduce_sgd_fast(RankArgs ra, int64_t total, Buckets bk, float inv, SgdArgs sa)
{
    static_assert(kUnroll == 1, "the fused kernel processes one vector per lane");
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    const int64_t tile = tile_of_block();
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

// Fused average + SGD step, one element per thread, element-aligned buffers
// of a single bucket, any N.
template <bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
reduce_sgd_scalar(RankArgs ra, int N, int64_t total, Buckets bk, float inv, SgdArgs sa)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    sgd_elems<IN, OUT, RING, MOM>(ra, N, total, bk, 0, inv, sa, i, 1);
}

// ---------------------------------------------------------------- accumulate
// Local accumulation between synchronisations ([DDP] 5.2, no_sync):
// dst[k] += src[k] for every buffer pair k (grid row k), one f32 add per
// element (bf16: widened, added, rounded to nearest even).
struct AccArgs {
    char *dst[DDP_MAX_RANKS];
    const char *src[DDP_MAX_RANKS];
};

template <int DT>
__device__ __forceinline__ void acc_elem(char *d, const char *s, int64_t i)
{
    store_elem<DT>(d, i, load_elem<DT>(d, i) + load_elem<DT>(s, i));
}

template <int DT>
__global__ void __launch_bounds__(kThreads) accumulate_vec(AccArgs a, int64_t len)
{
    constexpr int VEC = DT == kF32 ? 4 : 8;
    constexpr int ISZ = DT == kF32 ? 4 : 2;
    char *d = a.dst[blockIdx.y];
    const char *s = a.src[blockIdx.y];
    const int64_t i0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * VEC;
    if (i0 + VEC <= len) {
        const u32x4 x = ld_stream(d + i0 * ISZ), y = ld_stream(s + i0 * ISZ);
        u32x4 o;
        if (DT == kF32) {
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(__uint_as_float(x[w]) + __uint_as_float(y[w]));
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w)
                o[w] = bf16_rne(lane<kBF16>(x, 2 * w) + lane<kBF16>(y, 2 * w)) |
                       (bf16_rne(lane<kBF16>(x, 2 * w + 1) + lane<kBF16>(y, 2 * w + 1)) << 16);
        }
        st_stream(d + i0 * ISZ, o);
    } else {
        for (int64_t i = i0; i < len && i < i0 + VEC; ++i) acc_elem<DT>(d, s, i);
    }
}

template <int DT>
__global__ void __launch_bounds__(kThreads) accumulate_scalar(AccArgs a, int64_t len)
{
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < len) acc_elem<DT>(a.dst[blockIdx.y], a.src[blockIdx.y], i);
}

// Any N up to DDP_MAX_RANKS.  A wave makes one pass per ring segment its
// lanes lie in (usually one), so the rank order of each pass is
// wave-uniform, and folds with fold_looped.
template <bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
reduce_many(RankArgs ra, int N, int64_t total, Buckets bk, float inv, void *out)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    static_assert(kUnroll == 1, "one vector per lane");
    const int64_t tile = tile_of_block();
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
        fold_looped<IN, RING>(ra, N, pass == 0 ? sg.sa : sg.sb, mine ? i0 * ISZ : 0, acc);
        if (mine) store_vec<IN, OUT>(out, i0, acc, inv);
    }
    if (!in_a && !in_b && i0 < total)
        reduce_elems<IN, OUT, RING>(ra, N, total, bk, first_bucket(bk, tile), inv, out, i0, VEC);
    head_block<IN, OUT, RING>(ra, N, total, bk, inv, out);
}

// The fused average + SGD step for any N up to DDP_MAX_RANKS: the lane's
// parameter (and momentum) vectors are issued first, then the ranks are
// folded as in reduce_many and the epilogue of reduce_sgd_fast applied.
template <bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
reduce_sgd_many(RankArgs ra, int N, int64_t total, Buckets bk, float inv, SgdArgs sa)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    static_assert(kUnroll == 1, "one vector per lane");
    const int64_t tile = tile_of_block();
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
        fold_looped<IN, RING>(ra, N, pass == 0 ? sg.sa : sg.sb, mine ? i0 * ISZ : 0, y);
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
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= total) return;
    reduce_elems<IN, OUT, RING>(ra, N, total, bk, 0, inv, out, i, 1);
}

// ---------------------------------------------------------------- copies

__device__ __forceinline__ void copy16b(char *dst, const char *src, int64_t lo, int64_t hi)
{
    for (int64_t j = lo + 2 * (int64_t)threadIdx.x; j < hi; j += 2 * kCopyThreads)
        *reinterpret_cast<uint16_t *>(dst + j) = *reinterpret_cast<const uint16_t *>(src + j);
}

// Block-wide copy of nbytes (a multiple of 2) between 2-byte aligned addresses.
__device__ void block_copy(char *dst, const char *src, int64_t nbytes)
{
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
    const uintptr_t s = reinterpret_cast<uintptr_t>(src);
    const int tid = threadIdx.x;
    if (((d ^ s) & 15) == 0) {
        const int64_t head = min<int64_t>((16 - (d & 15)) & 15, nbytes);
        copy16b(dst, src, 0, head);
        const int64_t nvec = (nbytes - head) >> 4;
        const u32x4 *sv = reinterpret_cast<const u32x4 *>(src + head);
        u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
        int64_t j = tid;
        for (; j + kCopyThreads < nvec; j += 2 * kCopyThreads) {   // both loads before the stores
            const u32x4 a = __builtin_nontemporal_load(sv + j);
            const u32x4 b = __builtin_nontemporal_load(sv + j + kCopyThreads);
            __builtin_nontemporal_store(a, dv + j);
            __builtin_nontemporal_store(b, dv + j + kCopyThreads);
        }
        for (; j < nvec; j += kCopyThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(sv + j), dv + j);
        copy16b(dst, src, head + (nvec << 4), nbytes);
    } else if (((d ^ s) & 3) == 0) {
        const int64_t head = min<int64_t>((4 - (d & 3)) & 3, nbytes);
        copy16b(dst, src, 0, head);
        const int64_t nw = (nbytes - head) >> 2;
        const uint32_t *sw = reinterpret_cast<const uint32_t *>(src + head);
        uint32_t *dw = reinterpret_cast<uint32_t *>(dst + head);
        int64_t j = tid;
        for (; j + 3 * kCopyThreads < nw; j += 4 * kCopyThreads) {
            const uint32_t a = __builtin_nontemporal_load(sw + j);
            const uint32_t b = __builtin_nontemporal_load(sw + j + kCopyThreads);
            const uint32_t c = __builtin_nontemporal_load(sw + j + 2 * kCopyThreads);
            const uint32_t e = __builtin_nontemporal_load(sw + j + 3 * kCopyThreads);
            __builtin_nontemporal_store(a, dw + j);
            __builtin_nontemporal_store(b, dw + j + kCopyThreads);
            __builtin_nontemporal_store(c, dw + j + 2 * kCopyThreads);
            __builtin_nontemporal_store(e, dw + j + 3 * kCopyThreads);
        }
        for (; j < nw; j += kCopyThreads) __builtin_nontemporal_store(__builtin_nontemporal_load(sw + j), dw + j);
        copy16b(dst, src, head + (nw << 2), nbytes);
    } else {
        copy16b(dst, src, 0, nbytes);
    }
}

// kCopyBlocksPerUnit blocks per copy unit, each moving up to kCopyBlockElems
// elements of it (parts past a short unit's end return at once); to_flat
// selects flatten (param -> flat) or unflatten (flat -> param).  The blocks
// of one unit run on one XCD (workgroups are dealt to the XCDs round-robin,
// so block b runs on XCD b % 8), where the unit's table entry is then an L2
// hit for all but the first of them.  Units hold 4K elements: with many
// short parameters, bigger units mostly spawn blocks that find no work.
__global__ void __launch_bounds__(kCopyThreads)
copy_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, char *flat, int esize,
           int to_flat)
{
    const int64_t m = blockIdx.x / kXcds;
    const int64_t ui = (m / kCopyBlocksPerUnit) * kXcds + blockIdx.x % kXcds;
    if (ui >= n_units) return;
    const ddp_copy_unit u = units[first + ui];
    const int64_t lo = (m % kCopyBlocksPerUnit) * kCopyBlockElems;
    if (lo >= u.count) return;
    const int64_t n = min(u.count - lo, kCopyBlockElems);
    char *pp = reinterpret_cast<char *>(u.param_addr) + (u.param_elem + lo) * esize;
    char *fp = flat + (u.flat_elem + lo) * esize;
    const int64_t nbytes = n * esize;
    if (to_flat)
        block_copy(fp, pp, nbytes);
    else
        block_copy(pp, fp, nbytes);
}

// ---------------------------------------------------------------- host side

thread_local char g_last_error[256] = "";

// Records a failed HIP call for ddp_last_error() and maps it to a status.
ddp_status_t hip_fail(const char *what, hipError_t e, ddp_status_t st = DDP_ERR_HIP)
{
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return st;
}

ddp_status_t launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DDP_OK : hip_fail(what, e);
}

int dtype_size(int dt) { return dt == DDP_BF16 ? 2 : 4; }
bool dtype_ok(int dt) { return dt == DDP_F32 || dt == DDP_BF16; }
bool pair_ok(int in, int out)
{
    return (in == DDP_F32 && out == DDP_F32) || (in == DDP_BF16 && out == DDP_BF16) ||
           (in == DDP_F32 && out == DDP_BF16);
}
int64_t vec_elems(int in) { return in == DDP_F32 ? 4 : 8; }
int64_t tile_elems(int in) { return (int64_t)kThreads * kUnroll * vec_elems(in); }

// ---------------------------------------------------------------- occupancy
// These streaming kernels move the most bytes per second on gfx950 with fewer
// resident blocks per CU than registers alone would allow (up to 32 of these
// one-wave blocks): past a point, more concurrent waves only open more DRAM
// rows at once.  Each launch is therefore capped at k resident blocks per CU
// by asking for LDS_per_CU / k bytes of dynamic LDS, which the kernels do not
// touch.  k was measured per kernel and rank count on ResNet-50, many-small,
// GPT-1.3B and Llama-7B shapes; 0 means no cap.

// Reduce, N = 2..8 (one 16-byte load per rank and lane, one store); the
// looped kernel for N > 8.
int reduce_blocks_per_cu(int N, bool ring)
{
    static const int k[9] = {0, 0, 0, 16, 14, 12, 10, 9, 8};
    if (N < 0) return 0;
    if (N <= 8) return k[N];
    return N <= 11 ? (ring ? 12 : 10) : 8;
}

// Fused average + SGD step, N = 1..8 (also the parameter, momentum loads and
// stores); the looped kernel for N > 8.
int sgd_blocks_per_cu(int N, bool mom)
{
    static const int with_mom[9] = {0, 20, 14, 10, 8, 8, 7, 7, 6};
    static const int without[9] = {0, 0, 0, 0, 0, 10, 8, 8, 8};
    if (N < 0) return 0;
    if (N > 8) return N <= 11 ? (mom ? 10 : 12) : 8;
    return mom ? with_mom[N] : without[N];
}

// Flatten / unflatten (256-thread blocks).
constexpr int kCopyBlocksPerCU = 7;

constexpr int kMaxDevices = 64;

// DDP_OCCUPANCY_TUNED or DDP_OCCUPANCY_SHARED, process-wide.
std::atomic<int> g_occupancy{DDP_OCCUPANCY_TUNED};

// Dynamic LDS bytes that leave room for k blocks per CU on the current device
// (none under DDP_OCCUPANCY_SHARED).
unsigned lds_for_blocks(int k)
{
    static std::atomic<int> lds_per_cu[kMaxDevices];   // 0: not queried yet, -1: unknown
    if (k <= 0 || g_occupancy.load(std::memory_order_relaxed) != DDP_OCCUPANCY_TUNED) return 0;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
    int v = lds_per_cu[dev].load(std::memory_order_relaxed);
    if (v == 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
                hipSuccess ||
            v <= 0)
            v = -1;
        lds_per_cu[dev].store(v, std::memory_order_relaxed);
    }
    return v > 0 ? (unsigned)(v / k) : 0;
}

bool overlaps(uintptr_t a, int64_t na, uintptr_t b, int64_t nb)
{
    return a < b + (uintptr_t)nb && b < a + (uintptr_t)na;
}

// Output may be exactly one input (same dtype) or disjoint from all of them.
ddp_status_t check_alias(const void *const *in, int n, int64_t len, int isz, const void *out,
                         int osz)
{
    const uintptr_t o = reinterpret_cast<uintptr_t>(out);
    for (int r = 0; r < n; ++r) {
        const uintptr_t x = reinterpret_cast<uintptr_t>(in[r]);
        if (x == o && isz == osz) continue;
        if (overlaps(x, len * isz, o, len * osz)) return DDP_ERR_ALIAS;
    }
    return DDP_OK;
}

template <bool RING, int IN, int OUT>
ddp_status_t launch_typed(const RankArgs &ra, int N, int64_t total, const Buckets &bk, float inv,
                          void *out, hipStream_t st, bool vec_ok)
{
    if (vec_ok) {
        const int64_t tiles = (total + tile_elems(IN) - 1) / tile_elems(IN) +
                              (!bk.base && bk.lo < 0 ? 1 : 0);   // + the head block
        if (tiles > INT_MAX) return DDP_ERR_OVERFLOW;
        const dim3 g((unsigned)tiles), b(kThreads);
        const unsigned lds = lds_for_blocks(reduce_blocks_per_cu(N, RING));
        switch (N) {
        case 2: reduce_fast<2, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 3: reduce_fast<3, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 4: reduce_fast<4, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 5: reduce_fast<5, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 6: reduce_fast<6, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 7: reduce_fast<7, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        case 8: reduce_fast<8, RING, IN, OUT><<<g, b, lds, st>>>(ra, total, bk, inv, out); break;
        default: reduce_many<RING, IN, OUT><<<g, b, lds, st>>>(ra, N, total, bk, inv, out); break;
        }
    } else {
        const int64_t blocks = (total + kThreads - 1) / kThreads;
        if (blocks > INT_MAX) return DDP_ERR_OVERFLOW;
        reduce_scalar<RING, IN, OUT><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
            ra, N, total, bk, inv, out);
    }
    return launched("reduce kernel launch");
}

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

// One bucket of len elements.  The vector kernel wants its inputs 16-byte
// aligned (the vector width) and streams best from 128-byte aligned tiles
// (an L2 line: a misaligned 1 KiB wave load touches 9 lines instead of 8).
// When every rank buffer sits at the same offset from a 128-byte boundary
// -- a bucket at an unpadded offset into equally aligned flat buffers -- the
// vector path starts at the next boundary, h elements in, and numbers the
// bucket [-h, len - h) so that the ring chunks stay those of the whole
// bucket; the launch's extra head block reduces the first h elements one by
// one.  Sharing only the offset from a 16-byte boundary, it starts at the
// next 16-byte boundary instead.  Otherwise the per-element kernel takes it
// all.  The output must be aligned for the vector stores at the same point.
ddp_status_t launch_one_bucket(const RankArgs &ra, int N, int64_t len, int order, int in,
                               int out_dt, void *out, hipStream_t st)
{
    const int isz = dtype_size(in), osz = dtype_size(out_dt);
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(ra.p[0]);
    bool same128 = true, same16 = a0 % isz == 0;
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
    if (h < 0)
        return launch_reduce(ra, N, len, order, in, out_dt, single_bucket(0, len), out, st, false);
    RankArgs rest;
    std::memset(&rest, 0, sizeof(rest));
    for (int r = 0; r < N; ++r) rest.p[r] = static_cast<const char *>(ra.p[r]) + h * isz;
    return launch_reduce(rest, N, len - h, order, in, out_dt, single_bucket(-h, len - h),
                         static_cast<char *>(out) + h * osz, st, true);
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

template <bool RING, int IN, int OUT, bool MOM>
ddp_status_t launch_sgd_typed(const RankArgs &ra, int N, int64_t total, const Buckets &bk,
                              float inv, const SgdArgs &sa, hipStream_t st, bool vec_ok)
{
    if (vec_ok) {
        const int64_t tiles = (total + tile_elems(IN) - 1) / tile_elems(IN);
        if (tiles > INT_MAX) return DDP_ERR_OVERFLOW;
        const dim3 g((unsigned)tiles), b(kThreads);
        const unsigned lds = lds_for_blocks(sgd_blocks_per_cu(N, MOM));
        switch (N) {
        case 1: reduce_sgd_fast<1, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 2: reduce_sgd_fast<2, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 3: reduce_sgd_fast<3, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 4: reduce_sgd_fast<4, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 5: reduce_sgd_fast<5, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 6: reduce_sgd_fast<6, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 7: reduce_sgd_fast<7, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        case 8: reduce_sgd_fast<8, RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, total, bk, inv, sa); break;
        default: reduce_sgd_many<RING, IN, OUT, MOM><<<g, b, lds, st>>>(ra, N, total, bk, inv, sa); break;
        }
    } else {
        const int64_t blocks = (total + kThreads - 1) / kThreads;
        if (blocks > INT_MAX) return DDP_ERR_OVERFLOW;
        reduce_sgd_scalar<RING, IN, OUT, MOM><<<dim3((unsigned)blocks), dim3(kThreads), 0, st>>>(
            ra, N, total, bk, inv, sa);
    }
    return launched("fused SGD kernel launch");
}

template <bool RING, bool MOM>
ddp_status_t launch_sgd_pair(const RankArgs &ra, int N, int64_t total, int in, int out_dt,
                             const Buckets &bk, float inv, const SgdArgs &sa, hipStream_t st,
                             bool vec_ok)
{
    if (in == DDP_F32 && out_dt == DDP_F32)
        return launch_sgd_typed<RING, kF32, kF32, MOM>(ra, N, total, bk, inv, sa, st, vec_ok);
    if (in == DDP_BF16 && out_dt == DDP_BF16)
        return launch_sgd_typed<RING, kBF16, kBF16, MOM>(ra, N, total, bk, inv, sa, st, vec_ok);
    return launch_sgd_typed<RING, kF32, kBF16, MOM>(ra, N, total, bk, inv, sa, st, vec_ok);
}

ddp_status_t launch_sgd(const RankArgs &ra, int N, int64_t total, int order, int in, int out_dt,
                        const Buckets &bk, const SgdArgs &sa, hipStream_t st, bool vec_ok)
{
    const float inv = 1.0f / (float)N;
    const bool ring = order == DDP_ORDER_RING, mom = sa.mom != nullptr;
    if (ring)
        return mom ? launch_sgd_pair<true, true>(ra, N, total, in, out_dt, bk, inv, sa, st, vec_ok)
                   : launch_sgd_pair<true, false>(ra, N, total, in, out_dt, bk, inv, sa, st, vec_ok);
    return mom ? launch_sgd_pair<false, true>(ra, N, total, in, out_dt, bk, inv, sa, st, vec_ok)
               : launch_sgd_pair<false, false>(ra, N, total, in, out_dt, bk, inv, sa, st, vec_ok);
}

// Common validation of a reduce call.  Returns OK or an error code.  The
// output may be null only when out_optional is set.
ddp_status_t check_reduce(const void *const *ptrs, int32_t n, int64_t len, int order, int in,
                          int out_dt, const void *out, bool out_optional = false)
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
    int32_t b = 0;
    for (int64_t k = 0; k < entries; ++k) {
        const int64_t first = k * stride;
        while (plan->bucket_base[b + 1] <= first) ++b;   // skips empty buckets
        tb[k] = b;
    }
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

// Ring segments of every tile of a plan for n_ranks ranks, the word tile_segs
// reads: start ranks of the segment holding the tile's first element and of
// the next one, and where each ends inside the tile.  Segments are the
// non-empty ring chunks of every bucket in flat order (chunk c of a bucket of
// length L is [c*C, min((c+1)*C, L)) with C = ceil(L/N), started by rank
// (c+1) mod N).  The words are striped by XCD -- tile t at
// (t % 8) * stride + t / 8 -- so that each XCD's L2 fetches only lines of
// its own tiles.  Built on the host and uploaded once per device, tile size
// and rank count.
int64_t desc_stride(int64_t n_tiles) { return (n_tiles + kXcds - 1) / kXcds; }

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
    struct Seg {
        int64_t lo, hi;
        uint32_t start;
    };
    const int64_t total = plan->total, n_tiles = (total + tile - 1) / tile;
    std::vector<Seg> segs;
    std::vector<uint32_t> w;
    try {
        for (int32_t b = 0; b < plan->n_buckets(); ++b) {
            const int64_t base = plan->bucket_base[b], end = plan->bucket_base[b + 1];
            const int64_t C = (end - base + n_ranks - 1) / n_ranks;
            for (int c = 0; c < n_ranks && base + c * C < end; ++c)
                segs.push_back({base + c * C, std::min(base + (c + 1) * C, end),
                                (uint32_t)((c + 1) % n_ranks)});
        }
        w.assign((size_t)std::max<int64_t>(kXcds * desc_stride(n_tiles), 1), 0u);
    } catch (...) {
        return DDP_ERR_NOMEM;
    }
    // the segments cover [0, total) in order, so one forward pass finds them
    size_t j = 0;
    for (int64_t t = 0; t < n_tiles; ++t) {
        const int64_t t0 = t * tile, t1 = std::min(t0 + tile, total);
        while (segs[j].hi <= t0) ++j;
        const uint32_t cut_a = (uint32_t)(std::min(segs[j].hi, t1) - t0);
        uint32_t cut_b = cut_a, sb = 0;
        if (segs[j].hi < t1) {
            cut_b = (uint32_t)(std::min(segs[j + 1].hi, t1) - t0);
            sb = segs[j + 1].start;
        }
        w[(size_t)((t % kXcds) * desc_stride(n_tiles) + t / kXcds)] =
            segs[j].start | sb << 6 | cut_a << 12 | cut_b << 22;
    }
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
    *bk = {t->bucket_base, t->tile_bucket, desc, desc_stride(t->n_tiles), 0, plan->total,
           plan->n_buckets()};
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
    bool vec_ok = aligned(out, 16);
    for (int r = 0; r < n_ranks; ++r) {
        ra.p[r] = rank_ptrs[r];
        vec_ok = vec_ok && aligned(rank_ptrs[r], 16);
    }
    return launch_one_bucket(ra, n_ranks, len, order, in_dtype, out_dtype, out, st);
}

ddp_status_t ddp_plan_prepare(ddp_plan_t *plan)
{
    if (!plan) return DDP_ERR_INVALID_ARG;
    const ddp_dev_tables *t = nullptr;
    return plan_tables(plan, tile_elems(plan->dtype), &t);
}

ddp_status_t ddp_set_occupancy(ddp_occupancy_t policy)
{
    if (policy != DDP_OCCUPANCY_TUNED && policy != DDP_OCCUPANCY_SHARED) return DDP_ERR_INVALID_ARG;
    g_occupancy.store(policy, std::memory_order_relaxed);
    return DDP_OK;
}

ddp_occupancy_t ddp_get_occupancy(void)
{
    return static_cast<ddp_occupancy_t>(g_occupancy.load(std::memory_order_relaxed));
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
    if (n_ranks == 1) return copy_single(rank_flat[0], total, dtype_size(in), out_flat, st);

    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    bool vec_ok = aligned(out_flat, 16);
    for (int r = 0; r < n_ranks; ++r) {
        ra.p[r] = rank_flat[r];
        vec_ok = vec_ok && aligned(rank_flat[r], 16);
    }
    if (!vec_ok) {
        // element-aligned buffers: one per-element launch per bucket
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
    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    bool vec_ok = aligned(param_flat, 16) &&
                  (!momentum_flat || aligned(momentum_flat, 16)) && (!grad_out || aligned(grad_out, 16));
    for (int r = 0; r < n_ranks; ++r) {
        ra.p[r] = rank_flat[r];
        vec_ok = vec_ok && aligned(rank_flat[r], 16);
    }
    if (!vec_ok) {
        // element-aligned buffers: one per-element launch per bucket
        for (int32_t b = 0; b < plan->n_buckets(); ++b) {
            const int64_t base = plan->bucket_base[b], len = plan->bucket_base[b + 1] - base;
            if (len == 0) continue;
            RankArgs sub;
            std::memset(&sub, 0, sizeof(sub));
            for (int r = 0; r < n_ranks; ++r)
                sub.p[r] = static_cast<const char *>(rank_flat[r]) + base * isz;
            SgdArgs sa = {param_flat + base, momentum_flat ? momentum_flat + base : nullptr,
                          grad_out ? static_cast<char *>(grad_out) + base * osz : nullptr, lr,
                          momentum};
            ddp_status_t s2 = launch_sgd(sub, n_ranks, len, order, in, out_dtype,
                                         single_bucket(0, len), sa, st, false);
            if (s2 != DDP_OK) return s2;
        }
        return DDP_OK;
    }
    const SgdArgs sa = {param_flat, momentum_flat, grad_out, lr, momentum};
    if (order == DDP_ORDER_SEQUENTIAL || n_ranks == 1) {
        // neither depends on bucket boundaries (one rank: the input itself)
        return launch_sgd(ra, n_ranks, total, order, in, out_dtype, single_bucket(0, total), sa, st,
                          true);
    }
    Buckets bk;
    if ((stc = ring_buckets(plan, in, n_ranks, &bk)) != DDP_OK) return stc;
    return launch_sgd(ra, n_ranks, total, order, in, out_dtype, bk, sa, st, true);
}

ddp_status_t ddp_accumulate(void *const *dst, const void *const *src, int32_t n_bufs, int64_t len,
                            ddp_dtype_t dtype, void *stream)
{
    if (n_bufs < 1 || len < 0 || !dtype_ok(dtype)) return DDP_ERR_INVALID_ARG;
    if (n_bufs > DDP_MAX_RANKS) return DDP_ERR_UNSUPPORTED;
    if (len > INT64_MAX / 4) return DDP_ERR_OVERFLOW;
    if (len == 0) return DDP_OK;
    if (!dst || !src) return DDP_ERR_INVALID_ARG;
    const int esz = dtype_size(dtype);
    const int64_t nbytes = len * esz;
    AccArgs a;
    std::memset(&a, 0, sizeof(a));
    bool vec_ok = true;
    for (int k = 0; k < n_bufs; ++k) {
        if (!dst[k] || !src[k] || !aligned(dst[k], esz) || !aligned(src[k], esz))
            return DDP_ERR_INVALID_ARG;
        const uintptr_t dk = reinterpret_cast<uintptr_t>(dst[k]);
        for (int j = 0; j < n_bufs; ++j) {
            const uintptr_t sj = reinterpret_cast<uintptr_t>(src[j]);
            // a destination may be exactly its own source; it may overlap nothing else
            if (!(j == k && sj == dk) && overlaps(dk, nbytes, sj, nbytes)) return DDP_ERR_ALIAS;
            if (j != k && overlaps(dk, nbytes, reinterpret_cast<uintptr_t>(dst[j]), nbytes))
                return DDP_ERR_ALIAS;
        }
        a.dst[k] = static_cast<char *>(dst[k]);
        a.src[k] = static_cast<const char *>(src[k]);
        vec_ok = vec_ok && aligned(dst[k], 16) && aligned(src[k], 16);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t per = vec_ok ? (int64_t)kThreads * vec_elems(dtype) : kThreads;
    const int64_t blocks = (len + per - 1) / per;
    if (blocks > INT_MAX) return DDP_ERR_OVERFLOW;
    const dim3 g((unsigned)blocks, (unsigned)n_bufs), b(kThreads);
    if (dtype == DDP_F32) {
        if (vec_ok) accumulate_vec<kF32><<<g, b, 0, st>>>(a, len);
        else accumulate_scalar<kF32><<<g, b, 0, st>>>(a, len);
    } else {
        if (vec_ok) accumulate_vec<kBF16><<<g, b, 0, st>>>(a, len);
        else accumulate_scalar<kBF16><<<g, b, 0, st>>>(a, len);
    }
    return launched("accumulate kernel launch");
}

ddp_status_t ddp_bind_params(const ddp_plan_t *plan, void *const *param_grads, void *stream,
                             ddp_binding_t **out)
{
    (void)stream;
    if (!plan || !param_grads || !out) return DDP_ERR_INVALID_ARG;
    for (int32_t p = 0; p < plan->n_params; ++p) {
        if (plan->numel[p] > 0 && !param_grads[p]) return DDP_ERR_INVALID_ARG;
        if (!aligned(param_grads[p], 2)) return DDP_ERR_INVALID_ARG;
    }
    ddp_binding *bd = new (std::nothrow) ddp_binding();
    if (!bd) return DDP_ERR_NOMEM;
    bd->plan = plan;
    hipError_t e = hipGetDevice(&bd->device);
    if (e != hipSuccess) {
        delete bd;
        return hip_fail("hipGetDevice", e);
    }
    std::vector<ddp_copy_unit> units;
    try {
        const int32_t nb = plan->n_buckets();
        bd->bucket_first_unit.resize((size_t)nb + 1);
        for (int32_t b = 0; b < nb; ++b) {
            bd->bucket_first_unit[b] = (int64_t)units.size();
            int64_t flat = plan->bucket_base[b];
            for (int32_t s = plan->bucket_first_slot[b]; s < plan->bucket_first_slot[b + 1]; ++s) {
                const int32_t p = plan->slot_param[s];
                const int64_t n = plan->numel[p];
                for (int64_t off = 0; off < n; off += kCopyUnitElems) {
                    ddp_copy_unit u;
                    u.param_addr = reinterpret_cast<uint64_t>(param_grads[p]);
                    u.param_elem = off;
                    u.flat_elem = flat + off;
                    u.count = std::min<int64_t>(kCopyUnitElems, n - off);
                    units.push_back(u);
                }
                flat += n;
            }
        }
        bd->bucket_first_unit[nb] = (int64_t)units.size();
    } catch (...) {
        delete bd;
        return DDP_ERR_NOMEM;
    }
    bd->n_units = (int64_t)units.size();
    if (bd->n_units > 0) {
        const size_t bytes = sizeof(ddp_copy_unit) * units.size();
        if ((e = hipMalloc(&bd->units, bytes)) != hipSuccess) {
            delete bd;
            return hip_fail("hipMalloc (copy units)", e, DDP_ERR_NOMEM);
        }
        if ((e = hipMemcpy(bd->units, units.data(), bytes, hipMemcpyHostToDevice)) != hipSuccess) {
            (void)hipFree(bd->units);
            delete bd;
            return hip_fail("hipMemcpy (copy units)", e);
        }
    }
    *out = bd;
    return DDP_OK;
}

void ddp_binding_free(ddp_binding_t *binding)
{
    if (!binding) return;
    if (binding->units) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(binding->device);
        (void)hipFree(binding->units);
        if (cur >= 0) (void)hipSetDevice(cur);
    }
    delete binding;
}

static ddp_status_t run_copy(const ddp_plan_t *plan, const ddp_binding_t *bd, int32_t bucket,
                             void *flat, int dtype, void *stream, int to_flat)
{
    if (!plan || !bd || !flat || bd->plan != plan || !dtype_ok(dtype)) return DDP_ERR_INVALID_ARG;
    if (bucket < -1 || bucket >= plan->n_buckets()) return DDP_ERR_INVALID_ARG;
    if (!aligned(flat, dtype_size(dtype))) return DDP_ERR_INVALID_ARG;
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != bd->device) return DDP_ERR_INVALID_ARG;
    const int64_t first = bucket < 0 ? 0 : bd->bucket_first_unit[bucket];
    const int64_t last = bucket < 0 ? bd->n_units : bd->bucket_first_unit[bucket + 1];
    if (last <= first) return DDP_OK;
    // every XCD gets the same number of units (the last round padded)
    const int64_t blocks = (last - first + kXcds - 1) / kXcds * kXcds * kCopyBlocksPerUnit;
    if (blocks > INT_MAX) return DDP_ERR_OVERFLOW;
    copy_units<<<dim3((unsigned)blocks), dim3(kCopyThreads), lds_for_blocks(kCopyBlocksPerCU),
                 static_cast<hipStream_t>(stream)>>>(bd->units, first, last - first,
                                                      static_cast<char *>(flat), dtype_size(dtype),
                                                      to_flat);
    return launched("copy kernel launch");
}

ddp_status_t ddp_flatten(const ddp_plan_t *plan, const ddp_binding_t *binding, int32_t bucket,
                         void *flat_buf, ddp_dtype_t dtype, void *stream)
{
    return run_copy(plan, binding, bucket, flat_buf, dtype, stream, 1);
}

ddp_status_t ddp_unflatten(const ddp_plan_t *plan, const ddp_binding_t *binding, int32_t bucket,
                           const void *flat_out, ddp_dtype_t dtype, void *stream)
{
    return run_copy(plan, binding, bucket, const_cast<void *>(flat_out), dtype, stream, 0);
}

const char *ddp_last_error(void) { return g_last_error; }

}  // extern "C"
