// Device-side building blocks of libddp's kernels for gfx950 (MI355X):
// launch shape constants, the argument structs, streaming loads and stores,
// bf16 conversion, the ring-segment lookup, the fixed-order folds and the
// store epilogues.  Shared by reduce.hip, params.hip, accumulate.hip and
// copy.hip; not part of the ABI.
//
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
// order.  Every other vector -- one straddling a chunk or bucket boundary,
// or one lying past the second segment (a tile meeting three or more
// chunks, which needs a chunk shorter than a tile: a bucket of fewer than
// about N tiles) -- takes the
// per-element path (reduce_elems): each of its elements finds its own bucket
// and start rank (ring_start) and is folded on its own.  Either way each
// element gets the same additions in the same order, so the result is the
// same bits whichever path a vector takes.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ddp.h"

namespace ddp_detail {

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
constexpr int64_t kCopyBlockBytes = 8192;   // bytes per copy block: an f32 unit gets two
                                            // blocks, a bf16 unit one
__host__ __device__ constexpr int copy_blocks_per_unit(int esize)
{
    return (int)(kCopyUnitElems * esize / kCopyBlockBytes);
}
static_assert(copy_blocks_per_unit(2) == 1 && copy_blocks_per_unit(4) == 2,
              "a copy unit splits into whole blocks");

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
    int64_t first_block;          // grid-wide index of this launch's block 0: a grid
                                  // too large for one dispatch runs as several launches
};

// One bucket spanning [lo, hi) of a launch's elements.
__host__ __device__ inline Buckets single_bucket(int64_t lo, int64_t hi)
{
    return {nullptr, nullptr, nullptr, 0, lo, hi, 1, 0};
}

// Workgroups are dealt to the XCDs round-robin, so tile t runs on XCD t % 8.
constexpr int kXcds = 8;

// Tables of a plan's RING synchronisation, computed by the same code on the
// host (the tables a plan uploads once) and on the device (the tables
// ddp_sync_allreduce_avg_noalloc rebuilds in its static buffer).
//
// The bucket holding flat element i, 0 <= i < base[nb]: the smallest b with
// base[b + 1] > i, so empty buckets (base[b] == base[b + 1]) are skipped.
__host__ __device__ inline int32_t bucket_holding(const int64_t *base, int32_t nb, int64_t i)
{
    int32_t lo = 0, hi = nb - 1;
    while (lo < hi) {
        const int32_t mid = lo + (hi - lo) / 2;
        if (base[mid + 1] > i)
            hi = mid;
        else
            lo = mid + 1;
    }
    return lo;
}

__host__ __device__ inline int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

// Ring-segment word of tile t (tiles of `tile` elements over a flat layout of
// nb buckets, n_ranks >= 2), as tile_segs decodes it.  Segments are the
// non-empty ring chunks of every bucket in flat order: chunk c of a bucket
// of length L is [c*C, min((c+1)*C, L)) with C = ceil(L/N), started by rank
// (c+1) mod N.  Segment a holds the tile's first element; segment b is the
// next one when a ends inside the tile (the next chunk of the bucket, or
// chunk 0 of the next non-empty bucket).  Ends are relative to the tile.
__host__ __device__ inline uint32_t ring_tile_word(const int64_t *base, int32_t nb, int64_t tile,
                                                   int n_ranks, int64_t t)
{
    const int64_t total = base[nb];
    const int64_t t0 = t * tile, t1 = min64(t0 + tile, total);
    const int32_t b = bucket_holding(base, nb, t0);
    const int64_t bb = base[b], be = base[b + 1];
    const int64_t C = (be - bb + n_ranks - 1) / n_ranks;
    const int64_t c = (t0 - bb) / C;
    const int64_t a_hi = min64(bb + (c + 1) * C, be);
    const uint32_t sa = (uint32_t)((c + 1) % n_ranks);
    const uint32_t cut_a = (uint32_t)(min64(a_hi, t1) - t0);
    uint32_t sb = 0, cut_b = cut_a;
    if (a_hi < t1) {
        int64_t b_hi;
        if (a_hi < be) {   // the bucket's next chunk
            b_hi = min64(a_hi + C, be);
            sb = (uint32_t)((c + 2) % n_ranks);
        } else {           // chunk 0 of the next non-empty bucket
            const int32_t b2 = bucket_holding(base, nb, a_hi);
            const int64_t C2 = (base[b2 + 1] - base[b2] + n_ranks - 1) / n_ranks;
            b_hi = min64(base[b2] + C2, base[b2 + 1]);
            sb = (uint32_t)(1 % n_ranks);
        }
        cut_b = (uint32_t)(min64(b_hi, t1) - t0);
    }
    return sa | sb << 6 | cut_a << 12 | cut_b << 22;
}

// Tiles per XCD stripe of the word table: tile t's word sits at
// (t % kXcds) * stride + t / kXcds.
__host__ __device__ inline int64_t word_stride(int64_t n_tiles) { return (n_tiles + kXcds - 1) / kXcds; }

// The chunk segments a tile may meet on the vector path.
struct Segs {
    int64_t a_lo, a_hi, b_lo, b_hi;
    int sa, sb;
};

// Streaming 16-byte accesses of the reduce.  Every byte is touched once, so
// they are non-temporal (the `nt` cache policy): on gfx950 this lifts a pure
// streaming read from ~6.5 to ~7.2 TB/s and the reduce by ~15 %.  Loads and
// stores need only element alignment (2 bytes): gfx9 and later global
// accesses take any address, and the under-aligned types tell the compiler
// so (the instructions are the same global_load_dwordx4 and
// global_store_dwordx{2,4}).  Rank buffers of a bucket therefore need not
// share their offset from a 16-byte boundary, nor written buffers sit on one.
typedef u32x4 u32x4_ua __attribute__((aligned(2)));
template <typename V> struct under_aligned;
template <> struct under_aligned<u32x4> { typedef u32x4 type __attribute__((aligned(2))); };
template <> struct under_aligned<u32x2> { typedef u32x2 type __attribute__((aligned(2))); };

__device__ __forceinline__ u32x4 ld_stream(const char *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_ua *>(p));
}

// An 8-byte streaming load (four bf16 gradients of the fused step's split
// lane layout, sgd_vec_split).
__device__ __forceinline__ u32x2 ld_stream8(const char *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const typename under_aligned<u32x2>::type *>(p));
}

template <typename V>
__device__ __forceinline__ void st_stream(void *p, const V &v)
{
    typedef typename under_aligned<V>::type VU;
    __builtin_nontemporal_store(static_cast<VU>(v), reinterpret_cast<VU *>(p));
}

// The same accesses at a base that is either a pointer (a kernel argument,
// which the compiler knows to be global memory) or a 64-bit address read
// from a table, typed as global memory here so that the access is a global
// rather than a flat instruction.  Loads take a byte offset.
typedef __attribute__((address_space(1))) u32x4 g_u32x4;
typedef __attribute__((address_space(1))) u32x4_ua g_u32x4_ua;

__device__ __forceinline__ u32x4 ld_at(const void *p, int64_t off)
{
    return ld_stream(static_cast<const char *>(p) + off);
}
__device__ __forceinline__ u32x4 ld_at(uint64_t a, int64_t off)
{
    return __builtin_nontemporal_load(reinterpret_cast<const g_u32x4_ua *>(a + (uint64_t)off));
}
// Two 8-byte loads at byte offsets offA and offB, as one vector (the fused
// step's split lane layout for bf16 gradients).
__device__ __forceinline__ u32x4 ld_split(const void *p, int64_t offA, int64_t offB)
{
    const char *c = static_cast<const char *>(p);
    const u32x2 lo = ld_stream8(c + offA), hi = ld_stream8(c + offB);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}
__device__ __forceinline__ u32x4 ld_split(uint64_t a, int64_t offA, int64_t offB)
{
    typedef __attribute__((address_space(1))) typename under_aligned<u32x2>::type g_u32x2_ua;
    const u32x2 lo = __builtin_nontemporal_load(reinterpret_cast<const g_u32x2_ua *>(a + (uint64_t)offA));
    const u32x2 hi = __builtin_nontemporal_load(reinterpret_cast<const g_u32x2_ua *>(a + (uint64_t)offB));
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Stores take the element index i of a T array at the base.
template <typename T, typename V>
__device__ __forceinline__ void st_at(void *p, int64_t i, const V &v)
{
    st_stream(static_cast<T *>(p) + i, v);
}
template <typename T, typename V>
__device__ __forceinline__ void st_at(uint64_t a, int64_t i, const V &v)
{
    typedef __attribute__((address_space(1))) typename under_aligned<V>::type GV;
    __builtin_nontemporal_store(static_cast<typename under_aligned<V>::type>(v),
                                reinterpret_cast<GV *>(a + (uint64_t)i * sizeof(T)));
}

// Plain (cached) accesses of element i of a T array at either kind of base,
// for the per-element paths.
template <typename T>
__device__ __forceinline__ T ld_elem(const void *p, int64_t i)
{
    return static_cast<const T *>(p)[i];
}
template <typename T>
__device__ __forceinline__ T ld_elem(uint64_t a, int64_t i)
{
    typedef __attribute__((address_space(1))) T GT;
    return *reinterpret_cast<const GT *>(a + (uint64_t)i * sizeof(T));
}
template <typename T>
__device__ __forceinline__ void st_elem(void *p, int64_t i, T v)
{
    static_cast<T *>(p)[i] = v;
}
template <typename T>
__device__ __forceinline__ void st_elem(uint64_t a, int64_t i, T v)
{
    typedef __attribute__((address_space(1))) T GT;
    *reinterpret_cast<GT *>(a + (uint64_t)i * sizeof(T)) = v;
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

template <int IN, class A>
__device__ __forceinline__ float load_elem(A p, int64_t i)
{
    if (IN == kF32) return ld_elem<float>(p, i);
    return widen_bf16(ld_elem<uint16_t>(p, i));
}

template <int OUT, class A>
__device__ __forceinline__ void store_elem(A out, int64_t i, float y)
{
    if (OUT == kF32)
        st_elem<float>(out, i, y);
    else
        st_elem<uint16_t>(out, i, (uint16_t)bf16_rne(y));
}

__device__ __forceinline__ int wrap(int r, int n) { return r >= n ? r - n : r; }

// Ring start rank of element i (any bucket at or after b0).
__device__ __forceinline__ int ring_start(const Buckets &bk, int32_t b0, int N, int64_t i)
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

// The scaled average of element i of the ranks at bases p[0..N-1] (N >= 2),
// folded from rank r (RING: the element's ring start; SEQ: 0, after +0).
template <int IN, bool RING, class A>
__device__ __forceinline__ float avg_at(const A *p, int N, int r, float inv, int64_t i)
{
    float acc = load_elem<IN>(p[r], i);
    if (!RING) acc = 0.0f + acc;
    for (int k = 1; k < N; ++k) {
        r = wrap(r + 1, N);
        acc = acc + load_elem<IN>(p[r], i);
    }
    return acc * inv;
}

template <int IN, bool RING>
__device__ __forceinline__ float avg_elem(const RankArgs &ra, int N, int64_t total,
                                          const Buckets &bk, int32_t b0, float inv, int64_t i)
{
    return avg_at<IN, RING>(ra.p, N, RING ? ring_start(bk, b0, N, i) : 0, inv, i);
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

// Per-element epilogue of the fused step at element i: the average y stored
// to gout unless gout is null (bf16: rounded, and the step takes the rounded
// value), then the parameter (and momentum) updated.  Bases are pointers or
// table addresses.
template <int OUT, bool MOM, class A>
__device__ __forceinline__ void sgd_at(A gout, A param, A mom, int64_t i, float y, float lr,
                                       float mu)
{
    float g = y;
    if (OUT == kBF16) {
        const uint32_t h = bf16_rne(y);
        g = widen_bf16(h);
        if (gout != A()) st_elem<uint16_t>(gout, i, (uint16_t)h);
    } else if (gout != A()) {
        st_elem<float>(gout, i, y);
    }
    float m = MOM ? ld_elem<float>(mom, i) : 0.0f;
    st_elem<float>(param, i, sgd_elem<MOM>(ld_elem<float>(param, i), g, m, lr, mu));
    if (MOM) st_elem<float>(mom, i, m);
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
        sgd_at<OUT, MOM>(sa.grad_out, static_cast<void *>(sa.param), static_cast<void *>(sa.mom), i,
                         y, sa.lr, sa.mu);
    }
}

// Tile (vector kernels) or group of kThreads elements (per-element kernels)
// processed by this block.
__device__ __forceinline__ int64_t tile_of_block(const Buckets &bk)
{
    return bk.first_block + blockIdx.x;
}

// A single bucket that starts before the launch's element 0 (lo < 0: its
// first -lo elements sit just before the aligned address the vector path
// starts at) gets one extra block at the end of the grid.  Its tile, the
// only one that starts at or past the end (tile0 >= total), gives the vector
// path no work (its loads read the dummy vector), and this reduces the head
// elements one per lane.  The check comes after the vector path, so no other
// block waits on it before its loads.
template <int IN, int OUT, bool RING>
__device__ __forceinline__ void head_block(const RankArgs &ra, int N, int64_t total,
                                           const Buckets &bk, float inv, void *out,
                                           int64_t tile0)
{
    if (bk.base || bk.lo >= 0 || tile0 < total) return;
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
// the wave-uniform rank s, eight loads in flight at a time.  p[r] is rank r's
// base address (a pointer or a 64-bit address), read with a scalar load, and
// a short last group is cut by a uniform branch rather than dummy loads.
// Lanes not taking part pass off = 0 and re-read vector 0.
template <int IN, bool RING, class Ptrs>
__device__ __forceinline__ void fold_looped(const Ptrs &p, int N, int s, int64_t off, float *acc)
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
                v[j] = ld_at(p[r], off);
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

// fold_looped for bf16 gradients in the split lane layout: each rank's
// vector is four elements at byte offset offA and four at offB.
template <bool RING, class Ptrs>
__device__ __forceinline__ void fold_looped_split(const Ptrs &p, int N, int s, int64_t offA,
                                                  int64_t offB, float *acc)
{
    constexpr int G = 8;
#pragma unroll 1
    for (int k0 = 0; k0 < N; k0 += G) {
        u32x4 v[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (k0 + j < N) {
                int r = s + k0 + j;
                r = r >= N ? r - N : r;
                v[j] = ld_split(p[r], offA, offB);
            }
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (k0 + j < N) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = lane<kBF16>(v[j], e);
                    acc[e] = k0 + j > 0 ? acc[e] + x : (RING ? x : 0.0f + x);
                }
            }
        }
    }
}

// Convert and store one vector of scaled averages y at element i0 of the
// tensor at `out` (a pointer or a table address; nothing is written unless
// `write`); for a bf16 output y becomes the stored value widened back to f32
// either way.
template <int IN, int OUT, class A>
__device__ __forceinline__ void store_y(A out, int64_t i0, float *y, bool write)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    if (OUT == kF32) {
        u32x4 o;
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(y[e]);
        if (write) st_at<float>(out, i0, o);
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
            if (write) st_at<uint16_t>(out, i0, o);
        } else {
            u32x4 o;
            for (int w = 0; w < 4; ++w) o[w] = h[2 * w] | (h[2 * w + 1] << 16);
            if (write) st_at<uint16_t>(out, i0, o);
        }
    }
}

// Scale, convert and store one vector of accumulators at element i0.
template <int IN, int OUT, class A>
__device__ __forceinline__ void store_vec(A out, int64_t i0, const float *acc, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    float y[VEC];
    for (int e = 0; e < VEC; ++e) y[e] = acc[e] * inv;
    store_y<IN, OUT>(out, i0, y, true);
}

// The vector epilogue of the fused step: store the average y to gout unless
// gout is null (bf16: y becomes the stored value widened back), then update
// the lane's parameter vectors pv (and momentum mv), already loaded, and
// store them to param (and mom).  The three bases are pointers or table
// addresses.
template <int IN, int OUT, bool MOM, class A>
__device__ __forceinline__ void sgd_vec(A gout, A param, A mom, int64_t i0, float *y,
                                        const u32x4 *pv, const u32x4 *mv, float lr, float mu)
{
    constexpr int PV = (IN == kF32 ? 4 : 8) / 4;
    store_y<IN, OUT>(gout, i0, y, gout != A());
#pragma unroll
    for (int j = 0; j < PV; ++j) {
        u32x4 po, mo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float m = MOM ? __uint_as_float(mv[j][w]) : 0.0f;
            po[w] = __float_as_uint(sgd_elem<MOM>(__uint_as_float(pv[j][w]), y[4 * j + w], m, lr, mu));
            mo[w] = __float_as_uint(m);
        }
        st_at<float>(param, i0 + 4 * j, po);
        if (MOM) st_at<float>(mom, i0 + 4 * j, mo);
    }
}

// The same on the flat buffers of SgdArgs.
template <int IN, int OUT, bool MOM>
__device__ __forceinline__ void sgd_vec(const SgdArgs &sa, int64_t i0, float *y, const u32x4 *pv,
                                        const u32x4 *mv)
{
    sgd_vec<IN, OUT, MOM>(sa.grad_out, static_cast<void *>(sa.param),
                          static_cast<void *>(sa.mom), i0, y, pv, mv, sa.lr, sa.mu);
}

// The fused step's epilogue for bf16 gradients in the split lane layout: the
// lane's eight elements are [iA, iA + 4) and [iB, iB + 4), y[0..3] and
// y[4..7], with parameter (and momentum) vectors pv[0], pv[1] (mv) loaded
// from those two places.  With eight consecutive elements per lane a lane's
// two 16-byte parameter stores sit 32 bytes apart and each store instruction
// covers every other 16 bytes of its wave's range, so memory received a
// quarter of the 64-byte pieces in two halves; here every store instruction
// of a wave writes one contiguous range.  The average is rounded to bf16 and
// the step takes the rounded value, as store_y does.
template <bool MOM, class A>
__device__ __forceinline__ void sgd_vec_split(A gout, A param, A mom, int64_t iA, int64_t iB, float *y,
                                              const u32x4 *pv, const u32x4 *mv, float lr, float mu)
{
    uint32_t h[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = bf16_rne(y[e]);
        y[e] = widen_bf16(h[e]);
    }
    if (gout != A()) {
        st_at<uint16_t>(gout, iA, u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)});
        st_at<uint16_t>(gout, iB, u32x2{h[4] | (h[5] << 16), h[6] | (h[7] << 16)});
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        u32x4 po, mo;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            float m = MOM ? __uint_as_float(mv[j][w]) : 0.0f;
            po[w] = __float_as_uint(sgd_elem<MOM>(__uint_as_float(pv[j][w]), y[4 * j + w], m, lr, mu));
            mo[w] = __float_as_uint(m);
        }
        st_at<float>(param, j ? iB : iA, po);
        if (MOM) st_at<float>(mom, j ? iB : iA, mo);
    }
}

}  // namespace ddp_detail
