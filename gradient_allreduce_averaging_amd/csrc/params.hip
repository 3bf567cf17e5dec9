// The synchronisation over per-parameter tensors in one kernel.
//
// ddp_param_sync_*: every rank's gradients are read where they lie, with no
// flatten, folded in the fixed order their flat positions define, scaled,
// and written to per-parameter outputs, with no unflatten.  The result is
// that of flatten, then ddp_sync_allreduce_avg, then unflatten, bit for bit;
// the bytes moved are those of the sync alone (N reads and one write per
// element), where the three steps move 2N + N + 1 + 2 element-widths.
//
// ddp_param_sgd_*: the same average folded into a (momentum) SGD step on
// per-parameter f32 parameters, the per-parameter form of
// ddp_sync_sgd_update.
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel) 4.2 (the
//        gradients are copied into a flat bucket, averaged, and viewed back;
//        gradient_as_bucket_view drops a copy), 5.3 (the update rule);
//        [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn) 八
//        (gradients laid out by region so that no copy is needed), 九 (the
//        scale could be absorbed into the optimizer update).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <type_traits>
#include <vector>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

// Vectors per lane: a tile is kThreads * kPsUnroll vectors.  Two (half as
// many entries and blocks) measured 3-5 % slower than one at every cap.
constexpr int kPsUnroll = 1;

inline int64_t ps_tile_elems(int in) { return (int64_t)kThreads * kPsUnroll * vec_elems(in); }

// A parameter is cut into tiles of ps_tile_elems elements from its own start
// (the last one shorter), so every address inside a tile has the alignment
// of the parameter's address.  The table has two parts:
//
//   tile records, 8 bytes each, striped by XCD (tile t at
//   (t % kXcds) * rstride + t / kXcds, so that each XCD's L2 fetches lines
//   of its own tiles only): the tile's parameter entry and its ring word;
//
//   parameter entries, `pstride` bytes each (16-byte aligned), one per
//   parameter with elements, in flat order:
//     uint64_t addr[N + X]   ranks 0..N-1, then the X tensors written, at the
//                            parameter's first element:
//                              sync: the output (X = 1)
//                              SGD:  the averaged gradient (0 if not stored),
//                                    the parameters, the momentum (0 if none)
//                                    (X = 3)
//     PsParamMeta            below
//
// A tile's addresses are its parameter's plus the tile's first element j0 =
// (tile - first_tile) * ps_tile_elems, so the table costs 8 bytes per tile
// (0.09 % of the 9 KiB an f32 tile of 8 ranks moves) and a few dozen bytes
// per parameter.
struct PsTile {
    uint32_t param;   // parameter entry index
    uint32_t ring;    // the ring chunks the tile meets: start rank of chunk a
                      // (bits 0-5) and of chunk b (bits 6-11), where a (bits
                      // 12-21) and b (bits 22-31) end, relative to the tile's
                      // first element
};

struct PsParamMeta {
    int64_t pos0;         // position of the parameter's first element in its bucket
    int64_t blen;         // length of that bucket
    int64_t first_tile;   // the parameter's first tile
    int64_t numel;        // its elements
    uint32_t vec;         // 1: every written tensor of the parameter 2-byte aligned
    uint32_t pad;
};

// One tile's view of its entry, in registers.
struct PsMeta {
    int64_t pos;      // position of the tile's first element inside its bucket
    int64_t blen;     // length of that bucket
    int64_t j0;       // the tile's first element inside its parameter
    uint32_t count;   // elements in the tile, 1..tile
    uint32_t vec;
    uint32_t ring;
};

constexpr int kSyncExtra = 1, kSgdExtra = 3;

int64_t ps_pstride(int N, int extra)
{
    return (8 * (int64_t)(N + extra) + (int64_t)sizeof(PsParamMeta) + 15) / 16 * 16;
}

// Where tile t's record sits: XCD-striped.
__host__ __device__ inline int64_t ps_record(int64_t t, int64_t rstride)
{
    const uint64_t u = (uint64_t)t;   // t >= 0: unsigned division is a shift and a mask
    return (int64_t)((u % kXcds) * (uint64_t)rstride + u / kXcds);
}

__device__ __forceinline__ u32x4 gld_stream(uint64_t addr) { return ld_at(addr, 0); }

// The scaled average of tile element i, one element at a time (N >= 2); a
// holds the parameter's base addresses.
template <int IN, bool RING>
__device__ __forceinline__ float ps_avg_elem(const uint64_t *a, int N, const PsMeta &m, float inv,
                                             int64_t i)
{
    int r = 0;
    if (RING) {
        const int64_t C = (m.blen + N - 1) / N;
        r = (int)(((m.pos + i) / C + 1) % N);
    }
    return avg_at<IN, RING>(a, N, r, inv, m.j0 + i);
}

// Per-element path of the sync: tile elements [i0, i0 + cnt) clipped to the
// tile; a: the parameter entry's addresses (in memory).
template <int IN, int OUT, bool RING>
__device__ void params_elems(const uint64_t *a, int N, const PsMeta &m, float inv, int64_t i0,
                             int cnt)
{
    const uint64_t out = a[N];
    for (int e = 0; e < cnt; ++e) {
        const int64_t i = i0 + e;
        if (i >= (int64_t)m.count) break;
        if (N == 1) {   // the input, bit for bit (inputs and outputs share a dtype)
            if (IN == kF32)
                st_elem<uint32_t>(out, m.j0 + i, ld_elem<uint32_t>(a[0], m.j0 + i));
            else
                st_elem<uint16_t>(out, m.j0 + i, ld_elem<uint16_t>(a[0], m.j0 + i));
            continue;
        }
        store_elem<OUT>(out, m.j0 + i, ps_avg_elem<IN, RING>(a, N, m, inv, i));
    }
}

// Per-element path of the SGD step.  N == 1 takes the input as the average.
template <int IN, int OUT, bool RING, bool MOM>
__device__ void params_sgd_elems(const uint64_t *a, int N, const PsMeta &m, float inv, float lr,
                                 float mu, int64_t i0, int cnt)
{
    for (int e = 0; e < cnt; ++e) {
        const int64_t i = i0 + e;
        if (i >= (int64_t)m.count) break;
        const float y = N == 1 ? load_elem<IN>(a[0], m.j0 + i)
                               : ps_avg_elem<IN, RING>(a, N, m, inv, i);
        sgd_at<OUT, MOM>(a[N], a[N + 1], a[N + 2], m.j0 + i, y, lr, mu);
    }
}

struct PsSegs {
    int64_t a_hi, b_lo, b_hi;
    int sa, sb;
};

template <bool RING>
__device__ __forceinline__ PsSegs ps_segs(const PsMeta &m)
{
    PsSegs s;
    s.a_hi = s.b_lo = s.b_hi = m.count;
    s.sa = s.sb = 0;
    if (RING) {
        s.sa = __builtin_amdgcn_readfirstlane((int)(m.ring & 63u));
        s.sb = __builtin_amdgcn_readfirstlane((int)((m.ring >> 6) & 63u));
        s.a_hi = s.b_lo = (int64_t)((m.ring >> 12) & 1023u);
        s.b_hi = (int64_t)(m.ring >> 22);
    }
    return s;
}

// The table of one sync, as the kernels get it.
struct PsTable {
    const PsTile *tiles;   // XCD-striped records
    const char *params;    // parameter entries
    int64_t rstride;       // records per XCD stripe
    int64_t pstride;       // bytes per parameter entry
    int64_t n_tiles;
    int64_t tile_elems;
};

// The tile's entry: its record, then every address and the metadata of its
// parameter, fetched in one batch of scalar loads before any of them is used
// (a use behind a branch would otherwise wait for the flags before fetching
// its address).
template <int NA>
struct PsEntry {
    uint64_t ad[NA];
    PsMeta m;
    const char *pe;   // the parameter entry (per-element paths read addresses there)
};

template <int NA>
__device__ __forceinline__ PsEntry<NA> ps_entry(const PsTable &tb, int64_t tile)
{
    PsEntry<NA> t;
    const PsTile rec = tb.tiles[ps_record(tile, tb.rstride)];
    t.pe = tb.params + (int64_t)rec.param * tb.pstride;
    const uint64_t *a = reinterpret_cast<const uint64_t *>(t.pe);
#pragma unroll
    for (int k = 0; k < NA; ++k) t.ad[k] = a[k];
    const PsParamMeta pm = *reinterpret_cast<const PsParamMeta *>(t.pe + 8 * NA);
#pragma unroll
    for (int k = 0; k < NA; ++k) asm volatile("" : "+s"(t.ad[k]));
    t.m.j0 = (tile - pm.first_tile) * tb.tile_elems;
    t.m.pos = pm.pos0 + t.m.j0;
    t.m.blen = pm.blen;
    const int64_t left = pm.numel - t.m.j0;
    t.m.count = (uint32_t)(left < tb.tile_elems ? left : tb.tile_elems);
    t.m.vec = pm.vec;
    t.m.ring = rec.ring;
    return t;
}

// Tiles ahead of a block whose record it fetches into L2 (a multiple of 8,
// so the later block runs on the same XCD: blocks are dealt to the XCDs
// round-robin).
constexpr int64_t kPsPrefetch = 1024;

// From four ranks up, each block fetches the record of tile +
// kPsPrefetch, so that block's scalar record load finds it in L2 rather than
// HBM (parameter entries are few and stay in L2).  Every lane loads one of
// its two words (lane & 1), with no branch on the lane: a lane-dependent
// address makes it one vector load, which the wave does not wait for here (a
// uniform one would become a scalar load waited for at once).  The value is
// unused; consume() keeps it live until a point where the wave waits for its
// data loads anyway, so that the load has completed before its register is
// reused.
template <int NR>
__device__ __forceinline__ uint32_t prefetch_record(const PsTable &tb, int64_t tile)
{
    if constexpr (NR >= 4) {
        if (tile + kPsPrefetch < tb.n_tiles) {
            const PsTile *f = tb.tiles + ps_record(tile + kPsPrefetch, tb.rstride);
            return ld_elem<uint32_t>(reinterpret_cast<uint64_t>(f), threadIdx.x & 1);
        }
    }
    return 0;
}

__device__ __forceinline__ void consume(uint32_t x) { asm volatile("" ::"v"(x)); }

// Sync, N known at compile time (1..8).  After the entry, all NR *
// kPsUnroll vector loads of the lane go out before the ring chunks are
// looked at, as in the flat reduce.  A lane's vector past the tile's end
// reads the tile's first vector and drops it; a tile without the vector
// path reads 16 bytes of its parameter entry instead, and drops them (the
// loads are not behind a branch).
template <int NR, bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
params_fast(PsTable tb, int64_t first_block, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const int64_t tile = first_block + blockIdx.x;
    const uint32_t pf = prefetch_record<NR>(tb, tile);
    const PsEntry<NR + kSyncExtra> t = ps_entry<NR + kSyncExtra>(tb, tile);
    const PsMeta &m = t.m;
    const int64_t cnt = m.count;
    const bool vec = m.vec && cnt >= VEC;
    int64_t i0[kPsUnroll];
    u32x4 v[kPsUnroll][NR];
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        i0[u] = ((int64_t)u * kThreads + threadIdx.x) * VEC;
        const int64_t off = (m.j0 + (i0[u] + VEC <= cnt ? i0[u] : 0)) * ISZ;
#pragma unroll
        for (int k = 0; k < NR; ++k)
            v[u][k] = gld_stream(vec ? t.ad[k] + (uint64_t)off : reinterpret_cast<uint64_t>(t.pe));
    }
    const PsSegs sg = ps_segs<RING>(m);
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        const bool in_a = vec && i0[u] + VEC <= sg.a_hi;
        const bool in_b = RING && vec && i0[u] >= sg.b_lo && i0[u] + VEC <= sg.b_hi;
        if (in_a || in_b) {
            if constexpr (NR == 1 && IN == OUT) {
                st_at<std::conditional_t<IN == kF32, float, uint16_t>>(t.ad[1], m.j0 + i0[u],
                                                                       v[u][0]);
            } else {
                float acc[VEC];
                if (!RING)
                    fold_seq<NR, IN>(v[u], acc);
                else
                    fold_ring<NR, IN>(v[u], in_a ? sg.sa : sg.sb, acc);
                consume(pf);
                store_vec<IN, OUT>(t.ad[NR], m.j0 + i0[u], acc, inv);
            }
        } else {
            consume(pf);
            if (i0[u] < cnt)
                params_elems<IN, OUT, RING>(reinterpret_cast<const uint64_t *>(t.pe), NR, m, inv,
                                            i0[u], VEC);
        }
    }
}

// Sync, any N up to DDP_MAX_RANKS: one pass per ring chunk the wave's lanes
// meet, folded with fold_looped from the parameter entry's addresses.
template <bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
params_many(PsTable tb, int N, int64_t first_block, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const int64_t tile = first_block + blockIdx.x;
    const PsTile rec = tb.tiles[ps_record(tile, tb.rstride)];
    const char *pe = tb.params + (int64_t)rec.param * tb.pstride;
    const uint64_t *a = reinterpret_cast<const uint64_t *>(pe);
    const PsParamMeta pm = *reinterpret_cast<const PsParamMeta *>(pe + 8 * (N + kSyncExtra));
    PsMeta m;
    m.j0 = (tile - pm.first_tile) * tb.tile_elems;
    m.pos = pm.pos0 + m.j0;
    m.blen = pm.blen;
    m.count = (uint32_t)min(pm.numel - m.j0, tb.tile_elems);
    m.vec = pm.vec;
    m.ring = rec.ring;
    const int64_t cnt = m.count;
    const bool vec = m.vec && cnt >= VEC;
    const PsSegs sg = ps_segs<RING>(m);
#pragma unroll 1
    for (int u = 0; u < kPsUnroll; ++u) {
        const int64_t i0 = ((int64_t)u * kThreads + threadIdx.x) * VEC;
        const bool in_a = vec && i0 + VEC <= sg.a_hi;
        const bool in_b = RING && vec && i0 >= sg.b_lo && i0 + VEC <= sg.b_hi;
#pragma unroll 1
        for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
            const bool mine = pass == 0 ? in_a : in_b;
            if (!__builtin_amdgcn_ballot_w64(mine)) continue;   // no lane of the wave here
            float acc[VEC];
            // lanes not taking part re-read the tile's first vector
            fold_looped<IN, RING>(a, N, pass == 0 ? sg.sa : sg.sb, (m.j0 + (mine ? i0 : 0)) * ISZ,
                                  acc);
            if (mine) store_vec<IN, OUT>(a[N], m.j0 + i0, acc, inv);
        }
        if (!in_a && !in_b && i0 < cnt) params_elems<IN, OUT, RING>(a, N, m, inv, i0, VEC);
    }
}

// SGD, N known at compile time (1..8): the gradient vectors of every rank
// and the lane's parameter (and momentum) vectors are loaded together, the
// average folded and scaled, optionally stored, and the parameters updated.
// Parameters are f32: one 16-byte vector per 4 elements, so a bf16 lane (8
// elements) moves two.
// bf16 gradients: the split lane layout of the flat step (sgd_vec_split).
// Lane L takes the tile's elements [4L, 4L + 4) and [256 + 4L, 256 + 4L + 4),
// so that every parameter and momentum store of a wave writes one contiguous
// range.  A lane whose two groups are not in one ring segment of the tile,
// or reach past the parameter's end, folds them element by element.
template <int NR, bool RING, bool MOM>
__device__ __forceinline__ void params_sgd_tile_bf16(const PsTable &tb, int64_t first_block,
                                                     float inv, float lr, float mu)
{
    static_assert(kPsUnroll == 1, "one vector per lane");
    constexpr int H = kThreads * 4;   // the second group, 256 elements on
    const int64_t tile = first_block + blockIdx.x;
    const uint32_t pf = prefetch_record<NR>(tb, tile);
    const PsEntry<NR + kSgdExtra> t = ps_entry<NR + kSgdExtra>(tb, tile);
    const PsMeta &m = t.m;
    const uint64_t gout = t.ad[NR], param = t.ad[NR + 1], mom = t.ad[NR + 2];
    const uint64_t dummy = reinterpret_cast<uint64_t>(t.pe);
    const int64_t cnt = m.count;
    const int64_t iA = 4 * (int64_t)threadIdx.x, iB = iA + H;
    const bool vec = m.vec && cnt >= 8;
    // a lane past the parameter's end reads the tile's first elements (or,
    // without the vector path, the entry) and drops them
    const bool whole = iB + 4 <= cnt;
    const int64_t ja = m.j0 + (whole ? iA : 0), jb = m.j0 + (whole ? iB : 0);
    u32x4 v[NR], pv[2], mv[2];
    const int64_t oa = vec ? 2 * ja : 0, ob = vec ? 2 * jb : 0;
#pragma unroll
    for (int k = 0; k < NR; ++k) v[k] = ld_split(vec ? t.ad[k] : dummy, oa, ob);
    pv[0] = gld_stream(vec ? param + (uint64_t)(4 * ja) : dummy);
    pv[1] = gld_stream(vec ? param + (uint64_t)(4 * jb) : dummy);
    if (MOM) {
        mv[0] = gld_stream(vec ? mom + (uint64_t)(4 * ja) : dummy);
        mv[1] = gld_stream(vec ? mom + (uint64_t)(4 * jb) : dummy);
    }
    const PsSegs sg = ps_segs<RING>(m);
    const bool in_a = vec && iB + 4 <= sg.a_hi;
    const bool in_b = RING && vec && iA >= sg.b_lo && iB + 4 <= sg.b_hi;
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
        consume(pf);
        sgd_vec_split<MOM>(gout, param, mom, m.j0 + iA, m.j0 + iB, y, pv, mv, lr, mu);
    } else {
        consume(pf);
        const uint64_t *a = reinterpret_cast<const uint64_t *>(t.pe);
        if (iA < cnt) params_sgd_elems<kBF16, kBF16, RING, MOM>(a, NR, m, inv, lr, mu, iA, 4);
        if (iB < cnt) params_sgd_elems<kBF16, kBF16, RING, MOM>(a, NR, m, inv, lr, mu, iB, 4);
    }
}

template <int NR, bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
params_sgd_fast(PsTable tb, int64_t first_block, float inv, float lr, float mu)
{
    if constexpr (IN == kBF16) {
        static_assert(OUT == kBF16, "bf16 gradients average to bf16");
        params_sgd_tile_bf16<NR, RING, MOM>(tb, first_block, inv, lr, mu);
        return;
    }
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    const int64_t tile = first_block + blockIdx.x;
    const uint32_t pf = prefetch_record<NR>(tb, tile);
    const PsEntry<NR + kSgdExtra> t = ps_entry<NR + kSgdExtra>(tb, tile);
    const PsMeta &m = t.m;
    const uint64_t gout = t.ad[NR], param = t.ad[NR + 1], mom = t.ad[NR + 2];
    const uint64_t dummy = reinterpret_cast<uint64_t>(t.pe);
    const int64_t cnt = m.count;
    const bool vec = m.vec && cnt >= VEC;
    int64_t i0[kPsUnroll];
    u32x4 v[kPsUnroll][NR], pv[kPsUnroll][PV], mv[kPsUnroll][PV];
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        i0[u] = ((int64_t)u * kThreads + threadIdx.x) * VEC;
        const int64_t j = m.j0 + (i0[u] + VEC <= cnt ? i0[u] : 0);
        const int64_t go = j * ISZ, po = j * 4;
#pragma unroll
        for (int k = 0; k < NR; ++k) v[u][k] = gld_stream(vec ? t.ad[k] + (uint64_t)go : dummy);
#pragma unroll
        for (int q = 0; q < PV; ++q) {
            pv[u][q] = gld_stream(vec ? param + (uint64_t)(po + 16 * q) : dummy);
            if (MOM) mv[u][q] = gld_stream(vec ? mom + (uint64_t)(po + 16 * q) : dummy);
        }
    }
    const PsSegs sg = ps_segs<RING>(m);
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        const bool in_a = vec && i0[u] + VEC <= sg.a_hi;
        const bool in_b = RING && vec && i0[u] >= sg.b_lo && i0[u] + VEC <= sg.b_hi;
        if (in_a || in_b) {
            float y[VEC];
            if (!RING || NR == 1)
                fold_seq<NR, IN>(v[u], y);
            else
                fold_ring<NR, IN>(v[u], in_a ? sg.sa : sg.sb, y);
            if (NR > 1) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) y[k] = y[k] * inv;
            }
            consume(pf);
            sgd_vec<IN, OUT, MOM>(gout, param, mom, m.j0 + i0[u], y, pv[u], mv[u], lr, mu);
        } else {
            consume(pf);
            if (i0[u] < cnt)
                params_sgd_elems<IN, OUT, RING, MOM>(reinterpret_cast<const uint64_t *>(t.pe), NR,
                                                     m, inv, lr, mu, i0[u], VEC);
        }
    }
}

// SGD, any N up to DDP_MAX_RANKS: the lane's parameter (and momentum)
// vectors first, then the ranks folded as in params_many.
template <bool RING, int IN, int OUT, bool MOM>
__global__ void __launch_bounds__(kThreads)
params_sgd_many(PsTable tb, int N, int64_t first_block, float inv, float lr, float mu)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    constexpr int PV = VEC / 4;
    const int64_t tile = first_block + blockIdx.x;
    const PsTile rec = tb.tiles[ps_record(tile, tb.rstride)];
    const char *pe = tb.params + (int64_t)rec.param * tb.pstride;
    const uint64_t *a = reinterpret_cast<const uint64_t *>(pe);
    const PsParamMeta pm = *reinterpret_cast<const PsParamMeta *>(pe + 8 * (N + kSgdExtra));
    PsMeta m;
    m.j0 = (tile - pm.first_tile) * tb.tile_elems;
    m.pos = pm.pos0 + m.j0;
    m.blen = pm.blen;
    m.count = (uint32_t)min(pm.numel - m.j0, tb.tile_elems);
    m.vec = pm.vec;
    m.ring = rec.ring;
    const uint64_t gout = a[N], param = a[N + 1], mom = a[N + 2];
    const int64_t cnt = m.count;
    const bool vec = m.vec && cnt >= VEC;
    const PsSegs sg = ps_segs<RING>(m);
    if constexpr (IN == kBF16) {
        // the split lane layout of params_sgd_tile_bf16
        static_assert(OUT == kBF16 && kPsUnroll == 1, "bf16 gradients average to bf16");
        constexpr int H = kThreads * 4;
        const int64_t iA = 4 * (int64_t)threadIdx.x, iB = iA + H;
        const bool in_a = vec && iB + 4 <= sg.a_hi;
        const bool in_b = RING && vec && iA >= sg.b_lo && iB + 4 <= sg.b_hi;
        u32x4 pv[2], mv[2];
        if (vec) {   // a lane past the end reads the tile's first elements and drops them
            const bool whole = iB + 4 <= cnt;
            const int64_t ja = m.j0 + (whole ? iA : 0), jb = m.j0 + (whole ? iB : 0);
            pv[0] = gld_stream(param + (uint64_t)(4 * ja));
            pv[1] = gld_stream(param + (uint64_t)(4 * jb));
            if (MOM) {
                mv[0] = gld_stream(mom + (uint64_t)(4 * ja));
                mv[1] = gld_stream(mom + (uint64_t)(4 * jb));
            }
        }
#pragma unroll 1
        for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
            const bool mine = pass == 0 ? in_a : in_b;
            if (!__builtin_amdgcn_ballot_w64(mine)) continue;
            float y[8];
            fold_looped_split<RING>(a, N, pass == 0 ? sg.sa : sg.sb, 2 * (m.j0 + (mine ? iA : 0)),
                                    2 * (m.j0 + (mine ? iB : 0)), y);
            if (mine) {
#pragma unroll
                for (int k = 0; k < 8; ++k) y[k] = y[k] * inv;
                sgd_vec_split<MOM>(gout, param, mom, m.j0 + iA, m.j0 + iB, y, pv, mv, lr, mu);
            }
        }
        if (!in_a && !in_b) {
            if (iA < cnt) params_sgd_elems<kBF16, kBF16, RING, MOM>(a, N, m, inv, lr, mu, iA, 4);
            if (iB < cnt) params_sgd_elems<kBF16, kBF16, RING, MOM>(a, N, m, inv, lr, mu, iB, 4);
        }
        return;
    }
#pragma unroll 1
    for (int u = 0; u < kPsUnroll; ++u) {
        const int64_t i0 = ((int64_t)u * kThreads + threadIdx.x) * VEC;
        const bool in_a = vec && i0 + VEC <= sg.a_hi;
        const bool in_b = RING && vec && i0 >= sg.b_lo && i0 + VEC <= sg.b_hi;
        u32x4 pv[PV], mv[PV];
        if (vec) {   // a lane past the end reads the tile's first vectors and drops them
            const int64_t po = (m.j0 + (i0 + VEC <= cnt ? i0 : 0)) * 4;
#pragma unroll
            for (int q = 0; q < PV; ++q) {
                pv[q] = gld_stream(param + (uint64_t)(po + 16 * q));
                if (MOM) mv[q] = gld_stream(mom + (uint64_t)(po + 16 * q));
            }
        }
#pragma unroll 1
        for (int pass = 0; pass < (RING ? 2 : 1); ++pass) {
            const bool mine = pass == 0 ? in_a : in_b;
            if (!__builtin_amdgcn_ballot_w64(mine)) continue;
            float y[VEC];
            fold_looped<IN, RING>(a, N, pass == 0 ? sg.sa : sg.sb, (m.j0 + (mine ? i0 : 0)) * ISZ,
                                  y);
            if (mine) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) y[k] = y[k] * inv;
                sgd_vec<IN, OUT, MOM>(gout, param, mom, m.j0 + i0, y, pv, mv, lr, mu);
            }
        }
        if (!in_a && !in_b && i0 < cnt)
            params_sgd_elems<IN, OUT, RING, MOM>(a, N, m, inv, lr, mu, i0, VEC);
    }
}

// Entries [first, first + count) of a table: whole buckets.
struct TileRange {
    int64_t first, count;
};

// The table of a sync as the kernels take it.
PsTable ps_table(const ddp_param_sync *ps)
{
    PsTable tb;
    tb.tiles = reinterpret_cast<const PsTile *>(ps->table);
    tb.params = ps->table + ps->params_offset;
    tb.rstride = ps->rstride;
    tb.pstride = ps->pstride;
    tb.n_tiles = ps->n_tiles;
    tb.tile_elems = ps_tile_elems(ps->in);
    return tb;
}

template <bool RING, int IN, int OUT>
ddp_status_t launch_sync_typed(const ddp_param_sync *ps, TileRange tr, hipStream_t st)
{
    const int N = ps->n_ranks;
    const float inv = 1.0f / (float)N;
    const PsTable tb = ps_table(ps);
    const unsigned lds = lds_for_blocks(params_blocks_per_cu(N, RING));
    const dim3 b(kThreads);
    return launch_split(tr.count, kThreads, "parameter sync kernel launch",
                        [&](int64_t i, unsigned n) {
        const dim3 g(n);
        const int64_t b0 = tr.first + i;
        const bool fixed = with_rank_count<1, 8>(N, [&](auto nr) {
            params_fast<decltype(nr)::value, RING, IN, OUT><<<g, b, lds, st>>>(tb, b0, inv);
        });
        if (!fixed) params_many<RING, IN, OUT><<<g, b, lds, st>>>(tb, N, b0, inv);
    });
}

template <bool RING, int IN, int OUT, bool MOM>
ddp_status_t launch_sgd_typed(const ddp_param_sync *ps, TileRange tr, float lr, float mu,
                              hipStream_t st)
{
    const int N = ps->n_ranks;
    const float inv = 1.0f / (float)N;
    const PsTable tb = ps_table(ps);
    const unsigned lds = lds_for_blocks(params_sgd_blocks_per_cu(N, MOM));
    const dim3 b(kThreads);
    return launch_split(tr.count, kThreads, "parameter SGD kernel launch",
                        [&](int64_t i, unsigned n) {
        const dim3 g(n);
        const int64_t b0 = tr.first + i;
        const bool fixed = with_rank_count<1, 8>(N, [&](auto nr) {
            params_sgd_fast<decltype(nr)::value, RING, IN, OUT, MOM><<<g, b, lds, st>>>(
                tb, b0, inv, lr, mu);
        });
        if (!fixed) params_sgd_many<RING, IN, OUT, MOM><<<g, b, lds, st>>>(tb, N, b0, inv, lr, mu);
    });
}

template <bool RING>
ddp_status_t launch_sync(const ddp_param_sync *ps, TileRange tr, hipStream_t st)
{
    if (ps->in == DDP_F32 && ps->out == DDP_F32)
        return launch_sync_typed<RING, kF32, kF32>(ps, tr, st);
    if (ps->in == DDP_BF16) return launch_sync_typed<RING, kBF16, kBF16>(ps, tr, st);
    return launch_sync_typed<RING, kF32, kBF16>(ps, tr, st);
}

template <bool RING, bool MOM>
ddp_status_t launch_sgd(const ddp_param_sync *ps, TileRange tr, float lr, float mu, hipStream_t st)
{
    if (ps->in == DDP_F32 && ps->out == DDP_F32)
        return launch_sgd_typed<RING, kF32, kF32, MOM>(ps, tr, lr, mu, st);
    if (ps->in == DDP_BF16) return launch_sgd_typed<RING, kBF16, kBF16, MOM>(ps, tr, lr, mu, st);
    return launch_sgd_typed<RING, kF32, kBF16, MOM>(ps, tr, lr, mu, st);
}

// A set of per-parameter tensors the kernel writes.
struct Written {
    const ddp_binding_t *bd;   // null: not used
    int esz;                   // element size
    bool in_place_ok;          // may be exactly the same parameter's gradient of one rank
};

// Written tensors may not overlap each other, and may overlap an input only
// as the same parameter's gradient of one rank, exactly, where the set
// allows it (in place: each element is read before it is written, by the
// same thread).  Inputs may overlap each other: they are only read.
ddp_status_t check_param_alias(const ddp_plan *plan, const ddp_binding_t *const *ranks, int N,
                               int isz, const Written *w, int nw)
{
    struct Iv {
        uint64_t lo, hi;
        int32_t p;
        bool in_place_ok;
    };
    std::vector<Iv> outs;
    try {
        for (int k = 0; k < nw; ++k) {
            if (!w[k].bd) continue;
            for (int32_t p = 0; p < plan->n_params; ++p) {
                if (plan->numel[p] == 0) continue;
                const uint64_t lo = w[k].bd->param_addr[p];
                outs.push_back({lo, lo + (uint64_t)plan->numel[p] * (uint64_t)w[k].esz, p,
                                w[k].in_place_ok});
            }
        }
    } catch (...) {
        return DDP_ERR_NOMEM;
    }
    std::sort(outs.begin(), outs.end(), [](const Iv &x, const Iv &y) { return x.lo < y.lo; });
    for (size_t k = 1; k < outs.size(); ++k)
        if (outs[k].lo < outs[k - 1].hi) return DDP_ERR_ALIAS;
    // written intervals are disjoint and sorted, so their ends are sorted too
    for (int r = 0; r < N; ++r) {
        for (int32_t p = 0; p < plan->n_params; ++p) {
            if (plan->numel[p] == 0) continue;
            const uint64_t lo = ranks[r]->param_addr[p];
            const uint64_t hi = lo + (uint64_t)plan->numel[p] * (uint64_t)isz;
            auto it = std::upper_bound(outs.begin(), outs.end(), lo,
                                       [](uint64_t v, const Iv &x) { return v < x.hi; });
            for (; it != outs.end() && it->lo < hi; ++it)
                if (!(it->in_place_ok && it->lo == lo && it->hi == hi && it->p == p))
                    return DDP_ERR_ALIAS;
        }
    }
    return DDP_OK;
}

// The ring chunks met by bucket positions [t0, t0 + count) of a bucket of
// blen elements over N ranks, as a record's ring word.
uint32_t ring_word(int64_t t0, int64_t count, int64_t blen, int N)
{
    const int64_t C = (blen + N - 1) / N, t1 = t0 + count;
    const int64_t ca = t0 / C, a_end = std::min((ca + 1) * C, blen);
    const uint32_t cut_a = (uint32_t)(std::min(a_end, t1) - t0);
    uint32_t cut_b = cut_a, sb = 0;
    if (a_end < t1) {
        cut_b = (uint32_t)(std::min(std::min((ca + 2) * C, blen), t1) - t0);
        sb = (uint32_t)((ca + 2) % N);
    }
    return (uint32_t)((ca + 1) % N) | sb << 6 | cut_a << 12 | cut_b << 22;
}

// Validates the bindings and builds the device table of a per-parameter
// sync (w: the written sets, in entry order).
ddp_status_t create(const ddp_plan_t *plan, const ddp_binding_t *const *R, int32_t n_ranks,
                    const Written *w, int nw, ddp_order_t order, ddp_dtype_t out_dtype, bool sgd,
                    ddp_param_sync_t **out)
{
    if (n_ranks < 1 || !dtype_ok(out_dtype)) return DDP_ERR_INVALID_ARG;
    if (order != DDP_ORDER_SEQUENTIAL && order != DDP_ORDER_RING) return DDP_ERR_INVALID_ARG;
    if (n_ranks > DDP_MAX_RANKS) return DDP_ERR_UNSUPPORTED;
    const int in = plan->dtype;
    if (!pair_ok(in, out_dtype) || (n_ranks == 1 && in != out_dtype)) return DDP_ERR_UNSUPPORTED;
    int dev = -1;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return hip_fail("hipGetDevice", he);
    const int isz = dtype_size(in);
    auto usable = [&](const ddp_binding_t *bd, int esz) {
        if (bd->plan != plan || bd->device != dev) return false;
        for (int32_t p = 0; p < plan->n_params; ++p)
            if (plan->numel[p] > 0 && bd->param_addr[p] % (uint64_t)esz) return false;
        return true;
    };
    for (int r = 0; r < n_ranks; ++r)
        if (!R[r] || !usable(R[r], isz)) return DDP_ERR_INVALID_ARG;
    for (int k = 0; k < nw; ++k)
        if (w[k].bd && !usable(w[k].bd, w[k].esz)) return DDP_ERR_INVALID_ARG;
    ddp_status_t st = check_param_alias(plan, R, n_ranks, isz, w, nw);
    if (st != DDP_OK) return st;

    const int64_t T = ps_tile_elems(in), pstride = ps_pstride(n_ranks, nw);
    int64_t n_tiles = 0, n_entries = 0;
    for (int32_t p = 0; p < plan->n_params; ++p) {
        n_tiles += (plan->numel[p] + T - 1) / T;
        n_entries += plan->numel[p] > 0 ? 1 : 0;
    }
    if (n_tiles > (int64_t)UINT32_MAX * kXcds) return DDP_ERR_OVERFLOW;
    const int64_t rstride = word_stride(n_tiles);
    const int64_t rec_bytes = (kXcds * rstride * (int64_t)sizeof(PsTile) + 255) / 256 * 256;
    ddp_param_sync *ps = new (std::nothrow) ddp_param_sync();
    if (!ps) return DDP_ERR_NOMEM;
    ps->device = dev;
    ps->n_ranks = n_ranks;
    ps->order = order;
    ps->in = in;
    ps->out = out_dtype;
    ps->sgd = sgd;
    ps->momentum = sgd && w[2].bd != nullptr;
    ps->n_tiles = n_tiles;
    ps->rstride = rstride;
    ps->pstride = pstride;
    ps->params_offset = rec_bytes;
    std::vector<PsTile> recs;
    std::vector<char> ents;
    try {
        ps->bucket_tile.assign((size_t)plan->n_buckets() + 1, 0);
        recs.assign((size_t)(kXcds * rstride), PsTile{0u, 0u});
        ents.assign((size_t)(n_entries * pstride), 0);
    } catch (...) {
        delete ps;
        return DDP_ERR_NOMEM;
    }
    // Parameter entries in flat order; each parameter's tiles are consecutive.
    const bool ring = order == DDP_ORDER_RING && n_ranks > 1;
    int64_t t = 0, q = 0;
    for (int32_t b = 0; b < plan->n_buckets(); ++b) {
        const int64_t blen = plan->bucket_base[b + 1] - plan->bucket_base[b];
        for (int32_t s = plan->bucket_first_slot[b]; s < plan->bucket_first_slot[b + 1]; ++s) {
            const int32_t p = plan->slot_param[s];
            const int64_t n = plan->numel[p];
            if (n == 0) continue;
            char *ent = ents.data() + q * pstride;
            uint64_t *addr = reinterpret_cast<uint64_t *>(ent);
            for (int r = 0; r < n_ranks; ++r) addr[r] = R[r]->param_addr[p];
            // the vector path loads and stores 8- or 16-byte vectors at the
            // tensors' own element alignment, as gfx9 and later global
            // accesses allow (views carved out of one buffer sit at any
            // element offset; requiring a 16-byte boundary sent them down the
            // per-element path at 2.5 TB/s), so every bound tensor (2-byte
            // aligned) qualifies
            bool vec = true;
            for (int k = 0; k < nw; ++k) {
                addr[n_ranks + k] = w[k].bd ? w[k].bd->param_addr[p] : 0;
                vec = vec && (!w[k].bd || w[k].bd->param_addr[p] % 2 == 0);
            }
            PsParamMeta pm;
            std::memset(&pm, 0, sizeof(pm));
            pm.pos0 = plan->param_offset[p];
            pm.blen = blen;
            pm.first_tile = t;
            pm.numel = n;
            pm.vec = vec ? 1u : 0u;
            std::memcpy(ent + 8 * (n_ranks + nw), &pm, sizeof(pm));
            for (int64_t j0 = 0; j0 < n; j0 += T, ++t)
                recs[(size_t)ps_record(t, rstride)] =
                    PsTile{(uint32_t)q, ring ? ring_word(pm.pos0 + j0, std::min(T, n - j0), blen,
                                                         n_ranks)
                                             : 0u};
            ++q;
        }
        ps->bucket_tile[b + 1] = t;
    }
    if (n_tiles == 0) {
        *out = ps;
        return DDP_OK;
    }
    if ((he = hipMalloc(&ps->table, (size_t)(rec_bytes + n_entries * pstride))) != hipSuccess) {
        delete ps;
        return hip_fail("hipMalloc (parameter tiles)", he, DDP_ERR_NOMEM);
    }
    if ((he = hipMemcpy(ps->table, recs.data(), recs.size() * sizeof(PsTile),
                        hipMemcpyHostToDevice)) != hipSuccess ||
        (he = hipMemcpy(ps->table + rec_bytes, ents.data(), ents.size(),
                        hipMemcpyHostToDevice)) != hipSuccess) {
        ddp_param_sync_free(ps);
        return hip_fail("hipMemcpy (parameter tiles)", he);
    }
    *out = ps;
    return DDP_OK;
}

// Checks a run call and finds the entries of buckets [b0, b0 + nb) (nb < 0:
// every bucket).
ddp_status_t check_run(const ddp_param_sync_t *ps, bool sgd, int32_t b0, int32_t nb, TileRange *tr)
{
    if (!ps || ps->sgd != sgd) return DDP_ERR_INVALID_ARG;
    const int32_t n_buckets = (int32_t)ps->bucket_tile.size() - 1;
    if (nb < 0) {
        b0 = 0;
        nb = n_buckets;
    }
    if (b0 < 0 || b0 > n_buckets || nb > n_buckets - b0) return DDP_ERR_INVALID_ARG;
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != ps->device) return DDP_ERR_INVALID_ARG;
    tr->first = ps->bucket_tile[b0];
    tr->count = ps->bucket_tile[b0 + nb] - tr->first;
    return DDP_OK;
}

ddp_status_t run_sync(const ddp_param_sync_t *ps, int32_t b0, int32_t nb, void *stream)
{
    TileRange tr;
    const ddp_status_t s = check_run(ps, false, b0, nb, &tr);
    if (s != DDP_OK || tr.count == 0) return s;
    const OccupancyScope occ(ps->occupancy.load(std::memory_order_relaxed));
    hipStream_t st = static_cast<hipStream_t>(stream);
    return ps->order == DDP_ORDER_RING && ps->n_ranks > 1 ? launch_sync<true>(ps, tr, st)
                                                          : launch_sync<false>(ps, tr, st);
}

ddp_status_t run_sgd(const ddp_param_sync_t *ps, int32_t b0, int32_t nb, float lr, float mu,
                     void *stream)
{
    TileRange tr;
    const ddp_status_t s = check_run(ps, true, b0, nb, &tr);
    if (s != DDP_OK || tr.count == 0) return s;
    const OccupancyScope occ(ps->occupancy.load(std::memory_order_relaxed));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool ring = ps->order == DDP_ORDER_RING && ps->n_ranks > 1;
    if (ring)
        return ps->momentum ? launch_sgd<true, true>(ps, tr, lr, mu, st)
                            : launch_sgd<true, false>(ps, tr, lr, mu, st);
    return ps->momentum ? launch_sgd<false, true>(ps, tr, lr, mu, st)
                        : launch_sgd<false, false>(ps, tr, lr, mu, st);
}

}  // namespace

extern "C" {

ddp_status_t ddp_param_sync_create(const ddp_plan_t *plan, const ddp_binding_t *const *rank_bindings,
                                   int32_t n_ranks, const ddp_binding_t *out_binding,
                                   ddp_order_t order, ddp_dtype_t out_dtype,
                                   ddp_param_sync_t **out)
{
    if (!plan || !rank_bindings || !out_binding || !out) return DDP_ERR_INVALID_ARG;
    const Written w[kSyncExtra] = {{out_binding, dtype_size(out_dtype), true}};
    return create(plan, rank_bindings, n_ranks, w, kSyncExtra, order, out_dtype, false, out);
}

ddp_status_t ddp_param_sync_run(const ddp_param_sync_t *ps, void *stream)
{
    return run_sync(ps, 0, -1, stream);
}

ddp_status_t ddp_param_sync_run_buckets(const ddp_param_sync_t *ps, int32_t first_bucket,
                                        int32_t n_buckets, void *stream)
{
    if (n_buckets < 0) return DDP_ERR_INVALID_ARG;
    return run_sync(ps, first_bucket, n_buckets, stream);
}

ddp_status_t ddp_param_sgd_create(const ddp_plan_t *plan, const ddp_binding_t *const *rank_bindings,
                                  int32_t n_ranks, const ddp_binding_t *grad_out,
                                  const ddp_binding_t *params, const ddp_binding_t *momentum,
                                  ddp_order_t order, ddp_dtype_t out_dtype, ddp_param_sync_t **out)
{
    if (!plan || !rank_bindings || !params || !out) return DDP_ERR_INVALID_ARG;
    const Written w[kSgdExtra] = {{grad_out, dtype_size(out_dtype), true},
                                  {params, 4, false},
                                  {momentum, 4, false}};
    return create(plan, rank_bindings, n_ranks, w, kSgdExtra, order, out_dtype, true, out);
}

ddp_status_t ddp_param_sgd_run(const ddp_param_sync_t *ps, float lr, float momentum, void *stream)
{
    return run_sgd(ps, 0, -1, lr, momentum, stream);
}

ddp_status_t ddp_param_sgd_run_buckets(const ddp_param_sync_t *ps, int32_t first_bucket,
                                       int32_t n_buckets, float lr, float momentum, void *stream)
{
    if (n_buckets < 0) return DDP_ERR_INVALID_ARG;
    return run_sgd(ps, first_bucket, n_buckets, lr, momentum, stream);
}

ddp_status_t ddp_param_sync_set_occupancy(ddp_param_sync_t *ps, ddp_occupancy_t policy)
{
    if (!ps || (policy != DDP_OCCUPANCY_TUNED && policy != DDP_OCCUPANCY_SHARED &&
                policy != DDP_OCCUPANCY_DEFAULT))
        return DDP_ERR_INVALID_ARG;
    ps->occupancy.store(policy, std::memory_order_relaxed);
    return DDP_OK;
}

ddp_occupancy_t ddp_param_sync_get_occupancy(const ddp_param_sync_t *ps)
{
    return ps ? static_cast<ddp_occupancy_t>(ps->occupancy.load(std::memory_order_relaxed))
              : DDP_OCCUPANCY_DEFAULT;
}

void ddp_param_sync_free(ddp_param_sync_t *ps)
{
    if (!ps) return;
    if (ps->table) {
        int cur = -1;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(ps->device);
        (void)hipFree(ps->table);
        if (cur >= 0) (void)hipSetDevice(cur);
    }
    delete ps;
}

}  // extern "C"
