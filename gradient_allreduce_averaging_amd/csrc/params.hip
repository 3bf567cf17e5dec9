// The synchronisation over per-parameter gradient tensors in one kernel
// (ddp_param_sync_create / _run / _free).  Every rank's gradients are read
// where they lie, with no flatten, folded in the fixed order their flat
// positions define, scaled, and written to per-parameter outputs, with no
// unflatten.  The result is that of flatten, then ddp_sync_allreduce_avg,
// then unflatten, bit for bit; the bytes moved are those of the sync alone
// (N reads and one write per element), where the three steps move
// 2N + N + 1 + 2 element-widths per element.
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel) 4.2 (the
//        gradients are copied into a flat bucket, averaged, and viewed back;
//        gradient_as_bucket_view drops a copy);
//        [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn) 八
//        (gradients laid out by region so that no copy is needed).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
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
// of the parameter's address.  One table entry per tile, `stride` bytes
// (16-byte aligned):
//   uint64_t addr[N + 1]   ranks 0..N-1, then the output, at the tile's first element
//   PsMeta                 below
struct PsMeta {
    int64_t pos;      // position of the tile's first element inside its bucket
    int64_t blen;     // length of that bucket
    uint32_t count;   // elements in the tile, 1..tile
    uint32_t vec;     // 1: every address of the parameter 16-byte aligned
    uint32_t starts;  // the ring chunks the tile meets: start rank of chunk a
                      // (bits 0-5) and of chunk b (bits 6-11) ...
    uint32_t cuts;    // ... and where a (bits 0-15) and b (bits 16-31) end,
                      // relative to the tile's first element
};

int64_t ps_stride(int N) { return (8 * (int64_t)(N + 1) + (int64_t)sizeof(PsMeta) + 15) / 16 * 16; }

// Streaming accesses at an address read from the table, typed as global
// memory so that they compile to global (not flat) instructions.
typedef __attribute__((address_space(1))) u32x2 g_u32x2;
typedef __attribute__((address_space(1))) float g_f32;
typedef __attribute__((address_space(1))) uint32_t g_u32;
typedef __attribute__((address_space(1))) uint16_t g_u16;

__device__ __forceinline__ u32x4 gld_stream(uint64_t addr) { return ld_at(addr, 0); }
__device__ __forceinline__ void gst_stream(uint64_t addr, const u32x4 &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<g_u32x4 *>(addr));
}
__device__ __forceinline__ void gst_stream(uint64_t addr, const u32x2 &v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<g_u32x2 *>(addr));
}

// Scale, convert and store one vector of accumulators at tile element i0 of
// the output at `out` (the flat kernels' store_vec, on a table address).
template <int IN, int OUT>
__device__ __forceinline__ void gstore_vec(uint64_t out, int64_t i0, const float *acc, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    float y[VEC];
    for (int e = 0; e < VEC; ++e) y[e] = acc[e] * inv;
    if (OUT == kF32) {
        u32x4 o;
        for (int e = 0; e < 4; ++e) o[e] = __float_as_uint(y[e]);
        gst_stream(out + (uint64_t)i0 * 4, o);
    } else {
        uint32_t h[VEC];
        for (int e = 0; e < VEC; ++e) h[e] = bf16_rne(y[e]);
        if (VEC == 4) {
            u32x2 o;
            o[0] = h[0] | (h[1] << 16);
            o[1] = h[2] | (h[3] << 16);
            gst_stream(out + (uint64_t)i0 * 2, o);
        } else {
            u32x4 o;
            for (int w = 0; w < 4; ++w) o[w] = h[2 * w] | (h[2 * w + 1] << 16);
            gst_stream(out + (uint64_t)i0 * 2, o);
        }
    }
}

template <int IN>
__device__ __forceinline__ float gload_elem(uint64_t a, int64_t i)
{
    if (IN == kF32) return *reinterpret_cast<const g_f32 *>(a + (uint64_t)i * 4);
    return widen_bf16(*reinterpret_cast<const g_u16 *>(a + (uint64_t)i * 2));
}

// Per-element path: tile elements [i0, i0 + cnt) clipped to the tile.
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
                *reinterpret_cast<g_u32 *>(out + (uint64_t)i * 4) =
                    *reinterpret_cast<const g_u32 *>(a[0] + (uint64_t)i * 4);
            else
                *reinterpret_cast<g_u16 *>(out + (uint64_t)i * 2) =
                    *reinterpret_cast<const g_u16 *>(a[0] + (uint64_t)i * 2);
            continue;
        }
        int r = 0;
        if (RING) {
            const int64_t C = (m.blen + N - 1) / N;
            r = (int)(((m.pos + i) / C + 1) % N);
        }
        float acc = gload_elem<IN>(a[r], i);
        if (!RING) acc = 0.0f + acc;
        for (int k = 1; k < N; ++k) {
            r = wrap(r + 1, N);
            acc = acc + gload_elem<IN>(a[r], i);
        }
        const float y = acc * inv;
        if (OUT == kF32)
            *reinterpret_cast<g_f32 *>(out + (uint64_t)i * 4) = y;
        else
            *reinterpret_cast<g_u16 *>(out + (uint64_t)i * 2) = (uint16_t)bf16_rne(y);
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
        s.sa = __builtin_amdgcn_readfirstlane((int)(m.starts & 63u));
        s.sb = __builtin_amdgcn_readfirstlane((int)((m.starts >> 6) & 63u));
        s.a_hi = s.b_lo = (int64_t)(m.cuts & 0xffffu);
        s.b_hi = (int64_t)(m.cuts >> 16);
    }
    return s;
}

// N known at compile time (1..8).  The tile's entry (one batch of scalar
// loads) gives every address; then all NR * kPsUnroll vector loads of the
// lane go out before the ring chunks are looked at, as in the flat reduce.
// A lane's vector past the tile's end reads the tile's first vector and
// drops it.  The loads are not behind a branch (a branch would wait for the
// entry's flags before fetching its addresses): a tile without the vector
// path reads 16 bytes of its own entry instead, and drops them.
template <int NR, bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
params_fast(const char *__restrict__ table, int64_t stride, int64_t first_block, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const char *e = table + (first_block + blockIdx.x) * stride;
    const uint64_t *a = reinterpret_cast<const uint64_t *>(e);
    uint64_t ad[NR + 1];
#pragma unroll
    for (int k = 0; k <= NR; ++k) ad[k] = a[k];
    const PsMeta m = *reinterpret_cast<const PsMeta *>(e + 8 * (NR + 1));
    // every address is fetched in the entry's one batch of scalar loads,
    // before any of them is used
#pragma unroll
    for (int k = 0; k <= NR; ++k) asm volatile("" : "+s"(ad[k]));
    const int64_t cnt = m.count;
    const bool vec = m.vec && cnt >= VEC;
    int64_t i0[kPsUnroll];
    u32x4 v[kPsUnroll][NR];
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        i0[u] = ((int64_t)u * kThreads + threadIdx.x) * VEC;
        const int64_t off = i0[u] + VEC <= cnt ? i0[u] * ISZ : 0;
#pragma unroll
        for (int k = 0; k < NR; ++k)
            v[u][k] = gld_stream(vec ? ad[k] + (uint64_t)off : reinterpret_cast<uint64_t>(e));
    }
    const PsSegs sg = ps_segs<RING>(m);
#pragma unroll
    for (int u = 0; u < kPsUnroll; ++u) {
        const bool in_a = vec && i0[u] + VEC <= sg.a_hi;
        const bool in_b = RING && vec && i0[u] >= sg.b_lo && i0[u] + VEC <= sg.b_hi;
        if (in_a || in_b) {
            if constexpr (NR == 1 && IN == OUT) {
                gst_stream(ad[1] + (uint64_t)(i0[u] * ISZ), v[u][0]);
            } else {
                float acc[VEC];
                if (!RING)
                    fold_seq<NR, IN>(v[u], acc);
                else
                    fold_ring<NR, IN>(v[u], in_a ? sg.sa : sg.sb, acc);
                gstore_vec<IN, OUT>(ad[NR], i0[u], acc, inv);
            }
        } else if (i0[u] < cnt) {
            params_elems<IN, OUT, RING>(a, NR, m, inv, i0[u], VEC);
        }
    }
}

// Any N up to DDP_MAX_RANKS: one pass per ring chunk the wave's lanes meet,
// folded with fold_looped from the entry's addresses.
template <bool RING, int IN, int OUT>
__global__ void __launch_bounds__(kThreads)
params_many(const char *__restrict__ table, int64_t stride, int N, int64_t first_block, float inv)
{
    constexpr int VEC = IN == kF32 ? 4 : 8;
    constexpr int ISZ = IN == kF32 ? 4 : 2;
    const char *e = table + (first_block + blockIdx.x) * stride;
    const uint64_t *a = reinterpret_cast<const uint64_t *>(e);
    const PsMeta m = *reinterpret_cast<const PsMeta *>(e + 8 * (N + 1));
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
            fold_looped<IN, RING>(a, N, pass == 0 ? sg.sa : sg.sb, mine ? i0 * ISZ : 0, acc);
            if (mine) gstore_vec<IN, OUT>(a[N], i0, acc, inv);
        }
        if (!in_a && !in_b && i0 < cnt) params_elems<IN, OUT, RING>(a, N, m, inv, i0, VEC);
    }
}

template <bool RING, int IN, int OUT>
ddp_status_t launch_params_typed(const ddp_param_sync *ps, hipStream_t st)
{
    const int N = ps->n_ranks;
    const float inv = 1.0f / (float)N;
    const char *tb = ps->table;
    const int64_t sd = ps->stride;
    const unsigned lds = lds_for_blocks(params_blocks_per_cu(N, RING, IN == kBF16));
    const dim3 b(kThreads);
    return launch_split(ps->n_tiles, kThreads, "parameter sync kernel launch",
                        [&](int64_t b0, unsigned n) {
        const dim3 g(n);
        switch (N) {
        case 1: params_fast<1, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 2: params_fast<2, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 3: params_fast<3, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 4: params_fast<4, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 5: params_fast<5, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 6: params_fast<6, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 7: params_fast<7, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        case 8: params_fast<8, RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, b0, inv); break;
        default: params_many<RING, IN, OUT><<<g, b, lds, st>>>(tb, sd, N, b0, inv); break;
        }
    });
}

template <bool RING>
ddp_status_t launch_params(const ddp_param_sync *ps, hipStream_t st)
{
    if (ps->in == DDP_F32 && ps->out == DDP_F32) return launch_params_typed<RING, kF32, kF32>(ps, st);
    if (ps->in == DDP_BF16) return launch_params_typed<RING, kBF16, kBF16>(ps, st);
    return launch_params_typed<RING, kF32, kBF16>(ps, st);
}

// The outputs may not overlap each other, and may overlap an input only as
// the same parameter's gradient of one rank, exactly (in place: each element
// is read before it is written, by the same thread).  Inputs may overlap
// each other: they are only read.
ddp_status_t check_param_alias(const ddp_plan *plan, const ddp_binding_t *const *ranks, int N,
                               const ddp_binding_t *out, int isz, int osz)
{
    struct Iv {
        uint64_t lo, hi;
        int32_t p;
    };
    std::vector<Iv> outs;
    try {
        outs.reserve((size_t)plan->n_params);
        for (int32_t p = 0; p < plan->n_params; ++p) {
            if (plan->numel[p] == 0) continue;
            const uint64_t lo = out->param_addr[p];
            outs.push_back({lo, lo + (uint64_t)plan->numel[p] * (uint64_t)osz, p});
        }
    } catch (...) {
        return DDP_ERR_NOMEM;
    }
    std::sort(outs.begin(), outs.end(), [](const Iv &x, const Iv &y) { return x.lo < y.lo; });
    for (size_t k = 1; k < outs.size(); ++k)
        if (outs[k].lo < outs[k - 1].hi) return DDP_ERR_ALIAS;
    // outs are disjoint and sorted, so their ends are sorted too
    for (int r = 0; r < N; ++r) {
        for (int32_t p = 0; p < plan->n_params; ++p) {
            if (plan->numel[p] == 0) continue;
            const uint64_t lo = ranks[r]->param_addr[p];
            const uint64_t hi = lo + (uint64_t)plan->numel[p] * (uint64_t)isz;
            auto it = std::upper_bound(outs.begin(), outs.end(), lo,
                                       [](uint64_t v, const Iv &x) { return v < x.hi; });
            for (; it != outs.end() && it->lo < hi; ++it)
                if (!(it->lo == lo && it->hi == hi && it->p == p)) return DDP_ERR_ALIAS;
        }
    }
    return DDP_OK;
}

// The ring chunks met by bucket positions [t0, t0 + count) of a bucket of
// blen elements over N ranks: the entry's starts and cuts words.
void ring_words(int64_t t0, int64_t count, int64_t blen, int N, uint32_t *starts, uint32_t *cuts)
{
    const int64_t C = (blen + N - 1) / N, t1 = t0 + count;
    const int64_t ca = t0 / C, a_end = std::min((ca + 1) * C, blen);
    const uint32_t cut_a = (uint32_t)(std::min(a_end, t1) - t0);
    uint32_t cut_b = cut_a, sb = 0;
    if (a_end < t1) {
        cut_b = (uint32_t)(std::min(std::min((ca + 2) * C, blen), t1) - t0);
        sb = (uint32_t)((ca + 2) % N);
    }
    *starts = (uint32_t)((ca + 1) % N) | sb << 6;
    *cuts = cut_a | cut_b << 16;
}

}  // namespace

extern "C" {

ddp_status_t ddp_param_sync_create(const ddp_plan_t *plan, const ddp_binding_t *const *rank_bindings,
                                   int32_t n_ranks, const ddp_binding_t *out_binding,
                                   ddp_order_t order, ddp_dtype_t out_dtype,
                                   ddp_param_sync_t **out)
{
    if (!plan || !rank_bindings || !out_binding || !out) return DDP_ERR_INVALID_ARG;
    if (n_ranks < 1 || !dtype_ok(out_dtype)) return DDP_ERR_INVALID_ARG;
    if (order != DDP_ORDER_SEQUENTIAL && order != DDP_ORDER_RING) return DDP_ERR_INVALID_ARG;
    if (n_ranks > DDP_MAX_RANKS) return DDP_ERR_UNSUPPORTED;
    const int in = plan->dtype;
    if (!pair_ok(in, out_dtype) || (n_ranks == 1 && in != out_dtype)) return DDP_ERR_UNSUPPORTED;
    int dev = -1;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return hip_fail("hipGetDevice", he);
    const int isz = dtype_size(in), osz = dtype_size(out_dtype);
    const ddp_binding_t *const *R = rank_bindings;
    for (int r = 0; r <= n_ranks; ++r) {
        const ddp_binding_t *bd = r < n_ranks ? R[r] : out_binding;
        if (!bd || bd->plan != plan || bd->device != dev) return DDP_ERR_INVALID_ARG;
        const int esz = r < n_ranks ? isz : osz;
        for (int32_t p = 0; p < plan->n_params; ++p)
            if (plan->numel[p] > 0 && bd->param_addr[p] % (uint64_t)esz) return DDP_ERR_INVALID_ARG;
    }
    ddp_status_t st = check_param_alias(plan, R, n_ranks, out_binding, isz, osz);
    if (st != DDP_OK) return st;

    const int64_t T = ps_tile_elems(in), stride = ps_stride(n_ranks);
    int64_t n_tiles = 0;
    for (int32_t p = 0; p < plan->n_params; ++p) n_tiles += (plan->numel[p] + T - 1) / T;
    if (n_tiles > INT64_MAX / stride) return DDP_ERR_OVERFLOW;
    ddp_param_sync *ps = new (std::nothrow) ddp_param_sync();
    if (!ps) return DDP_ERR_NOMEM;
    ps->device = dev;
    ps->n_ranks = n_ranks;
    ps->order = order;
    ps->in = in;
    ps->out = out_dtype;
    ps->n_tiles = n_tiles;
    ps->stride = stride;
    if (n_tiles == 0) {
        *out = ps;
        return DDP_OK;
    }
    if ((he = hipMalloc(&ps->table, (size_t)(n_tiles * stride))) != hipSuccess) {
        delete ps;
        return hip_fail("hipMalloc (parameter tiles)", he, DDP_ERR_NOMEM);
    }
    // Entries in flat order, built and uploaded in pieces of at most 64 MiB.
    const int64_t per_chunk = std::max<int64_t>(1, (64 << 20) / stride);
    std::vector<char> host;
    try {
        host.assign((size_t)(std::min(per_chunk, n_tiles) * stride), 0);
    } catch (...) {
        ddp_param_sync_free(ps);
        return DDP_ERR_NOMEM;
    }
    int64_t done = 0, fill = 0;
    auto flush = [&]() -> ddp_status_t {
        const hipError_t e = hipMemcpy(ps->table + done * stride, host.data(),
                                       (size_t)(fill * stride), hipMemcpyHostToDevice);
        if (e != hipSuccess) return hip_fail("hipMemcpy (parameter tiles)", e);
        done += fill;
        fill = 0;
        std::memset(host.data(), 0, host.size());
        return DDP_OK;
    };
    const bool ring = order == DDP_ORDER_RING && n_ranks > 1;
    for (int32_t b = 0; b < plan->n_buckets(); ++b) {
        const int64_t blen = plan->bucket_base[b + 1] - plan->bucket_base[b];
        for (int32_t s = plan->bucket_first_slot[b]; s < plan->bucket_first_slot[b + 1]; ++s) {
            const int32_t p = plan->slot_param[s];
            const int64_t n = plan->numel[p];
            bool vec = out_binding->param_addr[p] % 16 == 0;
            for (int r = 0; r < n_ranks; ++r) vec = vec && R[r]->param_addr[p] % 16 == 0;
            for (int64_t j0 = 0; j0 < n; j0 += T) {
                char *ent = host.data() + fill * stride;
                uint64_t *addr = reinterpret_cast<uint64_t *>(ent);
                for (int r = 0; r < n_ranks; ++r)
                    addr[r] = R[r]->param_addr[p] + (uint64_t)(j0 * isz);
                addr[n_ranks] = out_binding->param_addr[p] + (uint64_t)(j0 * osz);
                PsMeta m;
                std::memset(&m, 0, sizeof(m));
                m.pos = plan->param_offset[p] + j0;
                m.blen = blen;
                m.count = (uint32_t)std::min(T, n - j0);
                m.vec = vec ? 1u : 0u;
                if (ring) ring_words(m.pos, m.count, blen, n_ranks, &m.starts, &m.cuts);
                std::memcpy(ent + 8 * (n_ranks + 1), &m, sizeof(m));
                if (++fill == per_chunk && (st = flush()) != DDP_OK) {
                    ddp_param_sync_free(ps);
                    return st;
                }
            }
        }
    }
    if (fill > 0 && (st = flush()) != DDP_OK) {
        ddp_param_sync_free(ps);
        return st;
    }
    *out = ps;
    return DDP_OK;
}

ddp_status_t ddp_param_sync_run(const ddp_param_sync_t *ps, void *stream)
{
    if (!ps) return DDP_ERR_INVALID_ARG;
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev != ps->device) return DDP_ERR_INVALID_ARG;
    if (ps->n_tiles == 0) return DDP_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    return ps->order == DDP_ORDER_RING && ps->n_ranks > 1 ? launch_params<true>(ps, st)
                                                          : launch_params<false>(ps, st);
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
