// Flatten and unflatten: per-parameter gradients <-> flat bucket buffers
// (ddp_bind_params, ddp_flatten, ddp_unflatten).  The flat buffer of a
// bucket holds its parameters' gradients back to back at the plan's
// offsets, with no padding; after the average it is viewed back onto the
// parameters' gradients.
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel), 4.2
//        (flat_grad built from the gradients, then viewed back).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

// ---------------------------------------------------------------- copies

constexpr int64_t kCopyRun = 64;   // consecutive copy units per XCD (unit_of_block)

static_assert(kCopyBlockBytes == 2 * 16 * kCopyThreads, "two vectors per thread cover a block");

// Block -> unit mapping of both copy kernels.  BPU blocks per copy unit
// (copy_blocks_per_unit: 8 KiB a block), each moving its share of the unit
// (parts past a short unit's end return at once).  Workgroups are dealt to
// the XCDs round-robin (block b runs on XCD b % 8).  Each XCD takes runs of
// `run` consecutive units (units [(8k + x) run, (8k + x + 1) run) go to XCD
// x), and the blocks of one unit run on one XCD, where the unit's table
// entry is then an L2 hit for all but the first of them.  Consecutive units
// touch neighbouring bytes: where a parameter's flat offset is not a
// multiple of the 128-byte line, the line two units share is written by one
// XCD's L2 inside a run instead of from two L2s, which measured 2-3 %
// faster with many small unaligned parameters (runs of 64; runs of 256, or
// one contiguous span per XCD, measured slower on large ones).  The units
// after the last whole round of 8 runs are shared out in runs of last_run =
// ceil(rest / 8), so that no XCD ends the launch with a whole run more than
// the others.  Units hold 4K elements: with many short parameters, bigger
// units mostly spawn blocks that find no work.
struct CopyMap {
    unsigned run, last_run;   // units per XCD run: whole rounds, the last round
    unsigned full_j;          // units of one XCD in whole rounds
};

template <int BPU>
__device__ __forceinline__ int64_t unit_of_block(const CopyMap &cm, int64_t *lo)
{
    constexpr int64_t kBlockElems = kCopyUnitElems / BPU;
    const unsigned m = blockIdx.x / kXcds, j = m / BPU;   // this XCD's j-th unit
    const unsigned x = blockIdx.x % kXcds;
    *lo = (m % BPU) * kBlockElems;
    if (j < cm.full_j) return (int64_t)((j / cm.run) * kXcds + x) * cm.run + j % cm.run;
    return (int64_t)cm.full_j * kXcds + (int64_t)x * cm.last_run + (j - cm.full_j);
}

// Unflatten, the chunks two or more parameters share: eight lanes per chunk,
// lane k copying the chunk's bytes [2k, 2k + 2) from the flat buffer where
// they belong to a parameter of the bucket, in one store instruction.  Run
// by the blocks of an unflatten launch past bulk_blocks.
struct UnflatEdges {
    const ddp_unflatten_edge *edges;
    int64_t n;
    unsigned bulk_blocks;   // the launch's copy blocks; the blocks after them take the edges
};

__device__ __forceinline__ void unflatten_edge(const UnflatEdges &ue, int64_t lane, const char *flat)
{
    const int64_t i = lane >> 3;
    if (i >= ue.n) return;
    const int k = (int)(lane & 7);
    const int64_t off = ue.edges[i].piece[k];
    if (off < 0) return;
    *reinterpret_cast<uint16_t *>(ue.edges[i].chunk + 2 * (uint64_t)k) =
        *reinterpret_cast<const uint16_t *>(flat + off);
}

// Unflatten (flat -> param), the bulk: the mirror of flatten_units with the
// roles of the buffers swapped.  Parameter views carved out of one buffer
// sit at any alignment, so a 16-byte chunk of parameter storage can hold
// bytes of two units of one parameter, or of two parameters.  Each block
// writes the chunks that start in its bytes [d0, d1) of the parameter and
// end inside it, one aligned store each, reading the flat buffer, where a
// parameter's units are contiguous, at its own alignment.  The chunks at the
// parameter's two ends are partial: one that holds no other parameter's
// bytes is written here, 2 bytes per lane in one store instruction; one that
// does (flags in the unit entry, for this element size) is left to the edge
// blocks (unflatten_edge).  Parameters that start on the allocator's alignment, as
// separate tensors do, have no first partial chunk and share no chunk.
template <int BPU>
__global__ void __launch_bounds__(kCopyThreads)
unflatten_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, CopyMap cm,
                const char *flat, int esize, UnflatEdges ue)
{
    if (blockIdx.x >= ue.bulk_blocks) {
        unflatten_edge(ue, (int64_t)(blockIdx.x - ue.bulk_blocks) * kCopyThreads + threadIdx.x, flat);
        return;
    }
    int64_t lo;
    const int64_t ui = unit_of_block<BPU>(cm, &lo);
    if (ui >= n_units) return;
    const ddp_copy_unit u = units[first + ui];
    if (lo >= u.count) return;
    const int64_t n = min((int64_t)u.count - lo, kCopyUnitElems / BPU);
    const char *src = flat + (u.flat_elem + lo) * esize;
    const uintptr_t d0 = (uintptr_t)u.param_addr + (uintptr_t)((u.param_elem + lo) * esize);
    const uintptr_t d1 = d0 + (uintptr_t)(n * esize);
    const int more = u.more & 0xff, sh = 8 + 2 * (esize >> 2);   // esize 2: bits 8-9, 4: 10-11
    const uintptr_t pend = d1 + (uintptr_t)(((int64_t)u.count - lo - n + more) * esize);
    const bool shared_head = (u.more >> sh) & 1, shared_tail = (u.more >> (sh + 1)) & 1;
    const uintptr_t cf = (d0 + 15) & ~(uintptr_t)15;
    const int tid = threadIdx.x;
    // the parameter's first chunk, partial, when no other parameter shares it
    if (u.param_elem + lo == 0 && cf != d0 && !shared_head) {
        const uintptr_t x = d0 + 2 * (uintptr_t)tid, xe = min(cf, pend);
        if (tid < 8 && x < xe)
            *reinterpret_cast<uint16_t *>(x) = *reinterpret_cast<const uint16_t *>(src + (x - d0));
    }
    if (cf >= d1) return;                                // no chunk starts here
    int64_t nch = (int64_t)((d1 - cf + 15) >> 4);        // chunks starting in [d0, d1), <= 512
    const uintptr_t cl = cf + 16 * (uintptr_t)(nch - 1);
    const bool tail = cl + 16 > pend;                    // the last holds the parameter's end
    if (tail) --nch;
    const int64_t k0 = tid, k1 = tid + kCopyThreads;
    const char *s = src + (cf - d0);
    u32x4 *dv = reinterpret_cast<u32x4 *>(cf);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    uint16_t t = 0;
    const uintptr_t xt = cl + 2 * (uintptr_t)(tid - (kCopyThreads - 8));
    const bool tl = tail && !shared_tail && tid >= kCopyThreads - 8 && xt < pend;
    if (k0 < nch) a = ld_stream(s + 16 * k0);
    if (k1 < nch) b = ld_stream(s + 16 * k1);
    if (tl) t = *reinterpret_cast<const uint16_t *>(src + (xt - d0));
    if (k0 < nch) __builtin_nontemporal_store(a, dv + k0);
    if (k1 < nch) __builtin_nontemporal_store(b, dv + k1);
    if (tl) *reinterpret_cast<uint16_t *>(xt) = t;       // the last 8 lanes: one store
}

// A parameter's start in the flat buffer: its first unit and flat element.
struct TensorStart {
    int64_t unit, flat_elem;
};

// The unit whose flat elements hold element f, walked to from unit w (the
// caller's first guess, right in all but layouts with parameters shorter
// than a 16-byte chunk).
__device__ __forceinline__ ddp_copy_unit unit_holding(const ddp_copy_unit *units, int64_t w,
                                                      int64_t f)
{
    ddp_copy_unit u = units[w];
    while (f < u.flat_elem) u = units[--w];
    while (f >= u.flat_elem + u.count) u = units[++w];
    return u;
}

// Flatten, the chunks flatten_units leaves, run by the blocks of a flatten
// launch past bulk_blocks.  Boundary i of the range is the first flat
// element of its i-th parameter, and after the last one the range's end.  A
// boundary inside a 16-byte chunk (not on its first byte) makes the chunk
// an edge chunk, which the chunk's first such boundary takes.  Eight lanes
// serve boundary i, lane p the chunk's bytes [2p, 2p + 2): bytes before the
// boundary come from the unit before it, bytes from it on from its
// parameter's first unit (or, where parameters are shorter than a chunk, a
// unit further off), none outside the range.  The eight lanes store in one
// instruction, so the chunk is written whole.
struct FlatEdges {
    const TensorStart *starts;   // the range's parameter starts
    int64_t nb;                  // their number
    int64_t first, last;         // the range's units
    int64_t r0e, r1e;            // the range's flat elements
    unsigned bulk_blocks;        // the launch's copy blocks; the blocks after them take the edges
};

__device__ __forceinline__ void flatten_edge(const ddp_copy_unit *units, const FlatEdges &fe,
                                             int64_t lane, char *flat, int esize)
{
    const int64_t i = lane >> 3;
    const int p = (int)(lane & 7);
    if (i > fe.nb) return;
    const uintptr_t fb = reinterpret_cast<uintptr_t>(flat);
    const TensorStart ts = i < fe.nb ? fe.starts[i] : TensorStart{fe.last, fe.r1e};
    const uintptr_t b = fb + (uintptr_t)(ts.flat_elem * esize);
    if ((b & 15) == 0) return;
    const uintptr_t c = b & ~(uintptr_t)15;
    if (i > 0 && fb + (uintptr_t)(fe.starts[i - 1].flat_elem * esize) > c)
        return;                                      // an earlier boundary in the chunk takes it
    const uintptr_t x = c + 2 * (uintptr_t)p;
    const uintptr_t r0 = fb + (uintptr_t)(fe.r0e * esize), r1 = fb + (uintptr_t)(fe.r1e * esize);
    if (x < r0 || x >= r1) return;
    // element f holds byte x; the unit before the boundary or the one at it
    const int64_t f = (int64_t)((x - fb) / (uintptr_t)esize);
    const ddp_copy_unit u = unit_holding(units, x < b ? ts.unit - 1 : ts.unit, f);
    const char *s = reinterpret_cast<const char *>(u.param_addr) + u.param_elem * esize +
                    (x - (fb + (uintptr_t)(u.flat_elem * esize)));
    *reinterpret_cast<uint16_t *>(x) = *reinterpret_cast<const uint16_t *>(s);
}

// Flatten (param -> flat), the bulk.  Parameters sit in the flat buffer at
// any element offset, so the 16-byte chunk that holds a parameter's last
// bytes often holds the next one's first bytes too.  Each block writes the
// chunks that start in its bytes [d0, d1) and end inside its parameter
// (counting the parameter's bytes past d1, `more` of them past the unit):
// one vector load from the source at its own alignment (any address) and
// an aligned 16-byte store each.  The chunk that holds a parameter's end
// when that end is not on a chunk boundary, and the chunk before the
// range's first byte, are left to the edge blocks (flatten_edge).  So every
// chunk has one writer and every store is whole, and a parameter whose
// bytes start and end on chunk boundaries needs no edge work at all.
template <int BPU>
__global__ void __launch_bounds__(kCopyThreads)
flatten_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, CopyMap cm,
              char *flat, int esize, FlatEdges fe)
{
    if (blockIdx.x >= fe.bulk_blocks) {
        flatten_edge(units, fe, (int64_t)(blockIdx.x - fe.bulk_blocks) * kCopyThreads + threadIdx.x,
                     flat, esize);
        return;
    }
    int64_t lo;
    const int64_t ui = unit_of_block<BPU>(cm, &lo);
    if (ui >= n_units) return;
    const ddp_copy_unit u = units[first + ui];
    if (lo >= u.count) return;
    const int64_t n = min((int64_t)u.count - lo, kCopyUnitElems / BPU);
    const char *src = reinterpret_cast<const char *>(u.param_addr) + (u.param_elem + lo) * esize;
    const uintptr_t d0 = reinterpret_cast<uintptr_t>(flat) + (uintptr_t)((u.flat_elem + lo) * esize);
    const uintptr_t d1 = d0 + (uintptr_t)(n * esize);
    const uintptr_t after = (uintptr_t)(((int64_t)u.count - lo - n + (u.more & 0xff)) * esize);
    const uintptr_t cf = (d0 + 15) & ~(uintptr_t)15;
    if (cf >= d1) return;                                // no chunk starts here
    int64_t nch = (int64_t)((d1 - cf + 15) >> 4);        // chunks starting in [d0, d1), <= 512
    if (cf + 16 * (uintptr_t)nch > d1 + after) --nch;    // the last holds the parameter's end
    const int tid = threadIdx.x;
    const int64_t k0 = tid, k1 = tid + kCopyThreads;
    const char *s = src + (cf - d0);
    u32x4 *dv = reinterpret_cast<u32x4 *>(cf);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (k0 < nch) a = ld_stream(s + 16 * k0);
    if (k1 < nch) b = ld_stream(s + 16 * k1);
    if (k0 < nch) __builtin_nontemporal_store(a, dv + k0);
    if (k1 < nch) __builtin_nontemporal_store(b, dv + k1);
}

// Unflatten's shared chunks for elements of `es` bytes: every 16-byte chunk
// of parameter storage that holds bytes of two or more bound parameters (a
// parameter's first or last chunk when it starts or ends off a 16-byte
// boundary).  Sets the parameters' shared-head and shared-tail flags and
// returns the chunks' edge entries grouped by bucket, with the start of
// each bucket's group in first[].
std::vector<ddp_unflatten_edge> unflatten_edges_for(const ddp_plan *plan, void *const *grads,
                                                    int64_t es, std::vector<uint8_t> &flags,
                                                    int shift, std::vector<int64_t> &first)
{
    const int32_t nb = plan->n_buckets();
    std::vector<int64_t> start((size_t)plan->n_params, 0);   // flat element of each parameter
    std::vector<int32_t> bucket_of((size_t)plan->n_params, -1);
    for (int32_t b = 0; b < nb; ++b) {
        int64_t flat = plan->bucket_base[b];
        for (int32_t sl = plan->bucket_first_slot[b]; sl < plan->bucket_first_slot[b + 1]; ++sl) {
            const int32_t q = plan->slot_param[sl];
            start[q] = flat;
            bucket_of[q] = b;
            flat += plan->numel[q];
        }
    }
    std::map<uint64_t, std::vector<int32_t>> chunks;   // partial chunk -> its parameters
    for (int32_t q = 0; q < plan->n_params; ++q) {
        if (plan->numel[q] == 0) continue;
        const uint64_t s0 = reinterpret_cast<uint64_t>(grads[q]), t = s0 + plan->numel[q] * es;
        if (s0 & 15) chunks[s0 & ~15ull].push_back(q);
        if ((t & 15) && (!(s0 & 15) || (t & ~15ull) != (s0 & ~15ull))) chunks[t & ~15ull].push_back(q);
    }
    std::vector<std::vector<ddp_unflatten_edge>> per((size_t)nb);
    for (const auto &kv : chunks) {
        if (kv.second.size() < 2) continue;
        const uint64_t c = kv.first;
        for (int32_t q : kv.second) {
            const uint64_t s0 = reinterpret_cast<uint64_t>(grads[q]), t = s0 + plan->numel[q] * es;
            if ((s0 & 15) && (s0 & ~15ull) == c) flags[q] |= (uint8_t)(1u << shift);
            if ((t & 15) && (t & ~15ull) == c) flags[q] |= (uint8_t)(2u << shift);
        }
        std::vector<int32_t> bs;
        for (int32_t q : kv.second)
            if (std::find(bs.begin(), bs.end(), bucket_of[q]) == bs.end()) bs.push_back(bucket_of[q]);
        for (int32_t b : bs) {
            ddp_unflatten_edge ed;
            ed.chunk = c;
            for (int k = 0; k < 8; ++k) {
                ed.piece[k] = -1;
                const uint64_t x = c + 2 * (uint64_t)k;
                for (int32_t q : kv.second) {
                    const uint64_t s0 = reinterpret_cast<uint64_t>(grads[q]);
                    if (bucket_of[q] == b && x >= s0 && x < s0 + plan->numel[q] * es)
                        ed.piece[k] = start[q] * es + (int64_t)(x - s0);
                }
            }
            per[b].push_back(ed);
        }
    }
    std::vector<ddp_unflatten_edge> all;
    first.assign((size_t)nb + 1, 0);
    for (int32_t b = 0; b < nb; ++b) {
        first[b] = (int64_t)all.size();
        all.insert(all.end(), per[b].begin(), per[b].end());
    }
    first[nb] = (int64_t)all.size();
    return all;
}

}  // namespace

extern "C" {

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
    std::vector<TensorStart> tfirst;   // each parameter's first unit and flat element
    std::vector<ddp_unflatten_edge> uedges[2];
    std::vector<uint8_t> pflags;       // per parameter: shared-chunk flags (unit `more` bits 8-11)
    try {
        pflags.assign((size_t)plan->n_params, 0);
        for (int k = 0; k < 2; ++k)
            uedges[k] = unflatten_edges_for(plan, param_grads, (int64_t)2 << k, pflags, 2 * k,
                                            bd->bucket_first_uedge[k]);
        bd->param_addr.resize((size_t)plan->n_params);
        for (int32_t p = 0; p < plan->n_params; ++p)
            bd->param_addr[p] = reinterpret_cast<uint64_t>(param_grads[p]);
        const int32_t nb = plan->n_buckets();
        bd->bucket_first_unit.resize((size_t)nb + 1);
        bd->bucket_first_tensor.resize((size_t)nb + 1);
        bd->bucket_edge_mask.assign((size_t)nb, 0);
        for (int32_t b = 0; b < nb; ++b) {
            bd->bucket_first_unit[b] = (int64_t)units.size();
            bd->bucket_first_tensor[b] = (int64_t)tfirst.size();
            int64_t flat = plan->bucket_base[b];
            for (int32_t s = plan->bucket_first_slot[b]; s < plan->bucket_first_slot[b + 1]; ++s) {
                const int32_t p = plan->slot_param[s];
                const int64_t n = plan->numel[p];
                if (n > 0) {
                    tfirst.push_back(TensorStart{(int64_t)units.size(), flat});
                    bd->bucket_edge_mask[b] |= (uint8_t)(1u << (flat & 7));
                }
                for (int64_t off = 0; off < n; off += kCopyUnitElems) {
                    ddp_copy_unit u;
                    u.param_addr = reinterpret_cast<uint64_t>(param_grads[p]);
                    u.param_elem = off;
                    u.flat_elem = flat + off;
                    u.count = (int32_t)std::min<int64_t>(kCopyUnitElems, n - off);
                    u.more = (int32_t)std::min<int64_t>(16, n - off - u.count) |
                             (int32_t)pflags[p] << 8;
                    units.push_back(u);
                }
                flat += n;
            }
            bd->bucket_edge_mask[b] |= (uint8_t)(1u << (flat & 7));   // the bucket's end
            bd->edge_mask |= bd->bucket_edge_mask[b];
        }
        bd->bucket_first_unit[nb] = (int64_t)units.size();
        bd->bucket_first_tensor[nb] = (int64_t)tfirst.size();
    } catch (...) {
        delete bd;
        return DDP_ERR_NOMEM;
    }
    bd->n_units = (int64_t)units.size();
    if (bd->n_units > 0) {
        // one allocation: the units, the parameters' starts, unflatten's
        // shared chunks for 2- and 4-byte elements
        const size_t ubytes = sizeof(ddp_copy_unit) * units.size();
        const size_t tbytes = sizeof(TensorStart) * tfirst.size();
        const size_t e0 = sizeof(ddp_unflatten_edge) * uedges[0].size();
        const size_t e1 = sizeof(ddp_unflatten_edge) * uedges[1].size();
        static_assert(sizeof(ddp_copy_unit) % alignof(TensorStart) == 0 &&
                          sizeof(TensorStart) % alignof(ddp_unflatten_edge) == 0,
                      "table alignment");
        if ((e = hipMalloc(&bd->units, ubytes + tbytes + e0 + e1)) != hipSuccess) {
            delete bd;
            return hip_fail("hipMalloc (copy units)", e, DDP_ERR_NOMEM);
        }
        char *base = reinterpret_cast<char *>(bd->units);
        bd->tensor_first = reinterpret_cast<int64_t *>(base + ubytes);
        bd->uedges[0] = reinterpret_cast<ddp_unflatten_edge *>(base + ubytes + tbytes);
        bd->uedges[1] = reinterpret_cast<ddp_unflatten_edge *>(base + ubytes + tbytes + e0);
        if ((e = hipMemcpy(bd->units, units.data(), ubytes, hipMemcpyHostToDevice)) != hipSuccess ||
            (e = hipMemcpy(bd->tensor_first, tfirst.data(), tbytes, hipMemcpyHostToDevice)) !=
                hipSuccess ||
            (e0 && (e = hipMemcpy(bd->uedges[0], uedges[0].data(), e0, hipMemcpyHostToDevice)) !=
                       hipSuccess) ||
            (e1 && (e = hipMemcpy(bd->uedges[1], uedges[1].data(), e1, hipMemcpyHostToDevice)) !=
                       hipSuccess)) {
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
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));
    // A launch takes at most max_launch_items() work-items, a multiple of
    // 4096, so cap (units per launch) is a multiple of kXcds; the run is
    // shortened where cap is below kXcds * kCopyRun, and every launch but the
    // last takes whole rounds of kXcds runs.
    const int esize = dtype_size(dtype), bpu = copy_blocks_per_unit(esize);
    const int64_t cap = max_launch_items() / (kCopyThreads * bpu);
    const int64_t run = std::min<int64_t>(kCopyRun, cap / kXcds);
    const int64_t round = kXcds * run, per = cap / round * round;
    char *fl = static_cast<char *>(flat);
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The edge work of the call.  Flatten: the chunks that hold a parameter
    // start or the range's end off a 16-byte boundary of this flat buffer.
    // Unflatten: the pieces of storage two parameters share.  It runs as
    // extra blocks after the last launch's copy blocks when they fit in the
    // launch, else as a launch of its own.
    const int32_t b0 = bucket < 0 ? 0 : bucket, b1 = bucket < 0 ? plan->n_buckets() : bucket + 1;
    FlatEdges fe{nullptr, 0, first, last, plan->bucket_base[b0], plan->bucket_base[b1], 0u};
    UnflatEdges ue{nullptr, 0, 0u};
    int64_t edge_lanes = 0;
    if (to_flat) {
        const unsigned mask = bucket < 0 ? bd->edge_mask : bd->bucket_edge_mask[bucket];
        bool edges = false;
        for (int k = 0; k < 8; ++k)
            if ((mask >> k & 1u) && ((reinterpret_cast<uintptr_t>(flat) + (uintptr_t)(k * esize)) & 15))
                edges = true;
        if (edges) {
            const int64_t t0 = bd->bucket_first_tensor[b0];
            fe.starts = reinterpret_cast<const TensorStart *>(bd->tensor_first) + t0;
            fe.nb = bd->bucket_first_tensor[b1] - t0;
            edge_lanes = 8 * (fe.nb + 1);   // 8 lanes per boundary; n_params < 2^31
        }
    } else {
        const int k = esize == 4 ? 1 : 0;
        const int64_t e0 = bd->bucket_first_uedge[k][b0];
        ue.edges = bd->uedges[k] + e0;
        ue.n = bd->bucket_first_uedge[k][b1] - e0;
        edge_lanes = 8 * ue.n;
    }
    const int64_t eblocks = (edge_lanes + kCopyThreads - 1) / kCopyThreads;
    bool edges_done = eblocks == 0;
    const unsigned lds = lds_for_blocks(kCopyBlocksPerCU);
    auto launch = [&](int64_t u0, int64_t n, const CopyMap &cm, unsigned bulk, unsigned extra) {
        const dim3 g(bulk + extra), b(kCopyThreads);
        fe.bulk_blocks = ue.bulk_blocks = bulk;
        if (to_flat && bpu == 1)
            flatten_units<1><<<g, b, lds, st>>>(bd->units, u0, n, cm, fl, esize, fe);
        else if (to_flat)
            flatten_units<2><<<g, b, lds, st>>>(bd->units, u0, n, cm, fl, esize, fe);
        else if (bpu == 1)
            unflatten_units<1><<<g, b, lds, st>>>(bd->units, u0, n, cm, fl, esize, ue);
        else
            unflatten_units<2><<<g, b, lds, st>>>(bd->units, u0, n, cm, fl, esize, ue);
        return launched("copy kernel launch");
    };
    for (int64_t u0 = first; u0 < last; u0 += per) {
        const int64_t n = std::min(per, last - u0);
        const int64_t whole = n / round, rest = n % round;
        const CopyMap cm{(unsigned)run, (unsigned)((rest + kXcds - 1) / kXcds), (unsigned)(whole * run)};
        const int64_t bulk = (whole * run + cm.last_run) * kXcds * bpu;
        int64_t extra = 0;
        if (u0 + per >= last && !edges_done && (bulk + eblocks) * kCopyThreads <= max_launch_items()) {
            extra = eblocks;
            edges_done = true;
        }
        const ddp_status_t s = launch(u0, n, cm, (unsigned)bulk, (unsigned)extra);
        if (s != DDP_OK) return s;
    }
    if (!edges_done) return launch(first, 0, CopyMap{(unsigned)run, 0u, 0u}, 0u, (unsigned)eblocks);
    return DDP_OK;
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

}  // extern "C"
