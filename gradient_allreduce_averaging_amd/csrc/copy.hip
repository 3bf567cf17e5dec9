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
#include <new>
#include <vector>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

// ---------------------------------------------------------------- copies

constexpr int64_t kCopyRun = 64;   // consecutive copy units per XCD (unit_of_block)

__device__ __forceinline__ void copy16b(char *dst, const char *src, int64_t lo, int64_t hi)
{
    for (int64_t j = lo + 2 * (int64_t)threadIdx.x; j < hi; j += 2 * kCopyThreads)
        *reinterpret_cast<uint16_t *>(dst + j) = *reinterpret_cast<const uint16_t *>(src + j);
}

// Block-wide copy of nbytes (a multiple of 2, at most kCopyBlockBytes)
// between 2-byte aligned addresses: 16-byte non-temporal accesses from the
// destination's first 16-byte boundary, at most two per thread, a thread's
// loads before its stores.  The loads run at whatever alignment the source
// has (gfx9 and later global loads take any address), so a tensor whose flat
// offset is not a multiple of 16 bytes still moves in 16-byte vectors; a head
// and tail of under 16 bytes move 2 bytes per thread.  A piece with neither
// (every piece of a 16-byte aligned tensor) takes a straight-line path; on
// the others the head goes first, which measured faster there than issuing
// the vector loads before it.
static_assert(kCopyBlockBytes == 2 * 16 * kCopyThreads, "two vectors per thread cover a block");
__device__ void block_copy(char *dst, const char *src, int64_t nbytes)
{
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst);
    const int tid = threadIdx.x;
    const int64_t head = min<int64_t>((16 - (d & 15)) & 15, nbytes);
    const int64_t nvec = (nbytes - head) >> 4;   // at most 2 * kCopyThreads
    const char *sv = src + head;
    u32x4 *dv = reinterpret_cast<u32x4 *>(dst + head);
    if (head == 0 && (nbytes & 15) == 0) {
        const int64_t j0 = tid, j1 = tid + kCopyThreads;
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (j0 < nvec) a = ld_stream(sv + 16 * j0);
        if (j1 < nvec) b = ld_stream(sv + 16 * j1);
        if (j0 < nvec) __builtin_nontemporal_store(a, dv + j0);
        if (j1 < nvec) __builtin_nontemporal_store(b, dv + j1);
        return;
    }
    copy16b(dst, src, 0, head);
    int64_t j = tid;
    for (; j + kCopyThreads < nvec; j += 2 * kCopyThreads) {
        const u32x4 a = ld_stream(sv + 16 * j);
        const u32x4 b = ld_stream(sv + 16 * (j + kCopyThreads));
        __builtin_nontemporal_store(a, dv + j);
        __builtin_nontemporal_store(b, dv + j + kCopyThreads);
    }
    for (; j < nvec; j += kCopyThreads) __builtin_nontemporal_store(ld_stream(sv + 16 * j), dv + j);
    copy16b(dst, src, head + (nvec << 4), nbytes);
}

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
// one contiguous span per XCD, measured slower on large ones).  Units hold
// 4K elements: with many short parameters, bigger units mostly spawn blocks
// that find no work.
template <int BPU>
__device__ __forceinline__ int64_t unit_of_block(unsigned run, int64_t *lo)
{
    constexpr int64_t kBlockElems = kCopyUnitElems / BPU;
    const unsigned m = blockIdx.x / kXcds, j = m / BPU;   // this XCD's j-th unit
    *lo = (m % BPU) * kBlockElems;
    return (int64_t)((j / run) * kXcds + blockIdx.x % kXcds) * run + j % run;
}

// Unflatten (flat -> param): each block copies its part of a unit into the
// parameter.  A parameter's storage usually starts on the allocator's
// alignment, so its pieces, all but its last, start and end on a 16-byte
// boundary and no two blocks share a chunk; block_copy takes any 2-byte
// alignment all the same.
template <int BPU>
__global__ void __launch_bounds__(kCopyThreads)
unflatten_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, unsigned run,
                const char *flat, int esize)
{
    int64_t lo;
    const int64_t ui = unit_of_block<BPU>(run, &lo);
    if (ui >= n_units) return;
    const ddp_copy_unit u = units[first + ui];
    if (lo >= u.count) return;
    const int64_t n = min(u.count - lo, kCopyUnitElems / BPU);
    block_copy(reinterpret_cast<char *>(u.param_addr) + (u.param_elem + lo) * esize,
               flat + (u.flat_elem + lo) * esize, n * esize);
}

// Loads through a generic pointer compile to flat instructions, which the
// scalar-load counter also tracks, so a wait for a scalar load would wait
// for them too; these take the global address space.
__device__ __forceinline__ u32x4 ld_stream_global(const char *p)
{
    typedef __attribute__((address_space(1))) const u32x4_ua gvec;
    return __builtin_nontemporal_load(reinterpret_cast<gvec *>(reinterpret_cast<uintptr_t>(p)));
}
__device__ __forceinline__ uint16_t ld_u16_global(const char *p)
{
    typedef __attribute__((address_space(1))) const uint16_t g16;
    return *reinterpret_cast<g16 *>(reinterpret_cast<uintptr_t>(p));
}

// A unit's flat bytes [beg, end) and the source address of beg.
struct UnitSpan {
    uintptr_t beg, end;
    const char *src;
};

__device__ __forceinline__ UnitSpan unit_span(const ddp_copy_unit &u, uintptr_t flat, int esize)
{
    const uintptr_t beg = flat + (uintptr_t)(u.flat_elem * esize);
    return {beg, beg + (uintptr_t)(u.count * esize),
            reinterpret_cast<const char *>(u.param_addr) + u.param_elem * esize};
}

// Source of flat byte x >= d1 (past the block's own bytes): in unit v0
// (cur), the unit after it (nxt, loaded with the block's own entry), or --
// where units are shorter than a chunk -- one further on, walked to up to
// range_end; null past the range's last unit.
__device__ const char *source_past(const ddp_copy_unit *units, int64_t v0, int64_t range_end,
                                   UnitSpan cur, UnitSpan nxt, uintptr_t flat, int esize,
                                   uintptr_t x)
{
    if (x < cur.end) return cur.src + (x - cur.beg);
    if (v0 + 1 >= range_end) return nullptr;
    if (x < nxt.end) return nxt.src + (x - nxt.beg);
    for (int64_t w = v0 + 2; w < range_end; ++w) {
        const UnitSpan sp = unit_span(units[w], flat, esize);
        if (x < sp.end) return sp.src + (x - sp.beg);
    }
    return nullptr;
}

// Flatten (param -> flat) with one writer per 16-byte chunk of the flat
// buffer.  Parameters sit in the flat buffer at any element offset, so a
// chunk often holds the end of one piece and the start of the next.  The
// block whose flat bytes [d0, d1) hold a chunk's first byte writes the whole
// chunk; the call's first block also writes the chunk holding the range's
// first byte.  Chunks inside [d0, d1) take one vector load from the source
// at its own alignment (any address) and an aligned store.  A chunk at an
// edge (the head chunk, and the one that runs past d1) is written by 8
// lanes, 2 bytes each, in one store instruction: bytes in [d0, d1) come
// from this block's source, bytes from d1 on from the unit that holds them,
// none before d0 (the head of a call's range) or past the range's last
// unit.  The next unit's entry is loaded with the block's own, and the
// edge lanes' loads go out with the vector loads, so a block makes one
// round trip to memory.  Bytes before a block's first chunk are left to the
// block before it.  Written in 2-byte pieces by two blocks each, as an
// earlier version did, such chunks cost many small unaligned parameters 3 %
// of their bandwidth.  A block with no edge chunk (every block of a tensor
// whose flat offset is a multiple of 16 bytes) takes a straight-line path:
// the edge bookkeeping ahead of its loads cost such tensors 5 %.
template <int BPU>
__global__ void __launch_bounds__(kCopyThreads)
flatten_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, unsigned run,
              int64_t range_first, int64_t range_end, char *flat, int esize)
{
    int64_t lo;
    const int64_t ui = unit_of_block<BPU>(run, &lo);
    if (ui >= n_units) return;
    const int64_t v0 = first + ui;
    const ddp_copy_unit u = units[v0];
    const ddp_copy_unit un = units[min(v0 + 1, range_end - 1)];
    // both entries arrive together, before any data load is in flight
    asm volatile("" ::"s"(un.param_addr), "s"(un.param_elem), "s"(un.flat_elem), "s"(un.count));
    if (lo >= u.count) return;
    const int64_t n = min(u.count - lo, kCopyUnitElems / BPU);
    const char *src = reinterpret_cast<const char *>(u.param_addr) + (u.param_elem + lo) * esize;
    const uintptr_t fb = reinterpret_cast<uintptr_t>(flat);
    const uintptr_t d0 = fb + (uintptr_t)((u.flat_elem + lo) * esize);
    const uintptr_t d1 = d0 + (uintptr_t)(n * esize);
    const bool head = v0 == range_first && lo == 0 && (d0 & 15);
    const uintptr_t cf = head ? (d0 & ~(uintptr_t)15) : ((d0 + 15) & ~(uintptr_t)15);
    if (cf >= d1) return;                                // no chunk starts here
    const int64_t nch = (int64_t)((d1 - cf + 15) >> 4);  // chunks [cf, cf + 16 nch), <= 513
    const bool spill = (d1 & 15) != 0;                   // the last chunk runs past d1
    const int64_t kb = head ? 1 : 0, ke = spill ? nch - 1 : nch;   // whole chunks [kb, ke)
    const int tid = threadIdx.x;
    if (((d0 | d1) & 15) == 0) {   // [d0, d1) is whole chunks: cf = d0, kb = 0, ke = nch
        const int64_t k0 = tid, k1 = tid + kCopyThreads;
        u32x4 *dv = reinterpret_cast<u32x4 *>(d0);
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (k0 < ke) a = ld_stream(src + 16 * k0);
        if (k1 < ke) b = ld_stream(src + 16 * k1);
        if (k0 < ke) __builtin_nontemporal_store(a, dv + k0);
        if (k1 < ke) __builtin_nontemporal_store(b, dv + k1);
        return;
    }
    // edge lanes: 0-7 the head chunk, the last 8 the chunk past d1 (unless
    // it is the head chunk too); their sources first, so that their loads
    // go out with the vector loads
    const int e = tid - (kCopyThreads - 8);
    uintptr_t x = 0;
    if (head && tid < 8) x = cf + 2 * (uintptr_t)tid;
    else if (spill && (nch > 1 || !head) && e >= 0) x = cf + 16 * (uintptr_t)(nch - 1) + 2 * e;
    const char *ps = nullptr;
    if (x >= d0 && x < d1)
        ps = src + (x - d0);
    else if (x >= d1)
        ps = source_past(units, v0, range_end, unit_span(u, fb, esize), unit_span(un, fb, esize),
                         fb, esize, x);
    const int64_t k0 = kb + tid, k1 = kb + tid + kCopyThreads;     // ke - kb <= 512
    // Lanes past the last whole chunk load it again (their loads merge with
    // its own), so both loads go out unconditionally and no lane waits for
    // one before the other is issued; only the stores are predicated.
    const int64_t klast = max(ke - 1, kb);
    u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
    if (ke > kb) {
        a = ld_stream_global(src + (cf + 16 * (uintptr_t)min(k0, klast) - d0));
        b = ld_stream_global(src + (cf + 16 * (uintptr_t)min(k1, klast) - d0));
    }
    uint16_t piece = 0;
    if (ps) piece = ld_u16_global(ps);
    u32x4 *cv = reinterpret_cast<u32x4 *>(cf);
    if (k0 < ke) __builtin_nontemporal_store(a, cv + k0);
    if (k1 < ke) __builtin_nontemporal_store(b, cv + k1);
    if (ps) *reinterpret_cast<uint16_t *>(x) = piece;
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
    try {
        bd->param_addr.resize((size_t)plan->n_params);
        for (int32_t p = 0; p < plan->n_params; ++p)
            bd->param_addr[p] = reinterpret_cast<uint64_t>(param_grads[p]);
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
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));
    // Every XCD gets the same number of runs (the last round of kXcds runs
    // padded).  A launch takes at most max_launch_items() work-items, a
    // multiple of 4096, so cap (units per launch) is a multiple of kXcds; the
    // run is shortened where cap is below kXcds * kCopyRun, and a launch
    // takes whole rounds.
    const int esize = dtype_size(dtype), bpu = copy_blocks_per_unit(esize);
    const int64_t cap = max_launch_items() / (kCopyThreads * bpu);
    const int64_t run = std::min<int64_t>(kCopyRun, cap / kXcds);
    const int64_t round = kXcds * run, per = cap / round * round;
    for (int64_t u0 = first; u0 < last; u0 += per) {
        const int64_t n = std::min(per, last - u0);
        const dim3 g((unsigned)((n + round - 1) / round * round * bpu)), b(kCopyThreads);
        const unsigned lds = lds_for_blocks(kCopyBlocksPerCU);
        char *fl = static_cast<char *>(flat);
        hipStream_t st = static_cast<hipStream_t>(stream);
        const unsigned r = (unsigned)run;
        if (to_flat && bpu == 1)
            flatten_units<1><<<g, b, lds, st>>>(bd->units, u0, n, r, first, last, fl, esize);
        else if (to_flat)
            flatten_units<2><<<g, b, lds, st>>>(bd->units, u0, n, r, first, last, fl, esize);
        else if (bpu == 1)
            unflatten_units<1><<<g, b, lds, st>>>(bd->units, u0, n, r, fl, esize);
        else
            unflatten_units<2><<<g, b, lds, st>>>(bd->units, u0, n, r, fl, esize);
        const ddp_status_t s = launched("copy kernel launch");
        if (s != DDP_OK) return s;
    }
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
