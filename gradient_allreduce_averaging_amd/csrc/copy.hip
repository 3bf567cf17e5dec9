// Flatten and unflatten: per-parameter gradients <-> flat bucket buffers
// (ddp_bind_params, ddp_flatten, ddp_unflatten).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <new>
#include <vector>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

// ---------------------------------------------------------------- copies

constexpr int64_t kCopyRun = 64;   // consecutive copy units per XCD (copy_units)

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

// BPU blocks per copy unit (copy_blocks_per_unit: 8 KiB a block), each
// moving its share of the unit (parts past a short unit's end return at
// once); to_flat selects flatten (param -> flat) or unflatten (flat ->
// param).  Workgroups are dealt to the XCDs round-robin (block b runs on
// XCD b % 8).  Each XCD takes runs of `run` consecutive units (units
// [(8k + x) run, (8k + x + 1) run) go to XCD x), and the blocks of one unit
// run on one XCD, where the unit's table entry is then an L2 hit for all
// but the first of them.  Consecutive units touch neighbouring bytes: where
// a parameter's flat offset is not a multiple of the 128-byte line, the
// line two units share is written whole by one XCD's L2 inside a run
// instead of in two partial writes from two L2s, which measured 2-3 %
// faster with many small unaligned parameters (runs of 64; runs of 256, or
// one contiguous span per XCD, measured slower on large ones).  Units hold
// 4K elements: with many short parameters, bigger units mostly spawn blocks
// that find no work.
template <int BPU>
__global__ void __launch_bounds__(kCopyThreads)
copy_units(const ddp_copy_unit *units, int64_t first, int64_t n_units, unsigned run, char *flat,
           int esize, int to_flat)
{
    constexpr int64_t kBlockElems = kCopyUnitElems / BPU;
    const unsigned m = blockIdx.x / kXcds, j = m / BPU;   // this XCD's j-th unit
    const int64_t ui = (int64_t)((j / run) * kXcds + blockIdx.x % kXcds) * run + j % run;
    if (ui >= n_units) return;
    const ddp_copy_unit u = units[first + ui];
    const int64_t lo = (m % BPU) * kBlockElems;
    if (lo >= u.count) return;
    const int64_t n = min(u.count - lo, kBlockElems);
    char *pp = reinterpret_cast<char *>(u.param_addr) + (u.param_elem + lo) * esize;
    char *fp = flat + (u.flat_elem + lo) * esize;
    const int64_t nbytes = n * esize;
    if (to_flat)
        block_copy(fp, pp, nbytes);
    else
        block_copy(pp, fp, nbytes);
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
        if (bpu == 1)
            copy_units<1><<<g, b, lds, st>>>(bd->units, u0, n, (unsigned)run, fl, esize, to_flat);
        else
            copy_units<2><<<g, b, lds, st>>>(bd->units, u0, n, (unsigned)run, fl, esize, to_flat);
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
