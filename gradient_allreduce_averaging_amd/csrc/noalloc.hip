// ddp_sync_allreduce_avg_noalloc: the whole synchronisation of a plan for
// callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc).
//
// Pages: [DDP] "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel);
//        [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn).
//
// A RING synchronisation reads three tables of the plan: the bucket bases,
// the coarse tile -> bucket table and the ring-segment word of every tile
// (device.h).  ddp_sync_allreduce_avg allocates them once per device and
// rank count; here they are rebuilt on every call, on the call's stream, in
// `scratch`, a fixed static device array:
//   1. the bucket bases travel as kernel arguments, kBasesPerLaunch per
//      launch, into the array;
//   2. one kernel writes every tile's word and every coarse-table entry from
//      the bases (ring_tile_word / bucket_holding, the functions the host
//      builds the plan's own tables with);
//   3. the reduce runs as ddp_sync_allreduce_avg's, reading the tables there.
// Every other case (SEQUENTIAL order, one rank, an empty plan, an output off
// a 16-byte boundary) reads no plan table, so it is ddp_sync_allreduce_avg's
// own path, which allocates nothing there.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>

#include "host.h"
#include "internal.h"

using namespace ddp_detail;

namespace {

constexpr int64_t kScratchBytes = DDP_NOALLOC_SCRATCH_BYTES;
constexpr int kScratchDevices = 64;

// One copy per device, held until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: kernels get the address
// hipGetSymbolAddress returns for the current device (scratch_on_device).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];

// The device address of `scratch` on the current device, looked up on the
// first call for that device.
ddp_status_t scratch_on_device(unsigned char **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kScratchDevices) return DDP_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail("hipGetSymbolAddress (scratch)", e);
        if (!p) return DDP_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<unsigned char *>(g_scratch_ptr[dev]);
    return DDP_OK;
}

constexpr int kBasesPerLaunch = 256;

// A batch of bucket bases, passed by value (2 KiB of kernel arguments).
struct BaseBatch {
    int64_t v[kBasesPerLaunch];
    int64_t first;   // index of v[0] in the base table
    int32_t n;       // entries used, 1..kBasesPerLaunch
};

__global__ void __launch_bounds__(kBasesPerLaunch) put_bases(BaseBatch batch, int64_t *base)
{
    const int i = threadIdx.x;
    if (i < batch.n) base[batch.first + i] = batch.v[i];
}

constexpr int kBuildThreads = 256;

// Thread t writes tile t's ring word (XCD-striped) and, for t < entries, the
// coarse table's entry t: the bucket holding element t * (tile << shift).
__global__ void __launch_bounds__(kBuildThreads)
build_ring_tables(const int64_t *base, int32_t nb, int64_t tile, int n_ranks, int64_t n_tiles,
                  int64_t stride, uint32_t *words, int32_t *tile_bucket, int64_t entries,
                  int64_t first_block)
{
    const int64_t t = (first_block + blockIdx.x) * kBuildThreads + threadIdx.x;
    if (t < n_tiles)
        words[(t % kXcds) * stride + t / kXcds] = ring_tile_word(base, nb, tile, n_ranks, t);
    if (t < entries) tile_bucket[t] = bucket_holding(base, nb, t * (tile << kTileTableShift));
}

int64_t round256(int64_t n) { return (n + 255) & ~(int64_t)255; }

}  // namespace

extern "C" {

ddp_status_t ddp_sync_allreduce_avg_noalloc(ddp_plan_t *plan, const void *const *rank_flat,
                                            int32_t n_ranks, ddp_order_t order,
                                            ddp_dtype_t out_dtype, void *out_flat, void *stream)
{
    if (!plan) return DDP_ERR_INVALID_ARG;
    const int in = plan->dtype;
    const int64_t total = plan->total;
    ddp_status_t stc = check_reduce(rank_flat, n_ranks, total, order, in, out_dtype, out_flat);
    if (stc != DDP_OK) return stc;
    if (order != DDP_ORDER_RING || n_ranks == 1 || total == 0 || !aligned(out_flat, 16))
        return ddp_sync_allreduce_avg(plan, rank_flat, n_ranks, order, out_dtype, out_flat,
                                      stream);

    // scratch layout: bases [nb + 1] int64 | coarse table [entries] int32 |
    // words [kXcds * stride] uint32, each part on a 256-byte boundary
    const int32_t nb = plan->n_buckets();
    const int64_t tile = tile_elems(in);
    const int64_t n_tiles = (total + tile - 1) / tile;
    const int64_t stride = word_stride(n_tiles);
    const int64_t entries = (total + (tile << kTileTableShift) - 1) / (tile << kTileTableShift);
    const int64_t off_tb = round256(8 * ((int64_t)nb + 1));
    const int64_t off_w = off_tb + round256(4 * entries);
    if (off_w + 4 * kXcds * stride > kScratchBytes) return DDP_ERR_CAPACITY;

    unsigned char *sp = nullptr;
    if ((stc = scratch_on_device(&sp)) != DDP_OK) return stc;
    int64_t *base = reinterpret_cast<int64_t *>(sp);
    int32_t *tile_bucket = reinterpret_cast<int32_t *>(sp + off_tb);
    uint32_t *words = reinterpret_cast<uint32_t *>(sp + off_w);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const OccupancyScope occ(plan->occupancy.load(std::memory_order_relaxed));

    BaseBatch batch;
    for (int64_t first = 0; first <= nb; first += kBasesPerLaunch) {
        std::memset(&batch, 0, sizeof(batch));
        batch.first = first;
        batch.n = (int32_t)std::min<int64_t>(kBasesPerLaunch, (int64_t)nb + 1 - first);
        std::memcpy(batch.v, plan->bucket_base.data() + first, sizeof(int64_t) * batch.n);
        put_bases<<<dim3(1), dim3(kBasesPerLaunch), 0, st>>>(batch, base);
        if ((stc = launched("bucket table launch")) != DDP_OK) return stc;
    }
    stc = launch_split((n_tiles + kBuildThreads - 1) / kBuildThreads, kBuildThreads,
                       "ring table launch", [&](int64_t b0, unsigned n) {
                           build_ring_tables<<<dim3(n), dim3(kBuildThreads), 0, st>>>(
                               base, nb, tile, n_ranks, n_tiles, stride, words, tile_bucket,
                               entries, b0);
                       });
    if (stc != DDP_OK) return stc;

    RankArgs ra;
    std::memset(&ra, 0, sizeof(ra));
    for (int r = 0; r < n_ranks; ++r) ra.p[r] = rank_flat[r];
    const Buckets bk = {base, tile_bucket, words, stride, 0, total, nb, 0};
    return launch_reduce(ra, n_ranks, total, order, in, out_dtype, bk, out_flat, st, true);
}

}  // extern "C"
