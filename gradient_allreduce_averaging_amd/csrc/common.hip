// Host-side helpers shared by libddp's launch code (declared in host.h),
// and the entry points for the occupancy policy and error text.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>

#include "host.h"

namespace ddp_detail {

thread_local char g_last_error[256] = "";

ddp_status_t hip_fail(const char *what, hipError_t e, ddp_status_t st)
{
    snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return st;
}

ddp_status_t launched(const char *what)
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? DDP_OK : hip_fail(what, e);
}

int64_t max_launch_items()
{
    static const int64_t items = [] {
        int64_t v = int64_t(1) << 30;
        if (const char *e = std::getenv("DDP_MAX_LAUNCH_ITEMS")) {
            char *end = nullptr;
            const long long x = std::strtoll(e, &end, 10);
            if (end != e && x > 0 && x < v) v = x < 4096 ? 4096 : x;
        }
        return v / 4096 * 4096;
    }();
    return items;
}

// ---------------------------------------------------------------- occupancy
// These streaming kernels move the most bytes per second on gfx950 with fewer
// resident blocks per CU than registers alone would allow (up to 32 of these
// one-wave blocks): past a point, more concurrent waves only open more DRAM
// rows at once.  Each launch is therefore capped at k resident blocks per CU
// by asking for LDS_per_CU / k bytes of dynamic LDS, which the kernels do not
// touch.  k was measured per kernel and rank count on ResNet-50, many-small,
// GPT-1.3B and Llama-7B shapes; 0 means no cap.

// Reduce, N = 2..16 (one 16-byte load per rank and lane, one store): for
// N = 9..12, 7 (8 for sequential order at N = 9, 10), and 6 for 13..16
// (ResNet-50 plan, swept 4-12); the looped kernel for N > 16.
int reduce_blocks_per_cu(int N, bool ring)
{
    static const int k[9] = {0, 0, 0, 16, 14, 12, 10, 9, 8};
    if (N < 0) return 0;
    if (N <= 8) return k[N];
    if (N <= 10) return ring ? 7 : 8;
    if (N <= 12) return 7;
    return N <= 16 ? 6 : 8;
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

// The per-parameter sync (params.hip): the reduce's pattern behind one
// table entry per block, whose scalar-load latency more resident blocks
// hide.  Measured at N = 4 (many-small: 16) and N = 8 (ResNet-50 and
// GPT-1.3B in f32, Llama-7B in bf16: 10); other N take the cap of the flat
// kernel of the same shape (unrolled up to 8, looped above) plus two.
int params_blocks_per_cu(int N, bool ring)
{
    if (N == 4) return 16;
    if (N == 8) return 10;
    if (N > 8) return N <= 11 ? (ring ? 14 : 12) : 10;   // the looped kernel's caps + 2
    const int k = reduce_blocks_per_cu(N, ring);
    return k > 0 ? std::min(k + 2, 16) : 0;
}

// The per-parameter fused SGD step: the flat step's caps, except with
// momentum at N = 4 (many-small: 10 gave 6.50 TB/s against 6.33 at the flat
// step's 8) and N = 8 (ResNet-50: 7 gave 6.36 against 6.31 at 6, GPT-1.3B
// level; fresh processes, two rounds).
int params_sgd_blocks_per_cu(int N, bool mom)
{
    if (N == 4 && mom) return 10;
    if (N == 8 && mom) return 7;
    return sgd_blocks_per_cu(N, mom);
}

constexpr int kMaxDevices = 64;

// DDP_OCCUPANCY_TUNED or DDP_OCCUPANCY_SHARED, process-wide: the policy of
// calls made without an object that has its own.
std::atomic<int> g_occupancy{DDP_OCCUPANCY_TUNED};

// The policy of the object (plan or per-parameter sync) whose entry point
// this thread is in, or -1.
thread_local int tl_occupancy = -1;

OccupancyScope::OccupancyScope(int policy) : prev_(tl_occupancy)
{
    if (policy == DDP_OCCUPANCY_TUNED || policy == DDP_OCCUPANCY_SHARED) tl_occupancy = policy;
}

OccupancyScope::~OccupancyScope() { tl_occupancy = prev_; }

int current_occupancy()
{
    return tl_occupancy >= 0 ? tl_occupancy : g_occupancy.load(std::memory_order_relaxed);
}

// Dynamic LDS bytes that leave room for k blocks per CU on the current device
// (none under DDP_OCCUPANCY_SHARED).
unsigned lds_for_blocks(int k)
{
    static std::atomic<int> lds_per_cu[kMaxDevices];   // 0: not queried yet, -1: unknown
    if (k <= 0 || current_occupancy() != DDP_OCCUPANCY_TUNED) return 0;
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

}  // namespace ddp_detail

using namespace ddp_detail;

extern "C" {

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

const char *ddp_last_error(void) { return g_last_error; }

}  // extern "C"
