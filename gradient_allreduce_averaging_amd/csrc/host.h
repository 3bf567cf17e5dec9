// Host-side helpers shared by libddp's launch code: error recording, dtype
// sizes, alias checks and the occupancy caps of the streaming kernels.  Not
// part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "ddp.h"
#include "device.h"

namespace ddp_detail {

// Records a failed HIP call for ddp_last_error() and maps it to a status.
ddp_status_t hip_fail(const char *what, hipError_t e, ddp_status_t st = DDP_ERR_HIP);

// The status of the last launch (hipGetLastError).
ddp_status_t launched(const char *what);

inline int dtype_size(int dt) { return dt == DDP_BF16 ? 2 : 4; }
inline bool dtype_ok(int dt) { return dt == DDP_F32 || dt == DDP_BF16; }
inline bool pair_ok(int in, int out)
{
    return (in == DDP_F32 && out == DDP_F32) || (in == DDP_BF16 && out == DDP_BF16) ||
           (in == DDP_F32 && out == DDP_BF16);
}
inline int64_t vec_elems(int in) { return in == DDP_F32 ? 4 : 8; }
inline int64_t tile_elems(int in) { return (int64_t)kThreads * kUnroll * vec_elems(in); }
inline bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
inline bool overlaps(uintptr_t a, int64_t na, uintptr_t b, int64_t nb)
{
    return a < b + (uintptr_t)nb && b < a + (uintptr_t)na;
}

// out may be exactly one of the n inputs (len elements of isz bytes each,
// out osz bytes each) and may overlap none of them otherwise.
ddp_status_t check_alias(const void *const *in, int n, int64_t len, int isz, const void *out,
                         int osz);

// The most work-items one launch is given (a dispatch packet counts its grid
// in 32-bit work-items): 2^30, or DDP_MAX_LAUNCH_ITEMS from the environment
// when that is smaller (rounded down to a multiple of 4096, at least 4096).
// A larger grid runs as several launches on the same stream, each told the
// grid-wide index of its first block.
int64_t max_launch_items();

// Launches a grid of `blocks` blocks of `threads` threads as consecutive
// launches of at most max_launch_items() work-items: launch(first_block, n)
// enqueues blocks [first_block, first_block + n).
template <class Launch>
ddp_status_t launch_split(int64_t blocks, int threads, const char *what, Launch &&launch)
{
    const int64_t per = max_launch_items() / threads;
    for (int64_t b0 = 0; b0 < blocks; b0 += per) {
        launch(b0, (unsigned)(blocks - b0 < per ? blocks - b0 : per));
        const ddp_status_t st = launched(what);
        if (st != DDP_OK) return st;
    }
    return DDP_OK;
}

// Calls f(std::integral_constant<int, K>()) for the K in [Lo, Hi] equal to
// n, so that a kernel templated on the rank count can be launched for a
// count known only at run time; false when n is outside [Lo, Hi].
template <int Lo, int Hi, class F>
bool with_rank_count(int n, F &&f)
{
    if constexpr (Lo > Hi) {
        (void)n;
        (void)f;
        return false;
    } else {
        if (n == Lo) {
            f(std::integral_constant<int, Lo>());
            return true;
        }
        return with_rank_count<Lo + 1, Hi>(n, f);
    }
}

// reduce.hip: the validation every reduce entry point shares (the output
// may be null only when out_optional is set), the N == 1 copy, and the
// reduce launch over the buckets bk (vec_ok: the vector kernels, else one
// element per thread; the bits are the same, the callers choose by output
// alignment and bucket length).
ddp_status_t check_reduce(const void *const *ptrs, int32_t n, int64_t len, int order, int in,
                          int out_dt, const void *out, bool out_optional = false);
ddp_status_t copy_single(const void *in, int64_t len, int esize, void *out, hipStream_t st);
ddp_status_t launch_reduce(const RankArgs &ra, int N, int64_t total, int order, int in, int out_dt,
                           const Buckets &bk, void *out, hipStream_t st, bool vec_ok);

// Resident blocks per CU each kernel family is capped at (0: no cap), and
// the dynamic-LDS request that imposes a cap of k (see common.hip).
int reduce_blocks_per_cu(int N, bool ring);
int sgd_blocks_per_cu(int N, bool mom);
int params_blocks_per_cu(int N, bool ring);
int params_sgd_blocks_per_cu(int N, bool mom);
constexpr int kCopyBlocksPerCU = 7;   // flatten / unflatten (256-thread blocks)
unsigned lds_for_blocks(int k);

// The occupancy policy of the launches made while it lives on this thread:
// an object's own (DDP_OCCUPANCY_TUNED or _SHARED), or, for
// DDP_OCCUPANCY_DEFAULT, the process-wide one.  Entry points that take a
// plan or a per-parameter sync open one with that object's policy.
class OccupancyScope {
public:
    explicit OccupancyScope(int policy);
    ~OccupancyScope();
    OccupancyScope(const OccupancyScope &) = delete;
    OccupancyScope &operator=(const OccupancyScope &) = delete;

private:
    int prev_;
};
int current_occupancy();

}  // namespace ddp_detail
