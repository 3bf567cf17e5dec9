// Host-side helpers shared by libddp's launch code: error recording, dtype
// sizes, alias checks and the occupancy caps of the streaming kernels.  Not
// part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

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

// Resident blocks per CU each kernel family is capped at (0: no cap), and
// the dynamic-LDS request that imposes a cap of k (see common.hip).
int reduce_blocks_per_cu(int N, bool ring);
int sgd_blocks_per_cu(int N, bool mom);
constexpr int kCopyBlocksPerCU = 7;   // flatten / unflatten (256-thread blocks)
unsigned lds_for_blocks(int k);

}  // namespace ddp_detail
