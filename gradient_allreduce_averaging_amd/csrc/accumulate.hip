// Local gradient accumulation between synchronisations (ddp_accumulate).
#include <hip/hip_runtime.h>

#include <cstring>

#include "host.h"

using namespace ddp_detail;

namespace {

// ---------------------------------------------------------------- accumulate
// Local accumulation between synchronisations ([DDP] 5.2, no_sync):
// dst[k] += src[k] for every buffer pair k (grid row k), one f32 add per
// element (bf16: widened, added, rounded to nearest even).  The buffers are
// read and written at whatever element alignment they have.
struct AccArgs {
    char *dst[DDP_MAX_RANKS];
    const char *src[DDP_MAX_RANKS];
};

template <int DT>
__device__ __forceinline__ void acc_elem(char *d, const char *s, int64_t i)
{
    store_elem<DT>(d, i, load_elem<DT>(d, i) + load_elem<DT>(s, i));
}

template <int DT>
__global__ void __launch_bounds__(kThreads) accumulate_vec(AccArgs a, int64_t len, int64_t first_block)
{
    constexpr int VEC = DT == kF32 ? 4 : 8;
    constexpr int ISZ = DT == kF32 ? 4 : 2;
    char *d = a.dst[blockIdx.y];
    const char *s = a.src[blockIdx.y];
    const int64_t i0 = ((first_block + blockIdx.x) * kThreads + threadIdx.x) * VEC;
    if (i0 + VEC <= len) {
        const u32x4 x = ld_stream(d + i0 * ISZ), y = ld_stream(s + i0 * ISZ);
        u32x4 o;
        if (DT == kF32) {
#pragma unroll
            for (int w = 0; w < 4; ++w) o[w] = __float_as_uint(__uint_as_float(x[w]) + __uint_as_float(y[w]));
        } else {
#pragma unroll
            for (int w = 0; w < 4; ++w)
                o[w] = bf16_rne(lane<kBF16>(x, 2 * w) + lane<kBF16>(y, 2 * w)) |
                       (bf16_rne(lane<kBF16>(x, 2 * w + 1) + lane<kBF16>(y, 2 * w + 1)) << 16);
        }
        st_stream(d + i0 * ISZ, o);
    } else {
        for (int64_t i = i0; i < len && i < i0 + VEC; ++i) acc_elem<DT>(d, s, i);
    }
}

}  // namespace

extern "C" {

ddp_status_t ddp_accumulate(void *const *dst, const void *const *src, int32_t n_bufs, int64_t len,
                            ddp_dtype_t dtype, void *stream)
{
    if (n_bufs < 1 || len < 0 || !dtype_ok(dtype)) return DDP_ERR_INVALID_ARG;
    if (n_bufs > DDP_MAX_RANKS) return DDP_ERR_UNSUPPORTED;
    if (len > INT64_MAX / 4) return DDP_ERR_OVERFLOW;
    if (len == 0) return DDP_OK;
    if (!dst || !src) return DDP_ERR_INVALID_ARG;
    const int esz = dtype_size(dtype);
    const int64_t nbytes = len * esz;
    AccArgs a;
    std::memset(&a, 0, sizeof(a));
    for (int k = 0; k < n_bufs; ++k) {
        if (!dst[k] || !src[k] || !aligned(dst[k], esz) || !aligned(src[k], esz))
            return DDP_ERR_INVALID_ARG;
        const uintptr_t dk = reinterpret_cast<uintptr_t>(dst[k]);
        for (int j = 0; j < n_bufs; ++j) {
            const uintptr_t sj = reinterpret_cast<uintptr_t>(src[j]);
            // a destination may be exactly its own source; it may overlap nothing else
            if (!(j == k && sj == dk) && overlaps(dk, nbytes, sj, nbytes)) return DDP_ERR_ALIAS;
            if (j != k && overlaps(dk, nbytes, reinterpret_cast<uintptr_t>(dst[j]), nbytes))
                return DDP_ERR_ALIAS;
        }
        a.dst[k] = static_cast<char *>(dst[k]);
        a.src[k] = static_cast<const char *>(src[k]);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int64_t per = (int64_t)kThreads * vec_elems(dtype);
    const dim3 b(kThreads);
    return launch_split((len + per - 1) / per, kThreads, "accumulate kernel launch",
                        [&](int64_t b0, unsigned n) {
                            const dim3 g(n, (unsigned)n_bufs);
                            if (dtype == DDP_F32)
                                accumulate_vec<kF32><<<g, b, 0, st>>>(a, len, b0);
                            else
                                accumulate_vec<kBF16><<<g, b, 0, st>>>(a, len, b0);
                        });
}

}  // extern "C"
