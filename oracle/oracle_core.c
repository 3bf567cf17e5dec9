/*
 * CPU ORACLE -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct C for the arithmetic of bucketed gradient
 * all-reduce averaging.  Only the tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this file's library; the product path never does.
 * It shares no code, header or table with the HIP library.
 *
 * Pages cited (title, section):
 *   [DDP]  "DDP" (sgdbs.github.io, AI_Infra/1.DataParallel)
 *   [TR24] "(24) NCCL通信与分布式数据并行" (tech-renaissance.cn)
 *
 * What is computed, per element i of a bucket of length L held by N ranks:
 *
 *   SEQUENTIAL  acc = +0.0f; for r = 0..N-1: acc = fl(acc + x_r[i])
 *               -- the sum-then-divide pseudocode of [TR24] section 一
 *               (grad_sync starts as zeros_like, ranks added in index order).
 *   RING        chunk length C = ceil(L/N), chunk c = floor(i/C),
 *               start rank s = (c+1) mod N;
 *               acc = x_s[i]; for k = 1..N-1: acc = fl(acc + x_{(s+k) mod N}[i])
 *               -- the reduce-scatter phase of [DDP] section 2.10/2.11 with
 *               round t sending chunk (i-t) mod N, rounds counted from 1, so
 *               the chunk's partial sum starts at the rank after its owner.
 *   scale       y = fl(acc * fl(1.0f/N))  -- [TR24] section 九 (inv = 1/N,
 *               dst *= inv after the sum), [DDP] section 4.2 (div by world size).
 *   output      float32 y, or bf16 = y rounded to nearest, ties to even.
 *   N == 1      output = input, bit for bit ([TR24] section 九 returns early
 *               when world_size <= 1).
 *   SGD step    (the optimizer update the average can be folded into, [TR24]
 *               section 九 note; update rule theta <- theta - eta * g of [DDP]
 *               section 5.3):  with momentum buffer m (optional):
 *                   v = fl(fl(mu * m) + g);  m = v;  g = v
 *               then  p = fl(p - fl(lr * g)),  where g is the averaged
 *               gradient exactly as stored (bf16 widened back to f32).
 *   accumulate  local gradient accumulation between synchronisations ([DDP]
 *               section 5.2, no_sync: backward adds into .grad):
 *               dst = fl(dst + src), f32; for bf16 both widened, one f32 add,
 *               one round to nearest even.
 *
 * Built with -O2 -ffp-contract=off and no fast-math flag: every addition and
 * multiplication is one IEEE-754 binary32 operation (SSE on x86-64), denormals
 * are kept, no FMA is formed.
 */
#include <stdint.h>
#include <string.h>

#define ORACLE_SEQ 0
#define ORACLE_RING 1
#define ORACLE_F32 0
#define ORACLE_BF16 1

static float bits_to_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f32_to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> f32 is exact: the bf16 pattern is the top half of an f32 pattern. */
static float widen_bf16(uint16_t h) { return bits_to_f32((uint32_t)h << 16); }

/* Round an f32 to the nearest bf16, ties to even.  NaN stays a NaN with its
 * sign (quiet bit set); +-Inf and +-0 map to themselves; overflow past the
 * largest finite bf16 rounds to Inf, as round-to-nearest requires. */
uint16_t oracle_rne_bf16(float y)
{
    uint32_t u = f32_to_bits(y);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u)           /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xFFFFu;                   /* the 16 bits dropped */
    uint32_t upper = u >> 16;                       /* truncated bf16 */
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;                                /* carries into the exponent correctly */
    return (uint16_t)upper;
}

void oracle_rne_bf16_array(const float *y, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_rne_bf16(y[i]);
}

static float load_elem(const void *base, int dtype, int64_t i)
{
    if (dtype == ORACLE_BF16) return widen_bf16(((const uint16_t *)base)[i]);
    return ((const float *)base)[i];
}

/* Start rank of the ring order for position pos of a bucket of length len. */
static int ring_start_rank(int64_t pos, int64_t len, int N)
{
    int64_t C = (len + N - 1) / N;
    int64_t c = pos / C;
    return (int)((c + 1) % N);
}

/* The fixed-order FP32 fold of one element; v[r] is rank r's value. */
static float fold(const float *v, int N, int order, int64_t pos, int64_t len)
{
    float acc;
    if (order == ORACLE_SEQ) {
        acc = 0.0f;
        for (int r = 0; r < N; ++r) acc = acc + v[r];
    } else {
        int s = ring_start_rank(pos, len, N);
        acc = v[s];
        for (int k = 1; k < N; ++k) acc = acc + v[(s + k) % N];
    }
    return acc;
}

static void store_elem(void *out, int dtype, int64_t i, float y)
{
    if (dtype == ORACLE_BF16) ((uint16_t *)out)[i] = oracle_rne_bf16(y);
    else ((float *)out)[i] = y;
}

static int check_args(int N, int order, int in_dtype, int out_dtype)
{
    if (N < 1 || N > 1024) return -1;
    if (order != ORACLE_SEQ && order != ORACLE_RING) return -1;
    if (in_dtype != ORACLE_F32 && in_dtype != ORACLE_BF16) return -1;
    if (out_dtype != ORACLE_F32 && out_dtype != ORACLE_BF16) return -1;
    return 0;
}

/* Average one bucket.  x[r] points at rank r's copy of the bucket (len
 * elements of in_dtype); out receives len elements of out_dtype. */
int oracle_bucket_avg(const void *const *x, int N, int64_t len, int order,
                      int in_dtype, int out_dtype, void *out)
{
    if (check_args(N, order, in_dtype, out_dtype) || len < 0) return -1;
    if (N == 1) {
        if (in_dtype != out_dtype) return -1;
        memcpy(out, x[0], (size_t)len * (in_dtype == ORACLE_BF16 ? 2u : 4u));
        return 0;
    }
    const float inv = 1.0f / (float)N;
    float v[1024];
    for (int64_t i = 0; i < len; ++i) {
        for (int r = 0; r < N; ++r) v[r] = load_elem(x[r], in_dtype, i);
        float acc = fold(v, N, order, i, len);
        store_elem(out, out_dtype, i, acc * inv);
    }
    return 0;
}

/* Average the piece [lo, lo + n) of a bucket of length len, for checking a
 * bucket too large to hold on the host in one piece.  x[r] points at rank
 * r's element lo (n elements of in_dtype); out receives n elements of
 * out_dtype.  Every element is folded exactly as in oracle_bucket_avg, with
 * its position lo + k in the whole bucket choosing its ring start, so the
 * pieces of a bucket together give oracle_bucket_avg's result. */
int oracle_bucket_range_avg(const void *const *x, int N, int64_t len, int64_t lo, int64_t n,
                            int order, int in_dtype, int out_dtype, void *out)
{
    if (check_args(N, order, in_dtype, out_dtype)) return -1;
    if (len < 0 || lo < 0 || n < 0 || lo > len || n > len - lo) return -1;
    if (N == 1) {   /* the input, bit for bit */
        if (in_dtype != out_dtype) return -1;
        memcpy(out, x[0], (size_t)n * (in_dtype == ORACLE_BF16 ? 2u : 4u));
        return 0;
    }
    const float scale = 1.0f / (float)N;
    float v[1024];
    for (int64_t k = 0; k < n; ++k) {
        for (int r = 0; r < N; ++r) v[r] = load_elem(x[r], in_dtype, k);
        float acc = fold(v, N, order, lo + k, len);
        store_elem(out, out_dtype, k, acc * scale);
    }
    return 0;
}

/* Average S sampled elements.  vals holds S rows of N input values (row s is
 * the N ranks' values of one element), pos[s] is that element's position in
 * its bucket and len[s] the bucket's length. */
int oracle_sampled_avg(const void *vals, const int64_t *pos, const int64_t *len,
                       int64_t S, int N, int order, int in_dtype, int out_dtype,
                       void *out)
{
    if (check_args(N, order, in_dtype, out_dtype) || S < 0) return -1;
    const float inv = 1.0f / (float)N;
    float v[1024];
    for (int64_t s = 0; s < S; ++s) {
        if (N == 1) {
            if (in_dtype != out_dtype) return -1;
            if (in_dtype == ORACLE_BF16) ((uint16_t *)out)[s] = ((const uint16_t *)vals)[s];
            else ((uint32_t *)out)[s] = ((const uint32_t *)vals)[s];
            continue;
        }
        for (int r = 0; r < N; ++r) v[r] = load_elem(vals, in_dtype, s * N + r);
        float acc = fold(v, N, order, pos[s], len[s]);
        store_elem(out, out_dtype, s, acc * inv);
    }
    return 0;
}

/* One SGD step over n elements: p[i] -= lr * g[i] (g of dtype g_dtype),
 * through the momentum buffer m when m != NULL. */
int oracle_sgd_step(float *p, float *m, const void *g, int g_dtype, int64_t n, float lr, float mu)
{
    if ((g_dtype != ORACLE_F32 && g_dtype != ORACLE_BF16) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        float gi = load_elem(g, g_dtype, i);
        if (m) {
            float v = mu * m[i];
            v = v + gi;
            m[i] = v;
            gi = v;
        }
        float step = lr * gi;
        p[i] = p[i] - step;
    }
    return 0;
}

/* dst[i] = dst[i] + src[i] over n elements of dtype (bf16: widened, added in
 * f32, rounded to nearest even). */
int oracle_accumulate(void *dst, const void *src, int dtype, int64_t n)
{
    if ((dtype != ORACLE_F32 && dtype != ORACLE_BF16) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) {
        float a = load_elem(dst, dtype, i);
        float b = load_elem(src, dtype, i);
        store_elem(dst, dtype, i, a + b);
    }
    return 0;
}
