/*
 * CPU oracle for the lightning-indexer logits -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg load this library.  The GPU library shares no code, header or table with
 * it, and nothing here is ever used as a fallback for the GPU path.
 *
 * It is a plain, slow, fp64 evaluation of the definition given on
 *   "[HIP] [JIT] fp8_paged_mqa_logits: hand-written gfx950 decode indexer
 *    kernel" (aiter PR 5047), section "Motivation", and on
 *   "[HIP] [JIT] fp8_mqa_logits: hand-written gfx950 prefill indexer kernel"
 *    (aiter PR 5046), section "Motivation":
 *
 *   logits[m, n] = sum_h relu(<Q[m,h,:], K[n,:]>) * kv_scale[n] * weights[m,h]
 *
 * for n inside row m's window, -inf elsewhere.
 *
 * Exactness: every fp8 e4m3fn value is an integer multiple of 2^-9 with
 * magnitude <= 448, so each product Q*K is a multiple of 2^-18 below 2^18 and a
 * 128-term dot product needs at most 43 significant bits: the fp64 dot is
 * exact.  The only roundings are the fp64 products with the weight and scale
 * and the 32-term head sum (about 1e-16 relative).
 *
 * The scale is applied inside the head sum (the unhoisted order written in the
 * definition) unless `hoist` is set, in which case it multiplies the head sum
 * once per column (the "kv-scale hoist" of both pages' "Technical Details").
 * The two agree because kv_scale >= 0 and relu is positive-homogeneous; the
 * tests check that they do.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- fp8 e4m3fn decode --------------------------------------------------
 * OCP 8-bit floating point format E4M3 ("fn": finite, no infinities):
 * sign bit, 4 exponent bits with bias 7, 3 mantissa bits.
 *   exponent field 0        -> subnormal  (-1)^s * m/8 * 2^(1-7)
 *   exponent 15, mantissa 7 -> NaN (the only non-finite codes: 0x7F, 0xFF)
 *   otherwise               -> (-1)^s * (1 + m/8) * 2^(e-7)
 * Largest finite magnitude: 1.75 * 2^8 = 448.
 */
double oracle_e4m3fn_value(uint8_t code)
{
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m / 8.0, 1 - 7);
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

void oracle_e4m3fn_table(double *out256)
{
    for (int c = 0; c < 256; ++c)
        out256[c] = oracle_e4m3fn_value((uint8_t)c);
}

static double table_fp8[256];
static int table_ready = 0;

static void ensure_table(void)
{
    if (!table_ready) {
        oracle_e4m3fn_table(table_fp8);
        table_ready = 1;
    }
}

/* One logit: q points at Q[m,0,0] ([H][D] fp8), k at K[n,0] ([D] fp8). */
static double one_logit(const uint8_t *q, const uint8_t *k, double scale,
                        const float *w, int H, int D, int hoist)
{
    double acc = 0.0;
    for (int h = 0; h < H; ++h) {
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
            dot += table_fp8[q[(int64_t)h * D + d]] * table_fp8[k[d]];
        double r = dot > 0.0 ? dot : 0.0; /* relu */
        if (hoist)
            acc += r * (double)w[h];
        else
            acc += r * scale * (double)w[h];
    }
    return hoist ? acc * scale : acc;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---- prefill ------------------------------------------------------------
 * Window of row m (aiter PR 5046 page, "Motivation"; edge cases from its
 * "Test Plan"): column n is valid iff  max(ks[m], 0) <= n < min(ke[m], N).
 * An empty or negative window leaves the whole row invalid.
 *
 * q [M,H,D] fp8, k [N,D] fp8, kv_scale [N], w [M,H], ks/ke [M], out [M,N].
 * clean != 0: invalid columns are written -inf; clean == 0: they are left as
 * the caller filled them.
 */
void oracle_prefill(const uint8_t *q, const uint8_t *k, const float *kv_scale,
                    const float *w, const int32_t *ks, const int32_t *ke,
                    int64_t M, int64_t N, int H, int D, int clean, int hoist,
                    double *out)
{
    ensure_table();
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        int64_t lo = ks[m] > 0 ? ks[m] : 0;
        int64_t hi = ke[m] < N ? ke[m] : N;
        for (int64_t n = 0; n < N; ++n) {
            double *o = &out[m * N + n];
            if (n >= lo && n < hi)
                *o = one_logit(q + m * H * D, k + n * D, (double)kv_scale[n],
                               w + m * H, H, D, hoist);
            else if (clean)
                *o = -INFINITY;
        }
    }
}

/* ---- paged decode -------------------------------------------------------
 * aiter PR 5047 page, "Technical Details": row j (0 <= j < next_n) of sequence
 * b covers KV positions p <= context_lens[b] - next_n + j (the issue page on
 * next_n tiling names the same bound "context_length - next_n + pid_next_n").
 * K and its per-token scale are read through block_tables; the cache layout is
 * block-split: block i is bs*(D+4) bytes, K rows of its bs slots first, then
 * the bs fp32 scales.  The K rows are either slot-major (layout 0: slot s's D
 * bytes at s*D) or tiled in 16 x 16 byte tiles (layout 1, the preshuffled
 * (16,16) cache the aiter PR 5047 page names under "Technical Details" for
 * 64-token blocks): the slots form groups of 16, group by group, each group
 * holding its 16-byte column granules in order, each granule holding the 16
 * slots' bytes of that granule one slot after the other.  So byte d of slot s
 * sits at  (s/16)*16*D + (d/16)*256 + (s%16)*16 + d%16.
 *
 * q [B,next_n,H,D], w [B*next_n,H], ctx [B], bt [B,mbps], out [B*next_n, mml].
 * Returns 0, -1 if a table entry that has to be read is out of range, or -2
 * for a layout the block shape cannot hold.
 */
int oracle_decode(const uint8_t *q, const uint8_t *cache, const float *w,
                  const int32_t *ctx, const int32_t *bt, int B, int next_n,
                  int H, int D, int bs, int layout, int64_t num_blocks, int mbps,
                  int64_t mml, int clean, int hoist, double *out)
{
    ensure_table();
    int bad = 0;
    if (layout != 0 && (layout != 1 || bs % 16 != 0 || D % 16 != 0 || D > 1024))
        return -2;
    int64_t block_bytes = (int64_t)bs * (D + 4);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t row = 0; row < (int64_t)B * next_n; ++row) {
        int64_t b = row / next_n;
        int64_t j = row % next_n;
        int64_t bound = (int64_t)ctx[b] - next_n + j; /* inclusive */
        for (int64_t p = 0; p < mml; ++p) {
            double *o = &out[row * mml + p];
            if (p >= 0 && p <= bound) {
                int64_t lb = p / bs;
                if (lb >= mbps) {
                    bad = 1;
                    continue;
                }
                int64_t blk = bt[b * mbps + lb];
                if (blk < 0 || blk >= num_blocks) {
                    bad = 1;
                    continue;
                }
                const uint8_t *base = cache + blk * block_bytes;
                int64_t slot = p % bs;
                float sc;
                memcpy(&sc, base + (int64_t)bs * D + slot * 4, 4);
                const uint8_t *krow = base + slot * D;
                uint8_t tiled[1024];
                if (layout == 1) {
                    for (int d = 0; d < D; ++d)
                        tiled[d] = base[(slot / 16) * 16 * D + (d / 16) * 256 +
                                        (slot % 16) * 16 + d % 16];
                    krow = tiled;
                }
                *o = one_logit(q + row * H * D, krow, (double)sc,
                               w + row * H, H, D, hoist);
            } else if (clean) {
                *o = -INFINITY;
            }
        }
    }
    return bad ? -1 : 0;
}
