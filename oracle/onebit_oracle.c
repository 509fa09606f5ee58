/*
 * onebit_oracle.c -- plain, slow, single-threaded CPU reference for the 1-bit Adam
 * hot path and the QSDP stochastic-rounding quantizer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls
 * this file; only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark do.  It shares no source with the HIP library.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fno-fast-math -fPIC -shared
 * (no fused multiply-add, no flush-to-zero: every "fl32(...)" below is exactly one
 * IEEE-754 binary32 operation with round-to-nearest-even, as on the GPU side).
 *
 * Sources ("the pages"):
 *  [1BA]  nubint.ai review "1-bit Adam: Communication Efficient Large-Scale Training
 *         with Adam's Convergence Speed", section "proposed method": Adam warmup,
 *         then the variance is frozen and used as a fixed preconditioner for
 *         error-compensated 1-bit compressed momentum SGD.
 *  [APM]  nubint.ai review "APMSqueeze", section "proposed method": during the
 *         preconditioning phase m_t and v_t are kept, afterwards v_t is frozen and
 *         m_t is compressed.
 *  [DSG]  yfxerp.com guide "DeepSpeed 1-bit Adam ... complete configuration guide",
 *         sec. 3.4 (parameter table: lr, betas, eps, weight_decay, bias_correction),
 *         sec. 3.5 (momentum mask), sec. 4 (the two phases of step(), the
 *         compressed all-reduce with worker_error / server_error, the update
 *         exp_avg / (sqrt(exp_avg_sq) + eps), 1 bit per value), sec. 7 (errors are
 *         reset on checkpoint load).
 *  [QSDP] nubint.ai review "Quantized Distributed Training of Large Models with
 *         Convergence Guarantees", section "proposed method": weights quantized by
 *         unbiased stochastic rounding to the nearest quantization levels.
 *  [QSGD] Alistarh, Grubic, Li, Tomioka, Vojnovic, "QSGD: Communication-Efficient
 *         SGD via Gradient Quantization and Encoding", NeurIPS 2017, sec. 3.1 (the
 *         stochastic quantizer Q_s) and its bucketed form; named by [QSDP] as the
 *         standard unbiased compressor applied to gradients.
 *  [LOCO] shd-paper.top summary of "LoCo: Low-Bit Communication Adaptor for Large-scale
 *         Model Training", core points and method details: before compressing, the
 *         local gradient is compensated with a moving average of the historical
 *         compensation errors, which estimates the current compression error.  The
 *         page gives no formula, window or weights (parity unpinned: the steps
 *         below are this oracle's reading, pinned only by its special cases).
 *  [PHX]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3",
 *         SC'11, section 4 (the Philox-4x32 bijection, 10 rounds).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - chunk scale = sqrt(sum c^2) / sqrt(n_chunk), sum taken in fp64 with compensated
 *    (Neumaier) summation, rounded once to fp32; the decompressed chunk then has
 *    the L2 norm of c;
 *  - a value is sent as bit 1 iff c < 0, so +0 and -0 decompress to +scale;
 *    32 bits per uint32 word, least significant bit first, every chunk starts on
 *    a word boundary, pad bits are 0;
 *  - after the compressed step m holds the decompressed momentum (the page's
 *    compressed_allreduce writes its result back into exp_avg);
 *  - eps is added to sqrt(v) (the page's formula lost its "+" sign);
 *  - bias correction, when enabled, applies to the warmup phase only;
 *  - weight decay is decoupled: update = m/(sqrt(v)+eps) + wd*x, x -= lr*update;
 *  - momentum mask per tensor: bits and scale come from the unmasked c, then m and
 *    e of masked tensors are set to 0;
 *  - server average: fp64 sum over workers in order 0..W-1, fp64 divide by W,
 *    one rounding to fp32;
 *  - QSDP: 2^b evenly spaced levels over [min, max] of each bucket; Philox key =
 *    seed, counter = (element index >> 2, 0, 0), output word (index & 3);
 *    round up iff u < floor(p * 2^32);
 *  - QSGD: per bucket the L2 norm (same fp64 sum, sqrt in fp64, one rounding to
 *    fp32); s = 2^(bits-1) - 1 levels of |g| / norm; code = sign bit (top bit of
 *    the code, set iff g < 0) and the level below it; same Philox stream layout as
 *    the weights (the caller picks a different seed); the dequantized value is
 *    the real number +-level * norm / s, and the average of W workers' values is
 *    (sum_w +-level_w * norm_w) / (s * W): each product level * norm is exact in
 *    fp64 (7 + 24 significant bits), the products are summed in fp64 in worker
 *    order, divided once by s * W in fp64 and rounded once to fp32.  Whenever
 *    that fp64 sum is exact the result is the exact average rounded once to fp32
 *    (the fp64 quotient cannot straddle a binary32 rounding boundary); the sum is
 *    exact for W = 1, and whenever W * 2^(31 + d) <= 2^53 with d the spread of the
 *    exponents of the W norms of the bucket (e.g. W <= 16 and d <= 18).
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_ERR_INVALID 1
#define ORACLE_ERR_NOMEM 4

/* ------------------------------------------------------------------ helpers */

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16; /* bf16 is the upper half of a binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays NaN (quiet). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u; /* carries into the exponent correctly, up to +inf */
    return (uint16_t)upper;
}

/* Neumaier's improvement of Kahan summation over non-negative fp64 terms. */
typedef struct {
    double sum;
    double comp;
} neumaier_t;

static void neumaier_add(neumaier_t *acc, double term)
{
    double t = acc->sum + term;
    if (fabs(acc->sum) >= fabs(term))
        acc->comp += (acc->sum - t) + term;
    else
        acc->comp += (term - t) + acc->sum;
    acc->sum = t;
}

static double neumaier_result(const neumaier_t *acc) { return acc->sum + acc->comp; }

/* scale_j = fl32( sqrt(S) / sqrt(n) ), S = exact-ish sum of fp64 squares. */
static float chunk_scale(const float *c, int64_t n)
{
    if (n <= 0)
        return 0.0f;
    neumaier_t acc = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i) {
        double ci = (double)c[i];
        neumaier_add(&acc, ci * ci); /* exact: 24-bit x 24-bit fits in 53 bits */
    }
    double s = neumaier_result(&acc);
    return (float)(sqrt(s) / sqrt((double)n));
}

static int64_t words_for(int64_t n) { return (n + 31) / 32; }

/* Validate a chunk table: [0] = 0, non-decreasing. */
static int check_offsets(const int64_t *off, int64_t count)
{
    if (!off || count < 0 || off[0] != 0)
        return 0;
    for (int64_t j = 0; j < count; ++j)
        if (off[j + 1] < off[j])
            return 0;
    return 1;
}

/* Expand a per-tensor keep table into a per-element flag for [0, n). */
static uint8_t *expand_keep(const int64_t *tensor_off, const uint8_t *keep, int64_t n_tensors, int64_t n)
{
    uint8_t *flag = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
    if (!flag)
        return NULL;
    memset(flag, 1, (size_t)(n > 0 ? n : 1));
    if (tensor_off && keep) {
        for (int64_t t = 0; t < n_tensors; ++t)
            for (int64_t i = tensor_off[t]; i < tensor_off[t + 1]; ++i)
                flag[i] = keep[t] ? 1 : 0;
    }
    return flag;
}

/* ------------------------------------------------------- O1: warmup Adam step
 * [DSG] sec. 4 (phase one: standard Adam first and second moments, full-precision
 * gradients) and sec. 3.4 (lr, betas, eps, weight_decay, bias_correction);
 * [APM] "proposed method" (m_t and v_t are both maintained while preconditioning).
 * step is 1-based.  m and v follow the exact fp32 operation sequence; x is the
 * decoupled-weight-decay Adam update.  Hyperparameters arrive as binary64 (as a
 * Python float does) and are each rounded to binary32 once; 1-beta is formed in
 * binary64 first, the way the page's exp_avg.mul_(beta1).add_(1 - beta1, grad)
 * forms it.  The bias-correction denominators 1-beta^t are formed in binary64.
 */
int oracle_adam_warmup_step(float *x, float *m, float *v, const float *g, int64_t n, double lr_d,
                            double beta1_d, double beta2_d, double eps_d, double weight_decay_d,
                            int bias_correction, int64_t step)
{
    if (n < 0 || step < 1 || (n > 0 && (!x || !m || !v || !g)))
        return ORACLE_ERR_INVALID;
    const float beta1 = (float)beta1_d, beta2 = (float)beta2_d;
    const float ob1 = (float)(1.0 - beta1_d); /* 1-beta formed in binary64, rounded once */
    const float ob2 = (float)(1.0 - beta2_d);
    const float lr = (float)lr_d, eps = (float)eps_d, weight_decay = (float)weight_decay_d;
    float bc1 = 1.0f, bc2 = 1.0f;
    if (bias_correction) {
        bc1 = (float)(1.0 - pow(beta1_d, (double)step));
        bc2 = (float)(1.0 - pow(beta2_d, (double)step));
    }
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g[i];
        const float mi = beta1 * m[i] + ob1 * gi;        /* fl32(fl32(b1*m) + fl32(ob1*g)) */
        const float vi = beta2 * v[i] + ob2 * (gi * gi); /* fl32(fl32(b2*v) + fl32(ob2*fl32(g*g))) */
        m[i] = mi;
        v[i] = vi;
        const float mhat = bias_correction ? mi / bc1 : mi;
        const float vhat = bias_correction ? vi / bc2 : vi;
        const float update = mhat / (sqrtf(vhat) + eps) + weight_decay * x[i];
        x[i] = x[i] - lr * update;
    }
    return ORACLE_OK;
}

/* ------------------------------------- O3: worker compress (+ frozen-v update)
 * [DSG] sec. 4 (phase two: exp_avg = beta1*exp_avg + (1-beta1)*grad; the momentum,
 * not the gradient, is compressed; the residual dropped by this round's
 * compression is kept in the error buffer and added back before the next one;
 * every value travels as 1 bit; then update = exp_avg / (sqrt(exp_avg_sq) + eps),
 * weight decay and lr applied), sec. 3.5 (the mask zeroes the momentum of masked
 * parameters after the all-reduce); [1BA] "proposed method" (error compensation on
 * the momentum; frozen variance as preconditioner).
 *
 * Compress-only mode (v == NULL and x == NULL): m is read but not written, x and v
 * untouched -- the worker half of the compressed all-reduce.
 * identity != 0 replaces the 1-bit compressor by the identity (q = c); used only by
 * the tests to pin the frozen-v phase to momentum SGD.  bits/scales are still
 * filled from c in that mode.
 */
int oracle_compress_update(const int64_t *chunk_off, int64_t n_chunks, const int64_t *tensor_off,
                           const uint8_t *tensor_keep, int64_t n_tensors, const float *g, float *m,
                           float *e, const float *v, float *x, uint16_t *x_bf16, uint32_t *bits,
                           float *scales, double lr_d, double beta1_d, double eps_d,
                           double weight_decay_d, int identity)
{
    if (!check_offsets(chunk_off, n_chunks))
        return ORACLE_ERR_INVALID;
    const int64_t n = chunk_off[n_chunks];
    const int update_mode = (v != NULL) || (x != NULL);
    if (update_mode && (!v || !x))
        return ORACLE_ERR_INVALID;
    if (tensor_off) {
        if (!check_offsets(tensor_off, n_tensors) || tensor_off[n_tensors] != n)
            return ORACLE_ERR_INVALID;
    }
    if (n > 0 && (!g || !m || !e || !bits || !scales))
        return ORACLE_ERR_INVALID;

    uint8_t *keep = expand_keep(tensor_off, tensor_keep, n_tensors, n);
    int64_t max_len = 1;
    for (int64_t j = 0; j < n_chunks; ++j)
        if (chunk_off[j + 1] - chunk_off[j] > max_len)
            max_len = chunk_off[j + 1] - chunk_off[j];
    float *c = (float *)malloc((size_t)max_len * sizeof(float));
    if (!keep || !c) {
        free(keep);
        free(c);
        return ORACLE_ERR_NOMEM;
    }

    const float beta1 = (float)beta1_d;
    const float ob1 = (float)(1.0 - beta1_d); /* 1-beta formed in binary64, rounded once */
    const float lr = (float)lr_d, eps = (float)eps_d, weight_decay = (float)weight_decay_d;
    int64_t wbase = 0;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t o = chunk_off[j];
        const int64_t len = chunk_off[j + 1] - o;

        /* 1. momentum and error compensation */
        for (int64_t k = 0; k < len; ++k) {
            const int64_t i = o + k;
            const float m1 = beta1 * m[i] + ob1 * g[i];
            c[k] = m1 + e[i];
        }

        /* 2. chunk scale */
        const float scale = chunk_scale(c, len);
        scales[j] = scale;

        /* 3. sign bits, LSB first, chunk starts on a word boundary, pad bits 0 */
        const int64_t nw = words_for(len);
        for (int64_t w = 0; w < nw; ++w)
            bits[wbase + w] = 0u;
        for (int64_t k = 0; k < len; ++k)
            if (c[k] < 0.0f)
                bits[wbase + (k >> 5)] |= 1u << (k & 31);

        /* 4-6. decompress, error, momentum, mask, update */
        for (int64_t k = 0; k < len; ++k) {
            const int64_t i = o + k;
            float q;
            if (identity)
                q = c[k];
            else
                q = (c[k] < 0.0f) ? -scale : scale;
            float e_new = c[k] - q;
            float m_new = q;
            if (!keep[i]) {
                m_new = 0.0f;
                e_new = 0.0f;
            }
            e[i] = e_new;
            if (update_mode) {
                m[i] = m_new;
                const float update = m_new / (sqrtf(v[i]) + eps) + weight_decay * x[i];
                x[i] = x[i] - lr * update;
                if (x_bf16)
                    x_bf16[i] = oracle_f32_to_bf16(x[i]);
            }
        }
        wbase += nw;
    }
    free(c);
    free(keep);
    return ORACLE_OK;
}

/* --------------------------------------------------------- O4: server stage
 * [DSG] sec. 4 (each GPU keeps a worker-side and a server-side error buffer; the
 * compressed all-reduce averages the workers' compressed momenta and compresses
 * the average again with the server error); [1BA] "proposed method" (custom
 * collective for the compressed exchange).
 * worker_bits: W rows of plan_words words; worker_scales: W rows of n_chunks.
 * m_out (nullable) receives the decompressed server result.
 */
int oracle_server_reduce(const int64_t *chunk_off, int64_t n_chunks, int W, const uint32_t *worker_bits,
                         const float *worker_scales, float *server_error, uint32_t *server_bits,
                         float *server_scales, float *m_out)
{
    if (!check_offsets(chunk_off, n_chunks) || W < 1)
        return ORACLE_ERR_INVALID;
    const int64_t n = chunk_off[n_chunks];
    int64_t plan_words = 0;
    int64_t max_len = 1;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t len = chunk_off[j + 1] - chunk_off[j];
        plan_words += words_for(len);
        if (len > max_len)
            max_len = len;
    }
    if (n > 0 && (!worker_bits || !worker_scales || !server_error || !server_bits || !server_scales))
        return ORACLE_ERR_INVALID;
    float *c = (float *)malloc((size_t)max_len * sizeof(float));
    if (!c)
        return ORACLE_ERR_NOMEM;

    int64_t wbase = 0;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t o = chunk_off[j];
        const int64_t len = chunk_off[j + 1] - o;
        for (int64_t k = 0; k < len; ++k) {
            double sum = 0.0;
            for (int w = 0; w < W; ++w) {
                const uint32_t word = worker_bits[(int64_t)w * plan_words + wbase + (k >> 5)];
                const double s = (double)worker_scales[(int64_t)w * n_chunks + j];
                sum += ((word >> (k & 31)) & 1u) ? -s : s;
            }
            const float a = (float)(sum / (double)W);
            c[k] = a + server_error[o + k];
        }
        const float scale = chunk_scale(c, len);
        server_scales[j] = scale;
        const int64_t nw = words_for(len);
        for (int64_t w = 0; w < nw; ++w)
            server_bits[wbase + w] = 0u;
        for (int64_t k = 0; k < len; ++k) {
            const int neg = c[k] < 0.0f;
            if (neg)
                server_bits[wbase + (k >> 5)] |= 1u << (k & 31);
            const float q = neg ? -scale : scale;
            server_error[o + k] = c[k] - q;
            if (m_out)
                m_out[o + k] = q;
        }
        wbase += nw;
    }
    free(c);
    return ORACLE_OK;
}

/* ------------------------------------- worker finish after the all-reduce
 * [DSG] sec. 3.5 and sec. 4: after the compressed all-reduce has written the
 * decompressed momentum back, the momentum is multiplied by exp_avg_mask (a 0/1
 * tensor of the parameter's shape; here one byte per element, non-zero = 1), then
 * update = m / (sqrt(v) + eps) + wd * x and x -= lr * update.
 * mask and x_bf16 are nullable (no mask = all ones).
 */
int oracle_momentum_update(float *m, const uint8_t *mask, const float *v, float *x, uint16_t *x_bf16, int64_t n,
                           double lr_d, double eps_d, double weight_decay_d)
{
    if (n < 0 || (n > 0 && (!m || !v || !x)))
        return ORACLE_ERR_INVALID;
    const float lr = (float)lr_d, eps = (float)eps_d, weight_decay = (float)weight_decay_d;
    for (int64_t i = 0; i < n; ++i) {
        if (mask)
            m[i] = m[i] * (mask[i] ? 1.0f : 0.0f);
        const float update = m[i] / (sqrtf(v[i]) + eps) + weight_decay * x[i];
        x[i] = x[i] - lr * update;
        if (x_bf16)
            x_bf16[i] = oracle_f32_to_bf16(x[i]);
    }
    return ORACLE_OK;
}

/* Decompress a packed stream (one worker's or the server's) into fp32. */
int oracle_decompress(const int64_t *chunk_off, int64_t n_chunks, const uint32_t *bits,
                      const float *scales, float *out)
{
    if (!check_offsets(chunk_off, n_chunks))
        return ORACLE_ERR_INVALID;
    int64_t wbase = 0;
    for (int64_t j = 0; j < n_chunks; ++j) {
        const int64_t o = chunk_off[j];
        const int64_t len = chunk_off[j + 1] - o;
        for (int64_t k = 0; k < len; ++k) {
            const uint32_t word = bits[wbase + (k >> 5)];
            out[o + k] = ((word >> (k & 31)) & 1u) ? -scales[j] : scales[j];
        }
        wbase += words_for(len);
    }
    return ORACLE_OK;
}

/* ----------------------------------------------------------- Philox4x32-10
 * [PHX] section 4: two 32x32->64 multiplies per round with multipliers
 * 0xD2511F53 and 0xCD9E8D57, the high halves xored with the other two counter words
 * and the round key, the round key advanced by the Weyl constants 0x9E3779B9 and
 * 0xBB67AE85 between rounds.
 */
void oracle_philox4x32_10(const uint32_t key_in[2], const uint32_t ctr_in[4], uint32_t out[4])
{
    uint32_t k0 = key_in[0], k1 = key_in[1];
    uint32_t x0 = ctr_in[0], x1 = ctr_in[1], x2 = ctr_in[2], x3 = ctr_in[3];
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)0xD2511F53u * (uint64_t)x0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * (uint64_t)x2;
        const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        const uint32_t y0 = hi1 ^ x1 ^ k0;
        const uint32_t y1 = lo1;
        const uint32_t y2 = hi0 ^ x3 ^ k1;
        const uint32_t y3 = lo0;
        x0 = y0;
        x1 = y1;
        x2 = y2;
        x3 = y3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = x0;
    out[1] = x1;
    out[2] = x2;
    out[3] = x3;
}

/* The uniform 32-bit word used for element i under seed s. */
uint32_t oracle_qsdp_uniform(uint64_t seed, int64_t i)
{
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    const uint64_t block = (uint64_t)i >> 2;
    const uint32_t ctr[4] = {(uint32_t)block, (uint32_t)(block >> 32), 0u, 0u};
    uint32_t out[4];
    oracle_philox4x32_10(key, ctr, out);
    return out[i & 3];
}

/* IEEE 754 totalOrder restricted to non-NaN values: like <, but -0 < +0.  The
 * pages do not say which zero is a bucket's minimum; this reading makes min and
 * max independent of the order in which the elements are visited. */
static int total_order_less(float a, float b)
{
    return a < b || (a == b && signbit(a) && !signbit(b));
}

/* ------------------------------------------------- O5: QSDP quantize
 * [QSDP] "proposed method": an unbiased operator that stochastically rounds each
 * weight to one of the two nearest quantization levels, so the expectation equals
 * the weight.  Levels: 2^bits evenly spaced over the bucket's [min, max].
 * first_index is the global index of x_bf16[0] (a multiple of the bucket): the
 * Philox counter uses global element indices, so a slice of a larger vector can
 * be checked on its own.
 */
int oracle_qsdp_quantize(const uint16_t *x_bf16, int64_t n, int bucket, int nbits, uint64_t seed,
                         int64_t first_index, uint8_t *codes, float *bucket_min, float *bucket_max)
{
    if (n < 0 || bucket < 1 || (nbits != 4 && nbits != 8) || first_index < 0 ||
        first_index % bucket != 0 || (nbits == 4 && first_index % 2 != 0))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!x_bf16 || !codes || !bucket_min || !bucket_max)
        return ORACLE_ERR_INVALID;
    const int L = (1 << nbits) - 1;
    const int64_t n_buckets = (n + bucket - 1) / bucket;
    const int64_t code_bytes = nbits == 4 ? (n + 1) / 2 : n;
    memset(codes, 0, (size_t)code_bytes);
    for (int64_t b = 0; b < n_buckets; ++b) {
        const int64_t lo = b * (int64_t)bucket;
        const int64_t hi = lo + bucket < n ? lo + bucket : n;
        float mn = oracle_bf16_to_f32(x_bf16[lo]), mx = mn;
        for (int64_t i = lo + 1; i < hi; ++i) {
            const float xi = oracle_bf16_to_f32(x_bf16[i]);
            if (total_order_less(xi, mn))
                mn = xi;
            if (total_order_less(mx, xi))
                mx = xi;
        }
        bucket_min[b] = mn;
        bucket_max[b] = mx;
        const float delta = (mx - mn) / (float)L;
        for (int64_t i = lo; i < hi; ++i) {
            uint32_t code = 0;
            if (delta != 0.0f) {
                const float d = oracle_bf16_to_f32(x_bf16[i]) - mn;
                const float t = d / delta;
                float k = floorf(t);
                if (k > (float)L)
                    k = (float)L;
                const float p = t - k;                                    /* exact */
                const uint64_t thr = (uint64_t)floor((double)p * 4294967296.0); /* exact */
                const uint32_t u = oracle_qsdp_uniform(seed, first_index + i);
                code = (uint32_t)k + ((uint64_t)u < thr ? 1u : 0u);
                if (code > (uint32_t)L)
                    code = (uint32_t)L;
            }
            if (nbits == 8)
                codes[i] = (uint8_t)code;
            else
                codes[i >> 1] |= (uint8_t)(code << ((i & 1) ? 4 : 0));
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------- O6: QSDP dequantize
 * y = fl32(min + fl32(code * delta)), delta recomputed as in quantize; output bf16
 * (round to nearest even) and, optionally, the fp32 y before rounding.
 */
int oracle_qsdp_dequantize(const uint8_t *codes, const float *bucket_min, const float *bucket_max,
                           int64_t n, int bucket, int nbits, uint16_t *out_bf16, float *out_f32)
{
    if (n < 0 || bucket < 1 || (nbits != 4 && nbits != 8))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!codes || !bucket_min || !bucket_max)
        return ORACLE_ERR_INVALID;
    const int L = (1 << nbits) - 1;
    for (int64_t i = 0; i < n; ++i) {
        const int64_t b = i / bucket;
        const float mn = bucket_min[b];
        const float delta = (bucket_max[b] - mn) / (float)L;
        uint32_t code;
        if (nbits == 8)
            code = codes[i];
        else
            code = (codes[i >> 1] >> ((i & 1) ? 4 : 0)) & 0xfu;
        const float y = mn + (float)code * delta;
        if (out_f32)
            out_f32[i] = y;
        if (out_bf16)
            out_bf16[i] = oracle_f32_to_bf16(y);
    }
    return ORACLE_OK;
}

/* --------------------------------------------- O7: QSGD gradient quantizer
 * [QSGD] sec. 3.1: with v a bucket of the gradient and l the integer such that
 * |v_i| / ||v||_2 lies in [l/s, (l+1)/s], the value sent is ||v||_2 sgn(v_i) xi_i / s,
 * where xi_i = l + 1 with probability |v_i| s / ||v||_2 - l and l otherwise, so
 * that its expectation is v_i.  Here (binary32 steps, as on the device side):
 *   t = fl32(|g| / norm);  u = fl32(t * s);  l = floor(u);  p = u - l (exact)
 *   level = l + (uniform < floor(p * 2^32));  code = (g < 0) << (bits-1) | level.
 * A bucket of zeros has norm 0 and all codes 0.  g: fp32 (dtype 0) or bf16 bits
 * (dtype 1).  4-bit codes are packed two per byte, even element in the low nibble.
 */
static double bucket_sum_squares(const float *v, int64_t n)
{
    neumaier_t acc = {0.0, 0.0};
    for (int64_t i = 0; i < n; ++i)
        neumaier_add(&acc, (double)v[i] * (double)v[i]);
    return neumaier_result(&acc);
}

int oracle_qsgd_quantize(const void *g, int g_dtype, int64_t n, int bucket, int nbits, uint64_t seed,
                         int64_t first_index, uint8_t *codes, float *norms)
{
    if (n < 0 || bucket < 1 || (nbits != 4 && nbits != 8) || (g_dtype != 0 && g_dtype != 1) || first_index < 0 ||
        first_index % bucket != 0 || (nbits == 4 && (bucket % 2 != 0 || first_index % 2 != 0)))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!g || !codes || !norms)
        return ORACLE_ERR_INVALID;
    const uint32_t s = (1u << (nbits - 1)) - 1u;
    float *v = (float *)malloc((size_t)bucket * sizeof(float));
    if (!v)
        return ORACLE_ERR_NOMEM;
    memset(codes, 0, (size_t)(nbits == 4 ? (n + 1) / 2 : n));
    const int64_t n_buckets = (n + bucket - 1) / bucket;
    for (int64_t b = 0; b < n_buckets; ++b) {
        const int64_t lo = b * (int64_t)bucket;
        const int64_t len = lo + bucket < n ? bucket : n - lo;
        for (int64_t k = 0; k < len; ++k)
            v[k] = g_dtype == 1 ? oracle_bf16_to_f32(((const uint16_t *)g)[lo + k]) : ((const float *)g)[lo + k];
        const float norm = (float)sqrt(bucket_sum_squares(v, len));
        norms[b] = norm;
        if (norm == 0.0f)
            continue;
        for (int64_t k = 0; k < len; ++k) {
            const float t = fabsf(v[k]) / norm;
            const float u = t * (float)s;
            const float l = floorf(u);
            const float p = u - l;
            const uint64_t thr = (uint64_t)floor((double)p * 4294967296.0);
            uint32_t level = (uint32_t)l + ((uint64_t)oracle_qsdp_uniform(seed, first_index + lo + k) < thr ? 1u : 0u);
            const uint32_t code = (v[k] < 0.0f ? 1u << (nbits - 1) : 0u) | level;
            const int64_t i = lo + k;
            if (nbits == 8)
                codes[i] = (uint8_t)code;
            else
                codes[i >> 1] |= (uint8_t)((i & 1) ? code << 4 : code);
        }
    }
    free(v);
    return ORACLE_OK;
}

/* The value worker w sent for element i, times s: +-level * norm, exact in fp64
 * (at most 7 + 24 significant bits). */
static double qsgd_value_times_s(const uint8_t *codes, const float *norms, int64_t i, int bucket, int nbits)
{
    const uint32_t s = (1u << (nbits - 1)) - 1u;
    const uint32_t code = nbits == 8 ? codes[i] : (uint32_t)((codes[i >> 1] >> ((i & 1) ? 4 : 0)) & 0xfu);
    const uint32_t level = code & s;
    const double y = (double)level * (double)norms[i / bucket];
    return (code >> (nbits - 1)) ? -y : y;
}

/* [QSGD] sec. 3.1 decoding: worker w's value is +-level_w * norm_w / s, averaged
 * over W workers' streams (the reduce half of a quantized gradient
 * reduce-scatter): out_i = fl32( (sum_w +-level_w * norm_w) / (s * W) ), the exact
 * products summed in fp64 in worker order, one fp64 division, one rounding to
 * fp32.  Worker w's codes start at codes + w * code_stride bytes, its norms at
 * norms + w * norm_stride.  W = 1 is plain dequantization. */
int oracle_qsgd_reduce(int W, const uint8_t *codes, int64_t code_stride, const float *norms, int64_t norm_stride,
                       int64_t n, int bucket, int nbits, float *out_f32, uint16_t *out_bf16)
{
    if (W < 1 || n < 0 || bucket < 1 || (nbits != 4 && nbits != 8) || (nbits == 4 && bucket % 2 != 0))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!codes || !norms || (!out_f32 && !out_bf16))
        return ORACLE_ERR_INVALID;
    const double sW = (double)((1u << (nbits - 1)) - 1u) * (double)W;
    for (int64_t i = 0; i < n; ++i) {
        double acc = 0.0;
        for (int w = 0; w < W; ++w)
            acc += qsgd_value_times_s(codes + (int64_t)w * code_stride, norms + (int64_t)w * norm_stride, i, bucket,
                                      nbits);
        const float y = (float)(acc / sW);
        if (out_f32)
            out_f32[i] = y;
        if (out_bf16)
            out_bf16[i] = oracle_f32_to_bf16(y);
    }
    return ORACLE_OK;
}

/* ------------------------------------- O9: the warmup phase's gradient average
 * [DSG] sec. 4, phase one: the Adam step runs on the gradient averaged over the
 * workers at full precision.  Reading: out_i = fl32( (sum_w g_{w,i}) / W ), the sum
 * taken in fp64 in worker order 0..W-1 (each fp32 value exact in fp64), one fp64
 * division, one rounding.  Row w of g starts w * row_stride values after g. */
int oracle_average_rows(const float *g, int W, int64_t row_stride, int64_t n, float *out)
{
    if (W < 1 || n < 0 || (W > 1 && row_stride < n))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!g || !out)
        return ORACLE_ERR_INVALID;
    for (int64_t i = 0; i < n; ++i) {
        double sum = 0.0;
        for (int w = 0; w < W; ++w)
            sum += (double)g[(int64_t)w * row_stride + i];
        const double mean = sum / (double)W;
        out[i] = (float)mean;
    }
    return ORACLE_OK;
}

/* ------------------------------- O8: LoCo-style compensated gradient quantizer
 * [LOCO] method details, steps 2-4: estimate the compression error by the moving
 * average of past errors, add it to the gradient, compress the sum.  Reading
 * (binary32, unfused; beta and 1 - beta formed in binary64, rounded once):
 *   h = fl32(g + err_avg);  (codes, norms) = QSGD of h, as O7;  y = decoded h as
 *   the W = 1 decode of O7 (fl32(+-level * norm / s));  err_avg = fl32( fl32(beta * err_avg) + fl32((1 - beta) * (h - y)) ).
 * beta = 0 is plain error feedback (err_avg = h - y).  err_avg: fp32 [n] in place.
 * first_index: global index of g[0], as in O7.
 */
int oracle_loco_quantize(const void *g, int g_dtype, float *err_avg, int64_t n, int bucket, int nbits, double beta_d,
                         uint64_t seed, int64_t first_index, uint8_t *codes, float *norms)
{
    if (n < 0 || (g_dtype != 0 && g_dtype != 1))
        return ORACLE_ERR_INVALID;
    if (n == 0)
        return ORACLE_OK;
    if (!g || !err_avg)
        return ORACLE_ERR_INVALID;
    float *h = (float *)malloc((size_t)n * sizeof(float));
    float *y = (float *)malloc((size_t)n * sizeof(float));
    if (!h || !y) {
        free(h);
        free(y);
        return ORACLE_ERR_NOMEM;
    }
    for (int64_t i = 0; i < n; ++i) {
        const float gi = g_dtype == 1 ? oracle_bf16_to_f32(((const uint16_t *)g)[i]) : ((const float *)g)[i];
        h[i] = gi + err_avg[i];
    }
    int rc = oracle_qsgd_quantize(h, 0, n, bucket, nbits, seed, first_index, codes, norms);
    if (rc == ORACLE_OK)
        rc = oracle_qsgd_reduce(1, codes, 0, norms, 0, n, bucket, nbits, y, NULL);
    if (rc == ORACLE_OK) {
        const float beta = (float)beta_d, one_minus_beta = (float)(1.0 - beta_d);
        for (int64_t i = 0; i < n; ++i)
            err_avg[i] = beta * err_avg[i] + one_minus_beta * (h[i] - y[i]);
    }
    free(h);
    free(y);
    return rc;
}
