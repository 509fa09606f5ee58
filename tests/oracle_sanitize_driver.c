/* Drives every function of the CPU oracle (oracle/onebit_oracle.c) over edge-case
 * inputs, for a build with -fsanitize=address,undefined: empty and one-element
 * vectors, lengths around the 32-bit word boundary, ragged and empty chunks, masked
 * tensors, 1..3 workers, odd QSDP / QSGD lengths (pad nibble), bucket sizes 2 and
 * 1024, LoCo, the finish with and without a mask, and the argument checks.  Every
 * output buffer is sized exactly, so an out-of-bounds access is reported by the
 * sanitizer.  Prints "ok" and exits 0 when every call returned the expected status.
 * Test infrastructure only. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_adam_warmup_step(float *x, float *m, float *v, const float *g, int64_t n, double lr, double beta1,
                            double beta2, double eps, double weight_decay, int bias_correction, int64_t step);
int oracle_compress_update(const int64_t *chunk_off, int64_t n_chunks, const int64_t *tensor_off,
                           const uint8_t *tensor_keep, int64_t n_tensors, const float *g, float *m, float *e,
                           const float *v, float *x, uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                           double beta1, double eps, double weight_decay, int identity);
int oracle_server_reduce(const int64_t *chunk_off, int64_t n_chunks, int W, const uint32_t *worker_bits,
                         const float *worker_scales, float *server_error, uint32_t *server_bits,
                         float *server_scales, float *m_out);
int oracle_momentum_update(float *m, const uint8_t *mask, const float *v, float *x, uint16_t *x_bf16, int64_t n,
                           double lr, double eps, double weight_decay);
int oracle_decompress(const int64_t *chunk_off, int64_t n_chunks, const uint32_t *bits, const float *scales,
                      float *out);
int oracle_qsdp_quantize(const uint16_t *x_bf16, int64_t n, int bucket, int nbits, uint64_t seed,
                         int64_t first_index, uint8_t *codes, float *bucket_min, float *bucket_max);
int oracle_qsdp_dequantize(const uint8_t *codes, const float *bucket_min, const float *bucket_max, int64_t n,
                           int bucket, int nbits, uint16_t *out_bf16, float *out_f32);
int oracle_qsgd_quantize(const void *g, int g_dtype, int64_t n, int bucket, int nbits, uint64_t seed,
                         int64_t first_index, uint8_t *codes, float *norms);
int oracle_qsgd_reduce(int W, const uint8_t *codes, int64_t code_stride, const float *norms, int64_t norm_stride,
                       int64_t n, int bucket, int nbits, float *out_f32, uint16_t *out_bf16);
int oracle_loco_quantize(const void *g, int g_dtype, float *err_avg, int64_t n, int bucket, int nbits, double beta,
                         uint64_t seed, int64_t first_index, uint8_t *codes, float *norms);

static int failures = 0;
static uint64_t rng_state = 0x1234567887654321ull;

static float frand(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return ((float)(int32_t)(rng_state >> 32)) * 4.6566e-10f * 1e-3f;
}

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "%s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

/* exactly sized heap copies, so that any overrun is caught */
static float *fvec(int64_t n)
{
    float *p = (float *)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i)
        p[i] = frand();
    return p;
}

static int64_t words_of(const int64_t *off, int64_t nc)
{
    int64_t w = 0;
    for (int64_t j = 0; j < nc; ++j)
        w += (off[j + 1] - off[j] + 31) / 32;
    return w;
}

static void compress_case(const int64_t *off, int64_t nc, const int64_t *toff, const uint8_t *keep, int64_t nt)
{
    const int64_t n = off[nc];
    const int64_t words = words_of(off, nc);
    float *g = fvec(n), *m = fvec(n), *e = fvec(n), *v = fvec(n), *x = fvec(n);
    for (int64_t i = 0; i < n; ++i)
        v[i] = v[i] * v[i] + 1e-7f;
    uint16_t *xb = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * 2);
    uint32_t *bits = (uint32_t *)malloc((size_t)(words > 0 ? words : 1) * 4);
    float *scales = (float *)malloc((size_t)(nc > 0 ? nc : 1) * 4);
    expect(oracle_compress_update(off, nc, toff, keep, nt, g, m, e, v, x, xb, bits, scales, 1e-3, 0.9, 1e-8, 0.01, 0),
           0, "compress update");
    expect(oracle_compress_update(off, nc, toff, keep, nt, g, m, e, NULL, NULL, NULL, bits, scales, 0.0, 0.9, 1e-8,
                                  0.0, 0),
           0, "compress only");
    expect(oracle_compress_update(off, nc, toff, keep, nt, g, m, e, v, x, NULL, bits, scales, 1e-3, 0.9, 1e-8, 0.0,
                                  1),
           0, "identity compressor");
    float *out = fvec(n);
    expect(oracle_decompress(off, nc, bits, scales, out), 0, "decompress");
    for (int W = 1; W <= 3; ++W) {
        uint32_t *wb = (uint32_t *)malloc((size_t)(W * (words > 0 ? words : 1)) * 4);
        float *ws = (float *)malloc((size_t)(W * (nc > 0 ? nc : 1)) * 4);
        for (int w = 0; w < W; ++w) {
            if (words > 0)
                memcpy(wb + w * words, bits, (size_t)words * 4);
            if (nc > 0)
                memcpy(ws + w * nc, scales, (size_t)nc * 4);
        }
        float *es = fvec(n), *mo = fvec(n);
        uint32_t *sb = (uint32_t *)malloc((size_t)(words > 0 ? words : 1) * 4);
        float *ss = (float *)malloc((size_t)(nc > 0 ? nc : 1) * 4);
        expect(oracle_server_reduce(off, nc, W, wb, ws, es, sb, ss, mo), 0, "server");
        expect(oracle_server_reduce(off, nc, W, wb, ws, es, sb, ss, NULL), 0, "server without m");
        free(wb), free(ws), free(es), free(mo), free(sb), free(ss);
    }
    uint8_t *mask = (uint8_t *)malloc((size_t)(n > 0 ? n : 1));
    for (int64_t i = 0; i < n; ++i)
        mask[i] = (uint8_t)(i % 3 != 0);
    expect(oracle_momentum_update(m, mask, v, x, xb, n, 1e-3, 1e-8, 0.01), 0, "finish with mask");
    expect(oracle_momentum_update(m, NULL, v, x, NULL, n, 1e-3, 1e-8, 0.0), 0, "finish");
    expect(oracle_adam_warmup_step(x, m, v, g, n, 1e-3, 0.9, 0.999, 1e-8, 0.01, 1, 3), 0, "warmup");
    free(g), free(m), free(e), free(v), free(x), free(xb), free(bits), free(scales), free(out), free(mask);
}

static void quant_case(int64_t n, int bucket)
{
    uint16_t *xb = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * 2);
    float *gf = fvec(n);
    for (int64_t i = 0; i < n; ++i)
        xb[i] = (uint16_t)(0x3c00u + (uint32_t)(i * 37u % 1024u));
    const int64_t nb = (n + bucket - 1) / bucket;
    for (int bits = 4; bits <= 8; bits += 4) {
        const int64_t cb = bits == 4 ? (n + 1) / 2 : n;
        uint8_t *codes = (uint8_t *)malloc((size_t)(cb > 0 ? cb : 1));
        float *mn = (float *)malloc((size_t)(nb > 0 ? nb : 1) * 4), *mx = (float *)malloc((size_t)(nb > 0 ? nb : 1) * 4);
        expect(oracle_qsdp_quantize(xb, n, bucket, bits, 99, 0, codes, mn, mx), 0, "qsdp quantize");
        uint16_t *yb = (uint16_t *)malloc((size_t)(n > 0 ? n : 1) * 2);
        float *yf = (float *)malloc((size_t)(n > 0 ? n : 1) * 4);
        expect(oracle_qsdp_dequantize(codes, mn, mx, n, bucket, bits, yb, yf), 0, "qsdp dequantize");
        expect(oracle_qsgd_quantize(gf, 0, n, bucket, bits, 7, 0, codes, mn), 0, "qsgd quantize f32");
        expect(oracle_qsgd_quantize(xb, 1, n, bucket, bits, 7, 0, codes, mn), 0, "qsgd quantize bf16");
        expect(oracle_qsgd_reduce(1, codes, 0, mn, 0, n, bucket, bits, yf, yb), 0, "qsgd reduce");
        uint8_t *c3 = (uint8_t *)malloc((size_t)(3 * (cb > 0 ? cb : 1)));
        float *n3 = (float *)malloc((size_t)(3 * (nb > 0 ? nb : 1)) * 4);
        for (int w = 0; w < 3; ++w) {
            if (cb > 0)
                memcpy(c3 + w * cb, codes, (size_t)cb);
            if (nb > 0)
                memcpy(n3 + w * nb, mn, (size_t)nb * 4);
        }
        expect(oracle_qsgd_reduce(3, c3, cb, n3, nb, n, bucket, bits, yf, NULL), 0, "qsgd reduce of 3");
        float *err = fvec(n);
        expect(oracle_loco_quantize(gf, 0, err, n, bucket, bits, 0.9, 5, 0, codes, mn), 0, "loco");
        expect(oracle_loco_quantize(xb, 1, err, n, bucket, bits, 0.0, 5, 0, codes, mn), 0, "loco bf16");
        free(codes), free(mn), free(mx), free(yb), free(yf), free(c3), free(n3), free(err);
    }
    free(xb), free(gf);
}

int main(void)
{
    const int64_t lens[] = {0, 1, 31, 32, 33, 63, 65, 4095, 4097};
    for (size_t a = 0; a < sizeof lens / sizeof lens[0]; ++a) {
        const int64_t off1[2] = {0, lens[a]};
        compress_case(off1, 1, NULL, NULL, 0);
    }
    const int64_t off[6] = {0, 3, 3, 40, 1070, 5000};     /* an empty chunk, unaligned starts */
    const int64_t toff[5] = {0, 10, 38, 2000, 5000};
    const uint8_t keep[4] = {1, 0, 0, 1};
    compress_case(off, 5, toff, keep, 4);
    compress_case(off, 5, NULL, NULL, 0);
    const int64_t none[1] = {0};
    compress_case(none, 0, NULL, NULL, 0);
    const int64_t qn[] = {0, 1, 2, 3, 1023, 1024, 1025, 2049};
    for (size_t a = 0; a < sizeof qn / sizeof qn[0]; ++a) {
        quant_case(qn[a], 1024);
        quant_case(qn[a], 2);
    }
    /* argument checks */
    const int64_t bad[3] = {0, 5, 3};
    float f[8] = {0};
    uint32_t b[2];
    float s[2];
    expect(oracle_compress_update(bad, 2, NULL, NULL, 0, f, f, f, NULL, NULL, NULL, b, s, 0, 0.9, 1e-8, 0, 0), 1,
           "decreasing offsets");
    expect(oracle_server_reduce(off, 5, 0, NULL, NULL, NULL, NULL, NULL, NULL), 1, "zero workers");
    expect(oracle_qsdp_quantize(NULL, 4, 0, 4, 0, 0, NULL, NULL, NULL), 1, "zero bucket");
    expect(oracle_qsgd_quantize(f, 0, 4, 3, 4, 0, 0, NULL, NULL), 1, "odd 4-bit bucket");
    if (failures) {
        fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
