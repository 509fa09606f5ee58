/*
 * onebit.h -- C ABI of the MI355X (gfx950) library for the data-parallel hot path
 * of 1-bit Adam and for a QSDP-style stochastic-rounding quantizer.
 *
 * Sources ("the pages"):
 *  [1BA]  nubint.ai review of "1-bit Adam: Communication Efficient Large-Scale
 *         Training with Adam's Convergence Speed", "proposed method": full-precision
 *         Adam warmup, then the frozen variance preconditions error-compensated
 *         1-bit compressed momentum SGD.
 *  [DSG]  yfxerp.com "DeepSpeed 1-bit Adam training optimisation ... complete
 *         configuration guide": sec. 3.4 (lr, betas, eps, weight_decay,
 *         bias_correction), sec. 3.5 (exp_avg_mask), sec. 4 (the two phases of
 *         step(), compressed_allreduce with worker_error / server_error,
 *         update = exp_avg / (sqrt(exp_avg_sq) + eps), 1 bit per value),
 *         sec. 7 (errors reset on checkpoint load).
 *  [QSDP] nubint.ai review of "Quantized Distributed Training of Large Models with
 *         Convergence Guarantees", "proposed method": weights rounded at random to
 *         one of the two nearest quantization levels, unbiased.
 *  [QSGD] Alistarh et al., "QSGD: Communication-Efficient SGD via Gradient Quantization
 *         and Encoding", NeurIPS 2017, sec. 3.1 (named by [QSDP] for gradients).
 *  [LOCO] shd-paper.top summary of "LoCo: Low-Bit Communication Adaptor for
 *         Large-scale Model Training", core points and method details.
 *  [PHX]  Salmon et al., "Parallel Random Numbers: As Easy as 1, 2, 3", SC'11.
 *
 * Conventions for every call:
 *  - Every data pointer is a DEVICE pointer owned by the caller unless marked
 *    (host).  Per-element arrays (x, m, v, e, g, x_bf16, server_error, m_out and
 *    the QSDP weights, codes and outputs) must be 16-byte aligned; packed words,
 *    scales and bucket min/max 4-byte aligned; the workspace 8-byte aligned
 *    (ONEBIT_ERR_ALIGN otherwise).  Chunk offsets inside the arrays may be
 *    arbitrary.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *    The returned status covers argument checks and launch errors; a fault during
 *    execution surfaces at the caller's next synchronisation.  Nothing here
 *    allocates device memory or synchronises, except onebit_plan_create /
 *    onebit_plan_destroy (which own the plan's tables).
 *  - Buffers passed to one call must not alias each other unless stated.
 *  - Non-finite inputs are not checked and propagate.
 *  - Hyperparameters are binary64 (as Python floats are); each is rounded to
 *    binary32 once, and 1-beta is formed in binary64 before that rounding.
 *  - Phase control is the caller's: warmup calls for steps t <= freeze_step, then
 *    compressed calls ([DSG] sec. 3.1, sec. 4).  The error reset that [DSG] sec. 7
 *    prescribes after a checkpoint load is the caller zeroing e and server_error.
 */
#ifndef ONEBIT_H
#define ONEBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ONEBIT_OK = 0,
    ONEBIT_ERR_INVALID = 1,     /* bad size, table, pointer or parameter */
    ONEBIT_ERR_ALIGN = 2,       /* a base pointer misses its required alignment */
    ONEBIT_ERR_HIP = 3,         /* a HIP runtime call or launch failed */
    ONEBIT_ERR_NOMEM = 4,       /* plan tables could not be allocated */
    ONEBIT_ERR_UNSUPPORTED = 5  /* valid request the library does not serve */
} onebit_status_t;

typedef enum { ONEBIT_F32 = 0, ONEBIT_BF16 = 1, ONEBIT_F16 = 2 } onebit_dtype_t;

/* Opaque plan: device copies of the chunk, tile and mask tables for one flat
 * parameter vector.  Library-owned, immutable after creation, usable from any
 * stream of the device that was current at creation. */
typedef struct onebit_plan_s *onebit_plan_t;

/* Human-readable name of a status code (static storage). */
const char *onebit_status_string(onebit_status_t status);

/* Build a plan for a flat vector of n = chunk_offsets[n_chunks] elements.
 *  chunk_offsets  (host) n_chunks+1 entries, [0] = 0, non-decreasing.  One fp32
 *                 scale per chunk; chunk j owns ceil(n_j/32) consecutive packed
 *                 words starting at sum_{k<j} ceil(n_k/32).
 *  tensor_offsets (host, nullable) n_tensors+1 entries, [0] = 0, non-decreasing,
 *                 last = n.  tensor_keep (host, nullable) n_tensors flags:
 *                 0 = masked (the momentum mask of [DSG] sec. 3.5, per tensor).
 *  n_chunks >= 0; n_chunks = 0 gives an empty plan whose calls do nothing.
 * Allocates device memory (the only allocating call besides the workspace the
 * caller provides). */
onebit_status_t onebit_plan_create(const int64_t *chunk_offsets, int64_t n_chunks,
                                   const int64_t *tensor_offsets, const uint8_t *tensor_keep,
                                   int64_t n_tensors, onebit_plan_t *out);
void onebit_plan_destroy(onebit_plan_t plan);

/* Host only (touches no device): the tables onebit_plan_create would build, for
 * inspection and host-side tests.  Same validation and status codes.  Outputs are
 * host arrays and nullable: *n_tiles, *n_words, *n_mask_iv; out_tiles
 * [n_tiles][6] = {first element, first packed word, length (0..2048), chunk,
 * mask_lo, mask_hi}, where masked intervals [mask_lo, mask_hi) touch the tile and
 * mask_lo = -1 means one masked interval covers it; out_mask_iv [n_mask_iv][2] =
 * merged masked element ranges [a, b).  Tiles are 2048 elements, each chunk cut
 * from its start (an empty chunk gets one empty tile). */
onebit_status_t onebit_plan_host_tables(const int64_t *chunk_offsets, int64_t n_chunks,
                                        const int64_t *tensor_offsets, const uint8_t *tensor_keep,
                                        int64_t n_tensors, int64_t *n_tiles, int64_t *n_words,
                                        int64_t *out_tiles, int64_t *n_mask_iv, int64_t *out_mask_iv);
int64_t onebit_plan_elements(onebit_plan_t plan); /* n */
int64_t onebit_plan_chunks(onebit_plan_t plan);   /* n_chunks */
int64_t onebit_plan_words(onebit_plan_t plan);    /* sum_j ceil(n_j / 32) */

/* Device scratch (bytes) that onebit_compress_update / onebit_server_reduce need
 * for this plan: per-tile partial norms and per-chunk published scales.  The
 * caller allocates it and must zero it once before first use (onebit_workspace_init
 * does that on a stream); every completed call leaves it ready for the next one,
 * for this or any other plan whose workspace size fits.  One workspace must not be
 * used by two calls that may overlap in time. */
size_t onebit_plan_workspace_bytes(onebit_plan_t plan);
onebit_status_t onebit_workspace_init(void *workspace, size_t bytes, void *stream);

/* Copy the workspace's error word to *out (host) and synchronise `stream`.
 * 0: every cross-workgroup wait of the calls since the workspace was zeroed
 * ended normally; non-zero: a bounded wait gave up (the outputs of that call are
 * not valid).  Intended for tests and diagnostics. */
onebit_status_t onebit_workspace_status(const void *workspace, uint64_t *out, void *stream);

/* Diagnostics: co-resident workgroups of the one-pass compression kernel on the
 * current device (the grid it is launched with at most), and a plan's tile
 * split: out6 (host) = {tiles, one-pass tiles, two-pass tiles, capacity used,
 * largest chunk in tiles, 1 if every chunk starts on a multiple of 4 elements}. */
int32_t onebit_device_resident_capacity(void);
void onebit_plan_stats(onebit_plan_t plan, int64_t *out6);
/* Largest chunk (elements) the one-pass path takes on the current device;
 * larger chunks take the two-pass path. */
int64_t onebit_onepass_max_elements(void);

/* Diagnostics: the number of re-polls after which a cross-workgroup wait gives up
 * (0 restores the default, 2^20).  A wait that gives up stores an error code in the
 * workspace (read it with onebit_workspace_status) and the call still completes,
 * with unspecified results; a workspace with an error must be re-initialized with
 * onebit_workspace_init before further use.  Applies to later calls from any host
 * thread. */
void onebit_set_spin_limit(uint32_t limit);

/* Diagnostics: launch the one-pass compression kernel with at most `cap`
 * workgroups (0 or a negative value removes the cap), so that the chunk-norm
 * exchange can be exercised with fewer resident workgroups than the device holds.
 * A call whose plan has a one-pass chunk of more than 3 * grid tiles (the most the
 * kernel's progress argument allows) returns ONEBIT_ERR_INVALID and launches
 * nothing.  Applies to later calls from any host thread. */
void onebit_set_grid_cap(int32_t cap);

/* Launch timing.  Between onebit_profile_begin and onebit_profile_end every kernel
 * the library launches is bracketed by two HIP events on its own stream.
 * onebit_profile_end synchronises on those events and returns, per kernel class,
 * the summed elapsed milliseconds and the launch count (host arrays of
 * ONEBIT_PROFILE_CLASSES entries, nullable).  Classes: 0 warmup, 1/2/3 worker
 * compression pass 1 / one-pass / pass 2, 4 quantize, 5 dequantize, 6/7/8 server
 * pass 1 / one-pass / pass 2, 9 chunk-norm finalization of two-pass chunks, 10
 * momentum update, 11 QSGD quantize, 12 QSGD reduce, 13 LoCo quantize.  A QSGD or
 * LoCo call with buckets of 1024 and a ragged last bucket launches two kernels (whole
 * buckets, then the last one) inside one bracket, counted as one launch.
 * onebit_profile_begin_classes brackets only the classes whose bit (1 << class) is
 * set in class_mask, so that a timed region carries the events of the kernel being
 * measured and no others (each event adds a few microseconds between launches).
 * Not thread-safe; diagnostics only. */
#define ONEBIT_PROFILE_CLASSES 14
void onebit_profile_begin(void);
void onebit_profile_begin_classes(uint32_t class_mask);
onebit_status_t onebit_profile_end(double *total_ms, int64_t *launches);

/* Diagnostics: a plain streaming kernel over `reads` fp32 input streams and `writes`
 * output streams of n elements each (out_k = sum of the inputs + k), to measure what
 * HBM delivers for that mix on this device.  in / out: DEVICE arrays of `reads` /
 * `writes` device pointers, each 16-byte aligned; n a multiple of 4.  Supported
 * mixes (reads + writes): 1 + 0 (read-only: the inputs are left unchanged unless a
 * sum equals -3e38), 0 + 1 (write-only), 1 + 1, 2 + 1, 3 + 1 (near the
 * compress-only worker's), 1 + 2, 2 + 2 (near the server stage's), 4 + 2 and 5 + 3
 * (the update-mode compression kernel's); others return ONEBIT_ERR_UNSUPPORTED.  grid:
 * number of workgroups; block: threads per workgroup, 256, 512 or 1024
 * (ONEBIT_ERR_INVALID otherwise).  policy 1: loads and stores use the streaming
 * (nontemporal) cache policy, as the compression kernels do; 0: the default
 * policy; 2: streaming policy with every wave's loads going straight into LDS
 * (the 16-byte global-to-LDS loads of gfx950), double-buffered, and read back from
 * there, so the next loads are in flight without holding registers (block must be
 * 256 and reads at least 1); any other policy or combination: ONEBIT_ERR_INVALID. */
onebit_status_t onebit_stream_probe(const float *const *in, int reads, float *const *out, int writes,
                                    int64_t n, int grid, int block, int policy, void *stream);

/* Diagnostics: the cost of the quantizers' random numbers alone (QSDP, "Proposed
 * method": unbiased stochastic rounding, here with Philox4x32-10 keyed by the
 * seed's low / high words and counter = block index).  Thread t of a grid of
 * grid x block threads draws the blocks t, t + T, t + 2T, ... below n_blocks
 * (T = grid x block) and stores the XOR of the four words of all its blocks to
 * out[t]: a DEVICE array of grid x block words.  One block serves four quantized
 * elements.  block: 256, 512 or 1024; grid >= 1; n_blocks >= 0 (else
 * ONEBIT_ERR_INVALID). */
onebit_status_t onebit_philox_probe(uint64_t seed, int64_t n_blocks, uint32_t *out, int grid, int block,
                                    void *stream);

/* Warmup step t (1-based) of full-precision Adam over n elements ([DSG] sec. 4,
 * phase one; [1BA]):  m = b1 m + (1-b1) g;  v = b2 v + (1-b2) g^2;
 *   x -= lr * ( mhat / (sqrt(vhat) + eps) + weight_decay * x ),
 * with mhat = m / (1-b1^t), vhat = v / (1-b2^t) when bias_correction != 0, else
 * mhat = m, vhat = v.  x, m, v: fp32 [n] in place.  g: [n] fp32, bf16 or fp16
 * (widened exactly). */
onebit_status_t onebit_adam_warmup_step(float *x, float *m, float *v, const void *g,
                                        onebit_dtype_t g_dtype, int64_t n, double lr,
                                        double beta1, double beta2, double eps,
                                        double weight_decay, int bias_correction, int64_t step,
                                        void *stream);

/* One compressed step on one worker's share ([DSG] sec. 4, phase two; sec. 3.5):
 *   m1 = b1 m + (1-b1) g;  c = m1 + e                       (binary32, unfused)
 *   scale_j = sqrt(sum_{i in j} c_i^2) / sqrt(n_j)          (fp64 sum, one rounding)
 *   bit_i = (c_i < 0);  q_i = bit_i ? -scale_j : +scale_j;  e = c - q;  m = q
 *   masked tensors: m = 0, e = 0 (bits and scale still from c)
 *   x -= lr * ( m / (sqrt(v) + eps) + weight_decay * x );  x_bf16 = bf16(x)
 * g: [n] fp32, bf16 or fp16 (widened exactly).  m, e, x: fp32 [n] in place; v: fp32
 * [n] read-only (frozen).
 * bits: uint32 [plan_words] out, least significant bit first, every chunk starting
 * on a word boundary, pad bits 0.  scales: fp32 [n_chunks] out.  x_bf16: uint16
 * [n] out, nullable.  Compress-only (the worker half of the compressed
 * all-reduce): pass v = x = x_bf16 = NULL; then m is read and NOT written and only
 * e, bits and scales are produced.  workspace: onebit_plan_workspace_bytes bytes. */
onebit_status_t onebit_compress_update(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                       float *m, float *e, const float *v, float *x,
                                       uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                       double beta1, double eps, double weight_decay,
                                       void *workspace, void *stream);

/* onebit_compress_update with the momentum kept in its compressed form.  After
 * every compressed step m is exactly the decompression of that step's sign words
 * and chunk scales (the worker's own in the fused single-worker step, 0 in masked
 * tensors; the server's in the W-worker step, times the element mask), so it need
 * not be stored as fp32: this call takes those words and scales as m,
 *   m_i = bit_i(m_bits) ? -m_scales[j] : +m_scales[j],  then
 *   m_i = m_i * 0 where m_mask[i] == 0 (m_mask: uint8 [n], 4-byte aligned, nullable; a signed zero,
 *   as onebit_momentum_update leaves it) and, in update mode, m_i = +0 in the
 *   plan's masked tensors (as onebit_compress_update leaves them),
 * performs the same step as onebit_compress_update (bits, scales, e, x, x_bf16
 * identical bit for bit) and writes no m.  Update mode (v, x given): the new
 * momentum is (bits, scales); 24.25 bytes per element instead of 32.125.
 * Compress-only mode (v = x = x_bf16 = NULL): the worker half of the all-reduce
 * with m the previous server result.  m_bits: uint32 [plan_words], m_scales: fp32
 * [n_chunks], both read-only and distinct from bits and scales (callers alternate
 * two pairs).  The first compressed step after the warmup, whose m is the fp32
 * Adam momentum, uses onebit_compress_update. */
onebit_status_t onebit_compress_update_packed(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                              const uint32_t *m_bits, const float *m_scales,
                                              const uint8_t *m_mask, float *e, const float *v, float *x,
                                              uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                              double beta1, double eps, double weight_decay,
                                              void *workspace, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): onebit_compress_update
 * with the same arguments and results, minus the workspace.  Its kernels use an
 * 8 MiB scratch area inside the library (one per device, held until the process
 * ends) instead; the call itself allocates nothing.  Limit: the plan's chunks +
 * tiles (one tile per 2048 elements of a chunk, rounded up) + 1 may not exceed
 * 2^20 (about 2.1e9 elements); a larger plan returns ONEBIT_ERR_NOMEM and launches
 * nothing.  Each call first clears the scratch words it uses (a kernel, no memset),
 * so a failed earlier call does not affect it.  wait_status: nullable DEVICE
 * uint64, 8-byte aligned; it receives the call's error word after the call's
 * kernels (0: every cross-workgroup wait ended normally; non-zero: a bounded wait
 * gave up and the outputs are not valid; 0 for a plan with no chunks).  Every call
 * on one GPU shares that GPU's scratch: calls that may overlap in time on one GPU
 * (several streams or host threads) race and give unspecified results.  Errors as
 * onebit_compress_update, plus ONEBIT_ERR_HIP if the scratch's address cannot be
 * obtained. */
onebit_status_t onebit_compress_update_static(onebit_plan_t plan, const void *g, onebit_dtype_t g_dtype,
                                              float *m, float *e, const float *v, float *x,
                                              uint16_t *x_bf16, uint32_t *bits, float *scales, double lr,
                                              double beta1, double eps, double weight_decay,
                                              uint64_t *wait_status, void *stream);

/* Server stage of the compressed all-reduce over W workers' streams held in one
 * GPU's memory ([DSG] sec. 4, server_error; [1BA] "proposed method"):
 *   a_i = fl32( (sum_{w=0..W-1} (bit_{w,i} ? -s_{w,j} : +s_{w,j})) / W )   (fp64)
 *   c = a + server_error;  then the compressor above with server_error as e;
 *   m_out = decompressed server result (nullable; may alias nothing else).
 * worker_bits: uint32 [W][plan_words] row-major; worker_scales: fp32 [W][n_chunks].
 * server_error: fp32 [n] in place; server_bits [plan_words], server_scales
 * [n_chunks] out.  1 <= W <= 1024. */
onebit_status_t onebit_server_reduce(onebit_plan_t plan, int W, const uint32_t *worker_bits,
                                     const float *worker_scales, float *server_error,
                                     uint32_t *server_bits, float *server_scales, float *m_out,
                                     void *workspace, void *stream);

/* The worker's finish after the compressed all-reduce ([DSG] sec. 3.5, exp_avg_mask;
 * sec. 4, phase two), elementwise over n elements, in binary32, unfused:
 *   m = m * mask;  x -= lr * ( m / (sqrt(v) + eps) + weight_decay * x );  x_bf16 = bf16(x)
 * m: fp32 [n] in place (the all-reduced momentum, e.g. m_out of the server stage
 * or its broadcast copy); written only when a mask is given.  mask: uint8 [n],
 * non-zero = keep, nullable (no mask).  v: fp32 [n] read-only (frozen).  x: fp32 [n]
 * in place.  x_bf16: uint16 [n] out, nullable.  All arrays 16-byte aligned.  With
 * no mask and the server's output as m, onebit_compress_update in compress-only
 * mode -> onebit_server_reduce -> this call reproduces onebit_compress_update's
 * own update for one worker bit for bit. */
onebit_status_t onebit_momentum_update(float *m, const uint8_t *mask, const float *v, float *x,
                                       uint16_t *x_bf16, int64_t n, double lr, double eps,
                                       double weight_decay, void *stream);

/* onebit_momentum_update with the all-reduced momentum in its compressed form (the
 * server's sign words and chunk scales of `plan`):
 *   m_i = (bit_i ? -m_scales[j] : +m_scales[j]) * (mask_i ? 1 : 0)   (mask nullable: all kept)
 *   x -= lr * ( m / (sqrt(v) + eps) + weight_decay * x );  x_bf16 = bf16(x)
 * with the same binary32 operations as onebit_momentum_update; no m is written (the
 * next step's workers take the same words, scales and mask as their packed m).
 * m_bits: uint32 [plan_words]; m_scales: fp32 [n_chunks]; mask: uint8 [n]; v: fp32
 * [n] read-only; x: fp32 [n] in place; x_bf16: uint16 [n] out, nullable.  v, x,
 * x_bf16 16-byte aligned. */
onebit_status_t onebit_momentum_update_packed(onebit_plan_t plan, const uint32_t *m_bits,
                                              const float *m_scales, const uint8_t *mask, const float *v,
                                              float *x, uint16_t *x_bf16, double lr, double eps,
                                              double weight_decay, void *stream);

/* Decompression of a plan's sign words and chunk scales (the all-gather-decompress
 * of the compressed all-reduce, [DSG] sec. 4: every value travels as one bit and
 * is rebuilt as +-scale; sec. 3.5: the momentum is then masked per element):
 *   out_i = (bit_i ? -scales[j] : +scales[j]) * (mask_i ? 1 : 0)   (mask nullable: +-scales[j])
 * with the product one binary32 multiplication (a masked negative value gives -0,
 * as onebit_momentum_update leaves it).  bits: uint32 [plan_words], 4-byte aligned;
 * scales: fp32 [n_chunks]; mask: uint8 [n]; out: fp32 [n], 16-byte aligned. */
onebit_status_t onebit_decompress(onebit_plan_t plan, const uint32_t *bits, const float *scales,
                                  const uint8_t *mask, float *out, void *stream);

/* The full-precision gradient exchange of the warmup phase ([DSG] sec. 4, phase
 * one: Adam runs on the workers' averaged gradient), simulated over W workers'
 * gradients held in one GPU's memory:
 *   out_i = fl32( (sum_{w=0..W-1} g_{w,i}) / W )
 * with the sum in fp64 in worker order (each value widened exactly), one fp64
 * division (a product with 1/W when W is a power of two, the same value), one
 * rounding.  g: W rows of n fp32, bf16 or fp16 values, row w starting
 * w * row_stride elements after g (row_stride >= n when W > 1); out: fp32 [n],
 * 16-byte aligned.  1 <= W <= 65536. */
onebit_status_t onebit_average_rows(const void *g, onebit_dtype_t g_dtype, int W, int64_t row_stride, int64_t n,
                                    float *out, void *stream);

/* QSGD gradient quantizer, the gradient side of QSDP ([QSDP] "proposed method":
 * gradients take the standard unbiased compressor of Alistarh et al. 2017; [QSGD]
 * sec. 3.1), per bucket of `bucket` elements (the last one may be short):
 *   norm = fl32( sqrt( sum g^2 ) )            (fp64 sum of exact squares, fp64 sqrt)
 *   s = 2^(bits-1) - 1;  t = fl32(|g| / norm);  v = fl32(t * s);  l = floor(v);  p = v - l
 *   u = Philox4x32-10(key = seed, counter = (i >> 2, 0, 0))[i & 3]      ([PHX])
 *   level = l + (u < floor(p * 2^32));  code = (g < 0) << (bits-1) | level
 *   a bucket of zeros: norm 0, codes 0.
 * g: [n] fp32, bf16 or fp16 (widened exactly), 16-byte aligned.  codes: uint8, bits 4:
 * two per byte, even element in the low nibble, ceil(n/2) bytes, pad nibble 0; bits
 * 8: n bytes; 16-byte aligned.  norms: fp32 [ceil(n/bucket)] out.  1 <= bucket <=
 * 65536, bucket even when bits == 4.  Use a seed distinct from the weights'. */
onebit_status_t qsgd_quantize(const void *g, onebit_dtype_t g_dtype, int64_t n, int bucket, int bits,
                              uint64_t seed, uint8_t *codes, float *norms, void *stream);

/* LoCo-style compensated gradient quantizer ([LOCO] method details: the gradient is
 * compensated, before compression, by a moving average of the past compression
 * errors; the page gives no formula, so these steps are this library's reading):
 *   h = fl32(g + err_avg);  codes, norms = qsgd_quantize of h (same seed use)
 *   y = h decoded (W = 1 of qsgd_reduce);  err_avg = fl32( fl32(beta err_avg) + fl32((1-beta)(h - y)) )
 * beta = 0 is plain error feedback.  err_avg: fp32 [n] in place, 16-byte aligned;
 * 0 <= beta <= 1 (rounded to binary32 once, 1 - beta formed in binary64).  Other
 * arguments as qsgd_quantize. */
onebit_status_t loco_quantize(const void *g, onebit_dtype_t g_dtype, float *err_avg, int64_t n, int bucket,
                              int bits, double beta, uint64_t seed, uint8_t *codes, float *norms,
                              void *stream);

/* Decode and average W workers' QSGD streams of the same n elements (the shard
 * owner's half of a quantized reduce-scatter; W = 1 is plain decoding):
 *   y_{w,i} = +-level * fl32(norm_{w,b} / s)   (exact in fp64; sign from the code's top bit)
 *   out_i = fl32( (sum_{w=0..W-1} y_{w,i}) / W )          (fp64 sum in worker order)
 * codes: worker w's codes at codes + w * code_stride bytes (code_stride >= code
 * bytes of n and a multiple of 16 when W > 1; base 16-byte aligned).  norms:
 * worker w's at norms + w * norm_stride (>= ceil(n/bucket) when W > 1).  out_f32
 * [n] and/or out_bf16 [n] (round to nearest even), at least one, 16-byte aligned.
 * 1 <= W <= 65536. */
onebit_status_t qsgd_reduce(int W, const uint8_t *codes, int64_t code_stride, const float *norms,
                            int64_t norm_stride, int64_t n, int bucket, int bits, float *out_f32,
                            uint16_t *out_bf16, void *stream);

/* QSDP-style unbiased stochastic rounding of bf16 weights ([QSDP] "proposed
 * method"), per bucket of `bucket` elements (the last one may be short):
 *   min, max of the bucket (exact);  delta = fl32(fl32(max - min) / L), L = 2^bits - 1
 *   t = fl32(fl32(x - min) / delta);  k = min(floor(t), L);  p = t - k
 *   u = Philox4x32-10(key = seed, counter = (i >> 2, 0, 0))[i & 3]   ([PHX])
 *   code = min(k + (u < floor(p * 2^32)), L);  code = 0 when delta == 0.
 * bits 4: codes packed two per byte, even element in the low nibble, pad nibble 0,
 * ceil(n/2) bytes.  bits 8: one byte per element.  bucket_min/max: fp32
 * [ceil(n/bucket)] out.  1 <= bucket <= 65536, bucket even when bits == 4. */
onebit_status_t qsdp_quantize(const uint16_t *x_bf16, int64_t n, int bucket, int bits,
                              uint64_t seed, uint8_t *codes, float *bucket_min, float *bucket_max,
                              void *stream);

/* Inverse map: y = fl32(min + fl32(code * delta)) with delta as above.
 * out_bf16: uint16 [n] (round to nearest even), nullable; out_f32: fp32 [n],
 * nullable. */
onebit_status_t qsdp_dequantize(const uint8_t *codes, const float *bucket_min,
                                const float *bucket_max, int64_t n, int bucket, int bits,
                                uint16_t *out_bf16, float *out_f32, void *stream);

/* Error statistics of one dequantized draw y (fp32 [n], e.g. out_f32 above)
 * against the bf16 weights x, for the unbiasedness measurement over repeated
 * seeds ([QSDP] "proposed method": the expectation of the quantized weight equals
 * the weight):  sums[0] += sum_i (y_i - x_i),  sums[1] += sum_i (y_i - x_i)^2,
 * both fp64 (device [2]); ysum (device fp64 [n], nullable): ysum_i += y_i.
 * partials: device scratch of 2 * QSDP_STATS_PARTIALS doubles.  The reduction
 * order is fixed, so results are bitwise reproducible.  x_bf16, y and ysum must be
 * 16-byte aligned (ONEBIT_ERR_ALIGN otherwise). */
#define QSDP_STATS_PARTIALS 1024
onebit_status_t qsdp_error_stats(const uint16_t *x_bf16, const float *y, int64_t n, double *ysum,
                                 double *sums, double *partials, void *stream);

/* *out (device fp64) = sum_i | ysum_i / seeds - x_i |: with the mean abs error of
 * the seed-averaged quantizer, divide by n.  Same partials scratch; x_bf16 and
 * ysum 16-byte aligned. */
onebit_status_t qsdp_mean_abs_error(const uint16_t *x_bf16, const double *ysum, int64_t n, int seeds,
                                    double *out, double *partials, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ONEBIT_H */
