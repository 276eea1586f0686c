/*
 * fp8q -- FP8 (E4M3) weight-quantized linear layers on AMD Instinct MI355X (gfx950).
 *
 * A C ABI over hand-written HIP kernels.  Every pointer argument is a DEVICE
 * pointer on the device that owns `stream` unless the comment says otherwise;
 * every call only enqueues work on `stream` and returns.  The library never
 * allocates, frees or synchronizes device memory: the caller owns every
 * buffer, including the scratch workspaces whose sizes the *_workspace_size
 * queries return.
 *
 * Layouts are row-major with a contiguous last dimension and a leading
 * dimension (row stride, in elements) `ld_*`.  A weight has the [out, in]
 * layout of a linear layer: row n holds output channel n.  The linear layer
 * computes Y = X . W^T.
 *
 * Sources (web pages on FP8 quantization of Llama 3):
 *   "FP8量化与长上下文实测：Llama 3 70B部署优化指南" (called "the deployment
 *   guide" below) §1.1 gives the E4M3 format, §1.2 the granularity (weights
 *   per channel, activations per tensor) and §3.1 the conversion recipe;
 *   "Llama 3 精读" FP8 + 128K write-up (called "the write-up") §3.1 step 3
 *   names the FP8 MatMul modes, §3.1 step 2 and §5.3 tip 2 the EMA
 *   activation scale; the deployment guide §3.2 gives the FP8 KV cache and
 *   §4.3 per-group weight scales.
 *
 * Errors.  Arguments are validated on the host before anything is enqueued;
 * on any error nothing is launched and a status other than FP8Q_OK is
 * returned.  fp8q_last_error() gives a thread-local description of the most
 * recent error.  NaN or infinite inputs are outside the method's domain: they
 * are reported through an optional device flag (set to 1, never cleared by
 * the library), and the codes they produce are unspecified.
 *
 * Pointer checks.  Every pointer a kernel dereferences is checked to be
 * device memory on the stream's device (hipPointerGetAttributes).  Each
 * thread remembers the last 32 device allocations it has checked, and a
 * pointer inside one of them is not queried again (the query costs
 * microseconds per pointer in a process with many allocations).  Not
 * detected while an allocation is remembered: freeing it and handing its
 * address range to host memory.  Setting the environment variable
 * FP8Q_POINTER_CACHE=0 turns the memory off.
 *
 * Threading.  Calls are thread-safe; the shared state is a per-device cache
 * of device properties (the pointer memory above is per thread).  Two calls
 * that share a workspace must be ordered on one stream.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 3

typedef enum {
    FP8Q_OK = 0,
    FP8Q_ERR_INVALID_ARG = 1,   /* null pointer, bad size/stride/alignment, host pointer,
                                   aliasing, wrong mode/scale combination */
    FP8Q_ERR_UNSUPPORTED = 2,   /* the stream's device is not a gfx950 GPU */
    FP8Q_ERR_HIP = 3,           /* a HIP runtime call or a kernel launch failed */
    FP8Q_ERR_WORKSPACE = 4,     /* workspace missing or smaller than the query returned */
    /* range sentinels, not statuses: they make every int a value of the type,
       so an unknown value passed through the ABI is still well defined */
    FP8Q_STATUS_INT_MIN_ = -0x7FFFFFFF - 1,
    FP8Q_STATUS_INT_MAX_ = 0x7FFFFFFF
} fp8q_status;

/* The FP8 MatMul modes of the write-up (§3.1 step 3). */
typedef enum {
    FP8Q_W8A16 = 0,             /* "fp8_w_bf16_a": E4M3 weight, bf16 activation and output */
    FP8Q_W8A8 = 1,              /* "fp8_w_fp8_a":  E4M3 weight and activation, bf16 output */
    FP8Q_W8A16_F16 = 2,         /* "fp8_w_fp16_a": E4M3 weight, fp16 activation and output */
    /* range sentinels, not modes (see fp8q_status) */
    FP8Q_MODE_INT_MIN_ = -0x7FFFFFFF - 1,
    FP8Q_MODE_INT_MAX_ = 0x7FFFFFFF
} fp8q_mode;

/* FP8Q_ABI_VERSION of the built library. */
int fp8q_abi_version(void);

/* Static description of a status code; never NULL. */
const char *fp8q_status_string(fp8q_status s);

/* Thread-local description of the last non-OK status returned on this thread
 * (an empty string if there was none).  Valid until the next call on the
 * same thread. */
const char *fp8q_last_error(void);

/*
 * Per-output-channel weight quantization (deployment guide §3.1, §1.2).
 *
 * For each row n of W (bf16 bit patterns, [n, k], row stride ld_w):
 *   amax      = max_k |W[n,k]|
 *   s         = max(fl32(amax / 448), 1e-12f)                 -> w_scale[n]  (fp32)
 *   w_fp8[n,k] = E4M3_RNE_saturating(fl32(W[n,k] / s))        (IEEE fp32 division,
 *                                                              then one RNE cast)
 * E4M3 is the OCP "e4m3fn" format of §1.1 (bias 7, max 448, no infinities);
 * the codes are raw bit patterns (viewable as torch.float8_e4m3fn).
 *
 *   w_bf16  [n, k] bf16, ld_w >= k
 *   w_fp8   [n, k] uint8 out, ld_q >= k
 *   (rows that are 16-byte aligned -- aligned pointers, ld_w % 8 == 0 and
 *   ld_q % 8 == 0 -- take the vectorized path; any other layout is handled
 *   element by element)
 *   w_scale [n] fp32 out
 *   nonfinite_flag  optional int32 (may be NULL): set to 1 if any input is NaN/Inf
 * n == 0 is a no-op; k must be >= 1.  Results are bit-exact and deterministic.
 */
fp8q_status fp8q_quantize_weight(const uint16_t *w_bf16, int64_t n, int64_t k, int64_t ld_w,
                                 uint8_t *w_fp8, int64_t ld_q, float *w_scale,
                                 int32_t *nonfinite_flag, hipStream_t stream);

/*
 * Per-group weight quantization (deployment guide §4.3 names per-group
 * granularity as the step beyond per-channel scales).  Each row of W is cut
 * along K into groups of `group` consecutive values (the last may be
 * shorter); each group gets the §3.1 scale over its own values:
 *   s[n,g]     = max(fl32(max_{k in g} |W[n,k]| / 448), 1e-12f)   -> w_scale[n*G + g]
 *   w_fp8[n,k] = E4M3_RNE_saturating(fl32(W[n,k] / s[n, k / group]))
 * with G = ceil(k / group).  group = 64, 128, 256 or 512.
 *
 *   w_bf16  [n, k] bf16, ld_w >= k;  w_fp8 [n, k] uint8 out, ld_q >= k
 *   w_scale [n, G] fp32 out, row-major; must lie inside one device allocation
 *   nonfinite_flag  optional, as above
 * n == 0 is a no-op; k must be >= 1.  Bit-exact.
 */
fp8q_status fp8q_quantize_weight_grouped(const uint16_t *w_bf16, int64_t n, int64_t k,
                                         int64_t ld_w, int64_t group, uint8_t *w_fp8,
                                         int64_t ld_q, float *w_scale, int32_t *nonfinite_flag,
                                         hipStream_t stream);

/*
 * Dynamic per-tensor activation quantization (deployment guide §1.2: one scale
 * for the whole activation tensor; the scale formula is the one of §3.1,
 * recomputed on every call).
 *   amax = max_{m,k} |X[m,k]|,  s = max(fl32(amax / 448), 1e-12f) -> *x_scale
 *   x_fp8[m,k] = E4M3_RNE_saturating(fl32(X[m,k] / s))
 *
 *   x_bf16  [m, k] bf16, ld_x >= k
 *   x_fp8   [m, k] uint8 out, ld_q >= k
 *   (16-byte aligned rows take the vectorized path, as for the weights)
 *   x_scale one fp32 out (device)
 *   workspace  device scratch of at least fp8q_quantize_act_workspace_size(m, k)
 *              bytes, 16-byte aligned; its contents need no initialisation
 *   nonfinite_flag  optional, as above
 * Two kernels run on `stream` (a global absmax, then the cast).  m == 0 writes
 * the scale of an empty tensor (1e-12f); k must be >= 1.  Bit-exact.
 */
size_t fp8q_quantize_act_workspace_size(int64_t m, int64_t k);
fp8q_status fp8q_quantize_act(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                              uint8_t *x_fp8, int64_t ld_q, float *x_scale,
                              void *workspace, size_t workspace_bytes,
                              int32_t *nonfinite_flag, hipStream_t stream);

/*
 * Static per-tensor activation quantization: the cast of fp8q_quantize_act with
 * a scale the caller holds instead of one recomputed from X (the per-tensor
 * activation scale of the deployment guide §1.2, kept across calls as the
 * write-up's §3.1 step 2 keeps it).  One pass over X:
 *   x_fp8[m,k] = E4M3_RNE_saturating(fl32(X[m,k] / *x_scale))
 * Values beyond 448 * scale saturate to +-448 (codes 0x7E / 0xFE).
 *
 *   x_bf16   [m, k] bf16, ld_x >= k;  x_fp8 [m, k] uint8 out, ld_q >= k
 *   x_scale  one fp32 (device), read only; it must be positive and finite
 *            (any other value gives unspecified codes)
 *   nonfinite_flag  optional, as above
 * m == 0 is a no-op; k must be >= 1.  Bit-exact.
 */
fp8q_status fp8q_quantize_act_static(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                     const float *x_scale, uint8_t *x_fp8, int64_t ld_q,
                                     int32_t *nonfinite_flag, hipStream_t stream);

/*
 * EMA-scaled per-tensor activation quantization (the write-up §3.1 step 2: the
 * activation scale is an exponential moving average, decay 0.9999 there;
 * §5.3 tip 2: a temperature T multiplies the new term by (1 + 0.1 T)).
 * `state` is one device fp32 that carries the average from call to call.
 *
 *   seed != 0: dynamic quantization of X exactly as fp8q_quantize_act;
 *              *x_scale and *state both receive X's dynamic scale.
 *   seed == 0: one pass over X casts it with s_old = *state (the scale lags
 *              one call behind, so X is read once), and the same pass finds
 *              max|X|; then a one-workgroup kernel sets
 *                *x_scale = s_old
 *                s_new    = max(fl32(max|X| / 448), 1e-12f)
 *                *state   = max(d*s_old + ((1-d)*s_new)*(1 + 0.1f*T), 1e-12f)
 *              in fp32, each operation rounded on its own (no fused
 *              multiply-add), in that order.
 * Pass *x_scale to fp8q_linear(FP8Q_W8A8, ...) with the codes.
 *
 *   decay        d in [0, 1]; 1 freezes the state, 0 follows the last tensor
 *   temperature  T, finite and >= 0 (0 gives the plain average)
 *   state        on a call with seed == 0 it must hold a positive finite scale
 *                (from a seeded call); read and written by the device
 *   workspace    at least fp8q_quantize_act_workspace_size(m, k) bytes,
 *                16-byte aligned, no initialisation needed
 *   x_fp8, x_scale, state and workspace must not overlap each other or x.
 * m == 0 counts as a tensor whose maximum is 0.  k must be >= 1.  Bit-exact.
 * Two kernels run on `stream` in either case; calls that share a state must be
 * ordered on one stream.
 */
fp8q_status fp8q_quantize_act_ema(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                  uint8_t *x_fp8, int64_t ld_q, float *x_scale, float *state,
                                  float decay, float temperature, int seed,
                                  void *workspace, size_t workspace_bytes,
                                  int32_t *nonfinite_flag, hipStream_t stream);

/*
 * FP8 KV-cache write with an online running-max scale (deployment guide §3.2:
 * KV values exist only at inference time, so each attention layer keeps a
 * running maximum that prefill batches raise and from which the scale is
 * computed; decode quantizes new K/V with the latest scale).  K and V keep a
 * running maximum each; scale and cast are those of §3.1.  One call writes
 * the new tokens of one layer.
 *
 *   k_bf16, v_bf16  [tokens, ld] bf16, token-major as the k/v projections
 *                   produce them; row t holds heads * head_dim values, head h
 *                   at columns h*head_dim ... ; 16-byte aligned, ld % 8 == 0
 *   slot     [tokens] int64: the cache row of each token (e.g. its position);
 *            rows must be distinct within a call (else which token lands
 *            there is unspecified).  A row outside [0, slots) is not written
 *            and sets flag bit 2.
 *   k_cache, v_cache  [heads, slots, head_dim] E4M3 codes of one layer (the
 *            contiguous [layers, kv_heads, seq_len, head_dim] layout of the
 *            "Some Technical Notes About Llama 3" commentary §3.2, one layer);
 *            8-byte aligned; each must lie inside one device allocation
 *   running_max  [2] fp32: max |K|, max |V| seen by calibrating calls (in/out;
 *            start at 0)
 *   scale_out    [2] fp32 out: the K and V scales this call's codes use,
 *            max(fl32(running / 448), 1e-12f)
 *   calibrate != 0 (prefill / warm-up): running = max(running, max|batch|)
 *            first, then the batch is cast with the raised scales (two passes
 *            over the batch, nothing saturates).
 *   calibrate == 0 (decode): one pass with the scales of the running maxima
 *            as they stand; values beyond 448 * scale saturate.  Before any
 *            calibrating call the scale is the 1e-12 floor (the page's cold
 *            start: warm up first).
 *   workspace  fp8q_kv_cache_workspace_size(tokens, heads, head_dim) bytes,
 *            16-byte aligned, no initialisation needed
 *   flags    optional int32, OR-ed: 1 = NaN/Inf input, 2 = slot out of range
 * head_dim must be a multiple of 8; tokens * heads * head_dim / 8 < 2^31.
 * Codes already in the cache keep the scale they were written with: a
 * calibrating call that raises the maximum does not rewrite them.  Bit-exact.
 */
size_t fp8q_kv_cache_workspace_size(int64_t tokens, int64_t heads, int64_t head_dim);
fp8q_status fp8q_kv_cache_write(const uint16_t *k_bf16, const uint16_t *v_bf16, int64_t tokens,
                                int64_t heads, int64_t head_dim, int64_t ld,
                                const int64_t *slot, uint8_t *k_cache, uint8_t *v_cache,
                                int64_t slots, float *running_max, float *scale_out,
                                int calibrate, void *workspace, size_t workspace_bytes,
                                int32_t *flags, hipStream_t stream);

/*
 * The scaled linear layer, Y = X . dequant(W)^T, in the write-up's modes
 * (§3.1 step 3), with the per-channel weight scale and per-tensor activation
 * scale of the deployment guide §1.2:
 *   FP8Q_W8A16: Y[m,n] = bf16_RNE( w_scale[n] * sum_k X[m,k] * dec(W[n,k]) )
 *               x = bf16 [m, k] (ld_x % 8 == 0); x_scale must be NULL.
 *   FP8Q_W8A8:  Y[m,n] = bf16_RNE( x_scale * w_scale[n] * sum_k dec(X[m,k]) * dec(W[n,k]) )
 *               x = E4M3 codes [m, k] (ld_x % 16 == 0); x_scale = device fp32[1];
 *               ld_x and ld_w must be below 2^23 in this mode.  Up to 64 activation
 *               rows run the decode kernels (codes widened exactly to bf16), more
 *               rows the FP8 MFMA GEMM (but see below); both compute the same sums.
 *   FP8Q_W8A16_F16: as FP8Q_W8A16 with x = fp16 [m, k] and y fp16 (RNE) instead of
 *               bf16 (E4M3 values are exact in fp16; |Y| must stay below 65504).
 * Products are exact and sums are accumulated in fp32; the result is within
 * 5e-3 relative Frobenius error of the exact value (see the tests).
 * Above 64 activation rows the 16-bit modes run a prefill GEMM on the 16-bit
 * MFMA (weights widened exactly to the activation type; it needs ld_x below
 * 2^22 and ld_w below 2^23).  From 65 to 1024 rows, where a GEMM's grid would
 * be one round of a few 256 x 256 tiles (a narrow N), the decode kernels run
 * instead, the rows in 64-row groups along their grid, when a cost estimate
 * fitted to MI355X measurements says they are faster (fp8q_linear_describe
 * names the kernel a shape gets).  In every mode ld_x and ld_w must be below 2^28
 * (the decode kernels address a few rows per load with 32-bit offsets);
 * larger strides return FP8Q_ERR_INVALID_ARG.
 *
 *   w_fp8   [n, k] E4M3 codes, ld_w >= k, ld_w % 16 == 0, 16-byte aligned
 *   w_scale [n] fp32
 *   y_bf16  [m, n] out (bf16, or fp16 in FP8Q_W8A16_F16), ld_y >= n, ld_y % 8 == 0,
 *           16-byte aligned; must not overlap any input
 *   workspace  device scratch of at least fp8q_linear_workspace_size(mode, m, n, k)
 *              bytes, 16-byte aligned (the size may be 0, then workspace may be
 *              NULL); needs no initialisation.  The decode kernels use it when
 *              they split K across workgroups (too few output tiles to fill
 *              the GPU): it then holds fp32 partial sums that a second kernel
 *              on `stream` adds up.
 * m == 0 or n == 0 is a no-op; k must be >= 1.  Deterministic: the same inputs
 * give the same bits on every call (K-split partial sums are added in split
 * order).
 */
size_t fp8q_linear_workspace_size(fp8q_mode mode, int64_t m, int64_t n, int64_t k);
fp8q_status fp8q_linear(fp8q_mode mode,
                        const void *x, int64_t m, int64_t k, int64_t ld_x, const float *x_scale,
                        const uint8_t *w_fp8, int64_t n, int64_t ld_w, const float *w_scale,
                        uint16_t *y_bf16, int64_t ld_y,
                        void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * fp8q_linear for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments without the workspace, the same kernels and results.  When
 * the plan splits K, the fp32 partial tiles go to a device-resident scratch
 * array of 8 MiB per GPU that the library holds until the process ends
 * (enough for the Llama-3 8B/70B decode shapes); a shape whose
 * fp8q_linear_workspace_size exceeds 8 MiB returns FP8Q_ERR_WORKSPACE and
 * launches nothing.  The first call on a device that needs the scratch looks
 * up its address (hipGetSymbolAddress); make that first call outside graph
 * capture.  Nothing is allocated, freed or cleared (the partial tiles need no
 * initialisation).  Every call on one GPU shares that GPU's scratch, which
 * keeps the last call's contents: calls that may overlap in time on one GPU
 * (different streams without ordering, several threads) race and give
 * undefined results; order them on one stream.
 */
fp8q_status fp8q_linear_noalloc(fp8q_mode mode,
                                const void *x, int64_t m, int64_t k, int64_t ld_x,
                                const float *x_scale, const uint8_t *w_fp8, int64_t n,
                                int64_t ld_w, const float *w_scale,
                                uint16_t *y_bf16, int64_t ld_y, hipStream_t stream);

/*
 * fp8_w_fp8_a (the write-up §3.1 step 3) on bf16 activations, with the dynamic
 * per-tensor activation quantization of the deployment guide §1.2 (scale by the
 * §3.1 formula) folded into the linear layer:
 *   s_x = max(fl32(max_{m,k} |X[m,k]| / 448), 1e-12f)
 *   Y[m,n] = bf16_RNE( s_x * w_scale[n] * sum_k dec(E4M3_RNE_SAT(fl32(X[m,k] / s_x))) * dec(W[n,k]) )
 * i.e. fp8q_quantize_act followed by fp8q_linear(FP8Q_W8A8, ...): the codes and
 * the scale are bit for bit those of fp8q_quantize_act, the sums are exact
 * products accumulated in fp32 (tolerance and determinism as fp8q_linear).
 * Up to 16 activation rows (decode) the decode GEMM's workgroups cast the
 * activations they load in registers, so the E4M3 activations never go
 * through memory: with at most 32768 activation values and the panel kernel
 * (fp8q_linear_w8a8_dynamic_describe says which) that is one kernel whose
 * workgroups each read all of X for its maximum, otherwise the absmax pass
 * runs first and the GEMM folds its maxima into s_x.  More rows run
 * fp8q_quantize_act into the workspace, then
 * the GEMM on the codes (the kernel fp8q_linear(FP8Q_W8A8, ...) runs for that
 * shape): every GEMM workgroup casts the rows it reads, and from 17 rows on
 * a whole column of workgroups reads each row, so one separate cast is cheaper.
 *
 *   x_bf16       [m, k] bf16, ld_x >= k, ld_x % 8 == 0, 16-byte aligned
 *   w_fp8, w_scale, y_bf16, ld_*   as fp8q_linear
 *   x_scale_out  optional device fp32[1]: receives s_x
 *   workspace    at least fp8q_linear_w8a8_dynamic_workspace_size(m, n, k) bytes,
 *                16-byte aligned, no initialisation needed; it must not overlap
 *                any other argument
 *   nonfinite_flag  optional; set to 1 if any |x| is NaN or Inf
 * m == 0 or n == 0 launches nothing (x_scale_out is then not written).
 */
size_t fp8q_linear_w8a8_dynamic_workspace_size(int64_t m, int64_t n, int64_t k);
fp8q_status fp8q_linear_w8a8_dynamic(const uint16_t *x_bf16, int64_t m, int64_t k, int64_t ld_x,
                                     const uint8_t *w_fp8, int64_t n, int64_t ld_w,
                                     const float *w_scale, uint16_t *y_bf16, int64_t ld_y,
                                     float *x_scale_out, void *workspace, size_t workspace_bytes,
                                     int32_t *nonfinite_flag, hipStream_t stream);

/*
 * The linear layer with per-group weight scales (w_scale [n, ceil(k/group)]
 * from fp8q_quantize_weight_grouped), in the same three modes:
 *   Y[m,n] = out_RNE( s_x * sum_g w_scale[n,g] * sum_{k in g} a(X[m,k]) * dec(W[n,k]) )
 * with s_x = *x_scale for FP8Q_W8A8 and 1 otherwise.  Each group's products
 * are summed in fp32 and multiplied by the group's scale as the group ends.
 * Arguments as fp8q_linear, plus group (64, 128, 256 or 512); w_scale must lie
 * inside one device allocation and hold positive finite scales.
 * FP8Q_W8A8 with more than 64 activation rows and group >= 128 runs the FP8
 * MFMA GEMM (from 65 to 1024 rows on a narrow weight the decode kernels
 * instead, by the cost estimate fp8q_linear uses, the GEMM's cost taken as
 * 1.25 times the per-channel one's): its accumulators are kept in units of the current group's scale,
 * multiplied by s[n][g-1] / s[n][g] (hardware reciprocal) as group g opens, and
 * scaled by the last group's scale at the end.  This needs adjacent group scales
 * of a row within a factor of about 1e28 of each other, which holds for weights
 * of magnitude below 1e16.  Every other case runs the decode kernels: the
 * panel kernel where fp8q_linear would and every 4-wave K range is a whole
 * number of groups (each wave's group scales preloaded into LDS where they
 * fit, else staged with each chunk), the rows kernel where fp8q_linear would
 * take it, else the tile kernel (at prefill sizes with group 64, W is then
 * re-read once per 64 activation rows).  fp8q_linear_grouped_describe names
 * the plan.
 * Tolerance and determinism as fp8q_linear.
 */
size_t fp8q_linear_grouped_workspace_size(fp8q_mode mode, int64_t m, int64_t n, int64_t k,
                                          int64_t group);
fp8q_status fp8q_linear_grouped(fp8q_mode mode,
                                const void *x, int64_t m, int64_t k, int64_t ld_x,
                                const float *x_scale, const uint8_t *w_fp8, int64_t n,
                                int64_t ld_w, const float *w_scale, int64_t group,
                                uint16_t *y_bf16, int64_t ld_y,
                                void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * The element cast used by both quantizers, exposed on its own: fp32 -> E4M3
 * code, round to nearest even, saturating to +-448 (deployment guide §1.1,
 * §3.1; the write-up §2.1 gives the [-448, 448] range).  The sign of zero is
 * kept.  NaN input gives an unspecified code.
 *   x   [count] fp32, 16-byte aligned;  out [count] uint8, 16-byte aligned.
 */
fp8q_status fp8q_cast_f32_to_e4m3(const float *x, int64_t count, uint8_t *out, hipStream_t stream);

/*
 * Describe the kernel configuration fp8q_linear would launch for these sizes
 * (kernel name, grid, split factor) into buf (host memory, NUL-terminated,
 * truncated to len).  Host-only; launches nothing.
 */
fp8q_status fp8q_linear_describe(fp8q_mode mode, int64_t m, int64_t n, int64_t k,
                                 char *buf, size_t len);

/*
 * The same for fp8q_linear_w8a8_dynamic (the absmax pass, then the GEMM that
 * casts the activations, or the quantizer and the GEMM on the codes above 16
 * rows).  Host-only; launches nothing.
 */
fp8q_status fp8q_linear_w8a8_dynamic_describe(int64_t m, int64_t n, int64_t k, char *buf,
                                              size_t len);

/*
 * The same for fp8q_linear_grouped with this group (64, 128, 256 or 512; any
 * other value is FP8Q_ERR_INVALID_ARG).  Host-only; launches nothing.
 */
fp8q_status fp8q_linear_grouped_describe(fp8q_mode mode, int64_t m, int64_t n, int64_t k,
                                         int64_t group, char *buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
