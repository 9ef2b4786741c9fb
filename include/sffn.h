/* sffn.h -- predictor-guided, neuron-aware sparse FFN for one MI355X (gfx950).
 *
 * C ABI of libsffn.so. Every entry point takes plain pointers and sizes; all
 * tensor pointers are DEVICE pointers owned by the caller, and the library
 * never allocates device memory. Calls enqueue work on `stream` (a
 * hipStream_t, NULL = the null stream) and return at once; results are valid
 * once the stream has reached them. No call synchronises the device, so a
 * sequence of calls can be captured into a HIP graph.
 *
 * The operation follows the PowerInfer pages:
 *   - "Online stage: neuron-aware inference engine" and "Adaptive sparsity
 *     predictors" (Turkish article): a small per-layer predictor runs on every
 *     token, marks the neurons that will be active, and the engine skips the
 *     rest;
 *   - "Neuron-aware operator" (same article): the sparse operators work on
 *     individual rows and columns of the weight matrices, never a dense copy;
 *   - "Neuron placement and management" (same article): neurons are stored in
 *     a chosen order and a table maps each back to its original position;
 *   - summary bullets and "Limitations/FAQ" (Indonesian digest): ReLU-family
 *     FFNs (ReLU, ReGLU, squared ReLU); "Quantization": INT4 Q4_0 weights.
 *
 * Notation. D = d_model, F = d_ffn (neurons), r = predictor rank, B = tokens
 * of one call (1 for decode; B > 1 computes every token over the union of the
 * per-token masks). "Stored order" is the caller's neuron order (a
 * permutation of the original one); the library never sees the permutation:
 * every per-neuron array (rows of P2, W_gate, W_up, W_down^T, b, c) must be
 * given in the same stored order, and the caller maps ids back.
 *
 * Layouts (row-major, contiguous):
 *   x        [B, D] fp32           token inputs
 *   P1       [r, D] fp16           predictor first factor
 *   P2       [F, r] fp16           predictor second factor (stored order)
 *   c        [F]    fp32 or NULL   predictor bias
 *   W_gate   [F, D] fp16           ReGLU gate rows (stored order), b_gate [F] fp32
 *   W_up     [F, D] fp16           up rows, b_up [F] fp32 (ReLU)
 *   W_downT  [F, D] fp16           W_down transposed: row k = column k of W_down
 *   mask     [ceil(F/64)] uint64   bit (k % 64) of word k / 64 = stored neuron k active
 *   y        [B, D] fp32
 * Q4_0 matrices (sffn_q4): blocks of 32 consecutive weights along d_model in
 * every neuron row, w = (q - 8) * s with q in 0..15:
 *   q  [F, D/2] uint8: for block j of a row, bytes 16j..16j+15; byte i holds
 *      element 32j+i in its low nibble and element 32j+16+i in its high nibble
 *   s  [F, D/32] fp16 scale of each block.
 *
 * Alignment: every tensor pointer 16-byte aligned; the workspace 256-byte
 * aligned. Limits: 1 <= B <= 64; 8 <= D <= 16384 with D % 8 == 0 (D % 32 == 0
 * for Q4_0); 1 <= F <= 1<<22; 8 <= r <= 1024 with r % 8 == 0; B * r <= 32768;
 * every weight matrix and the B x F activations below 2 GiB.
 *
 * Batches. B == 1 (decode) and B == 2 with 2 * D <= 16384 run the decode
 * kernels (vector ALU, x staged once per block); so do B in {4, 8} with
 * B * D <= 16384 when F > 32768. Every other B > 1 runs the union kernels on
 * the matrix cores ("Neuron-aware operator": each active row is read once for
 * the whole batch); these compact the whole mask inside one workgroup and
 * take F <= 32768 in sffn_forward / sffn_forward_q4. With fp16 weights and
 * up to 8 tokens the fp32 inputs and activations enter the matrix cores as
 * two fp16 halves (x = hi + lo), so those results match the decode kernels'
 * to within fp32 rounding; larger batches, and Q4_0 weights, take each as one
 * fp16 value after a per-token power-of-two scaling (relative 2^-11 per
 * value, inside the output tolerance the parity tests hold).
 *
 * Workspace (sffn_workspace_size bytes, 256-byte parts, caller-owned, no
 * state kept between calls): activations a [F, B] fp32 (for B == 1 at least
 * 4 KiB: sffn_decode keeps its per-block decision bitmaps there); for B > 1 the
 * normalised inputs [B, D]; partial sums of y, [256, D] fp32 for B == 1 (one
 * per block of the fused kernel) or [16, B, D] for B > 1 (row splits; the
 * union predictor also keeps its partial h there); for B > 1 the partial
 * pre-activations of the k-split union row kernel, [KS, 2, F, B] fp32 (KS = 8,
 * 4 or 2 shares for 7-8, 9-16 and 17-32 tokens, none otherwise), the union
 * row kernel's token operands (room for two fp16 planes of ceil(D/32) x
 * ceil(B/16) KiB, then 16 fp32 per 16 tokens) and its largest |a| per row
 * tile and token; the predictor's h [B, r] fp32 last. One workspace may serve
 * the predict and
 * forward calls of a layer in turn on one stream; calls that overlap in time
 * need separate workspaces.
 *
 * Errors: arguments are checked on the host before anything is enqueued; a
 * failed check returns its status and leaves the stream untouched. A failed
 * launch returns SFFN_ERR_HIP. sffn_last_error() gives the detail text of the
 * calling thread's last failure. No exception crosses the ABI.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SFFN_OK = 0,
  SFFN_ERR_NULL = 1,       /* a required pointer is NULL                      */
  SFFN_ERR_SHAPE = 2,      /* B, D, F or r outside the limits above            */
  SFFN_ERR_ALIGN = 3,      /* a pointer is not aligned as required             */
  SFFN_ERR_WORKSPACE = 4,  /* workspace smaller than sffn_workspace_size()     */
  SFFN_ERR_ACT = 5,        /* unknown activation, or operands it needs missing */
  SFFN_ERR_ARG = 6,        /* other bad argument (threshold outside (0, 1))    */
  SFFN_ERR_HIP = 7         /* the HIP runtime reported an error                */
} sffn_status;

typedef enum {
  SFFN_ACT_RELU = 0,   /* a_k = max(0, W_up[k] x + b_up[k])                        */
  SFFN_ACT_REGLU = 1,  /* a_k = max(0, W_gate[k] x + b_gate[k]) * (W_up[k] x)      */
  SFFN_ACT_SQRELU = 2  /* a_k = max(0, W_up[k] x + b_up[k])^2  (squared ReLU; operands as for RELU) */
} sffn_act;

/* One Q4_0 matrix (device pointers, layout above). */
typedef struct {
  const uint8_t* q;
  const void* s;
} sffn_q4;

/* Text of a status code (static storage). */
const char* sffn_status_string(int status);

/* Detail of the calling thread's last failure ("" if none). */
const char* sffn_last_error(void);

/* Bytes of workspace that sffn_predict / sffn_forward / sffn_forward_q4 need for these sizes. */
size_t sffn_workspace_size(int B, int D, int F, int r);

/* Number of 64-bit mask words for F neurons: ceil(F / 64). */
int sffn_mask_words(int F);

/* Which kernels sffn_forward (q4 = 0) or sffn_forward_q4 (q4 = 1) runs for these sizes:
 *   SFFN_PATH_FUSED (B == 1, F <= 32768, and D <= 5120 for fp16 ReGLU, D <= 8192 for fp16 ReLU and for Q4_0):
 *     one kernel gathers the gate/up rows, applies the activation and accumulates the W_downT rows into
 *     per-block partial sums of y; a second kernel adds the partials in fixed order (timing ids SFFN_K_ROWS and
 *     SFFN_K_COLS);
 *   SFFN_PATH_DECODE (other B == 1; B == 2 with 2 * D <= 16384; B in {4, 8} with B * D <= 16384 and
 *     F > 32768): row gather + activation, then the column gather;
 *   SFFN_PATH_UNION (every other B): matrix-core kernels over the union mask.
 * Returns -1 for an unknown activation. */
enum { SFFN_PATH_DECODE = 0, SFFN_PATH_FUSED = 1, SFFN_PATH_UNION = 2 };
int sffn_forward_path(int act, int q4, int B, int D, int F);

/* Activation predictor ("Adaptive sparsity predictors"; "Online stage").
 *   h[b, :] = P1 xn[b, :]                     (fp32 accumulate; h is never rounded)
 *   z[b, k] = P2[k, :] h[b, :] + c[k]         (c = NULL means 0)
 *   neuron k active  <=>  sigmoid(z[b, k]) > t for some token b
 *                    <=>  z[b, k] > ln(t / (1 - t))  (decided in logit space)
 * xn = x, or, if x_norm != 0, xn[b, :] = (x[b, :] - m) / sqrt(v + 1e-6) with m the mean and v the
 * (population) variance of x[b, :] -- the parameter-free normalisation between stacked layers, applied as the
 * input is loaded.
 * Outputs: mask (every word written, bits >= F zero); logits [B, F] fp32 if
 * non-NULL. Uses the workspace. Two kernels for B <= 8 (h, then z; a normalised input is normalised as it is
 * loaded); for B > 8 three (partial h over shares of d, their sum, z), after a normalisation pass with x_norm. */
int sffn_predict(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D, int F,
                 int r, float t, uint64_t* mask, float* logits, void* ws, size_t ws_bytes, void* stream);

/* sffn_predict with an always-active prefix ("Neuron placement and management", Turkish article: neurons are
 * stored in a chosen order, here hottest first). Stored neurons 0 .. n_hot-1 are set in the mask whatever the
 * predictor would say, and their rows of P2 and entries of c are never read (P2 and c must still span all F
 * rows; only rows >= n_hot are loaded). Their logits, if requested, are written as +infinity. Every other
 * neuron is decided exactly as by sffn_predict, which is this call with n_hot = 0. SFFN_ERR_ARG if n_hot is
 * outside 0..F. */
int sffn_predict_hot(const void* P1, const void* P2, const float* c, const float* x, int x_norm, int B, int D, int F,
                     int r, float t, int n_hot, uint64_t* mask, float* logits, void* ws, size_t ws_bytes,
                     void* stream);

/* Neuron-aware sparse FFN over the neurons set in `mask` ("Neuron-aware operator").
 *   compaction: active[0 .. n) = ascending stored ids of the set bits, *n_active = n
 *   a[b, j]  = act(row active[j] of W_gate / W_up, xn[b, :])   (only active rows are read)
 *   y[b, :]  = sum_j a[b, j] * W_downT[active[j], :]          (only active rows are read)
 * xn as in sffn_predict. W_gate / b_gate are used (and required) for REGLU only;
 * RELU and SQRELU read W_up and b_up; b_up may be NULL (0). active [F] int32 and n_active [1] int32 are device
 * outputs; y [B, D] is overwritten. Uses the workspace. Two kernels; the union kernels add a sum of the row-split partials (and a normalisation pass for x_norm). */
int sffn_forward(int act, const void* W_gate, const float* b_gate, const void* W_up, const float* b_up,
                 const void* W_downT, const float* x, int x_norm, int B, int D, int F, const uint64_t* mask,
                 int32_t* active, int32_t* n_active, float* y, void* ws, size_t ws_bytes, void* stream);

/* sffn_forward with Q4_0 weights ("Quantization": INT4 Q4_0); weights are
 * dequantised in registers, w = (q - 8) * s exactly in fp32. */
int sffn_forward_q4(int act, sffn_q4 W_gate, const float* b_gate, sffn_q4 W_up, const float* b_up, sffn_q4 W_downT,
                    const float* x, int x_norm, int B, int D, int F, const uint64_t* mask, int32_t* active,
                    int32_t* n_active, float* y, void* ws, size_t ws_bytes, void* stream);

/* One decode step of one layer for a single token: sffn_predict_hot (n_hot = 0: sffn_predict) followed by
 * sffn_forward, with the same operands, outputs and results ("Adaptive sparsity predictors" and "Neuron-aware
 * operator", Turkish article). mask, active, n_active, y and logits (if non-NULL) are written as the two calls
 * would write them. Where sffn_decode_path says SFFN_DECODE_FOLDED, the predictor's second stage runs inside
 * the row gather: each of the 256 workgroups decides the neurons it owns (stored neurons k with k % 256 equal to
 * its index) and gathers the active ones at once, so the layer takes three kernels instead of four and one
 * dependent round trip less; the mask and the ascending ids are assembled while the partial sums of y are added.
 * Otherwise the two calls run as they are. fp16 weights only (the Q4_0 forward keeps its separate calls). Uses
 * the workspace of sffn_workspace_size(1, D, F, r). Errors as sffn_predict and sffn_forward. */
enum { SFFN_DECODE_SEPARATE = 0, SFFN_DECODE_FOLDED = 1 };
int sffn_decode_path(int act, int q4, int D, int F, int r);   /* -1 for an unknown activation */
int sffn_decode(int act, const void* P1, const void* P2, const float* c, float t, int n_hot, const void* W_gate,
                const float* b_gate, const void* W_up, const float* b_up, const void* W_downT, const float* x,
                int x_norm, int D, int F, int r, uint64_t* mask, int32_t* active, int32_t* n_active, float* y,
                float* logits, void* ws, size_t ws_bytes, void* stream);

/* sffn_decode without a workspace argument, for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same operands, outputs and results as
 * sffn_decode. Its workspace is a scratch array of sffn_noalloc_scratch_bytes() bytes (16 MiB) in the library's
 * own device memory: one per GPU, allocated when the library is loaded on that GPU and held until the process
 * ends. The call allocates nothing. Sizes whose workspace (sffn_workspace_size(1, D, F, r)) exceeds the scratch
 * return SFFN_ERR_WORKSPACE before anything is enqueued (D = 8192, F = 32768, r = 1024 need 8.1 MiB). Every call
 * on one GPU shares that GPU's scratch, which keeps the last call's contents (no call needs them): calls that
 * overlap in time on one GPU (several streams or host threads) race on it and must be serialised by the caller.
 * The first call on a device looks up the scratch's address there (SFFN_ERR_HIP if that fails). */
size_t sffn_noalloc_scratch_bytes(void);
int sffn_decode_noalloc(int act, const void* P1, const void* P2, const float* c, float t, int n_hot,
                        const void* W_gate, const float* b_gate, const void* W_up, const float* b_up,
                        const void* W_downT, const float* x, int x_norm, int D, int F, int r, uint64_t* mask,
                        int32_t* active, int32_t* n_active, float* y, float* logits, void* stream);

/* Per-launch timing of one kernel (profiling aid; not needed for computing).
 * kernel: SFFN_K_PRED_H (P1 x), SFFN_K_PRED_Z (P2 h + c, threshold, mask), SFFN_K_ROWS (compaction + W_gate /
 * W_up row gather + activation), SFFN_K_COLS (W_downT column gather; in the union path the row-split down
 * projection, not the sum of its partials). In a folded sffn_decode the folded kernel (predictor stage 2 + row
 * gather) is SFFN_K_ROWS and the sum of partials with the mask assembly SFFN_K_COLS.
 * Between sffn_profile_begin and sffn_profile_end, every launch of that kernel made by the calling thread, up
 * to max_launches of them, is issued with a pair of HIP events that take the kernel's own start and end
 * timestamps (hipExtLaunchKernelGGL): the kernel's time on the device, without host-side queueing. The events
 * are created by sffn_profile_begin (host call; launches under graph capture are not timed: profile eager
 * calls). sffn_profile_end waits for the last event, writes the elapsed milliseconds of the launches to
 * ms[0 .. min(count, max)) and returns the count (negative status on error). Returns SFFN_ERR_ARG for a bad
 * kernel id or max_launches < 1. */
enum { SFFN_K_PRED_H = 0, SFFN_K_PRED_Z = 1, SFFN_K_ROWS = 2, SFFN_K_COLS = 3 };
int sffn_profile_begin(int kernel, int max_launches);
int sffn_profile_end(float* ms, int max);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
