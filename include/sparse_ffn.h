/*
 * sparse_ffn.h -- C ABI of the predictor-gated bank-wise sparse SwiGLU FFN
 * forward for AMD Instinct MI355X (gfx950).
 *
 * The operation is the FFN block of "Continual LLM Upcycling: A
 * Predictor-Gated Bank-Wise Sparsity Training Recipe for Dense-to-Sparse
 * LLMs" (gist.science technical summary, Methodologie > 1. Architectuur):
 * for every token t
 *
 *   z = x_t A^T                      predictor layer 1, R^d -> R^rank
 *   p = z B^T (+ bias)               predictor layer 2, R^rank -> R^{d_i},
 *                                    the channel routing logits
 *   m = bank top-k of p              d_i split into contiguous banks of 64,
 *                                    `keep` largest logits kept per bank
 *   h_j = m_j * s_j * u_j * v_j      u_j = x_t . W_g[j], v_j = x_t . W_u[j],
 *                                    s_j = sigmoid(p_j) (predictor gate, the
 *                                    routing signal replacing sigmoid(u)) or
 *                                    sigmoid(u_j) (plain SwiGLU gate)
 *   y_t = sum over kept j of h_j W_d[:, j]
 *
 * Inactive channels are exactly zero and their rows of W_g / W_u and columns
 * of W_d are never read (same summary, 3. Hardware Implicaties: gate, up and
 * down are all skipped for inactive channels).
 *
 * Conventions shared by every entry point
 * --------------------------------------
 * - Matrices are row-major, in nn.Linear layout [out, in].
 * - SFFN_BF16 tensors hold bfloat16 bit patterns (uint16 storage); SFFN_F32
 *   tensors hold IEEE binary32. Logits and the predictor bias are always fp32.
 * - Masks: one uint64 word per (token, bank); bit i of word (t, b) is channel
 *   64*b + i. Channel ids are uint16, ascending within a token.
 * - Ties in the top-k go to the lower channel index; -0 equals +0; NaN ranks
 *   below every number.
 * - All pointers named "device" are device memory owned by the caller; the
 *   library never allocates, frees or synchronises device memory except in
 *   sparse_ffn_create, which synchronises its stream once.
 * - Device pointers must be 16-byte aligned; the workspace 256-byte aligned.
 * - Work is enqueued on `hip_stream` (a hipStream_t; NULL = default stream)
 *   and runs asynchronously. Every argument is checked before anything is
 *   enqueued; a failed check returns an error and enqueues nothing.
 * - Return codes only: nothing aborts, nothing throws across the ABI. The
 *   detail of the last failure on the calling thread is returned by
 *   sparse_ffn_last_error().
 */
#ifndef SPARSE_FFN_H
#define SPARSE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SFFN_OK = 0,
    SFFN_ERR_INVALID_ARG = 1,  /* a null/misaligned pointer or bad size     */
    SFFN_ERR_UNSUPPORTED = 2,  /* a valid request this library cannot run   */
    SFFN_ERR_WORKSPACE = 3,    /* workspace or packed buffer too small      */
    SFFN_ERR_HIP = 4           /* the HIP runtime reported an error         */
} sffn_status_t;

typedef enum { SFFN_F32 = 0, SFFN_BF16 = 1 } sffn_dtype_t;

typedef enum {
    SFFN_GATE_PREDICTOR = 0,   /* h = m * sigmoid(p) * u * v                */
    SFFN_GATE_SILU = 1,        /* h = m * sigmoid(u) * u * v                */
    /* The Dense-4x baseline the method is compared against ("Continual LLM
     * Upcycling", gist.science technical summary, Resultaten: naive 4x
     * sparsity applied post hoc from activation amplitude). No predictor:
     * gate and up run for every channel, m is the bank top-k of
     * |sigmoid(u) * u * v| (fp32), h = m * sigmoid(u) * u * v, and down
     * reads the kept channels only. */
    SFFN_GATE_AMPLITUDE = 2
} sffn_gate_t;

/* Layer shape. The method's layer is d_i = 14336, rank = 448, bank = 64,
 * keep = 16 (Methodologie > 1. Architectuur); d is the model width.
 * Requirements: bank == 64; 1 <= keep <= 64; d_i % 64 == 0 and
 * d_i <= 65536; d % 64 == 0; rank % 32 == 0; all positive. */
/* Options of a layer (bits of sffn_config_t.flags). */
typedef enum {
    /* The packed buffer also holds W_g^T and W_u^T ([d, d_i] each, 4 d d_i
     * more bytes for bf16), so that sparse_ffn_backward does not transpose
     * them on every call. */
    SFFN_FLAG_BACKWARD = 1
} sffn_flag_t;

typedef struct {
    int32_t d;
    int32_t d_i;
    int32_t rank;
    int32_t bank;
    int32_t keep;
    sffn_dtype_t dtype;   /* element type of x, y and every weight */
    sffn_gate_t gate;
    int32_t flags;        /* SFFN_FLAG_* bits; 0 for none */
} sffn_config_t;

typedef struct sffn_layer* sffn_handle_t;

/* Bytes of the caller-owned buffer sparse_ffn_create packs the weights into,
 * or 0 when the config is invalid. */
size_t sparse_ffn_packed_size(const sffn_config_t* cfg);

/* Copy one layer's weights into `packed` (device, >= packed_size bytes) in
 * the layouts the kernels read, and return a handle.
 *   w_gate  [d_i, d], w_up [d_i, d], w_down [d, d_i]   (device, cfg->dtype)
 *   pred_a  [rank, d]  predictor layer 1               (device, cfg->dtype)
 *   pred_b  [d_i, rank] predictor layer 2              (device, cfg->dtype)
 *   pred_bias [d_i] fp32 or NULL                       (device)
 * With SFFN_GATE_AMPLITUDE pred_a and pred_b may be NULL (unused).
 * The weights may be freed after this call returns; `packed` must stay alive
 * and unmodified until sparse_ffn_destroy. Synchronises `hip_stream`.
 * *out is set only on SFFN_OK. */
sffn_status_t sparse_ffn_create(const sffn_config_t* cfg, const void* w_gate,
                                const void* w_up, const void* w_down,
                                const void* pred_a, const void* pred_b,
                                const float* pred_bias, void* packed,
                                size_t packed_bytes, void* hip_stream,
                                sffn_handle_t* out);

/* Workspace bytes sparse_ffn_forward needs for T tokens (0 for T <= 0 or a
 * null handle). */
size_t sparse_ffn_workspace_size(sffn_handle_t h, int64_t T);

/* Forward of T tokens: x [T, d] -> y [T, d] (device, cfg->dtype).
 *   mask_out   [T, d_i/64] uint64 or NULL: the top-k mask actually used
 *   logits_out [T, d_i] fp32 or NULL: the predictor logits p (with
 *              SFFN_GATE_AMPLITUDE: the amplitudes sigmoid(u) * u * v that
 *              were ranked)
 *   workspace  device scratch of >= sparse_ffn_workspace_size(h, T) bytes,
 *              not shared with a concurrent call
 * keep = 64 keeps every channel: with SFFN_GATE_PREDICTOR it is the
 * predictor-gated dense FFN of the training recipe's fourth stage
 * ("Continual LLM Upcycling", Methodologie > 2. Trainingsrecept); with
 * SFFN_GATE_SILU it is the plain dense SwiGLU, one reading of the single-
 * layer dense fallback (Belangrijkste Bijdragen, item 3). In the latter the
 * predictor runs only when logits_out is given; mask_out (if given) is all
 * ones.
 * T == 0 returns SFFN_OK and enqueues nothing. Calls on different streams
 * may overlap if each has its own workspace and outputs. */
sffn_status_t sparse_ffn_forward(sffn_handle_t h, const void* x, int64_t T,
                                 void* y, uint64_t* mask_out,
                                 float* logits_out, void* workspace,
                                 size_t ws_bytes, void* hip_stream);

/* sparse_ffn_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation). The scratch is a static array of
 * 16 MiB per GPU inside the library, allocated when the library's code is
 * loaded on that GPU and kept until the process ends; it covers every path
 * of the full layer (d = 4096, d_i = 14336, rank 448) up to T = 64. A call
 * whose sparse_ffn_workspace_size(h, T) exceeds it returns
 * SFFN_ERR_WORKSPACE and enqueues nothing. Every call on a GPU shares that
 * GPU's array: calls that may overlap on one GPU (different streams,
 * different threads) race and must not be issued; calls on one stream are
 * ordered and safe. The scratch keeps the last call's contents; every byte a
 * call reads is written earlier in the same call. The first call on a GPU
 * looks the array's address up (hipGetSymbolAddress on the stream's device);
 * no call allocates or frees device memory. Arguments and results are those
 * of sparse_ffn_forward. */
sffn_status_t sparse_ffn_forward_noalloc(sffn_handle_t h, const void* x, int64_t T,
                                         void* y, uint64_t* mask_out,
                                         float* logits_out, void* hip_stream);

/* Bank-wise hard top-k alone (Methodologie > 1. Architectuur, the bank rule):
 *   logits  [T, d_i] fp32 (device)
 *   mask_out [T, d_i/64] uint64 (device): exactly `keep` bits per word
 *   idx_out [T, (d_i/64)*keep] uint16 or NULL (device): kept channel ids,
 *           ascending per token
 * Requires d_i % 64 == 0, d_i <= 65536 (for ids), 1 <= keep <= 64, T >= 0. */
sffn_status_t bank_topk(const float* logits, int64_t T, int32_t d_i,
                        int32_t keep, uint64_t* mask_out, uint16_t* idx_out,
                        void* hip_stream);

/* Number of kernel stages in one forward (both execution paths). */
#define SFFN_STAGES 5

/* Per-stage timing, for profiling. When `events` is non-null it must hold
 * 2 * SFFN_STAGES hipEvent_t handles; every later sparse_ffn_forward on this
 * handle then launches the kernel of stage i with events[2i] / events[2i+1]
 * as its start / stop events (hipExtLaunchKernel: the timestamps of the
 * kernel's own dispatch, without host launch gaps). NULL turns recording
 * off. The events remain the caller's. Not thread-safe against concurrent
 * forwards on the same handle. */
sffn_status_t sparse_ffn_set_stage_events(sffn_handle_t h, void* const* events,
                                          int32_t n_events);

/* Name of stage i (0 <= i < SFFN_STAGES) of a forward of T tokens that asks
 * for no logits, e.g. "gateup"; "none" for a stage the chosen path does not
 * have (its two events are recorded back to back; with keep = 64 and the silu
 * gate these are the predictor and top-k stages); NULL when out of range. */
const char* sparse_ffn_stage_name(sffn_handle_t h, int64_t T, int32_t i);

/* Workspace bytes sparse_ffn_backward needs for T tokens (0 for T <= 0 or
 * a null handle). One fp32 and about ten bf16 [T, d_i] buffers, the
 * token-transposed operands and the transposed predictor weights, plus
 * W_g^T and W_u^T without SFFN_FLAG_BACKWARD: ~1.5 GB at T = 4096, d = 4096,
 * d_i = 14336 with the flag, ~1.75 GB without. */
size_t sparse_ffn_backward_workspace_size(sffn_handle_t h, int64_t T);

/* Backward pass of a forward of T tokens ("Continual LLM Upcycling",
 * gist.science technical summary, Methodologie > 1. Architectuur, Executie >
 * Backward Pass: the top-k is crossed by a soft, sigmoid-like local
 * gradient around the selection threshold so that the loss reaches the
 * predictor). Gradients of L = sum(y * g_y):
 *   x, g_y  [T, d] bf16 (device): the forward's input and dL/dy
 *   mask    [T, d_i/64] uint64 (device): the mask the forward returned
 *   tau     > 0: temperature of the surrogate (INFINITY: no surrogate term)
 *   g_x [T, d], g_A [rank, d], g_B [d_i, rank], g_W_g, g_W_u [d_i, d],
 *   g_W_d [d, d_i]: fp32 outputs (device, overwritten); g_bias [d_i] fp32 or
 *   NULL (the layer's bias gradient; zeros for a layer without bias)
 * The forward's hard mask is differentiated as sigmoid((p - theta) / tau),
 * theta the midpoint of the bank's smallest kept and largest dropped logit
 * (held constant); the mask gradient is taken for every channel, so gate and
 * up are recomputed densely; z's bf16 rounding passes gradients unchanged;
 * keep = 64 has no surrogate term. bf16 layers with the predictor or silu
 * gate only (SFFN_ERR_UNSUPPORTED otherwise). Asynchronous on hip_stream;
 * allocates nothing; T == 0 writes zero weight gradients (x, g_y, mask, g_x
 * and the workspace may then be NULL). */
sffn_status_t sparse_ffn_backward(sffn_handle_t h, const void* x, const void* g_y,
                                  const uint64_t* mask, int64_t T, float tau,
                                  float* g_x, float* g_A, float* g_B, float* g_bias,
                                  float* g_Wg, float* g_Wu, float* g_Wd,
                                  void* workspace, size_t ws_bytes, void* hip_stream);

/* Free the handle (host memory only; `packed` stays the caller's). */
void sparse_ffn_destroy(sffn_handle_t h);

/* Static description of a status code. */
const char* sparse_ffn_status_string(sffn_status_t s);

/* Detail of the last failure on the calling thread ("" if none). */
const char* sparse_ffn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_FFN_H */
