// Host-side launchers of the sparse FFN kernels. Each returns the
// hipGetLastError() of its launches; callers have validated every argument.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sffn {

enum class Dt { F32 = 0, BF16 = 1 };

constexpr int kStages = 5;

// gate values (sffn_gate_t)
constexpr int kGatePredictor = 0, kGateSilu = 1, kGateAmplitude = 2;

// Launches one stage's kernel. With profiling events attached, events[2i]
// and events[2i+1] take the start and end timestamps of this kernel's own
// dispatch (hipExtLaunchKernel), so host launch gaps are not counted.
// Records the start and stop events of stages [from, kStages) back to back,
// for a path with fewer kernels than kStages.
inline void skip_stages(void* const* events, int from, hipStream_t s) {
    if (!events) return;
    for (int i = 2 * from; i < 2 * kStages; ++i)
        (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
}

// Records the start and stop events of stages [from, to) back to back, for
// stages a call skips.
inline void skip_range(void* const* events, int from, int to, hipStream_t s) {
    if (!events) return;
    for (int i = 2 * from; i < 2 * to; ++i)
        (void)hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
}

// Compute units of the current device, asked once per device (every thread
// that races on the first call stores the same value).
inline int compute_units() {
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return 256;
        __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
    }
    return n;
}

// Every channel kept: n_words mask words of all ones.
hipError_t launch_fill_mask(uint64_t* mask, int64_t n_words, hipStream_t s);

template <typename F, typename... Args>
inline void xlaunch(void* const* events, int stage, F kernel, dim3 grid, dim3 block,
                    uint32_t shmem, hipStream_t s, Args... args) {
    hipEvent_t e0 = events ? static_cast<hipEvent_t>(events[2 * stage]) : nullptr;
    hipEvent_t e1 = events ? static_cast<hipEvent_t>(events[2 * stage + 1]) : nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, e0, e1, 0u, args...);
}

// ---- gate tiles ------------------------------------------------------------
// Gate input of the 256 x 128 gate/up GEMM tiles (d_i % 128 == 0), written by
// the fused predictor-layer-2 + top-k GEMM, one contiguous tile per output
// block (t / 256, j / 128) of 256 rows (tokens) of gate_row_bytes each. Rows
// t >= T of the last tile are not written.
//  * compact (keep <= kGateCompactMax): a row holds, for each of the block's
//    two banks, the kept channels' positions in the bank (one byte each, in
//    channel order, padded to gate_ids_bytes), then, for the predictor gate
//    only, for each bank their fp16 sigmoid(p) in the same order (padded to
//    gate_vals_bytes).
//  * full (keep > kGateCompactMax): fp16 G[t % 256][j % 128] = sigmoid(p)
//    (predictor gate) or 1 (silu gate) for kept channels, -1 for dropped ones.
constexpr int kGateTileRows = 256, kGateTileCols = 128;
constexpr uint16_t kGateDropped = 0xbc00;   // fp16 -1.0
constexpr int kGateCompactMax = 40;         // largest keep whose compact row fits 256 bytes
__host__ __device__ inline bool gate_compact(int keep) { return keep <= kGateCompactMax; }
__host__ __device__ inline int gate_ids_bytes(int keep) { return (keep + 15) / 16 * 16; }
__host__ __device__ inline int gate_vals_bytes(int keep) { return (2 * keep + 15) / 16 * 16; }
__host__ __device__ inline int gate_row_bytes(int keep, int gate) {
    return gate_compact(keep)
               ? 2 * gate_ids_bytes(keep) + (gate == kGatePredictor ? 2 * gate_vals_bytes(keep) : 0)
               : 2 * kGateTileCols;
}
// bytes of the gate tiles for T tokens
inline size_t gate_tiles_bytes(int64_t T, int d_i, int keep, int gate) {
    return (size_t)((T + kGateTileRows - 1) / kGateTileRows) * (size_t)(d_i / kGateTileCols) * kGateTileRows *
           (size_t)gate_row_bytes(keep, gate);
}

// ---- bank top-k of fp32 logits [T, d_i]: mask words, optional kept ids ------
hipError_t launch_bank_topk(const float* logits, int64_t T, int d_i, int keep,
                            uint64_t* mask, uint16_t* ids, hipStream_t s,
                            void* const* events = nullptr, int stage = 0);

// ---- token-gather path (VALU; decode and fp32 layers) ---------------------
struct GatherArgs {
    Dt dt;
    int d, d_i, rank, keep, gate;   // gate: 0 predictor, 1 silu
    int64_t T;
    const void* x;                  // [T, d]
    const void* A;                  // [rank, d]
    const void* B;                  // [d_i, rank]
    const float* bias;              // [d_i] or null
    const void* W_g;                // [d_i, d]
    const void* W_u;                // [d_i, d]
    const void* W_dT;               // [d_i, d] (W_d transposed)
    void* y;                        // [T, d]
    float* z;                       // [T, rank]       workspace
    uint64_t* mask;                 // [T, d_i/64]
    float* logits;                  // [T, d_i] or null
    uint16_t* ids;                  // [T, d_s]        workspace
    float* pk;                      // [T, d_s]        kept logits
    float* h;                       // [T, d_s]        kept activations
    float* partial;                 // [T, groups, d]  down partial sums
    float* amp;                     // [T, d_i] amplitudes (amplitude gate only)
    bool need_pred;                 // false: every channel kept with the silu gate
                                    // and no logits asked for, so no predictor
    bool mask_requested;            // mask points at the caller's mask_out
    void* const* events;            // null or 2 * kStages hipEvent_t
};
int gather_groups(int d_s);
bool fused_ok(const GatherArgs& a);   // the fused per-bank decode kernel applies
hipError_t launch_gather_forward(const GatherArgs& a, hipStream_t s);

// ---- dense-masked MFMA path (bf16, many tokens) ---------------------------
struct MfmaArgs {
    int d, d_i, rank, keep, gate;
    int64_t T;
    const uint16_t* x;      // [T, d]
    const uint16_t* A;      // [rank, d]
    const uint16_t* B;      // [d_i, rank]
    const float* bias;      // [d_i] or null
    const uint16_t* W_g;    // [d_i, d]
    const uint16_t* W_u;    // [d_i, d]
    const uint16_t* W_dT;   // [d_i, d]: W_d transposed, read K-major by the down GEMMs
    uint16_t* y;            // [T, d]
    uint16_t* z;            // [T, rank]   workspace
    float* logits;          // [T, d_i]
    uint64_t* mask;         // [T, d_i/64]
    uint16_t* h;            // [T, d_i]    workspace
    uint8_t* gate_tiles;    // gate tiles (see gate_row_bytes) or null
    uint64_t* union_w;      // skinny path: [d_i / 64] or of the batch's mask words
    float* z_partial;       // [z_splits, T, rank] K-split partials of z, or null
    bool logits_requested;  // logits points at the caller's logits_out
    bool need_pred;         // false: every channel kept with the silu gate and no
                            // logits asked for, so no predictor and no top-k
    bool mask_requested;    // mask points at the caller's mask_out
    void* const* events;    // null or 2 * kStages hipEvent_t
};
// K splits of predictor layer 1 on the MFMA path (1 = no split)
int z_splits(int64_t T, int d);
// predictor layer 2 and the bank top-k run as one kernel (with gate tiles)
bool mfma_fused_topk(int64_t T, int d, int d_i, int rank);
hipError_t launch_mfma_forward(const MfmaArgs& a, hipStream_t s);
// the Dense-4x baseline on the MFMA path: dense gate/up with the amplitude
// top-k in its epilogue (mask, masked bf16 h, amplitudes into logits when
// asked for), then the down GEMM
hipError_t launch_amp_mfma(const MfmaArgs& a, hipStream_t s);
// the same for 4 < T <= 64 on the skinny kernels (amplitudes through logits)
hipError_t launch_amp_skinny(const MfmaArgs& a, float* partial, hipStream_t s);
// bank top-k of |amp| [T, d_i]: mask words and the masked bf16 h [T, d_i]
hipError_t launch_amp_mask(const float* amp, int64_t T, int d_i, int keep, uint64_t* mask, uint16_t* h_dense,
                           hipStream_t s, void* const* events, int stage);

// ---- skinny MFMA path (bf16, 4 < T <= 64, rank % 64 == 0) -----------------
size_t skinny_partial_floats(int64_t T, int d, int rank, int d_i);
hipError_t launch_skinny_forward(const MfmaArgs& a, float* partial, hipStream_t s);

// ---- packing ---------------------------------------------------------------
// dst [cols][ld] = src [rows][cols] transposed; dst entries [rows, ld) of each
// row are zero (ld <= rows: ld = rows)
hipError_t launch_transpose(Dt dt, const void* src, void* dst, int rows, int cols,
                            hipStream_t s, int ld = 0);

// ---- plain GEMMs for the backward pass --------------------------------------
// C[M, N] (row stride N) = A[M, K] B[N, K]^T (+ bias[col] for F32), bf16
// operands (K contiguous), fp32 accumulation; K must be a multiple of 32.
// Thin shapes split K when `partial` holds gemm_nt_partial_floats(M, N, K)
// floats (null: no split).
enum class GemmOut { F32, F32_ACC, BF16 };   // store fp32, add to fp32, store bf16
size_t gemm_nt_partial_floats(int64_t M, int N, int K);
hipError_t launch_gemm_nt(const uint16_t* A, const uint16_t* B, int64_t M, int N, int K, void* C,
                          GemmOut out, hipStream_t s, const float* bias = nullptr, float* partial = nullptr);
// dense U = X W_g^T and V = X W_u^T, rounded to bf16 [T, d_i] each
hipError_t launch_uv_gemm(const uint16_t* x, const uint16_t* W_g, const uint16_t* W_u, int64_t T, int d_i,
                          int d, uint16_t* U, uint16_t* V, hipStream_t s);

// ---- backward pass (bf16 layers, predictor or silu gate) ----------------------
struct BwdArgs {
    int d, d_i, rank, keep, gate;
    int64_t T;
    float inv_tau;                  // 1 / tau (0: no surrogate term)
    const uint16_t* x;              // [T, d]
    const uint16_t* g_y;            // [T, d]
    const uint64_t* mask;           // [T, d_i/64] the forward's mask
    const uint16_t* A;              // [rank, d]
    const uint16_t* B;              // [d_i, rank]
    const float* bias;              // [d_i] or null
    const uint16_t* W_g;            // [d_i, d]
    const uint16_t* W_u;            // [d_i, d]
    const uint16_t* W_dT;           // [d_i, d]
    const uint16_t* W_gT;           // [d, d_i] or null (then transposed into the workspace)
    const uint16_t* W_uT;           // [d, d_i] or null
    float *g_x, *g_A, *g_B, *g_bias, *g_Wg, *g_Wu, *g_Wd;   // outputs (g_bias may be null)
    void* ws;                       // workspace of backward_workspace_bytes(...)
};
// weights_t: W_g^T and W_u^T come with the layer (no room for them needed)
size_t backward_workspace_bytes(int64_t T, int d, int d_i, int rank, bool weights_t);
hipError_t launch_backward(const BwdArgs& a, hipStream_t s);
// x[0 .. n) = 0
hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t s);

}  // namespace sffn
