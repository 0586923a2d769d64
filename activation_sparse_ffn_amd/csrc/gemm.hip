// Dense-masked MFMA path of the sparse FFN forward for many tokens (batched
// decode, prefill chunks). With independent per-token masks the union of
// kept channels over a tile of tokens is (nearly) every channel, so the
// contraction runs dense on the matrix cores and the mask is applied in the
// gate/up epilogue -- the GPU execution the method's authors describe
// ("Continual LLM Upcycling", gist.science technical summary,
// 3. Hardware Implicaties), with the gate taken from the predictor
// (Methodologie > 1. Architectuur) and off-mask channels exactly zero.
//
//   Z = bf16(X A^T)                 k_gemm<EPI_BF16>
//   P = Z B^T + bias (fp32)         k_gemm<EPI_F32_BIAS>
//   mask = bank top-k of P          k_bank_topk
//   H = select(m, s * U * V, 0)     k_gemm<EPI_GATEUP>, U = X W_g^T, V = X W_u^T
//   Y = bf16(H W_d^T)               k_gemm<EPI_BF16>
//
// Every GEMM is C[M, N] = A[M, K] B[N, K]^T with both operands K-contiguous
// bf16 and fp32 accumulation on v_mfma_f32_32x32x16_bf16.
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

enum { EPI_BF16 = 0, EPI_F32_BIAS = 1, EPI_GATEUP = 2 };

struct GemmParams {
    const uint16_t* A;   // [M, K]
    const uint16_t* B0;  // [N, K]
    const uint16_t* B1;  // [N, K] (gate/up: W_u) or null
    int64_t M;
    int N, K;
    // outputs / epilogue operands
    uint16_t* Cb;        // bf16 [M, N]
    float* Cf;           // fp32 [M, N]
    const float* bias;   // [N] or null
    const float* P;      // gate/up: logits [M, N]
    const uint64_t* mask;// gate/up: [M, N/64]
    int gate;            // 0 predictor, 1 silu
};

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDS_STRIDE = BK + 8;   // elements; 80-byte rows keep 16-byte alignment

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm(const GemmParams p) {
    constexpr int NB = (EPI == EPI_GATEUP) ? 2 : 1;
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[NB][BN * LDS_STRIDE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;
    const int n_tiles = (p.N + BN - 1) / BN;
    const int64_t mt = blockIdx.x % ((p.M + BM - 1) / BM);
    const int nt = (int)(blockIdx.x / ((p.M + BM - 1) / BM));
    if (nt >= n_tiles) return;
    const int64_t m0 = mt * BM;
    const int n0 = nt * BN;

    // global -> register staging: each thread moves 2 chunks of 8 elements
    // per operand tile (128 rows x 4 chunks)
    uint4 ra[2], rb[NB][2];
    auto load_tiles = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, kc = (c & 3) * 8;
            const int64_t gm = m0 + row;
            ra[i] = (gm < p.M) ? *reinterpret_cast<const uint4*>(p.A + gm * p.K + k0 + kc)
                               : make_uint4(0, 0, 0, 0);
            const int gn = n0 + row;
            rb[0][i] = (gn < p.N) ? *reinterpret_cast<const uint4*>(p.B0 + (int64_t)gn * p.K + k0 + kc)
                                  : make_uint4(0, 0, 0, 0);
            if constexpr (NB == 2)
                rb[1][i] = (gn < p.N) ? *reinterpret_cast<const uint4*>(p.B1 + (int64_t)gn * p.K + k0 + kc)
                                      : make_uint4(0, 0, 0, 0);
        }
    };
    auto store_tiles = [&]() {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + 256 * i;
            const int row = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<uint4*>(&As[row * LDS_STRIDE + kc]) = ra[i];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                *reinterpret_cast<uint4*>(&Bs[b][row * LDS_STRIDE + kc]) = rb[b][i];
        }
    };

    f32x16 acc[NB][2][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;

    const int kt_n = p.K / BK;
    load_tiles(0);
    for (int kt = 0; kt < kt_n; ++kt) {
        store_tiles();
        __syncthreads();
        if (kt + 1 < kt_n) load_tiles((kt + 1) * BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            const int ko = kk + 8 * (lane >> 5);
            bf16x8 af[2], bfr[NB][2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int row = wm * 64 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const bf16x8*>(&As[row * LDS_STRIDE + ko]);
            }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int row = wn * 64 + j * 32 + (lane & 31);
                    bfr[b][j] = *reinterpret_cast<const bf16x8*>(&Bs[b][row * LDS_STRIDE + ko]);
                }
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j],
                                                                               acc[b][i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // epilogue: lane holds column (lane & 31) and rows (v & 3) + 8 (v >> 2) + 4 (lane >> 5)
    const int nb64 = p.N / kBank;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = n0 + wn * 64 + j * 32 + (lane & 31);
            if (n >= p.N) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t m = m0 + wm * 64 + i * 32 + (v & 3) + 8 * (v >> 2) + 4 * (lane >> 5);
                if (m >= p.M) continue;
                const int64_t o = m * p.N + n;
                if constexpr (EPI == EPI_BF16) {
                    p.Cb[o] = f32_to_bf16(acc[0][i][j][v]);
                } else if constexpr (EPI == EPI_F32_BIAS) {
                    p.Cf[o] = acc[0][i][j][v] + (p.bias ? p.bias[n] : 0.f);
                } else {
                    const float u = acc[0][i][j][v];
                    const float vv = acc[NB - 1][i][j][v];
                    const bool keep = (p.mask[m * nb64 + (n >> 6)] >> (n & 63)) & 1ull;
                    const float s = p.gate ? sigmoidf_dev(u) : sigmoidf_dev(p.P[o]);
                    p.Cb[o] = keep ? f32_to_bf16(s * u * vv) : (uint16_t)0;
                }
            }
        }
}

template <int EPI>
static void gemm(const GemmParams& p, hipStream_t s, void* const* events, int stage) {
    const int64_t mt = (p.M + BM - 1) / BM;
    const int64_t nt = (p.N + BN - 1) / BN;
    xlaunch(events, stage, k_gemm<EPI>, dim3((unsigned)(mt * nt)), dim3(256), 0, s, p);
}

hipError_t launch_mfma_forward(const MfmaArgs& a, hipStream_t s) {
    GemmParams g{};
    // Z = bf16(X A^T)
    g.A = a.x; g.B0 = a.A; g.M = a.T; g.N = a.rank; g.K = a.d; g.Cb = a.z;
    gemm<EPI_BF16>(g, s, a.events, 0);
    // P = Z B^T + bias
    g = GemmParams{};
    g.A = a.z; g.B0 = a.B; g.M = a.T; g.N = a.d_i; g.K = a.rank; g.Cf = a.logits; g.bias = a.bias;
    gemm<EPI_F32_BIAS>(g, s, a.events, 1);
    // mask
    hipError_t e = launch_bank_topk(a.logits, a.T, a.d_i, a.keep, a.mask, nullptr, s, a.events, 2);
    if (e != hipSuccess) return e;
    // H = select(m, s u v, 0)
    g = GemmParams{};
    g.A = a.x; g.B0 = a.W_g; g.B1 = a.W_u; g.M = a.T; g.N = a.d_i; g.K = a.d; g.Cb = a.h;
    g.P = a.logits; g.mask = a.mask; g.gate = a.gate;
    gemm<EPI_GATEUP>(g, s, a.events, 3);
    // Y = bf16(H W_d^T)
    g = GemmParams{};
    g.A = a.h; g.B0 = a.W_d; g.M = a.T; g.N = a.d; g.K = a.d_i; g.Cb = a.y;
    gemm<EPI_BF16>(g, s, a.events, 4);
    return hipGetLastError();
}

}  // namespace sffn
