// Dense-masked MFMA path of the sparse FFN forward for many tokens (batched
// decode, prefill chunks). With independent per-token masks the union of
// kept channels over a tile of tokens is (nearly) every channel, so the
// contraction runs dense on the matrix cores and the mask is applied in the
// gate/up epilogue -- the GPU execution the method's authors describe
// ("Continual LLM Upcycling", gist.science technical summary,
// 3. Hardware Implicaties), with the gate taken from the predictor
// (Methodologie > 1. Architectuur) and off-mask channels exactly zero.
//
//   Z = bf16(X A^T)                 k_gemm<EPI_BF16>, or (T >= 256) K-split
//                                   k_gemm<EPI_PARTIAL> + k_sum_splits_bf16
//   P = Z B^T + bias (fp32)         k_gemm<EPI_F32_BIAS>
//   mask = bank top-k of P          k_bank_topk
//     (T >= 256, d_i % 128 == 0: P, the top-k and the gate tiles in one
//      kernel, k_gemm<EPI_TOPK>)
//   H = select(m, s * U * V, 0)     k_gemm<EPI_GATEUP> / k_gemm256<EPI_GATEUP>
//                                   (persistent with compact gate tiles),
//                                   U = X W_g^T, V = X W_u^T
//   Y = bf16(H W_d^T)               k_gemm256 / k_gemm <EPI_BF16, K-major W_d^T>
//
// Every GEMM is C[M, N] = A[M, K] B[N, K]^T with A K-contiguous bf16 and
// fp32 accumulation on v_mfma_f32_32x32x16_bf16. B is K-contiguous as well,
// except in the down projection (KMAJOR): there B is W_d^T [K = d_i][N = d],
// the layout the decode path gathers rows from, so the layer keeps one copy
// of W_d; its slabs land in LDS row for row and the fragments come out
// through transposed LDS reads (kmajor_frag).
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

enum { EPI_BF16 = 0, EPI_F32_BIAS = 1, EPI_GATEUP = 2, EPI_PARTIAL = 3, EPI_TOPK = 4, EPI_AMP = 5,
       EPI_F32_ACC = 6, EPI_UV = 7 };

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
    const uint8_t* G;    // gate/up, 256-row tiles: gate tiles instead of P and mask
    int gate;            // 0 predictor, 1 silu
    int kn;              // EPI_PARTIAL: K range of one split (blockIdx.y selects the split)
    // EPI_TOPK: logits (+ bias) go through LDS into the bank top-k; Cf receives
    // the logits only when non-null
    uint64_t* mask_w;    // [M, N/64]
    uint8_t* gate_w;     // gate tiles (layout: gate_row_bytes)
    int keep;            // EPI_TOPK, and the gate tiles' layout
    int dense;           // EPI_GATEUP without gate tiles: every channel kept (silu gate)
    uint16_t* Cb2;       // EPI_UV: bf16 [M, N] receives V (Cb receives U)
};

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kTopkPitch = 64 * 4 + 16;   // bytes per bank-row of the top-k epilogue's logit tile
constexpr int LDS_STRIDE = BK + 8;   // elements; 80-byte rows keep 16-byte alignment

// LDS slab layout shared by the LDS-direct loops: a slab holds rows of 64
// bf16 (128 bytes, eight 16-byte chunks); chunk g of row r sits in slot
// g ^ ((r >> 1) & 7), which spreads a fragment read over all LDS banks.
__device__ __forceinline__ int slab_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int slab_off(int r, int g) { return r * 128 + ((g ^ slab_swz(r)) << 4); }

constexpr int TKD = 64;                  // K step of the LDS-direct loops
constexpr int SLAB128 = BM * TKD * 2;    // one 128-row slab: 16 KB

// DMA: the LDS-direct loop (K range a multiple of 64): slabs go global ->
// LDS with global_load_lds_dwordx4 into two buffers (separate arrays, loop
// unrolled by two), fragment reads interleaved one per MFMA with the
// sub-step before, and the barrier before each step's last sub-step. Else
// the register-staged loop with 32-wide K steps.
template <int EPI, bool DMA, bool KMAJOR = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(EPI == EPI_TOPK ? 2 : 1))) void k_gemm(const GemmParams p) {
    constexpr int NB = (EPI == EPI_GATEUP || EPI == EPI_UV) ? 2 : 1;
    static_assert(!KMAJOR || (DMA && EPI == EPI_BF16), "a K-major B only for the plain bf16 GEMM, LDS-direct");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv >> 1, wn = wv & 1;
    const int r32 = lane & 31, hk = lane >> 5;
    const int n_tiles = (p.N + BN - 1) / BN;
    const int64_t mt = blockIdx.x % ((p.M + BM - 1) / BM);
    const int nt = (int)(blockIdx.x / ((p.M + BM - 1) / BM));
    if (nt >= n_tiles) return;
    const int64_t m0 = mt * BM;
    const int n0 = nt * BN;
    const int kn = EPI == EPI_PARTIAL ? p.kn : p.K;      // this workgroup's K range
    const int kb = EPI == EPI_PARTIAL ? (int)blockIdx.y * p.kn : 0;

    f32x16 acc[NB][2][2];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[b][i][j][v] = 0.f;
    auto mma = [&](const bf16x8 (&af)[2], const bf16x8 (&bfr)[NB][2]) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[b][j], acc[b][i][j], 0, 0, 0);
    };
    // EPI_TOPK: the fp32 logit tile as 256 bank-rows (64 floats + 16 bytes of
    // padding), rows 0..127 in `tile_lo`, 128..255 in `tile_hi` (the freed
    // staging buffers, enlarged to hold them)
    constexpr int TOPK_HALF = 128 * kTopkPitch;
    char* tile_lo;
    char* tile_hi;

    if constexpr (DMA) {
        constexpr int BUF = (EPI == EPI_TOPK && TOPK_HALF > (1 + NB) * SLAB128) ? TOPK_HALF : (1 + NB) * SLAB128;
        __shared__ __attribute__((aligned(16))) char buf0[BUF];
        __shared__ __attribute__((aligned(16))) char buf1[BUF];
        // per-thread fetch rows: chunk c = tid + 256 i -> row c / 8, slot c % 8
        // (lane l of a wave lands at base + 16 l). Rows past M or N read row
        // 0: their results are never stored.
        const int fs = tid & 7;
        const uint16_t* asrc[4];
        const uint16_t* bsrc[NB][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = (tid >> 3) + 32 * i;
            const int gch = fs ^ slab_swz(r);
            const int64_t m = m0 + r;
            asrc[i] = p.A + (m < p.M ? m : 0) * p.K + kb + 8 * gch;
            if constexpr (KMAJOR) {
                // K-major B: chunk c = tid + 256 i of the slab is K-row c / 16,
                // slot c % 16, holding chunk (c % 16) ^ (4 (row & 3)) of the
                // row's 128 columns; columns past N read column 0 (never stored)
                const int kr = (tid >> 4) + 16 * i;
                const int col = n0 + 8 * kmajor_slot<BN * 2>(kr, tid & 15);
                bsrc[0][i] = p.B0 + (size_t)(kb + kr) * p.N + (col < p.N ? col : 0);
            } else {
                const int n = n0 + r;
                const int64_t nr = n < p.N ? n : 0;
                bsrc[0][i] = p.B0 + nr * p.K + kb + 8 * gch;
                if constexpr (NB == 2) bsrc[1][i] = p.B1 + nr * p.K + kb + 8 * gch;
            }
        }
        const size_t bstep = KMAJOR ? (size_t)p.N : 1;     // B elements per unit of K
        auto fetch = [&](int k0, char* dst) {
            char* wbase = dst + wv * (kWave * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)(asrc[i] + k0),
                                                 (__attribute__((address_space(3))) void*)(wbase + i * 4096), 16, 0, 0);
#pragma unroll
                for (int b = 0; b < NB; ++b)
                    __builtin_amdgcn_global_load_lds(
                        (const __attribute__((address_space(1))) void*)(bsrc[b][i] + k0 * bstep),
                        (__attribute__((address_space(3))) void*)(wbase + (1 + b) * SLAB128 + i * 4096), 16, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        };
        auto frags = [&](const char* S, int sub, bf16x8 (&af)[2], bf16x8 (&bfr)[NB][2]) {
            const int gch = 2 * sub + hk;
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(S + slab_off(wm * 64 + i * 32 + r32, gch));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if constexpr (KMAJOR)
                        bfr[b][j] = kmajor_frag<BN * 2>(S + (1 + b) * SLAB128, wn * 64 + j * 32, sub, lane);
                    else
                        bfr[b][j] = *reinterpret_cast<const bf16x8*>(S + (1 + b) * SLAB128 +
                                                                      slab_off(wn * 64 + j * 32 + r32, gch));
                }
        };
        auto landed = [&]() {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        };
        auto interleave = [&]() {
            // LDS reads of a sub-step (a K-major B fragment takes two) and MFMAs
            constexpr int R = 2 + (KMAJOR ? 4 : 2) * NB, M = 4 * NB;
            constexpr int P = R < M ? R : M;
#pragma unroll
            for (int i = 0; i < P; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if constexpr (M > P) __builtin_amdgcn_sched_group_barrier(0x008, M - P, 0);
            if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        const int kt_n = kn / TKD;
        bf16x8 xa[2], xb[NB][2], ya[2], yb[NB][2];
        auto step = [&](char* cur, const char* nxt, int kt) {
            mma(xa, xb); frags(cur, 1, ya, yb); interleave();
            mma(ya, yb); frags(cur, 2, xa, xb); interleave();
            mma(xa, xb); frags(cur, 3, ya, yb); interleave();
            landed();                               // slab kt + 1 is in LDS, `cur` is free
            if (kt + 2 < kt_n) fetch((kt + 2) * TKD, cur);
            mma(ya, yb);
            frags(nxt, 0, xa, xb);                  // after the last step: stale, unused
            interleave();
        };
        fetch(0, buf0);
        landed();
        if (kt_n > 1) fetch(TKD, buf1);
        frags(buf0, 0, xa, xb);
        int kt = 0;
        for (; kt + 2 <= kt_n; kt += 2) {
            step(buf0, buf1, kt);
            step(buf1, buf0, kt + 1);
        }
        if (kt < kt_n) step(buf0, buf1, kt);
        __syncthreads();                           // every wave is done with the buffers
        tile_lo = buf0;
        tile_hi = buf1;
    } else {
        constexpr int STAGE_BYTES = (BM + NB * BN) * LDS_STRIDE * 2;
        constexpr int TILE_BYTES = EPI == EPI_TOPK ? 2 * TOPK_HALF : 0;   // fp32 logits tile
        __shared__ __attribute__((aligned(16))) char smem[STAGE_BYTES > TILE_BYTES ? STAGE_BYTES : TILE_BYTES];
        uint16_t* const As = reinterpret_cast<uint16_t*>(smem);
        auto BS = [&](int b) { return As + (BM + b * BN) * LDS_STRIDE; };
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
                    *reinterpret_cast<uint4*>(&BS(b)[row * LDS_STRIDE + kc]) = rb[b][i];
            }
        };
        const int kt_n = kn / BK;
        load_tiles(kb);
        for (int kt = 0; kt < kt_n; ++kt) {
            store_tiles();
            __syncthreads();
            if (kt + 1 < kt_n) load_tiles(kb + (kt + 1) * BK);
#pragma unroll
            for (int kk = 0; kk < BK; kk += 16) {
                const int ko = kk + 8 * hk;
                bf16x8 af[2], bfr[NB][2];
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int row = wm * 64 + i * 32 + r32;
                    af[i] = *reinterpret_cast<const bf16x8*>(&As[row * LDS_STRIDE + ko]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int row = wn * 64 + j * 32 + r32;
                        bfr[b][j] = *reinterpret_cast<const bf16x8*>(&BS(b)[row * LDS_STRIDE + ko]);
                    }
                mma(af, bfr);
            }
            __syncthreads();
        }
        tile_lo = smem;
        tile_hi = smem + TOPK_HALF;
    }

    // epilogue: lane holds column (lane & 31) and rows (v & 3) + 8 (v >> 2) + 4 (lane >> 5)
    const int nb64 = p.N / kBank;
    if constexpr (EPI == EPI_TOPK) {
        // logits (+ bias) into LDS as 256 bank-rows q = 2 row + (col >> 6),
        // kTopkPitch bytes apart; the staging buffers are free (the K loop
        // ended on a barrier). Wave wm holds rows 64 wm .. 64 wm + 63, all in
        // one half, and a value's address is a per-lane base plus a constant,
        // so the stores need no address arithmetic. The 16-byte padding puts
        // the two rows one store instruction touches (lanes 0-31 and 32-63,
        // rows 4 apart) on disjoint banks, and the 16 bank-rows of one quarter
        // of a 16-byte-per-lane read on distinct banks.
        char* const half = wm == 0 ? tile_lo : tile_hi;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int col = wn * 64 + j * 32 + (lane & 31);
                const int n = n0 + col;
                const float bj = (p.bias && n < p.N) ? p.bias[n] : 0.f;
                char* const base = half + (2 * (i * 32 + 4 * hk) + (col >> 6)) * kTopkPitch + (col & 63) * 4;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    *reinterpret_cast<float*>(base + (2 * ((v & 3) + 8 * (v >> 2))) * kTopkPitch) =
                        acc[0][i][j][v] + bj;
            }
        __syncthreads();
        // one bank-row per lane
        const int q = wv * kWave + lane;
        const int row = q >> 1, bsel = q & 1;
        const int64_t t = m0 + row;
        const int j0 = n0 + bsel * kBank;
        const char* trow = (q < 128 ? tile_lo : tile_hi) + (q & 127) * kTopkPitch;
        auto ld = [&](int c) { return *reinterpret_cast<const float4*>(trow + 16 * c); };
        const uint64_t sel = lane_select64(ld, p.keep);
        if (t >= p.M || j0 >= p.N) return;
        p.mask_w[t * nb64 + j0 / kBank] = sel;
        if (p.Cf != nullptr) {
#pragma unroll
            for (int c = 0; c < 16; ++c) reinterpret_cast<float4*>(p.Cf + t * p.N + j0)[c] = ld(c);
        }
        const int col_tiles = p.N / kGateTileCols;
        const int rb = gate_row_bytes(p.keep, p.gate);
        uint8_t* const grow = p.gate_w +
                              ((size_t)(t / kGateTileRows) * col_tiles + j0 / kGateTileCols) * (kGateTileRows * rb) +
                              (size_t)(t % kGateTileRows) * rb;
        if (gate_compact(p.keep)) {
            // compact row: this bank's kept channel positions in channel
            // order and (predictor gate) their sigmoid(p), built in registers
            const int ib = gate_ids_bytes(p.keep), vb = gate_vals_bytes(p.keep);
            const bool pred = p.gate == kGatePredictor;
            constexpr int IW = (kGateCompactMax + 15) / 16 * 4, VW = (2 * kGateCompactMax + 15) / 16 * 4;
            uint32_t idw[IW], vw[VW];
#pragma unroll
            for (int w = 0; w < IW; ++w) idw[w] = 0;
#pragma unroll
            for (int w = 0; w < VW; ++w) vw[w] = 0;
            uint64_t m = sel;
            // fully unrolled (register indices fixed at compile time), each
            // step under a uniform test instead of a loop exit
#pragma unroll
            for (int k = 0; k < kGateCompactMax; ++k) {
                if (k < p.keep) {
                    const int c = __builtin_ctzll(m);
                    m &= m - 1;
                    idw[k >> 2] |= (uint32_t)c << (8 * (k & 3));
                    if (pred) {
                        const float v = *reinterpret_cast<const float*>(trow + 4 * c);
                        vw[k >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sigmoidf_dev(v))
                                      << (16 * (k & 1));
                    }
                }
            }
            uint8_t* const gi = grow + bsel * ib;
#pragma unroll
            for (int c = 0; c < IW / 4; ++c)
                if (16 * c < ib)
                    *reinterpret_cast<uint4*>(gi + 16 * c) =
                        make_uint4(idw[4 * c], idw[4 * c + 1], idw[4 * c + 2], idw[4 * c + 3]);
            if (pred) {
                uint8_t* const gv = grow + 2 * ib + bsel * vb;
#pragma unroll
                for (int c = 0; c < VW / 4; ++c)
                    if (16 * c < vb)
                        *reinterpret_cast<uint4*>(gv + 16 * c) =
                            make_uint4(vw[4 * c], vw[4 * c + 1], vw[4 * c + 2], vw[4 * c + 3]);
            }
            return;
        }
        uint16_t* const gp = reinterpret_cast<uint16_t*>(grow) + j0 % kGateTileCols;
        // gate values: sigmoid(p) (predictor gate) or 1 (silu gate) where kept
        auto pack = [&](auto gate_of) {
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 v0 = ld(2 * c), v1 = ld(2 * c + 1);
                const float pv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t hw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint16_t h2[2];
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const int ch = 8 * c + 2 * e + k;
                        const float gv = gate_of(pv[2 * e + k]);
                        h2[k] = ((sel >> ch) & 1ull) ? __builtin_bit_cast(uint16_t, (_Float16)gv) : kGateDropped;
                    }
                    hw[e] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
                }
                *reinterpret_cast<uint4*>(gp + 8 * c) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            }
        };
        if (p.gate) pack([](float) { return 1.f; });
        else pack([](float v) { return sigmoidf_dev(v); });
        return;
    }
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
                if constexpr (EPI == EPI_PARTIAL) {
                    p.Cf[(int64_t)blockIdx.y * p.M * p.N + o] = acc[0][i][j][v];
                } else if constexpr (EPI == EPI_BF16) {
                    p.Cb[o] = f32_to_bf16(acc[0][i][j][v]);
                } else if constexpr (EPI == EPI_F32_BIAS) {
                    p.Cf[o] = acc[0][i][j][v] + (p.bias ? p.bias[n] : 0.f);
                } else if constexpr (EPI == EPI_F32_ACC) {
                    p.Cf[o] += acc[0][i][j][v];
                } else if constexpr (EPI == EPI_UV) {
                    p.Cb[o] = f32_to_bf16(acc[0][i][j][v]);
                    p.Cb2[o] = f32_to_bf16(acc[NB - 1][i][j][v]);
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

// ---------------------------------------------------------------------------
// 256 x 256 x 64 tiles for the large contractions (gate/up and down of a
// prefill chunk). 128 WN threads: WN waves along N and 2 along M, each
// owning a 128 x (256 / WN) block of C as accumulator tiles of
// v_mfma_f32_32x32x16_bf16. A K step moves a 256-row x
// 128-byte slab of each operand: eight lanes per row (whole 128-byte lines),
// into LDS with 16-byte chunks XOR-swizzled by row (chunk g of row r at slot
// g ^ ((r >> 1) & 7), so that the 16 consecutive rows one fragment read
// touches fall on distinct banks), double-buffered so the next slab's global
// loads are in flight while the matrix cores work on the current one.
// For the gate/up epilogue the 256 B-rows of a tile are, in blocks of 64,
// [W_g n0.., W_u n0.., W_g n0+64.., W_u n0+64..], so every wave holds u and v
// of the same 64 channels and 128 tokens.
// ---------------------------------------------------------------------------

template <bool B> struct BoolTag { static constexpr bool value = B; };

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int SLAB = TM * TK * 2;                  // bytes of one operand slab (32 KB)


// PERSIST (gate/up with gate tiles only): the grid is one workgroup per
// compute unit and workgroup g walks tiles g, g + G, g + 2 G, ... (G, the
// grid size, a multiple of 8, so every tile of a workgroup falls on the XCD
// that its number gives). When the epilogue has expanded a compact gate tile
// out of slab buffer 0, it requests the next tile's first slab into that
// buffer, so that the load's latency passes under the rest of the epilogue
// (the gate values, the H tile and its stores) instead of opening the next
// tile with an idle wait.
template <int EPI, int WN, bool KMAJOR = false, bool PERSIST = false>
__global__ __launch_bounds__(128 * WN) void k_gemm256(const GemmParams p, int m_tiles, int n_tiles) {
    static_assert(!KMAJOR || EPI == EPI_BF16, "a K-major B only for the plain bf16 GEMM");
    static_assert(!PERSIST || EPI == EPI_GATEUP, "persistent tiles only for gate/up");
    // WN waves along N (2 or 4), 2 along M: each wave owns 128 x (256 / WN) of C
    constexpr bool GU = EPI == EPI_GATEUP || EPI == EPI_AMP || EPI == EPI_UV;   // B = [W_g, W_u] blocks
    constexpr int NT = 128 * WN;                     // threads
    constexpr int WNC = TN / WN;                      // columns per wave
    constexpr int NJ = WNC / 32;                      // accumulator tiles along N
    constexpr int GB = WNC / 2;                       // gate/up interleave block (rows)
    constexpr int NF = TM * 8 / NT;                   // 16-byte fetches per thread per operand
    constexpr int TNC = GU ? TN / 2 : TN;             // output columns per tile
    // tid is opaque again at the top of each persistent tile (below), so that
    // what the epilogue and the gate-tile fetch derive from it is computed per
    // tile rather than held, or spilled, across the K loop
    int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wv / WN, wn = wv % WN;
    const int r32 = lane & 31, hk = lane >> 5;
    const int kt_n = p.K / TK;

    // Tile order: workgroups land on the 8 XCDs round-robin, so workgroup g
    // runs on XCD g % 8; each XCD gets a contiguous run gx of the tile order,
    // which walks groups of GM M-tiles, M fastest within a group. The 32
    // tiles that one XCD runs side by side then form an 8 x 4 block: each A
    // slab is shared by four of them and each B slab by eight in one L2
    // (against 2 and 16 for a plain M-fastest order), which cuts the L2
    // misses per K step by a third. Every 256 x 256 tile streams 64 KB per K
    // step through its compute unit, and the misses' latency is what limits
    // how fast that stream flows.
    const unsigned total = (unsigned)(m_tiles * n_tiles);
    constexpr int GM = 8;
    auto place = [&](unsigned g, int& mt, int& nt) {
        const unsigned gx = (total % 8 == 0) ? (g % 8) * (total / 8) + g / 8 : g;
        const int grp = (int)(gx / (unsigned)(GM * n_tiles));
        const int first_m = grp * GM;
        const int gm = min(m_tiles - first_m, GM);
        const int within = (int)(gx - (unsigned)grp * (unsigned)(GM * n_tiles));
        mt = first_m + within % gm;
        nt = within / gm;
    };
    unsigned tile = blockIdx.x;
    int mt, nt;
    place(tile, mt, nt);
    int64_t m0 = (int64_t)mt * TM;
    int n0 = nt * TNC;

    // per-thread fetch rows: chunk c = tid + NT i -> row c / 8, slot c % 8.
    // Gate/up B rows come in blocks of GB: [W_g, W_u] for channels n0 + GB b ..
    // Rows past M or N read row 0: their results are never stored.
    const int fs = tid & 7;
    const uint16_t* asrc[NF];
    const uint16_t* bsrc[NF];
    auto sources = [&](int64_t mb, int nb0) {
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            const int r = (tid >> 3) + (NT / 8) * i;
            const int gch = fs ^ slab_swz(r);
            const int64_t m = mb + r;
            asrc[i] = p.A + (m < p.M ? m : 0) * p.K + 8 * gch;
            if constexpr (KMAJOR) {
                // K-major B: chunk c = tid + NT i of the slab is K-row c / 32,
                // slot c % 32, holding chunk (c % 32) ^ (4 (row & 3)) of the
                // row's 256 columns; columns past N read column 0 (never stored)
                const int kr = (tid >> 5) + (NT / 32) * i;
                const int col = nb0 + 8 * kmajor_slot<TN * 2>(kr, tid & 31);
                bsrc[i] = p.B0 + (size_t)kr * p.N + (col < p.N ? col : 0);
                continue;
            }
            int n;
            const uint16_t* base;
            if constexpr (GU) {
                const int blk = r / GB;
                n = nb0 + (blk >> 1) * GB + (r % GB);
                base = (blk & 1) ? p.B1 : p.B0;
            } else {
                n = nb0 + r;
                base = p.B0;
            }
            bsrc[i] = base + (size_t)(n < p.N ? n : 0) * p.K + 8 * gch;
        }
    };
    const size_t bstep = KMAJOR ? (size_t)p.N : 1;     // B elements per unit of K
    // gate/up with gate tiles: the gate tile of a 256 x 128 output block is
    // one contiguous block of 256 rows (at most 64 KB)
    auto gate_tile = [&](int mtile, int ntile) -> const uint8_t* {
        if constexpr (EPI == EPI_GATEUP)
            if (p.G != nullptr)
                return p.G + ((size_t)mtile * (p.N / kGateTileCols) + ntile) * (TM * gate_row_bytes(p.keep, p.gate));
        return nullptr;
    };

    f32x16 acc[4][NJ];
    // fragments of sub-step s of the slab pair at As (A slab, then B slab)
    auto frags = [&](const char* As, int s, bf16x8 (&af)[4], bf16x8 (&bfr)[NJ]) {
        const char* Bs = As + SLAB;
        const int gch = 2 * s + hk;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const bf16x8*>(As + slab_off(wm * 128 + i * 32 + r32, gch));
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if constexpr (KMAJOR)
                bfr[j] = kmajor_frag<TN * 2>(Bs, wn * WNC + j * 32, s, lane);
            else
                bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + slab_off(wn * WNC + j * 32 + r32, gch));
        }
    };
    auto mma = [&](const bf16x8 (&af)[4], const bf16x8 (&bfr)[NJ]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    };
    // Slabs go from global memory straight into LDS (global_load_lds_dwordx4:
    // lane l of a wave writes the 16 bytes at base + 16 l, which is where the
    // swizzled layout puts thread tid's chunk), so a fetch holds no registers
    // and has a whole K step to land. The two buffers are separate arrays and
    // the loop is unrolled by two so that every LDS read names a buffer that
    // no load in flight writes.
    __shared__ __attribute__((aligned(16))) char buf0[2 * SLAB];
    __shared__ __attribute__((aligned(16))) char buf1[2 * SLAB];
    auto fetch = [&](int k0, char* dst) {
        char* wbase = dst + wv * (kWave * 16);
#pragma unroll
        for (int i = 0; i < NF; ++i) {
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(asrc[i] + k0),
                (__attribute__((address_space(3))) void*)(wbase + i * NT * 16), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(bsrc[i] + k0 * bstep),
                (__attribute__((address_space(3))) void*)(wbase + SLAB + i * NT * 16), 16, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);     // keep the loads ahead of the MFMAs
    };
    // the gate tile as a plain copy of its 16-byte chunks. The loop always
    // issues the full tile's count of loads (no branch in the K loop); past
    // a compact tile's end they repeat its last chunk into LDS bytes that
    // nothing reads.
    auto fetch_gate = [&](const uint8_t* gt, char* dst) {
        const int last = TM * gate_row_bytes(p.keep, p.gate) / 16 - 1;
        char* wbase = dst + wv * (kWave * 16);
#pragma unroll
        for (int i = 0; i < TM * kGateTileCols * 2 / (NT * 16); ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(gt + (size_t)min(tid + i * NT, last) * 16),
                (__attribute__((address_space(3))) void*)(wbase + i * NT * 16), 16, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    auto landed = [&]() {
        __builtin_amdgcn_s_waitcnt(0);            // this wave's loads and LDS reads are done
        __syncthreads();
    };
    // one MFMA group (a sub-step, 8 MFMAs) with the next group's fragment
    // reads interleaved, one read per MFMA
    auto interleave = [&]() {
        // LDS reads of a sub-step (a K-major B fragment takes two) and MFMAs
        constexpr int R = 4 + (KMAJOR ? 2 : 1) * NJ, M = 4 * NJ, P = R < M ? R : M;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);    // one LDS read
        }
        if constexpr (M > P) __builtin_amdgcn_sched_group_barrier(0x008, M - P, 0);
        if constexpr (R > P) __builtin_amdgcn_sched_group_barrier(0x100, R - P, 0);
        __builtin_amdgcn_sched_barrier(0);
    };
    bf16x8 xa[4], xb[NJ], ya[4], yb[NJ];
    const uint8_t* gtile = nullptr;           // gate tile of the current output block, if any
    bool compact = false;                     // gtile in the compact layout
    // A compact gate tile (at src) expanded into the full fp16 layout (at
    // dst), one (row, bank) per thread: -1 everywhere, then each kept
    // channel's value at its position.
    auto expand = [&](const char* src, char* dst) {
        const int ib = gate_ids_bytes(p.keep), vb = gate_vals_bytes(p.keep);
        const int rb = gate_row_bytes(p.keep, p.gate);
        const uint32_t dropped2 = (uint32_t)kGateDropped * 0x10001u;
        const bool pred = p.gate == kGatePredictor;
        for (int q = tid; q < 2 * TM; q += NT) {
            const int row = q >> 1, bsel = q & 1;
            const char* gi = src + row * rb + bsel * ib;
            const char* gv = src + row * rb + 2 * ib + bsel * vb;
            char* const er = dst + row * 256 + bsel * 128;
#pragma unroll
            for (int c = 0; c < 8; ++c)     // rotated by lane: neighbours start on different banks
                *reinterpret_cast<uint4*>(er + 16 * ((c + tid) & 7)) =
                    make_uint4(dropped2, dropped2, dropped2, dropped2);
            // 16 kept channels at a time: their positions (one 16-byte
            // chunk) and values (two), requested together
            for (int k0 = 0; k0 < p.keep; k0 += 16) {
                const uint4 ids = *reinterpret_cast<const uint4*>(gi + k0);
                const uint32_t iw[4] = {ids.x, ids.y, ids.z, ids.w};
                uint32_t vw[8];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    uint4 w = make_uint4(0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u);   // fp16 1: silu
                    if (pred && 2 * k0 + 16 * c < vb) w = *reinterpret_cast<const uint4*>(gv + 2 * k0 + 16 * c);
                    vw[4 * c] = w.x; vw[4 * c + 1] = w.y; vw[4 * c + 2] = w.z; vw[4 * c + 3] = w.w;
                }
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const int c = (iw[k >> 2] >> (8 * (k & 3))) & 63;
                    if (k0 + k < p.keep)
                        *reinterpret_cast<uint16_t*>(er + 2 * c) = (uint16_t)(vw[k >> 1] >> (16 * (k & 1)));
                }
            }
        }
    };
    // K step kt from slab `cur` (sub-step 0 already in x); the barrier sits
    // before the last sub-step, so that sub-step's MFMAs cover the barrier
    // and the first reads of the next slab
    auto step = [&](char* cur, const char* nxt, int kt) {
        mma(xa, xb); frags(cur, 1, ya, yb); interleave();
        mma(ya, yb); frags(cur, 2, xa, xb); interleave();
        mma(xa, xb); frags(cur, 3, ya, yb); interleave();
        landed();                                   // slab kt + 1 is in LDS, `cur` is free
        if (kt + 2 < kt_n) fetch((kt + 2) * TK, cur);
        else if (gtile != nullptr && (kt + 2 == kt_n || kt_n == 1)) fetch_gate(gtile, cur);
        mma(ya, yb);
        frags(nxt, 0, xa, xb);       // after the last step: stale, unused
        interleave();
    };

    // PERSIST: one pass per tile of the workgroup; otherwise one pass
    bool primed = false;    // the next tile's sources and first slab are requested
    for (bool first = true;; first = false) {
        if constexpr (PERSIST) asm volatile("" : "+v"(tid));
        if (!first) {
            tile += gridDim.x;
            if (tile >= total) return;
            place(tile, mt, nt);
            m0 = (int64_t)mt * TM;
            n0 = nt * TNC;
        }
        if (primed) {
            primed = false;               // sources and slab 0 already requested
        } else {
            sources(m0, n0);
            if (!first) __syncthreads();  // the previous tile's epilogue is done with buffer 0
            fetch(0, buf0);
        }
        gtile = gate_tile(mt, nt);
        compact = PERSIST || (gtile != nullptr && gate_compact(p.keep));   // PERSIST: launched for compact tiles
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
        landed();
        if (kt_n > 1) fetch(TK, buf1);
        frags(buf0, 0, xa, xb);
        int kt = 0;
        for (; kt + 2 <= kt_n; kt += 2) {
            step(buf0, buf1, kt);
            step(buf1, buf0, kt + 1);
        }
        if (kt < kt_n) step(buf0, buf1, kt);       // odd count: the last slab is in buf0
        // the gate tile went into the second-to-last step's `cur`, which is the
        // last step's `nxt` (one step only: that step's `cur`, buf0)
        char* gbuf = kt_n == 1 ? buf0 : ((kt_n & 1) ? buf1 : buf0);

        // epilogue: lane holds column (lane & 31) and rows (v & 3) + 8 (v >> 2)
        // + 4 (lane >> 5); for gate/up, tile j < NJ / 2 holds u and tile
        // j + NJ / 2 holds v of channels n0 + wn GB + 32 j + (lane & 31)
        if constexpr (EPI == EPI_AMP) {
            // Dense-4x baseline: a = SiLU(u) v of the 256 x 128 block goes to LDS
            // (both freed slab buffers) as 512 bank-rows q = 2 row + (col >> 6)
            // of 256 bytes, 16-byte chunks swizzled by q; thread q then ranks
            // |a| of its bank-row and writes the mask word, the masked bf16 h
            // and, when asked for, the amplitudes
            landed();
            auto arow = [&](int q) { return (q < 256 ? buf0 : buf1) + (q & 255) * 256; };
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int rt = wm * 128 + i * 32 + (v & 3) + 8 * (v >> 2) + 4 * hk;
#pragma unroll
                    for (int j = 0; j < NJ / 2; ++j) {
                        const int col = wn * GB + j * 32 + r32;
                        const int q = 2 * rt + (col >> 6), c64 = col & 63;
                        const float u = acc[i][j][v], vv = acc[i][j + NJ / 2][v];
                        *reinterpret_cast<float*>(arow(q) + (((c64 >> 2) ^ (q & 15)) << 4) + (c64 & 3) * 4) =
                            sigmoidf_dev(u) * u * vv;
                    }
                }
            __syncthreads();
            const int q = tid;                               // NT = 512 bank-rows
            const int64_t t = m0 + (q >> 1);
            const int j0 = n0 + (q & 1) * kBank;
            const char* r = arow(q);
            auto ld = [&](int c) { return *reinterpret_cast<const float4*>(r + ((c ^ (q & 15)) << 4)); };
            const uint64_t sel = lane_select64(
                [&](int c) {
                    const float4 f = ld(c);
                    return make_float4(fabsf(f.x), fabsf(f.y), fabsf(f.z), fabsf(f.w));
                },
                p.keep);
            if (t >= p.M || j0 >= p.N) return;
            p.mask_w[t * (p.N / kBank) + j0 / kBank] = sel;
            if (p.Cf != nullptr) {
#pragma unroll
                for (int c = 0; c < 16; ++c) reinterpret_cast<float4*>(p.Cf + t * p.N + j0)[c] = ld(c);
            }
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 v0 = ld(2 * c), v1 = ld(2 * c + 1);
                const float av[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
                uint32_t hw[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int ch = 8 * c + 2 * e;
                    const uint32_t lo = ((sel >> ch) & 1ull) ? f32_to_bf16(av[2 * e]) : 0u;
                    const uint32_t hi = ((sel >> (ch + 1)) & 1ull) ? f32_to_bf16(av[2 * e + 1]) : 0u;
                    hw[e] = lo | (hi << 16);
                }
                *reinterpret_cast<uint4*>(p.Cb + t * p.N + j0 + 8 * c) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            }
            return;
        }
        if constexpr (EPI == EPI_GATEUP) {
            if (compact) {
                // the compact gate tile, expanded into the full layout in the
                // other slab buffer. With two or more K steps the tile landed
                // before the last step's barrier, after which no wave reads that
                // buffer; a single step fetched it after its barrier.
                if (kt_n == 1) landed();
                char* const ebuf = gbuf == buf0 ? buf1 : buf0;
                expand(gbuf, ebuf);
                gbuf = ebuf;
            }
            if (PERSIST || gtile != nullptr || p.dense) {
                // H = select(kept, s u v, 0) with the gate values of the LDS
                // copy of the gate tile (at hb), written over them in place
                // (each element is read and written by one lane); the bf16
                // tile then leaves in 16-byte stores
                auto finish = [&](char* hb) {
                    // LDS addresses: element (row, channel) of the tile is at
                    // hb + 256 row + 2 channel, and the thread's 16-byte chunk
                    // i of the H rows at hb + 256 (ch >> 4) + 16 (ch & 15),
                    // ch = tid + NT i. The persistent kernel forms them as hb
                    // + an opaque per-lane base + a constant: a short address
                    // chain, along which the compiler still sees which LDS
                    // array an access names (a chain of one GEP per addend
                    // hides it, and each read then waits for every load in
                    // flight into LDS, the next tile's first slab included)
                    int eb = (wm * 128 + 4 * hk) * 256 + 2 * (wn * GB + r32);
                    int sb = (tid >> 4) * 256 + (tid & 15) * 16;
                    if constexpr (PERSIST) asm volatile("" : "+v"(eb), "+v"(sb));
                    auto elem = [&](int i, int j, int v) -> uint16_t* {
                        const int r = i * 32 + (v & 3) + 8 * (v >> 2);   // row within the wave's block
                        if constexpr (PERSIST) return reinterpret_cast<uint16_t*>(hb + eb + (r * 256 + 64 * j));
                        return reinterpret_cast<uint16_t*>(hb + (wm * 128 + r + 4 * hk) * 256) + wn * GB + j * 32 +
                               r32;
                    };
                    auto chunk = [&](int i) -> const uint4* {
                        if constexpr (PERSIST) return reinterpret_cast<const uint4*>(hb + sb + i * (NT / 16) * 256);
                        const int ch = tid + i * NT;
                        return reinterpret_cast<const uint4*>(hb + (ch >> 4) * 256 + (ch & 15) * 16);
                    };
                    // one copy of the element loop per gate, and the drop as a
                    // select of the value (bf16(0) = 0): no branch per element
                    auto compute = [&](auto silu) {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
#pragma unroll
                            for (int j = 0; j < NJ / 2; ++j) {
                                // 16 reads in flight, then the 16 writes
                                uint16_t* e[16];
                                uint16_t g[16];
#pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    e[v] = elem(i, j, v);
                                    g[v] = *e[v];
                                }
#pragma unroll
                                for (int v = 0; v < 16; ++v) {
                                    const float u = acc[i][j][v], vv = acc[i][j + NJ / 2][v];
                                    float sg;
                                    if constexpr (decltype(silu)::value) sg = sigmoidf_dev(u);
                                    else sg = (float)__builtin_bit_cast(_Float16, g[v]);
                                    const bool kept = p.dense || g[v] != kGateDropped;   // dense: no gate tile
                                    *e[v] = f32_to_bf16(kept ? sg * u * vv : 0.f);
                                }
                            }
                    };
                    if (p.gate == kGateSilu) compute(BoolTag<true>{});
                    else compute(BoolTag<false>{});
                    // this wave's LDS writes done, then the barrier; unlike
                    // __syncthreads it does not wait for the loads still in
                    // flight into the other buffer (the clobber keeps the
                    // compiler from moving memory accesses across it)
                    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
                    for (int i = 0; i < TM * 16 / NT; ++i) {
                        const int ch = tid + i * NT, row = ch >> 4, c16 = ch & 15;
                        const int64_t m = m0 + row;
                        const uint4 val = *chunk(i);
                        if (m < p.M) *reinterpret_cast<uint4*>(p.Cb + m * p.N + n0 + c16 * 8) = val;
                    }
                };
                landed();
                if constexpr (PERSIST) {
                    // Launched for compact gate tiles and an even count of K
                    // steps (or one) only, so the tile expanded out of buf0
                    // into buf1, and buf0 is free: the next tile's first slab
                    // goes there now. The epilogue's LDS reads name buf1
                    // itself, so that they need not wait for those loads.
                    primed = tile + gridDim.x < total;
                    if (primed) {
                        int nm, nn;
                        place(tile + gridDim.x, nm, nn);
                        sources((int64_t)nm * TM, nn * TNC);
                        fetch(0, buf0);
                    }
                    finish(buf1);
                    continue;
                }
                finish(gbuf);
                return;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < (GU ? NJ / 2 : NJ); ++j) {
                const int n = GU ? n0 + wn * GB + j * 32 + r32 : n0 + wn * WNC + j * 32 + r32;
                if (n >= p.N) continue;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t m = m0 + wm * 128 + i * 32 + (v & 3) + 8 * (v >> 2) + 4 * hk;
                    if (m >= p.M) continue;
                    const int64_t o = m * p.N + n;
                    if constexpr (EPI == EPI_BF16) {
                        p.Cb[o] = f32_to_bf16(acc[i][j][v]);
                    } else if constexpr (EPI == EPI_F32_BIAS) {
                        p.Cf[o] = acc[i][j][v] + (p.bias ? p.bias[n] : 0.f);
                    } else if constexpr (EPI == EPI_F32_ACC) {
                        p.Cf[o] += acc[i][j][v];
                    } else if constexpr (EPI == EPI_UV) {
                        p.Cb[o] = f32_to_bf16(acc[i][j][v]);
                        p.Cb2[o] = f32_to_bf16(acc[i][j + NJ / 2][v]);
                    } else {
                        const float u = acc[i][j][v];
                        const float vv = acc[i][j + NJ / 2][v];
                        const bool keep = (p.mask[m * (p.N / kBank) + (n >> 6)] >> (n & 63)) & 1ull;
                        const float sg = p.gate ? sigmoidf_dev(u) : sigmoidf_dev(p.P[o]);
                        p.Cb[o] = keep ? f32_to_bf16(sg * u * vv) : (uint16_t)0;
                    }
                }
            }
        if constexpr (!PERSIST) return;
    }
}

#ifndef SFFN_GEMM256_WN
#define SFFN_GEMM256_WN 4        // waves along N in the 256 x 256 tiles (2: 4 waves, 4: 8 waves)
#endif

template <int EPI, bool KMAJOR = false>
static void gemm256(const GemmParams& p, hipStream_t s, void* const* events, int stage) {
    constexpr int WN = SFFN_GEMM256_WN;
    const int m_tiles = (int)((p.M + TM - 1) / TM);
    constexpr int TNC = (EPI == EPI_GATEUP || EPI == EPI_AMP || EPI == EPI_UV) ? TN / 2 : TN;
    const int n_tiles = (p.N + TNC - 1) / TNC;
    if constexpr (EPI == EPI_GATEUP) {
        // compact gate tiles and more tiles than compute units: persistent
        // workgroups, one per compute unit (each holds 128 KB of LDS)
        const int n_cu = compute_units();
        const int kt_n = p.K / TK;
        if (p.G != nullptr && gate_compact(p.keep) && (kt_n % 2 == 0 || kt_n == 1) && m_tiles * n_tiles > n_cu &&
            n_cu % 8 == 0) {
            xlaunch(events, stage, k_gemm256<EPI, WN, KMAJOR, true>, dim3((unsigned)n_cu), dim3(128 * WN), 0, s,
                    p, m_tiles, n_tiles);
            return;
        }
    }
    xlaunch(events, stage, k_gemm256<EPI, WN, KMAJOR>, dim3((unsigned)(m_tiles * n_tiles)), dim3(128 * WN), 0, s,
            p, m_tiles, n_tiles);
}

template <int EPI>
static void gemm(const GemmParams& p, hipStream_t s, void* const* events, int stage) {
    const int64_t mt = (p.M + BM - 1) / BM;
    const int64_t nt = (p.N + BN - 1) / BN;
    if (p.K % TKD == 0)
        xlaunch(events, stage, k_gemm<EPI, true>, dim3((unsigned)(mt * nt)), dim3(256), 0, s, p);
    else
        xlaunch(events, stage, k_gemm<EPI, false>, dim3((unsigned)(mt * nt)), dim3(256), 0, s, p);
}

// Y = bf16(H W_d^T) with W_d^T given K-major ([d_i][d]; K = d_i is a
// multiple of 64 for every layer): 256-wide tiles for T >= 256, else 128-wide
static void down_gemm(const uint16_t* h, const uint16_t* WdT, int64_t T, int d, int d_i, uint16_t* y,
                      hipStream_t s, void* const* events, int stage) {
    GemmParams g{};
    g.A = h; g.B0 = WdT; g.M = T; g.N = d; g.K = d_i; g.Cb = y;
    if (T >= 256) {
        gemm256<EPI_BF16, true>(g, s, events, stage);
    } else {
        const int64_t mt = (T + BM - 1) / BM, nt = (d + BN - 1) / BN;
        xlaunch(events, stage, k_gemm<EPI_BF16, true, true>, dim3((unsigned)(mt * nt)), dim3(256), 0, s, g);
    }
}

// Sum of K-split partials in a fixed order, rounded to bf16.
__global__ __launch_bounds__(256) void k_sum_splits_bf16(const float* __restrict__ partial,
                                                         uint16_t* __restrict__ C, int splits,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float acc = sum_splits_in_order(partial + i, splits, n);
    C[i] = f32_to_bf16(acc);
}

bool mfma_fused_topk(int64_t T, int d, int d_i, int rank) {
    return T >= 256 && d % 64 == 0 && d_i % kGateTileCols == 0 && rank % BK == 0;
}

int z_splits(int64_t T, int d) {
    // split K of predictor layer 1 when the 128 x 128 tiles alone would leave
    // most compute units idle
    return (T >= 256 && d % (4 * BK) == 0) ? 4 : 1;
}

hipError_t launch_mfma_forward(const MfmaArgs& a, hipStream_t s) {
    // the 256-wide tiles need K to be a multiple of 64 and enough rows to fill them
    const bool big = a.T >= 256 && a.d % 64 == 0 && a.d_i % 64 == 0;
    const bool tiles = big && a.gate_tiles != nullptr && a.d_i % kGateTileCols == 0;
    GemmParams g{};
    if (!a.need_pred) {
        // every channel kept with the silu gate and no logits asked for: no
        // predictor and no top-k. The 256-wide gate/up epilogue keeps every
        // channel by itself when whole 128-column gate tiles cover d_i (its
        // in-place path stores all 128 columns of a tile); otherwise the
        // general epilogue reads the all-ones mask and skips columns >= d_i.
        // The mask is written when asked for or read.
        skip_range(a.events, 0, 3, s);
        const bool dense_tiles = big && a.d_i % kGateTileCols == 0;
        if (a.mask_requested || !dense_tiles) {
            const hipError_t e = launch_fill_mask(a.mask, a.T * (a.d_i / kBank), s);
            if (e != hipSuccess) return e;
        }
        g = GemmParams{};
        g.A = a.x; g.B0 = a.W_g; g.B1 = a.W_u; g.M = a.T; g.N = a.d_i; g.K = a.d; g.Cb = a.h;
        g.mask = a.mask; g.gate = a.gate; g.dense = dense_tiles ? 1 : 0;
        if (big) gemm256<EPI_GATEUP>(g, s, a.events, 3);
        else gemm<EPI_GATEUP>(g, s, a.events, 3);
        down_gemm(a.h, a.W_dT, a.T, a.d, a.d_i, a.y, s, a.events, 4);
        return hipGetLastError();
    }
    // Z = bf16(X A^T)
    g.A = a.x; g.B0 = a.A; g.M = a.T; g.N = a.rank; g.K = a.d; g.Cb = a.z;
    const int zs = z_splits(a.T, a.d);
    if (zs > 1 && a.z_partial != nullptr) {
        g.Cf = a.z_partial; g.kn = a.d / zs;
        const int64_t tiles = ((a.T + BM - 1) / BM) * ((a.rank + BN - 1) / BN);
        hipEvent_t e0 = a.events ? static_cast<hipEvent_t>(a.events[0]) : nullptr;
        hipEvent_t e1 = a.events ? static_cast<hipEvent_t>(a.events[1]) : nullptr;
        if (g.kn % TKD == 0)
            hipExtLaunchKernelGGL(k_gemm<EPI_PARTIAL, true>, dim3((unsigned)tiles, (unsigned)zs), dim3(256), 0,
                                  s, e0, nullptr, 0u, g);
        else
            hipExtLaunchKernelGGL(k_gemm<EPI_PARTIAL, false>, dim3((unsigned)tiles, (unsigned)zs), dim3(256), 0,
                                  s, e0, nullptr, 0u, g);
        const int64_t n = a.T * (int64_t)a.rank;
        hipExtLaunchKernelGGL(k_sum_splits_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                              nullptr, e1, 0u, (const float*)a.z_partial, a.z, zs, n);
    } else {
        gemm<EPI_BF16>(g, s, a.events, 0);
    }
    // P = Z B^T + bias
    g = GemmParams{};
    if (tiles && mfma_fused_topk(a.T, a.d, a.d_i, a.rank)) {
        // P, bank top-k and gate tiles in one kernel; the logits reach HBM
        // only when the caller asked for them
        g.A = a.z; g.B0 = a.B; g.M = a.T; g.N = a.d_i; g.K = a.rank; g.bias = a.bias;
        g.Cf = a.logits_requested ? a.logits : nullptr;
        g.mask_w = a.mask; g.gate_w = a.gate_tiles; g.keep = a.keep; g.gate = a.gate;
        gemm<EPI_TOPK>(g, s, a.events, 1);
        if (a.events) {
            (void)hipEventRecord(static_cast<hipEvent_t>(a.events[4]), s);
            (void)hipEventRecord(static_cast<hipEvent_t>(a.events[5]), s);
        }
    } else {
        g.A = a.z; g.B0 = a.B; g.M = a.T; g.N = a.d_i; g.K = a.rank; g.Cf = a.logits; g.bias = a.bias;
        gemm<EPI_F32_BIAS>(g, s, a.events, 1);
        // (gate tiles imply the fused branch above, so none are written here)
        hipError_t e = launch_bank_topk(a.logits, a.T, a.d_i, a.keep, a.mask, nullptr, s, a.events, 2);
        if (e != hipSuccess) return e;
    }
    // H = select(m, s u v, 0)
    g = GemmParams{};
    g.A = a.x; g.B0 = a.W_g; g.B1 = a.W_u; g.M = a.T; g.N = a.d_i; g.K = a.d; g.Cb = a.h;
    g.P = a.logits; g.mask = a.mask; g.gate = a.gate; g.keep = a.keep; g.G = tiles ? a.gate_tiles : nullptr;
    if (big) gemm256<EPI_GATEUP>(g, s, a.events, 3);
    else gemm<EPI_GATEUP>(g, s, a.events, 3);
    // Y = bf16(H W_d^T)
    down_gemm(a.h, a.W_dT, a.T, a.d, a.d_i, a.y, s, a.events, 4);
    return hipGetLastError();
}

// How launch_gemm_nt runs C = A B^T: 0 = the 256 x 256 kernel, which needs
// enough tiles to fill the chip; else the 128 x 128 kernel over that many K
// ranges (> 1: fp32 partials, then their sum in a fixed order). Thin GEMMs
// (one side the predictor rank) have only a few dozen 256 x 256 tiles.
static int nt_splits(int64_t M, int N, int K) {
    const int64_t t256 = ((M + TM - 1) / TM) * ((N + TN - 1) / TN);
    if (M >= TM && K % TK == 0 && t256 >= 192) return 0;
    const int64_t t128 = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int sp = 1;
    while (t128 * sp < 512 && K % (2 * sp * TKD) == 0 && K / (2 * sp) >= 256) sp *= 2;
    return sp;
}

size_t gemm_nt_partial_floats(int64_t M, int N, int K) {
    const int sp = nt_splits(M, N, K);
    return sp > 1 ? (size_t)sp * (size_t)M * (size_t)N : 0;
}

// C = (sum of the K-split partials in order) (+ bias[col]), stored as bf16,
// stored as fp32 or added to fp32
__global__ __launch_bounds__(256) void k_sum_splits_out(const float* __restrict__ partial, void* __restrict__ C,
                                                        int splits, int64_t n, int N, int mode,
                                                        const float* __restrict__ bias) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float acc = sum_splits_in_order(partial + i, splits, n);
    if (bias) acc += bias[i % N];
    if (mode == 2) static_cast<uint16_t*>(C)[i] = f32_to_bf16(acc);
    else if (mode == 1) static_cast<float*>(C)[i] += acc;
    else static_cast<float*>(C)[i] = acc;
}

hipError_t launch_gemm_nt(const uint16_t* A, const uint16_t* B, int64_t M, int N, int K, void* C,
                          GemmOut out, hipStream_t s, const float* bias, float* partial) {
    GemmParams g{};
    g.A = A; g.B0 = B; g.M = M; g.N = N; g.K = K; g.bias = bias;
    const int sp = nt_splits(M, N, K);
    if (sp > 1 && partial != nullptr) {
        g.Cf = partial; g.kn = K / sp;
        const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        if (g.kn % TKD == 0)
            hipExtLaunchKernelGGL(k_gemm<EPI_PARTIAL, true>, dim3((unsigned)tiles, (unsigned)sp), dim3(256), 0, s,
                                  nullptr, nullptr, 0u, g);
        else
            hipExtLaunchKernelGGL(k_gemm<EPI_PARTIAL, false>, dim3((unsigned)tiles, (unsigned)sp), dim3(256), 0, s,
                                  nullptr, nullptr, 0u, g);
        const int64_t n = M * (int64_t)N;
        const int mode = out == GemmOut::BF16 ? 2 : out == GemmOut::F32_ACC ? 1 : 0;
        hipLaunchKernelGGL(k_sum_splits_out, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           (const float*)partial, C, sp, n, N, mode, bias);
        return hipGetLastError();
    }
    const bool big = sp == 0;
    if (out == GemmOut::BF16) {
        g.Cb = static_cast<uint16_t*>(C);
        if (big) gemm256<EPI_BF16>(g, s, nullptr, 0);
        else gemm<EPI_BF16>(g, s, nullptr, 0);
    } else if (out == GemmOut::F32) {
        g.Cf = static_cast<float*>(C);
        if (big) gemm256<EPI_F32_BIAS>(g, s, nullptr, 0);
        else gemm<EPI_F32_BIAS>(g, s, nullptr, 0);
    } else {
        g.Cf = static_cast<float*>(C);
        if (big) gemm256<EPI_F32_ACC>(g, s, nullptr, 0);
        else gemm<EPI_F32_ACC>(g, s, nullptr, 0);
    }
    return hipGetLastError();
}

hipError_t launch_uv_gemm(const uint16_t* x, const uint16_t* W_g, const uint16_t* W_u, int64_t T, int d_i,
                          int d, uint16_t* U, uint16_t* V, hipStream_t s) {
    GemmParams g{};
    g.A = x; g.B0 = W_g; g.B1 = W_u; g.M = T; g.N = d_i; g.K = d; g.Cb = U; g.Cb2 = V;
    if (T >= 256 && d % TK == 0) gemm256<EPI_UV>(g, s, nullptr, 0);
    else gemm<EPI_UV>(g, s, nullptr, 0);
    return hipGetLastError();
}

hipError_t launch_amp_mfma(const MfmaArgs& a, hipStream_t s) {
    GemmParams g{};
    g.A = a.x; g.B0 = a.W_g; g.B1 = a.W_u; g.M = a.T; g.N = a.d_i; g.K = a.d; g.Cb = a.h;
    g.mask_w = a.mask; g.keep = a.keep; g.Cf = a.logits_requested ? a.logits : nullptr;
    gemm256<EPI_AMP>(g, s, a.events, 0);
    down_gemm(a.h, a.W_dT, a.T, a.d, a.d_i, a.y, s, a.events, 1);
    skip_stages(a.events, 2, s);
    return hipGetLastError();
}

}  // namespace sffn
