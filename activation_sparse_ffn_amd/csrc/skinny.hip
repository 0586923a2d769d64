// Skinny MFMA path of the sparse FFN forward: 4 < T <= 64 tokens (batched
// decode). The weight matrices are streamed once from HBM; the token
// operand (at most 64 rows) stays in the L2.
//
// C[M, N] = A[M, K] B[N, K]^T with M <= 64: a workgroup owns 32 columns of C
// (32 weight rows) and a K range; its four waves take interleaved 64-wide K
// steps. A step's operand tiles (32 rows x 128 bytes each) are fetched with
// eight lanes per row, so every load instruction covers eight whole 128-byte
// lines, then pass through a wave-private LDS tile (16-byte chunks
// XOR-swizzled by row pairs) into the v_mfma_f32_32x32x16_bf16 fragment layout:
// lane (r, h) of sub-step i takes row r, k = 32 h + 8 i .. + 8, for A and B
// alike (the MFMA only needs both operands to agree on which k each lane
// carries). The predictor GEMMs' loads run U steps ahead of the matrix cores
// (gate/up: one fetch per wave at a time). The four waves meet
// in LDS, where each wave finishes a quarter of the accumulator elements and
// runs the epilogue (or writes an fp32 partial when K is also split across
// workgroups).
//
// Same steps and epilogues as the dense-masked path ("Continual LLM
// Upcycling", gist.science technical summary, Methodologie > 1. Architectuur
// and 3. Hardware Implicaties):
//   Z = bf16(X A^T)  P = Z B^T + bias  mask = top-k(P)
//   H = select(m, s u v, 0) with U = X W_g^T, V = X W_u^T   Y = bf16(H W_d^T) (K-major W_d^T)
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

enum { SK_BF16 = 0, SK_F32_BIAS = 1, SK_GATEUP = 2, SK_PARTIAL = 3, SK_AMP = 4 };

struct SkinnyParams {
    const uint16_t* A;     // [M, K]
    const uint16_t* B0;    // [N, K]
    const uint16_t* B1;    // [N, K] (gate/up: W_u) or null
    int M, N, K;
    int k_split;           // K range per workgroup (multiple of 64)
    float* partial;        // [K / k_split, M, N] for SK_PARTIAL
    uint16_t* Cb;          // bf16 [M, N]
    float* Cf;             // fp32 [M, N]
    const float* bias;     // [N] or null
    const float* P;        // gate/up: logits [M, N]
    const uint64_t* mask;  // gate/up: [M, N / 64]
    int gate;              // 0 predictor, 1 silu
    // [N / 64 (gate/up) or K / 64 (down)] or null: the or of the batch's mask
    // words (written by the top-k); weight rows of channels no token keeps
    // are not read (their products with the token operand are exact zeros)
    uint64_t* unionw;
};

// byte offset of 16-byte chunk c of row r in a 32 x 128-byte LDS tile; the
// XOR with (r >> 1) & 7 spreads 16 consecutive rows over all banks
__device__ __forceinline__ int tile_off(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

#ifndef SFFN_SKINNY_U
#define SFFN_SKINNY_U 1          // K steps per fetch
#endif

template <int EPI, int NB, int MT>
__global__ __launch_bounds__(256) void k_skinny(const SkinnyParams p) {
    constexpr int U = SFFN_SKINNY_U;
    constexpr int NT = NB + MT;                  // operand tiles per step
    constexpr int TILE = 32 * 128;               // bytes per operand tile
    constexpr int STAGE = 4 * NT * TILE;         // all waves' staging tiles
    constexpr int RED = 4 * NB * MT * 16 * kWave * 4;
    __shared__ __attribute__((aligned(16))) char smem[STAGE > RED ? STAGE : RED];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 32;
    const int kb0 = blockIdx.y * p.k_split;
    const int steps = p.k_split / 64;
    char* stage = smem + wv * NT * TILE;

    // global fetch pattern: instruction q, lane l -> row 8 q + l / 8, chunk l % 8
    const int fr = lane >> 3, fc = lane & 7;
    const uint16_t* src[NT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
        src[b] = (b == 0 ? p.B0 : p.B1) + (size_t)(n0 + fr) * p.K + kb0 + 8 * fc;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)   // rows of A at or beyond M are zero-filled, never read
        src[NB + mt] = p.A + (size_t)(mt * 32 + fr) * p.K + kb0 + 8 * fc;
    const size_t rstride8 = (size_t)8 * p.K;      // 8 rows further down

    f32x16 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[b][mt][v] = 0.f;

    const int r = lane & 31, h = lane >> 5;
    // gate/up: this lane's weight rows 8 q + fr of the tile, kept by some token?
    uint32_t live = 0xfu;
    if constexpr (EPI == SK_GATEUP) {
        if (p.unionw != nullptr) {
            const uint64_t uw = p.unionw[n0 >> 6] >> (n0 & 63);
            live = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) live |= (uint32_t)((uw >> (8 * q + fr)) & 1ull) << q;
        }
    }
    // Workgroups start their K walk at different steps: rows of one weight
    // matrix sit a power-of-two stride apart, and if every workgroup read the
    // same K offset at the same time the requests would crowd a few HBM
    // channels. Step st of this workgroup is K step (st + rot) mod steps.
    const int rot = (int)((blockIdx.x * 37u) % (unsigned)steps);
    auto kstep = [&](int st) { const int k = st + rot; return k >= steps ? k - steps : k; };
    // U consecutive steps of this wave (st, st + 4, ...) per fetch
    auto fetch = [&](uint4 (&w)[U][NT][4], int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int s_ = st + 4 * u;
            if (s_ < steps) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const uint16_t* at = src[t] + q * rstride8 + 64 * kstep(s_);
                        if (t < NB) {
                            // weight rows: read once per call, streamed past the caches
                            if ((live >> q) & 1u) {
                                Raw<uint16_t> rw;
                                rw.load_stream(at);
                                w[u][t][q] = rw.w;
                            } else {
                                w[u][t][q] = make_uint4(0, 0, 0, 0);
                            }
                        } else {
                            // token rows: re-read by every workgroup from the L2
                            const bool valid = (t - NB) * 32 + 8 * q + fr < p.M;
                            w[u][t][q] = valid ? *reinterpret_cast<const uint4*>(at) : make_uint4(0, 0, 0, 0);
                        }
                    }
            }
        }
    };
    auto consume = [&](const uint4 (&w)[U][NT][4], int st) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (st + 4 * u < steps) {
#pragma unroll
                for (int t = 0; t < NT; ++t)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        *reinterpret_cast<uint4*>(stage + t * TILE + tile_off(8 * q + fr, fc)) = w[u][t][q];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    bf16x8 fb[NB], fa[MT];
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        fb[b] = *reinterpret_cast<const bf16x8*>(stage + b * TILE + tile_off(r, 4 * h + i));
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        fa[mt] = *reinterpret_cast<const bf16x8*>(stage + (NB + mt) * TILE + tile_off(r, 4 * h + i));
#pragma unroll
                    for (int b = 0; b < NB; ++b)
#pragma unroll
                        for (int mt = 0; mt < MT; ++mt)
                            acc[b][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[b], acc[b][mt], 0, 0, 0);
                }
            }
        }
    };
    // One weight tile per step (predictor GEMMs): two register buffers, so
    // the next U steps are in flight while the current U steps go through
    // LDS into the matrix cores. Two weight tiles per step (gate/up): one
    // buffer; the other waves of the compute unit keep the memory system
    // busy, and with two fetches in flight per wave (~44 MB requested across
    // the chip) the requests congest it: the 32-token gate/up took 41.3 us
    // double-buffered and 38.5 us single-buffered.
    constexpr int SPAN = 4 * U;                  // step distance covered by one fetch
    if constexpr (NB == 1) {
        uint4 w0[U][NT][4], w1[U][NT][4];
        fetch(w0, wv);
        for (int st = wv; st < steps; st += 2 * SPAN) {
            fetch(w1, st + SPAN);
            consume(w0, st);
            fetch(w0, st + 2 * SPAN);
            consume(w1, st + SPAN);
        }
    } else {
        for (int st = wv; st < steps; st += SPAN) {
            uint4 w0[U][NT][4];
            fetch(w0, st);
            consume(w0, st);
        }
    }

    // the four waves' partial sums meet in LDS; wave w finishes elements
    // v = 4 w .. 4 w + 3 of every accumulator tile
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);     // [4][NB * MT * 16][64]
    auto R = [&](int wave, int e, int ln) -> float& { return red[((size_t)wave * NB * MT * 16 + e) * kWave + ln]; };
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) R(wv, (b * MT + mt) * 16 + v, lane) = acc[b][mt][v];
    __syncthreads();

    const int n = n0 + r;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = 4 * wv + q;
            const int m = mt * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
            float val[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const int e = (b * MT + mt) * 16 + v;
                val[b] = (R(0, e, lane) + R(1, e, lane)) + (R(2, e, lane) + R(3, e, lane));
            }
            if (m >= p.M) continue;
            const size_t o = (size_t)m * p.N + n;
            if constexpr (EPI == SK_PARTIAL) {
                p.partial[(size_t)blockIdx.y * p.M * p.N + o] = val[0];
            } else if constexpr (EPI == SK_BF16) {
                p.Cb[o] = f32_to_bf16(val[0]);
            } else if constexpr (EPI == SK_F32_BIAS) {
                p.Cf[o] = val[0] + (p.bias ? p.bias[n] : 0.f);
            } else if constexpr (EPI == SK_AMP) {
                // Dense-4x baseline: the amplitude SiLU(u) v of every channel, fp32
                const float u = val[0], vv = val[NB - 1];
                p.Cf[o] = sigmoidf_dev(u) * u * vv;
            } else {
                const float u = val[0], vv = val[NB - 1];
                const bool keep = (p.mask[(size_t)m * (p.N / kBank) + (n >> 6)] >> (n & 63)) & 1ull;
                const float sg = p.gate ? sigmoidf_dev(u) : sigmoidf_dev(p.P[o]);
                p.Cb[o] = keep ? f32_to_bf16(sg * u * vv) : (uint16_t)0;
            }
        }
}

// Predictor layer 2 with the bank top-k in its epilogue: one workgroup of
// eight waves per bank computes the bank's M x 64 logits (+ bias) -- the
// waves take the rank's 64-wide K steps in turn, each step fetched like
// k_skinny's (two 32-row weight tiles and the token tiles) -- and after the
// waves' partial sums meet in LDS, one wave ranks them, lane t selecting
// token t's kept channels (lane_select64): the mask words, the or of the
// batch's mask words (the union) and the fp32 logits, which the gate/up
// epilogue reads for sigmoid(p).
template <int MT>
__global__ __launch_bounds__(512) void k_skinny_topk(const SkinnyParams p, int keep, uint64_t* __restrict__ mask) {
    constexpr int NW = 8, NB = 2, NT = NB + MT;
    constexpr int TILE = 32 * 128;                          // bytes per operand tile
    constexpr int STAGE = NW * NT * TILE;                   // every wave's staging tiles
    constexpr int RED = NW * NB * MT * 16 * kWave * 4;      // the waves' partial sums
    constexpr int PITCH = kBank * 4 + 16;                   // bytes per token row of the logit tile
    constexpr int LGT = 32 * MT * PITCH;
    __shared__ __attribute__((aligned(16))) char smem[STAGE > RED + LGT ? STAGE : RED + LGT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int bank = blockIdx.x, n0 = bank * kBank;
    const int steps = p.K / 64;
    char* stage = smem + wv * NT * TILE;

    // global fetch pattern: instruction q, lane l -> row 8 q + l / 8, chunk l % 8
    const int fr = lane >> 3, fc = lane & 7;
    const uint16_t* src[NT];
#pragma unroll
    for (int b = 0; b < NB; ++b) src[b] = p.B0 + (size_t)(n0 + 32 * b + fr) * p.K + 8 * fc;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) src[NB + mt] = p.A + (size_t)(mt * 32 + fr) * p.K + 8 * fc;
    const size_t rstride8 = (size_t)8 * p.K;

    f32x16 acc[NB][MT];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[b][mt][v] = 0.f;
    const int r = lane & 31, h = lane >> 5;
    for (int st = wv; st < steps; st += NW) {
        uint4 w[NT][4];
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint16_t* at = src[t] + q * rstride8 + 64 * st;
                if (t < NB) {
                    w[t][q] = *reinterpret_cast<const uint4*>(at);
                } else {
                    const bool valid = (t - NB) * 32 + 8 * q + fr < p.M;   // rows past M: zero
                    w[t][q] = valid ? *reinterpret_cast<const uint4*>(at) : make_uint4(0, 0, 0, 0);
                }
            }
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4*>(stage + t * TILE + tile_off(8 * q + fr, fc)) = w[t][q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x8 fb[NB], fa[MT];
#pragma unroll
            for (int b = 0; b < NB; ++b)
                fb[b] = *reinterpret_cast<const bf16x8*>(stage + b * TILE + tile_off(r, 4 * h + i));
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                fa[mt] = *reinterpret_cast<const bf16x8*>(stage + (NB + mt) * TILE + tile_off(r, 4 * h + i));
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[b][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[b], acc[b][mt], 0, 0, 0);
        }
    }

    // the waves' partial sums meet in LDS; wave w finishes elements
    // v = 2 w, 2 w + 1 of every accumulator tile into the logit tile
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);          // [NW][NB * MT * 16][64]
    char* const lg = smem + RED;                          // [32 MT][PITCH]
    auto R = [&](int wave, int e, int ln) -> float& { return red[((size_t)wave * NB * MT * 16 + e) * kWave + ln]; };
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) R(wv, (b * MT + mt) * 16 + v, lane) = acc[b][mt][v];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int v = 2 * wv + q;
                const int m = mt * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
                const int e = (b * MT + mt) * 16 + v;
                float val = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NW; ++w2) val += R(w2, e, lane);
                const int c = 32 * b + r;
                val += p.bias ? p.bias[n0 + c] : 0.f;
                *reinterpret_cast<float*>(lg + m * PITCH + 4 * c) = val;
                if (m < p.M) p.Cf[(size_t)m * p.N + n0 + c] = val;
            }
    __syncthreads();
    if (wv != 0) return;
    // lane t ranks token t (lanes past M repeat the last token and add
    // nothing to the union)
    const int t = lane < p.M ? lane : p.M - 1;
    const char* row = lg + t * PITCH;
    const uint64_t sel =
        lane_select64([&](int c) { return *reinterpret_cast<const float4*>(row + 16 * c); }, keep);
    if (lane < p.M) mask[(size_t)lane * (p.N / kBank) + bank] = sel;
    uint32_t lo = lane < p.M ? (uint32_t)sel : 0u, hi = lane < p.M ? (uint32_t)(sel >> 32) : 0u;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo |= (uint32_t)__shfl_xor((int)lo, o, kWave);
        hi |= (uint32_t)__shfl_xor((int)hi, o, kWave);
    }
    if (lane == 0 && p.unionw) p.unionw[bank] = ((uint64_t)hi << 32) | lo;
}

// The down projection Y = H W_d^T with W_d^T K-major ([K = d_i][N = d]): a
// workgroup owns 64 columns of Y (128-byte pieces of 64 consecutive K-rows
// per K step: whole cache lines) and a K range; its four waves take
// interleaved 64-wide K steps, U = 1 fetch ahead in registers. All
// workgroups walk their K range from its start, so the 64 workgroups of a K
// range read the 128-byte pieces of the same K-rows at about the same time
// (starting each at a different step, as k_skinny does for its row-major
// tiles, cost ~3% here). A step's
// weight tile (64 K-rows x 128 bytes, fetched eight lanes per row) goes to
// wave-private LDS with its chunks swizzled for the transposed fragment
// reads (kmajor_frag); the token tile (H, K-contiguous) as in k_skinny.
template <int EPI, int MT>
__global__ __launch_bounds__(256) void k_skinny_down(const SkinnyParams p) {
    static_assert(EPI == SK_BF16 || EPI == SK_PARTIAL, "plain or K-split output");
    constexpr int NC = 2;                           // 32-column output tiles per workgroup
    constexpr int WT = 64 * 128;                    // weight tile bytes
    constexpr int AT = 32 * 128;                    // token tile bytes
    constexpr int STAGE = 4 * (WT + MT * AT);
    constexpr int RED = 4 * NC * MT * 16 * kWave * 4;
    __shared__ __attribute__((aligned(16))) char smem[STAGE > RED ? STAGE : RED];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n0 = blockIdx.x * 64;
    const int kb0 = blockIdx.y * p.k_split;
    const int steps = p.k_split / 64;
    char* const wst = smem + wv * (WT + MT * AT);   // this wave's weight tile, then token tiles
    const int fr = lane >> 3, fc = lane & 7;
    // weight rows 8 q + fr of a step, chunk fc; token rows mt * 32 + 8 q + fr
    const uint16_t* wsrc = p.B0 + (size_t)(kb0 + fr) * p.N + n0 + 8 * fc;
    const uint16_t* asrc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) asrc[mt] = p.A + (size_t)(mt * 32 + fr) * p.K + kb0 + 8 * fc;
    const size_t wq = (size_t)8 * p.N, aq = (size_t)8 * p.K;

    f32x16 acc[NC][MT];
#pragma unroll
    for (int b = 0; b < NC; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[b][mt][v] = 0.f;
    const int r = lane & 31, h = lane >> 5;
    // union word of K step (bank) kb0 / 64 + lane, in lane `lane` (the K
    // range spans at most 64 banks when the union is given)
    const uint64_t uw_lane = (p.unionw != nullptr && lane < steps) ? p.unionw[kb0 / 64 + lane] : ~0ull;
    const uint32_t uw_lo = (uint32_t)uw_lane, uw_hi = (uint32_t)(uw_lane >> 32);
    struct Fetch { uint4 w[8]; uint4 a[MT][4]; };
    auto fetch = [&](Fetch& f, int st) {
        if (st >= steps) return;
        const int ks = st;
        // (readlane returns int: widen through uint32_t, not by sign extension)
        const uint64_t uw = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(uw_hi, ks) << 32) |
                            (uint32_t)__builtin_amdgcn_readlane(uw_lo, ks);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if ((uw >> (8 * q + fr)) & 1ull) {
                Raw<uint16_t> rw;
                rw.load_stream(wsrc + (size_t)64 * ks * p.N + q * wq);   // weights: read once per call
                f.w[q] = rw.w;
            } else {
                f.w[q] = make_uint4(0, 0, 0, 0);                        // no token keeps this channel
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const bool valid = mt * 32 + 8 * q + fr < p.M;
                f.a[mt][q] = valid ? *reinterpret_cast<const uint4*>(asrc[mt] + 64 * ks + q * aq)
                                   : make_uint4(0, 0, 0, 0);
            }
    };
    auto consume = [&](const Fetch& f, int st) {
        if (st >= steps) return;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int row = 8 * q + fr;
            *reinterpret_cast<uint4*>(wst + row * 128 + (kmajor_slot<128>(row, fc) << 4)) = f.w[q];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                *reinterpret_cast<uint4*>(wst + WT + mt * AT + tile_off(8 * q + fr, fc)) = f.a[mt][q];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            bf16x8 fb[NC], fa[MT];
#pragma unroll
            for (int b = 0; b < NC; ++b) fb[b] = kmajor_frag<128>(wst, 32 * b, i, lane);
            // lane (r, h) of sub-step i carries K = 16 i + 8 h .. + 8, the K that
            // the transposed weight fragment gives it
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
                fa[mt] = *reinterpret_cast<const bf16x8*>(wst + WT + mt * AT + tile_off(r, 2 * i + h));
#pragma unroll
            for (int b = 0; b < NC; ++b)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
                    acc[b][mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mt], fb[b], acc[b][mt], 0, 0, 0);
        }
    };
    Fetch f0, f1;
    fetch(f0, wv);
    for (int st = wv; st < steps; st += 8) {
        fetch(f1, st + 4);
        consume(f0, st);
        fetch(f0, st + 8);
        consume(f1, st + 4);
    }

    // the four waves' partial sums meet in LDS; wave w finishes elements
    // v = 4 w .. 4 w + 3 of every accumulator tile
    __syncthreads();
    float* red = reinterpret_cast<float*>(smem);     // [4][NC * MT * 16][64]
    auto R = [&](int wave, int e, int ln) -> float& { return red[((size_t)wave * NC * MT * 16 + e) * kWave + ln]; };
#pragma unroll
    for (int b = 0; b < NC; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 16; ++v) R(wv, (b * MT + mt) * 16 + v, lane) = acc[b][mt][v];
    __syncthreads();
#pragma unroll
    for (int b = 0; b < NC; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = 4 * wv + q;
                const int m = mt * 32 + (v & 3) + 8 * (v >> 2) + 4 * h;
                const int e = (b * MT + mt) * 16 + v;
                const float val = (R(0, e, lane) + R(1, e, lane)) + (R(2, e, lane) + R(3, e, lane));
                const int n = n0 + 32 * b + r;
                if (m >= p.M || n >= p.N) continue;
                const size_t o = (size_t)m * p.N + n;
                if constexpr (EPI == SK_PARTIAL) p.partial[(size_t)blockIdx.y * p.M * p.N + o] = val;
                else p.Cb[o] = f32_to_bf16(val);
            }
}

// Sum of the K-split partials in a fixed order, rounded to bf16.
__global__ __launch_bounds__(256) void k_skinny_sum_bf16(const float* __restrict__ partial,
                                                         uint16_t* __restrict__ C, int splits,
                                                         int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const float acc = sum_splits_in_order(partial + i, splits, n);
    C[i] = f32_to_bf16(acc);
}

template <int EPI, int NB>
static void skinny(SkinnyParams p, int splits, hipStream_t s, void* const* ev, int stage,
                   bool stop_here) {
    p.k_split = p.K / splits;
    const dim3 grid((unsigned)(p.N / 32), (unsigned)splits);
    // the stage's stop event goes on its last kernel
    hipEvent_t e0 = ev ? static_cast<hipEvent_t>(ev[2 * stage]) : nullptr;
    hipEvent_t e1 = (ev && stop_here) ? static_cast<hipEvent_t>(ev[2 * stage + 1]) : nullptr;
    if (p.M <= 32)
        hipExtLaunchKernelGGL(k_skinny<EPI, NB, 1>, grid, dim3(256), 0, s, e0, e1, 0u, p);
    else
        hipExtLaunchKernelGGL(k_skinny<EPI, NB, 2>, grid, dim3(256), 0, s, e0, e1, 0u, p);
}

static void sum_bf16(const float* partial, uint16_t* C, int splits, int64_t n, hipStream_t s,
                     void* const* ev, int stage) {
    hipEvent_t e1 = ev ? static_cast<hipEvent_t>(ev[2 * stage + 1]) : nullptr;
    hipExtLaunchKernelGGL(k_skinny_sum_bf16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                          nullptr, e1, 0u, partial, C, splits, n);
}

// Splits of K across workgroups so that a GEMM with few 32-column tiles still
// puts several hundred workgroups on the 256 compute units.
static int k_splits(int N, int K) {
    int s = 1;
    while ((N / 32) * s < 384 && K % (64 * 2 * s) == 0 && K / (2 * s) >= 256) s *= 2;
    return s;
}

// K splits of the K-major down projection (64 columns per workgroup)
static int down_splits(int N, int K) {
    int s = 1;
    while ((N / 64) * s < 384 && K % (64 * 2 * s) == 0 && K / (2 * s) >= 256) s *= 2;
    return s;
}

size_t skinny_partial_floats(int64_t T, int d, int rank, int d_i) {
    const size_t a = (size_t)k_splits(rank, d) * T * rank;
    const size_t b = (size_t)down_splits(d, d_i) * T * d;
    return a > b ? a : b;
}


// Y = bf16(H W_d^T), W_d^T K-major, as the stage `stage` of the events
static void skinny_down(const uint16_t* h, const uint16_t* WdT, int M, int d, int d_i, uint16_t* y, float* partial,
                        const uint64_t* unionw, hipStream_t s, void* const* ev, int stage) {
    SkinnyParams p{};
    p.A = h; p.B0 = WdT; p.M = M; p.N = d; p.K = d_i;
    const int sp = down_splits(d, d_i);
    p.k_split = d_i / sp;
    if (p.k_split / 64 <= kWave) p.unionw = const_cast<uint64_t*>(unionw);   // a lane per K step
    const dim3 grid((unsigned)(d / 64), (unsigned)sp);
    hipEvent_t e0 = ev ? static_cast<hipEvent_t>(ev[2 * stage]) : nullptr;
    hipEvent_t e1 = ev ? static_cast<hipEvent_t>(ev[2 * stage + 1]) : nullptr;
    if (sp == 1) {
        p.Cb = y;
        if (M <= 32) hipExtLaunchKernelGGL(k_skinny_down<SK_BF16, 1>, grid, dim3(256), 0, s, e0, e1, 0u, p);
        else hipExtLaunchKernelGGL(k_skinny_down<SK_BF16, 2>, grid, dim3(256), 0, s, e0, e1, 0u, p);
        return;
    }
    p.partial = partial;
    if (M <= 32) hipExtLaunchKernelGGL(k_skinny_down<SK_PARTIAL, 1>, grid, dim3(256), 0, s, e0, nullptr, 0u, p);
    else hipExtLaunchKernelGGL(k_skinny_down<SK_PARTIAL, 2>, grid, dim3(256), 0, s, e0, nullptr, 0u, p);
    sum_bf16(partial, y, sp, (int64_t)M * d, s, ev, stage);
}

hipError_t launch_skinny_forward(const MfmaArgs& a, float* partial, hipStream_t s) {
    const int M = (int)a.T;
    SkinnyParams p{};
    // the batch's union of kept channels per bank (every channel when the
    // dense fallback runs no top-k)
    uint64_t* const unionw = a.need_pred ? a.union_w : nullptr;
    if (!a.need_pred) {
        // every channel kept with the silu gate and no logits asked for: no
        // predictor and no top-k; the gate/up epilogue reads an all-ones mask
        skip_range(a.events, 0, 3, s);
        const hipError_t e = launch_fill_mask(a.mask, a.T * (a.d_i / kBank), s);
        if (e != hipSuccess) return e;
    } else {
        // Z = bf16(X A^T)
        {
            const int sp = k_splits(a.rank, a.d);
            p = SkinnyParams{};
            p.A = a.x; p.B0 = a.A; p.M = M; p.N = a.rank; p.K = a.d;
            if (sp == 1) {
                p.Cb = a.z;
                skinny<SK_BF16, 1>(p, 1, s, a.events, 0, true);
            } else {
                p.partial = partial;
                skinny<SK_PARTIAL, 1>(p, sp, s, a.events, 0, false);
                sum_bf16(partial, a.z, sp, (int64_t)M * a.rank, s, a.events, 0);
            }
        }
        // P = Z B^T + bias, the bank top-k (mask words and union) in the epilogue
        p = SkinnyParams{};
        p.A = a.z; p.B0 = a.B; p.M = M; p.N = a.d_i; p.K = a.rank; p.Cf = a.logits; p.bias = a.bias;
        p.unionw = unionw;
        const dim3 grid((unsigned)(a.d_i / kBank));
        if (M <= 32) xlaunch(a.events, 1, k_skinny_topk<1>, grid, dim3(512), 0, s, p, a.keep, a.mask);
        else xlaunch(a.events, 1, k_skinny_topk<2>, grid, dim3(512), 0, s, p, a.keep, a.mask);
        skip_range(a.events, 2, 3, s);
    }
    // H = select(m, s u v, 0)
    p = SkinnyParams{};
    p.A = a.x; p.B0 = a.W_g; p.B1 = a.W_u; p.M = M; p.N = a.d_i; p.K = a.d; p.Cb = a.h;
    p.P = a.logits; p.mask = a.mask; p.gate = a.gate; p.unionw = unionw;
    skinny<SK_GATEUP, 2>(p, 1, s, a.events, 3, true);
    // Y = bf16(H W_d^T)
    skinny_down(a.h, a.W_dT, M, a.d, a.d_i, a.y, partial, unionw, s, a.events, 4);
    return hipGetLastError();
}

hipError_t launch_amp_skinny(const MfmaArgs& a, float* partial, hipStream_t s) {
    const int M = (int)a.T;
    // amplitudes of every channel (fp32, into logits)
    SkinnyParams p{};
    p.A = a.x; p.B0 = a.W_g; p.B1 = a.W_u; p.M = M; p.N = a.d_i; p.K = a.d; p.Cf = a.logits;
    skinny<SK_AMP, 2>(p, 1, s, a.events, 0, true);
    // bank top-k of |a|: the mask and the masked bf16 h
    hipError_t e = launch_amp_mask(a.logits, a.T, a.d_i, a.keep, a.mask, a.h, s, a.events, 1);
    if (e != hipSuccess) return e;
    // Y = bf16(H W_d^T)
    skinny_down(a.h, a.W_dT, M, a.d, a.d_i, a.y, partial, nullptr, s, a.events, 2);
    skip_stages(a.events, 3, s);
    return hipGetLastError();
}

}  // namespace sffn
