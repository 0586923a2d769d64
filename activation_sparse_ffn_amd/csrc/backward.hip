// Backward pass of the predictor-gated sparse SwiGLU FFN ("Continual LLM
// Upcycling", gist.science technical summary, Methodologie > 1. Architectuur,
// Executie > Backward Pass): the hard top-k is crossed by a soft,
// sigmoid-like local gradient around the bank's selection threshold, so the
// loss reaches the predictor.
//
// Reading of the unstated form: the forward's hard mask m is differentiated
// as sigmoid((p - theta) / tau), theta the midpoint of the bank's smallest
// kept and largest dropped logit (its keep-th and (keep+1)-th largest; NaN
// counts lowest) held constant, tau the caller's temperature (1/tau = 0: no
// surrogate term). The mask gradient g_h * s * u * v is taken for every
// channel, so gate and up are evaluated densely. z's bf16 rounding passes
// gradients unchanged. A full bank (keep = 64) has no threshold.
//
// Steps, for T tokens (bf16 operands, fp32 accumulation, fp32 gradients):
//   z = bf16(x A^T), p = z B^T + bias          recomputed forward logits
//   g_h = g_y W_d                               every channel (W_d^T packed), bf16
//   U = x W_g^T, V = x W_u^T                    dense, bf16
//   k_bwd_tile: theta, h, g_u, g_v, g_p         one workgroup per (64 tokens, bank)
//   g_W_d = g_y^T h, g_W_g = g_u^T x, g_W_u = g_v^T x, g_B = g_p^T z,
//   g_z = g_p B, g_A = g_z^T x, g_bias = sum_t g_p,
//   g_x = g_z A + g_u W_g + g_v W_u
// Every product runs as C = A B^T on the MFMA GEMMs; operands that the
// tokens must contract over are token-transposed, zero-padded to a multiple
// of 64 tokens: h, g_u, g_v and g_p by k_bwd_tile itself, x, g_y, z and g_z
// by a transpose kernel.
#include <algorithm>

#include "common.hpp"
#include "launch.hpp"

namespace sffn {


// One workgroup per (block of 64 tokens, bank). Thread (token row tid / 8,
// chunk tid % 8) takes channels 8 c .. 8 c + 7 of one token per pass (two
// passes of 32 tokens), so every load and store moves 16 bytes (p 32 bytes);
// the bank's threshold comes from a reduction over the token's 8 lanes. g_u,
// g_v and g_p leave token-major (the A operands of g_x and g_z); h, g_u, g_v
// and g_p also leave transposed through LDS, [d_i][Tp] with zero columns past
// T (the operands of the weight gradients, which contract over tokens); g_p's
// column sums over the block, in a fixed order, go to colpart[block][d_i] for
// g_bias. In the LDS tiles ([channel][token], 128-byte rows) the 16-byte
// chunk of tokens 8 k .. 8 k + 7 of channel row ch sits at slot
// k ^ ((ch >> 3) & 7), so that the 8 lanes of one token, whose channels are 8
// rows apart, write to different banks.
constexpr int kBwdTok = 64;
__global__ __launch_bounds__(256) void k_bwd_tile(const float* __restrict__ p, const uint16_t* __restrict__ U,
                                                  const uint16_t* __restrict__ V, const uint16_t* __restrict__ g_h,
                                                  const uint64_t* __restrict__ mask, int64_t T, int nb, int Tp,
                                                  int gate, int keep, float inv_tau,
                                                  uint16_t* __restrict__ g_u, uint16_t* __restrict__ g_v,
                                                  uint16_t* __restrict__ g_p16, uint16_t* __restrict__ hT,
                                                  uint16_t* __restrict__ guT, uint16_t* __restrict__ gvT,
                                                  uint16_t* __restrict__ gpT, float* __restrict__ colpart) {
    constexpr int ROWS = 256 / 8;                    // tokens per pass
    __shared__ __attribute__((aligned(16))) uint16_t tile[4][kBank][kBwdTok];
    __shared__ float csum[ROWS][kBank + 1];
    const int tid = threadIdx.x;
    const int c8 = tid & 7, tr = tid >> 3;
    const int tb = blockIdx.x, b = blockIdx.y;
    const int d_i = nb * kBank;
    const int j0 = b * kBank + 8 * c8;               // this thread's first channel
    auto slot = [](int ch, int tl) { return (((tl >> 3) ^ ((ch >> 3) & 7)) << 3) + (tl & 7); };
    float colp[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) colp[e] = 0.f;
#pragma unroll
    for (int pass = 0; pass < kBwdTok / ROWS; ++pass) {
        const int tl = tr + ROWS * pass;             // token within the block
        const int64_t t = (int64_t)tb * kBwdTok + tl;
        uint16_t oh[8], ou[8], ov[8], op[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) oh[e] = ou[e] = ov[e] = op[e] = 0;
        if (t < T) {                                 // the same for the token's 8 lanes
            const int64_t o = t * (int64_t)d_i + j0;
            const float4 p0 = *reinterpret_cast<const float4*>(p + o);
            const float4 p1 = *reinterpret_cast<const float4*>(p + o + 4);
            Raw<uint16_t> ru, rv, rg;
            ru.load(U + o); rv.load(V + o); rg.load(g_h + o);
            const uint64_t mw = mask[t * nb + b];
            const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
            float u[8], v[8], gh[8];
            ru.decode(u); rv.decode(v); rg.decode(gh);
            // threshold: midpoint of the smallest kept and the largest dropped logit
            float kmin = __builtin_huge_valf(), dmax = -__builtin_huge_valf();
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float key = __builtin_isnan(pv[e]) ? -__builtin_huge_valf() : pv[e];
                const bool kept = (mw >> (8 * c8 + e)) & 1ull;
                kmin = kept ? fminf(kmin, key) : kmin;
                dmax = kept ? dmax : fmaxf(dmax, key);
            }
#pragma unroll
            for (int o2 = 1; o2 < 8; o2 <<= 1) {
                kmin = fminf(kmin, __shfl_xor(kmin, o2, kWave));
                dmax = fmaxf(dmax, __shfl_xor(dmax, o2, kWave));
            }
            const float theta = 0.5f * (kmin + dmax);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool kept = (mw >> (8 * c8 + e)) & 1ull;
                const float m = kept ? 1.f : 0.f;
                const float sp = sigmoidf_dev(pv[e]), su = sigmoidf_dev(u[e]);
                const float sg = gate ? su : sp;
                const float gm = gh[e] * sg * u[e] * v[e];   // dL/dm
                const float gu = gate ? m * gh[e] * v[e] * (su + u[e] * su * (1.f - su)) : m * gh[e] * sg * v[e];
                const float gv = m * gh[e] * sg * u[e];
                float gp = gate ? 0.f : m * gh[e] * u[e] * v[e] * sp * (1.f - sp);
                if (keep < kBank && inv_tau > 0.f) {
                    const float sa = sigmoidf_dev((pv[e] - theta) * inv_tau);
                    gp += gm * sa * (1.f - sa) * inv_tau;
                }
                colp[e] += gp;
                oh[e] = f32_to_bf16(m * sg * u[e] * v[e]);
                ou[e] = f32_to_bf16(gu);
                ov[e] = f32_to_bf16(gv);
                op[e] = f32_to_bf16(gp);
            }
            auto pack = [](const uint16_t (&h)[8]) {
                return make_uint4((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16),
                                  (uint32_t)h[4] | ((uint32_t)h[5] << 16), (uint32_t)h[6] | ((uint32_t)h[7] << 16));
            };
            *reinterpret_cast<uint4*>(g_u + o) = pack(ou);
            *reinterpret_cast<uint4*>(g_v + o) = pack(ov);
            *reinterpret_cast<uint4*>(g_p16 + o) = pack(op);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int ch = 8 * c8 + e;
            const int sl = slot(ch, tl);
            tile[0][ch][sl] = oh[e];
            tile[1][ch][sl] = ou[e];
            tile[2][ch][sl] = ov[e];
            tile[3][ch][sl] = op[e];
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) csum[tr][8 * c8 + e] = colp[e];
    __syncthreads();
    if (tid < kBank) {
        float sum = 0.f;
        for (int r = 0; r < ROWS; ++r) sum += csum[r][tid];
        colpart[(size_t)tb * d_i + b * kBank + tid] = sum;
    }
    // transposed tiles: 64 channel rows of 128 bytes per output, 16 bytes per thread
    uint16_t* const dst[4] = {hT, guT, gvT, gpT};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int c = tid + 256 * k;             // 512 chunks: row c / 8, chunk c % 8
            const int row = c >> 3, ch = c & 7;
            const uint4 val = *reinterpret_cast<const uint4*>(&tile[q][row][(ch ^ ((row >> 3) & 7)) << 3]);
            *reinterpret_cast<uint4*>(dst[q] + (size_t)(b * kBank + row) * Tp + (size_t)tb * kBwdTok + 8 * ch) = val;
        }
    }
}

// out[c] = sum over rows of x[r][c] in a fixed order: thread (column,
// eighth) sums every eighth row in order, then the eighths are summed in order
__global__ __launch_bounds__(256) void k_colsum(const float* __restrict__ x, int64_t rows, int cols,
                                                float* __restrict__ out) {
    __shared__ float red[8][32];
    const int cl = threadIdx.x & 31, q = threadIdx.x >> 5;
    const int c = blockIdx.x * 32 + cl;
    float a = 0.f;
    if (c < cols)
        for (int64_t r = q; r < rows; r += 8) a += x[r * cols + c];
    red[q][cl] = a;
    __syncthreads();
    if (q == 0 && c < cols) {
        float sum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) sum += red[k][cl];
        out[c] = sum;
    }
}

__global__ __launch_bounds__(256) void k_fill_f32(float* __restrict__ x, int64_t n, float v) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) x[i] = v;
}

namespace {
constexpr size_t kWsAlign = 256;
size_t up(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

struct BwdLayout {
    size_t z16, p32, gh16, U16, V16, gu16, gv16, gp16, gz16, colpart;
    size_t GT, hT, XT, guT, gvT, gpT, zT, gzT, BT, AT, WgT, WuT, total;
};

BwdLayout layout(int64_t T, int d, int d_i, int r, bool weights_t) {
    const size_t Tp = (size_t)((T + 63) / 64 * 64);
    const size_t tdi = (size_t)T * d_i;
    BwdLayout L{};
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off += up(bytes); return o; };
    L.z16 = take((size_t)T * r * 2);
    L.p32 = take(tdi * 4);
    L.gh16 = take(tdi * 2);
    // U16 is dead outside [UV GEMM, k_bwd_tile]: the other GEMMs use its
    // space for their fp32 K-split partials
    const int64_t Tq = (int64_t)Tp;
    const size_t part = std::max({gemm_nt_partial_floats(T, r, d), gemm_nt_partial_floats(T, d_i, r),
                                  gemm_nt_partial_floats(T, d_i, d), gemm_nt_partial_floats(d, d_i, (int)Tq),
                                  gemm_nt_partial_floats(d_i, d, (int)Tq), gemm_nt_partial_floats(d_i, r, (int)Tq),
                                  gemm_nt_partial_floats(T, r, d_i), gemm_nt_partial_floats(r, d, (int)Tq),
                                  gemm_nt_partial_floats(T, d, r), gemm_nt_partial_floats(T, d, d_i)});
    L.U16 = take(std::max(tdi * 2, part * 4));
    L.V16 = take(tdi * 2);
    L.gu16 = take(tdi * 2);
    L.gv16 = take(tdi * 2);
    L.colpart = take(Tp / 64 * (size_t)d_i * 4);
    L.gp16 = take(tdi * 2);
    L.gz16 = take((size_t)T * r * 2);
    L.GT = take((size_t)d * Tp * 2);
    L.hT = take((size_t)d_i * Tp * 2);
    L.XT = take((size_t)d * Tp * 2);
    L.guT = take((size_t)d_i * Tp * 2);
    L.gvT = take((size_t)d_i * Tp * 2);
    L.gpT = take((size_t)d_i * Tp * 2);
    L.zT = take((size_t)r * Tp * 2);
    L.gzT = take((size_t)r * Tp * 2);
    L.BT = take((size_t)r * d_i * 2);
    L.AT = take((size_t)d * r * 2);
    L.WgT = L.WuT = 0;
    if (!weights_t) {
        L.WgT = take((size_t)d * d_i * 2);
        L.WuT = take((size_t)d * d_i * 2);
    }
    L.total = off;
    return L;
}

template <typename P>
P* at(void* base, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}
}  // namespace

size_t backward_workspace_bytes(int64_t T, int d, int d_i, int rank, bool weights_t) {
    return layout(T, d, d_i, rank, weights_t).total;
}

hipError_t launch_backward(const BwdArgs& a, hipStream_t s) {
    const int64_t T = a.T;
    const int d = a.d, d_i = a.d_i, r = a.rank, nb = d_i / kBank;
    const int Tp = (int)((T + 63) / 64 * 64);
    const bool have_wt = a.W_gT != nullptr && a.W_uT != nullptr;
    const BwdLayout L = layout(T, d, d_i, r, have_wt);
    void* ws = a.ws;
    uint16_t* z16 = at<uint16_t>(ws, L.z16);
    float* p32 = at<float>(ws, L.p32);
    uint16_t* gh16 = at<uint16_t>(ws, L.gh16);
    uint16_t* U16 = at<uint16_t>(ws, L.U16);
    uint16_t* V16 = at<uint16_t>(ws, L.V16);
    float* split = at<float>(ws, L.U16);           // K-split partials of the other GEMMs
    uint16_t* gu16 = at<uint16_t>(ws, L.gu16);
    uint16_t* gv16 = at<uint16_t>(ws, L.gv16);
    float* colpart = at<float>(ws, L.colpart);
    uint16_t* gp16 = at<uint16_t>(ws, L.gp16);
    uint16_t* gz16 = at<uint16_t>(ws, L.gz16);
    uint16_t* GT = at<uint16_t>(ws, L.GT);
    uint16_t* hT = at<uint16_t>(ws, L.hT);
    uint16_t* XT = at<uint16_t>(ws, L.XT);
    uint16_t* guT = at<uint16_t>(ws, L.guT);
    uint16_t* gvT = at<uint16_t>(ws, L.gvT);
    uint16_t* gpT = at<uint16_t>(ws, L.gpT);
    uint16_t* zT = at<uint16_t>(ws, L.zT);
    uint16_t* gzT = at<uint16_t>(ws, L.gzT);
    uint16_t* BT = at<uint16_t>(ws, L.BT);
    uint16_t* AT = at<uint16_t>(ws, L.AT);
    const uint16_t* WgT = have_wt ? a.W_gT : at<uint16_t>(ws, L.WgT);
    const uint16_t* WuT = have_wt ? a.W_uT : at<uint16_t>(ws, L.WuT);
    hipError_t e = hipSuccess;
    auto ok = [&](hipError_t x) { if (e == hipSuccess) e = x; return e == hipSuccess; };

    // recomputed forward: z, p, dense U and V; g_h for every channel
    ok(launch_gemm_nt(a.x, a.A, T, r, d, z16, GemmOut::BF16, s, nullptr, split));
    ok(launch_gemm_nt(z16, a.B, T, d_i, r, p32, GemmOut::F32, s, a.bias, split));
    ok(launch_gemm_nt(a.g_y, a.W_dT, T, d_i, d, gh16, GemmOut::BF16, s, nullptr, split));
    ok(launch_uv_gemm(a.x, a.W_g, a.W_u, T, d_i, d, U16, V16, s));
    hipLaunchKernelGGL(k_bwd_tile, dim3((unsigned)(Tp / kBwdTok), (unsigned)nb), dim3(256), 0, s, p32, U16, V16,
                       gh16, a.mask, T, nb, Tp, a.gate, a.keep, a.inv_tau, gu16, gv16, gp16, hT, guT, gvT, gpT,
                       colpart);
    ok(hipGetLastError());
    if (a.g_bias) {
        hipLaunchKernelGGL(k_colsum, dim3((unsigned)((d_i + 31) / 32)), dim3(256), 0, s, colpart,
                           (int64_t)(Tp / kBwdTok), d_i, a.g_bias);
        ok(hipGetLastError());
    }
    // token-major operands transposed for the weight gradients (K = tokens)
    ok(launch_transpose(Dt::BF16, a.g_y, GT, (int)T, d, s, Tp));
    ok(launch_transpose(Dt::BF16, a.x, XT, (int)T, d, s, Tp));
    ok(launch_transpose(Dt::BF16, z16, zT, (int)T, r, s, Tp));
    ok(launch_gemm_nt(GT, hT, d, d_i, Tp, a.g_Wd, GemmOut::F32, s, nullptr, split));
    ok(launch_gemm_nt(guT, XT, d_i, d, Tp, a.g_Wg, GemmOut::F32, s, nullptr, split));
    ok(launch_gemm_nt(gvT, XT, d_i, d, Tp, a.g_Wu, GemmOut::F32, s, nullptr, split));
    ok(launch_gemm_nt(gpT, zT, d_i, r, Tp, a.g_B, GemmOut::F32, s, nullptr, split));
    // the predictor's input side
    ok(launch_transpose(Dt::BF16, a.B, BT, d_i, r, s));
    ok(launch_gemm_nt(gp16, BT, T, r, d_i, gz16, GemmOut::BF16, s, nullptr, split));
    ok(launch_transpose(Dt::BF16, gz16, gzT, (int)T, r, s, Tp));
    ok(launch_gemm_nt(gzT, XT, r, d, Tp, a.g_A, GemmOut::F32, s, nullptr, split));
    // g_x = g_z A + g_u W_g + g_v W_u
    ok(launch_transpose(Dt::BF16, a.A, AT, r, d, s));
    if (!have_wt) {
        ok(launch_transpose(Dt::BF16, a.W_g, at<uint16_t>(ws, L.WgT), d_i, d, s));
        ok(launch_transpose(Dt::BF16, a.W_u, at<uint16_t>(ws, L.WuT), d_i, d, s));
    }
    ok(launch_gemm_nt(gz16, AT, T, d, r, a.g_x, GemmOut::F32, s, nullptr, split));
    ok(launch_gemm_nt(gu16, WgT, T, d, d_i, a.g_x, GemmOut::F32_ACC, s, nullptr, split));
    ok(launch_gemm_nt(gv16, WuT, T, d, d_i, a.g_x, GemmOut::F32_ACC, s, nullptr, split));
    return e;
}

hipError_t launch_zero_f32(float* x, int64_t n, hipStream_t s) {
    if (x == nullptr || n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, x, n, 0.f);
    return hipGetLastError();
}

}  // namespace sffn
