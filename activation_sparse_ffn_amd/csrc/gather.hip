// Token-gather path of the sparse FFN forward: decode-sized batches (and
// every fp32 layer) on the vector ALUs, reading only the weight rows that
// each token's mask keeps.
//
// Steps per token, after "Continual LLM Upcycling" (gist.science technical
// summary, Methodologie > 1. Architectuur and 3. Hardware Implicaties):
//   k_pred1       z = x A^T                (predictor layer 1; bf16 layers
//                                           store z rounded to bf16)
//   k_pred2_topk  p = z B^T + bias, bank top-k, compact list of kept
//                 channel ids and their logits   (one workgroup per bank)
//   k_gateup      u, v on kept rows of W_g / W_u, h = s * u * v
//   k_down        partial y over groups of 64 kept channels, rows of W_d^T
//   k_reduce      y = sum of the partials, in a fixed order
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

// ---------------------------------------------------------------------------
// predictor layer 1: one wave per (token, rank row)
// ---------------------------------------------------------------------------
template <typename E, int NC>
__global__ __launch_bounds__(256) void k_pred1(const E* __restrict__ x, const E* __restrict__ A,
                                               float* __restrict__ z, int d, int rank,
                                               int64_t n_work, int round_bf16) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= n_work) return;
    const int64_t t = w / rank;
    const int q = (int)(w - t * rank);
    const E* xr = x + t * d;
    const E* ar = A + (int64_t)q * d;
    const int nch = d / 8;
    float acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * NC) {
        Raw<E> rx[NC], ra[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < nch) { rx[k].load(xr + 8 * c); ra[k].load(ar + 8 * c); }
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < nch) {
                float xv[8], av[8];
                rx[k].decode(xv);
                ra[k].decode(av);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(xv[e], av[e], acc);
            }
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) z[w] = round_bf16 ? bf16_to_f32(f32_to_bf16(acc)) : acc;
}

// Sixteen per-lane partial sums -> full wave sums. On return every lane
// holds the sum of row (lane >> 2) in r[0].
__device__ __forceinline__ void reduce16_rows(float (&r)[16], int lane) {
#pragma unroll
    for (int o = 32, n = 16; o >= 4; o >>= 1, n >>= 1) {
        const bool upper = (lane & o) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float give = upper ? r[i] : r[i + n / 2];
            const float mine = upper ? r[i + n / 2] : r[i];
            r[i] = mine + __shfl_xor(give, o, kWave);
        }
    }
    r[0] += __shfl_xor(r[0], 1, kWave);
    r[0] += __shfl_xor(r[0], 2, kWave);
}

// ---------------------------------------------------------------------------
// predictor layer 2 + bank top-k: one workgroup (4 waves x 16 rows) per
// (token, bank)
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void k_pred2_topk(const float* __restrict__ z,
                                                    const E* __restrict__ B,
                                                    const float* __restrict__ bias,
                                                    int rank, int d_i, int keep,
                                                    uint64_t* __restrict__ mask,
                                                    float* __restrict__ logits,
                                                    uint16_t* __restrict__ ids,
                                                    float* __restrict__ pk) {
    __shared__ float sp[kBank];
    const int nb = d_i / kBank;
    const int64_t t = blockIdx.x / nb;
    const int b = (int)(blockIdx.x - t * nb);
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* zt = z + t * rank;
    const int nch = rank / 8;
    const int64_t row0 = (int64_t)b * kBank + 16 * wv;

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int c = lane; c < nch; c += 64) {
        float zv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) zv[e] = zt[8 * c + e];
        Raw<E> rb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rb[i].load(B + (row0 + i) * rank + 8 * c);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float bv[8];
            rb[i].decode(bv);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i] = fmaf(zv[e], bv[e], acc[i]);
        }
    }
    reduce16_rows(acc, lane);
    if ((lane & 3) == 0) {
        const int r = lane >> 2;
        const float bj = bias ? bias[row0 + r] : 0.f;
        sp[16 * wv + r] = acc[0] + bj;
    }
    __syncthreads();
    if (wv == 0) {
        const float p = sp[lane];
        const uint64_t sel = wave_bank_topk(rank_key(p), keep);
        const int j = b * kBank + lane;
        if (logits) logits[t * d_i + j] = p;
        if (lane == 0) mask[t * nb + b] = sel;
        if ((sel >> lane) & 1ull) {
            const int64_t slot = t * (int64_t)(nb * keep) + (int64_t)b * keep + lanes_below(sel);
            ids[slot] = (uint16_t)j;
            pk[slot] = p;
        }
    }
}

// ---------------------------------------------------------------------------
// gate / up on kept rows: one wave per (token, kept channel)
// ---------------------------------------------------------------------------
template <typename E, int NC>
__global__ __launch_bounds__(256) void k_gateup(const E* __restrict__ x, const E* __restrict__ Wg,
                                                const E* __restrict__ Wu,
                                                const uint16_t* __restrict__ ids,
                                                const float* __restrict__ pk,
                                                float* __restrict__ h, int d, int d_s,
                                                int64_t n_work, int gate) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (w >= n_work) return;
    const int64_t t = w / d_s;
    const int64_t j = ids[w];
    const E* xr = x + t * d;
    const E* gr = Wg + j * d;
    const E* ur = Wu + j * d;
    const int nch = d / 8;
    float u = 0.f, v = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * NC) {
        Raw<E> rg[NC], ru[NC], rx[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < nch) { rg[k].load(gr + 8 * c); ru[k].load(ur + 8 * c); rx[k].load(xr + 8 * c); }
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (c < nch) {
                float xv[8], gv[8], uv[8];
                rx[k].decode(xv);
                rg[k].decode(gv);
                ru[k].decode(uv);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    u = fmaf(xv[e], gv[e], u);
                    v = fmaf(xv[e], uv[e], v);
                }
            }
        }
    }
    u = wave_sum(u);
    v = wave_sum(v);
    if (lane == 0) {
        const float s = gate ? sigmoidf_dev(u) : sigmoidf_dev(pk[w]);
        h[w] = s * u * v;
    }
}

// ---------------------------------------------------------------------------
// down projection: workgroup = (token, group of 64 kept channels, 512-column
// slice); each wave accumulates 16 rows of W_d^T, then the four waves are
// summed through LDS into one partial row.
// ---------------------------------------------------------------------------
constexpr int kGroup = 64;
constexpr int kSlice = 512;

template <typename E>
__global__ __launch_bounds__(256) void k_down(const E* __restrict__ WdT,
                                              const uint16_t* __restrict__ ids,
                                              const float* __restrict__ h,
                                              float* __restrict__ partial, int d, int d_s,
                                              int groups, int slices) {
    __shared__ float red[4][kSlice];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t blk = blockIdx.x;
    const int s = (int)(blk % slices);
    const int64_t tg = blk / slices;
    const int g = (int)(tg % groups);
    const int64_t t = tg / groups;
    const int col = s * kSlice + lane * 8;
    const bool active = col < d;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int slot0 = g * kGroup + 16 * wv;
    const int n_rows = min(16, d_s - slot0);
    if (active && n_rows > 0) {
        Raw<E> rw[16];
        float hv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < n_rows) {
                const int64_t slot = t * d_s + slot0 + i;
                const int64_t j = ids[slot];
                hv[i] = h[slot];
                rw[i].load(WdT + j * d + col);
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < n_rows) {
                float wv8[8];
                rw[i].decode(wv8);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[e] = fmaf(hv[i], wv8[e], acc[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) red[wv][lane * 8 + e] = acc[e];
    __syncthreads();
    float* out = partial + (t * groups + g) * (int64_t)d;
    for (int c = threadIdx.x; c < kSlice; c += 256) {
        const int gc = s * kSlice + c;
        if (gc < d) out[gc] = (red[0][c] + red[1][c]) + (red[2][c] + red[3][c]);
    }
}

template <typename E>
__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ partial, E* __restrict__ y,
                                                int d, int groups, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    const int64_t t = i / d;
    const int c = (int)(i - t * d);
    const float* p = partial + t * groups * (int64_t)d + c;
    float acc = 0.f;
    for (int g = 0; g < groups; ++g) acc += p[(int64_t)g * d];
    Elem<E>::store1(y + i, acc);
}

int gather_groups(int d_s) { return (d_s + kGroup - 1) / kGroup; }

template <typename E, int NC>
static hipError_t gather_forward(const GatherArgs& a, hipStream_t s) {
    const E* x = static_cast<const E*>(a.x);
    const int nb = a.d_i / kBank;
    const int d_s = nb * a.keep;
    const int64_t T = a.T;
    {
        const int64_t n = T * a.rank;
        xlaunch(a.events, 0, k_pred1<E, NC>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, x,
                           static_cast<const E*>(a.A), a.z, a.d, a.rank, n,
                           a.dt == Dt::BF16 ? 1 : 0);
    }
    xlaunch(a.events, 1, k_pred2_topk<E>, dim3((unsigned)(T * nb)), dim3(256), 0, s, a.z,
                       static_cast<const E*>(a.B), a.bias, a.rank, a.d_i, a.keep, a.mask,
                       a.logits, a.ids, a.pk);
    {
        const int64_t n = T * d_s;
        xlaunch(a.events, 2, k_gateup<E, NC>, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, x,
                           static_cast<const E*>(a.W_g), static_cast<const E*>(a.W_u), a.ids,
                           a.pk, a.h, a.d, d_s, n, a.gate);
    }
    const int groups = gather_groups(d_s);
    const int slices = (a.d + kSlice - 1) / kSlice;
    xlaunch(a.events, 3, k_down<E>, dim3((unsigned)(T * groups * slices)), dim3(256), 0, s,
                       static_cast<const E*>(a.W_dT), a.ids, a.h, a.partial, a.d, d_s, groups,
                       slices);
    {
        const int64_t n = T * a.d;
        xlaunch(a.events, 4, k_reduce<E>, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           a.partial, static_cast<E*>(a.y), a.d, groups, n);
    }
    return hipGetLastError();
}

hipError_t launch_gather_forward(const GatherArgs& a, hipStream_t s) {
    if (a.dt == Dt::BF16) return gather_forward<uint16_t, 8>(a, s);
    return gather_forward<float, 4>(a, s);
}

// ---------------------------------------------------------------------------
// packing: out-of-place transpose through LDS, 64 x 64 tiles
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ src, E* __restrict__ dst,
                                                   int rows, int cols) {
    __shared__ E tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int gr = r0 + r, gc = c0 + tx;
        if (gr < rows && gc < cols) tile[r][tx] = src[(int64_t)gr * cols + gc];
    }
    __syncthreads();
    for (int c = ty; c < 64; c += 4) {
        const int gc = c0 + c, gr = r0 + tx;
        if (gc < cols && gr < rows) dst[(int64_t)gc * rows + gr] = tile[tx][c];
    }
}

hipError_t launch_transpose(Dt dt, const void* src, void* dst, int rows, int cols, hipStream_t s) {
    dim3 grid((cols + 63) / 64, (rows + 63) / 64);
    if (dt == Dt::BF16)
        hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, cols);
    else
        hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s,
                           static_cast<const float*>(src), static_cast<float*>(dst), rows, cols);
    return hipGetLastError();
}

}  // namespace sffn
