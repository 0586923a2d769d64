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
// predictor layer 1: one workgroup per (token, rank row); the four waves split
// the d-long dot product and meet in LDS. EXACT: d/8 is a multiple of 256*NC.
// ---------------------------------------------------------------------------
template <typename E, int NC, bool EXACT>
__global__ __launch_bounds__(256) void k_pred1(const E* __restrict__ x, const E* __restrict__ A,
                                               float* __restrict__ z, int d, int rank,
                                               int round_bf16) {
    __shared__ float red[4];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const unsigned w = blockIdx.x;
    const unsigned t = w / (unsigned)rank;
    const unsigned q = w - t * (unsigned)rank;
    const E* xr = x + (size_t)t * d;
    const E* ar = A + (size_t)q * d;
    const int nch = d / 8;
    float acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 256 * NC) {
        Raw<E> rx[NC], ra[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + tid + 256 * k;
            if (EXACT || c < nch) { ra[k].load(ar + 8 * c); rx[k].load(xr + 8 * c); }
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + tid + 256 * k;
            if (EXACT || c < nch) {
                float xv[8], av[8];
                rx[k].decode(xv);
                ra[k].decode(av);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(xv[e], av[e], acc);
            }
        }
    }
    acc = wave_sum(acc);
    if (lane == 0) red[wv] = acc;
    __syncthreads();
    if (tid == 0) {
        const float v = (red[0] + red[1]) + (red[2] + red[3]);
        z[w] = round_bf16 ? bf16_to_f32(f32_to_bf16(v)) : v;
    }
}

// N per-lane partial sums (N a power of two) -> full wave sums. Each
// butterfly step trades half of the rows with the partner lane, so the whole
// reduction costs N - 1 + (6 - log2 N) shuffles. On return every lane holds
// the sum of row (lane >> (6 - log2 N)) in r[0].
template <int N>
__device__ __forceinline__ void reduce_rows(float (&r)[N], int lane) {
    constexpr int L = __builtin_ctz(N);
#pragma unroll
    for (int st = 0; st < L; ++st) {
        const int o = 32 >> st;
        const int h = (N >> st) / 2;
        const bool upper = (lane & o) != 0;
#pragma unroll
        for (int i = 0; i < h; ++i) {
            const float a = r[i], c = r[i + h];
            const float give = upper ? a : c;
            const float mine = upper ? c : a;
            r[i] = mine + __shfl_xor(give, o, kWave);
        }
    }
#pragma unroll
    for (int o = 1; o < (64 >> L); o <<= 1) r[0] += __shfl_xor(r[0], o, kWave);
}

// ---------------------------------------------------------------------------
// predictor layer 2 + bank top-k: one workgroup (4 waves x 16 rows) per
// (token, bank)
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_pred2_topk(const float* __restrict__ z,
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
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const float* zt = z + t * rank;
    const int nch = rank / 8;
    const int64_t row0 = (int64_t)b * kBank + 16 * wv;

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;
    for (int c = lane; c < nch; c += 64) {
        Raw<E> rb[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rb[i].load(B + (row0 + i) * rank + 8 * c);
        const float4 z0 = *reinterpret_cast<const float4*>(zt + 8 * c);
        const float4 z1 = *reinterpret_cast<const float4*>(zt + 8 * c + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float bv[8];
            rb[i].decode(bv);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i] = fmaf(zv[e], bv[e], acc[i]);
        }
    }
    reduce_rows<16>(acc, lane);
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
template <typename E, int NC, bool EXACT>
__global__ __launch_bounds__(256) void k_gateup(const E* __restrict__ x, const E* __restrict__ Wg,
                                                const E* __restrict__ Wu,
                                                const uint16_t* __restrict__ ids,
                                                const float* __restrict__ pk,
                                                float* __restrict__ h, int d, int d_s,
                                                int64_t n_work, int gate) {
    const int lane = threadIdx.x & 63;
    // wave-uniform work index: the id and logit below become scalar loads
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= n_work) return;
    const unsigned t = (unsigned)w / (unsigned)d_s;
    // no id list: every channel, in order
    const int64_t j = ids ? (int64_t)ids[w] : w - (int64_t)t * d_s;
    const E* xr = x + (size_t)t * d;
    const E* gr = Wg + j * d;
    const E* ur = Wu + j * d;
    const int nch = d / 8;
    float u = 0.f, v = 0.f;
    for (int c0 = 0; c0 < nch; c0 += 64 * NC) {
        Raw<E> rg[NC], ru[NC], rx[NC];
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (EXACT || c < nch) { rg[k].load(gr + 8 * c); ru[k].load(ur + 8 * c); rx[k].load(xr + 8 * c); }
        }
#pragma unroll
        for (int k = 0; k < NC; ++k) {
            const int c = c0 + lane + 64 * k;
            if (EXACT || c < nch) {
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

template <typename E, bool EXACT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 4))) void k_down(const E* __restrict__ WdT,
                                              const uint16_t* __restrict__ ids,
                                              const float* __restrict__ h,
                                              float* __restrict__ partial, int d, int d_s,
                                              int groups, int slices) {
    __shared__ float red[4][kSlice];
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int64_t blk = blockIdx.x;
    const int s = (int)(blk % slices);
    const int64_t tg = blk / slices;
    const int g = (int)(tg % groups);
    const int64_t t = tg / groups;
    const int col = s * kSlice + lane * 8;
    const bool active = EXACT || col < d;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    const int slot0 = g * kGroup + 16 * wv;
    const int n_rows = EXACT ? 16 : min(16, d_s - slot0);
    if (active && n_rows > 0) {
        Raw<E> rw[16];
        float hv[16];
        const size_t base = (size_t)t * d_s + slot0;
        if (ids == nullptr) {
            // every channel, in order: rows slot0 .. slot0 + 15
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (EXACT || i < n_rows) {
                    hv[i] = h[base + i];
                    rw[i].load(WdT + (size_t)(slot0 + i) * d + col);
                }
            }
        } else if constexpr (EXACT) {
            // sixteen ids as two 16-byte words, made wave-uniform so that the
            // row addresses live in scalar registers and all 16 row loads
            // issue back to back
            const uint4 i0 = *reinterpret_cast<const uint4*>(ids + base);
            const uint4 i1 = *reinterpret_cast<const uint4*>(ids + base + 8);
            const uint32_t iw[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t u = __builtin_amdgcn_readfirstlane(iw[k]);
                rw[2 * k].load(WdT + (size_t)(u & 0xffffu) * d + col);
                rw[2 * k + 1].load(WdT + (size_t)(u >> 16) * d + col);
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) hv[i] = h[base + i];
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if (i < n_rows) {
                    const int64_t j = ids[base + i];
                    hv[i] = h[base + i];
                    rw[i].load(WdT + j * d + col);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (EXACT || i < n_rows) {
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

// y = sum of the partial rows in a fixed order: workgroup = (token, 32
// columns) of 32 kReduceParts threads; thread (column, part) sums every
// kReduceParts-th partial row with all of its loads in flight, then LDS joins
// the parts in order. 16 parts (512 threads, 14 loads each for the 224 rows
// of the method's layer) step 0.5 us faster than 8 parts (256 threads, 28
// loads each), and the non-temporal hint on the loads another 0.2 us.
constexpr int kReduceParts = 16;
template <typename E>
__global__ __launch_bounds__(32 * kReduceParts) void k_reduce(const float* __restrict__ partial, E* __restrict__ y,
                                                              int d, int groups, int col_blocks) {
    constexpr int Q = kReduceParts, PER = 16;        // parts, loads per thread per pass
    __shared__ float red[Q][32];
    const int tid = threadIdx.x, cl = tid & 31, q = tid >> 5;
    const unsigned t = blockIdx.x / (unsigned)col_blocks;
    const int c = (int)(blockIdx.x - t * col_blocks) * 32 + cl;
    const bool active = c < d;
    const float* p = partial + (size_t)t * groups * d + (active ? c : 0);
    float acc = 0.f;
    for (int g0 = q; g0 < groups; g0 += Q * PER) {
        float v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int g = g0 + Q * k;
            v[k] = (active && g < groups) ? __builtin_nontemporal_load(p + (size_t)g * d) : 0.f;   // read once
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) acc += v[k];
    }
    red[q][cl] = acc;
    __syncthreads();
    if (q == 0 && active) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < Q; ++k) s += red[k][cl];
        Elem<E>::store1(y + (size_t)t * d + c, s);
    }
}

// ---------------------------------------------------------------------------
// Fused decode kernel for the method's layer width (d = 4096): one workgroup
// of KEEP waves per (token, bank) runs predictor layer 2 on the bank's 64 rows
// of B, the bank top-k, gate/up on the KEEP kept rows and the bank's share of
// the down projection over all d columns, written as one partial row of y.
// Every wave runs the bank top-k itself (the mask is wave-uniform, so the
// kept channels come out of it in scalar registers). Wave w computes u and v
// of kept channel w; the weight rows then stream through a bounded window:
// per thread, its 1 KB chunks of the wave's W_g and W_u rows and then its
// 16-byte pieces of its half of the kept W_d^T rows form one ordered stream
// of 16-byte loads, of which at most kFusedAhead groups of four are in
// flight (requesting a workgroup's ~400 KB at once congests the memory
// system). The two halves of the workgroup each sum half of the kept W_d^T
// rows over all d columns and meet in LDS. 16 waves per bank stream the
// weight rows ~2% faster than 8 waves with two kept channels each.
// ---------------------------------------------------------------------------
constexpr int kFusedD = 4096;
constexpr int kFusedAhead = 2;   // groups of four 16-byte loads in flight per thread

template <int KEEP>
__global__ __launch_bounds__(64 * KEEP)
void k_bank_fused(const uint16_t* __restrict__ x, const float* __restrict__ z,
                  const uint16_t* __restrict__ B, const float* __restrict__ bias,
                  const uint16_t* __restrict__ Wg, const uint16_t* __restrict__ Wu,
                  const uint16_t* __restrict__ WdT, int rank, int d_i, int gate,
                  uint64_t* __restrict__ mask, float* __restrict__ logits,
                  float* __restrict__ partial) {
    constexpr int D = kFusedD, NW = KEEP, NT = kWave * NW;
    constexpr int NCX = D / 8 / kWave;            // 16-byte chunks per lane of a gate/up row
    constexpr int RPW = kBank / NW;               // rows of B per wave
    constexpr int CPT = D / 8;                    // threads over the d columns (8 each)
    constexpr int HALVES = NT / CPT;              // thread groups splitting the kept W_d^T rows
    constexpr int DPH = KEEP / HALVES;            // kept W_d^T rows per thread
    constexpr int NS = NCX / 2 + DPH / 4;         // steps of the load stream
    static_assert(NT % CPT == 0 && HALVES == 2 && DPH % 4 == 0 && NCX % 2 == 0 && RPW >= 1,
                  "the layout of the method's layer: 16 kept of 64, d = 4096");
    __shared__ uint4 xs[D / 8];
    __shared__ float sp[kBank];
    __shared__ float sh[KEEP];
    __shared__ float4 comb[CPT][2];               // the upper half's sums
    const int tid = threadIdx.x, lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nb = d_i / kBank;
    const unsigned t = blockIdx.x / (unsigned)nb;
    const unsigned b = blockIdx.x - t * (unsigned)nb;
    const int nch = rank / 8;

    // predictor layer 2: wave wv takes rows 64 b + RPW wv .. + RPW
    const size_t row0 = (size_t)b * kBank + RPW * wv;
    float acc[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = 0.f;
    for (int c = lane; c < nch; c += kWave) {
        Raw<uint16_t> rb[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) rb[i].load_stream(B + (row0 + i) * rank + 8 * c);   // read once per token
        const float* zt = z + (size_t)t * rank + 8 * c;
        const float4 z0 = *reinterpret_cast<const float4*>(zt);
        const float4 z1 = *reinterpret_cast<const float4*>(zt + 4);
        const float zv[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            float bv[8];
            rb[i].decode(bv);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i] = fmaf(zv[e], bv[e], acc[i]);
        }
    }
    if (tid < CPT) xs[tid] = *reinterpret_cast<const uint4*>(x + (size_t)t * D + 8 * tid);
    reduce_rows<RPW>(acc, lane);
    if ((lane & (kWave / RPW - 1)) == 0) {
        const int r = lane / (kWave / RPW);
        sp[RPW * wv + r] = acc[0] + (bias ? bias[row0 + r] : 0.f);
    }
    __syncthreads();

    // bank top-k, run by every wave: the mask is wave-uniform, so each wave
    // finds the kept channels in it (slot k = the k-th set bit) without an
    // exchange through LDS
    const float pl = sp[lane];
    const uint64_t sel = wave_bank_topk(rank_key(pl), KEEP);
    if (wv == 0) {
        if (logits) logits[(size_t)t * d_i + (size_t)b * kBank + lane] = pl;
        if (lane == 0) mask[(size_t)t * nb + b] = sel;
    }
    auto drop = [](uint64_t m, int n) {          // m without its n lowest set bits
        for (int i = 0; i < n; ++i) m &= m - 1;
        return m;
    };
    // this wave's kept channel (slot wv) and its rows
    const int c0 = __builtin_ctzll(drop(sel, wv));
    const size_t j0 = (size_t)b * kBank + c0;
    const uint16_t* rows[2] = {Wg + j0 * D, Wu + j0 * D};
    // this thread's kept rows of W_d^T: slots DPH hf .. + DPH - 1, columns
    // 8 (tid % CPT) .. + 7
    const int hf = tid / CPT, col = 8 * (tid % CPT);
    const uint16_t* drow[DPH];
    {
        uint64_t m = drop(sel, DPH * hf);
#pragma unroll
        for (int k = 0; k < DPH; ++k) {
            drow[k] = WdT + ((size_t)b * kBank + __builtin_ctzll(m)) * D + col;
            m &= m - 1;
        }
    }
    // the ordered load stream: step s < NCX / 2 fetches chunks 2 s and 2 s + 1
    // of both gate/up rows, step NCX / 2 + q the W_d^T pieces 4 q .. 4 q + 3
    Raw<uint16_t> rc[NCX][2];
    Raw<uint16_t> rd[DPH];
    auto issue = [&](int st) {
        if (st < NCX / 2) {
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int k = 0; k < 2; ++k)
                    rc[2 * st + h][k].load_stream(rows[k] + 8 * (lane + kWave * (2 * st + h)));
        } else if (st < NS) {
#pragma unroll
            for (int k = 0; k < 4; ++k) rd[4 * (st - NCX / 2) + k].load_stream(drow[4 * (st - NCX / 2) + k]);
        }
    };
#pragma unroll
    for (int st = 0; st < kFusedAhead; ++st) issue(st);
    float u = 0.f, v = 0.f;
#pragma unroll
    for (int st = 0; st < NCX / 2; ++st) {
        // the scheduling barriers keep each step's loads behind the previous
        // step's arithmetic, so that the window stays bounded
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int m = 2 * st + h;
            const uint4 xw = xs[lane + kWave * m];
            const float xv[8] = {bf16_lo(xw.x), bf16_hi(xw.x), bf16_lo(xw.y), bf16_hi(xw.y),
                                 bf16_lo(xw.z), bf16_hi(xw.z), bf16_lo(xw.w), bf16_hi(xw.w)};
            float g[8], q[8];
            rc[m][0].decode(g);
            rc[m][1].decode(q);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u = fmaf(xv[e], g[e], u);
                v = fmaf(xv[e], q[e], v);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(st + kFusedAhead);
    }
#pragma unroll
    for (int st = NCX / 2 + kFusedAhead; st < NS; ++st) issue(st);
    __builtin_amdgcn_sched_barrier(0);
    {
        const float a0 = wave_sum(u), b0 = wave_sum(v);
        if (lane == 0) {
            const float p0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pl), c0));
            sh[wv] = (gate ? sigmoidf_dev(a0) : sigmoidf_dev(p0)) * a0 * b0;
        }
    }
    __syncthreads();

    // this bank's share of y over all columns, half of the kept rows per
    // thread group; the upper half's sums go through LDS
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
#pragma unroll
    for (int k = 0; k < DPH; ++k) {
        const float hk = sh[DPH * hf + k];
        float w8[8];
        rd[k].decode(w8);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = fmaf(hk, w8[e], o[e]);
    }
    if (hf == 1) {
        comb[tid - CPT][0] = make_float4(o[0], o[1], o[2], o[3]);
        comb[tid - CPT][1] = make_float4(o[4], o[5], o[6], o[7]);
    }
    __syncthreads();
    if (hf == 0) {
        const float4 q0 = comb[tid][0], q1 = comb[tid][1];
        float* out = partial + ((size_t)t * nb + b) * D + col;
        reinterpret_cast<float4*>(out)[0] = make_float4(o[0] + q0.x, o[1] + q0.y, o[2] + q0.z, o[3] + q0.w);
        reinterpret_cast<float4*>(out)[1] = make_float4(o[4] + q1.x, o[5] + q1.y, o[6] + q1.z, o[7] + q1.w);
    }
}

// ---------------------------------------------------------------------------
// Dense-4x baseline (post-hoc amplitude sparsity): one wave per (token,
// bank) ranks |a| of the bank's 64 amplitudes a = SiLU(u) v, writes the mask
// word, the kept channel ids in ascending order with their amplitudes (the h
// of the down projection), and the amplitudes themselves when asked for.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_amp_topk(const float* __restrict__ amp, int64_t n_words, int nb,
                                                  int keep, uint64_t* __restrict__ mask,
                                                  float* __restrict__ out_amp, uint16_t* __restrict__ ids,
                                                  float* __restrict__ hk, uint16_t* __restrict__ h_dense) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= n_words) return;
    const int64_t t = w / nb;
    const int b = (int)(w - t * nb);
    const int d_i = nb * kBank;
    const int j = b * kBank + lane;
    const float v = amp[t * d_i + j];
    const uint64_t sel = wave_bank_topk(rank_key(fabsf(v)), keep);
    const bool kept = (sel >> lane) & 1ull;
    if (lane == 0) mask[w] = sel;
    if (out_amp) out_amp[t * d_i + j] = v;
    if (h_dense) h_dense[t * d_i + j] = kept ? f32_to_bf16(v) : (uint16_t)0;
    if (ids && kept) {
        const int64_t slot = w * keep + lanes_below(sel);
        ids[slot] = (uint16_t)j;
        hk[slot] = v;
    }
}

hipError_t launch_amp_mask(const float* amp, int64_t T, int d_i, int keep, uint64_t* mask, uint16_t* h_dense,
                           hipStream_t s, void* const* events, int stage) {
    const int nb = d_i / kBank;
    xlaunch(events, stage, k_amp_topk, dim3((unsigned)((T * nb + 3) / 4)), dim3(256), 0, s, amp, T * nb, nb,
            keep, mask, nullptr, nullptr, nullptr, h_dense);
    return hipGetLastError();
}

int gather_groups(int d_s) { return (d_s + kGroup - 1) / kGroup; }

bool fused_ok(const GatherArgs& a) {
    return a.dt == Dt::BF16 && a.d == kFusedD && a.keep == 16 && a.rank % 8 == 0 && a.rank <= 512;
}

template <typename E, int NC>
static hipError_t gather_forward(const GatherArgs& a, hipStream_t s) {
    const E* x = static_cast<const E*>(a.x);
    const int nb = a.d_i / kBank;
    const int d_s = nb * a.keep;
    const int64_t T = a.T;
    const int nch = a.d / 8;
    const int rb = a.dt == Dt::BF16 ? 1 : 0;
    if (a.gate == kGateAmplitude) {
        // Dense-4x baseline: dense gate/up (a = SiLU(u) v for every channel),
        // the amplitude top-k, then down on the kept channels only
        const int64_t n = T * a.d_i;
        const dim3 grid((unsigned)((n + 3) / 4));
        if (nch % (64 * NC) == 0)
            xlaunch(a.events, 0, k_gateup<E, NC, true>, grid, dim3(256), 0, s, x,
                    static_cast<const E*>(a.W_g), static_cast<const E*>(a.W_u), nullptr, nullptr, a.amp,
                    a.d, a.d_i, n, 1);
        else
            xlaunch(a.events, 0, k_gateup<E, NC, false>, grid, dim3(256), 0, s, x,
                    static_cast<const E*>(a.W_g), static_cast<const E*>(a.W_u), nullptr, nullptr, a.amp,
                    a.d, a.d_i, n, 1);
        xlaunch(a.events, 1, k_amp_topk, dim3((unsigned)((T * nb + 3) / 4)), dim3(256), 0, s, a.amp,
                T * nb, nb, a.keep, a.mask, a.logits, a.ids, a.h, nullptr);
        const int groups = gather_groups(d_s);
        const int slices = (a.d + kSlice - 1) / kSlice;
        const dim3 dgrid((unsigned)(T * groups * slices));
        if (a.d % kSlice == 0 && d_s % kGroup == 0)
            xlaunch(a.events, 2, k_down<E, true>, dgrid, dim3(256), 0, s, static_cast<const E*>(a.W_dT),
                    a.ids, a.h, a.partial, a.d, d_s, groups, slices);
        else
            xlaunch(a.events, 2, k_down<E, false>, dgrid, dim3(256), 0, s, static_cast<const E*>(a.W_dT),
                    a.ids, a.h, a.partial, a.d, d_s, groups, slices);
        const int col_blocks = (a.d + 31) / 32;
        xlaunch(a.events, 3, k_reduce<E>, dim3((unsigned)(T * col_blocks)), dim3(32 * kReduceParts), 0, s, a.partial,
                static_cast<E*>(a.y), a.d, groups, col_blocks);
        skip_stages(a.events, 4, s);
        return hipGetLastError();
    }
    // every channel kept with the silu gate and no logits asked for: no
    // predictor and no top-k; gate/up and down walk all channels in order
    const bool dense = !a.need_pred;
    const uint16_t* ids = dense ? nullptr : a.ids;
    if (dense) {
        skip_range(a.events, 0, 2, s);
        if (a.mask_requested) {
            const hipError_t e = launch_fill_mask(a.mask, T * nb, s);
            if (e != hipSuccess) return e;
        }
    } else {
        if (nch % (256 * 2) == 0)
            xlaunch(a.events, 0, k_pred1<E, 2, true>, dim3((unsigned)(T * a.rank)), dim3(256), 0, s, x,
                    static_cast<const E*>(a.A), a.z, a.d, a.rank, rb);
        else
            xlaunch(a.events, 0, k_pred1<E, 2, false>, dim3((unsigned)(T * a.rank)), dim3(256), 0, s, x,
                    static_cast<const E*>(a.A), a.z, a.d, a.rank, rb);
        if constexpr (sizeof(E) == 2) {
            if (fused_ok(a)) {
                xlaunch(a.events, 1, k_bank_fused<16>, dim3((unsigned)(T * nb)), dim3(64 * 16), 0, s, x, a.z,
                        static_cast<const E*>(a.B), a.bias, static_cast<const E*>(a.W_g),
                        static_cast<const E*>(a.W_u), static_cast<const E*>(a.W_dT), a.rank, a.d_i,
                        a.gate, a.mask, a.logits, a.partial);
                const int col_blocks = (a.d + 31) / 32;
                xlaunch(a.events, 2, k_reduce<E>, dim3((unsigned)(T * col_blocks)), dim3(32 * kReduceParts), 0, s,
                        a.partial, static_cast<E*>(a.y), a.d, nb, col_blocks);
                skip_stages(a.events, 3, s);
                return hipGetLastError();
            }
        }
        xlaunch(a.events, 1, k_pred2_topk<E>, dim3((unsigned)(T * nb)), dim3(256), 0, s, a.z,
                static_cast<const E*>(a.B), a.bias, a.rank, a.d_i, a.keep, a.mask, a.logits, a.ids,
                a.pk);
    }
    {
        const int64_t n = T * d_s;
        const dim3 grid((unsigned)((n + 3) / 4));
        if (nch % (64 * NC) == 0)
            xlaunch(a.events, 2, k_gateup<E, NC, true>, grid, dim3(256), 0, s, x,
                    static_cast<const E*>(a.W_g), static_cast<const E*>(a.W_u), ids, a.pk, a.h,
                    a.d, d_s, n, a.gate);
        else
            xlaunch(a.events, 2, k_gateup<E, NC, false>, grid, dim3(256), 0, s, x,
                    static_cast<const E*>(a.W_g), static_cast<const E*>(a.W_u), ids, a.pk, a.h,
                    a.d, d_s, n, a.gate);
    }
    const int groups = gather_groups(d_s);
    const int slices = (a.d + kSlice - 1) / kSlice;
    {
        const dim3 grid((unsigned)(T * groups * slices));
        if (a.d % kSlice == 0 && d_s % kGroup == 0)
            xlaunch(a.events, 3, k_down<E, true>, grid, dim3(256), 0, s,
                    static_cast<const E*>(a.W_dT), ids, a.h, a.partial, a.d, d_s, groups, slices);
        else
            xlaunch(a.events, 3, k_down<E, false>, grid, dim3(256), 0, s,
                    static_cast<const E*>(a.W_dT), ids, a.h, a.partial, a.d, d_s, groups, slices);
    }
    {
        const int col_blocks = (a.d + 31) / 32;
        xlaunch(a.events, 4, k_reduce<E>, dim3((unsigned)(T * col_blocks)), dim3(32 * kReduceParts), 0, s,
                a.partial, static_cast<E*>(a.y), a.d, groups, col_blocks);
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
// dst[c][r] = src[r][c] with dst rows of ld >= rows entries; entries
// r in [rows, ld) are written as zero (K padding of a transposed operand)
template <typename E>
__global__ __launch_bounds__(256) void k_transpose(const E* __restrict__ src, E* __restrict__ dst,
                                                   int rows, int cols, int ld) {
    __shared__ E tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4) {
        const int gr = r0 + r, gc = c0 + tx;
        tile[r][tx] = (gr < rows && gc < cols) ? src[(int64_t)gr * cols + gc] : E(0);
    }
    __syncthreads();
    for (int c = ty; c < 64; c += 4) {
        const int gc = c0 + c, gr = r0 + tx;
        if (gc < cols && gr < ld) dst[(int64_t)gc * ld + gr] = tile[tx][c];
    }
}

// The same for bf16 with 16-byte global accesses (cols and ld multiples of 8,
// 16-byte aligned pointers): a thread moves 8 consecutive elements of a
// source row into LDS and later gathers 8 rows of one column from it.
__global__ __launch_bounds__(256) void k_transpose16(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
                                                     int rows, int cols, int ld) {
    constexpr int P = 64 + 2;                        // row pitch (elements): 132 bytes
    __shared__ __attribute__((aligned(16))) uint16_t tile[64 * P];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = threadIdx.x + 256 * k, r = q >> 3, cc = 8 * (q & 7);
        const int gr = r0 + r, gc = c0 + cc;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (gr < rows && gc < cols) v = *reinterpret_cast<const uint4*>(src + (int64_t)gr * cols + gc);
        uint32_t* t32 = reinterpret_cast<uint32_t*>(tile + r * P + cc);
        t32[0] = v.x; t32[1] = v.y; t32[2] = v.z; t32[3] = v.w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int q = threadIdx.x + 256 * k, c = q >> 3, rr = 8 * (q & 7);
        const int gc = c0 + c, gr = r0 + rr;
        if (gc >= cols || gr >= ld) continue;
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = tile[(rr + i) * P + c];
        *reinterpret_cast<uint4*>(dst + (int64_t)gc * ld + gr) =
            make_uint4((uint32_t)e[0] | ((uint32_t)e[1] << 16), (uint32_t)e[2] | ((uint32_t)e[3] << 16),
                       (uint32_t)e[4] | ((uint32_t)e[5] << 16), (uint32_t)e[6] | ((uint32_t)e[7] << 16));
    }
}

hipError_t launch_transpose(Dt dt, const void* src, void* dst, int rows, int cols, hipStream_t s, int ld) {
    if (ld < rows) ld = rows;
    dim3 grid((cols + 63) / 64, (ld + 63) / 64);
    const bool wide = dt == Dt::BF16 && cols % 8 == 0 && ld % 8 == 0 &&
                      (reinterpret_cast<uintptr_t>(src) & 15) == 0 && (reinterpret_cast<uintptr_t>(dst) & 15) == 0;
    if (wide)
        hipLaunchKernelGGL(k_transpose16, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src),
                           static_cast<uint16_t*>(dst), rows, cols, ld);
    else if (dt == Dt::BF16)
        hipLaunchKernelGGL(k_transpose<uint16_t>, grid, dim3(256), 0, s,
                           static_cast<const uint16_t*>(src), static_cast<uint16_t*>(dst), rows, cols, ld);
    else
        hipLaunchKernelGGL(k_transpose<float>, grid, dim3(256), 0, s,
                           static_cast<const float*>(src), static_cast<float*>(dst), rows, cols, ld);
    return hipGetLastError();
}

}  // namespace sffn
