// Standalone bank-wise hard top-k: one wave64 per (token, bank), one logit
// per lane. The rule is the bank top-k of "Continual LLM Upcycling"
// (gist.science technical summary, Methodologie > 1. Architectuur): the
// intermediate width is split into fixed banks of 64 channels and a hard
// top-k keeps `keep` channels of each bank.
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

// Each wave takes BPW consecutive (token, bank) words and requests all of
// their logits before the first selection, so the load latency is paid once
// per BPW banks.
template <int BPW>
__global__ __launch_bounds__(256) void k_bank_topk(const float* __restrict__ logits,
                                                   int64_t n_words, int keep,
                                                   uint64_t* __restrict__ mask,
                                                   uint16_t* __restrict__ ids, int nb,
                                                   uint16_t* __restrict__ gate, int gate_mode) {
    const int lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) * BPW;
    float v[BPW];
#pragma unroll
    for (int i = 0; i < BPW; ++i)
        v[i] = (w0 + i < n_words) ? logits[(w0 + i) * kBank + lane] : 0.f;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
        const int64_t gb = w0 + i;                  // (token, bank), wave-uniform
        if (gb >= n_words) break;
        const uint64_t sel = wave_bank_topk(rank_key(v[i]), keep);
        if (lane == 0) mask[gb] = sel;
        const bool kept = (sel >> lane) & 1ull;
        if (ids != nullptr && kept) {
            const int b = (int)(gb % nb);
            ids[gb * keep + lanes_below(sel)] = (uint16_t)(b * kBank + lane);
        }
        if (gate != nullptr) {
            const unsigned t = (unsigned)gb / (unsigned)nb;
            const unsigned j = ((unsigned)gb - t * (unsigned)nb) * kBank + lane;
            const unsigned col_tiles = (unsigned)nb * kBank / kGateTileCols;
            const size_t o = ((size_t)(t / kGateTileRows) * col_tiles + j / kGateTileCols) *
                                 (kGateTileRows * kGateTileCols) +
                             (t % kGateTileRows) * kGateTileCols + j % kGateTileCols;
            const float g = gate_mode ? 1.f : sigmoidf_dev(v[i]);
            gate[o] = kept ? __builtin_bit_cast(uint16_t, (_Float16)g) : kGateDropped;
        }
    }
}

// The 16th largest of 64 keys: sort four groups of 16 (descending bitonic
// networks), merge them pairwise keeping the top 16 (max against the other
// group reversed gives a bitonic sequence holding the top 16, which a
// half-cleaner network sorts), and at the last level only the minimum of the
// kept 16 is needed.
__device__ __forceinline__ void sort16_desc(uint32_t* a) {
#pragma unroll
    for (int sz = 2; sz <= 16; sz <<= 1)
#pragma unroll
        for (int j = sz >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const uint32_t x = a[i], y = a[l];
                    const bool desc = (i & sz) == 0;
                    a[i] = desc ? max(x, y) : min(x, y);
                    a[l] = desc ? min(x, y) : max(x, y);
                }
            }
}
// a, b sorted descending -> a holds the top 16 of both, sorted descending
__device__ __forceinline__ void merge_top16(uint32_t* a, const uint32_t* b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = max(a[i], b[15 - i]);
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
                const uint32_t x = a[i], y = a[l];
                a[i] = max(x, y);
                a[l] = min(x, y);
            }
        }
}
__device__ __forceinline__ uint32_t kth16(uint32_t (&k)[kBank]) {
    sort16_desc(k);
    sort16_desc(k + 16);
    sort16_desc(k + 32);
    sort16_desc(k + 48);
    merge_top16(k, k + 16);
    merge_top16(k + 32, k + 48);
    uint32_t t = max(k[0], k[47]);
#pragma unroll
    for (int i = 1; i < 16; ++i) t = min(t, max(k[i], k[47 - i]));
    return t;
}

// Many banks: one bank per lane. A wave stages the logits of 64 consecutive
// (token, bank) words (16 KB, read with whole-line loads) in wave-private LDS,
// 16-byte chunks XOR-swizzled by bank so that each lane can read its own bank
// without bank conflicts. Each lane sorts its 64 order-preserving keys with a
// bitonic network held in registers (max/min pairs, no branches), takes the
// keep-th largest key as the threshold, and rebuilds the mask in channel
// order: keys above the threshold are kept, keys equal to it are kept lowest
// channel first until `keep` are taken -- the same rule as wave_bank_topk.
__global__ __launch_bounds__(256) void k_bank_topk_lanes(const float* __restrict__ logits,
                                                         int64_t n_words, int keep,
                                                         uint64_t* __restrict__ mask,
                                                         uint16_t* __restrict__ ids, int nb,
                                                         uint16_t* __restrict__ gate,
                                                         int gate_mode) {
    __shared__ __attribute__((aligned(16))) float stage[4][kWave * kBank];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + wv) * kWave;      // first word of this wave
    float* st = stage[wv];
    char* stb = reinterpret_cast<char*>(st);

    // coalesced fetch: instruction q, lane l -> word q * 4 + l / 16, chunk l % 16
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int L = q * 4 + (lane >> 4), c = lane & 15;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (w0 + L < n_words) val = *reinterpret_cast<const float4*>(logits + (w0 + L) * kBank + 4 * c);
        *reinterpret_cast<float4*>(stb + L * 256 + ((c ^ (L & 15)) << 4)) = val;
    }
    const int64_t gw = w0 + lane;                  // this lane's word
    const bool live = gw < n_words;

    uint32_t k[kBank];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float4 val = *reinterpret_cast<const float4*>(stb + lane * 256 + ((c ^ (lane & 15)) << 4));
        k[4 * c + 0] = rank_key(val.x);
        k[4 * c + 1] = rank_key(val.y);
        k[4 * c + 2] = rank_key(val.z);
        k[4 * c + 3] = rank_key(val.w);
    }
    uint32_t thr;
    if (keep == 16) {
        thr = kth16(k);
    } else {
        // bitonic sort, descending
#pragma unroll
        for (int sz = 2; sz <= kBank; sz <<= 1)
#pragma unroll
            for (int j = sz >> 1; j > 0; j >>= 1)
#pragma unroll
                for (int i = 0; i < kBank; ++i) {
                    const int l = i ^ j;
                    if (l > i) {
                        const uint32_t a = k[i], b = k[l];
                        const bool desc = (i & sz) == 0;
                        k[i] = desc ? max(a, b) : min(a, b);
                        k[l] = desc ? min(a, b) : max(a, b);
                    }
                }
        thr = k[0];
#pragma unroll
        for (int i = 1; i < kBank; ++i) thr = (i == keep - 1) ? k[i] : thr;
    }

    // mask in channel order, comparing the logits against the threshold as
    // floats: -0 == +0 and NaN fails every compare, as under the keys; a
    // threshold key of 0 means the threshold lies among the NaNs
    const bool nan_thr = thr == 0u;
    const float thr_f = __uint_as_float((thr & 0x80000000u) ? (thr & 0x7fffffffu) : ~thr);
    float fv[kBank];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float4 val = *reinterpret_cast<const float4*>(stb + lane * 256 + ((c ^ (lane & 15)) << 4));
        fv[4 * c + 0] = val.x;
        fv[4 * c + 1] = val.y;
        fv[4 * c + 2] = val.z;
        fv[4 * c + 3] = val.w;
    }
    int n_gt = 0;
#pragma unroll
    for (int i = 0; i < kBank; ++i) n_gt += nan_thr ? !__builtin_isnan(fv[i]) : fv[i] > thr_f;
    const int need = keep - n_gt;
    int taken = 0;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < kBank; ++i) {
        const bool gt = nan_thr ? !__builtin_isnan(fv[i]) : fv[i] > thr_f;
        const bool eq = nan_thr ? __builtin_isnan(fv[i]) : fv[i] == thr_f;
        const bool eq_take = eq && taken < need;
        taken += eq_take;
        const uint32_t bit = (gt || eq_take) ? 1u : 0u;
        if (i < 32) lo |= bit << i; else hi |= bit << (i - 32);
    }
    const uint64_t sel = ((uint64_t)hi << 32) | lo;
    if (!live) return;
    mask[gw] = sel;
    const unsigned t = (unsigned)gw / (unsigned)nb;
    const unsigned b = (unsigned)gw - t * (unsigned)nb;
    if (ids != nullptr) {
        int slot = 0;
#pragma unroll
        for (int i = 0; i < kBank; ++i)
            if ((sel >> i) & 1ull) ids[gw * keep + slot++] = (uint16_t)(b * kBank + i);
    }
    if (gate != nullptr) {
        const unsigned col_tiles = (unsigned)nb * kBank / kGateTileCols;
        const unsigned j0 = b * kBank;
        uint16_t* gp = gate + ((size_t)(t / kGateTileRows) * col_tiles + j0 / kGateTileCols) *
                                  (kGateTileRows * kGateTileCols) +
                       (t % kGateTileRows) * kGateTileCols + j0 % kGateTileCols;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float4 v0 = *reinterpret_cast<const float4*>(stb + lane * 256 + (((2 * c) ^ (lane & 15)) << 4));
            const float4 v1 = *reinterpret_cast<const float4*>(stb + lane * 256 + (((2 * c + 1) ^ (lane & 15)) << 4));
            const float pv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t hw[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint16_t h2[2];
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const int i = 8 * c + 2 * e + q;
                    const float g = gate_mode ? 1.f : sigmoidf_dev(pv[2 * e + q]);
                    h2[q] = ((sel >> i) & 1ull) ? __builtin_bit_cast(uint16_t, (_Float16)g) : kGateDropped;
                }
                hw[e] = (uint32_t)h2[0] | ((uint32_t)h2[1] << 16);
            }
            *reinterpret_cast<uint4*>(gp + 8 * c) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        }
    }
}

size_t gate_tiles_bytes(int64_t T, int d_i) {
    return (size_t)((T + kGateTileRows - 1) / kGateTileRows) * kGateTileRows * d_i * 2;
}

hipError_t launch_bank_topk(const float* logits, int64_t T, int d_i, int keep,
                            uint64_t* mask, uint16_t* ids, hipStream_t s, void* const* events,
                            int stage, uint16_t* gate_tiles, int gate_mode) {
    const int nb = d_i / kBank;
    const int64_t n_words = T * nb;
    if (n_words >= 65536) {
        const int64_t blocks = (n_words + 4 * kWave - 1) / (4 * kWave);
        xlaunch(events, stage, k_bank_topk_lanes, dim3((unsigned)blocks), dim3(256), 0, s, logits,
                n_words, keep, mask, ids, nb, gate_tiles, gate_mode);
    } else {
        const int64_t blocks = (n_words + 3) / 4;
        xlaunch(events, stage, k_bank_topk<1>, dim3((unsigned)blocks), dim3(256), 0, s, logits,
                n_words, keep, mask, ids, nb, gate_tiles, gate_mode);
    }
    return hipGetLastError();
}

}  // namespace sffn
