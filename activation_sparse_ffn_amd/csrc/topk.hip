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

    const uint64_t sel = lane_select64(
        [stb, lane](int c) { return *reinterpret_cast<const float4*>(stb + lane * 256 + ((c ^ (lane & 15)) << 4)); },
        keep);
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

__global__ __launch_bounds__(256) void k_fill_mask(uint64_t* __restrict__ mask, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) mask[i] = ~0ull;
}

hipError_t launch_fill_mask(uint64_t* mask, int64_t n_words, hipStream_t s) {
    if (mask == nullptr || n_words <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_mask, dim3((unsigned)((n_words + 255) / 256)), dim3(256), 0, s, mask, n_words);
    return hipGetLastError();
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
