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

size_t gate_tiles_bytes(int64_t T, int d_i) {
    return (size_t)((T + kGateTileRows - 1) / kGateTileRows) * kGateTileRows * d_i * 2;
}

hipError_t launch_bank_topk(const float* logits, int64_t T, int d_i, int keep,
                            uint64_t* mask, uint16_t* ids, hipStream_t s, void* const* events,
                            int stage, uint16_t* gate_tiles, int gate_mode) {
    const int nb = d_i / kBank;
    const int64_t n_words = T * nb;
    if (n_words >= 65536) {
        constexpr int BPW = 8;
        const int64_t blocks = (n_words + 4 * BPW - 1) / (4 * BPW);
        xlaunch(events, stage, k_bank_topk<BPW>, dim3((unsigned)blocks), dim3(256), 0, s, logits,
                n_words, keep, mask, ids, nb, gate_tiles, gate_mode);
    } else {
        const int64_t blocks = (n_words + 3) / 4;
        xlaunch(events, stage, k_bank_topk<1>, dim3((unsigned)blocks), dim3(256), 0, s, logits,
                n_words, keep, mask, ids, nb, gate_tiles, gate_mode);
    }
    return hipGetLastError();
}

}  // namespace sffn
