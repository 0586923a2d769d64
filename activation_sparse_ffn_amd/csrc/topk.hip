// Standalone bank-wise hard top-k: one wave64 per (token, bank), one logit
// per lane. The rule is the bank top-k of "Continual LLM Upcycling"
// (gist.science technical summary, Methodologie > 1. Architectuur): the
// intermediate width is split into fixed banks of 64 channels and a hard
// top-k keeps `keep` channels of each bank.
#include "common.hpp"
#include "launch.hpp"

namespace sffn {

__global__ __launch_bounds__(256) void k_bank_topk(const float* __restrict__ logits,
                                                   int64_t n_words, int keep,
                                                   uint64_t* __restrict__ mask,
                                                   uint16_t* __restrict__ ids, int nb) {
    const int lane = threadIdx.x & 63;
    const int64_t gb = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (token, bank)
    if (gb >= n_words) return;                                        // wave-uniform
    const float v = logits[gb * kBank + lane];
    const uint64_t sel = wave_bank_topk(rank_key(v), keep);
    if (lane == 0) mask[gb] = sel;
    if (ids != nullptr && ((sel >> lane) & 1ull)) {
        const int b = (int)(gb % nb);
        ids[gb * keep + lanes_below(sel)] = (uint16_t)(b * kBank + lane);
    }
}

hipError_t launch_bank_topk(const float* logits, int64_t T, int d_i, int keep,
                            uint64_t* mask, uint16_t* ids, hipStream_t s, void* const* events,
                            int stage) {
    const int nb = d_i / kBank;
    const int64_t n_words = T * nb;
    const int64_t blocks = (n_words + 3) / 4;
    xlaunch(events, stage, k_bank_topk, dim3((unsigned)blocks), dim3(256), 0, s, logits, n_words,
            keep, mask, ids, nb);
    return hipGetLastError();
}

}  // namespace sffn
