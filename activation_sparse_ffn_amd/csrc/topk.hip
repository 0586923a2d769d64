// Standalone bank-wise hard top-k: one wave64 per (token, bank), one logit
// per lane. The rule is the bank top-k of "Continual LLM Upcycling"
// (gist.science technical summary, Methodologie > 1. Architectuur): the
// intermediate width is split into fixed banks of 64 channels and a hard
// top-k keeps `keep` channels of each bank.
#include <algorithm>
#include <utility>

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
                                                   uint16_t* __restrict__ ids, int nb) {
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
    }
}

// Many banks: one bank per lane. Each wave is a workgroup of its own and
// walks chunks of 64 consecutive (token, bank) words (16 KB), chunk c, c +
// n_waves, ...: a chunk's logits go from global memory straight into the
// wave's 16 KB LDS buffer (buffer loads to LDS, non-temporal, whole-line
// reads; 16-byte pieces XOR-swizzled by bank so that each lane reads its
// own bank without LDS bank conflicts). The wave copies its chunk into
// registers, starts the next chunk's loads into the freed buffer at once,
// and ranks from registers while they are in flight; with two such waves
// per SIMD the loads of one overlap the ranking of the other as well. Each
// lane sorts its 64 order-preserving keys with sorting networks held in
// registers (max/min pairs, no branches), takes the keep-th largest key as
// the threshold, and rebuilds the mask in channel order: keys above the
// threshold are kept, keys equal to it are kept lowest channel first until
// `keep` are taken -- the same rule as wave_bank_topk.
typedef float f4v __attribute__((ext_vector_type(4)));
// Sixteen 16-byte LDS reads, complete when the block ends. Written as one
// asm block so that the compiler's conservative wait before LDS reads that
// follow LDS-bound loads does not stall on the next chunk's loads; the
// caller orders the reads after an explicit wait for the chunk.
__device__ __forceinline__ void lds_read16(const uint32_t (&a)[16], f4v (&v)[16]) {
    asm volatile(
        "ds_read_b128 %0, %16\n\tds_read_b128 %1, %17\n\tds_read_b128 %2, %18\n\tds_read_b128 %3, %19\n\t"
        "ds_read_b128 %4, %20\n\tds_read_b128 %5, %21\n\tds_read_b128 %6, %22\n\tds_read_b128 %7, %23\n\t"
        "ds_read_b128 %8, %24\n\tds_read_b128 %9, %25\n\tds_read_b128 %10, %26\n\tds_read_b128 %11, %27\n\t"
        "ds_read_b128 %12, %28\n\tds_read_b128 %13, %29\n\tds_read_b128 %14, %30\n\tds_read_b128 %15, %31\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7]),
          "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]), "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
          "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]), "v"(a[15])
        : "memory");
}
// The lane's whole 256-byte word, piece c in v[c]; `key` is the word's LDS
// address with the lane's swizzle (bank % 16) * 16 or-ed in.
__device__ __forceinline__ void read_word(uint32_t key, f4v (&v)[16]) {
    asm volatile("" : "+v"(key));  // keep the 16 addresses out of the loop's live set
    uint32_t a[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) a[c] = key ^ (uint32_t)(c << 4);
    lds_read16(a, v);
}
// The 16 loads of one chunk, instruction Q = 4 a + r. The immediate offset
// moves both the source and the LDS destination, so the LDS base steps by
// 4096 only. Full chunks take the 4096 a part as the scalar offset; the
// last, partial chunk puts it in the lane offset, where the range check of
// the resource sees it, and its loads past the logits' end read zeros.
template <int... Q>
__device__ __forceinline__ void chunk_loads(__amdgpu_buffer_rsrc_t rs, __attribute__((address_space(3))) char* d3,
                                            const uint32_t (&voff)[4], bool full, std::integer_sequence<int, Q...>) {
    constexpr int kNonTemporal = 2;
    if (full)
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d3 + 4096 * (Q >> 2), 16, voff[Q & 3], 4096 * (Q >> 2),
                                                  1024 * (Q & 3), kNonTemporal),
         ...);
    else
        (__builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d3 + 4096 * (Q >> 2), 16, voff[Q & 3] + 4096 * (Q >> 2), 0,
                                                  1024 * (Q & 3), kNonTemporal),
         ...);
}
constexpr uint32_t kRawBufferWord3 = 0x00020000;  // 32-bit data format, untyped byte-addressed access
constexpr int kTopkLanesWaves = 8;  // two waves per SIMD: <= 256 registers and 16 KB of LDS each
__global__ __launch_bounds__(64) void k_bank_topk_lanes(const float* __restrict__ logits,
                                                        int64_t n_words, int keep,
                                                        uint64_t* __restrict__ mask,
                                                        uint16_t* __restrict__ ids, int nb) {
    __shared__ __attribute__((aligned(16))) char st0[kWave * kBank * 4];
    const int lane = threadIdx.x;
    const int64_t n_chunks = (n_words + kWave - 1) / kWave;
    const int64_t stride = gridDim.x;
    // Instruction q (q = 4 a + r) fills bytes [1024 q, 1024 q + 1024) of the
    // buffer: lane l lands in word L = 4 q + l / 16, slot l % 16, which holds
    // chunk (l % 16) ^ (L % 16) of that word. L % 16 = 4 r + l / 16, so the
    // lane's source offset is 4096 a + 1024 r + voff[r].
    uint32_t voff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        voff[r] = (uint32_t)((lane >> 4) * 256 + 16 * ((lane & 15) ^ (4 * r + (lane >> 4))));
    auto fetch = [&](int64_t ch, char* dst) {
        const int64_t w0 = ch * kWave;
        const int64_t left = n_words - w0;
        void* base = (void*)(logits + w0 * kBank);
        auto* d3 = (__attribute__((address_space(3))) char*)dst;
        const bool full = left >= kWave;
        const int nbytes = full ? kWave * kBank * 4 : (int)left * kBank * 4;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, kRawBufferWord3);
        chunk_loads(rs, d3, voff, full, std::make_integer_sequence<int, 16>{});
    };
    auto rank = [&](int64_t ch, const char* stb) {
        const int64_t gw = ch * kWave + lane;              // this lane's word
        const uint32_t key = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)stb + lane * 256 +
                             ((lane & 15) << 4);
        f4v buf[16];
        read_word(key, buf);
        if (ch + stride < n_chunks) fetch(ch + stride, st0);   // the buffer is free again
        const uint64_t sel = lane_select64(
            [&](int c) { return make_float4(buf[c].x, buf[c].y, buf[c].z, buf[c].w); }, keep);
        if (gw >= n_words) return;
        mask[gw] = sel;
        if (ids != nullptr) {
            const int b = (int)(gw % nb);
            int slot = 0;
#pragma unroll
            for (int i = 0; i < kBank; ++i)
                if ((sel >> i) & 1ull) ids[gw * keep + slot++] = (uint16_t)(b * kBank + i);
        }
    };
    // One wave per workgroup: the reads of a chunk complete inside
    // read_word, before the loads that overwrite the buffer are issued;
    // s_waitcnt(0) makes the chunk's loads (and the previous chunk's stores)
    // complete before it is read.
    if ((int64_t)blockIdx.x < n_chunks) fetch(blockIdx.x, st0);
    for (int64_t ch = blockIdx.x; ch < n_chunks; ch += stride) {
        __builtin_amdgcn_s_waitcnt(0);
        rank(ch, st0);
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

hipError_t launch_bank_topk(const float* logits, int64_t T, int d_i, int keep,
                            uint64_t* mask, uint16_t* ids, hipStream_t s, void* const* events,
                            int stage) {
    const int nb = d_i / kBank;
    const int64_t n_words = T * nb;
    if (n_words >= 65536) {
        const int n_cu = compute_units();
        const int64_t chunks = (n_words + kWave - 1) / kWave;
        const int64_t waves = std::min<int64_t>(chunks, (int64_t)n_cu * kTopkLanesWaves);
        xlaunch(events, stage, k_bank_topk_lanes, dim3((unsigned)waves), dim3(kWave), 0, s, logits,
                n_words, keep, mask, ids, nb);
    } else {
        const int64_t blocks = (n_words + 3) / 4;
        xlaunch(events, stage, k_bank_topk<1>, dim3((unsigned)blocks), dim3(256), 0, s, logits,
                n_words, keep, mask, ids, nb);
    }
    return hipGetLastError();
}

}  // namespace sffn
