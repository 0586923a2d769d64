// Shared device helpers of the sparse FFN kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sffn {

constexpr int kWave = 64;
constexpr int kBank = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------------------
// bf16 <-> fp32
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest even; NaN becomes the quiet NaN 0x7fc0.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------------------
// 8-element chunks: one 16-byte load for bf16, two for fp32
// ---------------------------------------------------------------------------

struct Chunk8 { float v[8]; };

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ void load8(const uint16_t* p, float* o) {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x);
        o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
        o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z);
        o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
    }
    static __device__ __forceinline__ void store1(uint16_t* p, float v) { *p = f32_to_bf16(v); }
};
template <> struct Elem<float> {
    static __device__ __forceinline__ void load8(const float* p, float* o) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
    static __device__ __forceinline__ void store1(float* p, float v) { *p = v; }
};

// Raw 16-byte words, loaded early and decoded later so that many loads are
// in flight before the first use.
template <typename T> struct Raw;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <> struct Raw<uint16_t> {
    uint4 w;
    __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
    // streaming load (nt): for data read once, so that it does not push
    // reusable lines out of the caches
    __device__ __forceinline__ void load_stream(const uint16_t* p) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        w = make_uint4(v.x, v.y, v.z, v.w);
    }
    __device__ __forceinline__ void decode(float* o) const {
        o[0] = bf16_lo(w.x); o[1] = bf16_hi(w.x);
        o[2] = bf16_lo(w.y); o[3] = bf16_hi(w.y);
        o[4] = bf16_lo(w.z); o[5] = bf16_hi(w.z);
        o[6] = bf16_lo(w.w); o[7] = bf16_hi(w.w);
    }
};
template <> struct Raw<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void decode(float* o) const {
        o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
        o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
    }
};

// ---------------------------------------------------------------------------
// K-major operands: fragments of v_mfma_f32_32x32x16_bf16 from a [K][N] tile
// ---------------------------------------------------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// An LDS slab of 64 K-rows of ROW_BYTES bytes (N contiguous, bf16), whose
// 16-byte chunk c of K-row r sits at slot kmajor_slot<ROW_BYTES>(r, c):
// c ^ (4 (r & 3)) for rows of 256 bytes or more, c ^ (4 ((r >> 1) & 1)) for
// 128-byte rows (eight chunks). The MFMA wants
// eight consecutive K of one column per lane (lane l: column col0 + l % 32,
// K 16 s + 8 (l >> 5) .. + 7). ds_read_b64_tr_b16 gathers that from rows:
// within each group of 16 lanes, lane i names the 8 bytes at K-row
// k + (i >> 2), columns n + 4 (i & 3) .. + 3, and lane j receives element
// j & 3 of the reads of lanes (j >> 2) + 4 e, e = 0..3, i.e. column n + j at
// K-rows k .. k + 3. Two such reads (K-rows + 0 and + 4) give the fragment.
// A group's 16 addresses cover 4 K-rows x 32 bytes; the swizzle puts the 4
// rows on disjoint LDS banks.
template <int ROW_BYTES>
__device__ __forceinline__ int kmajor_slot(int r, int c) {
    static_assert(ROW_BYTES == 128 || ROW_BYTES % 256 == 0, "rows of 128 bytes or whole 256-byte windows");
    return ROW_BYTES == 128 ? c ^ (4 * ((r >> 1) & 1)) : c ^ (4 * (r & 3));
}
template <int ROW_BYTES>
__device__ __forceinline__ bf16x8 kmajor_frag(const char* slab, int col0, int s, int lane) {
    const int i16 = lane & 15, g = lane >> 4;
    const int col = col0 + 16 * (g & 1) + 4 * (i16 & 3);
    const int kr = 16 * s + 8 * (g >> 1) + (i16 >> 2);
    // the slot depends on kr & 3 only, which K-row kr + 4 shares
    const int off = (kmajor_slot<ROW_BYTES>(kr, col >> 3) << 4) + (col & 7) * 2;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(slab + kr * ROW_BYTES + off));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(slab + (kr + 4) * ROW_BYTES + off));
    const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------------------
// wave reductions
// ---------------------------------------------------------------------------

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// 1 / (1 + e^-a) with the hardware reciprocal (1 ulp) instead of an IEEE
// division: the division sequence cost ~12 instructions per value in the
// top-k epilogue, which writes a sigmoid for every channel of the chunk.
// a = -inf gives rcp(inf) = 0, a = +inf gives 1, NaN stays NaN.
__device__ __forceinline__ float sigmoidf_dev(float a) { return __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

// Sum of `splits` K-split partials p[0], p[n], p[2 n], ... in that order.
// The loads of a group of 8 are all issued before its first add, so a
// thread waits for memory once per group instead of once per split.
__device__ __forceinline__ float sum_splits_in_order(const float* __restrict__ p, int splits, int64_t n) {
    constexpr int G = 8;
    float acc = 0.f;
    for (int s0 = 0; s0 < splits; s0 += G) {
        float v[G];
#pragma unroll
        for (int k = 0; k < G; ++k) v[k] = s0 + k < splits ? p[(size_t)(s0 + k) * n] : 0.f;
#pragma unroll
        for (int k = 0; k < G; ++k)
            if (s0 + k < splits) acc += v[k];
    }
    return acc;
}

// Order-preserving 32-bit key of a logit: larger value <=> larger key.
// -0 and +0 share a key; every NaN gets key 0, below -inf (0x007fffff).
__device__ __forceinline__ uint32_t rank_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if ((u & 0x7fffffffu) == 0u) return 0x80000000u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Bank-wise hard top-k of one 64-channel bank held one logit per lane.
// Returns the wave-uniform mask of the `keep` largest keys, equal keys taken
// lowest lane first. MSB-first radix search for the keep-th largest key,
// stopping as soon as the candidate prefix isolates exactly `keep` lanes.
__device__ __forceinline__ uint64_t wave_bank_topk(uint32_t key, int keep) {
    if (keep >= kBank) return ~0ull;
    uint32_t prefix = 0u;
#pragma unroll 1
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = prefix | (1u << bit);
        const uint64_t ge = __ballot(key >= cand);
        const int c = __popcll(ge);
        if (c >= keep) {
            prefix = cand;
            if (c == keep) return ge;
        }
    }
    // prefix is now the keep-th largest key; split its ties by lane
    const uint64_t gt = __ballot(key > prefix);
    const uint64_t eq = __ballot(key == prefix);
    const int need = keep - __popcll(gt);
    const bool take = (key == prefix) && ((int)lanes_below(eq) < need);
    return gt | __ballot(take);
}

// The 16th largest of 64 values: sort four groups of 16 (Batcher's odd-even
// merge sort, 63 compare-exchanges per group against 80 for a bitonic
// network), merge them pairwise keeping the top 16 (max against the other
// group reversed gives a bitonic sequence holding the top 16, which a
// half-cleaner network sorts), and at the last level only the minimum of the
// kept 16 is needed. The values hold no NaN, so max/min are plain compares.
__device__ __forceinline__ void sort16_desc(float* a) {
#pragma unroll
    for (int p = 1; p < 16; p <<= 1)
#pragma unroll
        for (int k = p; k >= 1; k >>= 1)
#pragma unroll
            for (int j = k % p; j + k < 16; j += 2 * k)
#pragma unroll
                for (int i = 0; i < k; ++i)
                    if (i + j + k < 16 && (i + j) / (2 * p) == (i + j + k) / (2 * p)) {
                        const float x = a[i + j], y = a[i + j + k];
                        a[i + j] = fmaxf(x, y);
                        a[i + j + k] = fminf(x, y);
                    }
}
// a, b sorted descending -> a holds the top 16 of both, sorted descending
__device__ __forceinline__ void merge_top16(float* a, const float* b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = fmaxf(a[i], b[15 - i]);
#pragma unroll
    for (int j = 8; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int l = i ^ j;
            if (l > i) {
                const float x = a[i], y = a[l];
                a[i] = fmaxf(x, y);
                a[l] = fminf(x, y);
            }
        }
}
__device__ __forceinline__ float kth16(float (&k)[kBank]) {
    sort16_desc(k);
    sort16_desc(k + 16);
    sort16_desc(k + 32);
    sort16_desc(k + 48);
    merge_top16(k, k + 16);
    merge_top16(k + 32, k + 48);
    float t = fmaxf(k[0], k[47]);
#pragma unroll
    for (int i = 1; i < 16; ++i) t = fminf(t, fmaxf(k[i], k[47 - i]));
    return t;
}

// The n lowest set bits of x.
__device__ __forceinline__ uint64_t lowest_bits(uint64_t x, int n) {
    uint64_t r = 0;
    for (int i = 0; i < n && x != 0; ++i) {
        const uint64_t b = x & (~x + 1);
        r |= b;
        x ^= b;
    }
    return r;
}

// Bit i of the result is (v[i] >= t) (GE) or (v[i] > t) for i < 32, false
// for NaN as in C. Each element costs one compare into VCC and one
// add-with-carry that shifts the word left and brings the compare in, i.e.
// acc = 2 acc + (compare); v[31] is taken first so that it ends in bit 31.
template <bool GE>
__device__ __forceinline__ uint32_t cmp_bits32(const float* v, float t) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 31; i >= 0; --i) {
        if constexpr (GE)
            asm("v_cmp_ge_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                : "+v"(acc) : "v"(v[i]), "v"(t) : "vcc");
        else
            asm("v_cmp_gt_f32 vcc, %1, %2\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
                : "+v"(acc) : "v"(v[i]), "v"(t) : "vcc");
    }
    return acc;
}

// Keep mask of one 64-channel bank held entirely by one lane. `load(c)`
// returns channels 4c .. 4c + 3 (c < 16) as a float4 and is called twice, so
// the logits need not stay in registers across the selection.
//
// The keep-th largest value is found by sorting networks over the logits
// with NaN mapped to -inf (fmaxf against -inf; -0 and +0 compare equal, as
// under the ranking order). The mask is then every channel whose logit
// compares >= that threshold. That set has exactly `keep` members unless
// logits tie at the threshold -- then the channels above it are kept and the
// tied ones lowest channel first -- or the threshold is -inf and NaNs are
// needed to reach `keep`; NaNs rank below -inf and are taken last, lowest
// channel first.
template <typename Load>
__device__ __forceinline__ uint64_t lane_select64(Load load, int keep) {
    if (keep >= kBank) return ~0ull;
    float k[kBank];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float4 val = load(c);
        k[4 * c + 0] = fmaxf(val.x, -__builtin_huge_valf());
        k[4 * c + 1] = fmaxf(val.y, -__builtin_huge_valf());
        k[4 * c + 2] = fmaxf(val.z, -__builtin_huge_valf());
        k[4 * c + 3] = fmaxf(val.w, -__builtin_huge_valf());
    }
    float thr;
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
                        const float a = k[i], b = k[l];
                        const bool desc = (i & sz) == 0;
                        k[i] = desc ? fmaxf(a, b) : fminf(a, b);
                        k[l] = desc ? fminf(a, b) : fmaxf(a, b);
                    }
                }
        thr = k[0];
#pragma unroll
        for (int i = 1; i < kBank; ++i) thr = (i == keep - 1) ? k[i] : thr;
    }
    // reload the logits rather than keep all 64 live across the sort
    // (a compiler-only memory barrier; no instruction)
    __asm__ __volatile__("" ::: "memory");
    float fv[kBank];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const float4 val = load(c);
        fv[4 * c + 0] = val.x;
        fv[4 * c + 1] = val.y;
        fv[4 * c + 2] = val.z;
        fv[4 * c + 3] = val.w;
    }
    const uint32_t lo = cmp_bits32<true>(fv, thr), hi = cmp_bits32<true>(fv + 32, thr);
    uint64_t sel = ((uint64_t)hi << 32) | lo;
    const int n_ge = __popcll(sel);
    if (n_ge == keep) return sel;
    if (n_ge > keep) {
        // ties at the threshold: everything above it, then the tied channels
        const uint32_t glo = cmp_bits32<false>(fv, thr), ghi = cmp_bits32<false>(fv + 32, thr);
        const uint64_t gt = ((uint64_t)ghi << 32) | glo;
        return gt | lowest_bits(sel & ~gt, keep - __popcll(gt));
    }
    // fewer than keep non-NaN logits: the NaNs fill up, lowest channel first
    uint32_t nlo = 0, nhi = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        nlo |= (uint32_t)__builtin_isnan(fv[i]) << i;
        nhi |= (uint32_t)__builtin_isnan(fv[32 + i]) << i;
    }
    return sel | lowest_bits(((uint64_t)nhi << 32) | nlo, keep - n_ge);
}

}  // namespace sffn
