// C ABI of the sparse FFN library: argument checks, weight packing,
// workspace carving and the choice between the two execution paths.
//
//   token-gather path  fp32 layers, and bf16 batches of at most
//                      kGatherMaxTokens tokens: only kept rows are read
//   skinny MFMA path   bf16 batches of up to kSkinnyMaxTokens tokens: the
//                      weights stream once through register-fed MFMA with
//                      split K (the union of the batch's masks is nearly
//                      every channel)
//   MFMA path          larger bf16 batches: tiled dense-masked contraction on
//                      the matrix cores
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/sparse_ffn.h"
#include "launch.hpp"

namespace {

constexpr int64_t kGatherMaxTokens = 4;
constexpr int64_t kSkinnyMaxTokens = 64;
constexpr size_t kAlign = 256;
constexpr int64_t kMaxGrid = (int64_t)1 << 31;

thread_local std::string g_last_error;

sffn_status_t fail(sffn_status_t st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(sffn_dtype_t dt) { return dt == SFFN_BF16 ? 2 : 4; }

template <typename Enum>
int as_int(const Enum& e) {
    static_assert(sizeof(Enum) == sizeof(int), "enums of the C ABI are int-sized");
    int v;
    std::memcpy(&v, &e, sizeof v);
    return v;
}

sffn_status_t check_config(const sffn_config_t* c) {
    if (!c) return fail(SFFN_ERR_INVALID_ARG, "config is null");
    if (c->d <= 0 || c->d_i <= 0 || c->rank <= 0)
        return fail(SFFN_ERR_INVALID_ARG, "d, d_i and rank must be positive (got %d, %d, %d)",
                    c->d, c->d_i, c->rank);
    if (c->bank != 64) return fail(SFFN_ERR_UNSUPPORTED, "bank must be 64 (got %d)", c->bank);
    if (c->keep < 1 || c->keep > 64)
        return fail(SFFN_ERR_INVALID_ARG, "keep must lie in [1, 64] (got %d)", c->keep);
    if (c->d_i % 64 != 0 || c->d_i > 65536)
        return fail(SFFN_ERR_INVALID_ARG, "d_i must be a multiple of 64 and <= 65536 (got %d)", c->d_i);
    if (c->d % 64 != 0) return fail(SFFN_ERR_INVALID_ARG, "d must be a multiple of 64 (got %d)", c->d);
    if (c->rank % 32 != 0)
        return fail(SFFN_ERR_INVALID_ARG, "rank must be a multiple of 32 (got %d)", c->rank);
    // the enum fields come from C callers as plain ints: read them as ints
    // (an out-of-range value read as a C++ enum is undefined behaviour)
    const int dtype = as_int(c->dtype), gate = as_int(c->gate);
    if (dtype != SFFN_F32 && dtype != SFFN_BF16)
        return fail(SFFN_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (gate != SFFN_GATE_PREDICTOR && gate != SFFN_GATE_SILU && gate != SFFN_GATE_AMPLITUDE)
        return fail(SFFN_ERR_INVALID_ARG, "unknown gate %d", gate);
    if (c->flags & ~SFFN_FLAG_BACKWARD) return fail(SFFN_ERR_INVALID_ARG, "unknown flags 0x%x", c->flags);
    return SFFN_OK;
}

// The packed weights: A, B, W_g, W_u, W_d^T (the only copy of the down
// projection: decode gathers its rows, the MFMA paths read it K-major), the
// bias, and with SFFN_FLAG_BACKWARD W_g^T and W_u^T.
struct PackedLayout {
    size_t A, B, Wg, Wu, WdT, bias, WgT, WuT, total;   // WgT, WuT: SFFN_FLAG_BACKWARD only
};

PackedLayout packed_layout(const sffn_config_t& c) {
    const size_t e = elem_size(c.dtype);
    const size_t d = (size_t)c.d, di = (size_t)c.d_i, r = (size_t)c.rank;
    PackedLayout L{};
    size_t off = 0;
    L.A = off;    off += align_up(r * d * e);
    L.B = off;    off += align_up(di * r * e);
    L.Wg = off;   off += align_up(di * d * e);
    L.Wu = off;   off += align_up(di * d * e);
    L.WdT = off;  off += align_up(di * d * e);
    L.bias = off; off += align_up(di * 4);
    L.WgT = L.WuT = 0;
    if (c.flags & SFFN_FLAG_BACKWARD) {
        L.WgT = off; off += align_up(d * di * e);
        L.WuT = off; off += align_up(d * di * e);
    }
    L.total = off;
    return L;
}

bool use_gather(const sffn_config_t& c, int64_t T) {
    return c.dtype == SFFN_F32 || T <= kGatherMaxTokens;
}

struct WsGather {
    size_t z, ids, pk, h, partial, mask, amp, logits, total;
};
struct WsMfma {
    size_t z, logits, mask, h, partial, gate, zpart, unionw, total;
};

bool use_skinny(const sffn_config_t& c, int64_t T) {
    // (rank % 64 only matters for the predictor, which the amplitude gate has not)
    return !use_gather(c, T) && T <= kSkinnyMaxTokens && (c.rank % 64 == 0 || c.gate == SFFN_GATE_AMPLITUDE);
}

WsGather ws_gather(const sffn_config_t& c, int64_t T) {
    const size_t nb = c.d_i / 64, ds = nb * c.keep;
    // partial rows of y: one per group of 64 kept channels (generic path) or
    // one per bank (fused path); the larger count covers both
    const size_t groups = std::max((size_t)sffn::gather_groups((int)ds), nb);
    WsGather w{};
    size_t off = 0;
    w.z = off;       off += align_up((size_t)T * c.rank * 4);
    w.ids = off;     off += align_up((size_t)T * ds * 2);
    w.pk = off;      off += align_up((size_t)T * ds * 4);
    w.h = off;       off += align_up((size_t)T * ds * 4);
    w.partial = off; off += align_up((size_t)T * groups * c.d * 4);
    w.mask = off;    off += align_up((size_t)T * nb * 8);
    w.amp = off;
    if (c.gate == SFFN_GATE_AMPLITUDE) off += align_up((size_t)T * c.d_i * 4);
    w.logits = off;  // gather path writes logits only when asked
    w.total = off;
    return w;
}

WsMfma ws_mfma(const sffn_config_t& c, int64_t T) {
    const size_t nb = c.d_i / 64;
    WsMfma w{};
    size_t off = 0;
    w.z = off;      off += align_up((size_t)T * c.rank * 2);
    w.logits = off; off += align_up((size_t)T * c.d_i * 4);
    w.mask = off;   off += align_up((size_t)T * nb * 8);
    w.h = off;      off += align_up((size_t)T * c.d_i * 2);
    w.partial = off;
    if (use_skinny(c, T)) off += align_up(sffn::skinny_partial_floats(T, c.d, c.rank, c.d_i) * 4);
    w.gate = off;
    if (!use_skinny(c, T) && c.d_i % sffn::kGateTileCols == 0)
        off += align_up(sffn::gate_tiles_bytes(T, c.d_i, c.keep, as_int(c.gate)));
    w.zpart = off;
    const int zs = use_skinny(c, T) ? 1 : sffn::z_splits(T, c.d);
    if (zs > 1) off += align_up((size_t)zs * T * c.rank * 4);
    w.unionw = off;
    if (use_skinny(c, T)) off += align_up(nb * 8);
    w.total = off;
    return w;
}

// Token counts a forward accepts: every launch's grid must fit in 31 bits,
// and T is bounded first so that none of the size products can overflow.
constexpr int64_t kMaxTokens = (int64_t)1 << 30;
bool tokens_fit(const sffn_config_t& c, int64_t T) {
    if (T > kMaxTokens) return false;
    const int64_t nb = c.d_i / 64, ds = nb * c.keep;
    const int64_t biggest = std::max(T * (int64_t)c.d_i, T * ds * 2);
    return biggest / 4 < kMaxGrid && T * nb * 8 < kMaxGrid;
}
// the backward pass: T tokens padded to 64, transposed operands of T columns
constexpr int64_t kMaxBackwardTokens = (int64_t)1 << 24;

sffn_status_t hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return SFFN_OK;
    return fail(SFFN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

template <typename P>
P* at(void* base, size_t off) {
    return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

// ---- static scratch of sparse_ffn_forward_noalloc ----------------------------
// The workspace of a forward, for callers that cannot allocate: one array per
// GPU, allocated when the library's code object is loaded on that GPU and
// held until the process ends. 16 MiB covers every path of the full layer
// (d = 4096, d_i = 14336, rank 448) up to T = 64: the token-gather path needs
// 14.2 MiB at T = 4, the skinny MFMA path 9.4 MiB at T = 64.
constexpr size_t kScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of `scratch` on each GPU (the host-side name `scratch` is a
// stand-in, never a device address), asked once per device with that device
// current.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

sffn_status_t scratch_for_stream(hipStream_t s, void** out) {
    int dev = -1, cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_status(e, "hipGetDevice");
    dev = cur;
    if (s != nullptr) {
        hipDevice_t sd = 0;
        e = hipStreamGetDevice(s, &sd);
        if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
        dev = (int)sd;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SFFN_ERR_UNSUPPORTED, "device %d is beyond the %d the static scratch serves", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (dev != cur) {
            const hipError_t back = hipSetDevice(cur);
            if (e == hipSuccess) e = back;
        }
        if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & (kAlign - 1)) != 0)
            return fail(SFFN_ERR_HIP, "the static scratch of device %d has no usable address", dev);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return SFFN_OK;
}

}  // namespace

struct sffn_layer {
    sffn_config_t cfg;
    void* packed;
    PackedLayout L;
    bool has_bias;
    void* events[2 * sffn::kStages];
    bool profiling;
};

extern "C" {

size_t sparse_ffn_packed_size(const sffn_config_t* cfg) {
    if (check_config(cfg) != SFFN_OK) return 0;
    return packed_layout(*cfg).total;
}

sffn_status_t sparse_ffn_create(const sffn_config_t* cfg, const void* w_gate, const void* w_up,
                                const void* w_down, const void* pred_a, const void* pred_b,
                                const float* pred_bias, void* packed, size_t packed_bytes,
                                void* hip_stream, sffn_handle_t* out) {
    sffn_status_t st = check_config(cfg);
    if (st != SFFN_OK) return st;
    if (!out) return fail(SFFN_ERR_INVALID_ARG, "out is null");
    // the amplitude gate (Dense-4x baseline) has no predictor: pred_a and
    // pred_b may then be null (the packed predictor sections stay unset)
    const bool amp = cfg->gate == SFFN_GATE_AMPLITUDE;
    const void* ptrs[] = {w_gate, w_up, w_down, pred_a, pred_b, packed};
    const char* names[] = {"w_gate", "w_up", "w_down", "pred_a", "pred_b", "packed"};
    for (int i = 0; i < 6; ++i) {
        if (!ptrs[i]) {
            if (amp && (i == 3 || i == 4)) continue;
            return fail(SFFN_ERR_INVALID_ARG, "%s is null", names[i]);
        }
        if (!aligned16(ptrs[i])) return fail(SFFN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (pred_bias && !aligned16(pred_bias))
        return fail(SFFN_ERR_INVALID_ARG, "pred_bias is not 16-byte aligned");
    const PackedLayout L = packed_layout(*cfg);
    if (packed_bytes < L.total)
        return fail(SFFN_ERR_WORKSPACE, "packed buffer holds %zu bytes, %zu needed", packed_bytes, L.total);

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const size_t e = elem_size(cfg->dtype);
    const size_t d = cfg->d, di = cfg->d_i, r = cfg->rank;
    const sffn::Dt dt = cfg->dtype == SFFN_BF16 ? sffn::Dt::BF16 : sffn::Dt::F32;
    hipError_t he = hipSuccess;
    auto cp = [&](size_t off, const void* src, size_t bytes) {
        if (he == hipSuccess) he = hipMemcpyAsync(at<char>(packed, off), src, bytes, hipMemcpyDeviceToDevice, s);
    };
    if (pred_a) cp(L.A, pred_a, r * d * e);
    if (pred_b) cp(L.B, pred_b, di * r * e);
    cp(L.Wg, w_gate, di * d * e);
    cp(L.Wu, w_up, di * d * e);
    if (pred_bias) cp(L.bias, pred_bias, di * 4);
    if (he == hipSuccess) he = sffn::launch_transpose(dt, w_down, at<char>(packed, L.WdT), cfg->d, cfg->d_i, s);
    if (cfg->flags & SFFN_FLAG_BACKWARD) {
        if (he == hipSuccess) he = sffn::launch_transpose(dt, w_gate, at<char>(packed, L.WgT), cfg->d_i, cfg->d, s);
        if (he == hipSuccess) he = sffn::launch_transpose(dt, w_up, at<char>(packed, L.WuT), cfg->d_i, cfg->d, s);
    }
    if (he == hipSuccess) he = hipStreamSynchronize(s);
    if (he != hipSuccess) return hip_status(he, "sparse_ffn_create");

    sffn_layer* h = new (std::nothrow) sffn_layer;
    if (!h) return fail(SFFN_ERR_INVALID_ARG, "out of host memory");
    h->cfg = *cfg;
    h->packed = packed;
    h->L = L;
    h->has_bias = pred_bias != nullptr;
    h->profiling = false;
    *out = h;
    g_last_error.clear();
    return SFFN_OK;
}

size_t sparse_ffn_workspace_size(sffn_handle_t h, int64_t T) {
    if (!h || T <= 0 || !tokens_fit(h->cfg, T)) return 0;
    return use_gather(h->cfg, T) ? ws_gather(h->cfg, T).total : ws_mfma(h->cfg, T).total;
}

sffn_status_t sparse_ffn_forward(sffn_handle_t h, const void* x, int64_t T, void* y,
                                 uint64_t* mask_out, float* logits_out, void* workspace,
                                 size_t ws_bytes, void* hip_stream) {
    if (!h) return fail(SFFN_ERR_INVALID_ARG, "handle is null");
    if (T < 0) return fail(SFFN_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (T == 0) return SFFN_OK;
    const sffn_config_t& c = h->cfg;
    if (!x || !y) return fail(SFFN_ERR_INVALID_ARG, "x and y must not be null");
    if (!aligned16(x) || !aligned16(y)) return fail(SFFN_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    if (mask_out && !aligned16(mask_out)) return fail(SFFN_ERR_INVALID_ARG, "mask_out is not 16-byte aligned");
    if (logits_out && !aligned16(logits_out))
        return fail(SFFN_ERR_INVALID_ARG, "logits_out is not 16-byte aligned");
    if (!workspace) return fail(SFFN_ERR_INVALID_ARG, "workspace is null");
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(SFFN_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (!tokens_fit(c, T)) return fail(SFFN_ERR_UNSUPPORTED, "T = %lld is too large for one call", (long long)T);
    const size_t need = sparse_ffn_workspace_size(h, T);
    if (ws_bytes < need)
        return fail(SFFN_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed for T = %lld", ws_bytes,
                    need, (long long)T);

    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const PackedLayout& L = h->L;
    // Every channel kept with the silu gate (the dense fallback): the mask is
    // all ones and the gate comes from u, so the predictor only runs when the
    // logits are asked for.
    const bool need_pred = !(c.gate == SFFN_GATE_SILU && c.keep == c.bank && logits_out == nullptr) &&
                           c.gate != SFFN_GATE_AMPLITUDE;
    void* pk = h->packed;
    const float* bias = h->has_bias ? at<float>(pk, L.bias) : nullptr;
    hipError_t he;
    if (use_gather(c, T)) {
        const WsGather w = ws_gather(c, T);
        sffn::GatherArgs a{};
        a.dt = c.dtype == SFFN_BF16 ? sffn::Dt::BF16 : sffn::Dt::F32;
        a.d = c.d; a.d_i = c.d_i; a.rank = c.rank; a.keep = c.keep; a.gate = (int)c.gate; a.T = T;
        a.x = x; a.A = at<char>(pk, L.A); a.B = at<char>(pk, L.B); a.bias = bias;
        a.W_g = at<char>(pk, L.Wg); a.W_u = at<char>(pk, L.Wu); a.W_dT = at<char>(pk, L.WdT);
        a.y = y;
        a.z = at<float>(workspace, w.z);
        a.mask = mask_out ? mask_out : at<uint64_t>(workspace, w.mask);
        a.logits = logits_out;
        a.ids = at<uint16_t>(workspace, w.ids);
        a.pk = at<float>(workspace, w.pk);
        a.h = at<float>(workspace, w.h);
        a.partial = at<float>(workspace, w.partial);
        a.amp = at<float>(workspace, w.amp);
        a.need_pred = need_pred;
        a.mask_requested = mask_out != nullptr;
        a.events = h->profiling ? h->events : nullptr;
        he = sffn::launch_gather_forward(a, s);
    } else {
        const WsMfma w = ws_mfma(c, T);
        sffn::MfmaArgs a{};
        a.d = c.d; a.d_i = c.d_i; a.rank = c.rank; a.keep = c.keep; a.gate = (int)c.gate; a.T = T;
        a.x = static_cast<const uint16_t*>(x);
        a.A = at<const uint16_t>(pk, L.A); a.B = at<const uint16_t>(pk, L.B); a.bias = bias;
        a.W_g = at<const uint16_t>(pk, L.Wg); a.W_u = at<const uint16_t>(pk, L.Wu);
        a.W_dT = at<const uint16_t>(pk, L.WdT);
        a.y = static_cast<uint16_t*>(y);
        a.z = at<uint16_t>(workspace, w.z);
        a.logits = logits_out ? logits_out : at<float>(workspace, w.logits);
        a.logits_requested = logits_out != nullptr;
        a.mask = mask_out ? mask_out : at<uint64_t>(workspace, w.mask);
        a.h = at<uint16_t>(workspace, w.h);
        a.gate_tiles = (!use_skinny(c, T) && c.d_i % sffn::kGateTileCols == 0)
                           ? at<uint8_t>(workspace, w.gate) : nullptr;
        a.z_partial = (!use_skinny(c, T) && sffn::z_splits(T, c.d) > 1) ? at<float>(workspace, w.zpart)
                                                                         : nullptr;
        a.union_w = use_skinny(c, T) ? at<uint64_t>(workspace, w.unionw) : nullptr;
        a.need_pred = need_pred;
        a.mask_requested = mask_out != nullptr;
        a.events = h->profiling ? h->events : nullptr;
        if (c.gate == SFFN_GATE_AMPLITUDE)
            he = use_skinny(c, T) ? sffn::launch_amp_skinny(a, at<float>(workspace, w.partial), s)
                                  : sffn::launch_amp_mfma(a, s);
        else if (use_skinny(c, T)) he = sffn::launch_skinny_forward(a, at<float>(workspace, w.partial), s);
        else he = sffn::launch_mfma_forward(a, s);
    }
    return hip_status(he, "sparse_ffn_forward");
}

sffn_status_t sparse_ffn_forward_noalloc(sffn_handle_t h, const void* x, int64_t T, void* y,
                                         uint64_t* mask_out, float* logits_out, void* hip_stream) {
    if (!h) return fail(SFFN_ERR_INVALID_ARG, "handle is null");
    if (T < 0) return fail(SFFN_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (T == 0) return SFFN_OK;
    if (!tokens_fit(h->cfg, T))
        return fail(SFFN_ERR_UNSUPPORTED, "T = %lld is too large for one call", (long long)T);
    const size_t need = sparse_ffn_workspace_size(h, T);
    if (need > kScratchBytes)
        return fail(SFFN_ERR_WORKSPACE, "T = %lld needs %zu bytes of scratch; the static scratch holds %zu",
                    (long long)T, need, kScratchBytes);
    void* ws = nullptr;
    const sffn_status_t st = scratch_for_stream(static_cast<hipStream_t>(hip_stream), &ws);
    if (st != SFFN_OK) return st;
    return sparse_ffn_forward(h, x, T, y, mask_out, logits_out, ws, kScratchBytes, hip_stream);
}

size_t sparse_ffn_backward_workspace_size(sffn_handle_t h, int64_t T) {
    if (!h || T <= 0 || T > kMaxBackwardTokens || T * h->cfg.d_i / 4 >= kMaxGrid) return 0;
    return sffn::backward_workspace_bytes(T, h->cfg.d, h->cfg.d_i, h->cfg.rank,
                                          (h->cfg.flags & SFFN_FLAG_BACKWARD) != 0);
}

sffn_status_t sparse_ffn_backward(sffn_handle_t h, const void* x, const void* g_y, const uint64_t* mask,
                                  int64_t T, float tau, float* g_x, float* g_A, float* g_B, float* g_bias,
                                  float* g_Wg, float* g_Wu, float* g_Wd, void* workspace, size_t ws_bytes,
                                  void* hip_stream) {
    if (!h) return fail(SFFN_ERR_INVALID_ARG, "handle is null");
    const sffn_config_t& c = h->cfg;
    if (c.dtype != SFFN_BF16) return fail(SFFN_ERR_UNSUPPORTED, "the backward pass needs a bf16 layer");
    if (c.gate == SFFN_GATE_AMPLITUDE)
        return fail(SFFN_ERR_UNSUPPORTED, "the backward pass has no amplitude-gate form");
    if (T < 0) return fail(SFFN_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (!(tau > 0.f)) return fail(SFFN_ERR_INVALID_ARG, "tau must be > 0 (got %g)", (double)tau);
    float* outs[] = {g_x, g_A, g_B, g_Wg, g_Wu, g_Wd};
    const char* names[] = {"g_x", "g_A", "g_B", "g_Wg", "g_Wu", "g_Wd"};
    for (int i = 0; i < 6; ++i) {
        if (!outs[i]) {
            if (i == 0 && T == 0) continue;          // g_x has no elements then
            return fail(SFFN_ERR_INVALID_ARG, "%s is null", names[i]);
        }
        if (!aligned16(outs[i])) return fail(SFFN_ERR_INVALID_ARG, "%s is not 16-byte aligned", names[i]);
    }
    if (g_bias && !aligned16(g_bias)) return fail(SFFN_ERR_INVALID_ARG, "g_bias is not 16-byte aligned");
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    const int64_t d = c.d, di = c.d_i, r = c.rank;
    if (T == 0) {
        hipError_t he = hipSuccess;
        const struct { float* p; int64_t n; } z[] = {{g_A, r * d}, {g_B, di * r}, {g_bias, di},
                                                      {g_Wg, di * d}, {g_Wu, di * d}, {g_Wd, d * di}};
        for (const auto& q : z)
            if (he == hipSuccess) he = sffn::launch_zero_f32(q.p, q.n, s);
        return hip_status(he, "sparse_ffn_backward");
    }
    if (!x || !g_y || !mask) return fail(SFFN_ERR_INVALID_ARG, "x, g_y and mask must not be null");
    if (!aligned16(x) || !aligned16(g_y) || !aligned16(mask))
        return fail(SFFN_ERR_INVALID_ARG, "x, g_y and mask must be 16-byte aligned");
    if (!workspace) return fail(SFFN_ERR_INVALID_ARG, "workspace is null");
    if ((reinterpret_cast<uintptr_t>(workspace) & (kAlign - 1)) != 0)
        return fail(SFFN_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (T > kMaxBackwardTokens || T * di / 4 >= kMaxGrid)
        return fail(SFFN_ERR_UNSUPPORTED, "T = %lld is too large for one call", (long long)T);
    const size_t need = sparse_ffn_backward_workspace_size(h, T);
    if (ws_bytes < need)
        return fail(SFFN_ERR_WORKSPACE, "workspace holds %zu bytes, %zu needed for T = %lld", ws_bytes, need,
                    (long long)T);
    const PackedLayout& L = h->L;
    void* pk = h->packed;
    sffn::BwdArgs a{};
    a.d = c.d; a.d_i = c.d_i; a.rank = c.rank; a.keep = c.keep; a.gate = (int)c.gate; a.T = T;
    a.inv_tau = std::isinf(tau) ? 0.f : 1.f / tau;
    a.x = static_cast<const uint16_t*>(x);
    a.g_y = static_cast<const uint16_t*>(g_y);
    a.mask = mask;
    a.A = at<const uint16_t>(pk, L.A); a.B = at<const uint16_t>(pk, L.B);
    a.bias = h->has_bias ? at<const float>(pk, L.bias) : nullptr;
    a.W_g = at<const uint16_t>(pk, L.Wg); a.W_u = at<const uint16_t>(pk, L.Wu);
    a.W_dT = at<const uint16_t>(pk, L.WdT);
    if (c.flags & SFFN_FLAG_BACKWARD) {
        a.W_gT = at<const uint16_t>(pk, L.WgT);
        a.W_uT = at<const uint16_t>(pk, L.WuT);
    }
    a.g_x = g_x; a.g_A = g_A; a.g_B = g_B; a.g_Wg = g_Wg; a.g_Wu = g_Wu; a.g_Wd = g_Wd;
    a.g_bias = h->has_bias ? g_bias : nullptr;
    a.ws = workspace;
    hipError_t he = sffn::launch_backward(a, s);
    if (he == hipSuccess && g_bias && !h->has_bias) he = sffn::launch_zero_f32(g_bias, di, s);
    return hip_status(he, "sparse_ffn_backward");
}

sffn_status_t bank_topk(const float* logits, int64_t T, int32_t d_i, int32_t keep,
                        uint64_t* mask_out, uint16_t* idx_out, void* hip_stream) {
    if (T < 0) return fail(SFFN_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    if (d_i <= 0 || d_i % 64 != 0 || d_i > 65536)
        return fail(SFFN_ERR_INVALID_ARG, "d_i must be a positive multiple of 64, <= 65536 (got %d)", d_i);
    if (keep < 1 || keep > 64) return fail(SFFN_ERR_INVALID_ARG, "keep must lie in [1, 64] (got %d)", keep);
    if (T == 0) return SFFN_OK;
    if (T > kMaxTokens) return fail(SFFN_ERR_UNSUPPORTED, "T = %lld is too large for one call", (long long)T);
    if (!logits || !mask_out) return fail(SFFN_ERR_INVALID_ARG, "logits and mask_out must not be null");
    if (!aligned16(logits) || !aligned16(mask_out) || (idx_out && !aligned16(idx_out)))
        return fail(SFFN_ERR_INVALID_ARG, "pointers must be 16-byte aligned");
    if ((T * (d_i / 64) + 3) / 4 >= kMaxGrid)
        return fail(SFFN_ERR_UNSUPPORTED, "T = %lld is too large for one call", (long long)T);
    return hip_status(sffn::launch_bank_topk(logits, T, d_i, keep, mask_out, idx_out,
                                             static_cast<hipStream_t>(hip_stream)),
                      "bank_topk");
}

sffn_status_t sparse_ffn_set_stage_events(sffn_handle_t h, void* const* events, int32_t n_events) {
    static_assert(sffn::kStages == SFFN_STAGES, "stage count");
    if (!h) return fail(SFFN_ERR_INVALID_ARG, "handle is null");
    if (!events) {
        h->profiling = false;
        return SFFN_OK;
    }
    if (n_events < 2 * sffn::kStages)
        return fail(SFFN_ERR_INVALID_ARG, "%d events given, %d needed", n_events, 2 * sffn::kStages);
    for (int i = 0; i < 2 * sffn::kStages; ++i) {
        if (!events[i]) return fail(SFFN_ERR_INVALID_ARG, "event %d is null", i);
        h->events[i] = events[i];
    }
    h->profiling = true;
    return SFFN_OK;
}

const char* sparse_ffn_stage_name(sffn_handle_t h, int64_t T, int32_t i) {
    static const char* gather[] = {"pred1", "pred2_topk", "gateup", "down", "reduce"};
    static const char* fused[] = {"pred1", "bank_fused", "reduce", "none", "none"};
    static const char* mfma[] = {"pred1_gemm", "pred2_gemm", "bank_topk", "gateup_gemm", "down_gemm"};
    static const char* mfma_fused[] = {"pred1_gemm", "pred2_topk_gemm", "none", "gateup_gemm", "down_gemm"};
    if (!h || i < 0 || i >= sffn::kStages) return nullptr;
    if (h->cfg.gate == SFFN_GATE_AMPLITUDE) {
        static const char* amp_gather[] = {"gateup_dense", "amp_topk", "down", "reduce", "none"};
        static const char* amp_mfma[] = {"gateup_amp_gemm", "down_gemm", "none", "none", "none"};
        static const char* amp_skinny[] = {"gateup_amp_gemm", "amp_topk", "down_gemm", "none", "none"};
        if (use_gather(h->cfg, T)) return amp_gather[i];
        return use_skinny(h->cfg, T) ? amp_skinny[i] : amp_mfma[i];
    }
    // the dense fallback skips the predictor (and top-k) stages unless the
    // logits are asked for
    const bool dense_silu = h->cfg.gate == SFFN_GATE_SILU && h->cfg.keep == h->cfg.bank;
    if (dense_silu && i < (use_gather(h->cfg, T) ? 2 : 3)) return "none";
    if (!use_gather(h->cfg, T)) {
        const sffn_config_t& c = h->cfg;
        // the skinny path (4 < T <= 64) always ranks in the predictor GEMM's epilogue
        const bool fused = use_skinny(c, T) || sffn::mfma_fused_topk(T, c.d, c.d_i, c.rank);
        return fused ? mfma_fused[i] : mfma[i];
    }
    sffn::GatherArgs a{};
    a.dt = h->cfg.dtype == SFFN_BF16 ? sffn::Dt::BF16 : sffn::Dt::F32;
    a.d = h->cfg.d; a.d_i = h->cfg.d_i; a.rank = h->cfg.rank; a.keep = h->cfg.keep;
    return sffn::fused_ok(a) ? fused[i] : gather[i];
}

void sparse_ffn_destroy(sffn_handle_t h) { delete h; }

const char* sparse_ffn_status_string(sffn_status_t status) {
    switch (as_int(status)) {
        case SFFN_OK: return "ok";
        case SFFN_ERR_INVALID_ARG: return "invalid argument";
        case SFFN_ERR_UNSUPPORTED: return "unsupported";
        case SFFN_ERR_WORKSPACE: return "buffer too small";
        case SFFN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char* sparse_ffn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
