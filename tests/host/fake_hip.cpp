// A stand-in for the HIP runtime and for the library's kernel launchers, so
// that the C ABI's host logic (argument checks, workspace carving, error
// propagation) can be built with the address and undefined-behaviour
// sanitizers and run on a machine without a GPU. Nothing here touches a
// device: every call records itself and returns the status the test asks for.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include <hip/hip_runtime_api.h>

#include "launch.hpp"

// Status that the next faked runtime call or kernel launch returns
// (hipSuccess: every call succeeds).
hipError_t g_fake_runtime_status = hipSuccess;
hipError_t g_fake_launch_status = hipSuccess;
int g_fake_launches = 0;

alignas(256) static unsigned char g_fake_scratch[256];
alignas(256) unsigned char fake_fatbin[64];

extern "C" {
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return g_fake_runtime_status; }
hipError_t hipStreamSynchronize(hipStream_t) { return g_fake_runtime_status; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "injected HIP error"; }
hipError_t hipGetDevice(int* d) { *d = 0; return g_fake_runtime_status; }
hipError_t hipSetDevice(int) { return g_fake_runtime_status; }
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* d) { *d = 0; return g_fake_runtime_status; }
hipError_t hipGetSymbolAddress(void** p, const void*) {
    if (g_fake_runtime_status != hipSuccess) return g_fake_runtime_status;
    *p = g_fake_scratch;
    return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
// registration of the (absent) device code object
void** __hipRegisterFatBinary(const void*) { static void* h = nullptr; return &h; }
void __hipUnregisterFatBinary(void**) {}
void __hipRegisterVar(void**, void*, char*, const char*, int, size_t, int, int) {}
}

namespace sffn {
static hipError_t launched() {
    ++g_fake_launches;
    return g_fake_launch_status;
}
hipError_t launch_fill_mask(uint64_t*, int64_t, hipStream_t) { return launched(); }
hipError_t launch_bank_topk(const float*, int64_t, int, int, uint64_t*, uint16_t*, hipStream_t, void* const*, int) {
    return launched();
}
int gather_groups(int d_s) { return (d_s + 63) / 64; }
bool fused_ok(const GatherArgs& a) { return a.dt == Dt::BF16 && a.d == 4096 && a.keep == 16; }
hipError_t launch_gather_forward(const GatherArgs&, hipStream_t) { return launched(); }
int z_splits(int64_t T, int d) { return (T >= 256 && d % 256 == 0) ? 4 : 1; }
bool mfma_fused_topk(int64_t T, int, int d_i, int) { return T >= 256 && d_i % 128 == 0; }
hipError_t launch_mfma_forward(const MfmaArgs&, hipStream_t) { return launched(); }
hipError_t launch_amp_mfma(const MfmaArgs&, hipStream_t) { return launched(); }
hipError_t launch_amp_skinny(const MfmaArgs&, float*, hipStream_t) { return launched(); }
size_t skinny_partial_floats(int64_t T, int d, int rank, int d_i) {
    (void)d_i;
    return (size_t)4 * T * (d > rank ? d : rank);
}
hipError_t launch_skinny_forward(const MfmaArgs&, float*, hipStream_t) { return launched(); }
hipError_t launch_transpose(Dt, const void*, void*, int, int, hipStream_t, int) { return launched(); }
size_t backward_workspace_bytes(int64_t T, int d, int d_i, int rank, bool) {
    return (size_t)T * (d + d_i + rank) * 16;
}
hipError_t launch_backward(const BwdArgs&, hipStream_t) { return launched(); }
hipError_t launch_zero_f32(float*, int64_t, hipStream_t) { return launched(); }
}  // namespace sffn
