// libfp8q C ABI (declared in include/fp8q.h): host-side validation, M-based
// dispatch between the decode (M <= 16) and tile (M > 16) kernels, and launch
// on the caller's stream.  No device memory is allocated and no host
// synchronization happens in any call.
#include <atomic>
#include <cstdio>
#include <cstring>

#include "common.hpp"
#include "fp8q.h"

using namespace fp8q;

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;
constexpr int kDecodeMaxM = 16;

thread_local char g_last_error[256] = "";

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

void note_error(const char* where, hipError_t e)
{
    std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%d)", where, hipGetErrorString(e),
                  (int)e);
}

// Per-device "is gfx950" cache: 0 = unknown, 1 = yes, 2 = no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

fp8q_status check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        note_error("hipGetDevice", e);
        return FP8Q_ERR_LAUNCH;
    }
    if (dev < 0 || dev >= kMaxDevices) return FP8Q_ERR_DEVICE;
    int state = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) {
            note_error("hipGetDeviceProperties", e);
            return FP8Q_ERR_LAUNCH;
        }
        state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (state == 2)
            std::snprintf(g_last_error, sizeof(g_last_error), "device %d is %s, not gfx950", dev,
                          prop.gcnArchName);
        g_arch_ok[dev].store(state, std::memory_order_relaxed);
    }
    return state == 1 ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

fp8q_status finish(const char* where, hipError_t e)
{
    if (e != hipSuccess) {
        note_error(where, e);
        return FP8Q_ERR_LAUNCH;
    }
    return FP8Q_OK;
}

// Shared size rule of the GEMM entry points.
fp8q_status check_gemm_sizes(int64_t M, int64_t N, int64_t K)
{
    if (M < 1 || N < 1 || K < 16 || (K % 16) != 0) return FP8Q_ERR_SHAPE;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim) return FP8Q_ERR_SHAPE;
    return FP8Q_OK;
}

#define FP8Q_TRY(expr)                     \
    do {                                   \
        const fp8q_status s_ = (expr);     \
        if (s_ != FP8Q_OK) return s_;      \
    } while (0)

}  // namespace

extern "C" {

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

const char* fp8q_status_str(int status)
{
    switch (status) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_NULL: return "null pointer argument";
    case FP8Q_ERR_SHAPE: return "size out of range";
    case FP8Q_ERR_ALIGN: return "pointer not 16-byte aligned";
    case FP8Q_ERR_DTYPE: return "unknown dtype";
    case FP8Q_ERR_LAUNCH: return "HIP call or kernel launch failed";
    case FP8Q_ERR_DEVICE: return "current device is not gfx950";
    default: return "unknown status";
    }
}

const char* fp8q_last_error(void) { return g_last_error; }

fp8q_status fp8_quantize_act(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                             float* amax, fp8q_stream stream)
{
    if (!x || !q || !scale || !amax) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale) || !aligned4(amax)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    return finish("fp8_quantize_act",
                  launch_quantize(x, dtype, n, q, scale, amax, (hipStream_t)stream));
}

fp8q_status fp8_gemm(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                     uint16_t* y, int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!qa || !sa || !qw || !sw || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(qa) || !aligned16(qw) || !aligned16(y) || !aligned4(sa) || !aligned4(sw))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = M <= kDecodeMaxM
                       ? launch_gemv_fp8(qa, sa, qw, sw, y, (int)M, (int)N, (int)K, WF_E4M3,
                                         OUT_BF16, st)
                       : launch_tile_fp8(qa, sa, qw, sw, y, (int)M, (int)N, (int)K, WF_E4M3,
                                         OUT_BF16, st);
    return finish("fp8_gemm", e);
}

fp8q_status nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                         fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    return finish("nested_split", launch_nested_split(w, hi, lo, n, (hipStream_t)stream));
}

fp8q_status nested_rebuild_fp16(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    return finish("nested_rebuild_fp16", launch_nested_rebuild(hi, lo, w, n, (hipStream_t)stream));
}

fp8q_status nested_gemm_fp16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!a || !hi || !lo || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(a) || !aligned16(hi) || !aligned16(lo) || !aligned16(y)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = M <= kDecodeMaxM
                       ? launch_gemv_nested16(a, hi, lo, y, (int)M, (int)N, (int)K, st)
                       : launch_tile_nested16(a, hi, lo, y, (int)M, (int)N, (int)K, st);
    return finish("nested_gemm_fp16", e);
}

fp8q_status nested_gemm_fp8(const uint8_t* qa, const float* sa, const uint8_t* hi, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!qa || !sa || !hi || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(qa) || !aligned16(hi) || !aligned16(y) || !aligned4(sa)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = M <= kDecodeMaxM
                       ? launch_gemv_fp8(qa, sa, hi, nullptr, y, (int)M, (int)N, (int)K, WF_E5M2,
                                         OUT_FP16, st)
                       : launch_tile_fp8(qa, sa, hi, nullptr, y, (int)M, (int)N, (int)K, WF_E5M2,
                                         OUT_FP16, st);
    return finish("nested_gemm_fp8", e);
}

fp8q_status fp8q_e4m3_encode_f32(const float* v, uint8_t* q, int64_t n, fp8q_stream stream)
{
    if (!v || !q) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(v) || !aligned16(q)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_device());
    return finish("fp8q_e4m3_encode_f32", launch_e4m3_encode_f32(v, q, n, (hipStream_t)stream));
}

}  // extern "C"
