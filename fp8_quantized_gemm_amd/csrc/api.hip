// libfp8q C ABI (declared in include/fp8q.h): host-side validation, M-based
// dispatch between the decode kernels (M <= 2 row-contiguous, M <= 16 MFMA
// GEMV) and the MFMA tile kernels (M > 16), and launch on the caller's stream.  No device memory is allocated and no host
// synchronization happens in any call.
#include <atomic>
#include <cstdio>
#include <cstring>

#include <initializer_list>
#include <utility>

#include "common.hpp"
#include "fp8q.h"

using namespace fp8q;

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;
// K bound: the kernels address a tile's rows through 32-bit buffer
// resources with byte offsets below 2^31.  The tallest tile, 256 rows of fp16
// activations in the NestedFP FP16 kernel, spans 256 * K * 2 = 2^31 bytes at
// K = 2^22 (the resource size is computed in 64 bits and still fits 32), and
// its last row starts at 255 * K * 2 < 2^31.
constexpr int64_t kMaxK = (int64_t)1 << 22;
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
    if (M > kMaxDim || N > kMaxDim || K > kMaxK) return FP8Q_ERR_SHAPE;
    return FP8Q_OK;
}

// FP8-operand GEMM dispatch on M: row-contiguous VALU path (M <= 2),
// MFMA GEMV (M <= 16), MFMA tile GEMM (larger M).
hipError_t dispatch_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                        uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                        hipStream_t st)
{
    if (M <= kRowkMaxM) return launch_rowk_fp8(qa, sa, qw, sw, y, M, N, K, wfmt, outf, rowscale, st);
    if (M <= kDecodeMaxM)
        return launch_gemv_fp8(qa, sa, qw, sw, y, M, N, K, wfmt, outf, rowscale, st);
    return launch_tile_fp8(qa, sa, qw, sw, y, M, N, K, wfmt, outf, rowscale, st);
}

#define FP8Q_TRY(expr)                     \
    do {                                   \
        const fp8q_status s_ = (expr);     \
        if (s_ != FP8Q_OK) return s_;      \
    } while (0)

// A buffer of a call: base pointer and byte count.  Byte counts are products
// of validated dimensions taken in unsigned arithmetic (M * N * 2 can pass
// 2^63 at the largest M and N).
struct Buf {
    const void* p;
    uint64_t n;
};

bool overlap(const Buf& a, const Buf& b)
{
    if (a.n == 0 || b.n == 0) return false;
    const uintptr_t ab = reinterpret_cast<uintptr_t>(a.p), bb = reinterpret_cast<uintptr_t>(b.p);
    return ab < bb + (uintptr_t)b.n && bb < ab + (uintptr_t)a.n;
}

// FP8Q_ERR_OVERLAP when an output shares a byte with another output or with
// one of the inputs (other workgroups would still read or write those bytes).
fp8q_status check_apart(std::initializer_list<Buf> outs, std::initializer_list<Buf> ins)
{
    for (auto o = outs.begin(); o != outs.end(); ++o) {
        for (auto o2 = o + 1; o2 != outs.end(); ++o2)
            if (overlap(*o, *o2)) return FP8Q_ERR_OVERLAP;
        for (const Buf& i : ins)
            if (overlap(*o, i)) return FP8Q_ERR_OVERLAP;
    }
    return FP8Q_OK;
}

uint64_t u64(int64_t v) { return (uint64_t)v; }

// The buffers of a linear layer (fp8_linear and its variants): outputs q,
// scale, amax apart from everything; y apart from those and from the weights,
// but allowed over the activation x (in place).  sbytes: bytes of scale and
// amax.
fp8q_status check_linear_apart(const void* x, int64_t xelem, const void* qw, const void* sw,
                               uint64_t swbytes, const void* y, const void* q, const void* scale,
                               const void* amax, uint64_t sbytes, int64_t M, int64_t N, int64_t K)
{
    const Buf bx{x, u64(M) * u64(K) * u64(xelem)}, bq{q, u64(M) * u64(K)},
        bw{qw, u64(N) * u64(K)}, bsw{sw, sw ? swbytes : 0}, by{y, u64(M) * u64(N) * 2},
        bs{scale, sbytes}, ba{amax, sbytes};
    FP8Q_TRY(check_apart({bq, bs, ba}, {bx, bw, bsw, by}));
    return check_apart({by}, {bw, bsw});
}

// quantize + GEMM of fp8_linear / nested_linear_fp8 (pointers already checked)
fp8q_status linear_common(const char* where, const void* x, int dtype, const uint8_t* qw,
                          const float* sw, uint16_t* y, uint8_t* q, float* scale, float* amax,
                          int64_t M, int64_t N, int64_t K, int wfmt, int outf, int rowscale,
                          hipStream_t st)
{
    // The caller has checked that q, *scale and *amax share no byte with any
    // other buffer and y none with them or the weights.  y may lie over x:
    // the one-launch paths read x while other workgroups already store y,
    // and the two-launch path lends y to the quantizer as scratch, so with
    // that overlap the quantizer runs without scratch and the GEMM follows.
    const bool y_free = !overlap({y, u64(M) * u64(N) * 2}, {x, u64(M) * u64(K) * 2});
    if (y_free && M <= kRowkMaxM && M * K <= kFusedMaxMK)
        return finish(where, launch_linear_fused(x, dtype, qw, sw, y, q, scale, amax, (int)M,
                                                 (int)N, (int)K, wfmt, outf, rowscale, st));
    if (y_free && !rowscale && M > kRowkMaxM && linear_gemv_fused_pays(M, N, K))
        return finish(where, launch_linear_gemv_fused(x, dtype, qw, sw, y, q, scale, amax, (int)M,
                                                      (int)N, (int)K, wfmt, outf, st));
    if (rowscale) {
        hipError_t e = launch_quantize_rows(x, dtype, M, K, q, scale, amax, st);
        if (e == hipSuccess)
            e = dispatch_fp8(q, scale, qw, sw, y, (int)M, (int)N, (int)K, wfmt, outf, 1, st);
        return finish(where, e);
    }
    hipError_t e = launch_quantize_scratch(x, dtype, M * K, q, scale, amax,
                                           y_free ? reinterpret_cast<float*>(y) : nullptr,
                                           M * N / 2, st);
    if (e == hipSuccess)
        e = dispatch_fp8(q, scale, qw, sw, y, (int)M, (int)N, (int)K, wfmt, outf, 0, st);
    return finish(where, e);
}

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
    case FP8Q_ERR_OVERLAP: return "an output buffer overlaps another buffer of the call";
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
    FP8Q_TRY(check_apart({{q, u64(n)}, {scale, 4}, {amax, 4}}, {{x, u64(n) * 2}}));
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
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}},
                         {{qa, u64(M) * u64(K)}, {sa, 4}, {qw, u64(N) * u64(K)}, {sw, 4}}));
    FP8Q_TRY(check_device());
    return finish("fp8_gemm", dispatch_fp8(qa, sa, qw, sw, y, (int)M, (int)N, (int)K, WF_E4M3,
                                           OUT_BF16, 0, (hipStream_t)stream));
}

fp8q_status fp8_linear(const void* x, int dtype, const uint8_t* qw, const float* sw, uint16_t* y,
                       uint8_t* q, float* scale, float* amax, int64_t M, int64_t N, int64_t K,
                       fp8q_stream stream)
{
    if (!x || !qw || !sw || !y || !q || !scale || !amax) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(x) || !aligned16(qw) || !aligned16(y) || !aligned16(q) || !aligned4(sw) ||
        !aligned4(scale) || !aligned4(amax))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_linear_apart(x, 2, qw, sw, 4, y, q, scale, amax, 4, M, N, K));
    FP8Q_TRY(check_device());
    return linear_common("fp8_linear", x, dtype, qw, sw, y, q, scale, amax, M, N, K, WF_E4M3,
                         OUT_BF16, 0, (hipStream_t)stream);
}

fp8q_status fp8_quantize_kv(const void* x, int dtype, int64_t tokens, int64_t heads,
                            int64_t head_dim, uint8_t* q, float* scale, float* amax,
                            fp8q_stream stream)
{
    if (!x || !q || !scale || !amax) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    if (tokens < 1 || heads < 1 || heads > ((int64_t)1 << 20) || head_dim < 8 ||
        (head_dim % 8) != 0 || head_dim > ((int64_t)1 << 16) ||
        tokens > ((int64_t)1 << 40) / (heads * head_dim))
        return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale) || !aligned4(amax)) return FP8Q_ERR_ALIGN;
    const uint64_t nkv = u64(tokens) * u64(heads) * u64(head_dim);
    FP8Q_TRY(check_apart({{q, nkv}, {scale, 4 * u64(heads)}, {amax, 4 * u64(heads)}}, {{x, 2 * nkv}}));
    FP8Q_TRY(check_device());
    return finish("fp8_quantize_kv", launch_quantize_kv(x, dtype, tokens, heads, head_dim, q, scale,
                                                        amax, (hipStream_t)stream));
}

// History lengths the delayed-scaling calls accept.
constexpr int64_t kMaxHistory = (int64_t)1 << 24;

fp8q_status fp8_quantize_act_delayed(const void* x, int dtype, int64_t n, uint8_t* q,
                                     float* scale, float* amax, float* history,
                                     int64_t history_len, uint32_t* state, fp8q_stream stream)
{
    if (!x || !q || !scale || !amax || !history || !state) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    if (n < 1 || n > ((int64_t)1 << 40) || history_len < 1 || history_len > kMaxHistory)
        return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale) || !aligned4(amax) ||
        !aligned4(history) || !aligned16(state))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{q, u64(n)}, {scale, 4}, {amax, 4}, {history, 4 * u64(history_len)},
                          {state, 4 * u64(FP8Q_DELAYED_STATE_WORDS)}},
                         {{x, u64(n) * 2}}));
    FP8Q_TRY(check_device());
    return finish("fp8_quantize_act_delayed",
                  launch_quantize_delayed(x, dtype, n, q, scale, amax, history, history_len, state,
                                          (hipStream_t)stream));
}

fp8q_status fp8_linear_delayed(const void* x, int dtype, const uint8_t* qw, const float* sw,
                               uint16_t* y, uint8_t* q, float* scale, float* amax,
                               float* history, int64_t history_len, uint32_t* state, int64_t M,
                               int64_t N, int64_t K, fp8q_stream stream)
{
    if (!x || !qw || !sw || !y || !q || !scale || !amax || !history || !state)
        return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (history_len < 1 || history_len > kMaxHistory) return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(qw) || !aligned16(y) || !aligned16(q) || !aligned4(sw) ||
        !aligned4(scale) || !aligned4(amax) || !aligned4(history) || !aligned16(state))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_linear_apart(x, 2, qw, sw, 4, y, q, scale, amax, 4, M, N, K));
    {
        const Buf bh{history, 4 * u64(history_len)},
            bst{state, 4 * u64(FP8Q_DELAYED_STATE_WORDS)};
        FP8Q_TRY(check_apart({bh, bst}, {{x, u64(M) * u64(K) * 2}, {qw, u64(N) * u64(K)}, {sw, 4},
                                         {y, u64(M) * u64(N) * 2}, {q, u64(M) * u64(K)},
                                         {scale, 4}, {amax, 4}}));
    }
    FP8Q_TRY(check_device());
    hipStream_t st = (hipStream_t)stream;
    // the fused kernel reads x while other workgroups store y
    if (M <= kRowkMaxM && M * K <= kFusedMaxMK &&
        !overlap({y, u64(M) * u64(N) * 2}, {x, u64(M) * u64(K) * 2}))
        return finish("fp8_linear_delayed",
                      launch_linear_fused_delayed(x, dtype, qw, sw, y, q, scale, amax, history,
                                                  history_len, state, (int)M, (int)N, (int)K, st));
    hipError_t e = launch_quantize_delayed(x, dtype, M * K, q, scale, amax, history, history_len,
                                           state, st);
    if (e == hipSuccess)
        e = dispatch_fp8(q, scale, qw, sw, y, (int)M, (int)N, (int)K, WF_E4M3, OUT_BF16, 0, st);
    return finish("fp8_linear_delayed", e);
}

fp8q_status fp8_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q,
                              float* scale, float* amax, fp8q_stream stream)
{
    if (!x || !q || !scale || !amax) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    if (rows < 1 || rows > kMaxDim || cols < 16 || (cols % 16) != 0 || cols > kMaxK)
        return FP8Q_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(q) || !aligned4(scale) || !aligned4(amax)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{q, u64(rows) * u64(cols)}, {scale, 4 * u64(rows)}, {amax, 4 * u64(rows)}},
                         {{x, u64(rows) * u64(cols) * 2}}));
    FP8Q_TRY(check_device());
    return finish("fp8_quantize_rows",
                  launch_quantize_rows(x, dtype, rows, cols, q, scale, amax, (hipStream_t)stream));
}

fp8q_status fp8_gemm_rowwise(const uint8_t* qa, const float* sa, const uint8_t* qw,
                             const float* sw, uint16_t* y, int64_t M, int64_t N, int64_t K,
                             fp8q_stream stream)
{
    if (!qa || !sa || !qw || !sw || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(qa) || !aligned16(qw) || !aligned16(y) || !aligned4(sa) || !aligned4(sw))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}}, {{qa, u64(M) * u64(K)}, {sa, 4 * u64(M)},
                                                      {qw, u64(N) * u64(K)}, {sw, 4 * u64(N)}}));
    FP8Q_TRY(check_device());
    return finish("fp8_gemm_rowwise", dispatch_fp8(qa, sa, qw, sw, y, (int)M, (int)N, (int)K,
                                                   WF_E4M3, OUT_BF16, 1, (hipStream_t)stream));
}

fp8q_status fp8_linear_rowwise(const void* x, int dtype, const uint8_t* qw, const float* sw,
                               uint16_t* y, uint8_t* q, float* sa, float* amax, int64_t M,
                               int64_t N, int64_t K, fp8q_stream stream)
{
    if (!x || !qw || !sw || !y || !q || !sa || !amax) return FP8Q_ERR_NULL;
    if (dtype != FP8Q_BF16 && dtype != FP8Q_FP16) return FP8Q_ERR_DTYPE;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(x) || !aligned16(qw) || !aligned16(y) || !aligned16(q) || !aligned4(sw) ||
        !aligned4(sa) || !aligned4(amax))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_linear_apart(x, 2, qw, sw, 4 * u64(N), y, q, sa, amax, 4 * u64(M), M, N, K));
    FP8Q_TRY(check_device());
    return linear_common("fp8_linear_rowwise", x, dtype, qw, sw, y, q, sa, amax, M, N, K, WF_E4M3,
                         OUT_BF16, 1, (hipStream_t)stream);
}

fp8q_status nested_linear_fp8(const uint16_t* a, const uint8_t* hi, uint16_t* y, uint8_t* q,
                              float* scale, float* amax, int64_t M, int64_t N, int64_t K,
                              fp8q_stream stream)
{
    if (!a || !hi || !y || !q || !scale || !amax) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(a) || !aligned16(hi) || !aligned16(y) || !aligned16(q) || !aligned4(scale) ||
        !aligned4(amax))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_linear_apart(a, 2, hi, nullptr, 0, y, q, scale, amax, 4, M, N, K));
    FP8Q_TRY(check_device());
    return linear_common("nested_linear_fp8", a, FP8Q_FP16, hi, nullptr, y, q, scale, amax, M, N,
                         K, WF_E5M2, OUT_FP16, 0, (hipStream_t)stream);
}

fp8q_status nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                         fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{hi, u64(n)}, {lo, u64(n)}}, {{w, 2 * u64(n)}}));
    FP8Q_TRY(check_device());
    return finish("nested_split", launch_nested_split(w, hi, lo, n, SP_PLAIN, nullptr,
                                                      (hipStream_t)stream));
}

fp8q_status nested_rebuild_fp16(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{w, 2 * u64(n)}}, {{hi, u64(n)}, {lo, u64(n)}}));
    FP8Q_TRY(check_device());
    return finish("nested_rebuild_fp16",
                  launch_nested_rebuild(hi, lo, w, n, SP_PLAIN, (hipStream_t)stream));
}

namespace {
// NestedFP FP16 mode on either split, dispatched on M like the FP8 GEMM.
hipError_t dispatch_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, int sp, hipStream_t st)
{
    return M <= kRowkMaxM     ? launch_rowk_nested16(a, hi, lo, y, (int)M, (int)N, (int)K, sp, st)
           : M <= kDecodeMaxM ? launch_gemv_nested16(a, hi, lo, y, (int)M, (int)N, (int)K, sp, st)
                              : launch_tile_nested16(a, hi, lo, y, (int)M, (int)N, (int)K, sp, st);
}
}  // namespace

fp8q_status nested_gemm_fp16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!a || !hi || !lo || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(a) || !aligned16(hi) || !aligned16(lo) || !aligned16(y)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}},
                         {{a, u64(M) * u64(K) * 2}, {hi, u64(N) * u64(K)}, {lo, u64(N) * u64(K)}}));
    FP8Q_TRY(check_device());
    return finish("nested_gemm_fp16",
                  dispatch_nested16(a, hi, lo, y, M, N, K, SP_PLAIN, (hipStream_t)stream));
}

fp8q_status nested_gemm_fp8(const uint8_t* qa, const float* sa, const uint8_t* hi, uint16_t* y,
                            int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!qa || !sa || !hi || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(qa) || !aligned16(hi) || !aligned16(y) || !aligned4(sa)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}},
                         {{qa, u64(M) * u64(K)}, {sa, 4}, {hi, u64(N) * u64(K)}}));
    FP8Q_TRY(check_device());
    return finish("nested_gemm_fp8", dispatch_fp8(qa, sa, hi, nullptr, y, (int)M, (int)N, (int)K,
                                                  WF_E5M2, OUT_FP16, 0, (hipStream_t)stream));
}

fp8q_status nested_split_e4m3(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                              uint64_t* out_of_range, fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo) ||
        (out_of_range != nullptr && (reinterpret_cast<uintptr_t>(out_of_range) & 7u) != 0))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{hi, u64(n)}, {lo, u64(n)}, {out_of_range, out_of_range ? 8u : 0u}},
                         {{w, 2 * u64(n)}}));
    FP8Q_TRY(check_device());
    return finish("nested_split_e4m3",
                  launch_nested_split(w, hi, lo, n, SP_E4M3,
                                      reinterpret_cast<unsigned long long*>(out_of_range),
                                      (hipStream_t)stream));
}

fp8q_status nested_rebuild_e4m3(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                fp8q_stream stream)
{
    if (!w || !hi || !lo) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(w) || !aligned16(hi) || !aligned16(lo)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{w, 2 * u64(n)}}, {{hi, u64(n)}, {lo, u64(n)}}));
    FP8Q_TRY(check_device());
    return finish("nested_rebuild_e4m3",
                  launch_nested_rebuild(hi, lo, w, n, SP_E4M3, (hipStream_t)stream));
}

fp8q_status nested_gemm_fp16_e4m3(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                  uint16_t* y, int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!a || !hi || !lo || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(a) || !aligned16(hi) || !aligned16(lo) || !aligned16(y)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}},
                         {{a, u64(M) * u64(K) * 2}, {hi, u64(N) * u64(K)}, {lo, u64(N) * u64(K)}}));
    FP8Q_TRY(check_device());
    return finish("nested_gemm_fp16_e4m3",
                  dispatch_nested16(a, hi, lo, y, M, N, K, SP_E4M3, (hipStream_t)stream));
}

fp8q_status nested_gemm_fp8_e4m3(const uint8_t* qa, const float* sa, const uint8_t* hi,
                                 uint16_t* y, int64_t M, int64_t N, int64_t K, fp8q_stream stream)
{
    if (!qa || !sa || !hi || !y) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(qa) || !aligned16(hi) || !aligned16(y) || !aligned4(sa)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{y, u64(M) * u64(N) * 2}},
                         {{qa, u64(M) * u64(K)}, {sa, 4}, {hi, u64(N) * u64(K)}}));
    FP8Q_TRY(check_device());
    return finish("nested_gemm_fp8_e4m3",
                  dispatch_fp8(qa, sa, hi, nullptr, y, (int)M, (int)N, (int)K, WF_E4M3_SC8,
                               OUT_FP16, 0, (hipStream_t)stream));
}

fp8q_status nested_linear_fp8_e4m3(const uint16_t* a, const uint8_t* hi, uint16_t* y, uint8_t* q,
                                   float* scale, float* amax, int64_t M, int64_t N, int64_t K,
                                   fp8q_stream stream)
{
    if (!a || !hi || !y || !q || !scale || !amax) return FP8Q_ERR_NULL;
    FP8Q_TRY(check_gemm_sizes(M, N, K));
    if (!aligned16(a) || !aligned16(hi) || !aligned16(y) || !aligned16(q) || !aligned4(scale) ||
        !aligned4(amax))
        return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_linear_apart(a, 2, hi, nullptr, 0, y, q, scale, amax, 4, M, N, K));
    FP8Q_TRY(check_device());
    return linear_common("nested_linear_fp8_e4m3", a, FP8Q_FP16, hi, nullptr, y, q, scale, amax, M,
                         N, K, WF_E4M3_SC8, OUT_FP16, 0, (hipStream_t)stream);
}

fp8q_status fp8q_e4m3_encode_f32(const float* v, uint8_t* q, int64_t n, fp8q_stream stream)
{
    if (!v || !q) return FP8Q_ERR_NULL;
    if (n < 1 || n > ((int64_t)1 << 40)) return FP8Q_ERR_SHAPE;
    if (!aligned16(v) || !aligned16(q)) return FP8Q_ERR_ALIGN;
    FP8Q_TRY(check_apart({{q, u64(n)}}, {{v, 4 * u64(n)}}));
    FP8Q_TRY(check_device());
    return finish("fp8q_e4m3_encode_f32", launch_e4m3_encode_f32(v, q, n, (hipStream_t)stream));
}

}  // extern "C"
