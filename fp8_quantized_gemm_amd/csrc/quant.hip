// Dynamic per-tensor E4M3 quantization: amax reduction, scale = amax/448,
// round-to-nearest-even with saturation (page on a 7B model on an RTX 4060,
// §2.2 and §6.1; the E4M3 converter keeps underflow as subnormals, page
// "NestedFP双精度推理框架" §4.1).
//
// Two paths:
//  - n <= kSmallN: one workgroup loads the whole tensor into registers,
//    reduces amax (DPP within waves, LDS across waves), then quantizes from
//    the same registers.  One launch, no atomics: the decode case.
//  - larger n: a one-thread init kernel zeroes *amax, a grid-stride kernel
//    reduces per workgroup and folds into *amax with an integer atomicMax on
//    the float bit pattern (monotone for non-negative floats), and a
//    grid-stride kernel quantizes.  Every element is read twice (HBM-bound).
//
// fl32(x / s) is the correctly rounded binary32 quotient (see Quotient in
// common.hpp), so codes are a function of (x, s) alone and independent of the
// launch shape.
#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallVecPerThread = 4;                                   // 8 elements each
constexpr int64_t kSmallN = (int64_t)kSmallThreads * kSmallVecPerThread * 8;  // 32768

constexpr int kBigThreads = 256;
constexpr int kBigUnroll = 4;

// ---------------------------------------------------------------- small path
template <int DT>
__global__ __launch_bounds__(kSmallThreads) void quant_small_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q,
    float* __restrict__ scale, float* __restrict__ amax_out)
{
    __shared__ float lds[kSmallThreads / 64];
    const int tid = threadIdx.x;
    const int64_t nvec = n >> 3;
    const int tail = (int)(n & 7);
    const v4i* xv = reinterpret_cast<const v4i*>(x);

    v4i v[kSmallVecPerThread];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kSmallVecPerThread; ++j) {
        const int64_t i = tid + (int64_t)j * kSmallThreads;
        v[j] = (i < nvec) ? xv[i] : v4i{0, 0, 0, 0};
        m = fmaxf(m, vec_absmax<DT>(v[j]));
    }
    uint16_t th = 0;
    if (tid < tail) {
        th = x[nvec * 8 + tid];
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(th)));
    }
    const float a = block_max<kSmallThreads>(m, lds);
    const float s = scale_from_amax(a);
    const Quotient d(s);

    v2i* qv = reinterpret_cast<v2i*>(q);
#pragma unroll
    for (int j = 0; j < kSmallVecPerThread; ++j) {
        const int64_t i = tid + (int64_t)j * kSmallThreads;
        if (i < nvec) qv[i] = vec_quantize<DT>(v[j], d);
    }
    if (tid < tail) q[nvec * 8 + tid] = scalar_quantize<DT>(th, d);
    if (tid == 0) {
        *scale = s;
        *amax_out = a;
    }
}

// ---------------------------------------------------------------- large path
__global__ void amax_init_kernel(float* amax) { *amax = 0.0f; }

template <int DT>
__global__ __launch_bounds__(kBigThreads) void amax_kernel(const uint16_t* __restrict__ x,
                                                           int64_t n, float* amax)
{
    __shared__ float lds[kBigThreads / 64];
    const int64_t nvec = n >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    const int64_t stride = (int64_t)gridDim.x * kBigThreads;
    float m = 0.0f;
    int64_t i = (int64_t)blockIdx.x * kBigThreads + threadIdx.x;
    for (; i + (kBigUnroll - 1) * stride < nvec; i += kBigUnroll * stride) {
        v4i v[kBigUnroll];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) v[u] = xv[i + u * stride];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) m = fmaxf(m, vec_absmax<DT>(v[u]));
    }
    for (; i < nvec; i += stride) m = fmaxf(m, vec_absmax<DT>(xv[i]));
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7))
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(x[nvec * 8 + threadIdx.x])));
    m = block_max<kBigThreads>(m, lds);
    if (threadIdx.x == 0) atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(m));
}

template <int DT>
__global__ __launch_bounds__(kBigThreads) void quant_kernel(const uint16_t* __restrict__ x,
                                                            int64_t n, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale,
                                                            const float* __restrict__ amax)
{
    const float s = scale_from_amax(*amax);
    const Quotient d(s);
    const int64_t nvec = n >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    v2i* qv = reinterpret_cast<v2i*>(q);
    const int64_t stride = (int64_t)gridDim.x * kBigThreads;
    int64_t i = (int64_t)blockIdx.x * kBigThreads + threadIdx.x;
    for (; i + (kBigUnroll - 1) * stride < nvec; i += kBigUnroll * stride) {
        v4i v[kBigUnroll];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) v[u] = xv[i + u * stride];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) qv[i + u * stride] = vec_quantize<DT>(v[u], d);
    }
    for (; i < nvec; i += stride) qv[i] = vec_quantize<DT>(xv[i], d);
    if (blockIdx.x == 0) {
        if (threadIdx.x < (int)(n & 7))
            q[nvec * 8 + threadIdx.x] = scalar_quantize<DT>(x[nvec * 8 + threadIdx.x], d);
        if (threadIdx.x == 0) *scale = s;
    }
}

// ---------------------------------------------------------------- large path, no atomics
// For callers that can lend G floats of scratch (fp8_linear lends its output
// y, which the GEMM writes only afterwards): each workgroup of the amax pass
// writes its partial maximum to part[blockIdx.x]; every workgroup of the
// quantize pass reduces the G partials itself (max is exact and
// order-free, so all of them get the same amax) and quantizes its share.
// Two launches instead of three, and no same-address atomics.
//
// Shape (measured on MI355X with graph-replayed launches over the prefill
// activations of Llama-7B and Qwen-32B, 512..2048 x 4096..25600): 1024-thread
// workgroups, at most 512 of them (two per CU), two vectors of 8 elements in
// flight per thread and step, and the quantize pass requests its first two
// vectors before it reads the partial maxima.  Against 256-thread workgroups
// with four vectors and up to 2048 workgroups: 2% faster at 512 x 4096, 17%
// at 2048 x 11008 and 1024 x 25600.  The quantize pass reads x for the last
// time, with non-temporal loads (prefill steps +0.5%).  Decode-sized
// activations (up to 65536 vectors) instead take one vector per thread of
// 256-thread workgroups: the 44032 elements of the Llama-7B down projection
// at M = 4 then spread over 22 workgroups instead of 3, since one CU streams
// only a few tens of GB/s (decode steps at M = 4 / 8 and Qwen-32B M = 16
// 1.5-5% faster).
constexpr int kPartThreads = 1024;
constexpr int kPartUnroll = 2;
constexpr int kPartMaxGrid = 512;
constexpr int kPartSmallThreads = 256;

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void amax_partial_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                          float* __restrict__ part)
{
    __shared__ float lds[NT / 64];
    const int64_t nvec = n >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    const int64_t stride = (int64_t)gridDim.x * NT;
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x; i < nvec; i += U * stride) {
        v4i v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = i + u * stride < nvec ? xv[i + u * stride] : v4i{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < U; ++u) m = fmaxf(m, vec_absmax<DT>(v[u]));
    }
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7))
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(x[nvec * 8 + threadIdx.x])));
    m = block_max<NT>(m, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

template <int DT, int NT, int U>
__global__ __launch_bounds__(NT) void quant_partial_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ amax_out, const float* __restrict__ part)
{
    __shared__ float lds[NT / 64];
    const int64_t nvec = n >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    v2i* qv = reinterpret_cast<v2i*>(q);
    const int64_t stride = (int64_t)gridDim.x * NT;
    int64_t i = (int64_t)blockIdx.x * NT + threadIdx.x;
    v4i v[U];
    auto load = [&]() {
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = i + u * stride < nvec ? __builtin_nontemporal_load(&xv[i + u * stride])
                                         : v4i{0, 0, 0, 0};
    };
    load();
    float m = 0.0f;
    for (int j = threadIdx.x; j < (int)gridDim.x; j += NT) m = fmaxf(m, part[j]);
    const float a = block_max<NT>(m, lds);
    const float s = scale_from_amax(a);
    const Quotient d(s);
    while (i < nvec) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i + u * stride < nvec) qv[i + u * stride] = vec_quantize<DT>(v[u], d);
        i += U * stride;
        if (i < nvec) load();
    }
    if (blockIdx.x == 0) {
        if (threadIdx.x < (int)(n & 7))
            q[nvec * 8 + threadIdx.x] = scalar_quantize<DT>(x[nvec * 8 + threadIdx.x], d);
        if (threadIdx.x == 0) {
            *scale = s;
            *amax_out = a;
        }
    }
}

// ---------------------------------------------------------------- FP8 KV cache
// A K or V block x[T, H, D] (tokens, heads, head dimension) with one scale per
// head over all its tokens ([RTX4060] §1 keeps the KV cache in FP8; [C++FP8]
// §4.2 builds with an FP8 KV-cache type).  Vector v of head h (8 elements)
// is token v / (D/8), elements 8 (v % (D/8)) .. +8 of that token's row of h.
// Heads of at most kSmallN elements: one workgroup per head holds the head in
// registers between its amax and its quantization (one launch).  Larger
// heads: C workgroups per head write their partial maxima into q, which is
// scratch until the last pass (H*C floats fit: every workgroup covers at
// least 8 elements of its head), one workgroup per head reduces them to
// amax[h] and scale[h], then C workgroups per head quantize.  No atomics: a
// burst of same-address atomics from thousands of short workgroups
// serializes (measured on MI355X: 43 us for a 4096 x 32 x 128 block with one
// atomicMax per workgroup).
// Element offset of vector j (8 elements) of a token range of head h that
// starts at token t0: token t0 + j / dv, elements 8 (j % dv) .. +8 of that
// token's row of head h (dv = D / 8; a shift when dv is a power of two).
struct KvIndex {
    int64_t H, D, h, t0;
    uint32_t dv;
    int shift;                       // log2(dv), or -1
    __device__ __forceinline__ int64_t operator()(uint32_t j) const
    {
        const uint32_t t = shift >= 0 ? j >> shift : j / dv;
        const uint32_t r = shift >= 0 ? j & (dv - 1) : j - t * dv;
        return ((t0 + t) * H + h) * D + (int64_t)r * 8;
    }
};

template <int DT>
__global__ __launch_bounds__(kSmallThreads) void quant_kv_small_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, int64_t D, int shift,
    uint8_t* __restrict__ q, float* __restrict__ scale, float* __restrict__ amax_out)
{
    __shared__ float lds[kSmallThreads / 64];
    const int64_t h = blockIdx.x;
    const KvIndex at{H, D, h, 0, (uint32_t)(D >> 3), shift};
    const uint32_t nv = (uint32_t)(T * (D >> 3));            // <= 4096 vectors
    v4i v[kSmallVecPerThread];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kSmallVecPerThread; ++j) {
        const uint32_t i = threadIdx.x + j * kSmallThreads;
        v[j] = i < nv ? *reinterpret_cast<const v4i*>(x + at(i)) : v4i{0, 0, 0, 0};
        m = fmaxf(m, vec_absmax<DT>(v[j]));
    }
    const float a = block_max<kSmallThreads>(m, lds);
    const float s = scale_from_amax(a);
    const Quotient d(s);
#pragma unroll
    for (int j = 0; j < kSmallVecPerThread; ++j) {
        const uint32_t i = threadIdx.x + j * kSmallThreads;
        if (i < nv) *reinterpret_cast<v2i*>(q + at(i)) = vec_quantize<DT>(v[j], d);
    }
    if (threadIdx.x == 0) {
        scale[h] = s;
        amax_out[h] = a;
    }
}

// Workgroup c of head h takes tokens [c * tpw, min(T, (c + 1) * tpw)).
template <int DT>
__global__ __launch_bounds__(kBigThreads) void kv_amax_partial_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, int64_t D, int shift, int C,
    int64_t tpw, float* __restrict__ part)
{
    __shared__ float lds[kBigThreads / 64];
    const int64_t h = blockIdx.x / C;
    const int64_t c = blockIdx.x - h * C;
    const int64_t t0 = c * tpw;
    const KvIndex at{H, D, h, t0, (uint32_t)(D >> 3), shift};
    const uint32_t nv = (uint32_t)(max((int64_t)0, min(T - t0, tpw)) * (D >> 3));
    float m = 0.0f;
    uint32_t i = threadIdx.x;
    for (; i + 3 * kBigThreads < nv; i += 4 * kBigThreads) {
        v4i v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const v4i*>(x + at(i + u * kBigThreads));
#pragma unroll
        for (int u = 0; u < 4; ++u) m = fmaxf(m, vec_absmax<DT>(v[u]));
    }
    for (; i < nv; i += kBigThreads)
        m = fmaxf(m, vec_absmax<DT>(*reinterpret_cast<const v4i*>(x + at(i))));
    m = block_max<kBigThreads>(m, lds);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

__global__ __launch_bounds__(kBigThreads) void kv_combine_kernel(
    const float* __restrict__ part, int C, float* __restrict__ scale, float* __restrict__ amax)
{
    __shared__ float lds[kBigThreads / 64];
    const int64_t h = blockIdx.x;
    float m = 0.0f;
    for (int c = threadIdx.x; c < C; c += kBigThreads) m = fmaxf(m, part[h * C + c]);
    m = block_max<kBigThreads>(m, lds);
    if (threadIdx.x == 0) {
        amax[h] = m;
        scale[h] = scale_from_amax(m);
    }
}

template <int DT>
__global__ __launch_bounds__(kBigThreads) void kv_quant_kernel(
    const uint16_t* __restrict__ x, int64_t T, int64_t H, int64_t D, int shift, int C,
    int64_t tpw, uint8_t* __restrict__ q, const float* __restrict__ scale)
{
    const int64_t h = blockIdx.x / C;
    const int64_t c = blockIdx.x - h * C;
    const Quotient d(scale[h]);
    const int64_t t0 = c * tpw;
    const KvIndex at{H, D, h, t0, (uint32_t)(D >> 3), shift};
    const uint32_t nv = (uint32_t)(max((int64_t)0, min(T - t0, tpw)) * (D >> 3));
    uint32_t i = threadIdx.x;
    for (; i + 3 * kBigThreads < nv; i += 4 * kBigThreads) {
        v4i v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const v4i*>(x + at(i + u * kBigThreads));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<v2i*>(q + at(i + u * kBigThreads)) = vec_quantize<DT>(v[u], d);
    }
    for (; i < nv; i += kBigThreads) {
        const int64_t e = at(i);
        *reinterpret_cast<v2i*>(q + e) = vec_quantize<DT>(*reinterpret_cast<const v4i*>(x + e), d);
    }
}

// Token-major quantization pass, for blocks whose tokens hold VT = H*D/8 >=
// 256 vectors: workgroup w quantizes whole tokens [w*tpw, (w+1)*tpw), which
// are contiguous in memory, so every wave reads and writes one contiguous
// stretch.  Thread tid takes vectors tid + 256 i (i < RPT) of each token;
// their heads, and so their scales, are the same for every token.  The codes
// go out with non-temporal stores (they are not read again here): measured on
// MI355X on a 4096 x 32 x 128 block this pass takes 9.9 us against 11.7 us for
// the head-major pass with ordinary stores.
template <int DT, int RPT>
__global__ __launch_bounds__(kBigThreads) void kv_quant_tokens_kernel(
    const uint16_t* __restrict__ x, int64_t T, uint32_t VT, uint32_t dv, int64_t tpw,
    uint8_t* __restrict__ q, const float* __restrict__ scale)
{
    const int tid = threadIdx.x;
    float s[RPT];
    bool in[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const uint32_t v = tid + i * kBigThreads;
        in[i] = v < VT;
        s[i] = scale[in[i] ? v / dv : 0];
    }
    const int64_t t0 = (int64_t)blockIdx.x * tpw;
    const int64_t nt = max((int64_t)0, min(T - t0, tpw));
    // per-workgroup resources: at most tpw * VT * 16 bytes of x
    const rsrc_t rx = make_rsrc(x + t0 * VT * 8, (uint32_t)(nt * VT * 16));
    const rsrc_t rq = make_rsrc(q + t0 * VT * 8, (uint32_t)(nt * VT * 8));
    for (int64_t t = 0; t < nt; t += 2) {
        v4i xv[2][RPT];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const uint32_t v = (uint32_t)((t + u) * VT) + tid + i * kBigThreads;
                xv[u][i] = buf_load16<CP_NT>(rx, in[i] ? v * 16 : kOOB);   // past nt: out of range
            }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const Quotient d(s[i]);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const uint32_t v = (uint32_t)((t + u) * VT) + tid + i * kBigThreads;
                __builtin_amdgcn_raw_buffer_store_b64(vec_quantize<DT>(xv[u][i], d), rq,
                                                      in[i] ? v * 8 : kOOB, 0, CP_NT);
            }
        }
    }
}

// ---------------------------------------------------------------- delayed scaling
// One pass over x: the scale comes from the amax history of earlier calls
// (delayed_scale), so every element is quantized as soon as it is loaded and
// the amax of x is only recorded.  Small n: one workgroup, which ends the
// call itself.  Larger n: a grid-stride pass in which every workgroup folds
// its maximum into the call's running max with integer atomicMax on the
// float bits (monotone for non-negative floats) and counts itself
// (delayed_arrive); the workgroup that arrives last publishes the call
// (delayed_publish).  Nothing waits for another workgroup, so the grid needs
// no co-residency.
template <int DT>
__global__ __launch_bounds__(kSmallThreads) void quant_small_delayed_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q,
    float* __restrict__ scale, float* __restrict__ amax_out, float* __restrict__ history,
    int64_t L, uint32_t* __restrict__ state)
{
    __shared__ float lds[kSmallThreads / 64];
    const int tid = threadIdx.x;
    const int64_t nvec = n >> 3;
    const int tail = (int)(n & 7);
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    const float s = delayed_scale(state);
    const DelayedView dv = delayed_view(history, L, state);
    const Quotient d(s);
    v2i* qv = reinterpret_cast<v2i*>(q);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < kSmallVecPerThread; ++j) {
        const int64_t i = tid + (int64_t)j * kSmallThreads;
        if (i < nvec) {
            const v4i v = xv[i];
            m = fmaxf(m, vec_absmax<DT>(v));
            qv[i] = vec_quantize<DT>(v, d);
        }
    }
    if (tid < tail) {
        const uint16_t th = x[nvec * 8 + tid];
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(th)));
        q[nvec * 8 + tid] = scalar_quantize<DT>(th, d);
    }
    const float a = block_max<kSmallThreads>(m, lds);
    __syncthreads();                                   // lds is reused below
    delayed_publish<kSmallThreads>(a, dv, history, L, state, lds);
    if (tid == 0) {
        *scale = s;
        *amax_out = a;
    }
}

template <int DT>
__global__ __launch_bounds__(kBigThreads) void quant_delayed_kernel(
    const uint16_t* __restrict__ x, int64_t n, uint8_t* __restrict__ q,
    float* __restrict__ scale, float* __restrict__ amax_out, float* __restrict__ history,
    int64_t L, uint32_t* __restrict__ state)
{
    __shared__ float lds[kBigThreads / 64];
    __shared__ int last;
    const float s = delayed_scale(state);
    const DelayedView dv = delayed_view(history, L, state);
    const Quotient d(s);
    const int64_t nvec = n >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    v2i* qv = reinterpret_cast<v2i*>(q);
    const int64_t stride = (int64_t)gridDim.x * kBigThreads;
    float m = 0.0f;
    int64_t i = (int64_t)blockIdx.x * kBigThreads + threadIdx.x;
    for (; i + (kBigUnroll - 1) * stride < nvec; i += kBigUnroll * stride) {
        v4i v[kBigUnroll];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) v[u] = xv[i + u * stride];
#pragma unroll
        for (int u = 0; u < kBigUnroll; ++u) {
            m = fmaxf(m, vec_absmax<DT>(v[u]));
            qv[i + u * stride] = vec_quantize<DT>(v[u], d);
        }
    }
    for (; i < nvec; i += stride) {
        const v4i v = xv[i];
        m = fmaxf(m, vec_absmax<DT>(v));
        qv[i] = vec_quantize<DT>(v, d);
    }
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7)) {
        const uint16_t th = x[nvec * 8 + threadIdx.x];
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(th)));
        q[nvec * 8 + threadIdx.x] = scalar_quantize<DT>(th, d);
    }
    m = block_max<kBigThreads>(m, lds);
    if (threadIdx.x == 0) last = delayed_arrive<1>(state, m, true);
    __syncthreads();
    if (last) {
        __threadfence();
        const float a = __uint_as_float(atomicMax(&state[1], 0u));   // every workgroup's max
        delayed_publish<kBigThreads>(a, dv, history, L, state, lds);
        if (threadIdx.x == 0) {
            *scale = s;
            *amax_out = a;
        }
    }
}

// ---------------------------------------------------------------- per-row scales
// One scale per row of a [rows, cols] matrix: the activation scale per token
// and the weight scale per output channel of the TensorRT-LLM build the page
// "C++与FP8量化" shows in §4.2 (its per-token and per-channel options).  One
// workgroup per row: the first kRowVec vectors of 8 elements per thread stay
// in registers between the amax pass and the quantization pass, the rest of a
// longer row is read again (from L2).  Codes and scales are those of
// fp8_quantize_act applied to each row on its own.
constexpr int kRowThreads = 256;
constexpr int kRowVec = 4;

template <int DT>
__global__ __launch_bounds__(kRowThreads) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int64_t cols, uint8_t* __restrict__ q,
    float* __restrict__ scale, float* __restrict__ amax_out)
{
    __shared__ float lds[kRowThreads / 64];
    const int64_t row = blockIdx.x;
    const int nvec = (int)(cols >> 3);                     // cols % 16 == 0
    const v4i* xv = reinterpret_cast<const v4i*>(x + row * cols);
    v2i* qv = reinterpret_cast<v2i*>(q + row * cols);
    const int t = threadIdx.x;
    v4i v[kRowVec];
    float m = 0.0f;
#pragma unroll
    for (int u = 0; u < kRowVec; ++u) {
        const int i = t + u * kRowThreads;
        v[u] = i < nvec ? xv[i] : v4i{0, 0, 0, 0};
        m = fmaxf(m, vec_absmax<DT>(v[u]));
    }
    for (int i = t + kRowVec * kRowThreads; i < nvec; i += kRowThreads)
        m = fmaxf(m, vec_absmax<DT>(xv[i]));
    const float a = block_max<kRowThreads>(m, lds);
    const float s = scale_from_amax(a);
    const Quotient d(s);
#pragma unroll
    for (int u = 0; u < kRowVec; ++u) {
        const int i = t + u * kRowThreads;
        if (i < nvec) qv[i] = vec_quantize<DT>(v[u], d);
    }
    for (int i = t + kRowVec * kRowThreads; i < nvec; i += kRowThreads)
        qv[i] = vec_quantize<DT>(xv[i], d);
    if (t == 0) {
        scale[row] = s;
        amax_out[row] = a;
    }
}

// ---------------------------------------------------------------- encoder export
__global__ __launch_bounds__(256) void e4m3_encode_kernel(const float* __restrict__ v,
                                                          uint8_t* __restrict__ q, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        q[i] = (uint8_t)(e4m3_pack4(v[i], 0.f, 0.f, 0.f) & 0xffu);
}

int grid_for(int64_t nvec, int per_block)
{
    int64_t g = (nvec + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > 2048) g = 2048;   // 8 workgroups per CU, grid-stride beyond
    return (int)g;
}

}  // namespace

hipError_t launch_quantize(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                           float* amax, hipStream_t stream)
{
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    if (n <= kSmallN) {
        if (dtype == DT_BF16)
            quant_small_kernel<DT_BF16><<<1, kSmallThreads, 0, stream>>>(xs, n, q, scale, amax);
        else
            quant_small_kernel<DT_FP16><<<1, kSmallThreads, 0, stream>>>(xs, n, q, scale, amax);
        return hipGetLastError();
    }
    const int g = grid_for(n >> 3, kBigThreads * kBigUnroll);
    amax_init_kernel<<<1, 1, 0, stream>>>(amax);
    if (dtype == DT_BF16) {
        amax_kernel<DT_BF16><<<g, kBigThreads, 0, stream>>>(xs, n, amax);
        quant_kernel<DT_BF16><<<g, kBigThreads, 0, stream>>>(xs, n, q, scale, amax);
    } else {
        amax_kernel<DT_FP16><<<g, kBigThreads, 0, stream>>>(xs, n, amax);
        quant_kernel<DT_FP16><<<g, kBigThreads, 0, stream>>>(xs, n, q, scale, amax);
    }
    return hipGetLastError();
}

hipError_t launch_quantize_scratch(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                                   float* amax, float* scratch, int64_t scratch_floats,
                                   hipStream_t stream)
{
    const int64_t nvec = n >> 3;
    // decode-sized activations: one vector per thread of 256-thread
    // workgroups, so that the tensor spreads over many CUs
    const bool small = nvec <= (int64_t)kPartSmallThreads * kPartMaxGrid / 2;
    const int64_t per = small ? kPartSmallThreads : (int64_t)kPartThreads * kPartUnroll;
    const int g = (int)std::min<int64_t>(kPartMaxGrid, std::max<int64_t>(1, (nvec + per - 1) / per));
    if (n <= kSmallN || scratch == nullptr || scratch_floats < g)
        return launch_quantize(x, dtype, n, q, scale, amax, stream);
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    auto go = [&](auto dt, auto nt, auto u) {
        constexpr int DT = decltype(dt)::value, NT = decltype(nt)::value, U = decltype(u)::value;
        amax_partial_kernel<DT, NT, U><<<g, NT, 0, stream>>>(xs, n, scratch);
        quant_partial_kernel<DT, NT, U><<<g, NT, 0, stream>>>(xs, n, q, scale, amax, scratch);
    };
    using BF = std::integral_constant<int, DT_BF16>;
    using FP = std::integral_constant<int, DT_FP16>;
    using NS = std::integral_constant<int, kPartSmallThreads>;
    using NB = std::integral_constant<int, kPartThreads>;
    using U1 = std::integral_constant<int, 1>;
    using UB = std::integral_constant<int, kPartUnroll>;
    if (dtype == DT_BF16) small ? go(BF{}, NS{}, U1{}) : go(BF{}, NB{}, UB{});
    else small ? go(FP{}, NS{}, U1{}) : go(FP{}, NB{}, UB{});
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q,
                                float* scale, float* amax, hipStream_t stream)
{
    if (rows < 1 || rows > 0x7fffffff || cols < 16 || (cols & 15) != 0) return hipErrorInvalidValue;
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    if (dtype == DT_BF16)
        quant_rows_kernel<DT_BF16><<<(unsigned)rows, kRowThreads, 0, stream>>>(xs, cols, q, scale, amax);
    else
        quant_rows_kernel<DT_FP16><<<(unsigned)rows, kRowThreads, 0, stream>>>(xs, cols, q, scale, amax);
    return hipGetLastError();
}

hipError_t launch_quantize_delayed(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                                   float* amax, float* history, int64_t L, uint32_t* state,
                                   hipStream_t stream)
{
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    if (n <= kSmallN) {
        if (dtype == DT_BF16)
            quant_small_delayed_kernel<DT_BF16><<<1, kSmallThreads, 0, stream>>>(
                xs, n, q, scale, amax, history, L, state);
        else
            quant_small_delayed_kernel<DT_FP16><<<1, kSmallThreads, 0, stream>>>(
                xs, n, q, scale, amax, history, L, state);
        return hipGetLastError();
    }
    // every workgroup ends with two same-address device atomics, which
    // serialize (measured on MI355X: 2048 workgroups take 3x longer than 256
    // on a 22.5 M-element tensor), so the grid is one workgroup per 2048
    // vectors, 64 to 256 workgroups
    const int64_t g = std::min<int64_t>(256, std::max<int64_t>(64, (n >> 3) / 2048));
    if (dtype == DT_BF16)
        quant_delayed_kernel<DT_BF16><<<g, kBigThreads, 0, stream>>>(xs, n, q, scale, amax, history,
                                                                     L, state);
    else
        quant_delayed_kernel<DT_FP16><<<g, kBigThreads, 0, stream>>>(xs, n, q, scale, amax, history,
                                                                     L, state);
    return hipGetLastError();
}

hipError_t launch_quantize_kv(const void* x, int dtype, int64_t T, int64_t H, int64_t D,
                              uint8_t* q, float* scale, float* amax, hipStream_t stream)
{
    const uint16_t* xs = static_cast<const uint16_t*>(x);
    const int64_t dv = D >> 3;
    int shift = -1;
    for (int k = 0; k < 31; ++k)
        if (((int64_t)1 << k) == dv) shift = k;
    if (T * D <= kSmallN) {
        if (dtype == DT_BF16)
            quant_kv_small_kernel<DT_BF16><<<(unsigned)H, kSmallThreads, 0, stream>>>(xs, T, H, D, shift, q, scale, amax);
        else
            quant_kv_small_kernel<DT_FP16><<<(unsigned)H, kSmallThreads, 0, stream>>>(xs, T, H, D, shift, q, scale, amax);
        return hipGetLastError();
    }
    // whole tokens per workgroup, about 8192 elements each (at most 2^31
    // vectors), at least one workgroup per head
    const int64_t tpw = std::max<int64_t>(1, std::min<int64_t>(((int64_t)1 << 31) / dv, 8192 / D));
    const int64_t C64 = (T + tpw - 1) / tpw;
    const int64_t grid = H * C64;
    if (C64 > 0x7fffffff || grid > 0x7fffffff) return hipErrorInvalidValue;
    const int C = (int)C64;
    // the partial maxima live in q until the quantization pass (H*C*4 <= T*H*D)
    float* part = reinterpret_cast<float*>(q);
    if (dtype == DT_BF16)
        kv_amax_partial_kernel<DT_BF16><<<(unsigned)grid, kBigThreads, 0, stream>>>(xs, T, H, D, shift, C, tpw, part);
    else
        kv_amax_partial_kernel<DT_FP16><<<(unsigned)grid, kBigThreads, 0, stream>>>(xs, T, H, D, shift, C, tpw, part);
    kv_combine_kernel<<<(unsigned)H, kBigThreads, 0, stream>>>(part, C, scale, amax);
    // quantization: token-major for 256 .. 2048 vectors per token (two tokens
    // per workgroup), else head-major like the partial maxima
    const int64_t VT = H * dv;
    if (VT >= kBigThreads && VT <= 8 * kBigThreads) {
        const int64_t g2 = (T + 1) / 2;
        if (g2 > 0x7fffffff) return hipErrorInvalidValue;
        auto go = [&](auto rpt) {
            constexpr int R = decltype(rpt)::value;
            if (dtype == DT_BF16)
                kv_quant_tokens_kernel<DT_BF16, R><<<(unsigned)g2, kBigThreads, 0, stream>>>(
                    xs, T, (uint32_t)VT, (uint32_t)dv, 2, q, scale);
            else
                kv_quant_tokens_kernel<DT_FP16, R><<<(unsigned)g2, kBigThreads, 0, stream>>>(
                    xs, T, (uint32_t)VT, (uint32_t)dv, 2, q, scale);
        };
        if (VT <= kBigThreads) go(std::integral_constant<int, 1>{});
        else if (VT <= 2 * kBigThreads) go(std::integral_constant<int, 2>{});
        else if (VT <= 4 * kBigThreads) go(std::integral_constant<int, 4>{});
        else go(std::integral_constant<int, 8>{});
    } else if (dtype == DT_BF16) {
        kv_quant_kernel<DT_BF16><<<(unsigned)grid, kBigThreads, 0, stream>>>(xs, T, H, D, shift, C, tpw, q, scale);
    } else {
        kv_quant_kernel<DT_FP16><<<(unsigned)grid, kBigThreads, 0, stream>>>(xs, T, H, D, shift, C, tpw, q, scale);
    }
    return hipGetLastError();
}

hipError_t launch_e4m3_encode_f32(const float* v, uint8_t* q, int64_t n, hipStream_t stream)
{
    e4m3_encode_kernel<<<grid_for(n, 256 * 4), 256, 0, stream>>>(v, q, n);
    return hipGetLastError();
}

}  // namespace fp8q
