// NestedFP byte planes (page "NestedFP双精度推理框架" §2.1): an fp16 weight
// word is stored as its upper byte (sign, 5 exponent bits, 2 mantissa bits:
// bit for bit an E5M2 code) and its lower byte (the remaining 8 mantissa
// bits).  The E4M3 split (the page also names E4M3 for the upper byte) keeps sign |
// bits 13..7 in the upper byte, the E4M3 code of w * 2^8 truncated to 3
// mantissa bits while the top exponent bit is clear, and bit 14 | bits 6..0
// in the lower byte, so the rebuild stays exact for every word; the FP8 mode
// needs |w| < 1.875 and the split counts the words beyond.  nested_split is
// the offline step; nested_rebuild runs the same in-register rebuild as the
// FP16-mode GEMMs, on its own.  Both stream 16-byte vectors (HBM-bound).
#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kThreads = 256;

// Word pair (w0 | w1 << 16) of the E4M3 split: bit 14 of each word moves to
// bit 7 and bits 13..7 up to 14..8, so that the plain byte split below
// yields hi = sign | bits 13..7 and lo = bit 14 | bits 6..0.
__device__ __forceinline__ uint32_t e4m3_split_arrange(uint32_t v)
{
    return (v & 0x807F807Fu) | ((v << 1) & 0x7F007F00u) | ((v >> 7) & 0x00800080u);
}

// words of a pair outside the E4M3 split's FP8 range |w| < 1.875 (NaN, inf,
// and every word whose magnitude bits reach 0x3F80)
__device__ __forceinline__ int e4m3_out_of_range(uint32_t v)
{
    return ((v & 0x7FFFu) >= 0x3F80u) + (((v >> 16) & 0x7FFFu) >= 0x3F80u);
}

template <int SP>
__global__ __launch_bounds__(kThreads) void split_kernel(const uint16_t* __restrict__ w,
                                                         uint8_t* __restrict__ hi,
                                                         uint8_t* __restrict__ lo, int64_t n,
                                                         unsigned long long* __restrict__ bad)
{
    __shared__ int red[kThreads / 64];
    const int64_t nvec = n >> 3;                   // 8 words per 16-byte vector
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const v4i* wv = reinterpret_cast<const v4i*>(w);
    v2i* hv = reinterpret_cast<v2i*>(hi);
    v2i* lv = reinterpret_cast<v2i*>(lo);
    int nbad = 0;
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        v4i v = wv[i];
        if constexpr (SP == SP_E4M3) {
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                nbad += e4m3_out_of_range((uint32_t)v[d]);
                v[d] = (int)e4m3_split_arrange((uint32_t)v[d]);
            }
        }
        // word pair (w0 | w1 << 16): upper bytes are bytes 1 and 3, lower bytes 0 and 2
        const uint32_t h01 = __builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x07050301u);
        const uint32_t l01 = __builtin_amdgcn_perm((uint32_t)v[1], (uint32_t)v[0], 0x06040200u);
        const uint32_t h23 = __builtin_amdgcn_perm((uint32_t)v[3], (uint32_t)v[2], 0x07050301u);
        const uint32_t l23 = __builtin_amdgcn_perm((uint32_t)v[3], (uint32_t)v[2], 0x06040200u);
        hv[i] = v2i{(int)h01, (int)h23};
        lv[i] = v2i{(int)l01, (int)l23};
    }
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7)) {
        const int64_t j = nvec * 8 + threadIdx.x;
        uint32_t v = w[j];
        if constexpr (SP == SP_E4M3) {
            nbad += e4m3_out_of_range(v);
            v = e4m3_split_arrange(v);
        }
        hi[j] = (uint8_t)(v >> 8);
        lo[j] = (uint8_t)(v & 0xffu);
    }
    if constexpr (SP == SP_E4M3) {
        if (bad != nullptr) {
            const int c = block_sum_int<kThreads>(nbad, red);
            if (threadIdx.x == 0 && c > 0) atomicAdd(bad, (unsigned long long)c);
        }
    }
}

template <int SP>
__global__ __launch_bounds__(kThreads) void rebuild_kernel(const uint8_t* __restrict__ hi,
                                                           const uint8_t* __restrict__ lo,
                                                           uint16_t* __restrict__ w, int64_t n)
{
    const int64_t nvec = n >> 3;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const v2i* hv = reinterpret_cast<const v2i*>(hi);
    const v2i* lv = reinterpret_cast<const v2i*>(lo);
    v4i* wv = reinterpret_cast<v4i*>(w);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const v2i h = hv[i], l = lv[i];
        uint32_t o[4];
        nested_rebuild4<SP>((uint32_t)h[0], (uint32_t)l[0], o[0], o[1]);
        nested_rebuild4<SP>((uint32_t)h[1], (uint32_t)l[1], o[2], o[3]);
        wv[i] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    }
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7)) {
        const int64_t j = nvec * 8 + threadIdx.x;
        uint32_t o01, o23;
        nested_rebuild4<SP>(hi[j], lo[j], o01, o23);
        w[j] = (uint16_t)(o01 & 0xffffu);
    }
}

int grid_for(int64_t nvec)
{
    int64_t g = (nvec + kThreads * 4 - 1) / (kThreads * 4);
    if (g < 1) g = 1;
    if (g > 4096) g = 4096;
    return (int)g;
}

}  // namespace

hipError_t launch_nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n, int sp,
                               unsigned long long* bad, hipStream_t stream)
{
    if (sp == SP_E4M3)
        split_kernel<SP_E4M3><<<grid_for(n >> 3), kThreads, 0, stream>>>(w, hi, lo, n, bad);
    else
        split_kernel<SP_PLAIN><<<grid_for(n >> 3), kThreads, 0, stream>>>(w, hi, lo, n, nullptr);
    return hipGetLastError();
}

hipError_t launch_nested_rebuild(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                 int sp, hipStream_t stream)
{
    if (sp == SP_E4M3)
        rebuild_kernel<SP_E4M3><<<grid_for(n >> 3), kThreads, 0, stream>>>(hi, lo, w, n);
    else
        rebuild_kernel<SP_PLAIN><<<grid_for(n >> 3), kThreads, 0, stream>>>(hi, lo, w, n);
    return hipGetLastError();
}

}  // namespace fp8q
