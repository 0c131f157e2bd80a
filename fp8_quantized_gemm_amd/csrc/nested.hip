// NestedFP byte planes (page "NestedFP双精度推理框架" §2.1): an fp16 weight
// word is stored as its upper byte (sign, 5 exponent bits, 2 mantissa bits:
// bit for bit an E5M2 code) and its lower byte (the remaining 8 mantissa
// bits).  nested_split is the offline step; nested_rebuild runs the same
// in-register rebuild (v_perm_b32) as the FP16-mode GEMMs, on its own.
// Both stream 16-byte vectors and are HBM-bound.
#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void split_kernel(const uint16_t* __restrict__ w,
                                                         uint8_t* __restrict__ hi,
                                                         uint8_t* __restrict__ lo, int64_t n)
{
    const int64_t nvec = n >> 3;                   // 8 words per 16-byte vector
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    const v4i* wv = reinterpret_cast<const v4i*>(w);
    v2i* hv = reinterpret_cast<v2i*>(hi);
    v2i* lv = reinterpret_cast<v2i*>(lo);
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
        const v4i v = wv[i];
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
        hi[j] = (uint8_t)(w[j] >> 8);
        lo[j] = (uint8_t)(w[j] & 0xffu);
    }
}

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
        nested_rebuild4((uint32_t)h[0], (uint32_t)l[0], o[0], o[1]);
        nested_rebuild4((uint32_t)h[1], (uint32_t)l[1], o[2], o[3]);
        wv[i] = v4i{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
    }
    if (blockIdx.x == 0 && threadIdx.x < (int)(n & 7)) {
        const int64_t j = nvec * 8 + threadIdx.x;
        uint32_t o01, o23;
        nested_rebuild4(hi[j], lo[j], o01, o23);
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

hipError_t launch_nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n,
                               hipStream_t stream)
{
    split_kernel<<<grid_for(n >> 3), kThreads, 0, stream>>>(w, hi, lo, n);
    return hipGetLastError();
}

hipError_t launch_nested_rebuild(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                 hipStream_t stream)
{
    rebuild_kernel<<<grid_for(n >> 3), kThreads, 0, stream>>>(hi, lo, w, n);
    return hipGetLastError();
}

}  // namespace fp8q
