// Decode-path GEMMs (M <= 16): weight-streaming GEMVs on the MFMA units.
//
// The FP8 GEMM of the page "C++与FP8量化" §3.3 (E4M3 operands, fp32
// accumulation, bf16 output, "tn" layout) and the NestedFP FP8/FP16 modes
// (page "NestedFP双精度推理框架" §2.1-§2.2) at decode sizes are bound by the
// bytes of the weight matrix, which is read exactly once.  The activation
// rows (M <= 16) are padded to the 16 rows of one v_mfma 16x16 tile: the
// wasted MFMA work is far below the MFMA peak, and the matrix units take FP8
// and BF8 bytes directly, so the weights are never decoded on the VALU.
//
// Work split: a workgroup owns 16 consecutive weight rows (16 output columns)
// and its WAVES waves interleave over the K dimension in blocks of 128 bytes
// (FP8) or 64 elements (fp16); each wave issues UNROLL blocks of 16-byte loads
// before its MFMAs, then the wave partials are summed in LDS and the
// epilogue scales and rounds.
//
// Operand layout of v_mfma_f32_16x16x128_f8f6f4 (and 16x16x32_f16): lane l
// supplies row (l % 16) of A and column (l % 16) of B, and the same slice of K
// for both; lane group g = l / 16 takes bytes [16g, 16g+16) and
// [64+16g, 64+16g+16) of each 128-byte K block, so every load instruction of
// a wave reads 64 contiguous bytes of each of 16 rows.  The result lane l
// holds D[4g + i][l % 16], i = 0..3.
#include "common.hpp"

namespace fp8q {
namespace {

template <int WFMT>
__device__ __forceinline__ v4f mfma_f8(const v8i& a, const v8i& b, const v4f& c)
{
    // A (activations) is always E4M3; B (weights) is E4M3 or E5M2.
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WF_E4M3, WFMT, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat(const v4i& lo, const v4i& hi)
{
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ v4i ld16(const uint8_t* p)
{
    return *reinterpret_cast<const v4i*>(p);
}

// ---------------------------------------------------------------- FP8 GEMV
// y[m, n] = out( sum_k qa[m,k] * W[n,k] * scale ),  scale = *sa * *sw (or *sa
// when sw == nullptr).
template <int WFMT, int OUTF, int WAVES, int UNROLL>
__global__ __launch_bounds__(WAVES * 64) void gemv_f8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K)
{
    __shared__ float red[WAVES][16][17];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;

    const bool wrow_ok = (n0 + r) < N;
    const bool arow_ok = r < M;
    const uint8_t* wrow = qw + (size_t)(wrow_ok ? n0 + r : 0) * K;
    const uint8_t* arow = qa + (size_t)(arow_ok ? r : 0) * K;

    const int nblk = (K + 127) >> 7;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const v4i z = {0, 0, 0, 0};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * UNROLL) {
        v4i wl[UNROLL], wh[UNROLL], al[UNROLL], ah[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            const int k0 = kb * 128 + g * 16;
            const int k1 = k0 + 64;
            const bool in0 = kb < nblk && k0 < K;
            const bool in1 = kb < nblk && k1 < K;
            wl[u] = (wrow_ok && in0) ? ld16(wrow + k0) : z;
            wh[u] = (wrow_ok && in1) ? ld16(wrow + k1) : z;
            al[u] = (arow_ok && in0) ? ld16(arow + k0) : z;
            ah[u] = (arow_ok && in1) ? ld16(arow + k1) : z;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            acc = mfma_f8<WFMT>(cat(al[u], ah[u]), cat(wl[u], wh[u]), acc);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
    __syncthreads();

    float s = *sa;
    if (sw != nullptr) s = s * *sw;
    for (int t = threadIdx.x; t < M * 16; t += WAVES * 64) {
        const int m = t >> 4, c = t & 15;
        if (n0 + c >= N) continue;
        float v = red[0][m][c];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[w][m][c];
        y[(size_t)m * N + n0 + c] = (uint16_t)f32_to_out_bits<OUTF>(v * s);
    }
}

// ---------------------------------------------------------------- NestedFP FP16 GEMV
// y[m, n] = fp16( sum_k a[m,k] * fp16((hi[n,k] << 8) | lo[n,k]) ).
// A K block is 64 elements: lane group g takes elements [16g, 16g+16) (16
// bytes of hi, 16 of lo, 32 of a) and feeds two 16x16x32 MFMAs.
template <int WAVES, int UNROLL>
__global__ __launch_bounds__(WAVES * 64) void gemv_nested16_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ hi,
    const uint8_t* __restrict__ lo, uint16_t* __restrict__ y, int M, int N, int K)
{
    __shared__ float red[WAVES][16][17];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;

    const bool wrow_ok = (n0 + r) < N;
    const bool arow_ok = r < M;
    const uint8_t* hrow = hi + (size_t)(wrow_ok ? n0 + r : 0) * K;
    const uint8_t* lrow = lo + (size_t)(wrow_ok ? n0 + r : 0) * K;
    const uint16_t* arow = a + (size_t)(arow_ok ? r : 0) * K;

    const int nblk = (K + 63) >> 6;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    const v4i z = {0, 0, 0, 0};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * UNROLL) {
        v4i hv[UNROLL], lv[UNROLL], a0[UNROLL], a1[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int kb = kb0 + u * WAVES;
            const int k0 = kb * 64 + g * 16;
            const bool in = kb < nblk && k0 < K;
            hv[u] = (wrow_ok && in) ? ld16(hrow + k0) : z;
            lv[u] = (wrow_ok && in) ? ld16(lrow + k0) : z;
            a0[u] = (arow_ok && in) ? *reinterpret_cast<const v4i*>(arow + k0) : z;
            a1[u] = (arow_ok && in) ? *reinterpret_cast<const v4i*>(arow + k0 + 8) : z;
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            uint32_t w[8];
            nested_rebuild4((uint32_t)hv[u][0], (uint32_t)lv[u][0], w[0], w[1]);
            nested_rebuild4((uint32_t)hv[u][1], (uint32_t)lv[u][1], w[2], w[3]);
            nested_rebuild4((uint32_t)hv[u][2], (uint32_t)lv[u][2], w[4], w[5]);
            nested_rebuild4((uint32_t)hv[u][3], (uint32_t)lv[u][3], w[6], w[7]);
            const v4i wlo = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
            const v4i whi = {(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a0[u]),
                                                         __builtin_bit_cast(v8h, wlo), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, a1[u]),
                                                         __builtin_bit_cast(v8h, whi), acc, 0, 0, 0);
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
    __syncthreads();

    for (int t = threadIdx.x; t < M * 16; t += WAVES * 64) {
        const int m = t >> 4, c = t & 15;
        if (n0 + c >= N) continue;
        float v = red[0][m][c];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[w][m][c];
        y[(size_t)m * N + n0 + c] = (uint16_t)f32_to_f16_bits(v);
    }
}

constexpr int kGemvWaves = 4;
constexpr int kGemvUnroll = 4;

}  // namespace

hipError_t launch_gemv_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf,
                           hipStream_t stream)
{
    const dim3 grid((N + 15) / 16), block(kGemvWaves * 64);
    if (wfmt == WF_E4M3 && outf == OUT_BF16)
        gemv_f8_kernel<WF_E4M3, OUT_BF16, kGemvWaves, kGemvUnroll>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K);
    else if (wfmt == WF_E5M2 && outf == OUT_FP16)
        gemv_f8_kernel<WF_E5M2, OUT_FP16, kGemvWaves, kGemvUnroll>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemv_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    gemv_nested16_kernel<kGemvWaves, kGemvUnroll>
        <<<dim3((N + 15) / 16), dim3(kGemvWaves * 64), 0, stream>>>(a, hi, lo, y, M, N, K);
    return hipGetLastError();
}

}  // namespace fp8q
