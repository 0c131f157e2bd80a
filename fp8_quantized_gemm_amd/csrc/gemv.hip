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
    constexpr int BF = mfma_format(WFMT);
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, WF_E4M3, BF, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i cat(const v4i& lo, const v4i& hi)
{
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- FP8 GEMV
// y[m, n] = out( sum_k qa[m,k] * W[n,k] * scale(m, n) ), scale(m, n) =
// fl32(*sa * *sw) (*sa when sw == nullptr), or fl32(sa[m] * sw[n]) with
// rowscale (a scale per activation row and per weight row).
//
// All loads are raw buffer loads: the weight resource spans only the valid
// rows of this workgroup's 16-row tile and the activation resource only the
// M valid rows, so padded rows read as zero, and a chunk past the end of K
// gets an always-out-of-range offset.  No load is predicated, so each wave
// issues its U blocks (2 x 16 bytes of weights per lane per block) back to
// back before the first MFMA waits on them.
template <int WFMT, int OUTF, int WAVES, int U, int CP>
__global__ __launch_bounds__(WAVES * 64) void gemv_f8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K, int rowscale)
{
    __shared__ float red[WAVES][16][17];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int rows = min(16, N - n0);

    const rsrc_t rw = make_rsrc(qw + (size_t)n0 * K, (uint32_t)(rows * K));
    const rsrc_t ra = make_rsrc(qa, (uint32_t)(M * K));
    const uint32_t row_off = (uint32_t)(r * K);   // past the resource for padded rows

    const int nblk = (K + 127) >> 7;
    v4f acc = {0.f, 0.f, 0.f, 0.f};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * U) {
        v4i w0[U], w1[U], a0[U], a1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k0 = (kb0 + u * WAVES) * 128 + g * 16;
            const int k1 = k0 + 64;
            const uint32_t o0 = k0 < K ? row_off + k0 : kOOB;
            const uint32_t o1 = k1 < K ? row_off + k1 : kOOB;
            w0[u] = buf_load16<CP>(rw, o0);
            w1[u] = buf_load16<CP>(rw, o1);
            a0[u] = buf_load16(ra, o0);
            a1[u] = buf_load16(ra, o1);
        }
        // keep every load of the batch ahead of the first MFMA
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc = mfma_f8<WFMT>(cat(a0[u], a1[u]), cat(w0[u], w1[u]), acc);
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
    __syncthreads();

    const float s_w = (sw != nullptr) ? *sw : implied_wscale(WFMT);
    for (int t = threadIdx.x; t < M * 16; t += WAVES * 64) {
        const int m = t >> 4, c = t & 15;
        if (c >= rows) continue;
        float v = red[0][m][c];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[w][m][c];
        const float s = rowscale ? sa[m] * sw[n0 + c] : *sa * s_w;
        y[(size_t)m * N + n0 + c] = (uint16_t)f32_to_out_bits<OUTF>(v * s);
    }
}

// ---------------------------------------------------------------- NestedFP FP16 GEMV
// y[m, n] = fp16( sum_k a[m,k] * fp16((hi[n,k] << 8) | lo[n,k]) ).
// A K block is 64 elements: lane group g takes elements [16g, 16g+16) (16
// bytes of hi, 16 of lo, 32 of a) and feeds two 16x16x32 MFMAs.  Same
// buffer-load scheme as the FP8 GEMV.
template <int WAVES, int U, int CP, int SP>
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
    const int rows = min(16, N - n0);

    const rsrc_t rh = make_rsrc(hi + (size_t)n0 * K, (uint32_t)(rows * K));
    const rsrc_t rl = make_rsrc(lo + (size_t)n0 * K, (uint32_t)(rows * K));
    const rsrc_t ra = make_rsrc(a, (uint32_t)(M * K * 2));
    const uint32_t row_off = (uint32_t)(r * K);

    const int nblk = (K + 63) >> 6;
    v4f acc = {0.f, 0.f, 0.f, 0.f};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * U) {
        v4i hv[U], lv[U], a0[U], a1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k0 = (kb0 + u * WAVES) * 64 + g * 16;
            const bool in = k0 < K;
            const uint32_t ow = in ? row_off + k0 : kOOB;
            const uint32_t oa = in ? 2 * (row_off + k0) : kOOB;
            hv[u] = buf_load16<CP>(rh, ow);
            lv[u] = buf_load16<CP>(rl, ow);
            a0[u] = buf_load16(ra, oa);
            a1[u] = buf_load16(ra, in ? oa + 16 : kOOB);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            uint32_t w[8];
            nested_rebuild4<SP>((uint32_t)hv[u][0], (uint32_t)lv[u][0], w[0], w[1]);
            nested_rebuild4<SP>((uint32_t)hv[u][1], (uint32_t)lv[u][1], w[2], w[3]);
            nested_rebuild4<SP>((uint32_t)hv[u][2], (uint32_t)lv[u][2], w[4], w[5]);
            nested_rebuild4<SP>((uint32_t)hv[u][3], (uint32_t)lv[u][3], w[6], w[7]);
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
        if (c >= rows) continue;
        float v = red[0][m][c];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) v += red[w][m][c];
        y[(size_t)m * N + n0 + c] = (uint16_t)f32_to_f16_bits(v);
    }
}

// Launch shapes measured on MI355X over the Llama-7B decode linears at M = 4
// and 8 (weights cold in HBM): the FP8 GEMV runs 16 waves of 2 blocks each
// per 16-row tile with the default cache policy (each 128-byte weight line is
// read by two load instructions, one per 64-byte half, and a non-temporal
// first half does not stay in L2 for the second: 18-22% slower on the large
// projections); the NestedFP FP16 GEMV keeps 4 waves of 4 blocks.
constexpr int kGemvWaves = 16;
constexpr int kGemvUnroll = 2;
constexpr int kNestedWaves = 4;
constexpr int kNestedUnroll = 4;

}  // namespace

hipError_t launch_gemv_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                           hipStream_t stream)
{
    const dim3 grid((unsigned)(((int64_t)N + 15) / 16)), block(kGemvWaves * 64);
    if (wfmt == WF_E4M3 && outf == OUT_BF16)
        gemv_f8_kernel<WF_E4M3, OUT_BF16, kGemvWaves, kGemvUnroll, CP_DEFAULT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, rowscale);
    else if (wfmt == WF_E5M2 && outf == OUT_FP16 && !rowscale)
        gemv_f8_kernel<WF_E5M2, OUT_FP16, kGemvWaves, kGemvUnroll, CP_DEFAULT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, 0);
    else if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && !rowscale)
        gemv_f8_kernel<WF_E4M3_SC8, OUT_FP16, kGemvWaves, kGemvUnroll, CP_DEFAULT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, 0);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_gemv_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream)
{
    const dim3 grid((unsigned)(((int64_t)N + 15) / 16)), block(kNestedWaves * 64);
    if (sp == SP_E4M3)
        gemv_nested16_kernel<kNestedWaves, kNestedUnroll, CP_NT, SP_E4M3>
            <<<grid, block, 0, stream>>>(a, hi, lo, y, M, N, K);
    else
        gemv_nested16_kernel<kNestedWaves, kNestedUnroll, CP_NT, SP_PLAIN>
            <<<grid, block, 0, stream>>>(a, hi, lo, y, M, N, K);
    return hipGetLastError();
}

}  // namespace fp8q
