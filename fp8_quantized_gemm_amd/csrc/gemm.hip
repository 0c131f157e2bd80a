// Prefill-path GEMMs (M > 16): LDS-staged, double-buffered MFMA tile GEMMs.
//
//  - FP8: y = out( (qa . W^T) * scale ) with E4M3 activations and E4M3 (FP8
//    GEMM, page "C++与FP8量化" §3.3) or E5M2 (NestedFP FP8 mode, page
//    "NestedFP双精度推理框架" §2.1) weights, v_mfma_f32_16x16x128_f8f6f4.
//  - NestedFP FP16 mode (same page, §2.1-§2.2): the weight tile is staged in
//    LDS as its two byte planes and rebuilt as fp16 (hi<<8)|lo with v_perm
//    while it is moved from LDS to registers, then v_mfma_f32_16x16x32_f16.
//
// A 256-thread workgroup computes a 128x128 output tile; its 4 waves form a
// 2x2 grid of 64x64 sub-tiles (4x4 MFMA tiles of 16x16 each).  Each K step
// stages the next tiles in registers while the current LDS buffer feeds the
// MFMAs, so one barrier per step suffices.  Rows of A and W are K-contiguous;
// LDS rows hold 16-byte units XOR-swizzled by row so that 16 lanes reading the
// same unit of 16 consecutive rows hit distinct banks.  Workgroup ids are
// remapped so that consecutive tiles (which share the weight tile) land on
// the same XCD and its L2.
#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;

__device__ __forceinline__ v8i cat(const v4i& lo, const v4i& hi)
{
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Workgroups are dispatched round-robin over the 8 XCDs; map the launch index
// so that each XCD receives a contiguous range of logical tile ids.
__device__ __forceinline__ int xcd_remap(int bid, int nb)
{
    const int q = nb >> 3, rem = nb & 7;
    const int xcd = bid & 7, idx = bid >> 3;
    return xcd < rem ? xcd * (q + 1) + idx : rem * (q + 1) + (xcd - rem) * q + idx;
}

// Byte offset of 16-byte unit `u` of row `row` in a tile with 128-byte rows.
__device__ __forceinline__ int swz128(int row, int u) { return row * 128 + ((u ^ (row & 7)) << 4); }
// ... with 64-byte rows (4 units).
__device__ __forceinline__ int swz64(int row, int u) { return row * 64 + ((u ^ ((row >> 1) & 3)) << 4); }

template <int OUTF>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ y, const v4f (&acc)[4][4], float s,
                                           int M, int N, int mb, int nb, int r, int g)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = nb + j * 16 + r;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int m = mb + i * 16 + 4 * g + e;
                if (m < M) y[(size_t)m * N + n] = (uint16_t)f32_to_out_bits<OUTF>(acc[i][j][e] * s);
            }
        }
    }
}

// ---------------------------------------------------------------- FP8 tile GEMM
template <int WFMT, int OUTF>
__global__ __launch_bounds__(kThreads) void gemm_f8_tile_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K)
{
    constexpr int BK = 128;                       // bytes = elements
    constexpr int STAGE = (kBM + kBN) * BK;       // 32 KiB
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (M + kBM - 1) / kBM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * kBM;
    const int n0 = (bid / tiles_m) * kBN;

    // global -> register staging: thread owns unit (tid & 7) of rows
    // (tid >> 3) + 32 j, j = 0..3, of both the A and the W tile.  Buffer
    // resources span the valid rows of each tile, so rows past M or N and
    // units past K (given an out-of-range offset) read as zero, unpredicated.
    const int su = tid & 7;
    const rsrc_t ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)(min(kBM, M - m0) * K));
    const rsrc_t rw = make_rsrc(qw + (size_t)n0 * K, (uint32_t)(min(kBN, N - n0) * K));
    uint32_t roff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) roff[j] = (uint32_t)(((tid >> 3) + 32 * j) * K + su * 16);
    v4i ra_[4], rw_[4];
    auto gload = [&](int kt) {
        const bool kin = kt * BK + su * 16 < K;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t o = kin ? roff[j] + kt * BK : kOOB;
            ra_[j] = buf_load16(ra, o);
            rw_[j] = buf_load16(rw, o);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* As = lds + buf * STAGE;
        uint8_t* Ws = As + kBM * BK;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = (tid >> 3) + 32 * j;
            *reinterpret_cast<v4i*>(As + swz128(row, su)) = ra_[j];
            *reinterpret_cast<v4i*>(Ws + swz128(row, su)) = rw_[j];
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* As = lds + cur * STAGE;
        const uint8_t* Ws = As + kBM * BK;
        v8i af[4], wf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = wm * 64 + i * 16 + r;
            af[i] = cat(*reinterpret_cast<const v4i*>(As + swz128(row, g)),
                        *reinterpret_cast<const v4i*>(As + swz128(row, g + 4)));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = wn * 64 + j * 16 + r;
            wf[j] = cat(*reinterpret_cast<const v4i*>(Ws + swz128(row, g)),
                        *reinterpret_cast<const v4i*>(Ws + swz128(row, g + 4)));
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], wf[j], acc[i][j], WF_E4M3, WFMT, 0, 0, 0, 0);
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    float s = *sa;
    if (sw != nullptr) s = s * *sw;
    store_tile<OUTF>(y, acc, s, M, N, m0 + wm * 64, n0 + wn * 64, r, g);
}

// ---------------------------------------------------------------- NestedFP FP16 tile GEMM
// K step = 64 elements: A tile 128 rows x 128 bytes, hi and lo tiles 128 rows
// x 64 bytes each.  MFMA s (s = 0, 1) of a step covers elements
// [32 s, 32 s + 32); lane group g supplies elements [32 s + 8 g, +8).
__global__ __launch_bounds__(kThreads) void gemm_nested16_tile_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ hi,
    const uint8_t* __restrict__ lo, uint16_t* __restrict__ y, int M, int N, int K)
{
    constexpr int BK = 64;                                   // elements
    constexpr int A_BYTES = kBM * BK * 2;                    // 16 KiB
    constexpr int P_BYTES = kBN * BK;                        // 8 KiB per plane
    constexpr int STAGE = A_BYTES + 2 * P_BYTES;             // 32 KiB
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (M + kBM - 1) / kBM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * kBM;
    const int n0 = (bid / tiles_m) * kBN;

    // A staging: unit (tid & 7) (8 elements) of rows (tid >> 3) + 32 j, j = 0..3
    // plane staging: unit (tid & 3) (16 bytes) of rows (tid >> 2) + 64 j, j = 0..1
    const int au = tid & 7, pu = tid & 3;
    const int mrows = min(kBM, M - m0), nrows = min(kBN, N - n0);
    const rsrc_t ra = make_rsrc(a + (size_t)m0 * K, (uint32_t)(mrows * K * 2));
    const rsrc_t rh = make_rsrc(hi + (size_t)n0 * K, (uint32_t)(nrows * K));
    const rsrc_t rl = make_rsrc(lo + (size_t)n0 * K, (uint32_t)(nrows * K));
    uint32_t aoff[4], poff[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) aoff[j] = (uint32_t)((((tid >> 3) + 32 * j) * K + au * 8) * 2);
#pragma unroll
    for (int j = 0; j < 2; ++j) poff[j] = (uint32_t)(((tid >> 2) + 64 * j) * K + pu * 16);
    v4i ra_[4], rh_[2], rl_[2];
    auto gload = [&](int kt) {
        const bool ain = kt * BK + au * 8 < K;
        const bool pin = kt * BK + pu * 16 < K;
#pragma unroll
        for (int j = 0; j < 4; ++j) ra_[j] = buf_load16(ra, ain ? aoff[j] + kt * BK * 2 : kOOB);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            rh_[j] = buf_load16(rh, pin ? poff[j] + kt * BK : kOOB);
            rl_[j] = buf_load16(rl, pin ? poff[j] + kt * BK : kOOB);
        }
    };
    auto lstore = [&](int buf) {
        uint8_t* As = lds + buf * STAGE;
        uint8_t* Hs = As + A_BYTES;
        uint8_t* Ls = Hs + P_BYTES;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            *reinterpret_cast<v4i*>(As + swz128((tid >> 3) + 32 * j, au)) = ra_[j];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int row = (tid >> 2) + 64 * j;
            *reinterpret_cast<v4i*>(Hs + swz64(row, pu)) = rh_[j];
            *reinterpret_cast<v4i*>(Ls + swz64(row, pu)) = rl_[j];
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint8_t* As = lds + cur * STAGE;
        const uint8_t* Hs = As + A_BYTES;
        const uint8_t* Ls = Hs + P_BYTES;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            // A: elements [32 s + 8 g, +8) = unit 4 s + g of the 128-byte row
            v8h af[4], wf[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = wm * 64 + i * 16 + r;
                af[i] = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i*>(As + swz128(row, 4 * s + g)));
            }
            // planes: bytes [32 s + 8 g, +8) = half (g & 1) of unit 2 s + (g >> 1)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int row = wn * 64 + j * 16 + r;
                const int off = swz64(row, 2 * s + (g >> 1)) + (g & 1) * 8;
                const v2i h = *reinterpret_cast<const v2i*>(Hs + off);
                const v2i l = *reinterpret_cast<const v2i*>(Ls + off);
                uint32_t w0, w1, w2, w3;
                nested_rebuild4((uint32_t)h[0], (uint32_t)l[0], w0, w1);
                nested_rebuild4((uint32_t)h[1], (uint32_t)l[1], w2, w3);
                wf[j] = __builtin_bit_cast(v8h, v4i{(int)w0, (int)w1, (int)w2, (int)w3});
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    store_tile<OUT_FP16>(y, acc, 1.0f, M, N, m0 + wm * 64, n0 + wn * 64, r, g);
}

int tile_grid(int M, int N)
{
    return ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
}

}  // namespace

hipError_t launch_tile_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf,
                           hipStream_t stream)
{
    const dim3 grid(tile_grid(M, N)), block(kThreads);
    if (wfmt == WF_E4M3 && outf == OUT_BF16)
        gemm_f8_tile_kernel<WF_E4M3, OUT_BF16><<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K);
    else if (wfmt == WF_E5M2 && outf == OUT_FP16)
        gemm_f8_tile_kernel<WF_E5M2, OUT_FP16><<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_tile_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    gemm_nested16_tile_kernel<<<dim3(tile_grid(M, N)), dim3(kThreads), 0, stream>>>(a, hi, lo, y,
                                                                                    M, N, K);
    return hipGetLastError();
}

}  // namespace fp8q
