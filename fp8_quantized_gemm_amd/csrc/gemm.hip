// Prefill-path GEMMs (M > 16): LDS-staged MFMA tile GEMMs.
//
//  - FP8: y = out( (qa . W^T) * scale ) with E4M3 activations and E4M3 (FP8
//    GEMM, page "C++与FP8量化" §3.3) or E5M2 (NestedFP FP8 mode, page
//    "NestedFP双精度推理框架" §2.1) weights: gemm_f8_kernel, 128x128 or
//    64x128 tiles by grid size (launch_tile_fmt), 16x16x128 MFMAs, operands
//    moved to LDS by direct-to-LDS loads in a 2-stage (activation) and a
//    3-stage (weight) ring.
//  - NestedFP FP16 mode (same page, §2.1-§2.2): gemm_nested16_tile_kernel,
//    128x128 tiles; the weight tile is staged in LDS as its two byte planes
//    and rebuilt as fp16 (hi<<8)|lo with v_perm while it is moved from LDS to
//    registers, then v_mfma_f32_16x16x32_f16.  Each K step stages the next
//    tiles in registers while the current LDS buffer feeds the MFMAs, so one
//    barrier per step suffices.
//
// Rows of A and W are K-contiguous; LDS rows hold 16-byte units XOR-swizzled
// by row so that 16 lanes reading the same unit of 16 consecutive rows hit
// distinct banks.  Workgroup ids are remapped so that consecutive tiles
// (which share the weight tile) land on the same XCD and its L2.
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

template <int OUTF, int FM = 4, int FN = 4>
__device__ __forceinline__ void store_tile(uint16_t* __restrict__ y, const v4f (&acc)[FM][FN], float s,
                                           int M, int N, int mb, int nb, int r, int g)
{
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
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

// ---------------------------------------------------------------- shared pieces
// The compiler does not order LDS reads after asynchronous direct-to-LDS
// loads, so a kernel that uses them waits explicitly (s_waitcnt vmcnt) for
// its own loads and then synchronizes the workgroup before reading.
template <int N_OUTSTANDING>
__device__ __forceinline__ void wait_vm()
{
    // s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (gfx9 encoding)
    static_assert(N_OUTSTANDING >= 0 && N_OUTSTANDING < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N_OUTSTANDING & 15) | ((N_OUTSTANDING >> 4) << 14) | (7 << 4) | (15 << 8));
}


// ---------------------------------------------------------------- FP8 tile GEMM
// BM x BN output tile (128 x 128, or 64 x 128 for small grids) per 256-thread
// workgroup; the 4 waves form a 2 x 2 grid of (BM/2) x (BN/2) wave tiles of
// 16x16x128 MFMAs, so each fragment read from LDS feeds BM/32 or BN/32
// MFMAs.  K advances 128 bytes per step.  Both operands reach LDS through
// direct global->LDS loads (buffer_load ... lds: no register staging, no LDS
// store instructions), in two rings: the activation tile (small, reused by
// every weight panel, L2-resident) has 2 stages, the weight tile (streamed
// from HBM) WST = 3 stages, so its loads are issued two steps ahead and have
// two steps of MFMAs to arrive.  Within a step the wave holds its A
// fragments and double-buffers the W fragments column by column.  LDS rows
// are 128 bytes, unit u of row r stored at position u ^ (r & 7), so the 16
// lanes reading one unit of 16 consecutive rows hit distinct banks; a DMA
// load writes lane l's 16 bytes to slot l of a 1 KiB block (8 rows), so each
// lane fetches the global unit that belongs in its slot.  For 128 x 128 tiles
// that is 80 KiB of LDS: two workgroups per CU.  Loads past the last step are
// still issued (with out-of-range offsets: zeros into a free stage) so the
// wait counts are the same every step.
template <int WFMT, int OUTF, int BM, int BN, int WST>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_f8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K)
{
    constexpr int BK = 128;
    constexpr int TM = BM / 2, TN = BN / 2;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ASTAGE = BM * BK, WSTAGE = BN * BK;
    constexpr int ABPW = BM / 32, WBPW = BN / 32;     // 1 KiB DMA blocks per wave per step
    static_assert(WST == 3, "the wait counts below assume a 3-stage weight ring");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* const a_lds = lds;                       // 2 stages
    uint8_t* const w_lds = lds + 2 * ASTAGE;          // WST stages

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (M + BM - 1) / BM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * BM;
    const int n0 = (bid / tiles_m) * BN;
    const rsrc_t ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
    const rsrc_t rw = make_rsrc(qw + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));

    // lane l of a DMA block lands in row 8b + l/8 at position l%8, which
    // holds unit (l%8) ^ (l/8) of that row
    const int du = (lane & 7) ^ (lane >> 3);
    const uint32_t rowoff = (uint32_t)((lane >> 3) * K + du * 16);
    const int nk = (K + BK - 1) / BK;
    auto dma_a = [&](int kt) {
        const bool kin = kt < nk && kt * BK + du * 16 < K;
        uint8_t* base = a_lds + (kt & 1) * ASTAGE + wave * ABPW * 1024;
#pragma unroll
        for (int j = 0; j < ABPW; ++j)
            dma_load16(ra, base + j * 1024,
                       kin ? (uint32_t)((wave * ABPW + j) * 8 * K) + rowoff + kt * BK : kOOB);
    };
    auto dma_w = [&](int kt) {
        const bool kin = kt < nk && kt * BK + du * 16 < K;
        uint8_t* base = w_lds + (kt % WST) * WSTAGE + wave * WBPW * 1024;
#pragma unroll
        for (int j = 0; j < WBPW; ++j)
            dma_load16(rw, base + j * 1024,
                       kin ? (uint32_t)((wave * WBPW + j) * 8 * K) + rowoff + kt * BK : kOOB);
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // issue order: A0 W0 .. W(WST-2) A1, then after step k: A(k+2) W(k+WST)
    dma_a(0);
#pragma unroll
    for (int p = 0; p < WST - 1; ++p) dma_w(p);
    dma_a(1);
    dma_w(WST - 1);
    // A0 and W0 done; outstanding: W1..W(WST-1), A1
    wait_vm<(WST - 1) * WBPW + ABPW>();
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t* As = a_lds + (kt & 1) * ASTAGE;
        const uint8_t* Ws = w_lds + (kt % WST) * WSTAGE;
        v8i af[FM];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * TM + i * 16 + r;
            af[i] = cat(*reinterpret_cast<const v4i*>(As + swz128(row, g)),
                        *reinterpret_cast<const v4i*>(As + swz128(row, g + 4)));
        }
        v8i wf[2];
        auto read_w = [&](int j, v8i& f) {
            const int row = wn * TN + j * 16 + r;
            f = cat(*reinterpret_cast<const v4i*>(Ws + swz128(row, g)),
                    *reinterpret_cast<const v4i*>(Ws + swz128(row, g + 4)));
        };
        read_w(0, wf[0]);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if (j + 1 < FN) read_w(j + 1, wf[(j + 1) & 1]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], wf[j & 1], acc[i][j], WF_E4M3, WFMT, 0, 0, 0, 0);
        }
        // issue order so far ends with ... W(k+1) A(k+1) W(k+2); A(k+1),
        // needed next, was issued one group ago, so only W(k+2) may stay in
        // flight (W(k+1) has had two steps)
        wait_vm<WBPW>();
        __syncthreads();                       // stage k of both rings is free
        dma_a(kt + 2);
        dma_w(kt + WST);
    }
    wait_vm<0>();                              // nothing left in flight into LDS

    float s = *sa;
    if (sw != nullptr) s = s * *sw;
    store_tile<OUTF, FM, FN>(y, acc, s, M, N, m0 + wm * TM, n0 + wn * TN, r, g);
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

template <int WFMT, int OUTF, int BM, int BN, int WST>
hipError_t launch_f8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                      uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    auto kern = gemm_f8_kernel<WFMT, OUTF, BM, BN, WST>;
    constexpr size_t lds = (2 * (size_t)BM + (size_t)WST * BN) * 128;
    static bool attr_set = false;        // idempotent host attribute, set on first use
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    kern<<<grid, 256, lds, stream>>>(qa, sa, qw, sw, y, M, N, K);
    return hipGetLastError();
}

template <int WFMT, int OUTF>
hipError_t launch_tile_fmt(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    // 128 x 128 tiles from 192 of them (measured faster from there on the
    // Llama-7B / Qwen-32B prefill shapes, M = 256..2048, weights cold in
    // HBM); below that 64 x 128, which doubles the workgroups per weight panel.
    const int64_t t128 = (int64_t)((M + 127) / 128) * ((N + 127) / 128);
    if (t128 >= 192) return launch_f8<WFMT, OUTF, 128, 128, 3>(qa, sa, qw, sw, y, M, N, K, stream);
    return launch_f8<WFMT, OUTF, 64, 128, 3>(qa, sa, qw, sw, y, M, N, K, stream);
}

hipError_t launch_tile_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf,
                           hipStream_t stream)
{
    if (wfmt == WF_E4M3 && outf == OUT_BF16)
        return launch_tile_fmt<WF_E4M3, OUT_BF16>(qa, sa, qw, sw, y, M, N, K, stream);
    if (wfmt == WF_E5M2 && outf == OUT_FP16)
        return launch_tile_fmt<WF_E5M2, OUT_FP16>(qa, sa, qw, sw, y, M, N, K, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_tile_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    gemm_nested16_tile_kernel<<<dim3(tile_grid(M, N)), dim3(kThreads), 0, stream>>>(a, hi, lo, y,
                                                                                    M, N, K);
    return hipGetLastError();
}

}  // namespace fp8q
