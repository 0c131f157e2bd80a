// Prefill-path GEMMs (M > 16): LDS-staged MFMA tile GEMMs.
//
//  - FP8: y = out( (qa . W^T) * scale ) with E4M3 activations and E4M3 (FP8
//    GEMM, page "C++与FP8量化" §3.3) or E5M2 (NestedFP FP8 mode, page
//    "NestedFP双精度推理框架" §2.1) weights: gemm_f8_kernel, tiles from
//    256x256 (8 waves) down to 64x64 (4 waves) picked per shape by the cost
//    of their rounds of workgroups (pick_tile_shape), 16x16x128 MFMAs, operands
//    moved to LDS by direct-to-LDS loads in an activation ring and a weight
//    ring of 2-4 stages each.
//  - NestedFP FP16 mode (same page, §2.1-§2.2): gemm_n16_kernel, tiles from
//    256x256 (8 waves) to 64x64 (4 waves) picked the same way; the
//    activation and the two weight byte planes reach LDS by
//    direct-to-LDS loads, and the weight words are rebuilt as fp16
//    (hi<<8)|lo with v_perm while they move from LDS to registers, then
//    v_mfma_f32_16x16x32_f16.
//
// Rows of A and W are K-contiguous; LDS rows hold 16-byte units XOR-swizzled
// by row so that 16 lanes reading the same unit of 16 consecutive rows hit
// distinct banks.  Workgroup ids are remapped so that consecutive tiles
// (which share the weight tile) land on the same XCD and its L2.
#include <atomic>

#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kCUs = 256;                // compute units of an MI355X


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
// BM x BN output tile per workgroup of WM x WN waves, each wave owning a
// (BM/WM) x (BN/WN) block of 16x16x128 MFMA tiles.  K advances 128 bytes per
// step.  Both operands reach LDS through direct global->LDS loads
// (buffer_load ... lds: no register staging, no LDS store instructions), in
// two rings: the activation tile (reused by every weight panel, L2-resident)
// has AST stages, the weight tile (streamed from HBM) WST >= AST stages, so
// its loads are issued WST - 1 steps ahead.  Within a step the wave keeps the
// fragments of the operand it has fewer of and streams the other one,
// double-buffered, so every streamed fragment feeds min(FM, FN) MFMAs.  LDS
// rows are 128 bytes, unit u of row r stored at position u ^ (r & 7), so the
// 16 lanes reading one unit of 16 consecutive rows hit distinct banks; a DMA
// load writes lane l's 16 bytes to slot l of a 1 KiB block (8 rows), so each
// lane fetches the global unit that belongs in its slot.  Loads past the last
// step are still issued (with out-of-range offsets: zeros into a free stage)
// so the wait counts are the same every step.
//
// The weight fragment is the MFMA's first operand, so a lane's four results
// are four consecutive output columns of one row: one 8-byte store each.
//
// Shapes in use: kTileShapes, chosen per call by pick_tile_shape.
template <int WFMT, int OUTF, int BM, int BN, int WM, int WN, int AST, int WST>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_f8_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K, int rowscale)
{
    constexpr int WF_MF = mfma_format(WFMT);   // MFMA format selector of the weight operand
    constexpr int NW = WM * WN;
    constexpr int BK = 128;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ASTAGE = BM * BK, WSTAGE = BN * BK;
    constexpr int ABPW = BM / 8 / NW, WBPW = BN / 8 / NW;   // 1 KiB DMA blocks per wave per step
    static_assert(ABPW * 8 * NW == BM && WBPW * 8 * NW == BN, "whole DMA blocks per wave");
    static_assert(AST >= 2 && WST >= AST, "ring depths");
    constexpr int ALLOW = (AST < WST ? WBPW : 0) + (AST - 2) * (ABPW + WBPW);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* const a_lds = lds;                       // AST stages
    uint8_t* const w_lds = lds + AST * ASTAGE;        // WST stages

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (int)(((int64_t)M + BM - 1) / BM);
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
        uint8_t* base = a_lds + (kt % AST) * ASTAGE + wave * ABPW * 1024;
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

    // loads go out in groups: the group issued after step j holds A(j + AST)
    // then W(j + WST); the prologue issues groups -WST .. -1 (skipping
    // negative steps), and loads past the last step are still issued with
    // out-of-range offsets, so the wait before every step is the same:
    // A(k+1) sits in group k + 1 - AST, after which only that group's W and
    // the AST - 2 later groups may still be in flight.
#pragma unroll
    for (int j = -WST; j < 0; ++j) {
        if (j + AST >= 0) dma_a(j + AST);
        dma_w(j + WST);
    }
    wait_vm<ALLOW + ABPW + WBPW>();            // the prologue has also issued group -1
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t* As = a_lds + (kt % AST) * ASTAGE;
        const uint8_t* Ws = w_lds + (kt % WST) * WSTAGE;
        auto frag = [&](const uint8_t* S, int row) {
            return cat(*reinterpret_cast<const v4i*>(S + swz128(row, g)),
                       *reinterpret_cast<const v4i*>(S + swz128(row, g + 4)));
        };
        if constexpr (FN <= FM) {
            // keep the FN weight fragments, stream the activation fragments
            v8i wf[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) wf[j] = frag(Ws, wn * TN + j * 16 + r);
            v8i af[2];
            af[0] = frag(As, wm * TM + r);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (i + 1 < FM) af[(i + 1) & 1] = frag(As, wm * TM + (i + 1) * 16 + r);
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf[j], af[i & 1], acc[i][j], WF_MF, WF_E4M3, 0, 0, 0, 0);
            }
        } else {
            // keep the FM activation fragments, stream the weight fragments
            v8i af[FM];
#pragma unroll
            for (int i = 0; i < FM; ++i) af[i] = frag(As, wm * TM + i * 16 + r);
            v8i wf[2];
            wf[0] = frag(Ws, wn * TN + r);
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                if (j + 1 < FN) wf[(j + 1) & 1] = frag(Ws, wn * TN + (j + 1) * 16 + r);
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf[j & 1], af[i], acc[i][j], WF_MF, WF_E4M3, 0, 0, 0, 0);
            }
        }
        wait_vm<ALLOW>();
        __syncthreads();                       // stage k of both rings is free
        dma_a(kt + AST);
        dma_w(kt + WST);
    }
    wait_vm<0>();                              // nothing left in flight into LDS

    // acc[i][j][e] is output row mb + 16 i + r, column nb + 16 j + 4 g + e;
    // scale_of(i, j, e) is the output scale of that element
    const int mb = m0 + wm * TM, nb = n0 + wn * TN;
    const bool vec = (N & 3) == 0;             // 8-byte aligned groups of 4 columns
    auto store = [&](auto scale_of) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = mb + i * 16 + r;
            if (m >= M) continue;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = nb + j * 16 + 4 * g;
                uint16_t* dst = y + (size_t)m * N + n;
                if (vec && n + 3 < N) {
                    const uint32_t lo = f32_to_out_bits<OUTF>(acc[i][j][0] * scale_of(i, j, 0)) |
                                        (f32_to_out_bits<OUTF>(acc[i][j][1] * scale_of(i, j, 1)) << 16);
                    const uint32_t hi = f32_to_out_bits<OUTF>(acc[i][j][2] * scale_of(i, j, 2)) |
                                        (f32_to_out_bits<OUTF>(acc[i][j][3] * scale_of(i, j, 3)) << 16);
                    *reinterpret_cast<v2i*>(dst) = v2i{(int)lo, (int)hi};
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N)
                            dst[e] = (uint16_t)f32_to_out_bits<OUTF>(acc[i][j][e] * scale_of(i, j, e));
                }
            }
        }
    };
    if (rowscale) {
        // the tile's row and column scales, loaded before the first store so
        // that no load waits behind the output stores
        float sam[FM], swn[FN][4];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = mb + i * 16 + r;
            sam[i] = m < M ? sa[m] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = nb + j * 16 + 4 * g + e;
                swn[j][e] = n < N ? sw[n] : 0.0f;
            }
        store([&](int i, int j, int e) { return sam[i] * swn[j][e]; });
    } else {
        const float s = *sa * ((sw != nullptr) ? *sw : implied_wscale(WFMT));
        store([&](int, int, int) { return s; });
    }
}

// ---------------------------------------------------------------- NestedFP FP16 GEMM, DMA rings
// The NestedFP FP16 mode on the structure of gemm_f8_kernel: BM x BN tiles,
// WM x WN waves of (BM/WM) x (BN/WN), K steps of 64 elements.  The fp16 activation
// tile (BM rows x 128 bytes) goes through an AST-stage ring and the weight
// byte planes (hi then lo, BN rows x 64 bytes each) through a WST-stage ring
// (WST >= AST >= 2), both filled by direct global->LDS loads.  MFMA s
// (s = 0, 1) of a step covers elements [32 s, 32 s + 32): lane group g
// supplies elements [32 s + 8 g, +8), i.e. unit 4 s + g of an activation row
// and half (g & 1) of unit 2 s + (g >> 1) of each plane row; the weight words
// are rebuilt as (hi << 8) | lo with v_perm while they move from LDS to
// registers.  Activation rows use the 128-byte swizzle (u ^ (r & 7)), plane
// rows the 64-byte one (u ^ ((r >> 1) & 3)); a DMA block is 8 activation rows
// or 16 plane rows.
//
// Loads are issued in groups: the group issued after step j holds A(j + AST)
// then W(j + WST) (the prologue issues groups j = -WST .. -1, skipping
// negative steps), and loads past the last step are still issued with
// out-of-range offsets, so before step k + 1 the wait is the same every
// step: A(k+1) sits in group k + 1 - AST, after which only that group's W
// and the AST - 2 later groups may still be in flight (when AST == WST the
// group's W is needed too).
template <int BM, int BN, int WM, int WN, int AST, int WST, int SP>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2)))
void gemm_n16_kernel(const uint16_t* __restrict__ a, const uint8_t* __restrict__ hi,
                     const uint8_t* __restrict__ lo, uint16_t* __restrict__ y, int M, int N, int K)
{
    static_assert(AST >= 2 && WST >= AST, "ring depths");
    constexpr int NW = WM * WN;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 16, FN = TN / 16;
    constexpr int ASTAGE = BM * 128, PLANE = BN * 64, WSTAGE = 2 * PLANE;
    constexpr int ABPW = BM / 8 / NW;             // activation blocks per wave per step
    constexpr int PBPW = BN / 16 / NW;            // blocks per plane per wave per step
    static_assert(ABPW * 8 * NW == BM && PBPW * 16 * NW == BN, "whole DMA blocks per wave");
    constexpr int WBPW = 2 * PBPW;
    constexpr int ALLOW = (AST < WST ? WBPW : 0) + (AST - 2) * (ABPW + WBPW);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    uint8_t* const a_lds = lds;
    uint8_t* const w_lds = lds + AST * ASTAGE;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (int)(((int64_t)M + BM - 1) / BM);
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * BM;
    const int n0 = (bid / tiles_m) * BN;
    const int nrows = min(BN, N - n0);
    // byte sizes in 64 bits: 256 fp16 rows at the largest K (2^22) span 2^31
    // bytes, which a buffer resource still holds (num_records is 32 bits)
    const rsrc_t ra = make_rsrc(a + (size_t)m0 * K, (uint32_t)((int64_t)min(BM, M - m0) * K * 2));
    const rsrc_t rh = make_rsrc(hi + (size_t)n0 * K, (uint32_t)((int64_t)nrows * K));
    const rsrc_t rl = make_rsrc(lo + (size_t)n0 * K, (uint32_t)((int64_t)nrows * K));

    const int dua = (lane & 7) ^ (lane >> 3);         // activation unit landing in slot l
    const int duw = (lane & 3) ^ ((lane >> 3) & 3);   // plane unit landing in slot l
    const uint32_t aoff = (uint32_t)((lane >> 3) * K * 2 + dua * 16);
    const uint32_t poff = (uint32_t)((lane >> 2) * K + duw * 16);
    const int nk = (K + 63) / 64;
    auto dma_a = [&](int kt) {
        const bool kin = kt < nk && kt * 64 + dua * 8 < K;
        uint8_t* base = a_lds + (kt % AST) * ASTAGE + wave * ABPW * 1024;
#pragma unroll
        for (int j = 0; j < ABPW; ++j)
            dma_load16(ra, base + j * 1024,
                       kin ? (uint32_t)((wave * ABPW + j) * 8 * K * 2) + aoff + kt * 128 : kOOB);
    };
    auto dma_w = [&](int kt) {
        const bool kin = kt < nk && kt * 64 + duw * 16 < K;
        uint8_t* base = w_lds + (kt % WST) * WSTAGE + wave * PBPW * 1024;
#pragma unroll
        for (int j = 0; j < PBPW; ++j) {
            const uint32_t o = kin ? (uint32_t)((wave * PBPW + j) * 16 * K) + poff + kt * 64 : kOOB;
            dma_load16(rh, base + j * 1024, o);
            dma_load16(rl, base + PLANE + j * 1024, o);
        }
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int j = -WST; j < 0; ++j) {
        if (j + AST >= 0) dma_a(j + AST);
        dma_w(j + WST);
    }
    wait_vm<ALLOW + ABPW + WBPW>();            // the prologue has also issued group -1
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const uint8_t* As = a_lds + (kt % AST) * ASTAGE;
        const uint8_t* Hs = w_lds + (kt % WST) * WSTAGE;
        const uint8_t* Ls = Hs + PLANE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            v8h af[FM], wf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int row = wm * TM + i * 16 + r;
                af[i] = __builtin_bit_cast(v8h, *reinterpret_cast<const v4i*>(As + swz128(row, 4 * s + g)));
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int row = wn * TN + j * 16 + r;
                const int off = swz64(row, 2 * s + (g >> 1)) + (g & 1) * 8;
                const v2i h = *reinterpret_cast<const v2i*>(Hs + off);
                const v2i l = *reinterpret_cast<const v2i*>(Ls + off);
                uint32_t w0, w1, w2, w3;
                nested_rebuild4<SP>((uint32_t)h[0], (uint32_t)l[0], w0, w1);
                nested_rebuild4<SP>((uint32_t)h[1], (uint32_t)l[1], w2, w3);
                wf[j] = __builtin_bit_cast(v8h, v4i{(int)w0, (int)w1, (int)w2, (int)w3});
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], wf[j], acc[i][j], 0, 0, 0);
        }
        wait_vm<ALLOW>();
        __syncthreads();                       // stage kt of both rings is free
        dma_a(kt + AST);
        dma_w(kt + WST);
    }
    wait_vm<0>();

    store_tile<OUT_FP16, FM, FN>(y, acc, 1.0f, M, N, m0 + wm * TM, n0 + wn * TN, r, g);
}

}  // namespace

template <int WFMT, int OUTF, int BM, int BN, int WM, int WN, int AST, int WST>
hipError_t launch_f8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                     uint16_t* y, int M, int N, int K, int rowscale, hipStream_t stream)
{
    auto kern = gemm_f8_kernel<WFMT, OUTF, BM, BN, WM, WN, AST, WST>;
    constexpr size_t lds = ((size_t)AST * BM + (size_t)WST * BN) * 128;
    static_assert(lds <= 160 * 1024, "LDS of one CU");
    static std::atomic<uint64_t> attr_devices{0};
    if (const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kern), lds, attr_devices);
        e != hipSuccess)
        return e;
    const int64_t grid = (((int64_t)M + BM - 1) / BM) * (((int64_t)N + BN - 1) / BN);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    kern<<<(int)grid, WM * WN * 64, lds, stream>>>(qa, sa, qw, sw, y, M, N, K, rowscale);
    return hipGetLastError();
}

// Tile shapes of the FP8 GEMM and the measured time of one round of their
// workgroups (one per CU, or two per CU for 64 x 64) at K = 4096 on MI355X,
// weights cold in HBM, medians over the Llama-7B / Qwen-32B prefill shapes.
// 64 x 64 appears twice: a grid of at most one workgroup per CU finishes its
// round much sooner than a full one.
struct TileShape { int bm, bn, per_cu; float round_us; };
constexpr TileShape kTileShapes[] = {
    {256, 256, 1, 55.8f},   // 8 waves of 128 x 64, 2 + 2 stages (128 KiB)
    {256, 192, 1, 45.3f},   // 8 waves of 128 x 48, 2 + 3 stages (136 KiB)
    {256, 128, 1, 33.9f},   // 8 waves of  64 x 64, 3 + 4 stages (160 KiB)
    {128, 192, 1, 29.6f},   // 8 waves of  64 x 48, 3 + 4 stages (144 KiB)
    {128, 128, 1, 22.9f},   // 8 waves of  64 x 32, 4 + 4 stages (128 KiB)
    {128,  64, 1, 16.5f},   // 8 waves of  32 x 32, 4 + 4 stages ( 96 KiB)
    { 64,  64, 2, 17.0f},   // 4 waves of  32 x 32, 4 + 4 stages ( 64 KiB)
    { 64,  64, 1, 10.2f},   // the same kernel, one workgroup per CU
};

// The shape of `shapes` whose rounds of workgroups cost least; tiles may not
// be taller than M rounded up to 64 rows.
inline int pick_tile_shape(const TileShape* shapes, int count, int M, int N)
{
    const int64_t mcap = ((int64_t)M + 63) / 64 * 64;
    int best = -1;
    float best_us = 0.f;
    for (int i = 0; i < count; ++i) {
        const TileShape& t = shapes[i];
        if (t.bm > mcap) continue;
        const int64_t tiles = (((int64_t)M + t.bm - 1) / t.bm) * (((int64_t)N + t.bn - 1) / t.bn);
        const int64_t slots = (int64_t)kCUs * t.per_cu;
        const float us = (float)((tiles + slots - 1) / slots) * t.round_us;
        if (best < 0 || us < best_us) { best = i; best_us = us; }
    }
    return best;
}

template <int WFMT, int OUTF>
hipError_t launch_tile_fmt(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int rowscale, hipStream_t stream)
{
    switch (pick_tile_shape(kTileShapes, sizeof(kTileShapes) / sizeof(kTileShapes[0]), M, N)) {
    case 0: return launch_f8<WFMT, OUTF, 256, 256, 2, 4, 2, 2>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    case 1: return launch_f8<WFMT, OUTF, 256, 192, 2, 4, 2, 3>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    case 2: return launch_f8<WFMT, OUTF, 256, 128, 4, 2, 3, 4>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    case 3: return launch_f8<WFMT, OUTF, 128, 192, 2, 4, 3, 4>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    case 4: return launch_f8<WFMT, OUTF, 128, 128, 2, 4, 4, 4>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    // 8 waves rather than 4 of 64 x 32: a third more LDS reading per step, but
    // two waves per SIMD (O and down projections at M = 512: 2.5% on the step)
    case 5: return launch_f8<WFMT, OUTF, 128, 64, 4, 2, 4, 4>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    default: return launch_f8<WFMT, OUTF, 64, 64, 2, 2, 4, 4>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    }
}

hipError_t launch_tile_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                           hipStream_t stream)
{
    if (wfmt == WF_E4M3 && outf == OUT_BF16)
        return launch_tile_fmt<WF_E4M3, OUT_BF16>(qa, sa, qw, sw, y, M, N, K, rowscale, stream);
    if (wfmt == WF_E5M2 && outf == OUT_FP16 && !rowscale)
        return launch_tile_fmt<WF_E5M2, OUT_FP16>(qa, sa, qw, sw, y, M, N, K, 0, stream);
    if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && !rowscale)
        return launch_tile_fmt<WF_E4M3_SC8, OUT_FP16>(qa, sa, qw, sw, y, M, N, K, 0, stream);
    return hipErrorInvalidValue;
}

template <int BM, int BN, int WM, int WN, int AST, int WST, int SP>
hipError_t launch_n16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo, uint16_t* y,
                      int M, int N, int K, hipStream_t stream)
{
    auto kern = gemm_n16_kernel<BM, BN, WM, WN, AST, WST, SP>;
    constexpr size_t lds = ((size_t)AST * BM + (size_t)WST * BN) * 128;
    static_assert(lds <= 160 * 1024, "LDS of one CU");
    static std::atomic<uint64_t> attr_devices{0};
    if (const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kern), lds, attr_devices);
        e != hipSuccess)
        return e;
    const int64_t grid = (((int64_t)M + BM - 1) / BM) * (((int64_t)N + BN - 1) / BN);
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    kern<<<(int)grid, WM * WN * 64, lds, stream>>>(a, hi, lo, y, M, N, K);
    return hipGetLastError();
}

// Tile shapes of the NestedFP FP16 GEMM with the measured time of one round
// of their workgroups at K = 4096 (MI355X, planes cold in HBM; Llama-7B
// shapes at M = 256 and 2048), picked like the FP8 shapes.
constexpr TileShape kN16Shapes[] = {
    {256, 256, 1, 115.0f},  // 8 waves of 128 x 64, 2 + 2 stages (128 KiB)
    {256, 128, 1, 76.0f},   // 8 waves of  64 x 64, 3 + 4 stages (160 KiB)
    {128, 128, 1, 48.5f},   // 8 waves of  64 x 32, 4 + 4 stages (128 KiB)
    { 64,  64, 2, 39.0f},   // 4 waves of  32 x 32, 4 + 4 stages ( 64 KiB)
    { 64,  64, 1, 25.0f},   // the same kernel, one workgroup per CU
};

template <int SP>
hipError_t launch_tile_nested16_sp(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                   uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    switch (pick_tile_shape(kN16Shapes, sizeof(kN16Shapes) / sizeof(kN16Shapes[0]), M, N)) {
    case 0: return launch_n16<256, 256, 2, 4, 2, 2, SP>(a, hi, lo, y, M, N, K, stream);
    case 1: return launch_n16<256, 128, 4, 2, 3, 4, SP>(a, hi, lo, y, M, N, K, stream);
    case 2: return launch_n16<128, 128, 2, 4, 4, 4, SP>(a, hi, lo, y, M, N, K, stream);
    default: return launch_n16<64, 64, 2, 2, 4, 4, SP>(a, hi, lo, y, M, N, K, stream);
    }
}

hipError_t launch_tile_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream)
{
    return sp == SP_E4M3 ? launch_tile_nested16_sp<SP_E4M3>(a, hi, lo, y, M, N, K, stream)
                         : launch_tile_nested16_sp<SP_PLAIN>(a, hi, lo, y, M, N, K, stream);
}

}  // namespace fp8q
