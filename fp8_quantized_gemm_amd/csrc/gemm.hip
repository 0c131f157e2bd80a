// Prefill-path GEMMs (M > 16): LDS-staged MFMA tile GEMMs.
//
//  - FP8: y = out( (qa . W^T) * scale ) with E4M3 activations and E4M3 (FP8
//    GEMM, page "C++与FP8量化" §3.3) or E5M2 (NestedFP FP8 mode, page
//    "NestedFP双精度推理框架" §2.1) weights.  Two kernels:
//      gemm_f8_tile_kernel  128x128 tiles, v_mfma_f32_16x16x128_f8f6f4,
//                           register-staged double buffer (grids below 512
//                           256x256 tiles);
//      gemm_f8_pipe_kernel  256x256 tiles, v_mfma_f32_32x32x64_f8f6f4, a
//                           4-stage LDS ring filled by direct global->LDS
//                           loads plus register double-buffered operands.
//  - NestedFP FP16 mode (same page, §2.1-§2.2): the weight tile is staged in
//    LDS as its two byte planes and rebuilt as fp16 (hi<<8)|lo with v_perm
//    while it is moved from LDS to registers, then v_mfma_f32_16x16x32_f16.
//
// 128x128 kernels: a 256-thread workgroup computes a 128x128 output tile; its
// 4 waves form a 2x2 grid of 64x64 sub-tiles (4x4 MFMA tiles of 16x16 each).
// Each K step stages the next tiles in registers while the current LDS buffer
// feeds the MFMAs, so one barrier per step suffices.  Rows of A and W are
// K-contiguous; LDS rows hold 16-byte units XOR-swizzled by row so that 16
// lanes reading the same unit of 16 consecutive rows hit distinct banks.
// Workgroup ids are remapped so that consecutive tiles (which share the
// weight tile) land on the same XCD and its L2.
#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;
constexpr int kThreads = 256;
constexpr int kBigTileMinGrid = 512;     // 256 x 256 tiles: two per CU
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

// ---------------------------------------------------------------- FP8 tile GEMM
// BM x BN output tile (BM, BN in {64, 128}) per 256-thread workgroup; the 4
// waves form a 2x2 grid of (BM/2) x (BN/2) sub-tiles of 16x16x128 MFMAs.
// The smaller tiles exist for grids that would otherwise leave CUs idle
// (M = 512 against N = 4096 is 128 tiles of 128x128 for 256 CUs).
template <int WFMT, int OUTF, int BM, int BN>
__global__ __launch_bounds__(kThreads) void gemm_f8_tile_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K)
{
    constexpr int BK = 128;                       // bytes = elements
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int FM = BM / 32, FN = BN / 32;     // 16x16 MFMA tiles per wave
    constexpr int JA = BM / 32, JW = BN / 32;     // 16-byte units per thread per step
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int r = lane & 15, g = lane >> 4;

    const int tiles_m = (M + BM - 1) / BM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * BM;
    const int n0 = (bid / tiles_m) * BN;

    // global -> register staging: thread owns unit (tid & 7) of rows
    // (tid >> 3) + 32 j of the A and the W tile.  Buffer resources span the
    // valid rows of each tile, so rows past M or N and units past K (given an
    // out-of-range offset) read as zero, unpredicated.
    const int su = tid & 7;
    const rsrc_t ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
    const rsrc_t rw = make_rsrc(qw + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));
    uint32_t roff[JA > JW ? JA : JW];
#pragma unroll
    for (int j = 0; j < (JA > JW ? JA : JW); ++j) roff[j] = (uint32_t)(((tid >> 3) + 32 * j) * K + su * 16);
    v4i ra_[JA], rw_[JW];
    auto gload = [&](int kt) {
        const bool kin = kt * BK + su * 16 < K;
#pragma unroll
        for (int j = 0; j < JA; ++j) ra_[j] = buf_load16(ra, kin ? roff[j] + kt * BK : kOOB);
#pragma unroll
        for (int j = 0; j < JW; ++j) rw_[j] = buf_load16(rw, kin ? roff[j] + kt * BK : kOOB);
    };
    auto lstore = [&](int buf) {
        uint8_t* As = lds + buf * STAGE;
        uint8_t* Ws = As + BM * BK;
#pragma unroll
        for (int j = 0; j < JA; ++j)
            *reinterpret_cast<v4i*>(As + swz128((tid >> 3) + 32 * j, su)) = ra_[j];
#pragma unroll
        for (int j = 0; j < JW; ++j)
            *reinterpret_cast<v4i*>(Ws + swz128((tid >> 3) + 32 * j, su)) = rw_[j];
    };

    v4f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + BK - 1) / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        gload(kt + 1);                 // past the end: out-of-range offsets, zeros
        const uint8_t* As = lds + cur * STAGE;
        const uint8_t* Ws = As + BM * BK;
        v8i af[FM], wf[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = wm * (BM / 2) + i * 16 + r;
            af[i] = cat(*reinterpret_cast<const v4i*>(As + swz128(row, g)),
                        *reinterpret_cast<const v4i*>(As + swz128(row, g + 4)));
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = wn * (BN / 2) + j * 16 + r;
            wf[j] = cat(*reinterpret_cast<const v4i*>(Ws + swz128(row, g)),
                        *reinterpret_cast<const v4i*>(Ws + swz128(row, g + 4)));
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af[i], wf[j], acc[i][j], WF_E4M3, WFMT, 0, 0, 0, 0);
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    float s = *sa;
    if (sw != nullptr) s = s * *sw;
    store_tile<OUTF, FM, FN>(y, acc, s, M, N, m0 + wm * (BM / 2), n0 + wn * (BN / 2), r, g);
}

// ---------------------------------------------------------------- FP8 pipelined big-tile GEMM
// BM x BN output tile per workgroup of WM x WN waves, each wave a
// (BM/WM) x (BN/WN) sub-tile of v_mfma_f32_32x32x64_f8f6f4 tiles (the 32x32
// shape reads half the LDS operand bytes per flop of the 16x16 one).
// Operand layout of the 32x32x64 MFMA: lane l supplies row (l % 32) of A (and
// of W) and 32 bytes of K; lane half h = l / 32 takes 16-byte units 2h, 2h+1
// of the 64-byte K step (the same units for A and W).  The result lane l
// holds D[8 (r/4) + 4 h + r % 4][l % 32], r = 0..15.
//
// K steps of 64 bytes flow through a STAGES-deep LDS ring filled by direct
// global->LDS loads (buffer_load ... lds): no register staging and no LDS
// store instructions; the loads of step kt + STAGES - 1 are in flight while
// step kt is multiplied.  LDS rows are 64 bytes (four 16-byte units), unit u
// of row r stored at position u ^ ((r >> 2) & 3), so 16 consecutive rows read
// at one unit touch 16 distinct 16-byte bank groups.  A DMA load writes lane
// l's 16 bytes to slot l of a 1 KiB block (16 rows), so each lane fetches the
// global unit that belongs in its slot.  The compiler does not order LDS
// reads after these asynchronous LDS writes, so every step waits explicitly
// (s_waitcnt vmcnt) for its own loads and then synchronizes the workgroup.
//
// On top of the ring, the MFMA operands are double-buffered in registers:
// after the barrier that publishes stage kt+1, the wave multiplies step kt
// from registers while it reads step kt+1's operands from LDS, the reads
// interleaved between the MFMAs (sched_group_barrier) so that they overlap
// the matrix unit instead of leaving it idle between steps.
constexpr int kDmaBK = 64;

template <int N_OUTSTANDING>
__device__ __forceinline__ void wait_vm()
{
    // s_waitcnt vmcnt(N) with expcnt and lgkmcnt left at their maxima (gfx9 encoding)
    static_assert(N_OUTSTANDING >= 0 && N_OUTSTANDING < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N_OUTSTANDING & 15) | ((N_OUTSTANDING >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <int WFMT, int OUTF, int BM, int BN, int WM, int WN, int STAGES>
__global__ __launch_bounds__(WM * WN * 64) void gemm_f8_pipe_kernel(
    const uint8_t* __restrict__ qa, const float* __restrict__ sa,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, int M, int N, int K)
{
    constexpr int NT = WM * WN * 64;
    constexpr int BK = kDmaBK;
    constexpr int TM = BM / WM, TN = BN / WN;
    constexpr int FM = TM / 32, FN = TN / 32;
    constexpr int STAGE = (BM + BN) * BK;
    constexpr int BLOCKS = STAGE / 1024;
    constexpr int BPW = BLOCKS / (NT / 64);
    static_assert(BPW * (NT / 64) == BLOCKS, "stage must split evenly over waves");
    static_assert(STAGES >= 3, "the ring needs a stage in use, one published and one loading");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int r32 = lane & 31, h = lane >> 5;

    const int tiles_m = (M + BM - 1) / BM;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int m0 = (bid % tiles_m) * BM;
    const int n0 = (bid / tiles_m) * BN;

    const rsrc_t ra = make_rsrc(qa + (size_t)m0 * K, (uint32_t)(min(BM, M - m0) * K));
    const rsrc_t rw = make_rsrc(qw + (size_t)n0 * K, (uint32_t)(min(BN, N - n0) * K));
    uint32_t goff[BPW];
    int gunit[BPW];
    bool is_a[BPW];
#pragma unroll
    for (int j = 0; j < BPW; ++j) {
        const int b = wave * BPW + j;
        const int row = b * 16 + (lane >> 2);
        gunit[j] = (lane & 3) ^ ((row >> 2) & 3);
        is_a[j] = row < BM;
        const int trow = is_a[j] ? row : row - BM;
        goff[j] = (uint32_t)(trow * K + gunit[j] * 16);
    }
    const int nk = (K + BK - 1) / BK;
    auto dma = [&](int kt) {
        uint8_t* st = lds + (kt % STAGES) * STAGE;
#pragma unroll
        for (int j = 0; j < BPW; ++j) {
            const bool kin = kt * BK + gunit[j] * 16 < K;
            dma_load16(is_a[j] ? ra : rw, st + (wave * BPW + j) * 1024,
                       kin ? goff[j] + kt * BK : kOOB);
        }
    };
    // LDS byte offsets (within a stage) of this lane's two units of operand
    // tile 0; tile i adds i * 32 rows.  Tile bases are multiples of 16 rows, so
    // the swizzle term ((row >> 2) & 3) depends on the lane alone.
    const int sw4 = (r32 >> 2) & 3;
    const int a_off0 = (wm * TM + r32) * BK + (((2 * h) ^ sw4) << 4);
    const int a_off1 = (wm * TM + r32) * BK + (((2 * h + 1) ^ sw4) << 4);
    const int w_off0 = (BM + wn * TN + r32) * BK + (((2 * h) ^ sw4) << 4);
    const int w_off1 = (BM + wn * TN + r32) * BK + (((2 * h + 1) ^ sw4) << 4);
    auto read_frags = [&](int kt, v8i (&af)[FM], v8i (&wf)[FN]) {
        const uint8_t* st = lds + (kt % STAGES) * STAGE;
#pragma unroll
        for (int i = 0; i < FM; ++i)
            af[i] = cat(*reinterpret_cast<const v4i*>(st + a_off0 + i * 32 * BK),
                        *reinterpret_cast<const v4i*>(st + a_off1 + i * 32 * BK));
#pragma unroll
        for (int j = 0; j < FN; ++j)
            wf[j] = cat(*reinterpret_cast<const v4i*>(st + w_off0 + j * 32 * BK),
                        *reinterpret_cast<const v4i*>(st + w_off1 + j * 32 * BK));
    };

    typedef float v16f __attribute__((ext_vector_type(16)));
    v16f acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    auto mfmas = [&](const v8i (&af)[FM], const v8i (&wf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    af[i], wf[j], acc[i][j], WF_E4M3, WFMT, 0, 0, 0, 0);
    };
    // wait until at most `later` steps' loads are still in flight
    auto wait_steps = [&](int later) {
        if (later >= 2) wait_vm<2 * BPW>();
        else if (later == 1) wait_vm<BPW>();
        else wait_vm<0>();
    };

#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
        if (p < nk) dma(p);

    v8i af0[FM], wf0[FN], af1[FM], wf1[FN];
    wait_steps(min(STAGES - 2, nk - 1));
    __syncthreads();
    read_frags(0, af0, wf0);

    auto interleave = [&]() {
#pragma unroll
        for (int q = 0; q < FM * FN; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);     // two LDS reads
        }
    };
    // one iteration = two K steps, so the two register sets swap roles by name
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
        // step kt: read step kt+1 into set 1 while multiplying set 0
        wait_steps(min(STAGES - 3, nk - 2 - kt));
        __syncthreads();                       // stage kt+1 published; stage kt-1 free
        if (kt + STAGES - 1 < nk) dma(kt + STAGES - 1);
        read_frags(kt + 1, af1, wf1);
        mfmas(af0, wf0);
        interleave();
        // step kt+1: read step kt+2 into set 0 while multiplying set 1
        if (kt + 2 < nk) {
            wait_steps(min(STAGES - 3, nk - 3 - kt));
            __syncthreads();
            if (kt + STAGES < nk) dma(kt + STAGES);
            read_frags(kt + 2, af0, wf0);
        }
        mfmas(af1, wf1);
        interleave();
    }
    if (kt < nk) mfmas(af0, wf0);              // odd number of steps: the last one

    float sc = *sa;
    if (sw != nullptr) sc = sc * *sw;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * TN + j * 32 + r32;
            if (n >= N) continue;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + wm * TM + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < M) y[(size_t)m * N + n] = (uint16_t)f32_to_out_bits<OUTF>(acc[i][j][e] * sc);
            }
        }
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

template <int WFMT, int OUTF, int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_pipe(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    auto kern = gemm_f8_pipe_kernel<WFMT, OUTF, BM, BN, WM, WN, STAGES>;
    constexpr size_t lds = (size_t)STAGES * (BM + BN) * kDmaBK;
    static bool attr_set = false;        // idempotent host attribute, set on first use
    if (!attr_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize,
                                                 (int)lds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    kern<<<grid, WM * WN * 64, lds, stream>>>(qa, sa, qw, sw, y, M, N, K);
    return hipGetLastError();
}

template <int WFMT, int OUTF, int BM, int BN>
hipError_t launch_tile(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    const int grid = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    gemm_f8_tile_kernel<WFMT, OUTF, BM, BN><<<grid, kThreads, 0, stream>>>(qa, sa, qw, sw, y, M, N, K);
    return hipGetLastError();
}

template <int WFMT, int OUTF>
hipError_t launch_tile_fmt(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, hipStream_t stream)
{
    auto tiles = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    // Tile shape by grid fill, from measurements on MI355X over the Llama-7B
    // and Qwen-32B prefill shapes: 256 x 256 pipelined tiles once there are
    // at least two per CU; 128 x 128 when its tiles fill whole rounds of the
    // 512 that fit at once (two per CU, 64 KiB of LDS each) to at least 90%;
    // else 128 x 64 if that still gives two workgroups per CU; else 64 x 64.
    const int64_t t128 = tiles(128, 128);
    const int64_t rounds = (t128 + 2 * kCUs - 1) / (2 * kCUs);
    if (tiles(256, 256) >= kBigTileMinGrid)
        return launch_pipe<WFMT, OUTF, 256, 256, 4, 2, 4>(qa, sa, qw, sw, y, M, N, K, stream);
    if (t128 >= 2 * kCUs && 10 * t128 >= 9 * rounds * 2 * kCUs)
        return launch_tile<WFMT, OUTF, 128, 128>(qa, sa, qw, sw, y, M, N, K, stream);
    if (tiles(128, 64) >= 2 * kCUs) return launch_tile<WFMT, OUTF, 128, 64>(qa, sa, qw, sw, y, M, N, K, stream);
    return launch_tile<WFMT, OUTF, 64, 64>(qa, sa, qw, sw, y, M, N, K, stream);
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
