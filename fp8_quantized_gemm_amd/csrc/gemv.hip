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
// [64+16g, 64+16g+16) of each 128-byte K block.  Loaded in that layout, an
// instruction would read 64 bytes of each of 16 rows, half of every line;
// the FP8 weights are instead loaded as whole lines and exchanged across
// lanes into it (wline, w_to_mfma), the activations directly.  The result
// lane l holds D[4g + i][l % 16], i = 0..3.
#include <algorithm>

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

// Weight loads of whole 128-byte lines.  For one 128-byte K block of a
// 16-row tile, load A takes rows 0..7 and load B rows 8..15: lane l reads the
// 16-byte unit l & 7 of row l >> 3 (A) and the unit ((l & 7) + 4) & 7 of row
// 8 + (l >> 3) (B), so that each instruction reads eight whole lines and the
// loads can be non-temporal (the operand layout's 64-byte halves needed the
// line kept in L2 between the two loads of each line).  WLine holds a lane's
// byte offsets within the tile and the K offsets of its units.
struct WLine {
    uint32_t oa, ob;   // byte offset in the tile of the lane's unit of A / B in block 0
    int ua, ub;        // K offset of that unit within a block
};
__device__ __forceinline__ WLine wline(int lane, int K)
{
    const int ua = lane & 7, ub = ((lane & 7) + 4) & 7;
    return WLine{(uint32_t)((lane >> 3) * K + ua * 16), (uint32_t)(((lane >> 3) + 8) * K + ub * 16),
                 ua * 16, ub * 16};
}

// The loaded units into the MFMA operand layout: lane L = r + 16 g gets
// units g (lo) and 4 + g (hi) of row r.  Rows r < 8 read from A and rows
// r >= 8 from B; with B's units rotated by four, the lanes that a lo (hi)
// exchange reads are all distinct, so a per-lane select of A or B on the
// source side (lanes with l & 4 give B to lo, A to hi) and one ds_bpermute
// per dword do it: 8 selects and 8 permutes per 2 KiB block.  The result is
// bit for bit the operand the 64-byte-half loads gave.
__device__ __forceinline__ v8i w_to_mfma(const v4i& a, const v4i& b, int lane)
{
    const int r = lane & 15, g = lane >> 4, up = r >> 3;
    const int base = (r & 7) * 8 + g;
    const int alo = (base + 4 * up) << 2, ahi = (base + 4 - 4 * up) << 2;
    const bool sel = (lane & 4) != 0;
    v8i w;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        w[d] = __builtin_amdgcn_ds_bpermute(alo, sel ? b[d] : a[d]);
        w[4 + d] = __builtin_amdgcn_ds_bpermute(ahi, sel ? a[d] : b[d]);
    }
    return w;
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
// back before the first MFMA waits on them.  With TPW = 2 a workgroup takes
// two adjacent tiles and each activation fragment feeds both tiles' MFMAs (a
// second tile past N has an empty resource and stores nothing).
template <int WFMT, int OUTF, int WAVES, int U, int CP, int TPW = 1>
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
    // TPW consecutive 16-row tiles; their weight loads share each activation load
    const int n0 = blockIdx.x * 16 * TPW;
    int rows[TPW];
    rsrc_t rw[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        rows[t] = max(0, min(16, N - n0 - 16 * t));
        rw[t] = make_rsrc(qw + (size_t)(n0 + 16 * t) * K, (uint32_t)(rows[t] * K));
    }
    const rsrc_t ra = make_rsrc(qa, (uint32_t)(M * K));
    const uint32_t row_off = (uint32_t)(r * K);   // past the resource for padded rows
    const WLine wl = wline(lane, K);

    const int nblk = (K + 127) >> 7;
    v4f acc[TPW];
#pragma unroll
    for (int t = 0; t < TPW; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * U) {
        v4i w0[TPW][U], w1[TPW][U], a0[U], a1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (kb0 + u * WAVES) * 128;
            const int k0 = kb + g * 16;
            const int k1 = k0 + 64;
            const uint32_t o0 = k0 < K ? row_off + k0 : kOOB;
            const uint32_t o1 = k1 < K ? row_off + k1 : kOOB;
            const uint32_t pa = kb + wl.ua < K ? wl.oa + kb : kOOB;
            const uint32_t pb = kb + wl.ub < K ? wl.ob + kb : kOOB;
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                w0[t][u] = buf_load16<CP>(rw[t], pa);
                w1[t][u] = buf_load16<CP>(rw[t], pb);
            }
            a0[u] = buf_load16(ra, o0);
            a1[u] = buf_load16(ra, o1);
        }
        // keep every load of the batch ahead of the first MFMA
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < TPW; ++t)
                acc[t] = mfma_f8<WFMT>(cat(a0[u], a1[u]), w_to_mfma(w0[t][u], w1[t][u], lane), acc[t]);
    }

    const float s_w = (sw != nullptr) ? *sw : implied_wscale(WFMT);
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        if (t > 0) __syncthreads();                // red is reused
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[t][i];
        __syncthreads();
        const int nt = n0 + 16 * t;
        for (int e = threadIdx.x; e < M * 16; e += WAVES * 64) {
            const int m = e >> 4, c = e & 15;
            if (c >= rows[t]) continue;
            float v = red[0][m][c];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) v += red[w][m][c];
            const float s = rowscale ? sa[m] * sw[nt + c] : *sa * s_w;
            y[(size_t)m * N + nt + c] = (uint16_t)f32_to_out_bits<OUTF>(v * s);
        }
    }
}

// ---------------------------------------------------------------- quantize + FP8 GEMV, one launch
// The whole linear layer (dynamic per-tensor activation quantization, then
// the GEMM) for 3 <= M <= 16 and M*K <= kFusedGemvMaxMK, on a grid of at
// most two workgroups per CU that loop over the 16-row weight tiles t =
// blockIdx.x, blockIdx.x + gridDim.x, ...  Each workgroup first reads all of
// x (from L2 after the first ones), reduces its amax and quantizes it into
// LDS with the standalone quantizer's scale and rounding, so its codes are
// bit-identical; workgroup 0 also stores q, *scale and *amax.  That prologue
// runs once per workgroup, not once per tile.  The weights stream as in
// gemv_f8_kernel, with the activation fragments read from LDS.
//
// Thread t handles vectors t, t + NT, ... (XV of them at most) of the
// row-major activation, 8 elements each (K % 16 == 0: a vector never
// straddles two rows).  Up to four vectors stay in registers from the amax
// to the quantization; with eight, x is read a second time (L2 hits) to
// quantize.  Loads return in order, so with one or two vectors the first
// batch of weight loads is issued right after the activation loads and is
// in flight during the prologue; with more it follows the prologue (beside
// the vectors it would not fit in 64 VGPRs, which keeps two workgroups per
// CU).  Each next tile's first batch is issued before the current tile's
// epilogue.
//
// LDS (at most 80 KiB): the codes, row m at m * K, its 16-byte unit c at
// unit c ^ (m & 15) within each complete group of 16 units (so the 16 rows
// of a fragment read fall on different banks); then the wave partials of the
// epilogue, whose first WAVES floats hold the per-wave maxima of the prologue.
__device__ __forceinline__ int code_unit(int m, int c, int units)
{
    return (c | 15) < units ? c ^ (m & 15) : c;
}

template <int DT, int WFMT, int OUTF, int WAVES, int U, int XV>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(8, 8)))
void gemv_f8_fused_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, uint8_t* __restrict__ q, float* __restrict__ scale,
    float* __restrict__ amax_out, int M, int N, int K)
{
    constexpr int NT = WAVES * 64;
    constexpr bool kHold = XV <= 4;            // vectors kept from amax to quantization
    constexpr bool kEarlyW = XV <= 2;          // first weight batch ahead of the prologue
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    float(*red)[16][16] = reinterpret_cast<float(*)[16][16]>(lds + M * K);
    float* const wmax = &red[0][0][0];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 15;
    const int g = lane >> 4;
    const int tiles = (N + 15) >> 4;
    const int units = K >> 4;

    const int nvec = (M * K) >> 3;
    const v4i* xv = reinterpret_cast<const v4i*>(x);
    auto load_x = [&](v4i (&v)[XV]) {
#pragma unroll
        for (int j = 0; j < XV; ++j) {
            const int i = tid + j * NT;
            v[j] = i < nvec ? xv[i] : v4i{0, 0, 0, 0};
        }
    };

    // weight loads: batch of blocks kb0, kb0 + WAVES, ... of the current tile
    // (whole lines, non-temporal; see wline)
    const int nblk = (K + 127) >> 7;
    v4i w0[U], w1[U];
    auto load_w = [&](const rsrc_t& rw, int kb0) {
        // the lane's offsets are recomputed for each batch rather than held
        // across the prologue and the tile loop (which spilled at 64 VGPRs)
        int l = lane;
        asm volatile("" : "+v"(l));
        const WLine wl = wline(l, K);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (kb0 + u * WAVES) * 128;
            w0[u] = buf_load16<CP_NT>(rw, kb + wl.ua < K ? wl.oa + kb : kOOB);
            w1[u] = buf_load16<CP_NT>(rw, kb + wl.ub < K ? wl.ob + kb : kOOB);
        }
    };
    auto tile_rsrc = [&](int t) {
        const int n0 = t * 16;
        return make_rsrc(qw + (size_t)n0 * K, (uint32_t)(min(16, N - n0) * K));
    };

    // amax of the whole activation
    v4i v[XV];
    load_x(v);
    __builtin_amdgcn_sched_barrier(0);
    rsrc_t rw = tile_rsrc(blockIdx.x);
    if constexpr (kEarlyW) load_w(rw, wave);
    __builtin_amdgcn_sched_barrier(0);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < XV; ++j) m = fmaxf(m, vec_absmax<DT>(v[j]));
    m = wave_max(m);
    if (lane == 0) wmax[wave] = m;
    lds_barrier();
    float a = wmax[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) a = fmaxf(a, wmax[w]);
    const float s = scale_from_amax(a);
    const Quotient d(s);

    // codes into LDS (and q from workgroup 0)
    if constexpr (!kHold) load_x(v);
    const int kv = K >> 3;
    v2i* const qv = reinterpret_cast<v2i*>(q);
#pragma unroll
    for (int j = 0; j < XV; ++j) {
        const int i = tid + j * NT;
        if (i < nvec) {
            const v2i c = vec_quantize<DT>(v[j], d);
            const int row = i / kv;
            const int col8 = i - row * kv;     // 8-byte half col8 & 1 of unit col8 >> 1
            *reinterpret_cast<v2i*>(lds + row * K + code_unit(row, col8 >> 1, units) * 16 +
                                    (col8 & 1) * 8) = c;
            if (blockIdx.x == 0) qv[i] = c;
        }
        // one vector at a time: interleaving them would need more than 64 VGPRs
        __builtin_amdgcn_sched_barrier(0);
    }
    if (blockIdx.x == 0 && tid == 0) {
        *scale = s;
        *amax_out = a;
    }
    if constexpr (!kEarlyW) load_w(rw, wave);
    lds_barrier();

    // activation row r of this lane (rows past M read as zero)
    const bool arow = r < M;
    const uint8_t* const ar = lds + (arow ? r : 0) * K;
    auto afrag = [&](int k) {
        const int c = k < K ? k >> 4 : 0;
        const v4i cv = *reinterpret_cast<const v4i*>(ar + code_unit(r, c, units) * 16);
        return (arow && k < K) ? cv : v4i{0, 0, 0, 0};
    };
    const float sc = s * ((sw != nullptr) ? *sw : implied_wscale(WFMT));

    for (int t = blockIdx.x; t < tiles; t += gridDim.x) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        for (int kb0 = wave;;) {
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k0 = (kb0 + u * WAVES) * 128 + g * 16;
                acc = mfma_f8<WFMT>(cat(afrag(k0), afrag(k0 + 64)), w_to_mfma(w0[u], w1[u], lane), acc);
                // one block's exchange at a time (64 VGPRs)
                __builtin_amdgcn_sched_barrier(0);
            }
            kb0 += WAVES * U;
            if (kb0 >= nblk) break;
            // the next batch reuses the registers of this one
            __builtin_amdgcn_sched_barrier(0);
            load_w(rw, kb0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][4 * g + i][r] = acc[i];
        __builtin_amdgcn_sched_barrier(0);
        // the next tile's first batch goes out before this tile's epilogue
        const int tn = t + (int)gridDim.x;
        if (tn < tiles) {
            rw = tile_rsrc(tn);
            load_w(rw, wave);
        }
        lds_barrier();
        const int n0 = t * 16;
        const int rows = min(16, N - n0);
        for (int e = tid; e < M * 16; e += NT) {
            const int mm = e >> 4, c = e & 15;
            if (c >= rows) continue;
            float vsum = red[0][mm][c];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) vsum += red[w][mm][c];
            y[(size_t)mm * N + n0 + c] = (uint16_t)f32_to_out_bits<OUTF>(vsum * sc);
        }
        lds_barrier();                         // red is free for the next tile
    }
}

// ---------------------------------------------------------------- NestedFP FP16 GEMV
// y[m, n] = fp16( sum_k a[m,k] * fp16((hi[n,k] << 8) | lo[n,k]) ).
// A K block is 128 elements, one 128-byte line of each plane row.  Each plane
// is read as whole lines with non-temporal loads: load A takes rows 0..7 of
// the tile, lane l the 16-byte unit l & 7 of row l >> 3, and load B rows
// 8..15 with the units of each pair swapped (unit (l & 7) ^ 1), and
// plane_to_mfma gives lane L = r + 16 g the units 2g and 2g + 1 of row r
// (elements [32g, 32g + 32) of the block); the activation elements of the
// same positions are loaded directly (four 16-byte pieces).  Each unit is
// rebuilt into 16 fp16 words and feeds two 16x16x32 MFMAs.
struct PLine {
    uint32_t oa, ob;   // byte offset in the tile of the lane's unit of A / B in block 0
    int ua, ub;        // K offset of that unit within a block
};
__device__ __forceinline__ PLine pline(int lane, int K)
{
    const int ua = lane & 7, ub = (lane & 7) ^ 1;
    return PLine{(uint32_t)((lane >> 3) * K + ua * 16), (uint32_t)(((lane >> 3) + 8) * K + ub * 16),
                 ua * 16, ub * 16};
}

// Lane L = r + 16 g gets units 2g (u0) and 2g + 1 (u1) of row r from the two
// whole-line loads: with B's pairs swapped the lanes each exchange reads are
// all distinct, so a per-lane select on the source side (odd lanes give B to
// u0, A to u1) and one ds_bpermute per dword do it.
__device__ __forceinline__ void plane_to_mfma(const v4i& a, const v4i& b, int lane, v4i& u0, v4i& u1)
{
    const int r = lane & 15, g = lane >> 4, up = r >> 3;
    const int base = (r & 7) * 8 + 2 * g;
    const int s0 = (base + up) << 2, s1 = (base + 1 - up) << 2;
    const bool odd = (lane & 1) != 0;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        u0[d] = __builtin_amdgcn_ds_bpermute(s0, odd ? b[d] : a[d]);
        u1[d] = __builtin_amdgcn_ds_bpermute(s1, odd ? a[d] : b[d]);
    }
}

// 16 bytes of each plane (16 elements) -> two MFMAs on activation pieces x0, x1
template <int SP>
__device__ __forceinline__ v4f nested_unit_mfma(const v4i& hv, const v4i& lv, const v4i& x0,
                                                const v4i& x1, v4f acc)
{
    uint32_t w[8];
    nested_rebuild4<SP>((uint32_t)hv[0], (uint32_t)lv[0], w[0], w[1]);
    nested_rebuild4<SP>((uint32_t)hv[1], (uint32_t)lv[1], w[2], w[3]);
    nested_rebuild4<SP>((uint32_t)hv[2], (uint32_t)lv[2], w[4], w[5]);
    nested_rebuild4<SP>((uint32_t)hv[3], (uint32_t)lv[3], w[6], w[7]);
    const v4i wlo = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    const v4i whi = {(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x0),
                                                 __builtin_bit_cast(v8h, wlo), acc, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(v8h, x1),
                                                  __builtin_bit_cast(v8h, whi), acc, 0, 0, 0);
}

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
    const uint32_t row_off = (uint32_t)(r * K);   // past the resource for padded rows
    const PLine pl = pline(lane, K);

    const int nblk = (K + 127) >> 7;
    v4f acc = {0.f, 0.f, 0.f, 0.f};

    for (int kb0 = wave; kb0 < nblk; kb0 += WAVES * U) {
        v4i ha[U], hb[U], la[U], lb[U], x[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kb = (kb0 + u * WAVES) * 128;
            const uint32_t pa = kb + pl.ua < K ? pl.oa + kb : kOOB;
            const uint32_t pb = kb + pl.ub < K ? pl.ob + kb : kOOB;
            ha[u] = buf_load16<CP>(rh, pa);
            hb[u] = buf_load16<CP>(rh, pb);
            la[u] = buf_load16<CP>(rl, pa);
            lb[u] = buf_load16<CP>(rl, pb);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int k = kb + 32 * g + 8 * j;   // K % 16 == 0: a piece is all in or all out
                x[u][j] = buf_load16(ra, k < K ? 2 * (row_off + k) : kOOB);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v4i h0, h1, l0, l1;
            plane_to_mfma(ha[u], hb[u], lane, h0, h1);
            plane_to_mfma(la[u], lb[u], lane, l0, l1);
            acc = nested_unit_mfma<SP>(h0, l0, x[u][0], x[u][1], acc);
            acc = nested_unit_mfma<SP>(h1, l1, x[u][2], x[u][3], acc);
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
// per 16-row tile; the NestedFP FP16 GEMV keeps 4 waves of 4 blocks.  The FP8
// weights are read as whole lines with non-temporal loads and exchanged into
// the operand layout (wline, w_to_mfma): decode steps at M = 4 / 8 3.55 ->
// 3.75 / 3.34 -> 3.53-3.67 TB/s, Qwen-32B M = 16 2.94 -> 3.51-3.64 TB/s,
// against loads of 64-byte halves in the operand layout, which needed the
// default cache policy to keep each line in L2 for its second half (with
// non-temporal halves 18-22% slower on the large projections).
constexpr int kGemvWaves = 16;
constexpr int kGemvUnroll = 2;
// workgroups of the one-launch linear: two per CU of an MI355X at most, the
// 16-row tiles dealt out to them in turn.  Each workgroup pays the prologue,
// so the grid is as small as the tiles allow (`per` tiles per workgroup)
// unless a full grid lowers the most tiles any CU streams: the dispatcher
// gives every CU one of the first 256 workgroups and one of the rest, so with
// 2 x 256 workgroups a CU streams at most ceil(tiles / 256) tiles (768 tiles:
// three per CU, where 384 workgroups of two left half the CUs with four;
// measured on the QKV projection at M = 4 / 8: 13.5 -> 12.0 / 14.8 -> 13.4 us).
constexpr int kCUs = 256;                  // compute units of an MI355X
constexpr int kGemvSlots = 2 * kCUs;
inline int64_t gemv_tiles_per_workgroup(int64_t N)
{
    const int64_t tiles = (N + 15) / 16;
    return (tiles + kGemvSlots - 1) / kGemvSlots;
}
inline int64_t gemv_grid(int64_t N)
{
    const int64_t tiles = (N + 15) / 16;
    const int64_t per = gemv_tiles_per_workgroup(N);
    const int64_t tight = (tiles + per - 1) / per;
    const int64_t most_tight = (tight > kCUs ? 2 : 1) * per;
    const int64_t most_full = (tiles + kCUs - 1) / kCUs;
    return most_full < most_tight ? std::min<int64_t>(tiles, kGemvSlots) : tight;
}
// From this many 16-row tiles (N >= 16384, at least 512 workgroups left) the
// E4M3 GEMV gives each workgroup two adjacent tiles, one block per wave
// step: 6 load instructions per 4 KiB of weights instead of 8.  Measured on
// the Qwen-32B gate+up projection (N = 55296, K = 5120) at M = 16, where
// half of a single tile's loads are activation fragments: decode step
// 2.70 -> 2.86-2.95 TB/s.
constexpr int64_t kGemvPairedTiles = 2 * kGemvSlots;
constexpr int kNestedWaves = 4;
constexpr int kNestedUnroll = 2;   // 128-element blocks: the bytes in flight of 4 blocks of 64

}  // namespace

hipError_t launch_gemv_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                           hipStream_t stream)
{
    const int64_t tiles = ((int64_t)N + 15) / 16;
    const dim3 block(kGemvWaves * 64), grid((unsigned)tiles);
    if (wfmt == WF_E4M3 && outf == OUT_BF16 && tiles >= kGemvPairedTiles)
        gemv_f8_kernel<WF_E4M3, OUT_BF16, kGemvWaves, 1, CP_NT, 2>
            <<<dim3((unsigned)((tiles + 1) / 2)), block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, rowscale);
    else if (wfmt == WF_E4M3 && outf == OUT_BF16)
        gemv_f8_kernel<WF_E4M3, OUT_BF16, kGemvWaves, kGemvUnroll, CP_NT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, rowscale);
    else if (wfmt == WF_E5M2 && outf == OUT_FP16 && !rowscale)
        gemv_f8_kernel<WF_E5M2, OUT_FP16, kGemvWaves, kGemvUnroll, CP_NT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, 0);
    else if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && !rowscale)
        gemv_f8_kernel<WF_E4M3_SC8, OUT_FP16, kGemvWaves, kGemvUnroll, CP_NT>
            <<<grid, block, 0, stream>>>(qa, sa, qw, sw, y, M, N, K, 0);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

namespace {

template <int DT, int WFMT, int OUTF, int XV>
hipError_t launch_gemv_fused_xv(const void* x, const uint8_t* qw, const float* sw, uint16_t* y,
                                uint8_t* q, float* scale, float* amax, int M, int N, int K,
                                hipStream_t stream)
{
    auto kern = gemv_f8_fused_kernel<DT, WFMT, OUTF, kGemvWaves, kGemvUnroll, XV>;
    constexpr size_t kRed = (size_t)kGemvWaves * 16 * 16 * 4;
    static_assert(kFusedGemvMaxMK + kRed <= 80 * 1024, "two workgroups per CU");
    const size_t lds = (size_t)M * K + kRed;
    static std::atomic<uint64_t> attr_devices{0};
    if (const hipError_t e = set_lds_limit_once(reinterpret_cast<const void*>(kern),
                                                (size_t)kFusedGemvMaxMK + kRed, attr_devices);
        e != hipSuccess)
        return e;
    kern<<<(unsigned)gemv_grid(N), kGemvWaves * 64, lds, stream>>>(static_cast<const uint16_t*>(x), qw,
                                                                   sw, y, q, scale, amax, M, N, K);
    return hipGetLastError();
}

template <int DT, int WFMT, int OUTF>
hipError_t launch_gemv_fused_fmt(const void* x, const uint8_t* qw, const float* sw, uint16_t* y,
                                 uint8_t* q, float* scale, float* amax, int M, int N, int K,
                                 hipStream_t stream)
{
    // vectors of 8 elements per thread
    const int per = (int)(((int64_t)M * K / 8 + kGemvWaves * 64 - 1) / (kGemvWaves * 64));
    if (per <= 1) return launch_gemv_fused_xv<DT, WFMT, OUTF, 1>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    if (per <= 2) return launch_gemv_fused_xv<DT, WFMT, OUTF, 2>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    if (per <= 4) return launch_gemv_fused_xv<DT, WFMT, OUTF, 4>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    return launch_gemv_fused_xv<DT, WFMT, OUTF, 8>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
}

}  // namespace

bool linear_gemv_fused_pays(int64_t M, int64_t N, int64_t K)
{
    // Measured on the Llama-7B decode linears at M = 4, 8, 16: with up to four
    // activation vectors per thread the one launch beats quantizer + GEMV on
    // every shape; with eight (x read twice, the first weight batch after the
    // prologue) only where a workgroup covers three or more tiles.
    if (M < 3 || M > 16 || (K & 15) != 0) return false;
    if (M * K <= 4 * 8 * kGemvWaves * 64) return true;
    return M * K <= kFusedGemvMaxMK && gemv_tiles_per_workgroup(N) >= 3;
}

hipError_t launch_linear_gemv_fused(const void* x, int dtype, const uint8_t* qw, const float* sw,
                                    uint16_t* y, uint8_t* q, float* scale, float* amax, int M,
                                    int N, int K, int wfmt, int outf, hipStream_t stream)
{
    static_assert(kFusedGemvMaxMK / 8 <= 8 * kGemvWaves * 64, "XV = 8 covers the largest activation");
    if (M < 1 || M > 16 || (int64_t)M * K > kFusedGemvMaxMK || (K & 15) != 0) return hipErrorInvalidValue;
    if (wfmt == WF_E4M3 && outf == OUT_BF16 && dtype == DT_BF16)
        return launch_gemv_fused_fmt<DT_BF16, WF_E4M3, OUT_BF16>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    if (wfmt == WF_E4M3 && outf == OUT_BF16 && dtype == DT_FP16)
        return launch_gemv_fused_fmt<DT_FP16, WF_E4M3, OUT_BF16>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    if (wfmt == WF_E5M2 && outf == OUT_FP16 && dtype == DT_FP16)
        return launch_gemv_fused_fmt<DT_FP16, WF_E5M2, OUT_FP16>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && dtype == DT_FP16)
        return launch_gemv_fused_fmt<DT_FP16, WF_E4M3_SC8, OUT_FP16>(x, qw, sw, y, q, scale, amax, M, N, K, stream);
    return hipErrorInvalidValue;
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
