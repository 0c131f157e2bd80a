// Decode path for M <= 2 activation rows: row-contiguous weight streaming,
// and the fused decode linear (dynamic activation quantization + FP8 GEMM in
// one launch).
//
// The weight matrix is read once and dominates the bytes (page "7B参数模型在
// 消费级GPU上的极限" §1: memory bandwidth is the first bottleneck of token
// generation), so the access pattern is chosen for HBM: each wave streams
// its weight rows with every lane reading 16 consecutive bytes, i.e. 1 KiB
// of one row per load instruction, rather than the 16-rows-by-64-bytes
// pattern the MFMA operand layout would impose.  The products still run on
// the matrix cores: with at most two activation rows an MFMA is computed on
// its diagonal (each lane pairs its own weight bytes with the activation
// codes of the same positions, see the main loop), one 16x16x128 FP8 MFMA
// per 2 KiB of weights and activation row, so the VALU does no per-element
// work.  (Measured on MI355X, Llama-7B decode step: decoding both operands to
// fp32 and multiplying on the VALU, 48 instructions per 16 weight bytes,
// held the stream back; fp16 pairs with v_dot2_f32_f16, 16 instructions,
// were 7% faster; the MFMA diagonal another 2%.)  Each wave finishes its dot
// products with a 64-lane sum.
//
// The fused variant quantizes the bf16/fp16 activation itself: every
// workgroup reduces amax over the whole activation (L2-resident), computes
// s = amax/448 and the E4M3 codes with the same device routines as
// fp8_quantize_act, keeps the codes in LDS, and workgroup 0 also writes the
// codes, scale and amax to memory.  The activation loads and then the first
// batch of weight loads are issued before this prologue, so the prologue
// waits only for the activation and HBM is busy while it runs.  The FP8 GEMM is the one
// of page "C++与FP8量化" §3.3; the quantization follows the page on a 7B
// model on an RTX 4060, §2.2 and §6.1.
#include <type_traits>

#include "common.hpp"

namespace fp8q {
namespace {

constexpr int kThreads = 256;     // NestedFP kernel: 4 waves, each owning ROWS weight rows
constexpr int kRows = 2;
constexpr int kUnroll = 4;        // 1 KiB chunks per row in flight per wave
constexpr int kWgThreads = 1024;  // FP8 kernel: 16 waves per workgroup
constexpr int kCUs = 256;         // compute units of an MI355X
// FP8 kernel configuration, measured on MI355X over the Llama-7B / Qwen-32B
// decode shapes: one activation row runs 2 KiB batches and two workgroups per
// CU (57 VGPRs, 32 waves per CU); two activation rows need more registers and
// run one workgroup per CU.
template <int MR> struct RowkCfg;
template <> struct RowkCfg<1> { static constexpr int U = 2, WPC = 2; };
template <> struct RowkCfg<2> { static constexpr int U = 2, WPC = 1; };
constexpr int kPartMax = 1024;    // per-workgroup partial sums of the split-K decode kernel

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ v8i cat8(const v4i& lo, const v4i& hi)
{
    return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// ---------------------------------------------------------------- FP8 / BF8 weights
// Activation source of the FP8 kernel.
enum : int {
    AS_GLOBAL = 0,   // E4M3 codes read from memory (L2) in the main loop
    AS_COPY = 1,     // E4M3 codes copied into LDS once per workgroup
    AS_BF16 = 2,     // bf16 activation quantized into LDS once per workgroup (fused)
    AS_FP16 = 3,     // fp16 activation quantized into LDS once per workgroup (fused)
};

// y[m, n] = out( sum_k dec(a[m,k]) * dec(W[n,k]) * scale(m, n) ), where
// scale(m, n) = fl32(s_a * s_w) with one activation scale and one weight scale
// (*sw, or 1 without weight scales), or, with rowscale set, fl32(s_a[m] *
// s_w[n]) with a scale per activation row (token) and per weight row (output
// channel).  The fused prologue then reduces amax per activation row.
//
// At most WPC workgroups of NT threads (W = NT / 64 waves) per CU: the
// activation prologue (copy or quantization into LDS) is paid once per
// workgroup and spread over its waves.  NT is 1024 or 512 and the batch U is
// 2, 3 or 4 KiB, chosen per call by launch_rowk.
// Each workgroup takes one contiguous span of weight rows, so that at any
// moment it streams one compact window of the weight matrix: measured on
// MI355X, block-contiguous streaming with non-temporal loads sustains about
// 7.1 TB/s where grid-strided streaming stays near 6 TB/s.  The K range of a
// row is cut into S = 2^ls equal segments (a multiple of 128 bytes each), so
// that a span holds S units per row; the W waves take consecutive units in
// turn, which keeps wave w on segment w % S.  A wave streams its segment in
// batches of U 1 KiB chunks; the 4 waves per SIMD overlap each other's loads
// and arithmetic.  With S = 1 a wave finishes a row itself; with S > 1 the
// per-segment sums go to LDS and are added in segment order after one
// barrier, so the result is deterministic.  The host picks S (see
// rowk_split_shift): splitting pays where a span has fewer rows than waves or
// a row's last batch is mostly empty.  The activation and then the first
// weight batch are requested before the prologue.
//
// With DS (delayed scaling, fused prologue only) the activation scale is the
// one the amax history gives (delayed_scale), so the prologue quantizes as
// soon as the activation arrives, without a block-wide amax first; each
// workgroup computes the amax of the whole activation in its prologue and
// counts itself at its end (delayed_arrive), and the one that arrives last
// publishes the call.
template <int NT, int WFMT, int OUTF, int AS, int MR, int U, int CP, int WPC, int XV, bool DS = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT / 256 * WPC)))
void rowk_f8_kernel(
    const void* __restrict__ act, const float* __restrict__ sa_in,
    const uint8_t* __restrict__ qw, const float* __restrict__ sw,
    uint16_t* __restrict__ y, uint8_t* __restrict__ q_out, float* __restrict__ sa_out,
    float* __restrict__ amax_out, int N, int K, int rpw, int ls, int kseg, int rowscale,
    float* __restrict__ history, int64_t hist_len, uint32_t* __restrict__ state, int act_first)
{
    constexpr bool FUSED = AS == AS_BF16 || AS == AS_FP16;
    static_assert(!DS || FUSED, "delayed scaling belongs to the fused prologue");
    constexpr bool IN_LDS = AS != AS_GLOBAL;
    constexpr int DT = AS == AS_BF16 ? DT_BF16 : DT_FP16;
    constexpr int W = NT / 64;
    extern __shared__ __attribute__((aligned(16))) uint8_t codes_lds[];   // IN_LDS: MR*K codes
    __shared__ float red[MR][W];
    __shared__ float part[kPartMax];   // S > 1: [m][row of the span][segment]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int S = 1 << ls;
    const int seg = wave & (S - 1);
    // rows [rbeg, rbeg + nrows) of this workgroup (rpw rows per workgroup;
    // 64-bit: N may come within a span of 2^31); the host computes rpw and
    // the segment length kseg, so that the setup every wave runs before its
    // first load (on the CU's one scalar unit) stays short
    const int64_t rbeg = (int64_t)blockIdx.x * rpw;
    const int nrows = (int)max((int64_t)0, min((int64_t)rpw, (int64_t)N - rbeg));
    const int nunits = nrows << ls;    // S > 1 only when MR * nrows * S <= kPartMax
    const int klo = min(K, seg * kseg), khi = min(K, klo + kseg);
    const int nkb = (khi - klo + 1024 * U - 1) / (1024 * U);

    v4i w[U];
    // weights of `row` at K offsets [kb, kb + U KiB) clipped to the segment;
    // an empty resource (!valid) makes every load read zero, and the loads
    // are still issued without a branch, which keeps the compiler's wait
    // counts exact for the activation loads issued before them
    auto load_w = [&](int64_t row, int kb, bool valid) {
        const rsrc_t rw = make_rsrc(qw + (size_t)row * K, valid ? (uint32_t)K : 0u);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + u * 1024 + lane * 16;
            w[u] = buf_load16<CP>(rw, k < khi ? (uint32_t)k : kOOB);
        }
    };

    // The activation (bf16/fp16 for the fused prologue, codes for AS_COPY) is
    // requested before the first weight batch, so its (L2-resident) lines
    // return first and the prologue waits for them alone while the weights
    // are still in flight.
    // XV 16-byte activation vectors per thread cover the activation: 8
    // elements each for the fused prologue, 16 codes each for AS_COPY (the
    // host picks the smallest of 1, 2, 4 that fits, which keeps registers
    // free for the prologue)
    constexpr int VPT = XV;
    constexpr int CPT = XV;
    const int nunit = MR * K / 8;
    const int ncopy = MR * K / 16;
    v4i xr[VPT];
    v4i cr[CPT];
    if constexpr (FUSED) {
        const rsrc_t rx = make_rsrc(act, (uint32_t)(MR * K * 2));
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + i * NT;
            xr[i] = buf_load16(rx, v < nunit ? (uint32_t)(v * 16) : kOOB);
        }
    } else if constexpr (AS == AS_COPY) {
        const rsrc_t rc = make_rsrc(act, (uint32_t)(MR * K));
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int v = tid + i * NT;
            cr[i] = buf_load16(rc, v < ncopy ? (uint32_t)(v * 16) : kOOB);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // The vector L1 returns a CU's loads in the order they were requested, so
    // a wave's activation queues behind the weight batches that waves started
    // earlier have already requested from HBM, and the prologue's reductions
    // wait for the last of them.  With act_first every wave of the workgroup
    // has requested its activation before any wave requests weights (a bare
    // s_barrier: nothing is waited for); the host sets it where each wave
    // streams at most two rows or row segments, so that the prologue, not the
    // stream, sets the launch's length.  It changes no arithmetic.
    if (act_first) asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);

    const int u0 = wave;
    load_w(rbeg + (min(u0, max(nunits - 1, 0)) >> ls), klo, u0 < nunits);   // unconditional: see load_w
    __builtin_amdgcn_sched_barrier(0);

    float s_a[MR];                    // the activation scale of each row (all equal without rowscale)
    DelayedView dview{};              // DS: the history as the call found it
    if constexpr (DS) {
        float xmax = 0.0f;
        const float sd = delayed_scale(state);
        dview = delayed_view(history, hist_len, state);
#pragma unroll
        for (int m = 0; m < MR; ++m) s_a[m] = sd;
        const Quotient d(sd);
        v2i* cl = reinterpret_cast<v2i*>(codes_lds);
        v2i* qg = reinterpret_cast<v2i*>(q_out);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + i * NT;
            xmax = fmaxf(xmax, vec_absmax<DT>(xr[i]));
            if (v < nunit) {
                const v2i c = vec_quantize<DT>(xr[i], d);
                cl[v] = c;
                if (blockIdx.x == 0) qg[v] = c;
            }
        }
        if (blockIdx.x == 0 && tid == 0) sa_out[0] = sd;
        // the waves' maxima wait in red[0] (untouched until the end) for the
        // workgroup that ends the call; the codes barrier publishes them too
        xmax = wave_max(xmax);
        if (lane == 0) red[0][wave] = xmax;
        __syncthreads();
    } else if constexpr (FUSED) {
        // per-row maxima (unit v belongs to row v / (K/8)), then one barrier
        // for all rows; without rowscale every row takes the overall max
        float mx[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) mx[m] = 0.0f;
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const float a = vec_absmax<DT>(xr[i]);
            if (MR == 1 || tid + i * NT < nunit / MR) mx[0] = fmaxf(mx[0], a);
            else mx[MR - 1] = fmaxf(mx[MR - 1], a);
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            mx[m] = wave_max(mx[m]);
            if (lane == 0) red[m][wave] = mx[m];
        }
        lds_barrier();
        float amax[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            amax[m] = red[m][0];
#pragma unroll
            for (int i = 1; i < W; ++i) amax[m] = fmaxf(amax[m], red[m][i]);
        }
        if (!rowscale) {
#pragma unroll
            for (int m = 1; m < MR; ++m) amax[0] = fmaxf(amax[0], amax[m]);
#pragma unroll
            for (int m = 1; m < MR; ++m) amax[m] = amax[0];
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) s_a[m] = scale_from_amax(amax[m]);
        const Quotient d0(s_a[0]), d1(s_a[MR - 1]);
        v2i* cl = reinterpret_cast<v2i*>(codes_lds);
        v2i* qg = reinterpret_cast<v2i*>(q_out);
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + i * NT;
            if (v < nunit) {
                const v2i c = vec_quantize<DT>(xr[i], (MR == 1 || v < nunit / MR) ? d0 : d1);
                cl[v] = c;
                if (blockIdx.x == 0) qg[v] = c;
            }
        }
        if (blockIdx.x == 0 && tid < (rowscale ? MR : 1)) {
            sa_out[tid] = s_a[tid];
            amax_out[tid] = amax[tid];
        }
        lds_barrier();
    } else {
#pragma unroll
        for (int m = 0; m < MR; ++m) s_a[m] = sa_in[rowscale ? m : 0];
        if constexpr (AS == AS_COPY) {
            v4i* dst = reinterpret_cast<v4i*>(codes_lds);
#pragma unroll
            for (int i = 0; i < CPT; ++i) {
                const int v = tid + i * NT;
                if (v < ncopy) dst[v] = cr[i];
            }
            lds_barrier();
        }
    }
    // output scale of activation row m and weight row `row`
    const float s_w = (sw != nullptr) ? *sw : implied_wscale(WFMT);
    auto out_scale = [&](int m, int64_t row) {
        return rowscale ? s_a[m] * sw[row] : s_a[m] * s_w;
    };
    const rsrc_t ra = make_rsrc(act, (uint32_t)(MR * K));

    constexpr int WMF = mfma_format(WFMT);   // MFMA format selector of the weight operand
    // lanes holding the diagonal of the 16x16 MFMA result: lane l holds
    // D[4 (l/16) + e][l % 16], e = 0..3, so D[i][i] sits in lane l with
    // e = l % 16 - 4 (l/16) in [0, 4)
    const int dg = (lane & 15) - 4 * (lane >> 4);
    for (int u = u0; u < nunits; u += W) {
        const int lr = u >> ls;
        const int64_t row = rbeg + lr;
        v4f acc[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[m] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int kbi = 0; kbi < nkb; ++kbi) {
            const int kb = klo + kbi * 1024 * U;
            if (kbi > 0) load_w(row, kb, true);   // (the first batch is already in flight)
            v4i a[MR][U];
#pragma unroll
            for (int uu = 0; uu < U; ++uu) {
                const int k = kb + uu * 1024 + lane * 16;
                const bool in = k < khi;
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    if constexpr (IN_LDS) {
                        const v4i v = *reinterpret_cast<const v4i*>(codes_lds + m * K + (in ? k : 0));
                        a[m][uu] = in ? v : v4i{0, 0, 0, 0};
                    } else {
                        a[m][uu] = buf_load16(ra, in ? (uint32_t)(m * K + k) : kOOB);
                    }
                }
            }
            // One MFMA per pair of 1 KiB chunks: lane l supplies the 32 weight
            // bytes it loaded (row positions kb + uu KiB + 16 l, 16 each) as
            // its A operand and the activation codes of the same positions as
            // its B operand.  A lane's A and B bytes meet in the same products,
            // so D[i][j] sums W at the positions of lanes {i + 16 g} times x at
            // those of lanes {j + 16 g}, and the diagonal D[i][i], i = 0..15,
            // holds the dot product over the 64 lanes' positions in 16 parts.
            // The weights stay in the streaming layout (1 KiB of one row per
            // load instruction) and nothing is decoded on the VALU.
#pragma unroll
            for (int uu = 0; uu < U; uu += 2) {
                // an odd last chunk pairs with zeros, which the compiler must
                // not see as constants (its combiner fails on a scaled MFMA
                // whose operand is partly known)
                v4i z = {0, 0, 0, 0};
                asm volatile("" : "+v"(z));
                const v8i wv = uu + 1 < U ? cat8(w[uu], w[uu + 1]) : cat8(w[uu], z);
#pragma unroll
                for (int m = 0; m < MR; ++m) {
                    const v8i av = uu + 1 < U ? cat8(a[m][uu], a[m][uu + 1]) : cat8(a[m][uu], z);
                    acc[m] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, av, acc[m], WMF, 0,
                                                                              0, 0, 0, 0);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) {
            const float dv = dg == 0 ? acc[m][0] : dg == 1 ? acc[m][1] : dg == 2 ? acc[m][2]
                           : dg == 3 ? acc[m][3] : 0.0f;
            const float v = wave_sum(dv);
            if (lane == 0) {
                if (S == 1) y[(size_t)m * N + row] = (uint16_t)f32_to_out_bits<OUTF>(v * out_scale(m, row));
                else part[(m * nrows + lr) * S + seg] = v;
            }
        }
        // next unit's first batch
        if (u + W < nunits) load_w(rbeg + ((u + W) >> ls), klo, true);
    }
    if (S > 1) {
        lds_barrier();
        for (int t = tid; t < MR * nrows; t += NT) {
            float v = 0.0f;
            for (int j = 0; j < S; ++j) v += part[t * S + j];
            const int m = t / nrows, lr = t - m * nrows;
            y[(size_t)m * N + rbeg + lr] = (uint16_t)f32_to_out_bits<OUTF>(v * out_scale(m, rbeg + lr));
        }
    }
    if constexpr (DS) {
        // every wave read state[0] in the prologue: count this workgroup now.
        // Counted right after the prologue, the atomic's return held up the
        // weight stream (vector-memory waits return in order, and one queue
        // of 512 same-address arrivals takes about 4 us): measured on the
        // Llama-7B decode step, 15.8 -> 12.4 us per launch with the count
        // here and in two levels.
        __shared__ int last;
        if (tid == 0) last = delayed_arrive<kDsGroups>(state, 0.0f, false);
        __syncthreads();
        if (last) {
            float a = red[0][0];
#pragma unroll
            for (int i = 1; i < W; ++i) a = fmaxf(a, red[0][i]);
            __syncthreads();                           // red is reused below
            delayed_publish<NT>(a, dview, history, hist_len, state, &red[0][0]);
            if (tid == 0) amax_out[0] = a;
        }
    }
}

// ---------------------------------------------------------------- NestedFP FP16 mode
// y[m, n] = fp16( sum_k a[m,k] * fp16((hi[n,k] << 8) | lo[n,k]) ): each lane
// reads 16 bytes of each plane (1 KiB of a plane row per instruction),
// rebuilds 16 fp16 words with v_perm and accumulates fp16 pairs with
// v_dot2_f32_f16 (fp32 accumulation).
template <int MR, int ROWS, int U, int CP, int SP>
__global__ __launch_bounds__(kThreads) void rowk_nested16_kernel(
    const uint16_t* __restrict__ a, const uint8_t* __restrict__ hi,
    const uint8_t* __restrict__ lo, uint16_t* __restrict__ y, int N, int K)
{
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = ((int64_t)blockIdx.x * (kThreads / 64) + wave) * ROWS;   // one group per wave
    const int nrow = (int)max((int64_t)0, min((int64_t)ROWS, (int64_t)N - row0));
    const size_t base = (size_t)min(row0, (int64_t)N - 1) * K;
    const rsrc_t rh = make_rsrc(hi + base, (uint32_t)(nrow * K));
    const rsrc_t rl = make_rsrc(lo + base, (uint32_t)(nrow * K));
    const rsrc_t ra = make_rsrc(a, (uint32_t)(MR * K * 2));

    float acc[MR][ROWS];
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < ROWS; ++j) acc[m][j] = 0.0f;

    for (int kb = 0; kb < K; kb += 1024 * U) {
        v4i hv[ROWS][U], lv[ROWS][U], av[MR][U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = kb + u * 1024 + lane * 16;
            const bool in = k < K;
#pragma unroll
            for (int j = 0; j < ROWS; ++j) {
                hv[j][u] = buf_load16<CP>(rh, in ? (uint32_t)(j * K + k) : kOOB);
                lv[j][u] = buf_load16<CP>(rl, in ? (uint32_t)(j * K + k) : kOOB);
            }
#pragma unroll
            for (int m = 0; m < MR; ++m) {
                av[m][u][0] = buf_load16(ra, in ? (uint32_t)(2 * (m * K + k)) : kOOB);
                av[m][u][1] = buf_load16(ra, in ? (uint32_t)(2 * (m * K + k) + 16) : kOOB);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int j = 0; j < ROWS; ++j) {
                uint32_t wv[8];
#pragma unroll
                for (int d = 0; d < 4; ++d)
                    nested_rebuild4<SP>((uint32_t)hv[j][u][d], (uint32_t)lv[j][u][d], wv[2 * d],
                                    wv[2 * d + 1]);
#pragma unroll
                for (int m = 0; m < MR; ++m)
#pragma unroll
                    for (int d = 0; d < 8; ++d)
                        acc[m][j] = __builtin_amdgcn_fdot2(
                            __builtin_bit_cast(h2, (int)av[m][u][d >> 2][d & 3]),
                            __builtin_bit_cast(h2, wv[d]), acc[m][j], false);
            }
        }
    }

#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int j = 0; j < ROWS; ++j) {
            const float v = wave_sum(acc[m][j]);
            if (lane == 0 && j < nrow) y[(size_t)m * N + row0 + j] = (uint16_t)f32_to_f16_bits(v);
        }
}

int rowk_grid(int N) { return (int)(((int64_t)N + kRows * (kThreads / 64) - 1) / (kRows * (kThreads / 64))); }

// Split of each weight row's K range over S = 2^ls waves.  A wave's work is
// ceil(units / 16) units of ceil(segment / batch) batches each.  A split is
// taken only where it at least halves the longest wave and that wave has at
// least 4 batches, and only while the partial sums fit in LDS.  Measured on
// MI355X inside the Llama-7B decode step: the down projection (8 rows of
// 11008 per workgroup, half the waves idle without a split) gains 10% with
// S = 2, while QKV (24 rows of 4096: 4 -> 3 batches) and O (8 rows of 4096:
// 2 -> 1 batch) lose about 4%, and S = 4 at 10-20 rows of 5120..8192 (Qwen-32B)
// loses although it shortens the longest wave a little.
// Batches of U KiB that the longest wave of a workgroup of W waves streams
// when each row's K range is cut into 2^ls segments.
int64_t rowk_wave_batches(int64_t rows_per_wg, int K, int U, int ls, int W)
{
    const int64_t units = rows_per_wg << ls;
    const int64_t kseg = ((((int64_t)K + (1 << ls) - 1) >> ls) + 127) & ~(int64_t)127;
    return ((units + W - 1) / W) * ((kseg + 1024 * U - 1) / (1024 * U));
}

int rowk_split_shift(int64_t rows_per_wg, int K, int MR, int U, int W)
{
    auto cost = [&](int ls) { return rowk_wave_batches(rows_per_wg, K, U, ls, W); };
    int best = 0;
    if (cost(0) < 4) return best;
    for (int ls = 1; ls <= 4; ++ls)
        if ((int64_t)MR * (rows_per_wg << ls) <= kPartMax && 2 * cost(ls) <= cost(best)) best = ls;
    return best;
}

template <int WFMT, int OUTF, int AS, int MR, bool DS = false>
void launch_rowk(const void* act, const float* sa_in, const uint8_t* qw, const float* sw,
                 uint16_t* y, uint8_t* q, float* sa_out, float* amax, int N, int K,
                 int rowscale, hipStream_t st, float* history = nullptr, int64_t hist_len = 0,
                 uint32_t* state = nullptr)
{
    using C = RowkCfg<MR>;
    const size_t lds = AS != AS_GLOBAL ? (size_t)MR * K : 0;
    // 16-byte activation vectors per thread: MR*K/8 bf16/fp16 vectors for the
    // fused prologue, MR*K/16 code vectors for AS_COPY (none for AS_GLOBAL)
    const int64_t vecs = AS == AS_GLOBAL ? 0 : (int64_t)MR * K / (AS == AS_COPY ? 16 : 8);
    auto go = [&](auto nt, auto wpc, auto u) {
        constexpr int NT = decltype(nt)::value, WPC = decltype(wpc)::value, U = decltype(u)::value;
        const int grid = min(N, kCUs * WPC);
        const int rpw = (int)(((int64_t)N + grid - 1) / grid);
        const int ls = rowk_split_shift(rpw, K, MR, U, NT / 64);
        const int kseg = (int)(((((int64_t)K + (1 << ls) - 1) >> ls) + 127) & ~(int64_t)127);
        // activation requested ahead of all weights where each wave streams at
        // most two rows or row segments (measured on MI355X, fused M = 1:
        // Llama-7B O 8.1 -> 6.5 us, down 13.8 -> 11.6, Qwen-32B O 11.1 -> 10.3;
        // with more rows per wave the stream dominates and the barrier only
        // delays it: gate+up 16.8 -> 18.1)
        const int act_first = (AS == AS_BF16 || AS == AS_FP16) &&
                              ((((int64_t)rpw << ls) + NT / 64 - 1) / (NT / 64)) <= 2;
        auto launch = [&](auto xv) {
            rowk_f8_kernel<NT, WFMT, OUTF, AS, MR, U, CP_NT, WPC, decltype(xv)::value, DS>
                <<<grid, NT, lds, st>>>(act, sa_in, qw, sw, y, q, sa_out, amax, N, K, rpw, ls, kseg,
                                        rowscale, history, hist_len, state, act_first);
        };
        if (vecs <= NT) launch(std::integral_constant<int, 1>{});
        else if (vecs <= 2 * NT) launch(std::integral_constant<int, 2>{});
        else launch(std::integral_constant<int, 4>{});
    };
    // Launch shape at M = 1 (measured on MI355X on 16 decode shapes, K = 2048
    // .. 12288, 4 .. 100 rows per workgroup, weights cold).  The reference is
    // 1024 threads streaming 2 KiB batches.  Rows of 3 .. 16 whole KiB instead
    // take 512 threads streaming 3 or 4 KiB batches (the size that leaves less
    // of a row's last batch empty; 4 on a tie) whenever the longest wave then
    // streams no more batches than with the reference: Llama-7B QKV 11.9 ->
    // 11.4 us, O 7.4 -> 6.6, gate+up 17.5 -> 16.9, Qwen-32B QKV 14.2 -> 13.2,
    // O 12.3 -> 10.7.  Where it would stream more (Qwen-32B gate+up: 100 rows
    // per workgroup), or rows end in a part of a KiB (down, K = 11008), or
    // are shorter than 3 KiB, the larger batches measured slower.  Otherwise,
    // where the reference leaves each wave at most two batches, 512 threads
    // with 2 KiB batches halve the waves that meet at the activation
    // prologue's barriers.  The choice depends on N and K only, never on the
    // activation source, so fp8_linear and fp8_quantize_act + fp8_gemm split
    // rows alike and stay bit-identical; K stays where the fused prologue (8
    // bf16 values per vector, at most 4 vectors per thread) fits 512 threads.
    using I512 = std::integral_constant<int, 512>;
    using I2 = std::integral_constant<int, 2>;
    if constexpr (MR == 1) {
        constexpr int W16 = kWgThreads / 64, W8 = 512 / 64;
        const int grid = min(N, kCUs * C::WPC);
        const int64_t rpw = ((int64_t)N + grid - 1) / grid;
        const int64_t ref = rowk_wave_batches(rpw, K, C::U, rowk_split_shift(rpw, K, MR, C::U, W16),
                                              W16);
        if (K % 1024 == 0 && K >= 3 * 1024 && K <= 4 * 512 * 8) {
            const int kb = K / 1024;
            const int u = ((kb + 2) / 3 * 3 - kb) < ((kb + 3) / 4 * 4 - kb) ? 3 : 4;
            if (rowk_wave_batches(rpw, K, u, rowk_split_shift(rpw, K, MR, u, W8), W8) <= ref) {
                if (u == 3) go(I512{}, I2{}, std::integral_constant<int, 3>{});
                else go(I512{}, I2{}, std::integral_constant<int, 4>{});
                return;
            }
        }
        if (K <= 4 * 512 * 8 && ref <= 2) {
            go(I512{}, I2{}, I2{});
            return;
        }
    }
    go(std::integral_constant<int, kWgThreads>{}, std::integral_constant<int, C::WPC>{},
       std::integral_constant<int, C::U>{});
}

// Unfused FP8 weights: codes staged in LDS when they fit, else read from L2.
template <int WFMT, int OUTF, int MR>
void launch_rowk_codes(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                       uint16_t* y, int N, int K, int rowscale, hipStream_t st)
{
    if ((int64_t)MR * K <= kFusedMaxMK)
        launch_rowk<WFMT, OUTF, AS_COPY, MR>(qa, sa, qw, sw, y, nullptr, nullptr, nullptr, N, K, rowscale, st);
    else
        launch_rowk<WFMT, OUTF, AS_GLOBAL, MR>(qa, sa, qw, sw, y, nullptr, nullptr, nullptr, N, K, rowscale, st);
}

}  // namespace

hipError_t launch_rowk_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                           hipStream_t stream)
{
    if (wfmt == WF_E4M3 && outf == OUT_BF16) {
        if (M == 1) launch_rowk_codes<WF_E4M3, OUT_BF16, 1>(qa, sa, qw, sw, y, N, K, rowscale, stream);
        else launch_rowk_codes<WF_E4M3, OUT_BF16, 2>(qa, sa, qw, sw, y, N, K, rowscale, stream);
    } else if (wfmt == WF_E5M2 && outf == OUT_FP16 && !rowscale) {
        if (M == 1) launch_rowk_codes<WF_E5M2, OUT_FP16, 1>(qa, sa, qw, sw, y, N, K, 0, stream);
        else launch_rowk_codes<WF_E5M2, OUT_FP16, 2>(qa, sa, qw, sw, y, N, K, 0, stream);
    } else if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && !rowscale) {
        if (M == 1) launch_rowk_codes<WF_E4M3_SC8, OUT_FP16, 1>(qa, sa, qw, sw, y, N, K, 0, stream);
        else launch_rowk_codes<WF_E4M3_SC8, OUT_FP16, 2>(qa, sa, qw, sw, y, N, K, 0, stream);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_rowk_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream)
{
    auto go = [&](auto mr, auto spc) {
        rowk_nested16_kernel<decltype(mr)::value, kRows, kUnroll, CP_NT, decltype(spc)::value>
            <<<rowk_grid(N), kThreads, 0, stream>>>(a, hi, lo, y, N, K);
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using P0 = std::integral_constant<int, SP_PLAIN>;
    using P1 = std::integral_constant<int, SP_E4M3>;
    if (M == 1) (sp == SP_E4M3) ? go(I1{}, P1{}) : go(I1{}, P0{});
    else (sp == SP_E4M3) ? go(I2{}, P1{}) : go(I2{}, P0{});
    return hipGetLastError();
}

hipError_t launch_linear_fused_delayed(const void* x, int dtype, const uint8_t* qw, const float* sw,
                                       uint16_t* y, uint8_t* q, float* scale, float* amax,
                                       float* history, int64_t L, uint32_t* state, int M, int N,
                                       int K, hipStream_t stream)
{
    if (dtype == DT_BF16) {
        if (M == 1)
            launch_rowk<WF_E4M3, OUT_BF16, AS_BF16, 1, true>(x, nullptr, qw, sw, y, q, scale, amax, N,
                                                             K, 0, stream, history, L, state);
        else
            launch_rowk<WF_E4M3, OUT_BF16, AS_BF16, 2, true>(x, nullptr, qw, sw, y, q, scale, amax, N,
                                                             K, 0, stream, history, L, state);
    } else {
        if (M == 1)
            launch_rowk<WF_E4M3, OUT_BF16, AS_FP16, 1, true>(x, nullptr, qw, sw, y, q, scale, amax, N,
                                                             K, 0, stream, history, L, state);
        else
            launch_rowk<WF_E4M3, OUT_BF16, AS_FP16, 2, true>(x, nullptr, qw, sw, y, q, scale, amax, N,
                                                             K, 0, stream, history, L, state);
    }
    return hipGetLastError();
}

hipError_t launch_linear_fused(const void* x, int dtype, const uint8_t* qw, const float* sw,
                               uint16_t* y, uint8_t* q, float* scale, float* amax, int M, int N,
                               int K, int wfmt, int outf, int rowscale, hipStream_t stream)
{
    if (rowscale && !(wfmt == WF_E4M3 && outf == OUT_BF16)) return hipErrorInvalidValue;
    if (wfmt == WF_E4M3 && outf == OUT_BF16 && dtype == DT_BF16) {
        if (M == 1)
            launch_rowk<WF_E4M3, OUT_BF16, AS_BF16, 1>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
        else
            launch_rowk<WF_E4M3, OUT_BF16, AS_BF16, 2>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
    } else if (wfmt == WF_E4M3 && outf == OUT_BF16 && dtype == DT_FP16) {
        if (M == 1)
            launch_rowk<WF_E4M3, OUT_BF16, AS_FP16, 1>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
        else
            launch_rowk<WF_E4M3, OUT_BF16, AS_FP16, 2>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
    } else if (wfmt == WF_E5M2 && outf == OUT_FP16 && dtype == DT_FP16) {
        // NestedFP FP8 mode: fp16 activation, hi plane as E5M2, no weight scale
        if (M == 1)
            launch_rowk<WF_E5M2, OUT_FP16, AS_FP16, 1>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
        else
            launch_rowk<WF_E5M2, OUT_FP16, AS_FP16, 2>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
    } else if (wfmt == WF_E4M3_SC8 && outf == OUT_FP16 && dtype == DT_FP16) {
        // the same mode on the E4M3 split: hi plane = E4M3 codes of w * 2^8
        if (M == 1)
            launch_rowk<WF_E4M3_SC8, OUT_FP16, AS_FP16, 1>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
        else
            launch_rowk<WF_E4M3_SC8, OUT_FP16, AS_FP16, 2>(x, nullptr, qw, sw, y, q, scale, amax, N, K, rowscale, stream);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fp8q
