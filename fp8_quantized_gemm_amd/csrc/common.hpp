// Internal header of libfp8q: device-side number-format helpers, wave
// reductions and the launcher declarations shared by the kernel files and the
// C ABI in api.hip.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8q.h"

namespace fp8q {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// Input dtype tags (same numbering as fp8q_dtype in the public header).
enum : int { DT_BF16 = 0, DT_FP16 = 1 };
// Weight format of the FP8 GEMMs: E4M3 codes, E5M2 codes (the NestedFP upper
// byte of the plain split), or E4M3 codes of w * 2^8 (the NestedFP upper byte
// of the E4M3 split), whose 2^-8 the epilogue applies when no weight scale is
// given.
enum : int { WF_E4M3 = 0, WF_E5M2 = 1, WF_E4M3_SC8 = 2 };
// The format selector (cbsz/blgp) of v_mfma_*_f8f6f4 for a weight format:
// 0 = FP8 E4M3, 1 = BF8 E5M2.
constexpr int mfma_format(int wf) { return wf == WF_E5M2 ? 1 : 0; }
// The weight scale a format implies when the call passes none.
constexpr float implied_wscale(int wf) { return wf == WF_E4M3_SC8 ? 0x1p-8f : 1.0f; }
// Output format of the GEMM epilogues.
enum : int { OUT_BF16 = 0, OUT_FP16 = 1 };

// ---------------------------------------------------------------- 16-bit floats
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

template <int DT>
__device__ __forceinline__ float half_bits_to_f32(uint32_t h)
{
    if constexpr (DT == DT_BF16) return bf16_bits_to_f32(h);
    else return f16_bits_to_f32(h);
}

// binary32 -> bfloat16, round to nearest even on the bit pattern (carry into
// the exponent gives the next binade or infinity); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// binary32 -> binary16 with the hardware conversion (round to nearest even,
// subnormal results kept, overflow to infinity).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f)
{
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

template <int OUTF>
__device__ __forceinline__ uint32_t f32_to_out_bits(float f)
{
    if constexpr (OUTF == OUT_BF16) return f32_to_bf16_bits(f);
    else return f32_to_f16_bits(f);
}

// ---------------------------------------------------------------- FP8 E4M3
// Saturate to the E4M3 range first (|v| > 448 and +-inf -> +-448; NaN passes
// through), then let the gfx950 packed converter round to nearest even into
// the OCP E4M3 encoding (subnormals kept).
__device__ __forceinline__ float e4m3_saturate(float v)
{
    return fabsf(v) > 448.0f ? copysignf(448.0f, v) : v;
}

// Four binary32 values already within [-448, 448] -> four E4M3 codes, value
// i in byte i.
__device__ __forceinline__ uint32_t e4m3_pack4_in_range(float a, float b, float c, float d)
{
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
    return (uint32_t)r;
}

// Four binary32 values -> four E4M3 codes, value i in byte i.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d)
{
    return e4m3_pack4_in_range(e4m3_saturate(a), e4m3_saturate(b), e4m3_saturate(c),
                               e4m3_saturate(d));
}

// ---------------------------------------------------------------- quantizer elements
// Shared by the stand-alone quantizer and the fused decode linear, so both
// produce the same codes: q = E4M3_rne_sat(fl32(x / s)), s = fl32(amax / 448)
// (1 when amax == 0), with fl32(x / s) the correctly rounded quotient.
//
// The quotient is computed with one reciprocal per scale and two FMAs per
// element (Markstein's correction step): r = RN(1/s), q0 = RN(x r),
// e = x - q0 s (exact through the FMA), q = RN(q0 + e r).  q equals the
// correctly rounded x / s for every bf16 and fp16 input significand and every
// fp32 divisor significand (checked exhaustively against IEEE division); the
// argument needs a finite r and an exact residual, which hold for
// 2^-80 <= s <= 2^120 and every quotient large enough to give a nonzero code.
// Scales outside that range use the IEEE division.
//
// The quantizer takes sat_div, which returns the quotient already saturated
// to [-448, 448] in six VALU operations and no branch or select:
//  - q0 is clamped to [-896, 896] first (a median of three).  Where that
//    changes q0 the true quotient is beyond 448 as well (q0 is within an ulp
//    of it) and the result saturates either way; the correction step must
//    not start from an infinite q0 (an input spike under a small delayed
//    scale, or an infinite input), where x - q0 s = -+inf and -+inf r +
//    q0 would give NaN.
//  - The result takes the sign of x: an exact zero quotient (x = -0) comes
//    out of the correction step as +0.
//  - The clamp to [-448, 448] is the saturation; the E4M3 converter then
//    only rounds.  NaN inputs, outside the quantizer's contract, come out as
//    whatever code the hardware median gives a NaN operand.
struct Quotient {
    float s, r;
    bool fast;
    __device__ __forceinline__ explicit Quotient(float s_) : s(s_)
    {
        r = 1.0f / s_;
        fast = s_ >= 0x1p-80f && s_ <= 0x1p120f;
    }
    __device__ __forceinline__ float sat_div(float x) const
    {
        const float q0 = __builtin_amdgcn_fmed3f(x * r, -896.0f, 896.0f);
        const float e = __builtin_fmaf(-q0, s, x);
        const float q = __builtin_copysignf(__builtin_fmaf(e, r, q0), x);
        return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f);
    }
};

template <int DT>
__device__ __forceinline__ float vec_absmax(const v4i& v)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        uint32_t u = (uint32_t)v[i];
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(u & 0xffffu)));
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(u >> 16)));
    }
    return m;
}

template <int DT>
__device__ __forceinline__ float vec_absmax(const v2i& v)
{
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint32_t u = (uint32_t)v[i];
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(u & 0xffffu)));
        m = fmaxf(m, fabsf(half_bits_to_f32<DT>(u >> 16)));
    }
    return m;
}

// 2*NW input halves (NW dwords) -> their E4M3 codes, four to a dword.  The
// quotients of the fast path are saturated already; the IEEE division of the
// other scales saturates in the converter's wrapper.
template <int DT, int NW>
__device__ __forceinline__ void vec_codes(const int (&w)[NW], const Quotient& d, int (&c)[NW / 2])
{
    float f[2 * NW];
    if (d.fast) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            f[2 * i] = d.sat_div(half_bits_to_f32<DT>((uint32_t)w[i] & 0xffffu));
            f[2 * i + 1] = d.sat_div(half_bits_to_f32<DT>((uint32_t)w[i] >> 16));
        }
#pragma unroll
        for (int i = 0; i < NW / 2; ++i)
            c[i] = (int)e4m3_pack4_in_range(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            f[2 * i] = half_bits_to_f32<DT>((uint32_t)w[i] & 0xffffu) / d.s;
            f[2 * i + 1] = half_bits_to_f32<DT>((uint32_t)w[i] >> 16) / d.s;
        }
#pragma unroll
        for (int i = 0; i < NW / 2; ++i)
            c[i] = (int)e4m3_pack4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
    }
}

// 8 input halves -> 8 E4M3 codes (two dwords)
template <int DT>
__device__ __forceinline__ v2i vec_quantize(const v4i& v, const Quotient& d)
{
    const int w[4] = {v[0], v[1], v[2], v[3]};
    int c[2];
    vec_codes<DT, 4>(w, d, c);
    return v2i{c[0], c[1]};
}

// 4 input halves -> 4 E4M3 codes (one dword)
template <int DT>
__device__ __forceinline__ uint32_t vec_quantize(const v2i& v, const Quotient& d)
{
    const int w[2] = {v[0], v[1]};
    int c[1];
    vec_codes<DT, 2>(w, d, c);
    return (uint32_t)c[0];
}

template <int DT>
__device__ __forceinline__ uint8_t scalar_quantize(uint16_t h, const Quotient& d)
{
    const float x = half_bits_to_f32<DT>(h);
    const uint32_t c = d.fast ? e4m3_pack4_in_range(d.sat_div(x), 0.f, 0.f, 0.f)
                              : e4m3_pack4(x / d.s, 0.f, 0.f, 0.f);
    return (uint8_t)(c & 0xffu);
}

__device__ __forceinline__ float scale_from_amax(float amax)
{
    return amax > 0.0f ? amax / 448.0f : 1.0f;
}

// ---------------------------------------------------------------- NestedFP rebuild
// Interleave four upper bytes (h) and four lower bytes (l) into two dwords
// holding the fp16 words (h_i << 8) | l_i, i = 0..3, little-endian.
// v_perm_b32 selects bytes from {src0 (bytes 4..7), src1 (bytes 0..3)}.
// With SP_E4M3 the planes come from the E4M3 split (hi = sign | bits 13..7,
// lo = bit 14 | bits 6..0), and each interleaved word hi << 8 | lo is put
// back in place: sign and bits 6..0 stay, hi's 7 bits move down by one, lo's
// top bit moves up to bit 14.
enum : int { SP_PLAIN = 0, SP_E4M3 = 1 };
// v_bfi_b32: (mask & a) | (~mask & b), one VALU instruction (the compiler
// does not form it from the C expression here); register operands only
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t a, uint32_t b)
{
    uint32_t d;
    asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(d) : "s"(mask), "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ uint32_t e4m3_split_words(uint32_t u)
{
    // bits 13..7 from u >> 1, then bit 14 from u << 7
    const uint32_t w = bit_insert(0x3F803F80u, u >> 1, u);
    return bit_insert(0x40004000u, u << 7, w);
}
template <int SP = SP_PLAIN>
__device__ __forceinline__ void nested_rebuild4(uint32_t h, uint32_t l, uint32_t& w01, uint32_t& w23)
{
    w01 = __builtin_amdgcn_perm(h, l, 0x05010400u);  // [l0, h0, l1, h1]
    w23 = __builtin_amdgcn_perm(h, l, 0x07030602u);  // [l2, h2, l3, h3]
    if constexpr (SP == SP_E4M3) {
        w01 = e4m3_split_words(w01);
        w23 = e4m3_split_words(w23);
    }
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resources (gfx9 V#: base, stride 0, num_records bytes, word 3 =
// 0x00020000).  A buffer load whose byte offset lies at or past num_records
// returns zeros without touching memory, which gives free zero padding for
// ragged rows and K tails without branches.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Callers pass wave-uniform base and size; readfirstlane states that to the
// compiler so the descriptor lives in SGPRs (no per-load waterfall loop).
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}

// An offset that always lies out of range (num_records < 2^31).
constexpr uint32_t kOOB = 0x80000000u;

// Cache policy bits of the buffer instructions (aux operand): 0 = default,
// 2 = non-temporal (streamed data that will not be reused).
enum : int { CP_DEFAULT = 0, CP_NT = 2 };

template <int CP = CP_DEFAULT>
__device__ __forceinline__ v4i buf_load16(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP = CP_DEFAULT>
__device__ __forceinline__ v2i buf_load8(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at
// lds_block + 16 l (the block is wave-uniform).  The compiler does not order
// later LDS reads after these asynchronous writes; callers wait (vmcnt) and
// synchronize explicitly.
__device__ __forceinline__ void dma_load16(rsrc_t r, void* lds_block, uint32_t off)
{
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_block, 16, off, 0, 0, 0);
}

// ---------------------------------------------------------------- reductions
// Max over a wave64 with DPP row operations; the result is valid in every lane.
#define FP8Q_DPP_MAX(v, ctrl, rowmask)                                                    \
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v),            \
                                                            __float_as_int(v), ctrl,      \
                                                            rowmask, 0xf, false)))

__device__ __forceinline__ float wave_max(float v)
{
    FP8Q_DPP_MAX(v, 0xB1, 0xf);   // quad_perm [1,0,3,2]
    FP8Q_DPP_MAX(v, 0x4E, 0xf);   // quad_perm [2,3,0,1]
    FP8Q_DPP_MAX(v, 0x141, 0xf);  // row_half_mirror
    FP8Q_DPP_MAX(v, 0x140, 0xf);  // row_mirror: lanes of each row of 16 hold its max
    FP8Q_DPP_MAX(v, 0x142, 0xa);  // row_bcast15 -> rows 1, 3
    FP8Q_DPP_MAX(v, 0x143, 0xc);  // row_bcast31 -> rows 2, 3: lane 63 holds the max
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Workgroup barrier for data exchanged through LDS only.  __syncthreads()
// also waits for every global load and store the wave still has in flight
// (s_waitcnt vmcnt(0) before s_barrier), which would hold a prologue behind
// weight loads issued ahead of it; LDS writes are complete once lgkmcnt is 0.
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Block-wide max for blockDim.x = NT threads; result valid in every thread.
template <int NT>
__device__ __forceinline__ float block_max(float v, float* lds)
{
    constexpr int W = NT / 64;
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) lds[wave] = v;
    __syncthreads();
    float m = lds[0];
#pragma unroll
    for (int i = 1; i < W; ++i) m = fmaxf(m, lds[i]);
    return m;
}

// Sum over a wave64 (butterfly through the LDS crossbar); valid in every lane.
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    return v;
}

// Block-wide integer sum for blockDim.x = NT threads; valid in every thread.
template <int NT>
__device__ __forceinline__ int block_sum_int(int v, int* lds)
{
    constexpr int W = NT / 64;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < W; ++i) t += lds[i];
    return t;
}

// ---------------------------------------------------------------- delayed scaling
// Delayed scaling with an amax history ([RTX4060] §6.1 asks for a history of
// at least 1024 values).  A call quantizes with the scale that the earlier
// calls' history gives, then records its own amax:
//   history[L]  the amax of the last L calls (zeros before any call)
//   state[0]    float bits of the scale the next call uses (0: none yet -> 1)
//   state[1]    float bits of the running max of the current call
//   state[2]    ring position
//   state[3]    groups of workgroups of the current call that have arrived
//   state[4]    float bits of max(history)
//   state[32 (1 + j)], state[32 (1 + j) + 1], j = 0..7: arrivals and running
//               max of group j (the workgroups blockIdx.x = j, j + 8, ...)
// Every word but [0], [2] and [4] is back at 0 when a call ends, so the caller
// only zero-fills state and history once.  Calls on one state must not
// overlap.
constexpr int kDsLine = 32;                         // words per 128-byte line
constexpr int kDsGroups = 8;
constexpr int kDsStateWords = kDsLine * (1 + kDsGroups);
static_assert(kDsStateWords == FP8Q_DELAYED_STATE_WORDS, "state layout of fp8q.h");

__device__ __forceinline__ float delayed_scale(const uint32_t* state)
{
    const float s = __uint_as_float(state[0]);
    return s > 0.0f ? s : 1.0f;
}

// The arrival of a workgroup of the current call, run by its thread 0 after
// the workgroup's last read of state[0]; with fold, m (the workgroup's
// maximum) is folded into the call's running max state[1] first.  Returns
// true in the workgroup that arrives last, which then ends the call
// (delayed_publish).  Only device-scope atomics pass information here, so
// their order suffices and no fence is needed (a fence would also write back
// the XCD's L2, behind the codes just stored): each atomic's returned value
// is consumed before the next one is issued, so a fold is performed before
// its count, and the last arrival sees every fold.  Same-address device-scope
// atomics serialize on MI355X (about 8 ns each).  With GROUPS = 8 a workgroup
// counts in the 128-byte line of its group (blockIdx.x % 8) and only the
// last of each group counts in state[3], so the longest queue is ceil(G / 8)
// + 8 atomics instead of G, at the price of a second round of dependent
// atomics: measured on the 512 workgroups of the fused decode kernel the two
// levels pay, on the 64-256 of the grid-stride quantizer one level is faster.
__device__ __forceinline__ void atomic_done(uint32_t v)
{
    asm volatile("" ::"v"(v));        // waits for the returned value, i.e. the atomic
}

template <int GROUPS>
__device__ __forceinline__ bool delayed_arrive(uint32_t* state, float m, bool fold)
{
    static_assert(GROUPS == 1 || GROUPS == kDsGroups, "one level or one line per group");
    const uint32_t G = gridDim.x;
    if constexpr (GROUPS == 1) {
        if (fold) atomic_done(atomicMax(&state[1], __float_as_uint(m)));
        return atomicAdd(&state[3], 1u) == G - 1;
    } else {
        const uint32_t j = blockIdx.x & (kDsGroups - 1);
        uint32_t* const line = state + kDsLine * (1 + j);
        if (fold) atomic_done(atomicMax(&line[1], __float_as_uint(m)));
        const uint32_t members = (G - j + kDsGroups - 1) / kDsGroups;
        if (atomicAdd(&line[0], 1u) != members - 1) return false;
        if (fold) atomic_done(atomicMax(&state[1], atomicMax(&line[1], 0u)));
        const uint32_t groups = G < (uint32_t)kDsGroups ? G : (uint32_t)kDsGroups;
        return atomicAdd(&state[3], 1u) == groups - 1;
    }
}

// What the workgroup that ends a call needs of the state as the call found
// it: every workgroup reads it at its start (nothing changes it before the
// call ends), so the end of the call waits for no further load.
struct DelayedView {
    uint32_t pos;      // ring position
    float evicted;     // history[pos], the entry this call replaces
    float hmax;        // max(history) = state[4]
};
__device__ __forceinline__ DelayedView delayed_view(const float* history, int64_t L,
                                                    const uint32_t* state)
{
    const uint32_t pos = (int64_t)state[2] < L ? state[2] : 0u;   // a corrupted position stays in range
    return DelayedView{pos, history[pos], __uint_as_float(state[4])};
}

// Run by every thread of the one workgroup that ends a call: history[pos] =
// amax, the next scale from the maximum of the new history, pos advanced,
// the accumulators cleared.  The new maximum is max(hmax, amax) unless the
// replaced entry held the maximum and amax is smaller; only then is the
// history scanned.
template <int NT>
__device__ __forceinline__ void delayed_publish(float amax, const DelayedView& v, float* history,
                                                int64_t L, uint32_t* state, float* lds)
{
    float m = fmaxf(v.hmax, amax);
    if (!(v.evicted < v.hmax || amax >= v.hmax)) {
        m = 0.0f;
        for (int64_t i = threadIdx.x; i < L; i += NT) m = fmaxf(m, i == v.pos ? amax : history[i]);
        m = block_max<NT>(m, lds);
    }
    static_assert(NT >= kDsGroups, "one thread per group line");
    if (threadIdx.x < kDsGroups) {
        state[kDsLine * (1 + threadIdx.x)] = 0u;
        state[kDsLine * (1 + threadIdx.x) + 1] = 0u;
    }
    if (threadIdx.x == 0) {
        history[v.pos] = amax;
        state[0] = __float_as_uint(scale_from_amax(m));
        state[1] = 0u;
        state[2] = (int64_t)v.pos + 1 == L ? 0u : v.pos + 1;
        state[3] = 0u;
        state[4] = __float_as_uint(m);
    }
}

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of hipGetLastError() after its launches.
hipError_t launch_quantize(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                           float* amax, hipStream_t stream);
// Same result; for n above the one-workgroup size it uses scratch_floats
// floats at `scratch` (device memory not overlapping x) for per-workgroup
// partial maxima instead of an atomic, when that is enough room.
hipError_t launch_quantize_scratch(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                                   float* amax, float* scratch, int64_t scratch_floats,
                                   hipStream_t stream);

// One scale per row of a [rows, cols] matrix (cols % 16 == 0): scale[r],
// amax[r] and the codes of row r as fp8_quantize_act would give for that row.
hipError_t launch_quantize_rows(const void* x, int dtype, int64_t rows, int64_t cols, uint8_t* q,
                                float* scale, float* amax, hipStream_t stream);

// FP8 KV-cache quantizer: x[T, H, D] with one scale per head (D % 8 == 0).
hipError_t launch_quantize_kv(const void* x, int dtype, int64_t T, int64_t H, int64_t D,
                              uint8_t* q, float* scale, float* amax, hipStream_t stream);

// Delayed-scaling quantizer (see delayed_scale): q, the scale it used and the
// amax of x; history and state advanced by one call.
hipError_t launch_quantize_delayed(const void* x, int dtype, int64_t n, uint8_t* q, float* scale,
                                   float* amax, float* history, int64_t L, uint32_t* state,
                                   hipStream_t stream);

// ---------------------------------------------------------------- launch helpers
// Raises a kernel's dynamic LDS limit to `lds` bytes once per device (the
// attribute is set for the current device).  `done` holds one bit per device
// id below 64; two threads racing on a first call both set it, which is
// harmless; devices 64 and up set it on every call.
inline hipError_t set_lds_limit_once(const void* kern, size_t lds, std::atomic<uint64_t>& done)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t)1 << dev : 0;
    if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
    return e;
}

// Row-contiguous decode path for M <= kRowkMaxM (see linear.hip).
constexpr int kRowkMaxM = 2;
// Largest M*K the fused decode linear quantizes in LDS.
constexpr int64_t kFusedMaxMK = 32768;
hipError_t launch_rowk_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw, const float* sw,
                           uint16_t* y, int M, int N, int K, int wfmt, int outf, int rowscale,
                           hipStream_t stream);
hipError_t launch_rowk_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream);
hipError_t launch_linear_fused(const void* x, int dtype, const uint8_t* qw, const float* sw,
                               uint16_t* y, uint8_t* q, float* scale, float* amax, int M, int N,
                               int K, int wfmt, int outf, int rowscale, hipStream_t stream);
// The fused decode linear with delayed scaling (E4M3 weights, bf16 output).
hipError_t launch_linear_fused_delayed(const void* x, int dtype, const uint8_t* qw, const float* sw,
                                       uint16_t* y, uint8_t* q, float* scale, float* amax,
                                       float* history, int64_t L, uint32_t* state, int M, int N,
                                       int K, hipStream_t stream);
hipError_t launch_e4m3_encode_f32(const float* v, uint8_t* q, int64_t n, hipStream_t stream);

// Decode path (M <= 16) and tile path (M > 16) of the FP8 GEMM; wfmt selects
// the weight format (E4M3 / E5M2), outf the output format (bf16 / fp16), and
// sw == nullptr means the scale is *sa alone.  With rowscale (E4M3 / bf16
// only) sa holds M scales and sw N scales, and element (m, n) is scaled by
// fl32(sa[m] * sw[n]).
hipError_t launch_gemv_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw,
                           const float* sw, uint16_t* y, int M, int N, int K, int wfmt,
                           int outf, int rowscale, hipStream_t stream);
// fp8_linear in one launch for 3 <= M <= 16 (see gemv.hip): quantizer and
// GEMV fused, per-tensor scales only; M * K at most kFusedGemvMaxMK, taken
// where linear_gemv_fused_pays says so.
constexpr int64_t kFusedGemvMaxMK = 65536;
bool linear_gemv_fused_pays(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_gemv_fused(const void* x, int dtype, const uint8_t* qw, const float* sw,
                                    uint16_t* y, uint8_t* q, float* scale, float* amax, int M,
                                    int N, int K, int wfmt, int outf, hipStream_t stream);
hipError_t launch_tile_fp8(const uint8_t* qa, const float* sa, const uint8_t* qw,
                           const float* sw, uint16_t* y, int M, int N, int K, int wfmt,
                           int outf, int rowscale, hipStream_t stream);

// sp selects the split (SP_PLAIN / SP_E4M3); with SP_E4M3 the split adds the
// number of words outside |w| < 1.875 to *bad (when bad is not null).
hipError_t launch_nested_split(const uint16_t* w, uint8_t* hi, uint8_t* lo, int64_t n, int sp,
                               unsigned long long* bad, hipStream_t stream);
hipError_t launch_nested_rebuild(const uint8_t* hi, const uint8_t* lo, uint16_t* w, int64_t n,
                                 int sp, hipStream_t stream);
hipError_t launch_gemv_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream);
hipError_t launch_tile_nested16(const uint16_t* a, const uint8_t* hi, const uint8_t* lo,
                                uint16_t* y, int M, int N, int K, int sp, hipStream_t stream);

}  // namespace fp8q
