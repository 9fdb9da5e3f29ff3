// kernels.hpp -- gfx950 kernels of the fused rank-sum + residual-add + RMSNorm
// epilogue (+ per-token or per-group FP8 E4M3, or MXFP4) and of the plain rank
// sum. Included by the per-dtype, per-epilogue translation units.
//
// Numerics (ROCm/aiter PR #6699 "gfx1250 fused all-reduce + RMSNorm", section
// Changes; PR #3462 "optimize fused AllReduce + RMSNorm", section Technical
// Details):
//   * ranks are summed per element in fp32 in rank order 0..R-1, the sum is
//     rounded to T (bf16/fp16) like an unfused all-reduce, added to the
//     residual in fp32 and rounded to T again (that value is residual_out);
//   * the row statistics are exact squares accumulated in fp64, so that
//     rstd = 1/sqrt(mean + eps) is good to ~1e-16 and the normalised output
//     y = RNE_T((h * w_eff) * rstd) is the single rounding of the fp64 value;
//   * the per-token FP8 epilogue quantises the T-rounded y with
//     scale = amax / 448 and an fp32 division per element.
// Fast branches (fp32 conversion of y, reciprocal multiply for FP8, hardware
// FP8 conversion) are taken only where they provably give the same bits;
// elements near a rounding tie take an exact branch (round-to-odd, IEEE
// division, software E4M3 encoder).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "launch.hpp"

namespace arrms {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

#define ARRMS_DEV static __device__ __forceinline__

// --------------------------------------------------------------------------
// Round to odd: fp64 -> fp32 by truncation toward zero, with the last bit set
// when the conversion is inexact. A following RNE to a format with at most
// 22 significant bits then equals the single RNE of the fp64 value (the odd
// fp32 value never sits on a tie of the narrower format).
ARRMS_DEV float f64_to_f32_odd(double v)
{
    float f = (float)v;
    double b = (double)f;
    if (b != v) {
        uint32_t u = __float_as_uint(f);
        if (__builtin_fabs(b) > __builtin_fabs(v))
            u -= 1u;  // RNE went away from zero: step back to the truncated value
        f = __uint_as_float(u | 1u);
    }
    return f;
}

// --------------------------------------------------------------------------
// Element formats. A 16-byte pack is 4 words; a word holds EPW elements.
template <int DT> struct Fmt;

template <> struct Fmt<DT_BF16> {
    static constexpr int EPW = 2;
    ARRMS_DEV void unpack(uint32_t w, float (&f)[2])
    {
        f[0] = __uint_as_float(w << 16);
        f[1] = __uint_as_float(w & 0xffff0000u);
    }
    ARRMS_DEV uint32_t pack(const float (&f)[2])  // RNE (v_cvt_pk_bf16_f32)
    {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    }
    // the lanes of the wave whose fp32 value f sits exactly halfway between
    // two bf16 values (bf16 drops 16 bits, in the normal and the subnormal
    // range alike), as a mask
    ARRMS_DEV uint64_t tie_mask(float f) { return __builtin_amdgcn_ballot_w64((__float_as_uint(f) & 0xffffu) == 0x8000u); }
    ARRMS_DEV float exact(double v) { return f64_to_f32_odd(v); }
};

template <> struct Fmt<DT_FP16> {
    static constexpr int EPW = 2;
    ARRMS_DEV void unpack(uint32_t w, float (&f)[2])
    {
        f16x2 h = __builtin_bit_cast(f16x2, w);
        f[0] = (float)h.x;
        f[1] = (float)h.y;
    }
    ARRMS_DEV uint32_t pack(const float (&f)[2])  // RNE
    {
        f32x2 v = {f[0], f[1]};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    }
    // lanes at risk, as a wave mask: a tie of the normal fp16 range (13
    // dropped bits, incl. 65520 -> inf), or anything below 2^-14 (fp16
    // subnormals drop more bits). One ballot per compare: each is then the
    // compare's own lane mask (a ballot of the OR would go through a register)
    ARRMS_DEV uint64_t tie_mask(float f)
    {
        return __builtin_amdgcn_ballot_w64((__float_as_uint(f) << 19) == 0x80000000u) |
               __builtin_amdgcn_ballot_w64(__builtin_fabsf(f) < 0x1p-14f);
    }
    ARRMS_DEV float exact(double v) { return f64_to_f32_odd(v); }
};

template <> struct Fmt<DT_FP32> {
    static constexpr int EPW = 1;
    ARRMS_DEV void unpack(uint32_t w, float (&f)[1]) { f[0] = __uint_as_float(w); }
    ARRMS_DEV uint32_t pack(const float (&f)[1]) { return __float_as_uint(f[0]); }
    ARRMS_DEV uint64_t tie_mask(float) { return 0; }
    ARRMS_DEV float exact(double v) { return (float)v; }  // one RNE fp64 -> fp32
};

// --------------------------------------------------------------------------
// FP8 E4M3 ("fn": bias 7, max 448, no infinities, S.1111.111 = NaN).
// Exact encoder written from the format: RNE, saturating to +-448. Every NaN
// gets the one code 0x7F: the sign of a NaN is not fixed by the arithmetic
// that produced it.
ARRMS_DEV uint32_t e4m3_encode(float x)
{
    uint32_t b = __float_as_uint(x);
    uint32_t s = (b >> 24) & 0x80u;
    float a = __builtin_fabsf(x);
    if (!(a == a))
        return 0x7fu;
    if (a >= 464.0f)  // midpoint of 448 and (unrepresentable) 480 and beyond
        return s | 0x7eu;
    if (a < 0.015625f) {  // below 2^-6: multiples of 2^-9 (code 8 = 2^-6)
        return s | (uint32_t)__builtin_rintf(a * 512.0f);
    }
    int e = (int)((b >> 23) & 0xffu) - 127;  // -6 .. 8
    uint32_t m = (uint32_t)__builtin_rintf(__builtin_ldexpf(a, 3 - e));  // 8 .. 16
    return s | (((uint32_t)(e + 7) << 3) + (m - 8u));
}

// --------------------------------------------------------------------------
// Wave (64-lane) reductions of fp64 values: DPP within rows of 16 lanes,
// permlane swaps across rows. Every lane ends with the same bits (each step
// adds the same two operands on both partner lanes).
template <int CTRL> ARRMS_DEV double dpp_f64(double v)
{
    u32x2 w = __builtin_bit_cast(u32x2, v);
    w.x = __builtin_amdgcn_update_dpp(0u, w.x, CTRL, 0xf, 0xf, false);
    w.y = __builtin_amdgcn_update_dpp(0u, w.y, CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, w);
}

// Partner value across 16-lane rows: v_permlane16_swap / v_permlane32_swap
// (gfx950) exchange a register between lanes i and i^16 / i^32 without LDS.
// Each builtin returns the two swapped registers; with both operands equal to
// v, the pair holds v of lane i and v of lane i^m in an order that depends on
// the lane, so a sum of the pair is the same on both partner lanes.
template <bool ROW32> ARRMS_DEV u32x2 swap_pair(uint32_t x)
{
    u32x2 r;
    if constexpr (ROW32) {
        auto t = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        r.x = t[0];
        r.y = t[1];
    } else {
        auto t = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        r.x = t[0];
        r.y = t[1];
    }
    return r;
}

// (value of this lane, value of the partner lane), in a lane-dependent order
template <bool ROW32> ARRMS_DEV void pair_f64(double v, double &a, double &b)
{
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    const u32x2 lo = swap_pair<ROW32>(w.x);
    const u32x2 hi = swap_pair<ROW32>(w.y);
    a = __builtin_bit_cast(double, u32x2{lo.x, hi.x});
    b = __builtin_bit_cast(double, u32x2{lo.y, hi.y});
}

template <bool ROW32> ARRMS_DEV double sum_across(double v)
{
    double a, b;
    pair_f64<ROW32>(v, a, b);
    return a + b;
}

ARRMS_DEV double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    v = sum_across<false>(v);  // rows 0+1, 2+3
    v = sum_across<true>(v);   // halves
    return v;
}

// Block barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its outstanding global loads and stores.
ARRMS_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Streaming (read-once / write-once) data: non-temporal accesses, so the rank
// inputs and the outputs do not displace the reused lines (weights) in the
// caches.
ARRMS_DEV u32x4 ld16_nt(const void *p, long long i)
{
    return __builtin_nontemporal_load((const u32x4 *)p + i);
}
ARRMS_DEV void st16_nt(void *p, long long i, u32x4 v) { __builtin_nontemporal_store(v, (u32x4 *)p + i); }

// --------------------------------------------------------------------------
// Row kernel. A block holds rpb row groups of tpr threads (tpr a multiple of
// 64); a row group owns one row and each of its threads owns PPT packs of it
// (pack j = lane_in_group + k * tpr). The grid has one block per row group, so
// all rows the device can hold are in flight at once and a finished block is
// replaced at once by the dispatcher; a lean register budget (the row's R+1
// input packs, its h values and its weights) keeps several blocks resident
// per compute unit. Every thread of a block runs the same barriers (rows past
// M are idle slots), so no barrier sits in divergent control flow (PR #5807
// Proposed modifications). A ragged row (tpr * PPT > packs per row) needs no
// separate variant: the buffer range check zero-fills the missing packs and
// drops their stores, and zeros add nothing to the sum of squares or the
// maximum. EPI selects the epilogue: T output only, FP8 only, or FP8 with the
// T mirror.
// EPI_FP8G: per-group FP8 (scale per 128 columns); EPI_MX4: MXFP4 (E8M0
// scale per 32 columns, E2M1 codes). Both write the T mirror when out is set.
enum Epilogue { EPI_T = 0, EPI_FP8 = 1, EPI_FP8_T = 2, EPI_FP8G = 3, EPI_MX4 = 4 };

struct RowCtx {
    int lt;      // thread index within the row group
    int tpr;     // threads per row group
    int P;       // packs per row
    int slot;    // row group index within the block
    int wave;    // wave index within the block
    int lane;
    int wpr;     // waves per row group
    int rpb;     // row groups per block
};

// Memory access of the row kernel: buffer instructions. A row's base address
// is wave-uniform, so each stream gets a buffer resource (4 scalar registers)
// covering exactly that row, and a lane adds its 32-bit byte offset: one
// offset register serves every stream. The hardware range check of the
// resource does the tail handling: a load past the row returns zero and a
// store past it is dropped, so ragged rows run the same instruction stream as
// aligned ones, with no predicates and no divergent barriers.
constexpr int kBufAuxNT = 2;               // cache policy: non-temporal
constexpr int kBufDword3 = 0x00020000;     // 32-bit data format, raw (untyped) access

// Resource covering row_bytes bytes of the row that starts at base + row * ld.
ARRMS_DEV __amdgpu_buffer_rsrc_t row_rsrc(const void *base, long long row, long long ld, int row_bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + row * ld), (short)0, row_bytes,
                                             kBufDword3);
}

ARRMS_DEV u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kBufAuxNT));
}

// Reused data (the weights): default cache policy.
ARRMS_DEV u32x4 bload_cached(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

ARRMS_DEV void bstore(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, kBufAuxNT);
}

ARRMS_DEV void bstore8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, kBufAuxNT);
}

ARRMS_DEV void bstore4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kBufAuxNT);
}

// Phase 1 keeps at most W 16-byte loads of a thread in flight (a sliding
// window over the row's loads, pack by pack, input streams in rank order).
// HBM on MI355X delivers the most when roughly 6-9 MB are outstanding across
// the device. When every row of a large launch is resident at once, a window
// of kWindowLow loads per thread is that amount (more measured slower: the
// DRAM pages of the many streams get interleaved; fewer starve the memory
// pipeline) -- for rows of at most 6 input streams; rows of more (R > 5)
// measured faster with the wide window. Large launches that run in several
// rounds of blocks take the wide window (the whole row, up to kWindowHigh
// loads), and so do small
// launches, for which it issues every load at once: a wait inside the row
// would add a memory round trip to their latency. A medium window
// (kWindowMid) is there on explicit request: with residual_out written after
// the row reduction it was 0.45 us faster than the wide one for the per-token
// FP8 epilogue on 2800 x 6144 fp16 rows, but with residual_out after the
// codes (as now) the wide window is 0.1 us faster still; it was 0.2 us slower
// for per-group FP8 and equal for MXFP4 and for 18-load bf16 rows.
// The narrow window: 2 loads per thread; 3 for the two-stage row pass (R = 1).
// Measured on 1024 x 6144 rows with residual_out written after the T output:
// R = 4 14.34 -> 14.13-14.15 us from 3 to 2 (4: 14.33-14.35), R = 3 12.40 ->
// 12.29, R = 2 10.65 -> 10.61; the R = 1 row pass was 1.5 us slower at 2.
constexpr int kWindowLow = 2;
constexpr int kWindowLowR1 = 3;
template <int R> constexpr int window_low() { return R == 1 ? kWindowLowR1 : kWindowLow; }
constexpr int kWindowMid = 8;
constexpr int kWindowHigh = 16;

template <int N> ARRMS_DEV void wait_vm()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Buffer resources of one row's streams: the inputs (R rank inputs, then the
// residual) and the outputs (residual_out, the T output, the FP8 codes). A
// row past M gets empty resources: its loads return zero and its stores are
// dropped, so idle row slots run the same code as real rows.
template <int R>
ARRMS_DEV void in_streams(const RowArgs &a, long long row, int rb, __amdgpu_buffer_rsrc_t (&s)[R + 1])
{
    const int n = row < a.M ? rb : 0;
#pragma unroll
    for (int r = 0; r < R; ++r)
        s[r] = row_rsrc(a.in[r], row, a.ld_in, n);
    s[R] = row_rsrc(a.residual, row, a.ld_res, n);
}

// Output resource of a row (rows past M: empty); bytes = the row's bytes in
// that output.
ARRMS_DEV __amdgpu_buffer_rsrc_t out_stream(const void *base, long long row, long long ld, int bytes,
                                            long long M)
{
    return row_rsrc(base, row, ld, row < M ? bytes : 0);
}

// Phase-1 arithmetic of one pack: rank sum in fp32, RNE to T, residual add,
// RNE to T (h), exact squares of h into fp64 partial sums.
template <int DT, int R>
ARRMS_DEV void reduce_pack(const u32x4 (&x)[R + 1], u32x4 &hv, double (&ssw)[4])
{
    using F = Fmt<DT>;
    constexpr int EPW = F::EPW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float acc[EPW];
        F::unpack(x[0][i], acc);
#pragma unroll
        for (int r = 1; r < R; ++r) {
            float t[EPW];
            F::unpack(x[r][i], t);
#pragma unroll
            for (int e = 0; e < EPW; ++e)
                acc[e] = acc[e] + t[e];
        }
        float av[EPW], rsd[EPW], hf[EPW];
        F::unpack(F::pack(acc), av);  // a = RNE_T(sum)
        F::unpack(x[R][i], rsd);
#pragma unroll
        for (int e = 0; e < EPW; ++e)
            acc[e] = av[e] + rsd[e];
        const uint32_t hw = F::pack(acc);  // h = RNE_T(a + res)
        hv[i] = hw;
        F::unpack(hw, hf);
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
            const double hd = (double)hf[e];
            ssw[i] = __builtin_fma(hd, hd, ssw[i]);  // h^2 is exact in fp64
        }
    }
}

// Per-token FP8 steps on 8 T values with their scale: q = E4M3_RNE_sat(fl32(y /
// scale)). y * (1/scale) rounds like y / scale when it lies in the normal E4M3
// range [2^-6, 464) and at least 4 fp32 ulps from an E4M3 tie: the 20 bits
// below E4M3's mantissa, moved to the top of a word and offset, land at or
// below 6 << 12 exactly when they are within 3 ulps of the halfway pattern
// 0x80000. fast == true promises a normal, finite scale = fl32(amax / 448)
// with amax >= |y| (the maximum of these very T values, as both callers
// compute it); then |y * (1/scale)| <= 448 (1 + 2^-22) < 464, so only the
// lower bound needs a test (a NaN fails it too). Elements that fail the test
// (rare) are recomputed alone by IEEE division and the exact encoder; fast ==
// false takes that path for all.
ARRMS_DEV bool e4m3_fast_bad(float cq)
{
    const uint32_t t = (__float_as_uint(cq) << 12) + 0x80003000u;
    return !(__builtin_fabsf(cq) >= 0x1p-6f) | (t <= 0x6000u);
}

ARRMS_DEV u32x2 quant8_e4m3(const float (&y)[8], float scale, float inv, bool fast)
{
    u32x2 q = {0u, 0u};
    if (fast) {
        float cq[8];
        uint64_t anybad = 0;  // wave mask
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            // the two halves of e4m3_fast_bad as separate ballots: each is then
            // the compare's own lane mask (a ballot of their OR would first
            // turn the mask into a register and back)
            cq[e] = y[e] * inv;
            const uint32_t t = (__float_as_uint(cq[e]) << 12) + 0x80003000u;
            anybad |= __builtin_amdgcn_ballot_w64(!(__builtin_fabsf(cq[e]) >= 0x1p-6f));
            anybad |= __builtin_amdgcn_ballot_w64(t <= 0x6000u);
        }
        q.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cq[0], cq[1], 0, false);
        q.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cq[2], cq[3], (int)q.x, true);
        q.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cq[4], cq[5], 0, false);
        q.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(cq[6], cq[7], (int)q.y, true);
        if (anybad != 0) {
            // the test again, on opaque copies: keeping its results from above
            // alive would cost registers and instructions on the common path
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float c = cq[e];
                asm volatile("" : "+v"(c));
                const bool bad = e4m3_fast_bad(c);
                if (__builtin_amdgcn_ballot_w64(bad) != 0 && bad) {
                    const uint32_t b = e4m3_encode(y[e] / scale);
                    const int sh = 8 * (e & 3);
                    if (e < 4)
                        q.x = (q.x & ~(0xffu << sh)) | (b << sh);
                    else
                        q.y = (q.y & ~(0xffu << sh)) | (b << sh);
                }
            }
        }
    } else {
        uint32_t qb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            qb[e] = scale == 0.0f ? ((__float_as_uint(y[e]) >> 24) & 0x80u) : e4m3_encode(y[e] / scale);
        q.x = qb[0] | (qb[1] << 8) | (qb[2] << 16) | (qb[3] << 24);
        q.y = qb[4] | (qb[5] << 8) | (qb[6] << 16) | (qb[7] << 24);
    }
    return q;
}

// max |y| of a pack of 8 T values, as T bits: with the sign cleared the
// integer order of the bits is the order of |y| (a NaN ranks above infinity);
// two 16-bit lanes per word
ARRMS_DEV uint32_t absmax_tbits(const u32x4 &yv)
{
    u16x2 m = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, yv[i] & 0x7fff7fffu));
    return m.x > m.y ? m.x : m.y;
}

// max over aligned groups of N lanes (N = 4 or 16) by DPP within 16-lane rows;
// every lane of a group ends with the group's maximum
template <int N> ARRMS_DEV uint32_t group_max_u32(uint32_t v)
{
    uint32_t t = __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);  // quad_perm [1,0,3,2]
    v = t > v ? t : v;
    t = __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);           // quad_perm [2,3,0,1]
    v = t > v ? t : v;
    if constexpr (N == 16) {
        t = __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xf, 0xf, false);      // row_half_mirror
        v = t > v ? t : v;
        t = __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xf, 0xf, false);      // row_mirror
        v = t > v ? t : v;
    }
    return v;
}

// max over the whole wave: 16-lane rows by DPP, then across rows
ARRMS_DEV uint32_t wave_max_u32(uint32_t v)
{
    v = group_max_u32<16>(v);
    u32x2 t = swap_pair<false>(v);
    v = t.x > t.y ? t.x : t.y;
    t = swap_pair<true>(v);
    return t.x > t.y ? t.x : t.y;
}

// E8M0 code of an MX block scale from the block's max |y| bits (OCP
// Microscaling Formats v1.0, section 6.3): 2^(floor(log2 amax) - 2) for E2M1,
// the exponent clamped at -127 (zero and tiny blocks: code 0); a NaN or an
// infinity in the block gives the E8M0 NaN code 0xFF.
ARRMS_DEV uint32_t mx_scale_code(uint32_t am)
{
    if (am >= 0x7f800000u)
        return 0xffu;
    const uint32_t biased = am >> 23;  // floor(log2 amax) + 127 for normal amax
    return biased >= 2u ? biased - 2u : 0u;
}

// E2M1 codes of 8 T values under the block scale: y / X exactly (X a power of
// two), then round to nearest, ties to even, saturating at 6 -- counted as the
// number of E2M1 decision points the magnitude passes (a tie goes up only when
// the upper neighbour's code is even); packed two per byte, the even column in
// the low nibble. A block with a NaN or an infinity (scale code 0xFF) gets
// +-6's code throughout with the sign of y, and 0x7 for a NaN element (its
// sign is not fixed by the arithmetic); such blocks take a separate,
// wave-uniform branch.
ARRMS_DEV uint32_t mx_pack8(const float (&y)[8], uint32_t code)
{
    const float f = __uint_as_float((254u - (code < 254u ? code : 253u)) << 23);  // 2^(127 - code)
    uint32_t word = 0;
    if (__builtin_amdgcn_ballot_w64(code == 0xffu) == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = __builtin_fabsf(y[e] * f);
            uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
            c |= (__float_as_uint(y[e]) >> 28) & 0x8u;
            word |= c << (4 * e);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float a = __builtin_fabsf(y[e] * f);
            uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                         (uint32_t)(a > 5.0f);
            const uint32_t sg = (__float_as_uint(y[e]) >> 28) & 0x8u;
            if (code == 0xffu)
                c = y[e] == y[e] ? (7u | sg) : 7u;
            else
                c |= sg;
            word |= c << (4 * e);
        }
    }
    return word;
}

// The rows of one block: row group g = blockIdx.x, then g + gridDim.x, ...
// (with the default grid of one block per row group the loop runs once).
template <int DT, int R, int PPT, int EPI, int WIN>
ARRMS_DEV void row_loop(const RowArgs &a, const RowCtx &c, double (&red)[2][kMaxWavesPerBlock],
                        uint32_t (&redm)[kMaxWavesPerBlock])
{
    using F = Fmt<DT>;
    constexpr int EPW = F::EPW;
    constexpr bool FP8 = (EPI == EPI_FP8 || EPI == EPI_FP8_T);  // per-token FP8
    constexpr bool GROUPQ = (EPI == EPI_FP8G || EPI == EPI_MX4);
    constexpr bool OUT_T = (EPI == EPI_T || EPI == EPI_FP8_T);   // GROUPQ: when out is set
    constexpr int NS = R + 1;        // input streams
    constexpr int NL = PPT * NS;     // loads per thread and row
    constexpr int W = WIN < NL ? WIN : NL;
    // Where residual_out is written. A row whose loads are throttled by the
    // window writes it only after its reads are over (measured faster on
    // MI355X: the DRAM gives more when a row's reads and writes do not
    // interleave) -- after the row reduction, or, with 2 to 6 ranks, after
    // the row's other outputs (the T output, or the quantised codes). The
    // quant epilogues do so even when every load of the row is in flight at
    // once. Measured on 1024 x 6144 bf16 rows (T output): after the reduction
    // 14.70-14.82 us, after the T output 14.41-14.47 (R = 2: 11.02 -> 10.76,
    // R = 3: 13.03 -> 12.50, R = 6: 21.70 -> 21.56); slower at R = 8 (26.36 ->
    // 26.66) and for the R = 1 row pass of the two-stage path (+1 us per
    // call), which keep the earlier place. On 2800 x 6144 fp16 gemma rows the
    // quant forms gain 0.17 (per-token FP8, against the medium window with
    // residual_out after the reduction), 0.27 (per-group FP8) and 0.8 us
    // (MXFP4); the T output with every load in flight loses 0.04-0.1 us by
    // waiting, so it writes residual_out pack by pack in phase 1.
    constexpr bool mid_ranks = R >= 2 && R <= 6;
    constexpr bool quant_out = FP8 || GROUPQ;
    constexpr bool rout_late = W < NL || (quant_out && mid_ranks);
    constexpr bool rout_after_y = rout_late && (EPI == EPI_T || quant_out) && mid_ranks;
    // w_eff = w + gadd: 1 under gemma_norm, else -0.0, which adds nothing to
    // any value (signed zeros included), so one fp64 add serves both modes
    const double gadd = a.gemma ? 1.0 : -0.0;
    // plain weights with 16-bit data: h * w needs no gemma add (and, for
    // fp16, no fp64 product)
    const bool plain_product = DT != DT_FP32 && !a.gemma;
    const bool exact_only = a.exact_only != 0;
    const int rb = c.P * 16;
    int parity = 0;

    // Every argument in scalar registers at once: one round of kernel-argument
    // loads before the first row's loads instead of a chain of dependent ones
    // (measured 0.1 us per call on 1024 x 6144 and 16 x 6144 bf16 rows).
#pragma unroll
    for (int r = 0; r < R; ++r)
        asm volatile("" ::"s"(a.in[r]));
    asm volatile("" ::"s"(a.residual), "s"(a.weight), "s"(a.residual_out), "s"(a.out));
    asm volatile("" ::"s"(a.M), "s"(a.P), "s"(a.H), "s"(a.ld_in), "s"(a.ld_res), "s"(a.ld_rout), "s"(a.ld_out));
    asm volatile("" ::"s"(a.eps), "s"(a.gemma), "s"(a.exact_only), "s"(a.groups));
    if constexpr (FP8 || GROUPQ)
        asm volatile("" ::"s"(a.fp8_out), "s"(a.fp8_scale), "s"(a.q_scale), "s"(a.qgroups), "s"(a.ld_q));
    for (long long g = blockIdx.x; g < a.groups; g += gridDim.x) {
        // The weights (the same columns for every row, from L2) are read per
        // row, once the inputs are all issued, so that they neither hold
        // registers through phase 1 nor sit in the load window.
        const __amdgpu_buffer_rsrc_t rw = row_rsrc(a.weight, 0, 0, rb);
        u32x4 w[PPT];
        const long long row = g * c.rpb + c.slot;
        __amdgpu_buffer_rsrc_t sin[NS];
        in_streams<R>(a, row, rb, sin);

        // ---- rank sum, residual add, sum of squares:
        // load i is stream i % NS of pack i / NS; after issuing load i the
        // window waits for load i - (W - 1), and a pack is reduced as soon
        // as its last stream has landed
        u32x4 x[PPT][NS];
        u32x4 hv[PPT];
        double ssw[4] = {0.0, 0.0, 0.0, 0.0};  // one partial sum of squares per word
        // steps i = 0 .. NL + W - 2, as (kk, r) with i = kk * NS + r
        constexpr int KK = (NL + W - 1 + NS - 1) / NS;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
            for (int r = 0; r < NS; ++r) {
                const int i = kk * NS + r;
                if (i >= NL + W - 1)
                    break;
                if (i < NL) {
                    x[kk][r] = bload(sin[r], (uint32_t)(c.lt + kk * c.tpr) * 16u);  // kk < PPT here
                    wait_vm<W - 1>();
                }
                if (i == NL - 1) {
#pragma unroll
                    for (int k = 0; k < PPT; ++k)
                        w[k] = bload_cached(rw, (uint32_t)(c.lt + k * c.tpr) * 16u);
                }
                const int j = i - (W - 1);
                if (j >= 0 && j % NS == NS - 1) {
                    const int k = j / NS;
                    reduce_pack<DT, R>(x[k], hv[k], ssw);
                    if constexpr (!rout_late)
                        bstore(hv[k], out_stream(a.residual_out, row, a.ld_rout, rb, a.M),
                               (uint32_t)(c.lt + k * c.tpr) * 16u);
                }
            }
        }

        // ---- row reduction: wave DPP tree, then the row group's waves via LDS
        double ss = (ssw[0] + ssw[1]) + (ssw[2] + ssw[3]);
        ss = wave_sum_f64(ss);
        if (c.wpr > 1) {
            if (c.lane == 0)
                red[parity][c.wave] = ss;
            lds_barrier();
            const int w0 = c.slot * c.wpr;
            ss = red[parity][w0];
            for (int w = 1; w < c.wpr; ++w)
                ss += red[parity][w0 + w];
            parity ^= 1;
        }

        // ---- normalise, write the T output, FP8 epilogue
        // (h is re-read from its packed T form: keeping phase 1's fp64
        // conversions alive across the reduction would cost 16 registers a pack)
        // (the same for the weights: their fp64 forms from phase 1 are not kept)
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            asm volatile("" : "+v"(hv[k]));
            asm volatile("" : "+v"(w[k]));
        }
        const __amdgpu_buffer_rsrc_t rout_t = out_stream(a.out, row, a.ld_out, rb, a.M);
        const __amdgpu_buffer_rsrc_t rout_q =
            out_stream(a.fp8_out, row, a.ld_q, EPI == EPI_MX4 ? rb / 4 : rb / 2, a.M);
        // residual_out of a late row (see rout_late above)
        const __amdgpu_buffer_rsrc_t rout = out_stream(a.residual_out, row, a.ld_rout, rb, a.M);
        if constexpr (rout_late && !rout_after_y) {
#pragma unroll
            for (int k = 0; k < PPT; ++k)
                bstore(hv[k], rout, (uint32_t)(c.lt + k * c.tpr) * 16u);
        }
        const double rstd = 1.0 / __builtin_sqrt(ss / (double)a.H + (double)a.eps);
        // per-token FP8: the T-rounded y of every pack is kept for the quant,
        // which needs the row's max |y| (taken on the T bits, absmax_tbits)
        u32x4 yk[FP8 ? PPT : 1];
        uint32_t ym = 0;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const uint32_t off = (uint32_t)(c.lt + k * c.tpr) * 16u;
            u32x4 yv;
            // lanes with an element on a rounding tie of T, as a wave mask: the
            // whole wave then recomputes the pack on the exact branch (same
            // bits for the other lanes), so the branch stays wave-uniform
            uint64_t risk = exact_only ? ~0ull : 0ull;
            if (plain_product) {
                // fp16: h * w is exact in fp32 (11 + 11 significant bits, and
                // fp16's range keeps the product inside fp32's normal range), so
                // fl64(h * w) = (double)(h * w): one conversion instead of two.
                // bf16 shares fp32's exponent range: an fp32 product can overflow
                // or lose bits below 2^-126 where h * w * rstd is an ordinary
                // number, so the product is formed in fp64 (exact: 8 + 8 bits).
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float hf[EPW], wf[EPW], yf[EPW];
                    F::unpack(hv[k][i], hf);
                    F::unpack(w[k][i], wf);
#pragma unroll
                    for (int e = 0; e < EPW; ++e) {
                        if constexpr (DT == DT_BF16)
                            yf[e] = (float)(((double)hf[e] * (double)wf[e]) * rstd);
                        else
                            yf[e] = (float)((double)(hf[e] * wf[e]) * rstd);
                        risk |= F::tie_mask(yf[e]);
                    }
                    yv[i] = F::pack(yf);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float hf[EPW], wf[EPW], yf[EPW];
                    F::unpack(hv[k][i], hf);
                    F::unpack(w[k][i], wf);
#pragma unroll
                    for (int e = 0; e < EPW; ++e) {
                        const double we = (double)wf[e] + gadd;
                        yf[e] = (float)(((double)hf[e] * we) * rstd);
                        risk |= F::tie_mask(yf[e]);
                    }
                    yv[i] = F::pack(yf);
                }
            }
            if (risk != 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float hf[EPW], wf[EPW], yf[EPW];
                    F::unpack(hv[k][i], hf);
                    F::unpack(w[k][i], wf);
#pragma unroll
                    for (int e = 0; e < EPW; ++e) {
                        const double we = (double)wf[e] + gadd;
                        yf[e] = F::exact(((double)hf[e] * we) * rstd);
                    }
                    yv[i] = F::pack(yf);
                }
            }
            if constexpr (OUT_T)
                bstore(yv, rout_t, off);
            if constexpr (GROUPQ)
                if (a.out)
                    bstore(yv, rout_t, off);
            if constexpr (FP8 && DT != DT_FP32) {
                yk[k] = yv;
                const uint32_t t = absmax_tbits(yv);
                ym = t > ym ? t : ym;
            }
            if constexpr (GROUPQ && DT != DT_FP32) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t[2];
                    F::unpack(yv[i], t);
                    y[2 * i] = t[0];
                    y[2 * i + 1] = t[1];
                }
                const int pack = c.lt + k * c.tpr;  // pack index in the row
                if constexpr (EPI == EPI_FP8G) {
                    // group max over the 16 lanes holding a group's 16 packs
                    float gm[EPW];
                    F::unpack(group_max_u32<16>(absmax_tbits(yv)), gm);  // the T value in the low half
                    const float gmax = gm[0];
                    const float gscale = gmax / 448.0f;
                    const bool gfast = !exact_only && gscale >= 1.17549435e-38f && gscale <= 3.0e38f;
                    bstore8(quant8_e4m3(y, gscale, 1.0f / gscale, gfast), rout_q, off / 2u);
                    if ((pack & 15) == 0 && pack < c.P && row < a.M)
                        ((float *)a.q_scale)[row * a.qgroups + (pack >> 4)] = gscale;
                } else {
                    // MXFP4: block max over the 4 lanes holding a block's 4 packs
                    float bm[EPW];
                    F::unpack(group_max_u32<4>(absmax_tbits(yv)), bm);
                    const uint32_t code = mx_scale_code(__float_as_uint(bm[0]));
                    bstore4(mx_pack8(y, code), rout_q, off / 4u);
                    if ((pack & 3) == 0 && pack < c.P && row < a.M)
                        ((uint8_t *)a.q_scale)[row * a.qgroups + (pack >> 2)] = (uint8_t)code;
                }
            }
        }
        if constexpr (rout_after_y && !FP8) {
#pragma unroll
            for (int k = 0; k < PPT; ++k)
                bstore(hv[k], rout, (uint32_t)(c.lt + k * c.tpr) * 16u);
        }
        if constexpr (FP8 && DT != DT_FP32) {
            // the row's max |y|: wave tree, then the row group's waves via LDS
            // (a second barrier; the row's waves have all read red by then)
            uint32_t am = wave_max_u32(ym);
            if (c.wpr > 1) {
                if (c.lane == 0)
                    redm[c.wave] = am;
                lds_barrier();
                const int w0 = c.slot * c.wpr;
                am = redm[w0];
                for (int w = 1; w < c.wpr; ++w)
                    am = redm[w0 + w] > am ? redm[w0 + w] : am;
            }
            float amx[EPW];
            F::unpack(am, amx);  // the T value in the low half
            const float scale = amx[0] / 448.0f;
            const float inv = 1.0f / scale;
            const bool qfast = !exact_only && scale >= 1.17549435e-38f && scale <= 3.0e38f;
            if (c.lt == 0 && row < a.M)
                a.fp8_scale[row] = scale;
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                float y[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t[2];
                    F::unpack(yk[k][i], t);
                    y[2 * i] = t[0];
                    y[2 * i + 1] = t[1];
                }
                bstore8(quant8_e4m3(y, scale, inv, qfast), rout_q, (uint32_t)(c.lt + k * c.tpr) * 8u);
            }
            if constexpr (rout_after_y) {
#pragma unroll
                for (int k = 0; k < PPT; ++k)
                    bstore(hv[k], rout, (uint32_t)(c.lt + k * c.tpr) * 16u);
            }
        }
    }
}

// Blocks of up to 1024 threads for one pack per thread (a whole wide row per
// block) and for fp32 rows (up to 16384 elements = 4096 packs: 1024 threads x
// 4 packs), 512 otherwise (more packs per thread hold more registers).
template <int DT, int PPT> constexpr int row_max_block() { return (PPT == 1 || DT == DT_FP32) ? 1024 : 512; }

template <int DT, int R, int PPT, int EPI, int WIN>
__global__ void __launch_bounds__((row_max_block<DT, PPT>())) row_kernel(const RowArgs a)
{
    RowCtx c;
    const int tid = threadIdx.x;
    c.tpr = a.tpr;
    c.wpr = c.tpr >> 6;
    c.rpb = a.rpb;
    // a wave never straddles two row groups (tpr is a multiple of 64), so the
    // row-group index is wave-uniform: keep it in a scalar register (and skip
    // the division for blocks of one row group, the common case)
    c.slot = c.rpb == 1 ? 0 : __builtin_amdgcn_readfirstlane((tid >> 6) / c.wpr);
    c.lt = tid - c.slot * c.tpr;
    c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    c.lane = tid & 63;
    c.P = a.P;

    __shared__ double red[2][kMaxWavesPerBlock];
    __shared__ uint32_t redm[kMaxWavesPerBlock];

    row_loop<DT, R, PPT, EPI, WIN>(a, c, red, redm);
}

// --------------------------------------------------------------------------
// Flat rank reduce (stage 1 of two-stage, PR #3462 Technical Details; and the
// sum-only rank all-reduce): every thread reduces whole packs across the R
// inputs in rank order in fp32, rounds to T and writes the destination. No
// LDS, no barrier. Block b takes tile b % tiles of row b / tiles; a tile is
// kFlatTile packs. TAIL=false is the aligned variant (P a multiple of the
// tile): no bounds checks. With TAIL only the last tile of a row checks its
// bounds, and every thread still runs the same code path (PR #5807 Proposed
// modifications: complete tiles unpredicated, leftover packs reduced by their
// owner threads).
template <int DT, int R>
ARRMS_DEV void flat_packs(const FlatArgs &a, long long src_row, long long dst_row,
                          const long long (&j)[kFlatPacksPerThread], const bool (&ok)[kFlatPacksPerThread])
{
    using F = Fmt<DT>;
    constexpr int EPW = F::EPW;
    constexpr int NP = kFlatPacksPerThread;
    constexpr int NL = NP * R;
    constexpr int W = kFlatWindow < NL ? kFlatWindow : NL;
    u32x4 xv[NP][R];
    u32x4 out[NP];
    // loads in a sliding window (pack-major, ranks in order); a pack is
    // reduced as soon as its last rank has landed; the stores follow the loads
    constexpr int KK = (NL + W - 1 + R - 1) / R;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = kk * R + r;
            if (i >= NL + W - 1)
                break;
            if (i < NL) {
                if (ok[kk])
                    xv[kk][r] = ld16_nt(a.in[r], src_row + j[kk]);  // kk < NP here
                wait_vm<W - 1>();
            }
            const int jj = i - (W - 1);
            if (jj >= 0 && jj % R == R - 1) {
                const int k = jj / R;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float acc[EPW];
                    F::unpack(xv[k][0][q], acc);
#pragma unroll
                    for (int rr = 1; rr < R; ++rr) {
                        float t[EPW];
                        F::unpack(xv[k][rr][q], t);
#pragma unroll
                        for (int e = 0; e < EPW; ++e)
                            acc[e] = acc[e] + t[e];
                    }
                    out[k][q] = F::pack(acc);
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        if (!ok[k])
            continue;
        st16_nt(a.dst, dst_row + j[k], out[k]);
    }
}

template <int DT, int R, bool TAIL>
__global__ void __launch_bounds__(kFlatThreads) flat_kernel(const FlatArgs a)
{
    // every argument in scalar registers at once (one round of kernel-argument
    // loads), and no division for contiguous data, which is one row
    // (0.1 us per call on a 4 x 12 MiB sum)
#pragma unroll
    for (int r = 0; r < R; ++r)
        asm volatile("" ::"s"(a.in[r]));
    asm volatile("" ::"s"(a.dst), "s"(a.rows), "s"(a.P), "s"(a.ld_in), "s"(a.ld_out), "s"(a.tiles));
    const long long b = blockIdx.x;
    const long long row = a.rows == 1 ? 0 : b / a.tiles;  // scalar: one division per block
    const long long tile = b - row * a.tiles;
    const long long base = tile * kFlatTile + threadIdx.x;
    long long j[kFlatPacksPerThread];
    bool ok[kFlatPacksPerThread];
    const bool last = TAIL && tile == a.tiles - 1;
#pragma unroll
    for (int k = 0; k < kFlatPacksPerThread; ++k) {
        j[k] = base + (long long)k * kFlatThreads;
        ok[k] = !last || j[k] < a.P;
    }
    flat_packs<DT, R>(a, row * a.ld_in, row * a.ld_out, j, ok);
}

// --------------------------------------------------------------------------
// Launch helpers (instantiated per dtype by kern_*.hip).

// LDS bytes of one compute unit and the most one block may reserve (cached
// per device; 0 if the runtime cannot tell).
static void device_lds(int &per_cu, int &per_block)
{
    static std::atomic<int> cu_cache[kMaxDevices], blk_cache[kMaxDevices];
    per_cu = per_block = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return;
    }
    int c = cu_cache[dev].load(std::memory_order_relaxed), b = blk_cache[dev].load(std::memory_order_relaxed);
    if (c == 0 || b == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess ||
            hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) {
            (void)hipGetLastError();
            return;
        }
        cu_cache[dev].store(c, std::memory_order_relaxed);
        blk_cache[dev].store(b, std::memory_order_relaxed);
    }
    per_cu = c;
    per_block = b;
}

// Blocks of row_kernel<DT, R, PPT, EPI, window> one compute unit of the current
// device holds at this block size (0 if the runtime cannot tell). Cached per
// device, window (1 narrow, 2 wide, 3 medium) and block size.
template <int DT, int R, int PPT, int EPI>
static int row_occupancy(int block, int win)
{
    static std::atomic<uint8_t> cache[kMaxDevices][3][1024 / 64 + 1];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return 0;
    }
    if (block < 64 || block > 1024 || block % 64 != 0 || win < 1 || win > 3)
        return 0;
    std::atomic<uint8_t> &slot = cache[dev][win - 1][block / 64];
    int n = slot.load(std::memory_order_relaxed);
    if (n == 0) {
        hipError_t e;
        if (win == 1)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_kernel<DT, R, PPT, EPI, window_low<R>()>, block, 0);
        else if (win == 3 && (R + 1) * PPT > kWindowMid)
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_kernel<DT, R, PPT, EPI, kWindowMid>, block, 0);
        else
            e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, row_kernel<DT, R, PPT, EPI, kWindowHigh>, block, 0);
        if (e != hipSuccess || n <= 0 || n > 255) {
            (void)hipGetLastError();
            return 0;
        }
        slot.store((uint8_t)n, std::memory_order_relaxed);
    }
    return n;
}

// Launch of a planned shape (api.cpp sets every field: the window, and cap16 for
// launches that hold at most 16 waves per compute unit).
template <int DT, int R, int PPT, int EPI>
static hipError_t row_go(const RowArgs &a, const RowShape &s, hipStream_t st)
{
    const int block = s.tpr * s.rpb;
    const long long groups = (a.M + s.rpb - 1) / s.rpb;
    const long long grid = (s.grid > 0 && s.grid < groups) ? s.grid : groups;
    if (grid > 0x7fffffffLL || block > row_max_block<DT, PPT>() || s.tpr != a.tpr || s.window < 1 || s.window > 3)
        return hipErrorInvalidValue;
    RowArgs b = a;
    b.rpb = s.rpb;
    b.groups = groups;
    // The occupancy cap: LDS that the kernel does not use, reserved so that no
    // more blocks fit than 16 waves per compute unit. Only for blocks of at most
    // 512 threads: the reservation then stays below 64 KiB, which a launch may
    // take without a per-kernel attribute.
    size_t smem = 0;
    if (s.cap16) {
        int lds_cu = 0, lds_block = 0;
        device_lds(lds_cu, lds_block);
        const int cap = 1024 / block;  // blocks per compute unit for 16 waves
        const size_t want = (size_t)lds_cu / (size_t)(cap + 1) + 1;  // cap + 1 blocks do not fit
        if (cap >= 2 && lds_cu > 0 && want <= (size_t)lds_block && want <= (64u << 10))
            smem = (want + 255) & ~(size_t)255;
    }
    const dim3 g((unsigned)grid), t((unsigned)block);
    if (s.window == 1) {
        hipLaunchKernelGGL((row_kernel<DT, R, PPT, EPI, window_low<R>()>), g, t, smem, st, b);
    } else if (s.window == 3) {
        // rows of at most kWindowMid loads per thread: the medium window is the wide one
        if constexpr ((R + 1) * PPT > kWindowMid)
            hipLaunchKernelGGL((row_kernel<DT, R, PPT, EPI, kWindowMid>), g, t, smem, st, b);
        else
            hipLaunchKernelGGL((row_kernel<DT, R, PPT, EPI, kWindowHigh>), g, t, smem, st, b);
    } else {
        hipLaunchKernelGGL((row_kernel<DT, R, PPT, EPI, kWindowHigh>), g, t, smem, st, b);
    }
    return hipGetLastError();
}

template <int DT, int R, int EPI>
static int row_occupancy_r(const RowShape &s)
{
    const int block = s.tpr * s.rpb;
    switch (s.ppt) {
    case 1: return row_occupancy<DT, R, 1, EPI>(block, s.window);
    case 2: return row_occupancy<DT, R, 2, EPI>(block, s.window);
    case 3: return row_occupancy<DT, R, 3, EPI>(block, s.window);
    case 4: return row_occupancy<DT, R, 4, EPI>(block, s.window);
    default: return 0;
    }
}

template <int DT, int EPI>
static int row_occupancy_epi(int R, const RowShape &s)
{
    switch (R) {
    case 1: return row_occupancy_r<DT, 1, EPI>(s);
    case 2: return row_occupancy_r<DT, 2, EPI>(s);
    case 3: return row_occupancy_r<DT, 3, EPI>(s);
    case 4: return row_occupancy_r<DT, 4, EPI>(s);
    case 5: return row_occupancy_r<DT, 5, EPI>(s);
    case 6: return row_occupancy_r<DT, 6, EPI>(s);
    case 7: return row_occupancy_r<DT, 7, EPI>(s);
    case 8: return row_occupancy_r<DT, 8, EPI>(s);
    default: return 0;
    }
}

template <int DT, int R, int EPI>
static hipError_t row_go_r(const RowArgs &a, const RowShape &s, hipStream_t st)
{
    switch (s.ppt) {
    case 1: return row_go<DT, R, 1, EPI>(a, s, st);
    case 2: return row_go<DT, R, 2, EPI>(a, s, st);
    case 3: return row_go<DT, R, 3, EPI>(a, s, st);
    case 4: return row_go<DT, R, 4, EPI>(a, s, st);
    default: return hipErrorInvalidValue;
    }
}

// One epilogue of one dtype: R = 1 .. 8.
template <int DT, int EPI>
static hipError_t row_launch_epi(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    switch (R) {
    case 1: return row_go_r<DT, 1, EPI>(a, s, st);
    case 2: return row_go_r<DT, 2, EPI>(a, s, st);
    case 3: return row_go_r<DT, 3, EPI>(a, s, st);
    case 4: return row_go_r<DT, 4, EPI>(a, s, st);
    case 5: return row_go_r<DT, 5, EPI>(a, s, st);
    case 6: return row_go_r<DT, 6, EPI>(a, s, st);
    case 7: return row_go_r<DT, 7, EPI>(a, s, st);
    case 8: return row_go_r<DT, 8, EPI>(a, s, st);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int R>
static hipError_t flat_go(const FlatArgs &a, hipStream_t st)
{
    const long long blocks = a.rows * a.tiles;
    if (blocks <= 0)
        return hipSuccess;
    if (blocks > 0x7fffffffLL)
        return hipErrorInvalidValue;
    const bool tail = a.P % kFlatTile != 0;
    dim3 grid((unsigned)blocks), block(kFlatThreads);
    if (tail)
        hipLaunchKernelGGL((flat_kernel<DT, R, true>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((flat_kernel<DT, R, false>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <int DT>
static hipError_t flat_launch(const FlatArgs &a, int R, hipStream_t st)
{
    switch (R) {
    case 1: return flat_go<DT, 1>(a, st);
    case 2: return flat_go<DT, 2>(a, st);
    case 3: return flat_go<DT, 3>(a, st);
    case 4: return flat_go<DT, 4>(a, st);
    case 5: return flat_go<DT, 5>(a, st);
    case 6: return flat_go<DT, 6>(a, st);
    case 7: return flat_go<DT, 7>(a, st);
    case 8: return flat_go<DT, 8>(a, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace arrms
