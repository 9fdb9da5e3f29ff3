// kernels.hpp -- gfx950 kernels of the fused rank-sum + residual-add + RMSNorm
// (+ per-token FP8 E4M3) epilogue. Included by the per-dtype translation units.
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

#include "launch.hpp"

namespace arrms {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

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
    // fp32 value exactly halfway between two bf16 values (bf16 drops 16 bits,
    // in the normal and the subnormal range alike)
    ARRMS_DEV bool tie_risk(float f) { return (__float_as_uint(f) & 0xffffu) == 0x8000u; }
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
    // a tie of the normal fp16 range (13 dropped bits, incl. 65520 -> inf),
    // or anything below 2^-14 (fp16 subnormals drop more bits): exact branch
    ARRMS_DEV bool tie_risk(float f)
    {
        uint32_t u = __float_as_uint(f) & 0x7fffffffu;
        return ((u & 0x1fffu) == 0x1000u) | (u < (113u << 23));
    }
    ARRMS_DEV float exact(double v) { return f64_to_f32_odd(v); }
};

template <> struct Fmt<DT_FP32> {
    static constexpr int EPW = 1;
    ARRMS_DEV void unpack(uint32_t w, float (&f)[1]) { f[0] = __uint_as_float(w); }
    ARRMS_DEV uint32_t pack(const float (&f)[1]) { return __float_as_uint(f[0]); }
    ARRMS_DEV bool tie_risk(float) { return false; }
    ARRMS_DEV float exact(double v) { return (float)v; }  // one RNE fp64 -> fp32
};

// RNE_T of one fp64 value, returned as its (exact) fp32 value.
template <int DT> ARRMS_DEV float round_one(double v, bool exact_only)
{
    using F = Fmt<DT>;
    float f = (float)v;
    if (exact_only || F::tie_risk(f))
        f = F::exact(v);
    float r[F::EPW] = {};
    float in[F::EPW] = {};
    in[0] = f;
    F::unpack(F::pack(in), r);
    return r[0];
}

// --------------------------------------------------------------------------
// FP8 E4M3 ("fn": bias 7, max 448, no infinities, S.1111.111 = NaN).
// Exact encoder written from the format: RNE, saturating to +-448.
ARRMS_DEV uint32_t e4m3_encode(float x)
{
    uint32_t b = __float_as_uint(x);
    uint32_t s = (b >> 24) & 0x80u;
    float a = __builtin_fabsf(x);
    if (!(a == a))
        return s | 0x7fu;
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
// ds_bpermute across rows. Every lane ends with the same bits (each step adds
// the same two operands on both partner lanes).
template <int CTRL> ARRMS_DEV double dpp_f64(double v)
{
    u32x2 w = __builtin_bit_cast(u32x2, v);
    w.x = __builtin_amdgcn_update_dpp(0u, w.x, CTRL, 0xf, 0xf, false);
    w.y = __builtin_amdgcn_update_dpp(0u, w.y, CTRL, 0xf, 0xf, false);
    return __builtin_bit_cast(double, w);
}

ARRMS_DEV double xor_lanes_f64(double v, int mask)
{
    int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    int addr = (lane ^ mask) << 2;
    u32x2 w = __builtin_bit_cast(u32x2, v);
    w.x = __builtin_amdgcn_ds_bpermute(addr, w.x);
    w.y = __builtin_amdgcn_ds_bpermute(addr, w.y);
    return __builtin_bit_cast(double, w);
}

ARRMS_DEV double wave_sum_f64(double v)
{
    v += dpp_f64<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f64<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f64<0x141>(v);  // row_half_mirror
    v += dpp_f64<0x140>(v);  // row_mirror
    v += xor_lanes_f64(v, 16);
    v += xor_lanes_f64(v, 32);
    return v;
}

ARRMS_DEV double wave_max_f64(double v)
{
    v = __builtin_fmax(v, dpp_f64<0xB1>(v));
    v = __builtin_fmax(v, dpp_f64<0x4E>(v));
    v = __builtin_fmax(v, dpp_f64<0x141>(v));
    v = __builtin_fmax(v, dpp_f64<0x140>(v));
    v = __builtin_fmax(v, xor_lanes_f64(v, 16));
    v = __builtin_fmax(v, xor_lanes_f64(v, 32));
    return v;
}

// Block barrier for LDS traffic only: waits for this wave's LDS operations,
// not for its outstanding global loads and stores.
ARRMS_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

ARRMS_DEV u32x4 ld16(const void *p, long long i) { return ((const u32x4 *)p)[i]; }
ARRMS_DEV void st16(void *p, long long i, u32x4 v) { ((u32x4 *)p)[i] = v; }

// --------------------------------------------------------------------------
// Row kernel. A block holds rpb row groups of tpr threads (tpr a multiple of
// 64); a row group owns one row at a time and each of its threads owns PPT
// packs of it (pack j = lane_in_group + k * tpr). Rows are visited with a
// grid stride; every thread runs the same number of loop trips and barriers
// (rows past M run as idle slots), so no barrier sits in divergent control
// flow (PR #5807 Proposed modifications). TAIL=false is the aligned variant
// (tpr * PPT == packs per row): no predicates at all.
template <int DT, int R, int PPT, bool TAIL>
__global__ void __launch_bounds__(512) row_kernel(const RowArgs a)
{
    using F = Fmt<DT>;
    constexpr int EPW = F::EPW;
    const int tid = threadIdx.x;
    const int tpr = a.tpr;
    const int wpr = tpr >> 6;
    const int rpb = (int)blockDim.x / tpr;
    const int slot = tid / tpr;
    const int lt = tid - slot * tpr;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int P = a.P;
    const bool gemma = a.gemma != 0;
    const bool fp8 = (DT != DT_FP32) && a.fp8 != 0;
    const bool exact_only = a.exact_only != 0;

    __shared__ double red[2][kMaxWavesPerBlock][2];

    u32x4 wv[PPT];
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
        const int j = lt + k * tpr;
        wv[k] = (!TAIL || j < P) ? ld16(a.weight, j) : u32x4{0u, 0u, 0u, 0u};
    }

    const long long groups = (a.M + rpb - 1) / rpb;
    int parity = 0;
    for (long long g = blockIdx.x; g < groups; g += gridDim.x) {
        const long long row = g * rpb + slot;
        const bool valid = row < a.M;
        const long long base = row * (long long)P;

        // ---- loads: all R inputs and the residual for this thread's packs
        u32x4 xv[R][PPT];
        u32x4 rv[PPT];
        if (valid) {
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int j = lt + k * tpr;
                if (!TAIL || j < P) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
                        xv[r][k] = ld16(a.in[r], base + j);
                    rv[k] = ld16(a.residual, base + j);
                }
            }
        }

        // ---- rank sum, residual add, sum of squares (and max |h * w_eff|)
        u32x4 hv[PPT];
        double ss = 0.0;
        double pm = 0.0;
        if (valid) {
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int j = lt + k * tpr;
                if (!TAIL || j < P) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float acc[EPW];
                        F::unpack(xv[0][k][i], acc);
#pragma unroll
                        for (int r = 1; r < R; ++r) {
                            float t[EPW];
                            F::unpack(xv[r][k][i], t);
#pragma unroll
                            for (int e = 0; e < EPW; ++e)
                                acc[e] = acc[e] + t[e];
                        }
                        float av[EPW], rs[EPW], hf[EPW];
                        F::unpack(F::pack(acc), av);  // a = RNE_T(sum)
                        F::unpack(rv[k][i], rs);
#pragma unroll
                        for (int e = 0; e < EPW; ++e)
                            acc[e] = av[e] + rs[e];
                        const uint32_t hw = F::pack(acc);  // h = RNE_T(a + res)
                        hv[k][i] = hw;
                        F::unpack(hw, hf);
#pragma unroll
                        for (int e = 0; e < EPW; ++e) {
                            const double hd = (double)hf[e];
                            ss = __builtin_fma(hd, hd, ss);  // h^2 is exact in fp64
                        }
                        if (fp8) {
                            float wf[EPW];
                            F::unpack(wv[k][i], wf);
#pragma unroll
                            for (int e = 0; e < EPW; ++e) {
                                const double we = gemma ? (double)wf[e] + 1.0 : (double)wf[e];
                                pm = __builtin_fmax(pm, __builtin_fabs((double)hf[e] * we));
                            }
                        }
                    }
                    st16(a.residual_out, base + j, hv[k]);
                }
            }
        }

        // ---- row reduction: wave DPP tree, then the row group's waves via LDS
        ss = wave_sum_f64(ss);
        if (fp8)
            pm = wave_max_f64(pm);
        if (wpr > 1) {
            if (lane == 0) {
                red[parity][wave][0] = ss;
                red[parity][wave][1] = pm;
            }
            lds_barrier();
            const int w0 = slot * wpr;
            ss = red[parity][w0][0];
            pm = red[parity][w0][1];
            for (int w = 1; w < wpr; ++w) {
                ss += red[parity][w0 + w][0];
                pm = __builtin_fmax(pm, red[parity][w0 + w][1]);
            }
            parity ^= 1;
        }

        // ---- normalise, write the T output, FP8 epilogue
        if (valid) {
            const double rstd = 1.0 / __builtin_sqrt(ss / (double)a.H + (double)a.eps);
            float scale = 0.0f, inv = 0.0f;
            bool qfast = false;
            if (fp8) {
                // max |y| = RNE_T(max |h * w_eff| * rstd): rounding is monotone
                const float amax = round_one<DT>(pm * rstd, exact_only);
                scale = amax / 448.0f;
                inv = 1.0f / scale;
                qfast = !exact_only && scale >= 1.17549435e-38f && scale <= 3.0e38f;
                if (lt == 0)
                    a.fp8_scale[row] = scale;
            }
#pragma unroll
            for (int k = 0; k < PPT; ++k) {
                const int j = lt + k * tpr;
                if (TAIL && j >= P)
                    continue;
                u32x4 yv;
                bool risk = exact_only;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float hf[EPW], wf[EPW], yf[EPW];
                    F::unpack(hv[k][i], hf);
                    F::unpack(wv[k][i], wf);
#pragma unroll
                    for (int e = 0; e < EPW; ++e) {
                        const double we = gemma ? (double)wf[e] + 1.0 : (double)wf[e];
                        yf[e] = (float)(((double)hf[e] * we) * rstd);
                        risk |= F::tie_risk(yf[e]);
                    }
                    yv[i] = F::pack(yf);
                }
                if (risk) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float hf[EPW], wf[EPW], yf[EPW];
                        F::unpack(hv[k][i], hf);
                        F::unpack(wv[k][i], wf);
#pragma unroll
                        for (int e = 0; e < EPW; ++e) {
                            const double we = gemma ? (double)wf[e] + 1.0 : (double)wf[e];
                            yf[e] = F::exact(((double)hf[e] * we) * rstd);
                        }
                        yv[i] = F::pack(yf);
                    }
                }
                if (a.out)
                    st16(a.out, base + j, yv);
                if constexpr (DT != DT_FP32) {
                    if (fp8) {
                        float y[8];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            float t[2];
                            F::unpack(yv[i], t);
                            y[2 * i] = t[0];
                            y[2 * i + 1] = t[1];
                        }
                        u32x2 q = {0u, 0u};
                        bool slow = !qfast;
                        if (qfast) {
                            float c[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                c[e] = y[e] * inv;
                                const uint32_t u = __float_as_uint(c[e]) & 0x7fffffffu;
                                const uint32_t lo = u & 0xfffffu;
                                // normal E4M3 range [2^-6, 464) and at least 4 fp32 ulps from
                                // an E4M3 tie: y * (1/scale) then rounds like y / scale
                                const bool ok = (u >= 0x3C800000u) & (u < 0x43E80000u) &
                                                ((lo + 3u - 0x80000u) > 6u);
                                slow |= !ok;
                            }
                            q.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
                            q.x = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], (int)q.x, true);
                            q.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
                            q.y = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], (int)q.y, true);
                        }
                        if (slow) {
                            uint32_t b[8];
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                b[e] = scale == 0.0f ? ((__float_as_uint(y[e]) >> 24) & 0x80u)
                                                     : e4m3_encode(y[e] / scale);
                            q.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
                            q.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
                        }
                        ((u32x2 *)a.fp8_out)[base + j] = q;
                    }
                }
            }
        }
    }
}

// --------------------------------------------------------------------------
// Flat rank reduce (stage 1 of two-stage, PR #3462 Technical Details): every
// thread reduces whole packs across the R inputs in rank order in fp32,
// rounds to T and writes the staging buffer. No LDS, no barrier. Tiles are
// kFlatTile packs; only the last block of a TAIL grid checks bounds.
template <int DT, int R>
ARRMS_DEV void flat_packs(const FlatArgs &a, const long long (&j)[kFlatPacksPerThread],
                          const bool (&ok)[kFlatPacksPerThread])
{
    using F = Fmt<DT>;
    constexpr int EPW = F::EPW;
    u32x4 xv[R][kFlatPacksPerThread];
#pragma unroll
    for (int k = 0; k < kFlatPacksPerThread; ++k)
        if (ok[k]) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                xv[r][k] = ld16(a.in[r], j[k]);
        }
#pragma unroll
    for (int k = 0; k < kFlatPacksPerThread; ++k) {
        if (!ok[k])
            continue;
        u32x4 out;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float acc[EPW];
            F::unpack(xv[0][k][i], acc);
#pragma unroll
            for (int r = 1; r < R; ++r) {
                float t[EPW];
                F::unpack(xv[r][k][i], t);
#pragma unroll
                for (int e = 0; e < EPW; ++e)
                    acc[e] = acc[e] + t[e];
            }
            out[i] = F::pack(acc);
        }
        st16(a.dst, j[k], out);
    }
}

template <int DT, int R, bool TAIL>
__global__ void __launch_bounds__(kFlatThreads) flat_kernel(const FlatArgs a)
{
    const long long base = (long long)blockIdx.x * kFlatTile + threadIdx.x;
    long long j[kFlatPacksPerThread];
    bool ok[kFlatPacksPerThread];
    const bool last = TAIL && blockIdx.x == gridDim.x - 1;
#pragma unroll
    for (int k = 0; k < kFlatPacksPerThread; ++k) {
        j[k] = base + (long long)k * kFlatThreads;
        ok[k] = !last || j[k] < a.npacks;
    }
    flat_packs<DT, R>(a, j, ok);
}

// --------------------------------------------------------------------------
// Launch helpers (instantiated per dtype by kern_*.hip).
template <int DT, int R, int PPT>
static hipError_t row_go(const RowArgs &a, const RowShape &s, hipStream_t st)
{
    if constexpr (PPT * (R + 1) > 45) {
        return hipErrorInvalidValue;  // register budget: never selected
    } else {
        dim3 grid((unsigned)s.grid), block((unsigned)(s.tpr * s.rpb));
        if (s.tail)
            hipLaunchKernelGGL((row_kernel<DT, R, PPT, true>), grid, block, 0, st, a);
        else
            hipLaunchKernelGGL((row_kernel<DT, R, PPT, false>), grid, block, 0, st, a);
        return hipGetLastError();
    }
}

template <int DT, int R>
static hipError_t row_go_r(const RowArgs &a, const RowShape &s, hipStream_t st)
{
    switch (s.ppt) {
    case 1: return row_go<DT, R, 1>(a, s, st);
    case 2: return row_go<DT, R, 2>(a, s, st);
    case 4: return row_go<DT, R, 4>(a, s, st);
    case 8: return row_go<DT, R, 8>(a, s, st);
    default: return hipErrorInvalidValue;
    }
}

template <int DT>
static hipError_t row_launch(const RowArgs &a, int R, const RowShape &s, hipStream_t st)
{
    switch (R) {
    case 1: return row_go_r<DT, 1>(a, s, st);
    case 2: return row_go_r<DT, 2>(a, s, st);
    case 3: return row_go_r<DT, 3>(a, s, st);
    case 4: return row_go_r<DT, 4>(a, s, st);
    case 5: return row_go_r<DT, 5>(a, s, st);
    case 6: return row_go_r<DT, 6>(a, s, st);
    case 7: return row_go_r<DT, 7>(a, s, st);
    case 8: return row_go_r<DT, 8>(a, s, st);
    default: return hipErrorInvalidValue;
    }
}

template <int DT, int R>
static hipError_t flat_go(const FlatArgs &a, hipStream_t st)
{
    const long long tiles = (a.npacks + kFlatTile - 1) / kFlatTile;
    const bool tail = a.npacks % kFlatTile != 0;
    dim3 grid((unsigned)tiles), block(kFlatThreads);
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
