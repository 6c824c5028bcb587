// sv_accept.h -- row merges, the accept decision and the residual element.
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ bool temperature_ok(float T) { return T >= 0.f && T != INFINITY; }

// ---------------------------------------------------------------------------
// Wave-level merges of one row's chunk partials `p[0..nc)` (lanes stride the
// chunks; the tail kernel stages them in LDS).  The same code merges target and draft rows, so equal rows merge to
// bitwise-equal statistics.

__device__ __forceinline__ void merge_sum(const RowPart *p, int nc, double c64, float &M, double &S)
{
    const int lane = threadIdx.x & 63;
    float m = -INFINITY;
    for (int c = lane; c < nc; c += 64) m = fmaxf(m, p[c].m);
    m = wave_max(m);
    double s = 0.0;
    for (int c = lane; c < nc; c += 64) {
        const RowPart r = p[c];
        if (r.m != -INFINITY && r.s != 0.0) s += r.s * exp2(((double)r.m - (double)m) * c64);
    }
    S = wave_sum(s);
    M = m;
}

__device__ __forceinline__ void merge_argmax(const RowPart *p, int nc, float &M, int &I)
{
    const int lane = threadIdx.x & 63;
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = lane; c < nc; c += 64) {
        const RowPart r = p[c];
        if (better(r.m, r.idx, v, i)) {
            v = r.m;
            i = r.idx;
        }
    }
    wave_argmax(v, i);
    M = v;
    I = i;
}

// A beta-weighted draft row.  Partials carry, per chunk, the chunk's top-4 and
// the sum over the chunk's other elements, so the mass outside the row's top-4
// is summed directly (never as S - S_top, which cancels when the top-4 hold
// nearly all the mass).  Returns the row max M, the row top-4, the mass
// outside it (S_rest) and inside it (S_top), all relative to exp2((z - M) c).
__device__ __forceinline__ void merge_weighted(const RowPart *p, const Top4 *tp, int nc, double c64,
                                               float &M, Top4 &row_top, double &S_rest,
                                               double &S_top)
{
    const int lane = threadIdx.x & 63;
    double s_excl;
    merge_sum(p, nc, c64, M, s_excl);
    Top4 t;
    top_clear(t);
    for (int c = lane; c < nc; c += 64) {
        const Top4 r = tp[c];
#pragma unroll
        for (int k = 0; k < 4; ++k) top_insert(t, r.v[k], r.i[k]);
    }
    row_top = wave_top4(t);
    double extra = 0.0;
    for (int c = lane; c < nc; c += 64) {
        const Top4 r = tp[c];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (r.i[k] != INT_MAX && r.v[k] != -INFINITY && !top_has(row_top, r.i[k]))
                extra += exp2(((double)r.v[k] - (double)M) * c64);
    }
    S_rest = s_excl + wave_sum(extra);
    double st = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (row_top.i[k] != INT_MAX && row_top.v[k] != -INFINITY)
            st += exp2(((double)row_top.v[k] - (double)M) * c64);
    S_top = st;
}

// ---------------------------------------------------------------------------
// One accept test ("Kangaroo: Self-Speculative Decoding via Shallow
// Sub-Networks", "3. Lossless Speculative Verification"; glossary
// "speculative decoding llm", "Why It Produces Identical Outputs"): accept x
// iff u <= p(x) / q'(x), formed in fp64 in the log domain,
//   ln p(x)  = (z_t(x) - m_t) / T - ln S_t,
//   ln q'(x) = (z_d(x) - m_d) / T + ln w(x) - ln D,
// with D = S_d unweighted, or S_rest + beta * S_top for the Saguaro-style
// draft ("Speculative Speculative Decoding", "Method"), w(x) = beta on the
// draft's top-4 and 1 elsewhere.  A token the draft law gives no mass is
// accepted (the ratio is +inf).
__device__ __forceinline__ bool decide(float T, float mt, double St, float md, double D,
                                       bool weighted_top, float beta, bool x_ok, float zt, float zd,
                                       float u, float &pt, float &pd)
{
    const double Td = (double)T;
    double ratio = 0.0;
    pt = NAN;
    pd = NAN;
    if (x_ok) {
        const double lpt = ((double)zt - (double)mt) / Td - log(St);
        double lpd = ((double)zd - (double)md) / Td - log(D);
        if (weighted_top) lpd += log((double)beta);
        ratio = (lpd == -INFINITY) ? INFINITY : exp(lpt - lpd);
        pt = (float)exp(lpt);
        pd = (float)exp(lpd);
    }
    return (double)u <= ratio;
}

// ---------------------------------------------------------------------------
// Residual of one element ("Kangaroo ...", "3. Lossless Speculative
// Verification", the corrected distribution max(0, p - q); "Speculative
// Speculative Decoding", "Key claims", the residual max(p_t - p_d, 0)):
// p_t in mode 2; in mode 1
//   r(v) = max(p_t(v) - q'(v), 0) = p_t(v) * (1 - 2^d(v))  for d(v) < 0, else 0,
// both returned times S_t (p_t(v) S_t = exp2((z_t(v) - m_t) log2e / T)): a
// factor common to the whole row, which cancels in the inverse CDF;
//   d(v) = log2 q'(v) - log2 p_t(v) = (z_d(v) - z_t(v)) log2e / T + k2 (+ log2 beta),
// so r keeps its relative accuracy when p_t and q' nearly cancel (small
// residual mass), where p_t - q' taken in fp32 would carry an absolute error
// of ~1e-7 of p_t.  d is formed in fp32 from constants split into hi + lo
// parts: fma(delta, c_hi, k_hi) rounds once, so d carries an error of a few
// ulp of d itself, not of its terms.

struct ResidualScale {
    float c_hi, c_lo;    // log2e / T
    float k_hi, k_lo;    // k2
    float kt_hi, kt_lo;  // k2 + log2 beta (draft top-4 tokens)
};

__device__ __forceinline__ ResidualScale make_residual_scale(const SeqState &st, const ExpScale &e)
{
    ResidualScale r;
    r.c_hi = e.hi;
    r.c_lo = e.lo;
    r.k_hi = (float)st.k2;
    r.k_lo = (float)(st.k2 - (double)r.k_hi);
    const double kt = st.k2 + (double)st.lbeta;  // -inf when beta == 0
    r.kt_hi = (float)kt;
    r.kt_lo = isfinite(kt) ? (float)(kt - (double)r.kt_hi) : 0.f;
    return r;
}

// 1 - 2^d for d < 0, to a few ulp: a degree-9 Taylor series of -expm1(d ln2)
// for d > -1 (truncation below 1e-8 relative), 1 - exp2(d) below, where
// 2^d <= 1/2 keeps the subtraction well conditioned.
__device__ __forceinline__ float one_minus_exp2(float d)
{
    const float y = d * 0.693147180559945f;
    float p = __builtin_fmaf(y, 1.f / 362880.f, 1.f / 40320.f);
    p = __builtin_fmaf(y, p, 1.f / 5040.f);
    p = __builtin_fmaf(y, p, 1.f / 720.f);
    p = __builtin_fmaf(y, p, 1.f / 120.f);
    p = __builtin_fmaf(y, p, 1.f / 24.f);
    p = __builtin_fmaf(y, p, 1.f / 6.f);
    p = __builtin_fmaf(y, p, 0.5f);
    p = __builtin_fmaf(y, p, 1.f);
    const float series = -(y * p);
    const float direct = 1.f - __builtin_amdgcn_exp2f(d);
    return d > -1.f ? series : direct;
}

template <bool TOP>
__device__ __forceinline__ float residual_at(float zt, float zd, int v, const SeqState &st,
                                             const ExpScale &e, const ResidualScale &rs, int mode)
{
    const float pt = exp_scaled(zt, st.m_t, e);  // p_t(v) * S_t
    if (mode == 2) return pt;
    const float delta = zd - zt;
    bool top = false;
    if (TOP) top = v == st.top[0] || v == st.top[1] || v == st.top[2] || v == st.top[3];
    const float khi = top ? rs.kt_hi : rs.k_hi;
    const float klo = top ? rs.kt_lo : rs.k_lo;
    const float d = __builtin_fmaf(delta, rs.c_hi, khi) + __builtin_fmaf(delta, rs.c_lo, klo);
    if (!(d < 0.f)) return 0.f;  // q' >= p_t, or a masked target token
    return pt * one_minus_exp2(d);
}

}  // namespace sv
