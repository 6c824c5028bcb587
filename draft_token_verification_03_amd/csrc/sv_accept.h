// sv_accept.h -- row merges, the accept decision and the residual element.
#pragma once

#include "sv_internal.h"

namespace sv {

__device__ __forceinline__ bool temperature_ok(float T) { return T >= 0.f && T != INFINITY; }

// ---------------------------------------------------------------------------
// Wave-level merges of one row's chunk partials `p[0..nc)` (lanes stride the
// chunks; the accept scan stages them in LDS).  A chunk's sum is relative to
// its own offset fp32(m_c c); the merged sum S is relative to the row's,
// fp32(M c).  The same code merges target and draft rows, so equal rows merge
// to bitwise-equal statistics.

__device__ __forceinline__ void merge_sum(const RowPart *p, int nc, const ExpScale &e, float &M, double &S)
{
    if (nc == 1) {  // a whole row per chunk: its partial is the row's statistic
        M = p[0].m;
        S = p[0].s;
        return;
    }
    const int lane = threadIdx.x & 63;
    float m = -INFINITY;
    for (int c = lane; c < nc; c += 64) m = fmaxf(m, p[c].m);
    m = wave_max(m);
    const double om = (double)row_offset(m, e);
    double s = 0.0;
    for (int c = lane; c < nc; c += 64) {
        const RowPart r = p[c];
        if (r.m != -INFINITY && r.s != 0.0) s += r.s * exp2((double)row_offset(r.m, e) - om);
    }
    S = wave_sum(s);
    M = m;
}

__device__ __forceinline__ void merge_argmax(const RowPart *p, int nc, float &M, int &I)
{
    if (nc == 1) {
        M = p[0].m;
        I = p[0].idx;
        return;
    }
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

// The normaliser D = S_rest + beta * S_top of a beta-weighted draft row from
// the mass outside its top-4 and the top-4 itself, relative to the offset om.
__device__ __forceinline__ double weighted_norm(double S_rest, const Top4 &t, double om, double c64,
                                                double beta)
{
    double st = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (t.i[k] != INT_MAX && t.v[k] != -INFINITY) st += exp_scaled64(t.v[k], om, c64);
    return S_rest + beta * st;
}

// A beta-weighted draft row.  Partials carry, per chunk, the chunk's top-4 and
// the sum over the chunk's other elements, so the mass outside the row's top-4
// is summed directly (never as S - S_top, which cancels when the top-4 hold
// nearly all the mass).  A row of one chunk already carries D (the streaming
// pass forms it).  Returns the row max M, the row top-4, D and the row's sum
// before the re-weighting Du, relative to exp2((z - M) c).  (Rows of more
// than one chunk only.)
__device__ __forceinline__ void merge_weighted(const RowPart *p, const Top4 *tp, int nc,
                                               const ExpScale &e, double beta, float &M, Top4 &row_top,
                                               double &D, double &Du)
{
    const int lane = threadIdx.x & 63;
    double s_excl;
    merge_sum(p, nc, e, M, s_excl);
    const double om = (double)row_offset(M, e);
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
                extra += exp_scaled64(r.v[k], om, e.c64);
    }
    const double s_rest = s_excl + wave_sum(extra);
    D = weighted_norm(s_rest, row_top, om, e.c64, beta);
    Du = weighted_norm(s_rest, row_top, om, e.c64, 1.0);
}

// ---------------------------------------------------------------------------
// One accept test ("Kangaroo: Self-Speculative Decoding via Shallow
// Sub-Networks", "3. Lossless Speculative Verification"; glossary
// "speculative decoding llm", "Why It Produces Identical Outputs"): accept x
// iff u <= p(x) / q'(x), with the ratio formed in fp64 in base 2,
//   log2 r = (z_t(x) c - o_t) - (z_d(x) c - o_d) + log2(D / S_t) - log2 w(x),
// where o_t, o_d are the rows' offsets, S_t the target row's sum relative to
// o_t, D the draft row's normaliser relative to o_d (S_d unweighted, or
// S_rest + beta * S_top for the Saguaro-style draft, "Speculative Speculative
// Decoding", "Method"), and w(x) = beta on the draft's top-4, 1 elsewhere
// (log2_beta from the host), and lq = log2(D / S_t) from the caller.  Only the
// final exponential is fp32: rounding
// log2 r to fp32 moves r by at most r |ln r| 2^-24 <= 2.2e-8 where r <= 1,
// below the uniforms' 2^-24 grid.  A token the draft law gives no mass is
// accepted (the ratio is +inf).  The diagnostics p(x), q'(x) are only formed
// when asked for.
__device__ __forceinline__ bool decide(const ExpScale &e, float ot, double St, float od, double D,
                                       double lq, bool weighted_top, double log2_beta, bool x_ok,
                                       float zt, float zd, float u, bool want_p, float &pt, float &pd)
{
    pt = NAN;
    pd = NAN;
    if (!x_ok) return false;
    const double lt = (double)zt * e.c64 - (double)ot;  // log2(p(x) S_t), zt c exact
    const double ld = (double)zd * e.c64 - (double)od;  // log2(q(x) D / w(x))
    const bool no_draft_mass = zd == -INFINITY || (weighted_top && log2_beta == -INFINITY);
    double lr = lt - ld + lq;
    if (weighted_top) lr -= log2_beta;
    const bool accept = no_draft_mass || (double)u <= (double)__builtin_amdgcn_exp2f((float)lr);
    if (want_p) {
        const double lpd = ld - log2(D) + (weighted_top ? log2_beta : 0.0);
        pt = __builtin_amdgcn_exp2f((float)(lt - log2(St)));
        pd = __builtin_amdgcn_exp2f((float)lpd);
    }
    return accept;
}

// ---------------------------------------------------------------------------
// Residual of one element ("Kangaroo ...", "3. Lossless Speculative
// Verification", the corrected distribution max(0, p - q); "Speculative
// Speculative Decoding", "Key claims", the residual max(p_t - p_d, 0)):
// p_t in mode 2; in mode 1
//   r(v) = max(p_t(v) - q'(v), 0) = p_t(v) * (1 - 2^d(v))  for d(v) < 0, else 0,
// both returned times S_t (p_t(v) S_t = exp2(z_t(v) c - o_t)): a
// factor common to the whole row, which cancels in the inverse CDF;
//   d(v) = log2 q'(v) - log2 p_t(v) = (z_d(v) - z_t(v)) c + k2 (+ log2 beta),
//   k2 = o_t - o_d + log2(S_t / D),
// so r keeps its relative accuracy when p_t and q' nearly cancel (small
// residual mass), where p_t - q' taken in fp32 would carry an absolute error
// of ~1e-7 of p_t.  k2 is split into fp32 hi + lo parts: fma(delta, c, k_hi)
// rounds once, so d carries an error of a few ulp of d itself, not of its
// terms.

struct ResidualScale {
    float c;             // fp32(log2e / T)
    float k_hi, k_lo;    // k2
    float kt_hi, kt_lo;  // k2 + log2 beta (draft top-4 tokens)
    int tq[4];           // 16-byte vector of each draft top-4 token, -1 for none
};

template <int VEC>
__device__ __forceinline__ ResidualScale make_residual_scale(const SeqState &st, const ExpScale &e)
{
    ResidualScale r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r.tq[k] = st.top[k] >= 0 ? st.top[k] / VEC : -1;
    r.c = e.c;
    r.k_hi = (float)st.k2;
    r.k_lo = (float)(st.k2 - (double)r.k_hi);
    const double kt = st.k2 + (double)st.lbeta;  // -inf when beta == 0
    r.kt_hi = (float)kt;
    r.kt_lo = isfinite(kt) ? (float)(kt - (double)r.kt_hi) : 0.f;
    return r;
}

// 1 - 2^d for d < 0, to ~2e-7 relative, clamped to [0, 1]: -d * P(d) on
// [-1, 0), with P a degree-5 fit of (2^d - 1)/d on that interval (fit error
// 1e-8, fp32 Horner rounding ~1e-7), and 1 - exp2(d) below -1, where
// 2^d <= 1/2 keeps the subtraction well conditioned.  d >= 0, and the NaN of
// a token masked in both rows, give 0: the clamp is the output modifier of
// the two producing operations (NaN clamps to 0).
__device__ __forceinline__ float one_minus_exp2(float d)
{
    float p = __builtin_fmaf(d, 1.145800052e-04f, 1.290776301e-03f);
    p = __builtin_fmaf(d, p, 9.596269578e-03f);
    p = __builtin_fmaf(d, p, 5.549895018e-02f);
    p = __builtin_fmaf(d, p, 2.402260602e-01f);
    p = __builtin_fmaf(d, p, 6.931471825e-01f);
    const float poly = __builtin_amdgcn_fmed3f(-d * p, 0.f, 1.f);
    const float direct = __builtin_amdgcn_fmed3f(1.f - __builtin_amdgcn_exp2f(d), 0.f, 1.f);
    return d >= -1.f ? poly : direct;
}

// MODE 1: max(p_t - q', 0) * S_t with the offset (k_hi, k_lo) of the token's
// draft weight; MODE 2: p_t * S_t.
template <int MODE>
__device__ __forceinline__ float residual_at(float zt, float zd, const SeqState &st, const ExpScale &e,
                                             const ResidualScale &rs, float khi, float klo)
{
    const float pt = exp_scaled(zt, st.o_t, e);  // p_t(v) * S_t
    if (MODE == 2) return pt;
    const float delta = zd - zt;
    const float d = __builtin_fmaf(delta, rs.c, khi) + klo;
    return pt * one_minus_exp2(d);  // q' >= p_t: no mass
}

}  // namespace sv
