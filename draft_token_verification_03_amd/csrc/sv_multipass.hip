// sv_multipass.hip -- the verify step as four launches, for any shape.
//
//   1. stats_kernel     streams every needed logit row once and reduces each
//                       (row, chunk) to a partial: (max, sum of
//                       exp2((z - max) log2e / T)) for sampling rows, (max,
//                       lowest argmax) for greedy rows, and for beta-weighted
//                       draft rows the chunk top-4 with the mass outside it.
//   2. accept_kernel    one workgroup per sequence merges its rows' partials in
//                       fp64, forms every accept ratio in the log domain, draws
//                       the Philox uniforms and finds the first rejection n.
//   3. residual_kernel  re-reads target row n and draft row n (or target row K
//                       after K acceptances) in chunks and sums the residual.
//   4. bonus_kernel     one workgroup per sequence scans the chunk sums, then
//                       the selected chunk, for the bonus token.
// The fused single-launch path is preferred; this one serves shapes it cannot
// hold (long drafts, very long rows) and the row-statistics entry point.
#include "sv_accept.h"

namespace sv {

template <int DT>
__device__ __forceinline__ uint4 neg_inf_raw_mp()
{
    return DT == 0 ? make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u)
                   : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
}

// kLoads vectors q = qb + u*kBlock + tid of a row, all loads issued before use;
// vectors at or beyond q1 read as -inf.
template <int DT>
__device__ __forceinline__ void load_step(const char *row, bool aligned, bool stream, int qb, int q1,
                                          int V, uint4 (&r)[kLoads])
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    if (aligned) {
        // every load is issued before any is used: vectors at or beyond q1
        // re-read vector q1 - 1 and are replaced by -inf afterwards
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = min(qb + u * kBlock + tid, q1 - 1);
            r[u] = stream ? load16_stream(row + (size_t)q * 16)
                          : *reinterpret_cast<const uint4 *>(row + (size_t)q * 16);
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            if (qb + u * kBlock + tid >= q1) r[u] = neg_inf_raw_mp<DT>();
    } else {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q < q1) {
                const char *p = row + (size_t)q * 16;
                const int valid = min(VEC, V - q * VEC);
                r[u] = load16_unaligned(p, ((uint32_t)((uintptr_t)p & 15)) +
                                               (uint32_t)valid * Elt<DT>::kBytes > 16u);
            } else {
                r[u] = neg_inf_raw_mp<DT>();
            }
        }
    }
}

// Unpack vector q; elements at or beyond V are -inf.
template <int DT>
__device__ __forceinline__ void unpack_masked(uint4 r, int q, int V, float (&x)[Elt<DT>::kVec])
{
    constexpr int VEC = Elt<DT>::kVec;
    Elt<DT>::unpack(r, x);
    if ((q + 1) * VEC > V) {
#pragma unroll
        for (int k = 0; k < VEC; ++k)
            if (q * VEC + k >= V) x[k] = -INFINITY;
    }
}

__device__ __forceinline__ const char *mp_target_row(const Args &a, int b, int i)
{
    return a.target + ((int64_t)b * (a.K + 1) + i) * a.row_bytes;
}

__device__ __forceinline__ const char *mp_draft_row(const Args &a, int b, int i)
{
    return a.draft + ((int64_t)b * a.K + i) * a.row_bytes;
}

// ---------------------------------------------------------------------------
// 1. Streaming pass.  Per lane the online (max, sum) is kept in (fp32, fp64):
// each vector's exponentials are summed in fp32 against the lane's running
// max and added to an fp64 sum that is rescaled in fp64 when the max grows.
// Lanes visit their elements in increasing index order, so argmax and top-4
// ties resolve to the lowest token id.  For a weighted draft row an element
// entering the lane's top-4 is left out of the sum and the element it evicts
// is added, so the sum is over elements outside the lane's top-4.

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void stats_kernel(const Args a)
{
    using E = Elt<DT>;
    constexpr int VEC = E::kVec;
    __shared__ float lds_f[4 + kWaves * 4];
    __shared__ int lds_i[4 + kWaves * 4];
    __shared__ double lds_d[kWaves];

    const int tid = threadIdx.x;
    const int chunk = blockIdx.x % a.nc;
    const int slot_row = blockIdx.x / a.nc;
    const int b = slot_row / a.R;
    const int j = slot_row - b * a.R;

    const float T = a.temperature[b];
    if (!temperature_ok(T)) return;
    const bool greedy = T == 0.f;
    const bool is_draft = j > a.K;
    if (is_draft && (greedy || a.draft == nullptr)) return;
    const int i = is_draft ? j - (a.K + 1) : j;
    const char *row = is_draft ? mp_draft_row(a, b, i) : mp_target_row(a, b, i);
    const bool aligned = ((uintptr_t)row & 15) == 0;
    const int q0 = chunk * a.cvec;
    const int q1 = min(a.nvec, q0 + a.cvec);
    RowPart *out = a.part + (int64_t)slot_row * a.nc + chunk;

    if (greedy) {
        float best = -INFINITY;
        int bi = INT_MAX;
        for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
            uint4 r[kLoads];
            load_step<DT>(row, aligned, true, qb, q1, a.V, r);
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int q = qb + u * kBlock + tid;
                float x[VEC];
                unpack_masked<DT>(r[u], q, a.V, x);
                float mx = x[0];
#pragma unroll
                for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[k]);
                if (mx > best) {
                    int kk = VEC - 1;
#pragma unroll
                    for (int k = VEC - 1; k >= 0; --k)
                        if (x[k] == mx) kk = k;
                    best = mx;
                    bi = q * VEC + kk;
                }
            }
        }
        block_argmax(best, bi, lds_f, lds_i);
        if (tid == 0) {
            RowPart r;
            r.m = best;
            r.idx = bi;
            r.s = 0.0;
            *out = r;
        }
        return;
    }

    const ExpScale e = make_scale(T);
    const bool track_top = TOP && is_draft;
    float m = -INFINITY;
    double s = 0.0;
    Top4 t4;
    top_clear(t4);
    for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
        uint4 r[kLoads];
        load_step<DT>(row, aligned, true, qb, q1, a.V, r);
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            float x[VEC];
            unpack_masked<DT>(r[u], q, a.V, x);
            float mx = x[0];
#pragma unroll
            for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[k]);
            if (mx > m) {
                if (s != 0.0) s *= exp2(((double)m - (double)mx) * e.c64);
                m = mx;
            }
            float acc[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k) acc[k] = 0.f;
            if (m != -INFINITY) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = exp_scaled(x[k], m, e);
            }
            if (track_top && (mx > t4.v[3] || (mx == t4.v[3] && t4.i[3] == INT_MAX))) {
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    const int idx = q * VEC + k;
                    if (idx < a.V && better(x[k], idx, t4.v[3], t4.i[3])) {
                        const float ev = t4.v[3];
                        const int ei = t4.i[3];
                        top_insert(t4, x[k], idx);
                        acc[k] = (m != -INFINITY && ei != INT_MAX) ? exp_scaled(ev, m, e) : 0.f;
                    }
                }
            }
#pragma unroll
            for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                for (int k = 0; k < w; ++k) acc[k] += acc[k + w];
            s += (double)acc[0];
        }
    }
    const float M = block_max(m, lds_f);
    double scaled = (m == -INFINITY) ? 0.0 : s * exp2(((double)m - (double)M) * e.c64);
    if (track_top) {
        const int lane = tid & 63, wave = tid >> 6;
        const Top4 w = wave_top4(t4);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lds_f[4 + wave * 4 + k] = w.v[k];
                lds_i[4 + wave * 4 + k] = w.i[k];
            }
        }
        __syncthreads();
        if (wave == 0) {
            Top4 c;
            top_clear(c);
            if (lane < kWaves * 4) {
                c.v[0] = lds_f[4 + lane];
                c.i[0] = lds_i[4 + lane];
            }
            const Top4 r = wave_top4(c);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lds_f[k] = r.v[k];
                    lds_i[k] = r.i[k];
                }
                a.top[((int64_t)b * a.K + i) * a.nc + chunk] = r;
            }
        }
        __syncthreads();
        Top4 ct;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            ct.v[k] = lds_f[k];
            ct.i[k] = lds_i[k];
        }
        // lane-top entries that did not make the chunk top-4 join the sum
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (t4.i[k] != INT_MAX && t4.v[k] != -INFINITY && !top_has(ct, t4.i[k]))
                scaled += exp2(((double)t4.v[k] - (double)M) * e.c64);
        __syncthreads();
    }
    const double S = block_sum(scaled, lds_d);
    if (tid == 0) {
        RowPart r;
        r.m = M;
        r.idx = -1;
        r.s = S;
        *out = r;
    }
}

// ---------------------------------------------------------------------------
// 2. Accept scan, one workgroup per sequence ("Kangaroo: Self-Speculative
// Decoding via Shallow Sub-Networks", "3. Lossless Speculative Verification";
// greedy: "LayerSkip Guide: Early Exit & Self-Speculative Decoding", "2. The
// Drafting and Single-Pass Verification Pipeline").  Every position's ratio
// is formed in parallel; n is the first rejection.

__global__ __launch_bounds__(kBlock) void accept_kernel(const Args a)
{
    __shared__ float s_m[kMaxSlots];
    __shared__ double s_S[kMaxSlots];
    __shared__ int s_idx[kMaxSlots];
    __shared__ Top4 s_top[kMaxK];
    __shared__ int s_acc[kMaxK];
    __shared__ int s_err[kMaxK];
    __shared__ float s_pt[kMaxK], s_pd[kMaxK];

    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    int32_t *out = a.out_tokens + (int64_t)b * (K + 1);
    const float T = a.temperature[b];
    const bool greedy = T == 0.f;
    const bool weighted = a.weighted && !greedy;

    int fail = 0;
    if (!temperature_ok(T)) fail = SV_ERR_TEMPERATURE;
    else if (!greedy && K > 0 && a.draft == nullptr) fail = SV_ERR_NO_DRAFT;

    if (!fail) {
        const int nslots = greedy ? K + 1 : 2 * K + 1;
        const double c64 = greedy ? 0.0 : kLog2e / (double)T;
        for (int slot = wave; slot < nslots; slot += kWaves) {
            const RowPart *p = a.part + ((int64_t)b * a.R + slot) * a.nc;
            if (greedy) {
                float M;
                int I;
                merge_argmax(p, a.nc, M, I);
                if (lane == 0) {
                    s_m[slot] = M;
                    s_idx[slot] = I;
                }
            } else if (weighted && slot > K) {
                const int i = slot - (K + 1);
                float M;
                Top4 rt4;
                double S_rest, S_top;
                merge_weighted(p, a.top + ((int64_t)b * K + i) * a.nc, a.nc, c64, M, rt4, S_rest,
                               S_top);
                if (lane == 0) {
                    s_m[slot] = M;
                    s_S[slot] = S_rest + (double)a.beta * S_top;
                    s_top[i] = rt4;
                }
            } else {
                float M;
                double S;
                merge_sum(p, a.nc, c64, M, S);
                if (lane == 0) {
                    s_m[slot] = M;
                    s_S[slot] = S;
                }
            }
        }
        __syncthreads();

        if (!greedy && tid < K) {
            const int i = tid;
            const float mt = s_m[i], md = s_m[K + 1 + i];
            int err = 0;
            if (!isfinite(mt)) err |= SV_ERR_ROW;
            if (!isfinite(md)) err |= SV_ERR_ROW;
            else if (!(s_S[K + 1 + i] > 0.0)) err |= SV_ERR_DRAFT_MASS;
            const int x = a.tokens[(int64_t)b * K + i];
            const bool x_ok = x >= 0 && x < a.V && err == 0;
            float zt = 0.f, zd = 0.f;
            if (x_ok) {
                if (a.dtype == SV_F32) {
                    zt = Elt<0>::scalar(mp_target_row(a, b, i), x);
                    zd = Elt<0>::scalar(mp_draft_row(a, b, i), x);
                } else {
                    zt = Elt<1>::scalar(mp_target_row(a, b, i), x);
                    zd = Elt<1>::scalar(mp_draft_row(a, b, i), x);
                }
            }
            const bool in_top = weighted && top_has(s_top[i], x);
            const float u = philox_uniform(a.seed, (uint32_t)b, (uint32_t)i, kPurposeAccept);
            float pt, pd;
            s_acc[i] = decide(T, mt, s_S[i], md, s_S[K + 1 + i], in_top, a.beta, x_ok, zt, zd, u,
                              pt, pd)
                           ? 1
                           : 0;
            s_err[i] = err;
            s_pt[i] = pt;
            s_pd[i] = pd;
        }
        __syncthreads();
    }

    if (tid != 0) return;

    int n = K;
    int err_bits = 0;
    if (!fail && greedy) {
        for (int i = 0; i <= K; ++i) {
            if (!isfinite(s_m[i])) {
                fail = SV_ERR_ROW;
                break;
            }
            if (i < K && a.tokens[(int64_t)b * K + i] == s_idx[i]) continue;
            n = i;
            break;
        }
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = a.tokens[(int64_t)b * K + i];
            if (n < K) {
                const int x = a.tokens[(int64_t)b * K + n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            out[n] = s_idx[n];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = NAN;
            if (a.aux_z) a.aux_z[b] = NAN;
            SeqState st = {};
            st.mode = 0;
            a.seq[b] = st;
        }
    } else if (!fail) {
        for (int i = 0; i < K; ++i) {
            if (s_err[i]) {  // rows of this position are unusable and it is reached
                fail = s_err[i];
                break;
            }
            if (!s_acc[i]) {
                n = i;
                break;
            }
        }
        if (!fail && n == K && !isfinite(s_m[K])) fail = SV_ERR_ROW;
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = a.tokens[(int64_t)b * K + i];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            out[n] = -1;  // the bonus kernel writes the drawn token
            if (n < K) {
                const int x = a.tokens[(int64_t)b * K + n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = i <= n ? s_pt[i] : NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = i <= n ? s_pd[i] : NAN;
            SeqState st = {};
            st.n = n;
            st.mode = n < K ? 1 : 2;
            st.m_t = s_m[n];
            st.inv_st = (float)(1.0 / s_S[n]);
            st.T = T;
            st.beta = a.beta;
            st.u_bonus = philox_uniform(a.seed, (uint32_t)b, (uint32_t)n, kPurposeBonus);
#pragma unroll
            for (int k = 0; k < 4; ++k) st.top[k] = -1;
            st.lbeta = (float)log2((double)a.beta);
            if (n < K) {
                st.m_d = s_m[K + 1 + n];
                st.inv_sd = (float)(1.0 / s_S[K + 1 + n]);
                st.k2 = ((double)s_m[n] - (double)s_m[K + 1 + n]) * (kLog2e / (double)T) +
                        log2(s_S[n]) - log2(s_S[K + 1 + n]);
                if (weighted) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        st.top[k] = s_top[n].i[k] == INT_MAX ? -1 : s_top[n].i[k];
                }
            }
            a.seq[b] = st;
        }
    }
    if (fail) {
        a.accepted_len[b] = 0;
        for (int i = 0; i <= K; ++i) out[i] = -1;
        if (a.aux_pt)
            for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = NAN;
        if (a.aux_pd)
            for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = NAN;
        if (a.aux_z) a.aux_z[b] = NAN;
        SeqState st = {};
        st.mode = 0;
        a.seq[b] = st;
        err_bits |= fail;
    }
    if (err_bits && a.error_word) atomicOr(a.error_word, err_bits);
}

// 3. Chunk sums of the residual: one workgroup per (sequence, chunk).
template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void residual_kernel(const Args a)
{
    constexpr int VEC = Elt<DT>::kVec;
    __shared__ double lds_d[kWaves];
    const int b = blockIdx.x / a.ncr;
    const int chunk = blockIdx.x - b * a.ncr;
    const SeqState st = a.seq[b];
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const char *trow = mp_target_row(a, b, st.n);
    const char *drow = st.mode == 1 ? mp_draft_row(a, b, st.n) : trow;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    const int q0 = chunk * a.rvec, q1 = min(a.nvec, q0 + a.rvec);
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
        uint4 rt[kLoads], rd[kLoads];
        load_step<DT>(trow, ta, false, qb, q1, a.V, rt);
        if (st.mode == 1) load_step<DT>(drow, da, false, qb, q1, a.V, rd);
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            float xt[VEC], xd[VEC], rv[VEC];
            unpack_masked<DT>(rt[u], q, a.V, xt);
            if (st.mode == 1) unpack_masked<DT>(rd[u], q, a.V, xd);
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                rv[k] = residual_at<TOP>(xt[k], st.mode == 1 ? xd[k] : 0.f, q * VEC + k, st, e,
                                         st.mode);
#pragma unroll
            for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                for (int k = 0; k < w; ++k) rv[k] += rv[k + w];
            s += (double)rv[0];
        }
    }
    const double S = block_sum(s, lds_d);
    if (tid == 0) a.res[(int64_t)b * a.ncr + chunk] = S;
}

// Scan the residual over vectors [q0, q1) in token order, starting from
// `base`, for the first element whose running sum reaches `thr`.  Returns that
// element (or INT_MAX), the range total, and the last element with mass.
template <int DT, bool TOP>
__device__ int scan_range(const Args &a, int b, const SeqState &st, int mode, const ExpScale &e,
                          int q0, int q1, double base, double thr, double &total, int &last_pos,
                          double *lds_d, int *lds_i)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const char *trow = mp_target_row(a, b, st.n);
    const char *drow = mode == 1 ? mp_draft_row(a, b, st.n) : trow;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    double run = base;
    int last = -1;
    for (int qb = q0; qb < q1; qb += kBlock) {
        const int q = qb + tid;
        double pre[VEC];
        double acc = 0.0;
        int mylast = -1;
        if (q < q1) {
            float xt[VEC], xd[VEC];
            load_vec<DT>(trow, ta, q, a.V, xt);
            if (mode == 1) load_vec<DT>(drow, da, q, a.V, xd);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float r = residual_at<TOP>(xt[k], mode == 1 ? xd[k] : 0.f, q * VEC + k, st, e,
                                                 mode);
                acc += (double)r;
                pre[k] = acc;
                if (r > 0.f) mylast = q * VEC + k;
            }
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) pre[k] = 0.0;
        }
        double tile_total;
        const double exc = block_exclusive_scan(acc, tile_total, lds_d);
        int cand = INT_MAX;
        if (q < q1) {
#pragma unroll
            for (int k = VEC - 1; k >= 0; --k)
                if (run + exc + pre[k] >= thr) cand = q * VEC + k;
        }
        cand = block_min_int(cand, lds_i);
        last = max(last, block_max_int(mylast, lds_i));
        if (cand != INT_MAX) {
            total = run + tile_total;
            last_pos = last;
            return cand;
        }
        run += tile_total;
    }
    total = run;
    last_pos = last;
    return INT_MAX;
}

// 4. Bonus draw by inverse CDF in ascending token id: the smallest v with
// C(v) >= u * Z, Z the total residual mass; zero mass falls back to p_t.
template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void bonus_kernel(const Args a)
{
    __shared__ double lds_d[kWaves];
    __shared__ int lds_i[kWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const SeqState st = a.seq[b];
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const double *rs = a.res + (int64_t)b * a.ncr;

    double Z = 0.0;
    for (int c0 = 0; c0 < a.ncr; c0 += kBlock) {
        const int c = c0 + tid;
        double tot;
        block_exclusive_scan(c < a.ncr ? rs[c] : 0.0, tot, lds_d);
        Z += tot;
    }
    int mode = st.mode;
    int token = -1;
    double total;
    int last;
    if (Z > 0.0) {
        const double thr = (double)st.u_bonus * Z;
        double run = 0.0;
        int cstar = INT_MAX, last_chunk = -1;
        double cbase = 0.0, last_base = 0.0;
        for (int c0 = 0; c0 < a.ncr && cstar == INT_MAX; c0 += kBlock) {
            const int c = c0 + tid;
            const double v = c < a.ncr ? rs[c] : 0.0;
            double tot;
            const double exc = block_exclusive_scan(v, tot, lds_d);
            int cand = (c < a.ncr && run + exc + v >= thr) ? c : INT_MAX;
            cand = block_min_int(cand, lds_i);
            const int lastc = block_max_int(v > 0.0 ? c : -1, lds_i);
            if (cand != INT_MAX || lastc > last_chunk) {
                if (c == cand) lds_d[0] = run + exc;
                if (c == lastc) lds_d[1] = run + exc;
                __syncthreads();
                if (cand != INT_MAX) cbase = lds_d[0];
                if (lastc > last_chunk) last_base = lds_d[1];
                __syncthreads();
            }
            if (cand != INT_MAX) cstar = cand;
            if (lastc > last_chunk) last_chunk = lastc;
            run += tot;
        }
        if (cstar == INT_MAX) {
            // rounding between the two summation orders left u * Z above the last
            // prefix: the draw falls in the last chunk that has mass
            cstar = last_chunk;
            cbase = last_base;
        }
        if (cstar >= 0) {
            const int q0 = cstar * a.rvec, q1 = min(a.nvec, q0 + a.rvec);
            token = scan_range<DT, TOP>(a, b, st, mode, e, q0, q1, cbase, thr, total, last, lds_d,
                                        lds_i);
            if (token == INT_MAX) token = last;  // same rounding inside the chunk
        }
    }
    if (token < 0) {
        // zero residual mass (only through rounding): draw from p_t instead
        mode = 2;
        scan_range<DT, TOP>(a, b, st, mode, e, 0, a.nvec, 0.0, INFINITY, total, last, lds_d, lds_i);
        Z = total;
        const double thr = (double)st.u_bonus * Z;
        token = scan_range<DT, TOP>(a, b, st, mode, e, 0, a.nvec, 0.0, thr, total, last, lds_d,
                                    lds_i);
        if (token == INT_MAX) token = last;
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + st.n] = token;
        if (a.aux_z) a.aux_z[b] = (float)Z;
    }
}

// Row-statistics entry point: finish the merge of each row's partials.
__global__ __launch_bounds__(64) void rowstats_finish_kernel(const Args a)
{
    const int r = blockIdx.x;
    const float T = a.temperature[r];
    const RowPart *p = a.part + (int64_t)r * a.nc;
    const int lane = threadIdx.x;
    if (!temperature_ok(T)) {
        if (lane == 0) {
            a.rs_max[r] = NAN;
            a.rs_logsum[r] = NAN;
            a.rs_argmax[r] = -1;
        }
        return;
    }
    if (T == 0.f) {
        float M;
        int I;
        merge_argmax(p, a.nc, M, I);
        if (lane == 0) {
            a.rs_max[r] = M;
            a.rs_logsum[r] = NAN;
            a.rs_argmax[r] = I;
        }
    } else {
        float M;
        double S;
        merge_sum(p, a.nc, kLog2e / (double)T, M, S);
        if (lane == 0) {
            a.rs_max[r] = M;
            a.rs_logsum[r] = log(S);
            a.rs_argmax[r] = -1;
        }
    }
}

__global__ void uniforms_kernel(uint64_t seed, int32_t B, int32_t P, float *out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)B * P * 2;
    if (t >= total) return;
    const uint32_t purpose = (uint32_t)(t & 1);
    const int64_t bp = t >> 1;
    const uint32_t pos = (uint32_t)(bp % P);
    const uint32_t b = (uint32_t)(bp / P);
    out[t] = philox_uniform(seed, b, pos, purpose);
}

__global__ void zero_kernel(uint32_t *p, size_t words)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// ---------------------------------------------------------------------------
// Host launchers.

template <int DT, bool TOP>
static void launch_all(const Args &a, const Plan &p, hipStream_t s, bool draw)
{
    stats_kernel<DT, TOP><<<(unsigned)((int64_t)p.B * p.R * p.nc), kBlock, 0, s>>>(a);
    accept_kernel<<<(unsigned)p.B, kBlock, 0, s>>>(a);
    if (draw) {
        residual_kernel<DT, TOP><<<(unsigned)((int64_t)p.B * p.ncr), kBlock, 0, s>>>(a);
        bonus_kernel<DT, TOP><<<(unsigned)p.B, kBlock, 0, s>>>(a);
    }
}

void launch_multipass(const Args &a, const Plan &p, hipStream_t s, bool draw)
{
    if (p.dtype == SV_F32) {
        if (a.weighted) launch_all<0, true>(a, p, s, draw);
        else launch_all<0, false>(a, p, s, draw);
    } else {
        if (a.weighted) launch_all<1, true>(a, p, s, draw);
        else launch_all<1, false>(a, p, s, draw);
    }
}

void launch_rowstats(const Args &a, const Plan &p, hipStream_t s)
{
    const unsigned grid = (unsigned)((int64_t)p.B * p.R * p.nc);
    if (p.dtype == SV_F32) stats_kernel<0, false><<<grid, kBlock, 0, s>>>(a);
    else stats_kernel<1, false><<<grid, kBlock, 0, s>>>(a);
    rowstats_finish_kernel<<<(unsigned)p.B, 64, 0, s>>>(a);
}

void launch_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, hipStream_t s)
{
    const int64_t total = (int64_t)B * P * 2;
    uniforms_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(seed, B, P, out);
}

void launch_zero(void *ptr, size_t bytes, hipStream_t s)
{
    const size_t words = bytes / 4;
    const unsigned blocks = (unsigned)std::min<size_t>(1024, (words + 255) / 256);
    if (words) zero_kernel<<<blocks > 0 ? blocks : 1, 256, 0, s>>>(static_cast<uint32_t *>(ptr), words);
}

}  // namespace sv
