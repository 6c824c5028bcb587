// sv_verify.hip -- the kernels of the verify step and their launchers.
//
//   1. stats_kernel     streams every needed logit row once, one workgroup per
//                       (row, chunk), and reduces it to a partial: (max, sum
//                       of exp2((z - max) log2e / T)) for sampling rows, (max,
//                       lowest argmax) for greedy rows, and for beta-weighted
//                       draft rows the chunk top-4 with the mass outside it.
//   2. accept           per sequence: merge its rows' partials in fp64, form
//                       every accept ratio in the log domain, draw the Philox
//                       uniforms and find the first rejection n.
//   3. residual_kernel  re-reads target row n and draft row n (or target row K
//                       after K acceptances) in chunks and sums the residual.
//   4. bonus            per sequence: scan the chunk sums, then the selected
//                       chunk, for the bonus token.
//
// The four launches are stream-ordered; every kernel reads only what earlier
// launches wrote, so no workgroup ever waits for another.
#include <algorithm>

#include "sv_accept.h"
#include "sv_tile.h"

namespace sv {

// kLoads vectors q = qb + u*kBlock + tid of a row, all loads issued before use;
// vectors at or beyond q1 and elements at or beyond V read as -inf.
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
            if (qb + u * kBlock + tid >= q1) r[u] = neg_inf_raw<DT>();
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
                r[u] = neg_inf_raw<DT>();
            }
        }
    }
    if (V % VEC) {
        const int last = (V - 1) / VEC;
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            if (qb + u * kBlock + tid == last) mask_raw<DT>(r[u], V - last * VEC);
    }
}

__device__ __forceinline__ const char *target_row(const Args &a, int b, int i)
{
    return a.target + ((int64_t)b * (a.K + 1) + i) * a.row_bytes;
}

__device__ __forceinline__ const char *draft_row(const Args &a, int b, int i)
{
    return a.draft + ((int64_t)b * a.K + i) * a.row_bytes;
}

// ---------------------------------------------------------------------------
// 2. Accept scan of sequence b by one workgroup ("Kangaroo: Self-Speculative
// Decoding via Shallow Sub-Networks", "3. Lossless Speculative Verification";
// greedy: "LayerSkip Guide: Early Exit & Self-Speculative Decoding", "2. The
// Drafting and Single-Pass Verification Pipeline").  Every position's ratio is
// formed in parallel; n is the first rejection.  C: the partials were
// published in the same launch.

struct AcceptLds {
    float m[kMaxSlots];
    double S[kMaxSlots];  // S_t, or the draft normaliser D
    int idx[kMaxSlots];
    Top4 top[kMaxK];
    int acc[kMaxK];
    int err[kMaxK];
    float pt[kMaxK], pd[kMaxK];
    int x[kMaxK];                // drafted tokens
    float zt[kMaxK], zd[kMaxK];  // their logits
};

__global__ __launch_bounds__(kBlock) void accept_kernel(const Args a)
{
    __shared__ __align__(16) unsigned char stage[kStageBytes];
    __shared__ AcceptLds L;
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, nc = a.nc;
    const uint32_t gb = (uint32_t)(a.b0 + b);  // Philox keys on the sequence's index in the call
    int32_t *out = a.out_tokens + (int64_t)b * (K + 1);
    const float T = a.temperature[b];
    const bool greedy = T == 0.f;
    const bool weighted = a.weighted && !greedy;

    int fail = 0;
    if (!temperature_ok(T)) fail = SV_ERR_TEMPERATURE;
    else if (!greedy && K > 0 && a.draft == nullptr) fail = SV_ERR_NO_DRAFT;

    if (!fail) {
        // One round trip: the sequence's partials and top-4 lists into LDS
        // (16-byte granules, every load issued before any is stored) and the
        // two logits of each drafted token.
        const int nslots = greedy ? K + 1 : 2 * K + 1;
        const int P = nslots * nc;
        const int PT = weighted ? K * nc : 0;
        const uint4 *gp = reinterpret_cast<const uint4 *>(a.part + (int64_t)b * a.R * nc);
        const uint4 *gt = reinterpret_cast<const uint4 *>(a.top + (int64_t)b * K * nc);
        uint4 *s4 = reinterpret_cast<uint4 *>(stage);
        const int total4 = P + 2 * PT;  // a RowPart is one granule, a Top4 two
        if (tid < K) {
            const int x = a.tokens[(int64_t)b * K + tid];
            L.x[tid] = x;
            float zt = 0.f, zd = 0.f;
            if (!greedy && x >= 0 && x < a.V) {
                if (a.dtype == SV_F32) {
                    zt = Elt<0>::scalar(target_row(a, b, tid), x);
                    zd = Elt<0>::scalar(draft_row(a, b, tid), x);
                } else {
                    zt = Elt<1>::scalar(target_row(a, b, tid), x);
                    zd = Elt<1>::scalar(draft_row(a, b, tid), x);
                }
            }
            L.zt[tid] = zt;
            L.zd[tid] = zd;
        }
        for (int base = 0; base < total4; base += 4 * kBlock) {
            uint4 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int jj = base + k * kBlock + tid;
                if (jj < total4) v[k] = jj < P ? gp[jj] : gt[jj - P];
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int jj = base + k * kBlock + tid;
                if (jj < total4) s4[jj] = v[k];
            }
        }
        __syncthreads();

        const RowPart *sp = reinterpret_cast<const RowPart *>(stage);
        const Top4 *stp = reinterpret_cast<const Top4 *>(stage + sizeof(RowPart) * (size_t)P);
        const double c64 = greedy ? 0.0 : kLog2e / (double)T;
        for (int slot = wave; slot < nslots; slot += kWaves) {
            const RowPart *p = sp + slot * nc;
            if (greedy) {
                float M;
                int I;
                merge_argmax(p, nc, M, I);
                if (lane == 0) {
                    L.m[slot] = M;
                    L.idx[slot] = I;
                }
            } else if (weighted && slot > K) {
                const int i = slot - (K + 1);
                float M;
                Top4 rt4;
                double S_rest, S_top;
                merge_weighted(p, stp + i * nc, nc, c64, M, rt4, S_rest, S_top);
                if (lane == 0) {
                    L.m[slot] = M;
                    L.S[slot] = S_rest + (double)a.beta * S_top;
                    L.top[i] = rt4;
                }
            } else {
                float M;
                double S;
                merge_sum(p, nc, c64, M, S);
                if (lane == 0) {
                    L.m[slot] = M;
                    L.S[slot] = S;
                }
            }
        }
        __syncthreads();

        if (!greedy) {
            for (int i = tid; i < K; i += kBlock) {
                const float mt = L.m[i], md = L.m[K + 1 + i];
                int err = 0;
                if (!isfinite(mt)) err |= SV_ERR_ROW;
                if (!isfinite(md)) err |= SV_ERR_ROW;
                else if (!(L.S[K + 1 + i] > 0.0)) err |= SV_ERR_DRAFT_MASS;
                const int x = L.x[i];
                const bool x_ok = x >= 0 && x < a.V && err == 0;
                const bool in_top = weighted && top_has(L.top[i], x);
                const float u = philox_uniform(a.seed, gb, (uint32_t)i, kPurposeAccept);
                float pt, pd;
                L.acc[i] = decide(T, mt, L.S[i], md, L.S[K + 1 + i], in_top, a.beta, x_ok, L.zt[i],
                                  L.zd[i], u, pt, pd)
                               ? 1
                               : 0;
                L.err[i] = err;
                L.pt[i] = pt;
                L.pd[i] = pd;
            }
        }
        __syncthreads();
    }

    if (tid != 0) return;

    int n = K;
    int err_bits = 0;
    SeqState st = {};
    st.mode = 0;
    if (!fail && greedy) {
        for (int i = 0; i <= K; ++i) {
            if (!isfinite(L.m[i])) {
                fail = SV_ERR_ROW;
                break;
            }
            if (i < K && L.x[i] == L.idx[i]) continue;
            n = i;
            break;
        }
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = L.x[i];
            if (n < K) {
                const int x = L.x[n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            out[n] = L.idx[n];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = NAN;
            if (a.aux_z) a.aux_z[b] = NAN;
        }
    } else if (!fail) {
        for (int i = 0; i < K; ++i) {
            if (L.err[i]) {  // rows of this position are unusable and it is reached
                fail = L.err[i];
                break;
            }
            if (!L.acc[i]) {
                n = i;
                break;
            }
        }
        if (!fail && n == K && !isfinite(L.m[K])) fail = SV_ERR_ROW;
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = L.x[i];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            out[n] = -1;  // the bonus step writes the drawn token
            if (n < K) {
                const int x = L.x[n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = i <= n ? L.pt[i] : NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = i <= n ? L.pd[i] : NAN;
            st.n = n;
            st.mode = n < K ? 1 : 2;
            st.m_t = L.m[n];
            st.inv_st = (float)(1.0 / L.S[n]);
            st.T = T;
            st.beta = a.beta;
            st.u_bonus = philox_uniform(a.seed, gb, (uint32_t)n, kPurposeBonus);
#pragma unroll
            for (int k = 0; k < 4; ++k) st.top[k] = -1;
            st.lbeta = (float)log2((double)a.beta);
            if (n < K) {
                st.m_d = L.m[K + 1 + n];
                st.inv_sd = (float)(1.0 / L.S[K + 1 + n]);
                st.k2 = ((double)L.m[n] - (double)L.m[K + 1 + n]) * (kLog2e / (double)T) +
                        log2(L.S[n]) - log2(L.S[K + 1 + n]);
                if (weighted) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) st.top[k] = L.top[n].i[k] == INT_MAX ? -1 : L.top[n].i[k];
                }
            }
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
        st = SeqState{};
        st.mode = 0;
        err_bits |= fail;
    }
    a.seq[b] = st;
    if (err_bits && a.error_word) atomicOr(a.error_word, err_bits);
}

// ---------------------------------------------------------------------------
// 1. Streaming pass, one workgroup per (row, chunk), with the per-thread tile
// reductions of sv_tile.h: a wave-uniform running max with per-lane fp64
// sums, lanes visiting their elements in increasing index order (so argmax
// and top-4 ties resolve to the lowest token id), and for a weighted draft row
// the lane top-4 kept out of the sum.  Rows a sequence does not use (draft
// rows in greedy mode or without draft logits, rows of a sequence with an
// invalid temperature) publish nothing.

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void stats_kernel(const Args a)
{
    __shared__ float lds_f[4 + kWaves * 4];
    __shared__ int lds_i[4 + kWaves * 4];
    __shared__ double lds_d[kWaves];

    const int tid = threadIdx.x;
    const int chunk = blockIdx.x % a.nc;
    const int slot_row = blockIdx.x / a.nc;
    const int b = slot_row / a.R;
    const int j = slot_row - b * a.R;

    const float T = a.temperature[b];
    const bool greedy = T == 0.f;
    const bool is_draft = j > a.K;
    const bool used = temperature_ok(T) && !(is_draft && (greedy || a.draft == nullptr));
    RowPart part;
    Top4 ct;
    const bool track_top = TOP && is_draft;
    if (used) {
        const int i = is_draft ? j - (a.K + 1) : j;
        const char *row = is_draft ? draft_row(a, b, i) : target_row(a, b, i);
        const bool aligned = ((uintptr_t)row & 15) == 0;
        const int q0 = chunk * a.cvec;
        const int q1 = min(a.nvec, q0 + a.cvec);
        if (greedy) {
            float best = -INFINITY;
            int bi = INT_MAX;
            for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
                uint4 r[kLoads];
                load_step<DT>(row, aligned, true, qb, q1, a.V, r);
                run_argmax_tile<DT, kLoads>(r, qb, best, bi);
            }
            block_argmax(best, bi, lds_f, lds_i);
            part.m = best;
            part.idx = bi;
            part.s = 0.0;
        } else {
            const ExpScale e = make_scale(T);
            RowRun run;
            run_clear(run);
            Top4 t4;
            top_clear(t4);
            for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
                uint4 r[kLoads];
                load_step<DT>(row, aligned, true, qb, q1, a.V, r);
                if (track_top) run_sum_top_tile<DT, kLoads>(r, qb, a.V, e, run, t4);
                else run_sum_tile<DT, kLoads>(r, e, run);
            }
            if (track_top) run_finish_top(run, t4, e, lds_f, lds_i, lds_d, part.m, part.s, ct);
            else run_finish(run, e, lds_f, lds_d, part.m, part.s);
            part.idx = -1;
        }
    }
    if (used && tid == 0) {
        a.part[(int64_t)slot_row * a.nc + chunk] = part;
        if (track_top && !greedy) a.top[((int64_t)b * a.K + (j - (a.K + 1))) * a.nc + chunk] = ct;
    }
}

// ---------------------------------------------------------------------------
// 4. Bonus draw by inverse CDF in ascending token id: the smallest v with
// C(v) >= u * Z, Z the total residual mass; zero mass falls back to p_t.

// Scan the residual over vectors [q0, q1), at most kBlock * kLoads of them,
// in token order, starting from `base`, for the first element whose running
// sum reaches `thr`.  All loads are issued before the scan.  Returns that
// element (or INT_MAX), the range total, and the last element with mass.
template <int DT, bool TOP>
__device__ int scan_chunk(const Args &a, int b, const SeqState &st, int mode, const ExpScale &e,
                          int q0, int q1, double base, double thr, double &total, int &last_pos,
                          double *lds_d, int *lds_i)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const char *trow = target_row(a, b, st.n);
    const char *drow = mode == 1 ? draft_row(a, b, st.n) : trow;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    uint4 rt[kLoads], rd[kLoads];
    load_step<DT>(trow, ta, false, q0, q1, a.V, rt);
    if (mode == 1) load_step<DT>(drow, da, false, q0, q1, a.V, rd);
    double run = base;
    int last = -1;
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
        float xt[VEC], xd[VEC];
        Elt<DT>::unpack(rt[u], xt);
        if (mode == 1) Elt<DT>::unpack(rd[u], xd);
        double pre[VEC];
        double acc = 0.0;
        int mylast = -1;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int v = elem_index(q0, u, k, VEC);
            const float r = residual_at<TOP>(xt[k], mode == 1 ? xd[k] : 0.f, v, st, e, mode);
            acc += (double)r;
            pre[k] = acc;
            if (r > 0.f) mylast = v;
        }
        double tile_total;
        const double exc = block_exclusive_scan(acc, tile_total, lds_d);
        int cand = INT_MAX;
#pragma unroll
        for (int k = VEC - 1; k >= 0; --k)
            if (run + exc + pre[k] >= thr) cand = elem_index(q0, u, k, VEC);
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

// The whole row range [0, nvec) in chunks of kBlock * kLoads vectors.
template <int DT, bool TOP>
__device__ int scan_row(const Args &a, int b, const SeqState &st, int mode, const ExpScale &e,
                        double thr, double &total, int &last_pos, double *lds_d, int *lds_i)
{
    double run = 0.0;
    int last = -1;
    for (int q0 = 0; q0 < a.nvec; q0 += kBlock * kLoads) {
        double t;
        int l;
        const int v = scan_chunk<DT, TOP>(a, b, st, mode, e, q0, min(a.nvec, q0 + kBlock * kLoads),
                                          run, thr, t, l, lds_d, lds_i);
        run = t;
        last = max(last, l);
        if (v != INT_MAX) {
            total = run;
            last_pos = last;
            return v;
        }
    }
    total = run;
    last_pos = last;
    return INT_MAX;
}

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
            token = scan_chunk<DT, TOP>(a, b, st, st.mode, e, q0, q1, cbase, thr, total, last, lds_d,
                                        lds_i);
            if (token == INT_MAX) token = last;  // same rounding inside the chunk
        }
    }
    if (token < 0) {
        // zero residual mass (only through rounding): draw from p_t instead
        scan_row<DT, TOP>(a, b, st, 2, e, INFINITY, total, last, lds_d, lds_i);
        Z = total;
        token = scan_row<DT, TOP>(a, b, st, 2, e, (double)st.u_bonus * Z, total, last, lds_d, lds_i);
        if (token == INT_MAX) token = last;
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + st.n] = token;
        if (a.aux_z) a.aux_z[b] = (float)Z;
    }
}

// ---------------------------------------------------------------------------
// 3. Chunk sums of the residual: one workgroup per (sequence, chunk);
// sequences with nothing to draw (greedy, failed) skip it.

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
    const char *trow = target_row(a, b, st.n);
    const char *drow = st.mode == 1 ? draft_row(a, b, st.n) : trow;
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
            float xt[VEC], xd[VEC], rv[VEC];
            Elt<DT>::unpack(rt[u], xt);
            if (st.mode == 1) Elt<DT>::unpack(rd[u], xd);
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                rv[k] = residual_at<TOP>(xt[k], st.mode == 1 ? xd[k] : 0.f, elem_index(qb, u, k, VEC),
                                         st, e, st.mode);
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

// ---------------------------------------------------------------------------
// Host launchers (one sub-batch of at most kMaxSeqPerLaunch sequences).

template <int DT, bool TOP>
static void launch_all(const Args &a, hipStream_t s, bool draw)
{
    stats_kernel<DT, TOP><<<(unsigned)((int64_t)a.B * a.R * a.nc), kBlock, 0, s>>>(a);
    accept_kernel<<<(unsigned)a.B, kBlock, 0, s>>>(a);
    if (draw) {
        residual_kernel<DT, TOP><<<(unsigned)((int64_t)a.B * a.ncr), kBlock, 0, s>>>(a);
        bonus_kernel<DT, TOP><<<(unsigned)a.B, kBlock, 0, s>>>(a);
    }
}

void launch_verify(const Args &a, hipStream_t s, bool draw)
{
    if (a.dtype == SV_F32) {
        if (a.weighted) launch_all<0, true>(a, s, draw);
        else launch_all<0, false>(a, s, draw);
    } else {
        if (a.weighted) launch_all<1, true>(a, s, draw);
        else launch_all<1, false>(a, s, draw);
    }
}

void launch_rowstats(const Args &a, hipStream_t s)
{
    const unsigned grid = (unsigned)((int64_t)a.B * a.R * a.nc);
    if (a.dtype == SV_F32) stats_kernel<0, false><<<grid, kBlock, 0, s>>>(a);
    else stats_kernel<1, false><<<grid, kBlock, 0, s>>>(a);
    rowstats_finish_kernel<<<(unsigned)a.B, 64, 0, s>>>(a);
}

void launch_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, hipStream_t s)
{
    const int64_t total = (int64_t)B * P * 2;
    uniforms_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(seed, B, P, out);
}

}  // namespace sv
