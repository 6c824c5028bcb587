// sv_fused.hip -- the verify step as one launch.
//
// The grid holds two kinds of workgroups, in this order:
//   streaming items (sequence b, slot p, chunk c): slots p < K are the row
//     pair (target p, draft p), slot K is target row K (the bonus position);
//     a chunk is kBlock * U consecutive 16-byte vectors of a row, which every
//     thread loads (nontemporal, all loads in flight at once) into registers
//     and reduces to partials: (max, sum of exp2((z - max) log2e / T)) for
//     sampling rows, (max, lowest argmax) for greedy rows and the chunk top-4
//     for beta-weighted draft rows.  It publishes them and arrives on the
//     sequence's counter; the last to arrive runs the accept scan of the
//     sequence, writes its accepted prefix and raises the sequence's flag.
//     Streaming items never wait for anything.
//   draw items (sequence b, chunk c), after all streaming items: each waits
//     for its sequence's flag, reads chunk c of the drawn rows (target and
//     draft row n, or target row K after K acceptances), sums the residual
//     over it and arrives on a second counter; the last to arrive draws the
//     bonus token by inverse CDF.
// A draw item only waits on streaming items, which always finish, and
// workgroups are dispatched in index order, so draw items cannot starve the
// work they wait for; each wait still has a spin budget and gives up with an
// error bit rather than hang.  Only per-sequence counters are touched
// atomically (no grid-wide counter), and each is returned to zero by its last
// user, so the control words are zero again when the launch ends.
#include "sv_accept.h"

namespace sv {


template <int DT>
__device__ __forceinline__ uint4 neg_inf_raw()
{
    return DT == 0 ? make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u)
                   : make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u);
}

__device__ __forceinline__ uint32_t &word_of(uint4 &r, int w)
{
    return w == 0 ? r.x : w == 1 ? r.y : w == 2 ? r.z : r.w;
}

// Set elements k >= keep of a raw vector to -inf.
template <int DT>
__device__ __forceinline__ void mask_raw(uint4 &r, int keep)
{
    constexpr int VEC = Elt<DT>::kVec;
#pragma unroll
    for (int k = 0; k < VEC; ++k) {
        if (k < keep) continue;
        if (DT == 0) {
            word_of(r, k) = 0xff800000u;
        } else {
            uint32_t &w = word_of(r, k >> 1);
            w = (k & 1) ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u);
        }
    }
}

// Load this thread's U vectors of a row chunk (vectors q0 + u*kBlock + tid).
template <int DT, int U>
__device__ __forceinline__ void load_chunk(const char *row, bool aligned, bool stream, int q0,
                                           int nvec, int V, uint4 (&r)[U])
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    if (aligned) {
        // every load is issued before any is used: vectors past the row end
        // re-read the row's last vector and are replaced by -inf afterwards
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = min(q0 + u * kBlock + tid, nvec - 1);
            r[u] = stream ? load16_stream(row + (size_t)q * 16)
                          : *reinterpret_cast<const uint4 *>(row + (size_t)q * 16);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (q0 + u * kBlock + tid >= nvec) r[u] = neg_inf_raw<DT>();
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int q = q0 + u * kBlock + tid;
            if (q < nvec) {
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
        const int last = nvec - 1;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (q0 + u * kBlock + tid == last) mask_raw<DT>(r[u], V - last * VEC);
    }
}

// Both rows of a slot: every load of both rows is issued before any value is
// examined, so a thread keeps 2U loads in flight.
template <int DT, int U>
__device__ __forceinline__ void load_pair(const char *trow, const char *drow, bool need_t,
                                          bool need_d, bool aligned, int q0, int nvec, int V,
                                          uint4 (&rt)[U], uint4 (&rd)[U])
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    if (!aligned) {
        if (need_t) load_chunk<DT, U>(trow, false, true, q0, nvec, V, rt);
        if (need_d) load_chunk<DT, U>(drow, false, true, q0, nvec, V, rd);
        return;
    }
    if (need_t) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            rt[u] = load16_stream(trow + (size_t)min(q0 + u * kBlock + tid, nvec - 1) * 16);
    }
    if (need_d) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            rd[u] = load16_stream(drow + (size_t)min(q0 + u * kBlock + tid, nvec - 1) * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kBlock + tid;
        if (q >= nvec) {
            rt[u] = neg_inf_raw<DT>();
            rd[u] = neg_inf_raw<DT>();
        } else if (V % VEC && q == nvec - 1) {
            mask_raw<DT>(rt[u], V - q * VEC);
            mask_raw<DT>(rd[u], V - q * VEC);
        }
    }
}

// Element index of value k of this thread's vector u.
__device__ __forceinline__ int elem_index(int q0, int u, int k, int vec)
{
    return (q0 + u * kBlock + (int)threadIdx.x) * vec + k;
}

// Partials of a sampling row chunk held in registers: block max M and the
// fp64 sum of exp2((z - M) c) over the chunk.
template <int DT, int U>
__device__ __forceinline__ void chunk_sum(const uint4 (&r)[U], const ExpScale &e, float *ldsf,
                                          double *ldsd, float &M, double &S)
{
    constexpr int VEC = Elt<DT>::kVec;
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) m = fmaxf(m, x[k]);
    }
    M = block_max(m, ldsf);
    double s = 0.0;
    if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC], ev[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], M, e);
#pragma unroll
            for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
            s += (double)ev[0];
        }
    }
    S = block_sum(s, ldsd);
}

// Weighted draft row chunk: max M, chunk top-4 and the mass outside the top-4.
// The smallest of the four wave maxima is a lower bound L4 on the chunk's 4th
// largest value (the wave maxima are four distinct elements), so only elements
// >= L4 can be in the chunk top-4.  They are compacted into LDS and one wave
// selects the top-4 from them; chunks with more than 64 such elements (ties,
// masked or tiny chunks) take a per-thread insertion path instead.
struct TopLds {
    float v[64];
    int i[64];
    int n;
};

template <int DT, int U>
__device__ __forceinline__ void chunk_sum_top(const uint4 (&r)[U], const ExpScale &e, int q0, int V,
                                              float *ldsf, int *ldsi, double *ldsd, TopLds &cand,
                                              float &M, double &S_excl, Top4 &ct)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) m = fmaxf(m, x[k]);
    }
    m = wave_max(m);
    if (tid == 0) cand.n = 0;
    if (lane == 0) ldsf[wave] = m;
    __syncthreads();
    M = ldsf[0];
    float L4 = ldsf[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
        M = fmaxf(M, ldsf[w]);
        L4 = fminf(L4, ldsf[w]);
    }
    __syncthreads();
    const bool fast = L4 != -INFINITY;
    if (fast) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (x[k] >= L4) {
                    const int idx = elem_index(q0, u, k, VEC);
                    if (idx < V) {
                        const int slot = atomicAdd(&cand.n, 1);
                        if (slot < 64) {
                            cand.v[slot] = x[k];
                            cand.i[slot] = idx;
                        }
                    }
                }
            }
        }
    }
    __syncthreads();
    const int ncand = cand.n;
    if (fast && ncand <= 64) {
        if (wave == 0) {
            Top4 c;
            top_clear(c);
            if (lane < ncand) {
                c.v[0] = cand.v[lane];
                c.i[0] = cand.i[lane];
            }
            const Top4 w = wave_top4(c);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ldsf[k] = w.v[k];
                    ldsi[k] = w.i[k];
                }
            }
        }
    } else {
        // per-thread lists in index order, then merged
        Top4 t;
        top_clear(t);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int idx = elem_index(q0, u, k, VEC);
                if (idx < V) top_insert(t, x[k], idx);
            }
        }
        const Top4 w = wave_top4(t);
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                ldsf[4 + wave * 4 + k] = w.v[k];
                ldsi[4 + wave * 4 + k] = w.i[k];
            }
        }
        __syncthreads();
        if (wave == 0) {
            Top4 c;
            top_clear(c);
            if (lane < kWaves * 4) {
                c.v[0] = ldsf[4 + lane];
                c.i[0] = ldsi[4 + lane];
            }
            const Top4 w2 = wave_top4(c);
            if (lane == 0) {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    ldsf[k] = w2.v[k];
                    ldsi[k] = w2.i[k];
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ct.v[k] = ldsf[k];
        ct.i[k] = ldsi[k];
    }
    __syncthreads();
    // mass outside the chunk top-4; its members are among the elements >= L4
    const float floor_v = fast ? L4 : -INFINITY;
    double s = 0.0;
    if (M != -INFINITY) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC], ev[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                ev[k] = exp_scaled(x[k], M, e);
                if (x[k] >= floor_v && top_has(ct, elem_index(q0, u, k, VEC))) ev[k] = 0.f;
            }
#pragma unroll
            for (int w2 = VEC / 2; w2 > 0; w2 >>= 1)
#pragma unroll
                for (int k = 0; k < w2; ++k) ev[k] += ev[k + w2];
            s += (double)ev[0];
        }
    }
    S_excl = block_sum(s, ldsd);
}

// Greedy row chunk: lowest index of the maximum.
template <int DT, int U>
__device__ __forceinline__ void chunk_argmax(const uint4 (&r)[U], int q0, float *ldsf, int *ldsi,
                                             float &M, int &I)
{
    constexpr int VEC = Elt<DT>::kVec;
    float best = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
        float mx = x[0];
#pragma unroll
        for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[k]);
        if (mx > best) {
            int kk = VEC - 1;
#pragma unroll
            for (int k = VEC - 1; k >= 0; --k)
                if (x[k] == mx) kk = k;
            best = mx;
            bi = elem_index(q0, u, kk, VEC);
        }
    }
    block_argmax(best, bi, ldsf, ldsi);
    M = best;
    I = bi;
}

// ---------------------------------------------------------------------------
// Accept scan of sequence b, run by the last workgroup to publish its partials.

struct AcceptLds {
    float m[2 * kFusedMaxK + 1];
    double S[2 * kFusedMaxK + 1];  // S_t, or the draft normaliser D
    int idx[2 * kFusedMaxK + 1];
    Top4 top[kFusedMaxK];
    int acc[kFusedMaxK];
    int err[kFusedMaxK];
    float pt[kFusedMaxK], pd[kFusedMaxK];
    int n, fail, err_bits;
};

template <bool TOP>
__device__ __forceinline__ void accept_sequence(const FusedArgs &a, int b, float T, unsigned char *stage,
                                AcceptLds &L, SeqState *st_lds)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, nc = a.schunks;
    const bool greedy = T == 0.f;
    const int gb = a.b0 + b;
    int32_t *out = a.out_tokens + (int64_t)b * (K + 1);

    int fail = 0;
    if (!temperature_ok(T)) fail = SV_ERR_TEMPERATURE;
    else if (!greedy && K > 0 && a.draft == nullptr) fail = SV_ERR_NO_DRAFT;

    const int R = greedy ? K + 1 : 2 * K + 1;
    const bool weighted = TOP && !greedy;
    RowPart *sp = reinterpret_cast<RowPart *>(stage);
    int x = -1;
    float2 zx = make_float2(0.f, 0.f);
    if (!fail) {
        // one round trip: partials, top-4 lists, drafted tokens and their logits
        const RowPart *gp = a.part + (int64_t)b * (2 * K + 1) * nc;
        const Top4 *gt = a.top + (int64_t)b * K * nc;
        const int P = R * nc, PT = weighted ? K * nc : 0;
        Top4 *stp = reinterpret_cast<Top4 *>(stage + sizeof(RowPart) * (size_t)P);
        // RowPart is one uint4 and Top4 two: both arrays are staged into LDS as
        // one index space of uint4, four loads in flight per thread per round
        const uint4 *gp4 = reinterpret_cast<const uint4 *>(gp);
        const uint4 *gt4 = reinterpret_cast<const uint4 *>(gt);
        uint4 *s4 = reinterpret_cast<uint4 *>(stage);  // partials, then top lists
        const int total4 = P + 2 * PT;
        if (tid < K) {
            x = a.tokens[(int64_t)b * K + tid];
            if (!greedy) {
                const uint32_t *zw = reinterpret_cast<const uint32_t *>(a.zx + (int64_t)b * K + tid);
                zx = make_float2(__uint_as_float(ld_agent(zw)), __uint_as_float(ld_agent(zw + 1)));
            }
        }
        for (int base = 0; base < total4; base += 4 * kBlock) {
            uint4 v0, v1, v2, v3;
            const int j0 = base + tid, j1 = j0 + kBlock, j2 = j0 + 2 * kBlock, j3 = j0 + 3 * kBlock;
            if (j0 < total4) v0 = ld_agent16(j0 < P ? gp4 + j0 : gt4 + (j0 - P));
            if (j1 < total4) v1 = ld_agent16(j1 < P ? gp4 + j1 : gt4 + (j1 - P));
            if (j2 < total4) v2 = ld_agent16(j2 < P ? gp4 + j2 : gt4 + (j2 - P));
            if (j3 < total4) v3 = ld_agent16(j3 < P ? gp4 + j3 : gt4 + (j3 - P));
            if (j0 < total4) s4[j0] = v0;
            if (j1 < total4) s4[j1] = v1;
            if (j2 < total4) s4[j2] = v2;
            if (j3 < total4) s4[j3] = v3;
        }
        __syncthreads();

        const double c64 = greedy ? 0.0 : kLog2e / (double)T;
        for (int slot = wave; slot < R; slot += kWaves) {
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

        if (tid < K) {
            const int i = tid;
            if (greedy) {
                L.acc[i] = (x == L.idx[i]) ? 1 : 0;
                L.err[i] = isfinite(L.m[i]) ? 0 : SV_ERR_ROW;
            } else {
                const float mt = L.m[i], md = L.m[K + 1 + i];
                int err = 0;
                if (!isfinite(mt)) err |= SV_ERR_ROW;
                if (!isfinite(md)) err |= SV_ERR_ROW;
                else if (!(L.S[K + 1 + i] > 0.0)) err |= SV_ERR_DRAFT_MASS;
                const bool x_ok = x >= 0 && x < a.V && err == 0;
                const bool in_top = weighted && top_has(L.top[i], x);
                const float u = philox_uniform(a.seed, (uint32_t)gb, (uint32_t)i, kPurposeAccept);
                float pt, pd;
                L.acc[i] = decide(T, mt, L.S[i], md, L.S[K + 1 + i], in_top, a.beta, x_ok, zx.x,
                                  zx.y, u, pt, pd)
                               ? 1
                               : 0;
                L.err[i] = err;
                L.pt[i] = pt;
                L.pd[i] = pd;
            }
        }
        __syncthreads();
    }

    if (tid == 0) {
        int n = K, err_bits = 0;
        if (!fail) {
            for (int i = 0; i < K; ++i) {
                if (L.err[i]) {
                    fail = L.err[i];
                    break;
                }
                if (!L.acc[i]) {
                    n = i;
                    break;
                }
            }
            if (!fail && n == K && !isfinite(L.m[K])) fail = SV_ERR_ROW;
            if (!fail && n < K) {
                const int xn = a.tokens[(int64_t)b * K + n];
                if (xn < 0 || xn >= a.V) err_bits |= SV_ERR_TOKEN;
            }
        }
        L.n = n;
        L.fail = fail;
        L.err_bits = err_bits | fail;
    }
    __syncthreads();
    const int n = L.n;
    fail = L.fail;

    // outputs, written in parallel
    if (tid <= K) {
        int v = -1;
        if (!fail) {
            if (tid < n) v = a.tokens[(int64_t)b * K + tid];
            else if (tid == n && greedy) v = L.idx[n];
        }
        // slot n of a sampling sequence is written again by the bonus draw
        // (another workgroup), so both writes go to the coherent point
        if (tid == n) st_agent(reinterpret_cast<uint32_t *>(out + tid), (uint32_t)v);
        else out[tid] = v;
    }
    if (tid < K) {
        const bool show = !fail && !greedy && tid <= n;
        if (a.aux_pt) a.aux_pt[(int64_t)b * K + tid] = show ? L.pt[tid] : NAN;
        if (a.aux_pd) a.aux_pd[(int64_t)b * K + tid] = show ? L.pd[tid] : NAN;
    }
    if (tid == 0) {
        a.accepted_len[b] = fail ? 0 : n;
        if (a.aux_z && (fail || greedy)) a.aux_z[b] = NAN;
        if (L.err_bits && a.error_word) atomicOr(a.error_word, L.err_bits);
        SeqState st = {};
        st.mode = 0;
        if (!fail && !greedy) {
            st.n = n;
            st.mode = n < K ? 1 : 2;
            st.m_t = L.m[n];
            st.inv_st = (float)(1.0 / L.S[n]);
            st.T = T;
            st.beta = a.beta;
            st.u_bonus = philox_uniform(a.seed, (uint32_t)gb, (uint32_t)n, kPurposeBonus);
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
                    for (int k = 0; k < 4; ++k)
                        st.top[k] = L.top[n].i[k] == INT_MAX ? -1 : L.top[n].i[k];
                }
            }
        }
        *st_lds = st;
    }
    __syncthreads();
    // publish the state (wave 0 stores it word by word, drains, raises the flag)
    if (tid < 16) st_agent(reinterpret_cast<uint32_t *>(a.state + b) + tid,
                           reinterpret_cast<const uint32_t *>(st_lds)[tid]);
    if (wave == 0) {
        drain_memory();
        if (tid == 0) {
            st_agent(&a.seqctl[b].count, 0u);
            st_agent(&a.seqctl[b].flag, 1u);
        }
    }
}

__device__ __forceinline__ double ld_res(const double *p)
{
    return __hip_atomic_load(const_cast<double *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Inverse-CDF scan of chunk c: the first element whose running residual sum,
// started at `base`, reaches `thr` (INT_MAX if none), the chunk total and the
// last element with mass.  Elements are visited in index order: vector u of
// every thread, thread by thread, then u + 1.
template <int DT, int U, bool TOP>
__device__ __forceinline__ int scan_chunk(const char *trow, const char *drow, bool aligned, int mode, int c,
                          int nvec, int V, const SeqState &st, const ExpScale &e, double base,
                          double thr, double &total, int &last_pos, double *ldsd, int *ldsi)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const int q0 = c * kBlock * U;
    uint4 rt[U], rd[U];
    load_chunk<DT, U>(trow, aligned, false, q0, nvec, V, rt);
    if (mode == 1) load_chunk<DT, U>(drow, aligned, false, q0, nvec, V, rd);
    double run = base;
    int last = -1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float xt[VEC], xd[VEC];
        Elt<DT>::unpack(rt[u], xt);
        if (mode == 1) Elt<DT>::unpack(rd[u], xd);
        double acc = 0.0;
        int mylast = -1;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int idx = elem_index(q0, u, k, VEC);
            const float rv = residual_at<TOP>(xt[k], mode == 1 ? xd[k] : 0.f, idx, st, e, mode);
            acc += (double)rv;
            if (rv > 0.f) mylast = idx;
        }
        double tile_total;
        const double exc = block_exclusive_scan(acc, tile_total, ldsd);
        int cand = INT_MAX;
        if (run + exc + acc >= thr) {
            // the crossing is inside this thread's vector: walk it again
            double pre = run + exc;
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int idx = elem_index(q0, u, k, VEC);
                pre += (double)residual_at<TOP>(xt[k], mode == 1 ? xd[k] : 0.f, idx, st, e, mode);
                if (pre >= thr && cand == INT_MAX) cand = idx;
            }
        }
        cand = block_min_int(cand, ldsi);
        last = max(last, block_max_int(mylast, ldsi));
        run += tile_total;
        if (cand != INT_MAX) {
            total = run;
            last_pos = last;
            return cand;
        }
    }
    total = run;
    last_pos = last;
    return INT_MAX;
}

// Bonus draw of sequence b, run by the last workgroup to publish a residual
// chunk sum: the smallest v with C(v) >= u * Z, C in ascending token id.
template <int DT, int U, bool TOP>
__device__ __forceinline__ void bonus_sequence(const FusedArgs &a, int b, const SeqState &st, double *ldsd,
                               int *ldsi)
{
    const int tid = threadIdx.x;
    const int nc = a.chunks;
    const ExpScale e = make_scale(st.T);
    const double *rs = a.res + (int64_t)b * nc;
    const char *trow = a.target + ((int64_t)b * (a.K + 1) + st.n) * a.row_bytes;
    const char *drow = st.mode == 1 ? a.draft + ((int64_t)b * a.K + st.n) * a.row_bytes : trow;
    const bool aligned = ((uintptr_t)trow & 15) == 0 && ((uintptr_t)drow & 15) == 0;

    double Z = 0.0;
    for (int c0 = 0; c0 < nc; c0 += kBlock) {
        double tot;
        block_exclusive_scan(c0 + tid < nc ? ld_res(rs + c0 + tid) : 0.0, tot, ldsd);
        Z += tot;
    }
    int token = -1, last = -1;
    double total;
    if (Z > 0.0) {
        const double thr = (double)st.u_bonus * Z;
        double run = 0.0, cbase = 0.0, last_base = 0.0;
        int cstar = INT_MAX, last_chunk = -1;
        for (int c0 = 0; c0 < nc && cstar == INT_MAX; c0 += kBlock) {
            const int c = c0 + tid;
            const double v = c < nc ? ld_res(rs + c) : 0.0;
            double tot;
            const double exc = block_exclusive_scan(v, tot, ldsd);
            int cand = (c < nc && run + exc + v >= thr) ? c : INT_MAX;
            cand = block_min_int(cand, ldsi);
            const int lastc = block_max_int(v > 0.0 ? c : -1, ldsi);
            if (cand != INT_MAX || lastc > last_chunk) {
                if (c == cand) ldsd[0] = run + exc;
                if (c == lastc) ldsd[1] = run + exc;
                __syncthreads();
                if (cand != INT_MAX) cbase = ldsd[0];
                if (lastc > last_chunk) last_base = ldsd[1];
                __syncthreads();
            }
            if (cand != INT_MAX) cstar = cand;
            if (lastc > last_chunk) last_chunk = lastc;
            run += tot;
        }
        if (cstar == INT_MAX) {  // u * Z above the last prefix through rounding
            cstar = last_chunk;
            cbase = last_base;
        }
        if (cstar >= 0) {
            token = scan_chunk<DT, U, TOP>(trow, drow, aligned, st.mode, cstar, a.nvec, a.V, st, e,
                                           cbase, thr, total, last, ldsd, ldsi);
            if (token == INT_MAX) token = last;
        }
    }
    if (token < 0) {
        // zero residual mass (only through rounding): draw from p_t of row n
        double run = 0.0;
        for (int c = 0; c < nc; ++c) {
            scan_chunk<DT, U, TOP>(trow, trow, aligned, 2, c, a.nvec, a.V, st, e, run, INFINITY,
                                   total, last, ldsd, ldsi);
            run = total;
        }
        Z = run;
        const double thr = (double)st.u_bonus * Z;
        double base = 0.0;
        int lastseen = -1;
        for (int c = 0; c < nc && token < 0; ++c) {
            const int t = scan_chunk<DT, U, TOP>(trow, trow, aligned, 2, c, a.nvec, a.V, st, e, base,
                                                 thr, total, last, ldsd, ldsi);
            if (last >= 0) lastseen = last;
            if (t != INT_MAX) token = t;
            base = total;
        }
        if (token < 0) token = lastseen;
    }
    if (tid == 0) {
        st_agent(reinterpret_cast<uint32_t *>(a.out_tokens + (int64_t)b * (a.K + 1) + st.n),
                 (uint32_t)token);
        if (a.aux_z) a.aux_z[b] = (float)Z;
    }
}

// Per-thread running statistics over the sub-tiles of a streaming item.
// Sampling rows: (max m, fp64 sum s of exp2((z - m) c)), rescaled when m grows.
template <int DT, int U>
__device__ __forceinline__ void thread_sum_tile(const uint4 (&r)[U], const ExpScale &e, float &m,
                                                double &s)
{
    constexpr int VEC = Elt<DT>::kVec;
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) mx = fmaxf(mx, x[k]);
    }
    if (mx > m) {
        if (s != 0.0) s *= exp2(((double)m - (double)mx) * e.c64);
        m = mx;
    }
    if (m == -INFINITY) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], m, e);
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        s += (double)ev[0];
    }
}

// Greedy rows: the thread's (max, lowest index) in increasing index order.
template <int DT, int U>
__device__ __forceinline__ void thread_argmax_tile(const uint4 (&r)[U], int q0, float &best, int &bi)
{
    constexpr int VEC = Elt<DT>::kVec;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
        float mx = x[0];
#pragma unroll
        for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[k]);
        if (mx > best) {
            int kk = VEC - 1;
#pragma unroll
            for (int k = VEC - 1; k >= 0; --k)
                if (x[k] == mx) kk = k;
            best = mx;
            bi = elem_index(q0, u, kk, VEC);
        }
    }
}

// Fold one sub-tile's (M_s, S_s, T_s) of a weighted draft row into the running
// (M, S, T): S is the mass outside T, so the entries that drop out of the
// top-4 join it.
__device__ __forceinline__ void top_run_merge(float &M, double &S, Top4 &T, float Ms, double Ss,
                                              const Top4 &Ts, double c64)
{
    const float Mn = fmaxf(M, Ms);
    if (Mn == -INFINITY) return;
    Top4 n = T;
#pragma unroll
    for (int k = 0; k < 4; ++k) top_insert(n, Ts.v[k], Ts.i[k]);
    double Sn = 0.0;
    if (M != -INFINITY && S != 0.0) Sn += S * exp2(((double)M - (double)Mn) * c64);
    if (Ms != -INFINITY && Ss != 0.0) Sn += Ss * exp2(((double)Ms - (double)Mn) * c64);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        if (T.i[k] != INT_MAX && T.v[k] != -INFINITY && !top_has(n, T.i[k]))
            Sn += exp2(((double)T.v[k] - (double)Mn) * c64);
        if (Ts.i[k] != INT_MAX && Ts.v[k] != -INFINITY && !top_has(n, Ts.i[k]))
            Sn += exp2(((double)Ts.v[k] - (double)Mn) * c64);
    }
    M = Mn;
    S = Sn;
    T = n;
}

// Streaming item (b, p, c): sub-tiles of kBlock * U vectors of the row(s) of
// slot p, vectors [c * span, (c + 1) * span) with span = sspan sub-tiles; then
// publish the partials and arrive; the last arriver runs the accept scan.
template <int DT, int U, bool TOP>
__device__ __forceinline__ void stream_item(const FusedArgs &a, int item, uint32_t *s_u, float *s_f,
                                            int *s_i, double *s_d, TopLds &s_top,
                                            unsigned char *s_stage, AcceptLds &s_acc,
                                            SeqState &s_st)
{
    constexpr int VEC = Elt<DT>::kVec;
    constexpr int kTile = kBlock * U;
    const int tid = threadIdx.x;
    const int ips = (a.K + 1) * a.schunks;
    const int b = item / ips;
    const int rem = item - b * ips;
    const int p = rem / a.schunks;
    const int c = rem - p * a.schunks;
    const int K = a.K;

    const float T = a.temperature[b];
    const bool tok = temperature_ok(T);
    const bool greedy = T == 0.f;
    const bool samp = tok && !greedy;
    const bool need_d = samp && p < K && a.draft != nullptr;
    const char *trow = a.target + ((int64_t)b * (K + 1) + p) * a.row_bytes;
    const char *drow = need_d ? a.draft + ((int64_t)b * K + p) * a.row_bytes : trow;
    const bool aligned = ((uintptr_t)trow & 15) == 0 && ((uintptr_t)drow & 15) == 0;
    const int v0 = c * a.sspan * kTile;
    const int v1 = min(a.nvec, v0 + a.sspan * kTile);
    const ExpScale e = make_scale(samp ? T : 1.f);

    // drafted token of this slot and, if this chunk holds it, its two logits
    bool gather = false;
    float zt = 0.f, zd = 0.f;
    if (samp && p < K) {
        const int x = a.tokens[(int64_t)b * K + p];
        gather = need_d && x >= v0 * VEC && x < min(a.V, v1 * VEC);
        if (gather && tid == 0) {
            zt = DT == 0 ? Elt<0>::scalar(trow, x) : Elt<1>::scalar(trow, x);
            zd = DT == 0 ? Elt<0>::scalar(drow, x) : Elt<1>::scalar(drow, x);
        }
    }

    float mt = -INFINITY, md = -INFINITY, bt = -INFINITY;
    double st = 0.0, sd = 0.0;
    int bit = INT_MAX;
    float Mw = -INFINITY;  // weighted draft row: running max, mass outside the top-4, top-4
    double Sw = 0.0;
    Top4 Tw;
    top_clear(Tw);
    for (int q0 = v0; q0 < v1; q0 += kTile) {
        uint4 rt[U], rd[U];
        load_pair<DT, U>(trow, drow, tok, need_d, aligned, q0, a.nvec, a.V, rt, rd);
        if (tok) {
            if (greedy) thread_argmax_tile<DT, U>(rt, q0, bt, bit);
            else thread_sum_tile<DT, U>(rt, e, mt, st);
        }
        if (need_d) {
            if (TOP) {
                float Ms;
                double Ss;
                Top4 Ts;
                chunk_sum_top<DT, U>(rd, e, q0, a.V, s_f, s_i, s_d, s_top, Ms, Ss, Ts);
                top_run_merge(Mw, Sw, Tw, Ms, Ss, Ts, e.c64);
            } else {
                thread_sum_tile<DT, U>(rd, e, md, sd);
            }
        }
    }

    RowPart *prow = a.part + (int64_t)b * (2 * K + 1) * a.schunks;
    if (tok) {
        RowPart pt;
        if (greedy) {
            block_argmax(bt, bit, s_f, s_i);
            pt.m = bt;
            pt.idx = bit;
            pt.s = 0.0;
        } else {
            const float M = block_max(mt, s_f);
            const double sc = (mt == -INFINITY) ? 0.0 : st * exp2(((double)mt - (double)M) * e.c64);
            pt.m = M;
            pt.idx = -1;
            pt.s = block_sum(sc, s_d);
        }
        if (tid == 0) st_agent_obj(prow + p * a.schunks + c, pt);
    }
    if (need_d) {
        RowPart pd;
        pd.idx = -1;
        if (TOP) {
            pd.m = Mw;
            pd.s = Sw;
            if (tid == 0) st_agent_obj(a.top + ((int64_t)b * K + p) * a.schunks + c, Tw);
        } else {
            const float M = block_max(md, s_f);
            const double sc = (md == -INFINITY) ? 0.0 : sd * exp2(((double)md - (double)M) * e.c64);
            pd.m = M;
            pd.s = block_sum(sc, s_d);
        }
        if (tid == 0) st_agent_obj(prow + (K + 1 + p) * a.schunks + c, pd);
    }
    if (gather && tid == 0) {
        uint32_t *zw = reinterpret_cast<uint32_t *>(a.zx + (int64_t)b * K + p);
        st_agent(zw, __float_as_uint(zt));
        st_agent(zw + 1, __float_as_uint(zd));
    }

    // publish and arrive; the last arriver runs the accept scan
    if (tid == 0) {
        drain_memory();
        const uint32_t old = atomicAdd(&a.seqctl[b].count, 1u);
        s_u[1] = (old == (uint32_t)ips - 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (s_u[1]) accept_sequence<TOP>(a, b, T, s_stage, s_acc, &s_st);
}

// Draw item: wait for the accept of sequence b, then the residual mass of
// chunk c of the drawn rows; the last chunk to publish draws the bonus.
template <int DT, int U, bool TOP>
__device__ __forceinline__ void draw_item(const FusedArgs &a, int item, uint32_t *s_u, double *s_d,
                                          int *s_i, SeqState &s_st)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const int b = item / a.chunks;
    const int c = item - b * a.chunks;
    const int K = a.K;
    SeqCtl &ctl = a.seqctl[b];

    if (tid == 0) {
        // poll with exponential backoff (64 to 4096 cycles between polls)
        uint32_t slept = 0, nap = 1, timeout = 0;
        while (ld_agent(&ctl.flag) == 0u) {  // state reads below are coherent loads too
            for (uint32_t k = 0; k < nap; ++k) __builtin_amdgcn_s_sleep(1);
            slept += nap;
            nap = nap < 64u ? nap * 2u : 64u;
            if (slept > a.spin_limit) {
                timeout = 1;
                break;
            }
        }
        if (timeout && a.error_word) atomicOr(a.error_word, kErrTimeout);
        s_u[2] = timeout;
    }
    __syncthreads();
    if (!s_u[2]) {
        // the state, read with lane-indexed loads into LDS
        if (tid < 16) {
            const uint32_t w = __hip_atomic_load(reinterpret_cast<uint32_t *>(a.state + b) + tid,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            reinterpret_cast<uint32_t *>(&s_st)[tid] = w;
        }
        __syncthreads();
        const SeqState st = s_st;
        if (st.n >= 0 && st.n <= K && ((st.mode == 1 && st.n < K) || (st.mode == 2 && st.n == K))) {
            const ExpScale e = make_scale(st.T);
            const char *trow = a.target + ((int64_t)b * (K + 1) + st.n) * a.row_bytes;
            const char *drow = st.mode == 1 ? a.draft + ((int64_t)b * K + st.n) * a.row_bytes : trow;
            const bool aligned = ((uintptr_t)trow & 15) == 0 && ((uintptr_t)drow & 15) == 0;
            const int q0 = c * kBlock * U;
            uint4 rt[U], rd[U];
            load_pair<DT, U>(trow, drow, true, st.mode == 1, aligned, q0, a.nvec, a.V, rt, rd);
            double acc = 0.0;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float xt[VEC], xd[VEC], rv[VEC];
                Elt<DT>::unpack(rt[u], xt);
                if (st.mode == 1) Elt<DT>::unpack(rd[u], xd);
#pragma unroll
                for (int k = 0; k < VEC; ++k)
                    rv[k] = residual_at<TOP>(xt[k], st.mode == 1 ? xd[k] : 0.f,
                                             elem_index(q0, u, k, VEC), st, e, st.mode);
#pragma unroll
                for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                    for (int k = 0; k < w; ++k) rv[k] += rv[k + w];
                acc += (double)rv[0];
            }
            const double Rc = block_sum(acc, s_d);
            if (tid == 0) {
                __hip_atomic_store(a.res + (int64_t)b * a.chunks + c, Rc, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                drain_memory();
                const uint32_t old = atomicAdd(&ctl.rcount, 1u);
                s_u[3] = (old == (uint32_t)a.chunks - 1u) ? 1u : 0u;
            }
            __syncthreads();
            if (s_u[3]) bonus_sequence<DT, U, TOP>(a, b, st, s_d, s_i);
        }
    }
    // the last draw item of the sequence returns its control words to zero
    __syncthreads();
    if (tid == 0) {
        drain_memory();
        const uint32_t old = atomicAdd(&ctl.dcount, 1u);
        if (old == (uint32_t)a.chunks - 1u) {
            __hip_atomic_store(&ctl.rcount, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctl.flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&ctl.dcount, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <int DT, int U, bool TOP>
__global__ __launch_bounds__(kBlock) void fused_kernel(const FusedArgs a)
{
    __shared__ uint32_t s_u[4];
    __shared__ float s_f[4 + kWaves * 4];
    __shared__ int s_i[4 + kWaves * 4];
    __shared__ double s_d[kWaves];
    __shared__ TopLds s_top;
    __shared__ __align__(16) unsigned char s_stage[kStageBytes];
    __shared__ AcceptLds s_acc;
    __shared__ SeqState s_st;

    const int item = (int)blockIdx.x;
    if (item < a.stream_items)
        stream_item<DT, U, TOP>(a, item, s_u, s_f, s_i, s_d, s_top, s_stage, s_acc, s_st);
    else
        draw_item<DT, U, TOP>(a, item - a.stream_items, s_u, s_d, s_i, s_st);
}

// ---------------------------------------------------------------------------
// Host side.

template <int DT, bool TOP>
static int resident_capacity()
{
    static int cap[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cap[dev] == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fused_kernel<DT, kFusedU, TOP>,
                                                         kBlock, 0) != hipSuccess)
            return 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cap[dev] = per_cu * cus;
    }
    return cap[dev];
}

bool fused_capacity_ok(const Plan &p, bool weighted)
{
    if (!p.fused_shape_ok) return false;
    int cap = 0;
    if (p.dtype == SV_F32) cap = weighted ? resident_capacity<0, true>() : resident_capacity<0, false>();
    else cap = weighted ? resident_capacity<1, true>() : resident_capacity<1, false>();
    return cap > 0;
}

void launch_fused(const FusedArgs &a, const Plan &p, hipStream_t s)
{
    const unsigned grid = (unsigned)(a.stream_items + a.B * a.chunks);
    if (p.dtype == SV_F32) {
        if (a.weighted) fused_kernel<0, kFusedU, true><<<grid, kBlock, 0, s>>>(a);
        else fused_kernel<0, kFusedU, false><<<grid, kBlock, 0, s>>>(a);
    } else {
        if (a.weighted) fused_kernel<1, kFusedU, true><<<grid, kBlock, 0, s>>>(a);
        else fused_kernel<1, kFusedU, false><<<grid, kBlock, 0, s>>>(a);
    }
}

}  // namespace sv
