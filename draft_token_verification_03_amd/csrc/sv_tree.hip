// sv_tree.hip -- tree (multi-draft) verification.
//
// The pages name tree-based speculative decoding ("Speculative Speculative
// Decoding", Key claims: SSD composes with Medusa-style trees) without a
// verify rule; this is the published recursive rejection sampling over a
// token tree (Miao et al., "SpecInfer", ASPLOS'24), which keeps the output
// law the target's when the children of every context are drawn i.i.d. from
// its draft law.  Node i < N has a parent in [-1, i-1] (-1: the root) and a
// token; context 0 is the root and context i + 1 is node i.  Target row c
// holds the target logits after context c, draft row c (c < N) the draft
// logits the children of context c were drawn from.  At a context the law
// starts as its target law p; its children are tried in node order, child j
// with token x being accepted iff u(b, j, 0) <= r(x) / q(x), and a rejection
// replaces r by max(r - q, 0) normalised.  An accepted child becomes the
// current context; when none is left the bonus is drawn from r by the
// inverse CDF in token order with u(b, d, 1), d the accepted depth.  Greedy
// sequences (T = 0) take the first child whose token is the target argmax.
// A chain (parent[i] = i - 1) is the verify step with K = N.
//
// One workgroup walks one sequence and reads only the rows of the contexts
// it visits: per context one pass over its target and draft rows for their
// statistics (the running-max sums of the streaming pass), one more pass per
// rejection for the mass of the next law (kept per tile step for the bonus
// search), and at the end the one tile step the bonus lies in.  Decisions
// are taken by thread 0 in fp64 from the two logits gathered at the token.
#include <hip/hip_ext.h>

#include "sv_accept.h"
#include "sv_stream.h"
#include "sv_tile.h"

namespace sv {

// One workgroup streams a sequence's rows on its own, so its rate is set by
// the bytes it has in flight.  512 threads (two waves per SIMD, up to 256
// registers a thread: the walk's decision and law state fit without spills,
// which a 1024-thread group's 128 registers do not) each take two vectors of
// each row per tile, and aligned rows stream through an LDS ring three tiles
// deep (below), ~96 KB of both rows in flight per workgroup.
constexpr int kTreeBlock = 512;
constexpr int kTreeWaves = kTreeBlock / 64;
constexpr int kTreeLoads = 2;
using TreeTile = PairTileU<kTreeLoads>;
static_assert(kTreeBlock * kTreeLoads == kTreeStepVecs, "tile step of the tree walk");

// The law at a context after L rejections that left mass.  With p, q the
// context's target and draft laws and z_i the mass of the i-th residual,
// r_{i+1} = max(r_i - q, 0) / z_i unrolls to
//   r_L = max(p - q A, 0) / P,   A = sum_{k<L} prod_{i<k} z_i,  P = prod_{i<L} z_i
// (A = 0, P = 1 for the target law itself; once p - q A_i <= 0 at a token it
// stays so, since A only grows), and a rejection's residual is
// max(r_L - q, 0) = max(p - q (A + P), 0) / P.  So every law is formed per
// element as one residual of the target and draft rows, like the verify
// step's, with relative accuracy where p and q A nearly cancel:
//   w(v) = exp2(z_t c - o_t) * max(1 - 2^{(z_d - z_t) c + kappa}, 0),
//   kappa = o_t - o_d + log2(S_t / S_d) + log2(A)     (= S_t P r_L(v)),
// the fp32 kappa split into hi + lo parts so that one fma rounds it once.
// A pass of kLawTarget forms w = exp2(z_t c - o_t) = S_t p(v) (A = 0).
constexpr int kLawTarget = 0, kLawResidual = 1;
constexpr int kWaveSteps = 64;  // tile steps a row may have for the barrier-free law pass

struct Law {
    ExpScale e;
    float ot;              // target row offset fp32(m_t c)
    float k_hi, k_lo;      // kappa
};

template <int MODE>
__device__ __forceinline__ float law_mass(float zt, float zd, const Law &w)
{
    const float pt = exp_scaled(zt, w.ot, w.e);
    if (MODE == kLawTarget) return pt;
    const float d = __builtin_fmaf(zd - zt, w.e.c, w.k_hi) + w.k_lo;
    return pt * one_minus_exp2(d);  // q A >= p (or a NaN of masked tokens): no mass
}

__device__ __forceinline__ void law_kappa(Law &w, double kappa)
{
    w.k_hi = (float)kappa;
    w.k_lo = (float)(kappa - (double)w.k_hi);
}

// Sum of w over the vector pair (fp32, pairwise).
template <int DT, int MODE>
__device__ __forceinline__ float law_vec(uint4 rt, uint4 rd, const Law &w, float (&m)[Elt<DT>::kVec])
{
    constexpr int VEC = Elt<DT>::kVec;
    float xt[VEC], xd[VEC];
    Elt<DT>::unpack(rt, xt);
    if (MODE != kLawTarget) Elt<DT>::unpack(rd, xd);
#pragma unroll
    for (int k = 0; k < VEC; ++k) m[k] = law_mass<MODE>(xt[k], MODE != kLawTarget ? xd[k] : 0.f, w);
    float s[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) s[k] = m[k];
#pragma unroll
    for (int h = VEC / 2; h > 0; h >>= 1)
#pragma unroll
        for (int k = 0; k < h; ++k) s[k] += s[k + h];
    return s[0];
}

// Aligned rows stream through a ring in LDS: each wave owns kRingStages
// stages of kTreeLoads 16-byte vectors per lane of the target row and of the
// draft row, filled by gfx950's 16-byte global-to-LDS loads, so that a
// thread has kRingStages - 1 tiles of both rows in flight without holding
// them in registers (register tiles reach two in flight).  The loads of a
// wave complete in order, so waiting until at most (kRingStages - 1) tiles'
// loads are outstanding leaves the oldest stage complete; the wave then reads
// its stage back, the only reader of its own stages, so no barrier is needed.
// The compiler's own wait before an LDS read of a global-to-LDS target is
// for every outstanding load, which would drain the ring each tile, so the
// ring is read by an assembly read that waits for itself, and the tile waits
// are explicit.  Past the row's last tile the loads repeat that tile's
// (in-bounds) addresses, which keeps the outstanding count the same on every
// tile; every load has landed before the pass returns.
constexpr int kRingStages = 4;
static_assert((kRingStages & (kRingStages - 1)) == 0, "ring stages: a power of two");

struct TreeRing {
    uint4 v[kTreeWaves][kRingStages][2][kTreeLoads][64];  // [wave][stage][target, draft][u][lane]
};
__shared__ TreeRing tree_ring;

template <int N>
__device__ __forceinline__ void wait_vmem()
{
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// A stage's vectors, read back by the lane that requested them.
__device__ __forceinline__ void ring_read2(const uint4 *p0, const uint4 *p1, uint4 &a, uint4 &b)
{
    const uint32_t a0 = (uint32_t)(uintptr_t)p0, a1 = (uint32_t)(uintptr_t)p1;
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(a), "=&v"(b)
                 : "v"(a0), "v"(a1)
                 : "memory");
}

template <int DT, bool PAIR, class Consume>
__device__ __forceinline__ void ring_pass(const char *trow, const char *drow, int nvec, int V, Consume &&consume)
{
    static_assert(kTreeLoads == 2, "the ring reads two vectors a row per thread and tile");
    constexpr int kStep = kTreeBlock * kTreeLoads;
    constexpr int kPerTile = kTreeLoads * (PAIR ? 2 : 1);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nt = (nvec + kStep - 1) / kStep;  // >= 1
    const int own = wave * 64 + lane;
    auto issue = [&](int t) {
        const int st = t & (kRingStages - 1);
        const int qb = min(t, nt - 1) * kStep + own;
#pragma unroll
        for (int u = 0; u < kTreeLoads; ++u) {
            const int q = min(qb + u * kTreeBlock, nvec - 1);
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(trow) + q,
                                             &tree_ring.v[wave][st][0][u][0], 16, 0, 0);
            if (PAIR)
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const uint4 *>(drow) + q,
                                                 &tree_ring.v[wave][st][1][u][0], 16, 0, 0);
        }
    };
    // the first kRingStages - 1 rounds only fill the ring
    for (int t = 1 - kRingStages; t < nt; ++t) {
        issue(t + kRingStages - 1);
        if (t < 0) continue;
        wait_vmem<kPerTile * (kRingStages - 1)>();
        const int st = t & (kRingStages - 1);
        TreeTile tl;
        ring_read2(&tree_ring.v[wave][st][0][0][lane], &tree_ring.v[wave][st][0][1][lane], tl.t[0], tl.t[1]);
        if (PAIR)
            ring_read2(&tree_ring.v[wave][st][1][0][lane], &tree_ring.v[wave][st][1][1][lane], tl.d[0], tl.d[1]);
        else
            tl.d[0] = tl.d[1] = tl.t[0];
        if (t == nt - 1) fix_pair<DT, PAIR, kTreeBlock>(t * kStep, nvec, V, tl);
        consume(tl, t * kStep);
    }
    wait_vmem<0>();
}

// A whole-row pass of the workgroup: aligned rows through the LDS ring,
// others through register tiles with funnel-shifted loads.
template <int DT, bool PAIR, class Consume>
__device__ __forceinline__ void row_pass(const char *trow, const char *drow, int nvec, int V, Consume &&consume)
{
    const bool aligned = ((uintptr_t)trow & 15) == 0 && (!PAIR || ((uintptr_t)drow & 15) == 0);
    if (aligned) {
        ring_pass<DT, PAIR>(trow, drow, nvec, V, consume);
    } else {
        TreeTile ra;
        issue_pair<DT, false, PAIR, kTreeBlock>(trow, drow, 0, nvec, V, ra);
        stream_pair<DT, false, PAIR, kTreeBlock>(trow, drow, 0, nvec, V, ra, consume);
    }
}

// Mass of a law per tile step into ssum[] (fp64 step sums of the threads'
// fp32 vector sums, the waves' sums added in wave order); returns the total
// (the step sums added in step order).  Rows of at most kWaveSteps steps keep
// each wave's step sums in wsum[] and add them up after the pass, so the waves
// stream without a barrier per step; longer rows reduce every step at once.
template <int DT, int MODE>
__device__ __forceinline__ double law_pass(const char *trow, const char *drow, int nvec, int V, const Law &w,
                                           double *ssum, double *wsum, double *lds_d)
{
    constexpr int VEC = Elt<DT>::kVec;
    constexpr int kStep = kTreeBlock * kTreeLoads;
    const int nsteps = (nvec + kStep - 1) / kStep;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    auto part_of = [&](TreeTile &tl) {
        double part = 0.0;
#pragma unroll
        for (int u = 0; u < kTreeLoads; ++u) {
            float m[VEC];
            part += (double)law_vec<DT, MODE>(tl.t[u], tl.d[u], w, m);
        }
        return part;
    };
    if (nsteps <= kWaveSteps) {
        auto consume = [&](TreeTile &tl, int qb) {
            const double ws = wave_sum(part_of(tl));
            if (lane == 0) wsum[(qb / kStep) * kTreeWaves + wave] = ws;
        };
        if (MODE == kLawTarget) row_pass<DT, false>(trow, nullptr, nvec, V, consume);
        else row_pass<DT, true>(trow, drow, nvec, V, consume);
        __syncthreads();
        for (int k = threadIdx.x; k < nsteps; k += kTreeBlock) {
            double v = wsum[k * kTreeWaves];
#pragma unroll
            for (int x = 1; x < kTreeWaves; ++x) v += wsum[k * kTreeWaves + x];
            ssum[k] = v;
        }
        __syncthreads();
        double total = 0.0;
        for (int k = 0; k < nsteps; ++k) total += ssum[k];
        return total;
    }
    double total = 0.0;
    auto consume = [&](TreeTile &tl, int qb) {
        const double s = block_sum<kTreeWaves>(part_of(tl), lds_d);
        if (threadIdx.x == 0) ssum[qb / kStep] = s;
        total += s;
    };
    if (MODE == kLawTarget) row_pass<DT, false>(trow, nullptr, nvec, V, consume);
    else row_pass<DT, true>(trow, drow, nvec, V, consume);
    return total;
}

// Greedy rows: the lane's (max, lowest index) over a tile of the walk.
template <int DT>
__device__ __forceinline__ void tree_argmax_tile(const uint4 (&r)[kTreeLoads], int q0, float &best, int &bi)
{
    constexpr int VEC = Elt<DT>::kVec;
#pragma unroll
    for (int u = 0; u < kTreeLoads; ++u) {
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
            bi = (q0 + u * kTreeBlock + (int)threadIdx.x) * VEC + kk;
        }
    }
}

// (max M, fp64 sum of exp2((z - M) c)) of a row from the threads' runs.
__device__ __forceinline__ void tree_run_finish(const RowRun &run, const ExpScale &e, float *lds_f, double *lds_d,
                                                float &M, double &S)
{
    M = block_max<kTreeWaves>(run.m, lds_f);
    const double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - (double)row_offset(M, e));
    S = block_sum<kTreeWaves>(sc, lds_d);
}

// Vector q (< nvec) of a row, elements at or beyond V as -inf.
template <int DT>
__device__ __forceinline__ uint4 tree_load(const char *row, int q, int nvec, int V)
{
    constexpr int VEC = Elt<DT>::kVec;
    const char *p = row + (size_t)q * 16;
    uint4 r;
    if (((uintptr_t)row & 15) == 0) {
        r = *reinterpret_cast<const uint4 *>(p);
    } else {
        const int valid = min(VEC, V - q * VEC);
        r = load16_unaligned(p, ((uint32_t)((uintptr_t)p & 15)) + (uint32_t)valid * Elt<DT>::kBytes > 16u);
    }
    if ((V % VEC) && q == nvec - 1) mask_raw<DT>(r, V - q * VEC);
    return r;
}

// The bonus: smallest v with C(v) >= thr, C the running sum of w in token
// order, from the step sums of the pass that formed them and one re-read
// step.  Within a step, token order is vector slot u first, then thread,
// then element.
template <int DT, int MODE>
__device__ __forceinline__ int law_draw(const char *trow, const char *drow, int nvec, int V, const Law &w,
                                        const double *ssum, double thr, double *lds_d, int *lds_i)
{
    constexpr int VEC = Elt<DT>::kVec;
    constexpr int kStep = kTreeBlock * kTreeLoads;
    const int nsteps = (nvec + kStep - 1) / kStep;
    const int tid = threadIdx.x;
    if (tid == 0) {
        double c = 0.0, c_last = 0.0;
        int s = -1, s_last = 0;
        for (int k = 0; k < nsteps; ++k) {
            if (ssum[k] > 0.0) {
                if (c + ssum[k] >= thr) {
                    s = k;
                    break;
                }
                s_last = k;
                c_last = c;
            }
            c += ssum[k];
        }
        if (s < 0) {  // rounding left thr above the total: the last step with mass, at its end
            s = s_last;
            c = c_last;
            thr = c_last + ssum[s_last];
        }
        lds_i[0] = s;
        lds_d[0] = thr - c;  // the threshold within the step
    }
    __syncthreads();
    const int s = lds_i[0];
    double rem = lds_d[0];
    __syncthreads();
    const int qb = s * kStep;
    int found = INT_MAX;  // lowest token whose running sum reaches rem, per thread
    int last = -1;        // the step's last token with mass (rounding fallback)
    for (int u = 0; u < kTreeLoads; ++u) {
        const int q = qb + u * kTreeBlock + tid;
        uint4 rt = neg_inf_raw<DT>(), rd = neg_inf_raw<DT>();
        const bool live = q < nvec;
        if (live) {
            rt = tree_load<DT>(trow, q, nvec, V);
            if (MODE != kLawTarget) rd = tree_load<DT>(drow, q, nvec, V);
        }
        float m[VEC];
        const float vs = law_vec<DT, MODE>(rt, rd, w, m);
        double tot;
        const double exc = block_exclusive_scan<kTreeWaves>((double)vs, tot, lds_d);
        if (rem <= tot) {  // the threshold lies in this slot
            if (found == INT_MAX && exc < rem && rem <= exc + (double)vs) {
                double c = exc;
                for (int k = 0; k < VEC; ++k) {
                    c += (double)m[k];
                    if (c >= rem && m[k] > 0.f) {
                        found = q * VEC + k;
                        break;
                    }
                }
                if (found == INT_MAX)  // rounding: the vector's last token with mass
                    for (int k = VEC - 1; k >= 0; --k)
                        if (m[k] > 0.f) {
                            found = q * VEC + k;
                            break;
                        }
            }
            rem = -1.0;  // found (or fall back below)
        } else {
            rem -= tot;
        }
        for (int k = 0; k < VEC; ++k)
            if (m[k] > 0.f) last = max(last, q * VEC + k);
    }
    const int f = block_min_int<kTreeWaves>(found, lds_i);
    const int l = block_max_int<kTreeWaves>(last, lds_i);
    return f != INT_MAX ? f : l;
}

// Decision data kept in LDS by thread 0 and read by all threads.
struct TreeShared {
    int32_t par[kMaxK], tok[kMaxK];
    int32_t path[kMaxK], out[kMaxK + 1];
    double wsum[kWaveSteps * kTreeWaves];      // the waves' step sums of a law pass
    double ssum[kMaxTreeSteps];
    int32_t next, err;
};

template <int DT>
__global__ __launch_bounds__(kTreeBlock) void tree_kernel(const TreeArgs t)
{
    __shared__ TreeShared sh;
    __shared__ float lds_f[4 + kTreeWaves * 4];
    __shared__ int lds_i[4 + kTreeWaves * 4];
    __shared__ double lds_d[kTreeWaves];
    const int b = blockIdx.x, N = t.N, V = t.V, tid = threadIdx.x;
    const float T = t.temperature[b];
    const char *tbase = t.target + (int64_t)b * (N + 1) * t.row_bytes;
    const char *dbase = t.draft ? t.draft + (int64_t)b * N * t.row_bytes : nullptr;
    if (tid < N) {
        sh.par[tid] = t.parent[(int64_t)b * N + tid];
        sh.tok[tid] = t.tokens[(int64_t)b * N + tid];
    }
    if (tid == 0) sh.err = 0;
    __syncthreads();
    if (tid == 0) {
        int e = 0;
        for (int i = 0; i < N; ++i)
            if (sh.par[i] < -1 || sh.par[i] >= i) e = SV_ERR_TREE;
        if (!e && !temperature_ok(T)) e = SV_ERR_TEMPERATURE;
        if (!e && T != 0.f && N > 0 && !dbase) e = SV_ERR_NO_DRAFT;
        sh.err = e;
    }
    __syncthreads();
    int fail = sh.err;
    int cur = -1, d = 0, bonus = -1;
    const bool greedy = T == 0.f;
    const ExpScale e = make_scale(greedy ? 1.f : T);
    int tok_err = 0;
    while (!fail) {
        const int ctx = cur + 1;
        const char *trow = tbase + (int64_t)ctx * t.row_bytes;
        // the context's first child (children are the later nodes with this parent)
        int first = -1;
        for (int j = ctx; j < N; ++j)
            if (sh.par[j] == cur) {
                first = j;
                break;
            }
        if (greedy) {
            float best = -INFINITY;
            int bi = INT_MAX;
            row_pass<DT, false>(trow, nullptr, t.nvec, V, [&](TreeTile &tl, int qb) {
                tree_argmax_tile<DT>(tl.t, qb, best, bi);
            });
            block_argmax<kTreeWaves>(best, bi, lds_f, lds_i);
            if (!isfinite(best)) {
                fail = SV_ERR_ROW;
                break;
            }
            int next = -1;
            for (int j = ctx; j < N && next < 0; ++j) {
                if (sh.par[j] != cur) continue;
                const int x = sh.tok[j];
                if (x < 0 || x >= V) tok_err = SV_ERR_TOKEN;
                if (x == bi) next = j;
            }
            if (next < 0) {
                bonus = bi;
                break;
            }
            if (tid == 0) {
                sh.out[d] = bi;
                sh.path[d] = next;
            }
            ++d;
            cur = next;
            continue;
        }
        const char *drow = first >= 0 ? dbase + (int64_t)ctx * t.row_bytes : nullptr;
        // statistics of the context's rows: one pass over both
        RowRun rt, rd;
        run_clear(rt);
        run_clear(rd);
        if (drow) {
            row_pass<DT, true>(trow, drow, t.nvec, V, [&](TreeTile &tl, int) {
                run_sum_tile<DT, kTreeLoads>(tl.t, e, rt);
                run_sum_tile<DT, kTreeLoads>(tl.d, e, rd);
            });
        } else {
            row_pass<DT, false>(trow, nullptr, t.nvec, V, [&](TreeTile &tl, int) {
                run_sum_tile<DT, kTreeLoads>(tl.t, e, rt);
            });
        }
        float Mt, Md = 0.f;
        double St, Sd = 1.0;
        tree_run_finish(rt, e, lds_f, lds_d, Mt, St);
        if (drow) tree_run_finish(rd, e, lds_f, lds_d, Md, Sd);
        if (!isfinite(Mt) || (drow && !isfinite(Md))) {
            fail = SV_ERR_ROW;
            break;
        }
        Law w;
        w.e = e;
        w.ot = row_offset(Mt, e);
        const float od = drow ? row_offset(Md, e) : 0.f;
        // kappa without its log2(A) term: log2(q(v) / p(v)) = (z_d - z_t) c + k0
        const double k0 = drow ? ((double)w.ot - (double)od) + log2(St / Sd) : 0.0;
        double A = 0.0, P = 1.0;  // the current law r = max(p - q A, 0) / P (identical in every thread)
        bool ssum_ready = false;  // ssum[] holds the current law's step masses (total ssum_total)
        double ssum_total = 0.0;
        int next = -1;
        for (int j = ctx; j < N && next < 0; ++j) {
            if (sh.par[j] != cur) continue;
            if (tid == 0) {
                // accept iff u <= r(x) / q(x) = max(p(x)/q(x) - A, 0) / P, in fp64 from the logits
                const int x = sh.tok[j];
                double ratio = 0.0;
                if (x < 0 || x >= V) {
                    sh.err |= SV_ERR_TOKEN;
                } else {
                    const float zt = Elt<DT>::scalar(trow, x), zd = Elt<DT>::scalar(drow, x);
                    if (zd == -INFINITY) {
                        ratio = INFINITY;  // no draft mass: cannot be rejected
                    } else {
                        const double pq = exp2(((double)zt - (double)zd) * e.c64 - k0);
                        ratio = A == 0.0 ? pq : fmax(pq - A, 0.0) / P;
                    }
                }
                const float u = philox_uniform(t.seed, (uint32_t)(t.b0 + b), (uint32_t)j, kPurposeAccept);
                sh.next = (double)u <= ratio ? 1 : 0;
            }
            __syncthreads();
            const bool acc = sh.next != 0;
            __syncthreads();
            if (acc) {
                next = j;
                break;
            }
            // rejected: the residual max(r - q, 0) = max(p - q (A + P), 0) / P, kept per
            // step for the bonus; its pass sums S_t P z, z the residual's mass
            const double A2 = A + P;
            law_kappa(w, k0 + log2(A2));
            const double sw = law_pass<DT, kLawResidual>(trow, drow, t.nvec, V, w, sh.ssum, sh.wsum, lds_d);
            if (sw > 0.0) {
                A = A2;
                P = sw / St;  // P z
                ssum_ready = true;
                ssum_total = sw;
            } else {
                ssum_ready = false;  // no mass: the law stays as it was
            }
        }
        if (next >= 0) {
            if (tid == 0) {
                sh.out[d] = sh.tok[next];
                sh.path[d] = next;
            }
            ++d;
            cur = next;
            continue;
        }
        // no child left: the bonus from the current law
        const float uB = philox_uniform(t.seed, (uint32_t)(t.b0 + b), (uint32_t)d, kPurposeBonus);
        if (A == 0.0) {
            const double tot = law_pass<DT, kLawTarget>(trow, nullptr, t.nvec, V, w, sh.ssum, sh.wsum, lds_d);
            bonus = law_draw<DT, kLawTarget>(trow, nullptr, t.nvec, V, w, sh.ssum, (double)uB * tot, lds_d, lds_i);
        } else {
            law_kappa(w, k0 + log2(A));
            double tot = ssum_total;
            if (!ssum_ready) tot = law_pass<DT, kLawResidual>(trow, drow, t.nvec, V, w, sh.ssum, sh.wsum, lds_d);
            bonus = law_draw<DT, kLawResidual>(trow, drow, t.nvec, V, w, sh.ssum, (double)uB * tot, lds_d, lds_i);
        }
        break;
    }
    __syncthreads();
    const int err = fail | tok_err | sh.err;
    int32_t *out = t.out_tokens + (int64_t)b * (N + 1);
    int32_t *path = t.path + (int64_t)b * N;
    if (fail) {
        for (int j = tid; j <= N; j += kTreeBlock) out[j] = -1;
        for (int j = tid; j < N; j += kTreeBlock) path[j] = -1;
        if (tid == 0) t.accepted_len[b] = 0;
    } else {
        for (int j = tid; j <= N; j += kTreeBlock) out[j] = j < d ? sh.out[j] : j == d ? bonus : -1;
        for (int j = tid; j < N; j += kTreeBlock) path[j] = j < d ? sh.path[j] : -1;
        if (tid == 0) t.accepted_len[b] = d;
    }
    if (err && tid == 0 && t.error_word) atomicOr(t.error_word, err);
}

void launch_tree(const TreeArgs &t, int32_t nb, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    if (t.dtype == SV_F32) {
        if (begin || end)
            hipExtLaunchKernelGGL(tree_kernel<0>, dim3((unsigned)nb), dim3(kTreeBlock), 0, s, begin, end, 0, t);
        else
            tree_kernel<0><<<(unsigned)nb, kTreeBlock, 0, s>>>(t);
    } else {
        if (begin || end)
            hipExtLaunchKernelGGL(tree_kernel<1>, dim3((unsigned)nb), dim3(kTreeBlock), 0, s, begin, end, 0, t);
        else
            tree_kernel<1><<<(unsigned)nb, kTreeBlock, 0, s>>>(t);
    }
}

}  // namespace sv
