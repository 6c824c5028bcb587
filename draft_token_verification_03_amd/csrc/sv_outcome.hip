// sv_outcome.hip -- the verification-outcome distribution of each sampling
// sequence ("Speculative Speculative Decoding", "Method": an outcome of a
// verification is the accepted prefix length together with the bonus
// token's identity, and the speculator prepares next-round drafts for the
// likeliest outcomes; "Key claims": the bonus follows the residual
// max(p_t - p_d, 0)).
//
// Over drafts drawn from the draft law q' that the verify step assumes,
// position j < K accepts with probability alpha_j = sum_v min(p_j, q'_j) and,
// on a rejection, emits v with probability r_j(v) / (1 - alpha_j), where
// r_j = max(p_j - q'_j, 0).  So P(n = k) = (prod_{j<k} alpha_j)(1 - alpha_k),
// P(n = K) = prod_j alpha_j, and the likeliest bonus tokens of position k are
// those of largest r_k (of p_K at k = K).
//
//   1. stats_kernel (the verify step's streaming pass) reads every target and
//      draft row once: row max, sum, and a weighted draft row's top-4.
//   2. outcome_kernel  one workgroup per (sequence, position, chunk): merges
//      the two rows' statistics, then streams both rows' chunk once more.
//      With a = z_t c - o_t and b = z_d c - o_d (offsets of the row maxima),
//      delta = log2(D / S_t) and w the token's beta weight,
//        min(p, q') D = exp2(min(a + delta, b + log2 w)),
//        r D          = exp2(a + delta) - exp2(b + log2 w)  where positive,
//      from the two exponentials of each token pair.  The chunk's best F
//      residuals are kept in LDS slots; a tile takes the exact path only
//      when some lane's r D reaches the slots' floor (or holds one of the
//      draft's beta-weighted top-4 tokens).  Position K keeps the F largest
//      target logits, since p_K ranks as its logits do.
//   3. outcome_finish_kernel  one workgroup per sequence: merges the chunks'
//      sorted lists and sums, and writes alpha, P(n = k) and the masses.
//
// The second read of the rows is inherent: the clamp in r and the order of
// the r values depend on both rows' normalisers, which are only known once
// both rows have been read.
#include <hip/hip_ext.h>

#include "sv_accept.h"
#include "sv_stream.h"
#include "sv_tile.h"

namespace sv {

// ---------------------------------------------------------------------------
// F shared slots of 64-bit keys (top_key order: value, then lower index),
// kept sorted in descending order, 0 = empty.  Every slot only rises, and a
// key enters slot s + 1 only after it was seen below slot s, so slot s >=
// slot s + 1 at every instant.  An insert skips the slots already above its
// key (found by a binary search: a slot read above the key stays above it,
// and by the order so do all slots before it) and walks down the rest with
// atomic maxima, carrying whichever key is displaced; at the end the slots
// hold the F largest keys ever inserted, under any interleaving.

__device__ __forceinline__ uint64_t slot_read(const uint64_t *s)
{
    return __hip_atomic_load(s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void slots_insert_f(uint64_t *slots, int F, uint64_t key)
{
    int lo = 0, hi = F;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (slot_read(&slots[mid]) > key) lo = mid + 1;
        else hi = mid;
    }
    for (int s = lo; s < F; ++s) {
        const uint64_t old = atomicMax((unsigned long long *)&slots[s], (unsigned long long)key);
        if (old < key) {
            if (old == 0) return;  // it took an empty slot: nothing was displaced
            key = old;
        }
    }
}

// The k-th largest (k in [1, 64]) of the lanes' values: a bitonic sort of the
// wave into descending lane order.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t wave_kth_largest(uint32_t x, int k)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int kk = 2; kk <= 64; kk <<= 1)
#pragma unroll
        for (int j = kk >> 1; j > 0; j >>= 1) {
            const uint32_t y = (uint32_t)__shfl_xor((int)x, j);
            const bool take_max = ((lane & j) == 0) == ((lane & kk) == 0);
            x = take_max ? max(x, y) : min(x, y);
        }
    return (uint32_t)__shfl((int)x, k - 1);
}

// A tile's candidates (keys above the slots' floor) are inserted one by one
// when the wave has a few.  When it has many (the first tiles of a chunk,
// rising rows) only those whose value reaches the F-th largest of the lanes'
// best candidates are: that value is at most the F-th best of the wave's
// tile, and any key below it has F better keys that are inserted, so it
// cannot be among the chunk's best F.

// Per-position constants, the same in every lane.
struct PosConst {
    ExpScale e;
    float ot, od;     // offsets of the target and draft row maxima
    float nad;        // fp32(delta - o_t), delta = log2(D / S_t): a + delta in one fma
    float lbeta;      // log2(beta) (-inf for beta == 0)
    float z4;         // a weighted draft row's 4th largest logit
    Top4 top;         // and its top-4
    int F;
};

// Position j < K: sum of min(p, q') D over the tile into `run`, candidates
// into the slots.  The fast path forms min(p, q') D and the unweighted r D of
// every token pair; a lane is flagged when its largest r D reaches the
// floor's value, or when it holds a logit at or above the draft's 4th
// largest (a token of the weighted top-4 has its weight applied on the
// exact path).  The exact path keys every token whose p D reaches the floor.
template <int DT, bool TOP>
__device__ __forceinline__ void pair_tile(const PairTile &tl, int qb, int V, const PosConst &pc,
                                          uint64_t *slots, double &run, double &tmass)
{
    constexpr int VEC = Elt<DT>::kVec;
    const uint64_t fkey = pc.F ? slot_read(&slots[pc.F - 1]) : 0;
    // a key above the floor needs r D > floor, hence p D = exp2(a + delta) > floor
    const float lf = pc.F == 0 ? INFINITY
                     : fkey == 0 ? -INFINITY
                                 : __builtin_amdgcn_logf(key_value(fkey)) - 0x1p-10f;
    float amax = -INFINITY, dmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC], y[VEC], ev[VEC];
        Elt<DT>::unpack(tl.t[u], x);
        Elt<DT>::unpack(tl.d[u], y);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float A = __builtin_fmaf(x[k], pc.e.c, pc.nad);
            const float B = __builtin_fmaf(y[k], pc.e.c, -pc.od);
            const float ea = __builtin_amdgcn_exp2f(A), eb = __builtin_amdgcn_exp2f(B);
            ev[k] = fminf(ea, eb);
            amax = fmaxf(amax, ea - eb);
            if (TOP) dmax = fmaxf(dmax, y[k]);
        }
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run += (double)ev[0];
    }
    const float fv = pc.F == 0 ? INFINITY : key_value(fkey);
    const bool flag = (amax > 0.f && amax >= fv) || (TOP && dmax >= pc.z4);
    if (__ballot(flag) == 0ull) return;

    uint64_t lmax = 0;
    int ncand = 0;
    double corr = 0.0;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC], y[VEC];
        Elt<DT>::unpack(tl.t[u], x);
        Elt<DT>::unpack(tl.d[u], y);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int idx = elem_index(qb, u, k, VEC);
            const float A = __builtin_fmaf(x[k], pc.e.c, pc.nad);
            const float B = __builtin_fmaf(y[k], pc.e.c, -pc.od);
            const bool mem = TOP && y[k] >= pc.z4 && top_has(pc.top, idx);
            if (mem) {  // replace the unweighted term summed above by the weighted one
                const float ea = __builtin_amdgcn_exp2f(A), ew = __builtin_amdgcn_exp2f(B + pc.lbeta);
                corr += (double)fminf(ea, ew) - (double)fminf(ea, __builtin_amdgcn_exp2f(B));
                tmass += (double)fmaxf(ea - ew, 0.f);  // r D of a top-4 token
            }
            if (A != -INFINITY && A >= lf) {
                const float rD = __builtin_amdgcn_exp2f(A) - __builtin_amdgcn_exp2f(mem ? B + pc.lbeta : B);
                if (rD > 0.f) {
                    const uint64_t key = top_key(rD, idx);
                    if (key > fkey) {
                        ++ncand;
                        lmax = max(lmax, key);
                    }
                }
            }
        }
    }
    run += corr;
    const int total = wave_sum_int(ncand);
    if (total == 0) return;
    const uint32_t thr = total > kSerialCandidates ? wave_kth_largest((uint32_t)(lmax >> 32), pc.F) : 0u;
    if (ncand == 0) return;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC], y[VEC];
        Elt<DT>::unpack(tl.t[u], x);
        Elt<DT>::unpack(tl.d[u], y);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const float A = __builtin_fmaf(x[k], pc.e.c, pc.nad);
            if (!(A != -INFINITY && A >= lf)) continue;
            const int idx = elem_index(qb, u, k, VEC);
            const float B = __builtin_fmaf(y[k], pc.e.c, -pc.od);
            const bool mem = TOP && y[k] >= pc.z4 && top_has(pc.top, idx);
            const float rD = __builtin_amdgcn_exp2f(A) - __builtin_amdgcn_exp2f(mem ? B + pc.lbeta : B);
            if (!(rD > 0.f)) continue;
            const uint64_t key = top_key(rD, idx);
            if (key > fkey && (uint32_t)(key >> 32) >= thr) slots_insert_f(slots, pc.F, key);
        }
    }
}

// Position K: the F largest finite target logits into the slots.
template <int DT>
__device__ __forceinline__ void last_tile(const PairTile &tl, int qb, int F, uint64_t *slots)
{
    constexpr int VEC = Elt<DT>::kVec;
    const uint64_t fkey = slot_read(&slots[F - 1]);
    const float fv = key_value(fkey);
    const int fi = key_index(fkey);
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC];
        Elt<DT>::unpack(tl.t[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) mx = fmaxf(mx, x[k]);
    }
    // the lane's first token of the tile is its lowest
    const bool maybe = mx != -INFINITY && (mx > fv || (mx == fv && elem_index(qb, 0, 0, VEC) < fi));
    if (__ballot(maybe) == 0ull) return;
    uint64_t lmax = 0;
    int ncand = 0;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC];
        Elt<DT>::unpack(tl.t[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            if (x[k] == -INFINITY) continue;
            const uint64_t key = top_key(x[k], elem_index(qb, u, k, VEC));
            if (key > fkey) {
                ++ncand;
                lmax = max(lmax, key);
            }
        }
    }
    const int total = wave_sum_int(ncand);
    if (total == 0) return;
    const uint32_t thr = total > kSerialCandidates ? wave_kth_largest((uint32_t)(lmax >> 32), F) : 0u;
    if (ncand == 0) return;
#pragma unroll
    for (int u = 0; u < kOutLoads; ++u) {
        float x[VEC];
        Elt<DT>::unpack(tl.t[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            if (x[k] == -INFINITY) continue;
            const uint64_t key = top_key(x[k], elem_index(qb, u, k, VEC));
            if (key > fkey && (uint32_t)(key >> 32) >= thr) slots_insert_f(slots, F, key);
        }
    }
}

// ---------------------------------------------------------------------------
// 2. The outcome pass.

struct PosStats {
    float mt, md;
    double St, D;
    Top4 top;
};

template <int DT, bool TOP, bool ALIGNED>
__device__ __forceinline__ void outcome_position(const OutArgs &o, const char *trow, const char *drow,
                                                 int b, int j, int chunk, float T)
{
    const Args &a = o.a;
    const int K = a.K;
    const bool pair = j < K;
    __shared__ uint64_t slots[kMaxOutcomeF];
    __shared__ PosStats ps;
    __shared__ double lds_d[kWaves];
    const int q0 = chunk * o.cvec2;
    const int q1 = min(a.nvec, q0 + o.cvec2);
    const int F = o.F;
    PairTile ra;
    // the first tile is requested before the statistics are merged
    if (pair) issue_pair<DT, ALIGNED, true>(trow, drow, q0, q1, a.V, ra);
    else if (F > 0) issue_pair<DT, ALIGNED, false>(trow, nullptr, q0, q1, a.V, ra);

    const ExpScale e = make_scale(T);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid < F) slots[tid] = 0;
    if (wave == 0) {
        float M;
        double S;
        merge_sum(a.part + ((int64_t)b * a.R + j) * a.nc, a.nc, e, M, S);
        if (lane == 0) {
            ps.mt = M;
            ps.St = S;
        }
    } else if (wave == 1 && pair) {
        const RowPart *p = a.part + ((int64_t)b * a.R + K + 1 + j) * a.nc;
        const Top4 *tp = a.top + ((int64_t)b * K + j) * a.nc;
        float M;
        double D;
        Top4 t;
        top_clear(t);
        if (TOP && a.nc > 1) {
            double Du;
            merge_weighted(p, tp, a.nc, e, (double)a.beta, M, t, D, Du);
        } else {
            merge_sum(p, a.nc, e, M, D);  // one chunk: the streaming pass formed D
            if (TOP) t = tp[0];
        }
        if (lane == 0) {
            ps.md = M;
            ps.D = D;
            ps.top = t;
        }
    }
    __syncthreads();
    const float mt = ps.mt;
    const double St = ps.St;
    int status = isfinite(mt) ? 0 : SV_ERR_ROW;
    float md = 0.f;
    double D = 0.0;
    if (pair) {
        md = ps.md;
        D = ps.D;
        if (!isfinite(md)) status |= SV_ERR_ROW;
        else if (!(D > 0.0)) status |= SV_ERR_DRAFT_MASS;
    }
    const int64_t posi = (int64_t)b * (K + 1) + j;
    if (chunk == 0 && tid == 0) {
        OutRow rr;
        rr.norm = pair ? D : St;
        rr.o = isfinite(mt) ? row_offset(mt, e) : 0.f;
        rr.status = status;
        o.rec[posi] = rr;
    }
    if (status || (!pair && F == 0)) return;

    uint64_t *keys = o.keys + (posi * o.nc2 + chunk) * F;
    if (pair) {
        PosConst pc;
        pc.e = e;
        pc.ot = row_offset(mt, e);
        pc.od = row_offset(md, e);
        pc.nad = (float)((log2(D) - log2(St)) - (double)pc.ot);
        pc.lbeta = (float)a.log2_beta;
        pc.top = ps.top;
        pc.z4 = TOP ? pc.top.v[3] : INFINITY;
        pc.F = F;
        double run = 0.0, tmass = 0.0;
        stream_pair<DT, ALIGNED, true>(trow, drow, q0, q1, a.V, ra, [&](PairTile &t, int qb) {
            pair_tile<DT, TOP>(t, qb, a.V, pc, slots, run, tmass);
        });
        const double s = block_sum(run, lds_d);  // its barrier orders every insert before the reads
        if (tid == 0) o.asum[posi * o.nc2 + chunk] = s;
        if (TOP) {
            __syncthreads();  // lds_d is reused
            const double tsum = block_sum(tmass, lds_d);
            if (tid == 0) o.tsum[posi * o.nc2 + chunk] = tsum;
        }
    } else {
        stream_pair<DT, ALIGNED, false>(trow, nullptr, q0, q1, a.V, ra, [&](PairTile &t, int qb) {
            last_tile<DT>(t, qb, F, slots);
        });
        __syncthreads();
    }
    if (tid < F) keys[tid] = slots[tid];
}

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void outcome_kernel(const OutArgs o)
{
    const Args &a = o.a;
    const int chunk = blockIdx.x % o.nc2;
    const int pos = blockIdx.x / o.nc2;
    const int b = pos / (a.K + 1);
    const int j = pos - b * (a.K + 1);
    const float T = a.temperature[b];
    // greedy sequences, invalid temperatures and missing draft logits: the
    // finishing kernel fills the outputs
    if (!temperature_ok(T) || T == 0.f || (a.K > 0 && !a.draft)) return;
    const char *trow = a.target + ((int64_t)b * (a.K + 1) + j) * a.row_bytes;
    const char *drow = j < a.K ? a.draft + ((int64_t)b * a.K + j) * a.row_bytes : nullptr;
    const bool aligned = ((uintptr_t)trow & 15) == 0 && (!drow || ((uintptr_t)drow & 15) == 0);
    if (aligned) outcome_position<DT, TOP, true>(o, trow, drow, b, j, chunk, T);
    else outcome_position<DT, TOP, false>(o, trow, drow, b, j, chunk, T);
}

// ---------------------------------------------------------------------------
// 3. Per sequence: alpha_j = (sum of the chunks' sums) / D, P(n = k), and the
// best F keys of each position from the chunks' sorted lists (one list: read
// as it is; several: a merge in which each lane follows the heads of its
// chunks' lists and the wave takes the largest head F times).  Keys of one
// position are distinct (they carry the token).

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)dpp_int<CTRL>((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)dpp_int<CTRL>((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int SPAN>
__device__ __forceinline__ uint64_t swap_max_u64(uint64_t v)
{
    const IntPair lo = swap_halves<SPAN>((int)(uint32_t)v);
    const IntPair hi = swap_halves<SPAN>((int)(uint32_t)(v >> 32));
    const uint64_t a = ((uint64_t)(uint32_t)hi.a << 32) | (uint32_t)lo.a;
    const uint64_t b = ((uint64_t)(uint32_t)hi.b << 32) | (uint32_t)lo.b;
    return a > b ? a : b;
}

// Wave maximum of 64-bit keys with the DPP and permlane butterflies of the
// float reductions (every lane gets it).  All 64 lanes must be active.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v)
{
    uint64_t w = dpp_u64<kDppQuadXor1>(v);
    v = w > v ? w : v;
    w = dpp_u64<kDppQuadXor2>(v);
    v = w > v ? w : v;
    w = dpp_u64<kDppRowHalfMirror>(v);
    v = w > v ? w : v;
    w = dpp_u64<kDppRowMirror>(v);
    v = w > v ? w : v;
    v = swap_max_u64<16>(v);
    return swap_max_u64<32>(v);
}

// Ranked slot f of position j from key `best` (0: none): the token and its
// mass, r D / D for j < K, exp2(z c - o_t) / S_t for j = K.
__device__ __forceinline__ void write_slot(const OutRow &rr, int j, int K, int f, int F, uint64_t best,
                                           const ExpScale &e, int32_t *tt, float *tm)
{
    int tok = -1;
    float mass = 0.f;
    if (best != 0) {
        tok = key_index(best);
        const double v = (double)key_value(best);
        mass = j < K ? (float)(v / rr.norm) : (float)(exp2(v * e.c64 - (double)rr.o) / rr.norm);
    }
    tt[j * F + f] = tok;
    tm[j * F + f] = mass;
}

__global__ __launch_bounds__(kBlock) void outcome_finish_kernel(const OutArgs o)
{
    const Args &a = o.a;
    const int b = blockIdx.x, K = a.K, F = o.F, P = K + 1;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ int err_s;
    __shared__ double alpha_s[kMaxK];
    float *ar = o.accept_rate + (int64_t)b * K;
    float *pl = o.p_len + (int64_t)b * P;
    int32_t *tt = o.top_tokens + (int64_t)b * P * F;
    float *tm = o.top_mass + (int64_t)b * P * F;
    const float T = a.temperature[b];
    int err = 0;
    bool none = false;
    if (!temperature_ok(T)) err = SV_ERR_TEMPERATURE;
    else if (T == 0.f) none = true;  // greedy: the drafts fix the outcome
    else if (K > 0 && !a.draft) err = SV_ERR_NO_DRAFT;
    if (!err && !none) {
        if (tid == 0) err_s = 0;
        __syncthreads();
        for (int j = tid; j < P; j += kBlock) {
            const int st = o.rec[(int64_t)b * P + j].status;
            if (st) atomicOr(&err_s, st);
        }
        __syncthreads();
        err = err_s;
    }
    if (err || none) {
        if (err && tid == 0 && a.error_word) atomicOr(a.error_word, err);
        for (int j = tid; j < K; j += kBlock) {
            ar[j] = NAN;
            if (o.draft_top_mass) o.draft_top_mass[(int64_t)b * K + j] = NAN;
        }
        for (int j = tid; j < P; j += kBlock) pl[j] = NAN;
        for (int j = tid; j < P * F; j += kBlock) {
            tt[j] = -1;
            tm[j] = 0.f;
        }
        return;
    }
    const ExpScale e = make_scale(T);
    for (int j = wave; j < P; j += kWaves) {
        const OutRow rr = o.rec[(int64_t)b * P + j];
        const int64_t base = ((int64_t)b * P + j) * o.nc2;
        if (j < K) {
            double s = 0.0;
            for (int c = lane; c < o.nc2; c += 64) s += o.asum[base + c];
            s = wave_sum(s);
            if (lane == 0) alpha_s[j] = fmin(fmax(s / rr.norm, 0.0), 1.0);
            if (o.draft_top_mass) {
                double t = 0.0;
                for (int c = lane; c < o.nc2; c += 64) t += o.tsum[base + c];
                t = wave_sum(t);
                if (lane == 0) o.draft_top_mass[(int64_t)b * K + j] = (float)(t / rr.norm);
            }
        }
        if (o.nc2 == 1) {  // one sorted list: lane f holds slot f
            const uint64_t *k0 = o.keys + base * F;
            for (int f = lane; f < F; f += 64) write_slot(rr, j, K, f, F, k0[f], e, tt, tm);
            continue;
        }
        // several lists: each lane follows the heads of its chunks' sorted lists
        const bool own0 = lane < o.nc2, own1 = lane + 64 < o.nc2;
        const uint64_t *k0 = o.keys + (base + lane) * F;
        const uint64_t *k1 = o.keys + (base + lane + 64) * F;
        int h0 = 0, h1 = 0;
        for (int f = 0; f < F; ++f) {
            const uint64_t c0 = (own0 && h0 < F) ? k0[h0] : 0;
            const uint64_t c1 = (own1 && h1 < F) ? k1[h1] : 0;
            const uint64_t mine = c0 > c1 ? c0 : c1;
            const uint64_t best = wave_max_u64(mine);
            if (best != 0 && mine == best) {
                if (c0 == best) ++h0;
                else ++h1;
            }
            if (lane == 0) write_slot(rr, j, K, f, F, best, e, tt, tm);
        }
    }
    __syncthreads();
    if (tid == 0) {
        double reach = 1.0;  // prod_{j<k} alpha_j
        for (int k = 0; k < K; ++k) {
            const double al = alpha_s[k];
            ar[k] = (float)al;
            pl[k] = (float)(reach * (1.0 - al));
            reach *= al;
        }
        pl[K] = (float)reach;
    }
}

// ---------------------------------------------------------------------------
// Host launcher of one sub-batch: streaming pass, outcome pass (events, if
// given, stamped by its dispatch), finish.

template <int DT, bool TOP>
static void launch_out(const OutArgs &o, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    launch_stats(o.a, s);
    const unsigned grid = (unsigned)((int64_t)o.a.B * (o.a.K + 1) * o.nc2);
    if (begin || end)
        hipExtLaunchKernelGGL(outcome_kernel<DT, TOP>, dim3(grid), dim3(kBlock), 0, s, begin, end, 0, o);
    else
        outcome_kernel<DT, TOP><<<grid, kBlock, 0, s>>>(o);
    outcome_finish_kernel<<<(unsigned)o.a.B, kBlock, 0, s>>>(o);
}

void launch_outcomes(const OutArgs &o, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    if (o.a.dtype == SV_F32) {
        if (o.a.weighted) launch_out<0, true>(o, s, begin, end);
        else launch_out<0, false>(o, s, begin, end);
    } else {
        if (o.a.weighted) launch_out<1, true>(o, s, begin, end);
        else launch_out<1, false>(o, s, begin, end);
    }
}

}  // namespace sv
