// sv_tile.h -- per-thread reductions of the streaming pass, shared by the
// two-launch and the four-launch paths.
//
// A tile is U 16-byte vectors per thread: vector u of thread t is row vector
// q0 + u * kBlock + t, so element k of it is token (q0 + u*kBlock + t)*VEC + k
// and every lane visits its tokens in increasing order.  Raw vectors hold -inf
// for tokens at or beyond V (the loaders mask them).
#pragma once

#include "sv_internal.h"

namespace sv {

// Raw vectors of -inf, and masking of the elements of a raw vector from
// `keep` on (the tail of a row whose length is not a multiple of VEC).
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

// Element k (run-time index) of a raw vector.
template <int DT>
__device__ __forceinline__ float elt_of(uint4 r, int k)
{
    if (DT == 0) return __uint_as_float(word_of(r, k));
    const uint32_t w = word_of(r, k >> 1);
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Element index of value k of this thread's vector u.
__device__ __forceinline__ int elem_index(int q0, int u, int k, int vec)
{
    return (q0 + u * kBlock + (int)threadIdx.x) * vec + k;
}

// Running statistics of one sampling row: the wave-uniform maximum m, its
// offset o = fp32(m c), and this lane's fp64 sum of exp2(z c - o).  Keeping m
// uniform across the wave makes the rare rescale when m grows a uniform branch
// (a per-lane maximum diverges on almost every tile and costs ~20% of the
// streaming rate on gfx950), and the cross-lane maximum is only formed when
// some lane's tile maximum exceeds m.  Each vector's exponentials are added
// pairwise in fp32 and the vector sum in fp64, so equal rows give
// bitwise-equal sums.
struct RowRun {
    float m, o;
    double s;
};

__device__ __forceinline__ void run_clear(RowRun &r)
{
    r.m = -INFINITY;
    r.o = -INFINITY;
    r.s = 0.0;
}

template <int DT, int U>
__device__ __forceinline__ float tile_lane_max(const uint4 (&r)[U])
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
    return mx;
}

__device__ __forceinline__ void run_raise(RowRun &run, float mw, const ExpScale &e)
{
    if (mw > run.m) {
        const float o = row_offset(mw, e);
        if (run.s != 0.0) run.s *= exp2((double)run.o - (double)o);
        run.m = mw;
        run.o = o;
    }
}

// Raise the running maximum to the wave's maximum of the lanes' tile maxima
// `lm`, reducing across lanes only when some lane exceeds it (a uniform test).
__device__ __forceinline__ void run_raise_lazy(RowRun &run, float lm, const ExpScale &e)
{
    if (__ballot(lm > run.m) != 0ull) run_raise(run, wave_max(lm), e);
}

template <int DT, int U>
__device__ __forceinline__ void run_sum_tile(const uint4 (&r)[U], const ExpScale &e, RowRun &run)
{
    constexpr int VEC = Elt<DT>::kVec;
    run_raise_lazy(run, tile_lane_max<DT, U>(r), e);
    if (run.m == -INFINITY) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], run.o, e);
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run.s += (double)ev[0];
    }
}

// Beta-weighted draft row: as run_sum_tile, and the wave keeps the top-4 W of
// the elements it has seen, by (value desc, index asc), identical in every
// lane; the lanes' sums cover the wave's elements outside W.  W's 4th entry
// is a threshold no later element reaches in most tiles (after t tiles a new
// tile holds a candidate with probability ~4/t), so most tiles take the plain
// sum.  A tile with a few candidates inserts them one at a time, in a
// wave-uniform loop; the first tile, or one with many candidates (rising
// rows), merges per-lane lists instead.  Whatever drops out of W, or never
// enters it, joins lane 0's sum.

__device__ __forceinline__ bool top_insert_out(Top4 &t, float v, int i, float &out_v, int &out_i)
{
    if (!better(v, i, t.v[3], t.i[3])) return false;
    out_v = t.v[3];
    out_i = t.i[3];
    top_insert(t, v, i);
    return true;
}

constexpr int kSerialCandidates = 16;

template <int DT, int U>
__device__ __forceinline__ void run_sum_top_tile(const uint4 (&r)[U], int q0, int V,
                                                 const ExpScale &e, RowRun &run, Top4 &W)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int lane = threadIdx.x & 63;
    const float mx = tile_lane_max<DT, U>(r);
    run_raise_lazy(run, mx, e);
    const bool have_m = run.m != -INFINITY;
    const float thr_v = W.v[3];
    const int thr_i = W.i[3];
    if (__ballot(mx >= thr_v) == 0ull) {  // no element can enter W
        if (!have_m) return;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC], ev[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], run.o, e);
#pragma unroll
            for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
            run.s += (double)ev[0];
        }
        return;
    }
    // candidates: elements that beat W's 4th entry; the others join the sum
    uint32_t cmask = 0;  // bit u * VEC + k
    int ncand = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int idx = elem_index(q0, u, k, VEC);
            const bool c = idx < V && better(x[k], idx, thr_v, thr_i);
            cmask |= (c ? 1u : 0u) << (u * VEC + k);
            ncand += c ? 1 : 0;
            ev[k] = (c || !have_m) ? 0.f : exp_scaled(x[k], run.o, e);
        }
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run.s += (double)ev[0];
    }
    double lost = 0.0;  // mass of candidates that end outside W
    if (W.i[3] != INT_MAX && wave_sum_int(ncand) <= kSerialCandidates) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                uint64_t bits = __ballot((cmask >> (u * VEC + k)) & 1u);
                while (bits) {
                    const int src = __ffsll((unsigned long long)bits) - 1;
                    bits &= bits - 1;
                    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k]), src));
                    const int idx = __builtin_amdgcn_readlane(elem_index(q0, u, k, VEC), src);
                    float ov = v;
                    int oi = idx;
                    top_insert_out(W, v, idx, ov, oi);  // on insertion (ov, oi) is the evicted entry
                    if (lane == 0 && oi != INT_MAX && ov != -INFINITY && have_m)
                        lost += (double)exp_scaled(ov, run.o, e);
                }
            }
        }
    } else {
        // per-lane lists of the candidates (lane 0 also holds W), then the
        // wave's top-4 of all of them
        Top4 t;
        top_clear(t);
        if (lane == 0) t = W;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (!((cmask >> (u * VEC + k)) & 1u)) continue;
                float ov = x[k];
                int oi = elem_index(q0, u, k, VEC);
                top_insert_out(t, x[k], oi, ov, oi);
                if (oi != INT_MAX && ov != -INFINITY && have_m) lost += (double)exp_scaled(ov, run.o, e);
            }
        }
        const Top4 nw = wave_top4(t);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (t.i[k] != INT_MAX && t.v[k] != -INFINITY && !top_has(nw, t.i[k]) && have_m)
                lost += (double)exp_scaled(t.v[k], run.o, e);
        W = nw;
    }
    run.s += lost;
}

// Greedy row: the lane's (max, lowest index).
template <int DT, int U>
__device__ __forceinline__ void run_argmax_tile(const uint4 (&r)[U], int q0, float &best, int &bi)
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

// ---------------------------------------------------------------------------
// Workgroup merges at the end of a chunk.  lds_f/lds_i hold 4 + 4*kWaves
// entries, lds_d kWaves.

// (block max M, fp64 sum of exp2((z - M) c)) of a sampling row chunk.
__device__ __forceinline__ void run_finish(const RowRun &run, const ExpScale &e, float *lds_f,
                                           double *lds_d, float &M, double &S)
{
    M = block_max(run.m, lds_f);
    const double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - (double)row_offset(M, e));
    S = block_sum(sc, lds_d);
}

// Weighted draft row chunk: block max M, the chunk's top-4 and the mass
// outside it (entries of the waves' top-4 lists that miss the chunk top-4
// join the sum).
__device__ __forceinline__ void run_finish_top(const RowRun &run, const Top4 &W, const ExpScale &e,
                                               float *lds_f, int *lds_i, double *lds_d, float &M,
                                               double &S_excl, Top4 &ct)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    M = block_max(run.m, lds_f);
    const double oM = (double)row_offset(M, e);
    double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - oM);
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            lds_f[4 + wave * 4 + k] = W.v[k];
            lds_i[4 + wave * 4 + k] = W.i[k];
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
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ct.v[k] = lds_f[k];
        ct.i[k] = lds_i[k];
    }
    __syncthreads();
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (W.i[k] != INT_MAX && W.v[k] != -INFINITY && !top_has(ct, W.i[k]))
                sc += exp_scaled64(W.v[k], oM, e.c64);
    }
    S_excl = block_sum(sc, lds_d);
}

}  // namespace sv
