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

// Element index of value k of this thread's vector u.
__device__ __forceinline__ int elem_index(int q0, int u, int k, int vec)
{
    return (q0 + u * kBlock + (int)threadIdx.x) * vec + k;
}

// Running statistics of one sampling row: the wave-uniform maximum m and
// this lane's fp64 sum of exp2((z - m) log2e / T).  Keeping m uniform across
// the wave makes the rare rescale when m grows a uniform branch (a per-lane
// maximum diverges on almost every tile and costs ~20% of the streaming rate
// on gfx950).  Each vector's exponentials are added pairwise in fp32 and the
// vector sum in fp64, so equal rows give bitwise-equal sums.
struct RowRun {
    float m;
    double s;
};

__device__ __forceinline__ void run_clear(RowRun &r)
{
    r.m = -INFINITY;
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
        if (run.s != 0.0) run.s *= exp2(((double)run.m - (double)mw) * e.c64);
        run.m = mw;
    }
}

template <int DT, int U>
__device__ __forceinline__ void run_sum_tile(const uint4 (&r)[U], const ExpScale &e, RowRun &run)
{
    constexpr int VEC = Elt<DT>::kVec;
    run_raise(run, wave_max(tile_lane_max<DT, U>(r)), e);
    if (run.m == -INFINITY) return;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], run.m, e);
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run.s += (double)ev[0];
    }
}

// Beta-weighted draft row: as run_sum_tile, and the lane keeps its top-4 by
// (value desc, index asc).  An element entering the lane's top-4 is left out
// of the sum and the element it evicts is added, so the sum covers the
// lane's elements outside its top-4.
template <int DT, int U>
__device__ __forceinline__ void run_sum_top_tile(const uint4 (&r)[U], int q0, int V,
                                                 const ExpScale &e, RowRun &run, Top4 &t4)
{
    constexpr int VEC = Elt<DT>::kVec;
    run_raise(run, wave_max(tile_lane_max<DT, U>(r)), e);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
        float mx = x[0];
#pragma unroll
        for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[k]);
#pragma unroll
        for (int k = 0; k < VEC; ++k) ev[k] = run.m == -INFINITY ? 0.f : exp_scaled(x[k], run.m, e);
        if (mx > t4.v[3] || (mx == t4.v[3] && t4.i[3] == INT_MAX)) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int idx = elem_index(q0, u, k, VEC);
                if (idx < V && better(x[k], idx, t4.v[3], t4.i[3])) {
                    const float out_v = t4.v[3];
                    const int out_i = t4.i[3];
                    top_insert(t4, x[k], idx);
                    ev[k] = (run.m != -INFINITY && out_i != INT_MAX) ? exp_scaled(out_v, run.m, e) : 0.f;
                }
            }
        }
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run.s += (double)ev[0];
    }
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
    const double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2(((double)run.m - (double)M) * e.c64);
    S = block_sum(sc, lds_d);
}

// Weighted draft row chunk: block max M, the chunk's top-4 and the mass
// outside it (lane-top entries that miss the chunk top-4 join the sum).
__device__ __forceinline__ void run_finish_top(const RowRun &run, const Top4 &t4, const ExpScale &e,
                                               float *lds_f, int *lds_i, double *lds_d, float &M,
                                               double &S_excl, Top4 &ct)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    M = block_max(run.m, lds_f);
    double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2(((double)run.m - (double)M) * e.c64);
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
        }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        ct.v[k] = lds_f[k];
        ct.i[k] = lds_i[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (t4.i[k] != INT_MAX && t4.v[k] != -INFINITY && !top_has(ct, t4.i[k]))
            sc += exp2(((double)t4.v[k] - (double)M) * e.c64);
    S_excl = block_sum(sc, lds_d);
}

}  // namespace sv
