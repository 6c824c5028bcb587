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

// Beta-weighted draft row: as run_sum_tile, and each wave keeps the top-4
// of the elements it has seen, by (value desc, index asc), in a list that
// every lane holds alike, out of its sums; at the end of the chunk the four
// waves' lists give the chunk's top-4 and their other entries join the sum
// (run_finish_top).  The 4th entry is a floor that most later tiles do not
// reach (after t tiles, a wave's next tile holds a new entry with probability
// ~4/t), so most tiles take the plain sum.  Elements that beat the floor
// when their tile arrives are inserted one at a time -- lanes in order, each
// lane's in token order -- or, when a tile holds many (the first tile,
// rising rows), through per-lane lists and the wave's top-4 of them.  An
// entry pushed out of the list, or a candidate that no longer makes it, has
// its mass added by a lane that the wave's own data fixes.  Every element
// thus reaches the sum, or the chunk's top-4, along a path and in an order
// that do not depend on how the waves are timed against each other: a call
// gives the same bits every time.

// Key of (v, i), i in [0, INT_MAX): larger keys are better entries; -0 counts
// as +0, as in `better`.  Key 0 is an empty slot.  (Used by the outcome pass.)
__device__ __forceinline__ uint64_t top_key(float v, int i)
{
    uint32_t b = __float_as_uint(v + 0.0f);
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)(0x7fffffff - i);
}

__device__ __forceinline__ float key_value(uint64_t k)
{
    if (k == 0) return -INFINITY;
    uint32_t b = (uint32_t)(k >> 32);
    b = (b & 0x80000000u) ? (b & 0x7fffffffu) : ~b;
    return __uint_as_float(b);
}

__device__ __forceinline__ int key_index(uint64_t k)
{
    return k == 0 ? INT_MAX : 0x7fffffff - (int)(uint32_t)k;
}

__device__ __forceinline__ bool top_insert_out(Top4 &t, float v, int i, float &out_v, int &out_i)
{
    if (!better(v, i, t.v[3], t.i[3])) return false;
    out_v = t.v[3];
    out_i = t.i[3];
    top_insert(t, v, i);
    return true;
}

constexpr int kSerialCandidates = 16;

// A wave's top-4 list, alike in every lane: four keys (top_key order: value,
// then lower index; 0 = empty, below every element's key), k0 the best, as
// scalars of one type so that the list stays in registers.
struct WaveTop {
    uint64_t k0, k1, k2, k3;
};

__device__ __forceinline__ void wtop_clear(WaveTop &w) { w.k0 = w.k1 = w.k2 = w.k3 = 0; }

// Insert key k; returns the key that leaves the list (k itself when it does
// not enter; 0 for an empty slot).  Branch-free: the list is sorted, so
// beating slot j implies beating every later one, and each slot keeps its
// key, takes k or takes the key above it.
__device__ __forceinline__ uint64_t wtop_insert(WaveTop &w, uint64_t k)
{
    const bool b3 = k > w.k3, b2 = k > w.k2, b1 = k > w.k1, b0 = k > w.k0;
    const uint64_t out = b3 ? w.k3 : k;
    const uint64_t n3 = !b3 ? w.k3 : !b2 ? k : w.k2;
    const uint64_t n2 = !b2 ? w.k2 : !b1 ? k : w.k1;
    const uint64_t n1 = !b1 ? w.k1 : !b0 ? k : w.k0;
    const uint64_t n0 = !b0 ? w.k0 : k;
    w.k0 = n0;
    w.k1 = n1;
    w.k2 = n2;
    w.k3 = n3;
    return out;
}

__device__ __forceinline__ bool wtop_has(const WaveTop &w, uint64_t k)
{
    return k != 0 && (w.k0 == k || w.k1 == k || w.k2 == k || w.k3 == k);
}

// One round of the wave merge: the best head of the lanes' lists (every
// lane gets it), popped from the list that holds it.
__device__ __forceinline__ uint64_t wtop_pop_best(WaveTop &t)
{
    // keys order as (value desc, index asc) pairs do: the wave argmax of the
    // decoded heads (DPP butterflies) finds the best key
    float v = key_value(t.k0);
    int i = key_index(t.k0);
    wave_argmax(v, i);
    const uint64_t best = i == INT_MAX ? 0 : top_key(v, i);
    if (best != 0 && t.k0 == best) {
        t.k0 = t.k1;
        t.k1 = t.k2;
        t.k2 = t.k3;
        t.k3 = 0;
    }
    return best;
}

// The wave's top-4 of the lanes' lists (every lane gets it).
__device__ __forceinline__ WaveTop wtop_wave_merge(WaveTop t)
{
    WaveTop out;
    out.k0 = wtop_pop_best(t);
    out.k1 = wtop_pop_best(t);
    out.k2 = wtop_pop_best(t);
    out.k3 = wtop_pop_best(t);
    return out;
}

// The floor a tile's elements must beat: the wave's 4th key, or the block's
// floor from the last exchange of the waves' lists when that is higher (an
// element below the block's 4th best of what all waves had seen then cannot
// be in the chunk's top-4).
template <int DT, int U>
__device__ __forceinline__ void run_sum_top_tile(const uint4 (&r)[U], int q0, int V,
                                                 const ExpScale &e, RowRun &run, WaveTop &wt,
                                                 uint64_t block_floor)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int lane = threadIdx.x & 63;
    const uint64_t floor_key = wt.k3 > block_floor ? wt.k3 : block_floor;
    const float fv = key_value(floor_key);
    const int fi = key_index(floor_key);
    const float mx = tile_lane_max<DT, U>(r);
    run_raise_lazy(run, mx, e);
    const bool have_m = run.m != -INFINITY;
    // the lane's first token of the tile is its lowest
    const bool maybe = mx > fv || (mx == fv && elem_index(q0, 0, 0, VEC) < fi);
    if (__ballot(maybe) == 0ull) {  // no element can enter the list
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
    // candidates: elements that beat the floor; the others join the sum
    uint32_t cmask = 0;  // bit u * VEC + k
    int ncand = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int idx = elem_index(q0, u, k, VEC);
            const bool c = idx < V && better(x[k], idx, fv, fi);
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
    double lost = 0.0;  // masses leaving the list that this lane adds
    if (wave_sum_int(ncand) <= kSerialCandidates) {
        // one candidate at a time, in a fixed order: element position of the
        // tile, then lane (the lists and every mass that leaves them are
        // alike in every lane; lane 0 adds those masses)
        double ulost = 0.0;
        const int wbase = (int)threadIdx.x & ~63;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (__ballot((cmask >> (u * VEC)) & ((1u << VEC) - 1u)) == 0ull) continue;
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                uint64_t m = __ballot((cmask >> (u * VEC + k)) & 1u);
                while (m != 0ull) {
                    const int L = __ffsll((unsigned long long)m) - 1;
                    m &= m - 1ull;
                    const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k]), L));
                    const int i = (q0 + u * kBlock + wbase + L) * VEC + k;
                    const uint64_t out = wtop_insert(wt, top_key(v, i));
                    if (out != 0 && have_m) ulost += (double)exp_scaled(key_value(out), run.o, e);
                }
            }
        }
        if (lane == 0) lost += ulost;
    } else {
        // many: each lane's candidates into its own list in token order, the
        // wave's top-4 of those lists merged with the wave list
        WaveTop t;
        wtop_clear(t);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[VEC];
            Elt<DT>::unpack(r[u], x);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                if (!((cmask >> (u * VEC + k)) & 1u)) continue;
                const uint64_t out = wtop_insert(t, top_key(x[k], elem_index(q0, u, k, VEC)));
                if (out != 0 && have_m) lost += (double)exp_scaled(key_value(out), run.o, e);
            }
        }
        const WaveTop nw = wtop_wave_merge(t);
        WaveTop m = wt;
        wtop_insert(m, nw.k0);
        wtop_insert(m, nw.k1);
        wtop_insert(m, nw.k2);
        wtop_insert(m, nw.k3);
        if (have_m) {
            if (t.k0 != 0 && !wtop_has(m, t.k0)) lost += (double)exp_scaled(key_value(t.k0), run.o, e);
            if (t.k1 != 0 && !wtop_has(m, t.k1)) lost += (double)exp_scaled(key_value(t.k1), run.o, e);
            if (t.k2 != 0 && !wtop_has(m, t.k2)) lost += (double)exp_scaled(key_value(t.k2), run.o, e);
            if (t.k3 != 0 && !wtop_has(m, t.k3)) lost += (double)exp_scaled(key_value(t.k3), run.o, e);
            if (lane == 0) {
                if (wt.k0 != 0 && !wtop_has(m, wt.k0)) lost += (double)exp_scaled(key_value(wt.k0), run.o, e);
                if (wt.k1 != 0 && !wtop_has(m, wt.k1)) lost += (double)exp_scaled(key_value(wt.k1), run.o, e);
                if (wt.k2 != 0 && !wtop_has(m, wt.k2)) lost += (double)exp_scaled(key_value(wt.k2), run.o, e);
                if (wt.k3 != 0 && !wtop_has(m, wt.k3)) lost += (double)exp_scaled(key_value(wt.k3), run.o, e);
            }
        }
        wt = m;
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

// Exchange of the waves' lists after a fixed number of tiles (the same in
// every wave, so the result is too): the 4th best of the four lists' keys.
// lds_keys holds 4 * kWaves 8-byte words.
__device__ __forceinline__ uint64_t block_floor_of(const WaveTop &wt, double *lds_keys)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t *keys = reinterpret_cast<uint64_t *>(lds_keys) + wave * 4;
    // a fixed field per lane (a select between fields by lane would become an
    // indexed access that keeps the list out of registers)
    if (lane == 0) keys[0] = wt.k0;
    if (lane == 1) keys[1] = wt.k1;
    if (lane == 2) keys[2] = wt.k2;
    if (lane == 3) keys[3] = wt.k3;
    __syncthreads();
    WaveTop c;
    wtop_clear(c);
    const uint64_t *all = reinterpret_cast<const uint64_t *>(lds_keys);
#pragma unroll
    for (int j = 0; j < 4 * kWaves; ++j) wtop_insert(c, all[j]);
    __syncthreads();  // lds_keys free again
    return c.k3;
}

// Weighted draft row chunk: block max M, the chunk's top-4 from the waves'
// lists (merged in wave order), and the mass outside it: the lanes' sums and
// the wave-list entries the chunk's top-4 does not keep.  lds_f holds kWaves
// entries, lds_keys 4 * kWaves 8-byte words.
__device__ __forceinline__ void run_finish_top(const RowRun &run, const WaveTop &wt, const ExpScale &e,
                                               float *lds_f, double *lds_keys, double *lds_d, float &M,
                                               double &S_excl, Top4 &ct)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    M = block_max(run.m, lds_f);  // uses entries 0..kWaves-1, ends with a barrier
    // each of lanes 0..3 stores one key of its wave's list (a fixed field
    // per lane: a select between fields by lane would become an indexed
    // access that keeps the list out of registers)
    uint64_t *keys = reinterpret_cast<uint64_t *>(lds_keys) + wave * 4;
    if (lane == 0) keys[0] = wt.k0;
    if (lane == 1) keys[1] = wt.k1;
    if (lane == 2) keys[2] = wt.k2;
    if (lane == 3) keys[3] = wt.k3;
    __syncthreads();
    WaveTop c;
    wtop_clear(c);
    const uint64_t *all = reinterpret_cast<const uint64_t *>(lds_keys);
#pragma unroll
    for (int j = 0; j < 4 * kWaves; ++j) wtop_insert(c, all[j]);
    const uint64_t ck[4] = {c.k0, c.k1, c.k2, c.k3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ct.v[j] = key_value(ck[j]);
        ct.i[j] = key_index(ck[j]);
    }
    const double oM = (double)row_offset(M, e);
    double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - oM);
    if (lane == 0) {
        const uint64_t wk[4] = {wt.k0, wt.k1, wt.k2, wt.k3};
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (wk[j] != 0 && key_value(wk[j]) != -INFINITY && !wtop_has(c, wk[j]))
                sc += exp_scaled64(key_value(wk[j]), oM, e.c64);
    }
    S_excl = block_sum(sc, lds_d);
}

}  // namespace sv
