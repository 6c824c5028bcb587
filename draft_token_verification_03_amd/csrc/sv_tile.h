// sv_tile.h -- per-thread tile reductions of the streaming pass, shared by
// the verify step, the outcome distribution and the tree walk.
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

// Pairwise fp32 sum of the exponentials of one raw vector.
template <int DT>
__device__ __forceinline__ float vec_sum_exp(uint4 r, float o, const ExpScale &e)
{
    constexpr int VEC = Elt<DT>::kVec;
    float x[VEC], ev[VEC];
    Elt<DT>::unpack(r, x);
#pragma unroll
    for (int k = 0; k < VEC; ++k) ev[k] = exp_scaled(x[k], o, e);
#pragma unroll
    for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
    return ev[0];
}

template <int DT, int U>
__device__ __forceinline__ void run_sum_tile(const uint4 (&r)[U], const ExpScale &e, RowRun &run)
{
    run_raise_lazy(run, tile_lane_max<DT, U>(r), e);
    if (run.m == -INFINITY) return;
#pragma unroll
    for (int u = 0; u < U; ++u) run.s += (double)vec_sum_exp<DT>(r[u], run.o, e);
}

// Beta-weighted draft row: as run_sum_tile, and each wave keeps the top-4
// of the elements it has seen, by (value desc, index asc), in a list that
// every lane holds alike, out of its sums; at the end of the chunk the four
// waves' lists give the chunk's top-4 and their other entries join the sum
// (run_finish_top).  The list's 4th entry is a floor that most later tiles
// do not reach (after t tiles a wave's next tile holds a new entry with
// probability ~4/t), so most vectors take the plain sum.  Elements that beat
// the floor when their vector is reached are inserted one at a time, in a
// fixed order (element position in the vector, then lane); when many lanes
// of a tile beat it (a wave's first tile, rising rows) the tile's floor is
// first raised to the 4th best of the lanes' best elements, below which no
// element of the tile can be in the top-4.  An entry pushed out of the
// list, or a candidate that no longer makes it, has its mass added by lane
// 0.  Every element thus reaches the sum, or the chunk's top-4, along a path
// and in an order that depend only on the data: a call gives the same bits
// every time.

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

// A floor decoded for `better`: elements (v, i) that beat it.
struct Floor {
    uint64_t key;
    float v;
    int i;
};

__device__ __forceinline__ Floor make_floor(uint64_t key)
{
    Floor f;
    f.key = key;
    f.v = key_value(key);
    f.i = key_index(key);
    return f;
}

// A value the same in every lane of the wave, held as such.
__device__ __forceinline__ uint64_t wave_uniform(uint64_t k)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)k);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(k >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// The key just below the 4th best of the lanes' best elements (value mx at
// the lane's lowest index bi; bi = INT_MAX for a lane without elements), or
// 0 when fewer than four lanes hold one.  Every element of the tile with a
// smaller key has four better ones in the tile.
__device__ __forceinline__ uint64_t seed_floor_keys(float mx, int bi)
{
    float v = mx;
    int i = bi;
    uint64_t k4 = 0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float bv = v;
        int bj = i;
        wave_argmax(bv, bj);
        bj = __builtin_amdgcn_readfirstlane(bj);
        bv = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bv)));
        if (bj == INT_MAX) return 0;
        if (i == bj) {  // indices are unique: the lane that held it drops out
            v = -INFINITY;
            i = INT_MAX;
        }
        k4 = top_key(bv, bj);
    }
    return k4 - 1;  // the low word is 0x7fffffff - bj > 0
}

// The 4th largest of the lanes' maxima by value (one lane dropping out per
// round), -inf when fewer than four lanes hold a finite one; `ties` tells
// whether another lane's maximum equals it.
__device__ __forceinline__ float seed_floor_value(float mx, bool &ties)
{
    const int lane = threadIdx.x & 63;
    float v = mx;
    float M = -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        M = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max(v))));
        if (M == -INFINITY) break;
        const uint64_t at = __ballot(v == M);
        if (lane == __ffsll((unsigned long long)at) - 1) v = -INFINITY;
    }
    ties = __ballot(v == M) != 0ull;
    return M;
}

// Per-vector lane maxima of a tile.
template <int DT, int U>
__device__ __forceinline__ void tile_vec_max(const uint4 (&r)[U], float (&vm)[U])
{
    constexpr int VEC = Elt<DT>::kVec;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
        float m = x[0];
#pragma unroll
        for (int k = 1; k < VEC; ++k) m = fmaxf(m, x[k]);
        vm[u] = m;
    }
}

// The lane's lowest token index (< V) holding value mx, INT_MAX if none.
template <int DT, int U>
__device__ __forceinline__ int lane_first_index(const uint4 (&r)[U], int q0, int V, float mx)
{
    constexpr int VEC = Elt<DT>::kVec;
    int bi = INT_MAX;
#pragma unroll
    for (int u = U - 1; u >= 0; --u) {
        float x[VEC];
        Elt<DT>::unpack(r[u], x);
#pragma unroll
        for (int k = VEC - 1; k >= 0; --k) {
            const int idx = elem_index(q0, u, k, VEC);
            if (x[k] == mx && idx < V) bi = idx;
        }
    }
    return bi;
}

// The floor a tile's elements must beat is the wave's 4th key, or the
// block's floor from the last exchange of the waves' lists when that is
// higher (an element below the block's 4th best of what all waves had seen
// then cannot be in the chunk's top-4).  Such a floor comes from lower token
// indices than any element of the tile, so an element beats it exactly when
// its value is larger; so does a list key taken after the tile's vectors up
// to u, for the vectors after u.  A floor seeded from the tile itself, or an
// empty one, is tested with indices (`full`).
template <int DT, int U>
__device__ __forceinline__ void run_sum_top_tile(const uint4 (&r)[U], int q0, int V,
                                                 const ExpScale &e, RowRun &run, WaveTop &wt,
                                                 uint64_t block_floor)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int lane = threadIdx.x & 63;
    float vm[U];
    tile_vec_max<DT, U>(r, vm);
    float mx = vm[0];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, vm[u]);
    run_raise_lazy(run, mx, e);
    const bool have_m = run.m != -INFINITY;
    Floor f = make_floor(wt.k3 > block_floor ? wt.k3 : block_floor);
    bool full = f.key == 0;
    const uint64_t lanes = __ballot(full ? !(mx < f.v) : mx > f.v);
    if (lanes == 0ull) {
        if (!have_m) return;
#pragma unroll
        for (int u = 0; u < U; ++u) run.s += (double)vec_sum_exp<DT>(r[u], run.o, e);
        return;
    }
    if (__popcll(lanes) > 4) {
        // many lanes: first raise this tile's floor from its lanes' maxima
        bool ties;
        const float v4 = seed_floor_value(mx, ties);
        // every element below v4 has four larger ones; elements equal to it
        // all stay candidates
        uint64_t s = v4 == -INFINITY ? 0 : top_key(v4, 0x7fffffff);
        if (ties) s = seed_floor_keys(mx, lane_first_index<DT, U>(r, q0, V, mx));
        if (s > f.key) {
            f = make_floor(s);
            full = true;
        }
    }
    const int wbase = __builtin_amdgcn_readfirstlane((int)threadIdx.x) & ~63;
    double ulost = 0.0;  // masses leaving the list, alike in every lane
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (__ballot(full ? !(vm[u] < f.v) : vm[u] > f.v) == 0ull) {
            if (have_m) run.s += (double)vec_sum_exp<DT>(r[u], run.o, e);
            continue;
        }
        float x[VEC], ev[VEC];
        Elt<DT>::unpack(r[u], x);
        uint64_t cm[VEC];  // lanes whose element k beats the floor
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const int idx = elem_index(q0, u, k, VEC);
            const bool c = full ? idx < V && better(x[k], idx, f.v, f.i) : x[k] > f.v;
            cm[k] = __ballot(c);
            ev[k] = (c || !have_m) ? 0.f : exp_scaled(x[k], run.o, e);
        }
#pragma unroll
        for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
            for (int k = 0; k < w; ++k) ev[k] += ev[k + w];
        run.s += (double)ev[0];
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            uint64_t m = cm[k];
            while (m != 0ull) {
                const int L = __ffsll((unsigned long long)m) - 1;
                m &= m - 1ull;
                const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k]), L));
                const int i = (q0 + u * kBlock + wbase + L) * VEC + k;
                const uint64_t out = wtop_insert(wt, top_key(v, i));
                if (out != 0 && have_m) ulost += (double)exp_scaled(key_value(out), run.o, e);
            }
        }
        if (wt.k3 > f.key) {  // later vectors face the risen floor
            f = make_floor(wt.k3);
            full = false;
        }
    }
    if (lane == 0) run.s += ulost;
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

// Lanes 0..3 of each wave store its list in lds_keys (a fixed field per
// lane: a select between fields by lane would become an indexed access that
// keeps the list out of registers); the four words after the waves' are
// cleared for top4_ranked.  lds_keys holds 4 * kWaves + 4 8-byte words.
__device__ __forceinline__ void store_wave_list(const WaveTop &wt, double *lds_keys)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t *keys = reinterpret_cast<uint64_t *>(lds_keys) + wave * 4;
    if (lane == 0) keys[0] = wt.k0;
    if (lane == 1) keys[1] = wt.k1;
    if (lane == 2) keys[2] = wt.k2;
    if (lane == 3) keys[3] = wt.k3;
    if (threadIdx.x < 4) reinterpret_cast<uint64_t *>(lds_keys)[4 * kWaves + threadIdx.x] = 0;
}

// The best four of the waves' 16 keys (stored, then a barrier): thread j < 16
// counts the keys above key j -- non-empty keys are distinct, so that is its
// place -- and the four best land in the cleared words after the lists.
// Every thread gets them after a second barrier.
__device__ __forceinline__ WaveTop top4_ranked(double *lds_keys)
{
    uint64_t *all = reinterpret_cast<uint64_t *>(lds_keys);
    const int tid = threadIdx.x;
    if (tid < 4 * kWaves) {
        const uint64_t k = all[tid];
        int rank = 0;
#pragma unroll
        for (int i = 0; i < 4 * kWaves; ++i) rank += all[i] > k ? 1 : 0;
        if (k != 0 && rank < 4) all[4 * kWaves + rank] = k;
    }
    __syncthreads();
    WaveTop c;
    c.k0 = all[4 * kWaves];
    c.k1 = all[4 * kWaves + 1];
    c.k2 = all[4 * kWaves + 2];
    c.k3 = all[4 * kWaves + 3];
    return c;
}

// Exchange of the waves' lists after a fixed number of tiles (the same in
// every wave, so the result is too): the 4th best of the four lists' keys.
__device__ __forceinline__ uint64_t block_floor_of(const WaveTop &wt, double *lds_keys)
{
    store_wave_list(wt, lds_keys);
    __syncthreads();
    const WaveTop c = top4_ranked(lds_keys);
    __syncthreads();  // lds_keys free again
    return wave_uniform(c.k3);
}

// Weighted draft row chunk: block max M, the chunk's top-4 from the waves'
// lists, and the mass outside it: the lanes' sums and the wave-list entries
// the chunk's top-4 does not keep (lanes 0..3 of each wave take one entry
// each, added as a quad).  lds_f holds kWaves entries, lds_keys 4 * kWaves +
// 4 8-byte words.
__device__ __forceinline__ void run_finish_top(const RowRun &run, const WaveTop &wt, const ExpScale &e,
                                               float *lds_f, double *lds_keys, double *lds_d, float &M,
                                               double &S_excl, Top4 &ct)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    store_wave_list(wt, lds_keys);
    M = block_max(run.m, lds_f);  // uses entries 0..kWaves-1, ends with a barrier
    const WaveTop c = top4_ranked(lds_keys);
    const uint64_t ck[4] = {c.k0, c.k1, c.k2, c.k3};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        ct.v[j] = key_value(ck[j]);
        ct.i[j] = key_index(ck[j]);
    }
    const double oM = (double)row_offset(M, e);
    double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - oM);
    double out = 0.0;
    if (lane < 4) {
        const uint64_t k = reinterpret_cast<const uint64_t *>(lds_keys)[wave * 4 + lane];
        if (k != 0 && key_value(k) != -INFINITY && !wtop_has(c, k)) out = exp_scaled64(key_value(k), oM, e.c64);
    }
    out += dpp_double<kDppQuadXor1>(out);
    out += dpp_double<kDppQuadXor2>(out);
    if (lane == 0) sc += out;
    S_excl = block_sum(sc, lds_d);
}

}  // namespace sv
