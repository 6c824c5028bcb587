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

// Beta-weighted draft row: as run_sum_tile, and the workgroup keeps the
// chunk's top-4 so far, by (value desc, index asc), in four LDS slots of
// 64-bit keys that every wave reads and updates.  A key orders like its
// (value, index) pair, so the slots take new entries with atomic maxima: an
// insert walks down the slots, and at each one the larger key stays and the
// smaller moves on, which keeps the slots plus the keys that fall off the end
// equal to everything inserted, and the slots the four best, under any
// interleaving of the waves.  The lanes' sums cover every element that
// never enters the slots or falls out of them.  The 4th slot is a floor no
// later element reaches in most tiles (one shared list sees four waves'
// elements, so after t tiles a wave's next tile holds a new entry with
// probability ~1/t), so most tiles take the plain sum.  A tile with a few
// candidates has each inserted by its own lane; the first tile, or one with
// many candidates (rising rows), reduces per-lane lists to the wave's top-4
// first and inserts those four.

// Key of (v, i), i in [0, INT_MAX): larger keys are better entries; -0 counts
// as +0, as in `better`.  Key 0 is an empty slot.
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

// Insert key k into the slots; returns the key that falls out (k itself if it
// does not enter, 0 if it took an empty slot).
__device__ __forceinline__ uint64_t slots_insert(uint64_t *slots, uint64_t k)
{
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t old = atomicMax((unsigned long long *)&slots[j], (unsigned long long)k);
        k = old < k ? old : k;
    }
    return k;
}

// The 4th slot as (value, index); a stale read is a lower bound of the
// current one, as slots only rise.
__device__ __forceinline__ void slots_floor(const uint64_t *slots, float &fv, int &fi)
{
    const uint64_t k = __hip_atomic_load(&slots[3], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    fv = key_value(k);
    fi = key_index(k);
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

template <int DT, int U>
__device__ __forceinline__ void run_sum_top_tile(const uint4 (&r)[U], int q0, int V,
                                                 const ExpScale &e, RowRun &run, uint64_t *slots)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int lane = threadIdx.x & 63;
    float fv;
    int fi;
    slots_floor(slots, fv, fi);
    const float mx = tile_lane_max<DT, U>(r);
    run_raise_lazy(run, mx, e);
    const bool have_m = run.m != -INFINITY;
    // the lane's first token of the tile is its lowest
    const bool maybe = mx > fv || (mx == fv && elem_index(q0, 0, 0, VEC) < fi);
    if (__ballot(maybe) == 0ull) {  // no element can enter the slots
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
    // keys that fall out of the slots, by the lane that inserted them; each
    // is at most the element inserted, so at most the wave's maximum
    double lost = 0.0;
    if (wave_sum_int(ncand) <= kSerialCandidates) {
        if (cmask != 0u) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float x[VEC];
                Elt<DT>::unpack(r[u], x);
#pragma unroll
                for (int k = 0; k < VEC; ++k) {
                    if (!((cmask >> (u * VEC + k)) & 1u)) continue;
                    const uint64_t out = slots_insert(slots, top_key(x[k], elem_index(q0, u, k, VEC)));
                    if (out != 0 && have_m) lost += (double)exp_scaled(key_value(out), run.o, e);
                }
            }
        }
    } else {
        // per-lane lists of the candidates, the wave's top-4 of them, and
        // lanes 0..3 insert its entries
        Top4 t;
        top_clear(t);
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
                if (oi != INT_MAX && have_m) lost += (double)exp_scaled(ov, run.o, e);
            }
        }
        const Top4 nw = wave_top4(t);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (t.i[k] != INT_MAX && !top_has(nw, t.i[k]) && have_m)
                lost += (double)exp_scaled(t.v[k], run.o, e);
        const float v = lane == 0 ? nw.v[0] : lane == 1 ? nw.v[1] : lane == 2 ? nw.v[2] : nw.v[3];
        const int i = lane == 0 ? nw.i[0] : lane == 1 ? nw.i[1] : lane == 2 ? nw.i[2] : nw.i[3];
        if (lane < 4 && i != INT_MAX) {
            const uint64_t out = slots_insert(slots, top_key(v, i));
            if (out != 0 && have_m) lost += (double)exp_scaled(key_value(out), run.o, e);
        }
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

// Weighted draft row chunk: block max M, the chunk's top-4 (the slots, once
// every wave has finished) and the mass outside it.
__device__ __forceinline__ void run_finish_top(const RowRun &run, const uint64_t *slots, const ExpScale &e,
                                               float *lds_f, double *lds_d, float &M, double &S_excl,
                                               Top4 &ct)
{
    M = block_max(run.m, lds_f);  // its barrier also orders every insert before the reads
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint64_t key = slots[k];
        ct.v[k] = key_value(key);
        ct.i[k] = key_index(key);
    }
    const double sc = (run.m == -INFINITY) ? 0.0 : run.s * exp2((double)run.o - (double)row_offset(M, e));
    S_excl = block_sum(sc, lds_d);
}

}  // namespace sv
