// sv_device.h -- device-side building blocks of libspecverify (gfx950, wave64).
//
// Private to the library: row loading, wave/block reductions and scans, the
// top-4 selection and the Philox4x32-10 counter generator.
#pragma once

#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

namespace sv {

constexpr int kBlock = 256;            // threads per workgroup: four wave64s
constexpr int kWaves = kBlock / 64;
constexpr int kLoads = 4;              // 16-byte loads in flight per thread per step
constexpr double kLog2e = 1.4426950408889634;

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds, each
// multiplying words 0 and 2 by fixed 32-bit constants (keeping both halves of
// the 64-bit products) and xoring the high halves into words 1 and 3 together
// with the key; the key advances by two Weyl increments between rounds.

__device__ __forceinline__ uint32_t philox_word0(uint64_t seed, uint32_t c0, uint32_t c1,
                                                 uint32_t c2, uint32_t c3)
{
    uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo_a = 0xD2511F53u * c0, hi_a = __umulhi(0xD2511F53u, c0);
        const uint32_t lo_b = 0xCD9E8D57u * c2, hi_b = __umulhi(0xCD9E8D57u, c2);
        c0 = hi_b ^ c1 ^ k0;
        c1 = lo_b;
        c2 = hi_a ^ c3 ^ k1;
        c3 = lo_a;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c0;
}

// Uniform in (0, 1] on a 2^-24 grid (exact in float) for counter (b, pos, purpose, 0).
__device__ __forceinline__ float philox_uniform(uint64_t seed, uint32_t b, uint32_t pos,
                                                uint32_t purpose)
{
    const uint32_t w = philox_word0(seed, b, pos, purpose, 0u);
    return (float)((w >> 8) + 1u) * 0x1p-24f;
}

// ---------------------------------------------------------------------------
// Row loading.  A row of V logits is read as 16-byte vectors; vector q holds
// elements [q*VEC, q*VEC + VEC).  The element-to-lane mapping depends only on
// the element index, never on the row's address, so two rows with equal
// values give bitwise-equal reductions wherever they sit in memory.

template <int DT> struct Elt;
template <> struct Elt<0> {  // fp32
    static constexpr int kVec = 4;
    static constexpr int kBytes = 4;
    __device__ static __forceinline__ void unpack(uint4 r, float (&x)[4])
    {
        x[0] = __uint_as_float(r.x);
        x[1] = __uint_as_float(r.y);
        x[2] = __uint_as_float(r.z);
        x[3] = __uint_as_float(r.w);
    }
    __device__ static __forceinline__ float scalar(const char *row, int64_t v)
    {
        return reinterpret_cast<const float *>(row)[v];
    }
};
template <> struct Elt<1> {  // bf16: the upper 16 bits of a float
    static constexpr int kVec = 8;
    static constexpr int kBytes = 2;
    __device__ static __forceinline__ void unpack(uint4 r, float (&x)[8])
    {
        x[0] = __uint_as_float(r.x << 16);
        x[1] = __uint_as_float(r.x & 0xffff0000u);
        x[2] = __uint_as_float(r.y << 16);
        x[3] = __uint_as_float(r.y & 0xffff0000u);
        x[4] = __uint_as_float(r.z << 16);
        x[5] = __uint_as_float(r.z & 0xffff0000u);
        x[6] = __uint_as_float(r.w << 16);
        x[7] = __uint_as_float(r.w & 0xffff0000u);
    }
    __device__ static __forceinline__ float scalar(const char *row, int64_t v)
    {
        const uint32_t bits = (uint32_t)reinterpret_cast<const uint16_t *>(row)[v] << 16;
        return __uint_as_float(bits);
    }
};

__device__ __forceinline__ uint32_t funnel_bytes(uint32_t lo, uint32_t hi, uint32_t r)
{
    return (uint32_t)((((uint64_t)hi << 32) | lo) >> (8u * r));
}

template <int W>
__device__ __forceinline__ uint4 pick4(const uint32_t (&d)[8], uint32_t r)
{
    return make_uint4(funnel_bytes(d[W], d[W + 1], r), funnel_bytes(d[W + 1], d[W + 2], r),
                      funnel_bytes(d[W + 2], d[W + 3], r), funnel_bytes(d[W + 3], d[W + 4], r));
}

// 16 bytes starting at a non-16-aligned address p, from the two aligned
// 16-byte blocks that hold them.  The second block is only read when it holds
// valid bytes (`need_second`), so no read leaves the pages the row lives in.
__device__ __forceinline__ uint4 load16_unaligned(const char *p, bool need_second)
{
    const uintptr_t a = (uintptr_t)p;
    const uint4 *blk = reinterpret_cast<const uint4 *>(a & ~(uintptr_t)15);
    const uint32_t sh = (uint32_t)(a & 15);
    const uint4 x = blk[0];
    const uint4 y = need_second ? blk[1] : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t d[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    const uint32_t r = sh & 3u;
    switch (sh >> 2) {
    case 0: return pick4<0>(d, r);
    case 1: return pick4<1>(d, r);
    case 2: return pick4<2>(d, r);
    default: return pick4<3>(d, r);
    }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load with the nontemporal hint: logits are streamed once, and on
// MI355X the hinted loads sustain ~7.1 TB/s against ~6.3 TB/s without it.
__device__ __forceinline__ uint4 load16_stream(const char *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------------------
// Exponentials of a row at temperature T are taken in base 2 with the scale
// c = fp32(log2(e) / T): an element z contributes exp2(z c - o), where the
// row offset o = fp32(m c) belongs to the row's (running) maximum m.  One fma
// per element forms the argument exactly and rounds it once.  Every later
// step (merges, accept ratio, residual) uses the same c and the same offsets
// in fp64, so the path is exactly the softmax at T' = log2(e) / c, within a
// relative 2^-24 of T: the accept ratios move by ~1e-7 at most.

struct ExpScale {
    float c;     // fp32(log2(e) / T)
    double c64;  // the same value in fp64
};

__device__ __forceinline__ ExpScale make_scale(float T)
{
    ExpScale e;
    e.c = (float)(kLog2e / (double)T);
    e.c64 = (double)e.c;
    return e;
}

// Row offset of a maximum m (-inf for an empty row).
__device__ __forceinline__ float row_offset(float m, const ExpScale &e) { return m * e.c; }

// exp2(x c - o) for an element x and a finite offset o.
__device__ __forceinline__ float exp_scaled(float x, float o, const ExpScale &e)
{
    return __builtin_amdgcn_exp2f(__builtin_fmaf(x, e.c, -o));
}

// exp2(x c - o) in fp64 (x c is exact in fp64) for merges of partial sums.
__device__ __forceinline__ double exp_scaled64(float x, double o, double c64)
{
    return exp2((double)x * c64 - o);
}

// ---------------------------------------------------------------------------
// Wave64 all-reductions without LDS: DPP within each 16-lane row (quad
// butterflies, then the half-row and row mirrors; after each step every lane
// of the group holds the group's value), then v_permlane16_swap and
// v_permlane32_swap across rows.  A swap of a register with itself returns
// the two halves being combined, so op(first, second) is the butterfly
// result on every lane.  Fixed trees: results are reproducible, and equal in
// every lane.  Callers run them with all 64 lanes active.

constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1, 0, 3, 2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ int dpp_int(int v)
{
    return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xf, 0xf, false);
}

template <int CTRL>
__device__ __forceinline__ float dpp_float(float v)
{
    return __int_as_float(dpp_int<CTRL>(__float_as_int(v)));
}

template <int CTRL>
__device__ __forceinline__ double dpp_double(double v)
{
    const int lo = dpp_int<CTRL>(__double2loint(v));
    const int hi = dpp_int<CTRL>(__double2hiint(v));
    return __hiloint2double(hi, lo);
}

// The two halves a row-pair (16) or wave-half (32) butterfly combines.
struct IntPair {
    int a, b;
};

template <int SPAN>
__device__ __forceinline__ IntPair swap_halves(int v)
{
    if (SPAN == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return {(int)p[0], (int)p[1]};
    }
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return {(int)p[0], (int)p[1]};
}

template <int SPAN>
__device__ __forceinline__ void swap_halves_float(float v, float &x, float &y)
{
    const IntPair p = swap_halves<SPAN>(__float_as_int(v));
    x = __int_as_float(p.a);
    y = __int_as_float(p.b);
}

template <int SPAN>
__device__ __forceinline__ void swap_halves_double(double v, double &x, double &y)
{
    const IntPair lo = swap_halves<SPAN>(__double2loint(v));
    const IntPair hi = swap_halves<SPAN>(__double2hiint(v));
    x = __hiloint2double(hi.a, lo.a);
    y = __hiloint2double(hi.b, lo.b);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = fmaxf(v, dpp_float<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_float<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_float<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_float<kDppRowMirror>(v));
    float x, y;
    swap_halves_float<16>(v, x, y);
    v = fmaxf(x, y);
    swap_halves_float<32>(v, x, y);
    return fmaxf(x, y);
}

__device__ __forceinline__ double wave_sum(double v)
{
    v += dpp_double<kDppQuadXor1>(v);
    v += dpp_double<kDppQuadXor2>(v);
    v += dpp_double<kDppRowHalfMirror>(v);
    v += dpp_double<kDppRowMirror>(v);
    double x, y;
    swap_halves_double<16>(v, x, y);
    v = x + y;
    swap_halves_double<32>(v, x, y);
    return x + y;
}

template <class Op>
__device__ __forceinline__ int wave_reduce_int(int v, Op op)
{
    v = op(v, dpp_int<kDppQuadXor1>(v));
    v = op(v, dpp_int<kDppQuadXor2>(v));
    v = op(v, dpp_int<kDppRowHalfMirror>(v));
    v = op(v, dpp_int<kDppRowMirror>(v));
    IntPair p = swap_halves<16>(v);
    v = op(p.a, p.b);
    p = swap_halves<32>(v);
    return op(p.a, p.b);
}

__device__ __forceinline__ int wave_min_int(int v)
{
    return wave_reduce_int(v, [](int x, int y) { return min(x, y); });
}

__device__ __forceinline__ int wave_sum_int(int v)
{
    return wave_reduce_int(v, [](int x, int y) { return x + y; });
}

__device__ __forceinline__ int wave_max_int(int v)
{
    return wave_reduce_int(v, [](int x, int y) { return max(x, y); });
}

// (value desc, index asc) order used for argmax and top-4.
__device__ __forceinline__ bool better(float v, int i, float w, int j)
{
    return v > w || (v == w && i < j);
}

__device__ __forceinline__ void argmax_step(float &v, int &i, float w, int j)
{
    if (better(w, j, v, i)) {
        v = w;
        i = j;
    }
}

template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float &v, int &i)
{
    const float w = dpp_float<CTRL>(v);
    const int j = dpp_int<CTRL>(i);
    argmax_step(v, i, w, j);
}

template <int SPAN>
__device__ __forceinline__ void argmax_swap(float &v, int &i)
{
    float x, y;
    swap_halves_float<SPAN>(v, x, y);
    const IntPair p = swap_halves<SPAN>(i);
    v = x;
    i = p.a;
    argmax_step(v, i, y, p.b);
}

__device__ __forceinline__ void wave_argmax(float &v, int &i)
{
    argmax_dpp<kDppQuadXor1>(v, i);
    argmax_dpp<kDppQuadXor2>(v, i);
    argmax_dpp<kDppRowHalfMirror>(v, i);
    argmax_dpp<kDppRowMirror>(v, i);
    argmax_swap<16>(v, i);
    argmax_swap<32>(v, i);
}

template <int NW = kWaves>
__device__ __forceinline__ float block_max(float v, float *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max(v);
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    float r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = fmaxf(r, lds[w]);
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ double block_sum(double v, double *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_sum(v);
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    double r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r += lds[w];
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_min_int(int v, int *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_min_int(v);
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = min(r, lds[w]);
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ int block_max_int(int v, int *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_max_int(v);
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = max(r, lds[w]);
    __syncthreads();
    return r;
}

template <int NW = kWaves>
__device__ __forceinline__ void block_argmax(float &v, int &i, float *ldsv, int *ldsi)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    wave_argmax(v, i);
    if (lane == 0) {
        ldsv[wave] = v;
        ldsi[wave] = i;
    }
    __syncthreads();
    v = ldsv[0];
    i = ldsi[0];
#pragma unroll
    for (int w = 1; w < NW; ++w)
        if (better(ldsv[w], ldsi[w], v, i)) {
            v = ldsv[w];
            i = ldsi[w];
        }
    __syncthreads();
}

// Inclusive prefix sum over the wave in lane order: Hillis-Steele shifts of
// 1, 2, 4, 8 lanes within each row (lanes without a source add 0), then the
// last lane of row 0 (2) is broadcast into row 1 (3), and the last lane of
// the lower half into rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_double_or0(double v)
{
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xf, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double wave_inclusive_scan(double v)
{
    v += dpp_double_or0<0x111, 0xf>(v);  // row_shr:1
    v += dpp_double_or0<0x112, 0xf>(v);  // row_shr:2
    v += dpp_double_or0<0x114, 0xf>(v);  // row_shr:4
    v += dpp_double_or0<0x118, 0xf>(v);  // row_shr:8
    v += dpp_double_or0<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_double_or0<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// Exclusive prefix sum over the workgroup in thread order; `total` receives
// the sum of all values.
template <int NW = kWaves>
__device__ __forceinline__ double block_exclusive_scan(double v, double &total, double *lds)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double inc = wave_inclusive_scan(v);
    const double exc = dpp_double_or0<0x138, 0xf>(inc);  // wave_shr:1, lane 0 gets 0
    if (lane == 63) lds[wave] = inc;
    __syncthreads();
    double off = 0.0;
    for (int w = 0; w < wave; ++w) off += lds[w];
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += lds[w];
    __syncthreads();
    total = tot;
    return off + exc;
}

// ---------------------------------------------------------------------------
// Top-4 lists kept sorted by (value desc, index asc); empty slots are
// (-inf, INT_MAX).

struct Top4 {
    float v[4];
    int i[4];
};

__device__ __forceinline__ void top_clear(Top4 &t)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        t.v[k] = -INFINITY;
        t.i[k] = INT_MAX;
    }
}

__device__ __forceinline__ void top_insert(Top4 &t, float v, int i)
{
    if (!better(v, i, t.v[3], t.i[3])) return;
    t.v[3] = v;
    t.i[3] = i;
#pragma unroll
    for (int k = 3; k > 0; --k) {
        if (better(t.v[k], t.i[k], t.v[k - 1], t.i[k - 1])) {
            const float tv = t.v[k];
            const int ti = t.i[k];
            t.v[k] = t.v[k - 1];
            t.i[k] = t.i[k - 1];
            t.v[k - 1] = tv;
            t.i[k - 1] = ti;
        }
    }
}

__device__ __forceinline__ bool top_has(const Top4 &t, int i)
{
    return i != INT_MAX && (t.i[0] == i || t.i[1] == i || t.i[2] == i || t.i[3] == i);
}

// Merge the per-lane lists of a wave into the wave's top-4 (every lane gets it).
__device__ __forceinline__ Top4 wave_top4(Top4 t)
{
    Top4 out;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float v = t.v[0];
        int i = t.i[0];
        wave_argmax(v, i);
        out.v[r] = v;
        out.i[r] = i;
        if (t.v[0] == v && t.i[0] == i && i != INT_MAX) {  // pop the winner's head
            t.v[0] = t.v[1];
            t.i[0] = t.i[1];
            t.v[1] = t.v[2];
            t.i[1] = t.i[2];
            t.v[2] = t.v[3];
            t.i[2] = t.i[3];
            t.v[3] = -INFINITY;
            t.i[3] = INT_MAX;
        }
    }
    return out;
}

}  // namespace sv
