// sv_stream.h -- pair tiles: the streaming of a target row and, optionally,
// the draft row of the same position in lockstep, U 16-byte vectors of each
// per thread per tile (kOutLoads for the outcome pass), with two tiles in
// flight.  Used by the outcome
// pass and the tree walk.
#pragma once

#include "sv_tile.h"

namespace sv {

// A tile is vectors q = qb + u*BLK + tid (u < U, BLK threads) of the target row
// and, when PAIR, of the draft row, loaded as the streaming pass loads its
// tiles: aligned rows with every load unconditional (indices clamped into
// the chunk) and the vectors past the chunk or the row masked to -inf by
// fix_pair on the last tile only; unaligned rows through funnel shifts.

template <int U>
struct PairTileU {
    uint4 t[U], d[U];
};
using PairTile = PairTileU<kOutLoads>;

template <int DT, bool ALIGNED, bool PAIR, int BLK = kBlock, int U>
__device__ __forceinline__ void issue_pair(const char *trow, const char *drow, int qb, int q1, int V,
                                           PairTileU<U> &r)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (ALIGNED) {
            const int q = min(qb + u * BLK + tid, q1 - 1);
            r.t[u] = load16_stream(trow + (size_t)q * 16);
            if (PAIR) r.d[u] = load16_stream(drow + (size_t)q * 16);
        } else {
            const int q = qb + u * BLK + tid;
            if (q < q1) {
                const int valid = min(VEC, V - q * VEC);
                const char *pt = trow + (size_t)q * 16;
                r.t[u] = load16_unaligned(pt, ((uint32_t)((uintptr_t)pt & 15)) +
                                                  (uint32_t)valid * Elt<DT>::kBytes > 16u);
                if (PAIR) {
                    const char *pd = drow + (size_t)q * 16;
                    r.d[u] = load16_unaligned(pd, ((uint32_t)((uintptr_t)pd & 15)) +
                                                      (uint32_t)valid * Elt<DT>::kBytes > 16u);
                }
            } else {
                r.t[u] = neg_inf_raw<DT>();
                if (PAIR) r.d[u] = neg_inf_raw<DT>();
            }
        }
    }
}

template <int DT, bool PAIR, int BLK = kBlock, int U>
__device__ __forceinline__ void fix_pair(int qb, int q1, int V, PairTileU<U> &r)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < U; ++u)
        if (qb + u * BLK + tid >= q1) {
            r.t[u] = neg_inf_raw<DT>();
            if (PAIR) r.d[u] = neg_inf_raw<DT>();
        }
    if (V % VEC) {
        const int last = (V - 1) / VEC;
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (qb + u * BLK + tid == last) {
                mask_raw<DT>(r.t[u], V - last * VEC);
                if (PAIR) mask_raw<DT>(r.d[u], V - last * VEC);
            }
    }
}

// Stream [q0, q1) through consume(tile, qb) with two tiles in flight; `ra`
// holds the already requested tile at q0.  As the streaming pass's loop: the
// steady state issues unconditionally (a load issued under a condition
// leaves its registers "loaded or not" at the join, where copies would wait
// for it), and the last one or two tiles are peeled.
template <int DT, bool ALIGNED, bool PAIR, int BLK = kBlock, int U, class Consume>
__device__ __forceinline__ void stream_pair(const char *trow, const char *drow, int q0, int q1, int V,
                                            PairTileU<U> &ra, Consume &&consume)
{
    constexpr int kStep = BLK * U;
    const int nt = (q1 - q0 + kStep - 1) / kStep;  // tiles, >= 1
    PairTileU<U> rb;
    int qb = q0;
    for (int t = 0; t + 2 < nt; t += 2, qb += 2 * kStep) {
        issue_pair<DT, ALIGNED, PAIR, BLK>(trow, drow, qb + kStep, q1, V, rb);
        consume(ra, qb);
        issue_pair<DT, ALIGNED, PAIR, BLK>(trow, drow, qb + 2 * kStep, q1, V, ra);
        consume(rb, qb + kStep);
    }
    if (qb + kStep < q1) {  // two tiles left
        issue_pair<DT, ALIGNED, PAIR, BLK>(trow, drow, qb + kStep, q1, V, rb);
        consume(ra, qb);
        fix_pair<DT, PAIR, BLK>(qb + kStep, q1, V, rb);
        consume(rb, qb + kStep);
    } else {
        fix_pair<DT, PAIR, BLK>(qb, q1, V, ra);
        consume(ra, qb);
    }
}

}  // namespace sv
