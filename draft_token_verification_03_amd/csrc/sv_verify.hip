// sv_verify.hip -- the kernels of the verify step and their launchers.
//
//   1. stats_kernel  streams every needed logit row once, one workgroup per
//                    (row, chunk), and reduces it to a partial: (max, sum of
//                    exp2((z - max) log2e / T)) for sampling rows, (max,
//                    lowest argmax) for greedy rows, and for beta-weighted
//                    draft rows the chunk top-4 with the mass outside it.
//   2. residual_kernel  several workgroups per sequence.  Each runs the
//                    sequence's accept scan: merge its rows' partials in fp64,
//                    form every accept ratio in the log domain, draw the
//                    Philox uniforms and find the first rejection n (all of
//                    them agree; the first publishes it).  Each then streams
//                    its share of target row n and draft row n (or of target
//                    row K after K acceptances) and writes the residual mass
//                    of every 1 KiB slot of it.
//   3. bonus_kernel  one workgroup per sequence: inverse CDF over the slot
//                    masses, then over the elements of the selected slot.
//
// Calls without draft rows (only greedy sequences can verify there) replace
// steps 2 and 3 by accept_kernel: the accept scan alone, one workgroup per
// sequence.
//
// The launches are stream-ordered; every kernel reads only what earlier
// launches wrote, so no workgroup ever waits for another.
#include <algorithm>

#include <hip/hip_ext.h>

#include "sv_accept.h"
#include "sv_tile.h"

namespace sv {

// Tiles of the streaming pass: kLoads vectors q = qb + u*kBlock + tid of a
// row per thread.  issue_tile only requests the loads (aligned rows: indices
// clamped into the chunk, so every load is unconditional); fix_tile, run by
// the consumer on a chunk's last tile only, turns the vectors at or beyond q1
// (re-reads of vector q1 - 1) and the elements at or beyond V into -inf.
// Masking right after issuing would make each load wait before the next tile
// could be requested.  Unaligned rows load through funnel shifts and are
// masked as they are loaded.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void issue_tile(const char *row, int qb, int q1, int V, uint4 (&r)[kLoads])
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    if (ALIGNED) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = min(qb + u * kBlock + tid, q1 - 1);
            r[u] = load16_stream(row + (size_t)q * 16);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q < q1) {
                const char *p = row + (size_t)q * 16;
                const int valid = min(VEC, V - q * VEC);
                r[u] = load16_unaligned(p, ((uint32_t)((uintptr_t)p & 15)) +
                                               (uint32_t)valid * Elt<DT>::kBytes > 16u);
            } else {
                r[u] = neg_inf_raw<DT>();
            }
        }
    }
}

template <int DT>
__device__ __forceinline__ void fix_tile(int qb, int q1, int V, uint4 (&r)[kLoads])
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
#pragma unroll
    for (int u = 0; u < kLoads; ++u)
        if (qb + u * kBlock + tid >= q1) r[u] = neg_inf_raw<DT>();
    if (V % VEC) {
        const int last = (V - 1) / VEC;
#pragma unroll
        for (int u = 0; u < kLoads; ++u)
            if (qb + u * kBlock + tid == last) mask_raw<DT>(r[u], V - last * VEC);
    }
}

// Stream the chunk [q0, q1) of a row through consume(tile, qb), two tiles
// in flight: the next tile is requested before the current one is consumed.
// `ra` holds the (already requested) tile at q0.  The row's alignment is a
// template parameter so that no loaded register passes a branch join (a
// join copies registers, and a copy waits for its load).
//
// The steady state issues its loads unconditionally: a load issued under a
// condition leaves its registers "loaded or not" at the join, and a consumer
// with branches of its own (the beta-weighted rows) then gets register
// copies there, which wait for the loads just issued -- one tile in flight
// instead of two.  The last one or two tiles are peeled.
template <int DT, bool ALIGNED, class Consume>
__device__ __forceinline__ void stream_chunk(const char *row, int q0, int q1, int V,
                                             uint4 (&ra)[kLoads], Consume &&consume)
{
    constexpr int kStep = kBlock * kLoads;
    const int nt = (q1 - q0 + kStep - 1) / kStep;  // tiles in the chunk, >= 1
    uint4 rb[kLoads];
    int qb = q0;
    for (int t = 0; t + 2 < nt; t += 2, qb += 2 * kStep) {
        issue_tile<DT, ALIGNED>(row, qb + kStep, q1, V, rb);
        consume(ra, qb);
        issue_tile<DT, ALIGNED>(row, qb + 2 * kStep, q1, V, ra);
        consume(rb, qb + kStep);
    }
    if (qb + kStep < q1) {  // two tiles left
        issue_tile<DT, ALIGNED>(row, qb + kStep, q1, V, rb);
        consume(ra, qb);
        fix_tile<DT>(qb + kStep, q1, V, rb);
        consume(rb, qb + kStep);
    } else {
        fix_tile<DT>(qb, q1, V, ra);
        consume(ra, qb);
    }
}

// Vector q of a row (q < nvec), with elements at or beyond V as -inf.
template <int DT>
__device__ __forceinline__ uint4 load_one(const char *row, bool aligned, int q, int nvec, int V)
{
    constexpr int VEC = Elt<DT>::kVec;
    const char *p = row + (size_t)q * 16;
    uint4 r;
    if (aligned) {
        r = *reinterpret_cast<const uint4 *>(p);
    } else {
        const int valid = min(VEC, V - q * VEC);
        r = load16_unaligned(p, ((uint32_t)((uintptr_t)p & 15)) + (uint32_t)valid * Elt<DT>::kBytes > 16u);
    }
    if ((V % VEC) && q == nvec - 1) mask_raw<DT>(r, V - q * VEC);
    return r;
}

// The vectors q[u] of a row for the lanes where live[u]; -inf elsewhere and at
// or beyond V.  Aligned rows load every vector unconditionally (indices
// clamped into the row), so all loads are in flight before any is used.
template <int DT, int U>
__device__ __forceinline__ void load_units(const char *row, bool aligned, const int (&q)[U],
                                           const bool (&live)[U], int nvec, int V, uint4 (&r)[U])
{
    constexpr int VEC = Elt<DT>::kVec;
    if (aligned) {
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = *reinterpret_cast<const uint4 *>(row + (size_t)min(q[u], nvec - 1) * 16);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (!live[u]) r[u] = neg_inf_raw<DT>();
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (live[u]) {
                const char *p = row + (size_t)q[u] * 16;
                const int valid = min(VEC, V - q[u] * VEC);
                r[u] = load16_unaligned(p, ((uint32_t)((uintptr_t)p & 15)) +
                                               (uint32_t)valid * Elt<DT>::kBytes > 16u);
            } else {
                r[u] = neg_inf_raw<DT>();
            }
        }
    }
    if (V % VEC) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (live[u] && q[u] == nvec - 1) mask_raw<DT>(r[u], V - q[u] * VEC);
    }
}

__device__ __forceinline__ const char *target_row(const Args &a, int b, int i)
{
    return a.target + ((int64_t)b * (a.K + 1) + i) * a.row_bytes;
}

__device__ __forceinline__ const char *draft_row(const Args &a, int b, int i)
{
    return a.draft + ((int64_t)b * a.K + i) * a.row_bytes;
}

// ---------------------------------------------------------------------------
// 1. Streaming pass, one workgroup per (row, chunk), with the per-thread tile
// reductions of sv_tile.h: a wave-uniform running max with per-lane fp64
// sums, lanes visiting their elements in increasing index order (so argmax
// and top-4 ties resolve to the lowest token id), and for a weighted draft row
// the workgroup's top-4 kept out of the sum.  The first tile is requested before
// the sequence's temperature is known, so the row stream starts one memory
// round trip earlier; a draft row of a greedy sequence (whose draft logits
// were passed anyway) wastes that one tile.  Rows a sequence does not use
// (draft rows in greedy mode or without draft logits, rows of a sequence with
// an invalid temperature, every row of a greedy sequence when only sampling
// sequences are wanted) publish nothing.

// One (row, chunk) of the streaming pass; the first tile is requested before
// the temperature is looked at.
template <int DT, bool TOP, bool ALIGNED>
__device__ __forceinline__ void stats_chunk(const Args &a, const char *row, int b, int i, int kb,
                                            bool is_draft, int slot_row, int chunk, float T)
{
    __shared__ float lds_f[4 + kWaves * 4];
    __shared__ int lds_i[4 + kWaves * 4];
    __shared__ double lds_d[kWaves];
    const int q0 = chunk * a.cvec;
    const int q1 = min(a.nvec, q0 + a.cvec);
    uint4 r[kLoads];
    issue_tile<DT, ALIGNED>(row, q0, q1, a.V, r);
    // a sampling row's logit at its drafted token, read while the first tile
    // is in flight, saves the accept step a dependent gather
    float zx = 0.f;
    if (chunk == 0 && i < kb && a.tokens && threadIdx.x == 0) {
        const int x = a.tokens[(int64_t)b * a.K + i];
        if (x >= 0 && x < a.V) zx = Elt<DT>::scalar(row, x);
    }

    const bool greedy = T == 0.f;
    if (!temperature_ok(T) || (greedy && (is_draft || a.sampling_only))) return;
    RowPart part;
    Top4 ct;
    const bool track_top = TOP && is_draft;
    if (greedy) {
        float best = -INFINITY;
        int bi = INT_MAX;
        stream_chunk<DT, ALIGNED>(row, q0, q1, a.V, r, [&](uint4 (&t)[kLoads], int qb) {
            run_argmax_tile<DT, kLoads>(t, qb, best, bi);
        });
        block_argmax(best, bi, lds_f, lds_i);
        part.m = best;
        part.idx = bi;
        part.s = 0.0;
    } else {
        const ExpScale e = make_scale(T);
        RowRun run;
        run_clear(run);
        if (track_top) {
            __shared__ double lds_keys[kWaves * 4 + 4];  // the waves' lists, exchanged, and their best four
            WaveTop wt;  // this wave's top-4 so far, alike in every lane
            wtop_clear(wt);
            uint64_t block_floor = 0;
            int tiles = 0;
            stream_chunk<DT, ALIGNED>(row, q0, q1, a.V, r, [&](uint4 (&t)[kLoads], int qb) {
                run_sum_top_tile<DT, kLoads>(t, qb, a.V, e, run, wt, block_floor);
                // the waves share their lists after the first tile: the block's
                // floor rises with four waves' data instead of one's (later
                // exchanges measured slower than the candidates they save)
                if (++tiles == 1) block_floor = block_floor_of(wt, lds_keys);
            });
            run_finish_top(run, wt, e, lds_f, lds_keys, lds_d, part.m, part.s, ct);
            if (threadIdx.x < 4) {
                // lane k: the mass of entry k, relative to the chunk's offset;
                // one chunk a row: the row's normaliser D (lane 0 adds the quad)
                const int k = threadIdx.x;
                const float v = k == 0 ? ct.v[0] : k == 1 ? ct.v[1] : k == 2 ? ct.v[2] : ct.v[3];
                const int ix = k == 0 ? ct.i[0] : k == 1 ? ct.i[1] : k == 2 ? ct.i[2] : ct.i[3];
                const double w = (ix != INT_MAX && v != -INFINITY)
                                     ? exp_scaled64(v, (double)row_offset(part.m, e), e.c64)
                                     : 0.0;
                if (a.nc == 1) {
                    double q = w + dpp_double<kDppQuadXor1>(w);
                    q += dpp_double<kDppQuadXor2>(q);
                    part.s += (double)a.beta * q;
                    if (k == 0)  // the top-4 mass itself, for the draft confidence (before beta)
                        reinterpret_cast<double *>(&a.tope[(int64_t)b * a.K + i])[0] = q;
                } else {
                    reinterpret_cast<double *>(&a.tope[((int64_t)b * a.K + i) * a.nc + chunk])[k] = w;
                }
            }
        } else {
            stream_chunk<DT, ALIGNED>(row, q0, q1, a.V, r, [&](uint4 (&t)[kLoads], int qb) {
                run_sum_tile<DT, kLoads>(t, e, run);
            });
            run_finish(run, e, lds_f, lds_d, part.m, part.s);
        }
        part.idx = __float_as_int(zx);
    }
    if (threadIdx.x == 0) {
        a.part[(int64_t)slot_row * a.nc + chunk] = part;
        if (track_top) a.top[((int64_t)b * a.K + i) * a.nc + chunk] = ct;
    }
}

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void stats_kernel(const Args a)
{
    // without draft logits only the target rows 0..K of each sequence are launched
    const int rl = a.draft ? a.R : a.K + 1;
    const int chunk = blockIdx.x % a.nc;
    const int b = (blockIdx.x / a.nc) / rl;
    const int j = blockIdx.x / a.nc - b * rl;
    const int slot_row = b * a.R + j;
    const bool is_draft = j > a.K;
    const int i = is_draft ? j - (a.K + 1) : j;
    int kb = a.K;
    if (a.draft_len) {  // ragged drafts: rows past the sequence's are not read
        kb = a.draft_len[b];
        if (kb < 0 || kb > a.K || i > kb || (is_draft && i == kb)) return;
    }
    const float T = a.temperature[b];
    const char *row = is_draft ? draft_row(a, b, i) : target_row(a, b, i);
    if (((uintptr_t)row & 15) == 0) stats_chunk<DT, TOP, true>(a, row, b, i, kb, is_draft, slot_row, chunk, T);
    else stats_chunk<DT, TOP, false>(a, row, b, i, kb, is_draft, slot_row, chunk, T);
}

// Calls without draft rows and with K > 0 drafts for every sequence (no
// ragged lengths): only greedy sequences can verify (a sampling sequence
// fails without its draft rows, in the accept scan), so only the argmax of
// target rows 0..K is needed, and every row is streamed without waiting for
// its sequence's temperature (the wait held back the second tile of every
// workgroup of a one-round grid).  The kernel holds none of the sampling
// code's registers.
template <int DT, bool ALIGNED>
__device__ __forceinline__ void argmax_chunk(const Args &a, const char *row, int slot_row, int chunk)
{
    __shared__ float lds_f[4 + kWaves * 4];
    __shared__ int lds_i[4 + kWaves * 4];
    const int q0 = chunk * a.cvec;
    const int q1 = min(a.nvec, q0 + a.cvec);
    uint4 r[kLoads];
    issue_tile<DT, ALIGNED>(row, q0, q1, a.V, r);
    float best = -INFINITY;
    int bi = INT_MAX;
    stream_chunk<DT, ALIGNED>(row, q0, q1, a.V, r, [&](uint4 (&t)[kLoads], int qb) {
        run_argmax_tile<DT, kLoads>(t, qb, best, bi);
    });
    block_argmax(best, bi, lds_f, lds_i);
    if (threadIdx.x == 0) {
        RowPart part;
        part.m = best;
        part.idx = bi;
        part.s = 0.0;
        a.part[(int64_t)slot_row * a.nc + chunk] = part;
    }
}

template <int DT>
__global__ __launch_bounds__(kBlock) void argmax_kernel(const Args a)
{
    const int chunk = blockIdx.x % a.nc;
    const int b = (blockIdx.x / a.nc) / (a.K + 1);
    const int j = blockIdx.x / a.nc - b * (a.K + 1);
    const char *row = target_row(a, b, j);
    if (((uintptr_t)row & 15) == 0) argmax_chunk<DT, true>(a, row, b * a.R + j, chunk);
    else argmax_chunk<DT, false>(a, row, b * a.R + j, chunk);
}

// ---------------------------------------------------------------------------
// 2. Accept scan of one sequence ("Kangaroo: Self-Speculative Decoding via
// Shallow Sub-Networks", "3. Lossless Speculative Verification"; greedy:
// "LayerSkip Guide: Early Exit & Self-Speculative Decoding", "2. The Drafting
// and Single-Pass Verification Pipeline"), run by every residual workgroup
// of the sequence (all reach the same outcome; the first writes it).  Thread
// i stands for position i <= K: it takes the statistics of target row i and
// draft row i, makes the accept test of drafted token x_i, and prepares the
// state of the bonus draw as if the scan stopped at i.  The first position
// that stops it (a rejection, an unusable row, or position K) is n; thread n
// publishes.  With a few chunks per row each thread loads and merges its own
// rows' partials; with more, the partials are staged in LDS and merged one row
// per wave first.  The LDS is laid out by accept_lds_layout(), sized from
// (R, K, nc).

struct AcceptLds {
    RowPart *part;  // [R][nc] staged partials (staged merges only)
    Top4 *ptop;     // [K][nc] staged chunk top-4 lists (weighted draft rows)
    double *S;      // [R] S_t, or the draft normaliser D
    float *m;       // [R]
    int *idx;       // [R]
    Top4 *top;      // [K] row top-4 of each weighted draft row
    double *Su;     // [K] a weighted draft row's sum before the beta re-weighting
    int *flag;      // [K + 1] 1: position stops the scan, 3: and its rows are unusable
    SeqState *st;
};

__host__ __device__ inline size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// Offsets of the AcceptLds arrays from `base` (nullptr: sizes only); returns
// the bytes used.
__host__ __device__ inline size_t accept_lds_layout(int R, int K, int nc, bool weighted,
                                                    unsigned char *base, AcceptLds *L)
{
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off = align16(off + bytes);
        return base ? base + o : nullptr;
    };
    static_assert(sizeof(RowPart) == 16 && sizeof(Top4) == 32, "16-byte staging granules");
    const bool staged = nc > kThreadMerge;
    unsigned char *p_part = take(staged ? sizeof(RowPart) * (size_t)R * nc : 0);  // ends on a granule:
    unsigned char *p_ptop = take(staged && weighted ? sizeof(Top4) * (size_t)K * nc : 0);  // contiguous
    unsigned char *p_S = take(staged ? sizeof(double) * (size_t)R : 0);
    unsigned char *p_m = take(staged ? sizeof(float) * (size_t)R : 0);
    unsigned char *p_idx = take(staged ? sizeof(int) * (size_t)R : 0);
    unsigned char *p_top = take(staged && weighted ? sizeof(Top4) * (size_t)K : 0);
    unsigned char *p_Su = take(staged && weighted ? sizeof(double) * (size_t)K : 0);
    unsigned char *p_flag = take(sizeof(int) * (size_t)(K + 1));
    unsigned char *p_st = take(sizeof(SeqState));
    if (L) {
        L->part = reinterpret_cast<RowPart *>(p_part);
        L->ptop = reinterpret_cast<Top4 *>(p_ptop);
        L->S = reinterpret_cast<double *>(p_S);
        L->m = reinterpret_cast<float *>(p_m);
        L->idx = reinterpret_cast<int *>(p_idx);
        L->top = reinterpret_cast<Top4 *>(p_top);
        L->Su = reinterpret_cast<double *>(p_Su);
        L->flag = reinterpret_cast<int *>(p_flag);
        L->st = reinterpret_cast<SeqState *>(p_st);
    }
    return off;
}

// Statistics of the rows of one position: target row i, and for i < K draft
// row i (max, sum S_t or normaliser D, its top-4 when weighted) and the
// logits at the drafted token, which chunk 0's partials carry.
struct PosRows {
    float mt, md, zt, zd;
    double St, D, Du;  // Du: the draft row's sum before the beta re-weighting
    int am;  // target argmax (greedy)
    Top4 top;
};

// Staged merges: the partials and top-4 lists of all 2K + 1 rows in LDS (16-byte
// granules; greedy sequences use the first K + 1 rows) and merge one row per
// wave.
template <int DT>
__device__ __forceinline__ void merge_rows(const Args &a, int b, float T, bool greedy, bool weighted,
                                           const AcceptLds &L)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K, nc = a.nc;
    {
        const int P = a.R * nc;
        const int PT = a.weighted ? K * nc : 0;
        const uint4 *gp = reinterpret_cast<const uint4 *>(a.part + (int64_t)b * a.R * nc);
        const uint4 *gt = reinterpret_cast<const uint4 *>(a.top + (int64_t)b * K * nc);
        uint4 *s4 = reinterpret_cast<uint4 *>(L.part);  // the top-4 lists follow the partials
        const int total4 = P + 2 * PT;                  // a RowPart is one granule, a Top4 two
        for (int base = 0; base < total4; base += 2 * kBlock) {
            const int j0 = base + tid, j1 = base + kBlock + tid;
            uint4 v0 = make_uint4(0u, 0u, 0u, 0u), v1 = v0;
            if (j0 < total4) v0 = j0 < P ? gp[j0] : gt[j0 - P];
            if (j1 < total4) v1 = j1 < P ? gp[j1] : gt[j1 - P];
            if (j0 < total4) s4[j0] = v0;
            if (j1 < total4) s4[j1] = v1;
        }
    }
    __syncthreads();
    const int nrows = greedy ? K + 1 : 2 * K + 1;
    const ExpScale e = make_scale(greedy ? 1.f : T);
    for (int r = wave; r < nrows; r += kWaves) {
        const RowPart *p = L.part + r * nc;
        if (greedy) {
            float M;
            int I;
            merge_argmax(p, nc, M, I);
            if (lane == 0) {
                L.m[r] = M;
                L.idx[r] = I;
            }
        } else if (weighted && r > K) {
            const int i = r - (K + 1);
            float M;
            Top4 rt4;
            double D, Du;
            merge_weighted(p, L.ptop + i * nc, nc, e, (double)a.beta, M, rt4, D, Du);
            if (lane == 0) {
                L.m[r] = M;
                L.S[r] = D;
                L.Su[i] = Du;
                L.top[i] = rt4;
            }
        } else {
            float M;
            double S;
            merge_sum(p, nc, e, M, S);
            if (lane == 0) {
                L.m[r] = M;
                L.S[r] = S;
            }
        }
    }
    __syncthreads();
}

// Rows of at most kThreadMerge chunks: each position thread loads and merges
// its own rows' partials (the same formulas as the wave merges, in chunk
// order).  Loads are issued before the temperature is known.

struct PosLoads {
    RowPart t[kThreadMerge], d[kThreadMerge];
    Top4 top[kThreadMerge];
    double4 tope[kThreadMerge];
};

__device__ __forceinline__ void load_position(const Args &a, int b, int i, PosLoads &pl)
{
    const int K = a.K, nc = a.nc;
    const RowPart *gt = a.part + ((int64_t)b * a.R + i) * nc;
    const RowPart *gd = a.part + ((int64_t)b * a.R + K + 1 + i) * nc;
    const Top4 *gtop = a.top + ((int64_t)b * K + i) * nc;
    const double4 *gtope = a.tope + ((int64_t)b * K + i) * nc;
#pragma unroll
    for (int c = 0; c < kThreadMerge; ++c) {
        pl.t[c] = RowPart{};
        pl.d[c] = RowPart{};
        top_clear(pl.top[c]);
        pl.tope[c] = make_double4(0.0, 0.0, 0.0, 0.0);
        if (c < nc) {
            pl.t[c] = gt[c];
            if (i < K) {
                pl.d[c] = gd[c];
                if (a.weighted) {
                    pl.top[c] = gtop[c];
                    pl.tope[c] = gtope[c];  // one chunk: .x is the row's top-4 mass
                }
            }
        }
    }
}

// M and S of a row from its chunk partials, and each chunk's factor
// f_c = exp2(o_c - o_M) (exactly 1 for a chunk that holds the row max).
__device__ __forceinline__ void thread_merge_sum(const RowPart (&p)[kThreadMerge], int nc, const ExpScale &e,
                                                 float &M, double &S, double (&f)[kThreadMerge])
{
    M = p[0].m;
#pragma unroll
    for (int c = 1; c < kThreadMerge; ++c)
        if (c < nc) M = fmaxf(M, p[c].m);
    const float oM = row_offset(M, e);
    S = 0.0;
#pragma unroll
    for (int c = 0; c < kThreadMerge; ++c) {
        f[c] = 0.0;
        if (c < nc && p[c].m != -INFINITY) {
            const float oc = row_offset(p[c].m, e);
            f[c] = oc == oM ? 1.0 : exp2((double)oc - (double)oM);
            if (p[c].s != 0.0) S += p[c].s * f[c];
        }
    }
}

// Insert (v, i) with mass w into the list t (masses tw); returns the mass
// that leaves it (w itself when (v, i) does not enter).
__device__ __forceinline__ double top_insert_mass(Top4 &t, double (&tw)[4], float v, int i, double w)
{
    if (!better(v, i, t.v[3], t.i[3])) return w;
    const double out = tw[3];
    t.v[3] = v;
    t.i[3] = i;
    tw[3] = w;
#pragma unroll
    for (int k = 3; k > 0; --k) {
        if (better(t.v[k], t.i[k], t.v[k - 1], t.i[k - 1])) {
            const float tv = t.v[k];
            const int ti = t.i[k];
            const double tm = tw[k];
            t.v[k] = t.v[k - 1];
            t.i[k] = t.i[k - 1];
            tw[k] = tw[k - 1];
            t.v[k - 1] = tv;
            t.i[k - 1] = ti;
            tw[k - 1] = tm;
        }
    }
    return out;
}

// Fill the position's row statistics from its loads (sampling rows need the
// temperature's scale e; greedy rows take the argmax).  A weighted draft row
// of several chunks merges the chunks' top-4 lists, whose entries carry their
// masses (relative to their chunk's offset, from the streaming pass): the
// row's top-4 form S_top, every other entry joins the mass outside it.
__device__ __forceinline__ void thread_rows(const PosLoads &pl, int nc, int i, int K, bool greedy,
                                            bool weighted, double beta, const ExpScale &e, PosRows &pr)
{
    pr.zt = __int_as_float(pl.t[0].idx);
    pr.zd = __int_as_float(pl.d[0].idx);
    if (greedy) {
        float v = pl.t[0].m;
        int j = pl.t[0].idx;
#pragma unroll
        for (int c = 1; c < kThreadMerge; ++c)
            if (c < nc && better(pl.t[c].m, pl.t[c].idx, v, j)) {
                v = pl.t[c].m;
                j = pl.t[c].idx;
            }
        pr.mt = v;
        pr.am = j;
        return;
    }
    double f[kThreadMerge];
    thread_merge_sum(pl.t, nc, e, pr.mt, pr.St, f);
    if (i >= K) return;
    double s;
    thread_merge_sum(pl.d, nc, e, pr.md, s, f);
    if (!weighted || nc == 1) {  // one chunk: the streaming pass formed D
        pr.D = pr.Du = s;
        if (weighted) {
            pr.top = pl.top[0];
            pr.Du = s + (1.0 - beta) * pl.tope[0].x;
        }
        return;
    }
    Top4 t = pl.top[0];
    double tw[4] = {pl.tope[0].x * f[0], pl.tope[0].y * f[0], pl.tope[0].z * f[0], pl.tope[0].w * f[0]};
    double extra = 0.0;
#pragma unroll
    for (int c = 1; c < kThreadMerge; ++c)
        if (c < nc) {
            const double w[4] = {pl.tope[c].x * f[c], pl.tope[c].y * f[c], pl.tope[c].z * f[c],
                                 pl.tope[c].w * f[c]};
#pragma unroll
            for (int k = 0; k < 4; ++k) extra += top_insert_mass(t, tw, pl.top[c].v[k], pl.top[c].i[k], w[k]);
        }
    pr.top = t;
    const double st = ((tw[0] + tw[1]) + tw[2]) + tw[3];
    pr.D = (s + extra) + beta * st;
    pr.Du = (s + extra) + st;
}

// Returns the outcome to every thread; `publish` writes the sequence's
// outputs (all but the bonus token of a sampling sequence) and its SeqState.
template <int DT>
__device__ __forceinline__ SeqState accept_sequence(const Args &a, int b, const AcceptLds &L, bool publish)
{
    const int tid = threadIdx.x, lane = tid & 63;
    const int K = a.K, nc = a.nc;  // K: drafts in the row layout, K + 1 output slots
    const uint32_t gb = (uint32_t)(a.b0 + b);  // Philox keys on the sequence's index in the call
    int32_t *out = a.out_tokens + (int64_t)b * (K + 1);

    // one round trip: temperature, this sequence's draft count, drafted token,
    // and (a few chunks per row) the position's partials
    const float T = a.temperature[b];
    const int kb = a.draft_len ? a.draft_len[b] : K;
    const bool kb_ok = kb >= 0 && kb <= K;
    const int Kp = kb_ok ? kb : 0;  // positions 0..Kp; position Kp is the bonus row
    const bool pos = tid <= Kp;     // this thread stands for position tid
    int x = -1;
    if (tid < K) x = a.tokens[(int64_t)b * K + tid];
    PosRows pr;
    pr.mt = pr.md = -INFINITY;
    pr.zt = pr.zd = 0.f;
    pr.St = pr.D = 0.0;
    pr.am = -1;
    top_clear(pr.top);
    const bool greedy = T == 0.f;
    const bool weighted = a.weighted && !greedy;
    const bool own = nc <= kThreadMerge;
    PosLoads pl;
    if (own && tid <= K) load_position(a, b, tid, pl);  // issued before kb is known
    int fail = 0;
    if (!kb_ok) fail = SV_ERR_DRAFT_LEN;
    else if (!temperature_ok(T)) fail = SV_ERR_TEMPERATURE;
    else if (!greedy && Kp > 0 && a.draft == nullptr) fail = SV_ERR_NO_DRAFT;
    if (own && pos && !fail)
        thread_rows(pl, nc, tid, Kp, greedy, weighted, (double)a.beta, make_scale(greedy ? 1.f : T), pr);
    if (!own && !fail) {
        merge_rows<DT>(a, b, T, greedy, weighted, L);
        if (pos) {
            pr.mt = L.m[tid];
            pr.St = L.S[tid];
            pr.am = L.idx[tid];
            pr.zt = __int_as_float(L.part[tid * nc].idx);
        }
        if (tid < Kp && !greedy) {
            pr.md = L.m[K + 1 + tid];
            pr.D = pr.Du = L.S[K + 1 + tid];
            pr.zd = __int_as_float(L.part[(K + 1 + tid) * nc].idx);
            if (weighted) {
                pr.top = L.top[tid];
                pr.Du = L.Su[tid];
            }
        }
    }

    // this position: does it stop the scan, and the bonus state if it is n
    int err = fail;
    bool stop = true;
    float ppt = NAN, ppd = NAN, conf = NAN;
    SeqState cs = {};
    cs.mode = 0;
    if (pos && !fail) {
        if (greedy) {
            if (!isfinite(pr.mt)) err = SV_ERR_ROW;
            stop = err != 0 || tid == Kp || x != pr.am;
        } else {
            const ExpScale e = make_scale(T);
            const float ot = row_offset(pr.mt, e);
            if (!isfinite(pr.mt)) err = SV_ERR_ROW;
            cs.n = tid;
            cs.o_t = ot;
            cs.inv_st = (float)(1.0 / pr.St);
            cs.T = T;
            cs.u_bonus = philox_uniform(a.seed, gb, (uint32_t)tid, kPurposeBonus);
            cs.lbeta = (float)a.log2_beta;
#pragma unroll
            for (int k = 0; k < 4; ++k) cs.top[k] = -1;
            if (tid < Kp) {
                if (!isfinite(pr.md)) err |= SV_ERR_ROW;
                else if (!(pr.D > 0.0)) err |= SV_ERR_DRAFT_MASS;
                const bool x_ok = x >= 0 && x < a.V;
                const bool in_top = weighted && top_has(pr.top, x);
                const float u = philox_uniform(a.seed, gb, (uint32_t)tid, kPurposeAccept);
                const float od = row_offset(pr.md, e);
                const double lq = log2(pr.D / pr.St);
                const bool want_p = publish && (a.aux_pt != nullptr || a.aux_pd != nullptr);
                const bool acc = decide(e, ot, pr.St, od, pr.D, lq, in_top, a.log2_beta, x_ok && err == 0,
                                        pr.zt, pr.zd, u, want_p, ppt, ppd);
                stop = err != 0 || !acc;
                cs.mode = 1;
                cs.o_d = od;
                cs.k2 = ((double)ot - (double)od) - lq;
                // draft confidence max_v p_d (before beta): exp2(m c - o_d) / S_d
                if (a.aux_conf && isfinite(pr.md))
                    conf = (float)(exp2((double)pr.md * e.c64 - (double)od) / pr.Du);
                if (weighted) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) cs.top[k] = pr.top.i[k] == INT_MAX ? -1 : pr.top.i[k];
                }
            } else {
                cs.mode = 2;
            }
        }
    }
    if (pos) L.flag[tid] = stop ? (err ? 3 : 1) : 0;
    __syncthreads();

    // n: the first position that stops the scan (position Kp always does)
    int n = Kp;
    for (int g0 = 0; g0 <= Kp; g0 += 64) {
        const int i = g0 + lane;
        const uint64_t m = __ballot(i <= Kp && L.flag[i] != 0);
        if (m != 0ull) {
            n = g0 + __ffsll((unsigned long long)m) - 1;
            break;
        }
    }
    const bool bad = (L.flag[n] & 2) != 0;  // failed: no outputs but -1
    if (publish && tid <= K) {  // every output slot, past the sequence's drafts too
        int v = -1;
        if (!bad && tid < n) v = x;
        if (!bad && greedy && tid == n) v = pr.am;
        out[tid] = v;
        if (tid < K) {
            const bool keep = !bad && !greedy && tid <= n;
            if (a.aux_pt) a.aux_pt[(int64_t)b * K + tid] = keep ? ppt : NAN;
            if (a.aux_pd) a.aux_pd[(int64_t)b * K + tid] = keep ? ppd : NAN;
            if (a.aux_conf) a.aux_conf[(int64_t)b * K + tid] = (!bad && !greedy) ? conf : NAN;
        }
    }
    if (tid == n) {
        int err_bits = err;
        SeqState st = cs;
        if (bad || greedy) {
            st = SeqState{};
            st.mode = 0;
        }
        if (!bad && n < Kp && (x < 0 || x >= a.V)) err_bits |= SV_ERR_TOKEN;
        *L.st = st;
        if (publish) {
            a.seq[b] = st;
            a.accepted_len[b] = bad ? 0 : n;
            if ((bad || greedy) && a.aux_z) a.aux_z[b] = NAN;
            if (err_bits && a.error_word) atomicOr(a.error_word, err_bits);
        }
    }
    __syncthreads();
    return *L.st;
}

// ---------------------------------------------------------------------------
// 3. Residual ("Kangaroo ...", "3. Lossless Speculative Verification";
// "Speculative Speculative Decoding", "Method"): max(p_t - q', 0) over target
// row n and draft row n, or p_t over target row K after K acceptances.

// Residual of the elements of one 16-byte vector pair; returns the fp32
// pairwise sum of the vector's values and fills r[].
template <int DT, bool TOP, int MODE>
__device__ __forceinline__ float residual_vec(uint4 rt, uint4 rd, int q, const SeqState &st,
                                              const ExpScale &e, const ResidualScale &rs,
                                              float (&r)[Elt<DT>::kVec])
{
    constexpr int VEC = Elt<DT>::kVec;
    float xt[VEC], xd[VEC];
    Elt<DT>::unpack(rt, xt);
    if (MODE == 1) Elt<DT>::unpack(rd, xd);
#pragma unroll
    for (int k = 0; k < VEC; ++k)
        r[k] = residual_at<MODE>(xt[k], MODE == 1 ? xd[k] : 0.f, st, e, rs, rs.k_hi, rs.k_lo);
    if (TOP && MODE == 1) {
        // a vector holding one of the draft's top-4 tokens (at most four per
        // row): recompute that token with its beta-weighted offset
        if (q == rs.tq[0] || q == rs.tq[1] || q == rs.tq[2] || q == rs.tq[3]) {
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const int v = q * VEC + k;
                if (v == st.top[0] || v == st.top[1] || v == st.top[2] || v == st.top[3])
                    r[k] = residual_at<MODE>(xt[k], xd[k], st, e, rs, rs.kt_hi, rs.kt_lo);
            }
        }
    }
    float s[VEC];
#pragma unroll
    for (int k = 0; k < VEC; ++k) s[k] = r[k];
#pragma unroll
    for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
        for (int k = 0; k < w; ++k) s[k] += s[k + w];
    return s[0];
}

// Residual mass of the slots [s_begin, s_end) of the row pair into slot[].
// Slot s covers the vectors [s*gs*kSlotVec, (s+1)*gs*kSlotVec); the NW waves
// of the workgroup take the slots in turn, and a wave's 64 lanes read
// kSlotVec consecutive vectors (1 KiB of each row) per load.  Item f = t*gs +
// j of a wave is unit j of its t-th slot, kResLoads items per batch (a second
// batch in flight measured slower: it costs occupancy).  FAST (aligned rows
// of whole vectors) loads without any branch (indices clamped into the row;
// items that are not live add nothing and load the batch's first vector
// again, so they cost no HBM traffic), so that no loaded register passes a
// branch join, which would make it wait for its load.  Each slot is summed
// by one wave in a fixed order (fp32 within a vector, fp64 across vectors
// and lanes).
template <int DT, int MODE>
struct ResBatch {
    uint4 rt[kResLoads], rd[kResLoads];
    int q[kResLoads], t[kResLoads];
    bool end[kResLoads], live[kResLoads];
};

template <int DT, int NW, int MODE, bool FAST>
__device__ __forceinline__ void residual_issue(ResBatch<DT, MODE> &B, const char *trow, const char *drow,
                                               bool ta, bool da, int V, int nvec, int s_begin, int gs,
                                               int items, int f0, int &t, int &j)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < kResLoads; ++u) {
        const int s = s_begin + wave + NW * t;
        B.q[u] = (s * gs + j) * kSlotVec + lane;
        B.t[u] = t;
        B.end[u] = j == gs - 1;
        B.live[u] = f0 + u < items && B.q[u] < nvec;
        if (++j == gs) {
            j = 0;
            ++t;
        }
    }
    if (FAST) {
        // the re-read streams too: nontemporal loads
#pragma unroll
        for (int u = 0; u < kResLoads; ++u)
            B.rt[u] = load16_stream(trow + (size_t)min(B.live[u] ? B.q[u] : B.q[0], nvec - 1) * 16);
        if (MODE == 1) {
#pragma unroll
            for (int u = 0; u < kResLoads; ++u)
                B.rd[u] = load16_stream(drow + (size_t)min(B.live[u] ? B.q[u] : B.q[0], nvec - 1) * 16);
        }
    } else {
        load_units<DT, kResLoads>(trow, ta, B.q, B.live, nvec, V, B.rt);
        if (MODE == 1) load_units<DT, kResLoads>(drow, da, B.q, B.live, nvec, V, B.rd);
    }
}

template <int DT, bool TOP, int NW, int MODE>
__device__ __forceinline__ void residual_consume(const ResBatch<DT, MODE> &B, int items, int f0, int s_begin,
                                                 const SeqState &st, const ExpScale &e,
                                                 const ResidualScale &rs, double &acc, double *slot)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int u = 0; u < kResLoads; ++u) {
        if (f0 + u >= items) break;
        float r[Elt<DT>::kVec];
        const float sum = residual_vec<DT, TOP, MODE>(B.rt[u], B.rd[u], B.q[u], st, e, rs, r);
        acc += B.live[u] ? (double)sum : 0.0;
        if (B.end[u]) {
            const double tot = wave_sum(acc);
            if (lane == 0) slot[s_begin + wave + NW * B.t[u]] = tot;
            acc = 0.0;
        }
    }
}

template <int DT, bool TOP, int NW, int MODE, bool FAST>
__device__ __forceinline__ void residual_slots_impl(const char *trow, const char *drow, int V, int nvec,
                                                    int s_begin, int s_end, int gs, const SeqState &st,
                                                    const ExpScale &e, const ResidualScale &rs,
                                                    double *slot)
{
    const int wave = threadIdx.x >> 6;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    const int ns = s_end - s_begin;
    const int my_slots = ns > wave ? (ns - wave + NW - 1) / NW : 0;
    const int items = my_slots * gs;
    if (items == 0) return;
    double acc = 0.0;
    int t = 0, j = 0;
    for (int f0 = 0; f0 < items; f0 += kResLoads) {
        ResBatch<DT, MODE> A;
        residual_issue<DT, NW, MODE, FAST>(A, trow, drow, ta, da, V, nvec, s_begin, gs, items, f0, t, j);
        residual_consume<DT, TOP, NW, MODE>(A, items, f0, s_begin, st, e, rs, acc, slot);
    }
}

template <int DT, bool TOP, int NW, int MODE>
__device__ __forceinline__ void residual_slots(const char *trow, const char *drow, int V, int nvec,
                                               int s_begin, int s_end, int gs, const SeqState &st,
                                               const ExpScale &e, const ResidualScale &rs, double *slot)
{
    const bool fast = ((uintptr_t)trow & 15) == 0 && (MODE == 2 || ((uintptr_t)drow & 15) == 0) &&
                      V % Elt<DT>::kVec == 0;
    if (fast)
        residual_slots_impl<DT, TOP, NW, MODE, true>(trow, drow, V, nvec, s_begin, s_end, gs, st, e, rs, slot);
    else
        residual_slots_impl<DT, TOP, NW, MODE, false>(trow, drow, V, nvec, s_begin, s_end, gs, st, e, rs, slot);
}

// One workgroup per (sequence, group of a.spg slots): the accept scan, then
// the group's slot masses.
template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void residual_kernel(const Args a)
{
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    const int b = blockIdx.x / a.ng;
    const int g = blockIdx.x - b * a.ng;
    AcceptLds L;
    accept_lds_layout(a.R, a.K, a.nc, a.weighted != 0, dyn_lds, &L);
    const SeqState st = accept_sequence<DT>(a, b, L, g == 0);
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const ResidualScale rs = make_residual_scale<Elt<DT>::kVec>(st, e);
    const char *trow = target_row(a, b, st.n);
    const char *drow = st.mode == 1 ? draft_row(a, b, st.n) : trow;
    const int s0 = g * a.spg, s1 = min(a.nslot, s0 + a.spg);
    double *slot = a.slot + (int64_t)b * a.nslot;
    if (st.mode == 1)
        residual_slots<DT, TOP, kWaves, 1>(trow, drow, a.V, a.nvec, s0, s1, a.gs, st, e, rs, slot);
    else
        residual_slots<DT, TOP, kWaves, 2>(trow, drow, a.V, a.nvec, s0, s1, a.gs, st, e, rs, slot);
}

// The accept scan alone, one workgroup per sequence: it writes the outputs
// (all but a sampling sequence's bonus token) and the sequence's outcome.
template <int DT>
__global__ __launch_bounds__(kBlock) void accept_kernel(const Args a)
{
    extern __shared__ __align__(16) unsigned char dyn_lds[];
    AcceptLds L;
    accept_lds_layout(a.R, a.K, a.nc, a.weighted != 0, dyn_lds, &L);
    accept_sequence<DT>(a, blockIdx.x, L, true);
}

// ---------------------------------------------------------------------------
// 4. Bonus draw by inverse CDF in ascending token id: the smallest v with
// C(v) >= u * Z, Z the total residual mass, first over the slot masses, then
// over the elements of the selected slot; zero mass (only through rounding)
// falls back to p_t.

// Ordered scan of the vectors [q0, q1) of the row pair, starting from `base`,
// for the first element with mass whose running sum reaches `thr`.  Returns
// that element, or INT_MAX when rounding leaves `thr` above the range; `last`
// receives the last element of the range with positive mass.
template <int DT, bool TOP, int MODE>
__device__ __forceinline__ int scan_range(const char *trow, const char *drow, int V, int nvec, int q0, int q1,
                          double base, double thr, const SeqState &st, const ExpScale &e,
                          const ResidualScale &rs, int &last, double *lds_d, int *lds_i)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    last = -1;
    for (int qb = q0; qb < q1; qb += kBlock) {
        const int q = qb + tid;
        const bool live = q < q1;
        const uint4 rt = live ? load_one<DT>(trow, ta, q, nvec, V) : neg_inf_raw<DT>();
        uint4 rd = neg_inf_raw<DT>();
        if (MODE == 1 && live) rd = load_one<DT>(drow, da, q, nvec, V);
        float r[VEC];
        residual_vec<DT, TOP, MODE>(rt, rd, q, st, e, rs, r);
        double pre[VEC];
        double acc = 0.0;
        int mylast = -1;
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            acc += (double)r[k];
            pre[k] = acc;
            if (r[k] > 0.f) mylast = q * VEC + k;
        }
        double tile_total;
        const double exc = block_exclusive_scan(acc, tile_total, lds_d);
        int cand = INT_MAX;
#pragma unroll
        for (int k = VEC - 1; k >= 0; --k)
            if (r[k] > 0.f && base + exc + pre[k] >= thr) cand = q * VEC + k;
        cand = block_min_int(cand, lds_i);
        last = max(last, block_max_int(mylast, lds_i));
        if (cand != INT_MAX) return cand;
        base += tile_total;
    }
    return INT_MAX;
}

// Inverse CDF over the slot masses in slot[0..nslot): returns the token (-1
// when the mass is 0) and Z, the total mass.
template <int DT, bool TOP, int MODE>
__device__ __forceinline__ int draw_token(const char *trow, const char *drow, int V, int nvec, int nslot, int gs,
                          float u, const SeqState &st, const ExpScale &e, const ResidualScale &rs,
                          const double *slot, double &Z, double *lds_d, int *lds_i)
{
    const int tid = threadIdx.x;
    const int per = (nslot + kBlock - 1) / kBlock;
    const int s0 = min(nslot, tid * per), s1 = min(nslot, s0 + per);
    double loc = 0.0;
    for (int s = s0; s < s1; ++s) loc += slot[s];
    double total;
    const double exc = block_exclusive_scan(loc, total, lds_d);
    Z = total;
    if (!(total > 0.0)) return -1;
    const double thr = (double)u * total;
    // the first slot with mass whose inclusive prefix reaches thr, else (by
    // rounding between summation orders) the last slot with mass
    int cand = INT_MAX, lastpos = -1;
    double cbase = 0.0, lbase = 0.0, run = exc;
    for (int s = s0; s < s1; ++s) {
        const double v = slot[s];
        if (v > 0.0) {
            if (cand == INT_MAX && run + v >= thr) {
                cand = s;
                cbase = run;
            }
            lastpos = s;
            lbase = run;
        }
        run += v;
    }
    const int c = block_min_int(cand, lds_i);
    const int lp = block_max_int(lastpos, lds_i);
    const int sel = c != INT_MAX ? c : lp;
    if (sel < 0) return -1;  // no slot with mass: only NaN masses get here
    if (sel >= s0 && sel < s1) lds_d[kWaves] = (c != INT_MAX) ? cbase : lbase;
    __syncthreads();
    const double base = lds_d[kWaves];
    __syncthreads();
    const int q0 = sel * gs * kSlotVec, q1 = min(nvec, q0 + gs * kSlotVec);
    int last;
    const int tok = scan_range<DT, TOP, MODE>(trow, drow, V, nvec, q0, q1, base, thr, st, e, rs, last,
                                              lds_d, lds_i);
    return tok != INT_MAX ? tok : last;
}

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void bonus_kernel(const Args a)
{
    __shared__ double slot[kMaxResSlots];
    __shared__ double lds_d[kWaves + 1];
    __shared__ int lds_i[kWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // the slot masses are requested together with the sequence's state
    const double *gslot = a.slot + (int64_t)b * a.nslot;
    for (int s = tid; s < a.nslot; s += kBlock) slot[s] = gslot[s];
    const SeqState st = a.seq[b];
    __syncthreads();
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const ResidualScale rs = make_residual_scale<Elt<DT>::kVec>(st, e);
    const char *trow = target_row(a, b, st.n);
    const char *drow = st.mode == 1 ? draft_row(a, b, st.n) : trow;
    double Z;
    int token = st.mode == 1
                    ? draw_token<DT, TOP, 1>(trow, drow, a.V, a.nvec, a.nslot, a.gs, st.u_bonus, st, e, rs,
                                             slot, Z, lds_d, lds_i)
                    : draw_token<DT, TOP, 2>(trow, drow, a.V, a.nvec, a.nslot, a.gs, st.u_bonus, st, e, rs,
                                             slot, Z, lds_d, lds_i);
    if (token < 0) {
        // zero residual mass: the slot masses of p_t, by this workgroup alone
        residual_slots<DT, TOP, kWaves, 2>(trow, trow, a.V, a.nvec, 0, a.nslot, a.gs, st, e, rs, slot);
        __syncthreads();
        token = draw_token<DT, TOP, 2>(trow, trow, a.V, a.nvec, a.nslot, a.gs, st.u_bonus, st, e, rs, slot,
                                       Z, lds_d, lds_i);
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + st.n] = token;
        if (a.aux_z) a.aux_z[b] = (float)(Z * (double)st.inv_st);
    }
}

// Row-statistics entry point: finish the merge of each row's partials.
__global__ __launch_bounds__(64) void rowstats_finish_kernel(const Args a)
{
    const int r = blockIdx.x;
    const float T = a.temperature[r];
    const RowPart *p = a.part + (int64_t)r * a.nc;
    const int lane = threadIdx.x;
    if (!temperature_ok(T)) {
        if (lane == 0) {
            a.rs_max[r] = NAN;
            a.rs_logsum[r] = NAN;
            a.rs_argmax[r] = -1;
        }
        return;
    }
    if (T == 0.f) {
        float M;
        int I;
        merge_argmax(p, a.nc, M, I);
        if (lane == 0) {
            a.rs_max[r] = M;
            a.rs_logsum[r] = NAN;
            a.rs_argmax[r] = I;
        }
    } else {
        const ExpScale e = make_scale(T);
        float M;
        double S;
        merge_sum(p, a.nc, e, M, S);
        if (lane == 0) {
            // S is relative to fp32(M c); the log-sum is relative to M c
            a.rs_max[r] = M;
            a.rs_logsum[r] = log(S) + ((double)row_offset(M, e) - (double)M * e.c64) * 0.6931471805599453;
            a.rs_argmax[r] = -1;
        }
    }
}

// The streaming pass's grid, rows, chunks, loads and tiles with its
// arithmetic taken out (each thread folds its vectors into one word): the
// floor that pass is measured against.  `sink` is written for one fold value
// in 2^32 only, which keeps the loads.
template <int DT>
__global__ __launch_bounds__(kBlock) void stream_probe_kernel(const Args a, uint32_t *sink)
{
    const int rl = a.draft ? a.R : a.K + 1;
    const int chunk = blockIdx.x % a.nc;
    const int b = (blockIdx.x / a.nc) / rl;
    const int j = blockIdx.x / a.nc - b * rl;
    const bool is_draft = j > a.K;
    const int i = is_draft ? j - (a.K + 1) : j;
    const char *row = is_draft ? draft_row(a, b, i) : target_row(a, b, i);
    const int q0 = chunk * a.cvec;
    const int q1 = min(a.nvec, q0 + a.cvec);
    uint32_t acc = 0;
    auto fold = [&](uint4 (&t)[kLoads], int) {
#pragma unroll
        for (int u = 0; u < kLoads; ++u) acc ^= t[u].x ^ t[u].y ^ t[u].z ^ t[u].w;
    };
    uint4 r[kLoads];
    if (((uintptr_t)row & 15) == 0) {
        issue_tile<DT, true>(row, q0, q1, a.V, r);
        stream_chunk<DT, true>(row, q0, q1, a.V, r, fold);
    } else {
        issue_tile<DT, false>(row, q0, q1, a.V, r);
        stream_chunk<DT, false>(row, q0, q1, a.V, r, fold);
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

__global__ void uniforms_kernel(uint64_t seed, int32_t B, int32_t P, float *out)
{
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t total = (int64_t)B * P * 2;
    if (t >= total) return;
    const uint32_t purpose = (uint32_t)(t & 1);
    const int64_t bp = t >> 1;
    const uint32_t pos = (uint32_t)(bp % P);
    const uint32_t b = (uint32_t)(bp / P);
    out[t] = philox_uniform(seed, b, pos, purpose);
}

// ---------------------------------------------------------------------------
// Host launchers (one sub-batch of at most kMaxSeqPerLaunch sequences).

template <int DT, bool TOP>
static void launch_all(const Args &a, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    const unsigned grid = (unsigned)((int64_t)a.B * (a.draft ? a.R : a.K + 1) * a.nc);
    const bool greedy_only = !a.draft && a.K > 0 && !a.draft_len;
    if (greedy_only) {
        if (begin || end)  // the dispatch itself stamps the kernel's start and end
            hipExtLaunchKernelGGL(argmax_kernel<DT>, dim3(grid), dim3(kBlock), 0, s, begin, end, 0, a);
        else
            argmax_kernel<DT><<<grid, kBlock, 0, s>>>(a);
    } else if (begin || end) {
        hipExtLaunchKernelGGL(stats_kernel<DT, TOP>, dim3(grid), dim3(kBlock), 0, s, begin, end, 0, a);
    } else {
        stats_kernel<DT, TOP><<<grid, kBlock, 0, s>>>(a);
    }
    const size_t lds = accept_lds_layout(a.R, a.K, a.nc, a.weighted != 0, nullptr, nullptr);
    if (greedy_only) {
        // every sequence is greedy or fails: the accept scan alone finishes
        // them, one workgroup per sequence, with no residual pass or bonus draw
        accept_kernel<DT><<<(unsigned)a.B, kBlock, lds, s>>>(a);
        return;
    }
    residual_kernel<DT, TOP><<<(unsigned)((int64_t)a.B * a.ng), kBlock, lds, s>>>(a);
    bonus_kernel<DT, TOP><<<(unsigned)a.B, kBlock, 0, s>>>(a);
}

void launch_verify(const Args &a, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    if (a.dtype == SV_F32) {
        if (a.weighted) launch_all<0, true>(a, s, begin, end);
        else launch_all<0, false>(a, s, begin, end);
    } else {
        if (a.weighted) launch_all<1, true>(a, s, begin, end);
        else launch_all<1, false>(a, s, begin, end);
    }
}

void launch_stats(const Args &a, hipStream_t s)
{
    const unsigned grid = (unsigned)((int64_t)a.B * (a.draft ? a.R : a.K + 1) * a.nc);
    if (a.dtype == SV_F32) {
        if (a.weighted) stats_kernel<0, true><<<grid, kBlock, 0, s>>>(a);
        else stats_kernel<0, false><<<grid, kBlock, 0, s>>>(a);
    } else {
        if (a.weighted) stats_kernel<1, true><<<grid, kBlock, 0, s>>>(a);
        else stats_kernel<1, false><<<grid, kBlock, 0, s>>>(a);
    }
}

void launch_rowstats(const Args &a, hipStream_t s)
{
    const unsigned grid = (unsigned)((int64_t)a.B * a.R * a.nc);
    if (a.dtype == SV_F32) stats_kernel<0, false><<<grid, kBlock, 0, s>>>(a);
    else stats_kernel<1, false><<<grid, kBlock, 0, s>>>(a);
    rowstats_finish_kernel<<<(unsigned)a.B, 64, 0, s>>>(a);
}

void launch_stream_probe(const Args &a, uint32_t *sink, hipStream_t s, hipEvent_t begin, hipEvent_t end)
{
    const unsigned grid = (unsigned)((int64_t)a.B * (a.draft ? a.R : a.K + 1) * a.nc);
    if (a.dtype == SV_F32)
        hipExtLaunchKernelGGL(stream_probe_kernel<0>, dim3(grid), dim3(kBlock), 0, s, begin, end, 0, a, sink);
    else
        hipExtLaunchKernelGGL(stream_probe_kernel<1>, dim3(grid), dim3(kBlock), 0, s, begin, end, 0, a, sink);
}

void launch_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, hipStream_t s)
{
    const int64_t total = (int64_t)B * P * 2;
    uniforms_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(seed, B, P, out);
}

}  // namespace sv
