// specverify.hip -- libspecverify: the speculative-sampling verify step on
// AMD Instinct MI355X (gfx950).  The operation and its conventions are stated
// in include/specverify.h; the per-step sources are cited at each kernel.
//
// One call enqueues four kernels on the caller's stream:
//   1. stats_kernel     streams every needed logit row once in 16-byte
//                       vectors and reduces each (row, chunk) to a partial:
//                       (max, sum of exp2((z - max) * log2e / T)) for
//                       sampling rows, (max, lowest argmax) for greedy rows,
//                       plus the chunk's top-4 for beta-weighted draft rows.
//   2. accept_kernel    one workgroup per sequence merges the partials of its
//                       rows in fp64, forms every accept ratio in the log
//                       domain, draws the Philox uniforms, finds the first
//                       rejection n and writes the accepted prefix.
//   3. residual_kernel  re-reads target row n and draft row n (or target row K
//                       after K acceptances) in chunks and sums the residual
//                       max(p_t - q', 0) (or p_t) per chunk in fp64.
//   4. bonus_kernel     one workgroup per sequence scans the chunk sums, then
//                       the selected chunk, for the smallest token whose
//                       running residual sum reaches u * Z.
// The workspace holds the partials between kernels; nothing is allocated.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>

#include "specverify.h"
#include "sv_device.h"

namespace sv {

constexpr int kMaxK = 128;              // drafted positions per sequence
constexpr int kMaxSlots = 2 * kMaxK + 1;
constexpr int kMaxChunks = 1024;        // streaming chunks per row
constexpr int kFillBlocks = 2048;       // workgroups a streaming grid aims for
constexpr uint32_t kPurposeAccept = 0u, kPurposeBonus = 1u;

// One (row, chunk) partial of the streaming pass.
struct RowPart {
    float m;      // chunk maximum
    int32_t idx;  // lowest index attaining m (greedy rows)
    double s;     // sum of exp2((z - m) * log2e / T) over the chunk (sampling rows)
};

// Per-sequence outcome of the accept scan, read by the residual and bonus kernels.
struct SeqState {
    int32_t n;     // accepted drafts
    int32_t mode;  // 0: nothing to draw, 1: residual max(p_t - q', 0), 2: p_t alone
    float m_t, m_d;
    float inv_st;  // 1 / S_t
    float inv_sd;  // 1 / (S_d * N)
    float beta;
    float u_bonus;
    int32_t top[4];
    float T;
    int32_t pad[3];
};
static_assert(sizeof(SeqState) == 64, "SeqState layout");

struct Plan {
    int32_t B, K, V, dtype, vec, R;
    int32_t nvec;           // 16-byte vectors per row (the last may be partial)
    int32_t nc, cvec;       // streaming chunks per row, vectors per chunk
    int32_t ncr, rvec;      // residual chunks per sequence, vectors per residual chunk
    int64_t row_bytes;
    size_t off_part, off_top, off_seq, off_res, bytes;
};

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan *p)
{
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return false;
    p->B = B;
    p->K = K;
    p->V = V;
    p->dtype = dtype;
    const int elt = dtype == SV_F32 ? 4 : 2;
    p->vec = 16 / elt;
    p->R = 2 * K + 1;
    p->row_bytes = (int64_t)V * elt;
    p->nvec = (int32_t)(((int64_t)V + p->vec - 1) / p->vec);
    const int64_t rows = std::max<int64_t>(1, (int64_t)B * p->R);
    int64_t nc = (kFillBlocks + rows - 1) / rows;
    const int64_t nc_max = std::max<int64_t>(1, p->nvec / kBlock);  // >= one vector per thread
    nc = std::min<int64_t>(std::min<int64_t>(nc, nc_max), kMaxChunks);
    p->cvec = (int32_t)((p->nvec + nc - 1) / nc);
    // a row longer than kMaxChunks * cvec cannot occur: nc was capped, cvec grows instead
    p->nc = (p->nvec + p->cvec - 1) / p->cvec;
    const int64_t ncr_want = (kFillBlocks + std::max(B, 1) - 1) / std::max(B, 1);
    int64_t rvec = (p->nvec + ncr_want - 1) / ncr_want;
    rvec = std::max<int64_t>(rvec, kBlock);
    rvec = std::min<int64_t>(rvec, (int64_t)kBlock * kLoads);
    p->rvec = (int32_t)rvec;
    p->ncr = (int32_t)((p->nvec + rvec - 1) / rvec);
    // every grid must fit a 32-bit workgroup count
    if ((int64_t)B * p->R * p->nc >= ((int64_t)1 << 31) || (int64_t)B * p->ncr >= ((int64_t)1 << 31))
        return false;
    size_t off = 0;
    p->off_part = off;
    off = align256(off + sizeof(RowPart) * (size_t)B * p->R * p->nc);
    p->off_top = off;
    off = align256(off + sizeof(Top4) * (size_t)B * K * p->nc);
    p->off_seq = off;
    off = align256(off + sizeof(SeqState) * (size_t)B);
    p->off_res = off;
    off = align256(off + sizeof(double) * (size_t)B * p->ncr);
    p->bytes = std::max<size_t>(off, 256);
    return true;
}

struct Args {
    const char *target;
    const char *draft;
    const int32_t *tokens;
    const float *temperature;
    int32_t B, K, V, R, nvec, nc, cvec, ncr, rvec, dtype;
    int64_t row_bytes;
    uint64_t seed;
    float beta;
    int32_t weighted;
    int32_t *accepted_len;
    int32_t *out_tokens;
    RowPart *part;
    Top4 *top;
    SeqState *seq;
    double *res;
    float *aux_pt, *aux_pd, *aux_z;
    int32_t *error_word;
    // row-statistics entry point outputs
    float *rs_max;
    double *rs_logsum;
    int32_t *rs_argmax;
};

__device__ __forceinline__ bool temperature_ok(float T) { return T >= 0.f && T != INFINITY; }

__device__ __forceinline__ const char *target_row(const Args &a, int b, int i)
{
    return a.target + ((int64_t)b * (a.K + 1) + i) * a.row_bytes;
}

__device__ __forceinline__ const char *draft_row(const Args &a, int b, int i)
{
    return a.draft + ((int64_t)b * a.K + i) * a.row_bytes;
}

// ---------------------------------------------------------------------------
// 1. Streaming pass: one workgroup per (row slot, chunk).  Row slots of a
// sequence are target rows 0..K then draft rows 0..K-1.  Per lane the online
// (max, sum) is kept in (fp32, fp64): each 16-byte vector's exponentials are
// summed in fp32 against the lane's running max and added to an fp64 sum,
// which is rescaled in fp64 when the max grows.  Lanes visit their elements
// in increasing index order, so argmax and top-4 ties resolve to the lowest
// token id.  (Row softmax: "Kangaroo: Self-Speculative Decoding via Shallow
// Sub-Networks", "3. Lossless Speculative Verification", p_i and q_i.)

template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void stats_kernel(const Args a)
{
    using E = Elt<DT>;
    constexpr int VEC = E::kVec;
    __shared__ float lds_f[kWaves * 4];
    __shared__ int lds_i[kWaves * 4];
    __shared__ double lds_d[kWaves];

    const int tid = threadIdx.x;
    const int chunk = blockIdx.x % a.nc;
    const int slot_row = blockIdx.x / a.nc;
    const int b = slot_row / a.R;
    const int j = slot_row - b * a.R;
    if (blockIdx.x == 0 && tid == 0 && a.error_word) *a.error_word = 0;

    const float T = a.temperature[b];
    if (!temperature_ok(T)) return;
    const bool greedy = T == 0.f;
    const bool is_draft = j > a.K;
    if (is_draft && (greedy || a.draft == nullptr)) return;
    const int i = is_draft ? j - (a.K + 1) : j;
    const char *row = is_draft ? draft_row(a, b, i) : target_row(a, b, i);
    const bool aligned = ((uintptr_t)row & 15) == 0;
    const int q0 = chunk * a.cvec;
    const int q1 = min(a.nvec, q0 + a.cvec);
    RowPart *out = a.part + (int64_t)slot_row * a.nc + chunk;

    if (greedy) {
        float best = -INFINITY;
        int bi = INT_MAX;
        for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
            float x[kLoads][VEC];
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int q = qb + u * kBlock + tid;
                if (q < q1) load_vec<DT>(row, aligned, q, a.V, x[u]);
            }
#pragma unroll
            for (int u = 0; u < kLoads; ++u) {
                const int q = qb + u * kBlock + tid;
                if (q >= q1) continue;
                float mx = x[u][0];
#pragma unroll
                for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[u][k]);
                if (mx > best) {
                    int kk = VEC - 1;
#pragma unroll
                    for (int k = VEC - 1; k >= 0; --k)
                        if (x[u][k] == mx) kk = k;
                    best = mx;
                    bi = q * VEC + kk;
                }
            }
        }
        block_argmax(best, bi, lds_f, lds_i);
        if (tid == 0) {
            RowPart r;
            r.m = best;
            r.idx = bi;
            r.s = 0.0;
            *out = r;
        }
        return;
    }

    const ExpScale e = make_scale(T);
    const bool track_top = TOP && is_draft;
    float m = -INFINITY;
    double s = 0.0;
    Top4 t4;
    top_clear(t4);
    for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
        float x[kLoads][VEC];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q < q1) load_vec<DT>(row, aligned, q, a.V, x[u]);
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q >= q1) continue;
            float mx = x[u][0];
#pragma unroll
            for (int k = 1; k < VEC; ++k) mx = fmaxf(mx, x[u][k]);
            if (mx > m) {
                if (s != 0.0) s *= exp2(((double)m - (double)mx) * e.c64);
                m = mx;
            }
            if (m != -INFINITY) {
                float acc[VEC];
#pragma unroll
                for (int k = 0; k < VEC; ++k) acc[k] = exp_scaled(x[u][k], m, e);
#pragma unroll
                for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                    for (int k = 0; k < w; ++k) acc[k] += acc[k + w];
                s += (double)acc[0];
            }
            if (track_top) {
                if (mx > t4.v[3] || (mx == t4.v[3] && t4.i[3] == INT_MAX)) {
#pragma unroll
                    for (int k = 0; k < VEC; ++k) top_insert(t4, x[u][k], q * VEC + k);
                }
            }
        }
    }
    const float M = block_max(m, lds_f);
    const double scaled = (m == -INFINITY) ? 0.0 : s * exp2(((double)m - (double)M) * e.c64);
    const double S = block_sum(scaled, lds_d);
    if (tid == 0) {
        RowPart r;
        r.m = M;
        r.idx = -1;
        r.s = S;
        *out = r;
    }
    if (track_top) {
        const Top4 w = wave_top4(t4);
        const int lane = tid & 63, wave = tid >> 6;
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lds_f[wave * 4 + k] = w.v[k];
                lds_i[wave * 4 + k] = w.i[k];
            }
        }
        __syncthreads();
        if (wave == 0) {
            Top4 c;
            top_clear(c);
            if (lane < kWaves * 4) {
                c.v[0] = lds_f[lane];
                c.i[0] = lds_i[lane];
            }
            const Top4 r = wave_top4(c);
            if (lane == 0) a.top[((int64_t)b * a.K + i) * a.nc + chunk] = r;
        }
    }
}

// ---------------------------------------------------------------------------
// Wave-level merges of a row's chunk partials (same code for target and draft
// rows, so equal rows merge to equal values).

__device__ __forceinline__ void merge_sum(const RowPart *p, int nc, double c64, float &M, double &S)
{
    const int lane = threadIdx.x & 63;
    float m = -INFINITY;
    for (int c = lane; c < nc; c += 64) m = fmaxf(m, p[c].m);
    m = wave_max(m);
    double s = 0.0;
    for (int c = lane; c < nc; c += 64) {
        const RowPart r = p[c];
        if (r.m != -INFINITY) s += r.s * exp2(((double)r.m - (double)m) * c64);
    }
    S = wave_sum(s);
    M = m;
}

__device__ __forceinline__ void merge_argmax(const RowPart *p, int nc, float &M, int &I)
{
    const int lane = threadIdx.x & 63;
    float v = -INFINITY;
    int i = INT_MAX;
    for (int c = lane; c < nc; c += 64) {
        const RowPart r = p[c];
        if (better(r.m, r.idx, v, i)) {
            v = r.m;
            i = r.idx;
        }
    }
    wave_argmax(v, i);
    M = v;
    I = i;
}

__device__ __forceinline__ Top4 merge_top(const Top4 *p, int nc)
{
    const int lane = threadIdx.x & 63;
    Top4 t;
    top_clear(t);
    for (int c = lane; c < nc; c += 64) {
        const Top4 r = p[c];
#pragma unroll
        for (int k = 0; k < 4; ++k) top_insert(t, r.v[k], r.i[k]);
    }
    return wave_top4(t);
}

// ---------------------------------------------------------------------------
// 2. Accept scan, one workgroup per sequence.
// Sampling ("Kangaroo ...", "3. Lossless Speculative Verification"; glossary
// "speculative decoding llm", "Why It Produces Identical Outputs"): accept x_i
// iff u_i <= p_i(x_i) / q'_i(x_i), the ratio formed in fp64 as
//   ln p - ln q' = (z_t(x) - m_t)/T - ln S_t - (z_d(x) - m_d)/T + ln S_d
//                  - ln w(x) + ln N,
// with the beta weights w and N = sum_v w(v) q(v) of the Saguaro-style draft
// ("Speculative Speculative Decoding", "Method").  Every position's ratio is
// formed in parallel; n is the first rejection.
// Greedy ("LayerSkip Guide ...", "2. The Drafting and Single-Pass
// Verification Pipeline"): accept while x_i equals the target argmax.

__global__ __launch_bounds__(kBlock) void accept_kernel(const Args a)
{
    __shared__ float s_m[kMaxSlots];
    __shared__ double s_S[kMaxSlots];
    __shared__ int s_idx[kMaxSlots];
    __shared__ Top4 s_top[kMaxK];
    __shared__ int s_acc[kMaxK];
    __shared__ int s_err[kMaxK];
    __shared__ float s_pt[kMaxK], s_pd[kMaxK];
    __shared__ double s_invsd[kMaxK];

    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int K = a.K;
    int32_t *out = a.out_tokens + (int64_t)b * (K + 1);
    const float T = a.temperature[b];
    const bool greedy = T == 0.f;

    int fail = 0;
    if (!temperature_ok(T)) fail = SV_ERR_TEMPERATURE;
    else if (!greedy && K > 0 && a.draft == nullptr) fail = SV_ERR_NO_DRAFT;

    if (!fail) {
        const int nslots = greedy ? K + 1 : 2 * K + 1;
        const double c64 = greedy ? 0.0 : kLog2e / (double)T;
        for (int slot = wave; slot < nslots; slot += kWaves) {
            const RowPart *p = a.part + ((int64_t)b * a.R + slot) * a.nc;
            if (greedy) {
                float M;
                int I;
                merge_argmax(p, a.nc, M, I);
                if (lane == 0) {
                    s_m[slot] = M;
                    s_idx[slot] = I;
                }
            } else {
                float M;
                double S;
                merge_sum(p, a.nc, c64, M, S);
                if (lane == 0) {
                    s_m[slot] = M;
                    s_S[slot] = S;
                }
                if (a.weighted && slot > K) {
                    const int i = slot - (K + 1);
                    const Top4 t = merge_top(a.top + ((int64_t)b * K + i) * a.nc, a.nc);
                    if (lane == 0) s_top[i] = t;
                }
            }
        }
        __syncthreads();

        if (!greedy && tid < K) {
            const int i = tid;
            const double Td = (double)T;
            const float mt = s_m[i], md = s_m[K + 1 + i];
            const double St = s_S[i], Sd = s_S[K + 1 + i];
            int err = 0;
            if (!isfinite(mt)) err |= SV_ERR_ROW;
            double lnN = 0.0;
            bool in_top = false;
            const int x = a.tokens[(int64_t)b * K + i];
            if (!isfinite(md)) {
                err |= SV_ERR_ROW;
            } else if (a.weighted) {
                const Top4 t = s_top[i];
                double top_mass = 0.0;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    if (t.i[k] == INT_MAX) continue;
                    top_mass += exp(((double)t.v[k] - (double)md) / Td) / Sd;
                    if (t.i[k] == x) in_top = true;
                }
                const double N = 1.0 + ((double)a.beta - 1.0) * top_mass;
                if (!(N > 0.0)) err |= SV_ERR_DRAFT_MASS;
                else lnN = log(N);
                s_invsd[i] = 1.0 / (Sd * N);
            } else {
                s_invsd[i] = 1.0 / Sd;
            }
            double ratio = 0.0;
            float pt = NAN, pd = NAN;
            if (x >= 0 && x < a.V && err == 0) {
                double z_t, z_d;
                if (a.dtype == SV_F32) {
                    z_t = (double)Elt<0>::scalar(target_row(a, b, i), x);
                    z_d = (double)Elt<0>::scalar(draft_row(a, b, i), x);
                } else {
                    z_t = (double)Elt<1>::scalar(target_row(a, b, i), x);
                    z_d = (double)Elt<1>::scalar(draft_row(a, b, i), x);
                }
                const double lpt = (z_t - (double)mt) / Td - log(St);
                double lpd = (z_d - (double)md) / Td - log(Sd);
                if (a.weighted) lpd += (in_top ? log((double)a.beta) : 0.0) - lnN;
                ratio = (lpd == -INFINITY) ? INFINITY : exp(lpt - lpd);
                pt = (float)exp(lpt);
                pd = (float)exp(lpd);
            }
            const float u = philox_uniform(a.seed, (uint32_t)b, (uint32_t)i, kPurposeAccept);
            s_acc[i] = ((double)u <= ratio) ? 1 : 0;
            s_err[i] = err;
            s_pt[i] = pt;
            s_pd[i] = pd;
        }
        __syncthreads();
    }

    if (tid != 0) return;

    int n = K;
    int err_bits = 0;
    if (!fail && greedy) {
        for (int i = 0; i <= K; ++i) {
            if (!isfinite(s_m[i])) {
                fail = SV_ERR_ROW;
                break;
            }
            if (i < K && a.tokens[(int64_t)b * K + i] == s_idx[i]) continue;
            n = i;
            break;
        }
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = a.tokens[(int64_t)b * K + i];
            if (n < K) {
                const int x = a.tokens[(int64_t)b * K + n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            out[n] = s_idx[n];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = NAN;
            if (a.aux_z) a.aux_z[b] = NAN;
            SeqState st = {};
            st.mode = 0;
            a.seq[b] = st;
        }
    } else if (!fail) {
        for (int i = 0; i < K; ++i) {
            if (s_err[i]) {  // rows of this position are unusable and it is reached
                fail = s_err[i];
                break;
            }
            if (!s_acc[i]) {
                n = i;
                break;
            }
        }
        if (!fail && n == K && !isfinite(s_m[K])) fail = SV_ERR_ROW;
        if (!fail) {
            for (int i = 0; i < n; ++i) out[i] = a.tokens[(int64_t)b * K + i];
            for (int i = n + 1; i <= K; ++i) out[i] = -1;
            out[n] = -1;  // the bonus kernel writes the drawn token
            if (n < K) {
                const int x = a.tokens[(int64_t)b * K + n];
                if (x < 0 || x >= a.V) err_bits |= SV_ERR_TOKEN;
            }
            a.accepted_len[b] = n;
            if (a.aux_pt)
                for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = i <= n ? s_pt[i] : NAN;
            if (a.aux_pd)
                for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = i <= n ? s_pd[i] : NAN;
            SeqState st = {};
            st.n = n;
            st.mode = n < K ? 1 : 2;
            st.m_t = s_m[n];
            st.inv_st = (float)(1.0 / s_S[n]);
            st.T = T;
            st.beta = a.beta;
            st.u_bonus = philox_uniform(a.seed, (uint32_t)b, (uint32_t)n, kPurposeBonus);
#pragma unroll
            for (int k = 0; k < 4; ++k) st.top[k] = -1;
            if (n < K) {
                st.m_d = s_m[K + 1 + n];
                st.inv_sd = (float)s_invsd[n];
                if (a.weighted) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        st.top[k] = s_top[n].i[k] == INT_MAX ? -1 : s_top[n].i[k];
                }
            }
            a.seq[b] = st;
        }
    }
    if (fail) {
        a.accepted_len[b] = 0;
        for (int i = 0; i <= K; ++i) out[i] = -1;
        if (a.aux_pt)
            for (int i = 0; i < K; ++i) a.aux_pt[(int64_t)b * K + i] = NAN;
        if (a.aux_pd)
            for (int i = 0; i < K; ++i) a.aux_pd[(int64_t)b * K + i] = NAN;
        if (a.aux_z) a.aux_z[b] = NAN;
        SeqState st = {};
        st.mode = 0;
        a.seq[b] = st;
        err_bits |= fail;
    }
    if (err_bits && a.error_word) atomicOr(a.error_word, err_bits);
}

// ---------------------------------------------------------------------------
// Residual of one element: max(p_t - q', 0) in mode 1, p_t in mode 2, with
// p = exp2((z - m) * log2e / T) / S ("Kangaroo ...", "3. Lossless Speculative
// Verification", the corrected distribution; "Speculative Speculative
// Decoding", "Key claims", the residual max(p_t - p_d, 0)).

template <bool TOP>
__device__ __forceinline__ float residual_at(float zt, float zd, int v, const SeqState &st,
                                             const ExpScale &e, int mode)
{
    const float pt = exp_scaled(zt, st.m_t, e) * st.inv_st;
    if (mode == 2) return pt;
    float w = 1.f;
    if (TOP && (v == st.top[0] || v == st.top[1] || v == st.top[2] || v == st.top[3])) w = st.beta;
    const float pd = exp_scaled(zd, st.m_d, e) * st.inv_sd * w;
    return fmaxf(pt - pd, 0.f);
}

// 3. Chunk sums of the residual: one workgroup per (sequence, chunk).
template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void residual_kernel(const Args a)
{
    constexpr int VEC = Elt<DT>::kVec;
    __shared__ double lds_d[kWaves];
    const int b = blockIdx.x / a.ncr;
    const int chunk = blockIdx.x - b * a.ncr;
    const SeqState st = a.seq[b];
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const char *trow = target_row(a, b, st.n);
    const char *drow = st.mode == 1 ? draft_row(a, b, st.n) : trow;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    const int q0 = chunk * a.rvec, q1 = min(a.nvec, q0 + a.rvec);
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int qb = q0; qb < q1; qb += kBlock * kLoads) {
        float xt[kLoads][VEC], xd[kLoads][VEC];
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q < q1) {
                load_vec<DT>(trow, ta, q, a.V, xt[u]);
                if (st.mode == 1) load_vec<DT>(drow, da, q, a.V, xd[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < kLoads; ++u) {
            const int q = qb + u * kBlock + tid;
            if (q >= q1) continue;
            float acc[VEC];
#pragma unroll
            for (int k = 0; k < VEC; ++k)
                acc[k] = residual_at<TOP>(xt[u][k], st.mode == 1 ? xd[u][k] : 0.f, q * VEC + k, st,
                                          e, st.mode);
#pragma unroll
            for (int w = VEC / 2; w > 0; w >>= 1)
#pragma unroll
                for (int k = 0; k < w; ++k) acc[k] += acc[k + w];
            s += (double)acc[0];
        }
    }
    const double S = block_sum(s, lds_d);
    if (tid == 0) a.res[(int64_t)b * a.ncr + chunk] = S;
}

// Scan the residual over vectors [q0, q1) in token order, starting from
// `base`, for the first element whose running sum reaches `thr`.  Returns that
// element (or INT_MAX), the range total, and the last element with mass.
template <int DT, bool TOP>
__device__ int scan_range(const Args &a, int b, const SeqState &st, int mode, const ExpScale &e,
                          int q0, int q1, double base, double thr, double &total, int &last_pos,
                          double *lds_d, int *lds_i)
{
    constexpr int VEC = Elt<DT>::kVec;
    const int tid = threadIdx.x;
    const char *trow = target_row(a, b, st.n);
    const char *drow = mode == 1 ? draft_row(a, b, st.n) : trow;
    const bool ta = ((uintptr_t)trow & 15) == 0, da = ((uintptr_t)drow & 15) == 0;
    double run = base;
    int last = -1;
    for (int qb = q0; qb < q1; qb += kBlock) {
        const int q = qb + tid;
        double pre[VEC];
        double acc = 0.0;
        int mylast = -1;
        if (q < q1) {
            float xt[VEC], xd[VEC];
            load_vec<DT>(trow, ta, q, a.V, xt);
            if (mode == 1) load_vec<DT>(drow, da, q, a.V, xd);
#pragma unroll
            for (int k = 0; k < VEC; ++k) {
                const float r = residual_at<TOP>(xt[k], mode == 1 ? xd[k] : 0.f, q * VEC + k, st, e,
                                                 mode);
                acc += (double)r;
                pre[k] = acc;
                if (r > 0.f) mylast = q * VEC + k;
            }
        } else {
#pragma unroll
            for (int k = 0; k < VEC; ++k) pre[k] = 0.0;
        }
        double tile_total;
        const double exc = block_exclusive_scan(acc, tile_total, lds_d);
        int cand = INT_MAX;
        if (q < q1) {
#pragma unroll
            for (int k = VEC - 1; k >= 0; --k)
                if (run + exc + pre[k] >= thr) cand = q * VEC + k;
        }
        cand = block_min_int(cand, lds_i);
        last = max(last, block_max_int(mylast, lds_i));
        if (cand != INT_MAX) {
            total = run + tile_total;
            last_pos = last;
            return cand;
        }
        run += tile_total;
    }
    total = run;
    last_pos = last;
    return INT_MAX;
}

// 4. Bonus draw by inverse CDF in ascending token id: the smallest v with
// C(v) >= u * Z, Z the total residual mass; zero mass falls back to p_t.
template <int DT, bool TOP>
__global__ __launch_bounds__(kBlock) void bonus_kernel(const Args a)
{
    __shared__ double lds_d[kWaves];
    __shared__ int lds_i[kWaves];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const SeqState st = a.seq[b];
    if (st.mode == 0) return;
    const ExpScale e = make_scale(st.T);
    const double *rs = a.res + (int64_t)b * a.ncr;

    // Z: running sum of the chunk sums in chunk order.
    double Z = 0.0;
    for (int c0 = 0; c0 < a.ncr; c0 += kBlock) {
        const int c = c0 + tid;
        double tot;
        block_exclusive_scan(c < a.ncr ? rs[c] : 0.0, tot, lds_d);
        Z += tot;
    }
    int mode = st.mode;
    int token = -1;
    double total;
    int last;
    if (Z > 0.0) {
        const double thr = (double)st.u_bonus * Z;
        // the first chunk whose inclusive prefix reaches thr
        double run = 0.0;
        int cstar = INT_MAX, last_chunk = -1;
        double cbase = 0.0, last_base = 0.0;
        for (int c0 = 0; c0 < a.ncr && cstar == INT_MAX; c0 += kBlock) {
            const int c = c0 + tid;
            const double v = c < a.ncr ? rs[c] : 0.0;
            double tot;
            const double exc = block_exclusive_scan(v, tot, lds_d);
            int cand = (c < a.ncr && run + exc + v >= thr) ? c : INT_MAX;
            cand = block_min_int(cand, lds_i);
            const int lastc = block_max_int(v > 0.0 ? c : -1, lds_i);
            if (cand != INT_MAX || lastc > last_chunk) {
                if (c == cand) lds_d[0] = run + exc;
                if (c == lastc) lds_d[1] = run + exc;
                __syncthreads();
                if (cand != INT_MAX) cbase = lds_d[0];
                if (lastc > last_chunk) last_base = lds_d[1];
                __syncthreads();
            }
            if (cand != INT_MAX) cstar = cand;
            if (lastc > last_chunk) last_chunk = lastc;
            run += tot;
        }
        if (cstar == INT_MAX) {
            // rounding between the two summation orders left u * Z above the last
            // prefix: the draw falls in the last chunk that has mass
            cstar = last_chunk;
            cbase = last_base;
        }
        const int q0 = cstar * a.rvec, q1 = min(a.nvec, q0 + a.rvec);
        token = scan_range<DT, TOP>(a, b, st, mode, e, q0, q1, cbase, thr, total, last, lds_d, lds_i);
        if (token == INT_MAX) token = last;  // same rounding inside the chunk
    }
    if (token < 0) {
        // zero residual mass (only through rounding): draw from p_t instead
        mode = 2;
        scan_range<DT, TOP>(a, b, st, mode, e, 0, a.nvec, 0.0, INFINITY, total, last, lds_d, lds_i);
        Z = total;
        const double thr = (double)st.u_bonus * Z;
        token = scan_range<DT, TOP>(a, b, st, mode, e, 0, a.nvec, 0.0, thr, total, last, lds_d,
                                    lds_i);
        if (token == INT_MAX) token = last;
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)b * (a.K + 1) + st.n] = token;
        if (a.aux_z) a.aux_z[b] = (float)Z;
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
        float M;
        double S;
        merge_sum(p, a.nc, kLog2e / (double)T, M, S);
        if (lane == 0) {
            a.rs_max[r] = M;
            a.rs_logsum[r] = log(S);
            a.rs_argmax[r] = -1;
        }
    }
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
// Host side.

template <int DT, bool TOP>
static void launch_all(const Args &a, const Plan &p, hipStream_t s, bool draw)
{
    stats_kernel<DT, TOP><<<(unsigned)((int64_t)p.B * p.R * p.nc), kBlock, 0, s>>>(a);
    accept_kernel<<<(unsigned)p.B, kBlock, 0, s>>>(a);
    if (draw) {
        residual_kernel<DT, TOP><<<(unsigned)((int64_t)p.B * p.ncr), kBlock, 0, s>>>(a);
        bonus_kernel<DT, TOP><<<(unsigned)p.B, kBlock, 0, s>>>(a);
    }
}

static Args base_args(const Plan &p, void *ws)
{
    Args a = {};
    char *w = static_cast<char *>(ws);
    a.B = p.B;
    a.K = p.K;
    a.V = p.V;
    a.R = p.R;
    a.nvec = p.nvec;
    a.nc = p.nc;
    a.cvec = p.cvec;
    a.ncr = p.ncr;
    a.rvec = p.rvec;
    a.dtype = p.dtype;
    a.row_bytes = p.row_bytes;
    a.part = reinterpret_cast<RowPart *>(w + p.off_part);
    a.top = reinterpret_cast<Top4 *>(w + p.off_top);
    a.seq = reinterpret_cast<SeqState *>(w + p.off_seq);
    a.res = reinterpret_cast<double *>(w + p.off_res);
    return a;
}

}  // namespace sv

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype)
{
    sv::Plan p;
    if (B < 0 || !sv::make_plan(B, K, V, dtype, &p)) return 0;
    return p.bytes;
}

int32_t spec_verify(const void *target_logits, const void *draft_logits,
                    const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                    uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    const sv_aux *aux, void *stream)
{
    if (B < 0 || K < 0 || K > sv::kMaxK || V < 1) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (!(beta >= 0.f && beta <= 1.f)) return SV_EINVAL;
    if ((int64_t)B * (K + 1) * (int64_t)V > ((int64_t)1 << 40)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !accepted_len || !out_tokens) return SV_EINVAL;
    if (K > 0 && !draft_tokens) return SV_EINVAL;
    const size_t elt = dtype == SV_F32 ? 4 : 2;
    if (((uintptr_t)target_logits % elt) || (draft_logits && ((uintptr_t)draft_logits % elt)))
        return SV_EINVAL;
    sv::Plan p;
    if (!sv::make_plan(B, K, V, dtype, &p)) return SV_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < p.bytes)
        return SV_EWORKSPACE;

    sv::Args a = sv::base_args(p, workspace);
    a.target = static_cast<const char *>(target_logits);
    a.draft = static_cast<const char *>(draft_logits);
    a.tokens = draft_tokens;
    a.temperature = temperature;
    a.seed = seed;
    a.beta = beta;
    a.weighted = (beta < 1.f && K > 0) ? 1 : 0;
    a.accepted_len = accepted_len;
    a.out_tokens = out_tokens;
    if (aux) {
        a.aux_pt = aux->p_target;
        a.aux_pd = aux->p_draft;
        a.aux_z = aux->residual_mass;
        a.error_word = aux->error_word;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    // With no draft logits every sequence is greedy or fails; nothing to draw.
    const bool draw = !(K > 0 && draft_logits == nullptr);
    if (dtype == SV_F32) {
        if (a.weighted) sv::launch_all<0, true>(a, p, s, draw);
        else sv::launch_all<0, false>(a, p, s, draw);
    } else {
        if (a.weighted) sv::launch_all<1, true>(a, p, s, draw);
        else sv::launch_all<1, false>(a, p, s, draw);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t spec_verify_row_stats(const void *logits, int32_t rows, int32_t V, int32_t dtype,
                              const float *temperature, float *row_max, double *row_logsum,
                              int32_t *row_argmax, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    if (rows < 0 || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return SV_EINVAL;
    if (rows == 0) return SV_OK;
    if (!logits || !temperature || !row_max || !row_logsum || !row_argmax) return SV_EINVAL;
    const size_t elt = dtype == SV_F32 ? 4 : 2;
    if ((uintptr_t)logits % elt) return SV_EINVAL;
    sv::Plan p;
    if (!sv::make_plan(rows, 0, V, dtype, &p)) return SV_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < p.bytes)
        return SV_EWORKSPACE;
    sv::Args a = sv::base_args(p, workspace);
    a.target = static_cast<const char *>(logits);
    a.temperature = temperature;
    a.rs_max = row_max;
    a.rs_logsum = row_logsum;
    a.rs_argmax = row_argmax;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dtype == SV_F32)
        sv::stats_kernel<0, false><<<(unsigned)((int64_t)p.B * p.R * p.nc), sv::kBlock, 0, s>>>(a);
    else
        sv::stats_kernel<1, false><<<(unsigned)((int64_t)p.B * p.R * p.nc), sv::kBlock, 0, s>>>(a);
    sv::rowstats_finish_kernel<<<(unsigned)rows, 64, 0, s>>>(a);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t spec_verify_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, void *stream)
{
    if (B < 0 || P < 0) return SV_EINVAL;
    const int64_t total = (int64_t)B * P * 2;
    if (total == 0) return SV_OK;
    if (!out || total > ((int64_t)1 << 31)) return SV_EINVAL;
    const unsigned blocks = (unsigned)((total + 255) / 256);
    sv::uniforms_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(seed, B, P, out);
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

const char *spec_verify_status_str(int32_t status)
{
    switch (status) {
    case SV_OK: return "SV_OK: success";
    case SV_EINVAL: return "SV_EINVAL: invalid argument (nothing enqueued)";
    case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing, misaligned or too small";
    case SV_EHIP: return "SV_EHIP: HIP runtime error on launch";
    default: return "unknown status";
    }
}

}  // extern "C"
