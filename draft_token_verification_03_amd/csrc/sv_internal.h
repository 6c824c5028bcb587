// sv_internal.h -- shared host/device declarations of libspecverify.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "specverify.h"
#include "sv_device.h"

namespace sv {

constexpr int kMaxK = 128;               // drafted positions per sequence
constexpr int kMaxSlots = 2 * kMaxK + 1;
constexpr int kMaxChunks = 1024;         // streaming chunks per row
constexpr int kFillBlocks = 768;         // workgroups the streaming grid aims for (one round)
constexpr int kArgmaxFill = 1280;        // the same for the greedy-only grid (five per CU)
constexpr int kCUs = 256;                // compute units of the chip
constexpr int64_t kSplitRowBytes = 256 * 1024;  // rows this long take at least two chunks
constexpr int kMaxSeqPerLaunch = 8192;   // sequences per sub-batch of launches
constexpr int kStageBytes = 24 * 1024;   // LDS staging of one sequence's partials
constexpr int kResFill = 1024;           // workgroups the residual grid aims for (one round)
constexpr int kResLoads = 4;             // residual units in flight per lane (per row)
constexpr int kSlotVec = 64;             // 16-byte vectors per residual slot unit (one per lane)
constexpr int kSlotUnits = 4;            // units per slot when the batch alone fills the grid
constexpr int kMaxResSlots = 4096;       // residual slots per row (coarser slots beyond)
constexpr int kThreadMerge = 4;          // chunks per row the accept scan merges per thread
constexpr uint32_t kPurposeAccept = 0u, kPurposeBonus = 1u;

// One (row, chunk) partial of the streaming pass.
struct RowPart {
    float m;      // chunk maximum
    int32_t idx;  // lowest index attaining m (greedy rows); in chunk 0 of a sampling
                  // row i < K, the bits of the fp32 logit at drafted token x_i
    double s;     // sum of exp2((z - m) * log2e / T) over the chunk; for a beta-weighted
                  // draft row, over the chunk's elements outside the chunk's top-4
};

// Per-sequence outcome of the accept scan, handed to the bonus step.
struct SeqState {
    int32_t n;     // accepted drafts
    int32_t mode;  // 0: nothing to draw, 1: residual max(p_t - q', 0), 2: p_t alone
    float o_t, o_d;  // row offsets fp32(m c) of target row n and draft row n
    double k2;       // log2 q'(v) - log2 p_t(v) = (z_d(v) - z_t(v)) c + k2 (+ log2 beta on the top-4)
    float inv_st;  // 1 / S_t: residual masses are summed relative to p_t * S_t
    float u_bonus;
    int32_t top[4];
    float T;
    float lbeta;   // log2(beta), -inf for beta == 0
    int32_t pad[2];
};
static_assert(sizeof(SeqState) == 64, "SeqState layout");

// Launch geometry and workspace layout for one sub-batch of sB sequences.
struct Plan {
    int32_t B, K, V, dtype, vec, R;
    int32_t sB;             // sequences per sub-batch: min(B, kMaxSeqPerLaunch)
    int32_t nvec;           // 16-byte vectors per row (the last may be partial)
    int64_t row_bytes;
    int32_t nc, cvec;       // streaming chunks per row, vectors per chunk
    int32_t nslot, gs;      // residual slots per row, kSlotVec-vector units per slot
    int32_t ng, spg;        // residual workgroups per sequence, slots per workgroup
    size_t off_part, off_top, off_tope, off_seq, off_slot;
    size_t bytes;           // total workspace
};

// greedy_only: a call without draft rows (and K > 0, no ragged lengths),
// whose streaming pass launches only target rows 0..K (argmax_kernel)
bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan *p, bool greedy_only = false,
               bool weighted = false);

struct Args {
    const char *target;     // the sub-batch's first target row
    const char *draft;
    const int32_t *tokens;
    const int32_t *draft_len;   // [B] drafts of each sequence (K_b <= K), or null for K
    const float *temperature;
    int32_t B, K, V, R, nvec, nc, cvec, nslot, gs, ng, spg, dtype;
    int32_t b0;             // index of the sub-batch's first sequence in the call
    int64_t row_bytes;
    uint64_t seed;
    float beta;
    double log2_beta;       // log2(beta), -inf for beta == 0
    int32_t weighted;
    int32_t sampling_only;  // the streaming pass skips the rows of greedy sequences
    int32_t *accepted_len;
    int32_t *out_tokens;
    RowPart *part;          // [sB][R][nc]
    Top4 *top;              // [sB][K][nc]
    double4 *tope;          // [sB][K][nc] exp2((v - m_c) c) of each chunk top-4 entry (nc > 1)
    SeqState *seq;          // [sB]
    double *slot;           // [sB][nslot] residual mass of each slot
    float *aux_pt, *aux_pd, *aux_z, *aux_conf;
    int32_t *error_word;    // error bits are OR-ed in
    // row-statistics entry point outputs
    float *rs_max;
    double *rs_logsum;
    int32_t *rs_argmax;
};

// ---------------------------------------------------------------------------
// Verification-outcome distribution: per (sequence, position) records and
// per (sequence, position, chunk) partial sums and best-F residual keys.

constexpr int kMaxOutcomeF = 32;     // ranked bonus tokens per position
constexpr int kMaxOutChunks = 128;   // outcome-pass chunks per position
constexpr int kOutLoads = 2;         // 16-byte vectors per thread per row per tile

struct OutRow {
    double norm;     // position j < K: draft normaliser D; j == K: target sum S_t
    float o;         // j == K: offset fp32(m_t c) of target row K
    int32_t status;  // SV_ERR_ROW / SV_ERR_DRAFT_MASS bits of the position's rows
};

struct OutPlan {
    Plan p;                   // the streaming pass (its part/top/tope regions)
    int32_t F, nc2, cvec2;    // ranked tokens; outcome chunks per position, vectors per chunk
    size_t off_rec, off_asum, off_tsum, off_keys;
    size_t bytes;
};

bool make_outcome_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, int32_t F, OutPlan *p);

struct OutArgs {
    Args a;                   // rows, temperatures, beta and the streaming-pass partials
    int32_t F, nc2, cvec2;
    OutRow *rec;              // [sB][K+1]
    double *asum;             // [sB][K+1][nc2] sum of min(p, q') D over the chunk (j < K)
    double *tsum;             // [sB][K+1][nc2] r D summed over the draft's top-4 in the chunk (j < K)
    uint64_t *keys;           // [sB][K+1][nc2][F] the chunk's best keys, descending, 0 = none
    float *accept_rate;       // [sB][K]
    float *p_len;             // [sB][K+1]
    int32_t *top_tokens;      // [sB][K+1][F]
    float *top_mass;          // [sB][K+1][F]
    float *draft_top_mass;    // [sB][K] r summed over each draft row's top-4, or null
};

// ---------------------------------------------------------------------------
// Tree verification: one workgroup walks one sequence's token tree.

constexpr int kMaxTreeSteps = 2048;  // tile steps per row whose masses the bonus search keeps
constexpr int kTreeStepVecs = 1024;     // 16-byte vectors per tile step of the tree walk

struct TreeArgs {
    const char *target;        // the sub-batch's first target row: [sB][N+1][V]
    const char *draft;         // [sB][N][V] or null
    const int32_t *parent;     // [sB][N]
    const int32_t *tokens;     // [sB][N]
    const float *temperature;  // [sB]
    int32_t N, V, nvec, dtype;
    int32_t b0;                // index of the sub-batch's first sequence in the call
    int64_t row_bytes;
    uint64_t seed;
    int32_t *accepted_len;     // [sB]
    int32_t *out_tokens;       // [sB][N+1]
    int32_t *path;             // [sB][N]
    int32_t *error_word;
};

// Launchers of one sub-batch: the verify step (non-null events are recorded
// around the streaming launch), the streaming pass alone, the outcome
// distribution (events around the outcome pass), the row-statistics entry
// point, the uniforms.
void launch_verify(const Args &a, hipStream_t s, hipEvent_t begin, hipEvent_t end);
void launch_stats(const Args &a, hipStream_t s);
void launch_outcomes(const OutArgs &o, hipStream_t s, hipEvent_t begin, hipEvent_t end);
void launch_tree(const TreeArgs &t, int32_t nb, hipStream_t s, hipEvent_t begin, hipEvent_t end);
void launch_rowstats(const Args &a, hipStream_t s);
void launch_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, hipStream_t s);
void launch_stream_probe(const Args &a, uint32_t *sink, hipStream_t s, hipEvent_t begin, hipEvent_t end);

}  // namespace sv
