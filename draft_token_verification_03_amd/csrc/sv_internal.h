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
constexpr int kMaxChunks = 1024;         // streaming chunks per row (multi-pass path)
constexpr int kFillBlocks = 2048;        // workgroups a streaming grid aims for
constexpr int kFusedFill = 8192;         // streaming items the fused grid aims for
constexpr int kMaxSeqPerLaunch = 8192;   // sequences per fused launch
constexpr int kFusedU = 4;               // fused path: 16-byte vectors per thread per row chunk
constexpr int kFusedMaxK = 16;           // fused path: drafted positions per sequence
constexpr int kStageBytes = 12 * 1024;   // fused path: LDS staging of one sequence's partials
constexpr uint32_t kPurposeAccept = 0u, kPurposeBonus = 1u;

// Error bit for a wait that exceeded its spin budget (fused path only).
constexpr int kErrTimeout = 32;

// One (row, chunk) partial of the streaming pass.
struct RowPart {
    float m;      // chunk maximum
    int32_t idx;  // lowest index attaining m (greedy rows)
    double s;     // sum of exp2((z - m) * log2e / T) over the chunk; for a beta-weighted
                  // draft row, over the chunk's elements outside the chunk's top-4
};

// Per-sequence outcome of the accept scan, read by the residual and bonus steps.
struct SeqState {
    int32_t n;     // accepted drafts
    int32_t mode;  // 0: nothing to draw, 1: residual max(p_t - q', 0), 2: p_t alone
    float m_t, m_d;
    double k2;     // log2 q'(v) - log2 p_t(v) = (z_d(v) - z_t(v)) log2e / T + k2 (+ log2 beta on the top-4)
    float inv_st;  // 1 / S_t
    float inv_sd;  // 1 / (S_d * N): the weighted draft normaliser
    float beta;
    float u_bonus;
    int32_t top[4];
    float T;
    float lbeta;   // log2(beta), -inf for beta == 0
};
static_assert(sizeof(SeqState) == 64, "SeqState layout");

// Control words of one sequence on the fused path, one 128-byte line each so
// that different sequences' atomics never share a line.  They are zero before
// a launch and returned to zero by their last users.
struct SeqCtl {
    uint32_t count;   // streaming items of the sequence that have published
    uint32_t rcount;  // draw items that have published a residual chunk sum
    uint32_t dcount;  // draw items done
    uint32_t flag;    // 1 once the accept scan of the sequence is done
    uint32_t pad[28];
};
static_assert(sizeof(SeqCtl) == 128, "SeqCtl layout");
constexpr size_t kPersistBytes = sizeof(SeqCtl) * (size_t)kMaxSeqPerLaunch;

struct Plan {
    int32_t B, K, V, dtype, vec, R;
    int32_t nvec;           // 16-byte vectors per row (the last may be partial)
    int64_t row_bytes;
    // multi-pass path
    int32_t nc, cvec;       // streaming chunks per row, vectors per chunk
    int32_t ncr, rvec;      // residual chunks per sequence, vectors per residual chunk
    size_t off_part, off_top, off_seq, off_res, mp_bytes;
    // fused path (per launch of at most kMaxSeqPerLaunch sequences)
    int32_t fu;             // 16-byte vectors per thread per sub-tile
    int32_t fchunks;        // draw chunks (one sub-tile each) per row
    int32_t fspan;          // sub-tiles per streaming chunk
    int32_t fschunks;       // streaming chunks per row
    int32_t fitems;         // streaming items per sequence: (K + 1) * fschunks
    int32_t fB;             // sequences per launch
    size_t foff_part, foff_top, foff_state, foff_res, foff_zx, f_bytes;
    bool fused_shape_ok;
    size_t bytes;           // total workspace
};

bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan *p);

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

struct FusedArgs {
    const char *target;
    const char *draft;
    const int32_t *tokens;
    const float *temperature;
    int32_t B, K, V, nvec;
    int32_t chunks;        // draw chunks per row (kBlock * U vectors each)
    int32_t sspan;         // sub-tiles per streaming chunk
    int32_t schunks;       // streaming chunks per row
    int32_t stream_items, b0;
    int64_t row_bytes;
    uint64_t seed;
    float beta;
    int32_t weighted;
    uint32_t spin_limit;
    int32_t *accepted_len;
    int32_t *out_tokens;
    float *aux_pt, *aux_pd, *aux_z;
    int32_t *error_word;   // error bits are OR-ed in
    SeqCtl *seqctl;
    RowPart *part;   // [B][2K+1][schunks]
    Top4 *top;       // [B][K][schunks]
    SeqState *state; // [B]
    double *res;     // [B][chunks]
    float2 *zx;      // [B][K]: (target, draft) logit of the drafted token
};

// Multi-pass path (any shape).
void launch_multipass(const Args &a, const Plan &p, hipStream_t s, bool draw);
void launch_rowstats(const Args &a, const Plan &p, hipStream_t s);
void launch_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, hipStream_t s);
void launch_zero(void *ptr, size_t bytes, hipStream_t s);

// Fused single-launch path: returns false (nothing enqueued) when the shape or
// the device's resident-workgroup capacity does not allow it.
bool fused_capacity_ok(const Plan &p, bool weighted);
void launch_fused(const FusedArgs &a, const Plan &p, hipStream_t s);

}  // namespace sv
