// sv_api.hip -- the C ABI of libspecverify: argument validation, the launch
// plan, the workspace layout and the split into sub-batches.  The operation is specified in include/specverify.h.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sv_internal.h"

namespace sv {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool make_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, Plan *p, bool greedy_only, bool weighted)
{
    if (B < 0 || K < 0 || K > kMaxK || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return false;
    *p = Plan{};
    p->B = B;
    p->K = K;
    p->V = V;
    p->dtype = dtype;
    const int elt = dtype == SV_F32 ? 4 : 2;
    p->vec = 16 / elt;
    p->R = 2 * K + 1;
    p->sB = std::min(std::max(B, 1), kMaxSeqPerLaunch);
    p->row_bytes = (int64_t)V * elt;
    p->nvec = (int32_t)(((int64_t)V + p->vec - 1) / p->vec);

    // streaming: ~kFillBlocks workgroups per sub-batch (one round of resident
    // workgroups; kArgmaxFill for the lighter greedy-only kernel, which
    // launches only target rows), >= one vector per thread, and one
    // sequence's partials and top-4 lists within the accept scan's LDS staging
    const int64_t rows = (int64_t)p->sB * (greedy_only ? K + 1 : p->R);
    const int64_t fill = greedy_only ? kArgmaxFill : kFillBlocks;
    int64_t nc = (fill + rows - 1) / rows;
    // rows enough to cover the chip with a few chunks each: at most as many as
    // the accept scan merges per thread
    if (rows * kThreadMerge >= kCUs) nc = std::min<int64_t>(nc, kThreadMerge);
    // long rows in a batch that fills the grid by itself: two chunks a row
    // halve the size of the grid's workgroups, so its last round leaves less
    // of the chip idle
    if (nc == 1 && p->row_bytes >= kSplitRowBytes) {
        nc = 2;
        // beta-weighted draft rows keep top-4 lists per chunk, whose upkeep
        // grows with the number of chunks: one chunk a row unless that leaves
        // a larger share of the last round idle
        auto idle = [](int64_t w) { return (kFillBlocks - w % kFillBlocks) % kFillBlocks; };
        if (weighted && 2 * idle(rows) <= idle(2 * rows)) nc = 1;
    }
    const int64_t nc_max = std::max<int64_t>(1, p->nvec / kBlock);
    const int64_t nc_stage =
        kStageBytes / ((int64_t)sizeof(RowPart) * p->R + (int64_t)sizeof(Top4) * K);
    nc = std::min<int64_t>(std::min<int64_t>(nc, nc_max), std::min<int64_t>(kMaxChunks, nc_stage));
    nc = std::max<int64_t>(nc, 1);
    p->cvec = (int32_t)((p->nvec + nc - 1) / nc);
    p->nc = (p->nvec + p->cvec - 1) / p->cvec;
    // residual: slots of gs units of kSlotVec vectors (kSlotUnits units, or
    // single units when a small batch needs the finer split to fill the
    // grid), at most kMaxResSlots per row; ~kResFill workgroups in all
    const int64_t units = (p->nvec + kSlotVec - 1) / kSlotVec;
    const int64_t ng_fill = (kResFill + p->sB - 1) / p->sB;
    int64_t gs = (units / kSlotUnits >= ng_fill) ? kSlotUnits : 1;
    gs = std::max<int64_t>(gs, (units + kMaxResSlots - 1) / kMaxResSlots);
    p->gs = (int32_t)gs;
    p->nslot = (int32_t)((units + gs - 1) / gs);
    // at least one slot per wave: a workgroup's waves take its slots in turn,
    // and one with fewer slots than waves still pays the whole accept scan
    const int64_t ng_max = (p->nslot + kWaves - 1) / kWaves;
    p->ng = (int32_t)std::max<int64_t>(1, std::min<int64_t>(ng_fill, ng_max));
    p->spg = (p->nslot + p->ng - 1) / p->ng;
    p->ng = (p->nslot + p->spg - 1) / p->spg;
    if ((int64_t)p->sB * p->R * p->nc >= ((int64_t)1 << 31) || (int64_t)p->sB * p->ng >= ((int64_t)1 << 31))
        return false;
    size_t off = 0;
    p->off_part = off;
    off = align256(off + sizeof(RowPart) * (size_t)p->sB * p->R * p->nc);
    p->off_top = off;
    off = align256(off + sizeof(Top4) * (size_t)p->sB * K * p->nc);
    p->off_tope = off;
    off = align256(off + sizeof(double4) * (size_t)p->sB * K * p->nc);
    p->off_seq = off;
    off = align256(off + sizeof(SeqState) * (size_t)p->sB);
    p->off_slot = off;
    off = align256(off + sizeof(double) * (size_t)p->sB * p->nslot);
    p->bytes = off;
    return true;
}

// The outcome distribution: the streaming pass's plan, then ~kFillBlocks
// outcome workgroups (one chunk per position once the positions fill the
// grid: a longer chunk lets its slots' floor rise further before most of its
// elements arrive, so fewer of them are inserted), and the outcome pass's
// records, sums and keys after the streaming pass's regions.
bool make_outcome_plan(int32_t B, int32_t K, int32_t V, int32_t dtype, int32_t F, OutPlan *op)
{
    if (F < 0 || F > kMaxOutcomeF) return false;
    *op = OutPlan{};
    if (!make_plan(B, K, V, dtype, &op->p)) return false;
    const Plan &p = op->p;
    op->F = F;
    const int64_t pos = (int64_t)p.sB * (K + 1);
    int64_t nc2 = (kFillBlocks + pos - 1) / pos;
    const int64_t nc_max = std::max<int64_t>(1, p.nvec / (kBlock * kOutLoads));
    nc2 = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(nc2, nc_max), kMaxOutChunks));
    op->cvec2 = (int32_t)((p.nvec + nc2 - 1) / nc2);
    op->nc2 = (p.nvec + op->cvec2 - 1) / op->cvec2;
    if (pos * op->nc2 >= ((int64_t)1 << 31)) return false;
    size_t off = p.bytes;
    op->off_rec = off;
    off = align256(off + sizeof(OutRow) * (size_t)pos);
    op->off_asum = off;
    off = align256(off + sizeof(double) * (size_t)pos * op->nc2);
    op->off_tsum = off;
    off = align256(off + sizeof(double) * (size_t)pos * op->nc2);
    op->off_keys = off;
    off = align256(off + sizeof(uint64_t) * (size_t)pos * op->nc2 * F);
    op->bytes = off;
    return true;
}

// Arguments of the sub-batch of sequences [b0, b0 + nb).
static Args sub_args(const Plan &p, void *ws, int32_t b0, int32_t nb)
{
    Args a = {};
    char *w = static_cast<char *>(ws);
    a.B = nb;
    a.K = p.K;
    a.V = p.V;
    a.R = p.R;
    a.nvec = p.nvec;
    a.nc = p.nc;
    a.cvec = p.cvec;
    a.nslot = p.nslot;
    a.gs = p.gs;
    a.ng = p.ng;
    a.spg = p.spg;
    a.dtype = p.dtype;
    a.b0 = b0;
    a.row_bytes = p.row_bytes;
    a.part = reinterpret_cast<RowPart *>(w + p.off_part);
    a.top = reinterpret_cast<Top4 *>(w + p.off_top);
    a.tope = reinterpret_cast<double4 *>(w + p.off_tope);
    a.seq = reinterpret_cast<SeqState *>(w + p.off_seq);
    a.slot = reinterpret_cast<double *>(w + p.off_slot);
    return a;
}

// Checks shared by the verify entry points; SV_OK means "go on".
static int32_t validate(const void *target_logits, const void *draft_logits,
                        const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                        const float *temperature, float beta, int32_t *accepted_len,
                        int32_t *out_tokens)
{
    if (B < 0 || K < 0 || K > kMaxK || V < 1) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (!(beta >= 0.f && beta <= 1.f)) return SV_EINVAL;
    if ((int64_t)B * (K + 1) * (int64_t)V > ((int64_t)1 << 40)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !accepted_len || !out_tokens) return SV_EINVAL;
    if (K > 0 && !draft_tokens) return SV_EINVAL;
    const size_t elt = dtype == SV_F32 ? 4 : 2;
    if (((uintptr_t)target_logits % elt) || (draft_logits && ((uintptr_t)draft_logits % elt)))
        return SV_EINVAL;
    return SV_OK;
}

static int32_t verify(const void *target_logits, const void *draft_logits,
                      const int32_t *draft_tokens, const int32_t *draft_len, int32_t B, int32_t K,
                      int32_t V, int32_t dtype,
                      uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                      int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                      const sv_aux *aux, void *stream)
{
    const int32_t v = validate(target_logits, draft_logits, draft_tokens, B, K, V, dtype,
                               temperature, beta, accepted_len, out_tokens);
    if (v != SV_OK || B == 0) return v;
    Plan p;
    if (!make_plan(B, K, V, dtype, &p, !draft_logits && K > 0 && !draft_len, beta < 1.f && K > 0))
        return SV_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < p.bytes)
        return SV_EWORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    for (int32_t b0 = 0; b0 < B; b0 += p.sB) {
        const int32_t nb = std::min(p.sB, B - b0);
        Args a = sub_args(p, workspace, b0, nb);
        a.target = static_cast<const char *>(target_logits) + (int64_t)b0 * (K + 1) * p.row_bytes;
        a.draft = draft_logits ? static_cast<const char *>(draft_logits) + (int64_t)b0 * K * p.row_bytes
                               : nullptr;
        a.tokens = draft_tokens ? draft_tokens + (int64_t)b0 * K : nullptr;
        a.draft_len = draft_len ? draft_len + b0 : nullptr;
        a.temperature = temperature + b0;
        a.seed = seed;
        a.beta = beta;
        a.log2_beta = std::log2((double)beta);
        a.weighted = (beta < 1.f && K > 0) ? 1 : 0;
        a.accepted_len = accepted_len + b0;
        a.out_tokens = out_tokens + (int64_t)b0 * (K + 1);
        if (aux) {
            a.aux_pt = aux->p_target ? aux->p_target + (int64_t)b0 * K : nullptr;
            a.aux_pd = aux->p_draft ? aux->p_draft + (int64_t)b0 * K : nullptr;
            a.aux_z = aux->residual_mass ? aux->residual_mass + b0 : nullptr;
            a.aux_conf = aux->draft_conf ? aux->draft_conf + (int64_t)b0 * K : nullptr;
            a.error_word = aux->error_word;
        }
        hipEvent_t begin = nullptr, end = nullptr;
        if (aux && b0 == 0) {
            begin = static_cast<hipEvent_t>(aux->pass_begin);
            end = static_cast<hipEvent_t>(aux->pass_end);
        }
        launch_verify(a, s, begin, end);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

// Scratch of spec_verify_noalloc: a file-scope device array (each GPU the
// library runs on holds its own copy until the process ends).  Host code
// never passes the array's name to a kernel -- on the host it is a stand-in,
// not a device address -- but the address hipGetSymbolAddress returns for the
// current device, taken once per device and kept here.
constexpr size_t kScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static void *g_scratch[kMaxDevices];
static std::mutex g_scratch_mutex;

// This device's copy of scratch, or nullptr when HIP reports an error.
static void *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch[dev] = ptr;
    }
    return g_scratch[dev];
}

}  // namespace sv

extern "C" {

size_t spec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype)
{
    sv::Plan p, pg;
    if (B < 0 || !sv::make_plan(B, K, V, dtype, &p) || !sv::make_plan(B, K, V, dtype, &pg, true)) return 0;
    return std::max(p.bytes, pg.bytes);
}

int32_t spec_verify(const void *target_logits, const void *draft_logits,
                    const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                    uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    const sv_aux *aux, void *stream)
{
    return sv::verify(target_logits, draft_logits, draft_tokens, nullptr, B, K, V, dtype, seed,
                      temperature, beta, accepted_len, out_tokens, workspace, workspace_bytes, aux,
                      stream);
}

int32_t spec_verify_ragged(const void *target_logits, const void *draft_logits,
                           const int32_t *draft_tokens, const int32_t *draft_len, int32_t B,
                           int32_t K, int32_t V, int32_t dtype, uint64_t seed,
                           const float *temperature, float beta, int32_t *accepted_len,
                           int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                           const sv_aux *aux, void *stream)
{
    return sv::verify(target_logits, draft_logits, draft_tokens, draft_len, B, K, V, dtype, seed,
                      temperature, beta, accepted_len, out_tokens, workspace, workspace_bytes, aux,
                      stream);
}

size_t spec_verify_noalloc_max_scratch(void) { return sv::kScratchBytes; }

int32_t spec_verify_noalloc(const void *target_logits, const void *draft_logits,
                            const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                            uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                            int32_t *out_tokens, const sv_aux *aux, void *stream)
{
    const int32_t v = sv::validate(target_logits, draft_logits, draft_tokens, B, K, V, dtype, temperature,
                                   beta, accepted_len, out_tokens);
    if (v != SV_OK || B == 0) return v;
    // the plans of both streaming kernels must fit the static scratch
    const size_t need = spec_verify_workspace_size(B, K, V, dtype);
    if (need == 0) return SV_EINVAL;
    if (need > sv::kScratchBytes) return SV_ESCRATCH;
    void *ws = sv::device_scratch();
    if (!ws) return SV_EHIP;
    return sv::verify(target_logits, draft_logits, draft_tokens, nullptr, B, K, V, dtype, seed, temperature,
                      beta, accepted_len, out_tokens, ws, sv::kScratchBytes, aux, stream);
}

size_t spec_verify_outcomes_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype, int32_t F)
{
    sv::OutPlan op;
    if (B < 0 || !sv::make_outcome_plan(B, K, V, dtype, F, &op)) return 0;
    return op.bytes;
}

int32_t spec_verify_outcomes(const void *target_logits, const void *draft_logits, int32_t B, int32_t K,
                             int32_t V, int32_t dtype, const float *temperature, float beta, int32_t F,
                             float *accept_rate, float *p_len, int32_t *top_tokens, float *top_mass,
                             float *draft_top_mass, int32_t *error_word, void *workspace,
                             size_t workspace_bytes, void *pass_begin, void *pass_end, void *stream)
{
    if (B < 0 || K < 0 || K > sv::kMaxK || V < 1) return SV_EINVAL;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_EINVAL;
    if (!(beta >= 0.f && beta <= 1.f) || F < 0 || F > sv::kMaxOutcomeF) return SV_EINVAL;
    if ((int64_t)B * (K + 1) * (int64_t)V > ((int64_t)1 << 40)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !p_len || (K > 0 && !accept_rate) ||
        (F > 0 && (!top_tokens || !top_mass)))
        return SV_EINVAL;
    const size_t elt = dtype == SV_F32 ? 4 : 2;
    if (((uintptr_t)target_logits % elt) || (draft_logits && ((uintptr_t)draft_logits % elt)))
        return SV_EINVAL;
    sv::OutPlan op;
    if (!sv::make_outcome_plan(B, K, V, dtype, F, &op)) return SV_EINVAL;
    if (!workspace || ((uintptr_t)workspace & 255) || workspace_bytes < op.bytes) return SV_EWORKSPACE;
    const sv::Plan &p = op.p;
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *w = static_cast<char *>(workspace);
    for (int32_t b0 = 0; b0 < B; b0 += p.sB) {
        const int32_t nb = std::min(p.sB, B - b0);
        sv::OutArgs o = {};
        o.a = sv::sub_args(p, workspace, b0, nb);
        sv::Args &a = o.a;
        a.target = static_cast<const char *>(target_logits) + (int64_t)b0 * (K + 1) * p.row_bytes;
        a.draft = draft_logits ? static_cast<const char *>(draft_logits) + (int64_t)b0 * K * p.row_bytes
                               : nullptr;
        a.temperature = temperature + b0;
        a.beta = beta;
        a.log2_beta = std::log2((double)beta);
        // the draft rows' top-4 are tracked for beta < 1, and for their residual mass
        a.weighted = ((beta < 1.f || draft_top_mass) && K > 0) ? 1 : 0;
        a.sampling_only = 1;
        a.error_word = error_word;
        o.F = F;
        o.nc2 = op.nc2;
        o.cvec2 = op.cvec2;
        o.rec = reinterpret_cast<sv::OutRow *>(w + op.off_rec);
        o.asum = reinterpret_cast<double *>(w + op.off_asum);
        o.tsum = reinterpret_cast<double *>(w + op.off_tsum);
        o.keys = reinterpret_cast<uint64_t *>(w + op.off_keys);
        o.accept_rate = accept_rate ? accept_rate + (int64_t)b0 * K : nullptr;
        o.p_len = p_len + (int64_t)b0 * (K + 1);
        o.top_tokens = top_tokens ? top_tokens + (int64_t)b0 * (K + 1) * F : nullptr;
        o.top_mass = top_mass ? top_mass + (int64_t)b0 * (K + 1) * F : nullptr;
        o.draft_top_mass = draft_top_mass ? draft_top_mass + (int64_t)b0 * K : nullptr;
        sv::launch_outcomes(o, s, b0 == 0 ? static_cast<hipEvent_t>(pass_begin) : nullptr,
                            b0 == 0 ? static_cast<hipEvent_t>(pass_end) : nullptr);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t spec_verify_tree(const void *target_logits, const void *draft_logits, const int32_t *parent,
                         const int32_t *tokens, int32_t B, int32_t N, int32_t V, int32_t dtype,
                         uint64_t seed, const float *temperature, int32_t *accepted_len,
                         int32_t *out_tokens, int32_t *path, int32_t *error_word, void *pass_begin,
                         void *pass_end, void *stream)
{
    if (B < 0 || N < 0 || N > sv::kMaxK || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return SV_EINVAL;
    const int64_t elt = dtype == SV_F32 ? 4 : 2;
    const int64_t nvec = ((int64_t)V * elt + 15) / 16;
    if (nvec > (int64_t)sv::kMaxTreeSteps * sv::kTreeStepVecs) return SV_EINVAL;
    if ((int64_t)B * (N + 1) * (int64_t)V > ((int64_t)1 << 40) || B >= (1 << 30)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !temperature || !accepted_len || !out_tokens || (N > 0 && (!parent || !tokens || !path)))
        return SV_EINVAL;
    if (((uintptr_t)target_logits % elt) || (draft_logits && ((uintptr_t)draft_logits % elt))) return SV_EINVAL;
    sv::TreeArgs t = {};
    t.target = static_cast<const char *>(target_logits);
    t.draft = static_cast<const char *>(draft_logits);
    t.parent = parent;
    t.tokens = tokens;
    t.temperature = temperature;
    t.N = N;
    t.V = V;
    t.nvec = (int32_t)nvec;
    t.dtype = dtype;
    t.b0 = 0;
    t.row_bytes = (int64_t)V * elt;
    t.seed = seed;
    t.accepted_len = accepted_len;
    t.out_tokens = out_tokens;
    t.path = path;
    t.error_word = error_word;
    sv::launch_tree(t, B, static_cast<hipStream_t>(stream), static_cast<hipEvent_t>(pass_begin),
                    static_cast<hipEvent_t>(pass_end));
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
    for (int32_t r0 = 0; r0 < rows; r0 += p.sB) {
        const int32_t nr = std::min(p.sB, rows - r0);
        sv::Args a = sv::sub_args(p, workspace, r0, nr);
        a.target = static_cast<const char *>(logits) + (int64_t)r0 * p.row_bytes;
        a.temperature = temperature + r0;
        a.rs_max = row_max + r0;
        a.rs_logsum = row_logsum + r0;
        a.rs_argmax = row_argmax + r0;
        sv::launch_rowstats(a, static_cast<hipStream_t>(stream));
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t spec_verify_stream_probe(const void *target_logits, const void *draft_logits, int32_t B, int32_t K,
                                 int32_t V, int32_t dtype, uint32_t *sink, void *begin, void *end,
                                 void *stream)
{
    if (B < 0 || K < 0 || K > sv::kMaxK || V < 1 || (dtype != SV_F32 && dtype != SV_BF16)) return SV_EINVAL;
    if (B == 0) return SV_OK;
    if (!target_logits || !sink) return SV_EINVAL;
    const size_t elt = dtype == SV_F32 ? 4 : 2;
    if (((uintptr_t)target_logits % elt) || (draft_logits && ((uintptr_t)draft_logits % elt)))
        return SV_EINVAL;
    sv::Plan p;
    if (!sv::make_plan(B, K, V, dtype, &p, !draft_logits && K > 0)) return SV_EINVAL;
    for (int32_t b0 = 0; b0 < B; b0 += p.sB) {
        const int32_t nb = std::min(p.sB, B - b0);
        sv::Args a = {};
        a.B = nb;
        a.K = K;
        a.V = V;
        a.R = p.R;
        a.nvec = p.nvec;
        a.nc = p.nc;
        a.cvec = p.cvec;
        a.dtype = dtype;
        a.row_bytes = p.row_bytes;
        a.target = static_cast<const char *>(target_logits) + (int64_t)b0 * (K + 1) * p.row_bytes;
        a.draft = draft_logits ? static_cast<const char *>(draft_logits) + (int64_t)b0 * K * p.row_bytes
                               : nullptr;
        sv::launch_stream_probe(a, sink, static_cast<hipStream_t>(stream),
                                b0 == 0 ? static_cast<hipEvent_t>(begin) : nullptr,
                                b0 == 0 ? static_cast<hipEvent_t>(end) : nullptr);
    }
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

int32_t spec_verify_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, void *stream)
{
    if (B < 0 || P < 0) return SV_EINVAL;
    const int64_t total = (int64_t)B * P * 2;
    if (total == 0) return SV_OK;
    if (!out || total > ((int64_t)1 << 31)) return SV_EINVAL;
    sv::launch_uniforms(seed, B, P, out, static_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? SV_OK : SV_EHIP;
}

const char *spec_verify_status_str(int32_t status)
{
    switch (status) {
    case SV_OK: return "SV_OK: success";
    case SV_EINVAL: return "SV_EINVAL: invalid argument (nothing enqueued)";
    case SV_EWORKSPACE: return "SV_EWORKSPACE: workspace missing, misaligned or too small";
    case SV_EHIP: return "SV_EHIP: HIP runtime error on launch";
    case SV_ESCRATCH:
        return "SV_ESCRATCH: these sizes need more scratch than spec_verify_noalloc's static buffer "
               "holds (spec_verify_noalloc_max_scratch() bytes); call spec_verify with a workspace";
    default: return "unknown status";
    }
}

}  // extern "C"
