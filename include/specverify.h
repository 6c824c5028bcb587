/*
 * specverify.h -- C ABI of libspecverify, the speculative-sampling verify
 * step for AMD Instinct MI355X (gfx950).
 *
 * The operation (sources cited by page title and section):
 *  - "Kangaroo: Self-Speculative Decoding via Shallow Sub-Networks",
 *    "3. Lossless Speculative Verification": draft token x_i is accepted when
 *    a uniform u satisfies u <= min(1, p_i(x_i) / q_i(x_i)); at the first
 *    rejection one token is drawn from max(0, p_i - q_i) normalised over the
 *    vocabulary and verification stops.  The simulation listing on the same
 *    page counts one guaranteed bonus token per verification.
 *  - glossary "speculative decoding llm", "How Speculative Decoding Works" and
 *    "Why It Produces Identical Outputs": the same rule, whose output law is
 *    exactly the target model's.
 *  - "Speculative Speculative Decoding", "Method": the verification outcome
 *    is (accepted prefix length, bonus token); the bonus comes from the
 *    residual max(p_t - p_d, 0); Saguaro sampling down-weights the most
 *    likely draft probabilities by a factor beta.
 *  - "LayerSkip Guide: Early Exit & Self-Speculative Decoding", "2. The
 *    Drafting and Single-Pass Verification Pipeline": greedy verification
 *    accepts drafts while they equal the target argmax and replaces the first
 *    mismatch by the target argmax.
 *
 * Per sequence b with temperature T = temperature[b] and K drafted tokens
 * x_i = draft_tokens[b, i]:
 *   p_i = softmax(target_logits[b, i, :] / T)   for i = 0..K,
 *   q_i = softmax(draft_logits[b, i, :] / T)    for i = 0..K-1; when beta < 1
 *         the probabilities of the 4 largest draft logits of the row (ties to
 *         the lower token id) are multiplied by beta and q_i is renormalised.
 *   For i = 0, 1, ...: accept x_i iff u(b, i, 0) <= p_i(x_i) / q_i(x_i).
 *   n = index of the first rejection, or K if all are accepted.
 *   The bonus token is the smallest v with C(v) >= u(b, n, 1) * C(V-1), where
 *   C is the running sum in ascending token id of r(v) = max(p_n - q_n, 0)
 *   (n < K) or r(v) = p_K(v) (n == K).  If r has zero mass the bonus is drawn
 *   from p_n the same way.
 *   T == 0 selects greedy mode for that sequence: n = first i with
 *   x_i != argmax p_i (lowest token id on ties), else K; the bonus is the
 *   argmax of target row n; draft logits and beta are not used.
 *   u(b, pos, purpose) = ((w >> 8) + 1) * 2^-24 in (0, 1], where w is the
 *   first output word of Philox4x32-10 (Salmon et al., SC'11) with key
 *   (seed & 0xffffffff, seed >> 32) and counter (b, pos, purpose, 0).
 *
 * Memory and ownership: every array argument is a DEVICE pointer owned by the
 * caller, unless noted.  Arrays are dense and row-major.  Logits are fp32 or
 * bf16 (dtype) and must be aligned to their element size.  Logits may hold
 * -inf (masked tokens); every row that is used needs a finite maximum; NaN or
 * +inf logits give unspecified results.  The library never allocates device
 * memory and never synchronises: all work is enqueued on `stream` (a
 * hipStream_t; NULL is the default stream) and results are ready when the
 * stream is synchronised.  Calls are re-entrant; calls that may overlap in
 * time need distinct workspaces.
 *
 * Workspace: a caller-owned device buffer of spec_verify_workspace_size()
 * bytes, 256-byte aligned, used as scratch (row partials, per-sequence state,
 * residual chunk sums).  Its contents before a call do not matter; a call
 * that is still running owns it.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Logit element types. */
#define SV_F32 0
#define SV_BF16 1

/* Status codes returned synchronously by the host entry points. */
#define SV_OK 0
#define SV_EINVAL (-1)      /* an argument is invalid; nothing was enqueued     */
#define SV_EWORKSPACE (-2)  /* workspace NULL, misaligned or too small         */
#define SV_EHIP (-3)        /* the HIP runtime reported an error on launch     */
#define SV_ESCRATCH (-4)    /* spec_verify_noalloc: sizes beyond its static scratch */

/* Bits of the device-side error word (see sv_aux.error_word). */
#define SV_ERR_TOKEN 1          /* a draft token outside [0, V): treated as rejected    */
#define SV_ERR_TEMPERATURE 2    /* T < 0, NaN or infinite: sequence outputs are -1      */
#define SV_ERR_ROW 4            /* a used row has no finite maximum: outputs are -1     */
#define SV_ERR_DRAFT_MASS 8     /* beta == 0 left a draft row with zero mass: outputs -1 */
#define SV_ERR_NO_DRAFT 16      /* T > 0 but draft_logits is NULL: outputs are -1       */
#define SV_ERR_DRAFT_LEN 32     /* a ragged draft length outside [0, K]: outputs are -1 */
#define SV_ERR_TREE 64          /* a tree parent outside [-1, i-1]: outputs are -1      */

/* Optional per-call diagnostics; every field may be NULL. */
typedef struct sv_aux {
    float *p_target;      /* [B, K] p_i(x_i) at evaluated positions, NaN elsewhere and in greedy mode */
    float *p_draft;       /* [B, K] q_i(x_i) (beta-weighted) at evaluated positions, else NaN         */
    float *residual_mass; /* [B]    C(V-1) of the bonus draw; NaN in greedy mode                      */
    int32_t *error_word;  /* [1]    SV_ERR_* bits are OR-ed in: zero it before the call           */
    void *pass_begin;     /* hipEvent_t stamped with the start of the streaming-pass kernel      */
    void *pass_end;       /* and with its end (first sub-batch only): times the dominant kernel  */
    float *draft_conf;    /* [B, K] draft confidence max_v p_d(v) of each drafted position at the
                             sequence temperature, before the beta re-weighting (every drafted
                             position, reached or not); NaN past the sequence's drafts, in greedy
                             mode and for failed sequences.  Appended last: zero-initialise the
                             whole struct. */
} sv_aux;

/*
 * Bytes of device workspace spec_verify needs for these sizes (0 if the sizes
 * are invalid).  Pure host function.
 */
size_t spec_verify_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype);

/*
 * The verify step.
 *   target_logits  [B, K+1, V] dtype
 *   draft_logits   [B, K, V]   dtype; may be NULL when every temperature is 0
 *   draft_tokens   [B, K]      int32; may be NULL when K == 0
 *   temperature    [B]         float; 0 = greedy for that sequence
 *   beta           host float in [0, 1]; 1 = no draft re-weighting
 *   accepted_len   [B]         int32 out: n in [0, K]
 *   out_tokens     [B, K+1]    int32 out: x_0..x_{n-1}, the bonus token, then -1
 *   workspace      device buffer of >= spec_verify_workspace_size(...) bytes
 *                  (see "Workspace" above)
 *   aux            host pointer to an sv_aux, or NULL
 * B == 0 is a no-op.  Returns SV_OK after enqueuing the work: three kernel
 * launches per sub-batch of at most 8192 sequences (streaming pass; accept
 * scan and residual slot masses; bonus draw), the last one skipped when
 * draft_logits is NULL and K > 0 (every sequence is then greedy or fails).
 */
int32_t spec_verify(const void *target_logits, const void *draft_logits,
                    const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                    uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                    int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                    const sv_aux *aux, void *stream);

/*
 * The verify step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * spec_verify without the workspace arguments.  Its scratch is a static
 * device array of spec_verify_noalloc_max_scratch() bytes (32 MiB) inside the
 * library, one per GPU, held until the process ends; the call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine).  The caller
 * passes inputs and outputs exactly as for spec_verify and gets the same
 * results, bit for bit.  Sizes whose workspace (spec_verify_workspace_size)
 * exceeds the static scratch return SV_ESCRATCH before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (other streams, other host threads) race and give
 * undefined results; serialise them, or use spec_verify with distinct
 * workspaces.  The scratch's contents before a call do not matter.  The
 * first call on a device looks up that device's copy (hipGetSymbolAddress;
 * SV_EHIP if that fails).
 */
size_t spec_verify_noalloc_max_scratch(void);

int32_t spec_verify_noalloc(const void *target_logits, const void *draft_logits,
                            const int32_t *draft_tokens, int32_t B, int32_t K, int32_t V, int32_t dtype,
                            uint64_t seed, const float *temperature, float beta, int32_t *accepted_len,
                            int32_t *out_tokens, const sv_aux *aux, void *stream);

/*
 * The verify step with ragged draft lengths ("Kangaroo: Self-Speculative
 * Decoding via Shallow Sub-Networks", its second early exit stops drafting
 * when the draft's confidence falls below a threshold, so a round carries
 * K_b <= K drafts per sequence):
 *   draft_len      [B] int32 device array: K_b in [0, K] (out of range:
 *                  SV_ERR_DRAFT_LEN, the sequence's outputs are -1); NULL
 *                  means K for every sequence (exactly spec_verify)
 * The logit tensors keep their [B, K+1, V] and [B, K, V] layouts; sequence b
 * verifies drafts 0..K_b-1 and, after K_b acceptances, draws its bonus from
 * target row K_b; rows past those are never read.  out_tokens keeps K+1
 * slots (-1 after the bonus), uniforms are keyed as for K = K_b, and
 * draft_logits may be NULL when every sampling sequence has K_b == 0.
 * Everything else as spec_verify.
 */
int32_t spec_verify_ragged(const void *target_logits, const void *draft_logits,
                           const int32_t *draft_tokens, const int32_t *draft_len, int32_t B,
                           int32_t K, int32_t V, int32_t dtype, uint64_t seed,
                           const float *temperature, float beta, int32_t *accepted_len,
                           int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                           const sv_aux *aux, void *stream);

/*
 * Per-row statistics of `rows` rows of V logits (the streaming pass of the
 * verify step on its own, for parity checks of the row reduction):
 *   row_max[r]    = max_v z[r, v]
 *   row_logsum[r] = ln sum_v exp((z[r, v] - row_max[r]) / temperature[r]) when
 *                   temperature[r] > 0, else NaN
 *   row_argmax[r] = lowest v attaining row_max[r] when temperature[r] == 0, else -1
 * All output pointers are device pointers and may not be NULL.
 * Workspace: >= spec_verify_workspace_size(rows, 0, V, dtype) bytes.
 */
int32_t spec_verify_row_stats(const void *logits, int32_t rows, int32_t V, int32_t dtype,
                              const float *temperature, float *row_max, double *row_logsum,
                              int32_t *row_argmax, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * The uniforms the verify step draws: out[(b * P + pos) * 2 + purpose] =
 * u(b, pos, purpose) for b < B, pos < P, purpose in {0 (accept), 1 (bonus)}.
 */
int32_t spec_verify_uniforms(uint64_t seed, int32_t B, int32_t P, float *out, void *stream);

/*
 * Measurement aid: the streaming pass of spec_verify for these arguments
 * (same grid, rows, chunks, 16-byte loads and tiles, every target row and,
 * when draft_logits is not NULL, every draft row) with its arithmetic taken
 * out, so that its duration is the read floor the pass runs against.
 *   sink         one device uint32; written only for one input pattern in
 *                2^32 (it keeps the loads), so its contents are meaningless
 *   begin, end   hipEvent_t or NULL: stamped with the start and end of the
 *                first sub-batch's kernel
 * Validation as for spec_verify (no workspace).  Returns after enqueuing.
 */
int32_t spec_verify_stream_probe(const void *target_logits, const void *draft_logits, int32_t B, int32_t K,
                                 int32_t V, int32_t dtype, uint32_t *sink, void *begin, void *end,
                                 void *stream);

/*
 * The verification-outcome distribution ("Speculative Speculative Decoding",
 * "Method": a verification outcome is the accepted prefix length together
 * with the bonus token, and the speculator prepares drafts for the likeliest
 * outcomes).  For each sequence with T > 0, over drafts drawn from the
 * (beta-weighted) draft law q'_j the verify step assumes:
 *   accept_rate [B, K]      alpha_j = sum_v min(p_j(v), q'_j(v))
 *   p_len       [B, K+1]    P(n = k) = (prod_{j<k} alpha_j)(1 - alpha_k),
 *                           P(n = K) = prod_j alpha_j
 *   top_tokens  [B, K+1, F] int32: per position k, the F tokens of largest
 *                           r_k(v) = max(p_k(v) - q'_k(v), 0) (k < K) or
 *                           p_K(v) (k = K), in descending order, ties to the
 *                           lower token id; -1 past the positive ones
 *   top_mass    [B, K+1, F] those r_k(v) (p_K(v)), 0 past the positive ones;
 *                           P(n = k, bonus = v) = prod_{j<k} alpha_j * r_k(v)
 *   draft_top_mass [B, K]   optional (NULL: not formed): sum of r_k(v) over
 *                           the 4 largest logits of draft row k (ties to the
 *                           lower id), the tokens beta down-weights; the bonus
 *                           of a rejection at k is one of them with probability
 *                           draft_top_mass_k / (1 - alpha_k) ("Key claims":
 *                           Saguaro sampling concentrates the residual there
 *                           to raise the speculation cache's hit rate)
 * p, q' and beta as in spec_verify; all K positions of every sequence are
 * used, whatever was drafted.  Outputs are float32 (alpha clamped to [0, 1]);
 * the r values are ranked as computed in fp32, so tokens whose masses agree
 * to ~1e-6 may appear in either order.  Greedy sequences (T == 0, whose
 * outcome their drafts fix) get NaN, -1 and 0; so do failed ones, whose
 * failures (SV_ERR_TEMPERATURE, SV_ERR_ROW, SV_ERR_DRAFT_MASS, and
 * SV_ERR_NO_DRAFT when T > 0, K > 0 and draft_logits is NULL) are OR-ed into
 * *error_word when error_word is not NULL.
 *   target_logits  [B, K+1, V] dtype;  draft_logits [B, K, V] dtype or NULL
 *   temperature    [B] float;  beta host float in [0, 1]
 *   F              ranked tokens per position, 0..32 (top_tokens and
 *                  top_mass may be NULL when F == 0; accept_rate when K == 0)
 *   workspace      device buffer of >= spec_verify_outcomes_workspace_size()
 *                  bytes, 256-byte aligned (scratch)
 *   pass_begin, pass_end  hipEvent_t or NULL: stamped with the start and end
 *                  of the outcome-pass kernel of the first sub-batch
 * Device pointers, stream ordering and ownership as for spec_verify.
 * Three kernel launches per sub-batch of at most 8192 sequences: the
 * streaming pass of spec_verify, the outcome pass (a second read of every
 * row: the clamp and the ranking need both rows' normalisers), and a
 * per-sequence finish.  Returns SV_OK after enqueuing the work.
 */
size_t spec_verify_outcomes_workspace_size(int32_t B, int32_t K, int32_t V, int32_t dtype, int32_t F);

int32_t spec_verify_outcomes(const void *target_logits, const void *draft_logits, int32_t B, int32_t K,
                             int32_t V, int32_t dtype, const float *temperature, float beta, int32_t F,
                             float *accept_rate, float *p_len, int32_t *top_tokens, float *top_mass,
                             float *draft_top_mass, int32_t *error_word, void *workspace,
                             size_t workspace_bytes, void *pass_begin, void *pass_end, void *stream);

/*
 * Tree (multi-draft) verification.  The pages name tree-based speculative
 * decoding ("Speculative Speculative Decoding", Key claims: SSD composes with
 * Medusa-style trees) without its verify rule; this is the published
 * recursive rejection sampling over a token tree (Miao et al., "SpecInfer",
 * ASPLOS'24), lossless when the children of every context are drawn i.i.d.
 * from that context's draft law.
 *   parent        [B, N] int32: parent of node i in [-1, i-1] (-1: the root);
 *                 otherwise SV_ERR_TREE and the sequence's outputs are -1
 *   tokens        [B, N] int32: the token of node i
 *   target_logits [B, N+1, V] dtype: row c = target logits after context c
 *                 (context 0: the root, context i + 1: node i)
 *   draft_logits  [B, N, V] dtype: row c = the draft logits the children of
 *                 context c were drawn from (rows of contexts without
 *                 children are never read); NULL when every temperature is 0
 *   temperature   [B] float; 0 = greedy
 *   accepted_len  [B] int32 out: d, the number of accepted nodes
 *   out_tokens    [B, N+1] int32 out: the accepted tokens, the bonus, then -1
 *   path          [B, N] int32 out: the accepted nodes, then -1
 *   error_word    device int32 or NULL: SV_ERR_* bits OR-ed in (TOKEN, TEMPERATURE,
 *                 ROW, NO_DRAFT, TREE as for spec_verify)
 *   pass_begin, pass_end  hipEvent_t or NULL, stamped with the kernel's start and end
 * At the current context (first the root) the law r starts as its target
 * law p = softmax(target row / T).  Its children are tried in ascending node
 * index: child j with token x is accepted iff u(b, j, 0) <= r(x) / q(x),
 * q = softmax(draft row / T); a rejection replaces r by max(r - q, 0)
 * normalised (unchanged if that has no mass).  An accepted child becomes the
 * current context.  When no child is left, the bonus is the smallest v with
 * C(v) >= u(b, d, 1) C(V-1), C the running sum of r in token order.  Greedy
 * sequences accept the first child whose token is the target argmax and emit
 * the final context's argmax.  u as for spec_verify; a chain (parent[i] =
 * i - 1) gives exactly spec_verify with K = N.  Only the rows of the
 * contexts the walk visits are read.  N <= 128; V up to 2048 * 1024 16-byte
 * vectors.  One kernel launch (one workgroup per sequence); no workspace.
 * Returns SV_OK after enqueuing the work.
 */
int32_t spec_verify_tree(const void *target_logits, const void *draft_logits, const int32_t *parent,
                         const int32_t *tokens, int32_t B, int32_t N, int32_t V, int32_t dtype,
                         uint64_t seed, const float *temperature, int32_t *accepted_len,
                         int32_t *out_tokens, int32_t *path, int32_t *error_word, void *pass_begin,
                         void *pass_end, void *stream);

/* Static description of a status code. */
const char *spec_verify_status_str(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
