/*
 * sv.h -- C ABI of the batched speculative-sampling verifier for AMD Instinct MI355X (gfx950).
 *
 * The rule (Leviathan et al., as restated on the page "Uno: the draft model was already inside the target model",
 * section "What 'lossless' actually has to mean"): a drafted token x, proposed from q, is accepted when a uniform
 * u satisfies u < min(1, p(x)/q(x)); the block is cut at the first rejection (DFlash/DFlash2 guide, section 4.4),
 * where one replacement token is drawn from max(p - q, 0) renormalised; when every draft is accepted, one bonus
 * token is drawn from the target's next distribution (same guide, section 2: tokens per cycle in [1, gamma + 1]).
 * Dense calls form p = softmax(z_target / T) and q = softmax(z_draft / T) (same guide, section 9 Q3: temperature on
 * both sides before the ratio).
 *
 * Conventions shared by every entry point
 * - Every array argument is a DEVICE pointer owned by the caller. The library allocates nothing, keeps no state of
 *   its own between calls (what a call leaves for the next one lives in the caller's workspace, see
 *   sv_workspace_bytes) and may be called from several host threads on different streams.
 * - Work is enqueued on `stream` (a hipStream_t, or NULL for the null stream) of the current device; outputs are
 *   valid once that stream has reached the enqueued work. No call synchronises the host.
 * - The return value is 0 (SV_OK) or a negative SV_ERR_* code. Argument errors are detected on the host BEFORE any
 *   HIP call, so nothing has been enqueued when one is returned. SV_ERR_HIP means a launch failed.
 * - Data faults inside the tensors do not fail the call; they are reported per sequence in `flags` (SV_FLAG_*).
 *   A sequence with SV_FLAG_NONFINITE or SV_FLAG_ID_RANGE is not verified: n_accepted = -1, out_token = -1,
 *   accept = 0 for all its rows, p_draft / q_draft (or p_spec / q_spec / correction_probs) = NaN.
 * - The index of a draw is the smallest i whose inclusive running sum of the draw's weights exceeds t = u * (total
 *   weight), in vocabulary order (dense) or in the given support-slot order (sparse); if rounding leaves no such i,
 *   the last index with positive weight is taken. An empty residual (zero total) draws from p instead and sets
 *   SV_FLAG_EMPTY_RESIDUAL.
 * - The accept test is strict (u == min(1, ratio) rejects), as in the engine routine printed on the Uno page.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------------------------------- */
#define SV_OK             0
#define SV_ERR_NULL      (-1)   /* a required pointer is NULL                                                     */
#define SV_ERR_SHAPE     (-2)   /* B, gamma, V, k or a stride out of range, or a size product overflows          */
#define SV_ERR_DTYPE     (-3)   /* dtype is not SV_F32 or SV_BF16                                                 */
#define SV_ERR_TEMP      (-4)   /* temperature is not finite or is <= 0                                           */
#define SV_ERR_ALIGN     (-5)   /* a pointer is not aligned to its element size (workspace: to 256 bytes)        */
#define SV_ERR_WORKSPACE (-6)   /* workspace smaller than sv_workspace_bytes() or NULL while bytes are needed     */
#define SV_ERR_HIP       (-7)   /* a kernel launch failed                                                         */
#define SV_ERR_ARG       (-8)   /* any other invalid argument (bonus not 0/1, unknown kind)                       */
#define SV_ERR_SCRATCH   (-9)   /* the call needs more scratch than SV_NOALLOC_SCRATCH_BYTES (no-allocation call)  */

/* ---- logit element types ------------------------------------------------------------------------------------ */
#define SV_F32  0
#define SV_BF16 1

/* ---- workspace kinds ---------------------------------------------------------------------------------------- */
#define SV_KIND_DENSE  0
#define SV_KIND_ONEHOT 1
#define SV_KIND_SPARSE 2
#define SV_KIND_GREEDY 3
#define SV_KIND_TREE   4

/* ---- per-sequence flags ------------------------------------------------------------------------------------- */
#define SV_FLAG_NONFINITE      1u  /* NaN or +inf logit (or a row all -inf) in a row that was read; for sparse, a
                                      NaN, infinite or negative probability. Fatal for the sequence, except in the
                                      bonus row, where it only voids the bonus token (out_token = -1).           */
#define SV_FLAG_ID_RANGE       2u  /* a draft / spec id outside [0, V) (sparse: outside [0, vocab_size) when given,
                                      for spec and support ids), `order` not a permutation of [0, gamma), or
                                      start outside [0, gamma]. Fatal for the sequence.                          */
#define SV_FLAG_EMPTY_RESIDUAL 4u  /* the residual had zero mass and the draw used p instead. Informational.      */
#define SV_FLAG_Q_ZERO         8u  /* q was exactly 0 at a verified draft (ratio 0, rejected). Informational.     */
#define SV_FLAG_INTERNAL      16u  /* a hand-off between the workgroups of the call failed its check or timed out
                                      (workspace shared by concurrent calls, or overwritten during the call): the
                                      sequence was not verified (n_accepted = -1, out_token = -1). Fatal.         */

/* ---- limits ------------------------------------------------------------------------------------------------- */
#define SV_MAX_GAMMA 1024        /* drafted positions per sequence                                                */
#define SV_MAX_K     256         /* support size of a sparse row (kp, kq)                                          */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)   /* scratch each GPU holds for sv_verify_dense_noalloc               */
#define SV_MAX_TREE_NODES 1024   /* nodes of one token tree (the root included)                                    */

/*
 * Bytes of device workspace a call of `kind` needs for B sequences of gamma drafts over V_or_k (V for dense,
 * one-hot and greedy, the p-support size kp for sparse). Depends only on these arguments. Returns 0 when no workspace is
 * needed and (size_t)-1 for arguments the calls would reject. The workspace holds the call's work-queue counters
 * and scratch records; its first 256 bytes are a header naming the layout of those counters. Its initial contents
 * do not matter: the first workgroup of every call compares the header with the call's layout and, when they
 * differ (first use, another kind or shape of call, or an earlier call that stopped early), zeroes the counters
 * inside the same launch before any other workgroup uses them. Every call leaves its counters at zero, so the same
 * workspace serves any number of later calls of any kind and shape it is large enough for. Apart from the header
 * and the counters its contents are meaningless after a call. It must not be shared by calls that may run
 * concurrently (they would race on the counters; a sequence whose hand-off then fails its checks is flagged
 * SV_FLAG_INTERNAL).
 */
size_t sv_workspace_bytes(int kind, int64_t B, int32_t gamma, int64_t V_or_k);

/* Static text for a status code. */
const char* sv_status_string(int status);

/*
 * Dense verification: p and q from full logit rows.
 *
 * target_logits  [B][gamma + bonus][V] of `dtype`; element (b, r, i) at target_logits[b*t_seq + r*t_row + i].
 *                Row gamma is read only for a bonus draw. Rows of slots before `start` are not read.
 * draft_logits   [B][gamma][V] of `dtype`, at draft_logits[b*d_seq + r*d_row + i].
 * dtype          SV_F32 or SV_BF16 (both tensors). Pointers aligned to the element size; rows need no further
 *                alignment (strides are in elements and must be >= 1; V is contiguous).
 * B, gamma, V    1 <= B <= 2^31-1, 1 <= gamma <= SV_MAX_GAMMA, 1 <= V <= 2^31-1.
 * draft_ids      [B][gamma] int32, the drafted token of each storage row.
 * u_accept       [B][gamma] float uniforms in [0, 1) for the accept tests, by storage row.
 * u_sample       [B][gamma + 1] float uniforms in [0, 1): a residual draw at slot k reads u_sample[b][order[k]],
 *                the bonus draw reads u_sample[b][gamma].
 * temperature    T > 0, finite: p = softmax(z_target / T), q = softmax(z_draft / T).
 * bonus          1: draw a bonus token from target row gamma when every verified slot is accepted; 0: no bonus
 *                (out_token = -1 then), and the target needs only gamma rows.
 * start          [B] int32 or NULL (= all 0). Slots start[b] .. gamma-1 are verified. On return start[b] is set to
 *                min(gamma, k + 1), k = the first rejected slot (gamma if none), so that consecutive calls chain
 *                verification rounds over one window (Self-Speculative Masked Diffusions, 关键设计 2 and 4). A
 *                sequence with start[b] == gamma is finished: nothing is read, n = 0, out_token = -1, start kept.
 * order          [B][gamma] int32 or NULL (= identity): slot s verifies storage row order[b][s].
 * accept         [B][gamma] uint8 or NULL: the raw test of every verified row (0 for rows before start).
 * n_accepted     [B] int32 (required): accepted drafts from start up to the first rejection.
 * out_token      [B] int32 (required): the residual or bonus token, or -1.
 * p_draft/q_draft [B][gamma] float or NULL: p(x) and q(x) at each verified row (0 elsewhere).
 * flags          [B] uint32 or NULL.
 * workspace      >= sv_workspace_bytes(SV_KIND_DENSE, B, gamma, V) bytes of device memory, 256-byte aligned.
 */
int sv_verify_dense(const void* target_logits, int64_t t_seq, int64_t t_row,
                    const void* draft_logits, int64_t d_seq, int64_t d_row,
                    int dtype, int64_t B, int32_t gamma, int64_t V,
                    const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                    float temperature, int32_t bonus,
                    int32_t* start, const int32_t* order,
                    uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                    float* p_draft, float* q_draft, uint32_t* flags,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * sv_verify_dense without a workspace, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same arguments, outputs and errors as
 * sv_verify_dense, minus workspace / workspace_bytes: the call's scratch is a static device array of
 * SV_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the process ends. Its address is looked
 * up once per device, on the first call with that device current; the call itself allocates nothing (no hipMalloc,
 * hipFree or allocating library routine). Returns SV_ERR_SCRATCH when sv_workspace_bytes(SV_KIND_DENSE, B, gamma,
 * V) exceeds SV_NOALLOC_SCRATCH_BYTES (16 MiB: B = 64, gamma = 16, V = 151936 needs 1.8 MiB), and SV_ERR_HIP when the
 * scratch's address cannot be found. All calls on one GPU share that GPU's array: calls that may overlap on one GPU
 * (different streams, or host threads) race on it and must not be made; calls ordered on one stream are safe. The
 * array keeps the last call's contents, and each call clears the control words it needs inside its own launch.
 */
int sv_verify_dense_noalloc(const void* target_logits, int64_t t_seq, int64_t t_row,
                            const void* draft_logits, int64_t d_seq, int64_t d_row,
                            int dtype, int64_t B, int32_t gamma, int64_t V,
                            const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                            float temperature, int32_t bonus,
                            int32_t* start, const int32_t* order,
                            uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                            float* p_draft, float* q_draft, uint32_t* flags, void* stream);

/*
 * Greedy-draft verification (the last paragraph of the Uno page's section "What 'lossless' actually has to mean":
 * a greedy drafter makes q one-hot, and the rule must be applied to that q): q = e_d at the draft id d, so the
 * test is u < p(d) and the residual is p with d removed, renormalised. No draft logits exist and only target rows
 * are read. Arguments as for sv_verify_dense without the draft tensor and q_draft.
 * workspace >= sv_workspace_bytes(SV_KIND_ONEHOT, B, gamma, V).
 */
int sv_verify_onehot_draft(const void* target_logits, int64_t t_seq, int64_t t_row,
                           int dtype, int64_t B, int32_t gamma, int64_t V,
                           const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                           float temperature, int32_t bonus,
                           int32_t* start, const int32_t* order,
                           uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                           float* p_draft, uint32_t* flags,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse verification on top-k supports, following the engine routine printed on the Uno page (section "What
 * 'lossless' actually has to mean"): p_spec and q_spec are the support probabilities whose id equals the drafted
 * id (summed in slot order); accept iff q_spec > 0 and u < min(1, p_spec / q_spec), evaluated exactly as
 * u * q_spec < p_spec in float64; the correction distribution on p's support is max(p_i - q_on_p_i, 0) renormalised,
 * with q_on_p_i the q probability of p's i-th id. Probabilities are used as given (no renormalisation of p or q).
 * All arithmetic is float64 in slot order, so every output equals the float64 evaluation of these definitions.
 *
 * p_ids, p_probs  [B][gamma + bonus][kp] int32 / float, contiguous (row gamma only read for a bonus draw).
 * q_ids, q_probs  [B][gamma][kq] int32 / float, contiguous.
 * kp, kq          1 .. SV_MAX_K.
 * vocab_size      > 0: spec and support ids outside [0, vocab_size) flag SV_FLAG_ID_RANGE; 0: ids unchecked.
 * spec_ids        [B][gamma] int32 drafted ids; u_accept [B][gamma]; u_sample [B][gamma + 1] (column k for a
 *                 residual draw at slot k, column gamma for the bonus).
 * accept          [B][gamma] uint8 or NULL; n_accepted, out_token [B] int32 (required).
 * correction_probs [B][gamma][kp] float or NULL: the draw distribution of each row (p's fallback when empty).
 * p_spec, q_spec  [B][gamma] float or NULL.  flags [B] uint32 or NULL.
 * workspace       unused (sv_workspace_bytes returns 0); may be NULL.
 */
int sv_verify_sparse(const int32_t* p_ids, const float* p_probs,
                     const int32_t* q_ids, const float* q_probs,
                     int64_t B, int32_t gamma, int32_t kp, int32_t kq, int64_t vocab_size,
                     const int32_t* spec_ids, const float* u_accept, const float* u_sample, int32_t bonus,
                     uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                     float* correction_probs, float* p_spec, float* q_spec, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k / top-p support builder: dense logit rows to the (ids, probs) supports that sv_verify_sparse takes. The
 * sampler settings are those of the throughput test on the Uno page (section "The speedup, without the 'up to'":
 * temperature 1, top-p 0.95, top-k 50), whose sparse verify routine (section "What 'lossless' actually has to mean")
 * takes p and q as such supports; the temperature divides the logits first (DFlash/DFlash2 guide, section 9 Q3).
 * The pages name the parameters only; the procedure is the usual sampler's, in this order:
 * - top-k: the k largest logits of the row, equal logits ordered by ascending id, listed in descending order
 *   (the order is the same at every T > 0);
 * - top-p on the top-k distribution t_j = e_j / sum(e), e_j = exp(z_j / T - z_0 / T): slot j is kept when j = 0 or
 *   t_0 + ... + t_{j-1} < top_p, i.e. the shortest prefix whose mass reaches top_p, the crossing slot included;
 *   the cumulative sums and the comparison are float64;
 * - probs of kept slots: renorm = 1, e_j over the sum of the kept e (they sum to 1); renorm = 0, the row's full
 *   softmax probability exp(z_j / T) / sum over all V of exp(z_i / T) (they sum to the kept mass). Slots past the
 *   kept ones keep their ids and get probability 0, so every output row is a valid support of k slots.
 *
 * logits       rows of V logits of `dtype`, row r at logits + r * ld elements (ld >= V; V contiguous); pointer
 *              aligned to the element size.
 * rows, V      1 <= rows, V <= 2^31-1.   k: 1 .. min(SV_MAX_K, V).
 * temperature  T > 0, finite.   top_p: in (0, 1] (1: no cut beyond rounding).   renorm: 0 or 1.
 * ids          [rows][k] int32 (required): the top-k ids in descending order.
 * probs        [rows][k] float (required).
 * count        [rows] int32 or NULL: kept slots (1 .. k).
 * flags        [rows] uint32 or NULL: SV_FLAG_NONFINITE for a row with a NaN or +inf logit, or all -inf; such a
 *              row gets ids -1, probs NaN, count 0 (so a sparse verify of it flags the sequence). 0 otherwise.
 * workspace    >= sv_support_workspace_bytes(rows, V, k) bytes, 256-byte aligned, any initial contents (the same
 *              contract as sv_workspace_bytes; a workspace may alternate between this call and the verify calls).
 */
size_t sv_support_workspace_bytes(int64_t rows, int64_t V, int32_t k);
int sv_build_support(const void* logits, int64_t ld, int dtype, int64_t rows, int64_t V,
                     float temperature, int32_t k, float top_p, int32_t renorm,
                     int32_t* ids, float* probs, int32_t* count, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same support builder over two sets of rows in one launch: the target's rows and the draft's that one sparse
 * verify takes as p and q (Uno page, section "What 'lossless' actually has to mean"), under the same settings. Each
 * output row is the one sv_build_support gives for that row alone; one launch lets the second set's rows fill the
 * schedule the first set's leave partly empty, and pays one launch and one tail instead of two.
 *
 * logits_a, ld_a, rows_a   the first set, as logits, ld, rows of sv_build_support; ids_a, probs_a, count_a, flags_a
 *                          its outputs, as there.
 * logits_b ... flags_b     the second set, the same way (rows_b >= 1; rows_a + rows_b <= 2^31-1).
 * dtype, V, temperature, k, top_p, renorm   shared by both sets, as in sv_build_support.
 * workspace                >= sv_support_workspace_bytes(rows_a + rows_b, V, k) bytes, as in sv_build_support.
 * The two sets' outputs must not overlap each other; their logits may (the rows are only read).
 * Errors: those of sv_build_support, for either set; SV_ERR_SHAPE also when rows_b < 1 or the two sets together
 * pass 2^31-1 rows.
 */
int sv_build_support_pair(const void* logits_a, int64_t ld_a, int64_t rows_a,
                          const void* logits_b, int64_t ld_b, int64_t rows_b,
                          int dtype, int64_t V, float temperature, int32_t k, float top_p, int32_t renorm,
                          int32_t* ids_a, float* probs_a, int32_t* count_a, uint32_t* flags_a,
                          int32_t* ids_b, float* probs_b, int32_t* count_b, uint32_t* flags_b,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verification at temperature 0 (DFlash/DFlash2 guide, section 4.4: under greedy decoding a drafted token is
 * kept exactly when it is the target's most likely token; the block is cut at the first one that is not). The
 * target's choice at a row is the argmax of its logits, equal maxima going to the lowest id. Slots start[b] ..
 * gamma-1 are checked in `order`; at the first mismatching slot k the target's argmax there is emitted; when every
 * checked draft matches and bonus = 1, the argmax of target row gamma is emitted (section 2: up to gamma + 1 tokens
 * per cycle). No draft logits, uniforms or temperature are involved: every output is an integer decision that the
 * logits fix exactly.
 *
 * target_logits  [B][gamma + bonus][V] of `dtype` at target_logits[b*t_seq + r*t_row + i]; pointer aligned to the
 *                element size (rows need no further alignment; strides >= 1; V contiguous). Every row of a slot
 *                >= start is read, and row gamma whenever the sequence is live (bonus = 1), even if unused.
 * dtype          SV_F32 or SV_BF16.
 * B, gamma, V    1 <= B <= 2^31-1, 1 <= gamma <= SV_MAX_GAMMA, 1 <= V <= 2^31-1.
 * draft_ids      [B][gamma] int32, the drafted token of each storage row.
 * bonus          0 or 1 (with 0 the target needs only gamma rows and out_token is -1 after a full match).
 * start          [B] int32 or NULL (= all 0), updated to min(gamma, k + 1) as for sv_verify_dense; a sequence with
 *                start[b] == gamma is finished (nothing read, n = 0, out_token = -1).
 * order          [B][gamma] int32 or NULL (= identity): slot s checks storage row order[b][s].
 * accept         [B][gamma] uint8 or NULL: 1 where a checked row's draft equals its argmax (0 for rows before start).
 * n_accepted     [B] int32 (required): matches from start up to the first mismatch; -1 for a fault.
 * out_token      [B] int32 (required): the argmax at the first mismatch, the bonus argmax, or -1.
 * flags          [B] uint32 or NULL: SV_FLAG_ID_RANGE (a draft id outside [0, V) in a checked slot, order not a
 *                permutation, start outside [0, gamma]) and SV_FLAG_NONFINITE (a NaN or +inf logit, or a row all
 *                -inf, in a checked row; in row gamma only when the bonus is taken from it). Either one in a
 *                checked slot makes the sequence fail: n = -1, out_token = -1, accept 0, start unchanged; a bad bonus
 *                row only sets the flag and leaves out_token = -1.
 * workspace      >= sv_workspace_bytes(SV_KIND_GREEDY, B, gamma, V) bytes of device memory, 256-byte aligned,
 *                any initial contents (same contract as the other calls).
 * Errors: SV_ERR_NULL, SV_ERR_DTYPE, SV_ERR_SHAPE, SV_ERR_ARG (bonus), SV_ERR_ALIGN, SV_ERR_WORKSPACE, SV_ERR_HIP,
 * all returned before anything is launched except SV_ERR_HIP.
 */
int sv_verify_greedy(const void* target_logits, int64_t t_seq, int64_t t_row,
                     int dtype, int64_t B, int32_t gamma, int64_t V,
                     const int32_t* draft_ids, int32_t bonus,
                     int32_t* start, const int32_t* order,
                     uint8_t* accept, int32_t* n_accepted, int32_t* out_token, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Confidence-threshold commit of block diffusion (SDAR-style block diffusion page, section 5 "Decoding timeline":
 * each pass gives a distribution over the vocabulary at every masked slot of the block; slots whose confidence
 * reaches tau are committed, at least the most confident one, so every pass makes progress). This is the decoding
 * rule of a masked-diffusion pass, not a verifier: it is lossy by design.
 * Per masked slot j of block b: token = argmax of the logits (equal maxima to the lowest id) and confidence = its
 * softmax probability 1 / sum_i exp(z_i - max) (temperature 1), merged in float64. Committed: the masked slots with
 * confidence >= tau; if there are none, the single most confident masked slot (equal confidences: the lowest j).
 *
 * logits      [B][W][V] of `dtype` at logits[b*l_seq + j*l_row + i]; pointer aligned to the element size, rows need
 *             no further alignment; only masked slots are read.
 * B, W, V     1 <= B <= 2^31-1, 1 <= W <= SV_MAX_GAMMA, 1 <= V <= 2^31-1.
 * masked      [B][W] uint8 or NULL (= every slot masked): nonzero = the slot is still masked.
 * tau         in [0, 1] (float; compared with the float64 confidence), else SV_ERR_ARG.
 * commit      [B][W] uint8 or NULL: 1 for a committed slot.
 * token       [B][W] int32 (required): the committed token, -1 elsewhere.
 * confidence  [B][W] float or NULL: the confidence of each masked slot (rounded to float), NaN elsewhere.
 * n_commit    [B] int32 (required): committed slots (0 when none is masked), -1 for a fault.
 * flags       [B] uint32 or NULL: SV_FLAG_NONFINITE for a NaN or +inf logit, or a row all -inf, in a masked slot;
 *             such a block commits nothing (token -1, confidence NaN).
 * workspace   >= sv_workspace_bytes(SV_KIND_GREEDY, B, W, V) bytes, 256-byte aligned, any initial contents (same
 *             contract as the other calls; it may alternate with sv_verify_greedy and the others).
 * Errors: SV_ERR_NULL, SV_ERR_DTYPE, SV_ERR_SHAPE, SV_ERR_ARG, SV_ERR_ALIGN, SV_ERR_WORKSPACE, SV_ERR_HIP.
 */
int sv_confidence_commit(const void* logits, int64_t l_seq, int64_t l_row, int dtype, int64_t B, int32_t W,
                         int64_t V, const uint8_t* masked, float tau, uint8_t* commit, int32_t* token,
                         float* confidence, int32_t* n_commit, uint32_t* flags,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Tree (multi-candidate) verification. The pages verify trees of drafted tokens (the Uno page's B = 16 tree sampler,
 * section "One backbone, two pathways"; EAGLE-2's dynamic draft trees, DFlash/DFlash2 guide section 3; DFlash2's
 * top-m candidates per position submitted as a dense verification tree, section 5.2) but state the acceptance rule
 * for one candidate per position, with its one-hot form for a greedy drafter (Uno, "What 'lossless' actually has to
 * mean"). For several candidates the rule is SpecInfer's multi-step speculative sampling (Miao et al., ASPLOS 2024)
 * with q one-hot at each candidate (candidates chosen deterministically, as top-m drafters choose them):
 * - node 0 is the root; row i of the target logits is the target's distribution after the path to node i, and
 *   p_i = softmax(row_i / T);
 * - at node u the children of u are tested in increasing node index: child c with token x passes when
 *   u_accept[c] < min(1, p'(x)), p' = p_u without the tokens of the children of u already rejected, renormalised
 *   (a token already rejected has p'(x) = 0 and fails); a passing child is accepted and the walk continues there;
 * - where every child fails, or at a node without children, one token is drawn from p' (p_u without the rejected
 *   tokens; at a leaf, p_u itself) by the draw rule above, at t = u_sample[u] * (mass of p').
 * With distinct candidates the emitted tokens follow the target's own law (Leviathan et al.'s guarantee).
 *
 * target_logits  [B][N][V] of `dtype` at target_logits[b*t_seq + i*t_row + v]; pointer aligned to the element size
 *                (rows need no further alignment; strides >= 1; V contiguous). Every row is read once, the stop
 *                node's row twice.
 * B, N, V        1 <= B <= 2^31-1, 1 <= N <= SV_MAX_TREE_NODES, 1 <= V <= 2^31-1.
 * parent, token  [B][N] int32: parent[b][i] in [0, i) and token[b][i] in [0, V) for i >= 1 (element 0 unused),
 *                else the sequence is flagged SV_FLAG_ID_RANGE and not verified.
 * u_accept       [B][N] float in [0, 1): the test of node i (element 0 unused).
 * u_sample       [B][N] float in [0, 1): the draw when the walk stops at node i.
 * temperature    T > 0, finite.
 * accept         [B][N] uint8 (required): 1 for the accepted nodes, 0 elsewhere.
 * n_accepted     [B] int32 (required): accepted nodes (the depth of the stop node), -1 for a failed sequence.
 * path           [B][N] int32 (required): the accepted nodes from the root down, -1 after them.
 * out_token      [B] int32 (required): the token drawn at the stop node, -1 for a failed sequence.
 * p_test         [B][N] float or NULL: p'(x) of every tested node, NaN for nodes not tested.
 * flags          [B] uint32 or NULL: SV_FLAG_ID_RANGE (tree or token out of range), SV_FLAG_NONFINITE (a NaN or
 *                +inf logit, or a row all -inf, in a row the walk reaches; rows off the walk are not checked),
 *                SV_FLAG_EMPTY_RESIDUAL (the rejected tokens held all of p at the stop node: drawn from p).
 * workspace      >= sv_workspace_bytes(SV_KIND_TREE, B, N, V) bytes, 256-byte aligned, any initial contents (same
 *                contract as the other calls).
 * Two kernels on `stream`: the row statistics with the walk, then the draw.
 * Errors: SV_ERR_NULL, SV_ERR_DTYPE, SV_ERR_SHAPE, SV_ERR_TEMP, SV_ERR_ALIGN, SV_ERR_WORKSPACE, SV_ERR_HIP.
 */
int sv_verify_tree(const void* target_logits, int64_t t_seq, int64_t t_row, int dtype, int64_t B, int32_t N,
                   int64_t V, const int32_t* parent, const int32_t* token, const float* u_accept,
                   const float* u_sample, float temperature, uint8_t* accept, int32_t* n_accepted, int32_t* path,
                   int32_t* out_token, float* p_test, uint32_t* flags, void* workspace, size_t workspace_bytes,
                   void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
