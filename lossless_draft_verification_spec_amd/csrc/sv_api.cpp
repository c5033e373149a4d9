// Exported C entry points of the verifier library: argument validation on the host (before any HIP call),
// workspace sizing and launch sequencing. The kernels live in sv_dense.hip, sv_sparse.hip and sv_support.hip.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <limits>

#include "sv.h"
#include "sv_greedy.h"
#include "sv_internal.h"

namespace {

constexpr int64_t kMaxI32 = std::numeric_limits<int32_t>::max();

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by the dense and one-hot calls. Returns SV_OK or an error code.
int check_dense_common(const void* tgt, int64_t t_seq, int64_t t_row, int dtype, int64_t B, int32_t gamma, int64_t V,
                       const int32_t* ids, const float* ua, const float* us, float temperature, int32_t bonus,
                       int32_t* start, const int32_t* order, uint8_t* accept, int32_t* n_acc, int32_t* token,
                       float* p_draft, uint32_t* flags) {
  if (!tgt || !ids || !ua || !us || !n_acc || !token) return SV_ERR_NULL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || B > kMaxI32 || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > kMaxI32) return SV_ERR_SHAPE;
  if (t_seq < 1 || t_row < 1) return SV_ERR_SHAPE;
  if (bonus != 0 && bonus != 1) return SV_ERR_ARG;
  if (!std::isfinite(temperature) || !(temperature > 0.f)) return SV_ERR_TEMP;
  // the largest element offset must fit in int64 (and the per-sequence work in the grid)
  const double last = double(B - 1) * double(t_seq) + double(gamma + bonus - 1) * double(t_row) + double(V);
  if (last > 9.0e18) return SV_ERR_SHAPE;
  const size_t es = dtype == SV_BF16 ? 2 : 4;
  if (!aligned(tgt, es)) return SV_ERR_ALIGN;
  if (!aligned(ids, 4) || !aligned(ua, 4) || !aligned(us, 4) || !aligned(n_acc, 4) || !aligned(token, 4) ||
      (start && !aligned(start, 4)) || (order && !aligned(order, 4)) || (p_draft && !aligned(p_draft, 4)) ||
      (flags && !aligned(flags, 4)))
    return SV_ERR_ALIGN;
  (void)accept;
  return SV_OK;
}

// Grids of the plan must fit the launch limits.
// The work queue (one workgroup per item) must fit a one-dimensional grid of int32 indices.
int check_grid(const sv::DensePlan& p) {
  if (double(p.B) * (double(p.n1) + 1.0) + double(p.nslots) > double(kMaxI32)) return SV_ERR_SHAPE;
  return SV_OK;
}

int check_workspace(void* ws, size_t bytes, size_t need) {
  if (need == 0) return SV_OK;
  if (!ws) return SV_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return SV_ERR_ALIGN;
  if (bytes < need) return SV_ERR_WORKSPACE;
  return SV_OK;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int kind, int64_t B, int32_t gamma, int64_t V_or_k) {
  const size_t bad = static_cast<size_t>(-1);
  if (B < 1 || B > kMaxI32 || gamma < 1 || gamma > SV_MAX_GAMMA || V_or_k < 1) return bad;
  switch (kind) {
    case SV_KIND_DENSE:
    case SV_KIND_ONEHOT:
      if (V_or_k > kMaxI32) return bad;
      return sv::make_dense_plan(B, gamma, V_or_k, kind == SV_KIND_DENSE ? 2 : 1, SV_F32, 1).total;
    case SV_KIND_SPARSE:
      if (V_or_k > SV_MAX_K) return bad;
      return 0;
    case SV_KIND_GREEDY:
      if (V_or_k > kMaxI32) return bad;
      return sv::greedy_workspace_bytes(B, gamma, V_or_k);
    case SV_KIND_TREE:
      if (V_or_k > kMaxI32 || gamma > SV_MAX_TREE_NODES) return bad;
      return sv::make_tree_plan(B, gamma, V_or_k, SV_F32, 1).total;
    default:
      return bad;
  }
}

const char* sv_status_string(int status) {
  switch (status) {
    case SV_OK: return "ok";
    case SV_ERR_NULL: return "a required pointer is NULL";
    case SV_ERR_SHAPE: return "shape or stride out of range";
    case SV_ERR_DTYPE: return "unsupported dtype";
    case SV_ERR_TEMP: return "temperature must be finite and > 0";
    case SV_ERR_ALIGN: return "misaligned pointer";
    case SV_ERR_WORKSPACE: return "workspace missing or too small";
    case SV_ERR_HIP: return "HIP launch failed";
    case SV_ERR_ARG: return "invalid argument";
    case SV_ERR_SCRATCH: return "the call needs more scratch than the no-allocation entry point holds";
    default: return "unknown status";
  }
}

int sv_verify_dense(const void* target_logits, int64_t t_seq, int64_t t_row,
                    const void* draft_logits, int64_t d_seq, int64_t d_row,
                    int dtype, int64_t B, int32_t gamma, int64_t V,
                    const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                    float temperature, int32_t bonus,
                    int32_t* start, const int32_t* order,
                    uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                    float* p_draft, float* q_draft, uint32_t* flags,
                    void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense_common(target_logits, t_seq, t_row, dtype, B, gamma, V, draft_ids, u_accept, u_sample,
                              temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, flags);
  if (st != SV_OK) return st;
  if (!draft_logits) return SV_ERR_NULL;
  if (d_seq < 1 || d_row < 1) return SV_ERR_SHAPE;
  if (double(B - 1) * double(d_seq) + double(gamma - 1) * double(d_row) + double(V) > 9.0e18) return SV_ERR_SHAPE;
  if (!aligned(draft_logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  if (q_draft && !aligned(q_draft, 4)) return SV_ERR_ALIGN;
  const sv::DensePlan plan = sv::make_dense_plan(B, gamma, V, 2, dtype, sv::resident_workgroups());
  st = check_grid(plan);
  if (st != SV_OK) return st;
  st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;

  sv::DenseArgs a{target_logits, t_seq, t_row, draft_logits, d_seq, d_row, dtype, draft_ids, u_accept, u_sample,
                  temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, q_draft, flags,
                  static_cast<char*>(workspace)};
  return sv::launch_dense(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_verify_dense_noalloc(const void* target_logits, int64_t t_seq, int64_t t_row,
                            const void* draft_logits, int64_t d_seq, int64_t d_row,
                            int dtype, int64_t B, int32_t gamma, int64_t V,
                            const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                            float temperature, int32_t bonus,
                            int32_t* start, const int32_t* order,
                            uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                            float* p_draft, float* q_draft, uint32_t* flags, void* stream) {
  int st = check_dense_common(target_logits, t_seq, t_row, dtype, B, gamma, V, draft_ids, u_accept, u_sample,
                              temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, flags);
  if (st != SV_OK) return st;
  if (!draft_logits) return SV_ERR_NULL;
  if (d_seq < 1 || d_row < 1) return SV_ERR_SHAPE;
  if (double(B - 1) * double(d_seq) + double(gamma - 1) * double(d_row) + double(V) > 9.0e18) return SV_ERR_SHAPE;
  if (!aligned(draft_logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  if (q_draft && !aligned(q_draft, 4)) return SV_ERR_ALIGN;
  // the scratch must hold the largest plan of this shape (the float32 one), whatever the dtype of this call
  if (sv::make_dense_plan(B, gamma, V, 2, SV_F32, 1).total > size_t(SV_NOALLOC_SCRATCH_BYTES)) return SV_ERR_SCRATCH;
  const sv::DensePlan plan = sv::make_dense_plan(B, gamma, V, 2, dtype, sv::resident_workgroups());
  st = check_grid(plan);
  if (st != SV_OK) return st;
  char* ws = nullptr;
  if (sv::noalloc_scratch(&ws) != hipSuccess) return SV_ERR_HIP;
  sv::DenseArgs a{target_logits, t_seq, t_row, draft_logits, d_seq, d_row, dtype, draft_ids, u_accept, u_sample,
                  temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, q_draft, flags, ws};
  return sv::launch_dense(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_verify_onehot_draft(const void* target_logits, int64_t t_seq, int64_t t_row,
                           int dtype, int64_t B, int32_t gamma, int64_t V,
                           const int32_t* draft_ids, const float* u_accept, const float* u_sample,
                           float temperature, int32_t bonus,
                           int32_t* start, const int32_t* order,
                           uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                           float* p_draft, uint32_t* flags,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dense_common(target_logits, t_seq, t_row, dtype, B, gamma, V, draft_ids, u_accept, u_sample,
                              temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, flags);
  if (st != SV_OK) return st;
  const sv::DensePlan plan = sv::make_dense_plan(B, gamma, V, 1, dtype, sv::resident_workgroups());
  st = check_grid(plan);
  if (st != SV_OK) return st;
  st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;
  sv::DenseArgs a{target_logits, t_seq, t_row, nullptr, 0, 0, dtype, draft_ids, u_accept, u_sample,
                  temperature, bonus, start, order, accept, n_accepted, out_token, p_draft, nullptr, flags,
                  static_cast<char*>(workspace)};
  return sv::launch_dense(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_verify_sparse(const int32_t* p_ids, const float* p_probs,
                     const int32_t* q_ids, const float* q_probs,
                     int64_t B, int32_t gamma, int32_t kp, int32_t kq, int64_t vocab_size,
                     const int32_t* spec_ids, const float* u_accept, const float* u_sample, int32_t bonus,
                     uint8_t* accept, int32_t* n_accepted, int32_t* out_token,
                     float* correction_probs, float* p_spec, float* q_spec, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!p_ids || !p_probs || !q_ids || !q_probs || !spec_ids || !u_accept || !u_sample || !n_accepted || !out_token)
    return SV_ERR_NULL;
  if (B < 1 || B > kMaxI32 || gamma < 1 || gamma > SV_MAX_GAMMA || kp < 1 || kp > SV_MAX_K || kq < 1 ||
      kq > SV_MAX_K || vocab_size < 0 || vocab_size > kMaxI32)
    return SV_ERR_SHAPE;
  if (bonus != 0 && bonus != 1) return SV_ERR_ARG;
  if (double(B) * double(gamma + 1) * double(kp > kq ? kp : kq) > 9.0e18) return SV_ERR_SHAPE;
  const void* ptrs[] = {p_ids, p_probs, q_ids, q_probs, spec_ids, u_accept, u_sample, n_accepted, out_token,
                        correction_probs, p_spec, q_spec, flags};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SV_ERR_ALIGN;
  sv::SparseArgs a{p_ids, p_probs, q_ids, q_probs, B, gamma, kp, kq, vocab_size, spec_ids, u_accept, u_sample, bonus,
                   accept, n_accepted, out_token, correction_probs, p_spec, q_spec, flags};
  return sv::launch_sparse(a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

size_t sv_support_workspace_bytes(int64_t rows, int64_t V, int32_t k) {
  if (rows < 1 || rows > kMaxI32 || V < 1 || V > kMaxI32 || k < 1 || k > SV_MAX_K || k > V)
    return static_cast<size_t>(-1);
  return sv::make_support_plan(rows, V, k, SV_F32, 1).total;
}

namespace {

// Checks one row set of a support build; SV_OK or the status to return.
int check_support_rows(const void* logits, int64_t ld, int64_t rows, int dtype, int64_t V, const int32_t* ids,
                       const float* probs, const int32_t* count, const uint32_t* flags) {
  if (!logits || !ids || !probs) return SV_ERR_NULL;
  if (rows < 1 || rows > kMaxI32 || ld < V) return SV_ERR_SHAPE;
  if (double(rows - 1) * double(ld) + double(V) > 9.0e18) return SV_ERR_SHAPE;
  if (!aligned(logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  const void* ptrs[] = {ids, probs, count, flags};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SV_ERR_ALIGN;
  return SV_OK;
}

// The shared part of sv_build_support and sv_build_support_pair: settings, plan, workspace, launch.
int build_support(const sv::SupportRows& a, const sv::SupportRows& b, int dtype, int64_t V, float temperature,
                  int32_t k, float top_p, int32_t renorm, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (V < 1 || V > kMaxI32 || k < 1 || k > SV_MAX_K || k > V) return SV_ERR_SHAPE;
  int st = check_support_rows(a.logits, a.ld, a.rows, dtype, V, a.ids, a.probs, a.count, a.flags);
  if (st != SV_OK) return st;
  if (b.rows != 0) {
    st = check_support_rows(b.logits, b.ld, b.rows, dtype, V, b.ids, b.probs, b.count, b.flags);
    if (st != SV_OK) return st;
  }
  const int64_t rows = a.rows + b.rows;
  if (rows > kMaxI32) return SV_ERR_SHAPE;
  if (!std::isfinite(temperature) || !(temperature > 0.f)) return SV_ERR_TEMP;
  if (!(top_p > 0.f && top_p <= 1.f)) return SV_ERR_ARG;
  if (renorm != 0 && renorm != 1) return SV_ERR_ARG;
  const sv::SupportPlan plan = sv::make_support_plan(rows, V, k, dtype, sv::resident_workgroups());
  if (double(plan.items) > double(kMaxI32)) return SV_ERR_SHAPE;
  st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;
  sv::SupportArgs args{{a, b}, dtype, temperature, top_p, renorm, static_cast<char*>(workspace)};
  return sv::launch_support(plan, args, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // namespace

int sv_build_support(const void* logits, int64_t ld, int dtype, int64_t rows, int64_t V,
                     float temperature, int32_t k, float top_p, int32_t renorm,
                     int32_t* ids, float* probs, int32_t* count, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const sv::SupportRows a{logits, ld, rows, ids, probs, count, flags};
  const sv::SupportRows none{nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr};
  return build_support(a, none, dtype, V, temperature, k, top_p, renorm, workspace, workspace_bytes, stream);
}

int sv_build_support_pair(const void* logits_a, int64_t ld_a, int64_t rows_a,
                          const void* logits_b, int64_t ld_b, int64_t rows_b,
                          int dtype, int64_t V, float temperature, int32_t k, float top_p, int32_t renorm,
                          int32_t* ids_a, float* probs_a, int32_t* count_a, uint32_t* flags_a,
                          int32_t* ids_b, float* probs_b, int32_t* count_b, uint32_t* flags_b,
                          void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits_b || !ids_b || !probs_b) return SV_ERR_NULL;
  if (rows_b < 1) return SV_ERR_SHAPE;
  const sv::SupportRows a{logits_a, ld_a, rows_a, ids_a, probs_a, count_a, flags_a};
  const sv::SupportRows b{logits_b, ld_b, rows_b, ids_b, probs_b, count_b, flags_b};
  return build_support(a, b, dtype, V, temperature, k, top_p, renorm, workspace, workspace_bytes, stream);
}

int sv_verify_greedy(const void* target_logits, int64_t t_seq, int64_t t_row,
                     int dtype, int64_t B, int32_t gamma, int64_t V,
                     const int32_t* draft_ids, int32_t bonus,
                     int32_t* start, const int32_t* order,
                     uint8_t* accept, int32_t* n_accepted, int32_t* out_token, uint32_t* flags,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (!target_logits || !draft_ids || !n_accepted || !out_token) return SV_ERR_NULL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || B > kMaxI32 || gamma < 1 || gamma > SV_MAX_GAMMA || V < 1 || V > kMaxI32) return SV_ERR_SHAPE;
  if (t_seq < 1 || t_row < 1) return SV_ERR_SHAPE;
  if (bonus != 0 && bonus != 1) return SV_ERR_ARG;
  if (double(B - 1) * double(t_seq) + double(gamma + bonus - 1) * double(t_row) + double(V) > 9.0e18)
    return SV_ERR_SHAPE;
  if (!aligned(target_logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  const void* ptrs[] = {draft_ids, start, order, n_accepted, out_token, flags};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SV_ERR_ALIGN;
  const sv::GreedyPlan plan = sv::make_greedy_plan(B, gamma, V, bonus, dtype);
  if (double(plan.items) > double(kMaxI32)) return SV_ERR_SHAPE;
  const int st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;
  sv::GreedyArgs a{target_logits, t_seq, t_row, dtype, bonus, draft_ids, start, order, accept, n_accepted, out_token,
                   flags, static_cast<char*>(workspace)};
  return sv::launch_greedy(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_confidence_commit(const void* logits, int64_t l_seq, int64_t l_row, int dtype, int64_t B, int32_t W,
                         int64_t V, const uint8_t* masked, float tau, uint8_t* commit, int32_t* token,
                         float* confidence, int32_t* n_commit, uint32_t* flags,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (!logits || !token || !n_commit) return SV_ERR_NULL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || B > kMaxI32 || W < 1 || W > SV_MAX_GAMMA || V < 1 || V > kMaxI32) return SV_ERR_SHAPE;
  if (l_seq < 1 || l_row < 1) return SV_ERR_SHAPE;
  if (double(B - 1) * double(l_seq) + double(W - 1) * double(l_row) + double(V) > 9.0e18) return SV_ERR_SHAPE;
  if (!(tau >= 0.f && tau <= 1.f)) return SV_ERR_ARG;
  if (!aligned(logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  const void* ptrs[] = {token, confidence, n_commit, flags};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SV_ERR_ALIGN;
  const sv::GreedyPlan plan = sv::make_greedy_plan(B, W, V, 0, dtype);
  if (double(plan.items) > double(kMaxI32)) return SV_ERR_SHAPE;
  const int st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;
  sv::GreedyArgs a{logits, l_seq, l_row, dtype, 0, nullptr, nullptr, nullptr, nullptr, n_commit, token, flags,
                   static_cast<char*>(workspace)};
  a.conf_mode = true;
  a.masked = masked;
  a.tau = tau;
  a.commit = commit;
  a.conf = confidence;
  return sv::launch_greedy(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

int sv_verify_tree(const void* target_logits, int64_t t_seq, int64_t t_row, int dtype, int64_t B, int32_t N,
                   int64_t V, const int32_t* parent, const int32_t* token, const float* u_accept,
                   const float* u_sample, float temperature, uint8_t* accept, int32_t* n_accepted, int32_t* path,
                   int32_t* out_token, float* p_test, uint32_t* flags, void* workspace, size_t workspace_bytes,
                   void* stream) {
  if (!target_logits || !parent || !token || !u_accept || !u_sample || !accept || !n_accepted || !path || !out_token)
    return SV_ERR_NULL;
  if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
  if (B < 1 || B > kMaxI32 || N < 1 || N > SV_MAX_TREE_NODES || V < 1 || V > kMaxI32) return SV_ERR_SHAPE;
  if (t_seq < 1 || t_row < 1) return SV_ERR_SHAPE;
  if (double(B - 1) * double(t_seq) + double(N - 1) * double(t_row) + double(V) > 9.0e18) return SV_ERR_SHAPE;
  if (double(B) * double(N) > double(kMaxI32)) return SV_ERR_SHAPE;
  if (!std::isfinite(temperature) || !(temperature > 0.f)) return SV_ERR_TEMP;
  if (!aligned(target_logits, dtype == SV_BF16 ? 2 : 4)) return SV_ERR_ALIGN;
  const void* ptrs[] = {parent, token, u_accept, u_sample, n_accepted, path, out_token, p_test, flags};
  for (const void* p : ptrs)
    if (p && !aligned(p, 4)) return SV_ERR_ALIGN;
  const sv::TreePlan plan = sv::make_tree_plan(B, N, V, dtype, sv::tree_resident_workgroups(dtype));
  if (double(plan.items) + double(plan.tasks) > double(kMaxI32)) return SV_ERR_SHAPE;
  const int st = check_workspace(workspace, workspace_bytes, plan.total);
  if (st != SV_OK) return st;
  sv::TreeArgs a{target_logits, t_seq, t_row, dtype, parent, token, u_accept, u_sample, temperature, accept,
                 n_accepted, path, out_token, p_test, flags, static_cast<char*>(workspace)};
  return sv::launch_tree(plan, a, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_ERR_HIP;
}

}  // extern "C"
