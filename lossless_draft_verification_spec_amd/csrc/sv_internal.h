// Internal declarations shared by the host entry points and the kernel launchers of the verifier library.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

namespace sv {

// Kinds of draw a sequence needs after the accept/first-reject scan.
enum JobKind : int32_t {
  JOB_NONE = 0,      // nothing to draw (finished, fatal, or no bonus)
  JOB_RESID = 1,     // residual max(p - q, 0) at a rejected row, q from draft logits
  JOB_ONEHOT = 2,    // residual p with the draft id removed (q one-hot)
  JOB_BONUS = 3,     // bonus draw from p of target row gamma
};

// What the scan of one sequence decides, published to the sequence's draw tasks. 64 bytes: four 16-byte groups, each
// ending in a seal word (1 once the scan has written the job, 0 again at the end of the call).
struct alignas(16) Job {
  int32_t kind;      // JobKind
  int32_t row;       // storage row of the draw (gamma for the bonus)
  int32_t d;         // draft id at that row (one-hot residual)
  uint32_t seal0;
  float u;           // the uniform of the draw
  float m_t;         // exact max of the target row (from the statistics pass; unused for the bonus)
  float m_d;         // exact max of the draft row
  uint32_t seal1;
  double kappa;      // S_d / S_t of the row pair as estimated by the statistics pass (float32 sums)
  int32_t new_start; // start for the next call (-1: leave unchanged)
  uint32_t seal2;
  uint32_t flags;    // the sequence's SV_FLAG_* bits from the scan
  uint32_t pad0, pad1;
  uint32_t seal3;
};
constexpr int kJobStride = 64;     // bytes per job in the workspace (one cache line each)
static_assert(sizeof(Job) == kJobStride && offsetof(Job, seal0) == 12 && offsetof(Job, seal1) == 28 &&
              offsetof(Job, seal2) == 44 && offsetof(Job, seal3) == 60, "job layout");

// Sizes, work queue and workspace layout of one dense / one-hot call. Depends only on (B, gamma, V, number of
// tensors, dtype); the float32 plan is the larger, so it sizes the workspace for both dtypes.
struct DensePlan {
  int64_t B = 0;
  int32_t G = 0;
  int64_t V = 0;
  int32_t ntens = 0;     // 2: target + draft; 1: target only (one-hot)
  int32_t nseg1 = 1;     // statistics items (segments) per row
  int64_t n1 = 1;        // statistics items per sequence: ntens * G * nseg1
  int32_t ntask = 1;     // draw tasks per sequence (all but the last tailq sequences)
  int32_t ntask2 = 1;    // draw tasks of each of the last tailq sequences (smaller tasks)
  int32_t chunks1 = 16;  // chunks per draw task of the other sequences
  int64_t tailq = 1;     // sequences with the smaller draw tasks
  int64_t ntot = 1;      // draw tasks in all
  int64_t nch = 1;       // 512-element chunks per row in the draw
  int64_t nslots = 1;    // draw slots of the work queue (at least B * ntask)
  size_t off_ready = 0;  // int32 per b (one per 256 bytes): statistics items finished, + 1 once the job is published
  size_t off_done = 0;   // int32 per b (one per 256 bytes): draw tasks finished
  size_t off_tickets = 0; // int32: draw slots started in this call
  size_t off_jobs = 0;   // Job per b, kJobStride bytes apart
  size_t off_part1 = 0;  // (max, logit at the id, float64 sum) per (tensor, b, row, segment)
  size_t off_part2 = 0;  // double4 (m_task, S_t, m_d, S_d) per (b, task)
  size_t off_recA = 0;   // double per (b, chunk): the chunk's A (see the draw's chunk records)
  size_t off_recD = 0;   // double per (b, chunk): the chunk's D
  size_t off_recN = 0;   // int32 per (b, chunk): the chunk's undecided elements
  size_t off_recU = 0;   // 4 (e_t, e_d) pairs per (b, chunk): the undecided elements themselves
  size_t off_masses = 0; // double per (b, chunk)
  size_t total = 0;
};

// resident: workgroups resident on the device at once (it sets the draw task sizes; the workspace size does not
// depend on it).
DensePlan make_dense_plan(int64_t B, int32_t G, int64_t V, int32_t ntens, int dtype, int64_t resident);
int resident_workgroups();

// Kinds of control layout kept in a workspace (see sv_wshdr.h): the workspace header names one of them, with the
// size that places its control words.
constexpr uint64_t kLayoutDense = 0xcbf29ce484222325ull;     // FNV-1a offset basis, one per kind of layout
constexpr uint64_t kLayoutSupport = 0x84222325cbf29ce4ull;
inline uint64_t layout_mix(uint64_t sig, uint64_t v) { return (sig ^ v) * 1099511628211ull; }

struct DenseArgs {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;     // dft == nullptr: one-hot drafts
  int dtype;
  const int32_t* ids; const float* ua; const float* us;
  float temperature; int32_t bonus;
  int32_t* start; const int32_t* order;
  uint8_t* accept; int32_t* n_acc; int32_t* token;
  float* p_draft; float* q_draft; uint32_t* flags;
  char* ws;
};

hipError_t launch_dense(const DensePlan& plan, const DenseArgs& a, hipStream_t stream);
// Device address of the current device's no-allocation scratch (SV_NOALLOC_SCRATCH_BYTES), looked up once per device.
hipError_t noalloc_scratch(char** out);

struct SparseArgs {
  const int32_t* p_ids; const float* p_probs;
  const int32_t* q_ids; const float* q_probs;
  int64_t B; int32_t G; int32_t kp; int32_t kq; int64_t vocab;
  const int32_t* spec; const float* ua; const float* us; int32_t bonus;
  uint8_t* accept; int32_t* n_acc; int32_t* token;
  float* corr; float* p_spec; float* q_spec; uint32_t* flags;
};

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream);

// Top-k / top-p support builder (sv_support.hip): sizes and workspace layout of one call.
struct SupportPlan {
  int64_t rows = 0;
  int64_t V = 0;
  int32_t k = 0;
  int64_t head_rows = 0;   // rows taken whole, one workgroup each (full resident rounds)
  int32_t nseg = 1;        // segments of each later row
  int32_t nlay = 1;        // segment records per row in the workspace
  int64_t items = 0;       // workgroups of the launch
  size_t off_ctr = 0;      // int32 per row (one per 256 bytes): segments finished, returned to 0 by the row's merge
  size_t ctr_bytes = 0;    // header + control region [0, ctr_bytes)
  size_t off_keys = 0;     // per (row, segment): up to k uint64 keys
  size_t off_part = 0;     // per (row, segment): the segment's statistics
  size_t total = 0;
};

// resident: workgroups resident on the device at once (it sets which rows are cut into segments; the workspace size
// depends on neither it nor the dtype).
SupportPlan make_support_plan(int64_t rows, int64_t V, int32_t k, int dtype, int64_t resident);

// One set of logit rows and its outputs. A launch takes two sets; the rows of the second follow those of the first
// (rows = 0 for a launch of one set).
struct SupportRows {
  const void* logits; int64_t ld; int64_t rows;
  int32_t* ids; float* probs; int32_t* count; uint32_t* flags;
};

struct SupportArgs {
  SupportRows set[2];
  int dtype;
  float temperature; float top_p; int32_t renorm;
  char* ws;
};

hipError_t launch_support(const SupportPlan& plan, const SupportArgs& a, hipStream_t stream);

// Tree verification (sv_tree.hip): per-row statistics outside the node's child tokens, the draw job of a sequence,
// the sizes and workspace layout of one call.
constexpr uint64_t kLayoutTree = 0x62325cbf29ce4842ull;

struct alignas(16) TreeRow {
  float m;          // max of the row's logits outside its node's child tokens (-inf when there are none)
  uint32_t bad;     // 1: a NaN or +inf among them
  double s;         // sum over them of 2^((z - m) * c), c = log2(e)/T rounded to float
};

struct alignas(16) TreeJob {
  int32_t stop;     // node where the walk stopped (-1: nothing to draw)
  float m;          // max of the stop node's whole row
  float u;          // the draw's uniform
  uint32_t flags;   // the sequence's flags from the walk
  int32_t n;        // accepted nodes (-1: a failed sequence)
};

struct TreePlan {
  int64_t B = 0;
  int32_t N = 0;
  int64_t V = 0;
  int64_t head_rows = 0;    // rows taken whole by the row items (rows b * N + u below it)
  int32_t nseg = 1;         // pieces of every later row (1: those rows are whole too)
  int64_t items = 0;        // row items (workgroups before the draw tasks in the launch)
  int64_t nch = 0;          // 512-element chunks per row in the draw
  int32_t ntask = 1;        // draw tasks per sequence (all but the last tailq sequences)
  int32_t task_chunks = 16; // chunks per draw task
  int32_t tailq = 0;        // the last sequences, whose rows finish last: smaller draw tasks
  int32_t ntask2 = 1;       // draw tasks of each of them
  int32_t task_chunks2 = 8; // chunks per such task
  int64_t tasks = 0;        // draw tasks of the launch
  size_t off_ctr1 = 0;      // int32 per sequence: rows finished, N + 1 once the walk published the job; back to 0
                            // after the pick
  size_t off_ctr2 = 0;      // int32 per sequence: draw tasks finished, back to 0 after the pick
  size_t off_rctr = 0;      // int32 per cut row: pieces finished, back to 0 after the row's merge
  size_t ctl_end = 0;       // the control region is [header end, ctl_end)
  size_t off_rows = 0;      // TreeRow per (b, node)
  size_t off_piece = 0;     // TreeRow per (cut row, piece)
  size_t off_jobs = 0;      // TreeJob per b
  size_t off_chunk = 0;     // double per (b, chunk)
  size_t total = 0;
};

// Row item `item` of the tree launch: row r = b * N + u and piece seg of it. The whole rows come first (r = item
// below head_rows), then the pieces of the later rows, the nseg pieces of one row together.
__host__ __device__ inline void tree_item(int64_t item, int64_t head_rows, int32_t nseg, int64_t* r, int32_t* seg) {
  if (item < head_rows || nseg <= 1) {
    *r = item;
    *seg = 0;
  } else {
    const int64_t j = item - head_rows;
    *r = head_rows + j / nseg;
    *seg = int32_t(j % nseg);
  }
}

// Draw task j of the tree launch: sequence b, its task t of nt, chunks [c0, c1). The first B - tailq sequences have
// ntask tasks of task_chunks chunks, the last tailq have ntask2 of task_chunks2, in sequence order.
struct TreeTask {
  int64_t b;
  int32_t t, nt;
  int64_t c0, c1;
};
__host__ __device__ inline TreeTask tree_task(int64_t j, int64_t B, int32_t tailq, int32_t ntask, int32_t ntask2,
                                              int32_t task_chunks, int32_t task_chunks2, int64_t nch) {
  const int64_t head = (B - tailq) * int64_t(ntask);
  TreeTask k;
  int64_t per;
  if (j < head) {
    k.b = j / ntask;
    k.t = int32_t(j % ntask);
    k.nt = ntask;
    per = task_chunks;
  } else {
    const int64_t j2 = j - head;
    k.b = B - tailq + j2 / ntask2;
    k.t = int32_t(j2 % ntask2);
    k.nt = ntask2;
    per = task_chunks2;
  }
  k.c0 = int64_t(k.t) * per;
  k.c1 = k.c0 + per < nch ? k.c0 + per : nch;
  return k;
}

// resident: workgroups of the tree launch resident on the device at once (it sets which rows are cut into pieces;
// the workspace size depends on neither it nor the dtype).
TreePlan make_tree_plan(int64_t B, int32_t N, int64_t V, int dtype, int64_t resident);
int tree_resident_workgroups(int dtype);

struct TreeArgs {
  const void* tgt; int64_t t_seq, t_row; int dtype;
  const int32_t* parent; const int32_t* token; const float* ua; const float* us;
  float temperature;
  uint8_t* accept; int32_t* n_acc; int32_t* path; int32_t* out_token; float* p_test; uint32_t* flags;
  char* ws;
};

hipError_t launch_tree(const TreePlan& plan, const TreeArgs& a, hipStream_t stream);

}  // namespace sv
