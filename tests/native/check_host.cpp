// Host-side checks of the verifier library, built with AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_host_sanitized.py builds and runs it; no GPU is needed and no call here reaches a HIP call):
//  1. the check applied to a draw job read back from the workspace (job_valid), on random and garbage words: every
//     job it accepts names only rows and ids inside the call's tensors;
//  2. the count check of the support builder's segment records (clamp_count), and the item map, piece sizes and
//     workspace regions of the tree's first launch over many shapes and residencies;
//  3. every entry point with arguments it must reject on the host (NULLs, shapes, dtypes, strides, alignment,
//     temperatures, workspace sizes), and workspace sizing over extreme shapes, so that the sanitizers see the size
//     arithmetic of every plan.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <vector>

#include "sv.h"
#include "sv_internal.h"
#include "sv_wshdr.h"

static int g_fail = 0;
#define CHECK(c)                                                               \
  do {                                                                         \
    if (!(c)) {                                                                \
      std::fprintf(stderr, "FAILED %s:%d: %s\n", __FILE__, __LINE__, #c);      \
      ++g_fail;                                                                \
    }                                                                          \
  } while (0)

using sv::Job;

// What a job that passes the check may do: every address or index it forms stays inside the call's tensors.
static bool job_is_safe(const Job& j, int32_t G, int64_t V, int32_t bonus, bool dense) {
  if (j.new_start < -1 || j.new_start > G) return false;
  switch (j.kind) {
    case sv::JOB_NONE: return true;
    case sv::JOB_RESID: return dense && 0 <= j.row && j.row < G;
    case sv::JOB_ONEHOT: return !dense && 0 <= j.row && j.row < G && 0 <= j.d && j.d < V;
    case sv::JOB_BONUS: return bonus == 1 && j.row == G;
    default: return false;
  }
}

static void check_jobs() {
  std::mt19937_64 rng(12345);
  const int32_t Gs[] = {1, 4, 16, 1024};
  const int64_t Vs[] = {1, 9, 151936, 2147483647};
  int64_t accepted = 0;
  for (int it = 0; it < 400000; ++it) {
    Job j;
    uint32_t w[16];
    for (uint32_t& x : w) x = uint32_t(rng());
    // half the jobs: garbage words as they might sit in a stale workspace; the other half: near-valid jobs with one
    // field pushed to or past its bounds
    if (it & 1) {
      const int32_t G = Gs[rng() % 4];
      const int64_t V = Vs[rng() % 4];
      w[0] = uint32_t(rng() % 6) - 1u;                    // kind in [-1, 4]
      w[1] = uint32_t(int32_t(rng() % (G + 3)) - 1);      // row in [-1, G + 1]
      w[2] = uint32_t(int64_t(rng() % 5) - 2 + (rng() & 1 ? V : 0));   // d near 0 or near V
      w[10] = uint32_t(int32_t(rng() % (G + 4)) - 2);     // new_start in [-2, G + 1]
    }
    std::memcpy(&j, w, sizeof(j));
    for (int32_t G : Gs)
      for (int64_t V : Vs)
        for (int32_t bonus = 0; bonus < 2; ++bonus)
          for (int dense = 0; dense < 2; ++dense) {
            const bool ok = sv::job_valid(j, G, V, bonus, dense != 0);
            CHECK(ok == job_is_safe(j, G, V, bonus, dense != 0));
            accepted += ok;
          }
  }
  CHECK(accepted > 0);
  // what the scan publishes is accepted
  Job r{};
  r.kind = sv::JOB_RESID; r.row = 15; r.new_start = 16;
  CHECK(sv::job_valid(r, 16, 151936, 1, true));
  CHECK(!sv::job_valid(r, 16, 151936, 1, false));       // a residual draw only exists with draft logits
  Job o{};
  o.kind = sv::JOB_ONEHOT; o.row = 0; o.d = 128255; o.new_start = 1;
  CHECK(sv::job_valid(o, 8, 128256, 1, false));
  o.d = 128256;
  CHECK(!sv::job_valid(o, 8, 128256, 1, false));
  Job b{};
  b.kind = sv::JOB_BONUS; b.row = 16; b.new_start = 16;
  CHECK(sv::job_valid(b, 16, 151936, 1, true));
  CHECK(!sv::job_valid(b, 16, 151936, 0, true));        // no bonus row without a bonus
  Job n{};
  n.kind = sv::JOB_NONE; n.new_start = -1;
  CHECK(sv::job_valid(n, 1, 1, 0, true));
}

static void check_counts() {
  for (int32_t k = 1; k <= SV_MAX_K; ++k)
    for (int32_t n : {std::numeric_limits<int32_t>::min(), -1, 0, 1, k - 1, k, k + 1,
                      std::numeric_limits<int32_t>::max()}) {
      const int32_t c = sv::clamp_count(n, k);
      CHECK(c >= 0 && c <= k);
      if (n >= 0 && n <= k) CHECK(c == n);
    }
}

static void check_signatures() {
  // distinct kinds and sizes give distinct, nonzero signatures
  const uint64_t kinds[] = {sv::kLayoutDense, sv::kLayoutSupport};
  for (uint64_t kind : kinds)
    for (uint64_t n = 0; n < 5000; ++n) {
      CHECK(sv::ws_signature(kind, n) != 0);
      CHECK(sv::ws_signature(kind, n) != sv::ws_signature(kind, n + 1));
    }
  CHECK(sv::ws_signature(sv::kLayoutDense, 64) != sv::ws_signature(sv::kLayoutSupport, 64));
}

// The tree's first launch over many shapes and residencies: its items cover every piece of every row exactly once,
// in order, the piece and row-counter indexes stay inside their workspace regions, every piece of a cut row holds at
// least 512 vectors at any alignment, and the workspace size depends on neither the dtype nor the residency.
static void check_tree_plans() {
  int64_t cut_plans = 0;
  for (int64_t B : {int64_t(1), int64_t(3), int64_t(64), int64_t(100), int64_t(1000)})
    for (int32_t N : {1, 2, 17, 64, 200})
      for (int64_t V : {int64_t(1), int64_t(9), int64_t(4099), int64_t(50000), int64_t(151936), int64_t(2147483647)}) {
        const size_t total = sv::make_tree_plan(B, N, V, SV_F32, 1).total;
        for (int dt : {SV_F32, SV_BF16})
          for (int64_t W : {int64_t(1), int64_t(7), int64_t(1024), int64_t(2048), int64_t(100000)}) {
            const sv::TreePlan pl = sv::make_tree_plan(B, N, V, dt, W);
            CHECK(pl.total == total);
            const int64_t R = B * N;
            CHECK(pl.nseg >= 1 && pl.nseg <= 64 && pl.head_rows >= 0 && pl.head_rows <= R);
            if (pl.nseg == 1) CHECK(pl.head_rows == R && pl.items == R);
            const int64_t epv = dt == SV_BF16 ? 8 : 4;
            const int64_t nvec_min = (V - (epv - 1)) / epv;
            if (pl.nseg > 1) {
              ++cut_plans;
              CHECK(nvec_min / pl.nseg >= 512);
            }
            const size_t piece_cap = (pl.off_jobs - pl.off_piece) / sizeof(sv::TreeRow);
            const size_t rctr_cap = (pl.ctl_end - pl.off_rctr) / sizeof(int32_t);
            CHECK((pl.off_piece - pl.off_rows) / sizeof(sv::TreeRow) >= size_t(R));
            CHECK(pl.off_rctr >= pl.off_ctr2 + size_t(B) * 4 && pl.off_ctr2 >= pl.off_ctr1 + size_t(B) * 4);
            std::vector<int32_t> seen(size_t(R), 0);
            for (int64_t it = 0; it < pl.items; ++it) {
              int64_t r = -1;
              int32_t seg = -1;
              sv::tree_item(it, pl.head_rows, pl.nseg, &r, &seg);
              if (!(r >= 0 && r < R)) { CHECK(r >= 0 && r < R); break; }
              const int32_t nseg = it < pl.head_rows ? 1 : pl.nseg;
              CHECK(seg >= 0 && seg < nseg);
              CHECK(seg == seen[size_t(r)]);          // the pieces of a row come in order, each once
              ++seen[size_t(r)];
              if (nseg > 1) {
                CHECK(size_t((r - pl.head_rows) * nseg + seg) < piece_cap);
                CHECK(size_t(r - pl.head_rows) < rctr_cap);
              }
            }
            for (int64_t r = 0; r < R; ++r) CHECK(seen[size_t(r)] == (r < pl.head_rows ? 1 : pl.nseg));
            // draw tasks: every chunk of every sequence's row in exactly one task, the tasks of a sequence in order
            CHECK(pl.tailq >= 0 && pl.tailq <= B && pl.ntask >= 1 && pl.ntask2 >= 1);
            CHECK(pl.tasks == (B - pl.tailq) * int64_t(pl.ntask) + int64_t(pl.tailq) * pl.ntask2);
            if (pl.tasks <= 2000000) {
              int64_t prev_b = -1, next_c = 0;
              int32_t next_t = 0;
              for (int64_t j = 0; j < pl.tasks; ++j) {
                const sv::TreeTask k = sv::tree_task(j, B, pl.tailq, pl.ntask, pl.ntask2, pl.task_chunks,
                                                     pl.task_chunks2, pl.nch);
                if (k.b != prev_b) {
                  if (prev_b >= 0) CHECK(next_c == pl.nch);
                  CHECK(k.b == prev_b + 1);
                  prev_b = k.b;
                  next_c = 0;
                  next_t = 0;
                }
                CHECK(k.t == next_t && k.t < k.nt);
                CHECK(k.nt == (k.b < B - pl.tailq ? pl.ntask : pl.ntask2));
                CHECK(k.c0 == next_c && k.c1 > k.c0 && k.c1 <= pl.nch);
                next_c = k.c1;
                ++next_t;
              }
              CHECK(prev_b == B - 1 && next_c == pl.nch);
            }
          }
      }
  CHECK(cut_plans > 100);
}

static void check_entry_points() {
  // fake device pointers: never dereferenced, because every call below fails its host checks first
  alignas(256) static unsigned char buf[1 << 16];
  void* p = buf;
  const int32_t* ip = reinterpret_cast<const int32_t*>(buf);
  const float* fp = reinterpret_cast<const float*>(buf);
  int32_t* op = reinterpret_cast<int32_t*>(buf);
  uint8_t* u8 = buf;
  void* mis = buf + 1;
  const size_t big = size_t(1) << 40;
  const float nan = std::numeric_limits<float>::quiet_NaN();

  // dense
  CHECK(sv_verify_dense(nullptr, 1, 1, p, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_dense(p, 1, 1, nullptr, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, 7, 1, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op, nullptr,
                        nullptr, nullptr, p, big, nullptr) == SV_ERR_DTYPE);
  for (int64_t B : {int64_t(0), int64_t(-1), int64_t(1) << 31})
    CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, B, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                          nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_SHAPE);
  for (int32_t G : {0, -5, SV_MAX_GAMMA + 1})
    CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 1, G, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                          nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_verify_dense(p, 0, 1, p, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_verify_dense(p, int64_t(1) << 62, 1, p, 1, 1, SV_F32, 1000, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr,
                        nullptr, op, op, nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_SHAPE);
  for (float T : {0.f, -1.f, nan, std::numeric_limits<float>::infinity()})
    CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, T, 1, nullptr, nullptr, nullptr, op, op,
                          nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_TEMP);
  CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, 1.f, 2, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_ARG);
  CHECK(sv_verify_dense(mis, 1, 1, p, 1, 1, SV_F32, 1, 1, 1, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, big, nullptr) == SV_ERR_ALIGN);
  CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 4, 4, 1000, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, nullptr, 0, nullptr) == SV_ERR_WORKSPACE);
  CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 4, 4, 1000, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, p, 16, nullptr) == SV_ERR_WORKSPACE);
  CHECK(sv_verify_dense(p, 1, 1, p, 1, 1, SV_F32, 4, 4, 1000, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                        nullptr, nullptr, nullptr, buf + 16, big, nullptr) == SV_ERR_ALIGN);
  // one-hot
  CHECK(sv_verify_onehot_draft(p, 1, 1, SV_BF16, 1, 1, 1, nullptr, fp, fp, 1.f, 1, nullptr, nullptr, nullptr, op, op,
                               nullptr, nullptr, p, big, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_onehot_draft(p, 1, 1, SV_BF16, 1, 1, int64_t(1) << 31, ip, fp, fp, 1.f, 1, nullptr, nullptr, nullptr,
                               op, op, nullptr, nullptr, p, big, nullptr) == SV_ERR_SHAPE);
  // sparse
  CHECK(sv_verify_sparse(ip, fp, ip, fp, 1, 1, 0, 1, 0, ip, fp, fp, 1, nullptr, op, op, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_verify_sparse(ip, fp, ip, fp, 1, 1, SV_MAX_K + 1, 1, 0, ip, fp, fp, 1, nullptr, op, op, nullptr, nullptr,
                         nullptr, nullptr, nullptr, 0, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_verify_sparse(ip, fp, ip, fp, 1, 1, 4, 4, -1, ip, fp, fp, 1, nullptr, op, op, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0, nullptr) == SV_ERR_SHAPE);
  CHECK(sv_verify_sparse(nullptr, fp, ip, fp, 1, 1, 4, 4, 0, ip, fp, fp, 1, nullptr, op, op, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0, nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_sparse(ip, fp, ip, fp, 1, 1, 4, 4, 0, ip, fp, fp, 3, nullptr, op, op, nullptr, nullptr, nullptr,
                         nullptr, nullptr, 0, nullptr) == SV_ERR_ARG);
  CHECK(sv_verify_sparse(ip, fp, ip, fp, 1, 1, 4, 4, 0, ip, fp, fp, 1, nullptr, op, op,
                         reinterpret_cast<float*>(buf + 2), nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
        SV_ERR_ALIGN);
  // support builder
  CHECK(sv_build_support(p, 10, SV_F32, 1, 10, 1.f, 11, 0.9f, 1, op, reinterpret_cast<float*>(buf), nullptr, nullptr,
                         p, big, nullptr) == SV_ERR_SHAPE);                                           // k > V
  CHECK(sv_build_support(p, 9, SV_F32, 1, 10, 1.f, 4, 0.9f, 1, op, reinterpret_cast<float*>(buf), nullptr, nullptr,
                         p, big, nullptr) == SV_ERR_SHAPE);                                           // ld < V
  for (float tp : {0.f, -0.5f, 1.5f, nan})
    CHECK(sv_build_support(p, 10, SV_F32, 1, 10, 1.f, 4, tp, 1, op, reinterpret_cast<float*>(buf), nullptr, nullptr,
                           p, big, nullptr) == SV_ERR_ARG);
  CHECK(sv_build_support(p, 10, SV_F32, 1, 10, 1.f, 4, 0.9f, 2, op, reinterpret_cast<float*>(buf), nullptr, nullptr,
                         p, big, nullptr) == SV_ERR_ARG);
  CHECK(sv_build_support(p, 10, SV_F32, 3, 10, 1.f, 4, 0.9f, 1, op, reinterpret_cast<float*>(buf), nullptr, nullptr,
                         p, 8, nullptr) == SV_ERR_WORKSPACE);
  // greedy and commit
  CHECK(sv_verify_greedy(p, 1, 1, SV_F32, 1, 1, 1, nullptr, 1, nullptr, nullptr, nullptr, op, op, nullptr, p, big,
                         nullptr) == SV_ERR_NULL);
  CHECK(sv_verify_greedy(p, 1, 1, SV_F32, 1, 1, 1, ip, 5, nullptr, nullptr, nullptr, op, op, nullptr, p, big,
                         nullptr) == SV_ERR_ARG);
  CHECK(sv_verify_greedy(p, 1, 1, SV_F32, 2, 3, 100, ip, 1, nullptr, nullptr, nullptr, op, op, nullptr, p, 4,
                         nullptr) == SV_ERR_WORKSPACE);
  for (float tau : {-0.1f, 1.1f, nan})
    CHECK(sv_confidence_commit(p, 1, 1, SV_F32, 1, 1, 1, u8, tau, u8, op, nullptr, op, nullptr, p, big, nullptr) ==
          SV_ERR_ARG);
  CHECK(sv_confidence_commit(p, 1, 1, SV_F32, 1, SV_MAX_GAMMA + 1, 1, u8, 0.5f, u8, op, nullptr, op, nullptr, p, big,
                             nullptr) == SV_ERR_SHAPE);
  // status strings exist for every code
  for (int s = -9; s <= 0; ++s) CHECK(sv_status_string(s) != nullptr && std::strlen(sv_status_string(s)) > 0);

  // workspace sizes: defined for every accepted shape, (size_t)-1 for rejected ones, monotone in B
  const size_t bad = static_cast<size_t>(-1);
  for (int kind : {SV_KIND_DENSE, SV_KIND_ONEHOT, SV_KIND_GREEDY})
    for (int64_t V : {int64_t(1), int64_t(511), int64_t(512), int64_t(151936), int64_t(2147483647)})
      for (int32_t G : {1, 16, SV_MAX_GAMMA}) {
        size_t prev = 0;
        for (int64_t B : {int64_t(1), int64_t(64), int64_t(4096)}) {
          const size_t n = sv_workspace_bytes(kind, B, G, V);
          CHECK(n != bad && n >= prev && n % 256 == 0);
          prev = n;
        }
      }
  CHECK(sv_workspace_bytes(SV_KIND_DENSE, 0, 1, 1) == bad);
  CHECK(sv_workspace_bytes(SV_KIND_DENSE, 1, 1, int64_t(1) << 31) == bad);
  CHECK(sv_workspace_bytes(99, 1, 1, 1) == bad);
  CHECK(sv_workspace_bytes(SV_KIND_SPARSE, 1, 1, SV_MAX_K) == 0);
  CHECK(sv_support_workspace_bytes(1, 10, 11) == bad);
  for (int64_t rows : {int64_t(1), int64_t(1088), int64_t(100000)})
    for (int32_t k : {1, 50, SV_MAX_K}) CHECK(sv_support_workspace_bytes(rows, 151936, k) != bad);
}

int main() {
  check_jobs();
  check_counts();
  check_signatures();
  check_tree_plans();
  check_entry_points();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("ALL HOST CHECKS PASSED\n");
  return 0;
}
