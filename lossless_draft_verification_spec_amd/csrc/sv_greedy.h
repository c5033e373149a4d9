// Host-side declarations of the greedy verifier (sv_greedy.hip): sizes and workspace layout of one call, and its
// launcher.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "sv_internal.h"

namespace sv {

constexpr uint64_t kLayoutGreedy = 0x2325cbf29ce48422ull;   // workspace control layout kind (see sv_wshdr.h)
constexpr int64_t kGreedyMaxSeg = 64;          // segments per row at most (longer rows get longer segments)
constexpr int64_t kGreedyTargetItems = 1024;   // workgroups a launch aims at (about the resident count)

struct GreedyPlan {
  int64_t B = 0;
  int32_t G = 0;
  int32_t R = 0;           // target rows per sequence: gamma + bonus
  int64_t V = 0;
  int64_t seg_elems = 0;   // logits per segment (a multiple of 256 vectors)
  int32_t S = 1;           // segments per row
  int64_t items = 0;       // workgroups of the launch: B * R * S
  size_t ctr_bytes = 0;    // header + control region [0, ctr_bytes): int32 per sequence, returned to 0 by its merge
  size_t off_part = 0;     // uint64 key per (sequence, row, segment)
  size_t off_part2 = 0;    // float2 (segment maximum, sum of exp(z - maximum)) per (sequence, row, segment)
  size_t total = 0;
};

GreedyPlan make_greedy_plan(int64_t B, int32_t G, int64_t V, int32_t bonus, int dtype);
// The largest plan over both dtypes and both bonus settings: the workspace size for (B, gamma, V).
size_t greedy_workspace_bytes(int64_t B, int32_t G, int64_t V);

struct GreedyArgs {
  const void* tgt; int64_t t_seq, t_row;
  int dtype; int32_t bonus;
  const int32_t* ids;
  int32_t* start; const int32_t* order;
  uint8_t* accept; int32_t* n_acc; int32_t* token; uint32_t* flags;
  char* ws;
  // confidence-threshold commit: gamma = W slots, bonus 0, n_acc = committed count, token [B][W]
  bool conf_mode = false;
  const uint8_t* masked = nullptr; float tau = 0.f; uint8_t* commit = nullptr; float* conf = nullptr;
};

hipError_t launch_greedy(const GreedyPlan& plan, const GreedyArgs& a, hipStream_t stream);

}  // namespace sv
