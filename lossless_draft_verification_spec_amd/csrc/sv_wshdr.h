// The workspace header: the first 256-byte line of every workspace that holds control words (work-queue counters,
// draw tickets, job slots), and the checks applied to the words that pass between workgroups of one launch.
//
// Every call leaves its control words at zero when it ends, so a workspace can serve any number of calls without a
// clearing pass. What those words mean, and where they sit, depends on the kind of call and on its shape: the header
// names the layout (a 64-bit signature) that the zeros belong to. Workgroup 0 of each launch compares the header
// with its own layout; when they differ (first use, garbage, another kind or shape of call before), or when the dirty
// word says that an earlier call stopped before returning its words to zero, it zeroes the control region and then
// publishes the signature. Every other workgroup waits until the header holds its layout, clean, before it touches a
// control word. Workgroup 0 is dispatched before all others, so every such wait ends. The library keeps no state of
// its own between calls: all of it lives in the caller's workspace.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "sv_internal.h"

namespace sv {

constexpr size_t kWsHeaderBytes = 256;

struct WsHeader {
  uint64_t sig;      // layout whose control words are at zero (0: none)
  uint32_t dirty;    // nonzero: a call gave up waiting and may have left control words set
  uint32_t pad;
};

// Signature of a control layout: the kind of call and the one size that places its control words (sequences or
// rows). Never 0, so that a zeroed header matches no layout.
inline uint64_t ws_signature(uint64_t kind, uint64_t n) {
  const uint64_t s = layout_mix(layout_mix(kind, n), 0x9e3779b97f4a7c15ull);
  return s == 0 ? 1 : s;
}

// Polls of a header or counter wait before the wait gives up (only a broken dispatch order could exhaust them).
constexpr int32_t kWsSpinCap = 1 << 20;

__device__ __forceinline__ uint64_t ws_ld_sig(const WsHeader* h) {
  return __hip_atomic_load(const_cast<uint64_t*>(&h->sig), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ws_ld_dirty(const WsHeader* h) {
  return __hip_atomic_load(const_cast<uint32_t*>(&h->dirty), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// By every thread of workgroup 0, before anything else touches a control word: if the header does not name this
// layout as clean, zero [kWsHeaderBytes, ctl_end) with device-scope stores, wait for them, then publish the layout.
__device__ __forceinline__ void ws_claim(char* ws, uint64_t sig, size_t ctl_end, int* sh_flag) {
  WsHeader* h = reinterpret_cast<WsHeader*>(ws);
  if (threadIdx.x == 0) *sh_flag = (ws_ld_sig(h) != sig) || (ws_ld_dirty(h) != 0u);
  __syncthreads();
  if (*sh_flag) {
    uint64_t* w = reinterpret_cast<uint64_t*>(ws + kWsHeaderBytes);
    const int64_t n = int64_t((ctl_end - kWsHeaderBytes) / 8);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x)
      __hip_atomic_store(w + i, uint64_t(0), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
      __hip_atomic_store(&h->dirty, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
      __hip_atomic_store(&h->sig, sig, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);
    }
  }
  __syncthreads();
}

// A plain (cached) read of the header. Within one launch the header only ever changes to "this layout, clean"
// (workgroup 0's claim), and the caches hold nothing older than the launch, so a copy that already shows this layout
// clean is exact whatever its age; any other value is confirmed with ws_ready.
__device__ __forceinline__ bool ws_seen_clean(const char* ws, uint64_t sig) {
  const WsHeader* h = reinterpret_cast<const WsHeader*>(ws);
  return h->sig == sig && h->dirty == 0u;
}

// By one thread: true once the header names this layout as clean (at once, unless workgroup 0 is clearing it);
// false after kWsSpinCap polls.
__device__ __forceinline__ bool ws_ready(const char* ws, uint64_t sig) {
  const WsHeader* h = reinterpret_cast<const WsHeader*>(ws);
  for (int32_t polls = 0; polls < kWsSpinCap; ++polls) {
    if (ws_ld_sig(h) == sig && ws_ld_dirty(h) == 0u) return true;
    __builtin_amdgcn_s_sleep(8);
  }
  return false;
}

// By one thread of a workgroup that gave up a wait: the next call clears the control region before using it.
__device__ __forceinline__ void ws_mark_dirty(char* ws) {
  WsHeader* h = reinterpret_cast<WsHeader*>(ws);
  __hip_atomic_store(&h->dirty, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ----------------------------------------------------------------------------------------------------------------
// checks of the words handed between workgroups
// ----------------------------------------------------------------------------------------------------------------

// A draw job read from the workspace, checked before any of its fields becomes an address or an index: the kind is
// one the call can produce; a residual or one-hot draw names a verified row in [0, gamma) (and a one-hot draw a
// draft id in [0, V)); a bonus draw names row gamma and only when the call draws a bonus; the new start lies in
// [-1, gamma]. `dense`: the call has draft logits (residual draws), else one-hot drafts.
__host__ __device__ inline bool job_valid(const Job& j, int32_t G, int64_t V, int32_t bonus, bool dense) {
  if (j.new_start < -1 || j.new_start > G) return false;
  switch (j.kind) {
    case JOB_NONE:
      return true;
    case JOB_RESID:
      return dense && j.row >= 0 && j.row < G;
    case JOB_ONEHOT:
      return !dense && j.row >= 0 && j.row < G && j.d >= 0 && int64_t(j.d) < V;
    case JOB_BONUS:
      return bonus != 0 && j.row == G;
    default:
      return false;
  }
}

// A count of candidate keys read back from a segment record of the support builder: clamped into [0, k].
__host__ __device__ inline int32_t clamp_count(int32_t n, int32_t k) { return n < 0 ? 0 : (n > k ? k : n); }

}  // namespace sv
