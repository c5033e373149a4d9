// Device helpers shared by the verifier's kernels: typed 16-byte loads of logit rows, wave-level reductions and
// scans through DPP, workgroup reductions, and the device-scope loads, stores and counters that pass records between
// workgroups of one launch. gfx950 only: 64-lane waves.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace sv {

// ----------------------------------------------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------------------------------------------

// Loads through the global address space. The logit rows are always global memory; saying so keeps the loads
// global_load instructions (not flat ones) wherever the compiler cannot see where a pointer came from.
#define SV_GLOBAL __attribute__((address_space(1)))
template <typename V>
__device__ __forceinline__ V gload(const V* p) {
  return *(const SV_GLOBAL V*)(p);
}

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int kEPV = 4;                                  // elements per 16-byte vector
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return gload(p); }
};
template <> struct Vec<uint16_t> {
  static constexpr int kEPV = 8;
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xFFFF0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return __uint_as_float(uint32_t(gload(p)) << 16); }
};

__device__ __forceinline__ float ex2f(float x) { return __builtin_amdgcn_exp2f(x); }

// Element i of a row of V logits, -inf for i >= V. The load address is clamped into the row and the value selected
// afterwards, so a run of such loads issues without a branch (and a wait) per element.
template <typename T>
__device__ __forceinline__ float elem_or_ninf(const T* row, int64_t i, int64_t V) {
  const float z = Vec<T>::load1(row + (i < V ? i : V - 1));
  return i < V ? z : -INFINITY;
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 gload4(const uint4* p) {
  const u32x4 r = *(const SV_GLOBAL u32x4*)(p);
  return make_uint4(r.x, r.y, r.z, r.w);
}

// A 16-byte load; NT: non-temporal (streamed data, not kept in the caches).
template <bool NT>
__device__ __forceinline__ uint4 load_vec(const uint4* p) {
  const SV_GLOBAL u32x4* q = (const SV_GLOBAL u32x4*)(p);
  u32x4 r;
  if constexpr (NT) r = __builtin_nontemporal_load(q);
  else r = *q;
  return make_uint4(r.x, r.y, r.z, r.w);
}

// ----------------------------------------------------------------------------------------------------------------
// wave-level reductions and scans through DPP: data-parallel-primitive moves between the lanes of a row of 16 inside
// the VALU (a few cycles each, where a cross-lane shuffle is an LDS round trip); rows are combined with readlane.
// All 64 lanes must be active. The operation order is fixed, so results are bitwise reproducible and identical in
// every lane.
// ----------------------------------------------------------------------------------------------------------------

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <- lane 7 - i within each 8
constexpr int kDppMirror = 0x140;      // row_mirror: lane i <- lane 15 - i within each row
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;   // row_shr:n
constexpr int kDppBcast15 = 0x142;     // row_bcast:15: lane 15 of the previous row
constexpr int kDppBcast31 = 0x143;     // row_bcast:31: lane 31

// v moved by the DPP control CTRL; lanes outside ROWS, or whose source lies outside the row, get `old`.
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __int_as_float(dpp_i<CTRL, ROWS>(__float_as_int(old), __float_as_int(v)));
}
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ double dpp_d(double old, double v) {
  return __hiloint2double(dpp_i<CTRL, ROWS>(__double2hiint(old), __double2hiint(v)),
                          dpp_i<CTRL, ROWS>(__double2loint(old), __double2loint(v)));
}
// v moved by CTRL where every lane's source lies inside its row and every row takes part (no `old` operand needed).
template <int CTRL>
__device__ __forceinline__ double dpp_full_d(double v) {
  return __hiloint2double(__builtin_amdgcn_mov_dpp(__double2hiint(v), CTRL, 0xF, 0xF, true),
                          __builtin_amdgcn_mov_dpp(__double2loint(v), CTRL, 0xF, 0xF, true));
}
// v from the first active lane, in scalar registers. readfirstlane returns an int: each half is taken back as an
// unsigned 32-bit value before widening, so a low half at or above 2^31 does not spill into the high half.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
  const uint64_t u = uint64_t(v);
  const uint32_t hi = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(u >> 32)));
  const uint32_t lo = uint32_t(__builtin_amdgcn_readfirstlane(uint32_t(u)));
  return int64_t((uint64_t(hi) << 32) | uint64_t(lo));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                          __builtin_amdgcn_readlane(__double2loint(v), l));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_full_d<kDppXor1>(v);
  v += dpp_full_d<kDppXor2>(v);
  v += dpp_full_d<kDppHalfMirror>(v);
  v += dpp_full_d<kDppMirror>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}

__device__ __forceinline__ double wave_max_d(double v) {
  v = fmax(v, dpp_d<kDppXor1>(v, v));
  v = fmax(v, dpp_d<kDppXor2>(v, v));
  v = fmax(v, dpp_d<kDppHalfMirror>(v, v));
  v = fmax(v, dpp_d<kDppMirror>(v, v));
  return fmax(fmax(readlane_d(v, 0), readlane_d(v, 16)), fmax(readlane_d(v, 32), readlane_d(v, 48)));
}

__device__ __forceinline__ float wave_max_f(float v) {
  v = fmaxf(v, dpp_f<kDppXor1>(v, v));
  v = fmaxf(v, dpp_f<kDppXor2>(v, v));
  v = fmaxf(v, dpp_f<kDppHalfMirror>(v, v));
  v = fmaxf(v, dpp_f<kDppMirror>(v, v));
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

__device__ __forceinline__ int wave_min_i(int v) {
  v = min(v, dpp_i<kDppXor1>(v, v));
  v = min(v, dpp_i<kDppXor2>(v, v));
  v = min(v, dpp_i<kDppHalfMirror>(v, v));
  v = min(v, dpp_i<kDppMirror>(v, v));
  return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
             min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Inclusive running sum over the lanes in lane order (Hillis-Steele inside each row, then row carries).
__device__ __forceinline__ double wave_incl_scan(double v) {
  v += dpp_d<kDppShr1>(0.0, v);
  v += dpp_d<kDppShr2>(0.0, v);
  v += dpp_d<kDppShr4>(0.0, v);
  v += dpp_d<kDppShr8>(0.0, v);
  v += dpp_d<kDppBcast15, 0xA>(0.0, v);
  v += dpp_d<kDppBcast31, 0xC>(0.0, v);
  return v;
}
__device__ __forceinline__ int wave_incl_scan_i(int v) {
  v += dpp_i<kDppShr1>(0, v);
  v += dpp_i<kDppShr2>(0, v);
  v += dpp_i<kDppShr4>(0, v);
  v += dpp_i<kDppShr8>(0, v);
  v += dpp_i<kDppBcast15, 0xA>(0, v);
  v += dpp_i<kDppBcast31, 0xC>(0, v);
  return v;
}

// Wave-wide vote and the rank of this lane among the lanes whose vote is set.
__device__ __forceinline__ uint64_t wave_ballot(bool p) { return __builtin_amdgcn_ballot_w64(p); }
__device__ __forceinline__ int lane_rank(uint64_t m) {
  return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// ----------------------------------------------------------------------------------------------------------------
// block reductions (fixed order, so results are bitwise reproducible)
// ----------------------------------------------------------------------------------------------------------------

template <int BLOCK>
__device__ __forceinline__ float block_max(float v, float* sh) {
  v = wave_max_f(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  float r = sh[0];
#pragma unroll
  for (int i = 1; i < BLOCK / 64; ++i) r = fmaxf(r, sh[i]);
  return r;
}

template <int BLOCK>
__device__ __forceinline__ double block_sum(double v, double* sh) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < BLOCK / 64; ++i) r += sh[i];
  return r;
}

// ----------------------------------------------------------------------------------------------------------------
// passing records between workgroups of one kernel
// ----------------------------------------------------------------------------------------------------------------
// Each XCD has its own write-back L2, so a plain store from one workgroup may not be visible to a workgroup on
// another XCD before the kernel ends. Records handed over inside a kernel are stored and loaded at device scope
// (written through to, and read from, the level where all XCDs agree); the writer waits for its stores to complete
// and then counts itself on a per-sequence counter (a system-scope atomic, performed where all XCDs agree); the
// workgroup that brings the count to its total reads the records. Nobody waits on a counter.
template <typename V>
__device__ __forceinline__ void st_dev(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename V>
__device__ __forceinline__ V ld_dev(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// System-scope forms, for the counters that workgroups poll (they are updated with system-scope atomics).
template <typename V>
__device__ __forceinline__ void st_sys(V* p, V v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
template <typename V>
__device__ __forceinline__ V ld_sys(const V* p) {
  return __hip_atomic_load(const_cast<V*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ int32_t ctr_add(int32_t* p) {
  return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

}  // namespace sv
