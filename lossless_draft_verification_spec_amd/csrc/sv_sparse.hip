// Sparse (top-k support) speculative-sampling verification for gfx950 (MI355X).
//
// Follows the engine routine printed on "Uno: the draft model was already inside the target model" (section "What
// 'lossless' actually has to mean"): the probabilities of the drafted id are gathered from each support by id
// equality (p_spec, q_spec), the ratio is 0 when q_spec is 0, the test is the strict u < min(1, ratio), and the
// correction distribution is clamp(p - q_on_p, 0) renormalised on p's support. On top of that routine this kernel
// adds the first-rejection scan and the draw from the correction distribution at that slot (or a bonus draw from p's
// support of row gamma), as the dense path does.
//
// One workgroup (4 waves) per sequence; each wave handles one slot at a time with the slot's supports staged in LDS.
// Every sum is float64 and runs strictly in slot order, so all outputs equal the float64 evaluation of the
// definitions: the accept test u * q_spec < p_spec is exact for float32 inputs, and the draw index is chosen on
// the same running sums a sequential CPU evaluation forms. Ids are matched by direct comparison (no sorting).

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "sv.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

struct WaveLds {
  int32_t pid[SV_MAX_K];
  float pp[SV_MAX_K];
  int32_t qid[SV_MAX_K];
  float qp[SV_MAX_K];
  double w[SV_MAX_K];     // draw weights of the slot (correction, or p when the correction is empty)
};

__device__ __forceinline__ bool bad_prob(float v) { return !(v >= 0.f) || v == INFINITY; }   // NaN, <0, inf

// Stage row j's supports into the wave's LDS area.
__device__ __forceinline__ void stage(WaveLds& L, const int32_t* pi, const float* pp, int kp, const int32_t* qi,
                                      const float* qp, int kq, int lane) {
  for (int i = lane; i < kp; i += 64) { L.pid[i] = pi[i]; L.pp[i] = pp[i]; }
  if (qi)
    for (int i = lane; i < kq; i += 64) { L.qid[i] = qi[i]; L.qp[i] = qp[i]; }
}

// Correction weights max(p_i - q_on_p_i, 0) of the staged row into L.w; returns their slot-order sum.
__device__ __forceinline__ double correction(WaveLds& L, int kp, int kq, int lane) {
#pragma clang fp contract(off)
  for (int i = lane; i < kp; i += 64) {
    const int id = L.pid[i];
    double qop = 0.0;
    for (int l = 0; l < kq; ++l) qop += (L.qid[l] == id) ? double(L.qp[l]) : 0.0;
    const double r = double(L.pp[i]) - qop;
    L.w[i] = r > 0.0 ? r : 0.0;
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double s = 0.0;
  for (int i = 0; i < kp; ++i) s += L.w[i];
  return s;
}

// Replace the weights by p (the empty-residual fallback); returns the slot-order sum.
__device__ __forceinline__ double weights_from_p(WaveLds& L, int kp, int lane) {
  for (int i = lane; i < kp; i += 64) L.w[i] = double(L.pp[i]);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  double s = 0.0;
  for (int i = 0; i < kp; ++i) s += L.w[i];
  return s;
}

// Smallest slot whose slot-order running sum of L.w exceeds t; the last positive slot if none (rounding).
__device__ __forceinline__ int draw_slot(const WaveLds& L, int kp, double t) {
  double acc = 0.0;
  int found = -1, last = -1;
  for (int i = 0; i < kp; ++i) {
    const double w = L.w[i];
    acc += w;
    if (w > 0.0) last = i;
    if (found < 0 && acc > t) found = i;
  }
  return found >= 0 ? found : last;
}

struct SpParams {
  SparseArgs a;
};

__global__ __launch_bounds__(kBlock) void k_sparse(SparseArgs a) {
  __shared__ WaveLds lds[kWaves];
  __shared__ uint8_t s_acc[SV_MAX_GAMMA];
  __shared__ int s_k;

  const int64_t b = blockIdx.x;
  const int G = a.G, kp = a.kp, kq = a.kq;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int rows_p = G + (a.bonus ? 1 : 0);
  const int32_t* P_ids = a.p_ids + b * int64_t(rows_p) * kp;
  const float* P_pr = a.p_probs + b * int64_t(rows_p) * kp;
  const int32_t* Q_ids = a.q_ids + b * int64_t(G) * kq;
  const float* Q_pr = a.q_probs + b * int64_t(G) * kq;

  // validation of every verified row (rows 0 .. G-1) before anything is written
  int bad_id = 0, bad_nf = 0;
  for (int64_t i = tid; i < int64_t(G) * kp; i += kBlock) {
    bad_nf |= bad_prob(P_pr[i]);
    if (a.vocab > 0) bad_id |= (P_ids[i] < 0 || P_ids[i] >= a.vocab);
  }
  for (int64_t i = tid; i < int64_t(G) * kq; i += kBlock) {
    bad_nf |= bad_prob(Q_pr[i]);
    if (a.vocab > 0) bad_id |= (Q_ids[i] < 0 || Q_ids[i] >= a.vocab);
  }
  if (a.vocab > 0)
    for (int j = tid; j < G; j += kBlock) bad_id |= (a.spec[b * G + j] < 0 || a.spec[b * G + j] >= a.vocab);
  bad_id = __syncthreads_or(bad_id);
  bad_nf = __syncthreads_or(bad_nf);
  const bool fatal = bad_id || bad_nf;
  uint32_t flg = (bad_id ? SV_FLAG_ID_RANGE : 0u) | (bad_nf ? SV_FLAG_NONFINITE : 0u);

  if (fatal) {
    for (int j = tid; j < G; j += kBlock) {
      if (a.accept) a.accept[b * G + j] = 0;
      if (a.p_spec) a.p_spec[b * G + j] = NAN;
      if (a.q_spec) a.q_spec[b * G + j] = NAN;
    }
    if (a.corr)
      for (int64_t i = tid; i < int64_t(G) * kp; i += kBlock) a.corr[b * int64_t(G) * kp + i] = NAN;
    if (tid == 0) {
      a.n_acc[b] = -1;
      a.token[b] = -1;
      if (a.flags) a.flags[b] = flg;
    }
    return;
  }

  WaveLds& L = lds[wv];
  int qzero_any = 0;
  for (int j0 = 0; j0 < G; j0 += kWaves) {
    const int j = j0 + wv;
    if (j < G) {
      stage(L, P_ids + int64_t(j) * kp, P_pr + int64_t(j) * kp, kp, Q_ids + int64_t(j) * kq,
            Q_pr + int64_t(j) * kq, kq, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int x = a.spec[b * G + j];
      double ps = 0.0, qs = 0.0;
      for (int i = 0; i < kp; ++i) ps += (L.pid[i] == x) ? double(L.pp[i]) : 0.0;
      for (int l = 0; l < kq; ++l) qs += (L.qid[l] == x) ? double(L.qp[l]) : 0.0;
      const double u = double(a.ua[b * G + j]);
      const bool acc = (qs > 0.0) && (u * qs < ps);
      qzero_any |= (qs == 0.0);
      double S = correction(L, kp, kq, lane);
      if (!(S > 0.0)) S = weights_from_p(L, kp, lane);
      if (a.corr)
        for (int i = lane; i < kp; i += 64) a.corr[(b * G + j) * int64_t(kp) + i] = float(L.w[i] / S);
      if (lane == 0) {
        s_acc[j] = acc ? 1 : 0;
        if (a.accept) a.accept[b * G + j] = acc ? 1 : 0;
        if (a.p_spec) a.p_spec[b * G + j] = float(ps);
        if (a.q_spec) a.q_spec[b * G + j] = float(qs);
      }
    }
    __syncthreads();
  }
  qzero_any = __syncthreads_or(qzero_any);
  if (qzero_any) flg |= SV_FLAG_Q_ZERO;

  // first rejection; then the draw, by wave 0
  if (tid == 0) {
    int k = G;
    for (int j = 0; j < G; ++j)
      if (!s_acc[j]) { k = j; break; }
    s_k = k;
  }
  __syncthreads();
  const int k = s_k;
  if (wv != 0) return;
  int tok = -1;
  if (k < G) {
    stage(L, P_ids + int64_t(k) * kp, P_pr + int64_t(k) * kp, kp, Q_ids + int64_t(k) * kq, Q_pr + int64_t(k) * kq,
          kq, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double S = correction(L, kp, kq, lane);
    if (!(S > 0.0)) {
      S = weights_from_p(L, kp, lane);
      flg |= SV_FLAG_EMPTY_RESIDUAL;
    }
    const double t = double(a.us[b * (G + 1) + k]) * S;
    const int slot = draw_slot(L, kp, t);
    tok = slot >= 0 ? L.pid[slot] : -1;
  } else if (a.bonus) {
    const int32_t* bi = P_ids + int64_t(G) * kp;
    const float* bp = P_pr + int64_t(G) * kp;
    int bad = 0, badid = 0;
    for (int i = lane; i < kp; i += 64) {
      bad |= bad_prob(bp[i]);
      if (a.vocab > 0) badid |= (bi[i] < 0 || bi[i] >= a.vocab);
    }
    bad = __any(bad);          // wave-wide
    badid = __any(badid);
    if (bad) {
      flg |= SV_FLAG_NONFINITE;
    } else if (badid) {
      flg |= SV_FLAG_ID_RANGE;
    } else {
      stage(L, bi, bp, kp, nullptr, nullptr, 0, lane);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const double S = weights_from_p(L, kp, lane);
      const double t = double(a.us[b * (G + 1) + G]) * S;
      const int slot = draw_slot(L, kp, t);
      tok = slot >= 0 ? L.pid[slot] : -1;
    }
  }
  if (lane == 0) {
    a.n_acc[b] = k;
    a.token[b] = tok;
    if (a.flags) a.flags[b] = flg;
  }
}

}  // namespace

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(k_sparse, dim3(unsigned(a.B)), dim3(kBlock), 0, stream, a);
  return hipGetLastError();
}

}  // namespace sv
