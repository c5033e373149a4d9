// Sparse (top-k support) speculative-sampling verification for gfx950 (MI355X).
//
// Follows the engine routine printed on "Uno: the draft model was already inside the target model" (section "What
// 'lossless' actually has to mean"): the probabilities of the drafted id are gathered from each support by id
// equality (p_spec, q_spec), the ratio is 0 when q_spec is 0, the test is the strict u < min(1, ratio), and the
// correction distribution is clamp(p - q_on_p, 0) renormalised on p's support. On top of that routine this kernel
// adds the first-rejection scan and the draw from the correction distribution at that slot (or a bonus draw from p's
// support of row gamma), as the dense path does.
//
// One workgroup of 8 waves per sequence (four fit a compute unit for supports of up to 64 entries, so that a thousand
// sequences run in one round); the slots go in batches whose correction weights fit the LDS table (one batch for the
// usual sizes, e.g. 16 slots of 64-entry supports).
//  1. a wave per slot (slots wave, wave + 8, ...), the slot's supports in its lanes (entry e in lane e % 64,
//     register e / 64): the rows are checked; p_spec and q_spec come from a ballot of the entries whose id is the
//     drafted one; the accept test; then each p entry's q probability through the wave's bucket index of q (see
//     slot_weights), and the weights max(p - q_on_p, 0) into the LDS table with their ids (p's probabilities when no
//     weight is positive). With one batch, the checks of every row end before any output is written; with several, all
//     rows are checked in a pass before.
//  2. one thread per slot sums its weights in slot order (and keeps the running sums of the slot to be drawn from);
//     the outputs and the normalised correction distribution are written by all threads.
//  3. the draw, by one wave: a ballot over the stored running sums finds the first that exceeds t.
// Every float64 sum runs strictly in support-slot order, as a sequential CPU evaluation forms it (a q_on_p term has
// one matching q entry unless q's ids repeat, in which case that slot's matches are summed in slot order as well),
// so all outputs equal the float64 evaluation of the definitions: the accept test u * q_spec < p_spec is exact for
// float32 inputs, and the draw index is chosen on the same running sums.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "sv.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kBlock = 512;
constexpr int kWaves = kBlock / 64;
constexpr int kEntMax = SV_MAX_K / 64;  // support entries per lane for the largest supports
constexpr int kTable = 1536;            // float64 weights (and their ids) the LDS tables hold: a batch of slots
constexpr int kBatchMax = 256;          // slots per batch at most

__device__ __forceinline__ bool bad_prob(float v) { return !(v >= 0.f) || v == INFINITY; }   // NaN, <0, inf

// One support row in the lanes of a wave: entry e = 64 m + lane in (id[m], pr[m]); entries past k are id -1, 0.
// kEnt entries per lane hold supports of up to 64 kEnt entries.
template <int kEnt>
struct Row {
  int32_t id[kEnt];
  float pr[kEnt];
};
template <int kEnt>
__device__ __forceinline__ Row<kEnt> load_row(const int32_t* ids, const float* pr, int k, int lane) {
  Row<kEnt> r;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    const int e = m * 64 + lane;
    r.id[m] = e < k ? ids[e] : -1;
    r.pr[m] = e < k ? pr[e] : 0.f;
  }
  return r;
}
// Whether a row holds a probability that is NaN, negative or +inf (bad_nf), or an id outside [0, vocab) (bad_id).
template <int kEnt>
__device__ __forceinline__ void check_row(const Row<kEnt>& r, int k, int64_t vocab, int& bad_nf, int& bad_id) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    if (m * 64 + lane < k) {
      bad_nf |= bad_prob(r.pr[m]);
      if (vocab > 0) bad_id |= (r.id[m] < 0 || r.id[m] >= vocab);
    }
  }
}

// Sum, in slot order, of the probabilities of the entries whose id is x (usually one entry or none).
template <int kEnt>
__device__ __forceinline__ double match_sum(const Row<kEnt>& r, int k, int32_t x) {
  double s = 0.0;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    if (m * 64 >= k) break;
    uint64_t hit = __ballot(r.id[m] == x && m * 64 + int(threadIdx.x & 63) < k);
    while (hit) {
      const int l = __builtin_ctzll(hit);
      hit &= hit - 1;
      s += double(__uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(r.pr[m]), l)));
    }
  }
  return s;
}

// Buckets of a wave's index of q (an entry number each): four per entry of the widest q support, so that few
// entries share a bucket.
template <int kEnt> constexpr int kQBuckets = 256 * kEnt;
template <int kEnt> constexpr int kQBucketBits = kEnt == 1 ? 8 : kEnt == 2 ? 9 : 10;

// Sized for supports of up to 64 kEnt entries, so that the narrow layouts leave room for more workgroups.
template <int kEnt>
struct SpShared {
  double w[kTable];                    // weights of the batch's slots, row stride ldw
  int32_t pid[kTable];                 // their p ids
  double S[kBatchMax];                 // per slot of the batch: its normaliser
  double cum[64 * kEnt];               // the drawn slot's running sums of its weights (slot order)
  int32_t qb[kWaves][kQBuckets<kEnt>]; // per wave: the index of its slot's q support (entry per bucket)
  float ps[kBatchMax], qs[kBatchMax];  // per slot of the batch: p_spec, q_spec
  float us[kBatchMax];                 // per slot of the batch: its draw uniform
  uint8_t acc[SV_MAX_GAMMA];
  uint8_t empty[kBatchMax];            // per slot of the batch: no leftover mass (the weights are p)
  int32_t k;
  int32_t tok;
};

// Sum of n weights in slot order (one thread), their values requested eight at a time; with cum, every running sum
// is stored too.
__device__ __forceinline__ double seq_sum(const double* w, int n, double* cum) {
  double s = 0.0;
  int e = 0;
  for (; e + 8 <= n; e += 8) {
    double v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = w[e + i];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      s += v[i];
      if (cum) cum[e + i] = s;
    }
  }
  for (; e < n; ++e) {
    s += w[e];
    if (cum) cum[e] = s;
  }
  return s;
}

// The draw over a row of n weights whose running sums are in cum (by one wave): the smallest slot whose running sum
// exceeds t; the last slot with positive weight if none (rounding); -1 when no weight is positive.
__device__ __forceinline__ int wave_draw(const double* w, const double* cum, int n, double t) {
  const int lane = threadIdx.x & 63;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const uint64_t hit = __ballot(e0 + lane < n && cum[e0 + lane] > t);
    if (hit) return e0 + __builtin_ctzll(hit);
  }
  for (int e0 = (n - 1) / 64 * 64; e0 >= 0; e0 -= 64) {
    const uint64_t pos = __ballot(e0 + lane < n && w[e0 + lane] > 0.0);
    if (pos) return e0 + 63 - __builtin_clzll(pos);
  }
  return -1;
}

template <int kEnt>
__device__ __forceinline__ uint32_t q_bucket(int32_t id) {
  return (uint32_t(id) * 0x9E3779B1u) >> (32 - kQBucketBits<kEnt>);
}

// q entry e (taken mod 64 kEnt) for every lane: id and probability, read across lanes from the lane that holds it.
template <int kEnt>
__device__ __forceinline__ void q_entry(const Row<kEnt>& Q, int e, int32_t& id, float& pr) {
  const int src = (e & 63) << 2;
  id = -1;
  pr = 0.f;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    const int i = __builtin_amdgcn_ds_bpermute(src, Q.id[m]);
    const int f = __builtin_amdgcn_ds_bpermute(src, __float_as_int(Q.pr[m]));
    if (((e >> 6) & (kEnt - 1)) == m) {
      id = i;
      pr = __int_as_float(f);
    }
  }
}

// The correction weights max(p_e - q_on_p_e, 0) of one slot (by one wave) into w, and the p ids into ids. Each p
// entry's q probability is found through the wave's index of q (qb, an entry number per bucket of the id's hash): every
// q entry writes its index at its bucket, and an entry that reads back another's has lost the bucket; each p entry
// reads its bucket and checks the id of the q entry named there (so the index needs no clearing: a stale or
// uninitialised word names an entry whose id does not match, or one that does and is a true match); the q entries that
// lost their bucket (a few) are then compared with every p entry one at a time. When q repeats an id, every q_on_p is
// summed again in float64 in q's slot order instead, each q entry read across lanes. With no positive weight (no
// leftover mass) the weights become p's probabilities and the result is true (the same for every lane).
template <int kEnt>
__device__ __forceinline__ bool slot_weights(const Row<kEnt>& P, const Row<kEnt>& Q, int kp, int kq, int32_t* qb,
                                             double* w, int32_t* ids) {
  const int lane = threadIdx.x & 63;
  // lanes talk through the index, so every access is a relaxed atomic (never merged with this lane's own earlier
  // write by the compiler); every write of the wave lands before its reads: the LDS executes one wave's operations
  // in issue order
  auto put = [&](int b, int v) { __hip_atomic_store(qb + b, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT); };
  auto get = [&](int b) { return __hip_atomic_load(qb + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT); };
#pragma unroll
  for (int m = 0; m < kEnt; ++m)
    if (m * 64 + lane < kq) put(q_bucket<kEnt>(Q.id[m]), m * 64 + lane);
  uint64_t lost[kEnt];
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    const int e = m * 64 + lane;
    lost[m] = __ballot(e < kq && get(q_bucket<kEnt>(Q.id[m])) != e);
  }
  float qm[kEnt];
  int nm[kEnt];
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    const bool ok = m * 64 + lane < kp;
    const int c = ok ? get(q_bucket<kEnt>(P.id[m])) : 0;
    int32_t qid;
    float qpr;
    q_entry<kEnt>(Q, c, qid, qpr);
    const bool hit = ok && c >= 0 && c < kq && qid == P.id[m];
    qm[m] = hit ? qpr : 0.f;
    nm[m] = hit ? 1 : 0;
  }
#pragma unroll
  for (int mq = 0; mq < kEnt; ++mq) {
    uint64_t left = lost[mq];
    while (left) {
      const int l = __builtin_ctzll(left);
      left &= left - 1;
      const int32_t qid = __builtin_amdgcn_readlane(Q.id[mq], l);
      const float qpr = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(Q.pr[mq]), l));
#pragma unroll
      for (int m = 0; m < kEnt; ++m) {
        const bool hit = m * 64 + lane < kp && P.id[m] == qid;
        qm[m] = hit ? qpr : qm[m];
        nm[m] += hit ? 1 : 0;
      }
    }
  }
  bool multi = false;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) multi |= nm[m] > 1;
  double qop[kEnt];
#pragma unroll
  for (int m = 0; m < kEnt; ++m) qop[m] = double(qm[m]);
  if (__any(multi)) {
#pragma unroll
    for (int m = 0; m < kEnt; ++m) qop[m] = 0.0;
#pragma unroll
    for (int mq = 0; mq < kEnt; ++mq) {
      const int n = min(64, kq - 64 * mq);
      for (int l = 0; l < n; ++l) {
        const int32_t qid = __builtin_amdgcn_readlane(Q.id[mq], l);
        const double qpr = double(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(Q.pr[mq]), l)));
#pragma unroll
        for (int m = 0; m < kEnt; ++m) qop[m] += (P.id[m] == qid) ? qpr : 0.0;
      }
    }
  }
  double r[kEnt];
  bool pos = false;
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
#pragma clang fp contract(off)
    const double d = double(P.pr[m]) - qop[m];
    r[m] = d > 0.0 ? d : 0.0;
    pos |= m * 64 + lane < kp && r[m] > 0.0;
  }
  const bool empty = !__any(pos);
#pragma unroll
  for (int m = 0; m < kEnt; ++m) {
    const int e = m * 64 + lane;
    if (e < kp) {
      w[e] = empty ? double(P.pr[m]) : r[m];
      ids[e] = P.id[m];
    }
  }
  return empty;
}

// Waves per SIMD asked of each layout: the narrowest (supports of up to 64 entries) fits four workgroups per compute
// unit, so that a thousand sequences run in one round.
template <int kEnt> constexpr int kSparseWpe = kEnt == 1 ? 8 : 1;

template <int kEnt>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(kSparseWpe<kEnt>)))
void k_sparse(SparseArgs kargs) {
  (void)kargs;
  // the arguments are read in place from the argument segment, each when it is used, instead of being held in
  // scalar registers for the whole kernel
  const SparseArgs& a = *(const SparseArgs*)(__builtin_amdgcn_kernarg_segment_ptr());
  __shared__ SpShared<kEnt> sh;

  const int64_t b = blockIdx.x;
  const int G = a.G, kp = a.kp, kq = a.kq;
  // the wave index in a scalar register: every slot index, row address and loop bound of a wave is then scalar
  const int tid = threadIdx.x, lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rows_p = G + (a.bonus ? 1 : 0);
  const int32_t* P_ids = a.p_ids + b * int64_t(rows_p) * kp;
  const float* P_pr = a.p_probs + b * int64_t(rows_p) * kp;
  const int32_t* Q_ids = a.q_ids + b * int64_t(G) * kq;
  const float* Q_pr = a.q_probs + b * int64_t(G) * kq;
  const int ldw = kp | 1;                            // odd row stride: the lanes of the normaliser step use distinct banks
  const int nb = min(kTable / ldw, kBatchMax);       // slots per batch
  const bool single = G <= nb;                       // one batch: checked while it is read (the usual case)
  const bool weights = single || a.corr;             // weights of every slot (else only the rejected slot's, at the end)

  int bad_id = 0, bad_nf = 0;
  auto fail = [&]() {
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
      if (a.flags) a.flags[b] = (bad_id ? SV_FLAG_ID_RANGE : 0u) | (bad_nf ? SV_FLAG_NONFINITE : 0u);
    }
  };
  if (!single) {                                     // every verified row is checked before anything is written
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
    if (bad_id || bad_nf) { fail(); return; }
  }

  uint32_t flg = 0;
  int qzero_any = 0;
  if (tid == 0) { sh.k = G; sh.tok = -1; }
  for (int j0 = 0; j0 < G; j0 += nb) {
    const int j1 = min(j0 + nb, G);
    // 1. a wave per slot: accept test and, when needed, the correction weights
    for (int j = j0 + wv; j < j1; j += kWaves) {
      const Row<kEnt> P = load_row<kEnt>(P_ids + int64_t(j) * kp, P_pr + int64_t(j) * kp, kp, lane);
      const Row<kEnt> Q = load_row<kEnt>(Q_ids + int64_t(j) * kq, Q_pr + int64_t(j) * kq, kq, lane);
      const int32_t x = a.spec[b * G + j];
      const float u = a.ua[b * G + j];
      const float uds = a.us[b * (G + 1) + j];
      if (single) {
        check_row(P, kp, a.vocab, bad_nf, bad_id);
        check_row(Q, kq, a.vocab, bad_nf, bad_id);
        if (a.vocab > 0) bad_id |= (x < 0 || x >= a.vocab);
      }
      const double ps = match_sum(P, kp, x);
      const double qs = match_sum(Q, kq, x);
      const bool acc = (qs > 0.0) && (double(u) * qs < ps);
      qzero_any |= (qs == 0.0);
      if (lane == 0) {
        sh.acc[j] = acc ? 1 : 0;
        sh.ps[j - j0] = float(ps);
        sh.qs[j - j0] = float(qs);
        sh.us[j - j0] = uds;
      }
      if (weights) {
        const bool em = slot_weights(P, Q, kp, kq, sh.qb[wv], sh.w + (j - j0) * ldw, sh.pid + (j - j0) * ldw);
        if (lane == 0) sh.empty[j - j0] = em ? 1 : 0;
      }
    }
    if (single) {
      bad_id = __syncthreads_or(bad_id);
      bad_nf = __syncthreads_or(bad_nf);
      if (bad_id || bad_nf) { fail(); return; }
    }
    __syncthreads();
    if (single && wv == 0) {                         // the first rejection (G: none)
      int k = G;
      for (int i0 = 0; i0 < G; i0 += 64) {
        const uint64_t rej = __ballot(i0 + lane < G && sh.acc[i0 + lane] == 0);
        if (rej) {
          k = i0 + __builtin_ctzll(rej);
          break;
        }
      }
      if (lane == 0) sh.k = k;
    }
    __syncthreads();
    const int k = sh.k;                              // known here only with a single batch
    // 2. normalisers, one thread per slot
    if (weights) {
      for (int s = tid; s < j1 - j0; s += kBlock)
        sh.S[s] = seq_sum(sh.w + s * ldw, kp, j0 + s == k ? sh.cum : nullptr);
    }
    __syncthreads();
    // 3. the batch's outputs, then (single batch) the draw
    for (int s = tid; s < j1 - j0; s += kBlock) {
      if (a.accept) a.accept[b * G + j0 + s] = sh.acc[j0 + s];
      if (a.p_spec) a.p_spec[b * G + j0 + s] = sh.ps[s];
      if (a.q_spec) a.q_spec[b * G + j0 + s] = sh.qs[s];
    }
    if (a.corr) {
      for (int i = tid; i < (j1 - j0) * kp; i += kBlock) {
        const int s = i / kp, e = i - s * kp;
        a.corr[(b * G + j0 + s) * int64_t(kp) + e] = float(sh.w[s * ldw + e] / sh.S[s]);
      }
    }
    if (single && k < G && wv == 0) {
      const int sl = k - j0;
      const int e = wave_draw(sh.w + sl * ldw, sh.cum, kp, double(sh.us[sl]) * sh.S[sl]);
      if (lane == 0) sh.tok = e >= 0 ? sh.pid[sl * ldw + e] : -1;
      if (sh.empty[sl]) flg |= SV_FLAG_EMPTY_RESIDUAL;
    }
    __syncthreads();
  }
  qzero_any = __syncthreads_or(qzero_any);
  if (qzero_any) flg |= SV_FLAG_Q_ZERO;
  if (wv != 0) return;
  int k = sh.k;
  if (!single) {                                     // several batches: the first rejection, then its correction
    k = G;
    for (int i0 = 0; i0 < G; i0 += 64) {
      const uint64_t rej = __ballot(i0 + lane < G && sh.acc[i0 + lane] == 0);
      if (rej) {
        k = i0 + __builtin_ctzll(rej);
        break;
      }
    }
    if (k < G) {
      const Row<kEnt> P = load_row<kEnt>(P_ids + int64_t(k) * kp, P_pr + int64_t(k) * kp, kp, lane);
      const Row<kEnt> Q = load_row<kEnt>(Q_ids + int64_t(k) * kq, Q_pr + int64_t(k) * kq, kq, lane);
      const bool empty = slot_weights(P, Q, kp, kq, sh.qb[0], sh.w, sh.pid);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      double S = 0.0;
      if (lane == 0) S = seq_sum(sh.w, kp, sh.cum);
      S = __shfl(S, 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int e = wave_draw(sh.w, sh.cum, kp, double(a.us[b * (G + 1) + k]) * S);
      if (lane == 0) sh.tok = e >= 0 ? sh.pid[e] : -1;
      if (empty) flg |= SV_FLAG_EMPTY_RESIDUAL;
    }
  }
  if (k == G && a.bonus) {                           // every slot accepted: the bonus draw from p's row gamma (wave 0)
    const Row<kEnt> P = load_row<kEnt>(P_ids + int64_t(G) * kp, P_pr + int64_t(G) * kp, kp, lane);
    int bad = 0, badid = 0;
    check_row(P, kp, a.vocab, bad, badid);
    bad = __any(bad);
    badid = __any(badid);
    if (bad) {
      flg |= SV_FLAG_NONFINITE;
    } else if (badid) {
      flg |= SV_FLAG_ID_RANGE;
    } else {
#pragma unroll
      for (int m = 0; m < kEnt; ++m)
        if (m * 64 + lane < kp) sh.w[m * 64 + lane] = double(P.pr[m]);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      double S = 0.0;
      if (lane == 0) S = seq_sum(sh.w, kp, sh.cum);
      S = __shfl(S, 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int e = wave_draw(sh.w, sh.cum, kp, double(a.us[b * (G + 1) + G]) * S);
      int32_t id = -1;
#pragma unroll
      for (int m = 0; m < kEnt; ++m)
        if (e >= m * 64 && e < m * 64 + 64) id = __builtin_amdgcn_readlane(P.id[m], e - m * 64);
      if (lane == 0) sh.tok = id;
    }
  }
  if (lane != 0) return;
  a.n_acc[b] = k;
  a.token[b] = sh.tok;
  if (a.flags) a.flags[b] = flg;
}

}  // namespace

hipError_t launch_sparse(const SparseArgs& a, hipStream_t stream) {
  // the narrowest register layout that holds both supports
  const int k = a.kp > a.kq ? a.kp : a.kq;
  if (k <= 64) {
    hipLaunchKernelGGL(k_sparse<1>, dim3(unsigned(a.B)), dim3(kBlock), 0, stream, a);
  } else if (k <= 128) {
    hipLaunchKernelGGL(k_sparse<2>, dim3(unsigned(a.B)), dim3(kBlock), 0, stream, a);
  } else {
    hipLaunchKernelGGL(k_sparse<kEntMax>, dim3(unsigned(a.B)), dim3(kBlock), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace sv
