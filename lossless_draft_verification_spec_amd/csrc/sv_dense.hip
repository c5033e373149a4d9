// Dense and one-hot speculative-sampling verification for gfx950 (MI355X).
//
// The rule is Leviathan et al.'s, as restated on "Uno: the draft model was already inside the target model"
// (section "What 'lossless' actually has to mean"): accept a draft x with probability min(1, p(x)/q(x)), cut the
// block at the first rejection (DFlash/DFlash2 guide, section 4.4) and draw the replacement from max(p - q, 0)
// renormalised there, or a bonus token from the next target row when every draft is accepted (same guide,
// section 2). p and q are softmaxes of the logits divided by the temperature (same guide, section 9 Q3).
//
// Three launches, all on the caller's stream:
//  1. k_stats     : one read of every verified logit row. Per (row, segment) it keeps a running max and a running
//                   sum of exp2((z - max) * log2(e)/T) in float32, folds the threads together in float64 and writes
//                   (max, sum, logit at the draft id). 16-byte non-temporal loads, a two-group ping-pong per thread.
//                   This pass moves almost all the bytes; it is bound by HBM bandwidth.
//  2. k_draw_mass : one-wave workgroups. Each first evaluates p(x), q(x) and the strict test u < min(1, p/q) for
//                   every verified slot of its sequence and finds the first rejection from `start` along `order`
//                   (the first workgroup of the sequence writes the per-row outputs and the draw job); it then
//                   computes, in float64, the exact softmax normalisers and the residual mass of its chunks of the
//                   row(s) the draw needs (at most one row pair per sequence).
//  3. k_draw_pick : one workgroup per sequence: chunk masses, their running sum, and a search inside the one chunk
//                   that holds t = u * (total mass).
// The float64 draw exists because a token boundary of the residual CDF often lies within 1e-7 of t at these
// vocabulary sizes; float32 sums would pick a neighbouring token far more often than the float64 reference does.

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>

#include "sv.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kStatsBlock = 256;
constexpr int kUnroll = 4;          // 16-byte vectors per thread per group
#ifndef SV_STATS_NT
#define SV_STATS_NT 1
#endif
constexpr bool kNonTemporal = SV_STATS_NT != 0;   // streaming loads that bypass cache retention
constexpr int kStatsWpe = 4;        // waves per SIMD the statistics kernel is compiled for (more waves stream worse)
constexpr int kStatsWgPerCu = 0;    // persistent grid cap per CU (0: one workgroup per work item)
constexpr int kDrawBlock = 256;

struct alignas(16) Partial1 {
  float m;        // exact max of the segment's logits (raw, before the temperature)
  float zx;       // segment 0 only: the row's logit at its draft id (NaN when the id is out of range)
  double s;       // sum over the segment of 2^((z - m) * c), c = log2(e)/T rounded to float
};

// ----------------------------------------------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------------------------------------------

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int kEPV = 4;                                  // elements per 16-byte vector
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
};
template <> struct Vec<uint16_t> {
  static constexpr int kEPV = 8;
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xFFFF0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
};

__device__ __forceinline__ float ex2f(float x) { return __builtin_amdgcn_exp2f(x); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------------------------------------------
// block reductions (fixed order, so results are bitwise reproducible)
// ----------------------------------------------------------------------------------------------------------------

template <int BLOCK>
__device__ __forceinline__ float block_max(float v, float* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
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
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
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
// 1. row statistics
// ----------------------------------------------------------------------------------------------------------------

struct StatsParams {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;
  int64_t B; int32_t G; int64_t V; int32_t nseg; int32_t ntens;
  float c;                                  // log2(e) / T, rounded to float
  const int32_t* start; const int32_t* order;
  const int32_t* ids;                       // [B][G] draft ids (the logit at the id is gathered with segment 0)
  Partial1* part;                           // [ntens][B][G][nseg]
};

// Running state of one thread: max m, mc = fl(m * c), s = sum of 2^(z*c - mc).
struct Run {
  float m, mc, s;
};

template <int N>
__device__ __forceinline__ void absorb(Run& st, const float* v, float c) {
  float cm = v[0];
#pragma unroll
  for (int k = 1; k < N; ++k) cm = fmaxf(cm, v[k]);
  const float mn = fmaxf(st.m, cm);
  if (mn == -INFINITY) {                             // only -inf (or NaN) so far: nothing to add, but keep NaN
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (v[k] != v[k]) st.s = NAN;
    return;
  }
  const float mnc = __fmul_rn(mn, c);
  if (mn != st.m) {                                  // new maximum: rescale what was summed
    st.s *= ex2f(st.mc - mnc);
    st.m = mn;
    st.mc = mnc;
  }
  float t[N];
#pragma unroll
  for (int k = 0; k < N; ++k) t[k] = ex2f(fmaf(v[k], c, -mnc));
#pragma unroll
  for (int w = 1; w < N; w <<= 1)
#pragma unroll
    for (int k = 0; k + w < N; k += 2 * w) t[k] += t[k + w];
  st.s += t[0];
}

template <bool NT>
__device__ __forceinline__ uint4 load_vec(const uint4* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  u32x4 r;
  if constexpr (NT) r = __builtin_nontemporal_load(q);
  else r = *q;
  return make_uint4(r.x, r.y, r.z, r.w);
}

// One work item: segment `seg` of one row. Returns without writing when the row's slot lies before start.
template <typename T, int BLOCK, int U, bool NT>
__device__ __forceinline__ void stats_item(const StatsParams& prm, int64_t item, float* sh_f, double* sh_d) {
  using VT = Vec<T>;
  constexpr int EPV = VT::kEPV;

  int64_t w = item;
  const int seg = int(w % prm.nseg); w /= prm.nseg;
  const int row = int(w % prm.G);    w /= prm.G;
  const int64_t b = w % prm.B;
  const int tens = int(w / prm.B);

  if (prm.start) {                                   // rows of slots before start are not read
    const int st = prm.start[b];
    if (st < 0 || st > prm.G) return;                // reported by the scan (uniform: the block skips the item)
    if (st > 0) {
      int hit = 0;
      if (prm.order) {
        for (int s = threadIdx.x; s < st; s += BLOCK) hit |= (prm.order[b * prm.G + s] == row);
      } else {
        hit = row < st;
      }
      if (__syncthreads_or(hit)) return;
    }
  }

  const T* base = tens == 0
      ? static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(row) * prm.t_row
      : static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(row) * prm.d_row;
  const int64_t V = prm.V;
  const float c = prm.c;

  // head (until 16-byte alignment), vector body, tail
  const uintptr_t addr = reinterpret_cast<uintptr_t>(base);
  int64_t head = int64_t(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int64_t nvec = (V - head) / EPV;
  const int64_t v0 = nvec * seg / prm.nseg, v1 = nvec * (seg + 1) / prm.nseg;

  Run st{-INFINITY, -INFINITY, 0.f};
  if (seg == 0) {
    for (int64_t i = threadIdx.x; i < head; i += BLOCK) { float z = VT::load1(base + i); absorb<1>(st, &z, c); }
  }
  if (seg == prm.nseg - 1) {
    for (int64_t i = head + nvec * EPV + threadIdx.x; i < V; i += BLOCK) {
      float z = VT::load1(base + i);
      absorb<1>(st, &z, c);
    }
  }

  // Vector body. Each thread walks vectors v0+tid, v0+tid+BLOCK, ... in groups of U; full groups run in a two-group
  // ping-pong (one group is processed while the other is in flight), the few vectors left run one at a time.
  const uint4* vp = reinterpret_cast<const uint4*>(base + head);
  constexpr int64_t kStep = int64_t(U) * BLOCK;
  int64_t v = v0 + threadIdx.x;
  const int64_t span = v1 - v - int64_t(U - 1) * BLOCK;
  const int64_t ngroups = span > 0 ? (span + kStep - 1) / kStep : 0;
  if (ngroups > 0) {
    uint4 ga[U], gb[U];
    float z[U * EPV];
#pragma unroll
    for (int k = 0; k < U; ++k) ga[k] = load_vec<NT>(vp + v + int64_t(k) * BLOCK);
    int64_t g = 1;
    for (; g + 1 < ngroups; g += 2) {
      const uint4* pb = vp + v + g * kStep;
#pragma unroll
      for (int k = 0; k < U; ++k) gb[k] = load_vec<NT>(pb + int64_t(k) * BLOCK);
#pragma unroll
      for (int k = 0; k < U; ++k) VT::unpack(ga[k], z + k * EPV);
      absorb<U * EPV>(st, z, c);
      const uint4* pa = pb + kStep;
#pragma unroll
      for (int k = 0; k < U; ++k) ga[k] = load_vec<NT>(pa + int64_t(k) * BLOCK);
#pragma unroll
      for (int k = 0; k < U; ++k) VT::unpack(gb[k], z + k * EPV);
      absorb<U * EPV>(st, z, c);
    }
    if (g < ngroups) {
      const uint4* pb = vp + v + g * kStep;
#pragma unroll
      for (int k = 0; k < U; ++k) gb[k] = load_vec<NT>(pb + int64_t(k) * BLOCK);
#pragma unroll
      for (int k = 0; k < U; ++k) VT::unpack(ga[k], z + k * EPV);
      absorb<U * EPV>(st, z, c);
#pragma unroll
      for (int k = 0; k < U; ++k) VT::unpack(gb[k], z + k * EPV);
      absorb<U * EPV>(st, z, c);
    } else {
#pragma unroll
      for (int k = 0; k < U; ++k) VT::unpack(ga[k], z + k * EPV);
      absorb<U * EPV>(st, z, c);
    }
    v += ngroups * kStep;
  }
  for (; v < v1; v += BLOCK) {
    const uint4 w1 = load_vec<NT>(vp + v);
    float z[EPV];
    VT::unpack(w1, z);
    absorb<EPV>(st, z, c);
  }

  // Fold the threads: common max M, then each thread rescales its sum to 2^(z*c - M*c) in float64.
  const float M = block_max<BLOCK>(st.m, sh_f);
  double s = 0.0;
  if (st.m != -INFINITY && M != -INFINITY) {
    s = double(st.s) * exp2(double(st.mc) - double(M) * double(c));
  } else if (isnan(st.s)) {
    s = NAN;
  }
  s = block_sum<BLOCK>(s, sh_d);
  if (threadIdx.x == 0) {
    Partial1 out;
    out.m = M;
    out.zx = NAN;
    if (seg == 0) {
      const int x = prm.ids[b * prm.G + row];
      if (x >= 0 && int64_t(x) < V) out.zx = VT::load1(base + x);
    }
    out.s = s;
    prm.part[((int64_t(tens) * prm.B + b) * prm.G + row) * prm.nseg + seg] = out;
  }
}

// Persistent over work items (row, segment): workgroup g handles items g, g + gridDim.x, ... The grid is sized by
// the launcher to the device (WPE waves per SIMD, i.e. WPE * 4 / (BLOCK / 64) workgroups per CU).
template <typename T, int BLOCK, int U, bool NT, int WPE>
__global__ __launch_bounds__(BLOCK) __attribute__((amdgpu_waves_per_eu(WPE, WPE))) void k_stats(StatsParams prm) {
  __shared__ float sh_f[BLOCK / 64];
  __shared__ double sh_d[BLOCK / 64];
  const int64_t n_items = int64_t(prm.ntens) * prm.B * prm.G * prm.nseg;
  for (int64_t item = blockIdx.x; item < n_items; item += gridDim.x) {
    stats_item<T, BLOCK, U, NT>(prm, item, sh_f, sh_d);
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------------------------------
// 2. draw: accept tests and first-rejection scan, then the float64 draw (mass pass + pick)
// ----------------------------------------------------------------------------------------------------------------
//
// The rows are cut into chunks of kChunk = 1024 consecutive elements (one wave, 16 consecutive elements per lane).
// The mass pass starts, in every workgroup, with the accept tests of its sequence (from the statistics pass's
// per-row max, sum and draft-id logit) and the scan for the first rejection; the workgroup of the sequence's first
// segment writes the per-row outputs and the draw job. It then computes, per chunk of the draw's row(s), A = sum
// of e_t and D = sum of e_d over the elements where the residual is positive, with e = exp((z - max) / T) in
// float64, together with the exact normalisers S_t and S_d; a chunk's residual mass is then A / S_t - D / S_d.
// Whether p_i > q_i, i.e. e_t * (S_d / S_t) > e_d, is decided with the statistics pass's estimate of S_d / S_t,
// which is within 1e-5 of the exact ratio; an element within kBand of the boundary marks its chunk, and the pick
// recomputes that chunk exactly. The pick forms every chunk's mass, scans them in order, finds the chunk that
// holds t = u * (total mass) and searches it with one wave.

constexpr int kChunk = 1024;        // elements per chunk
constexpr int kPer = 16;            // elements per lane in a chunk
constexpr double kBand = 3.0e-5;    // relative width of the undecided zone of the residual's sign test
constexpr int kTile = 4096;         // chunks held in LDS at a time by the pick

struct DenseParams {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;     // dft == nullptr: one-hot drafts
  int64_t B; int32_t G; int64_t V; int32_t nseg1; int32_t bonus;
  float c;                                    // log2(e) / T, rounded to float (statistics pass)
  double invT;                                // 1 / T in float64 (draw)
  const int32_t* ids; const float* ua; const float* us;
  int32_t* start; const int32_t* order;
  uint8_t* accept; int32_t* n_acc; int32_t* token; float* p_draft; float* q_draft; uint32_t* flags;
  const Partial1* part1;
  Job* jobs;
  int32_t nseg2; int32_t cpw; int64_t nch;
  double4* part2a;     // per (b, seg): reference max m_seg, sum e_t (relative to m_seg), m_d, sum e_d
  struct ChunkRec* chunks;   // per (b, chunk), see ChunkRec
  double* masses;            // per (b, chunk): chunk masses, written by the pick when the chunks exceed one tile
};

// Combine the segment partials of one row: exact max m and S = sum 2^((z - m) * c) in float64; zx from segment 0.
__device__ __forceinline__ void row_stats(const Partial1* p, int nseg, double c, float& m, double& S, float& zx) {
  float mm = -INFINITY;
  for (int i = 0; i < nseg; ++i) mm = fmaxf(mm, p[i].m);
  double s = 0.0;
  bool nan = false;
  for (int i = 0; i < nseg; ++i) {
    nan |= isnan(p[i].s);
    if (p[i].m == mm) s += p[i].s;
    else if (p[i].m != -INFINITY) s += p[i].s * exp2((double(p[i].m) - double(mm)) * c);
  }
  m = mm;
  S = nan ? NAN : s;
  zx = p[0].zx;
}

struct SlotEval {
  float P, Q;
  bool acc, qzero, bad_id, nonfinite;
};

// 2^x for a float64 x, to float32 accuracy at any magnitude: the integer part is applied exactly with ldexp, only
// the fraction in [0, 1) goes through the hardware exp2.
__device__ __forceinline__ float exp2_split(double x) {
  if (!(x > -160.0)) return x != x ? NAN : 0.f;
  if (x > 130.0) return INFINITY;
  const double n = floor(x);
  return ldexpf(ex2f(float(x - n)), int(n));
}

// p(x), q(x) and the strict test u < min(1, p/q) of storage row r. The log-probabilities are assembled in float64
// from the row statistics; the hardware float32 log2/exp2 finish them (relative error ~1e-6 on the ratio and on
// p(x), q(x)).
__device__ __forceinline__ SlotEval eval_slot(const DenseParams& prm, int64_t b, int r) {
  SlotEval e{NAN, NAN, false, false, false, false};
  const int G = prm.G;
  const double c = double(prm.c);
  const int x = prm.ids[b * G + r];
  float mt, zt, md = 0.f, zd = 0.f;
  double St, Sd = 1.0;
  row_stats(prm.part1 + (b * G + r) * prm.nseg1, prm.nseg1, c, mt, St, zt);
  e.nonfinite = isnan(St) || mt == INFINITY || mt == -INFINITY;
  if (prm.dft) {
    row_stats(prm.part1 + ((prm.B + b) * G + r) * prm.nseg1, prm.nseg1, c, md, Sd, zd);
    e.nonfinite |= isnan(Sd) || md == INFINITY || md == -INFINITY;
  }
  if (x < 0 || int64_t(x) >= prm.V) {
    e.bad_id = true;
    return e;
  }
  const double lp = (double(zt) - double(mt)) * c - double(__builtin_amdgcn_logf(float(St)));   // log2 p(x)
  double lq = 0.0;                                                                              // one-hot: q(x) = 1
  if (prm.dft) {
    e.qzero = (zd == -INFINITY);
    lq = (double(zd) - double(md)) * c - double(__builtin_amdgcn_logf(float(Sd)));
  }
  e.P = exp2_split(lp);
  e.Q = prm.dft ? exp2_split(lq) : 1.f;
  float ratio = e.qzero ? 0.f : exp2_split(lp - lq);
  if (ratio != ratio) ratio = 0.f;
  e.acc = prm.ua[b * G + r] < fminf(1.f, ratio);
  return e;
}

__device__ __forceinline__ int wave_min_i(int v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

// Accept tests and first-rejection scan of sequence b by one wave (every wave of the sequence computes the same
// result). The leader wave writes the per-row outputs, n_accepted, flags, out_token = -1 and the job record; the
// new start is stored in the job and written by the pick, after every wave of this kernel has read the old one.
__device__ Job seq_scan(const DenseParams& prm, int64_t b, bool leader, uint32_t* seen) {
  const int lane = threadIdx.x & 63;
  const int G = prm.G;
  const int32_t* ord = prm.order ? prm.order + b * G : nullptr;
  const int st = prm.start ? prm.start[b] : 0;
  int bad = (st < 0 || st > G);
  if (ord) {                                      // order must be a permutation of 0 .. G-1
    for (int i = lane; i < (G + 31) / 32; i += 64) seen[i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int s = lane; s < G; s += 64) {
      const int r = ord[s];
      if (r < 0 || r >= G) {
        bad = 1;
      } else {
        const uint32_t bit = 1u << (r & 31);
        if (atomicOr(&seen[r >> 5], bit) & bit) bad = 1;
      }
    }
  }
  bad = __any(bad);
  const bool done = !bad && st == G;
  int bad_id = 0, nf = 0, qz = 0, kmin = G;
  if (!bad && !done) {
    for (int s = st + lane; s < G; s += 64) {
      const SlotEval e = eval_slot(prm, b, ord ? ord[s] : s);
      bad_id |= e.bad_id;
      nf |= e.nonfinite;
      qz |= e.qzero;
      if (!e.acc) kmin = min(kmin, s);
    }
  }
  bad_id = __any(bad_id);
  nf = __any(nf);
  qz = __any(qz);
  const int k = wave_min_i(kmin);
  const bool fatal = bad || bad_id || nf;
  uint32_t flg = (bad || bad_id ? SV_FLAG_ID_RANGE : 0u) | (nf ? SV_FLAG_NONFINITE : 0u);
  if (!fatal && qz) flg |= SV_FLAG_Q_ZERO;

  Job job{};
  job.kind = JOB_NONE;
  job.new_start = -1;
  if (!fatal && !done) {
    job.new_start = min(G, k + 1);
    if (k < G) {
      const int r = ord ? ord[k] : k;
      job.kind = prm.dft ? JOB_RESID : JOB_ONEHOT;
      job.row = r;
      job.d = prm.ids[b * G + r];
      job.u = prm.us[b * (G + 1) + r];
      double S_t, S_d = 1.0;
      float zx;
      row_stats(prm.part1 + (b * G + r) * prm.nseg1, prm.nseg1, double(prm.c), job.m_t, S_t, zx);
      if (prm.dft) row_stats(prm.part1 + ((prm.B + b) * G + r) * prm.nseg1, prm.nseg1, double(prm.c), job.m_d, S_d, zx);
      job.kappa = S_d / S_t;
    } else if (prm.bonus) {
      job.kind = JOB_BONUS;
      job.row = G;
      job.u = prm.us[b * (G + 1) + G];
    }
  }
  if (leader) {
    for (int s = lane; s < G; s += 64) {
      const int r = ord && !bad ? ord[s] : s;
      uint8_t a = 0;
      float P = 0.f, Q = 0.f;
      if (fatal) {
        P = Q = NAN;
      } else if (!done && s >= st) {
        const SlotEval e = eval_slot(prm, b, r);
        a = e.acc ? 1 : 0;
        P = e.P;
        Q = e.Q;
      }
      if (prm.accept) prm.accept[b * G + r] = a;
      if (prm.p_draft) prm.p_draft[b * G + r] = P;
      if (prm.q_draft) prm.q_draft[b * G + r] = Q;
    }
    if (lane == 0) {
      prm.n_acc[b] = fatal ? -1 : (done ? 0 : k - st);
      prm.token[b] = -1;
      if (prm.flags) prm.flags[b] = flg;
      prm.jobs[b] = job;
    }
  }
  return job;
}

// exp(x) in float64 by Tang's table-driven method (P. T. P. Tang, "Table-driven implementation of the exponential
// function in IEEE floating-point arithmetic", ACM TOMS 15(2), 1989): x = (64 e + j) ln2/64 + r with |r| <= ln2/128,
// exp(x) = 2^e * 2^(j/64) * (1 + expm1(r)), expm1(r) by its degree-5 Taylor polynomial (truncation < 4e-17).
// kExp2Tab[j] = 2^(j/64) correctly rounded; each workgroup copies it to LDS for the per-lane lookups.
__constant__ double kExp2Tab[64] = {
    0x1.0000000000000p+0, 0x1.02c9a3e778061p+0, 0x1.059b0d3158574p+0, 0x1.0874518759bc8p+0,
    0x1.0b5586cf9890fp+0, 0x1.0e3ec32d3d1a2p+0, 0x1.11301d0125b51p+0, 0x1.1429aaea92de0p+0,
    0x1.172b83c7d517bp+0, 0x1.1a35beb6fcb75p+0, 0x1.1d4873168b9aap+0, 0x1.2063b88628cd6p+0,
    0x1.2387a6e756238p+0, 0x1.26b4565e27cddp+0, 0x1.29e9df51fdee1p+0, 0x1.2d285a6e4030bp+0,
    0x1.306fe0a31b715p+0, 0x1.33c08b26416ffp+0, 0x1.371a7373aa9cbp+0, 0x1.3a7db34e59ff7p+0,
    0x1.3dea64c123422p+0, 0x1.4160a21f72e2ap+0, 0x1.44e086061892dp+0, 0x1.486a2b5c13cd0p+0,
    0x1.4bfdad5362a27p+0, 0x1.4f9b2769d2ca7p+0, 0x1.5342b569d4f82p+0, 0x1.56f4736b527dap+0,
    0x1.5ab07dd485429p+0, 0x1.5e76f15ad2148p+0, 0x1.6247eb03a5585p+0, 0x1.6623882552225p+0,
    0x1.6a09e667f3bcdp+0, 0x1.6dfb23c651a2fp+0, 0x1.71f75e8ec5f74p+0, 0x1.75feb564267c9p+0,
    0x1.7a11473eb0187p+0, 0x1.7e2f336cf4e62p+0, 0x1.82589994cce13p+0, 0x1.868d99b4492edp+0,
    0x1.8ace5422aa0dbp+0, 0x1.8f1ae99157736p+0, 0x1.93737b0cdc5e5p+0, 0x1.97d829fde4e50p+0,
    0x1.9c49182a3f090p+0, 0x1.a0c667b5de565p+0, 0x1.a5503b23e255dp+0, 0x1.a9e6b5579fdbfp+0,
    0x1.ae89f995ad3adp+0, 0x1.b33a2b84f15fbp+0, 0x1.b7f76f2fb5e47p+0, 0x1.bcc1e904bc1d2p+0,
    0x1.c199bdd85529cp+0, 0x1.c67f12e57d14bp+0, 0x1.cb720dcef9069p+0, 0x1.d072d4a07897cp+0,
    0x1.d5818dcfba487p+0, 0x1.da9e603db3285p+0, 0x1.dfc97337b9b5fp+0, 0x1.e502ee78b3ff6p+0,
    0x1.ea4afa2a490dap+0, 0x1.efa1bee615a27p+0, 0x1.f50765b6e4540p+0, 0x1.fa7c1819e90d8p+0,
};

__device__ __forceinline__ void exp_table_init(double* tab) {
  if (threadIdx.x < 64) tab[threadIdx.x] = kExp2Tab[threadIdx.x];
  __syncthreads();
}

// exp(d * invT) for d = z - max <= 0. kC = invT * 64/ln2. The nearest integer k of d * kC comes from adding
// 1.5 * 2^52 (its low mantissa bits then hold k); r = d * invT - k * ln2/64 is formed with one rounding because
// k * L1 is exact (L1 keeps 36 bits, |k| < 2^17). Inputs at or below -746 (after scaling), -inf and NaN are
// evaluated on garbage and replaced at the end by 0 (NaN stays NaN).
struct ExpArg {
  double invT, kC;
};

// Core of the evaluation, valid for finite d with d * invT >= -745 (no special-value handling).
__device__ __forceinline__ double fexp_core(double d, const ExpArg& ea, const double* tab) {
  const double kMagic = 6755399441055744.0;                     // 1.5 * 2^52
  const double y = fma(d, ea.kC, kMagic);
  const int k = int(__double2loint(y));
  const double kd = y - kMagic;
  double r = fma(d, ea.invT, -kd * 0x1.62e42fefa0000p-7);
  r = fma(-kd, 0x1.cf79abc9e3b3ap-46, r);
  double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  q = fma(q, r, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  const double em1 = q * r;
  const double t = tab[k & 63];
  return ldexp(fma(t, em1, t), k >> 6);
}

__device__ __forceinline__ double fexp_scaled(double d, const ExpArg& ea, const double* tab) {
  const double kMagic = 6755399441055744.0;                     // 1.5 * 2^52
  const double y = fma(d, ea.kC, kMagic);
  const int k = int(__double2loint(y));
  const double kd = y - kMagic;
  double r = fma(d, ea.invT, -kd * 0x1.62e42fefa0000p-7);       // ln2/64, leading 36 bits (product exact)
  r = fma(-kd, 0x1.cf79abc9e3b3ap-46, r);                       // ln2/64, remainder
  double q = fma(r, 1.0 / 120.0, 1.0 / 24.0);
  q = fma(q, r, 1.0 / 6.0);
  q = fma(q, r, 0.5);
  q = fma(q, r, 1.0);
  const double em1 = q * r;
  const double t = tab[k & 63];
  const double res = ldexp(fma(t, em1, t), k >> 6);
  const double x = d * ea.invT;
  return (x >= -746.0) ? res : (x != x ? x : 0.0);
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_incl_scan(double v, int lane) {
  for (int o = 1; o < 64; o <<= 1) {
    const double n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  return v;
}

template <int BLOCK>
__device__ __forceinline__ double block_max_d(double v, double* sh) {
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) sh[w] = v;
  __syncthreads();
  double r = sh[0];
#pragma unroll
  for (int i = 1; i < BLOCK / 64; ++i) r = fmax(r, sh[i]);
  return r;
}

// Exclusive scan of doubles over the block in thread order; also returns the total.
template <int BLOCK>
__device__ __forceinline__ double block_excl_scan(double v, double* sh, double& total) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double incl = wave_incl_scan(v, l);
  __syncthreads();
  if (l == 63) sh[w] = incl;
  __syncthreads();
  double base = 0.0, tot = 0.0;
#pragma unroll
  for (int i = 0; i < BLOCK / 64; ++i) {
    if (i < w) base += sh[i];
    tot += sh[i];
  }
  total = tot;
  return base + incl - v;
}

// 16 consecutive logits starting at element i0 of a row, as float; -inf past the end of the row.
template <typename T>
__device__ __forceinline__ void load16(const T* row, int64_t i0, int64_t V, bool vec, float* z) {
  if (vec && i0 + kPer <= V) {
    const uint4* p = reinterpret_cast<const uint4*>(row + i0);
    constexpr int NV = kPer / Vec<T>::kEPV;
#pragma unroll
    for (int k = 0; k < NV; ++k) Vec<T>::unpack(p[k], z + k * Vec<T>::kEPV);
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) z[e] = (i0 + e < V) ? Vec<T>::load1(row + i0 + e) : -INFINITY;
  }
}

// Exact draw weights of the lane's 16 elements of chunk c (relative to the common reference max mt): the residual
// max(p_i - q_i, 0), or p_i when use_p. Compiled without contraction so repeated evaluations agree bit for bit.
template <typename T>
__device__ __forceinline__ void chunk_weights(const Job& job, const T* rt, const T* rd, bool vec, int64_t c, int lane,
                                              int64_t V, double mt, double inv_st, double md, double inv_sd,
                                              double invT, bool use_p, const double* tab, double* w) {
#pragma clang fp contract(off)
  const int64_t i0 = c * kChunk + int64_t(lane) * kPer;
  float zt[kPer], zd[kPer];
  load16<T>(rt, i0, V, vec, zt);
  const bool resid = job.kind == JOB_RESID && !use_p;
  if (resid) load16<T>(rd, i0, V, vec, zd);
  const ExpArg ea{invT, invT * 92.332482616893656};
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const double p = fexp_scaled(double(zt[e]) - mt, ea, tab) * inv_st;
    double q = 0.0;
    if (resid) q = fexp_scaled(double(zd[e]) - md, ea, tab) * inv_sd;
    else if (!use_p && job.kind == JOB_ONEHOT) q = (i0 + e == job.d) ? 1.0 : 0.0;
    const double r = use_p ? p : p - q;
    w[e] = r > 0.0 ? r : 0.0;
  }
}

__device__ __forceinline__ double lane_sum16(const double* w) {
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) s += w[e];
  return s;
}

// Per-chunk record of the mass pass. A = sum of e_t and D = sum of e_d over the elements whose residual is positive;
// up to kAmbMax elements whose sign could not be decided are kept as (e_t, e_d) pairs (n_amb of them); n_amb > kAmbMax
// means the chunk must be recomputed from the logits.
constexpr int kAmbMax = 4;
struct alignas(16) ChunkRec {
  double A, D;
  int32_t n_amb, pad0;
  double pad1;
  double et[kAmbMax], ed[kAmbMax];
};

// Elements of the lane: all finite and within exp's range of the reference max (so the guard-free core applies).
__device__ __forceinline__ bool lane_safe(const float* z, double m, double invT) {
  float lo = z[0], hi = z[0];
#pragma unroll
  for (int e = 1; e < kPer; ++e) { lo = fminf(lo, z[e]); hi = fmaxf(hi, z[e]); }
  // NaN makes both comparisons false; +inf fails the upper bound check; -inf fails the lower one
  return (double(lo) - m) * invT >= -740.0 && double(hi) <= m && hi == hi && lo == lo;
}

// One lane's 16 elements: exp of both logits, the residual's sign test and the sums.
template <int KIND, bool SAFE>
__device__ __forceinline__ void mass_lane(const float* zt, const float* zd, double mt, double md, int64_t i0, int32_t d,
                                          const ExpArg& ea, const double* tab, double k_lo, double k_hi, double& st,
                                          double& sd, double& A, double& D, uint32_t& amb) {
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const double et = SAFE ? fexp_core(double(zt[e]) - mt, ea, tab) : fexp_scaled(double(zt[e]) - mt, ea, tab);
    st += et;
    if constexpr (KIND == JOB_RESID) {
      const double ed = SAFE ? fexp_core(double(zd[e]) - md, ea, tab) : fexp_scaled(double(zd[e]) - md, ea, tab);
      sd += ed;
      // r_e > 0 iff et * (S_d / S_t) > ed; kappa brackets S_d / S_t within kBand
      const bool pos = et * k_lo > ed;
      const bool neg = et * k_hi <= ed;
      A += pos ? et : 0.0;
      D += pos ? ed : 0.0;
      amb |= (!(pos || neg) ? 1u : 0u) << e;
    } else if constexpr (KIND == JOB_ONEHOT) {
      A += (i0 + e == d) ? 0.0 : et;
    } else {
      A += et;
    }
  }
}

// Chunk loop of the mass pass for one kind of draw (KIND is uniform per sequence).
template <typename T, int KIND>
__device__ __forceinline__ void mass_chunks(const DenseParams& prm, const Job& job, int64_t b, int64_t c0, int64_t c1,
                                            const T* rt, const T* rd, bool vec, double mt, const double* tab,
                                            double& st, double& sd) {
  const int lane = threadIdx.x;
  const int64_t V = prm.V;
  const double md = job.m_d;
  const ExpArg ea{prm.invT, prm.invT * 92.332482616893656};
  const double k_lo = job.kappa * (1.0 - kBand), k_hi = job.kappa * (1.0 + kBand);
  float zt[kPer], zd[kPer];
  for (int64_t c = c0; c < c1; ++c) {
    const int64_t i0 = c * kChunk + int64_t(lane) * kPer;
    load16<T>(rt, i0, V, vec, zt);
    if constexpr (KIND == JOB_RESID) load16<T>(rd, i0, V, vec, zd);
    bool safe = i0 + kPer <= V && lane_safe(zt, mt, prm.invT);
    if constexpr (KIND == JOB_RESID) safe = safe && lane_safe(zd, md, prm.invT);
    safe = __all(safe);
    double A = 0.0, D = 0.0;
    uint32_t amb = 0;                                  // bit e: element e undecided
    if (safe)
      mass_lane<KIND, true>(zt, zd, mt, md, i0, job.d, ea, tab, k_lo, k_hi, st, sd, A, D, amb);
    else
      mass_lane<KIND, false>(zt, zd, mt, md, i0, job.d, ea, tab, k_lo, k_hi, st, sd, A, D, amb);
    A = wave_sum(A);
    if constexpr (KIND == JOB_RESID) D = wave_sum(D);
    ChunkRec* rec = prm.chunks + b * prm.nch + c;
    int namb = 0;
    if constexpr (KIND == JOB_RESID) {
      if (__any(amb != 0)) {                           // rare: list the undecided elements in element order
        const int mine = __popc(amb);
        int before = mine;                             // inclusive prefix over lanes
        for (int o = 1; o < 64; o <<= 1) {
          const int n = __shfl_up(before, o);
          if (lane >= o) before += n;
        }
        namb = __shfl(before, 63);
        int pos = before - mine;
        for (int e = 0; e < kPer; ++e) {
          if ((amb >> e) & 1u) {                       // recomputed exactly as in mass_lane
            if (pos < kAmbMax) {
              rec->et[pos] = fexp_scaled(double(zt[e]) - mt, ea, tab);
              rec->ed[pos] = fexp_scaled(double(zd[e]) - md, ea, tab);
            }
            ++pos;
          }
        }
      }
    }
    if (lane == 0) {
      rec->A = A;
      rec->D = D;
      rec->n_amb = namb;
    }
  }
}

// One wave per workgroup; each workgroup handles cpw consecutive chunks of one sequence's draw row(s), after the
// sequence's scan.
template <typename T>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_draw_mass(DenseParams prm) {
  __shared__ double tab[64];
  __shared__ uint32_t seen[SV_MAX_GAMMA / 32];
  const int seg = int(blockIdx.x % prm.nseg2);
  const int64_t b = blockIdx.x / prm.nseg2;
  exp_table_init(tab);
  const Job job = seq_scan(prm, b, seg == 0, seen);
  if (job.kind == JOB_NONE) return;
  const int lane = threadIdx.x;
  const int64_t V = prm.V;
  const int64_t c0 = int64_t(seg) * prm.cpw, c1 = min<int64_t>(prm.nch, c0 + prm.cpw);
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const bool resid = job.kind == JOB_RESID;
  const T* rd = resid ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(rt) & 15u) == 0 &&
                   (!resid || (reinterpret_cast<uintptr_t>(rd) & 15u) == 0);

  double mt = job.m_t;
  int has_nan = 0;
  if (job.kind == JOB_BONUS) {            // the bonus row was not in the statistics pass: this segment's max
    float zt[kPer];
    float m = -INFINITY;
    for (int64_t c = c0; c < c1; ++c) {
      load16<T>(rt, c * kChunk + int64_t(lane) * kPer, V, vec, zt);
#pragma unroll
      for (int e = 0; e < kPer; ++e) { m = fmaxf(m, zt[e]); has_nan |= (zt[e] != zt[e]); }
    }
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    mt = m;
    has_nan = __any(has_nan);
  }
  double st = 0.0, sd = 0.0;
  if (mt == -INFINITY) {                  // a segment of -inf only (bonus row): no mass
    for (int64_t c = c0 + lane; c < c1; c += 64) {
      prm.chunks[b * prm.nch + c].A = 0.0;
      prm.chunks[b * prm.nch + c].D = 0.0;
      prm.chunks[b * prm.nch + c].n_amb = 0;
    }
  } else if (job.kind == JOB_RESID) {
    mass_chunks<T, JOB_RESID>(prm, job, b, c0, c1, rt, rd, vec, mt, tab, st, sd);
  } else if (job.kind == JOB_ONEHOT) {
    mass_chunks<T, JOB_ONEHOT>(prm, job, b, c0, c1, rt, rd, vec, mt, tab, st, sd);
  } else {
    mass_chunks<T, JOB_BONUS>(prm, job, b, c0, c1, rt, rd, vec, mt, tab, st, sd);
  }
  st = wave_sum(st);
  if (resid) sd = wave_sum(sd);
  if (lane == 0) prm.part2a[b * prm.nseg2 + seg] = make_double4(mt, has_nan ? NAN : st, job.m_d, sd);
}

template <typename T, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_draw_pick(DenseParams prm) {
  constexpr int NW = BLOCK / 64;
  __shared__ double tab[64];
  __shared__ double sh_d[NW];
  __shared__ double s_mass[kTile];
  __shared__ int s_amb[kTile];
  __shared__ int s_namb, s_cand, s_last;
  __shared__ double s_base;
  const int64_t b = blockIdx.x;
  const Job job = prm.jobs[b];
  if (prm.start && job.new_start >= 0 && threadIdx.x == 0) prm.start[b] = job.new_start;
  if (job.kind == JOB_NONE) return;
  exp_table_init(tab);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nseg = prm.nseg2;
  const int64_t nch = prm.nch, V = prm.V;
  const ChunkRec* ch = prm.chunks + b * nch;
  double* mg = prm.masses + b * nch;
  const double4* ps = prm.part2a + b * nseg;
  const double invT = prm.invT;
  const bool resid = job.kind == JOB_RESID, bonus = job.kind == JOB_BONUS;
  const ExpArg eaP{invT, invT * 92.332482616893656};

  // normalisers from the segment partials, combined in a fixed order
  double lm = -INFINITY;
  int bad = 0;
  for (int s = tid; s < nseg; s += BLOCK) {
    const double4 p = ps[s];
    lm = fmax(lm, p.x);
    bad |= isnan(p.y) || isnan(p.w);
  }
  const double mt = block_max_d<BLOCK>(lm, sh_d);
  bad = __syncthreads_or(bad);
  double lst = 0.0, lsd = 0.0;
  for (int s = tid; s < nseg; s += BLOCK) {
    const double4 p = ps[s];
    const double f = (!bonus || p.x == mt) ? 1.0 : (p.x == -INFINITY ? 0.0 : fexp_scaled(p.x - mt, eaP, tab));
    lst += p.y * f;
    lsd += p.w;
  }
  const double St = block_sum<BLOCK>(lst, sh_d);
  const double Sd = block_sum<BLOCK>(lsd, sh_d);
  if (bad || !(St > 0.0) || isinf(mt) || (resid && !(Sd > 0.0))) {    // only a bonus row can be bad here
    if (tid == 0) {
      prm.token[b] = -1;
      if (prm.flags) prm.flags[b] |= SV_FLAG_NONFINITE;
    }
    return;
  }
  const double inv_st = 1.0 / St, inv_sd = resid ? 1.0 / Sd : 0.0;
  const double md = job.m_d;
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const T* rd = resid ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(rt) & 15u) == 0 &&
                   (!resid || (reinterpret_cast<uintptr_t>(rd) & 15u) == 0);
  const bool one_tile = nch <= kTile;
  double w[kPer];

  // Masses of the chunks of one tile into s_mass (and back to global memory when there are several tiles).
  auto tile_masses = [&](int64_t t0, int n, bool use_p) {
    if (tid == 0) s_namb = 0;
    __syncthreads();
    for (int i = tid; i < n; i += BLOCK) {
      const int64_t c = t0 + i;
      const ChunkRec& rc = ch[c];
      const int namb = rc.n_amb;
      if (use_p || namb > kAmbMax) {
        s_amb[atomicAdd(&s_namb, 1)] = i;
      } else {
        const double f = bonus ? fexp_scaled(ps[c / prm.cpw].x - mt, eaP, tab) : 1.0;
        double m = f * (rc.A * inv_st - rc.D * inv_sd);
        for (int q = 0; q < namb; ++q) {               // undecided elements, exactly: max(p - q, 0)
          const double r = rc.et[q] * inv_st - rc.ed[q] * inv_sd;
          m += r > 0.0 ? r : 0.0;
        }
        s_mass[i] = m;
      }
    }
    __syncthreads();
    const int namb = s_namb;
    for (int q = wave; q < namb; q += NW) {
      const int i = s_amb[q];
      chunk_weights<T>(job, rt, rd, vec, t0 + i, lane, V, mt, inv_st, md, inv_sd, invT, use_p, tab, w);
      const double m = wave_sum(lane_sum16(w));
      if (lane == 0) s_mass[i] = m;
    }
    __syncthreads();
    if (!one_tile)
      for (int i = tid; i < n; i += BLOCK) mg[t0 + i] = s_mass[i];
  };
  // Running sum over one tile: thread-contiguous ranges, exclusive base per thread, tile total.
  auto tile_scan = [&](int n, double& mine_excl, int& ia, int& ib) {
    const int per = (n + BLOCK - 1) / BLOCK;
    ia = min(n, per * tid);
    ib = min(n, per * (tid + 1));
    double mine = 0.0;
    for (int i = ia; i < ib; ++i) mine += s_mass[i];
    double tot;
    mine_excl = block_excl_scan<BLOCK>(mine, sh_d, tot);
    return tot;
  };

  bool use_p = false;
  double total = 0.0, excl = 0.0;
  int ia = 0, ib = 0;
  for (int pass = 0; pass < 2; ++pass) {
    total = 0.0;
    for (int64_t t0 = 0; t0 < nch; t0 += kTile) {
      const int n = int(min<int64_t>(kTile, nch - t0));
      tile_masses(t0, n, use_p);
      total += tile_scan(n, excl, ia, ib);
    }
    if (total > 0.0) break;
    use_p = true;                                         // empty residual: draw from p instead
  }
  const double t = double(job.u) * total;

  // Locate the chunk whose running sum first exceeds t (else the last chunk with mass).
  if (tid == 0) { s_cand = INT_MAX; s_last = -1; }
  __syncthreads();
  double run = 0.0;
  for (int64_t t0 = 0; t0 < nch; t0 += kTile) {
    const int n = int(min<int64_t>(kTile, nch - t0));
    double tile_total = 0.0;
    if (!one_tile) {
      __threadfence_block();
      __syncthreads();
      for (int i = tid; i < n; i += BLOCK) s_mass[i] = *reinterpret_cast<const volatile double*>(&mg[t0 + i]);
      __syncthreads();
      tile_total = tile_scan(n, excl, ia, ib);
    }
    double acc = run + excl;
    int cand = INT_MAX, last = -1;
    double cbase = 0.0;
    for (int i = ia; i < ib; ++i) {
      const double m = s_mass[i];
      if (m > 0.0) last = int(t0 + i);
      if (cand == INT_MAX && acc + m > t) { cand = int(t0 + i); cbase = acc; }
      acc += m;
    }
    atomicMin(&s_cand, cand);
    atomicMax(&s_last, last);
    __syncthreads();
    if (cand != INT_MAX && cand == s_cand) s_base = cbase;
    __syncthreads();
    if (s_cand != INT_MAX) break;
    run += tile_total;
  }
  const bool clamp = s_cand == INT_MAX;
  const int64_t cstar = clamp ? s_last : s_cand;
  if (wave != 0) return;
  if (cstar < 0) {
    if (lane == 0) prm.token[b] = -1;
    return;
  }
  // exact search inside the chunk, one wave
  chunk_weights<T>(job, rt, rd, vec, cstar, lane, V, mt, inv_st, md, inv_sd, invT, use_p, tab, w);
  const double lsum = lane_sum16(w);
  const double incl = wave_incl_scan(lsum, lane);
  double acc = (clamp ? 0.0 : s_base) + (incl - lsum);
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    acc += w[e];
    if (w[e] > 0.0) lastpos = e;
    if (hit < 0 && !clamp && w[e] > 0.0 && acc > t) hit = e;
  }
  const uint64_t hm = __ballot(hit >= 0);
  const uint64_t pm = __ballot(lastpos >= 0);
  int64_t tok = -1;
  if (hm) {
    const int l = __builtin_ctzll(hm);
    tok = cstar * kChunk + int64_t(l) * kPer + __shfl(hit, l);
  } else if (pm) {
    const int l = 63 - __builtin_clzll(pm);
    tok = cstar * kChunk + int64_t(l) * kPer + __shfl(lastpos, l);
  }
  if (lane == 0) {
    prm.token[b] = int32_t(tok);
    if (use_p && prm.flags) prm.flags[b] |= SV_FLAG_EMPTY_RESIDUAL;
  }
}

// Workgroups of the statistics pass: every work item, capped at kStatsWgPerCu per compute unit (the kernel then
// loops over items).
int64_t stats_grid(int64_t items) {
  int dev = 0, ncu = 0;
  if (kStatsWgPerCu <= 0 || hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0)
    return items;
  const int64_t cap = int64_t(ncu) * kStatsWgPerCu;
  return items < cap ? items : cap;
}

template <typename T>
hipError_t launch_typed(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  char* ws = a.ws;
  Partial1* part1 = reinterpret_cast<Partial1*>(ws + plan.off_part1);
  Job* jobs = reinterpret_cast<Job*>(ws + plan.off_jobs);
  double4* part2a = reinterpret_cast<double4*>(ws + plan.off_part2a);
  ChunkRec* chunks = reinterpret_cast<ChunkRec*>(ws + plan.off_chunks);
  double* masses = reinterpret_cast<double*>(ws + plan.off_masses);
  const double T_ = double(a.temperature);
  const float c = float(1.4426950408889634074 / T_);          // log2(e) / T

  StatsParams sp{a.tgt, a.t_seq, a.t_row, a.dft, a.d_seq, a.d_row, plan.B, plan.G, plan.V, plan.nseg1, plan.ntens,
                 c, a.start, a.order, a.ids, part1};
  const int64_t g1 = int64_t(plan.ntens) * plan.B * plan.G * plan.nseg1;
  const int64_t grid1 = stats_grid(g1);
  if (a.ev_start) {      // events taken from the dispatch packet itself: no marker packets around the kernel
    hipExtLaunchKernelGGL((k_stats<T, kStatsBlock, kUnroll, kNonTemporal, kStatsWpe>), dim3(unsigned(grid1)),
                          dim3(kStatsBlock), 0, stream, static_cast<hipEvent_t>(a.ev_start),
                          static_cast<hipEvent_t>(a.ev_stop), 0, sp);
  } else {
    hipLaunchKernelGGL((k_stats<T, kStatsBlock, kUnroll, kNonTemporal, kStatsWpe>), dim3(unsigned(grid1)),
                       dim3(kStatsBlock), 0, stream, sp);
  }

  DenseParams dp{a.tgt, a.t_seq, a.t_row, a.dft, a.d_seq, a.d_row, plan.B, plan.G, plan.V, plan.nseg1, a.bonus, c,
                 1.0 / T_, a.ids, a.ua, a.us, a.start, a.order, a.accept, a.n_acc, a.token, a.p_draft, a.q_draft,
                 a.flags, part1, jobs, plan.nseg2, plan.cpw, plan.nch, part2a, chunks, masses};
  const int64_t g2 = plan.B * plan.nseg2;
  hipLaunchKernelGGL((k_draw_mass<T>), dim3(unsigned(g2)), dim3(64), 0, stream, dp);
  hipLaunchKernelGGL((k_draw_pick<T, kDrawBlock>), dim3(unsigned(plan.B)), dim3(kDrawBlock), 0, stream, dp);
  return hipGetLastError();
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

DensePlan make_dense_plan(int64_t B, int32_t G, int64_t V, int32_t ntens) {
  DensePlan p;
  p.B = B; p.G = G; p.V = V; p.ntens = ntens;
  const int64_t rows = int64_t(ntens) * B * G;
  // statistics pass: aim for >= 2048 workgroups (8 per CU on 256 CUs), segments of >= 8192 elements
  int64_t s1 = (2048 + rows - 1) / rows;
  const int64_t cap1 = V / 8192 > 1 ? V / 8192 : 1;
  if (s1 > cap1) s1 = cap1;
  if (s1 < 1) s1 = 1;
  p.nseg1 = int32_t(s1);
  // draw pass: rows cut into chunks of kChunk elements; one-wave workgroups of cpw chunks each, cpw chosen so that
  // the B row pairs give about 8192 workgroups
  p.nch = (V + kChunk - 1) / kChunk;
  int64_t cpw = (int64_t(B) * p.nch + 8191) / 8192;
  if (cpw < 1) cpw = 1;
  if (cpw > 64) cpw = 64;
  p.cpw = int32_t(cpw);
  p.nseg2 = int32_t((p.nch + cpw - 1) / cpw);
  size_t off = 0;
  p.off_part1 = off; off = align_up(off + size_t(rows) * p.nseg1 * sizeof(Partial1), 256);
  p.off_jobs = off;  off = align_up(off + size_t(B) * sizeof(Job), 256);
  p.off_part2a = off; off = align_up(off + size_t(B) * p.nseg2 * sizeof(double4), 256);
  p.off_chunks = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(ChunkRec), 256);
  p.off_masses = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(double), 256);
  p.total = off;
  return p;
}

hipError_t launch_dense(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  if (a.dtype == SV_BF16) return launch_typed<uint16_t>(plan, a, stream);
  return launch_typed<float>(plan, a, stream);
}

}  // namespace sv
