// Dense and one-hot speculative-sampling verification for gfx950 (MI355X).
//
// The rule is Leviathan et al.'s, as restated on "Uno: the draft model was already inside the target model"
// (section "What 'lossless' actually has to mean"): accept a draft x with probability min(1, p(x)/q(x)), cut the
// block at the first rejection (DFlash/DFlash2 guide, section 4.4) and draw the replacement from max(p - q, 0)
// renormalised there, or a bonus token from the next target row when every draft is accepted (same guide,
// section 2). p and q are softmaxes of the logits divided by the temperature (same guide, section 9 Q3).
//
// Four launches, all on the caller's stream:
//  1. k_stats   : one read of every verified logit row. Per (row, segment) it keeps a running max and a running sum
//                 of exp2((z - max) * log2(e)/T) in float32, folds the threads together in float64 and writes
//                 (max, sum). 16-byte loads, -inf padding instead of bounds checks in the hot loop. This pass
//                 moves almost all the bytes; it is bound by HBM bandwidth.
//  2. k_scan    : one workgroup per sequence. Combines the segment partials in a fixed order (float64), evaluates
//                 p(x), q(x) and the strict test u < min(1, p/q) for every verified slot, finds the first
//                 rejection from `start` along `order`, writes the per-row outputs and one draw job per sequence.
//  3. k_draw_stats + k_draw_mass + k_draw_pick : only for the row(s) a draw needs (at most one row pair per
//                 sequence). Float64 throughout: exact softmax normalisers, the residual's mass per segment, then
//                 a search inside the one segment that holds t = u * (total mass).
// The float64 draw pass exists because a token boundary of the residual CDF often lies within 1e-7 of t at these
// vocabulary sizes; float32 sums would pick a neighbouring token far more often than the float64 reference does.

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
constexpr int kScanBlock = 256;
constexpr int kDrawBlock = 256;

struct alignas(16) Partial1 {
  float m;        // exact max of the segment's logits (raw, before the temperature)
  float pad;
  double s;       // sum over the segment of 2^((z - m) * c), c = log2(e)/T rounded to float
};

// ----------------------------------------------------------------------------------------------------------------
// element access
// ----------------------------------------------------------------------------------------------------------------

template <typename T> struct Vec;
template <> struct Vec<float> {
  static constexpr int kEPV = 4;                                  // elements per 16-byte vector
  static constexpr uint32_t kNegInf = 0xFF800000u;                // pattern of -inf
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
    v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
  }
  __device__ static __forceinline__ float load1(const float* p) { return *p; }
};
template <> struct Vec<uint16_t> {
  static constexpr int kEPV = 8;
  static constexpr uint32_t kNegInf = 0xFF80FF80u;                // two bf16 -inf
  __device__ static __forceinline__ void unpack(const uint4& w, float* v) {
    v[0] = __uint_as_float(w.x << 16); v[1] = __uint_as_float(w.x & 0xFFFF0000u);
    v[2] = __uint_as_float(w.y << 16); v[3] = __uint_as_float(w.y & 0xFFFF0000u);
    v[4] = __uint_as_float(w.z << 16); v[5] = __uint_as_float(w.z & 0xFFFF0000u);
    v[6] = __uint_as_float(w.w << 16); v[7] = __uint_as_float(w.w & 0xFFFF0000u);
  }
  __device__ static __forceinline__ float load1(const uint16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }
};

__device__ __forceinline__ float ex2f(float x) { return __builtin_amdgcn_exp2f(x); }

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

template <typename T, int BLOCK, int U>
__global__ __launch_bounds__(BLOCK) void k_stats(StatsParams prm) {
  using VT = Vec<T>;
  constexpr int EPV = VT::kEPV;
  __shared__ float sh_f[BLOCK / 64];
  __shared__ double sh_d[BLOCK / 64];

  int64_t w = blockIdx.x;
  const int seg = int(w % prm.nseg); w /= prm.nseg;
  const int row = int(w % prm.G);    w /= prm.G;
  const int64_t b = w % prm.B;
  const int tens = int(w / prm.B);

  if (prm.start) {                                   // rows of slots before start are not read
    const int st = prm.start[b];
    if (st < 0 || st > prm.G) return;                // reported by the scan
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

  const uint4* vp = reinterpret_cast<const uint4*>(base + head);
  const uint4 pad = make_uint4(VT::kNegInf, VT::kNegInf, VT::kNegInf, VT::kNegInf);
  uint4 cur[U], nxt[U];
  int64_t v = v0 + threadIdx.x;
#pragma unroll
  for (int k = 0; k < U; ++k) cur[k] = (v + int64_t(k) * BLOCK < v1) ? vp[v + int64_t(k) * BLOCK] : pad;
  for (; v < v1; v += int64_t(U) * BLOCK) {
    const int64_t vn = v + int64_t(U) * BLOCK;
#pragma unroll
    for (int k = 0; k < U; ++k) nxt[k] = (vn + int64_t(k) * BLOCK < v1) ? vp[vn + int64_t(k) * BLOCK] : pad;
    float z[U * EPV];
#pragma unroll
    for (int k = 0; k < U; ++k) VT::unpack(cur[k], z + k * EPV);
    absorb<U * EPV>(st, z, c);
#pragma unroll
    for (int k = 0; k < U; ++k) cur[k] = nxt[k];
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
    out.pad = 0.f;
    out.s = s;
    prm.part[((int64_t(tens) * prm.B + b) * prm.G + row) * prm.nseg + seg] = out;
  }
}

// ----------------------------------------------------------------------------------------------------------------
// 2. accept test and first-reject scan
// ----------------------------------------------------------------------------------------------------------------

struct ScanParams {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;
  int64_t B; int32_t G; int64_t V; int32_t nseg; int32_t bonus;
  float c;
  const int32_t* ids; const float* ua; const float* us;
  int32_t* start; const int32_t* order;
  uint8_t* accept; int32_t* n_acc; int32_t* token; float* p_draft; float* q_draft; uint32_t* flags;
  const Partial1* part;
  Job* jobs;
};

template <typename T>
__device__ __forceinline__ float load_elem(const void* base, int64_t off) {
  return Vec<T>::load1(static_cast<const T*>(base) + off);
}

// Combine the segment partials of one row: exact max m and S = sum 2^((z - m) * c) in float64.
__device__ __forceinline__ void row_stats(const Partial1* p, int nseg, double c, float& m, double& S) {
  float mm = -INFINITY;
  for (int i = 0; i < nseg; ++i) mm = fmaxf(mm, p[i].m);
  double s = 0.0;
  bool nan = false;
  for (int i = 0; i < nseg; ++i) {
    nan |= isnan(p[i].s);
    if (p[i].m != -INFINITY) s += p[i].s * exp2((double(p[i].m) - double(mm)) * c);
  }
  m = mm;
  S = nan ? NAN : s;
}

template <typename T, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_scan(ScanParams prm) {
  __shared__ uint8_t s_acc[SV_MAX_GAMMA];
  __shared__ int32_t s_slot[SV_MAX_GAMMA];     // slot of each storage row (inverse of order)
  __shared__ float s_p[SV_MAX_GAMMA];
  __shared__ float s_q[SV_MAX_GAMMA];
  __shared__ int s_k;

  const int64_t b = blockIdx.x;
  const int G = prm.G;
  const int tid = threadIdx.x;
  const int32_t* ord = prm.order ? prm.order + b * G : nullptr;
  const int st = prm.start ? prm.start[b] : 0;

  // argument checks that make the sequence unverifiable
  int bad = (st < 0 || st > G);
  for (int r = tid; r < G; r += BLOCK) s_slot[r] = ord ? -1 : r;
  if (tid == 0) s_k = G;
  __syncthreads();
  if (ord) {
    for (int s = tid; s < G; s += BLOCK) {
      const int r = ord[s];
      if (r < 0 || r >= G) bad = 1;
      else if (atomicCAS(&s_slot[r], -1, s) != -1) bad = 1;   // a repeated row
    }
  }
  bad = __syncthreads_or(bad);
  uint32_t flg = 0;
  bool fatal = bad != 0;
  if (bad) flg |= SV_FLAG_ID_RANGE;

  const bool done = !fatal && st == G;
  const double c = double(prm.c);
  int local_bad_id = 0, local_nf = 0, local_qz = 0;
  if (!fatal && !done) {
    for (int s = st + tid; s < G; s += BLOCK) {
      const int r = ord ? ord[s] : s;
      const int x = prm.ids[b * G + r];
      const Partial1* pt = prm.part + (b * G + r) * prm.nseg;
      float mt; double St;
      row_stats(pt, prm.nseg, c, mt, St);
      if (isnan(St) || mt == INFINITY || mt == -INFINITY) local_nf = 1;
      float md = 0.f; double Sd = 1.0;
      if (prm.dft) {
        const Partial1* pd = prm.part + ((prm.B + b) * G + r) * prm.nseg;
        row_stats(pd, prm.nseg, c, md, Sd);
        if (isnan(Sd) || md == INFINITY || md == -INFINITY) local_nf = 1;
      }
      float P = NAN, Q = NAN;
      uint8_t acc = 0;
      if (x < 0 || int64_t(x) >= prm.V) {
        local_bad_id = 1;
      } else {
        const float zt = load_elem<T>(prm.tgt, b * prm.t_seq + int64_t(r) * prm.t_row + x);
        const double lp = (double(zt) - double(mt)) * c - log2(St);        // log2 p(x)
        double lq = 0.0;                                                    // one-hot: q(x) = 1
        bool qzero = false;
        if (prm.dft) {
          const float zd = load_elem<T>(prm.dft, b * prm.d_seq + int64_t(r) * prm.d_row + x);
          qzero = (zd == -INFINITY);
          lq = (double(zd) - double(md)) * c - log2(Sd);
        }
        P = float(exp2(lp));
        Q = prm.dft ? float(exp2(lq)) : 1.f;
        double ratio = qzero ? 0.0 : exp2(lp - lq);
        if (isnan(ratio)) ratio = 0.0;
        acc = double(prm.ua[b * G + r]) < fmin(1.0, ratio) ? 1 : 0;
        local_qz |= qzero;
      }
      s_acc[s] = acc;
      s_p[s] = P;
      s_q[s] = Q;
    }
  }
  const int any_id = __syncthreads_or(local_bad_id);
  const int any_nf = __syncthreads_or(local_nf);
  const int any_qz = __syncthreads_or(local_qz);
  if (any_id) flg |= SV_FLAG_ID_RANGE;
  if (any_nf) flg |= SV_FLAG_NONFINITE;
  fatal = fatal || any_id || any_nf;
  if (!fatal && any_qz) flg |= SV_FLAG_Q_ZERO;

  if (fatal) {
    for (int r = tid; r < G; r += BLOCK) {
      if (prm.accept) prm.accept[b * G + r] = 0;
      if (prm.p_draft) prm.p_draft[b * G + r] = NAN;
      if (prm.q_draft) prm.q_draft[b * G + r] = NAN;
    }
    if (tid == 0) {
      prm.n_acc[b] = -1;
      prm.token[b] = -1;
      if (prm.flags) prm.flags[b] = flg;
      prm.jobs[b].kind = JOB_NONE;
    }
    return;
  }

  // first rejected slot at or after start
  int kmin = G;
  if (!done)
    for (int s = st + tid; s < G; s += BLOCK)
      if (!s_acc[s]) kmin = min(kmin, s);
  atomicMin(&s_k, kmin);
  __syncthreads();
  const int k = s_k;

  for (int r = tid; r < G; r += BLOCK) {
    const int s = s_slot[r];
    const bool ver = !done && s >= st;
    if (prm.accept) prm.accept[b * G + r] = ver ? s_acc[s] : 0;
    if (prm.p_draft) prm.p_draft[b * G + r] = ver ? s_p[s] : 0.f;
    if (prm.q_draft) prm.q_draft[b * G + r] = ver ? s_q[s] : 0.f;
  }
  if (tid == 0) {
    Job job{};
    job.kind = JOB_NONE;
    if (done) {
      prm.n_acc[b] = 0;
    } else {
      prm.n_acc[b] = k - st;
      if (k < G) {
        const int r = ord ? ord[k] : k;
        job.kind = prm.dft ? JOB_RESID : JOB_ONEHOT;
        job.row = r;
        job.d = prm.ids[b * G + r];
        job.u = prm.us[b * (G + 1) + r];
        double S;
        row_stats(prm.part + (b * G + r) * prm.nseg, prm.nseg, c, job.m_t, S);
        if (prm.dft) row_stats(prm.part + ((prm.B + b) * G + r) * prm.nseg, prm.nseg, c, job.m_d, S);
      } else if (prm.bonus) {
        job.kind = JOB_BONUS;
        job.row = G;
        job.u = prm.us[b * (G + 1) + G];
      }
      if (prm.start) prm.start[b] = min(G, k + 1);
    }
    prm.token[b] = -1;
    if (prm.flags) prm.flags[b] = flg;
    prm.jobs[b] = job;
  }
}

// ----------------------------------------------------------------------------------------------------------------
// 3. float64 draw: normalisers, segment masses, search
// ----------------------------------------------------------------------------------------------------------------

struct DrawParams {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;
  int64_t B; int64_t V; int32_t nseg;
  double invT;
  const Job* jobs;
  double4* part2a;     // per (b, seg): m_t, S_t, m_d, S_d
  double2* part2b;     // per (b, seg): residual mass, p mass
  int32_t* token; uint32_t* flags;
};

__device__ __forceinline__ int64_t seg_lo(int64_t V, int nseg, int seg) { return V * seg / nseg; }

// Normalisers of the job's rows from the per-segment partials (fixed order).
__device__ __forceinline__ void draw_norms(const DrawParams& prm, int64_t b, double& mt, double& St, double& md,
                                           double& Sd) {
  const double4* p = prm.part2a + b * prm.nseg;
  double m1 = -INFINITY, m2 = -INFINITY;
  for (int i = 0; i < prm.nseg; ++i) { m1 = fmax(m1, p[i].x); m2 = fmax(m2, p[i].z); }
  double s1 = 0.0, s2 = 0.0;
  bool nan = false;
  for (int i = 0; i < prm.nseg; ++i) {
    nan |= isnan(p[i].y) || isnan(p[i].w);
    if (p[i].x != -INFINITY) s1 += (p[i].x == m1) ? p[i].y : p[i].y * exp((p[i].x - m1) * prm.invT);
    if (p[i].z != -INFINITY) s2 += (p[i].z == m2) ? p[i].w : p[i].w * exp((p[i].z - m2) * prm.invT);
  }
  mt = m1; md = m2;
  St = nan ? NAN : s1;
  Sd = nan ? NAN : s2;
}

// Weight of element i in the draw: the residual max(p_i - q_i, 0), or p_i when `use_p`. One definition for the
// mass pass and the search, compiled without contraction so that both see identical values.
template <typename T>
__device__ __forceinline__ double draw_weight(const Job& job, const T* rt, const T* rd, int64_t i, double mt,
                                              double inv_st, double md, double inv_sd, double invT, bool use_p,
                                              double* p_out) {
#pragma clang fp contract(off)
  const double zt = double(Vec<T>::load1(rt + i));
  const double p = exp((zt - mt) * invT) * inv_st;
  *p_out = p;
  if (use_p) return p;
  double q = 0.0;
  if (job.kind == JOB_RESID) {
    const double zd = double(Vec<T>::load1(rd + i));
    q = exp((zd - md) * invT) * inv_sd;
  } else if (job.kind == JOB_ONEHOT) {
    q = (i == job.d) ? 1.0 : 0.0;
  }
  const double r = p - q;
  return r > 0.0 ? r : 0.0;
}

template <typename T, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_draw_stats(DrawParams prm) {
  __shared__ float sh_f[BLOCK / 64];
  __shared__ double sh_d[BLOCK / 64];
  const int seg = int(blockIdx.x % prm.nseg);
  const int64_t b = blockIdx.x / prm.nseg;
  const Job job = prm.jobs[b];
  if (job.kind == JOB_NONE) return;
  const int64_t lo = seg_lo(prm.V, prm.nseg, seg), hi = seg_lo(prm.V, prm.nseg, seg + 1);
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;

  float mt = job.m_t;
  int has_nan = 0;
  if (job.kind == JOB_BONUS) {                      // the bonus row was not in the statistics pass
    float m = -INFINITY;
    for (int64_t i = lo + threadIdx.x; i < hi; i += BLOCK) {
      const float z = Vec<T>::load1(rt + i);
      m = fmaxf(m, z);
      has_nan |= (z != z);
    }
    mt = block_max<BLOCK>(m, sh_f);
    has_nan = __syncthreads_or(has_nan);
  }
  double st = 0.0;
  if (mt != -INFINITY)
    for (int64_t i = lo + threadIdx.x; i < hi; i += BLOCK)
      st += exp((double(Vec<T>::load1(rt + i)) - double(mt)) * prm.invT);
  st = block_sum<BLOCK>(st, sh_d);
  if (has_nan) st = NAN;
  double sd = 0.0;
  float md = -INFINITY;
  if (job.kind == JOB_RESID) {
    const T* rd = static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row;
    md = job.m_d;
    for (int64_t i = lo + threadIdx.x; i < hi; i += BLOCK)
      sd += exp((double(Vec<T>::load1(rd + i)) - double(md)) * prm.invT);
    sd = block_sum<BLOCK>(sd, sh_d);
  }
  if (threadIdx.x == 0) prm.part2a[b * prm.nseg + seg] = make_double4(mt, st, md, sd);
}

template <typename T, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_draw_mass(DrawParams prm) {
  __shared__ double sh_d[BLOCK / 64];
  const int seg = int(blockIdx.x % prm.nseg);
  const int64_t b = blockIdx.x / prm.nseg;
  const Job job = prm.jobs[b];
  if (job.kind == JOB_NONE) return;
  double mt, St, md, Sd;
  draw_norms(prm, b, mt, St, md, Sd);
  if (isnan(St) || isinf(mt) || (job.kind == JOB_RESID && isnan(Sd))) return;   // bad bonus row: k_draw_pick
  const double inv_st = 1.0 / St, inv_sd = (job.kind == JOB_RESID) ? 1.0 / Sd : 0.0;
  const int64_t lo = seg_lo(prm.V, prm.nseg, seg), hi = seg_lo(prm.V, prm.nseg, seg + 1);
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const T* rd = job.kind == JOB_RESID
      ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  double R = 0.0, Pm = 0.0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += BLOCK) {
    double p;
    R += draw_weight<T>(job, rt, rd, i, mt, inv_st, md, inv_sd, prm.invT, false, &p);
    Pm += p;
  }
  R = block_sum<BLOCK>(R, sh_d);
  Pm = block_sum<BLOCK>(Pm, sh_d);
  if (threadIdx.x == 0) prm.part2b[b * prm.nseg + seg] = make_double2(R, Pm);
}

// Inclusive block scan of doubles in thread order.
template <int BLOCK>
__device__ __forceinline__ double block_inclusive_scan(double v, double* sh) {
  const int l = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const double n = __shfl_up(v, o);
    if (l >= o) v += n;
  }
  __syncthreads();
  if (l == 63) sh[w] = v;
  __syncthreads();
  double base = 0.0;
  for (int i = 0; i < w; ++i) base += sh[i];
  return base + v;
}

template <typename T, int BLOCK>
__global__ __launch_bounds__(BLOCK) void k_draw_pick(DrawParams prm) {
  __shared__ double sh_d[BLOCK / 64];
  __shared__ int s_seg, s_clamp, s_cand, s_last;
  __shared__ double s_base, s_t;
  const int64_t b = blockIdx.x;
  const Job job = prm.jobs[b];
  if (job.kind == JOB_NONE) return;
  const int tid = threadIdx.x;
  double mt, St, md, Sd;
  draw_norms(prm, b, mt, St, md, Sd);
  if (isnan(St) || isinf(mt) || (job.kind == JOB_RESID && isnan(Sd))) {     // only a bonus row can get here
    if (tid == 0) {
      prm.token[b] = -1;
      if (prm.flags) prm.flags[b] |= SV_FLAG_NONFINITE;
    }
    return;
  }
  const double2* mass = prm.part2b + b * prm.nseg;
  const int nseg = prm.nseg;
  // total residual mass; an empty residual falls back to p
  double tot_r = 0.0, tot_p = 0.0;
  for (int i = 0; i < nseg; ++i) { tot_r += mass[i].x; tot_p += mass[i].y; }
  const bool use_p = !(tot_r > 0.0);
  if (tid == 0) {
    const double total = use_p ? tot_p : tot_r;
    const double t = double(job.u) * total;
    double cum = 0.0;
    int seg = -1, last = -1;
    double base = 0.0;
    for (int i = 0; i < nseg; ++i) {
      const double w = use_p ? mass[i].y : mass[i].x;
      if (w > 0.0) last = i;
      if (seg < 0 && cum + w > t) { seg = i; base = cum; }
      cum += w;
    }
    s_clamp = seg < 0;
    if (seg < 0) {
      seg = last;
      base = 0.0;
    }
    s_seg = seg;
    s_base = base;
    s_t = t;
    s_cand = INT_MAX;
    s_last = -1;
  }
  __syncthreads();
  const int seg = s_seg;
  if (seg < 0) {                                    // no positive weight anywhere (cannot happen for finite rows)
    if (tid == 0) prm.token[b] = -1;
    return;
  }
  const double t = s_t;
  const int64_t lo = seg_lo(prm.V, nseg, seg), hi = seg_lo(prm.V, nseg, seg + 1);
  const int64_t n = hi - lo;
  const int64_t per = (n + BLOCK - 1) / BLOCK;
  const int64_t i0 = lo + min<int64_t>(n, per * tid), i1 = lo + min<int64_t>(n, per * (tid + 1));
  const double inv_st = 1.0 / St, inv_sd = (job.kind == JOB_RESID) ? 1.0 / Sd : 0.0;
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const T* rd = job.kind == JOB_RESID
      ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  double mine = 0.0;
  int last = -1;
  for (int64_t i = i0; i < i1; ++i) {
    double p;
    const double w = draw_weight<T>(job, rt, rd, i, mt, inv_st, md, inv_sd, prm.invT, use_p, &p);
    mine += w;
    if (w > 0.0) last = int(i);
  }
  const double incl = block_inclusive_scan<BLOCK>(mine, sh_d);
  int cand = INT_MAX;
  if (!s_clamp) {
    double acc = s_base + (incl - mine);
    for (int64_t i = i0; i < i1; ++i) {
      double p;
      acc += draw_weight<T>(job, rt, rd, i, mt, inv_st, md, inv_sd, prm.invT, use_p, &p);
      if (acc > t) { cand = int(i); break; }
    }
  }
  atomicMin(&s_cand, cand);
  atomicMax(&s_last, last);
  __syncthreads();
  if (tid == 0) {
    const int tok = s_cand != INT_MAX ? s_cand : s_last;
    prm.token[b] = tok;
    if (use_p && prm.flags) prm.flags[b] |= SV_FLAG_EMPTY_RESIDUAL;
  }
}

template <typename T>
hipError_t launch_typed(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  char* ws = a.ws;
  Partial1* part1 = reinterpret_cast<Partial1*>(ws + plan.off_part1);
  Job* jobs = reinterpret_cast<Job*>(ws + plan.off_jobs);
  double4* part2a = reinterpret_cast<double4*>(ws + plan.off_part2a);
  double2* part2b = reinterpret_cast<double2*>(ws + plan.off_part2b);
  const double T_ = double(a.temperature);
  const float c = float(1.4426950408889634074 / T_);          // log2(e) / T

  StatsParams sp{a.tgt, a.t_seq, a.t_row, a.dft, a.d_seq, a.d_row, plan.B, plan.G, plan.V, plan.nseg1, plan.ntens,
                 c, a.start, a.order, part1};
  const int64_t g1 = int64_t(plan.ntens) * plan.B * plan.G * plan.nseg1;
  if (a.ev_start) (void)hipEventRecord(static_cast<hipEvent_t>(a.ev_start), stream);
  hipLaunchKernelGGL((k_stats<T, kStatsBlock, kUnroll>), dim3(unsigned(g1)), dim3(kStatsBlock), 0, stream, sp);
  if (a.ev_stop) (void)hipEventRecord(static_cast<hipEvent_t>(a.ev_stop), stream);

  ScanParams cp{a.tgt, a.t_seq, a.t_row, a.dft, a.d_seq, a.d_row, plan.B, plan.G, plan.V, plan.nseg1, a.bonus, c,
                a.ids, a.ua, a.us, a.start, a.order, a.accept, a.n_acc, a.token, a.p_draft, a.q_draft, a.flags,
                part1, jobs};
  hipLaunchKernelGGL((k_scan<T, kScanBlock>), dim3(unsigned(plan.B)), dim3(kScanBlock), 0, stream, cp);

  DrawParams dp{a.tgt, a.t_seq, a.t_row, a.dft, a.d_seq, a.d_row, plan.B, plan.V, plan.nseg2, 1.0 / T_, jobs,
                part2a, part2b, a.token, a.flags};
  const int64_t g2 = plan.B * plan.nseg2;
  hipLaunchKernelGGL((k_draw_stats<T, kDrawBlock>), dim3(unsigned(g2)), dim3(kDrawBlock), 0, stream, dp);
  hipLaunchKernelGGL((k_draw_mass<T, kDrawBlock>), dim3(unsigned(g2)), dim3(kDrawBlock), 0, stream, dp);
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
  // draw pass: aim for >= 2048 workgroups over B row pairs, segments of >= 2048 elements, at most 256 segments
  int64_t s2 = (2048 + B - 1) / B;
  const int64_t cap2 = V / 2048 > 1 ? V / 2048 : 1;
  if (s2 > cap2) s2 = cap2;
  if (s2 > 256) s2 = 256;
  if (s2 < 1) s2 = 1;
  p.nseg2 = int32_t(s2);
  size_t off = 0;
  p.off_part1 = off; off = align_up(off + size_t(rows) * p.nseg1 * sizeof(Partial1), 256);
  p.off_jobs = off;  off = align_up(off + size_t(B) * sizeof(Job), 256);
  p.off_part2a = off; off = align_up(off + size_t(B) * p.nseg2 * sizeof(double4), 256);
  p.off_part2b = off; off = align_up(off + size_t(B) * p.nseg2 * sizeof(double2), 256);
  p.total = off;
  return p;
}

hipError_t launch_dense(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  if (a.dtype == SV_BF16) return launch_typed<uint16_t>(plan, a, stream);
  return launch_typed<float>(plan, a, stream);
}

}  // namespace sv
