// Dense and one-hot speculative-sampling verification for gfx950 (MI355X).
//
// The rule is Leviathan et al.'s, as restated on "Uno: the draft model was already inside the target model"
// (section "What 'lossless' actually has to mean"): accept a draft x with probability min(1, p(x)/q(x)), cut the
// block at the first rejection (DFlash/DFlash2 guide, section 4.4) and draw the replacement from max(p - q, 0)
// renormalised there, or a bonus token from the next target row when every draft is accepted (same guide,
// section 2). p and q are softmaxes of the logits divided by the temperature (same guide, section 9 Q3).
//
// One launch on the caller's stream: one 256-thread workgroup per work item, in a queue order that the hardware's
// in-order dispatch turns into a schedule. Three kinds of item:
//  - statistics item (one segment of one verified logit row): a running max and a running sum of
//    exp2((z - max) * log2(e)/T) in float32, folded over the workgroup in float64, written as (max, sum, logit at the
//    draft id). 16-byte non-temporal loads, a two-group ping-pong per thread. These items move almost all the bytes;
//    they are bound by HBM bandwidth.
//  - scan (one per sequence, queued about one resident round after the sequence's statistics items): evaluates p(x),
//    q(x) and the strict test u < min(1, p/q) of every verified slot, finds the first rejection from `start` along
//    `order`, writes the per-row outputs and publishes the sequence's draw job.
//  - draw task (a range of 512-element chunks of the row or row pair the draw needs; queued after every statistics
//    item): float64 residual masses of its chunks and partial softmax normalisers. The last task of a sequence to
//    finish forms the chunk masses and their running sum, and searches the one chunk that holds t = u * (total mass).
// Draw tasks start on the compute units that the last statistics items leave free, so the float64 draw overlaps the
// tail of the streaming phase instead of waiting for a second launch.
// The float64 draw exists because a token boundary of the residual CDF often lies within 1e-7 of t at these
// vocabulary sizes; float32 sums would pick a neighbouring token far more often than the float64 reference does.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cfloat>
#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "sv.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_wshdr.h"
#include "sv_fexp.h"

// Scratch of the no-allocation entry point (sv_verify_dense_noalloc): every GPU the library runs on holds its own copy
// until the process ends. Host code never passes this name to a kernel: it looks the device address up with
// hipGetSymbolAddress (noalloc_scratch) and passes that.
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace sv {
namespace {

constexpr int kStatsBlock = 256;
constexpr int kUnroll = 4;          // 16-byte vectors per thread per group
constexpr bool kNonTemporal = true; // streaming loads that bypass cache retention
constexpr int kWpe = 4;             // waves per SIMD the kernel is compiled for
constexpr int kDrawBlock = 256;     // threads per workgroup, both kinds of item
constexpr int64_t kItemBytes = 1048576;   // target bytes of logits per statistics item
// Draw task sizes, in chunks. Most sequences take tasks of kTaskChunks, doubled (up to kTaskChunksMax) while the launch
// would hold more than kTasksPerSlot tasks per resident workgroup (a task costs ~4 us of hand-off and set-up besides
// its float64 work); the last sequences, whose draws end the launch, take tasks of kTailChunks: as many sequences as
// hold about kTailSlots chunks per resident workgroup.
constexpr int64_t kTaskChunks = 16;
constexpr int64_t kTaskChunksMax = 64;
constexpr int64_t kTasksPerSlot = 2;
constexpr int64_t kTailChunks = 8;
constexpr int64_t kTailSlots = 3;
constexpr int kScanLagRounds = 1;   // resident rounds of statistics items between a sequence's statistics and its scan
constexpr int64_t kDrawSlackPct = 25;   // draw slots beyond the draw tasks, in percent of them ...
constexpr int64_t kDrawSlackMax = 256;  // ... and at most this many
constexpr int kCtrStride = 64;          // int32 slots between per-sequence counters (one 256-byte line each)
constexpr int kSleep = 16;              // s_sleep units between polls of a wait
constexpr int32_t kSpinCap = kWsSpinCap;   // polls before a wait gives up (never reached when the hardware
                                           // dispatches workgroups in index order, as documented)

struct alignas(16) Partial1 {
  float m;        // exact max of the segment's logits (raw, before the temperature)
  float zx;       // segment 0 only: the row's logit at its draft id (NaN when the id is out of range)
  double s;       // sum over the segment of 2^((z - m) * c), c = log2(e)/T rounded to float
};

// ----------------------------------------------------------------------------------------------------------------
// helpers that depend on the job record
// ----------------------------------------------------------------------------------------------------------------

// The job's fields are the same in every lane (read from shared memory after a barrier): moved to scalar registers,
// so that branches on them are uniform.
__device__ __forceinline__ Job uniform_job(const Job& j) {
  Job r;
  const uint32_t* s = reinterpret_cast<const uint32_t*>(&j);
  uint32_t* d = reinterpret_cast<uint32_t*>(&r);
#pragma unroll
  for (int i = 0; i < int(sizeof(Job) / 4); ++i) d[i] = __builtin_amdgcn_readfirstlane(s[i]);
  return r;
}


// ----------------------------------------------------------------------------------------------------------------
// 1. row statistics
// ----------------------------------------------------------------------------------------------------------------

// Everything one call needs, shared by both kinds of work item.
struct DenseParams {
  const void* tgt; int64_t t_seq, t_row;
  const void* dft; int64_t d_seq, d_row;     // dft == nullptr: one-hot drafts
  int64_t B; int32_t G; int64_t V; int32_t nseg1; int32_t ntens; int32_t bonus;
  float c;                                    // log2(e) / T, rounded to float (statistics items)
  double c2;                                  // log2(e) / T in float64 (draw: weights are 2^((z - max) * c2))
  const int32_t* ids; const float* ua; const float* us;
  int32_t* start; const int32_t* order;
  uint8_t* accept; int32_t* n_acc; int32_t* token; float* p_draft; float* q_draft; uint32_t* flags;
  // work queue: per sequence n1 statistics items, one scan and ntask draw tasks, in the order of decode_item
  int32_t n1; int32_t ntask; int32_t lag1; int32_t n_items;
  int32_t ntask2;                             // draw tasks of each of the last tailq sequences (>= ntask)
  int32_t chunks1;                            // chunks per draw task of the other sequences
  int32_t tailq;                              // sequences with small draw tasks (the last ones)
  int64_t ntot;                               // draw tasks in all
  int64_t nch;                                // kChunk-element chunks per row
  int32_t* ready;                             // per b (stride kCtrStride): statistics items finished
  int32_t* done;                              // per b (stride kCtrStride): draw tasks finished
  int32_t* tickets;                           // draw slots started in this call (each takes one ticket)
  int32_t nslots;                             // draw slots in the queue (at least B * ntask)
  Job* jobs;                                  // per b (one per kJobStride bytes): the draw job, sealed
  Partial1* part1;                            // per (tensor, b, row, segment)
  double4* part2;            // per (b, task): reference max, sum e_t (relative to it), m_d, sum e_d
  // chunk records of the mass pass, one array per field so that the pick reads them coalesced (see chunk_body)
  double* recA;              // per (b, chunk)
  double* recD;              // per (b, chunk)
  int32_t* recN;             // per (b, chunk)
  double2* recU;             // per (b, chunk, kAmbMax)
  double* masses;            // per (b, chunk): chunk masses, written by the pick when the chunks exceed one tile
  char* ws;                  // the workspace: its header (the control layout at zero) leads the control words
  uint64_t sig;              // this call's control layout
  int64_t ctl_end;           // control words fill [kWsHeaderBytes, ctl_end)
};

// The parameters are read in place from the kernel-argument segment (constant address space) by every function,
// inlined or not, instead of being copied to per-lane private memory for the functions that are not inlined.
typedef const __attribute__((address_space(4))) DenseParams DP;

// The kernel's parameters, read in place from its kernel-argument segment. Only the kernel itself may ask for that
// segment's address; functions that are not inlined receive the reference as an argument (in vector registers) and
// make it uniform again with uniform_params, so that their parameter reads are scalar loads.
__device__ __forceinline__ DP& kernel_params() { return *(DP*)(__builtin_amdgcn_kernarg_segment_ptr()); }

__device__ __forceinline__ DP& uniform_params(DP& p) {
  const uint64_t a = reinterpret_cast<uint64_t>(&p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(a >> 32));
  return *reinterpret_cast<DP*>((uint64_t(hi) << 32) | lo);
}

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

// One work item: segment `seg` of one row. Returns without writing when the row's slot lies before start.
template <typename T, int BLOCK, int U, bool NT>
__device__ __forceinline__ void stats_item(DP& prm, int64_t b, int item, float* sh_f, double* sh_d) {
  using VT = Vec<T>;
  constexpr int EPV = VT::kEPV;

  const int seg = item % prm.nseg1;
  const int row = (item / prm.nseg1) % prm.G;
  const int tens = item / (prm.nseg1 * prm.G);

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
  const int64_t v0 = nvec * seg / prm.nseg1, v1 = nvec * (seg + 1) / prm.nseg1;

  Run st{-INFINITY, -INFINITY, 0.f};
  if (seg == 0) {
    for (int64_t i = threadIdx.x; i < head; i += BLOCK) { float z = VT::load1(base + i); absorb<1>(st, &z, c); }
  }
  if (seg == prm.nseg1 - 1) {
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
  if (threadIdx.x == 0) {          // read by other workgroups of this launch: device-scope stores
    float zx = NAN;
    if (seg == 0) {
      const int x = prm.ids[b * prm.G + row];
      if (x >= 0 && int64_t(x) < V) zx = VT::load1(base + x);
    }
    Partial1* out = prm.part1 + ((int64_t(tens) * prm.B + b) * prm.G + row) * prm.nseg1 + seg;
    st_dev(&out->m, M);
    st_dev(&out->zx, zx);
    st_dev(&out->s, s);
  }
}

// ----------------------------------------------------------------------------------------------------------------
// 2. draw: accept tests and first-rejection scan, then the float64 draw (mass pass + pick)
// ----------------------------------------------------------------------------------------------------------------
//
// The rows are cut into chunks of kChunk = 512 consecutive elements (one wave, 8 consecutive elements per lane).
// The mass pass starts, in every workgroup, with the accept tests of its sequence (from the statistics pass's
// per-row max, sum and draft-id logit) and the scan for the first rejection; the workgroup of the sequence's first
// segment writes the per-row outputs and the draw job. It then computes, per chunk of the draw's row(s), A = sum
// of e_t and D = sum of e_d over the elements where the residual is positive, with e = exp((z - max) / T) in
// float64, together with the exact normalisers S_t and S_d; a chunk's residual mass is then A / S_t - D / S_d.
// Whether p_i > q_i, i.e. e_t * (S_d / S_t) > e_d, is decided with the statistics pass's estimate of S_d / S_t,
// which is within 1e-5 of the exact ratio; an element within kBand of the boundary marks its chunk, and the pick
// recomputes that chunk exactly. The pick forms every chunk's mass, scans them in order, finds the chunk that
// holds t = u * (total mass) and searches it with one wave.

constexpr int kChunk = 512;         // elements per chunk
constexpr int kPer = 8;             // elements per lane in a chunk
constexpr double kBand = 3.0e-5;    // relative width of the undecided zone of the residual's sign test
constexpr int kTile = 1024;         // chunks held in LDS at a time by the pick
constexpr int kDrawWaves = kDrawBlock / 64;


// 2^x for a float64 x, to float32 accuracy at any magnitude: the integer part is applied exactly with ldexp, only
// the fraction in [0, 1) goes through the hardware exp2.
__device__ __forceinline__ float exp2_split(double x) {
  if (!(x > -160.0)) return x != x ? NAN : 0.f;
  if (x > 130.0) return INFINITY;
  const double n = floor(x);
  return ldexpf(ex2f(float(x - n)), int(n));
}

// 2^((m - M) * c) for a segment max m <= M: exactly 1 when m == M, 0 for an empty segment, else to float32 accuracy
// (the scan needs the row sums only to float32 accuracy; the draw forms its own float64 normalisers).
__device__ __forceinline__ double seg_scale(float m, float M, double c) {
  if (m == M) return 1.0;
  if (m == -INFINITY) return 0.0;
  return double(exp2_split((double(m) - double(M)) * c));
}

// Row statistics of a target row and (dense) its draft row from their segment partials, written by other
// workgroups of this launch (device-scope loads): exact max m and S = sum 2^((z - m) * c) over the row. The partials
// of both rows are requested together, four segments at a time, so rows of up to four segments cost one round trip.
// Identical rows give identical results.
struct RowPair {
  float mt, zt, md, zd;   // max and logit at the draft id of the target and draft rows
  double St, Sd;          // sums relative to the max (NaN when a segment saw NaN)
};

__device__ __forceinline__ RowPair row_pair_stats(const Partial1* pt, const Partial1* pd, int nseg, double c) {
  constexpr int K = 4;
  const Partial1* qd = pd ? pd : pt;             // one-hot: loads of the target row stand in, results unused
  RowPair r;
  r.zt = ld_dev(&pt[0].zx);
  const float zd0 = ld_dev(&qd[0].zx);
  r.zd = pd ? zd0 : 0.f;
  if (nseg == 1) {                               // one statistics item per row: its partial is the row's
    r.mt = ld_dev(&pt[0].m);
    r.St = ld_dev(&pt[0].s);
    const float md = ld_dev(&qd[0].m);
    const double sd = ld_dev(&qd[0].s);
    r.md = pd ? md : 0.f;
    r.Sd = pd ? sd : 1.0;
    return r;
  }
  float Mt = -INFINITY, Md = -INFINITY;
  double St = 0.0, Sd = 0.0;
  bool nt = false, nd = false;
  for (int i0 = 0; i0 < nseg; i0 += K) {
    float mt[K], md[K];
    double st[K], sd[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {                 // clamped indices: every load is issued, none is conditional
      const int i = min(i0 + k, nseg - 1);
      mt[k] = ld_dev(&pt[i].m);
      st[k] = ld_dev(&pt[i].s);
      md[k] = ld_dev(&qd[i].m);
      sd[k] = ld_dev(&qd[i].s);
    }
    float bt = Mt, bd = Md;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if (i0 + k >= nseg) { mt[k] = md[k] = -INFINITY; st[k] = sd[k] = 0.0; }
      bt = fmaxf(bt, mt[k]);
      bd = fmaxf(bd, md[k]);
    }
    St *= seg_scale(Mt, bt, c);
    Sd *= seg_scale(Md, bd, c);
#pragma unroll
    for (int k = 0; k < K; ++k) {
      nt |= isnan(st[k]);
      nd |= isnan(sd[k]);
      St += st[k] * seg_scale(mt[k], bt, c);
      Sd += sd[k] * seg_scale(md[k], bd, c);
    }
    Mt = bt;
    Md = bd;
  }
  r.mt = Mt;
  r.St = nt ? NAN : St;
  r.md = pd ? Md : 0.f;
  r.Sd = pd ? (nd ? NAN : Sd) : 1.0;
  return r;
}

struct SlotEval {
  float P, Q;
  bool acc, qzero, bad_id, nonfinite;
  RowPair rs;
  int32_t x;
  float us;               // the row's draw uniform
};


// p(x), q(x) and the strict test u < min(1, p/q) of storage row r. The log-probabilities are assembled in float64
// from the row statistics; the hardware float32 log2/exp2 finish them (relative error ~1e-6 on the ratio and on
// p(x), q(x)).
__device__ __forceinline__ SlotEval eval_slot(const DP& prm, int64_t b, int r) {
  SlotEval e;
  e.P = e.Q = NAN;
  e.acc = e.qzero = e.bad_id = e.nonfinite = false;
  const int G = prm.G;
  const double c = double(prm.c);
  const int x = prm.ids[b * G + r];
  const float u = prm.ua[b * G + r];
  e.us = prm.us[b * (G + 1) + r];
  e.x = x;
  e.rs = row_pair_stats(prm.part1 + (b * G + r) * prm.nseg1,
                        prm.dft ? prm.part1 + ((prm.B + b) * G + r) * prm.nseg1 : nullptr, prm.nseg1, c);
  const RowPair& rs = e.rs;
  e.nonfinite = isnan(rs.St) || rs.mt == INFINITY || rs.mt == -INFINITY;
  if (prm.dft) e.nonfinite |= isnan(rs.Sd) || rs.md == INFINITY || rs.md == -INFINITY;
  if (x < 0 || int64_t(x) >= prm.V) {
    e.bad_id = true;
    return e;
  }
  const double lp = (double(rs.zt) - double(rs.mt)) * c - double(__builtin_amdgcn_logf(float(rs.St)));   // log2 p(x)
  double lq = 0.0;                                                                                       // one-hot
  if (prm.dft) {
    e.qzero = (rs.zd == -INFINITY);
    lq = (double(rs.zd) - double(rs.md)) * c - double(__builtin_amdgcn_logf(float(rs.Sd)));
  }
  e.P = exp2_split(lp);
  e.Q = prm.dft ? exp2_split(lq) : 1.f;
  float ratio = e.qzero ? 0.f : exp2_split(lp - lq);
  if (ratio != ratio) ratio = 0.f;
  e.acc = u < fminf(1.f, ratio);
  return e;
}

// Accept tests and first-rejection scan of sequence b by one wave (lane l takes slots start + l, start + l + 64, ...).
// Every draw task of the sequence computes the same record; the leader also writes the per-row outputs and
// n_accepted. out_token, flags and the new start are written once, by the sequence's last draw task.
__device__ __forceinline__ Job seq_scan(DP& prm, int64_t b, bool leader, uint32_t* seen) {
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
  RowPair krs{};                                   // statistics of this lane's first rejected slot
  int32_t kx = 0;
  float ku = 0.f;
  const float u_bonus = prm.us[b * (G + 1) + G];
  // Every slot is evaluated, whatever start is, so that all loads go out together; slots before start (whose rows
  // were not read) and every slot of a sequence with a bad order or start are then ignored.
  for (int s = lane; s < G; s += 64) {
    int r = ord ? ord[s] : s;
    r = (r >= 0 && r < G) ? r : 0;                 // addresses stay in range under an invalid order
    const SlotEval e = eval_slot(prm, b, r);
    if (bad || done || s < st) continue;
    bad_id |= e.bad_id;
    nf |= e.nonfinite;
    qz |= e.qzero;
    if (!e.acc && kmin == G) { kmin = s; krs = e.rs; kx = e.x; ku = e.us; }
    if (leader) {
      if (prm.accept) prm.accept[b * G + r] = e.acc ? 1 : 0;
      if (prm.p_draft) prm.p_draft[b * G + r] = e.P;
      if (prm.q_draft) prm.q_draft[b * G + r] = e.Q;
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
  job.flags = flg;
  if (!fatal && !done) {
    job.new_start = min(G, k + 1);
    if (k < G) {
      const int kl = k & 63;                       // the lane that evaluated slot k
      job.kind = prm.dft ? JOB_RESID : JOB_ONEHOT;
      job.row = ord ? ord[k] : k;
      job.d = __builtin_amdgcn_readlane(kx, kl);
      job.u = readlane_f(ku, kl);
      job.m_t = readlane_f(krs.mt, kl);
      job.m_d = readlane_f(krs.md, kl);
      const double S_t = readlane_d(krs.St, kl), S_d = prm.dft ? readlane_d(krs.Sd, kl) : 1.0;
      job.kappa = S_d / S_t;
    } else if (prm.bonus) {
      job.kind = JOB_BONUS;
      job.row = G;
      job.u = u_bonus;
    }
  }
  if (leader) {
    if (fatal) __builtin_amdgcn_s_waitcnt(0);       // the per-slot stores above land before they are overwritten
    // rows not verified (before start, or every row when nothing is left), and every row of a failed sequence
    for (int s = lane; s < G; s += 64) {
      if (!(fatal || done || s < st)) continue;
      const int r = ord && !bad ? ord[s] : s;
      const float pq = fatal ? NAN : 0.f;
      if (prm.accept) prm.accept[b * G + r] = 0;
      if (prm.p_draft) prm.p_draft[b * G + r] = pq;
      if (prm.q_draft) prm.q_draft[b * G + r] = pq;
    }
    if (lane == 0) prm.n_acc[b] = fatal ? -1 : (done ? 0 : k - st);
  }
  return job;
}

template <int BLOCK>
__device__ __forceinline__ double block_max_d(double v, double* sh) {
  v = wave_max_d(v);
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
  const double incl = wave_incl_scan(v);
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

// kPer consecutive logits starting at element i0 of a row, as float; -inf past the end of the row.
template <typename T>
__device__ __forceinline__ void load_lane(const T* row, int64_t i0, int64_t V, bool vec, float* z) {
  if (vec && i0 + kPer <= V) {
    const uint4* p = reinterpret_cast<const uint4*>(row + i0);
    constexpr int NV = kPer / Vec<T>::kEPV;
#pragma unroll
    for (int k = 0; k < NV; ++k) Vec<T>::unpack(gload4(p + k), z + k * Vec<T>::kEPV);
  } else {
#pragma unroll
    for (int e = 0; e < kPer; ++e) z[e] = elem_or_ninf<T>(row, i0 + e, V);
  }
}

// Exact draw weights of the lane's kPer elements of chunk c (relative to the common reference max mt): the residual
// max(p_i - q_i, 0), or p_i when use_p. Compiled without contraction so repeated evaluations agree bit for bit.
template <typename T>
__device__ __forceinline__ void chunk_weights(const Job& job, const T* rt, const T* rd, bool vec, int64_t c, int lane,
                                              int64_t V, double mt, double inv_st, double md, double inv_sd,
                                              double c2, bool use_p, double* w) {
#pragma clang fp contract(off)
  const int64_t i0 = c * kChunk + int64_t(lane) * kPer;
  float zt[kPer], zd[kPer];
  load_lane<T>(rt, i0, V, vec, zt);
  const bool resid = job.kind == JOB_RESID && !use_p;
  if (resid) load_lane<T>(rd, i0, V, vec, zd);
  const double nmt = -(mt * c2), nmd = -(md * c2);
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const double p = fexp_scaled(xarg(zt[e], c2, nmt)) * inv_st;
    double q = 0.0;
    if (resid) q = fexp_scaled(xarg(zd[e], c2, nmd)) * inv_sd;
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

// Per-chunk record of the mass pass: A = sum of e_t and D = sum of e_d over the elements whose residual is known to be
// positive (bonus and one-hot: A = sum of e_t over every element but the one-hot id, D = 0); N = number of elements
// whose sign could not be decided, kept as (e_t, e_d) pairs in U when N <= kAmbMax (N > kAmbMax: the chunk must be
// recomputed from the logits). The exps are relative to the draw row's max, except for a bonus row, where they are
// relative to the max of the chunk's draw task (the first field of that task's partial).
constexpr int kAmbMax = 4;

// The draw tasks of sequence b: the sequences before the last tailq cut their rows into tasks of kTaskChunks chunks,
// the last tailq (whose draws end the launch) into tasks of kTailChunks, so that their draws take less time. The
// task partials of sequence b sit at b * ntask2 + task.
struct TaskShape {
  int32_t ntask;     // tasks of the sequence
  int32_t chunks;    // chunks per task (a power of two; the last task may hold fewer)
  int32_t shift;     // log2(chunks)
};
__device__ __forceinline__ TaskShape task_shape(DP& prm, int64_t b) {
  const int32_t c = b < prm.B - prm.tailq ? prm.chunks1 : int32_t(kTailChunks);
  return TaskShape{b < prm.B - prm.tailq ? prm.ntask : prm.ntask2, c, __builtin_ctz(uint32_t(c))};
}
// The draw task that chunk c belongs to (task t holds chunks t * chunks .. t * chunks + chunks - 1).
__device__ __forceinline__ int task_of_chunk(int64_t c, const TaskShape& shp) { return int(c >> shp.shift); }

__device__ __forceinline__ double4 ld_task(const double4* p) {
  const double* d = reinterpret_cast<const double*>(p);
  return make_double4(ld_dev(d), ld_dev(d + 1), ld_dev(d + 2), ld_dev(d + 3));
}
__device__ __forceinline__ void st_task(double4* p, double4 v) {
  double* d = reinterpret_cast<double*>(p);
  st_dev(d, v.x);
  st_dev(d + 1, v.y);
  st_dev(d + 2, v.z);
  st_dev(d + 3, v.w);
}

// One lane's kPer elements: exp of both logits, the residual's sign test and the sums. For a residual draw A and D are
// accumulated as fma(e, w, .) with w = 1 where the residual is positive and 0 elsewhere; amb is set when an element's
// sign could not be decided (the caller recomputes which one). Bonus and one-hot draws only sum e_t here.
template <int KIND>
__device__ __forceinline__ void mass_lane(const float* zt, const float* zd, double c2, double nmt, double nmd,
                                          double k_lo, double k_hi, double& st, double& sd,
                                          double& A, double& D, bool& amb) {
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const double et = fexp_scaled(xarg(zt[e], c2, nmt));
    st += et;
    if constexpr (KIND == JOB_RESID) {
      const double ed = fexp_scaled(xarg(zd[e], c2, nmd));
      sd += ed;
      // r_e > 0 iff et * (S_d / S_t) > ed; kappa brackets S_d / S_t within kBand
      const bool pos = et * k_lo > ed;
      const bool neg = et * k_hi <= ed;
      const double w = pos ? 1.0 : 0.0;
      A = fma(et, w, A);
      D = fma(ed, w, D);
      amb |= !(pos || neg);
    }
    // the sums are pinned here every two elements: otherwise the compiler defers them to the end of the chunk and
    // holds every exp of the lane at once, past the loop's register budget (other waves on the SIMD hide latency)
    if (e & 1) asm volatile("" : "+v"(st), "+v"(sd), "+v"(A), "+v"(D));
  }
}

// One chunk of the mass pass, its kPer elements per lane in zt (and zd): the sums, the undecided elements and the
// chunk's record.
template <int KIND>
__device__ __forceinline__ void chunk_body(DP& prm, const Job& job, int64_t b, int64_t c, int64_t i0,
                                           const float* zt, const float* zd, double mt, double c2, double nmt,
                                           double nmd, double k_lo, double k_hi, double& st, double& sd) {
  const int lane = threadIdx.x & 63;
  double A = 0.0, D = 0.0, cst = 0.0, csd = 0.0;     // this chunk's sums
  bool amb = false;
  mass_lane<KIND>(zt, zd, c2, nmt, nmd, k_lo, k_hi, cst, csd, A, D, amb);
  st += cst;
  sd += csd;
  if constexpr (KIND != JOB_RESID) A = cst;          // the bonus draws from p: the chunk's whole sum
  if constexpr (KIND == JOB_ONEHOT) {
    // q is one-hot at the draft id d, so the residual is p without element d: in the chunk that holds d, the lane
    // that holds it sums its other elements again (same operations, so the same bits for every other element)
    if (c == job.d / kChunk) {
      const int64_t ed = int64_t(job.d) - i0;
      if (ed >= 0 && ed < kPer) {
        double a = 0.0;
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
          float z = zt[e];
          asm volatile("" : "+v"(z));
          const double et = fexp_scaled(xarg(z, c2, nmt));
          if (e != ed) a += et;
        }
        A = a;
      }
    }
  }
  A = wave_sum(A);
  if constexpr (KIND == JOB_RESID) D = wave_sum(D);
  const int64_t rc = b * prm.nch + c;
  int namb = 0;
  if constexpr (KIND == JOB_RESID) {
    if (__any(amb)) {                                // rare: list the undecided elements in element order
      uint32_t bits = 0;                             // bit e: element e undecided, recomputed exactly as above
      double et[kPer], ed[kPer];
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        // the logits pass through an empty asm so that the compiler recomputes here instead of keeping the main
        // loop's exps alive across the reductions (same operations on the same values: the same bits)
        float a = zt[e], d = zd[e];
        asm volatile("" : "+v"(a), "+v"(d));
        et[e] = fexp_scaled(xarg(a, c2, nmt));
        ed[e] = fexp_scaled(xarg(d, c2, nmd));
        const bool pos = et[e] * k_lo > ed[e];
        const bool neg = et[e] * k_hi <= ed[e];
        bits |= (!(pos || neg) ? 1u : 0u) << e;
      }
      const int mine = __popc(bits);
      int before = mine;                             // inclusive prefix over lanes
      for (int o = 1; o < 64; o <<= 1) {
        const int n = __shfl_up(before, o);
        if (lane >= o) before += n;
      }
      namb = __shfl(before, 63);
      int pos = before - mine;
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if ((bits >> e) & 1u) {
          if (pos < kAmbMax) {
            st_dev(&prm.recU[rc * kAmbMax + pos].x, et[e]);
            st_dev(&prm.recU[rc * kAmbMax + pos].y, ed[e]);
          }
          ++pos;
        }
      }
    }
  }
  // every lane stores the same values (no branch around the stores: a store skipped on some path would leave the
  // compiler's count of outstanding memory operations too low, and the next chunk's wait would also wait for the
  // loads still in flight)
  st_dev(&prm.recA[rc], A);
  st_dev(&prm.recD[rc], D);
  st_dev(&prm.recN[rc], namb);
}

// Chunk loop of the mass pass for one kind of draw (KIND is uniform per sequence): chunks c0, c0 + stride, ... below
// c1. Chunks that lie wholly inside a 16-byte aligned row take the vector loop, with the next two chunks' loads in
// flight while the current one is evaluated; a partial last chunk, or a row off the 16-byte grid, takes element loads.
template <typename T, int KIND>
__device__ __forceinline__ void mass_chunks(DP& prm, const Job& job, int64_t b, int64_t c0, int64_t c1,
                                            int stride, const T* rt, const T* rd, bool vec, double mt,
                                            double& st, double& sd) {
  constexpr int NV = kPer / Vec<T>::kEPV;
  constexpr int EPV = Vec<T>::kEPV;
  const int lane = threadIdx.x & 63;
  const int64_t V = prm.V;
  const double md = job.m_d;
  const double c2 = prm.c2;
  const double nmt = -(mt * c2), nmd = -(md * c2);
  const double k_lo = job.kappa * (1.0 - kBand), k_hi = job.kappa * (1.0 + kBand);
  const int64_t step = int64_t(stride) * kChunk;
  float zt[kPer], zd[kPer];
  // the chunk range is the same in every lane of the wave: kept in scalar registers, so the loop's branches are uniform
  c0 = uniform_i64(c0);
  c1 = uniform_i64(c1);
  const int64_t c_vec = uniform_i64(vec ? min<int64_t>(c1, V / kChunk) : c0);   // chunks below V / kChunk are whole
  int64_t c = c0;
  int64_t i0 = c0 * kChunk + int64_t(lane) * kPer;
  if (c < c_vec) {
    // two buffer sets used in turn (the loop is unrolled twice so that no register copy waits on a load): while
    // chunk c is evaluated, the loads of chunks c + stride and c + 2 * stride are in flight
    uint4 xt[2][NV], xd[2][NV];
    const uint4* pt = reinterpret_cast<const uint4*>(rt + i0);
    const uint4* pd = KIND == JOB_RESID ? reinterpret_cast<const uint4*>(rd + i0) : pt;
    const int64_t vstep = step / EPV;                // in 16-byte vectors
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t ahead = (h == 1 && c + stride < c_vec) ? vstep : 0;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        xt[h][k] = gload4(pt + ahead + k);
        if constexpr (KIND == JOB_RESID) xd[h][k] = gload4(pd + ahead + k);
      }
    }
    // chunk c from buffer set h: unpack, refill the set with the chunk after next (past the last chunk: the current
    // one again, so that every load is unconditional), evaluate
    auto half = [&](uint4 (&bt)[NV], uint4 (&bd)[NV]) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        Vec<T>::unpack(bt[k], zt + k * EPV);
        if constexpr (KIND == JOB_RESID) Vec<T>::unpack(bd[k], zd + k * EPV);
      }
      const int64_t ahead = c + 2 * stride < c_vec ? 2 * vstep : 0;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        bt[k] = gload4(pt + ahead + k);
        if constexpr (KIND == JOB_RESID) bd[k] = gload4(pd + ahead + k);
      }
      chunk_body<KIND>(prm, job, b, c, i0, zt, zd, mt, c2, nmt, nmd, k_lo, k_hi, st, sd);
      c += stride;
      i0 += step;
      pt += vstep;
      pd += vstep;
    };
    while (c + stride < c_vec) {                     // two chunks per pass, one from each set
      half(xt[0], xd[0]);
      half(xt[1], xd[1]);
    }
    if (c < c_vec) half(xt[0], xd[0]);               // an odd last chunk
  }
  for (; c < c1; c += stride, i0 += step) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) zt[e] = elem_or_ninf<T>(rt, i0 + e, V);
    if constexpr (KIND == JOB_RESID) {
#pragma unroll
      for (int e = 0; e < kPer; ++e) zd[e] = elem_or_ninf<T>(rd, i0 + e, V);
    }
    chunk_body<KIND>(prm, job, b, c, i0, zt, zd, mt, c2, nmt, nmd, k_lo, k_hi, st, sd);
  }
}

// Draw weights of the kPT consecutive elements of chunk c that thread tid holds in the search (elements
// kPT * tid .. kPT * tid + kPT - 1), evaluated exactly as chunk_weights does. Every load is issued before the first
// weight is formed.
constexpr int kPT = kChunk / kDrawBlock;
constexpr int kLeanChunks = 512;    // the lean pick: at most 8 chunks per lane (and at most 64 tasks)
template <typename T>
__device__ __forceinline__ void chunk_weights_t(const Job& job, const T* rt, const T* rd, int64_t c, int tid, int64_t V,
                                                double mt, double inv_st, double md, double inv_sd, double c2,
                                                bool use_p, double* w) {
#pragma clang fp contract(off)
  const int64_t i0 = c * kChunk + int64_t(tid) * kPT;
  const bool resid = job.kind == JOB_RESID && !use_p;
  const double nmt = -(mt * c2), nmd = -(md * c2);
  float zt[kPT], zd[kPT];
#pragma unroll
  for (int e = 0; e < kPT; ++e) zt[e] = elem_or_ninf<T>(rt, i0 + e, V);
  if (resid) {
#pragma unroll
    for (int e = 0; e < kPT; ++e) zd[e] = elem_or_ninf<T>(rd, i0 + e, V);
  }
#pragma unroll
  for (int e = 0; e < kPT; ++e) {
    const int64_t i = i0 + e;
    const double p = fexp_scaled(xarg(zt[e], c2, nmt)) * inv_st;
    double q = 0.0;
    if (resid) {
      q = fexp_scaled(xarg(zd[e], c2, nmd)) * inv_sd;
    } else if (!use_p && job.kind == JOB_ONEHOT) {
      q = (i == job.d) ? 1.0 : 0.0;
    }
    const double r = use_p ? p : p - q;
    w[e] = r > 0.0 ? r : 0.0;
  }
}

struct PickShared {
  double mass[kTile];
  int amb[kTile];
  double red[kDrawWaves];
  double base;
  int namb, cand, last, hit, lastpos;
};
__shared__ PickShared s_pick;     // at file scope: reached with LDS instructions from the functions not inlined

// The sequence's drawn token and flags (the scan's bits plus what the draw adds), written once.
__device__ __forceinline__ void finish(DP& prm, int64_t b, const Job& job, int32_t tok, uint32_t extra) {
  prm.token[b] = tok;
  if (prm.flags) prm.flags[b] = job.flags | extra;
  if (job.flags & SV_FLAG_INTERNAL) prm.n_acc[b] = -1;
}

// The exact search inside chunk cstar by the whole workgroup (thread tid holds kPT consecutive elements): the first
// element whose running sum from cbase exceeds t, else (clamp, or rounding) the chunk's last element with weight.
template <typename T>
__device__ __forceinline__ void search_chunk(DP& prm, int64_t b, const Job& job, int64_t cstar, double cbase, bool clamp, double t,
                             double mt, double inv_st, double md, double inv_sd, bool use_p) {
  PickShared& sh = s_pick;
  constexpr int BLOCK = kDrawBlock;
  const int tid = threadIdx.x;
  const bool resid = job.kind == JOB_RESID;
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const T* rd = resid ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  if (tid == 0) { sh.hit = INT_MAX; sh.lastpos = -1; }
  double w[kPT];
  chunk_weights_t<T>(job, rt, rd, cstar, tid, prm.V, mt, inv_st, md, inv_sd, prm.c2, use_p, w);
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kPT; ++e) mine += w[e];
  double tot;
  double acc = cbase + block_excl_scan<BLOCK>(mine, sh.red, tot);
  int hit = INT_MAX, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPT; ++e) {
    acc += w[e];
    if (w[e] > 0.0) lastpos = tid * kPT + e;
    if (hit == INT_MAX && !clamp && w[e] > 0.0 && acc > t) hit = tid * kPT + e;
  }
  if (hit != INT_MAX) atomicMin(&sh.hit, hit);
  if (lastpos >= 0) atomicMax(&sh.lastpos, lastpos);
  __syncthreads();
  if (tid == 0) {
    const int e = sh.hit != INT_MAX ? sh.hit : sh.lastpos;
    finish(prm, b, job, e >= 0 ? int32_t(cstar * kChunk + e) : -1, use_p ? SV_FLAG_EMPTY_RESIDUAL : 0u);
  }
}

// The pick of sequence b by one workgroup, after every task of the sequence has finished: normalisers from the task
// partials, chunk masses, their running sum, the chunk that holds t = u * total, and an exact search inside it.
template <typename T>
__device__ __forceinline__ void pick_seq(DP& prm_arg, int64_t b, const Job& job_arg) {
  PickShared& sh = s_pick;
  const Job job = uniform_job(job_arg);
  DP& prm = uniform_params(prm_arg);
  constexpr int BLOCK = kDrawBlock, NW = kDrawWaves;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const TaskShape shp = task_shape(prm, b);
  const int ntask = shp.ntask;
  const int64_t nch = prm.nch, V = prm.V;
  const double* rA = prm.recA + b * nch;
  const double* rD = prm.recD + b * nch;
  const int32_t* rN = prm.recN + b * nch;
  const double2* rU = prm.recU + b * nch * kAmbMax;
  double* mg = prm.masses + b * nch;
  const double4* ps = prm.part2 + b * prm.ntask2;
  const double c2 = prm.c2;
  const bool resid = job.kind == JOB_RESID, bonus = job.kind == JOB_BONUS;

  // normalisers from the task partials, combined in a fixed order
  double lm = -INFINITY;
  int bad = 0;
  for (int s = tid; s < ntask; s += BLOCK) {
    const double4 p = ld_task(ps + s);
    lm = fmax(lm, p.x);
    bad |= isnan(p.y) || isnan(p.w);
  }
  const double mt = block_max_d<BLOCK>(lm, sh.red);
  bad = __syncthreads_or(bad);
  double lst = 0.0, lsd = 0.0;
  for (int s = tid; s < ntask; s += BLOCK) {
    const double4 p = ld_task(ps + s);
    const double f = (!bonus || p.x == mt) ? 1.0 : (p.x == -INFINITY ? 0.0 : fexp_scaled((p.x - mt) * c2));
    lst += p.y * f;
    lsd += p.w;
  }
  const double St = block_sum<BLOCK>(lst, sh.red);
  const double Sd = block_sum<BLOCK>(lsd, sh.red);
  if (bad || !(St > 0.0) || isinf(mt) || (resid && !(Sd > 0.0))) {    // only a bonus row can be bad here
    if (tid == 0) {
      finish(prm, b, job, -1, SV_FLAG_NONFINITE);
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

  // Masses of the chunks of one tile into sh.mass (and to global memory when there are several tiles).
  auto tile_masses = [&](int64_t t0, int n, bool use_p) {
    if (tid == 0) sh.namb = 0;
    __syncthreads();
    for (int i = tid; i < n; i += BLOCK) {
      const int64_t c = t0 + i;
      const int namb = ld_dev(rN + c);
      if (use_p || namb > kAmbMax) {
        sh.amb[atomicAdd(&sh.namb, 1)] = i;
      } else {
        double f = 1.0;
        if (bonus) {                                   // the chunk's exps are relative to its task's max
          const double mref = ld_dev(reinterpret_cast<const double*>(ps + task_of_chunk(c, shp)));
          f = mref == -INFINITY ? 0.0 : fexp_scaled((mref - mt) * c2);
        }
        double m = f * (ld_dev(rA + c) * inv_st - ld_dev(rD + c) * inv_sd);
        for (int q = 0; q < namb; ++q) {               // undecided elements, exactly: max(p - q, 0)
          const double r = ld_dev(&rU[c * kAmbMax + q].x) * inv_st - ld_dev(&rU[c * kAmbMax + q].y) * inv_sd;
          m += r > 0.0 ? r : 0.0;
        }
        sh.mass[i] = m;
      }
    }
    __syncthreads();
    const int namb = sh.namb;
    for (int q = wave; q < namb; q += NW) {
      const int i = sh.amb[q];
      chunk_weights<T>(job, rt, rd, vec, t0 + i, lane, V, mt, inv_st, md, inv_sd, c2, use_p, w);
      const double m = wave_sum(lane_sum16(w));
      if (lane == 0) sh.mass[i] = m;
    }
    __syncthreads();
    if (!one_tile)
      for (int i = tid; i < n; i += BLOCK) mg[t0 + i] = sh.mass[i];
  };
  // Running sum over one tile: thread-contiguous ranges, exclusive base per thread, tile total.
  auto tile_scan = [&](int n, double& mine_excl, int& ia, int& ib) {
    const int per = (n + BLOCK - 1) / BLOCK;
    ia = min(n, per * tid);
    ib = min(n, per * (tid + 1));
    double mine = 0.0;
    for (int i = ia; i < ib; ++i) mine += sh.mass[i];
    double tot;
    mine_excl = block_excl_scan<BLOCK>(mine, sh.red, tot);
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
  if (tid == 0) { sh.cand = INT_MAX; sh.last = -1; }
  __syncthreads();
  double run = 0.0;
  for (int64_t t0 = 0; t0 < nch; t0 += kTile) {
    const int n = int(min<int64_t>(kTile, nch - t0));
    double tile_total = 0.0;
    if (!one_tile) {
      __threadfence_block();
      __syncthreads();
      for (int i = tid; i < n; i += BLOCK) sh.mass[i] = *reinterpret_cast<const volatile double*>(&mg[t0 + i]);
      __syncthreads();
      tile_total = tile_scan(n, excl, ia, ib);
    }
    double acc = run + excl;
    int cand = INT_MAX, last = -1;
    double cbase = 0.0;
    for (int i = ia; i < ib; ++i) {
      const double m = sh.mass[i];
      if (m > 0.0) last = int(t0 + i);
      if (cand == INT_MAX && acc + m > t) { cand = int(t0 + i); cbase = acc; }
      acc += m;
    }
    atomicMin(&sh.cand, cand);
    atomicMax(&sh.last, last);
    __syncthreads();
    if (cand != INT_MAX && cand == sh.cand) sh.base = cbase;
    __syncthreads();
    if (sh.cand != INT_MAX) break;
    run += tile_total;
  }
  const bool clamp = sh.cand == INT_MAX;
  const int64_t cstar = clamp ? sh.last : sh.cand;
  if (cstar < 0) {
    if (tid == 0) finish(prm, b, job, -1, 0u);
    return;
  }
  search_chunk<T>(prm, b, job, cstar, clamp ? 0.0 : sh.base, clamp, t, mt, inv_st, md, inv_sd, use_p);
}

// The common case of the pick, for rows of at most kLeanChunks chunks and at most 64 draw tasks whose chunk records
// need no recomputation, by wave 0 alone (no barrier, no shared memory): one round of loads brings the task partials
// and every chunk record (lane l holds chunks l, l + 64, l + 128, ...: each load of a record field is 64 consecutive
// values); the normalisers, the chunk masses, their running sum in chunk order (one wave scan per group of 64
// chunks) and the chunk that holds t = u * total follow with wave-level operations; that chunk is then searched with
// the mass pass's layout (lane l holds its kPer consecutive elements). Returns 0 when done (token and flags
// written), 1 when the general pick must run instead (an undecided chunk, an empty residual), with nothing written.
template <typename T>
__device__ __forceinline__ int pick_lean(DP& prm, int64_t b, const Job& job) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = prm.nch, V = prm.V;
  const TaskShape shp = task_shape(prm, b);
  const int ntask = shp.ntask;
  const double c2 = prm.c2;
  const bool resid = job.kind == JOB_RESID, bonus = job.kind == JOB_BONUS;
  const double* rA = prm.recA + b * nch;
  const double* rD = prm.recD + b * nch;
  const int32_t* rN = prm.recN + b * nch;
  constexpr int KM = kLeanChunks / 64;
  const int kb = int((nch + 63) / 64);               // groups of 64 chunks in use (uniform)
  int namb[KM];
  double A[KM], D[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {                     // clamped indices: every load is issued, none is conditional
    namb[k] = 0;
    A[k] = D[k] = 0.0;
    if (k < kb) {
      const int64_t c = min<int64_t>(int64_t(k) * 64 + lane, nch - 1);
      namb[k] = ld_dev(rN + c);
      A[k] = ld_dev(rA + c);
      D[k] = ld_dev(rD + c);
    }
  }
  const bool has_task = lane < ntask;
  const double4 p = ld_task(prm.part2 + b * prm.ntask2 + min(lane, ntask - 1));
  const double mt = wave_max_d(has_task ? p.x : -INFINITY);
  const int bad = __any(has_task && (isnan(p.y) || isnan(p.w)));
  double lst = 0.0, lsd = 0.0, ftask = 1.0;          // ftask: rescaling of task lane's exps to the row max (bonus)
  if (has_task) {
    ftask = (!bonus || p.x == mt) ? 1.0 : (p.x == -INFINITY ? 0.0 : fexp_scaled((p.x - mt) * c2));
    lst = p.y * ftask;
    lsd = p.w;
  }
  const double St = wave_sum(lst), Sd = wave_sum(lsd);
  if (bad || !(St > 0.0) || isinf(mt) || (resid && !(Sd > 0.0))) {     // only a bonus row can be bad here
    if (lane == 0) finish(prm, b, job, -1, SV_FLAG_NONFINITE);
    return 0;
  }
  const double inv_st = 1.0 / St, inv_sd = resid ? 1.0 / Sd : 0.0;
  double m[KM];
  int slow = 0;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    m[k] = 0.0;
    if (k >= kb) continue;
    const int64_t c = int64_t(k) * 64 + lane;
    // the task's rescaling factor, from the lane that holds that task's partial (every lane takes part)
    double f = 1.0;
    if (bonus) f = __shfl(ftask, task_of_chunk(min<int64_t>(c, nch - 1), shp));
    if (c >= nch) continue;
    if (namb[k] > kAmbMax) {
      slow = 1;
      continue;
    }
    m[k] = f * (A[k] * inv_st - D[k] * inv_sd);
    for (int u = 0; u < namb[k]; ++u) {              // undecided elements, exactly: max(p - q, 0)
      const double2* pu = prm.recU + (b * nch + c) * kAmbMax + u;
      const double r = ld_dev(&pu->x) * inv_st - ld_dev(&pu->y) * inv_sd;
      m[k] += r > 0.0 ? r : 0.0;
    }
  }
  if (__any(slow)) return 1;
  // running sums: inclusive scan of each group of 64 chunks, groups in order
  double incl[KM], tot[KM];
  double total = 0.0;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    incl[k] = tot[k] = 0.0;
    if (k >= kb) continue;
    incl[k] = wave_incl_scan(m[k]);
    tot[k] = readlane_d(incl[k], 63);
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) total += tot[k];
  if (!(total > 0.0)) return 1;                      // empty residual: the general pick draws from p
  const double t = double(job.u) * total;

  // the chunk whose running sum first exceeds t (else, rounding, the last chunk with mass)
  int64_t cstar = -1, last = -1;
  double cbase = 0.0, carry = 0.0;
  bool found = false;
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k >= kb) continue;
    if (m[k] > 0.0) last = int64_t(k) * 64 + lane;
    if (!found && carry + tot[k] > t) {
      const uint64_t hm = __ballot(carry + incl[k] > t);
      const int l = hm ? __builtin_ctzll(hm) : 63;
      cstar = int64_t(k) * 64 + l;
      cbase = carry + (readlane_d(incl[k], l) - readlane_d(m[k], l));
      found = true;
    }
    carry += tot[k];
  }
  bool clamp = false;
  if (!found) {
    clamp = true;
    const uint64_t pm = __ballot(last >= 0);
    cstar = -1;
    if (pm) {                                        // the largest chunk index with mass over all lanes
      int64_t best = last;
      for (int o = 1; o < 64; o <<= 1) best = max<int64_t>(best, __shfl_xor(best, o));
      cstar = best;
    }
  }
  if (cstar < 0) {
    if (lane == 0) finish(prm, b, job, -1, 0u);
    return 0;
  }

  // the exact search inside chunk cstar: the first element whose running sum from cbase exceeds t, else (clamp,
  // or rounding) the chunk's last element with weight
  const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
  const T* rd = resid ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(rt) & 15u) == 0 &&
                   (!resid || (reinterpret_cast<uintptr_t>(rd) & 15u) == 0);
  double w[kPer];
  chunk_weights<T>(job, rt, rd, vec, cstar, lane, V, mt, inv_st, double(job.m_d), inv_sd, c2, false, w);
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) mine += w[e];
  const double inc2 = wave_incl_scan(mine);
  double run = cbase + (inc2 - mine);
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    run += w[e];
    if (w[e] > 0.0) lastpos = e;
    if (hit < 0 && !clamp && w[e] > 0.0 && run > t) hit = e;
  }
  int32_t tok = -1;
  const uint64_t hh = __ballot(hit >= 0);
  if (hh) {
    const int l = __builtin_ctzll(hh);
    tok = int32_t(cstar * kChunk + int64_t(l) * kPer + __shfl(hit, l));
  } else {
    const uint64_t lp = __ballot(lastpos >= 0);
    if (lp) {
      const int l = 63 - __builtin_clzll(lp);
      tok = int32_t(cstar * kChunk + int64_t(l) * kPer + __shfl(lastpos, l));
    }
  }
  if (lane == 0) finish(prm, b, job, tok, 0u);
  return 0;
}

// Per-sequence counters. They start at zero (the workspace is zero-filled before its first use) and every launch
// leaves them at zero again: the last draw task of a sequence clears that sequence's counters.
__device__ __forceinline__ int32_t ld_ctr(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The job of sequence b fills a 64-byte aligned slot (one cache line): four 16-byte groups, each with a seal word. The
// scan writes the whole slot with one store instruction (lane i: word i, seals set), and a draw task reads it with one
// load instruction; a 16-byte group moves as a unit, so a group whose seal reads 1 holds this call's words, and a job
// is taken only when all four seals read 1. The sequence's last draw task clears the slot once every task has read
// it (the workspace starts zero-filled: unsealed).
constexpr int kJobWords = int(sizeof(Job) / 4);
static_assert(kJobWords == 16, "a job is four 16-byte groups");
__device__ __forceinline__ uint32_t* job_slot(DP& prm, int64_t b) {
  return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(prm.jobs) + b * kJobStride);
}
// By every lane of one wave; j is the same in every lane.
__device__ __forceinline__ void st_job(uint32_t* slot, const Job& j) {
  const int lane = threadIdx.x & 63;
  Job s = j;
  s.seal0 = s.seal1 = s.seal2 = s.seal3 = 1u;
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&s);
  uint32_t v = 0;
#pragma unroll
  for (int i = 0; i < kJobWords; ++i) v = lane == i ? w[i] : v;
  if (lane < kJobWords) st_dev(slot + lane, v);
}
// By every lane of one wave. Polls until sealed (at most kSpinCap times); returns false when it gave up.
__device__ __forceinline__ bool ld_job_sealed(const uint32_t* slot, Job& j) {
  const int lane = threadIdx.x & 63;
  uint32_t w = 0;
  int32_t polls = 0;
  for (;;) {
    w = lane < kJobWords ? ld_dev(slot + lane) : 0u;
    const bool sealed = (__builtin_amdgcn_readlane(w, 3) & __builtin_amdgcn_readlane(w, 7) &
                         __builtin_amdgcn_readlane(w, 11) & __builtin_amdgcn_readlane(w, 15)) != 0u;
    if (sealed || ++polls >= kSpinCap) break;
    __builtin_amdgcn_s_sleep(kSleep);
  }
  uint32_t* d = reinterpret_cast<uint32_t*>(&j);
#pragma unroll
  for (int i = 0; i < kJobWords; ++i) d[i] = __builtin_amdgcn_readlane(w, i);
  return polls < kSpinCap;
}

// What workgroup i does. The queue holds, in this order: steps s = 0 .. B-1, each the statistics items of sequence s
// followed by the scan of sequence s - lag1 (when s >= lag1), so that a scan comes about one resident round of
// statistics items after its own; then the scans of the last lag1 sequences; then the draw slots. The hardware
// dispatches each XCD's share of the workgroups in index order, so every scan waits only on lower-indexed items. A
// draw slot takes the next draw task from a ticket counter when it starts (tasks in sequence order), which keeps the
// XCDs busy until the last task whatever their relative speed; its job's scan lies before every draw slot.
enum ItemKind : int32_t { ITEM_STATS = 0, ITEM_SCAN = 1, ITEM_DRAW = 2 };
struct ItemRef {
  int32_t kind;
  int32_t b;
  int32_t sub;    // statistics item within the sequence (draw slots: unused)
};
__device__ __forceinline__ ItemRef decode_item(uint32_t i, uint32_t B, uint32_t n1, uint32_t lag1) {
  const uint32_t head = lag1 * n1;                         // steps before the first scan: statistics only
  const uint32_t body = head + (B - lag1) * (n1 + 1);
  if (i < head) return ItemRef{ITEM_STATS, int32_t(i / n1), int32_t(i % n1)};
  if (i < body) {
    const uint32_t j = i - head, s = lag1 + j / (n1 + 1), k = j % (n1 + 1);
    if (k < n1) return ItemRef{ITEM_STATS, int32_t(s), int32_t(k)};
    return ItemRef{ITEM_SCAN, int32_t(s - lag1), 0};
  }
  if (i < body + lag1) return ItemRef{ITEM_SCAN, int32_t(B - lag1 + (i - body)), 0};
  return ItemRef{ITEM_DRAW, 0, 0};
}

struct DrawShared {
  Job job;
  int32_t ticket;
  float max[kDrawWaves];
  int nan[kDrawWaves];
  double sum[kDrawWaves][2];
};
// Workgroup-shared state of the draw tasks and the pick, at file scope so that the functions that are not inlined
// reach it with LDS instructions (a reference parameter would be a generic pointer: flat accesses through the vector
// memory path).
__shared__ DrawShared s_draw;
__shared__ int s_flag;


__device__ __forceinline__ void ctr_inc(int32_t* p) {
  (void)__hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Waits (thread 0 polls, the others hold at the barrier) until the counter reaches `target`. Returns false when it
// gave up after kSpinCap polls, which only happens if the hardware broke the dispatch order; the workspace is then
// marked so that the next call clears its control words.
// With sig != 0 the header is confirmed first (the counter is a control word).
__device__ __forceinline__ bool wait_count(const int32_t* ctr, int32_t target, char* ws, uint64_t sig = 0) {
  if (threadIdx.x == 0) {
    int32_t polls = 0;
    if (sig != 0 && !ws_seen_clean(ws, sig) && !ws_ready(ws, sig)) polls = kSpinCap;
    while (polls < kSpinCap && ld_ctr(ctr) < target) {
      __builtin_amdgcn_s_sleep(kSleep);
      ++polls;
    }
    s_flag = polls < kSpinCap;
    if (!s_flag) ws_mark_dirty(ws);
  }
  __syncthreads();
  return s_flag != 0;
}

// The job of a sequence that could not be verified because a hand-off inside the launch failed: nothing is drawn.
__device__ __forceinline__ Job internal_fault_job() {
  Job j{};
  j.kind = JOB_NONE;
  j.flags = SV_FLAG_INTERNAL;
  j.new_start = -1;
  return j;
}

// Draw task `task` of sequence b, once its job is published: the float64 masses of the task's chunks of the draw
// row(s) (see task_shape), dealt to the waves in turn, and the task's partial normalisers. Returns true in the
// workgroup of the sequence's last task once every task of the sequence has counted itself.
template <typename T>
__device__ __forceinline__ bool draw_task(DP& prm_arg, int64_t b, int task, const Job& job_arg) {
  DP& prm = uniform_params(prm_arg);
  const Job job = uniform_job(job_arg);
  DrawShared& ds = s_draw;
  constexpr int NW = kDrawWaves;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (job.kind != JOB_NONE) {                       // uniform over the workgroup
    const int64_t V = prm.V;
    const TaskShape shp = task_shape(prm, b);
    const int64_t cbeg = int64_t(task) * shp.chunks;
    const int64_t c1 = min<int64_t>(cbeg + shp.chunks, prm.nch);
    const int64_t c0 = cbeg + (wave + NW / 2) % NW;
    const T* rt = static_cast<const T*>(prm.tgt) + b * prm.t_seq + int64_t(job.row) * prm.t_row;
    const bool resid = job.kind == JOB_RESID;
    const T* rd = resid ? static_cast<const T*>(prm.dft) + b * prm.d_seq + int64_t(job.row) * prm.d_row : nullptr;
    const bool vec = (reinterpret_cast<uintptr_t>(rt) & 15u) == 0 &&
                     (!resid || (reinterpret_cast<uintptr_t>(rd) & 15u) == 0);
    double mt = job.m_t;
    int has_nan = 0;
    if (job.kind == JOB_BONUS) {            // the bonus row was not in the statistics items: this task's max
      float zt[kPer];
      float m = -INFINITY;
      for (int64_t c = c0; c < c1; c += NW) {
        load_lane<T>(rt, c * kChunk + int64_t(lane) * kPer, V, vec, zt);
#pragma unroll
        for (int e = 0; e < kPer; ++e) { m = fmaxf(m, zt[e]); has_nan |= (zt[e] != zt[e]); }
      }
      m = wave_max_f(m);
      has_nan = __any(has_nan);
      if (lane == 0) { ds.max[wave] = m; ds.nan[wave] = has_nan; }
      __syncthreads();
      m = ds.max[0];
      has_nan = ds.nan[0];
      for (int i = 1; i < NW; ++i) { m = fmaxf(m, ds.max[i]); has_nan |= ds.nan[i]; }
      mt = m;
    }
    double st = 0.0, sd = 0.0;
    if (mt == -INFINITY) {                  // a task of -inf only (bonus row): no mass
      if (lane == 0) {
        for (int64_t c = c0; c < c1; c += NW) {
          st_dev(&prm.recA[b * prm.nch + c], 0.0);
          st_dev(&prm.recD[b * prm.nch + c], 0.0);
          st_dev(&prm.recN[b * prm.nch + c], 0);
        }
      }
    } else if (resid) {
      mass_chunks<T, JOB_RESID>(prm, job, b, c0, c1, NW, rt, rd, vec, mt, st, sd);
    } else if (job.kind == JOB_ONEHOT) {
      mass_chunks<T, JOB_ONEHOT>(prm, job, b, c0, c1, NW, rt, rd, vec, mt, st, sd);
    } else {
      mass_chunks<T, JOB_BONUS>(prm, job, b, c0, c1, NW, rt, rd, vec, mt, st, sd);
    }
    st = wave_sum(st);
    if (resid) sd = wave_sum(sd);
    if (lane == 0) { ds.sum[wave][0] = st; ds.sum[wave][1] = sd; }
    __syncthreads();
    if (tid == 0) {
      double S = 0.0, D = 0.0;
      for (int i = 0; i < NW; ++i) { S += ds.sum[i][0]; D += ds.sum[i][1]; }
      st_task(prm.part2 + b * prm.ntask2 + task, make_double4(mt, has_nan ? NAN : S, job.m_d, D));
    }
  }
  // this workgroup's records are complete before it is counted (the count does not wait for a reply); the
  // sequence's last task picks once every task has counted itself (the others were dispatched before it)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  int32_t* done = prm.done + b * kCtrStride;
  if (tid == 0) ctr_inc(done);
  const int32_t nt_b = task_shape(prm, b).ntask;
  if (task != nt_b - 1) return false;
  if (!wait_count(done, nt_b, prm.ws)) {            // gave up: report the sequence as not verified
    if (tid == 0) {
      prm.token[b] = -1;
      prm.n_acc[b] = -1;
      if (prm.flags) prm.flags[b] = SV_FLAG_INTERNAL;
    }
    return false;
  }
  return true;
}


// One workgroup per work item, in the queue order of decode_item (the hardware dispatches workgroups in index
// order, so everything a workgroup waits for was dispatched before it and is running or done):
//  - statistics item: streams its segment, writes its partial and counts itself on the sequence's counter;
//  - scan: once the sequence's statistics are all counted, the accept tests, the first-rejection scan, the per-row
//    outputs and the draw job, published by one more count;
//  - draw task: once the job is published, the float64 masses of its chunks; the last task of the sequence picks the
//    token and returns the sequence's counters to zero.
template <typename T>
__global__ __launch_bounds__(kDrawBlock) __attribute__((amdgpu_waves_per_eu(kWpe, kWpe))) void k_verify(DenseParams kp) {
  (void)kp;
  DP& prm = kernel_params();
  __shared__ float sh_f[kDrawWaves];
  __shared__ double sh_d[kDrawWaves];
  __shared__ uint32_t seen[SV_MAX_GAMMA / 32];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const ItemRef it = decode_item(blockIdx.x, uint32_t(prm.B), uint32_t(prm.n1), uint32_t(prm.lag1));
  const int64_t b = it.b;
  int32_t* ready = prm.ready + b * kCtrStride;
  // workgroup 0 (a statistics item) makes sure the control words are at zero for this call's layout; every other
  // workgroup sees the header name this layout as clean before it touches a control word
  if (blockIdx.x == 0) ws_claim(prm.ws, prm.sig, size_t(prm.ctl_end), &s_flag);
  if (it.kind == ITEM_STATS) {
    const bool seen = blockIdx.x == 0 || ws_seen_clean(prm.ws, prm.sig);   // read while the segment streams
    stats_item<T, kStatsBlock, kUnroll, kNonTemporal>(prm, b, it.sub, sh_f, sh_d);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      if (seen || ws_ready(prm.ws, prm.sig)) ctr_inc(ready);
      else ws_mark_dirty(prm.ws);                    // not counted: the scan gives up and flags the sequence
    }
    return;
  }
  if (it.kind == ITEM_SCAN) {
    // the scan and the pick are short serial chains on the critical path: their waves get issue priority over the
    // streaming and float64 waves that share their SIMDs
    __builtin_amdgcn_s_setprio(3);
    const bool ok = wait_count(ready, prm.n1, prm.ws, prm.sig);
    if (wave == 0) {
      Job j;
      if (ok) {
        j = seq_scan(prm, b, true, seen);
      } else {                                       // gave up waiting: report the sequence as not verified
        j = internal_fault_job();
      }
      st_job(job_slot(prm, b), j);                   // published: the draw tasks take it once sealed
    }
    return;
  }
  // draw slot: the next draw task from the ticket counter (tickets in sequence order, task order within a sequence),
  // then that sequence's job. There are more draw slots than tasks: the XCDs that run faster start more slots and take more of
  // the tasks; a slot that finds none left ends at once.
  fexp_fill_table();                                 // the draw's exp2 table
  const int64_t ntot = prm.ntot;
  const int64_t head = (prm.B - prm.tailq) * int64_t(prm.ntask);    // tickets of the sequences with large tasks
  auto seq_of = [&](int64_t t) { return t < head ? t / prm.ntask : prm.B - prm.tailq + (t - head) / prm.ntask2; };
  auto task_of = [&](int64_t t) { return int(t < head ? t % prm.ntask : (t - head) % prm.ntask2); };
  if (wave == 0) {
    int32_t tk = 0;
    if (lane == 0) {
      if (ws_seen_clean(prm.ws, prm.sig) || ws_ready(prm.ws, prm.sig)) {
        tk = __hip_atomic_fetch_add(prm.tickets, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the slot that takes the last ticket of this call returns the counter to zero for the next call (every
        // other slot has taken its ticket already)
        if (tk == prm.nslots - 1) st_dev(prm.tickets, 0);
      } else {
        tk = -1;                                     // no ticket: the sequences' last tasks give up and flag them
        ws_mark_dirty(prm.ws);
      }
    }
    tk = __builtin_amdgcn_readfirstlane(tk);
    Job j{};
    if (tk >= 0 && tk < ntot) {
      const bool sealed = ld_job_sealed(job_slot(prm, seq_of(tk)), j);
      // every field that becomes an address or an index is checked first: a job that gave up waiting or does not
      // fit this call is not drawn from, and its sequence is reported as not verified
      if (!sealed || !job_valid(j, prm.G, prm.V, prm.bonus, prm.dft != nullptr)) {
        if (!sealed && lane == 0) ws_mark_dirty(prm.ws);
        j = internal_fault_job();
      }
    }
    if (lane == 0) { s_draw.job = j; s_draw.ticket = tk; }
  }
  __syncthreads();
  const int32_t tk = __builtin_amdgcn_readfirstlane(s_draw.ticket);
  if (tk < 0 || tk >= ntot) return;
  const int64_t bd = seq_of(tk);
  const Job job = uniform_job(s_draw.job);
  if (draw_task<T>(prm, bd, task_of(tk), job)) {
    const int64_t b = bd;
    __builtin_amdgcn_s_setprio(3);
    if (tid == 0 && prm.start && job.new_start >= 0) prm.start[b] = job.new_start;
    if (job.kind == JOB_NONE) {
      if (tid == 0) finish(prm, b, job, -1, 0u);
    } else {
      int general = 1;
      if (prm.nch <= kLeanChunks && task_shape(prm, b).ntask <= 64) {
        if (wave == 0) {
          const int r = pick_lean<T>(prm, b, job);
          if (lane == 0) s_flag = r;
        }
        __syncthreads();
        general = s_flag;
      }
      if (general) pick_seq<T>(prm, b, job);
    }
    if (tid == 0) {                                  // every item of sequence b has finished
      st_dev(prm.ready + b * kCtrStride, 0);
      st_dev(prm.done + b * kCtrStride, 0);
    }
    if (tid < kJobWords) st_dev(job_slot(prm, b) + tid, 0u);
  }
}


template <typename T>
hipError_t launch_typed(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  char* ws = a.ws;
  const double T_ = double(a.temperature);
  const float c = float(1.4426950408889634074 / T_);          // log2(e) / T
  DenseParams dp{};
  dp.tgt = a.tgt; dp.t_seq = a.t_seq; dp.t_row = a.t_row;
  dp.dft = a.dft; dp.d_seq = a.d_seq; dp.d_row = a.d_row;
  dp.B = plan.B; dp.G = plan.G; dp.V = plan.V; dp.nseg1 = plan.nseg1; dp.ntens = plan.ntens; dp.bonus = a.bonus;
  dp.c = c; dp.c2 = 1.4426950408889634074 / T_;
  dp.ids = a.ids; dp.ua = a.ua; dp.us = a.us; dp.start = a.start; dp.order = a.order;
  dp.accept = a.accept; dp.n_acc = a.n_acc; dp.token = a.token; dp.p_draft = a.p_draft; dp.q_draft = a.q_draft;
  dp.flags = a.flags;
  dp.n1 = plan.n1; dp.ntask = plan.ntask; dp.nch = plan.nch; dp.nslots = int32_t(plan.nslots);
  dp.ntask2 = plan.ntask2; dp.tailq = int32_t(plan.tailq); dp.ntot = plan.ntot; dp.chunks1 = plan.chunks1;
  const int R = resident_workgroups();
  auto lag_for = [&](int64_t rounds) {          // sequences whose statistics fill `rounds` resident rounds
    if (rounds <= 0) return int64_t(plan.B);
    int64_t l = (int64_t(R) * rounds + plan.n1 - 1) / plan.n1;
    return l < 1 ? int64_t(1) : (l > plan.B ? plan.B : l);
  };
  dp.lag1 = int32_t(lag_for(kScanLagRounds));
  dp.n_items = int32_t(plan.B * (int64_t(plan.n1) + 1) + plan.nslots);
  dp.ready = reinterpret_cast<int32_t*>(ws + plan.off_ready);
  dp.done = reinterpret_cast<int32_t*>(ws + plan.off_done);
  dp.tickets = reinterpret_cast<int32_t*>(ws + plan.off_tickets);
  dp.jobs = reinterpret_cast<Job*>(ws + plan.off_jobs);
  dp.part1 = reinterpret_cast<Partial1*>(ws + plan.off_part1);
  dp.part2 = reinterpret_cast<double4*>(ws + plan.off_part2);
  dp.recA = reinterpret_cast<double*>(ws + plan.off_recA);
  dp.recD = reinterpret_cast<double*>(ws + plan.off_recD);
  dp.recN = reinterpret_cast<int32_t*>(ws + plan.off_recN);
  dp.recU = reinterpret_cast<double2*>(ws + plan.off_recU);
  dp.masses = reinterpret_cast<double*>(ws + plan.off_masses);
  // the control words (per-sequence counters, the draw ticket, the job slots) sit at positions set by B alone
  dp.ws = ws;
  dp.sig = ws_signature(kLayoutDense, uint64_t(plan.B));
  dp.ctl_end = int64_t(plan.off_part1);
  const unsigned grid = unsigned(dp.n_items);
  auto kern = k_verify<T>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kDrawBlock), 0, stream, dp);
  return hipGetLastError();
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace

// Resident workgroups of the kernel on the current device (compute units x workgroups per compute unit).
int resident_workgroups() {
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
  return ncu * kWpe;                 // kWpe 4-wave workgroups per compute unit at kWpe waves per SIMD
}

DensePlan make_dense_plan(int64_t B, int32_t G, int64_t V, int32_t ntens, int dtype, int64_t resident) {
  DensePlan p;
  p.B = B; p.G = G; p.V = V; p.ntens = ntens;
  const int64_t es = dtype == SV_BF16 ? 2 : 4;
  // statistics items of about kItemBytes of logits, at least 8192 elements each
  int64_t s1 = (V * es + kItemBytes - 1) / kItemBytes;
  const int64_t cap1 = V / 8192 > 1 ? V / 8192 : 1;
  if (s1 > cap1) s1 = cap1;
  if (s1 < 1) s1 = 1;
  p.nseg1 = int32_t(s1);
  p.n1 = int64_t(ntens) * G * s1;
  // draw: rows cut into chunks of kChunk elements, consecutive chunks per task
  p.nch = (V + kChunk - 1) / kChunk;
  const int64_t R = std::max<int64_t>(1, resident);
  int64_t chunks1 = kTaskChunks;
  while (chunks1 < kTaskChunksMax && B * ((p.nch + chunks1 - 1) / chunks1) > kTasksPerSlot * R) chunks1 *= 2;
  p.chunks1 = int32_t(chunks1);
  int64_t ntask = (p.nch + chunks1 - 1) / chunks1;
  if (ntask < 1) ntask = 1;
  p.ntask = int32_t(ntask);
  int64_t ntask2 = (p.nch + kTailChunks - 1) / kTailChunks;
  if (ntask2 < ntask) ntask2 = ntask;
  p.ntask2 = int32_t(ntask2);
  p.tailq = std::max<int64_t>(1, std::min<int64_t>(B, (kTailSlots * R + p.nch - 1) / p.nch));
  p.ntot = (B - p.tailq) * ntask + p.tailq * ntask2;
  // draw slots: the tasks plus kDrawSlackPct percent more, so that a faster XCD can take more than its share
  p.nslots = p.ntot + std::min<int64_t>((p.ntot * kDrawSlackPct + 99) / 100, kDrawSlackMax);
  size_t off = kWsHeaderBytes;
  p.off_ready = off; off = align_up(off + size_t(B) * kCtrStride * sizeof(int32_t), 256);
  p.off_done = off;  off = align_up(off + size_t(B) * kCtrStride * sizeof(int32_t), 256);
  p.off_tickets = off; off = align_up(off + kCtrStride * sizeof(int32_t), 256);
  p.off_jobs = off;  off = align_up(off + size_t(B) * kJobStride, 256);
  p.off_part1 = off; off = align_up(off + size_t(ntens) * size_t(B) * G * p.nseg1 * sizeof(Partial1), 256);
  p.off_part2 = off; off = align_up(off + size_t(B) * p.ntask2 * sizeof(double4), 256);
  p.off_recA = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(double), 256);
  p.off_recD = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(double), 256);
  p.off_recN = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(int32_t), 256);
  p.off_recU = off; off = align_up(off + size_t(B) * size_t(p.nch) * kAmbMax * sizeof(double2), 256);
  p.off_masses = off; off = align_up(off + size_t(B) * size_t(p.nch) * sizeof(double), 256);
  p.total = off;
  return p;
}

// The current device's copy of `scratch`, looked up once per device (with that device current) and kept.
hipError_t noalloc_scratch(char** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static char* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<char*>(p);
  }
  *out = addr[dev];
  return hipSuccess;
}

hipError_t launch_dense(const DensePlan& plan, const DenseArgs& a, hipStream_t stream) {
  if (a.dtype == SV_BF16) return launch_typed<uint16_t>(plan, a, stream);
  return launch_typed<float>(plan, a, stream);
}

}  // namespace sv
