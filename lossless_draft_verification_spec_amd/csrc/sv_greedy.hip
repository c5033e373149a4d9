// Greedy (T = 0) verification (DFlash/DFlash2 guide, section 4.4: under greedy decoding a drafted token is kept
// exactly when it is the target's most likely token, and the block is cut at the first token that is not; the
// target's choice is emitted there, or the bonus token when every draft is kept, section 2).
//
// One launch, one streaming pass over the target rows. The only per-row statistic is the argmax (equal maxima go to
// the lowest id), so the kernel is a plain HBM-bound reduction: no exponentials, no second pass.
//
//  * Work items: every target row of every sequence is cut into S equal segments, S the smallest count that gives
//    the launch about as many workgroups as the device holds at once (S = 1, whole rows, once there are that many
//    rows: every workgroup pays a start-up and a hand-over latency, so fewer and longer items stream faster); one
//    workgroup per (sequence, row, segment), segment index fastest, so the rows of a sequence finish together.
//  * A segment is streamed in 16 KB chunks of 16-byte non-temporal loads, the next chunk's loads in flight while the
//    current one is folded (a misaligned head or tail of a few elements is read singly). Each thread folds a chunk
//    with the NaN-propagating maximum (v_maximum3_f32: one instruction per two logits) and, only when that beats its
//    running maximum, finds the chunk's first element equal to it, so every thread ends with its maximum and the
//    lowest index holding it. A NaN or +inf makes a chunk maximum NaN or +inf: that is the fault test.
//  * The segment's result is one 64-bit key: the order-preserving code of M in the high word and the complement of
//    its index in the low word, so the largest key is the row maximum with the lowest index; a faulty segment
//    writes the largest key of all. Keys go to the workspace (device-scope stores); a per-sequence counter elects
//    the sequence's last workgroup, which merges the keys of every row in LDS, walks the slots in
//    verification order and writes the outputs. It returns the counter to 0, so the workspace is ready for the next
//    call without a clearing pass.
//  * Rows of slots before `start` are not read (their workgroups only count themselves in); the bonus row is read
//    with the others whenever the sequence is live, and used only when every verified draft matches.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "sv.h"
#include "sv_device.h"
#include "sv_greedy.h"
#include "sv_internal.h"
#include "sv_wshdr.h"

namespace sv {
namespace {

constexpr int kGrBlock = 256;
constexpr int kGrWaves = kGrBlock / 64;
constexpr int kGrU = 4;                                     // 16-byte vectors per thread per chunk
constexpr int64_t kGrChunkVec = int64_t(kGrBlock) * kGrU;   // vectors per chunk (16 KB)
constexpr uint64_t kFaultKey = ~0ull;                       // a segment holding a NaN or +inf
constexpr uint32_t kOrdNegInf = 0x007FFFFFu;                // ord_bits(-inf)
constexpr float kLog2e = 1.4426950408889634f;

struct GreedyParams {
  const void* tgt;
  int64_t t_seq, t_row;
  int64_t V;
  int64_t seg_elems;           // elements per segment (a multiple of the chunk)
  int32_t G, R, S;             // gamma, rows per sequence (gamma + bonus), segments per row
  int32_t bonus;
  const int32_t* ids;
  int32_t* start;
  const int32_t* order;
  uint8_t* accept;
  int32_t* n_acc;
  int32_t* token;
  uint32_t* flags;
  char* ws;                    // the workspace; its header names the control layout at zero
  uint64_t sig;                // this call's control layout
  int64_t ctl_end;             // control words (the counters) fill [kWsHeaderBytes, ctl_end)
  int32_t* ctr;                // per sequence: workgroups finished
  uint64_t* part;              // per (sequence, row, segment): the segment's key
  // confidence-threshold commit (CONF kernels): W = G slots, no bonus row
  const uint8_t* masked;       // [B][W] or null (all masked)
  double tau;
  uint8_t* commit;             // [B][W] or null
  float* conf;                 // [B][W] or null
  float2* part2;               // per (sequence, row, segment): (segment maximum, sum of exp(z - maximum))
};

struct GrShared {
  uint64_t wkey[kGrWaves];
  uint32_t wfault[kGrWaves];
  int32_t slot;                // verification slot of this workgroup's row
  int32_t last;                // this workgroup merges the sequence
  int32_t kmin;                // first mismatching slot
  uint32_t fl;                 // the sequence's flags
  float wsum[kGrWaves];
  uint32_t seen[SV_MAX_GAMMA / 32];
  uint64_t rowkey[SV_MAX_GAMMA + 1];
  double rowconf[SV_MAX_GAMMA];   // CONF merge: the slot's confidence
  uint64_t best;                  // CONF merge: the largest confidence (its bits)
  int32_t bestj;
  int32_t any;
};

// Order-preserving code of a float's bits (larger float, larger code), -0 taken as +0 so that equal values tie.
__device__ __forceinline__ uint32_t ord_bits(float x) {
  const uint32_t u = __float_as_uint(x == 0.0f ? 0.0f : x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float maximum3(float a, float b, float c) {
  return __builtin_elementwise_maximum(a, __builtin_elementwise_maximum(b, c));
}

template <typename T>
__device__ __forceinline__ uint4 ninf_vec() {
  const uint32_t w = sizeof(T) == 2 ? 0xFF80FF80u : 0xFF800000u;   // -inf in every element
  return make_uint4(w, w, w, w);
}

// One chunk of the thread's vectors: vector u of chunk c is vp[c * kGrChunkVec + u * kGrBlock + t]. Vectors past
// the segment's end read its last vector instead (fold_chunk counts them as -inf). Branch-free, so that the
// compiler's wait counts see the same loads on every path. Requires nv >= 1.
__device__ __forceinline__ void load_chunk(uint4 (&w)[kGrU], const uint4* vp, int c, int64_t nv, int t) {
  const int64_t base = int64_t(c) * kGrChunkVec + t;
#pragma unroll
  for (int u = 0; u < kGrU; ++u) {
    const int64_t j = base + int64_t(u) * kGrBlock;
    w[u] = load_vec<true>(vp + (j < nv ? j : nv - 1));
  }
}

// Folds one chunk into the thread's running (maximum m, lowest index mi holding it). The chunk maximum is
// NaN-propagating, so a NaN or +inf sets `bad`; only a chunk whose maximum beats m is searched for its first
// element equal to that maximum (elements are visited last to first, so the final match is the lowest index).
template <typename T, bool CONF>
__device__ __forceinline__ void fold_chunk(const uint4 (&w)[kGrU], int c, int64_t nv, int t, int64_t elem0, float& m,
                                          int64_t& mi, bool& bad, float& sum) {
  constexpr int E = Vec<T>::kEPV;
  const int64_t base = int64_t(c) * kGrChunkVec + t;
  const bool full = int64_t(c + 1) * kGrChunkVec <= nv;
  float v[kGrU][E];
#pragma unroll
  for (int u = 0; u < kGrU; ++u) {
    uint4 x = w[u];
    if (!full) {                           // uniform: only a segment's last chunk can run past its end
      const bool ok = base + int64_t(u) * kGrBlock < nv;
      const uint4 ni = ninf_vec<T>();
      x.x = ok ? x.x : ni.x;
      x.y = ok ? x.y : ni.y;
      x.z = ok ? x.z : ni.z;
      x.w = ok ? x.w : ni.w;
    }
    Vec<T>::unpack(x, v[u]);
  }
  float cm = -INFINITY;
#pragma unroll
  for (int u = 0; u < kGrU; ++u)
#pragma unroll
    for (int e = 0; e < E; e += 2) cm = maximum3(cm, v[u][e], v[u][e + 1]);
  bad |= !(cm < INFINITY);
  if (cm > m) {
    int pos = 0;
#pragma unroll
    for (int u = kGrU - 1; u >= 0; --u)
#pragma unroll
      for (int e = E - 1; e >= 0; --e)
        if (v[u][e] == cm) pos = u * kGrBlock * E + e;
    if constexpr (CONF) sum *= ex2f((m - cm) * kLog2e);   // m = -inf the first time: the empty sum stays 0
    m = cm;
    mi = elem0 + pos;
  }
  if constexpr (CONF) {                    // sum of exp(z - m) with m the running maximum (masked-off lanes: -inf)
    if (m > -INFINITY) {
      // exp(z - m) = 2^(z log2(e) - m log2(e)): one fused multiply-add per element before the exp2
      const float nml = -(m * kLog2e);
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < kGrU; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) acc += ex2f(fmaf(v[u][e], kLog2e, nml));
      sum += acc;
    }
  }
}

__device__ __forceinline__ uint64_t make_key(float v, int64_t i) {
  return (uint64_t(ord_bits(v)) << 32) | (i < 0 ? 0ull : uint64_t(~uint32_t(i)));
}

__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
  uint32_t hi = uint32_t(v >> 32), lo = uint32_t(v);
#define SV_GR_STEP(CTRL)                                                                              \
  {                                                                                                   \
    const uint32_t oh = uint32_t(dpp_i<CTRL>(int(hi), int(hi))), ol = uint32_t(dpp_i<CTRL>(int(lo), int(lo))); \
    const bool take = oh > hi || (oh == hi && ol > lo);                                               \
    hi = take ? oh : hi;                                                                              \
    lo = take ? ol : lo;                                                                              \
  }
  SV_GR_STEP(kDppXor1)
  SV_GR_STEP(kDppXor2)
  SV_GR_STEP(kDppHalfMirror)
  SV_GR_STEP(kDppMirror)
#undef SV_GR_STEP
  uint64_t best = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint64_t k = (uint64_t(uint32_t(__builtin_amdgcn_readlane(int(hi), 16 * r))) << 32) |
                       uint64_t(uint32_t(__builtin_amdgcn_readlane(int(lo), 16 * r)));
    best = k > best ? k : best;
  }
  return best;
}

// The key of logits [e0, e1) of one row (see the file comment). Every thread of the workgroup calls it. CONF: also
// the segment's sum of exp(z - M), M its maximum, in `ssum`.
template <typename T, bool CONF>
__device__ uint64_t segment_key(const T* row, int64_t e0, int64_t e1, GrShared& sh, float& ssum) {
  constexpr int E = Vec<T>::kEPV;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;

  // 16-byte aligned vector part [v0, v1) and up to 2 (E - 1) single elements around it.
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(row + e0);
  int64_t v0 = e0 + int64_t(((16u - uint32_t(a0 & 15u)) & 15u) / sizeof(T));
  if (v0 > e1) v0 = e1;
  const int64_t nv = (e1 - v0) / E;
  const int64_t v1 = v0 + nv * E;
  const uint4* vp = reinterpret_cast<const uint4*>(row + v0);
  const int nh = int(v0 - e0), ns = nh + int(e1 - v1);
  const int nch = int((nv + kGrChunkVec - 1) / kGrChunkVec);

  // The first chunk's loads go out before anything waits; the single elements follow (branch-free: threads
  // without one read element e0 and ignore it).
  uint4 cur[kGrU];
  if (nch > 0) load_chunk(cur, vp, 0, nv, t);
  const bool has_s = t < ns;
  const int64_t sidx = has_s ? (t < nh ? e0 + t : v1 + (t - nh)) : -1;
  const float sraw = Vec<T>::load1(row + (has_s ? sidx : e0));

  // Stream the chunks through two register buffers, the next chunk's loads in flight while the current one is
  // folded. The loads are unconditional (a chunk index past the end reads the segment's last vector in every lane:
  // one cache line), so that the wait counts are exact on every path; only the folds are skipped.
  float m = -INFINITY;
  int64_t mi = -1;
  bool bad = false;
  float sum = 0.0f;
  uint4 nxt[kGrU];
  for (int c = 0; c < nch; c += 2) {
    load_chunk(nxt, vp, c + 1, nv, t);
    fold_chunk<T, CONF>(cur, c, nv, t, v0 + (int64_t(c) * kGrChunkVec + t) * E, m, mi, bad, sum);
    load_chunk(cur, vp, c + 2, nv, t);
    if (c + 1 < nch)
      fold_chunk<T, CONF>(nxt, c + 1, nv, t, v0 + (int64_t(c + 1) * kGrChunkVec + t) * E, m, mi, bad, sum);
  }

  // Workgroup maximum key and fault test.
  const float sval = has_s ? sraw : -INFINITY;
  bad |= !(sval < INFINITY);
  uint64_t key = make_key(m, mi);
  const uint64_t ks = make_key(sval, sidx);
  key = ks > key ? ks : key;
  const uint64_t fb = __ballot(bad);
  const uint64_t wk = wave_max_key(key);
  if (lane == 0) {
    sh.wkey[wave] = wk;
    sh.wfault[wave] = fb != 0;
  }
  __syncthreads();
  uint64_t best = sh.wkey[0];
  uint32_t anyf = sh.wfault[0];
#pragma unroll
  for (int w = 1; w < kGrWaves; ++w) {
    best = sh.wkey[w] > best ? sh.wkey[w] : best;
    anyf |= sh.wfault[w];
  }
  if (anyf) return kFaultKey;
  if constexpr (CONF) {
    // the workgroup's sum, every thread's sum rescaled to the segment maximum (taken from the key)
    const uint32_t hb = uint32_t(best >> 32);
    const float M = __uint_as_float((hb & 0x80000000u) ? (hb & 0x7FFFFFFFu) : ~hb);
    float mine = sum > 0.0f ? sum * ex2f((m - M) * kLog2e) : 0.0f;
    if (has_s && sval > -INFINITY) mine += ex2f((sval - M) * kLog2e);
    const float ws = float(wave_sum(double(mine)));
    __syncthreads();
    if (lane == 0) sh.wsum[wave] = ws;
    __syncthreads();
    float tot = 0.0f;
#pragma unroll
    for (int w = 0; w < kGrWaves; ++w) tot += sh.wsum[w];
    ssum = tot;
  }
  return best;
}

__device__ __forceinline__ bool key_fault(uint64_t k) { return k == kFaultKey || uint32_t(k >> 32) == kOrdNegInf; }
__device__ __forceinline__ int32_t key_index(uint64_t k) { return int32_t(~uint32_t(k)); }

// The sequence's last workgroup: merge the row keys, check the arguments of the sequence, walk the slots.
__device__ void resolve(const GreedyParams& p, int64_t b, int32_t st, GrShared& sh) {
  const int t = threadIdx.x;
  const int G = p.G, R = p.R, S = p.S;
  for (int i = t; i < R; i += kGrBlock) sh.rowkey[i] = 0;
  for (int i = t; i < (G + 31) / 32; i += kGrBlock) sh.seen[i] = 0;
  if (t == 0) {
    sh.kmin = G;
    sh.fl = 0;
  }
  __syncthreads();
  const uint64_t* part = p.part + b * R * S;
  for (int i = t; i < R * S; i += kGrBlock) atomicMax(reinterpret_cast<unsigned long long*>(&sh.rowkey[i / S]),
                                                       static_cast<unsigned long long>(ld_dev(part + i)));
  const int32_t* ord = p.order ? p.order + b * G : nullptr;
  for (int s = t; s < G; s += kGrBlock) {
    const int v = ord ? ord[s] : s;
    if (v < 0 || v >= G) {
      atomicOr(&sh.fl, SV_FLAG_ID_RANGE);
    } else {
      const uint32_t bit = 1u << (v & 31);
      if (atomicOr(&sh.seen[v >> 5], bit) & bit) atomicOr(&sh.fl, SV_FLAG_ID_RANGE);   // repeated row
    }
  }
  __syncthreads();
  const bool bad_args = st < 0 || st > G || sh.fl != 0;
  const int32_t* ids = p.ids + b * G;
  if (!bad_args && st < G) {
    for (int s = st + t; s < G; s += kGrBlock) {
      const int row = ord ? ord[s] : s;
      const uint64_t k = sh.rowkey[row];
      const int32_t x = ids[row];
      if (x < 0 || int64_t(x) >= p.V) atomicOr(&sh.fl, SV_FLAG_ID_RANGE);
      if (key_fault(k)) atomicOr(&sh.fl, SV_FLAG_NONFINITE);
      if (x != key_index(k)) atomicMin(&sh.kmin, s);
    }
  }
  __syncthreads();
  const uint32_t fl = bad_args ? uint32_t(SV_FLAG_ID_RANGE) : sh.fl;
  const bool fatal = fl != 0;
  const bool live = !fatal && st < G;
  if (p.accept) {
    uint8_t* acc = p.accept + b * G;
    if (!live) {
      for (int r = t; r < G; r += kGrBlock) acc[r] = 0;
    } else {
      for (int s = t; s < G; s += kGrBlock) {
        const int row = ord ? ord[s] : s;
        acc[row] = s >= st && ids[row] == key_index(sh.rowkey[row]);
      }
    }
  }
  if (t == 0) {
    uint32_t f = fl;
    int32_t n = fatal ? -1 : 0, tok = -1;
    if (live) {
      const int k = sh.kmin;
      n = k - st;
      if (k < G) {
        tok = key_index(sh.rowkey[ord ? ord[k] : k]);
      } else if (p.bonus) {
        const uint64_t kb = sh.rowkey[G];
        if (key_fault(kb)) f |= SV_FLAG_NONFINITE;
        else tok = key_index(kb);
      }
      if (p.start) p.start[b] = min(G, k + 1);
    }
    p.n_acc[b] = n;
    p.token[b] = tok;
    if (p.flags) p.flags[b] = f;
    st_dev(p.ctr + b, int32_t(0));          // ready for the next call
  }
}

// Confidence-threshold commit, the last workgroup of a block: per masked slot the merged argmax and confidence
// 1 / sum exp(z - max) (float64 merge of the segment sums), then commit the slots at or above tau, or else the single
// most confident one (lowest slot on ties).
__device__ void resolve_conf(const GreedyParams& p, int64_t b, GrShared& sh) {
  const int t = threadIdx.x;
  const int W = p.G, S = p.S;
  for (int i = t; i < W; i += kGrBlock) sh.rowkey[i] = 0;
  if (t == 0) {
    sh.fl = 0;
    sh.best = 0;
    sh.bestj = W;
    sh.any = 0;
  }
  __syncthreads();
  const uint64_t* part = p.part + b * W * S;
  const float2* part2 = p.part2 + b * W * S;
  const uint8_t* msk = p.masked ? p.masked + b * W : nullptr;
  for (int i = t; i < W * S; i += kGrBlock)
    if (!msk || msk[i / S]) atomicMax(reinterpret_cast<unsigned long long*>(&sh.rowkey[i / S]),
                                      static_cast<unsigned long long>(ld_dev(part + i)));
  __syncthreads();
  for (int j = t; j < W; j += kGrBlock) {
    double c = -1.0;
    if (!msk || msk[j]) {
      const uint64_t k = sh.rowkey[j];
      if (key_fault(k)) {
        atomicOr(&sh.fl, SV_FLAG_NONFINITE);
      } else {
        const uint32_t hb = uint32_t(k >> 32);
        const double M = double(__uint_as_float((hb & 0x80000000u) ? (hb & 0x7FFFFFFFu) : ~hb));
        double acc = 0.0;
        for (int s = 0; s < S; ++s) {
          const float2 q = make_float2(ld_dev(&part2[j * S + s].x), ld_dev(&part2[j * S + s].y));
          if (q.y > 0.0f) acc += double(q.y) * exp(double(q.x) - M);
        }
        c = 1.0 / acc;
        if (c >= p.tau) atomicOr(&sh.any, 1);
        atomicMax(reinterpret_cast<unsigned long long*>(&sh.best), static_cast<unsigned long long>(__double_as_longlong(c)));
      }
    }
    sh.rowconf[j] = c;
  }
  __syncthreads();
  const bool fatal = sh.fl != 0;
  const bool any = sh.any != 0;
  const double best = __longlong_as_double(static_cast<long long>(sh.best));
  if (!fatal && !any)
    for (int j = t; j < W; j += kGrBlock)
      if (sh.rowconf[j] >= 0.0 && sh.rowconf[j] == best) atomicMin(&sh.bestj, j);
  __syncthreads();
  int cnt = 0;
  for (int j = t; j < W; j += kGrBlock) {
    const double c = sh.rowconf[j];
    const bool read = c >= 0.0;
    const bool take = !fatal && read && (any ? c >= p.tau : j == sh.bestj);
    cnt += take;
    if (p.commit) p.commit[b * W + j] = take;
    p.token[b * W + j] = take ? key_index(sh.rowkey[j]) : -1;
    if (p.conf) p.conf[b * W + j] = read && !fatal ? float(c) : NAN;
  }
  // block count of commits
  const int wc = int(wave_sum(double(cnt)));
  __syncthreads();
  if ((t & 63) == 0) sh.wsum[t >> 6] = float(wc);
  __syncthreads();
  if (t == 0) {
    int n = 0;
    for (int w = 0; w < kGrWaves; ++w) n += int(sh.wsum[w]);
    p.n_acc[b] = fatal ? -1 : n;
    if (p.flags) p.flags[b] = sh.fl;
    st_dev(p.ctr + b, int32_t(0));          // ready for the next call
  }
}

template <typename T, bool CONF>
__global__ __launch_bounds__(kGrBlock) void k_greedy(GreedyParams p) {
  __shared__ GrShared sh;
  const int t = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int s = int(item % p.S);
  const int64_t br = item / p.S;
  const int r = int(br % p.R);
  const int64_t b = br / p.R;
  const int G = p.G;
  const int32_t st = (!CONF && p.start) ? p.start[b] : 0;
  // workgroup 0 makes sure the counters are at zero for this call's layout; the others confirm it before counting
  if (item == 0) ws_claim(p.ws, p.sig, size_t(p.ctl_end), &sh.last);
  const bool seen = item == 0 || ws_seen_clean(p.ws, p.sig);

  // Is this row verified (or the bonus row of a live sequence; CONF: a masked slot)?
  bool read;
  if constexpr (CONF) {
    read = !p.masked || p.masked[b * G + r] != 0;
  } else if (st < 0 || st >= G) {
    read = false;
  } else if (r == G || st == 0) {
    read = true;
  } else if (!p.order) {
    read = r >= st;
  } else {
    if (t == 0) sh.slot = G;
    __syncthreads();
    for (int j = t; j < G; j += kGrBlock)
      if (p.order[b * G + j] == r) sh.slot = j;
    __syncthreads();
    read = sh.slot >= st && sh.slot < G;    // a row missing from order: the sequence fails its argument check
  }

  uint64_t key = 0;
  float ssum = 0.0f, smax = -INFINITY;
  if (read) {
    const T* row = static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(r) * p.t_row;
    const int64_t e0 = int64_t(s) * p.seg_elems;
    const int64_t e1 = min(p.V, e0 + p.seg_elems);
    key = segment_key<T, CONF>(row, e0, e1, sh, ssum);
    if (CONF && key != kFaultKey) {
      const uint32_t hb = uint32_t(key >> 32);
      smax = __uint_as_float((hb & 0x80000000u) ? (hb & 0x7FFFFFFFu) : ~hb);
    }
  }
  // The key is a device-scope store, complete (waitcnt) before the counter counts it; the merging workgroup reads
  // the keys with device-scope loads issued after it has seen the count. No release or acquire fence: at agent
  // scope those write back and invalidate the whole L2, which would cost far more than the pass itself.
  if (t == 0) {
    if (read) {
      st_dev(p.part + item, key);
      if (CONF) {
        st_dev(&p.part2[item].x, smax);
        st_dev(&p.part2[item].y, ssum);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (seen || ws_ready(p.ws, p.sig)) {
      sh.last = ctr_add(p.ctr + b) == p.R * p.S - 1;
    } else {                                  // never counted: the sequence is not resolved in this call
      ws_mark_dirty(p.ws);
      sh.last = 0;
    }
  }
  __syncthreads();
  if (!sh.last) return;
  if constexpr (CONF) resolve_conf(p, b, sh);
  else resolve(p, b, st, sh);
}

}  // namespace

GreedyPlan make_greedy_plan(int64_t B, int32_t G, int64_t V, int32_t bonus, int dtype) {
  GreedyPlan pl;
  pl.B = B; pl.G = G; pl.V = V; pl.R = G + (bonus ? 1 : 0);
  const int64_t E = dtype == SV_BF16 ? 8 : 4;                           // logits per 16-byte vector
  const int64_t rows = B * pl.R;
  const int64_t nchunk = (V + kGrChunkVec * E - 1) / (kGrChunkVec * E);
  int64_t S = (kGreedyTargetItems + rows - 1) / rows;
  S = std::min<int64_t>(S, std::min<int64_t>(nchunk, kGreedyMaxSeg));
  S = std::max<int64_t>(S, 1);
  const int64_t gran = int64_t(kGrBlock) * E;                           // one vector per thread
  pl.seg_elems = ((V + S - 1) / S + gran - 1) / gran * gran;
  pl.S = int32_t((V + pl.seg_elems - 1) / pl.seg_elems);
  pl.items = rows * pl.S;
  pl.ctr_bytes = kWsHeaderBytes + size_t((B * 4 + 255) / 256 * 256);
  pl.off_part = pl.ctr_bytes;
  pl.off_part2 = (pl.off_part + size_t(pl.items) * 8 + 255) / 256 * 256;
  pl.total = (pl.off_part2 + size_t(pl.items) * 8 + 255) / 256 * 256;
  return pl;
}

size_t greedy_workspace_bytes(int64_t B, int32_t G, int64_t V) {
  size_t n = 0;
  for (int bonus = 0; bonus < 2; ++bonus)
    for (int dtype : {SV_F32, SV_BF16}) n = std::max(n, make_greedy_plan(B, G, V, bonus, dtype).total);
  return n;
}

hipError_t launch_greedy(const GreedyPlan& plan, const GreedyArgs& a, hipStream_t stream) {
  GreedyParams p{};
  p.ws = a.ws;
  p.sig = ws_signature(kLayoutGreedy, uint64_t(plan.B));
  p.ctl_end = int64_t(plan.ctr_bytes);
  p.tgt = a.tgt; p.t_seq = a.t_seq; p.t_row = a.t_row;
  p.V = plan.V; p.seg_elems = plan.seg_elems;
  p.G = plan.G; p.R = plan.R; p.S = plan.S; p.bonus = a.bonus;
  p.ids = a.ids; p.start = a.start; p.order = a.order;
  p.accept = a.accept; p.n_acc = a.n_acc; p.token = a.token; p.flags = a.flags;
  p.masked = a.masked; p.tau = double(a.tau); p.commit = a.commit; p.conf = a.conf;
  p.ctr = reinterpret_cast<int32_t*>(a.ws + kWsHeaderBytes);
  p.part = reinterpret_cast<uint64_t*>(a.ws + plan.off_part);
  p.part2 = reinterpret_cast<float2*>(a.ws + plan.off_part2);
  auto kern = a.conf_mode ? (a.dtype == SV_BF16 ? k_greedy<uint16_t, true> : k_greedy<float, true>)
                          : (a.dtype == SV_BF16 ? k_greedy<uint16_t, false> : k_greedy<float, false>);
  const unsigned grid = unsigned(plan.items);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kGrBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
