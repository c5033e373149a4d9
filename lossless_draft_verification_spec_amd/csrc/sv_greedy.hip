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

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdint>

#include "sv.h"
#include "sv_device.h"
#include "sv_greedy.h"
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kGrBlock = 256;
constexpr int kGrWaves = kGrBlock / 64;
#ifndef SV_GR_U
#define SV_GR_U 4
#endif
constexpr int kGrU = SV_GR_U;                               // 16-byte vectors per thread per chunk
constexpr int64_t kGrChunkVec = int64_t(kGrBlock) * kGrU;   // vectors per chunk (16 KB)
constexpr uint64_t kFaultKey = ~0ull;                       // a segment holding a NaN or +inf
constexpr uint32_t kOrdNegInf = 0x007FFFFFu;                // ord_bits(-inf)

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
  int32_t* ctr;                // per sequence: workgroups finished
  uint64_t* part;              // per (sequence, row, segment): the segment's key
};

struct GrShared {
  uint64_t wkey[kGrWaves];
  uint32_t wfault[kGrWaves];
  int32_t slot;                // verification slot of this workgroup's row
  int32_t last;                // this workgroup merges the sequence
  int32_t kmin;                // first mismatching slot
  uint32_t fl;                 // the sequence's flags
  uint32_t seen[SV_MAX_GAMMA / 32];
  uint64_t rowkey[SV_MAX_GAMMA + 1];
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
template <typename T>
__device__ __forceinline__ void fold_chunk(const uint4 (&w)[kGrU], int c, int64_t nv, int t, int64_t elem0, float& m,
                                          int64_t& mi, bool& bad) {
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
    m = cm;
    mi = elem0 + pos;
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

// The key of logits [e0, e1) of one row (see the file comment). Every thread of the workgroup calls it.
template <typename T>
__device__ uint64_t segment_key(const T* row, int64_t e0, int64_t e1, GrShared& sh) {
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
  uint4 nxt[kGrU];
  for (int c = 0; c < nch; c += 2) {
    load_chunk(nxt, vp, c + 1, nv, t);
    fold_chunk<T>(cur, c, nv, t, v0 + (int64_t(c) * kGrChunkVec + t) * E, m, mi, bad);
    load_chunk(cur, vp, c + 2, nv, t);
    if (c + 1 < nch) fold_chunk<T>(nxt, c + 1, nv, t, v0 + (int64_t(c + 1) * kGrChunkVec + t) * E, m, mi, bad);
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
  return anyf ? kFaultKey : best;
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

template <typename T>
__global__ __launch_bounds__(kGrBlock) void k_greedy(GreedyParams p) {
  __shared__ GrShared sh;
  const int t = threadIdx.x;
  const int64_t item = blockIdx.x;
  const int s = int(item % p.S);
  const int64_t br = item / p.S;
  const int r = int(br % p.R);
  const int64_t b = br / p.R;
  const int G = p.G;
  const int32_t st = p.start ? p.start[b] : 0;

  // Is this row verified (or the bonus row of a live sequence)?
  bool read;
  if (st < 0 || st >= G) {
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
  if (read) {
    const T* row = static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(r) * p.t_row;
    const int64_t e0 = int64_t(s) * p.seg_elems;
    const int64_t e1 = min(p.V, e0 + p.seg_elems);
    key = segment_key<T>(row, e0, e1, sh);
  }
  // The key is a device-scope store, complete (waitcnt) before the counter counts it; the merging workgroup reads
  // the keys with device-scope loads issued after it has seen the count. No release or acquire fence: at agent
  // scope those write back and invalidate the whole L2, which would cost far more than the pass itself.
  if (t == 0) {
    if (read) st_dev(p.part + item, key);
    __builtin_amdgcn_s_waitcnt(0);
    sh.last = ctr_add(p.ctr + b) == p.R * p.S - 1;
  }
  __syncthreads();
  if (!sh.last) return;
  resolve(p, b, st, sh);
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
  pl.ctr_bytes = size_t((B * 4 + 255) / 256 * 256);
  pl.off_part = pl.ctr_bytes;
  pl.total = pl.off_part + size_t(pl.items) * 8;
  return pl;
}

size_t greedy_workspace_bytes(int64_t B, int32_t G, int64_t V) {
  size_t n = 0;
  for (int bonus = 0; bonus < 2; ++bonus)
    for (int dtype : {SV_F32, SV_BF16}) n = std::max(n, make_greedy_plan(B, G, V, bonus, dtype).total);
  return n;
}

hipError_t launch_greedy(const GreedyPlan& plan, const GreedyArgs& a, hipStream_t stream) {
  if (workspace_layout_changed(a.ws, layout_mix(kLayoutGreedy, uint64_t(plan.B)))) {
    const hipError_t e = clear_control(a.ws, plan.ctr_bytes, stream);
    if (e != hipSuccess) return e;
  }
  GreedyParams p{};
  p.tgt = a.tgt; p.t_seq = a.t_seq; p.t_row = a.t_row;
  p.V = plan.V; p.seg_elems = plan.seg_elems;
  p.G = plan.G; p.R = plan.R; p.S = plan.S; p.bonus = a.bonus;
  p.ids = a.ids; p.start = a.start; p.order = a.order;
  p.accept = a.accept; p.n_acc = a.n_acc; p.token = a.token; p.flags = a.flags;
  p.ctr = reinterpret_cast<int32_t*>(a.ws);
  p.part = reinterpret_cast<uint64_t*>(a.ws + plan.off_part);
  auto kern = a.dtype == SV_BF16 ? k_greedy<uint16_t> : k_greedy<float>;
  const unsigned grid = unsigned(plan.items);
  if (a.ev_start) {
    hipExtLaunchKernelGGL(kern, dim3(grid), dim3(kGrBlock), 0, stream, static_cast<hipEvent_t>(a.ev_start),
                          static_cast<hipEvent_t>(a.ev_stop), 0, p);
  } else {
    hipLaunchKernelGGL(kern, dim3(grid), dim3(kGrBlock), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace sv
