// Top-k / top-p support builder for gfx950 (MI355X): dense logit rows become the sparse (ids, probs) supports that
// the sparse verifier takes.
//
// What it computes. The sampler settings are those of the throughput test on "Uno: the draft model was already
// inside the target model" (section "The speedup, without the 'up to'": temperature 1, top-p 0.95, top-k 50); the
// sparse verify routine printed on that page (section "What 'lossless' actually has to mean") takes p and q as such
// supports; the temperature divides the logits before the probabilities are formed (DFlash/DFlash2 guide, section 9
// Q3). Per row: the k largest logits, ties to the lower id, in descending order; over them the top-k distribution
// e_j / sum(e), e_j = exp(z_j / T - z_0 / T); slot j is kept when j = 0 or the cumulative probability of slots
// 0..j-1 is below top_p (the shortest prefix that reaches top_p); a kept slot gets its probability renormalised over
// the kept slots (renorm = 1) or its full-vocabulary softmax probability (renorm = 0), every other slot 0.
//
// How. One launch on the caller's stream, one 256-thread workgroup per item: one segment of one row (the segments of a
// row are consecutive items). A launch may take two sets of rows with the same settings (a target's rows and a
// draft's), the second numbered after the first, so that the two share one schedule and one tail. Each wave streams its
// share of the segment with 16-byte non-temporal loads and keeps candidate keys in its own LDS buffer. A key holds the
// logit, mapped to an order-preserving unsigned integer, in its high 32 bits and the complement of the id in its low
// 32, so keys are distinct and a larger key is a larger logit or, for equal logits, the lower id. An element enters the
// buffer only if its key exceeds the wave's threshold, the k-th largest key the wave (or another wave of the workgroup)
// has kept so far; a 16-byte vector is tested first through its maximum, so once the threshold has risen, within the
// first few thousand elements of a row, nearly every vector costs one compare. When a buffer fills, its wave raises the
// threshold by a radix select over the buffer, without a barrier. At the end of the segment the waves' candidates (on
// these rows a few dozen past k) are put in order in one pass, each thread counting the keys above its own; with
// several segments per row the last segment to finish (a counter per row) merges the segments' keys the same way, after
// a radix select when they are more than one per thread. The row's probabilities are then formed in float64 and the
// top-p cut taken in float64.
//
// Bound: HBM. Algorithmic bytes: every logit of every row once (V * s per row, s = 2 bf16, 4 fp32), plus k ids and
// k probabilities written per row.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "sv.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_wshdr.h"

namespace sv {
namespace {

constexpr int kSupBlock = 256;
constexpr int kSupWaves = kSupBlock / 64;
constexpr int kWaveCap = 768;                      // candidate keys per wave buffer
constexpr int kMergeCap = kSupWaves * kWaveCap;    // keys one merge holds (the wave buffers side by side)
// 16-byte vectors per thread per load round (two rounds in flight): fewer for bf16, whose 8 elements per vector
// take more registers in the candidate path.
template <typename T> constexpr int kRoundVecs = sizeof(T) == 2 ? 2 : 4;
// The rows of a last, partial resident round are cut into segments that are items of their own, queued before the
// whole rows.
constexpr int kSupCtrStride = 64;                  // int32 slots between row counters (one 256-byte line each)
constexpr int kMaxSeg = 16;                        // segments per row
constexpr int64_t kMinSegBytes = 32768;            // smallest segment worth a workgroup
static_assert(SV_MAX_K + 8 * 64 <= kWaveCap, "a wave buffer holds k keys plus one 16-byte vector per lane");
static_assert(SV_MAX_K * kSupWaves <= kMergeCap, "the waves' candidates fit one merge");

struct SupPartial {
  float m;        // max of the segment's logits (NaN ignored)
  int32_t nk;     // keys the segment passed on (min(k, its non-NaN elements))
  uint32_t nan;   // 1 when the segment holds a NaN
  uint32_t pad;
  double s;       // sum over the segment of 2^(z * c - m * c), c = log2(e) / T in float32 (renorm = 0 only)
};

struct SupportParams {
  SupportRows s0, s1;   // the row sets: global rows 0 .. rows0 - 1 are s0's, the rest s1's
  int64_t rows0;
  int64_t rows; int64_t V;
  int32_t k; int32_t renorm;
  int64_t head_rows;  // rows 0 .. head_rows - 1: one item each (the whole row)
  int32_t nseg;       // segments of each later row
  int64_t items;      // items (workgroups) in the launch
  int32_t nlay;       // segment records per row in the workspace (>= nseg)
  float c;          // log2(e) / T rounded to float32: the full-row sums
  double T;         // the temperature, widened
  double top_p;     // top_p as received (float32), widened
  char* ws;         // the workspace; its header names the control layout at zero
  uint64_t sig;     // this call's control layout
  int64_t ctl_end;  // control words (the row counters) fill [kWsHeaderBytes, ctl_end)
  int32_t* ctr;     // per row, kSupCtrStride apart: segments finished in this call
  uint64_t* keys;   // per (row, segment): up to k keys
  SupPartial* part; // per (row, segment)
};

struct SupShared {
  uint64_t buf[kMergeCap];             // wave w's candidates at w * kWaveCap; as one array, the merge area
  uint64_t uni[kSupWaves * SV_MAX_K];  // the waves' candidates side by side at the end of a segment
  uint64_t sorted[SV_MAX_K];           // the row's keys in descending order
  uint32_t hist[kSupWaves][256];       // one radix histogram per wave
  uint64_t theta[kSupWaves];           // each wave's threshold (read by the other waves)
  int32_t cnt[kSupWaves];
  int32_t segoff[kMaxSeg + 1];
  double redd[kSupWaves];
  double dval;
  float redf[kSupWaves];
  float mval;
  int32_t ival;
  int32_t flag;
  int32_t pool_n;                      // keys the waves have added to the pilot's pool in uni (whole rows)
  int32_t pool_in;                     // waves that have added theirs
};

// The workgroup's shared state, at file scope so that functions that are not inlined address it as LDS too.
__shared__ SupShared g_sup;

// ----------------------------------------------------------------------------------------------------------------
// keys
// ----------------------------------------------------------------------------------------------------------------

// Order-preserving map of a non-NaN float to an unsigned integer (-0 ranks as +0).
__device__ __forceinline__ uint32_t ord_of(float z) {
  uint32_t u = __float_as_uint(z);
  u = u == 0x80000000u ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t key_of(float z, uint32_t id) {
  return (uint64_t(ord_of(z)) << 32) | uint64_t(~id);
}
__device__ __forceinline__ float val_of(uint64_t key) {
  const uint32_t o = uint32_t(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}
__device__ __forceinline__ int32_t id_of(uint64_t key) { return int32_t(~uint32_t(key)); }
// The smallest logit that can still beat threshold key t (key 0 lies below every key).
__device__ __forceinline__ float floor_of(uint64_t t) { return t == 0 ? -INFINITY : val_of(t); }

__device__ __forceinline__ uint64_t lds_load_u64(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_store_u64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Wave-wide min / max of 64-bit keys: DPP exchanges inside each row of 16 lanes, then the four rows' results
// combined from scalar reads (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(v)), CTRL, 0xF, 0xF, true));
  const uint32_t hi = uint32_t(__builtin_amdgcn_mov_dpp(int(uint32_t(v >> 32)), CTRL, 0xF, 0xF, true));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<kDppXor1>(v); v = o < v ? o : v;
  o = dpp_u64<kDppXor2>(v); v = o < v ? o : v;
  o = dpp_u64<kDppHalfMirror>(v); v = o < v ? o : v;
  o = dpp_u64<kDppMirror>(v); v = o < v ? o : v;
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16), c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a < b ? a : b, cd = c < d ? c : d;
  return ab < cd ? ab : cd;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint64_t o;
  o = dpp_u64<kDppXor1>(v); v = o > v ? o : v;
  o = dpp_u64<kDppXor2>(v); v = o > v ? o : v;
  o = dpp_u64<kDppHalfMirror>(v); v = o > v ? o : v;
  o = dpp_u64<kDppMirror>(v); v = o > v ? o : v;
  const uint64_t a = readlane_u64(v, 0), b = readlane_u64(v, 16), c = readlane_u64(v, 32), d = readlane_u64(v, 48);
  const uint64_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Moves the keys >= t of a[0..n) to the front, in order, and returns how many there are. A round's writes land at or
// below its reads. One wave, all lanes active.
__device__ __forceinline__ int keep_from(uint64_t* a, int n, uint64_t t) {
  const int lane = threadIdx.x & 63;
  int out = 0;
  for (int j0 = 0; j0 < n; j0 += 64) {
    const int j = j0 + lane;
    const uint64_t key = j < n ? a[j] : 0ull;
    const bool keep = j < n && key >= t;
    const uint64_t m = wave_ballot(keep);
    __builtin_amdgcn_wave_barrier();
    if (keep) a[out + lane_rank(m)] = key;
    out += __builtin_popcountll(m);
  }
  __builtin_amdgcn_wave_barrier();
  return out;
}

__device__ __forceinline__ int wave_sum_i(int v) {
  v += dpp_i<kDppXor1>(0, v);
  v += dpp_i<kDppXor2>(0, v);
  v += dpp_i<kDppHalfMirror>(0, v);
  v += dpp_i<kDppMirror>(0, v);
  return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
         (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// The largest logit code t (the high 32 bits of a key) such that at least k of the n keys a[0..n) have a code >= t,
// n >= k >= 1, kWaveCap >= n: a bisection over the codes, each step one compare per key held in registers and one
// wave sum (no LDS traffic after the first read).
__device__ __forceinline__ uint32_t wave_code_floor(const uint64_t* a, int n, int k) {
  const int lane = threadIdx.x & 63;
  constexpr int J = kWaveCap / 64;
  uint32_t o[J];
  uint32_t lo = ~0u, hi = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int idx = j * 64 + lane;
    o[j] = idx < n ? uint32_t(a[idx] >> 32) : 0u;
    if (idx < n) {
      lo = o[j] < lo ? o[j] : lo;
      hi = o[j] > hi ? o[j] : hi;
    }
  }
  lo = uint32_t(wave_min_u64(lo));                   // the answer lies in [min code, max code]
  hi = uint32_t(wave_max_u64(hi));
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo + 1u) / 2u;
    int c = 0;
#pragma unroll
    for (int j = 0; j < J; ++j) c += o[j] >= mid;
    if (wave_sum_i(c) >= k) lo = mid;
    else hi = mid - 1u;
  }
  return lo;
}

// The k-th largest of the n distinct keys a[0..n), n > k >= 1, by a most-significant-digit-first radix select with
// 8-bit digits over a 256-bin histogram in LDS; with `move`, the k largest keys are then moved to a[0..k), in no
// particular order (the pilots, which only need the threshold, leave the keys where they are). One wave, all 64
// lanes active, no barrier: the LDS executes one wave's operations in issue order. The keys of a buffer lie close
// together and share their high bits, so the digits start at the highest bit where the smallest and the largest key
// differ: the first histogram spreads over its bins instead of piling every key into one (whose atomic adds would
// serialise).
__device__ __forceinline__ uint64_t wave_select(uint64_t* a, int n, int k, uint32_t* hist, bool move = true) {
  const int lane = threadIdx.x & 63;
  uint64_t lo = ~0ull, hi_key = 0ull;
  for (int j = lane; j < n; j += 64) {
    const uint64_t key = a[j];
    lo = key < lo ? key : lo;
    hi_key = key > hi_key ? key : hi_key;
  }
  lo = wave_min_u64(lo);
  hi_key = wave_max_u64(hi_key);
  const int top = 63 - __builtin_clzll(lo ^ hi_key);       // lo != hi_key: n >= 2 distinct keys
  uint64_t prefix = top == 63 ? 0ull : (hi_key & (~0ull << (top + 1)));   // the bits every key shares
  int rank = k;           // rank, from the top, of the wanted key among the keys that match the prefix
  uint64_t theta = 0;
  bool found = false;
  for (int shift = top - 7; shift > -8; shift -= 8) {   // at most 8 digits: the loop ends whatever the keys
    const int sh = shift < 0 ? 0 : shift;                   // this digit: bits [sh, shift + 7]
    const uint64_t hi = shift + 8 >= 64 ? 0ull : (~0ull << (shift + 8));
    const uint32_t dmask = shift < 0 ? ((1u << (shift + 8)) - 1u) : 255u;
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0u;
    __builtin_amdgcn_wave_barrier();
    for (int j = lane; j < n; j += 64) {
      const uint64_t key = a[j];
      if ((key & hi) == prefix)
        __hip_atomic_fetch_add(&hist[uint32_t(key >> sh) & dmask], 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    __builtin_amdgcn_wave_barrier();
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = hist[lane * 4 + i];
    const int c = int(h[0] + h[1] + h[2] + h[3]);
    const int incl = wave_incl_scan_i(c);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    const int from_here = total - incl + c;                // matching keys whose digit is >= 4 * lane
    const uint64_t m = wave_ballot(from_here >= rank);     // lane 0 always votes: total >= rank
    const int L = 63 - __builtin_clzll(m);                 // the digit lies in [4L, 4L + 3]
    int above = __builtin_amdgcn_readlane(from_here, L) - __builtin_amdgcn_readlane(c, L);
    const int h3 = __builtin_amdgcn_readlane(int(h[3]), L), h2 = __builtin_amdgcn_readlane(int(h[2]), L);
    const int h1 = __builtin_amdgcn_readlane(int(h[1]), L), h0 = __builtin_amdgcn_readlane(int(h[0]), L);
    int dig, hd;
    if (above + h3 >= rank) { dig = 3; hd = h3; }
    else if (above + h3 + h2 >= rank) { above += h3; dig = 2; hd = h2; }
    else if (above + h3 + h2 + h1 >= rank) { above += h3 + h2; dig = 1; hd = h1; }
    else { above += h3 + h2 + h1; dig = 0; hd = h0; }
    rank -= above;
    prefix |= uint64_t(4 * L + dig) << sh;
    if (hd == rank) {       // every key with this prefix is among the k: the threshold is the smallest of them
      const uint64_t mask = ~0ull << sh;
      uint64_t mn = ~0ull;
      for (int j = lane; j < n; j += 64) {
        const uint64_t key = a[j];
        if ((key & mask) == prefix) mn = key < mn ? key : mn;
      }
      theta = wave_min_u64(mn);
      found = true;
      break;                // reached at the last digit at the latest (distinct keys: one key per full prefix)
    }
  }
  if (!found) theta = prefix;                       // only with repeated keys, which callers never pass
  if (move) keep_from(a, n, theta);                // exactly k keys
  return theta;
}

// ----------------------------------------------------------------------------------------------------------------
// streaming candidates
// ----------------------------------------------------------------------------------------------------------------

struct WaveCands {
  uint64_t theta;   // the wave's threshold key (0: none yet, every element enters)
  float floor;      // its logit (-inf when none)
  uint32_t tid;     // its id (0xFFFFFFFF when none)
  int cnt;          // keys in the wave's buffer
  bool exact;       // ties of the threshold's logit are filtered by id (once a compaction left the logit unchanged)
  bool seeded;      // the first round has set a threshold from its vector maxima
};

__device__ __forceinline__ void set_theta(WaveCands& wc, uint64_t t) {
  wc.theta = t;
  wc.floor = floor_of(t);
  wc.tid = t == 0 ? 0xFFFFFFFFu : uint32_t(id_of(t));
}

// Takes the highest threshold of the workgroup's waves: each is the k-th largest of keys that stay in the segment's
// candidates, so any of them bounds the segment's k-th largest from below.
__device__ __forceinline__ void refresh(WaveCands& wc) {
  uint64_t t = wc.theta;
#pragma unroll
  for (int w = 0; w < kSupWaves; ++w) {
    const uint64_t o = lds_load_u64(&g_sup.theta[w]);
    t = o > t ? o : t;
  }
  t = uint64_t(uniform_i64(int64_t(t)));
  if (t != wc.theta) set_theta(wc, t);
}

// The same bits, opaque to the compiler (an empty volatile asm that claims to change them): used to unpack a vector
// again instead of keeping earlier unpacked values live, and to pin where a loaded vector is first waited for.
__device__ __forceinline__ uint4 opaque(uint4 v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
  return v;
}

// Shrinks wave w's buffer (cnt > k keys) to the keys whose logit code reaches the k-th largest code (at least k of
// them) and raises the wave's threshold to that code, published for the other waves. If ties of that code would
// leave more than `limit` keys, an exact select keeps the k largest keys instead and the wave filters ties by id
// from then on.
struct Compacted {
  uint64_t theta;   // the new threshold key (exact: the k-th largest key; otherwise a code << 32)
  int cnt;          // keys kept
  int exact;        // 1: ties were broken by id
};

// Out of line: reached a few times per row at most, and one copy serves every call site.
__device__ __noinline__ Compacted compact_keys(int w, int cnt, int k, int limit) {
  w = __builtin_amdgcn_readfirstlane(w);
  cnt = __builtin_amdgcn_readfirstlane(cnt);
  k = __builtin_amdgcn_readfirstlane(k);
  limit = __builtin_amdgcn_readfirstlane(limit);
  uint64_t* a = g_sup.buf + w * kWaveCap;
  const uint64_t t = uint64_t(wave_code_floor(a, cnt, k)) << 32;     // every key with the k-th largest code passes
  const int kept = keep_from(a, cnt, t);
  if (kept <= limit) return Compacted{t, kept, 0};
  return Compacted{wave_select(a, kept, k, g_sup.hist[w]), k, 1};     // ties of one logit: break them by id
}

__device__ __forceinline__ void compact(int w, WaveCands& wc, int k, int limit) {
  const Compacted c = compact_keys(w, wc.cnt, k, limit);
  const uint64_t t = uint64_t(uniform_i64(int64_t(c.theta)));
  set_theta(wc, t > wc.theta ? t : wc.theta);
  wc.cnt = __builtin_amdgcn_readfirstlane(c.cnt);
  wc.exact = wc.exact || __builtin_amdgcn_readfirstlane(c.exact) != 0;
  if ((threadIdx.x & 63) == 0) lds_store_u64(&g_sup.theta[w], wc.theta);
}

// Offers N elements per lane (ids id0 .. id0 + N - 1; lanes with ok) to the wave's buffer. Every element whose key
// exceeds the threshold must enter: every element whose logit reaches the threshold's does (ties with a higher id
// are harmless extra keys), unless a tie flood has put the wave in exact mode, where those ties stay out. Each
// element slot's candidates are the lane mask of one compare; they are counted first, and nothing is written
// (false) when they would not fit. Only the slots with candidates write.
template <int N>
__device__ __forceinline__ bool try_offer(int w, WaveCands& wc, const float* z, uint32_t id0, bool ok) {
  uint64_t m[N];
  int total = 0;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    m[e] = wave_ballot(ok && z[e] >= wc.floor);      // NaN never passes
    if (wc.exact && m[e] != 0) m[e] &= ~wave_ballot(z[e] == wc.floor && id0 + uint32_t(e) >= wc.tid);
    total += __builtin_popcountll(m[e]);
  }
  if (wc.cnt + total > kWaveCap) return false;
  int base = w * kWaveCap + wc.cnt;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    if (m[e] == 0) continue;
    if ((m[e] >> (threadIdx.x & 63)) & 1u) g_sup.buf[base + lane_rank(m[e])] = key_of(z[e], id0 + uint32_t(e));
    base += __builtin_popcountll(m[e]);
  }
  wc.cnt += total;
  return true;
}

// Running full-row sum of one thread (renorm = 0): max m, mc = fl(m * c), s = sum of 2^(z * c - mc).
struct RowRun {
  float m, mc, s;
};

template <int N>
__device__ __forceinline__ void sum_absorb(RowRun& st, const float* v, float cm, float c) {
  const float mn = fmaxf(st.m, cm);
  if (mn == -INFINITY) return;                       // nothing but -inf (and NaN, tracked apart) so far
  const float mnc = __fmul_rn(mn, c);
  if (mn != st.m) {                                  // a new maximum: rescale what was summed
    st.s *= ex2f(st.mc - mnc);
    st.m = mn;
    st.mc = mnc;
  }
  float t[N];
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = ex2f(fmaf(v[i], c, -mnc));
#pragma unroll
  for (int w = 1; w < N; w <<= 1)
#pragma unroll
    for (int i = 0; i + w < N; i += 2 * w) t[i] += t[i + w];
  st.s += t[0];
}

// The first round's threshold: the largest logit code t such that at least k of the wave's vector maxima (one per
// lane and vector, -inf for vectors past the segment) have a code >= t. Those maxima are k distinct elements, so the
// row's k-th largest key exceeds t << 32: every element below t can be dropped from the start, instead of the whole
// first round filling the buffer. A bisection over the codes; each step counts with one ballot per vector.
template <int U>
__device__ __forceinline__ void seed(int w, WaveCands& wc, int k, const float* vmax) {
  wc.seeded = true;
  uint32_t c[U];
  uint32_t lo = ~0u, hi = 0u;
  int n = 0;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool real = vmax[u] == vmax[u] && vmax[u] > -INFINITY;      // a finite or +inf maximum
    c[u] = real ? ord_of(vmax[u]) : 0u;
    if (real) {
      lo = c[u] < lo ? c[u] : lo;
      hi = c[u] > hi ? c[u] : hi;
    }
    n += __builtin_popcountll(wave_ballot(real));
  }
  if (n < k) return;                                 // too few: no threshold yet
  lo = uint32_t(wave_min_u64(lo));
  hi = uint32_t(wave_max_u64(hi));
  while (lo < hi) {
    const uint32_t mid = lo + (hi - lo + 1u) / 2u;
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) cnt += __builtin_popcountll(wave_ballot(c[u] >= mid));
    if (cnt >= k) lo = mid;
    else hi = mid - 1u;
  }
  const uint64_t t = uint64_t(lo) << 32;
  if (t > wc.theta) {
    set_theta(wc, t);
    if ((threadIdx.x & 63) == 0) lds_store_u64(&g_sup.theta[w], t);
  }
}

// Ranks the n distinct keys a[0..n), n <= kSupBlock, one per thread: thread tid counts the keys above a[tid],
// reading all n as broadcasts, four per step, and calls f(key, rank). All threads of the workgroup, with the same n;
// a[] is only read. Every thread reads every key, so this pays only for the few dozen keys left at the end of a
// segment; larger sets go through a radix select first.
template <typename F>
__device__ __forceinline__ void rank_keys(const uint64_t* a, int n, F f) {
  const int tid = threadIdx.x;
  const uint64_t key = tid < n ? a[tid] : ~0ull;
  int r = 0, j = 0;
  for (; j + 4 <= n; j += 4) {
    const uint64_t a0 = a[j], a1 = a[j + 1], a2 = a[j + 2], a3 = a[j + 3];
    r += int(a0 > key) + int(a1 > key) + int(a2 > key) + int(a3 > key);
  }
  for (; j < n; ++j) r += a[j] > key;
  if (tid < n) f(key, r);
}

// After the first rounds of a segment: one exact threshold for the whole workgroup. The waves' candidates so far go
// side by side (a wave with more than SV_MAX_K is compacted first), one wave selects their k-th largest, and every
// wave takes it as its threshold. That is the k-th largest key of every element the workgroup has seen, a bound
// each wave alone would only reach after seeing four times as many; the logits of the rows at hand (largest at low
// ids) make it close to the segment's final k-th largest, so that later rounds rarely offer anything.
// The same threshold for a whole row, without a barrier: each wave adds its candidates (at most SV_MAX_K, compacted
// first if need be) to a pool in uni and counts itself in; the last wave to arrive selects the pool's k-th largest
// and publishes it as its own threshold, which the others take at their next refresh, streaming on meanwhile. The
// waves of a workgroup reach this point at different times (their loads return unevenly), and the barrier pair
// would hold the early ones; a segment's few remaining rounds would mostly pass before the threshold arrived, so
// segments keep the barrier form.
__device__ __forceinline__ void pilot_async(int w, WaveCands& wc, int k) {
  const int lane = threadIdx.x & 63;
  if (wc.cnt > SV_MAX_K) compact(w, wc, k, SV_MAX_K);
  int off = 0;
  if (lane == 0)
    off = __hip_atomic_fetch_add(&g_sup.pool_n, wc.cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  off = __builtin_amdgcn_readfirstlane(off);
  for (int j = lane; j < wc.cnt; j += 64) g_sup.uni[off + j] = g_sup.buf[w * kWaveCap + j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");      // the copies land before the wave counts itself in
  int last = 0;
  if (lane == 0)
    last = __hip_atomic_fetch_add(&g_sup.pool_in, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == kSupWaves - 1;
  if (!__builtin_amdgcn_readfirstlane(last)) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  const int n = __builtin_amdgcn_readfirstlane(
      __hip_atomic_load(&g_sup.pool_n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
  if (n <= k) return;
  // the wave's own histogram: other waves may be compacting with theirs meanwhile
  const uint64_t t = uint64_t(uniform_i64(int64_t(wave_select(g_sup.uni, n, k, g_sup.hist[w], false))));
  if (t > wc.theta) {
    set_theta(wc, t);
    if (lane == 0) lds_store_u64(&g_sup.theta[w], t);
  }
}

__device__ __forceinline__ void pilot(int w, WaveCands& wc, int k) {
  const int lane = threadIdx.x & 63;
  if (wc.cnt > SV_MAX_K) compact(w, wc, k, SV_MAX_K);
  if (lane == 0) g_sup.cnt[w] = wc.cnt;
  __syncthreads();
  int off = 0, n = 0;
#pragma unroll
  for (int i = 0; i < kSupWaves; ++i) {
    const int ci = g_sup.cnt[i];
    if (i < w) off += ci;
    n += ci;
  }
  for (int j = lane; j < wc.cnt; j += 64) g_sup.uni[off + j] = g_sup.buf[w * kWaveCap + j];
  __syncthreads();
  if (w == 0 && n > k) {
    const uint64_t t = wave_select(g_sup.uni, n, k, g_sup.hist[0], false);
    if (lane == 0) lds_store_u64(&g_sup.theta[0], t > wc.theta ? t : wc.theta);
  }
  __syncthreads();
  refresh(wc);
}

// One round of U vectors per thread: statistics, then the elements of the vectors whose maximum reaches the
// threshold are offered (unpacked again from the raw vectors, so that no element array stays live). PART: a round
// past the end of the segment for some vectors (valid[u] false: ignored).
template <typename T, bool SUM, bool PART>
__device__ __forceinline__ void take_round(int w, WaveCands& wc, RowRun& st, bool& nan, int k, float c,
                                           const uint4* g, uint32_t id0, const bool* valid) {
  using VT = Vec<T>;
  constexpr int EPV = VT::kEPV;
  constexpr int U = kRoundVecs<T>;
  float vmax[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool ok = !PART || valid[u];
    float z[EPV];
    VT::unpack(g[u], z);
    float mx = z[0];
#pragma unroll
    for (int e = 1; e < EPV; ++e) mx = fmaxf(mx, z[e]);
    bool bad = false;                                // one unordered compare covers two elements
#pragma unroll
    for (int e = 0; e < EPV; e += 2) bad |= __builtin_isunordered(z[e], z[e + 1]);
    vmax[u] = ok ? mx : -INFINITY;
    nan |= ok && bad;
    if constexpr (SUM) {
      if (ok) sum_absorb<EPV>(st, z, mx, c);
    }
  }
  if (!wc.seeded) seed<U>(w, wc, k, vmax);
  float gm = vmax[0];
#pragma unroll
  for (int u = 1; u < U; ++u) gm = fmaxf(gm, vmax[u]);
  if (wave_ballot(gm >= wc.floor) == 0) return;
  refresh(wc);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (wave_ballot(vmax[u] >= wc.floor) == 0) continue;
    float z[EPV];
    VT::unpack(opaque(g[u]), z);
    const uint32_t idu = id0 + uint32_t(u * kSupBlock * EPV);
    const bool ok = !PART || valid[u];
    if (!try_offer<EPV>(w, wc, z, idu, ok)) {        // no room: compact, the threshold rises, then it fits
      compact(w, wc, k, kWaveCap - EPV * 64);
      try_offer<EPV>(w, wc, z, idu, ok);
    }
  }
}

// ----------------------------------------------------------------------------------------------------------------
// the row's support from its k keys
// ----------------------------------------------------------------------------------------------------------------

// The set that global row `row` belongs to; r: the row's index within it.
__device__ __forceinline__ SupportRows row_set(const SupportParams& p, int64_t row, int64_t& r) {
  const bool second = row >= p.rows0;
  r = second ? row - p.rows0 : row;
  return second ? p.s1 : p.s0;
}

// The k largest of the n distinct keys a[0..n) in descending order to g_sup.sorted[0..min(n, k)). All threads of
// the workgroup. Up to kSupBlock keys: one rank pass. More: one wave's radix select moves the k largest to a[0..k)
// first, and those are ranked.
__device__ __forceinline__ void top_sorted(uint64_t* a, int n, int k) {
  if (n > kSupBlock) {
    if (threadIdx.x < 64) wave_select(a, n, k, g_sup.hist[0]);
    n = k;
    __syncthreads();
  }
  rank_keys(a, n, [&](uint64_t key, int r) {
    if (r < k) g_sup.sorted[r] = key;
  });
  __syncthreads();
}

// g_sup.sorted[0..kk): the row's largest keys in descending order, kk = min(k, keys the row offered); S: the row's
// sum of 2^((z - M) * c) with M its max (renorm = 0); nan: a NaN was seen. All threads of the workgroup.
__device__ __forceinline__ void finish_row(const SupportParams& p, int64_t grow, int kk, double S, bool nan) {
  const int tid = threadIdx.x, w = tid >> 6, k = p.k;
  int64_t row;
  const SupportRows rs = row_set(p, grow, row);
  const float z0 = kk > 0 ? val_of(g_sup.sorted[0]) : NAN;
  int32_t* ids = rs.ids + row * k;
  float* probs = rs.probs + row * k;
  if (nan || kk < k || !(z0 < INFINITY) || z0 == -INFINITY) {   // NaN, +inf, or a row all -inf
    for (int j = tid; j < k; j += kSupBlock) {
      ids[j] = -1;
      probs[j] = NAN;
    }
    if (tid == 0) {
      if (rs.count) rs.count[row] = 0;
      if (rs.flags) rs.flags[row] = SV_FLAG_NONFINITE;
    }
    return;
  }
  const bool mine = tid < k;
  const uint64_t key = mine ? g_sup.sorted[tid] : 0ull;
  const double a0 = double(z0) / p.T;
  const double e = mine ? exp(double(val_of(key)) / p.T - a0) : 0.0;
  // inclusive running sum over the slots (threads at and past k add 0)
  double incl = wave_incl_scan(e);
  if ((tid & 63) == 63) g_sup.redd[w] = incl;
  __syncthreads();
  double carry = 0.0, total = 0.0;
#pragma unroll
  for (int i = 0; i < kSupWaves; ++i) {
    const double t = g_sup.redd[i];
    if (i < w) carry += t;
    total += t;
  }
  const double cum = incl + carry;
  const bool below = tid < k - 1 && cum / total < p.top_p;
  const int count = 1 + __syncthreads_count(below);
  if (tid == count - 1) g_sup.dval = cum;
  __syncthreads();
  if (mine) {
    float pr = 0.f;
    if (tid < count) pr = float(p.renorm ? e / g_sup.dval : e / S);
    ids[tid] = id_of(key);
    probs[tid] = pr;
  }
  if (tid == 0) {
    if (rs.count) rs.count[row] = count;
    if (rs.flags) rs.flags[row] = 0u;
  }
}

template <typename T, bool SUM>
__device__ __forceinline__ void support_item(const SupportParams& p, int64_t row, int seg, int nseg, bool seen) {
  using VT = Vec<T>;
  constexpr int EPV = VT::kEPV;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int64_t rec = row * p.nlay + seg;            // this segment's records in the workspace
  const int k = p.k;
  int64_t srow;
  const SupportRows rs = row_set(p, row, srow);
  const T* base = static_cast<const T*>(rs.logits) + srow * rs.ld;
  const int64_t V = p.V;

  if (lane == 0) lds_store_u64(&g_sup.theta[w], 0ull);
  if (tid == 0) {
    g_sup.pool_n = 0;
    g_sup.pool_in = 0;
  }
  WaveCands wc;
  set_theta(wc, 0ull);
  wc.cnt = 0;
  wc.exact = false;
  wc.seeded = false;
  RowRun st{-INFINITY, -INFINITY, 0.f};
  bool nan = false;

  // head (until 16-byte alignment: segment 0), vector body, tail (the last segment)
  const uintptr_t addr = reinterpret_cast<uintptr_t>(base);
  int64_t head = int64_t(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int64_t nvec = (V - head) / EPV;
  const int64_t v0 = nvec * seg / nseg, v1 = nvec * (seg + 1) / nseg;
  const int64_t tail0 = head + nvec * EPV;

  auto scalar_part = [&](int64_t i0, int64_t i1) {   // fewer than EPV elements: one pass of the block
    const int64_t i = i0 + tid;
    const bool valid = i < i1;
    const float z = valid ? VT::load1(base + i) : -INFINITY;
    nan |= valid && z != z;
    if constexpr (SUM) {
      if (valid) sum_absorb<1>(st, &z, z, p.c);
    }
    refresh(wc);
    if (!try_offer<1>(w, wc, &z, uint32_t(i), valid)) {
      compact(w, wc, k, kWaveCap - 64);
      try_offer<1>(w, wc, &z, uint32_t(i), valid);   // fits: at most kWaveCap - 64 keys are kept
    }
  };
  __syncthreads();                                   // thresholds cleared before any wave reads them
  if (seg == 0 && head > 0) scalar_part(0, head);
  if (seg == nseg - 1 && tail0 < V) scalar_part(tail0, V);

  // Vector body: thread tid takes vectors v0 + tid + u * BLOCK (u < U) of each round of U * BLOCK vectors. Full
  // rounds go in pairs, the next round's loads in flight while a round is evaluated (the loads are unconditional:
  // the last pair reloads its second round instead of loading past it); the rounds left over run one at a time,
  // masked where they pass the end of the segment.
  const uint4* vp = reinterpret_cast<const uint4*>(base + head);
  constexpr int U = kRoundVecs<T>;
  constexpr int64_t kStep = int64_t(U) * kSupBlock;
  const int64_t nround = (v1 - v0 + kStep - 1) / kStep;
  const int64_t npair = (v1 - v0) / kStep / 2;       // pairs of full rounds
  const int64_t v = v0 + tid;
  const uint32_t id_v = uint32_t(head + v * EPV);    // id of this thread's first element
  constexpr uint32_t kIdStep = uint32_t(kStep * EPV);
  // round r's vectors for this thread; addresses past the segment reload its last vector (masked out later)
  auto load_round = [&](uint4* g, int64_t r) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t vi = v + r * kStep + int64_t(u) * kSupBlock;
      g[u] = load_vec<true>(vp + (vi < v1 ? vi : v1 - 1));
    }
  };
  auto masks = [&](bool* valid, int64_t r) {
#pragma unroll
    for (int u = 0; u < U; ++u) valid[u] = v + r * kStep + int64_t(u) * kSupBlock < v1;
  };
  uint4 ga[U], gb[U];
  if (nround > 0) load_round(ga, 0);
  for (int64_t r = 0; r < 2 * npair; r += 2) {
    load_round(gb, r + 1);
    // the next round's loads issue before this round's data is waited for: nothing is scheduled across this point
    __builtin_amdgcn_sched_barrier(0);
    take_round<T, SUM, false>(w, wc, st, nan, k, p.c, ga, id_v + uint32_t(r) * kIdStep, nullptr);
    load_round(ga, r + 2 < nround ? r + 2 : r + 1);  // the next pair's first round, or the first round left over
    __builtin_amdgcn_sched_barrier(0);
    take_round<T, SUM, false>(w, wc, st, nan, k, p.c, gb, id_v + uint32_t(r + 1) * kIdStep, nullptr);
    if (r == 0 && npair > 1) {
      if (nseg == 1) pilot_async(w, wc, k);
      else pilot(w, wc, k);
    }
  }
  // at most two rounds left (a full one and the partial one); the first is already in ga
  for (int64_t r = 2 * npair; r < nround; ++r) {
    if (r > 2 * npair) load_round(ga, r);
    bool valid[U];
    masks(valid, r);
    take_round<T, SUM, true>(w, wc, st, nan, k, p.c, ga, id_v + uint32_t(r) * kIdStep, valid);
  }

  // each wave drops its keys below the workgroup's best threshold (the segment's k largest are all at or above
  // it) and keeps at most SV_MAX_K; the waves' keys side by side; the segment's k largest, in order
  refresh(wc);
  if (wc.theta != 0) wc.cnt = keep_from(g_sup.buf + w * kWaveCap, wc.cnt, wc.theta);
  if (wc.cnt > SV_MAX_K) compact(w, wc, k, SV_MAX_K);
  if (lane == 0) g_sup.cnt[w] = wc.cnt;
  const bool seg_nan = __syncthreads_or(nan) != 0;
  int off = 0, n = 0;
#pragma unroll
  for (int i = 0; i < kSupWaves; ++i) {
    const int ci = g_sup.cnt[i];
    if (i < w) off += ci;
    n += ci;
  }
  for (int j = lane; j < wc.cnt; j += 64) g_sup.uni[off + j] = (g_sup.buf + w * kWaveCap)[j];
  __syncthreads();
  top_sorted(g_sup.uni, n, k);
  const int kk = n < k ? n : k;

  // the segment's full-row statistics (renorm = 0): common max, then each thread's sum rescaled in float64
  float Mseg = -INFINITY;
  double Sseg = 0.0;
  if constexpr (SUM) {
    Mseg = block_max<kSupBlock>(st.m, g_sup.redf);
    double sv = 0.0;
    if (st.m != -INFINITY && Mseg != -INFINITY) sv = double(st.s) * exp2(double(st.mc) - double(Mseg) * double(p.c));
    Sseg = block_sum<kSupBlock>(sv, g_sup.redd);
  }
  __syncthreads();

  if (nseg == 1) {
    finish_row(p, row, kk, Sseg, seg_nan);
    return;
  }

  // several segments: publish this one's keys and statistics, count it; the row's last segment merges
  uint64_t* kout = p.keys + rec * k;
  for (int j = tid; j < kk; j += kSupBlock) st_dev(kout + j, g_sup.sorted[j]);
  if (tid == 0) {
    SupPartial* pp = p.part + rec;
    st_dev(&pp->m, Mseg);
    st_dev(&pp->nk, int32_t(kk));
    st_dev(&pp->nan, uint32_t(seg_nan));
    st_dev(&pp->s, Sseg);
  }
  __builtin_amdgcn_s_waitcnt(0);                     // this segment's records are complete before it is counted
  __syncthreads();
  int32_t* ctr = p.ctr + row * kSupCtrStride;
  if (tid == 0) {
    if (seen || ws_ready(p.ws, p.sig)) {
      g_sup.flag = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) == nseg - 1;
    } else {                                         // never counted: the row is not merged in this call
      ws_mark_dirty(p.ws);
      g_sup.flag = 0;
    }
  }
  __syncthreads();
  if (!g_sup.flag) return;
  // every segment of the row has counted itself: wave 0 reads their statistics, one lane per segment (in parallel)
  const int64_t item0 = row * p.nlay;
  if (w == 0) {
    int nk = 0;
    float m = -INFINITY;
    uint32_t nn = 0;
    double sv = 0.0;
    if (lane < nseg) {
      const SupPartial* pp = p.part + item0 + lane;
      nk = clamp_count(ld_dev(&pp->nk), k);        // a count read back is never trusted as an extent
      m = ld_dev(&pp->m);
      nn = ld_dev(&pp->nan);
      if (SUM) sv = ld_dev(&pp->s);
    }
    const int incl = wave_incl_scan_i(nk);
    if (lane < nseg) g_sup.segoff[lane] = incl - nk;
    if (lane == 0) g_sup.segoff[nseg] = __builtin_amdgcn_readlane(incl, 63);
    const float M = wave_max_f(m);
    double term = 0.0;
    if (SUM && m != -INFINITY && M != -INFINITY) term = sv * exp2(double(m) * double(p.c) - double(M) * double(p.c));
    const double S = SUM ? wave_sum(term) : 0.0;
    const bool anynan = wave_ballot(nn != 0u) != 0;
    if (lane == 0) {
      st_dev(ctr, 0);
      g_sup.dval = S;
      g_sup.ival = int32_t(anynan);
    }
  }
  __syncthreads();
  const bool row_nan = g_sup.ival != 0;
  const double S = g_sup.dval;
  // the segments' keys side by side in the merge area: every load issued before any is used (a flat index per
  // thread and step, its segment found from the offsets; indices past the end reload the first key)
  uint64_t* merge = g_sup.buf;
  const int nall = g_sup.segoff[nseg];
  int so[kMaxSeg];
#pragma unroll
  for (int t = 0; t < kMaxSeg; ++t) so[t] = t < nseg ? g_sup.segoff[t] : INT32_MAX;
  constexpr int KPT = kMergeCap / kSupBlock;
  uint64_t kv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int f = i * kSupBlock + tid;
    const int fc = f < nall ? f : 0;
    int sidx = 0, base = 0;
#pragma unroll
    for (int t = 1; t < kMaxSeg; ++t)
      if (fc >= so[t]) { sidx = t; base = so[t]; }
    kv[i] = nall > 0 ? ld_dev(p.keys + (item0 + sidx) * k + (fc - base)) : 0ull;
  }
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int f = i * kSupBlock + tid;
    if (f < nall) merge[f] = kv[i];
  }
  __syncthreads();
  top_sorted(merge, nall, k);
  finish_row(p, row, nall < k ? nall : k, S, row_nan);
}

template <typename T, bool SUM>
__global__ __launch_bounds__(kSupBlock) __attribute__((amdgpu_waves_per_eu(4, 4))) void k_support(SupportParams p) {
  const int64_t item = int64_t(blockIdx.x);
  // workgroup 0 makes sure the row counters are at zero for this call's layout; the others confirm it before
  // counting (only rows cut into segments count)
  if (item == 0) ws_claim(p.ws, p.sig, size_t(p.ctl_end), &g_sup.flag);
  // the segments of the rows past the head first, then the whole rows
  const int64_t nfirst = p.items - p.head_rows;
  if (item >= nfirst) {
    support_item<T, SUM>(p, item - nfirst, 0, 1, true);
  } else {
    const bool seen = item == 0 || ws_seen_clean(p.ws, p.sig);   // read while the segment streams
    support_item<T, SUM>(p, p.head_rows + item / p.nseg, int(item % p.nseg), p.nseg, seen);
  }
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Segments per row that the row's bytes and the merge area allow.
int32_t max_segments(int64_t V, int64_t es, int32_t k) {
  int64_t n = V * es / kMinSegBytes;
  n = std::min<int64_t>(n, kMaxSeg);
  n = std::min<int64_t>(n, kMergeCap / std::max<int32_t>(k, 1));
  return int32_t(std::max<int64_t>(n, 1));
}

}  // namespace

SupportPlan make_support_plan(int64_t rows, int64_t V, int32_t k, int dtype, int64_t resident) {
  SupportPlan p;
  p.rows = rows; p.V = V; p.k = k;
  const int32_t nlayout = max_segments(V, 4, k);     // the float32 bound sizes the workspace for both dtypes
  const int32_t ncap = max_segments(V, dtype == SV_BF16 ? 2 : 4, k);
  // Whole rows, one workgroup each, in full resident rounds. The rows of a last, partial round would stream alone at
  // one workgroup's rate, so they are cut into segments, items of their own queued before the whole rows.
  const int64_t R = std::max<int64_t>(resident, 1);
  const int64_t tail = rows % R;
  p.head_rows = rows - tail;
  p.nlay = nlayout;
  if (tail == 0) {
    p.nseg = 1;
    p.items = rows;
  } else {
    p.nseg = int32_t(std::min<int64_t>(ncap, std::max<int64_t>(1, R / tail)));
    p.items = p.head_rows + tail * p.nseg;
  }
  size_t off = kWsHeaderBytes;
  p.off_ctr = off;  off = align_up(off + size_t(rows) * kSupCtrStride * sizeof(int32_t), 256);
  p.ctr_bytes = off;
  p.off_keys = off; off = align_up(off + size_t(rows) * nlayout * size_t(k) * sizeof(uint64_t), 256);
  p.off_part = off; off = align_up(off + size_t(rows) * nlayout * sizeof(SupPartial), 256);
  p.total = off;
  return p;
}

hipError_t launch_support(const SupportPlan& plan, const SupportArgs& a, hipStream_t stream) {
  char* ws = a.ws;
  SupportParams p{};
  p.ws = ws;
  p.sig = ws_signature(kLayoutSupport, uint64_t(plan.rows));
  p.ctl_end = int64_t(plan.ctr_bytes);
  p.s0 = a.set[0]; p.s1 = a.set[1]; p.rows0 = a.set[0].rows;
  p.rows = plan.rows; p.V = plan.V;
  p.k = plan.k; p.renorm = a.renorm;
  p.head_rows = plan.head_rows; p.nseg = plan.nseg; p.nlay = plan.nlay; p.items = plan.items;
  const double T = double(a.temperature);
  p.c = float(1.4426950408889634074 / T);
  p.T = T;
  p.top_p = double(a.top_p);
  p.ctr = reinterpret_cast<int32_t*>(ws + plan.off_ctr);
  p.keys = reinterpret_cast<uint64_t*>(ws + plan.off_keys);
  p.part = reinterpret_cast<SupPartial*>(ws + plan.off_part);
  const unsigned grid = unsigned(plan.items);
  auto kern = a.dtype == SV_BF16 ? (a.renorm ? k_support<uint16_t, false> : k_support<uint16_t, true>)
                                 : (a.renorm ? k_support<float, false> : k_support<float, true>);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kSupBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
