// Tree (multi-candidate) verification for gfx950 (MI355X).
//
// The rule. The pages verify trees of drafted tokens (the Uno page's B = 16 tree sampler, section "One backbone, two
// pathways"; EAGLE-2's dynamic trees and DFlash2's top-m candidates per position, DFlash/DFlash2 guide sections 3 and
// 5.2) but state the acceptance rule for one candidate per position only, and its one-hot form for a greedy drafter
// (Uno, "What 'lossless' actually has to mean"). For several candidates this is SpecInfer's multi-step speculative
// sampling (Miao et al., ASPLOS 2024) with q one-hot at each candidate: at node u the children are tested in node
// order, child c with token x passing when u_accept[c] < min(1, p'(x)), p' = softmax(z_u / T) renormalised outside the
// tokens of the children already rejected at u; the walk continues at a passing child; where every child fails (or at
// a leaf) one token is drawn from p' by inverse CDF at t = u_sample[u] * (its mass).
//
// Two launches on the caller's stream, no waits inside either:
//  - k_tree_rows: one 256-thread workgroup per node row (sequence b, node u). It streams the row once with 16-byte
//    non-temporal loads and keeps the running max and the float32 running sum of 2^((z - max) * log2(e)/T) over the
//    row WITHOUT the drafted tokens of u's children (each thread lists the few child tokens that fall in its share of
//    the row and masks them as it streams), and gathers the logit of every child. Every denominator of the walk is
//    then a sum of positive terms (the rest of the row, plus the children not rejected yet), so a child holding most
//    of the mass cannot leave a remainder that cancels. The last row of a sequence to finish (a counter) walks the
//    tree in float64 and publishes where it stopped.
//  - k_tree_draw: per sequence, tasks of at least 4 chunks of 512 elements of the stop row (all tasks about one
//    resident round): float64 weights (table-driven
//    2^y) with the rejected children's tokens removed, one sum per chunk; the last task of the sequence finds the
//    chunk holding t, recomputes it and searches it.
// Bound: HBM, B * N * V * s bytes in the first launch (every node row once); the draw re-reads one row per sequence.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>

#include "sv.h"
#include "sv_device.h"
#include "sv_internal.h"
#include "sv_wshdr.h"
#include "sv_fexp.h"

namespace sv {
namespace {

constexpr int kTBlock = 256;
constexpr int kTWaves = kTBlock / 64;
constexpr int kTU = 4;                 // 16-byte vectors per thread per group of the row stream
constexpr int kHits = 8;               // masked elements one thread keeps in its list (more: the exact slow path)
constexpr int kTChunk = 512;           // elements per chunk of the draw (8 per lane of a wave)
constexpr int kTPer = kTChunk / 64;

struct TreeParams {
  const void* tgt; int64_t t_seq, t_row;
  int64_t B; int32_t N; int64_t V;
  float c;                             // log2(e) / T rounded to float: the row sums and the walk's weights
  double c2;                           // log2(e) / T in float64: the draw's weights
  const int32_t* parent; const int32_t* token; const float* ua; const float* us;
  uint8_t* accept; int32_t* n_acc; int32_t* path; int32_t* out_token; float* p_test; uint32_t* flags;
  char* ws; uint64_t sig; int64_t ctl_end;
  int32_t* ctr1;                       // per sequence: rows finished (first launch)
  int32_t* ctr2;                       // per sequence: draw tasks finished (second launch)
  TreeRow* rows;                       // per (b, node): the row's statistics outside its children's tokens
  float* zc;                           // per (b, node c >= 1): logit of c's token in its parent's row
  TreeJob* jobs;                       // per b: where the walk stopped
  double* chunk;                       // per (b, chunk): float64 weight of the chunk of the stop row
  int64_t nch;                         // chunks per row
  int32_t ntask;                       // draw tasks per sequence
  int32_t task_chunks;                 // chunks per draw task
};

struct TreeShared {
  int32_t par[SV_MAX_TREE_NODES];
  int32_t tok[SV_MAX_TREE_NODES];
  union {
    struct {                           // the row pass (and the draw)
      int32_t xs[SV_MAX_TREE_NODES];   // masked tokens: the child tokens of the row's node (or of the stop node)
      int32_t hits[kTBlock][kHits];    // per thread: the masked elements it streams, (group << 8) | slot
    } rp;
    struct {                           // the walk, after the row pass of the same workgroup
      float rm[SV_MAX_TREE_NODES];     // per node: max of its row outside its children's tokens (NaN: bad row)
      double rs[SV_MAX_TREE_NODES];    // per node: the sum relative to it
      float zk[SV_MAX_TREE_NODES];     // per node >= 1: its logit in its parent's row
      int32_t kid[SV_MAX_TREE_NODES];  // the children of the current node in node order
      double pk[SV_MAX_TREE_NODES];    // p'(x) of each of them
    } wk;
  } u;
  double redd[kTWaves];
  float redf[kTWaves];
  int32_t nx, overflow, flag;
};
__shared__ TreeShared g_tree;          // at file scope: functions that are not inlined reach it as LDS

// Running state of one thread: max m, mc = fl(m * c), s = sum of 2^(z*c - mc) (the dense verifier's one-pass form).
struct TRun {
  float m, mc, s;
};
template <int K>
__device__ __forceinline__ void t_absorb(TRun& st, const float* v, float c) {
  float cm = v[0];
#pragma unroll
  for (int k = 1; k < K; ++k) cm = fmaxf(cm, v[k]);
  const float mn = fmaxf(st.m, cm);
  if (mn == -INFINITY) {                             // only -inf (or NaN) so far: nothing to add, but keep NaN
#pragma unroll
    for (int k = 0; k < K; ++k)
      if (v[k] != v[k]) st.s = NAN;
    return;
  }
  const float mnc = __fmul_rn(mn, c);
  if (mn != st.m) {
    st.s *= ex2f(st.mc - mnc);
    st.m = mn;
    st.mc = mnc;
  }
  float t[K];
#pragma unroll
  for (int k = 0; k < K; ++k) t[k] = ex2f(fmaf(v[k], c, -mnc));
#pragma unroll
  for (int w = 1; w < K; w <<= 1)
#pragma unroll
    for (int k = 0; k + w < K; k += 2 * w) t[k] += t[k + w];
  st.s += t[0];
}

__device__ __forceinline__ bool in_list(const int32_t* xs, int n, int64_t i) {
  for (int j = 0; j < n; ++j)
    if (xs[j] == i) return true;
  return false;
}

// One group of the row stream: the thread's kTU vectors tid + (g * kTU + k) * kTBlock; vectors past the row's last
// one read that vector again (every load is unconditional) and count as -inf.
template <typename T>
__device__ __forceinline__ void t_load_group(uint4 (&w)[kTU], const uint4* vp, int64_t g, int64_t nvec) {
#pragma unroll
  for (int k = 0; k < kTU; ++k) {
    const int64_t v = int64_t(threadIdx.x) + (g * kTU + k) * kTBlock;
    w[k] = load_vec<true>(vp + (v < nvec ? v : nvec - 1));
  }
}
template <typename T>
__device__ __forceinline__ void t_fold_group(TRun& st, const uint4 (&w)[kTU], int64_t g, int64_t nvec, int nh,
                                             const int32_t* hits, float c) {
  constexpr int EPV = Vec<T>::kEPV;
  float z[kTU * EPV];
#pragma unroll
  for (int k = 0; k < kTU; ++k) {
    Vec<T>::unpack(w[k], z + k * EPV);
    const int64_t v = int64_t(threadIdx.x) + (g * kTU + k) * kTBlock;
    if (v >= nvec)
#pragma unroll
      for (int e = 0; e < EPV; ++e) z[k * EPV + e] = -INFINITY;
  }
  if (nh > 0) {                                      // rare: a child token in this thread's share
    for (int j = 0; j < nh; ++j) {
      const int h = hits[j];
      if ((h >> 8) != int(g)) continue;
      const int slot = h & 255;
#pragma unroll
      for (int q = 0; q < kTU * EPV; ++q) z[q] = q == slot ? -INFINITY : z[q];
    }
  }
  t_absorb<kTU * EPV>(st, z, c);
}

// The statistics of row (b, u) outside the tokens of u's children, and the logit of every child: by every thread.
template <typename T>
__device__ void tree_row_pass(const TreeParams& p, int64_t b, int u) {
  TreeShared& sh = g_tree;
  constexpr int EPV = Vec<T>::kEPV;
  const int tid = threadIdx.x;
  const int N = p.N;
  const int64_t V = p.V;
  const T* row = static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(u) * p.t_row;
  if (tid == 0) { sh.nx = 0; sh.overflow = 0; }
  for (int i = tid; i < N; i += kTBlock) {
    sh.par[i] = p.parent[b * N + i];
    sh.tok[i] = p.token[b * N + i];
  }
  __syncthreads();
  // the children of u: their logits (device-scope stores, read by the walk) and the tokens to mask
  for (int ci = 1 + tid; ci < N; ci += kTBlock) {
    if (sh.par[ci] != u) continue;
    const int x = sh.tok[ci];
    float z = NAN;
    if (x >= 0 && int64_t(x) < V) {
      z = Vec<T>::load1(row + x);
      sh.u.rp.xs[atomicAdd(&sh.nx, 1)] = x;
    }
    st_dev(p.zc + b * N + ci, z);
  }
  __syncthreads();
  const int nx = sh.nx;

  // layout: head elements up to 16-byte alignment, vectors (groups of kTU per thread), tail elements
  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int64_t head = int64_t(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int64_t nvec = (V - head) / EPV;
  const int64_t tail0 = head + nvec * EPV;
  const int64_t ngroups = (nvec + int64_t(kTU) * kTBlock - 1) / (int64_t(kTU) * kTBlock);
  const uint4* vp = reinterpret_cast<const uint4*>(row + head);

  // the masked elements this thread streams
  int nh = 0;
  for (int j = 0; j < nx; ++j) {
    const int64_t x = sh.u.rp.xs[j];
    if (x < head || x >= tail0) continue;
    const int64_t vx = (x - head) / EPV;
    if (int(vx % kTBlock) != tid) continue;
    const int g = int(vx / (int64_t(kTU) * kTBlock)), k = int((vx / kTBlock) % kTU), e = int((x - head) % EPV);
    if (nh < kHits) sh.u.rp.hits[tid][nh] = (g << 8) | (k * EPV + e);
    ++nh;
  }
  if (nh > kHits) atomicOr(&sh.overflow, 1);
  __syncthreads();
  const bool slow = sh.overflow != 0;

  TRun st{-INFINITY, -INFINITY, 0.f};
  const float c = p.c;
  if (!slow) {
    for (int64_t i = tid; i < head; i += kTBlock) {
      float z = Vec<T>::load1(row + i);
      if (in_list(sh.u.rp.xs, nx, i)) z = -INFINITY;
      t_absorb<1>(st, &z, c);
    }
    if (ngroups > 0) {
      // two register sets in turn: while one group is folded the next one's loads are in flight
      uint4 wa[kTU], wb[kTU];
      t_load_group<T>(wa, vp, 0, nvec);
      int64_t g = 0;
      for (; g + 1 < ngroups; g += 2) {
        t_load_group<T>(wb, vp, g + 1, nvec);
        t_fold_group<T>(st, wa, g, nvec, nh, sh.u.rp.hits[tid], c);
        if (g + 2 < ngroups) t_load_group<T>(wa, vp, g + 2, nvec);
        t_fold_group<T>(st, wb, g + 1, nvec, nh, sh.u.rp.hits[tid], c);
      }
      if (g < ngroups) t_fold_group<T>(st, wa, g, nvec, nh, sh.u.rp.hits[tid], c);
    }
    for (int64_t i = tail0 + tid; i < V; i += kTBlock) {
      float z = Vec<T>::load1(row + i);
      if (in_list(sh.u.rp.xs, nx, i)) z = -INFINITY;
      t_absorb<1>(st, &z, c);
    }
  } else {                                           // many child tokens in one thread's share: element by element
    for (int64_t i = tid; i < V; i += kTBlock) {
      float z = Vec<T>::load1(row + i);
      if (in_list(sh.u.rp.xs, nx, i)) z = -INFINITY;
      t_absorb<1>(st, &z, c);
    }
  }

  // fold the threads: common max M, each thread's sum rescaled to it in float64
  const float M = block_max<kTBlock>(st.m, sh.redf);
  double s = 0.0;
  if (st.m != -INFINITY && M != -INFINITY) s = double(st.s) * exp2(double(st.mc) - double(M) * double(c));
  else if (isnan(st.s)) s = NAN;
  s = block_sum<kTBlock>(s, sh.redd);
  if (tid == 0) {
    TreeRow* r = p.rows + b * N + u;
    st_dev(&r->m, M);
    st_dev(&r->bad, uint32_t(isnan(s) || M == INFINITY));
    st_dev(&r->s, s);
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The walk of sequence b by wave 0 of the workgroup of its last row (sh.par / sh.tok hold its tree), with no barrier:
// every row record and child logit the walk may read comes into LDS in one round of loads; at each node the children
// are listed in node order (ballots), the tests are evaluated for all of them at once (p'(x) over the mass outside
// the earlier siblings' tokens: the rest of the row plus a suffix sum of the later siblings' weights, positive terms
// only), and the first passing child is found with a ballot. Writes the outputs of every node and the draw job.
__device__ void tree_walk(const TreeParams& p, int64_t b) {
  TreeShared& sh = g_tree;
  const int lane = threadIdx.x & 63;
  const int N = p.N;
  const int64_t V = p.V;
  const double c = double(p.c);
  int bad = 0;
  for (int i = lane; i < N; i += 64) {
    const TreeRow* r = p.rows + b * N + i;
    const float m = ld_dev(&r->m);
    const double s = ld_dev(&r->s);
    const uint32_t rb = ld_dev(&r->bad);
    const float z = i > 0 ? ld_dev(p.zc + b * N + i) : 0.f;
    sh.u.wk.rm[i] = rb ? NAN : m;
    sh.u.wk.rs[i] = s;
    sh.u.wk.zk[i] = z;
    if (i > 0) bad |= !(sh.par[i] >= 0 && sh.par[i] < i) || !(sh.tok[i] >= 0 && int64_t(sh.tok[i]) < V);
    p.accept[b * N + i] = 0;
    p.path[b * N + i] = -1;
    if (p.p_test) p.p_test[b * N + i] = NAN;
  }
  bad = __any(bad);
  wave_sync();
  uint32_t fl = bad ? SV_FLAG_ID_RANGE : 0u;
  int cur = 0, n = 0, stop = -1;
  float mstop = 0.f;
  while (!bad) {
    wave_sync();                                     // the previous level's reads of kid / pk are done
    // children of cur in node order
    int nk = 0;
    for (int c0 = 1; c0 < N; c0 += 64) {
      const int ci = c0 + lane;
      const bool hit = ci < N && sh.par[ci] == cur;
      const uint64_t m = wave_ballot(hit);
      if (hit) sh.u.wk.kid[nk + lane_rank(m)] = ci;
      nk += __popcll(m);
    }
    wave_sync();
    // the row's maximum (the rest's and the children's) and its faults
    float mk = -INFINITY;
    int kbad = 0;
    for (int j = lane; j < nk; j += 64) {
      const float z = sh.u.wk.zk[sh.u.wk.kid[j]];
      kbad |= !(z < INFINITY);
      mk = fmaxf(mk, z);
    }
    mk = wave_max_f(mk);
    kbad = __any(kbad);
    const float mr = sh.u.wk.rm[cur];
    const float M = fmaxf(mr, mk);
    if (mr != mr || kbad || M == -INFINITY) {        // a NaN or +inf in the row, or nothing but -inf
      fl |= SV_FLAG_NONFINITE;
      stop = -1;
      break;
    }
    const double rest = mr == -INFINITY ? 0.0 : sh.u.wk.rs[cur] * exp2((double(mr) - double(M)) * c);
    // p'(x) of every child, chunks of 64 from the last: a child's denominator is the rest plus the weights of the
    // first holders of the tokens of it and of its later siblings (reverse scan within a chunk, carry across chunks)
    double carry = 0.0;
    for (int c0 = ((nk + 63) / 64 - 1) * 64; c0 >= 0; c0 -= 64) {
      const int j = c0 + lane;
      const bool valid = j < nk;
      const int ci = valid ? sh.u.wk.kid[j] : 0;
      int first = valid;
      for (int i = 0; i < j && first && valid; ++i) first = sh.tok[sh.u.wk.kid[i]] != sh.tok[ci];
      const double ex = first ? exp2((double(sh.u.wk.zk[ci]) - double(M)) * c) : 0.0;
      const double rev = wave_incl_scan(__shfl(ex, 63 - lane));   // suffix sums, read back in lane order
      const double suffix = __shfl(rev, 63 - lane);
      if (valid) sh.u.wk.pk[j] = first ? ex / (rest + (carry + suffix)) : 0.0;
      carry += readlane_d(rev, 63);
    }
    wave_sync();
    // the tests in node order: the first passing child is accepted
    int next = -1;
    for (int c0 = 0; c0 < nk && next < 0; c0 += 64) {
      const int j = c0 + lane;
      const bool valid = j < nk;
      const int ci = valid ? sh.u.wk.kid[j] : 0;
      const double P = valid ? sh.u.wk.pk[j] : 0.0;
      const float u = valid ? p.ua[b * N + ci] : 1.f;
      const uint64_t pass = wave_ballot(valid && double(u) < fmin(1.0, P));
      const int jstar = pass ? c0 + __builtin_ctzll(pass) : INT_MAX;
      if (valid && j <= jstar && p.p_test) p.p_test[b * N + ci] = float(P);
      if (pass) next = __builtin_amdgcn_readlane(ci, __builtin_ctzll(pass));
    }
    if (next < 0) {
      stop = cur;
      mstop = M;
      break;
    }
    if (lane == 0) {
      p.accept[b * N + next] = 1;
      p.path[b * N + n] = next;
    }
    ++n;
    cur = next;
  }
  if (lane == 0) {
    const bool fatal = stop < 0;
    TreeJob jb{};
    jb.stop = stop;
    jb.m = fatal ? 0.f : mstop;
    jb.u = fatal ? 0.f : p.us[b * N + stop];
    jb.flags = fl;
    p.jobs[b] = jb;
    p.n_acc[b] = fatal ? -1 : n;
    p.out_token[b] = -1;
    if (p.flags) p.flags[b] = fl;
  }
  if (stop < 0) {                                    // a failed sequence: no accepted node, no tested node
    __builtin_amdgcn_s_waitcnt(0);
    for (int i = lane; i < N; i += 64) {
      p.accept[b * N + i] = 0;
      p.path[b * N + i] = -1;
      if (p.p_test) p.p_test[b * N + i] = NAN;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(kTBlock) void k_tree_rows(TreeParams p) {
  TreeShared& sh = g_tree;
  const int64_t item = blockIdx.x;
  const int64_t b = item / p.N;
  const int u = int(item % p.N);
  // workgroup 0 makes sure the counters are at zero for this call's layout; the others confirm it before counting
  if (item == 0) ws_claim(p.ws, p.sig, size_t(p.ctl_end), &sh.flag);
  const bool seen = item == 0 || ws_seen_clean(p.ws, p.sig);
  tree_row_pass<T>(p, b, u);
  __builtin_amdgcn_s_waitcnt(0);                     // this row's records are complete before it is counted
  __syncthreads();
  if (threadIdx.x == 0) {
    if (seen || ws_ready(p.ws, p.sig)) {
      sh.flag = ctr_add(p.ctr1 + b) == p.N - 1;
    } else {                                         // never counted: the sequence is not walked in this call
      ws_mark_dirty(p.ws);
      sh.flag = 0;
    }
  }
  __syncthreads();
  if (!sh.flag || threadIdx.x >= 64) return;       // the walk is wave 0's
  tree_walk(p, b);
  if (threadIdx.x == 0) st_dev(p.ctr1 + b, int32_t(0));   // ready for the next call
}

// The float64 weights of the lane's kTPer elements of chunk c of the stop row, the stop node's child tokens (sh.xs,
// nx of them) removed unless `all`; the same operations every time, so repeated evaluations agree bit for bit.
template <typename T>
__device__ __forceinline__ void t_chunk_weights(const T* row, bool vec, int64_t V, int64_t c, double c2, double nm,
                                                int nx, bool all, double* w) {
  const int lane = threadIdx.x & 63;
  const int64_t i0 = c * kTChunk + int64_t(lane) * kTPer;
  float z[kTPer];
  if (vec && i0 + kTPer <= V) {
    constexpr int NV = kTPer / Vec<T>::kEPV;
    const uint4* q = reinterpret_cast<const uint4*>(row + i0);
#pragma unroll
    for (int k = 0; k < NV; ++k) Vec<T>::unpack(gload4(q + k), z + k * Vec<T>::kEPV);
  } else {
#pragma unroll
    for (int e = 0; e < kTPer; ++e) z[e] = elem_or_ninf<T>(row, i0 + e, V);
  }
#pragma unroll
  for (int e = 0; e < kTPer; ++e) w[e] = fexp_scaled(xarg(z[e], c2, nm));
  if (!all) {
    for (int j = 0; j < nx; ++j) {
      const int64_t d = int64_t(g_tree.u.rp.xs[j]) - i0;
#pragma unroll
      for (int e = 0; e < kTPer; ++e) w[e] = d == e ? 0.0 : w[e];
    }
  }
}

// The pick of sequence b by wave 0 of its last draw task: the chunk whose running sum crosses t = u * total, then the
// element inside it (the chunk recomputed with the same operations). Returns the token (-1 when nothing has weight).
template <typename T>
__device__ int32_t tree_pick(const TreeParams& p, int64_t b, const TreeJob& job, const T* row, bool vec, int nx,
                             bool all) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = p.nch;
  const double* cs = p.chunk + b * nch;
  const double c2 = p.c2, nm = -(double(job.m) * c2);
  // running sums over the chunks in order, a wave scan per group of 64
  double carry = 0.0;
  int64_t cstar = -1, last = -1;
  double cbase = 0.0, total = 0.0;
  for (int64_t g0 = 0; g0 < nch; g0 += 64) total += wave_sum(g0 + lane < nch ? ld_dev(cs + g0 + lane) : 0.0);
  const double t = double(job.u) * total;
  for (int64_t g0 = 0; g0 < nch; g0 += 64) {
    const int64_t ci = g0 + lane;
    const double m = ci < nch ? ld_dev(cs + ci) : 0.0;
    const double incl = wave_incl_scan(m);
    const uint64_t pos = wave_ballot(m > 0.0);
    if (pos) last = g0 + 63 - __builtin_clzll(pos);
    if (cstar < 0) {
      const uint64_t hm = wave_ballot(m > 0.0 && carry + incl > t);
      if (hm) {
        const int l = __builtin_ctzll(hm);
        cstar = g0 + l;
        cbase = carry + (readlane_d(incl, l) - readlane_d(m, l));
      }
    }
    carry += readlane_d(incl, 63);
  }
  const bool clamp = cstar < 0;
  if (clamp) cstar = last;
  if (cstar < 0) return -1;
  double w[kTPer];
  t_chunk_weights<T>(row, vec, p.V, cstar, c2, nm, nx, all, w);
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kTPer; ++e) mine += w[e];
  double run = cbase + (wave_incl_scan(mine) - mine);
  int hit = -1, lastpos = -1;
#pragma unroll
  for (int e = 0; e < kTPer; ++e) {
    run += w[e];
    if (w[e] > 0.0) lastpos = e;
    if (hit < 0 && !clamp && w[e] > 0.0 && run > t) hit = e;
  }
  const uint64_t hh = wave_ballot(hit >= 0);
  if (hh) {
    const int l = __builtin_ctzll(hh);
    return int32_t(cstar * kTChunk + int64_t(l) * kTPer + __shfl(hit, l));
  }
  const uint64_t lp = wave_ballot(lastpos >= 0);
  if (!lp) return -1;
  const int l = 63 - __builtin_clzll(lp);
  return int32_t(cstar * kTChunk + int64_t(l) * kTPer + __shfl(lastpos, l));
}

template <typename T>
__global__ __launch_bounds__(kTBlock) void k_tree_draw(TreeParams p) {
  TreeShared& sh = g_tree;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int64_t b = int64_t(blockIdx.x) / p.ntask;
  const int task = int(int64_t(blockIdx.x) % p.ntask);
  const int N = p.N;
  // the job (written by the first launch) and the tree are requested together: the children of the stop node (all
  // rejected) give the tokens to remove
  const TreeJob job = p.jobs[b];
  for (int i = tid; i < N; i += kTBlock) {
    sh.par[i] = p.parent[b * N + i];
    sh.tok[i] = p.token[b * N + i];
  }
  fexp_fill_table();
  if (tid == 0) sh.nx = 0;
  __syncthreads();
  if (job.stop >= 0 && job.stop < N) {
    for (int ci = 1 + tid; ci < N; ci += kTBlock)
      if (sh.par[ci] == job.stop) {
        const int x = sh.tok[ci];
        if (x >= 0 && int64_t(x) < p.V) sh.u.rp.xs[atomicAdd(&sh.nx, 1)] = x;
      }
  }
  __syncthreads();
  const int nx = sh.nx;
  const bool live = job.stop >= 0 && job.stop < N;
  const T* row = live ? static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(job.stop) * p.t_row : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const double c2 = p.c2, nm = -(double(job.m) * c2);
  if (live) {
    const int64_t c0 = int64_t(task) * p.task_chunks, c1 = std::min<int64_t>(c0 + p.task_chunks, p.nch);
    for (int64_t ci = c0 + wave; ci < c1; ci += kTWaves) {
      double w[kTPer];
      t_chunk_weights<T>(row, vec, p.V, ci, c2, nm, nx, false, w);
      double s = 0.0;
#pragma unroll
      for (int e = 0; e < kTPer; ++e) s += w[e];
      s = wave_sum(s);
      st_dev(p.chunk + b * p.nch + ci, s);           // every lane stores the same value
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) sh.flag = ctr_add(p.ctr2 + b) == p.ntask - 1;
  __syncthreads();
  if (!sh.flag) return;
  // the last task of the sequence: the pick (wave 0)
  if (live && wave == 0) {
    uint32_t extra = 0;
    int32_t tok = tree_pick<T>(p, b, job, row, vec, nx, false);
    if (tok < 0) {                                   // the removed tokens held every weight: draw from p itself
      extra = SV_FLAG_EMPTY_RESIDUAL;
      for (int64_t ci = 0; ci < p.nch; ++ci) {
        double w[kTPer];
        t_chunk_weights<T>(row, vec, p.V, ci, c2, nm, nx, true, w);
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < kTPer; ++e) s += w[e];
        s = wave_sum(s);
        st_dev(p.chunk + b * p.nch + ci, s);
      }
      __builtin_amdgcn_s_waitcnt(0);
      tok = tree_pick<T>(p, b, job, row, vec, nx, true);
    }
    if ((threadIdx.x & 63) == 0) {
      p.out_token[b] = tok;
      if (p.flags) p.flags[b] = job.flags | extra;
    }
  }
  if (tid == 0) st_dev(p.ctr2 + b, int32_t(0));     // ready for the next call
}

}  // namespace

TreePlan make_tree_plan(int64_t B, int32_t N, int64_t V) {
  TreePlan pl;
  pl.B = B; pl.N = N; pl.V = V;
  pl.nch = (V + kTChunk - 1) / kTChunk;
  // draw tasks: the sequences' tasks together about fill one resident round (1024 workgroups), each task at least
  // 4 chunks (one per wave)
  const int64_t want = std::max<int64_t>(1, 1024 / std::max<int64_t>(B, 1));
  int64_t tc = std::max<int64_t>(4, (pl.nch + want - 1) / want);
  pl.task_chunks = int32_t(std::min<int64_t>(tc, std::max<int64_t>(pl.nch, 1)));
  pl.ntask = int32_t((pl.nch + pl.task_chunks - 1) / pl.task_chunks);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t off = kWsHeaderBytes;
  pl.off_ctr1 = off; off = up(off + size_t(B) * 4);
  pl.off_ctr2 = off; off = up(off + size_t(B) * 4);
  pl.ctl_end = off;
  pl.off_rows = off; off = up(off + size_t(B) * size_t(N) * sizeof(TreeRow));
  pl.off_zc = off; off = up(off + size_t(B) * size_t(N) * sizeof(float));
  pl.off_jobs = off; off = up(off + size_t(B) * sizeof(TreeJob));
  pl.off_chunk = off; off = up(off + size_t(B) * size_t(pl.nch) * sizeof(double));
  pl.total = off;
  return pl;
}

hipError_t launch_tree(const TreePlan& plan, const TreeArgs& a, hipStream_t stream) {
  TreeParams p{};
  p.tgt = a.tgt; p.t_seq = a.t_seq; p.t_row = a.t_row;
  p.B = plan.B; p.N = plan.N; p.V = plan.V;
  const double T = double(a.temperature);
  p.c = float(1.4426950408889634074 / T);
  p.c2 = 1.4426950408889634074 / T;
  p.parent = a.parent; p.token = a.token; p.ua = a.ua; p.us = a.us;
  p.accept = a.accept; p.n_acc = a.n_acc; p.path = a.path; p.out_token = a.out_token; p.p_test = a.p_test;
  p.flags = a.flags;
  p.ws = a.ws;
  p.sig = ws_signature(kLayoutTree, uint64_t(plan.B));
  p.ctl_end = int64_t(plan.ctl_end);
  p.ctr1 = reinterpret_cast<int32_t*>(a.ws + plan.off_ctr1);
  p.ctr2 = reinterpret_cast<int32_t*>(a.ws + plan.off_ctr2);
  p.rows = reinterpret_cast<TreeRow*>(a.ws + plan.off_rows);
  p.zc = reinterpret_cast<float*>(a.ws + plan.off_zc);
  p.jobs = reinterpret_cast<TreeJob*>(a.ws + plan.off_jobs);
  p.chunk = reinterpret_cast<double*>(a.ws + plan.off_chunk);
  p.nch = plan.nch; p.ntask = plan.ntask; p.task_chunks = plan.task_chunks;
  const unsigned g1 = unsigned(plan.B * plan.N), g2 = unsigned(plan.B * plan.ntask);
  if (a.dtype == SV_BF16) {
    hipLaunchKernelGGL(k_tree_rows<uint16_t>, dim3(g1), dim3(kTBlock), 0, stream, p);
    hipLaunchKernelGGL(k_tree_draw<uint16_t>, dim3(g2), dim3(kTBlock), 0, stream, p);
  } else {
    hipLaunchKernelGGL(k_tree_rows<float>, dim3(g1), dim3(kTBlock), 0, stream, p);
    hipLaunchKernelGGL(k_tree_draw<float>, dim3(g2), dim3(kTBlock), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace sv
