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
// One launch on the caller's stream; its workgroups, in dispatch order:
//  - row items: 256-thread workgroups over the node rows (sequence b, node u). A workgroup streams its row (or its
//    piece of a row) once with 16-byte non-temporal loads and keeps the running max and the float32 running sum of
//    2^((z - max) * log2(e)/T) WITHOUT the drafted tokens of u's children (each thread lists the few child tokens
//    that fall in its share and masks them as it streams). Every denominator of the walk is then a sum of positive
//    terms (the rest of the row, plus the children not rejected yet), so a child holding most of the mass cannot
//    leave a remainder that cancels. Rows are taken whole in full resident rounds; the rows of a last, partial round
//    are cut into equal pieces queued after them, which fill the slots the whole rows free (a piece pays a memory
//    round trip before it streams and two after, so smaller items everywhere cost more than they balance). The last
//    piece of a row (a counter) merges the pieces' records; the last row of a sequence to finish (a counter) walks
//    the tree in float64 and publishes where it stopped.
//  - draw tasks: per sequence, tasks of at least 4 chunks of 512 elements of the stop row. A task waits until its
//    sequence's walk has published the stop node (every row item is dispatched before any draw task, so the wait
//    ends), then computes float64 weights (table-driven 2^y) with the rejected children's tokens removed, one sum per
//    chunk; the last task of the sequence finds the chunk holding t, recomputes it and searches it. The draws are
//    float64-arithmetic bound; in the same launch they run while the row items' last pieces still stream.
// Bound: HBM, B * N * V * s bytes of the row items (every node row once); the draw re-reads one row per sequence.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
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
constexpr int64_t kTTailChunks = 8;    // chunks per draw task of the sequences that walk last
constexpr int64_t kTTailPerSlot = 3;   // their chunks in all, per resident workgroup
constexpr int kTPer = kTChunk / 64;
constexpr int kTMaxSeg = 64;           // pieces of one row at most (one lane each in the merge)
constexpr int64_t kTMinSegVec = 512;   // 16-byte vectors of one piece at least (2 per thread)
constexpr int64_t kTPieceCap = 8192;   // piece records the workspace holds

struct TreeParams {
  const void* tgt; int64_t t_seq, t_row;
  int64_t B; int32_t N; int64_t V;
  float c;                             // log2(e) / T rounded to float: the row sums and the walk's weights
  double c2;                           // log2(e) / T in float64: the draw's weights
  const int32_t* parent; const int32_t* token; const float* ua; const float* us;
  uint8_t* accept; int32_t* n_acc; int32_t* path; int32_t* out_token; float* p_test; uint32_t* flags;
  char* ws; uint64_t sig; int64_t ctl_end;
  int32_t* ctr1;                       // per sequence: rows finished, then N + 1 once its walk published the job
  int32_t* ctr2;                       // per sequence: draw tasks finished
  int32_t* rctr;                       // per cut row: pieces finished
  int64_t head_rows;                   // rows taken whole (rows b * N + u below it)
  int32_t nseg;                        // pieces of every later row (1: those rows are whole too)
  TreeRow* rows;                       // per (b, node): the row's statistics outside its children's tokens
  TreeRow* piece;                      // per (cut row, piece): the same over the piece
  TreeJob* jobs;                       // per b: where the walk stopped
  double* chunk;                       // per (b, chunk): float64 weight of the chunk of the stop row
  int64_t nch;                         // chunks per row
  int32_t ntask;                       // draw tasks per sequence (all but the last tailq)
  int32_t task_chunks;                 // chunks per draw task
  int32_t tailq, ntask2, task_chunks2; // the last sequences' smaller tasks
  int64_t row_items;                   // workgroups of the row pass (the draw tasks follow them)
};

struct TreeShared {
  int32_t par[SV_MAX_TREE_NODES];
  int32_t tok[SV_MAX_TREE_NODES];
  union {
    struct {                           // the row pass
      int32_t xs[SV_MAX_TREE_NODES];   // masked tokens: the child tokens of the row's node
      int32_t hits[kTBlock][kHits];    // per thread: the masked elements it streams, (group << 8) | slot
    } rp;
    struct {                           // a draw task
      int32_t xs[SV_MAX_TREE_NODES];   // the stop node's child tokens: removed from the draw
      double tab[256];                 // the float64 exp table
    } dr;
    struct {                           // the walk of a tree of at most 64 nodes, per node:
      uint64_t kids[64];               // its children (bit c for child c)
      float z[64];                     // its logit in its parent's row
      float M[64];                     // its row's max, its children's logits included
      double rest[64];                 // the weight of its row outside its children's tokens, relative to M
      double ex[64];                   // its weight in its parent's row (0 unless the first holder of its token)
    } sw;
    struct {                           // the walk, after the row pass of the same workgroup
      float rm[SV_MAX_TREE_NODES];     // per node: max of its row outside its children's tokens (NaN: bad row)
      double rs[SV_MAX_TREE_NODES];    // per node: the sum relative to it
      float zk[SV_MAX_TREE_NODES];     // per node >= 1: its logit in its parent's row
      float ua[SV_MAX_TREE_NODES];     // per node: its acceptance uniform
      int16_t kid[SV_MAX_TREE_NODES];  // the children of the current node in node order
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

// The statistics of piece `seg` of `nseg` of row (b, u) outside the tokens of u's children, into *out: by every
// thread. The row is laid out as head elements up to 16-byte alignment, 16-byte vectors and tail elements; piece s
// takes vectors [nvec * s / nseg, nvec * (s + 1) / nseg), the first piece the head elements and the last the tail
// elements. The loads of the piece's first group are issued before the tree is read, so that the two wait together.
template <typename T>
__device__ void tree_row_pass(const TreeParams& p, int64_t b, int u, int seg, int nseg, TreeRow* out) {
  TreeShared& sh = g_tree;
  constexpr int EPV = Vec<T>::kEPV;
  const int tid = threadIdx.x;
  const int N = p.N;
  const int64_t V = p.V;
  const T* row = static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(u) * p.t_row;

  const uintptr_t addr = reinterpret_cast<uintptr_t>(row);
  int64_t head = int64_t(((16u - (addr & 15u)) & 15u) / sizeof(T));
  if (head > V) head = V;
  const int64_t nvec = (V - head) / EPV;
  const int64_t tail0 = head + nvec * EPV;
  const int64_t v0 = nvec * seg / nseg, v1 = nvec * (seg + 1) / nseg;
  const int64_t nv = v1 - v0;
  const int64_t x0 = head + v0 * EPV, x1 = head + v1 * EPV;       // the piece's vector elements
  const bool first = seg == 0, last = seg == nseg - 1;
  const int64_t ngroups = (nv + int64_t(kTU) * kTBlock - 1) / (int64_t(kTU) * kTBlock);
  const uint4* vp = reinterpret_cast<const uint4*>(row + head) + v0;
  uint4 wa[kTU], wb[kTU];
  if (ngroups > 0) t_load_group<T>(wa, vp, 0, nv);

  // the children of u: the tokens to mask
  if (tid == 0) { sh.nx = 0; sh.overflow = 0; }
  for (int i = tid; i < N; i += kTBlock) {
    sh.par[i] = p.parent[b * N + i];
    sh.tok[i] = p.token[b * N + i];
  }
  __syncthreads();
  for (int ci = 1 + tid; ci < N; ci += kTBlock) {
    if (sh.par[ci] != u) continue;
    const int x = sh.tok[ci];
    if (x >= 0 && int64_t(x) < V) sh.u.rp.xs[atomicAdd(&sh.nx, 1)] = x;
  }
  __syncthreads();
  const int nx = sh.nx;

  // the masked elements this thread streams
  int nh = 0;
  for (int j = 0; j < nx; ++j) {
    const int64_t x = sh.u.rp.xs[j];
    if (x < x0 || x >= x1) continue;
    const int64_t vx = (x - head) / EPV - v0;
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
    if (first)
      for (int64_t i = tid; i < head; i += kTBlock) {
        float z = Vec<T>::load1(row + i);
        if (in_list(sh.u.rp.xs, nx, i)) z = -INFINITY;
        t_absorb<1>(st, &z, c);
      }
    if (ngroups > 0) {
      // two register sets in turn: while one group is folded the next one's loads are in flight
      int64_t g = 0;
      for (; g + 1 < ngroups; g += 2) {
        t_load_group<T>(wb, vp, g + 1, nv);
        t_fold_group<T>(st, wa, g, nv, nh, sh.u.rp.hits[tid], c);
        if (g + 2 < ngroups) t_load_group<T>(wa, vp, g + 2, nv);
        t_fold_group<T>(st, wb, g + 1, nv, nh, sh.u.rp.hits[tid], c);
      }
      if (g < ngroups) t_fold_group<T>(st, wa, g, nv, nh, sh.u.rp.hits[tid], c);
    }
    if (last)
      for (int64_t i = tail0 + tid; i < V; i += kTBlock) {
        float z = Vec<T>::load1(row + i);
        if (in_list(sh.u.rp.xs, nx, i)) z = -INFINITY;
        t_absorb<1>(st, &z, c);
      }
  } else {                                           // many child tokens in one thread's share: element by element
    const int64_t e0 = first ? 0 : x0, e1 = last ? V : x1;
    for (int64_t i = e0 + tid; i < e1; i += kTBlock) {
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
    st_dev(&out->m, M);
    st_dev(&out->bad, uint32_t(isnan(s) || M == INFINITY));
    st_dev(&out->s, s);
  }
}

// The record of cut row r from its nseg piece records, by wave 0 of the workgroup of its last piece: the common max,
// the bad flags OR-ed, and each piece's sum rescaled to the common max in float64, summed in lane (piece) order.
__device__ void tree_merge_pieces(const TreeParams& p, int64_t r) {
  const int lane = threadIdx.x & 63;
  const int nseg = p.nseg;
  const TreeRow* pr = p.piece + (r - p.head_rows) * nseg;
  float m = -INFINITY;
  double s = 0.0;
  uint32_t bad = 0;
  if (lane < nseg) {
    m = ld_dev(&pr[lane].m);
    s = ld_dev(&pr[lane].s);
    bad = ld_dev(&pr[lane].bad);
  }
  const float M = wave_max_f(m);
  const int anybad = __any(bad != 0u);
  double w = 0.0;
  if (m != -INFINITY && M != -INFINITY) w = s * exp2((double(m) - double(M)) * double(p.c));
  w = wave_sum(w);
  if (lane == 0) {
    TreeRow* o = p.rows + r;
    st_dev(&o->m, M);
    st_dev(&o->bad, uint32_t(anybad || M == INFINITY));
    st_dev(&o->s, w);
  }
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The walk of sequence b by wave 0 of the workgroup of its last row (sh.par / sh.tok hold its tree), with no barrier:
// every row record, child logit (read from the target row of its parent) and acceptance uniform the walk may use
// comes into LDS in one round of loads; at each node the children
// are listed in node order (ballots), the tests are evaluated for all of them at once (p'(x) over the mass outside
// the earlier siblings' tokens: the rest of the row plus a suffix sum of the later siblings' weights, positive terms
// only), and the first passing child is found with a ballot. Writes the outputs of every node and the draw job.
template <typename T>
__device__ void tree_walk(const TreeParams& p, int64_t b) {
  TreeShared& sh = g_tree;
  __builtin_amdgcn_s_setprio(3);                     // the walk is on the call's critical path
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
    const int pa = sh.par[i], x = sh.tok[i];
    const bool zok = i > 0 && pa >= 0 && pa < N && x >= 0 && int64_t(x) < V;
    // every lane loads (element 0 of the sequence's first row where the node names no element), so that all the
    // walk's loads are in flight together
    const float zr = Vec<T>::load1(static_cast<const T*>(p.tgt) + b * p.t_seq + (zok ? int64_t(pa) * p.t_row + x : 0));
    const float ua = p.ua[b * N + i];
    const float z = i == 0 ? 0.f : (zok ? zr : NAN);
    sh.u.wk.rm[i] = rb ? NAN : m;
    sh.u.wk.rs[i] = s;
    sh.u.wk.zk[i] = z;
    sh.u.wk.ua[i] = ua;
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
      if (hit) sh.u.wk.kid[nk + lane_rank(m)] = int16_t(ci);
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
      const int tk = valid ? sh.tok[ci] : -1;
      // first holder of its token: no earlier sibling holds it (the earlier siblings' tokens come 64 at a time into
      // registers and are read back lane by lane)
      bool first = valid;
      for (int d0 = 0; d0 <= c0; d0 += 64) {
        const int dt = d0 == c0 ? tk : sh.tok[sh.u.wk.kid[d0 + lane]];
        const int lim = nk - d0 < 64 ? nk - d0 : 64;
        for (int q = 0; q < lim; ++q) first = first && !(d0 + q < j && __builtin_amdgcn_readlane(dt, q) == tk);
      }
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
      const float u = valid ? sh.u.wk.ua[ci] : 1.f;
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
    TreeJob* jb = p.jobs + b;
    st_dev(&jb->stop, int32_t(stop));
    st_dev(&jb->m, fatal ? 0.f : mstop);
    st_dev(&jb->u, fatal ? 0.f : p.us[b * N + stop]);
    st_dev(&jb->flags, fl);
    st_dev(&jb->n, fatal ? -1 : n);                  // n, the token and the flags are output by the draw's pick
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

// The walk of a tree of at most 64 nodes, lane i for node i, by wave 0 of the workgroup of the sequence's last row;
// same rule and outputs as tree_walk. A child's p'(x) depends only on its parent's row and siblings, not on the path to
// the parent, so every node's test is evaluated at once: as a parent, the lane forms its row's max M (the rest of the
// row and its children's logits) and the rest's weight; as a child, its own weight and denominator (the parent's rest
// plus the weights of the first holders of the tokens of it and of its later siblings, summed from the last sibling
// down) and its test; as a parent again, its first passing child. The walk is then a chain of lane reads. Each lane
// loops over its own children or siblings only (bit masks built in LDS), never over the whole tree.
template <typename T>
__device__ void tree_walk_small(const TreeParams& p, int64_t b) {
  TreeShared& sh = g_tree;
  __builtin_amdgcn_s_setprio(3);                     // the walk is on the call's critical path
  const int lane = threadIdx.x & 63;
  const int N = p.N;
  const int64_t V = p.V;
  const double c = double(p.c);
  const bool in = lane < N;
  const int i = in ? lane : 0;
  // one round of loads: the node's row record, its logit in its parent's row, its uniform
  const TreeRow* r = p.rows + b * N + i;
  const float m = ld_dev(&r->m);
  const double s = ld_dev(&r->s);
  const uint32_t rb = ld_dev(&r->bad);
  const int pa = in ? sh.par[i] : -1, tk = in ? sh.tok[i] : -1;
  const bool child = in && lane > 0;
  const bool zok = child && pa >= 0 && pa < N && tk >= 0 && int64_t(tk) < V;
  const float zr = Vec<T>::load1(static_cast<const T*>(p.tgt) + b * p.t_seq + (zok ? int64_t(pa) * p.t_row + tk : 0));
  const float ua = p.ua[b * N + i];
  const int bad = __any(child && (!(pa >= 0 && pa < lane) || !(tk >= 0 && int64_t(tk) < V)));
  const bool linked = child && pa >= 0 && pa < lane;  // a parent index that can be used (always, unless bad)
  const int src = linked ? pa : 0;
  sh.u.sw.kids[lane] = 0;
  wave_sync();
  if (linked) atomicOr(reinterpret_cast<unsigned long long*>(&sh.u.sw.kids[pa]), 1ull << lane);
  const float mr = in ? (rb ? NAN : m) : -INFINITY;
  const float z = zok ? zr : NAN;
  sh.u.sw.z[lane] = z;
  wave_sync();
  // as a parent: the row's max over the rest and the children's logits, a NaN or +inf among the children's logits
  const uint64_t kids = sh.u.sw.kids[lane];
  float M = mr;
  int kb = 0;
  for (uint64_t q = kids; q; q &= q - 1) {
    const float zq = sh.u.sw.z[__builtin_ctzll(q)];
    M = fmaxf(M, zq);
    kb |= !(zq < INFINITY);
  }
  const bool nodebad = mr != mr || kb || M == -INFINITY;
  const double rest = (mr == -INFINITY || nodebad) ? 0.0 : s * exp2((double(mr) - double(M)) * c);
  sh.u.sw.M[lane] = M;
  sh.u.sw.rest[lane] = rest;
  wave_sync();
  // as a child of pa: first holder of its token among its siblings, its weight, the denominator, the test
  const float Mu = sh.u.sw.M[src];
  const double restu = sh.u.sw.rest[src];
  const uint64_t sib = linked ? sh.u.sw.kids[src] : 0;
  bool first = linked;
  for (uint64_t q = sib & ((1ull << lane) - 1); q && first; q &= q - 1) first = sh.tok[__builtin_ctzll(q)] != tk;
  const double ex = first ? exp2((double(z) - double(Mu)) * c) : 0.0;
  sh.u.sw.ex[lane] = ex;
  wave_sync();
  double S = 0.0;
  for (uint64_t q = (sib >> lane) << lane; q;) {     // this child and its later siblings, from the last down
    const int k = 63 - __builtin_clzll(q);
    S += sh.u.sw.ex[k];
    q &= ~(1ull << k);
  }
  const double P = first ? ex / (restu + S) : 0.0;
  const uint64_t passm = wave_ballot(linked && double(ua) < fmin(1.0, P));
  const uint64_t badm = wave_ballot(in && nodebad);
  // as a parent: the first passing child in node order
  const uint64_t okk = kids & passm;
  const int next = okk ? __builtin_ctzll(okk) : -1;
  // the walk
  uint32_t fl = bad ? SV_FLAG_ID_RANGE : 0u;
  int cur = 0, n = 0, stop = -1, pathv = -1;
  float mstop = 0.f;
  uint64_t onpath = 0;
  while (!bad) {
    if ((badm >> cur) & 1ull) {                      // a NaN or +inf in the row, or nothing but -inf
      fl |= SV_FLAG_NONFINITE;
      stop = -1;
      break;
    }
    const int nx = __builtin_amdgcn_readlane(next, cur);
    if (nx < 0) {                                    // every child rejected (or a leaf): draw at cur
      stop = cur;
      mstop = readlane_f(M, cur);
      break;
    }
    onpath |= 1ull << nx;
    if (lane == n) pathv = nx;
    ++n;
    cur = nx;
  }
  // outputs: the children of the visited nodes are tested up to the accepted one (all of them at the stop node)
  const bool fatal = stop < 0;
  const int nextpa = __shfl(next, src);
  const bool tested = linked && (((onpath | 1ull) >> src) & 1ull) && (nextpa < 0 || lane <= nextpa);
  if (in) {
    p.accept[b * N + lane] = (!fatal && ((onpath >> lane) & 1ull)) ? 1 : 0;
    p.path[b * N + lane] = (!fatal && lane < n) ? pathv : -1;
    if (p.p_test) p.p_test[b * N + lane] = (!fatal && tested) ? float(P) : NAN;
  }
  if (lane == 0) {
    TreeJob* jb = p.jobs + b;
    st_dev(&jb->stop, int32_t(stop));
    st_dev(&jb->m, fatal ? 0.f : mstop);
    st_dev(&jb->u, fatal ? 0.f : p.us[b * N + stop]);
    st_dev(&jb->flags, fl);
    st_dev(&jb->n, fatal ? -1 : n);                  // n, the token and the flags are output by the draw's pick
  }
}

// A row item: a whole row or one piece of a row; the row's last piece merges, the sequence's last row walks.
template <typename T>
__device__ void tree_row_item(const TreeParams& p, int64_t item) {
  TreeShared& sh = g_tree;
  int64_t r;
  int32_t seg;
  tree_item(item, p.head_rows, p.nseg, &r, &seg);
  const int nseg = item < p.head_rows ? 1 : p.nseg;
  const int64_t b = r / p.N;
  const int u = int(r % p.N);
  // workgroup 0 makes sure the counters are at zero for this call's layout; the others confirm it before counting
  if (item == 0) ws_claim(p.ws, p.sig, size_t(p.ctl_end), &sh.flag);
  const bool seen = item == 0 || ws_seen_clean(p.ws, p.sig);
  tree_row_pass<T>(p, b, u, seg, nseg, nseg == 1 ? p.rows + r : p.piece + (r - p.head_rows) * nseg + seg);
  __builtin_amdgcn_s_waitcnt(0);                     // this piece's records are complete before it is counted
  __syncthreads();
  if (threadIdx.x == 0) {
    if (seen || ws_ready(p.ws, p.sig)) {
      sh.flag = nseg == 1 || ctr_add(p.rctr + (r - p.head_rows)) == nseg - 1;
    } else {                                         // never counted: the sequence is not walked in this call
      ws_mark_dirty(p.ws);
      sh.flag = 0;
    }
  }
  __syncthreads();
  if (!sh.flag) return;
  if (nseg > 1) {                                    // the row's last piece: its record from the pieces' records
    if (threadIdx.x < 64) {
      tree_merge_pieces(p, r);
      if (threadIdx.x == 0) st_sys(p.rctr + (r - p.head_rows), int32_t(0));   // ready for the next call
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (threadIdx.x == 0) sh.flag = ctr_add(p.ctr1 + b) == p.N - 1;
  __syncthreads();
  if (!sh.flag || threadIdx.x >= 64) return;       // the walk is wave 0's
  if (p.N <= 64)
    tree_walk_small<T>(p, b);
  else
    tree_walk<T>(p, b);
  if (threadIdx.x == 0) {                            // the job is complete before the draw tasks may read it
    __builtin_amdgcn_s_waitcnt(0);
    st_sys(p.ctr1 + b, p.N + 1);
  }
}

// The lane's kTPer elements of chunk c of the stop row as 16-byte vectors, when they are whole vectors (aligned row,
// not past the row's end); t_chunk_eval turns them into weights (or loads the elements one by one otherwise). Split
// so that the loads of several chunks are in flight together.
template <typename T>
struct TRaw {
  uint4 v[kTPer / Vec<T>::kEPV];
};
template <typename T>
__device__ __forceinline__ void t_chunk_load(TRaw<T>& r, const T* row, bool vec, int64_t V, int64_t c) {
  const int64_t i0 = c * kTChunk + int64_t(threadIdx.x & 63) * kTPer;
  if (vec && i0 + kTPer <= V) {
    const uint4* q = reinterpret_cast<const uint4*>(row + i0);
#pragma unroll
    for (int k = 0; k < kTPer / Vec<T>::kEPV; ++k) r.v[k] = gload4(q + k);
  }
}

// The float64 weights of the lane's kTPer elements of chunk c of the stop row (r from t_chunk_load of the same chunk),
// the stop node's child tokens (the draw's xs, nx of them) removed unless `all`; the same operations every time, so
// repeated evaluations agree bit for bit.
template <typename T>
__device__ __forceinline__ void t_chunk_eval(const TRaw<T>& r, const T* row, bool vec, int64_t V, int64_t c,
                                             double c2, double nm, int nx, bool all, double* w) {
  const int lane = threadIdx.x & 63;
  const int64_t i0 = c * kTChunk + int64_t(lane) * kTPer;
  float z[kTPer];
  if (vec && i0 + kTPer <= V) {
#pragma unroll
    for (int k = 0; k < kTPer / Vec<T>::kEPV; ++k) Vec<T>::unpack(r.v[k], z + k * Vec<T>::kEPV);
  } else {
#pragma unroll
    for (int e = 0; e < kTPer; ++e) z[e] = elem_or_ninf<T>(row, i0 + e, V);
  }
#pragma unroll
  for (int e = 0; e < kTPer; ++e) w[e] = fexp_scaled_at(g_tree.u.dr.tab, xarg(z[e], c2, nm));
  if (!all) {
    for (int j = 0; j < nx; ++j) {
      const int64_t d = int64_t(g_tree.u.dr.xs[j]) - i0;
#pragma unroll
      for (int e = 0; e < kTPer; ++e) w[e] = d == e ? 0.0 : w[e];
    }
  }
}

template <typename T>
__device__ __forceinline__ void t_chunk_weights(const T* row, bool vec, int64_t V, int64_t c, double c2, double nm,
                                                int nx, bool all, double* w) {
  TRaw<T> r;
  t_chunk_load<T>(r, row, vec, V, c);
  t_chunk_eval<T>(r, row, vec, V, c, c2, nm, nx, all, w);
}

// The pick of sequence b by wave 0 of its last draw task: the chunk whose running sum crosses t = u * total, then the
// element inside it (the chunk recomputed with the same operations). Returns the token (-1 when nothing has weight).
// Each lane first sums a contiguous block of the chunk sums (eight loads in flight at a time); a scan over the lanes
// finds the block that crosses t, and a second pass scans that block's chunks one per lane.
template <typename T>
__device__ int32_t tree_pick(const TreeParams& p, int64_t b, const TreeJob& job, const T* row, bool vec, int nx,
                             bool all) {
  const int lane = threadIdx.x & 63;
  const int64_t nch = p.nch;
  const double* cs = p.chunk + b * nch;
  const double c2 = p.c2, nm = -(double(job.m) * c2);
  const int64_t per = (nch + 63) / 64;
  const int64_t l0 = int64_t(lane) * per, l1 = l0 + per < nch ? l0 + per : nch;
  double bsum = 0.0;
  int64_t blast = -1;                                // the block's last chunk with weight
  for (int64_t k0 = l0; k0 < l1; k0 += 8) {
    double m[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) m[k] = ld_dev(cs + (k0 + k < l1 ? k0 + k : l1 - 1));
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k0 + k < l1) {
        bsum += m[k];
        if (m[k] > 0.0) blast = k0 + k;
      }
  }
  const double incl = wave_incl_scan(bsum);
  const double total = readlane_d(incl, 63);
  const double t = double(job.u) * total;
  int64_t last = blast;                              // the last chunk with weight of the whole row
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t x = __shfl_xor(last, o);
    last = x > last ? x : last;
  }
  int64_t cstar = -1;
  double cbase = 0.0;
  const uint64_t bhit = wave_ballot(bsum > 0.0 && incl > t);
  if (bhit) {
    const int L = __builtin_ctzll(bhit);
    const int64_t b0 = int64_t(L) * per, b1 = b0 + per < nch ? b0 + per : nch;
    double base = readlane_d(incl, L) - readlane_d(bsum, L);
    for (int64_t g0 = b0; g0 < b1 && cstar < 0; g0 += 64) {
      const int64_t ci = g0 + lane;
      const double mv = ld_dev(cs + (ci < b1 ? ci : b1 - 1));
      const double m = ci < b1 ? mv : 0.0;
      const double inc = wave_incl_scan(m);
      const uint64_t hm = wave_ballot(m > 0.0 && base + inc > t);
      if (hm) {
        const int l = __builtin_ctzll(hm);
        cstar = g0 + l;
        cbase = base + (readlane_d(inc, l) - readlane_d(m, l));
      }
      base += readlane_d(inc, 63);
    }
    // (no crossing inside the block: t lies within rounding of the block's end; the row's last weighted chunk of
    // that block is taken as at the end of the row)
    if (cstar < 0) last = __shfl(blast, L);
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

// A draw task: chunks [task * task_chunks, ...) of the stop row of sequence b, after the sequence's walk has published
// where it stopped (the tree and the exp table are set up while it may still run); the last task of the sequence
// picks the token and returns the sequence's counters to zero.
template <typename T>
__device__ void tree_draw_item(const TreeParams& p, int64_t j) {
  TreeShared& sh = g_tree;
  const int tid = threadIdx.x, wave = tid >> 6;
  const TreeTask tk = tree_task(j, p.B, p.tailq, p.ntask, p.ntask2, p.task_chunks, p.task_chunks2, p.nch);
  const int64_t b = tk.b;
  const int N = p.N;
  const bool seen = ws_seen_clean(p.ws, p.sig);
  for (int i = tid; i < N; i += kTBlock) {
    sh.par[i] = p.parent[b * N + i];
    sh.tok[i] = p.token[b * N + i];
  }
  fexp_fill_table_at(sh.u.dr.tab);
  if (tid == 0) {
    sh.nx = 0;
    // every row item is dispatched before any draw task, so this wait ends (the cap only guards a broken order)
    int ok = seen || ws_ready(p.ws, p.sig);
    for (int32_t polls = 0; ok && ld_sys(p.ctr1 + b) != N + 1; ++polls) {
      if (polls >= kWsSpinCap) ok = 0;
      __builtin_amdgcn_s_sleep(8);
    }
    if (!ok) {                                       // not drawn: the sequence is reported, the next call clears
      ws_mark_dirty(p.ws);
      p.n_acc[b] = -1;
      p.out_token[b] = -1;
      if (p.flags) p.flags[b] = SV_FLAG_INTERNAL;
    }
    sh.flag = ok;
  }
  __syncthreads();
  if (!sh.flag) return;
  TreeJob job;
  job.stop = ld_dev(&p.jobs[b].stop);
  job.m = ld_dev(&p.jobs[b].m);
  job.u = ld_dev(&p.jobs[b].u);
  job.flags = ld_dev(&p.jobs[b].flags);
  job.n = ld_dev(&p.jobs[b].n);
  const bool live = job.stop >= 0 && job.stop < N;
  if (live) {
    for (int ci = 1 + tid; ci < N; ci += kTBlock)
      if (sh.par[ci] == job.stop) {
        const int x = sh.tok[ci];
        if (x >= 0 && int64_t(x) < p.V) sh.u.dr.xs[atomicAdd(&sh.nx, 1)] = x;
      }
  }
  __syncthreads();
  const int nx = sh.nx;
  const T* row = live ? static_cast<const T*>(p.tgt) + b * p.t_seq + int64_t(job.stop) * p.t_row : nullptr;
  const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0;
  const double c2 = p.c2, nm = -(double(job.m) * c2);
  if (live) {
    const int64_t c0 = tk.c0, c1 = tk.c1;
    // the wave's chunks c0 + wave + 4k, kTBatch of them in flight at a time
    constexpr int kTBatch = 4;
    for (int64_t cb = c0 + wave; cb < c1; cb += int64_t(kTBatch) * kTWaves) {
      TRaw<T> raw[kTBatch];
#pragma unroll
      for (int k = 0; k < kTBatch; ++k) {
        const int64_t ci = cb + int64_t(k) * kTWaves;
        if (ci < c1) t_chunk_load<T>(raw[k], row, vec, p.V, ci);
      }
#pragma unroll
      for (int k = 0; k < kTBatch; ++k) {
        const int64_t ci = cb + int64_t(k) * kTWaves;
        if (ci >= c1) break;
        double w[kTPer];
        t_chunk_eval<T>(raw[k], row, vec, p.V, ci, c2, nm, nx, false, w);
        double s = 0.0;
#pragma unroll
        for (int e = 0; e < kTPer; ++e) s += w[e];
        s = wave_sum(s);
        st_dev(p.chunk + b * p.nch + ci, s);         // every lane stores the same value
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) sh.flag = ctr_add(p.ctr2 + b) == tk.nt - 1;
  __syncthreads();
  if (!sh.flag) return;
  // the last task of the sequence: the pick (wave 0), and the sequence's outputs that the walk left to it (one writer
  // for each output word: workgroups on different XCDs do not share a cache)
  if (wave == 0) {
    __builtin_amdgcn_s_setprio(3);                   // on the call's critical path
    uint32_t extra = 0;
    int32_t tok = live ? tree_pick<T>(p, b, job, row, vec, nx, false) : -1;
    if (live && tok < 0) {                           // the removed tokens held every weight: draw from p itself
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
      p.n_acc[b] = job.n;
      p.out_token[b] = tok;
      if (p.flags) p.flags[b] = job.flags | extra;
    }
  }
  if (tid == 0) {                                    // ready for the next call
    st_sys(p.ctr1 + b, int32_t(0));
    st_sys(p.ctr2 + b, int32_t(0));
  }
}

// One launch: the row items (whole rows, then the pieces of the cut rows), then the draw tasks of every sequence.
template <typename T>
__global__ __launch_bounds__(kTBlock) void k_tree(TreeParams p) {
  const int64_t item = blockIdx.x;
  if (item < p.row_items) tree_row_item<T>(p, item);
  else tree_draw_item<T>(p, item - p.row_items);
}

}  // namespace

TreePlan make_tree_plan(int64_t B, int32_t N, int64_t V, int dtype, int64_t resident) {
  TreePlan pl;
  pl.B = B; pl.N = N; pl.V = V;
  // the row items: whole rows in full resident rounds, the rows of a last, partial round cut into pieces (as many
  // as fill the round, each at least kTMinSegVec vectors); the workspace holds the most pieces any residency gives
  const int64_t R = B * int64_t(N);
  const int64_t W = std::max<int64_t>(resident, 1);
  const int64_t tail = R % W;
  const int64_t epv = dtype == SV_BF16 ? 8 : 4;
  const int64_t segcap = std::max<int64_t>(1, (V / epv - 1) / kTMinSegVec);
  int64_t nseg = tail > 0 ? W / tail : 1;
  nseg = std::max<int64_t>(1, std::min<int64_t>({nseg, int64_t(kTMaxSeg), segcap, tail > 0 ? kTPieceCap / tail : 1}));
  pl.nseg = int32_t(nseg);
  pl.head_rows = nseg > 1 ? R - tail : R;
  pl.items = pl.head_rows + (nseg > 1 ? tail * nseg : 0);
  pl.nch = (V + kTChunk - 1) / kTChunk;
  // draw tasks: the sequences' tasks together about fill one resident round (1024 workgroups), each task at least
  // 4 chunks (one per wave)
  const int64_t want = std::max<int64_t>(1, 1024 / std::max<int64_t>(B, 1));
  int64_t tc = std::max<int64_t>(4, (pl.nch + want - 1) / want);
  pl.task_chunks = int32_t(std::min<int64_t>(tc, std::max<int64_t>(pl.nch, 1)));
  pl.ntask = int32_t((pl.nch + pl.task_chunks - 1) / pl.task_chunks);
  // the sequences whose rows finish last (the walks come last) take tasks of kTTailChunks chunks: about
  // kTTailPerSlot chunks per resident workgroup in all, so the end of the launch is many short tasks
  pl.task_chunks2 = int32_t(std::min<int64_t>(kTTailChunks, std::max<int64_t>(pl.nch, 1)));
  pl.ntask2 = int32_t((pl.nch + pl.task_chunks2 - 1) / pl.task_chunks2);
  pl.tailq = pl.ntask2 > pl.ntask
      ? int32_t(std::min<int64_t>(B, (kTTailPerSlot * W + pl.nch - 1) / std::max<int64_t>(pl.nch, 1)))
      : 0;
  pl.tasks = (B - pl.tailq) * int64_t(pl.ntask) + int64_t(pl.tailq) * pl.ntask2;
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t ncut = size_t(std::min<int64_t>(R, kTPieceCap / 2));      // cut rows at most (2 pieces or more each)
  const size_t npiece = size_t(std::min<int64_t>(R * kTMaxSeg, kTPieceCap));
  size_t off = kWsHeaderBytes;
  pl.off_ctr1 = off; off = up(off + size_t(B) * 4);
  pl.off_ctr2 = off; off = up(off + size_t(B) * 4);
  pl.off_rctr = off; off = up(off + ncut * 4);
  pl.ctl_end = off;
  pl.off_rows = off; off = up(off + size_t(R) * sizeof(TreeRow));
  pl.off_piece = off; off = up(off + npiece * sizeof(TreeRow));
  pl.off_jobs = off; off = up(off + size_t(B) * sizeof(TreeJob));
  pl.off_chunk = off; off = up(off + size_t(B) * size_t(pl.nch) * sizeof(double));
  pl.total = off;
  return pl;
}

int tree_resident_workgroups(int dtype) {
  static std::atomic<int> cache[2][64];             // per dtype and device (0: not asked yet)
  int dev = 0, ncu = 0, per = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  const int di = dtype == SV_BF16 ? 1 : 0;
  if (dev >= 0 && dev < 64) {
    const int w = cache[di][dev].load(std::memory_order_relaxed);
    if (w > 0) return w;
  }
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
  const hipError_t e = dtype == SV_BF16
      ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_tree<uint16_t>, kTBlock, 0)
      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_tree<float>, kTBlock, 0);
  if (e != hipSuccess || per <= 0) per = 4;
  const int w = ncu * per;
  if (dev >= 0 && dev < 64) cache[di][dev].store(w, std::memory_order_relaxed);
  return w;
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
  p.sig = ws_signature(kLayoutTree, layout_mix(uint64_t(plan.B), uint64_t(plan.ctl_end)));
  p.ctl_end = int64_t(plan.ctl_end);
  p.ctr1 = reinterpret_cast<int32_t*>(a.ws + plan.off_ctr1);
  p.ctr2 = reinterpret_cast<int32_t*>(a.ws + plan.off_ctr2);
  p.rctr = reinterpret_cast<int32_t*>(a.ws + plan.off_rctr);
  p.head_rows = plan.head_rows; p.nseg = plan.nseg;
  p.rows = reinterpret_cast<TreeRow*>(a.ws + plan.off_rows);
  p.piece = reinterpret_cast<TreeRow*>(a.ws + plan.off_piece);
  p.jobs = reinterpret_cast<TreeJob*>(a.ws + plan.off_jobs);
  p.chunk = reinterpret_cast<double*>(a.ws + plan.off_chunk);
  p.nch = plan.nch; p.ntask = plan.ntask; p.task_chunks = plan.task_chunks;
  p.tailq = plan.tailq; p.ntask2 = plan.ntask2; p.task_chunks2 = plan.task_chunks2;
  p.row_items = plan.items;
  const unsigned grid = unsigned(plan.items + plan.tasks);
  if (a.dtype == SV_BF16)
    hipLaunchKernelGGL(k_tree<uint16_t>, dim3(grid), dim3(kTBlock), 0, stream, p);
  else
    hipLaunchKernelGGL(k_tree<float>, dim3(grid), dim3(kTBlock), 0, stream, p);
  return hipGetLastError();
}

}  // namespace sv
