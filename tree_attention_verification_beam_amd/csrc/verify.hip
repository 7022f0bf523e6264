// verify.hip -- acceptance, selection and residual resampling over the packed tree.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 5: token matches (greedy)
// or rejection sampling per token; the longest accepted prefix over all
// candidates wins.  ResiSpec (paperpeel 2608.24411), section 4: candidates of
// one position are checked in order, and after each rejection the target
// becomes the residual max(0, p - q) / sum max(0, p - q).
//
// Kernels, in stream order:
//   k_vstats  the vocabulary stream: every needed logits row is read once, in
//             chunks; each chunk yields (max, argmax with the lowest index on
//             ties, sum exp(l - max)).  Coalesced 16-byte loads; exp in fp32,
//             sums in fp64.  A draft row is read only when it is the draft row
//             of a node with a child.
//   k_vselect P workgroups per sequence (P = 1 for greedy): validate the tree,
//             merge the chunk partials of the needed rows into row statistics
//             (all threads, staged in LDS), gather p and q of every node's
//             own token (fp64 exp), run the mode's tests and the path select,
//             and do the residual passes and the inverse-CDF draw over the stop
//             row pair in fp64.  With P > 1 the workgroups of a sequence split
//             the vocabulary and exchange per-pass partial sums through
//             tagged slots (cleared by k_vstats): every 64-bit slot word holds
//             one 32-bit half of a value beside the exchange's round number,
//             so a reader needs no separate arrival count.  Every workgroup
//             then holds the same totals and takes the same decisions.  The
//             grid is sized to be resident at once (occupancy query) and every
//             wait is bounded.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "common.hpp"

namespace spec {

// greedy walk (verify_walk.hip)
int launch_verify_walk(int B, int T_cap, int V, const float* tgt, const int32_t* n_nodes,
                       const int32_t* parent, const int32_t* token, const int32_t* depth,
                       int32_t* acc_len, int32_t* acc_path, int32_t* next_token, float* p_tok,
                       float* q_tok, int8_t* decision, int32_t* near_tie, void* ws,
                       size_t ws_bytes, int32_t* status, hipStream_t s);
size_t verify_walk_workspace_size(int B);

namespace {

constexpr int kStatThreads = 256;
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxP = 32;
constexpr int kMergeEntries = 1024;  // chunk partials staged in LDS per merge batch
constexpr int kSyncWords = 2 * kMaxP * 4;  // [2 parities][kMaxP][4 tagged halves]
constexpr size_t kSyncStride = kSyncWords * 8;  // bytes of sync area per sequence
// rejection-mode walks: rows scanned per exchange (target and draft rows of up
// to kScanRows / 2 frontier nodes), 4 tagged 32-bit words per row
constexpr int kScanRows = 8;
constexpr int kXWords = 4 * kScanRows;
// Per sequence the walks keep [2 parities][Pb][4] words for exchange() and
// [2 parities][Pb][kXWords] for exchange_words(), Pb = the most workgroups a
// sequence can get at this vocabulary size
__host__ __device__ inline int walk_p_bound(int V) { return V / 2048 < 1 ? 1 : (V / 2048 > kMaxP ? kMaxP : V / 2048); }
__host__ __device__ inline size_t walk_stride(int V) { return (size_t)walk_p_bound(V) * (2 * 4 + 2 * kXWords) * 8; }
constexpr double kNearTie = 1e-5;
constexpr double kCdfNearTie = 1e-9;
constexpr float kLog2e = 1.4426950408889634f;

struct Partial {
  double S;  // sum of exp(l - m) over the chunk
  float m;   // chunk maximum
  int arg;   // lowest index attaining m
};

struct VerifyPlan {
  int ept;       // floats per thread in k_vstats
  int chunk;     // floats per chunk
  int n_chunks;  // chunks per row
  long n_units;  // rows: B*T_cap target rows, then B*R draft rows
  size_t off_part, off_sync, total;
};

VerifyPlan make_plan(int mode, int B, int T_cap, int V, int R) {
  VerifyPlan p{};
  const int Rr = mode == SPEC_GREEDY ? 0 : R;
  p.n_units = (long)B * T_cap + (long)B * Rr;
  p.ept = 64;
  // about one workgroup per CU at least; larger chunks keep the row merges short
  while (p.ept > 4 && p.n_units * ((V + p.ept * kStatThreads - 1) / (p.ept * kStatThreads)) < 256)
    p.ept >>= 1;
  p.chunk = p.ept * kStatThreads;
  p.n_chunks = (V + p.chunk - 1) / p.chunk;
  while (p.n_chunks > kMergeEntries && p.ept < 64) {  // very large vocabularies
    p.ept <<= 1;
    p.chunk = p.ept * kStatThreads;
    p.n_chunks = (V + p.chunk - 1) / p.chunk;
  }
  size_t off = 0;
  p.off_part = off;
  off += round_up((size_t)p.n_units * p.n_chunks * sizeof(Partial), 256);
  p.off_sync = off;
  off += (size_t)B * kSyncStride;
  p.total = off;
  return p;
}

// ------------------------------------------------------------------ block reductions

__device__ __forceinline__ double block_sum_f64(double v, double* s_red) {
  v = wave_sum_f64(v);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) s_red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < kSelWaves; ++w) t += s_red[w];
  return t;
}

// two sums at once
__device__ __forceinline__ void block_sum2_f64(double& a, double& b, double* s_red) {
  a = wave_sum_f64(a);
  b = wave_sum_f64(b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) {
    s_red[wave] = a;
    s_red[kSelWaves + wave] = b;
  }
  __syncthreads();
  double ta = 0.0, tb = 0.0;
  for (int w = 0; w < kSelWaves; ++w) {
    ta += s_red[w];
    tb += s_red[kSelWaves + w];
  }
  a = ta;
  b = tb;
}

// exclusive scan over the block's threads (in thread order), fp64; returns the
// total and leaves every thread's inclusive value in s_buf[tid].  Each wave
// scans its lanes with shuffles (Hillis-Steele over 64 lanes), then adds the
// totals of the waves before it.
__device__ __forceinline__ double block_exclusive_scan_f64(double v, double* s_buf, double& excl) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  double inc = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double add = __shfl_up(inc, off, 64);
    if (lane >= off) inc += add;
  }
  __shared__ double s_wave[kSelWaves];
  __syncthreads();
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  double before = 0.0, total = 0.0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    if (w < wave) before += s_wave[w];
    total += s_wave[w];
  }
  inc += before;
  s_buf[tid] = inc;
  excl = inc - v;
  __syncthreads();
  return total;
}

// ------------------------------------------------------------------ k_vstats

template <int EPT, bool VEC>
__global__ __launch_bounds__(kStatThreads) void k_vstats(
    int B, int T_cap, int V, int Rr, int n_chunks, const float* __restrict__ tgt,
    const float* __restrict__ dft, const int32_t* __restrict__ n_nodes,
    const int32_t* __restrict__ parent, const int32_t* __restrict__ dft_row,
    Partial* __restrict__ part, unsigned char* __restrict__ sync) {
  __shared__ int s_need;
  __shared__ float s_m[kStatThreads / 64];
  __shared__ int s_a[kStatThreads / 64];
  __shared__ double s_s[kStatThreads / 64];
  const long unit = blockIdx.x / n_chunks;
  const int c = blockIdx.x - (int)(unit * n_chunks);
  const float* row;
  const long n_tgt = (long)B * T_cap;
  const int tid = threadIdx.x;
  if (unit < n_tgt) {
    const int b = (int)(unit / T_cap), t = (int)(unit - (long)b * T_cap);
    if (t > 0 && t >= n_nodes[b]) return;
    // the sequence's root row, first chunk: clear the select's exchange slots
    // (round tags start again at one)
    if (t == 0 && c == 0)
      for (int i = tid; i < kSyncWords; i += kStatThreads)
        store_coherent(reinterpret_cast<uint64_t*>(sync + (size_t)b * kSyncStride) + i, 0);
    row = tgt + unit * (long)V;
  } else {
    // a draft row is needed iff it is the draft row of some node with a child;
    // the node count, parents and draft rows are read in one round trip and
    // the parents' rows looked up in LDS
    const long u2 = unit - n_tgt;
    const int b = (int)(u2 / Rr), r = (int)(u2 - (long)b * Rr);
    __shared__ int s_row[SPEC_MAX_TREE];
    static_assert(kStatThreads >= SPEC_MAX_TREE, "one tree row per thread");
    const int T_n = n_nodes[b];
    int my_par = -1, my_row = -1;
    if (tid < T_cap) {
      my_par = parent[(size_t)b * T_cap + tid];
      my_row = dft_row[(size_t)b * T_cap + tid];
    }
    if (tid == 0) s_need = 0;
    if (tid < T_cap) s_row[tid] = my_row;
    __syncthreads();
    const int T = min(T_n, T_cap);
    if (tid >= 1 && tid < T && my_par >= 0 && my_par < tid && s_row[my_par] == r) s_need = 1;
    __syncthreads();
    if (!s_need) return;
    row = dft + u2 * (long)V;
  }
  const int base = c * EPT * kStatThreads;
  float x[EPT];
  int idx0[EPT / 4];
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      const int e = base + 4 * (tid + kStatThreads * j);
      idx0[j] = e;
      f32x4 v4 = e < V ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + e))
                       : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      x[4 * j] = v4[0];
      x[4 * j + 1] = v4[1];
      x[4 * j + 2] = v4[2];
      x[4 * j + 3] = v4[3];
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      const int e = base + 4 * (tid + kStatThreads * j);
      idx0[j] = e;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[4 * j + i] = e + i < V ? row[e + i] : -INFINITY;
    }
  }
  // Row maximum, then (in one more pass over the registers) the sum of
  // exp(l - m) and the lowest index holding the maximum.  Padding past V is
  // -inf: it never raises the maximum and, having the highest indices, never
  // wins a tie, so only the sum needs the range test, and only in the last
  // chunk of a row.
  float tm = x[0];  // this thread's maximum
#pragma unroll
  for (int e = 1; e < EPT; ++e) tm = fmaxf(tm, x[e]);
  float m = wave_max_f32(tm);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) s_m[wave] = m;
  __syncthreads();
  m = s_m[0];
  for (int w = 1; w < kStatThreads / 64; ++w) m = fmaxf(m, s_m[w]);
  // sum of exp(l - m): exp in fp32 (v_exp_f32 on the log2 argument), sums in
  // fp64; both passes run in increasing index order
  float loc = 0.0f;
  const float mb = m * kLog2e;
  const bool full = base + EPT * kStatThreads <= V;  // uniform
  if (full) {
#pragma unroll
    for (int e = 0; e < EPT; ++e) loc += __builtin_amdgcn_exp2f(__builtin_fmaf(x[e], kLog2e, -mb));
  } else {
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (idx0[j] + i < V) loc += __builtin_amdgcn_exp2f(__builtin_fmaf(x[4 * j + i], kLog2e, -mb));
  }
  // the lowest index holding the maximum: only lanes whose own maximum is it
  // search (usually one lane of one wave)
  int a = 0x7fffffff;
  if (tm == m) {
#pragma unroll
    for (int j = EPT / 4 - 1; j >= 0; --j)
#pragma unroll
      for (int i = 3; i >= 0; --i) a = x[4 * j + i] == m ? idx0[j] + i : a;
  }
  a = wave_min_i32(a);
  double s = wave_sum_f64((double)loc);
  if (lane == 0) {
    s_s[wave] = s;
    s_a[wave] = a;
  }
  __syncthreads();
  a = s_a[0];
  for (int w = 1; w < kStatThreads / 64; ++w) a = min(a, s_a[w]);
  if (a == 0x7fffffff) a = base;  // no element equals the maximum (NaN logits): stay in range
  if (tid == 0) {
    double tot = 0.0;
    for (int w = 0; w < kStatThreads / 64; ++w) tot += s_s[w];
    Partial p;
    p.S = tot;
    p.m = m;
    p.arg = a;
    part[unit * n_chunks + c] = p;
  }
}

// ------------------------------------------------------------------ k_vselect

struct SelArgs {
  int B, T_cap, V, Rr, n_chunks, P, cache;
  int slice;           // walks: vocabulary entries per workgroup (a multiple of 4)
  uint32_t tag_base;   // walks: this call's exchange-tag base (bits 12..31), never 0
  const float* tgt;
  const float* dft;
  const int32_t* dft_row;
  const int32_t* n_nodes;
  const int32_t* parent;
  const int32_t* token;
  const int32_t* depth;
  const float* u_node;
  const float* u_final;
  const Partial* part;
  unsigned char* sync;
  int32_t* acc_len;
  int32_t* acc_path;
  int32_t* next_token;
  float* p_tok;
  float* q_tok;
  int8_t* decision;
  int32_t* near_tie;
  int32_t* status;
};

// Shared state of one sequence inside a select workgroup.
struct SelShared {
  int row[SPEC_MAX_TREE];  // draft row of every node (rejection modes)
  int par[SPEC_MAX_TREE];
  int tok[SPEC_MAX_TREE];
  int dep[SPEC_MAX_TREE];
  int nch[SPEC_MAX_TREE];
  int arg_p[SPEC_MAX_TREE];
  float m_p[SPEC_MAX_TREE];
  float m_q[SPEC_MAX_TREE];
  double S_p[SPEC_MAX_TREE];
  double S_q[SPEC_MAX_TREE];
  double pt[SPEC_MAX_TREE];
  double qt[SPEC_MAX_TREE];
  float u[SPEC_MAX_TREE];       // the nodes' acceptance uniforms (rejection modes)
  float own_lp[SPEC_MAX_TREE];  // a child's token logits in its parent's target and draft rows
  float own_lq[SPEC_MAX_TREE];
  int dec[SPEC_MAX_TREE];
  double red[2 * kSelWaves];
  double scan[kSelThreads];
  double slots[2 * kMaxP];
  double invN[64];
  double xsum;  // reduce_exchange's total
  // row-statistics merge: jobs are the needed rows, entries their chunk partials
  Partial ent[kMergeEntries];
  int job_unit[2 * SPEC_MAX_TREE];
  int job_node[2 * SPEC_MAX_TREE];  // node t; draft rows of node t stored as -1 - t
  float job_m[2 * SPEC_MAX_TREE];
  int n_jobs;
  int near_count;
  int stop;
  // rejection-mode walks: frontier, scan list, per-workgroup row statistics
  // and the word exchange
  int front[SPEC_MAX_TREE];
  int scan_node[SPEC_MAX_TREE];
  int in_batch[SPEC_MAX_TREE];
  int n_front, n_scan;
  float sc_m[kScanRows];
  int sc_a[kScanRows];
  double sc_S[kScanRows];
  float wm[kSelWaves];
  int wa[kSelWaves];
  double wsum[kSelWaves];
  uint32_t xw_mine[kXWords];
  uint32_t xw_all[kMaxP * kXWords];
};

// Cross-workgroup meeting point of the P workgroups of one sequence.
struct SeqSync {
  uint64_t* slot;   // [2 parities][kMaxP][4]: low/high halves of a, then of b
  uint64_t* wslot;  // [2 parities][kMaxP][kXWords] (the walks' word exchange)
  int P, w, rounds;
  int pmax;           // workgroup capacity of the slot areas (>= P)
  uint32_t tag_base;  // 0 when the slots are cleared before the call, else a per-call epoch
  int32_t* status;

  // Everyone publishes nw (<= kXWords) 32-bit words, waits for the other
  // workgroups and returns all P x nw words in `all` ([P][nw], identical in
  // every workgroup).  Tags and parities as in exchange() below.
  __device__ __forceinline__ void exchange_words(const uint32_t* mine, int nw, uint32_t* all) {
    if (P == 1) {
      for (int i = threadIdx.x; i < nw; i += kSelThreads) all[i] = mine[i];
      __syncthreads();
      ++rounds;
      return;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint32_t tag = tag_base + (uint32_t)rounds + 1u;
      uint64_t* base = wslot + (size_t)(rounds & 1) * pmax * kXWords;
      for (int i = lane; i < nw; i += 64)
        store_coherent(base + (size_t)w * kXWords + i, ((uint64_t)tag << 32) | mine[i]);
      // every workgroup's words, lane-strided: all loads of a polling round
      // are issued together (one coherent round trip per round)
      constexpr int kPer = kMaxP * kXWords / 64;
      const int n = P * nw;
      uint64_t v[kPer];
      bool ok[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        ok[j] = lane + 64 * j >= n;
        v[j] = 0;
      }
      int spins = 0;
      for (;;) {
        bool done = true;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const int i = lane + 64 * j;
          if (!ok[j]) v[j] = load_coherent(base + (size_t)(i / nw) * kXWords + (i - (i / nw) * nw));
        }
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          if (!ok[j]) ok[j] = (uint32_t)(v[j] >> 32) == tag;
          done = done && ok[j];
        }
        if (done) break;
        if (++spins > (1 << 22)) {
          raise_status(status, SPEC_DEV_SYNC_TIMEOUT);
          break;
        }
      }
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const int i = lane + 64 * j;
        if (i < n) all[i] = (uint32_t)v[j];
      }
    }
    __syncthreads();
    ++rounds;
  }

  // Everyone publishes (a, b), waits for the other workgroups and returns the
  // per-workgroup values in s_slots (identical in every workgroup).  Word k of
  // a workgroup's slot holds 32 bits of its values in the low half and the
  // round number plus one in the high half: a word read at the coherent level
  // with the current tag is this round's, whatever order the stores landed in.
  // Round r + 2 reuses round r's parity only after every workgroup has
  // published round r + 1, i.e. after every reader is done with round r.
  __device__ __forceinline__ void exchange(double a, double b, double* s_slots) {
    if (P == 1) {
      if (threadIdx.x == 0) {
        s_slots[0] = a;
        s_slots[1] = b;
      }
      __syncthreads();
      ++rounds;
      return;
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const uint32_t tag = tag_base + (uint32_t)rounds + 1u;
      uint64_t* base = slot + (size_t)(rounds & 1) * pmax * 4;
      if (lane < 4) {
        const uint64_t bits = (uint64_t)__double_as_longlong(lane < 2 ? a : b);
        const uint32_t half = (lane & 1) ? (uint32_t)(bits >> 32) : (uint32_t)bits;
        store_coherent(base + w * 4 + lane, ((uint64_t)tag << 32) | half);
      }
      // the 4P words of this parity, two per lane
      const int n = 4 * P;
      uint64_t v0 = 0, v1 = 0;
      bool ok0 = lane >= n, ok1 = lane + 64 >= n;
      int spins = 0;
      while (!(ok0 && ok1)) {
        if (!ok0) {
          v0 = load_coherent(base + lane);
          ok0 = (uint32_t)(v0 >> 32) == tag;
        }
        if (!ok1) {
          v1 = load_coherent(base + lane + 64);
          ok1 = (uint32_t)(v1 >> 32) == tag;
        }
        if (++spins > (1 << 22)) {
          raise_status(status, SPEC_DEV_SYNC_TIMEOUT);
          break;
        }
      }
      // word k is 32-bit element k of the little-endian double array
      uint32_t* dst = reinterpret_cast<uint32_t*>(s_slots);
      if (lane < n) dst[lane] = (uint32_t)v0;
      if (lane + 64 < n) dst[lane + 64] = (uint32_t)v1;
    }
    __syncthreads();
    ++rounds;
  }
};

// Block sum of x, then its sum over the P workgroups (identical in every
// workgroup): each wave's sum goes through LDS to wave 0, which publishes the
// workgroup's total, waits for the others and adds them in a fixed lane order;
// lane 0 leaves the total in *out and its reciprocal in *inv_out.  Two
// barriers in all.  Slot words, tags and parities as in SeqSync::exchange.
__device__ __forceinline__ double reduce_exchange(SeqSync& sy, double x, double* s_red, double* out,
                                                  double* inv_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  x = wave_sum_f64(x);
  __syncthreads();
  if (lane == 0) s_red[wave] = x;
  __syncthreads();
  if (tid < 64) {
    double wg = 0.0;
    for (int w = 0; w < kSelWaves; ++w) wg += s_red[w];
    double total = wg;
    if (sy.P > 1) {
      const uint32_t tag = sy.tag_base + (uint32_t)sy.rounds + 1u;
      uint64_t* base = sy.slot + (size_t)(sy.rounds & 1) * sy.pmax * 4;
      if (lane < 2) {
        const uint64_t bits = (uint64_t)__double_as_longlong(wg);
        const uint32_t half = lane ? (uint32_t)(bits >> 32) : (uint32_t)bits;
        store_coherent(base + sy.w * 4 + lane, ((uint64_t)tag << 32) | half);
      }
      // lane i < P reads workgroup i's two words
      uint64_t lo = 0, hi = 0;
      bool ok = lane >= sy.P;
      int spins = 0;
      while (!ok) {
        lo = load_coherent(base + lane * 4);
        hi = load_coherent(base + lane * 4 + 1);
        ok = (uint32_t)(lo >> 32) == tag && (uint32_t)(hi >> 32) == tag;
        if (!ok && ++spins > (1 << 22)) {
          raise_status(sy.status, SPEC_DEV_SYNC_TIMEOUT);
          break;
        }
      }
      const double mine =
          lane < sy.P ? __longlong_as_double((long long)(((hi & 0xffffffffull) << 32) | (lo & 0xffffffffull)))
                      : 0.0;
      total = wave_sum_f64(mine);
    }
    if (lane == 0) {
      *out = total;
      *inv_out = 1.0 / total;
    }
  }
  __syncthreads();
  ++sy.rounds;
  return *out;
}

// One row pair (target row of node s and its draft row) with its statistics.
struct RowPair {
  const float* lp;
  const float* lq;
  double mp, mq;
  double invSp, invSq;  // accurate (fp64) normalisers once known
};

// p(v), q(v) and the residual after k rejections, r_k(v), in fp64, from the
// token's logits lp_v, lq_v in the row pair.
__device__ inline double eval_r_logits(const RowPair& rp, float lp_v, float lq_v, int k,
                                       const double* invN, double& qv) {
  double r = exp((double)lp_v - rp.mp) * rp.invSp;
  qv = exp((double)lq_v - rp.mq) * rp.invSq;
  for (int j = 0; j < k; ++j) {
    const double w = r - qv;
    r = w > 0.0 ? w * invN[j] : 0.0;
  }
  return r;
}

__device__ inline double eval_r(const RowPair& rp, int v, int k, const double* invN, double& qv) {
  double r = exp((double)rp.lp[v] - rp.mp) * rp.invSp;
  qv = exp((double)rp.lq[v] - rp.mq) * rp.invSq;
  for (int j = 0; j < k; ++j) {
    const double w = r - qv;
    r = w > 0.0 ? w * invN[j] : 0.0;
  }
  return r;
}

// Weight of v in the final draw: unnormalised p (k < 0) or max(0, r_k - q).
__device__ inline double draw_weight(const RowPair& rp, int v, int k, const double* invN) {
  if (k < 0) return exp((double)rp.lp[v] - rp.mp);
  double qv;
  const double r = eval_r(rp, v, k, invN, qv);
  const double w = r - qv;
  return w > 0.0 ? w : 0.0;
}

struct Slice {
  int lo, hi;
};

__device__ inline Slice slice_of(int V, int P, int w) {
  Slice s;
  s.lo = (int)((long)V * w / P);
  s.hi = (int)((long)V * (w + 1) / P);
  return s;
}

// Sums over the P exchanged slots, in slot order.  The slots are read eight
// at a time with every read of a group issued before its adds (a loop bounded
// by P would wait out one LDS round trip per slot); a slot past P adds +0.0,
// which leaves a sum of non-negative values unchanged.
__device__ __forceinline__ void slot_sums(const double* slots, int P, double& ta, double& tb) {
  static_assert(kMaxP % 8 == 0, "whole groups of slots");
  ta = 0.0;
  tb = 0.0;
  for (int i0 = 0; i0 < P; i0 += 8) {
    double a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = slots[2 * (i0 + j)];
      b[j] = slots[2 * (i0 + j) + 1];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      ta += i0 + j < P ? a[j] : 0.0;
      tb += i0 + j < P ? b[j] : 0.0;
    }
  }
}

__device__ __forceinline__ double slot_sum(const double* slots, int P) {
  double t = 0.0;
  for (int i0 = 0; i0 < P; i0 += 8) {
    double a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = slots[2 * (i0 + j)];
#pragma unroll
    for (int j = 0; j < 8; ++j) t += i0 + j < P ? a[j] : 0.0;
  }
  return t;
}

// The slice holding the draw's threshold thr: the first slot js with weight
// whose running total passes thr, and the total before it (base); past the
// end (rounding), the last slot with weight (overshoot).  Slots read as in
// slot_sums.
__device__ __forceinline__ bool find_slice(const double* slots, int P, double thr, int& js,
                                           double& base) {
  base = 0.0;
  js = -1;
  int jlast = -1;
  double base_last = 0.0;
  for (int i0 = 0; i0 < P; i0 += 8) {
    double t[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) t[j] = slots[2 * (i0 + j)];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + j;
      const double ti = t[j];
      if (i >= P) continue;
      if (ti > 0.0) {
        jlast = i;
        base_last = base;
      }
      if (js < 0 && ti > 0.0 && base + ti > thr) js = i;
      if (js < 0) base += ti;
    }
  }
  const bool overshoot = js < 0;
  if (overshoot) {
    js = jlast;
    base = base_last;
  }
  return overshoot;
}

// Accurate softmax normalisers of a row pair: sum exp(l - m) in fp64 over V.
__device__ __forceinline__ void pass_normalisers(RowPair& rp, bool with_q, SeqSync& sy, SelShared& sh, int V) {
  const Slice sl = slice_of(V, sy.P, sy.w);
  double a = 0.0, b = 0.0;
  for (int v = sl.lo + threadIdx.x; v < sl.hi; v += kSelThreads) {
    a += exp((double)rp.lp[v] - rp.mp);
    if (with_q) b += exp((double)rp.lq[v] - rp.mq);
  }
  block_sum2_f64(a, b, sh.red);
  sy.exchange(a, b, sh.slots);
  double ta, tb;
  slot_sums(sh.slots, sy.P, ta, tb);
  rp.invSp = 1.0 / ta;
  if (with_q) rp.invSq = 1.0 / tb;
  __syncthreads();
}

// Normaliser of the next residual: sum_v max(0, r_k(v) - q(v)).
__device__ __forceinline__ double pass_residual_mass(const RowPair& rp, int k, const double* invN, SeqSync& sy,
                                     SelShared& sh, int V) {
  const Slice sl = slice_of(V, sy.P, sy.w);
  double a = 0.0;
  for (int v = sl.lo + threadIdx.x; v < sl.hi; v += kSelThreads) {
    double qv;
    const double r = eval_r(rp, v, k, invN, qv);
    const double w = r - qv;
    if (w > 0.0) a += w;
  }
  a = block_sum_f64(a, sh.red);
  sy.exchange(a, 0.0, sh.slots);
  const double t = slot_sum(sh.slots, sy.P);
  __syncthreads();
  return t;
}

// Inverse-CDF draw over draw_weight(.., k, ..) in ascending vocabulary order.
// Each thread owns a contiguous range of its workgroup's slice.  Returns true in
// the one workgroup that found the token (written to *out_tok / *out_near);
// *total_out gets the total weight (all workgroups).
__device__ __forceinline__ bool pass_draw(const RowPair& rp, int k, const double* invN, double u, SeqSync& sy,
                          SelShared& sh, int V, int* out_tok, int* out_near, double* total_out) {
  const Slice sl = slice_of(V, sy.P, sy.w);
  const int n = sl.hi - sl.lo;
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int t0 = sl.lo + threadIdx.x * per;
  const int t1 = min(sl.hi, t0 + per);
  double mine = 0.0;
  for (int v = t0; v < t1; ++v) mine += draw_weight(rp, v, k, invN);
  double excl;
  const double slice_total = block_exclusive_scan_f64(mine, sh.scan, excl);
  sy.exchange(slice_total, 0.0, sh.slots);
  const double total = slot_sum(sh.slots, sy.P);
  *total_out = total;
  if (!(total > 0.0)) {
    __syncthreads();
    return false;
  }
  const double thr = u * total;
  const double eps = kCdfNearTie * total;
  // the slice holding the threshold (or, past the end, the last slice with weight)
  int js;
  double base;
  const bool overshoot = find_slice(sh.slots, sy.P, thr, js, base);
  __syncthreads();
  if (js != sy.w) return false;
  // the thread holding the threshold
  __shared__ int s_found_tok, s_found_near;
  if (threadIdx.x == 0) {
    s_found_tok = -1;
    s_found_near = 0;
  }
  __syncthreads();
  // thread ranges [base + incl[t-1], base + incl[t]) partition the slice exactly
  const double lo_run = base + (threadIdx.x > 0 ? sh.scan[threadIdx.x - 1] : 0.0);
  const double hi_run = base + sh.scan[threadIdx.x];
  (void)excl;
  if (!overshoot && mine > 0.0 && lo_run <= thr && thr < hi_run) {
    double run = lo_run;
    int found = -1, last_pos = -1, near = 1;
    for (int v = t0; v < t1; ++v) {
      const double w = draw_weight(rp, v, k, invN);
      if (!(w > 0.0)) continue;
      last_pos = v;
      const double before = run;
      run += w;
      if (run > thr) {
        found = v;
        near = (fabs(run - thr) < eps || fabs(before - thr) < eps) ? 1 : 0;
        break;
      }
    }
    s_found_tok = found >= 0 ? found : last_pos;
    s_found_near = near;
  }
  __syncthreads();
  if (s_found_tok < 0) {
    // overshoot through rounding: the last token with positive weight of this slice
    __shared__ int s_last;
    if (threadIdx.x == 0) s_last = -1;
    __syncthreads();
    int last = -1;
    for (int v = t0; v < t1; ++v)
      if (draw_weight(rp, v, k, invN) > 0.0) last = v;
    if (last >= 0) atomicMax(&s_last, last);
    __syncthreads();
    if (threadIdx.x == 0) {
      s_found_tok = s_last < 0 ? sl.lo : s_last;
      s_found_near = 1;
    }
    __syncthreads();
  }
  *out_tok = s_found_tok;
  *out_near = s_found_near;
  return true;
}

// ------------------------------------------------------------------ cached row pair
// When a workgroup's slice of the vocabulary fits, every thread keeps its
// contiguous range of the stop row pair in registers, in fp64: the target side
// (p, then each residual) and the draft side q.  The exponentials are taken
// once per node; each residual pass is then a few FMAs per entry, applied in
// the same operation order as eval_r.
constexpr int kCacheE = 20;  // entries per thread

struct RowCache {
  double r[kCacheE];
  double q[kCacheE];
  int v0, n;
};

// this thread's contiguous range of its workgroup's slice (the draw's partition)
__device__ inline void cache_range(RowCache& c, int V, const SeqSync& sy) {
  const Slice sl = slice_of(V, sy.P, sy.w);
  const int per = (sl.hi - sl.lo + kSelThreads - 1) / kSelThreads;
  c.v0 = sl.lo + (int)threadIdx.x * per;
  c.n = max(0, min(sl.hi, c.v0 + per) - c.v0);
}

// exp(l - m) of the row pair (q side only when with_q); with `normalise` the
// fp64 totals are exchanged and both sides become p and q
__device__ __forceinline__ void cache_load(RowCache& c, RowPair& rp, bool with_q, bool normalise, SeqSync& sy,
                           SelShared& sh) {
  double a = 0.0, bq = 0.0;
#pragma unroll
  for (int e = 0; e < kCacheE; ++e) {
    c.r[e] = 0.0;
    c.q[e] = 0.0;
    if (e < c.n) {
      c.r[e] = exp((double)rp.lp[c.v0 + e] - rp.mp);
      a += c.r[e];
      if (with_q) {
        c.q[e] = exp((double)rp.lq[c.v0 + e] - rp.mq);
        bq += c.q[e];
      }
    }
  }
  if (!normalise) return;
  block_sum2_f64(a, bq, sh.red);
  sy.exchange(a, bq, sh.slots);
  double ta, tb;
  slot_sums(sh.slots, sy.P, ta, tb);
  rp.invSp = 1.0 / ta;
  rp.invSq = 1.0 / tb;
#pragma unroll
  for (int e = 0; e < kCacheE; ++e) {
    c.r[e] *= rp.invSp;
    c.q[e] *= rp.invSq;
  }
  __syncthreads();
}

// this thread's part of sum max(0, r - q)
__device__ inline double cache_mass_local(const RowCache& c) {
  double a = 0.0;
#pragma unroll
  for (int e = 0; e < kCacheE; ++e) {
    const double w = c.r[e] - c.q[e];
    if (w > 0.0) a += w;
  }
  return a;
}

// one rejection and this thread's part of the next residual's mass, in one pass
__device__ inline double cache_step_mass(RowCache& c, double invN) {
  double a = 0.0;
#pragma unroll
  for (int e = 0; e < kCacheE; ++e) {
    const double w = c.r[e] - c.q[e];
    c.r[e] = w > 0.0 ? w * invN : 0.0;
    const double w2 = c.r[e] - c.q[e];
    if (w2 > 0.0) a += w2;
  }
  return a;
}

__device__ inline double cache_weight(const RowCache& c, int e, bool resid) {
  if (!resid) return c.r[e];
  const double w = c.r[e] - c.q[e];
  return w > 0.0 ? w : 0.0;
}

// The inverse-CDF draw of pass_draw over cached weights: r itself (resid ==
// false) or max(0, r - q).
__device__ __forceinline__ bool cache_draw(const RowCache& c, bool resid, double u, SeqSync& sy, SelShared& sh,
                           int V, int* out_tok, int* out_near, double* total_out) {
  const Slice sl = slice_of(V, sy.P, sy.w);
  double mine = 0.0;
#pragma unroll
  for (int e = 0; e < kCacheE; ++e)
    if (e < c.n) mine += cache_weight(c, e, resid);
  double excl;
  const double slice_total = block_exclusive_scan_f64(mine, sh.scan, excl);
  (void)excl;
  sy.exchange(slice_total, 0.0, sh.slots);
  const double total = slot_sum(sh.slots, sy.P);
  *total_out = total;
  if (!(total > 0.0)) {
    __syncthreads();
    return false;
  }
  const double thr = u * total;
  const double eps = kCdfNearTie * total;
  int js;
  double base;
  const bool overshoot = find_slice(sh.slots, sy.P, thr, js, base);
  __syncthreads();
  if (js != sy.w) return false;
  __shared__ int s_found_tok, s_found_near, s_last;
  if (threadIdx.x == 0) {
    s_found_tok = -1;
    s_found_near = 0;
    s_last = -1;
  }
  __syncthreads();
  const double lo_run = base + (threadIdx.x > 0 ? sh.scan[threadIdx.x - 1] : 0.0);
  const double hi_run = base + sh.scan[threadIdx.x];
  if (!overshoot && mine > 0.0 && lo_run <= thr && thr < hi_run) {
    double run = lo_run;
    int found = -1, last_pos = -1, near = 1;
    bool done = false;
#pragma unroll
    for (int e = 0; e < kCacheE; ++e) {
      if (done || e >= c.n) continue;
      const double w = cache_weight(c, e, resid);
      if (!(w > 0.0)) continue;
      last_pos = c.v0 + e;
      const double before = run;
      run += w;
      if (run > thr) {
        found = c.v0 + e;
        near = (fabs(run - thr) < eps || fabs(before - thr) < eps) ? 1 : 0;
        done = true;
      }
    }
    s_found_tok = found >= 0 ? found : last_pos;
    s_found_near = near;
  }
  __syncthreads();
  if (s_found_tok < 0) {
    // overshoot through rounding: the last token with positive weight of this slice
    int last = -1;
#pragma unroll
    for (int e = 0; e < kCacheE; ++e)
      if (e < c.n && cache_weight(c, e, resid) > 0.0) last = c.v0 + e;
    if (last >= 0) atomicMax(&s_last, last);
    __syncthreads();
    if (threadIdx.x == 0) {
      s_found_tok = s_last < 0 ? sl.lo : s_last;
      s_found_near = 1;
    }
    __syncthreads();
  }
  *out_tok = s_found_tok;
  *out_near = s_found_near;
  return true;
}

// Sequential checking of the children of node s ([ResiSpec] section 4): in
// node-index order against the running target p' (p_s at first), p' <-
// norm(max(0, p' - q_s)) after each rejection.  sh.pt / sh.qt of the children
// and the statistics of s's rows must be in place.  Returns true (and the
// child in next_s) on an acceptance; otherwise the draw description for s:
// draw_k (-1: from p_s) and whether rc holds the row pair.
__device__ __forceinline__ bool test_children_seq(const SelArgs& A, size_t nb, int s, int T, RowPair& rp,
                                  RowCache& rc, SeqSync& sy, SelShared& sh, int& draw_k,
                                  bool& cached, int& next_s) {
  const int tid = threadIdx.x;
  const int V = A.V;
  const int b = (int)(nb / A.T_cap);
  const double* invN = sh.invN;
  int k = 0;
  draw_k = -1;
  cached = false;
  bool dead = false, have_norm = false, moved = false;
  rp.lp = A.tgt + (nb + s) * V;
  rp.mp = sh.m_p[s];
  if (sh.nch[s] > 0) {
    const int r = sh.row[s];
    rp.lq = A.dft + ((size_t)b * A.Rr + r) * V;
    rp.mq = sh.m_q[s];
  }
  // Every child's own logits in both rows, gathered once: the tests after a
  // rejection read them from LDS instead of a global round trip each (the
  // loads stay in flight until the first rejection's exchanges are done).
  const bool own = tid > s && tid < T && sh.par[tid] == s;
  float own_lp = 0.0f, own_lq = 0.0f;
  if (own && sh.nch[s] > 1) {
    own_lp = rp.lp[sh.tok[tid]];
    own_lq = rp.lq[sh.tok[tid]];
  }
  bool own_stored = false;
  double mass_next = 0.0;  // cached path: this thread's part of the next residual mass
  int remaining = sh.nch[s];
  for (int ch = s + 1; ch < T && remaining > 0; ++ch) {
    if (sh.par[ch] != s) continue;
    --remaining;
    if (dead) {
      if (tid == 0) sh.dec[ch] = 0;
      continue;
    }
    const int x = sh.tok[ch];
    double ratio;
    if (k == 0) {
      const double p = sh.pt[ch], q = sh.qt[ch];
      ratio = q > 0.0 ? p / q : (p > 0.0 ? INFINITY : 0.0);
    } else {
      double qv;
      const double r = eval_r_logits(rp, sh.own_lp[ch], sh.own_lq[ch], k, invN, qv);
      ratio = qv > 0.0 ? r / qv : (r > 0.0 ? INFINITY : 0.0);
    }
    (void)x;
    const double u = (double)sh.u[ch];  // loaded with the tree
    if (tid == 0 && fabs(ratio - u) < kNearTie) sh.near_count++;
    if (u < ratio) {
      if (tid == 0) sh.dec[ch] = 1;
      next_s = ch;
      moved = true;
      break;
    }
    if (tid == 0) sh.dec[ch] = 0;
    if (!have_norm) {
      if (A.cache) {
        cache_load(rc, rp, true, true, sy, sh);
        cached = true;
        mass_next = cache_mass_local(rc);
      } else {
        pass_normalisers(rp, true, sy, sh, V);
      }
      have_norm = true;
    }
    if (!own_stored) {
      // read at k >= 1, after the residual mass exchange's barriers
      if (own) {
        sh.own_lp[tid] = own_lp;
        sh.own_lq[tid] = own_lq;
      }
      own_stored = true;
    }
    if (remaining == 0) {
      // last child rejected: the draw uses max(0, r_k - q) unnormalised
      draw_k = k;
      break;
    }
    // cached: one exchange per rejection (it also leaves 1 / N in invN[k]),
    // then the residual step and the next mass in one pass over the cache
    const double N = A.cache ? reduce_exchange(sy, mass_next, sh.red, &sh.xsum, &sh.invN[k])
                             : pass_residual_mass(rp, k, invN, sy, sh, V);
    if (!(N > 0.0) || k >= 63) {
      dead = true;
      if (tid == 0) raise_status(A.status, SPEC_DEV_RESIDUAL_ZERO);
    } else {
      if (A.cache) {
        mass_next = cache_step_mass(rc, sh.invN[k]);
      } else {
        if (tid == 0) sh.invN[k] = 1.0 / N;
        __syncthreads();
      }
      ++k;
    }
  }
  __syncthreads();
  if (moved) return true;
  if (dead) draw_k = -1;
  return false;
}

// The next token at the stop node: its greedy token (greedy mode, or a bad
// sequence), else an inverse-CDF draw with u_final from the residual after
// draw_k rejections (draw_k >= 0; with `cached` the row pair sits in rc) or
// from p_stop (draw_k < 0).  rp.lp, rp.mp (and the q side for draw_k >= 0)
// describe the stop rows.  Returns true in the workgroup that holds the token.
__device__ __forceinline__ bool final_token(bool greedy, const SelArgs& A, size_t nb, int stop, bool bad,
                            int draw_k, bool cached, RowPair& rp, RowCache& rc, SeqSync& sy,
                            SelShared& sh, bool lead, int& next, int& cdf_near) {
  const int tid = threadIdx.x;
  const int V = A.V;
  const double* invN = sh.invN;
  const int b = (int)(nb / A.T_cap);
  if (greedy || bad) {
    next = sh.arg_p[stop];
    return lead;
  }
  rp.lp = A.tgt + (nb + stop) * V;
  rp.mp = sh.m_p[stop];
  const double u = (double)A.u_final[b];
  double total = 0.0;
  int tok = 0, near = 0;
  bool found;
  if (A.cache && draw_k >= 0 && cached) {
    found = cache_draw(rc, true, u, sy, sh, V, &tok, &near, &total);
  } else if (A.cache && draw_k < 0) {
    cache_load(rc, rp, false, false, sy, sh);
    found = cache_draw(rc, false, u, sy, sh, V, &tok, &near, &total);
  } else {
    found = pass_draw(rp, draw_k, invN, u, sy, sh, V, &tok, &near, &total);
  }
  if (!(total > 0.0) && draw_k >= 0) {
    // nothing left in the residual (rounding only): draw from p_stop
    if (lead && tid == 0) raise_status(A.status, SPEC_DEV_RESIDUAL_ZERO);
    found = pass_draw(rp, -1, invN, u, sy, sh, V, &tok, &near, &total);
  }
  if (found) {
    next = tok;
    cdf_near = near;
  }
  return found;
}

template <int MODE>
__global__ __launch_bounds__(kSelThreads) void k_vselect(SelArgs A) {
  __shared__ SelShared sh;
  const int b = blockIdx.x / A.P;
  const int w = blockIdx.x - b * A.P;
  const int tid = threadIdx.x;
  const int T_cap = A.T_cap, V = A.V;
  SeqSync sy;
  sy.slot = reinterpret_cast<uint64_t*>(A.sync + (size_t)b * kSyncStride);
  sy.P = A.P;
  sy.w = w;
  sy.rounds = 0;
  sy.pmax = kMaxP;
  sy.tag_base = 0;  // k_vstats cleared the slots
  sy.wslot = nullptr;
  sy.status = A.status;
  const bool lead = w == 0;

  const size_t nb = (size_t)b * T_cap;
  __shared__ int s_bad;
  static_assert(kSelThreads >= SPEC_MAX_TREE, "one tree row per thread");
  // One round trip for the tree and, in greedy mode, for the chunk partials of
  // every target row the tree can have (rows past n_nodes are never used).
  const int T_in = A.n_nodes[b];
  int my_par = -1, my_tok = 0, my_dep = 0, my_row = 0;
  float my_u = 0.0f;
  if (tid < T_cap) {
    my_par = tid == 0 ? -1 : A.parent[nb + tid];
    my_tok = A.token[nb + tid];
    my_dep = tid == 0 ? 0 : A.depth[nb + tid];
    if (MODE != SPEC_GREEDY) {
      my_row = A.dft_row[nb + tid];
      my_u = A.u_node[nb + tid];
    }
  }
  const bool staged = MODE == SPEC_GREEDY && T_cap * A.n_chunks <= kMergeEntries;
  if (staged)
    for (int e = tid; e < T_cap * A.n_chunks; e += kSelThreads)
      sh.ent[e] = A.part[nb * A.n_chunks + e];
  int T = T_in < 1 ? 1 : (T_in > T_cap ? T_cap : T_in);

  // ---------------------------------------------------------------- tree + row stats
  for (int t = tid; t < SPEC_MAX_TREE; t += kSelThreads) {
    sh.nch[t] = 0;
    sh.dec[t] = -1;
    sh.pt[t] = 0.0;
    sh.qt[t] = 0.0;
  }
  if (tid == 0) {
    sh.near_count = 0;
    s_bad = (T_in < 1 || T_in > T_cap) ? SPEC_DEV_BAD_TREE : 0;
  }
  __syncthreads();
  if (tid < T) {
    sh.par[tid] = my_par;
    sh.tok[tid] = my_tok;
    sh.dep[tid] = my_dep;
    sh.row[tid] = my_row;
    sh.u[tid] = my_u;
  }
  __syncthreads();
  // validate the tree against the vocabulary and the draft rows; a bad
  // sequence accepts nothing and takes the greedy token at the root
  for (int t = tid + 1; t < T; t += kSelThreads) {
    const int p = sh.par[t];
    if (p < 0 || p >= t) {
      atomicOr(&s_bad, SPEC_DEV_BAD_TREE);
    } else {
      if (sh.dep[t] != sh.dep[p] + 1) atomicOr(&s_bad, SPEC_DEV_BAD_TREE);
      atomicAdd(&sh.nch[p], 1);
    }
    if (sh.tok[t] < 0 || sh.tok[t] >= V) atomicOr(&s_bad, SPEC_DEV_BAD_TOKEN);
  }
  __syncthreads();
  if (MODE != SPEC_GREEDY) {
    for (int t = tid; t < T; t += kSelThreads) {
      if (sh.nch[t] == 0) continue;
      const int r = sh.row[t];
      if (r < 0 || r >= A.Rr) atomicOr(&s_bad, SPEC_DEV_BAD_ROW);
    }
    __syncthreads();
  }
  const bool bad = s_bad != 0;
  if (bad) {
    if (lead && tid == 0) raise_status(A.status, s_bad);
    T = 1;
    for (int t = tid; t < SPEC_MAX_TREE; t += kSelThreads) sh.nch[t] = 0;
    __syncthreads();
  }
  // The logits of every node's own token under its parent, issued now so
  // they arrive while the row statistics are merged.
  double lp_own = 0.0, lq_own = 0.0;
  if (tid + 1 < T) {
    const int t = tid + 1, sp = sh.par[t], x = sh.tok[t];
    lp_own = A.tgt[(nb + sp) * V + x];
    if (MODE != SPEC_GREEDY) lq_own = A.dft[((size_t)b * A.Rr + sh.row[sp]) * V + x];
  }
  // Row statistics from the vocabulary pass's chunk partials, with all threads:
  // the partials of a batch of rows are staged in LDS, then per row the
  // maximum and lowest argmax (chunks in index order), per partial its sum
  // rescaled to the row maximum (fp64), and per row the total.
  if (tid == 0) sh.n_jobs = T;
  for (int t = tid; t < T; t += kSelThreads) {
    sh.job_unit[t] = (int)(nb + t);
    sh.job_node[t] = t;
  }
  __syncthreads();
  if (MODE != SPEC_GREEDY) {
    for (int t = tid; t < T; t += kSelThreads) {
      if (sh.nch[t] == 0) continue;
      const int j = atomicAdd(&sh.n_jobs, 1);
      sh.job_unit[j] = (int)((size_t)A.B * T_cap + (size_t)b * A.Rr + sh.row[t]);
      sh.job_node[j] = -1 - t;
    }
    __syncthreads();
  }
  {
    const int n_jobs = sh.n_jobs, nc = A.n_chunks;
    const int per_batch = min(kMergeEntries / nc, 2 * SPEC_MAX_TREE);
    for (int j0 = 0; j0 < n_jobs; j0 += per_batch) {
      const int nj = min(per_batch, n_jobs - j0);
      if (!staged) {  // staged: the target rows' partials are in LDS already
        for (int e = tid; e < nj * nc; e += kSelThreads) {
          const int j = j0 + e / nc, cc = e - (e / nc) * nc;
          sh.ent[e] = A.part[(size_t)sh.job_unit[j] * nc + cc];
        }
        __syncthreads();
      }
      for (int k = tid; k < nj; k += kSelThreads) {
        float m = -INFINITY;
        int arg = 0;
        for (int cc = 0; cc < nc; ++cc) {
          const Partial& q = sh.ent[k * nc + cc];
          if (q.m > m) {
            m = q.m;
            arg = q.arg;
          }
        }
        sh.job_m[k] = m;
        const int node = sh.job_node[j0 + k];
        if (node >= 0) {
          sh.m_p[node] = m;
          sh.arg_p[node] = arg;
        } else {
          sh.m_q[-1 - node] = m;
        }
      }
      __syncthreads();
      for (int e = tid; e < nj * nc; e += kSelThreads) {
        const int k = e / nc;
        const float mc = sh.ent[e].m;
        sh.ent[e].S = mc == -INFINITY ? 0.0 : sh.ent[e].S * exp((double)mc - (double)sh.job_m[k]);
      }
      __syncthreads();
      for (int k = tid; k < nj; k += kSelThreads) {
        double S = 0.0;
        for (int cc = 0; cc < nc; ++cc) S += sh.ent[k * nc + cc].S;
        const int node = sh.job_node[j0 + k];
        if (node >= 0) sh.S_p[node] = S;
        else sh.S_q[-1 - node] = S;
      }
      __syncthreads();
    }
  }
  // p and q of every node's own token under its parent (fp64 exp, merged sums)
  if (tid + 1 < T) {
    const int t = tid + 1, sp = sh.par[t];
    sh.pt[t] = exp(lp_own - (double)sh.m_p[sp]) / sh.S_p[sp];
    if (MODE != SPEC_GREEDY) sh.qt[t] = exp(lq_own - (double)sh.m_q[sp]) / sh.S_q[sp];
  }
  __syncthreads();

  int stop = 0;
  // draw description for the final token
  int draw_k = -1;          // -1: draw from p_stop; k >= 0: from max(0, r_k - q)
  RowPair rp{};
  RowCache rc;
  bool cached = false;  // rc holds the current node's normalised pair (residual after k steps)
  cache_range(rc, V, sy);

  if (MODE == SPEC_GREEDY || MODE == SPEC_REJECT_PATH) {
    for (int t = tid + 1; t < T; t += kSelThreads) {
      int acc;
      if (MODE == SPEC_GREEDY) {
        acc = sh.tok[t] == sh.arg_p[sh.par[t]];
      } else {
        const double p = sh.pt[t], q = sh.qt[t];
        const double ratio = q > 0.0 ? p / q : (p > 0.0 ? INFINITY : 0.0);
        const double u = (double)sh.u[t];
        acc = u < ratio;
        if (fabs(ratio - u) < kNearTie) atomicAdd(&sh.near_count, 1);
      }
      sh.dec[t] = acc;
    }
    __syncthreads();
    // a node survives when it and all its ancestors are accepted; the deepest
    // survivor wins, the lowest node index on ties (one thread per node, each
    // walking its own ancestors, then a max over keys depth*1024 + (1023 - t))
    if (tid == 0) sh.stop = 1023;  // key of the root: depth 0, node 0
    __syncthreads();
    for (int t = tid + 1; t < T; t += kSelThreads) {
      int ok = 1;
      for (int u = t; u > 0 && ok; u = sh.par[u]) ok = sh.dec[u];
      if (ok) atomicMax(&sh.stop, sh.dep[t] * 1024 + (1023 - t));
    }
    __syncthreads();
    if (tid == 0) sh.stop = 1023 - (sh.stop & 1023);
    __syncthreads();
    stop = sh.stop;
    if (MODE == SPEC_REJECT_PATH && !bad) {
      rp.lp = A.tgt + (nb + stop) * V;
      rp.mp = sh.m_p[stop];
      if (sh.nch[stop] > 0) {
        const int r = sh.row[stop];
        rp.lq = A.dft + ((size_t)b * A.Rr + r) * V;
        rp.mq = sh.m_q[stop];
        if (A.cache) {
          cache_load(rc, rp, true, true, sy, sh);
          cached = true;
        } else {
          pass_normalisers(rp, true, sy, sh, V);
        }
        draw_k = 0;
      }
    }
  } else {
    // sequential multi-candidate verification with residual renormalisation
    int s = 0;
    for (;;) {
      int next_s = s;
      if (test_children_seq(A, nb, s, T, rp, rc, sy, sh, draw_k, cached, next_s)) {
        s = next_s;
        continue;
      }
      stop = s;
      break;
    }
  }

  // ---------------------------------------------------------------- final token
  int next = 0, cdf_near = 0;
  const bool have_next = final_token(MODE == SPEC_GREEDY, A, nb, stop, bad, draw_k, cached, rp,
                                     rc, sy, sh, lead, next, cdf_near);

  // ---------------------------------------------------------------- outputs
  const int near_total = sh.near_count + cdf_near;
  if (have_next && tid == 0) {
    A.next_token[b] = next;
    if (A.near_tie) A.near_tie[b] = near_total;
  }
  if (!lead) return;
  if (tid == 0) A.acc_len[b] = sh.dep[stop];
  for (int t = tid; t < T_cap; t += kSelThreads) {
    int pv = -1;
    if (!bad && t <= sh.dep[stop]) {
      int cur = stop;
      while (sh.dep[cur] > t) cur = sh.par[cur];
      pv = cur;
    }
    if (bad && t == 0) pv = 0;
    A.acc_path[nb + t] = pv;
    if (A.decision) A.decision[nb + t] = (int8_t)((t < T && !bad) ? sh.dec[t] : -1);
    if (A.p_tok) A.p_tok[nb + t] = (t < T && !bad) ? (float)sh.pt[t] : 0.0f;
    if (A.q_tok) A.q_tok[nb + t] = (t < T && !bad) ? (float)sh.qt[t] : 0.0f;
  }
}


// ------------------------------------------------------------------ rejection-mode walks
// Rejection sampling that reads only the rows the decisions need
// ([ReDrafter] "The Full Speculative Decoding Loop", Step 5, rejection
// sampling; [ResiSpec] section 4, sequential checking).  The acceptance, stop
// node and next token equal k_vselect's in the same mode; only the tested
// nodes (children of nodes whose rows are read) get decision, p_tok and q_tok.
// P workgroups per sequence split every scanned row into aligned slices: each
// scans its slice of a batch of rows for (max, lowest argmax, sum exp(l - max)),
// the P partial statistics are exchanged through tagged words, and every
// workgroup merges them in workgroup order into the same row statistics.
// Exchange tags carry a per-call epoch, so the workspace needs no initial
// contents.

constexpr int kScanBatch = 4;  // 16-byte loads per thread per batch
constexpr int kScanBufs = 4;   // batches in flight

__device__ inline __amdgpu_buffer_rsrc_t scan_rsrc(const float* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, n * 4, 0x00020000);
}

__device__ inline void scan_issue(__amdgpu_buffer_rsrc_t rs, f32x4 (&buf)[kScanBatch], int j0) {
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j)
    buf[j] = __builtin_bit_cast(
        f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                   rs, ((j0 + j) * kSelThreads + (int)threadIdx.x) * 16, 0, kLoadOnce));
}

// Fold one batch (chunk positions relative to the slice; >= n masked) into a
// running (max m, lowest argmax a, sum S of exp(l - m)); exp in fp32, S in fp64.
__device__ inline void scan_fold(const f32x4 (&buf)[kScanBatch], int j0, int n, int base,
                                 float& m, int& a, double& S) {
  float bm = -INFINITY;
  int ba = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) {
    const int pos = ((j0 + j) * kSelThreads + (int)threadIdx.x) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float l = pos + e < n ? buf[j][e] : -INFINITY;
      if (l > bm) {
        bm = l;
        ba = base + pos + e;
      }
    }
  }
  if (bm == -INFINITY) return;
  if (bm > m) {
    S = m == -INFINITY ? 0.0 : S * (double)__builtin_amdgcn_exp2f((m - bm) * kLog2e);
    m = bm;
    a = ba;
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < kScanBatch; ++j) {
    const int pos = ((j0 + j) * kSelThreads + (int)threadIdx.x) * 4;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      sum += pos + e < n ? __builtin_amdgcn_exp2f((buf[j][e] - m) * kLog2e) : 0.0f;
  }
  S += (double)sum;
}

// Workgroup statistics of row i from the threads' (m, a, S) into sh.sc_*[i].
__device__ inline void scan_reduce(float m, int a, double S, int i, SelShared& sh) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float wm = m;
  int wa = a;
  wave_argmax(wm, wa);
  if (lane == 0) {
    sh.wm[wave] = wm;
    sh.wa[wave] = wa;
  }
  __syncthreads();
  float M = sh.wm[0];
  int Aa = sh.wa[0];
  for (int k = 1; k < kSelWaves; ++k) argmax_merge(M, Aa, sh.wm[k], sh.wa[k]);
  double part = (m == -INFINITY || M == -INFINITY)
                    ? 0.0
                    : S * (double)__builtin_amdgcn_exp2f((m - M) * kLog2e);
  part = wave_sum_f64(part);
  if (lane == 0) sh.wsum[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int k = 0; k < kSelWaves; ++k) t += sh.wsum[k];
    sh.sc_m[i] = M;
    sh.sc_a[i] = Aa;
    sh.sc_S[i] = t;
  }
}

// Statistics of nr (<= kScanRows) rows over this workgroup's slice [lo, lo + n);
// row_of(i) gives row i's first entry.  kScanBufs batches of loads in flight:
// the batches of the next rows are issued before the current one is folded.
template <bool VEC, typename RowOf>
__device__ __forceinline__ void scan_rows(int nr, RowOf row_of, int lo, int n, SelShared& sh) {
  const int tid = threadIdx.x;
  if constexpr (VEC) {
    const int n_per = ((n >> 2) + kSelThreads - 1) / kSelThreads;  // 16-byte chunks per thread
    const int nbat = n_per > 0 ? (n_per + kScanBatch - 1) / kScanBatch : 1;
    const int items = nr * nbat;
    auto issue = [&](int q, f32x4 (&buf)[kScanBatch]) {
      const int i = q / nbat, jb = q - (q / nbat) * nbat;
      scan_issue(scan_rsrc(row_of(i) + lo, n), buf, jb * kScanBatch);
    };
    float m = -INFINITY;
    int a = 0x7fffffff;
    double S = 0.0;
    auto fold_item = [&](int q, const f32x4 (&buf)[kScanBatch]) {
      const int i = q / nbat, jb = q - (q / nbat) * nbat;
      scan_fold(buf, jb * kScanBatch, n, lo, m, a, S);
      if (jb == nbat - 1) {
        scan_reduce(m, a, S, i, sh);
        m = -INFINITY;
        a = 0x7fffffff;
        S = 0.0;
      }
    };
    // kScanBufs batches in flight: batch q + kScanBufs - 1 is issued into the
    // registers batch q - 1 has just left
    f32x4 L[kScanBufs][kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBufs - 1; ++u)
      if (u < items) issue(u, L[u]);
    for (int q0 = 0; q0 < items; q0 += kScanBufs) {
#pragma unroll
      for (int u = 0; u < kScanBufs; ++u) {
        const int q = q0 + u;
        if (q + kScanBufs - 1 < items) issue(q + kScanBufs - 1, L[(u + kScanBufs - 1) % kScanBufs]);
        __builtin_amdgcn_sched_barrier(0);
        if (q < items) fold_item(q, L[u]);
      }
    }
  } else {
    for (int i = 0; i < nr; ++i) {
      const float* row = row_of(i);
      float m = -INFINITY;
      int a = 0x7fffffff;
      double S = 0.0;
      for (int v = tid; v < n; v += kSelThreads) {
        const float l = row[lo + v];
        if (l > m) {
          S = m == -INFINITY ? 0.0 : S * (double)__builtin_amdgcn_exp2f((m - l) * kLog2e);
          m = l;
          a = lo + v;
        }
        if (l != -INFINITY) S += (double)__builtin_amdgcn_exp2f((l - m) * kLog2e);
      }
      scan_reduce(m, a, S, i, sh);
    }
  }
}

template <int MODE, bool VEC>
__global__ __launch_bounds__(kSelThreads) void k_vrwalk(SelArgs A) {
  __shared__ SelShared sh;
  __shared__ int s_bad;
  const int b = blockIdx.x / A.P;
  const int w = blockIdx.x - b * A.P;
  const int tid = threadIdx.x;
  const int T_cap = A.T_cap, V = A.V, P = A.P;
  const int pb = walk_p_bound(V);
  unsigned char* area = A.sync + (size_t)b * walk_stride(V);
  SeqSync sy;
  sy.slot = reinterpret_cast<uint64_t*>(area);
  sy.wslot = reinterpret_cast<uint64_t*>(area + (size_t)pb * 2 * 4 * 8);
  sy.pmax = pb;
  sy.P = P;
  sy.w = w;
  sy.rounds = 0;
  sy.tag_base = A.tag_base;
  sy.status = A.status;
  const bool lead = w == 0;
  const size_t nb = (size_t)b * T_cap;
  const int lo = w * A.slice;
  const int n = max(0, min(A.slice, V - lo));
  static_assert(kSelThreads >= SPEC_MAX_TREE, "one tree row per thread");

  // ---------------------------------------------------------------- tree
  const int T_in = A.n_nodes[b];
  int my_par = -1, my_tok = 0, my_dep = 0, my_row = 0;
  float my_u = 0.0f;
  if (tid < T_cap) {
    my_par = tid == 0 ? -1 : A.parent[nb + tid];
    my_tok = A.token[nb + tid];
    my_dep = tid == 0 ? 0 : A.depth[nb + tid];
    my_row = A.dft_row[nb + tid];
    my_u = A.u_node[nb + tid];
  }
  int T = T_in < 1 ? 1 : (T_in > T_cap ? T_cap : T_in);
  for (int t = tid; t < SPEC_MAX_TREE; t += kSelThreads) {
    sh.nch[t] = 0;
    sh.dec[t] = -1;
    sh.pt[t] = 0.0;
    sh.qt[t] = 0.0;
  }
  if (tid == 0) {
    sh.near_count = 0;
    s_bad = (T_in < 1 || T_in > T_cap) ? SPEC_DEV_BAD_TREE : 0;
  }
  __syncthreads();
  if (tid < T) {
    sh.par[tid] = my_par;
    sh.tok[tid] = my_tok;
    sh.dep[tid] = my_dep;
    sh.row[tid] = my_row;
    sh.u[tid] = my_u;
  }
  __syncthreads();
  // the validation of k_vselect: a bad sequence accepts nothing and takes the
  // greedy token at the root
  for (int t = tid + 1; t < T; t += kSelThreads) {
    const int p = sh.par[t];
    if (p < 0 || p >= t) {
      atomicOr(&s_bad, SPEC_DEV_BAD_TREE);
    } else {
      if (sh.dep[t] != sh.dep[p] + 1) atomicOr(&s_bad, SPEC_DEV_BAD_TREE);
      atomicAdd(&sh.nch[p], 1);
    }
    if (sh.tok[t] < 0 || sh.tok[t] >= V) atomicOr(&s_bad, SPEC_DEV_BAD_TOKEN);
  }
  __syncthreads();
  for (int t = tid; t < T; t += kSelThreads) {
    if (sh.nch[t] == 0) continue;
    const int r = sh.row[t];
    if (r < 0 || r >= A.Rr) atomicOr(&s_bad, SPEC_DEV_BAD_ROW);
  }
  __syncthreads();
  const bool bad = s_bad != 0;
  if (bad) {
    if (lead && tid == 0) raise_status(A.status, s_bad);
    T = 1;
    for (int t = tid; t < SPEC_MAX_TREE; t += kSelThreads) sh.nch[t] = 0;
    __syncthreads();
  }

  // ---------------------------------------------------------------- row scans
  // Nodes sh.scan_node[i0 .. i0 + nn): target rows, and with_q their draft
  // rows; the merged statistics land in m_p / arg_p / S_p (and m_q / S_q).
  auto scan_nodes = [&](int i0, int nn, bool with_q) {
    const int nr = with_q ? 2 * nn : nn;
    auto row_of = [&](int i) -> const float* {
      const int node = sh.scan_node[i0 + (with_q ? (i >> 1) : i)];
      if (with_q && (i & 1)) return A.dft + ((size_t)b * A.Rr + sh.row[node]) * V;
      return A.tgt + (nb + node) * V;
    };
    scan_rows<VEC>(nr, row_of, lo, n, sh);
    __syncthreads();
    if (tid < nr) {
      const uint64_t sb = (uint64_t)__double_as_longlong(sh.sc_S[tid]);
      sh.xw_mine[4 * tid] = __float_as_uint(sh.sc_m[tid]);
      sh.xw_mine[4 * tid + 1] = (uint32_t)sh.sc_a[tid];
      sh.xw_mine[4 * tid + 2] = (uint32_t)sb;
      sh.xw_mine[4 * tid + 3] = (uint32_t)(sb >> 32);
    }
    const int nw = 4 * nr;
    sy.exchange_words(sh.xw_mine, nw, sh.xw_all);
    if (tid < nr) {
      // merge the P slices in workgroup order (ascending vocabulary)
      float M = -INFINITY;
      int Aa = 0x7fffffff;
      for (int k = 0; k < P; ++k)
        argmax_merge(M, Aa, __uint_as_float(sh.xw_all[k * nw + 4 * tid]),
                     (int)sh.xw_all[k * nw + 4 * tid + 1]);
      double S = 0.0;
      for (int k = 0; k < P; ++k) {
        const float mk = __uint_as_float(sh.xw_all[k * nw + 4 * tid]);
        const uint64_t sb = ((uint64_t)sh.xw_all[k * nw + 4 * tid + 3] << 32) |
                            sh.xw_all[k * nw + 4 * tid + 2];
        if (mk != -INFINITY) S += __longlong_as_double((long long)sb) * exp((double)mk - (double)M);
      }
      const int node = sh.scan_node[i0 + (with_q ? (tid >> 1) : tid)];
      if (with_q && (tid & 1)) {
        sh.m_q[node] = M;
        sh.S_q[node] = S;
      } else {
        sh.m_p[node] = M;
        sh.arg_p[node] = Aa;
        sh.S_p[node] = S;
      }
    }
    __syncthreads();
  };
  // p and q of the own token of every child of the nodes in the batch, from
  // logits gathered before the scan (fp64 exp, merged sums)
  auto child_of_batch = [&](int t, int i0, int nn) {
    if (t < 1 || t >= T) return false;
    const int p = sh.par[t];
    for (int i = 0; i < nn; ++i)
      if (sh.scan_node[i0 + i] == p) return true;
    return false;
  };

  RowPair rp{};
  RowCache rc;
  cache_range(rc, V, sy);
  int stop = 0, draw_k = -1;
  bool cached = false;

  if (MODE == SPEC_REJECT_PATH) {
    // ------------------------------------------------------------ per-path walk
    if (tid == 0) {
      sh.front[0] = 0;
      sh.n_front = 1;
    }
    __syncthreads();
    int d = 0;
    while (sh.n_front > 0) {
      const int nf = sh.n_front;
      stop = sh.front[0];  // the lowest-index survivor of this depth
      if (tid == 0) {
        int c = 0;
        for (int i = 0; i < nf; ++i)
          if (sh.nch[sh.front[i]] > 0) sh.scan_node[c++] = sh.front[i];
        sh.n_scan = c;
      }
      __syncthreads();
      const int ns = sh.n_scan;
      for (int i0 = 0; i0 < ns; i0 += kScanRows / 2) {
        const int nn = min(kScanRows / 2, ns - i0);
        const bool mine = child_of_batch(tid, i0, nn);
        double lp_own = 0.0, lq_own = 0.0;
        if (mine) {
          const int sp = sh.par[tid], x = sh.tok[tid];
          lp_own = A.tgt[(nb + sp) * V + x];
          lq_own = A.dft[((size_t)b * A.Rr + sh.row[sp]) * V + x];
        }
        scan_nodes(i0, nn, true);
        if (mine) {
          const int t = tid, sp = sh.par[t];
          const double p = exp(lp_own - (double)sh.m_p[sp]) / sh.S_p[sp];
          const double q = exp(lq_own - (double)sh.m_q[sp]) / sh.S_q[sp];
          sh.pt[t] = p;
          sh.qt[t] = q;
          const double ratio = q > 0.0 ? p / q : (p > 0.0 ? INFINITY : 0.0);
          const double u = (double)sh.u[t];
          sh.dec[t] = u < ratio;
          if (fabs(ratio - u) < kNearTie) atomicAdd(&sh.near_count, 1);
        }
        __syncthreads();
      }
      // next frontier: the accepted children of this depth, in node order
      if (tid < kWave) {
        const int t0 = tid, t1 = tid + kWave;
        const bool a0 = t0 >= 1 && t0 < T && sh.dep[t0] == d + 1 && sh.dec[t0] == 1;
        const bool a1 = t1 < T && sh.dep[t1] == d + 1 && sh.dec[t1] == 1;
        const uint64_t m0 = __ballot(a0), m1 = __ballot(a1);
        const uint64_t below = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
        const int n0 = __popcll(m0);
        if (a0) sh.front[__popcll(m0 & below)] = t0;
        if (a1) sh.front[n0 + __popcll(m1 & below)] = t1;
        if (tid == 0) sh.n_front = n0 + __popcll(m1);
      }
      __syncthreads();
      ++d;
    }
    if (!bad && sh.nch[stop] > 0) {
      // every child of the stop node was rejected: norm(max(0, p_s - q_s)),
      // from the rows its frontier scan read
      rp.lp = A.tgt + (nb + stop) * V;
      rp.mp = sh.m_p[stop];
      rp.lq = A.dft + ((size_t)b * A.Rr + sh.row[stop]) * V;
      rp.mq = sh.m_q[stop];
      if (A.cache) {
        cache_load(rc, rp, true, true, sy, sh);
        cached = true;
      } else {
        pass_normalisers(rp, true, sy, sh, V);
      }
      draw_k = 0;
    }
  } else {
    // ------------------------------------------------------------ sequential walk
    int s = 0;
    while (!bad) {
      if (sh.nch[s] > 0) {
        if (tid == 0) sh.scan_node[0] = s;
        __syncthreads();
        const bool mine = tid >= 1 && tid < T && sh.par[tid] == s;
        double lp_own = 0.0, lq_own = 0.0;
        if (mine) {
          lp_own = A.tgt[(nb + s) * V + sh.tok[tid]];
          lq_own = A.dft[((size_t)b * A.Rr + sh.row[s]) * V + sh.tok[tid]];
        }
        scan_nodes(0, 1, true);
        if (mine) {
          sh.pt[tid] = exp(lp_own - (double)sh.m_p[s]) / sh.S_p[s];
          sh.qt[tid] = exp(lq_own - (double)sh.m_q[s]) / sh.S_q[s];
        }
        __syncthreads();
      }
      int next_s = s;
      if (test_children_seq(A, nb, s, T, rp, rc, sy, sh, draw_k, cached, next_s)) {
        s = next_s;
        continue;
      }
      stop = s;
      break;
    }
  }
  if (bad || sh.nch[stop] == 0) {
    // a stop node without children (or a bad sequence's root): its target row
    if (tid == 0) sh.scan_node[0] = stop;
    __syncthreads();
    scan_nodes(0, 1, false);
    draw_k = -1;
    cached = false;
  }

  // ---------------------------------------------------------------- final token
  int next = 0, cdf_near = 0;
  const bool have_next = final_token(false, A, nb, stop, bad, draw_k, cached, rp, rc, sy, sh,
                                     lead, next, cdf_near);

  // ---------------------------------------------------------------- outputs
  const int near_total = sh.near_count + cdf_near;
  if (have_next && tid == 0) {
    A.next_token[b] = next;
    if (A.near_tie) A.near_tie[b] = near_total;
  }
  if (!lead) return;
  if (tid == 0) A.acc_len[b] = sh.dep[stop];
  for (int t = tid; t < T_cap; t += kSelThreads) {
    int pv = -1;
    if (!bad && t <= sh.dep[stop]) {
      int cur = stop;
      while (sh.dep[cur] > t) cur = sh.par[cur];
      pv = cur;
    }
    if (bad && t == 0) pv = 0;
    A.acc_path[nb + t] = pv;
    if (A.decision) A.decision[nb + t] = (int8_t)((t < T && !bad) ? sh.dec[t] : -1);
    // only tested nodes carry p and q (a sequential walk gathers them for
    // every child of a node it reads, also those after the accepted one)
    const bool tested = t < T && !bad && sh.dec[t] >= 0;
    if (A.p_tok) A.p_tok[nb + t] = tested ? (float)sh.pt[t] : 0.0f;
    if (A.q_tok) A.q_tok[nb + t] = tested ? (float)sh.qt[t] : 0.0f;
  }
}

// Largest P with B * P co-resident select workgroups (the occupancy of the
// mode's own kernel), at most kMaxP, and at least 2048 vocabulary entries per
// workgroup.
int choose_p(int mode, int B, int V) {
  if (mode == SPEC_GREEDY) return 1;
  thread_local int cached_capacity[2] = {-1, -1};  // per host thread: no shared state
  thread_local int cached_device[2] = {-1, -1};
  const int slot = mode == SPEC_REJECT_PATH ? 0 : 1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (cached_device[slot] != dev) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 1;
    const void* fn = slot == 0 ? reinterpret_cast<const void*>(k_vselect<SPEC_REJECT_PATH>)
                               : reinterpret_cast<const void*>(k_vselect<SPEC_REJECT_RECURSIVE>);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kSelThreads, 0) != hipSuccess)
      return 1;
    cached_capacity[slot] = cus * per_cu;
    cached_device[slot] = dev;
  }
  int P = cached_capacity[slot] / (B > 0 ? B : 1);
  const int by_v = V / 2048;
  if (P > by_v) P = by_v;
  if (P > kMaxP) P = kMaxP;
  if (P < 1) P = 1;
  return P;
}

// Largest P with B * P co-resident walk workgroups, at most kMaxP, and at
// least 2048 vocabulary entries per workgroup.
// (per walk kernel: the two modes differ in registers and so in occupancy)
int choose_walk_p(int B, int V, const void* fn) {
  thread_local const void* cached_fn[2] = {nullptr, nullptr};
  thread_local int cached_capacity[2] = {-1, -1};  // per host thread: no shared state
  thread_local int cached_device[2] = {-1, -1};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  int slot = cached_fn[0] == fn ? 0 : (cached_fn[1] == fn ? 1 : -1);
  if (slot < 0 || cached_device[slot] != dev) {
    if (slot < 0) slot = cached_fn[0] == nullptr ? 0 : 1;
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kSelThreads, 0) != hipSuccess)
      return 1;
    cached_fn[slot] = fn;
    cached_capacity[slot] = cus * per_cu;
    cached_device[slot] = dev;
  }
  int P = cached_capacity[slot] / (B > 0 ? B : 1);
  if (P > walk_p_bound(V)) P = walk_p_bound(V);
  if (P < 1) P = 1;
  return P;
}

int launch_reject_walk(int mode, SelArgs A, hipStream_t s) {
  // 16-byte chunk offsets of a row slice must fit the 32-bit buffer range
  if ((long long)A.V * 4 > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  const bool vec = (A.V % 4 == 0) && aligned(A.tgt, 16) && aligned(A.dft, 16);
  const void* fn;
  if (mode == SPEC_REJECT_PATH_WALK)
    fn = vec ? reinterpret_cast<const void*>(k_vrwalk<SPEC_REJECT_PATH, true>)
             : reinterpret_cast<const void*>(k_vrwalk<SPEC_REJECT_PATH, false>);
  else
    fn = vec ? reinterpret_cast<const void*>(k_vrwalk<SPEC_REJECT_RECURSIVE, true>)
             : reinterpret_cast<const void*>(k_vrwalk<SPEC_REJECT_RECURSIVE, false>);
  A.P = choose_walk_p(A.B, A.V, fn);
  int slice = (A.V + A.P - 1) / A.P;
  A.slice = (slice + 3) & ~3;  // slices start on 16-byte boundaries of 16-byte-aligned rows
  {
    const int cslice = (A.V + A.P - 1) / A.P;  // the draw's slicing (slice_of)
    A.cache = (cslice + kSelThreads - 1) / kSelThreads <= kCacheE ? 1 : 0;
  }
  // a new tag base for every call (bits 12..31, never 0): exchange words left
  // by an earlier call never match this call's tags
  static std::atomic<uint32_t> calls{0};
  uint32_t e = (calls.fetch_add(1, std::memory_order_relaxed) + 1) & 0xfffffu;
  if (e == 0) e = 1;
  A.tag_base = e << 12;
  void* args[] = {&A};
  const dim3 grid((unsigned)(A.B * A.P));
  hipError_t err;
  if (A.P > 1)
    err = launch_meeting_kernel(fn, grid, dim3(kSelThreads), args, s);
  else
    err = hipLaunchKernel(fn, grid, dim3(kSelThreads), args, 0, s);
  return err == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

template <int EPT>
void launch_stats(const VerifyPlan& pl, bool vec, int B, int T_cap, int V, int Rr,
                  const float* tgt, const float* dft, const int32_t* n_nodes,
                  const int32_t* parent, const int32_t* dft_row, Partial* part,
                  unsigned char* sync, hipStream_t s) {
  const dim3 grid((unsigned)(pl.n_units * pl.n_chunks));
  if (vec)
    hipLaunchKernelGGL((k_vstats<EPT, true>), grid, dim3(kStatThreads), 0, s, B, T_cap, V, Rr,
                       pl.n_chunks, tgt, dft, n_nodes, parent, dft_row, part, sync);
  else
    hipLaunchKernelGGL((k_vstats<EPT, false>), grid, dim3(kStatThreads), 0, s, B, T_cap, V, Rr,
                       pl.n_chunks, tgt, dft, n_nodes, parent, dft_row, part, sync);
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_verify_workspace_size(int mode, int B, int T_cap, int V, int R) {
  if (mode == SPEC_GREEDY_WALK && B >= 1) return verify_walk_workspace_size(B);
  if ((mode == SPEC_REJECT_PATH_WALK || mode == SPEC_REJECT_RECURSIVE_WALK) && B >= 1 &&
      T_cap >= 1 && V >= 1)
    return (size_t)B * walk_stride(V);
  if (mode < SPEC_GREEDY || mode > SPEC_REJECT_RECURSIVE || B < 1 || T_cap < 1 || V < 1)
    return 0;
  const VerifyPlan pl = make_plan(mode, B, T_cap, V, R);
  return pl.n_chunks > kMergeEntries ? 0 : pl.total;
}

extern "C" int spec_verify(int mode, int B, int T_cap, int V, int R, const float* tgt,
                           const float* dft, const int32_t* dft_row, const int32_t* n_nodes,
                           const int32_t* parent, const int32_t* token, const int32_t* depth,
                           const float* u_node, const float* u_final, int32_t* acc_len,
                           int32_t* acc_path, int32_t* next_token, float* p_tok, float* q_tok,
                           int8_t* decision, int32_t* near_tie, void* ws, size_t ws_bytes,
                           int32_t* status, void* stream) {
  if (mode < SPEC_GREEDY || mode > SPEC_REJECT_RECURSIVE_WALK) return SPEC_ERR_INVALID;
  if (B < 0 || T_cap < 1 || V < 1 || R < 0) return SPEC_ERR_INVALID;
  if (T_cap > SPEC_MAX_TREE) return SPEC_ERR_CAPACITY;
  if (B == 0) return SPEC_OK;
  if (!tgt || !n_nodes || !parent || !token || !depth || !acc_len || !acc_path || !next_token)
    return SPEC_ERR_INVALID;
  status = status_or_library(status);
  if (mode == SPEC_REJECT_PATH_WALK || mode == SPEC_REJECT_RECURSIVE_WALK) {
    if (!dft || !dft_row || R < 1 || !u_node || !u_final) return SPEC_ERR_INVALID;
    if (!ws || ws_bytes < (size_t)B * walk_stride(V) || !aligned(ws, 256)) return SPEC_ERR_WORKSPACE;
    SelArgs A{};
    A.B = B;
    A.T_cap = T_cap;
    A.V = V;
    A.Rr = R;
    A.tgt = tgt;
    A.dft = dft;
    A.dft_row = dft_row;
    A.n_nodes = n_nodes;
    A.parent = parent;
    A.token = token;
    A.depth = depth;
    A.u_node = u_node;
    A.u_final = u_final;
    A.sync = static_cast<unsigned char*>(ws);
    A.acc_len = acc_len;
    A.acc_path = acc_path;
    A.next_token = next_token;
    A.p_tok = p_tok;
    A.q_tok = q_tok;
    A.decision = decision;
    A.near_tie = near_tie;
    A.status = status;
    return launch_reject_walk(mode, A, as_stream(stream));
  }
  if (mode == SPEC_GREEDY_WALK)
    return launch_verify_walk(B, T_cap, V, tgt, n_nodes, parent, token, depth, acc_len,
                              acc_path, next_token, p_tok, q_tok, decision, near_tie, ws,
                              ws_bytes, status, as_stream(stream));
  if (mode != SPEC_GREEDY) {
    if (!dft || !dft_row || R < 1 || !u_node || !u_final) return SPEC_ERR_INVALID;
  }
  const VerifyPlan pl = make_plan(mode, B, T_cap, V, R);
  // a row's chunk partials are merged in LDS batches of kMergeEntries: a
  // vocabulary with more chunks than that (V > 64 * 256 * 1024) is refused
  if (pl.n_chunks > kMergeEntries) return SPEC_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < pl.total || !aligned(ws, 256)) return SPEC_ERR_WORKSPACE;
  const int Rr = mode == SPEC_GREEDY ? 0 : R;
  char* w = static_cast<char*>(ws);
  Partial* part = reinterpret_cast<Partial*>(w + pl.off_part);
  unsigned char* sync = reinterpret_cast<unsigned char*>(w + pl.off_sync);
  hipStream_t s = as_stream(stream);

  const bool vec = (V % 4 == 0) && aligned(tgt, 16) && (Rr == 0 || aligned(dft, 16));
#define SPEC_STATS(E)                                                                       \
  launch_stats<E>(pl, vec, B, T_cap, V, Rr, tgt, dft, n_nodes, parent, dft_row, part, sync, s)
  switch (pl.ept) {
    case 64: SPEC_STATS(64); break;
    case 32: SPEC_STATS(32); break;
    case 16: SPEC_STATS(16); break;
    case 8: SPEC_STATS(8); break;
    default: SPEC_STATS(4); break;
  }
#undef SPEC_STATS
  int rc = launch_status();
  if (rc != SPEC_OK) return rc;

  SelArgs A;
  A.B = B;
  A.T_cap = T_cap;
  A.V = V;
  A.Rr = Rr;
  A.n_chunks = pl.n_chunks;
  A.P = choose_p(mode, B, V);
  {
    const int slice = (V + A.P - 1) / A.P;
    A.cache = (slice + kSelThreads - 1) / kSelThreads <= kCacheE ? 1 : 0;
  }
  A.tgt = tgt;
  A.dft = dft;
  A.dft_row = dft_row;
  A.n_nodes = n_nodes;
  A.parent = parent;
  A.token = token;
  A.depth = depth;
  A.u_node = u_node;
  A.u_final = u_final;
  A.part = part;
  A.sync = sync;
  A.acc_len = acc_len;
  A.acc_path = acc_path;
  A.next_token = next_token;
  A.p_tok = p_tok;
  A.q_tok = q_tok;
  A.decision = decision;
  A.near_tie = near_tie;
  A.status = status;
  const dim3 grid((unsigned)(B * A.P));
  const void* fn = mode == SPEC_GREEDY ? reinterpret_cast<const void*>(k_vselect<SPEC_GREEDY>)
                   : mode == SPEC_REJECT_PATH
                       ? reinterpret_cast<const void*>(k_vselect<SPEC_REJECT_PATH>)
                       : reinterpret_cast<const void*>(k_vselect<SPEC_REJECT_RECURSIVE>);
  void* args[] = {&A};
  hipError_t e;
  if (A.P > 1)
    e = launch_meeting_kernel(fn, grid, dim3(kSelThreads), args, s);
  else
    e = hipLaunchKernel(fn, grid, dim3(kSelThreads), args, 0, s);
  return e == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

// ------------------------------------------------------------------ no-allocation variant
// spec_verify for callers that cannot allocate (code under stream capture,
// tight serving loops): the workspace is a file-scope device array of
// kNoAllocScratchBytes, one per device, held until the process ends.  Host
// code never passes the array's name to a kernel (on the host it only stands
// for the symbol): its device address is looked up once per device with that
// device current and kept.

namespace {
constexpr size_t kNoAllocScratchBytes = 4u << 20;  // every mode of every workload above fits
constexpr int kNoAllocMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];

// Device address of `scratch` on the current device (nullptr on failure).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int spec_verify_noalloc(int mode, int B, int T_cap, int V, int R, const float* tgt,
                                   const float* dft, const int32_t* dft_row,
                                   const int32_t* n_nodes, const int32_t* parent,
                                   const int32_t* token, const int32_t* depth,
                                   const float* u_node, const float* u_final, int32_t* acc_len,
                                   int32_t* acc_path, int32_t* next_token, float* p_tok,
                                   float* q_tok, int8_t* decision, int32_t* near_tie,
                                   int32_t* status, void* stream) {
  if (mode < SPEC_GREEDY || mode > SPEC_REJECT_RECURSIVE_WALK) return SPEC_ERR_INVALID;
  if (B < 0 || T_cap < 1 || V < 1 || R < 0) return SPEC_ERR_INVALID;
  if (T_cap > SPEC_MAX_TREE) return SPEC_ERR_CAPACITY;
  if (B == 0) return SPEC_OK;
  const size_t need = spec_verify_workspace_size(mode, B, T_cap, V, R);
  if (need == 0) return SPEC_ERR_UNSUPPORTED;  // a vocabulary beyond the row merge
  if (need > kNoAllocScratchBytes) return SPEC_ERR_CAPACITY;
  void* ws = scratch_on_current_device();
  if (!ws) return SPEC_ERR_HIP;
  // no mode needs initial workspace contents: whatever the previous call on
  // this device left in the array is overwritten before it is read
  return spec_verify(mode, B, T_cap, V, R, tgt, dft, dft_row, n_nodes, parent, token, depth,
                     u_node, u_final, acc_len, acc_path, next_token, p_tok, q_tok, decision,
                     near_tie, ws, kNoAllocScratchBytes, status, stream);
}
