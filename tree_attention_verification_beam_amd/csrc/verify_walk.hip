// verify_walk.hip -- greedy verification that reads only the rows it needs.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 5 (token matches): a node
// is accepted when its token is the target's greedy token after its parent,
// and the deepest node whose whole path is accepted wins.  Only the target
// rows of nodes whose path is accepted so far can change that answer, so the
// tree is walked depth by depth: the frontier starts at the root; each frontier
// node's row is scanned once for (max, argmax with the lowest index on ties,
// sum exp(l - max)); its children are tested against the argmax; the accepted
// ones form the next frontier.  The stop node is the lowest-index node of the
// deepest non-empty frontier and the next token is its greedy token.  A tree
// whose draft tokens rarely match reads one row per sequence instead of one per
// node.
//
// k_vwalk: P workgroups per sequence split every scanned row into P slices (a
// single CU streams only some 20 GB/s from HBM, so one row needs many CUs).
// Each scan ends in a meeting of the P workgroups: each publishes its slice's
// (max, argmax, sum) as four 64-bit words, 32 bits of payload beside a 32-bit
// tag made of the call's epoch (a host counter, new for every call) and the
// meeting's number, and one wave then polls the 4P words of the meeting until
// every tag matches; every workgroup combines the P entries in the same order
// and takes the same decisions.  Entries of meeting r sit in parity r & 1:
// meeting r + 2 overwrites them only after all P workgroups have published
// meeting r + 1, i.e. after every reader is done with meeting r.  Words left
// by an earlier call, even one that ended at a wait bound with late
// workgroups still publishing, carry another epoch and never match, so the
// workspace needs no initial contents and no reset.  The grid is sized to be
// resident at once (occupancy query) and every wait is bounded.
//
// A slice scan keeps two batches of 16-byte buffer loads in flight; loads past
// the slice end return zeros and are masked to -inf.  The logits of the tested
// children's own tokens are gathered while the row streams, for p_tok.
#include <atomic>

#include "common.hpp"

namespace spec {

int launch_verify_walk(int B, int T_cap, int V, const float* tgt, const int32_t* n_nodes,
                       const int32_t* parent, const int32_t* token, const int32_t* depth,
                       int32_t* acc_len, int32_t* acc_path, int32_t* next_token, float* p_tok,
                       float* q_tok, int8_t* decision, int32_t* near_tie, void* ws,
                       size_t ws_bytes, int32_t* status, hipStream_t s);
size_t verify_walk_workspace_size(int B);

namespace {

constexpr int kWalkThreads = 256;
constexpr int kWalkWaves = kWalkThreads / kWave;
constexpr int kWalkMaxP = 32;
constexpr int kBatch = 4;  // 16-byte loads per thread per batch (two batches in flight)
constexpr float kLog2eW = 1.4426950408889634f;
constexpr int kBufWord3 = 0x00020000;  // buffer resource word 3, raw 32-bit loads
// per sequence: [2 parities][P][4] tagged entry words
constexpr size_t kWalkStride = 2 * kWalkMaxP * 4 * 8;

struct WalkArgs {
  int B, T_cap, V, P, slice;  // slice: vocabulary entries per workgroup (multiple of 4)
  uint32_t epoch;             // this call's tag base (bits 8..31), never 0
  const float* tgt;
  const int32_t* n_nodes;
  const int32_t* parent;
  const int32_t* token;
  const int32_t* depth;
  int32_t* acc_len;
  int32_t* acc_path;
  int32_t* next_token;
  float* p_tok;
  float* q_tok;
  int8_t* decision;
  int32_t* near_tie;
  unsigned char* ws;
  int32_t* status;
};

struct WalkShared {
  int par[SPEC_MAX_TREE], tok[SPEC_MAX_TREE], dep[SPEC_MAX_TREE];
  int dec[SPEC_MAX_TREE];
  float pt[SPEC_MAX_TREE];
  int greedy[SPEC_MAX_TREE];
  int front[SPEC_MAX_TREE];
  int n_front, bad, stop;
  float wm[kWalkWaves];
  int wa[kWalkWaves];
  double ws[kWalkWaves];
  float M;
  int arg;
  double S;
  uint32_t xw[2 * kWave];  // a meeting's entry words
};

// Fold 4 logits (slice positions pos .. pos+3, those >= n masked) into a running
// (max m, lowest argmax a) in vocabulary indices base + pos.
__device__ inline void fold4(const f32x4& v, int pos, int n, int base, float& m, int& a) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float l = pos + e < n ? v[e] : -INFINITY;
    if (l > m) {
      m = l;
      a = base + pos + e;
    }
  }
}

struct SliceLoads {
  f32x4 b0[kBatch], b1[kBatch];
};

__device__ inline __amdgpu_buffer_rsrc_t slice_rsrc(const float* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), (short)0, n * 4, kBufWord3);
}

__device__ inline void load_batch(__amdgpu_buffer_rsrc_t rs, f32x4 (&buf)[kBatch], int j0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < kBatch; ++j)
    buf[j] = __builtin_bit_cast(
        f32x4,
        __builtin_amdgcn_raw_buffer_load_b128(rs, ((j0 + j) * kWalkThreads + tid) * 16, 0, kLoadOnce));
}

// First two batches of a slice's loads (16-byte path); callers overlap them
// with other loads.
template <bool VEC>
__device__ inline void slice_issue(__amdgpu_buffer_rsrc_t rs, SliceLoads& L) {
  if constexpr (VEC) {
    load_batch(rs, L.b0, 0);  // past the slice: zero-range loads, masked when folded
    load_batch(rs, L.b1, kBatch);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The slice [base, base + n) of a row: (max, lowest argmax, sum exp(l - max))
// of this workgroup into sh.M, sh.arg, sh.S.  Thread j owns 16-byte chunks j,
// j + 256, ...; within a thread positions rise and a strict > keeps the lowest
// index among equal values.  Exponentials in fp32 (exp2 form), sums in fp64.
template <bool VEC>
__device__ void slice_finish(const float* row, int base, int n, __amdgpu_buffer_rsrc_t rs,
                             SliceLoads& L, WalkShared& sh) {
  const int tid = threadIdx.x;
  float m = -INFINITY;
  int a = 0x7fffffff;
  double S = 0.0;
  if constexpr (VEC) {
    const int n_per = ((n >> 2) + kWalkThreads - 1) / kWalkThreads;  // chunks per thread
    auto fold = [&](const f32x4 (&buf)[kBatch], int j0) {
      float bm = -INFINITY;
      int ba = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
        fold4(buf[j], ((j0 + j) * kWalkThreads + tid) * 4, n, base, bm, ba);
      if (bm == -INFINITY) return;
      if (bm > m) {
        S = m == -INFINITY ? 0.0 : S * (double)__builtin_amdgcn_exp2f((m - bm) * kLog2eW);
        m = bm;
        a = ba;
      }
      float s = 0.0f;
#pragma unroll
      for (int j = 0; j < kBatch; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int pos = ((j0 + j) * kWalkThreads + tid) * 4 + e;
          s += pos < n ? __builtin_amdgcn_exp2f((buf[j][e] - m) * kLog2eW) : 0.0f;
        }
      S += (double)s;
    };
    for (int j0 = 0; j0 < n_per; j0 += 2 * kBatch) {
      fold(L.b0, j0);
      if (j0 + 2 * kBatch < n_per) load_batch(rs, L.b0, j0 + 2 * kBatch);
      __builtin_amdgcn_sched_barrier(0);
      if (j0 + kBatch < n_per) fold(L.b1, j0 + kBatch);
      if (j0 + 3 * kBatch < n_per) load_batch(rs, L.b1, j0 + 3 * kBatch);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    for (int i = tid; i < n; i += kWalkThreads) {
      const float l = row[base + i];
      if (l > m) {
        S = m == -INFINITY ? 0.0 : S * (double)__builtin_amdgcn_exp2f((m - l) * kLog2eW);
        m = l;
        a = base + i;
      }
      if (l != -INFINITY) S += (double)__builtin_amdgcn_exp2f((l - m) * kLog2eW);
    }
  }
  // workgroup (max, lowest argmax), then the sum rescaled to the common max
  float wm = m;
  int wa = a;
  wave_argmax(wm, wa);
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) {
    sh.wm[wave] = wm;
    sh.wa[wave] = wa;
  }
  __syncthreads();
  if (tid < kWave) {
    float M = tid < kWalkWaves ? sh.wm[tid] : -INFINITY;
    int A = tid < kWalkWaves ? sh.wa[tid] : 0x7fffffff;
    wave_argmax(M, A);
    if (tid == 0) {
      sh.M = M;
      sh.arg = A;
    }
  }
  __syncthreads();
  const float M = sh.M;
  double part = (m == -INFINITY || M == -INFINITY)
                    ? 0.0
                    : S * (double)__builtin_amdgcn_exp2f((m - M) * kLog2eW);
  part = wave_sum_f64(part);
  if (lane == 0) sh.ws[wave] = part;
  __syncthreads();
  if (tid < kWave) {
    double t = tid < kWalkWaves ? sh.ws[tid] : 0.0;
    t = wave_sum_f64(t);
    if (tid == 0) sh.S = t;
  }
  __syncthreads();
}

// Meeting `round` of the P workgroups of a sequence: publish this workgroup's
// (M, arg, S), wait for all P, combine them in workgroup order (the same result
// in every workgroup) into sh.M, sh.arg, sh.S.  Word k of a workgroup's entry
// holds 32 bits of its values in the low half and the tag epoch | round in the
// high half, so a word read at the coherent level with the current tag belongs
// to this meeting, whatever order the stores landed in.
__device__ void meet(uint64_t* seq, int P, int w, uint32_t epoch, int round, WalkShared& sh,
                     int32_t* status) {
  if (P == 1) return;
  uint64_t* entries = seq + (size_t)(round & 1) * kWalkMaxP * 4;
  const uint64_t tag = (uint64_t)(epoch | (uint32_t)(round & 0xff)) << 32;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    if (lane < 4) {
      const uint64_t sbits = (uint64_t)__double_as_longlong(sh.S);
      const uint32_t half = lane == 0   ? __float_as_uint(sh.M)
                            : lane == 1 ? (uint32_t)sh.arg
                            : lane == 2 ? (uint32_t)sbits
                                        : (uint32_t)(sbits >> 32);
      store_coherent(entries + 4 * w + lane, tag | half);
    }
    // the 4P words of this parity, two per lane
    const int n = 4 * P;
    uint64_t v0 = 0, v1 = 0;
    bool ok0 = lane >= n, ok1 = lane + 64 >= n;
    int spins = 0;
    while (!(ok0 && ok1)) {
      if (!ok0) {
        v0 = load_coherent(entries + lane);
        ok0 = (v0 & 0xffffffff00000000ull) == tag;
      }
      if (!ok1) {
        v1 = load_coherent(entries + lane + 64);
        ok1 = (v1 & 0xffffffff00000000ull) == tag;
      }
      if (++spins > (1 << 22)) {
        raise_status(status, SPEC_DEV_SYNC_TIMEOUT);
        break;
      }
    }
    // word 4i + k (workgroup i, word k) through LDS to lane i
    sh.xw[lane] = (uint32_t)v0;
    sh.xw[lane + 64] = (uint32_t)v1;
    __builtin_amdgcn_wave_barrier();
    float m = -INFINITY;
    int a = 0x7fffffff;
    double S = 0.0;
    if (lane < P) {
      m = __uint_as_float(sh.xw[4 * lane]);
      a = (int)sh.xw[4 * lane + 1];
      S = __longlong_as_double(
          (long long)(((uint64_t)sh.xw[4 * lane + 3] << 32) | sh.xw[4 * lane + 2]));
    }
    float M = m;
    int A = a;
    wave_argmax(M, A);
    double part = (lane < P && m != -INFINITY && M != -INFINITY)
                      ? S * (double)__builtin_amdgcn_exp2f((m - M) * kLog2eW)
                      : 0.0;
    part = wave_sum_f64(part);
    if (lane == 0) {
      sh.M = M;
      sh.arg = A;
      sh.S = part;
    }
  }
  __syncthreads();
}

template <bool VEC>
__global__ __launch_bounds__(kWalkThreads) void k_vwalk(WalkArgs A) {
  __shared__ WalkShared sh;
  const int b = blockIdx.x / A.P;
  const int w = blockIdx.x - b * A.P;
  const int tid = threadIdx.x;
  const int T_cap = A.T_cap, V = A.V, P = A.P;
  const size_t nb = (size_t)b * T_cap;
  const bool lead = w == 0;
  uint64_t* seq = reinterpret_cast<uint64_t*>(A.ws + (size_t)b * kWalkStride);
  static_assert(kWalkThreads >= SPEC_MAX_TREE, "one tree row per thread");
  // this workgroup's slice of every row
  const int base = w * A.slice;
  const int n = max(0, min(A.slice, V - base));

  // the root's row is always scanned first: its loads go out with the tree's
  SliceLoads L;
  auto rs = slice_rsrc(A.tgt + nb * V + base, n);
  slice_issue<VEC>(rs, L);
  const int T_in = A.n_nodes[b];
  int my_par = -1, my_tok = 0, my_dep = 0;
  if (tid < T_cap) {
    my_par = tid == 0 ? -1 : A.parent[nb + tid];
    my_tok = A.token[nb + tid];
    my_dep = tid == 0 ? 0 : A.depth[nb + tid];
  }
  int T = T_in < 1 ? 1 : (T_in > T_cap ? T_cap : T_in);
  if (tid < SPEC_MAX_TREE) {
    sh.dec[tid] = -1;
    sh.pt[tid] = 0.0f;
    sh.par[tid] = my_par;
    sh.tok[tid] = my_tok;
    sh.dep[tid] = my_dep;
  }
  if (tid == 0) {
    sh.bad = (T_in < 1 || T_in > T_cap) ? SPEC_DEV_BAD_TREE : 0;
    sh.front[0] = 0;
    sh.n_front = 1;
    sh.stop = 0;
  }
  __syncthreads();
  // the same validation as the one-pass select: a bad sequence accepts nothing
  // and takes the greedy token at the root
  if (tid >= 1 && tid < T) {
    const int p = sh.par[tid];
    if (p < 0 || p >= tid || sh.dep[tid] != sh.dep[p] + 1) atomicOr(&sh.bad, SPEC_DEV_BAD_TREE);
    if (sh.tok[tid] < 0 || sh.tok[tid] >= V) atomicOr(&sh.bad, SPEC_DEV_BAD_TOKEN);
  }
  __syncthreads();
  const bool bad = sh.bad != 0;
  if (bad) {
    if (lead && tid == 0) raise_status(A.status, sh.bad);
    T = 1;
  }

  // ---------------------------------------------------------------- walk
  // (uniform control flow: every bound below is read from LDS after a barrier,
  // and every workgroup of the sequence takes the same decisions)
  int round = 0;
  while (sh.n_front > 0) {
    const int n_front = sh.n_front;
    if (tid == 0) sh.stop = sh.front[0];  // lowest-index survivor of this depth
    for (int i = 0; i < n_front; ++i) {
      const int f = __builtin_amdgcn_readfirstlane(sh.front[i]);
      const float* row = A.tgt + (nb + f) * V;
      if (f != 0) {  // (the root's loads are in flight since the start)
        rs = slice_rsrc(row + base, n);
        slice_issue<VEC>(rs, L);
      }
      // the children's own logits, gathered while the row streams
      const bool child = tid >= 1 && tid < T && sh.par[tid] == f;
      const float lx = child ? row[sh.tok[tid]] : 0.0f;
      slice_finish<VEC>(row, base, n, rs, L, sh);
      meet(seq, P, w, A.epoch, round++, sh, A.status);
      if (tid == 0) sh.greedy[f] = sh.arg < V ? sh.arg : 0;  // every logit -inf: index 0
      if (child) {
        sh.dec[tid] = sh.tok[tid] == sh.arg;
        sh.pt[tid] = (float)(exp((double)lx - (double)sh.M) / sh.S);
      }
      __syncthreads();
    }
    // next frontier: the accepted children of this depth's frontier, in node
    // order (wave 0 compacts nodes t and 64 + t with ballots)
    if (tid < kWave) {
      const int d = sh.dep[sh.front[0]] + 1;
      const int t0 = tid, t1 = tid + kWave;
      const bool a0 = t0 >= 1 && t0 < T && sh.dep[t0] == d && sh.dec[t0] == 1;
      const bool a1 = t1 < T && sh.dep[t1] == d && sh.dec[t1] == 1;
      const uint64_t m0 = __ballot(a0), m1 = __ballot(a1);
      const uint64_t below = (tid == 0) ? 0ull : (~0ull >> (64 - tid));
      const int n0 = __popcll(m0);
      if (a0) sh.front[__popcll(m0 & below)] = t0;
      if (a1) sh.front[n0 + __popcll(m1 & below)] = t1;
      if (tid == 0) sh.n_front = n0 + __popcll(m1);
    }
    __syncthreads();
  }

  // ---------------------------------------------------------------- leave
  if (!lead) return;

  // ---------------------------------------------------------------- outputs
  const int stop = sh.stop;
  if (tid == 0) {
    A.acc_len[b] = sh.dep[stop];
    A.next_token[b] = sh.greedy[stop];
    if (A.near_tie) A.near_tie[b] = 0;
  }
  if (tid < T_cap) {
    const int t = tid;
    int pv = -1;
    if (t <= sh.dep[stop]) {
      int cur = stop;
      while (sh.dep[cur] > t) cur = sh.par[cur];
      pv = cur;
    }
    A.acc_path[nb + t] = pv;
    const bool live = t < T && !bad;
    if (A.decision) A.decision[nb + t] = (int8_t)(live ? sh.dec[t] : -1);
    if (A.p_tok) A.p_tok[nb + t] = live ? sh.pt[t] : 0.0f;
    if (A.q_tok) A.q_tok[nb + t] = 0.0f;
  }
}

// Largest P with B * P co-resident workgroups, at most kWalkMaxP, and at least
// 2048 vocabulary entries per workgroup.
int choose_walk_p(int B, int V) {
  thread_local int cached_capacity = -1;  // per host thread: no shared state
  thread_local int cached_device = -1;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  if (cached_device != dev) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void*>(k_vwalk<true>), kWalkThreads, 0) !=
        hipSuccess)
      return 1;
    cached_capacity = cus * per_cu;
    cached_device = dev;
  }
  int P = cached_capacity / (B > 0 ? B : 1);
  const int by_v = V / 2048;
  if (P > by_v) P = by_v;
  if (P > kWalkMaxP) P = kWalkMaxP;
  if (P < 1) P = 1;
  return P;
}

}  // namespace

size_t verify_walk_workspace_size(int B) { return (size_t)B * kWalkStride; }

int launch_verify_walk(int B, int T_cap, int V, const float* tgt, const int32_t* n_nodes,
                       const int32_t* parent, const int32_t* token, const int32_t* depth,
                       int32_t* acc_len, int32_t* acc_path, int32_t* next_token, float* p_tok,
                       float* q_tok, int8_t* decision, int32_t* near_tie, void* ws,
                       size_t ws_bytes, int32_t* status, hipStream_t s) {
  // 16-byte chunk offsets of a row must fit the 32-bit buffer range
  if ((long long)V * 4 > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < verify_walk_workspace_size(B) || !aligned(ws, 256))
    return SPEC_ERR_WORKSPACE;
  const int P = choose_walk_p(B, V);
  int slice = (V + P - 1) / P;
  slice = (slice + 3) & ~3;  // slices start on 16-byte boundaries of 16-byte-aligned rows
  // a new tag base for every call: bits 8..31 of the tag, never 0 (a
  // zero-filled workspace never matches)
  static std::atomic<uint32_t> calls{0};
  uint32_t e = (calls.fetch_add(1, std::memory_order_relaxed) + 1) & 0xffffffu;
  if (e == 0) e = 1;
  WalkArgs A{};
  A.epoch = e << 8;
  A.B = B;
  A.T_cap = T_cap;
  A.V = V;
  A.P = P;
  A.slice = slice;
  A.tgt = tgt;
  A.n_nodes = n_nodes;
  A.parent = parent;
  A.token = token;
  A.depth = depth;
  A.acc_len = acc_len;
  A.acc_path = acc_path;
  A.next_token = next_token;
  A.p_tok = p_tok;
  A.q_tok = q_tok;
  A.decision = decision;
  A.near_tie = near_tie;
  A.ws = static_cast<unsigned char*>(ws);
  A.status = status;
  const bool vec = V % 4 == 0 && aligned(tgt, 16);
  const void* fn = vec ? reinterpret_cast<const void*>(k_vwalk<true>)
                       : reinterpret_cast<const void*>(k_vwalk<false>);
  void* args[] = {&A};
  const dim3 grid((unsigned)(B * P));
  hipError_t err;
  if (P > 1)
    err = launch_meeting_kernel(fn, grid, dim3(kWalkThreads), args, s);
  else
    err = hipLaunchKernel(fn, grid, dim3(kWalkThreads), args, 0, s);
  return err == hipSuccess ? SPEC_OK : SPEC_ERR_HIP;
}

}  // namespace spec
