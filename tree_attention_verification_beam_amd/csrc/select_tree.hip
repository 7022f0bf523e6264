// select_tree.hip -- dynamic draft-tree selection under a node budget.
//
// "Speculative Decoding, Part 2: A History of Drafters", the EAGLE-2
// paragraph: a branch is scored by the product of the drafter's confidences
// along its path from the root and the highest-scoring branches are kept; a
// parent always scores at least as high as its children, so the kept set
// holds its parents.  "Clover: Regressive Lightweight Speculative Decoding
// with Sequential Knowledge" sizes its tree by a node budget.  In log form the
// path score is S(root) = 0, S(node) = S(parent) + logp(node), an fp32 sum
// taken from the root down; the N_keep candidates with the highest S are kept
// (the lower index on ties) and leave as an explicit candidate list for
// spec_build_tree, renumbered in their original order.
//
// k_select_tree: one workgroup per sequence, everything in LDS.  Scores are
// computed level by level (a node is summed in the round after its parent),
// so each sum happens in the same order as the definition; the rank of a node
// is the number of nodes ahead of it (one 64-bit key per node, read from LDS
// two at a time, one compare each);
// kept nodes are numbered by a ballot scan in node order.
#include "common.hpp"

namespace spec {
namespace {

constexpr int kSelTreeThreads = 256;
constexpr int kSelTreeWaves = kSelTreeThreads / kWave;
constexpr int kPerThread = SPEC_MAX_SELECT / kSelTreeThreads;  // candidates per thread

__global__ __launch_bounds__(kSelTreeThreads) void k_select_tree(
    int N, int N_keep, const int32_t* __restrict__ cand_parent,
    const int32_t* __restrict__ cand_token, const float* __restrict__ cand_logp,
    int32_t* __restrict__ keep_parent, int32_t* __restrict__ keep_token,
    int32_t* __restrict__ keep_src, float* __restrict__ keep_score, int32_t* status) {
  __shared__ float s_S[SPEC_MAX_SELECT + 1];    // path score of node n (node 0 = root)
  __shared__ __align__(16) uint64_t s_K[SPEC_MAX_SELECT];  // rank key of candidate u, 0 padded
  __shared__ int s_round[SPEC_MAX_SELECT + 1];  // round in which node n was scored, -1 not yet
  __shared__ int s_par[SPEC_MAX_SELECT];
  __shared__ int s_new[SPEC_MAX_SELECT];        // new node number of candidate i (0: dropped)
  __shared__ int s_wsum[kSelTreeWaves];
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (size_t)b * N;

  int par[kPerThread];
  float lp[kPerThread];
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int i = r * kSelTreeThreads + tid;
    par[r] = i < N ? cand_parent[base + i] : 0;
    lp[r] = i < N ? cand_logp[base + i] : 0.0f;
  }
  if (tid == 0) {
    s_bad = 0;
    s_S[0] = 0.0f;
    s_round[0] = 0;
  }
#pragma unroll
  for (int r = 0; r < kPerThread; ++r) {
    const int i = r * kSelTreeThreads + tid;
    if (i < N) {
      s_par[i] = par[r];
      s_round[i + 1] = -1;
      if (par[r] < 0 || par[r] > i || !(lp[r] <= 0.0f)) atomicOr(&s_bad, 1);
    }
  }
  __syncthreads();
  const bool bad = s_bad != 0;

  if (!bad) {
    // ---------------------------------------------------------------- scores
    // round q scores the nodes whose parent was scored in an earlier round
    for (int q = 1;; ++q) {
      int left = 0;
#pragma unroll
      for (int r = 0; r < kPerThread; ++r) {
        const int i = r * kSelTreeThreads + tid;
        if (i < N && s_round[i + 1] < 0) {
          const int pr = s_round[par[r]];
          if (pr >= 0 && pr < q) {
            s_S[i + 1] = s_S[par[r]] + lp[r];
            s_round[i + 1] = q;
          } else {
            left = 1;
          }
        }
      }
      if (!__syncthreads_or(left)) break;
    }

    // ---------------------------------------------------------------- rank
    // one 64-bit key per candidate, larger = ahead: the score's bits in an
    // unsigned order above the complement of the index (a lower index wins a
    // tie); -0.0 ranks as +0.0.  Zero pads the copy to a multiple of 8, and a
    // zero key is never ahead.
    const int n_pad = (N + 7) & ~7;
    for (int u = tid; u < n_pad; u += kSelTreeThreads) {
      uint64_t key = 0;
      if (u < N) {
        uint32_t bits = __float_as_uint(s_S[u + 1]);
        if (bits == 0x80000000u) bits = 0;
        const uint32_t o = (bits & 0x80000000u) ? ~bits : (bits | 0x80000000u);
        key = ((uint64_t)o << 32) | (uint64_t)(~(uint32_t)u);
      }
      s_K[u] = key;
    }
    __syncthreads();
    bool keep[kPerThread];
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int i = r * kSelTreeThreads + tid;
      keep[r] = false;
      if (i < N) {
        const uint64_t ki = s_K[i];
        int ahead = 0;
        for (int u0 = 0; u0 < n_pad; u0 += 8) {
          uint64_t c[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const auto two = *reinterpret_cast<const u32x4*>(s_K + u0 + 2 * q);
            c[2 * q] = ((uint64_t)two[1] << 32) | two[0];
            c[2 * q + 1] = ((uint64_t)two[3] << 32) | two[2];
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) ahead += c[e] > ki ? 1 : 0;
        }
        keep[r] = ahead < N_keep;
      }
    }

    // ---------------------------------------------------------------- number
    // kept candidates in index order i = r * 256 + tid: a ballot scan per block
    int running = 0;
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const uint64_t m = __ballot(keep[r]);
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      if (lane == 0) s_wsum[wave] = __popcll(m);
      __syncthreads();
      int before = running;
      for (int w2 = 0; w2 < wave; ++w2) before += s_wsum[w2];
      int total = 0;
      for (int w2 = 0; w2 < kSelTreeWaves; ++w2) total += s_wsum[w2];
      const int i = r * kSelTreeThreads + tid;
      if (i < N) s_new[i] = keep[r] ? before + __popcll(m & below) + 1 : 0;
      running += total;
      __syncthreads();
    }

    // ---------------------------------------------------------------- write
#pragma unroll
    for (int r = 0; r < kPerThread; ++r) {
      const int i = r * kSelTreeThreads + tid;
      if (i < N && keep[r]) {
        const int k = s_new[i] - 1;
        const int p = par[r];
        const int np = p == 0 ? 0 : s_new[p - 1];
        if (p > 0 && np == 0) atomicOr(&s_bad, 2);  // a dropped parent (not for logp <= 0)
        keep_parent[(size_t)b * N_keep + k] = np;
        keep_token[(size_t)b * N_keep + k] = cand_token[base + i];
        if (keep_src) keep_src[(size_t)b * N_keep + k] = i;
        if (keep_score) keep_score[(size_t)b * N_keep + k] = s_S[i + 1];
      }
    }
    __syncthreads();
  }
  if (s_bad) {
    // invalid input: parents that spec_build_tree rejects as not topological
    for (int k = tid; k < N_keep; k += kSelTreeThreads) {
      keep_parent[(size_t)b * N_keep + k] = -1;
      keep_token[(size_t)b * N_keep + k] = 0;
      if (keep_src) keep_src[(size_t)b * N_keep + k] = -1;
      if (keep_score) keep_score[(size_t)b * N_keep + k] = -INFINITY;
    }
    if (tid == 0) raise_status(status, SPEC_DEV_BAD_PARENT);
  }
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" int spec_select_tree(int B, int N, int N_keep, const int32_t* cand_parent,
                                const int32_t* cand_token, const float* cand_logp,
                                int32_t* keep_parent, int32_t* keep_token, int32_t* keep_src,
                                float* keep_score, int32_t* status, void* stream) {
  if (B < 0 || N < 1 || N_keep < 1 || N_keep > N) return SPEC_ERR_INVALID;
  if (N > SPEC_MAX_SELECT || N_keep > SPEC_MAX_TREE - 1) return SPEC_ERR_CAPACITY;
  if (B == 0) return SPEC_OK;
  if (!cand_parent || !cand_token || !cand_logp || !keep_parent || !keep_token)
    return SPEC_ERR_INVALID;
  status = status_or_library(status);
  hipLaunchKernelGGL(k_select_tree, dim3(B), dim3(kSelTreeThreads), 0, as_stream(stream), N,
                     N_keep, cand_parent, cand_token, cand_logp, keep_parent, keep_token,
                     keep_src, keep_score, status);
  return launch_status();
}
