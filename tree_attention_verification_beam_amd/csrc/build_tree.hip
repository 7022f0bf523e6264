// build_tree.hip -- pack draft candidates into a token tree on the GPU.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "Dynamic Tree Attention": candidates of equal length share prefixes;
// the packed beam keeps each distinct prefix once and the tree mask lets a token
// see only its own prefix.  That section builds the packed beam from tensor
// operations instead of pointer-chasing trie inserts; this kernel does the same
// with one thread per candidate token: each thread finds the smallest candidate
// sharing its prefix, a block scan numbers the first appearances in beam-major
// order, and every node writes its parent, depth and ancestor mask.
//
// One workgroup of SPEC_MAX_TREE threads per sequence; everything lives in LDS.
// The prefix test is split in two data-parallel passes so that no thread walks
// a chain of dependent LDS reads: first every candidate pair (i2 < i) finds the
// first position where the two differ, then token (i, k) takes the smallest i2
// whose first difference lies past k.  The scan is two wave ballots.
#include "common.hpp"

namespace spec {
namespace {

constexpr int kThreads = SPEC_MAX_TREE;

static_assert(kThreads == 2 * kWave, "the scan below covers two waves");

// Inclusive scan of a 0/1 flag over the block's two waves.  Returns the
// inclusive count for this thread and the block total in *total.
__device__ int block_flag_scan(int flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const uint64_t bal = __ballot(flag);
  const uint64_t upto = lane == kWave - 1 ? ~0ull : ((1ull << (lane + 1)) - 1ull);
  int incl = __popcll(bal & upto);
  if (lane == 0) s_wave[wave] = __popcll(bal);
  __syncthreads();
  if (wave == 1) incl += s_wave[0];
  *total = s_wave[0] + s_wave[1];
  return incl;
}

// Writes node t's row (parent, token, depth, mask) given the node's parent
// chain in LDS; padding rows for t >= T.
__device__ void write_node(int t, int T, int T_cap, int n_words, const int* s_par,
                           const int* s_tok, int32_t* parent, int32_t* token, int32_t* depth,
                           uint64_t* anc) {
  uint64_t w0 = 0, w1 = 0;
  int d = -1, par = -1, tok = -1;
  if (t < T) {
    par = s_par[t];
    tok = s_tok[t];
    d = 0;
    int cur = t;
    for (;;) {
      if (cur < 64) w0 |= 1ull << cur; else w1 |= 1ull << (cur - 64);
      if (cur == 0) break;
      cur = s_par[cur];
      ++d;
    }
  }
  parent[t] = par;
  token[t] = tok;
  depth[t] = d;
  anc[(size_t)t * n_words] = w0;
  if (n_words > 1) anc[(size_t)t * n_words + 1] = w1;
}

__global__ __launch_bounds__(kThreads) void k_build_beams(
    int W, int L, int T_cap, const int32_t* __restrict__ beams,
    const int32_t* __restrict__ root_token, int32_t* __restrict__ n_nodes,
    int32_t* __restrict__ parent, int32_t* __restrict__ token, int32_t* __restrict__ depth,
    uint64_t* __restrict__ anc, int32_t* __restrict__ beam_node) {
  __shared__ int s_cand[kThreads];  // candidate tokens, beam-major
  __shared__ int s_wave[2];
  __shared__ int s_node[kThreads];  // node id of every (i, k)
  __shared__ int s_par[kThreads];   // per node
  __shared__ int s_tok[kThreads];
  // first differing position of candidates i2 < i, at [i2 * W + i] (W * W <= 127^2)
  __shared__ unsigned char s_fm[(kThreads - 1) * (kThreads - 1)];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n = W * L;
  const int n_words = (T_cap + 63) / 64;
  const size_t base = (size_t)b * n;
  const int root = tid == 0 ? root_token[b] : 0;  // in flight with the candidates
  if (tid < n) s_cand[tid] = beams[base + tid];
  __syncthreads();

  // pass 1: first position where candidates i2 < i differ (L if they never do);
  // every compare is independent, so the LDS reads pipeline
  for (int p = tid; p < W * W; p += kThreads) {
    const int i2 = p / W, i1 = p - (p / W) * W;
    if (i2 >= i1) continue;
    int fm = L;
    for (int j = L - 1; j >= 0; --j)
      if (s_cand[i2 * L + j] != s_cand[i1 * L + j]) fm = j;
    s_fm[p] = (unsigned char)fm;
  }
  __syncthreads();

  // pass 2: the smallest candidate sharing token (i, k)'s prefix of length k+1
  const int i = tid / L, k = tid - (tid / L) * L;
  int src = i;
  if (tid < n) {
    for (int i2 = i - 1; i2 >= 0; --i2)
      if (s_fm[i2 * W + i] > k) src = i2;
  }
  const int is_new = (tid < n && src == i) ? 1 : 0;
  int total_new;
  const int incl = block_flag_scan(is_new, s_wave, &total_new);
  // first appearances get ids 1, 2, ... in beam-major order
  if (is_new) s_node[tid] = incl;
  __syncthreads();
  // a repeated prefix reuses the node of the smallest sharing candidate,
  // which is itself a first appearance
  if (tid < n && !is_new) s_node[tid] = s_node[src * L + k];
  __syncthreads();
  const int T = 1 + total_new;
  if (tid == 0) {
    s_par[0] = -1;
    s_tok[0] = root;
  }
  if (is_new) {
    const int id = s_node[tid];
    s_par[id] = k == 0 ? 0 : s_node[tid - 1];
    s_tok[id] = s_cand[tid];
  }
  if (tid < n && beam_node) beam_node[base + tid] = s_node[tid];
  __syncthreads();
  const size_t row = (size_t)b * T_cap;
  for (int t = tid; t < T_cap; t += kThreads)
    write_node(t, T, T_cap, n_words, s_par, s_tok, parent + row, token + row, depth + row,
               anc + row * n_words);
  if (tid == 0) n_nodes[b] = T;
}

__global__ __launch_bounds__(kThreads) void k_build_explicit(
    int N, int T_cap, const int32_t* __restrict__ cand_token,
    const int32_t* __restrict__ cand_parent, const int32_t* __restrict__ root_token,
    int32_t* __restrict__ n_nodes, int32_t* __restrict__ parent, int32_t* __restrict__ token,
    int32_t* __restrict__ depth, uint64_t* __restrict__ anc, int32_t* __restrict__ status) {
  __shared__ int s_par[kThreads];
  __shared__ int s_tok[kThreads];
  __shared__ int s_bad;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int n_words = (T_cap + 63) / 64;
  // all global reads in one round trip
  const int root = tid == 0 ? root_token[b] : 0;
  const int p = tid < N ? cand_parent[(size_t)b * N + tid] : 0;
  const int tok = tid < N ? cand_token[(size_t)b * N + tid] : 0;
  if (tid == 0) {
    s_bad = 0;
    s_par[0] = -1;
    s_tok[0] = root;
  }
  __syncthreads();
  if (tid < N) {
    if (p < 0 || p > tid) atomicOr(&s_bad, 1);
    s_par[tid + 1] = p;
    s_tok[tid + 1] = tok;
  }
  __syncthreads();
  const int T = s_bad ? 1 : N + 1;
  if (tid == 0 && s_bad) raise_status(status, SPEC_DEV_BAD_PARENT);
  const size_t row = (size_t)b * T_cap;
  for (int t = tid; t < T_cap; t += kThreads)
    write_node(t, T, T_cap, n_words, s_par, s_tok, parent + row, token + row, depth + row,
               anc + row * n_words);
  if (tid == 0) n_nodes[b] = T;
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" int spec_build_tree(int kind, int B, int W, int L, int T_cap,
                               const int32_t* cand_token, const int32_t* cand_parent,
                               const int32_t* root_token, int32_t* n_nodes, int32_t* parent,
                               int32_t* token, int32_t* depth, uint64_t* anc,
                               int32_t* beam_node, int32_t* status, void* stream) {
  if (B < 0 || W < 1 || L < 1 || T_cap < 1) return SPEC_ERR_INVALID;
  if (T_cap > SPEC_MAX_TREE) return SPEC_ERR_CAPACITY;
  if ((long long)W * L + 1 > T_cap) return SPEC_ERR_CAPACITY;
  if (B == 0) return SPEC_OK;
  if (!cand_token || !root_token || !n_nodes || !parent || !token || !depth || !anc)
    return SPEC_ERR_INVALID;
  hipStream_t s = as_stream(stream);
  if (kind == SPEC_TREE_BEAMS) {
    if (cand_parent) return SPEC_ERR_INVALID;
    hipLaunchKernelGGL(k_build_beams, dim3(B), dim3(kThreads), 0, s, W, L, T_cap, cand_token,
                       root_token, n_nodes, parent, token, depth, anc, beam_node);
  } else if (kind == SPEC_TREE_EXPLICIT) {
    if (!cand_parent || beam_node) return SPEC_ERR_INVALID;
    status = status_or_library(status);
    hipLaunchKernelGGL(k_build_explicit, dim3(B), dim3(kThreads), 0, s, W * L, T_cap,
                       cand_token, cand_parent, root_token, n_nodes, parent, token, depth, anc,
                       status);
  } else {
    return SPEC_ERR_INVALID;
  }
  return launch_status();
}
