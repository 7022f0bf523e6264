// beam_topk.hip -- the pruning step of beam search over a batch of sequences.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "Beam Search During Inference", steps 1 and 3: every extension of
// beam j by token v scores the cumulative log-probability score[j] +
// logp[j][v], and the K best of the K_in x |V| extensions become the next
// beams.  Scores are fp32 sums; equal scores go to the lower flattened index
// j * V + v.  The result feeds the tree build: parent beam, token, score, and
// optionally each new beam's token history.
//
// A candidate is one 64-bit key: the score's bits mapped to an unsigned order
// in the high half, and the bitwise complement of the flattened index in the
// low half, so the largest key is the best score with the lowest index and
// every key is distinct and nonzero (zero marks an empty entry).
//
// k_topk_slices: one workgroup per (sequence, beam, vocabulary slice).  Each
// wave streams its threads' 16-byte chunks of the slice and keeps its best KM
// keys; an element scoring below the wave's current K-th best costs one
// compare, the rest are compacted into a per-wave LDS buffer that is merged
// into the wave's list when full (KM rounds of a wave maximum, in which the
// lane holding the winner drops it).  The four waves' lists are merged the
// same way, and the slice's best KM keys go to the workspace.
// k_topk_merge: one workgroup per sequence selects the final K_out from the
// slices' keys (per-thread sorted lists, then the same rounds) and writes the
// outputs and histories.
#include "common.hpp"

namespace spec {
namespace {

constexpr int kTopThreads = 256;
constexpr int kTopWaves = kTopThreads / kWave;
constexpr int kMinSlice = 2048;   // vocabulary entries per slice workgroup, at least
constexpr int kWantSlices = 512;  // slice workgroups per call, about
constexpr int kBufWord3T = 0x00020000;
constexpr int kCandCap = 256;     // candidate buffer per wave (keys)

__device__ inline uint64_t score_key(float s, uint32_t idx) {
  uint32_t b = __float_as_uint(s);
  if (b == 0x80000000u) b = 0;  // -0.0 ranks as +0.0
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(~idx);
}
__device__ inline float key_score(uint64_t k) {
  const uint32_t o = (uint32_t)(k >> 32);
  const uint32_t b = (o & 0x80000000u) ? (o & 0x7fffffffu) : ~o;
  return __uint_as_float(b);
}
__device__ inline uint32_t key_index(uint64_t k) { return ~(uint32_t)k; }

template <int KM>
struct TopList {
  uint64_t k[KM];  // descending; zeros are empty
};

template <int KM>
__device__ inline void tl_clear(TopList<KM>& t) {
#pragma unroll
  for (int i = 0; i < KM; ++i) t.k[i] = 0;
}

template <int KM>
__device__ inline void tl_push(TopList<KM>& t, uint64_t key) {
  if (key <= t.k[KM - 1]) return;
  t.k[KM - 1] = key;
#pragma unroll
  for (int i = KM - 1; i > 0; --i) {
    const uint64_t a = t.k[i - 1], c = t.k[i];
    const bool sw = c > a;
    t.k[i - 1] = sw ? c : a;
    t.k[i] = sw ? a : c;
  }
}

template <int KM>
__device__ inline void tl_pop(TopList<KM>& t) {
#pragma unroll
  for (int i = 0; i < KM - 1; ++i) t.k[i] = t.k[i + 1];
  t.k[KM - 1] = 0;
}

// Wave maximum of a 32-bit value, uniform in every lane: a running maximum
// along each 16-lane row by DPP row shifts (a lane whose source lies outside
// its row keeps its own value), then the four rows' last lanes.  A few cycles
// per step, where a shuffle is an LDS-crossbar round trip.
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  uint32_t w;
  w = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v = w > v ? w : v;
  w = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v = w > v ? w : v;
  w = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v = w > v ? w : v;
  w = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v = w > v ? w : v;
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 15);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 31);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 47);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return ab > cd ? ab : cd;
}

// Wave maximum of a 64-bit key: the high halves first, then the low halves of
// the lanes holding the highest high half.
__device__ inline uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// The workgroup's best n (<= KM) keys, in order, into out[0..n) (LDS), from
// every thread's list.  Keys are distinct, so the owner of a round's maximum
// is unique.
template <int KM>
__device__ void block_select(TopList<KM>& t, int n, uint64_t* s_wave, uint64_t* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int r = 0; r < n; ++r) {
    const uint64_t m = wave_max_u64(t.k[0]);
    if (m != 0 && t.k[0] == m) tl_pop(t);
    if (lane == 0) s_wave[wave * KM + r] = m;
  }
  __syncthreads();
  if (wave == 0) {
    uint64_t mine = 0;
    if (lane < kTopWaves * KM && (lane % KM) < n) mine = s_wave[lane];
    for (int r = 0; r < n; ++r) {
      const uint64_t m = wave_max_u64(mine);
      if (m != 0 && mine == m) mine = 0;
      if (lane == 0) out[r] = m;
    }
  }
  __syncthreads();
}

// A wave's running top KM (in LDS, descending) merged with its candidate
// buffer: KM rounds in which every lane offers the largest key it holds, the
// wave maximum is taken and its (unique) holder drops it.  Returns the new
// K-th key (0 while fewer than KM keys exist).
template <int KM>
__device__ uint64_t wave_reduce(uint64_t* cand, int n_c, uint64_t* top) {
  const int lane = threadIdx.x & 63;
  constexpr int R = kCandCap / kWave + 1;
  uint64_t r[R];
#pragma unroll
  for (int i = 0; i < R - 1; ++i) r[i] = lane + kWave * i < n_c ? cand[lane + kWave * i] : 0ull;
  r[R - 1] = lane < KM ? top[lane] : 0ull;
  uint64_t kth = 0;
  for (int q = 0; q < KM; ++q) {
    uint64_t best = r[0];
#pragma unroll
    for (int i = 1; i < R; ++i) best = r[i] > best ? r[i] : best;
    const uint64_t m = wave_max_u64(best);
    if (m != 0 && best == m) {
      bool done = false;
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const bool hit = !done && r[i] == m;
        r[i] = hit ? 0ull : r[i];
        done = done || hit;
      }
    }
    if (lane == 0) top[q] = m;
    kth = m;
  }
  return kth;
}

template <int KM, bool VEC>
__global__ __launch_bounds__(kTopThreads) void k_topk_slices(int K_in, int V, int Pv, int slice,
                                                             int K_out, const float* __restrict__ logp,
                                                             const float* __restrict__ beam_score,
                                                             uint64_t* __restrict__ ws) {
  __shared__ uint64_t s_cand[kTopWaves][kCandCap];
  __shared__ uint64_t s_top[kTopWaves][KM];
  __shared__ uint64_t s_out[KM];
  const int unit = blockIdx.x;  // (b * K_in + j) * Pv + pv
  const int pv = unit % Pv;
  const int bj = unit / Pv;
  const int j = bj % K_in;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float base = beam_score ? beam_score[bj] : 0.0f;
  const float* row = logp + (size_t)bj * V;
  const int v0 = pv * slice;
  const int n = max(0, min(slice, V - v0));
  const uint32_t idx0 = (uint32_t)j * (uint32_t)V + (uint32_t)v0;
  uint64_t* cand = s_cand[wave];
  uint64_t* top = s_top[wave];
  if (lane < KM) top[lane] = 0;

  // Each wave keeps its own top KM.  An element whose score is below the
  // wave's K-th best score (tau) cannot enter it: that costs one compare.  The
  // others are compacted into the wave's candidate buffer, which is merged
  // into the top list when it could overflow.
  float tau = -INFINITY;
  uint64_t kth = 0;
  int n_c = 0;
  auto offer = [&](float sc, int p) {
    const bool live = p < n && sc >= tau;
    const uint64_t key = score_key(sc, idx0 + (uint32_t)p);
    const bool pass = live && key > kth;
    const uint64_t mask = __ballot(pass);
    if (mask) {
      const uint64_t below = lane == 0 ? 0ull : (~0ull >> (64 - lane));
      if (pass) cand[n_c + __popcll(mask & below)] = key;
      n_c += __popcll(mask);
      if (n_c > kCandCap - kWave) {
        kth = wave_reduce<KM>(cand, n_c, top);
        tau = kth ? key_score(kth) : -INFINITY;
        n_c = 0;
      }
    }
  };
  if constexpr (VEC) {
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(row + v0), (short)0,
                                                      n * 4, kBufWord3T);
    const int n_chunks = (n + 3) >> 2;
    constexpr int U = 4;  // 16-byte loads per thread per step
    f32x4 x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      x[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, (u * kTopThreads + tid) * 16, 0, kLoadOnce));
    for (int c0 = 0; c0 < n_chunks; c0 += U * kTopThreads) {
      // the next step's loads go out before this step's elements are offered
#pragma unroll
      for (int u = 0; u < U; ++u)
        y[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rs, (c0 + (U + u) * kTopThreads + tid) * 16, 0, kLoadOnce));
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) offer(base + x[u][e], (c0 + u * kTopThreads + tid) * 4 + e);
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = y[u];
    }
  } else {
    for (int p0 = 0; p0 < n; p0 += kTopThreads) {
      const int p = p0 + tid;
      offer(p < n ? base + row[v0 + p] : -INFINITY, p);
    }
  }
  wave_reduce<KM>(cand, n_c, top);
  __syncthreads();
  // the four waves' lists: KM rounds of the wave maximum in wave 0
  const int keep = K_out < KM ? K_out : KM;
  if (wave == 0) {
    uint64_t mine = lane < kTopWaves * KM ? s_top[lane / KM][lane % KM] : 0ull;
    for (int r = 0; r < keep; ++r) {
      const uint64_t m = wave_max_u64(mine);
      if (m != 0 && mine == m) mine = 0;
      if (lane == 0) s_out[r] = m;
    }
  }
  __syncthreads();
  if (tid < KM) ws[(size_t)unit * KM + tid] = tid < keep ? s_out[tid] : 0ull;
}

template <int KM>
__global__ __launch_bounds__(kTopThreads) void k_topk_merge(int K_in, int V, int n_slices, int K_out,
                                                            const uint64_t* __restrict__ ws,
                                                            int32_t* __restrict__ out_parent,
                                                            int32_t* __restrict__ out_token,
                                                            float* __restrict__ out_score,
                                                            const int32_t* __restrict__ hist_in,
                                                            int len,
                                                            int32_t* __restrict__ hist_out) {
  __shared__ uint64_t s_wave[kTopWaves * KM];
  __shared__ uint64_t s_out[KM];
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const uint64_t* keys = ws + (size_t)b * n_slices * KM;
  TopList<KM> t;
  tl_clear(t);
  for (int i = tid; i < n_slices * KM; i += kTopThreads) tl_push(t, keys[i]);
  block_select(t, K_out, s_wave, s_out);
  if (tid < K_out) {
    const uint64_t k = s_out[tid];
    const uint32_t idx = key_index(k);
    const int j = (int)(idx / (uint32_t)V), v = (int)(idx % (uint32_t)V);
    out_parent[(size_t)b * K_out + tid] = j;
    out_token[(size_t)b * K_out + tid] = v;
    out_score[(size_t)b * K_out + tid] = key_score(k);
  }
  if (hist_out) {
    // new beam k: the parent's history, then the new token
    for (int e = tid; e < K_out * (len + 1); e += kTopThreads) {
      const int k = e / (len + 1), i = e - k * (len + 1);
      const uint32_t idx = key_index(s_out[k]);
      const int j = (int)(idx / (uint32_t)V);
      hist_out[((size_t)b * K_out + k) * (len + 1) + i] =
          i < len ? hist_in[((size_t)b * K_in + j) * len + i] : (int)(idx % (uint32_t)V);
    }
  }
}

struct TopkPlan {
  int Pv, slice, n_slices, KM;
  size_t ws_bytes;
};

TopkPlan topk_plan(int B, int K_in, int K_out, int V) {
  TopkPlan p{};
  p.KM = K_out <= 8 ? 8 : 16;
  const long rows = (long)B * K_in;
  long want = (kWantSlices + rows - 1) / rows;
  long by_v = (V + kMinSlice - 1) / kMinSlice;
  if (want > by_v) want = by_v;
  if (want < 1) want = 1;
  int slice = (int)((V + want - 1) / want);
  slice = (slice + 3) & ~3;  // slices start on 16-byte boundaries
  p.slice = slice;
  p.Pv = (V + slice - 1) / slice;
  p.n_slices = K_in * p.Pv;
  p.ws_bytes = round_up((size_t)B * p.n_slices * p.KM * sizeof(uint64_t), 256);
  return p;
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_beam_topk_workspace_size(int B, int K_in, int K_out, int V) {
  if (B < 1 || K_in < 1 || K_out < 1 || K_out > SPEC_MAX_BEAM_TOPK || V < 1) return 0;
  return topk_plan(B, K_in, K_out, V).ws_bytes;
}

extern "C" int spec_beam_topk(int B, int K_in, int K_out, int V, const float* logp,
                              const float* beam_score, int32_t* out_parent, int32_t* out_token,
                              float* out_score, const int32_t* hist_in, int hist_len,
                              int32_t* hist_out, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || K_in < 1 || K_out < 1 || V < 1 || hist_len < 0) return SPEC_ERR_INVALID;
  if (K_out > SPEC_MAX_BEAM_TOPK || (long long)K_out > (long long)K_in * V)
    return SPEC_ERR_CAPACITY;
  if ((long long)K_in * V >= 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  if (B == 0) return SPEC_OK;
  if (!logp || !out_parent || !out_token || !out_score) return SPEC_ERR_INVALID;
  if (hist_in && !hist_out) return SPEC_ERR_INVALID;
  if (hist_out && hist_len > 0 && !hist_in) return SPEC_ERR_INVALID;
  const TopkPlan p = topk_plan(B, K_in, K_out, V);
  if (!ws || ws_bytes < p.ws_bytes || !aligned(ws, 256)) return SPEC_ERR_WORKSPACE;
  hipStream_t s = as_stream(stream);
  uint64_t* keys = static_cast<uint64_t*>(ws);
  const bool vec = V % 4 == 0 && aligned(logp, 16);
  const dim3 grid1((unsigned)((long)B * K_in * p.Pv));
#define SPEC_TOPK(KM_)                                                                          \
  if (vec)                                                                                     \
    hipLaunchKernelGGL((k_topk_slices<KM_, true>), grid1, dim3(kTopThreads), 0, s, K_in, V,    \
                       p.Pv, p.slice, K_out, logp, beam_score, keys);                          \
  else                                                                                         \
    hipLaunchKernelGGL((k_topk_slices<KM_, false>), grid1, dim3(kTopThreads), 0, s, K_in, V,   \
                       p.Pv, p.slice, K_out, logp, beam_score, keys);                          \
  hipLaunchKernelGGL((k_topk_merge<KM_>), dim3(B), dim3(kTopThreads), 0, s, K_in, V,            \
                     p.n_slices, K_out, keys, out_parent, out_token, out_score, hist_in,        \
                     hist_len, hist_out);
  if (p.KM == 8) {
    SPEC_TOPK(8)
  } else {
    SPEC_TOPK(16)
  }
#undef SPEC_TOPK
  return launch_status();
}
