// tree_attention.hip -- tree-masked GQA attention of the packed tree's queries
// over the KV cache plus the tree's own K/V.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 4: the target runs one
// forward pass over the packed beam under the tree mask; each token's result
// equals the one it would get had its own prefix been decoded token by token.
// "Clover: Regressive Lightweight Speculative Decoding with Sequential
// Knowledge", causal mask construction: M_ij = 1 iff j is an ancestor of i or
// i = j.
//
// bf16 path (gfx950 MFMA).  For one (sequence, KV head) the G query heads of the
// group times the T tree nodes form an M = G*T row block that shares every key,
// so Q K^T and P V are real dense contractions and every K/V byte is read once
// for all of them.  A workgroup of NW waves owns a slice of those rows (QT
// 16-row MFMA tiles per wave) and a range of keys: it streams 64-key K and V
// tiles through LDS (double-buffered; V stored transposed so the P V operand is
// a contiguous LDS read; for wide GQA groups at D = 128 the tiles are loaded
// straight into LDS as they lie in memory and the V^T operand comes from
// transposing LDS reads), computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 so
// that each lane owns one query row, runs the online softmax in fp32 in exp2
// form (row sums of P in fp32 per lane, added across lanes after the key
// loop), and accumulates O^T = V^T P^T with the same MFMA.  When few rows exist
// (no GQA, small trees) the waves split each key tile instead (KG key groups)
// and combine through LDS at the end.  The running maximum is only moved when
// a score exceeds it by more than 2^8, so most tiles skip the rescale of the
// accumulators; the result is the same softmax (on the direct-load plan the
// exponentials are taken first and the test is an integer maximum of their
// bits, exceeding 2^8).  Context keys are unmasked;
// only tiles that reach the tree slots test the ancestor bits.  Long contexts
// are split across workgroups (chosen so the grid fills the 256 CUs evenly) and
// a merge kernel combines the (max, sum, O) partials.
//
// fp32 path: one wavefront per output row, plain FMA, for the small fp32 case.
#include "attn_bf16.hpp"

namespace spec {
namespace {

using namespace attn;

constexpr int kNumCU = 256;       // MI355X compute units
constexpr int kMaxSplits = 32;    // context splits per (sequence, KV head)

// ------------------------------------------------------------------ geometry

struct AttnPlan {
  int NW;        // waves per workgroup
  int QT;        // 16-row query tiles per wave
  int KG;        // key groups (waves splitting one key tile)
  int PF;        // tiles of global loads in flight per workgroup (1 or 2)
  int NS;        // LDS stages of direct-to-LDS tiles, scores one tile ahead (2; 0: staged through registers)
  int n_mt;      // row blocks (workgroups sharing one key range)
  int n_splits;  // context splits
  int tiles_per_split;
  int n_kv;      // B * Hkv * n_splits, the key-stream work units
  int n_slots;   // workgroups launched (n_kv padded to a multiple of 8, times n_mt)
};

void finish_plan(AttnPlan& p, int B, int T_cap, int H, int Hkv, int max_ctx, int want_splits) {
  const int nq = (H / Hkv * T_cap + 15) / 16;
  const int per_wg = p.NW / p.KG * p.QT;
  p.n_mt = (nq + per_wg - 1) / per_wg;
  const int n_tiles = (max_ctx + T_cap + kKeyTile - 1) / kKeyTile;
  int s = want_splits < 1 ? 1 : want_splits;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s > n_tiles) s = n_tiles;
  p.tiles_per_split = (n_tiles + s - 1) / s;
  p.n_splits = (n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  p.n_kv = B * Hkv * p.n_splits;
  p.n_slots = ((p.n_kv + 7) / 8) * 8 * p.n_mt;
}

// Shape-driven choice of the tiling: enough query tiles per wave to reuse each
// K/V tile across the whole G*T row block, and enough context splits that the
// busy workgroups cover every CU about once (or twice for 4-wave groups).
AttnPlan make_plan(int B, int T_cap, int H, int Hkv, int D, int max_ctx) {
  AttnPlan p{};
  const int nq = (H / Hkv * T_cap + 15) / 16;
  p.NW = 8;
  if (nq <= 4) {
    // few rows: waves pair up on each key tile (two key groups)
    p.KG = 2; p.QT = 1; p.PF = 1;
    // many independent key streams (the grid runs in several rounds, bound by
    // the stream rate) and at most 32 rows: 4-wave groups with two tiles of
    // loads in flight stream faster
    if (nq <= 2 && (long)B * Hkv >= 4L * kNumCU) { p.NW = 4; p.PF = 2; }
  } else if (nq <= 8 || (nq <= 16 && D != 128)) {
    // one row block: two query tiles per wave, two tiles of loads in flight
    p.KG = 1; p.QT = 2; p.PF = 2;
  } else {
    // many rows (wide GQA groups; at D = 128 from 9 query tiles on): 128-row
    // blocks of 4 waves with two query tiles each read the same key range, two
    // workgroups per CU; at D = 128 the tiles go straight to LDS, which frees
    // the staging registers and the stores from the waves, and the scores of
    // the next tile run beside the softmax and P V of this one.  With 9 to 16
    // query tiles this beats one 8-wave block of register-staged tiles (196
    // rows, 32k keys: 157 -> 149 us), and an 8-wave block of direct loads
    // (161 us).
    p.NW = 4; p.KG = 1; p.QT = 2; p.PF = 2;
    if (D == 128) p.NS = 2;
  }
  const long units = (long)B * Hkv;
  const int n_tiles = (max_ctx + T_cap + kKeyTile - 1) / kKeyTile;
  // enough context splits that the workgroups (units x row blocks x splits)
  // cover every CU once, or twice for 4-wave groups
  const int per_wg = p.NW / p.KG * p.QT;
  const long n_mt = (nq + per_wg - 1) / per_wg;
  const long slots_wanted = (long)kNumCU * (p.NW == 4 ? 2 : 1);
  long want = (slots_wanted + units * n_mt - 1) / (units * n_mt);
  const long by_len = n_tiles / 2 > 0 ? n_tiles / 2 : 1;  // at least 2 tiles per split
  if (want > by_len) want = by_len;
  finish_plan(p, B, T_cap, H, Hkv, max_ctx, (int)want);
  // a grid of at most about two workgroups per CU runs short, latency-bound
  // streams: keep two tiles of loads in flight there
  if (p.KG == 2 && p.n_slots <= 2 * kNumCU) p.PF = 2;
  return p;
}

size_t partial_bytes(const AttnPlan& p, int B, int T_cap, int H, int Hkv, int D) {
  if (p.n_splits <= 1) return 0;
  const size_t rows = (size_t)(H / Hkv) * T_cap;
  const size_t units = (size_t)B * Hkv * p.n_splits;
  return round_up(units * rows * D * sizeof(float), 256) +
         2 * round_up(units * rows * sizeof(float), 256);
}

template <int D, int MAXS>
__global__ __launch_bounds__(256) void k_attn_merge(int T_cap, int H, int Hkv, int cache_cap,
                                                    int max_ctx, int n_splits,
                                                    const int32_t* __restrict__ ctx_len,
                                                    const int32_t* __restrict__ n_nodes,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_m,
                                                    const float* __restrict__ part_l,
                                                    bf16_t* __restrict__ out) {
  constexpr int TPR = D / 4;          // threads per row
  constexpr int RPB = 256 / TPR;      // rows per block
  const int G = H / Hkv;
  const int M_cap = G * T_cap;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, g_kv = bh - (bh / Hkv) * Hkv;
  const int r = blockIdx.x * RPB + threadIdx.x / TPR;
  const int d0 = 4 * (threadIdx.x % TPR);
  if (r >= M_cap) return;
  float ms[MAXS], ls[MAXS];
  f32x4 os[MAXS];
#pragma unroll
  for (int s = 0; s < MAXS; ++s) {
    ms[s] = -INFINITY;
    ls[s] = 0.0f;
    os[s] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (s < n_splits) {  // uniform
      const size_t u = (size_t)bh * n_splits + s;
      ms[s] = part_m[u * M_cap + r];
      ls[s] = part_l[u * M_cap + r];
      os[s] = *reinterpret_cast<const f32x4*>(part_o + (u * M_cap + r) * D + d0);
    }
  }
  const int ctx = ctx_len[b], T = n_nodes[b];
  const bool bad = T < 1 || T > T_cap || ctx < 0 || ctx > max_ctx || ctx + T > cache_cap;
  const int rows_valid = bad ? 0 : G * T;
  const int t = r / G, gq = r - t * G;
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < MAXS; ++s)
    if (s < n_splits) M = fmaxf(M, ms[s]);
  f32x4 o{0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (r < rows_valid && M != -INFINITY) {
#pragma unroll
    for (int s = 0; s < MAXS; ++s) {
      const bool use = s < n_splits && ms[s] != -INFINITY;
      const float w = use ? __builtin_amdgcn_exp2f(ms[s] - M) : 0.0f;
      L += use ? ls[s] * w : 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] += use ? os[s][e] * w : 0.0f;
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    o *= inv;
  }
  bf16x4 ob{(bf16_t)o[0], (bf16_t)o[1], (bf16_t)o[2], (bf16_t)o[3]};
  *reinterpret_cast<bf16x4*>(out + (((size_t)b * T_cap + t) * H + g_kv * G + gq) * D + d0) = ob;
}

// ------------------------------------------------------------------ fp32 path

// One wavefront per (b, t, h) output row; lanes split the head dimension.
__global__ __launch_bounds__(256) void k_attn_f32(int B, int T_cap, int H, int Hkv, int D,
                                                  int cache_cap, int max_ctx,
                                                  const float* __restrict__ q,
                                                  const float* __restrict__ kc,
                                                  const float* __restrict__ vc,
                                                  const int32_t* __restrict__ ctx_len,
                                                  const int32_t* __restrict__ n_nodes,
                                                  const uint64_t* __restrict__ anc, float scale,
                                                  float* __restrict__ out,
                                                  int32_t* __restrict__ status) {
  constexpr int MAXD = 4;  // up to 256 dims, 4 per lane
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= B * T_cap * H) return;
  const int b = row / (T_cap * H);
  const int t = (row / H) % T_cap;
  const int h = row % H;
  const int g = h / (H / Hkv);
  const int n_words = (T_cap + 63) / 64;
  const int ctx = ctx_len[b], T = n_nodes[b];
  const bool bad = T < 1 || T > T_cap || ctx < 0 || ctx > max_ctx || ctx + T > cache_cap;
  float* orow = out + (size_t)row * D;
  if (bad || t >= T) {
    if (bad && t == 0 && h == 0 && lane == 0) raise_status(status, SPEC_DEV_CTX_RANGE);
    for (int d = lane; d < D; d += 64) orow[d] = 0.0f;
    return;
  }
  const float* qrow = q + (size_t)row * D;
  float qv[MAXD], acc[MAXD];
#pragma unroll
  for (int j = 0; j < MAXD; ++j) {
    const int d = lane + 64 * j;
    qv[j] = d < D ? qrow[d] : 0.0f;
    acc[j] = 0.0f;
  }
  const uint64_t* arow = anc + ((size_t)b * T_cap + t) * n_words;
  const float* kb = kc + ((size_t)b * Hkv + g) * cache_cap * D;
  const float* vb = vc + ((size_t)b * Hkv + g) * cache_cap * D;
  const int n_keys = ctx + T;
  float m = -INFINITY, l = 0.0f;
  // keys in chunks of KC: every K and V load of a chunk is issued before any
  // is used, so a chunk costs one memory round trip
  constexpr int KC = 16;
  for (int j0 = 0; j0 < n_keys; j0 += KC) {
    float kv[KC][MAXD], vv[KC][MAXD];
    bool vis[KC];
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const int j = j0 + c;
      bool v = j < n_keys;
      if (v && j >= ctx) {
        const int aa = j - ctx;
        v = (arow[aa >> 6] >> (aa & 63)) & 1ull;
      }
      vis[c] = v;
#pragma unroll
      for (int jj = 0; jj < MAXD; ++jj) {
        const int d = lane + 64 * jj;
        const bool in = j < n_keys && d < D;
        kv[c][jj] = in ? kb[(size_t)j * D + d] : 0.0f;
        vv[c][jj] = in ? vb[(size_t)j * D + d] : 0.0f;
      }
    }
    float sc[KC];
    float cmax = -INFINITY;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      float part = 0.0f;
#pragma unroll
      for (int jj = 0; jj < MAXD; ++jj) part += qv[jj] * kv[c][jj];
      sc[c] = wave_sum_f32(part) * scale;
      if (vis[c]) cmax = fmaxf(cmax, sc[c]);
    }
    if (cmax == -INFINITY) continue;  // no visible key in the chunk (uniform)
    const float m_new = fmaxf(m, cmax);
    const float alpha = __expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int jj = 0; jj < MAXD; ++jj) acc[jj] *= alpha;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      const float p = vis[c] ? __expf(sc[c] - m_new) : 0.0f;
      l += p;
#pragma unroll
      for (int jj = 0; jj < MAXD; ++jj) acc[jj] += p * vv[c][jj];
    }
    m = m_new;
  }
#pragma unroll
  for (int jj = 0; jj < MAXD; ++jj) {
    const int d = lane + 64 * jj;
    if (d < D) orow[d] = acc[jj] / l;
  }
}

// ------------------------------------------------------------------ launchers

// The plans make_plan can choose.  A key range read by one row block only
// (n_mt == 1) is streamed with non-temporal loads; row blocks that share a key
// range keep the default policy so the others find its tiles in L2.
template <int D>
int dispatch_main(const AttnPlan& p, const AttnArgs& args, hipStream_t s) {
  const bool once = p.n_mt == 1;
#define SPEC_ATTN_CASE(NW_, QT_, KG_, PF_, NS_)                                           \
  if (p.NW == NW_ && p.QT == QT_ && p.KG == KG_ && p.PF == PF_ && p.NS == NS_)            \
    return once ? launch_main<D, NW_, QT_, KG_, PF_, NS_, true>(p.n_slots, args, s)       \
                : launch_main<D, NW_, QT_, KG_, PF_, NS_, false>(p.n_slots, args, s);
  SPEC_ATTN_CASE(8, 1, 2, 1, 0)
  SPEC_ATTN_CASE(8, 1, 2, 2, 0)
  SPEC_ATTN_CASE(4, 1, 2, 2, 0)
  SPEC_ATTN_CASE(8, 2, 1, 2, 0)
  if constexpr (D == 64) {
    SPEC_ATTN_CASE(4, 2, 1, 2, 0)
  } else {
    if (p.NW == 4 && p.QT == 2 && p.KG == 1 && p.PF == 2 && p.NS == 2)
      return launch_direct(once, p.n_slots, args, s);
  }
#undef SPEC_ATTN_CASE
  return SPEC_ERR_UNSUPPORTED;
}

template <int D>
int launch_merge(const AttnPlan& p, const AttnArgs& a, hipStream_t s) {
  constexpr int RPB = 256 / (D / 4);
  const int G = a.H / a.Hkv;
  dim3 grid((G * a.T_cap + RPB - 1) / RPB, a.B * a.Hkv);
#define SPEC_MERGE_CASE(MAXS_)                                                                  \
  if (p.n_splits <= MAXS_) {                                                                   \
    hipLaunchKernelGGL((k_attn_merge<D, MAXS_>), grid, dim3(256), 0, s, a.T_cap, a.H, a.Hkv,   \
                       a.cache_cap, a.max_ctx, p.n_splits, a.ctx_len, a.n_nodes, a.part_o,     \
                       a.part_m, a.part_l, a.out);                                             \
    return launch_status();                                                                    \
  }
  SPEC_MERGE_CASE(2)
  SPEC_MERGE_CASE(4)
  SPEC_MERGE_CASE(8)
  SPEC_MERGE_CASE(16)
  SPEC_MERGE_CASE(32)
#undef SPEC_MERGE_CASE
  return SPEC_ERR_UNSUPPORTED;
}

// Validated launch of the bf16 path with a given plan (ws already checked).
int run_bf16(const AttnPlan& p, int B, int T_cap, int H, int Hkv, int D, int cache_cap,
             int max_ctx, const void* q, const void* k_cache, const void* v_cache,
             const int32_t* ctx_len, const int32_t* n_nodes, const uint64_t* anc, float scale,
             void* out, void* ws, int32_t* status, hipStream_t s) {
  AttnArgs a{};
  a.B = B;
  a.T_cap = T_cap;
  a.H = H;
  a.Hkv = Hkv;
  a.cache_cap = cache_cap;
  a.max_ctx = max_ctx;
  a.n_splits = p.n_splits;
  a.tiles_per_split = p.tiles_per_split;
  a.n_kv = p.n_kv;
  a.n_mt = p.n_mt;
  a.scale_log2 = scale * kLog2e;
  a.q = static_cast<const bf16_t*>(q);
  a.kc = static_cast<const bf16_t*>(k_cache);
  a.vc = static_cast<const bf16_t*>(v_cache);
  a.ctx_len = ctx_len;
  a.n_nodes = n_nodes;
  a.anc = anc;
  a.out = static_cast<bf16_t*>(out);
  a.status = status;
  if (p.n_splits > 1) {
    const size_t rows = (size_t)(H / Hkv) * T_cap;
    const size_t units = (size_t)B * Hkv * p.n_splits;
    char* w = static_cast<char*>(ws);
    a.part_o = reinterpret_cast<float*>(w);
    w += round_up(units * rows * D * sizeof(float), 256);
    a.part_m = reinterpret_cast<float*>(w);
    w += round_up(units * rows * sizeof(float), 256);
    a.part_l = reinterpret_cast<float*>(w);
  }
  int rc = D == 128 ? dispatch_main<128>(p, a, s) : dispatch_main<64>(p, a, s);
  if (rc != SPEC_OK || p.n_splits <= 1) return rc;
  return D == 128 ? launch_merge<128>(p, a, s) : launch_merge<64>(p, a, s);
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_tree_attention_workspace_size(int dt, int B, int T_cap, int H, int Hkv,
                                                     int D, int max_ctx) {
  if (dt != SPEC_BF16 || B < 1 || T_cap < 1 || H < 1 || Hkv < 1 || H % Hkv || max_ctx < 0)
    return 0;
  const AttnPlan p = make_plan(B, T_cap, H, Hkv, D, max_ctx);
  return partial_bytes(p, B, T_cap, H, Hkv, D);
}

extern "C" int spec_tree_attention(int dt, int B, int T_cap, int H, int Hkv, int D,
                                   int cache_cap, int max_ctx, const void* q,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* ctx_len, const int32_t* n_nodes,
                                   const uint64_t* anc, float scale, void* out, void* ws,
                                   size_t ws_bytes, int32_t* status, void* stream) {
  if (B < 0 || T_cap < 1 || H < 1 || Hkv < 1 || D < 1 || max_ctx < 0 || cache_cap < 1)
    return SPEC_ERR_INVALID;
  if (H % Hkv) return SPEC_ERR_INVALID;
  if (T_cap > SPEC_MAX_TREE) return SPEC_ERR_CAPACITY;
  if ((long long)max_ctx + T_cap > cache_cap) return SPEC_ERR_CAPACITY;
  if (B == 0) return SPEC_OK;
  if (!q || !k_cache || !v_cache || !ctx_len || !n_nodes || !anc || !out) return SPEC_ERR_INVALID;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf((float)D);
  hipStream_t s = as_stream(stream);
  status = status_or_library(status);
  if (dt == SPEC_F32) {
    if (D > 256) return SPEC_ERR_UNSUPPORTED;
    const int rows = B * T_cap * H;
    hipLaunchKernelGGL(k_attn_f32, dim3((rows + 3) / 4), dim3(256), 0, s, B, T_cap, H, Hkv, D,
                       cache_cap, max_ctx, static_cast<const float*>(q),
                       static_cast<const float*>(k_cache), static_cast<const float*>(v_cache),
                       ctx_len, n_nodes, anc, scale, static_cast<float*>(out), status);
    return launch_status();
  }
  if (dt != SPEC_BF16) return SPEC_ERR_INVALID;
  if (D != 64 && D != 128) return SPEC_ERR_UNSUPPORTED;
  // tile loads address one (b, KV head) row block through 32-bit buffer ranges
  if ((long long)cache_cap * D * 2 > 0x7fffffffLL) return SPEC_ERR_UNSUPPORTED;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return SPEC_ERR_INVALID;
  const AttnPlan p = make_plan(B, T_cap, H, Hkv, D, max_ctx);
  const size_t need = partial_bytes(p, B, T_cap, H, Hkv, D);
  if (need && (!ws || ws_bytes < need || !aligned(ws, 256))) return SPEC_ERR_WORKSPACE;
  return run_bf16(p, B, T_cap, H, Hkv, D, cache_cap, max_ctx, q, k_cache, v_cache, ctx_len,
                  n_nodes, anc, scale, out, ws, status, s);
}
