// tree_attention.hip -- tree-masked GQA attention of the packed tree's queries
// over the KV cache plus the tree's own K/V.
//
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 4: the target runs one
// forward pass over the packed beam under the tree mask; each token's result
// equals the one it would get had its own prefix been decoded token by token.
// "Clover: Regressive Lightweight Speculative Decoding with Sequential
// Knowledge", Figure 4: mask M_ij = 1 iff j is an ancestor of i or i = j.
//
// bf16 path (gfx950 MFMA).  For one (sequence, KV head) the G query heads of the
// group times the T tree nodes form an M = G*T row block that shares every key,
// so Q K^T and P V are real dense contractions.  A workgroup of 4 waves owns a
// slice of those rows (16-row MFMA tiles) and a slice of the keys: it streams
// 64-key K and V tiles through LDS (double-buffered, V stored transposed so the
// P V operand is a contiguous LDS read), computes S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 so that each lane ends up owning one query row,
// runs the online softmax in fp32 in exp2 form, and accumulates O^T = V^T P^T
// with the same MFMA.  Context keys are unmasked; only the last tiles, which
// hold the tree slots, test the ancestor bits.  Long contexts are split across
// workgroups; a merge kernel combines the (max, sum, O) partials.
//
// fp32 path: one wavefront per output row, plain FMA, for the small fp32 case.
#include "common.hpp"

namespace spec {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeyTile = 64;   // keys per LDS stage
constexpr int kThreads = 256;  // 4 waves

// ------------------------------------------------------------------ geometry

struct AttnPlan {
  int KG;        // key groups per workgroup (waves splitting a key tile)
  int QT;        // 16-row query tiles per wave
  int n_mt;      // row tiles (workgroups) per (b, kv head)
  int n_splits;  // context splits
  int tiles_per_split;
  int n_kv;      // B * Hkv * n_splits, the key-stream work units
  int n_slots;   // workgroups launched (n_kv padded to a multiple of 8, times n_mt)
};

AttnPlan make_plan(int B, int T_cap, int H, int Hkv, int max_ctx) {
  AttnPlan p{};
  const int G = H / Hkv;
  const int rows = G * T_cap;
  const int nq = (rows + 15) / 16;
  if (nq <= 4) {
    p.KG = 2;
    p.QT = (nq + 1) / 2;
    p.n_mt = 1;
  } else {
    p.KG = 1;
    p.QT = 2;
    const int per_wg = 4 * p.QT;
    p.n_mt = (nq + per_wg - 1) / per_wg;
  }
  const int total_keys = max_ctx + T_cap;
  const int n_tiles = (total_keys + kKeyTile - 1) / kKeyTile;
  const long base = (long)B * Hkv * p.n_mt;
  int want = (int)((512 + base - 1) / base);
  if (want < 1) want = 1;
  // at least 4 tiles (256 keys) per split
  int max_splits = (n_tiles + 3) / 4;
  if (max_splits < 1) max_splits = 1;
  if (want > max_splits) want = max_splits;
  p.tiles_per_split = (n_tiles + want - 1) / want;
  p.n_splits = (n_tiles + p.tiles_per_split - 1) / p.tiles_per_split;
  p.n_kv = B * Hkv * p.n_splits;
  p.n_slots = ((p.n_kv + 7) / 8) * 8 * p.n_mt;
  return p;
}

size_t partial_bytes(const AttnPlan& p, int B, int T_cap, int H, int Hkv, int D) {
  if (p.n_splits <= 1) return 0;
  const size_t rows = (size_t)(H / Hkv) * T_cap;
  const size_t units = (size_t)B * Hkv * p.n_splits;
  return round_up(units * rows * D * sizeof(float), 256) +
         2 * round_up(units * rows * sizeof(float), 256);
}

// ------------------------------------------------------------------ bf16 MFMA kernel

template <int D>
struct Lds {
  static constexpr int kPitchK = D + 8;         // bf16 elements per K row
  static constexpr int kPitchV = kKeyTile + 4;  // bf16 elements per transposed V row
  static constexpr int kStageK = kKeyTile * kPitchK;
  static constexpr int kStageV = D * kPitchV;
  static constexpr int kStage = kStageK + kStageV;
  static constexpr int kBytes = 2 * kStage * 2;  // two stages of bf16
};

__device__ inline f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Map a workgroup slot to (kv unit, row tile) so that the row tiles sharing one
// key stream land on the same XCD (slots are dealt round-robin over 8 XCDs).
__device__ inline void slot_to_work(int slot, int n_mt, int& kv_unit, int& mt) {
  const int xcd = slot & 7;
  const int j = slot >> 3;
  kv_unit = xcd + 8 * (j / n_mt);
  mt = j - (j / n_mt) * n_mt;
}

template <int D, int QT, int KG>
__global__ __launch_bounds__(kThreads, 2) void k_attn_bf16(
    int B, int T_cap, int H, int Hkv, int cache_cap, int max_ctx, int n_splits,
    int tiles_per_split, int n_kv, int n_mt, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ n_nodes,
    const uint64_t* __restrict__ anc, float scale_log2, bf16_t* __restrict__ out,
    float* __restrict__ part_o, float* __restrict__ part_m, float* __restrict__ part_l,
    int32_t* __restrict__ status) {
  constexpr int RG = 4 / KG;            // row groups
  constexpr int KSTEPS = D / 32;        // k-steps of Q K^T
  constexpr int DT = D / 16;            // 16-wide d tiles of the output
  constexpr int KEYS_W = kKeyTile / KG; // keys per wave per tile
  constexpr int SUB = KEYS_W / 16;      // 16-key sub-tiles per wave per tile
  constexpr int PV_STEPS = KEYS_W / 32; // 32-key k-steps of P V per tile
  static_assert(KG == 1 || KG == 2, "key groups");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);

  int kv_unit, mt;
  slot_to_work(blockIdx.x, n_mt, kv_unit, mt);
  if (kv_unit >= n_kv) return;
  const int sp = kv_unit % n_splits;
  const int bh = kv_unit / n_splits;
  const int b = bh / Hkv;
  const int g_kv = bh - b * Hkv;
  const int G = H / Hkv;
  const int M_cap = G * T_cap;
  const int n_words = (T_cap + 63) / 64;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int rg = wave / KG;
  const int kg = wave - rg * KG;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  const int ctx = ctx_len[b];
  const int T = n_nodes[b];
  const bool bad = T < 1 || T > T_cap || ctx < 0 || ctx > max_ctx || ctx + T > cache_cap;
  const int rows_valid = bad ? 0 : G * T;
  const int nq_valid = (rows_valid + 15) >> 4;
  const int n_keys = ctx + T;
  const int k_begin = sp * tiles_per_split * kKeyTile;
  int k_end = k_begin + tiles_per_split * kKeyTile;
  if (k_end > n_keys) k_end = n_keys;
  if (bad && sp == 0 && mt == 0 && tid == 0) raise_status(status, SPEC_DEV_CTX_RANGE);

  // this wave's query tiles: interleaved over the row groups of the workgroup
  int qt_idx[QT];
  bool qt_on[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    qt_idx[i] = mt * RG * QT + i * RG + rg;
    qt_on[i] = qt_idx[i] < nq_valid && k_begin < k_end;
  }
  const int wg_first_q = mt * RG * QT * 16;
  const bool wg_active = wg_first_q < rows_valid && k_begin < k_end;

  // ---------------------------------------------------------------- empty work
  if (!wg_active) {
    if (n_splits == 1) {
      // zero the output rows of this row tile (padding nodes / bad sequences)
      const int r0 = wg_first_q, r1 = min(M_cap, r0 + RG * QT * 16);
      for (int e = tid; e < (r1 - r0) * D; e += kThreads) {
        const int r = r0 + e / D, d = e % D;
        const int t = r / G, gq = r - t * G;
        out[(((size_t)b * T_cap + t) * H + g_kv * G + gq) * D + d] = (bf16_t)0.0f;
      }
    } else {
      const size_t ubase = (size_t)kv_unit * M_cap;
      const int r0 = wg_first_q, r1 = min(M_cap, r0 + RG * QT * 16);
      for (int r = r0 + tid; r < r1; r += kThreads) {
        part_m[ubase + r] = -INFINITY;
        part_l[ubase + r] = 0.0f;
      }
    }
    return;
  }

  // ---------------------------------------------------------------- Q fragments
  // B operand of S^T = K Q^T: lane (query l16, group lg) holds Q[row][32s + 8lg .. +8]
  bf16x8 qf[QT][KSTEPS];
  uint64_t mask0[QT], mask1[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    const int r = qt_idx[i] * 16 + l16;
    const int t = r / G;
    const int gq = r - t * G;
    const bool live = qt_on[i] && r < rows_valid;
    const bf16_t* qrow = q + (((size_t)b * T_cap + t) * H + g_kv * G + gq) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      if (live) {
        qf[i][s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * lg);
      } else {
        qf[i][s] = bf16x8{};
      }
    }
    mask0[i] = live ? anc[((size_t)b * T_cap + t) * n_words] : 0ull;
    mask1[i] = (live && n_words > 1) ? anc[((size_t)b * T_cap + t) * n_words + 1] : 0ull;
  }

  // ---------------------------------------------------------------- state
  f32x4 acc[QT][DT];
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
#pragma unroll
    for (int d = 0; d < DT; ++d) acc[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const bf16_t* kbase = kc + (size_t)bh * cache_cap * D;
  const bf16_t* vbase = vc + (size_t)bh * cache_cap * D;

  // ---------------------------------------------------------------- tile loader
  // K: 64 keys x D, unit = (key, 8-wide d octet); V: unit = (4 keys, d octet).
  constexpr int OCT = D / 8;
  constexpr int K_TOTAL = kKeyTile * OCT;                          // 16-byte K units per tile
  constexpr int V_TOTAL = (kKeyTile / 4) * OCT;                    // 4-key V units per tile
  constexpr int K_UNITS = (K_TOTAL + kThreads - 1) / kThreads;     // per thread
  constexpr int V_UNITS = (V_TOTAL + kThreads - 1) / kThreads;
  bf16x8 kreg[K_UNITS];
  bf16x8 vreg[V_UNITS][4];

  auto load_tile = [&](int kt0) {
#pragma unroll
    for (int u = 0; u < K_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int key = unit / OCT, oc = unit - (unit / OCT) * OCT;
      const int kidx = kt0 + key;
      kreg[u] = (unit < K_TOTAL && kidx < k_end)
                    ? *reinterpret_cast<const bf16x8*>(kbase + (size_t)kidx * D + oc * 8)
                    : bf16x8{};
    }
#pragma unroll
    for (int u = 0; u < V_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int kq = unit / OCT, oc = unit - (unit / OCT) * OCT;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kidx = kt0 + 4 * kq + j;
        vreg[u][j] = (unit < V_TOTAL && kidx < k_end)
                         ? *reinterpret_cast<const bf16x8*>(vbase + (size_t)kidx * D + oc * 8)
                         : bf16x8{};
      }
    }
  };
  auto store_tile = [&](int stage) {
    bf16_t* sk = smem + stage * Lds<D>::kStage;
    bf16_t* sv = sk + Lds<D>::kStageK;
#pragma unroll
    for (int u = 0; u < K_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      if (unit >= K_TOTAL) continue;
      const int key = unit / OCT, oc = unit - (unit / OCT) * OCT;
      *reinterpret_cast<bf16x8*>(sk + key * Lds<D>::kPitchK + oc * 8) = kreg[u];
    }
#pragma unroll
    for (int u = 0; u < V_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      if (unit >= V_TOTAL) continue;
      const int kq = unit / OCT, oc = unit - (unit / OCT) * OCT;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x4 w{vreg[u][0][e], vreg[u][1][e], vreg[u][2][e], vreg[u][3][e]};
        *reinterpret_cast<bf16x4*>(sv + (oc * 8 + e) * Lds<D>::kPitchV + 4 * kq) = w;
      }
    }
  };

  const int n_tiles = (k_end - k_begin + kKeyTile - 1) / kKeyTile;
  load_tile(k_begin);
  store_tile(0);
  __syncthreads();

  for (int it = 0; it < n_tiles; ++it) {
    const int kt0 = k_begin + it * kKeyTile;
    const bool more = it + 1 < n_tiles;
    if (more) load_tile(kt0 + kKeyTile);
    const bf16_t* sk = smem + (it & 1) * Lds<D>::kStage;
    const bf16_t* sv = sk + Lds<D>::kStageK;
    const int wkey0 = kg * KEYS_W;  // first key of this wave inside the tile
    const bool need_mask = kt0 + kKeyTile > ctx || kt0 + kKeyTile > k_end;

    // S^T = K Q^T for this wave's SUB sub-tiles
    f32x4 sacc[QT][SUB];
#pragma unroll
    for (int st = 0; st < SUB; ++st) {
      bf16x8 kf[KSTEPS];
      const bf16_t* krow = sk + (wkey0 + 16 * st + l16) * Lds<D>::kPitchK + 8 * lg;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(krow + 32 * s);
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        f32x4 c{0.f, 0.f, 0.f, 0.f};
        if (qt_on[i]) {
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) c = mfma16x16x32(kf[s], qf[i][s], c);
        }
        sacc[i][st] = c;
      }
    }

    // online softmax (exp2 form); lane owns query l16, keys 16*st + 4*lg + e
#pragma unroll
    for (int i = 0; i < QT; ++i) {
      if (!qt_on[i]) continue;
      float tmax = -INFINITY;
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s = sacc[i][st][e] * scale_log2;
          if (need_mask) {
            const int key = kt0 + wkey0 + 16 * st + 4 * lg + e;
            bool vis = key < k_end;
            if (vis && key >= ctx) {
              const int a = key - ctx;
              const uint64_t w = a < 64 ? mask0[i] : mask1[i];
              vis = (w >> (a & 63)) & 1ull;
            }
            if (!vis) s = -INFINITY;
          }
          sacc[i][st][e] = s;
          tmax = fmaxf(tmax, s);
        }
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, kWave));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, kWave));
      const float m_new = fmaxf(m_run[i], tmax);
      float alpha = 1.0f;
      if (m_new != -INFINITY) {
        alpha = __builtin_amdgcn_exp2f(m_run[i] - m_new);
      }
      float psum = 0.0f;
#pragma unroll
      for (int st = 0; st < SUB; ++st) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pv = m_new == -INFINITY ? 0.0f
                                              : __builtin_amdgcn_exp2f(sacc[i][st][e] - m_new);
          sacc[i][st][e] = pv;
          psum += pv;
        }
      }
      m_run[i] = m_new;
      l_run[i] = l_run[i] * alpha + psum;
#pragma unroll
      for (int d = 0; d < DT; ++d) acc[i][d] *= alpha;
    }

    // O^T += V^T P^T: one 32-key k-step pairs sub-tiles (2j, 2j+1)
#pragma unroll
    for (int j = 0; j < PV_STEPS; ++j) {
      bf16x8 pf[QT];
#pragma unroll
      for (int i = 0; i < QT; ++i) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[i][e] = (bf16_t)sacc[i][2 * j][e];
          pf[i][4 + e] = (bf16_t)sacc[i][2 * j + 1][e];
        }
      }
      const int key_a = wkey0 + 32 * j + 4 * lg;  // keys of sub-tile 2j owned by this lane group
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        const bf16_t* vrow = sv + (16 * d + l16) * Lds<D>::kPitchV;
        const bf16x4 lo = *reinterpret_cast<const bf16x4*>(vrow + key_a);
        const bf16x4 hi = *reinterpret_cast<const bf16x4*>(vrow + key_a + 16);
        const bf16x8 vf{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
        for (int i = 0; i < QT; ++i)
          if (qt_on[i]) acc[i][d] = mfma16x16x32(vf, pf[i], acc[i][d]);
      }
    }

    if (more) store_tile((it + 1) & 1);
    __syncthreads();
  }

  // ---------------------------------------------------------------- combine lanes
  // the 4 lane groups of a query hold partial sums over their own keys
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    l_run[i] += __shfl_xor(l_run[i], 16, kWave);
    l_run[i] += __shfl_xor(l_run[i], 32, kWave);
  }

  // ---------------------------------------------------------------- combine key groups
  if constexpr (KG == 2) {
    float* xs = reinterpret_cast<float*>(smem_raw);  // LDS reused after the loop
    // per row group: QT * (DT*4*64 acc floats + 64 m + 64 l)
    constexpr int PER_QT = DT * 4 * 64 + 128;
    float* mine = xs + rg * QT * PER_QT;
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        float* p = mine + i * PER_QT;
#pragma unroll
        for (int d = 0; d < DT; ++d)
#pragma unroll
          for (int e = 0; e < 4; ++e) p[(d * 4 + e) * 64 + lane] = acc[i][d][e];
        p[DT * 4 * 64 + lane] = m_run[i];
        p[DT * 4 * 64 + 64 + lane] = l_run[i];
      }
    }
    __syncthreads();
    if (kg == 1) return;
#pragma unroll
    for (int i = 0; i < QT; ++i) {
      const float* p = mine + i * PER_QT;
      const float m2 = p[DT * 4 * 64 + lane];
      const float l2 = p[DT * 4 * 64 + 64 + lane];
      const float m_new = fmaxf(m_run[i], m2);
      const float a1 = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
      const float a2 = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - m_new);
#pragma unroll
      for (int d = 0; d < DT; ++d)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][d][e] = acc[i][d][e] * a1 + p[(d * 4 + e) * 64 + lane] * a2;
      m_run[i] = m_new;
      l_run[i] = l_run[i] * a1 + l2 * a2;
    }
  }

  // ---------------------------------------------------------------- write
  // lane owns query l16 and output dims 16*d + 4*lg + e
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    const int r = qt_idx[i] * 16 + l16;
    if (qt_idx[i] * 16 >= M_cap || r >= M_cap) continue;
    const int t = r / G;
    const int gq = r - t * G;
    if (n_splits == 1) {
      bf16_t* orow = out + (((size_t)b * T_cap + t) * H + g_kv * G + gq) * D;
      const bool live = qt_on[i] && r < rows_valid;
      const float inv = (live && l_run[i] > 0.f) ? 1.0f / l_run[i] : 0.0f;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (bf16_t)(live ? acc[i][d][e] * inv : 0.0f);
        *reinterpret_cast<bf16x4*>(orow + 16 * d + 4 * lg) = o;
      }
    } else {
      const size_t ubase = (size_t)kv_unit * M_cap;
      const bool live = qt_on[i] && r < rows_valid;
      float* po = part_o + (ubase + r) * D;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        f32x4 o = live ? acc[i][d] : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(po + 16 * d + 4 * lg) = o;
      }
      if (lg == 0) {
        part_m[ubase + r] = live ? m_run[i] : -INFINITY;
        part_l[ubase + r] = live ? l_run[i] : 0.0f;
      }
    }
  }
}

// Combine the per-split partials of one (b, kv head, row) and write bf16 rows.
__global__ __launch_bounds__(256) void k_attn_merge(int B, int T_cap, int H, int Hkv, int D,
                                                    int cache_cap, int max_ctx, int n_splits,
                                                    const int32_t* __restrict__ ctx_len,
                                                    const int32_t* __restrict__ n_nodes,
                                                    const float* __restrict__ part_o,
                                                    const float* __restrict__ part_m,
                                                    const float* __restrict__ part_l,
                                                    bf16_t* __restrict__ out) {
  const int G = H / Hkv;
  const int M_cap = G * T_cap;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, g_kv = bh - (bh / Hkv) * Hkv;
  const int ctx = ctx_len[b], T = n_nodes[b];
  const bool bad = T < 1 || T > T_cap || ctx < 0 || ctx > max_ctx || ctx + T > cache_cap;
  const int rows_valid = bad ? 0 : G * T;
  const int per_block = 256 / D > 0 ? 256 / D : 1;
  const int r = blockIdx.x * per_block + threadIdx.x / D;
  const int d = threadIdx.x % D;
  if (r >= M_cap || threadIdx.x >= per_block * D) return;
  const int t = r / G, gq = r - t * G;
  float val = 0.0f;
  if (r < rows_valid) {
    float M = -INFINITY;
    for (int s = 0; s < n_splits; ++s) {
      const size_t u = (size_t)bh * n_splits + s;
      M = fmaxf(M, part_m[u * M_cap + r]);
    }
    float L = 0.0f, O = 0.0f;
    if (M != -INFINITY) {
      for (int s = 0; s < n_splits; ++s) {
        const size_t u = (size_t)bh * n_splits + s;
        const float ms = part_m[u * M_cap + r];
        if (ms == -INFINITY) continue;
        const float w = __builtin_amdgcn_exp2f(ms - M);
        L += part_l[u * M_cap + r] * w;
        O += part_o[(u * M_cap + r) * D + d] * w;
      }
    }
    val = L > 0.0f ? O / L : 0.0f;
  }
  out[(((size_t)b * T_cap + t) * H + g_kv * G + gq) * D + d] = (bf16_t)val;
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
  float m = -INFINITY, l = 0.0f;
  for (int j = 0; j < ctx + T; ++j) {
    if (j >= ctx) {
      const int a = j - ctx;
      if (!((arow[a >> 6] >> (a & 63)) & 1ull)) continue;
    }
    float part = 0.0f;
#pragma unroll
    for (int jj = 0; jj < MAXD; ++jj) {
      const int d = lane + 64 * jj;
      if (d < D) part += qv[jj] * kb[(size_t)j * D + d];
    }
    const float s = wave_sum_f32(part) * scale;
    const float m_new = fmaxf(m, s);
    const float alpha = __expf(m - m_new);
    const float p = __expf(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int jj = 0; jj < MAXD; ++jj) {
      const int d = lane + 64 * jj;
      if (d < D) acc[jj] = acc[jj] * alpha + p * vb[(size_t)j * D + d];
    }
    m = m_new;
  }
#pragma unroll
  for (int jj = 0; jj < MAXD; ++jj) {
    const int d = lane + 64 * jj;
    if (d < D) orow[d] = acc[jj] / l;
  }
}

template <int D, int QT, int KG>
int launch_bf16(const AttnPlan& p, int B, int T_cap, int H, int Hkv, int cache_cap, int max_ctx,
                const void* q, const void* k, const void* v, const int32_t* ctx_len,
                const int32_t* n_nodes, const uint64_t* anc, float scale_log2, void* out,
                float* po, float* pm, float* pl, int32_t* status, hipStream_t s) {
  auto kern = k_attn_bf16<D, QT, KG>;
  const int lds = Lds<D>::kBytes;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                      hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(kern, dim3(p.n_slots), dim3(kThreads), lds, s, B, T_cap, H, Hkv, cache_cap,
                     max_ctx, p.n_splits, p.tiles_per_split, p.n_kv, p.n_mt,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), ctx_len, n_nodes, anc, scale_log2,
                     static_cast<bf16_t*>(out), po, pm, pl, status);
  return launch_status();
}

template <int D>
int dispatch_bf16(const AttnPlan& p, int B, int T_cap, int H, int Hkv, int cache_cap,
                  int max_ctx, const void* q, const void* k, const void* v,
                  const int32_t* ctx_len, const int32_t* n_nodes, const uint64_t* anc,
                  float scale_log2, void* out, float* po, float* pm, float* pl, int32_t* status,
                  hipStream_t s) {
#define SPEC_ATTN_CASE(QT_, KG_)                                                              \
  if (p.QT == QT_ && p.KG == KG_)                                                             \
    return launch_bf16<D, QT_, KG_>(p, B, T_cap, H, Hkv, cache_cap, max_ctx, q, k, v, ctx_len, \
                                    n_nodes, anc, scale_log2, out, po, pm, pl, status, s);
  SPEC_ATTN_CASE(1, 2)
  SPEC_ATTN_CASE(2, 2)
  SPEC_ATTN_CASE(2, 1)
#undef SPEC_ATTN_CASE
  return SPEC_ERR_UNSUPPORTED;
}

}  // namespace
}  // namespace spec

using namespace spec;

extern "C" size_t spec_tree_attention_workspace_size(int dt, int B, int T_cap, int H, int Hkv,
                                                     int D, int max_ctx) {
  if (dt != SPEC_BF16 || B < 1 || T_cap < 1 || H < 1 || Hkv < 1 || H % Hkv || max_ctx < 0)
    return 0;
  const AttnPlan p = make_plan(B, T_cap, H, Hkv, max_ctx);
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
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16))
    return SPEC_ERR_INVALID;
  const AttnPlan p = make_plan(B, T_cap, H, Hkv, max_ctx);
  const size_t need = partial_bytes(p, B, T_cap, H, Hkv, D);
  float *po = nullptr, *pm = nullptr, *pl = nullptr;
  if (need) {
    if (!ws || ws_bytes < need || !aligned(ws, 256)) return SPEC_ERR_WORKSPACE;
    const size_t rows = (size_t)(H / Hkv) * T_cap;
    const size_t units = (size_t)B * Hkv * p.n_splits;
    char* w = static_cast<char*>(ws);
    po = reinterpret_cast<float*>(w);
    w += round_up(units * rows * D * sizeof(float), 256);
    pm = reinterpret_cast<float*>(w);
    w += round_up(units * rows * sizeof(float), 256);
    pl = reinterpret_cast<float*>(w);
  }
  const float scale_log2 = scale * kLog2e;
  int rc = D == 128 ? dispatch_bf16<128>(p, B, T_cap, H, Hkv, cache_cap, max_ctx, q, k_cache,
                                         v_cache, ctx_len, n_nodes, anc, scale_log2, out, po, pm,
                                         pl, status, s)
                    : dispatch_bf16<64>(p, B, T_cap, H, Hkv, cache_cap, max_ctx, q, k_cache,
                                        v_cache, ctx_len, n_nodes, anc, scale_log2, out, po, pm,
                                        pl, status, s);
  if (rc != SPEC_OK || p.n_splits <= 1) return rc;
  const int G = H / Hkv;
  const int per_block = 256 / D;
  dim3 grid((G * T_cap + per_block - 1) / per_block, B * Hkv);
  hipLaunchKernelGGL(k_attn_merge, grid, dim3(256), 0, s, B, T_cap, H, Hkv, D, cache_cap,
                     max_ctx, p.n_splits, ctx_len, n_nodes, po, pm, pl,
                     static_cast<bf16_t*>(out));
  return launch_status();
}
