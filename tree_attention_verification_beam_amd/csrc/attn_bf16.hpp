// attn_bf16.hpp -- the bf16 MFMA kernel of the tree attention and its
// launcher, shared by the compile units that instantiate its plans: the
// register-staged plans in tree_attention.hip (which states the method and
// chooses the plan) and the direct-to-LDS plan in attn_direct.hip, which the
// build compiles with a scheduling strategy of its own.
//
// The kernel computes the one forward pass over the packed tree of
// "Recurrent Drafter for Fast Speculative Decoding in Large Language Models",
// section "The Full Speculative Decoding Loop", Step 4, under the ancestor
// mask of "Clover: Regressive Lightweight Speculative Decoding with
// Sequential Knowledge" (causal mask construction).
#pragma once
#include "common.hpp"
#include "tile_mask.hpp"

namespace spec {
namespace attn {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kKeyTile = 64;      // keys per LDS stage
constexpr float kRescale = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 for raw 32-bit-format loads (gfx9 family)

// ------------------------------------------------------------------ bf16 MFMA kernel

// Key order and LDS layout of one 32-key chunk.  Row m of the S^T MFMA's
// sub-tile st (m = 4 q + r) is the chunk key 8 q + 4 (st ^ h(q)) + r, with
// h(q) = (q >> 1) & 1.  The lane group q of the output then holds 8 of the
// chunk's keys, 8 q .. 8 q + 7, so its P values form one 16-byte operand read
// of a transposed V row, provided V^T stores key k at column vcol(k) below,
// which swaps the two 4-key halves of every 8-key block with h = 1.  The row
// pitches and the V^T row swizzle swz keep the K operand reads, the V^T
// stores and the V^T operand reads of a wave free of bank conflicts.  The
// pitches come from a conflict rule measured on gfx950 with
// SQ_LDS_BANK_CONFLICT: 64 banks of 4 bytes; a 16-byte read is served in four
// passes of 16 lanes, and a bank group hit from different lane positions in
// different passes costs extra passes.  Rows of D + 16 and 64 + 16 elements
// read these patterns conflict-free; D + 8 and 64 + 8 read them 2-way.
template <int D>
struct Lds {
  static constexpr int kPitchK = D + 16;         // bf16 elements per K row
  static constexpr int kPitchV = kKeyTile + 16;  // bf16 elements per transposed V row
  static __device__ constexpr int swz(int row) { return ((row >> 4) & 7) * 8; }
  static __device__ constexpr int vcol(int key, int row) {
    return key ^ (((key >> 4) & 1) * 4) ^ swz(row);
  }
  static constexpr int kStageK = kKeyTile * kPitchK;
  static constexpr int kStageV = D * kPitchV;
  static constexpr int kStage = kStageK + kStageV;
  static constexpr int kBytes = 2 * kStage * 2;  // two stages of bf16
};

// Direct-to-LDS layout (one key group, D = 128): a stage holds the tile's K
// and V rows as loaded, 64 rows of 256 bytes each, K first.  A 16-byte load
// writes lane l's bytes at slot l of a 1 KB block (four rows), so the layout
// is row-major with no padding; instead the 16-byte chunk c of key row k sits
// at position c ^ swz(k) of its row, swz(k) = 2 ((k & 3) | ((k >> 3) & 1) << 2).
// With it the K operand reads (16 bytes) and the V operand reads (transposing
// 8-byte reads of 16-bit elements) are free of bank conflicts (measured on
// gfx950 with SQ_LDS_BANK_CONFLICT).
struct LdsDirect {
  static constexpr int kRow = 256;                 // bytes per key row
  static constexpr int kStageK = kKeyTile * kRow;  // 16 KB
  static constexpr int kStage = 2 * kStageK;       // K + V
  static __device__ constexpr int swz(int key) { return ((key & 3) << 1) | (((key >> 3) & 1) << 3); }
};

struct AttnArgs {
  int B, T_cap, H, Hkv, cache_cap, max_ctx, n_splits, tiles_per_split, n_kv, n_mt;
  float scale_log2;
  const bf16_t* q;
  const bf16_t* kc;
  const bf16_t* vc;
  const int32_t* ctx_len;
  const int32_t* n_nodes;
  const uint64_t* anc;
  bf16_t* out;
  float* part_o;
  float* part_m;
  float* part_l;
  int32_t* status;
};

__device__ inline f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Workgroup barrier for LDS hand-over: waits for this wave's LDS operations
// only (not its outstanding global loads, which may stay in flight across it).
__device__ inline void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N vector memory operations of this wave are outstanding
// (loads into LDS complete in issue order).
template <int N>
__device__ inline void wait_loads() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One 16-byte-per-lane load into LDS: lane l's bytes land at LDS byte address
// lds + 16 l; the buffer resource's range check returns zeros past its end.
// Written in assembly so that the compiler's wait insertion does not take the
// loads for pending writes to all of LDS (it would then wait for them before
// every transposing read): the kernel waits for them itself (wait_loads)
// before the barrier that hands a stage over.  M0 carries the LDS address and
// is restored; the leading s_nop covers a VALU write of the resource's SGPRs
// (5 wait states), the one after the M0 write the LDS-DMA hazard.
template <bool NT>
__device__ inline void load_lds_b128(u32x4 rsrc, unsigned lds, int voffset) {
  unsigned saved;
  if constexpr (NT)
    asm volatile("s_nop 4\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen nt lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
  else
    asm volatile("s_nop 4\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, 0 offen lds\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(lds), "v"(voffset), "s"(rsrc) : "memory");
}

// Map a workgroup slot to (kv unit, row block) so that the row blocks sharing
// one key stream land on the same XCD (slots are dealt round-robin over 8 XCDs).
__device__ inline void slot_to_work(int slot, int n_mt, int& kv_unit, int& mt) {
  const int xcd = slot & 7;
  const int j = slot >> 3;
  kv_unit = xcd + 8 * (j / n_mt);
  mt = j - (j / n_mt) * n_mt;
}

template <int S>
struct StageC {
  static constexpr int value = S;
};

template <int D, int NW, int QT, int KG, int PF, int NS, bool ONCE>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void k_attn_bf16(AttnArgs a) {
  constexpr int kThreads = NW * 64;
  constexpr bool DL = NS > 0;  // direct-to-LDS tiles
  static_assert(!DL || (KG == 1 && D == 128 && NS == 2), "direct-load plans: one key group, D = 128, two stages");
  constexpr int RG = NW / KG;           // row groups
  constexpr int KSTEPS = D / 32;        // k-steps of Q K^T
  constexpr int DT = D / 16;            // 16-wide d tiles of the output
  constexpr int KEYS_W = kKeyTile / KG; // keys per wave per tile
  constexpr int PV_STEPS = KEYS_W / 32; // 32-key k-steps of P V per tile
  static_assert(KG == 1 || KG == 2, "key groups");
  static_assert(NW % KG == 0, "waves per key group");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  bf16_t* smem = reinterpret_cast<bf16_t*>(smem_raw);

  int kv_unit, mt;
  slot_to_work(blockIdx.x, a.n_mt, kv_unit, mt);
  if (kv_unit >= a.n_kv) return;
  const int n_splits = a.n_splits;
  const int sp = kv_unit % n_splits;
  const int bh = kv_unit / n_splits;
  const int Hkv = a.Hkv, T_cap = a.T_cap, H = a.H;
  const int b = bh / Hkv;
  const int g_kv = bh - b * Hkv;
  const int G = H / Hkv;
  const int M_cap = G * T_cap;
  const int n_words = (T_cap + 63) / 64;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps per-wave choices scalar
  const int lane = tid & 63;
  const int rg = wave / KG;
  const int kg = wave - rg * KG;
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  // Everything this workgroup reads before its first tile is issued here, in
  // one round trip: the sequence's lengths, the Q fragments and ancestor words
  // of its rows (row indices clamped into the tensors; rows that turn out dead
  // are zeroed below) and the first key tile (clamped into the cache; keys past
  // the range are zeroed before they reach LDS).
  const int ctx = a.ctx_len[b];
  const int T = a.n_nodes[b];
  const bf16_t* kbase = a.kc + (size_t)bh * a.cache_cap * D;
  const bf16_t* vbase = a.vc + (size_t)bh * a.cache_cap * D;
  const int k_begin = sp * a.tiles_per_split * kKeyTile;

  // ---------------------------------------------------------------- tile loader
  // K: 64 keys x D, unit = (key, 8-wide d octet); V: unit = (VK keys, d octet),
  // sized so every thread owns exactly one V unit.  A tile is read with buffer
  // loads through a resource that starts at the tile's first key and ends at
  // `limit` keys: every thread's byte offset inside a tile is fixed, the
  // resource is built with scalar ops, and the hardware range check returns
  // zeros for keys at or past `limit`.  So the loads never branch or clamp (a
  // full and a partial tile run the same code, and prefetched loads stay in
  // flight), and keys past the range reach LDS as zeros, to be masked to -inf
  // before the softmax.  PF register sets keep PF tiles in flight.  When this
  // workgroup is the only reader of its key range (one row block), the loads
  // are non-temporal.
  constexpr int OCT = D / 8;
  constexpr int K_TOTAL = kKeyTile * OCT;                          // 16-byte K units per tile
  constexpr int K_UNITS = K_TOTAL / kThreads;                      // per thread
  constexpr int VK = kKeyTile * OCT / kThreads;                    // keys per V unit
  static_assert(K_TOTAL % kThreads == 0 && VK >= 1 && VK <= 4, "tile split");
  constexpr int kRowBytes = D * 2;
  constexpr int kCpol = ONCE ? kLoadOnce : 0;

  int koff[K_UNITS], voff[VK];  // byte offsets inside a tile
#pragma unroll
  for (int u = 0; u < K_UNITS; ++u) {
    const int unit = tid + u * kThreads;
    koff[u] = (unit / OCT) * kRowBytes + (unit % OCT) * 16;
  }
#pragma unroll
  for (int j = 0; j < VK; ++j) voff[j] = (VK * (tid / OCT) + j) * kRowBytes + (tid % OCT) * 16;

  auto tile_rsrc = [&](const bf16_t* base, int kt0, int limit) {
    const int rows = limit - kt0 > 0 ? limit - kt0 : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(base + (size_t)kt0 * D), (short)0,
                                             rows * kRowBytes, kBufferWord3);
  };
  auto load_tile = [&](bf16x8 (&kr)[K_UNITS], bf16x8 (&vr)[VK], int kt0, int limit) {
    const auto rk = tile_rsrc(kbase, kt0, limit);
    const auto rv = tile_rsrc(vbase, kt0, limit);
#pragma unroll
    for (int u = 0; u < K_UNITS; ++u)
      kr[u] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, koff[u], 0, kCpol));
#pragma unroll
    for (int j = 0; j < VK; ++j)
      vr[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[j], 0, kCpol));
  };
  // zero the keys of a speculatively loaded tile that lie past `last` (cache
  // slots past the sequence may hold any bits, NaN included)
  auto sanitize_tile = [&](bf16x8 (&kr)[K_UNITS], bf16x8 (&vr)[VK], int kt0, int last) {
#pragma unroll
    for (int u = 0; u < K_UNITS; ++u) {
      const int key = (tid + u * kThreads) / OCT;
      if (kt0 + key > last) kr[u] = bf16x8{};
    }
    const int kq = tid / OCT;
#pragma unroll
    for (int j = 0; j < VK; ++j)
      if (kt0 + VK * kq + j > last) vr[j] = bf16x8{};
  };

  // Direct-to-LDS loads: the tile's K (and V) rows form 16 blocks of 1 KB
  // (four rows); wave w issues blocks w, w + NW, ...  Lane l of a block loads
  // the chunk that belongs at slot l (row 4 R + l / 16, position l % 16), so
  // the swizzle costs nothing; every voffset is fixed per thread.
  constexpr int DL_BLOCKS = DL ? kKeyTile * LdsDirect::kRow / 1024 / NW : 1;  // per wave, K or V
  int dl_off[DL_BLOCKS];
  if constexpr (DL) {
#pragma unroll
    for (int u = 0; u < DL_BLOCKS; ++u) {
      const int row = 4 * (u * NW + wave) + (lane >> 4);
      dl_off[u] = row * LdsDirect::kRow + 16 * ((lane & 15) ^ LdsDirect::swz(row));
    }
  }
  const unsigned lds0 = (unsigned)(size_t)((__attribute__((address_space(3))) unsigned char*)smem_raw);
  auto rsrc_words = [&](const bf16_t* base, int kt0, int limit) {
    const int rows = limit - kt0 > 0 ? limit - kt0 : 0;
    const unsigned long long addr = (unsigned long long)(base + (size_t)kt0 * D);
    return u32x4{(unsigned)addr, (unsigned)(addr >> 32) & 0xffffu, (unsigned)(rows * kRowBytes),
                 (unsigned)kBufferWord3};
  };
  auto issue_tile = [&](int stage, int kt0, int limit) {
    const u32x4 rk = rsrc_words(kbase, kt0, limit);
    const u32x4 rv = rsrc_words(vbase, kt0, limit);
    const unsigned st = lds0 + stage * LdsDirect::kStage;
#pragma unroll
    for (int u = 0; u < DL_BLOCKS; ++u) {
      const unsigned blk = st + (u * NW + wave) * 1024;
      load_lds_b128<ONCE>(rk, blk, dl_off[u]);
      load_lds_b128<ONCE>(rv, blk + LdsDirect::kStageK, dl_off[u]);
    }
  };
  // K or V rows alone (the pipelined loop keeps K one tile ahead of V)
  auto issue_rows = [&](const bf16_t* base, int stage, bool v_part, int kt0, int limit) {
    const u32x4 rs = rsrc_words(base, kt0, limit);
    const unsigned st = lds0 + stage * LdsDirect::kStage + (v_part ? LdsDirect::kStageK : 0);
#pragma unroll
    for (int u = 0; u < DL_BLOCKS; ++u) load_lds_b128<ONCE>(rs, st + (u * NW + wave) * 1024, dl_off[u]);
  };

  bf16x8 kA[DL ? 1 : K_UNITS], vA[DL ? 1 : VK];
  if constexpr (DL)
    issue_tile(0, k_begin, a.cache_cap);  // every cache slot: rows past the range zeroed below
  else
    load_tile(kA, vA, k_begin, a.cache_cap);  // every cache slot: sanitized below

  // Q fragments: B operand of S^T = K Q^T; lane (query l16, group lg) holds
  // Q[row][32s + 8lg .. +8]
  int qt_idx[QT];
  bf16x8 qf[QT][KSTEPS];
  uint64_t mask0[QT], mask1[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    qt_idx[i] = mt * RG * QT + rg * QT + i;
    const int r = min(qt_idx[i] * 16 + l16, M_cap - 1);
    const int t = r / G;
    const int gq = r - t * G;
    const bf16_t* qrow = a.q + (((size_t)b * T_cap + t) * H + g_kv * G + gq) * D;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[i][s] = *reinterpret_cast<const bf16x8*>(qrow + 32 * s + 8 * lg);
    mask0[i] = a.anc[((size_t)b * T_cap + t) * n_words];
    mask1[i] = n_words > 1 ? a.anc[((size_t)b * T_cap + t) * n_words + 1] : 0ull;
  }

  const bool bad =
      T < 1 || T > T_cap || ctx < 0 || ctx > a.max_ctx || ctx + T > a.cache_cap;
  const int rows_valid = bad ? 0 : G * T;
  const int nq_valid = (rows_valid + 15) >> 4;
  const int n_keys = ctx + T;
  int k_end = k_begin + a.tiles_per_split * kKeyTile;
  if (k_end > n_keys) k_end = n_keys;
  if (bad && sp == 0 && mt == 0 && tid == 0) raise_status(a.status, SPEC_DEV_CTX_RANGE);

  // this wave's query tiles: consecutive tiles of the row block per row group,
  // so the dead tiles past a short sequence's rows fall on whole waves, which
  // skip their tile work and leave their SIMD to the other waves
  bool qt_on[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    qt_on[i] = qt_idx[i] < nq_valid && k_begin < k_end;
    const int r = qt_idx[i] * 16 + l16;
    const bool live = qt_on[i] && r < rows_valid;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qf[i][s] = live ? qf[i][s] : bf16x8{};
    mask0[i] = live ? mask0[i] : 0ull;
    mask1[i] = live ? mask1[i] : 0ull;
  }
  bool wave_on = false;
#pragma unroll
  for (int i = 0; i < QT; ++i) wave_on = wave_on || qt_on[i];
  const int wg_first_row = mt * RG * QT * 16;
  const int wg_end_row = min(M_cap, wg_first_row + RG * QT * 16);
  const bool wg_active = wg_first_row < rows_valid && k_begin < k_end;

  // ---------------------------------------------------------------- empty work
  if (!wg_active) {
    if (n_splits == 1) {
      // zero the output rows of this row block (padding nodes / bad sequences)
      for (int e = tid; e < (wg_end_row - wg_first_row) * D; e += kThreads) {
        const int r = wg_first_row + e / D, d = e % D;
        const int t = r / G, gq = r - t * G;
        a.out[(((size_t)b * T_cap + t) * H + g_kv * G + gq) * D + d] = (bf16_t)0.0f;
      }
    } else {
      const size_t ubase = (size_t)kv_unit * M_cap;
      for (int r = wg_first_row + tid; r < wg_end_row; r += kThreads) {
        a.part_m[ubase + r] = -INFINITY;
        a.part_l[ubase + r] = 0.0f;
      }
    }
    if constexpr (DL) wait_loads<0>();  // no load into LDS outlives the workgroup
    return;
  }
  const int klast = k_end - 1;
  if constexpr (!DL) sanitize_tile(kA, vA, k_begin, klast);

  // ---------------------------------------------------------------- state
  f32x4 acc[QT][DT];
  // l_run: each lane's fp32 sum of its own exponentials (before bf16 rounding);
  // the 4 lane groups holding a query are added after the key loop.  An extra
  // MFMA per chunk against an all-ones operand gives the same sums complete in
  // every lane, but the kernel ran slower with it on every plan.
  float m_run[QT], l_run[QT];
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
#pragma unroll
    for (int d = 0; d < DT; ++d) acc[i][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto store_tile = [&](const bf16x8 (&kr)[K_UNITS], const bf16x8 (&vr)[VK], int stage) {
    bf16_t* sk = smem + stage * Lds<D>::kStage;
    bf16_t* sv = sk + Lds<D>::kStageK;
#pragma unroll
    for (int u = 0; u < K_UNITS; ++u) {
      const int unit = tid + u * kThreads;
      const int key = unit / OCT, oc = unit - (unit / OCT) * OCT;
      *reinterpret_cast<bf16x8*>(sk + key * Lds<D>::kPitchK + oc * 8) = kr[u];
    }
    const int kq = tid / OCT, oc = tid - (tid / OCT) * OCT;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int row = oc * 8 + e;
      bf16_t* dst = sv + row * Lds<D>::kPitchV + Lds<D>::vcol(VK * kq, row);
      if constexpr (VK == 4) {
        *reinterpret_cast<bf16x4*>(dst) = bf16x4{vr[0][e], vr[1][e], vr[2][e], vr[3][e]};
      } else if constexpr (VK == 2) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<bf16x2*>(dst) = bf16x2{vr[0][e], vr[1][e]};
      } else {
        *dst = vr[0][e];
      }
    }
  };

  const float c = a.scale_log2;
  const int wkey0 = kg * KEYS_W;  // first key of this wave inside a tile

  // One 64-key tile from LDS stage `stage` (first key kt0).  Each 32-key chunk of
  // this wave's keys: S^T = K Q^T (two 16-key sub-tiles), online softmax, then
  // O^T += V^T P^T with the chunk as one 32-key k-step.
  // Visibility of the 64 keys of the tile at kt0 for query tile i of this lane,
  // bit p <-> key kt0 + p: context keys before ctx, tree keys whose ancestor bit
  // is set, and nothing at or past k_end.  All shift amounts are uniform.
  auto tile_vis = [&](int i, int kt0) -> uint64_t {
    return tile_vis_bits(ctx - kt0, k_end - kt0, mask0[i], mask1[i]);
  };

  // Direct-load operand addresses (bytes inside a stage).  K: lane (l16, lg)
  // reads key 32 j + 8 q + 4 st + r (q = l16 / 4, r = l16 % 4) at chunk
  // 4 s + lg.  V^T: each transposing read covers 16 rows of 4 elements per
  // 16-lane group; lane r of group lg names row (key 32 j + 8 lg + 4 hf + r / 4,
  // dims 16 dt + 4 (r % 4) .. + 3), and lane m of the group receives the four
  // keys' values of dim 16 dt + m, that is elements 4 hf .. 4 hf + 3 of its
  // V^T operand.
  int dl_k[DL ? KSTEPS : 1], dl_v[DL ? DT : 1];
  if constexpr (DL) {
    const int q = l16 >> 2, r = l16 & 3;
    const int swk = LdsDirect::swz(8 * q + r);
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) dl_k[s] = (8 * q + r) * LdsDirect::kRow + 16 * ((4 * s + lg) ^ swk);
    const int ra = l16 & 3, rk = l16 >> 2;
    const int s2 = LdsDirect::swz(8 * lg + rk) >> 1;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      dl_v[dt] = LdsDirect::kStageK + (8 * lg + rk) * LdsDirect::kRow + 32 * (dt ^ s2) + 8 * ra;
  }

  // One 64-key tile in three phases: the scores S^T = K Q^T of all this
  // wave's keys of the tile (per 32-key chunk j, two 16-key sub-tiles st), one
  // online-softmax step over them (one maximum check and rescale per tile),
  // then O^T += V^T P^T with each chunk as one 32-key k-step.  The pipelined
  // loop below runs the scores of the next tile beside the softmax and P V of
  // this one.
  typedef f32x4 Scores[PV_STEPS][QT][2];
  typedef bf16x8 Probs[PV_STEPS][QT];
  // K of the tile in LDS stage `stage`
  auto tile_scores = [&](int stage, Scores& sacc) {
    const bf16_t* sk = smem + stage * Lds<D>::kStage;
    const unsigned char* sb = smem_raw + stage * LdsDirect::kStage;
    (void)sk; (void)sb;
#pragma unroll
    for (int j = 0; j < PV_STEPS; ++j) {
      const int ck0 = wkey0 + 32 * j;  // first key of the chunk inside the tile
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        bf16x8 kf[KSTEPS];
        if constexpr (DL) {
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s)
            kf[s] = *reinterpret_cast<const bf16x8*>(sb + dl_k[s] + ck0 * LdsDirect::kRow + st * 4 * LdsDirect::kRow);
        } else {
          const int q = l16 >> 2;
          const int kk = ck0 + 8 * q + 4 * (st ^ ((q >> 1) & 1)) + (l16 & 3);  // this lane's key row
          const bf16_t* krow = sk + kk * Lds<D>::kPitchK + 8 * lg;
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(krow + 32 * s);
        }
#pragma unroll
        for (int i = 0; i < QT; ++i) {
          // a dead tile of a live wave has zero Q: its scores are computed
          // and discarded (its rows are never written)
          f32x4 cc{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KSTEPS; ++s) cc = mfma16x16x32(kf[s], qf[i][s], cc);
          sacc[j][i][st] = cc;
        }
      }
    }
  };

  // the tile's first key is kt0
  auto tile_softmax = [&](int kt0, Scores& sacc, Probs& pf) {
    const bool need_mask = kt0 + kKeyTile > ctx || kt0 + kKeyTile > k_end;
    // keys past the range or outside the node's ancestor set score -inf; this
    // lane's keys of chunk j are wkey0 + 32 j + 8 lg + 4 (st ^ h) + e (h = 0
    // for the direct-load layout, else (lg >> 1) & 1); bit 32 j + 4 st + e of
    // lvis[i] is that key's
    if (need_mask) {
      uint64_t lvis[QT];
#pragma unroll
      for (int i = 0; i < QT; ++i)
        lvis[i] = DL ? lane_vis_bits_direct(tile_vis(i, kt0), lg) : lane_vis_bits(tile_vis(i, kt0), wkey0, lg);
#pragma unroll
      for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
        for (int i = 0; i < QT; ++i)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int c = 32 * j + 4 * st + e;  // compile-time bit position
              const uint32_t word = c < 32 ? (uint32_t)lvis[i] : (uint32_t)(lvis[i] >> 32);
              const bool vis = (word >> (c & 31)) & 1u;
              sacc[j][i][st][e] = vis ? sacc[j][i][st][e] : -INFINITY;
            }
    }

    if constexpr (DL) {
      // online softmax in exp2 form; lane owns query l16 and, in chunk j, keys
      // wkey0 + 32 j + 8 lg + 4 (st ^ h) + e.  The exponentials are taken
      // against the running maximum first, and the maximum moves only when one
      // of them exceeds 2^kRescale (or on a row's first tile): an integer
      // maximum over the bit patterns of these non-negative values orders them
      // as floats and, unlike a float maximum of the MFMA results, needs no
      // quieting of each operand.  A growing query tile then takes its row
      // maximum (the 4 lane groups holding the row agree on it), rescales its
      // accumulators and takes its exponentials again; one uniform branch
      // covers every query tile's rescale.
      static_assert(kRescale == 8.0f, "growth threshold bits below");
      constexpr uint32_t kGrowBits = 0x43800000u;  // 2^kRescale as fp32 bits
      bool grow[QT];
      bool any_grow = false;
      float psum[QT];
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        const float nmu = m_run[i] == -INFINITY ? 0.0f : -m_run[i];
        uint32_t pmax = 0u;
        psum[i] = 0.0f;
#pragma unroll
        for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][i][st][e], c, nmu));
              pf[j][i][4 * st + e] = (bf16_t)pv;
              pmax = max(pmax, __builtin_bit_cast(uint32_t, pv));
              psum[i] += pv;
            }
        grow[i] = __builtin_amdgcn_ballot_w64(pmax > kGrowBits || m_run[i] == -INFINITY) != 0ull;
        any_grow = any_grow || grow[i];
      }
      if (any_grow) {
#pragma unroll
        for (int i = 0; i < QT; ++i) {
          if (!grow[i]) continue;
          float lmax = -INFINITY;
#pragma unroll
          for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int e = 0; e < 4; ++e) lmax = fmaxf(lmax, sacc[j][i][st][e]);
          lmax *= c;
          float tmax = fmaxf(lmax, partner_f32<4>(lmax));  // lane l ^ 16
          tmax = fmaxf(tmax, partner_f32<5>(tmax));        // lane l ^ 32
          const float m_new = fmaxf(m_run[i], tmax);
          const float alpha =
              (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
          l_run[i] *= alpha;
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[i][d] *= alpha;
          m_run[i] = m_new;
          const float nmu = m_new == -INFINITY ? 0.0f : -m_new;
          psum[i] = 0.0f;
#pragma unroll
          for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][i][st][e], c, nmu));
                pf[j][i][4 * st + e] = (bf16_t)pv;
                psum[i] += pv;
              }
        }
      }
#pragma unroll
      for (int i = 0; i < QT; ++i) l_run[i] += psum[i];
    } else {
      // online softmax in exp2 form; lane owns query l16 and, in chunk j, keys
      // wkey0 + 32 j + 8 lg + 4 (st ^ h) + e.  A row maximum moves only when some
      // lane outgrew it by 2^kRescale; then the 4 lane groups holding the row
      // agree on the new maximum.  One uniform branch covers every query tile's
      // rescale, so the exponentials of all tiles share one basic block with
      // whatever MFMA work follows.
      float lmax[QT];
      bool grow[QT];
      bool any_grow = false;
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        lmax[i] = -INFINITY;
#pragma unroll
        for (int j = 0; j < PV_STEPS; ++j)
          lmax[i] = fmaxf(lmax[i], fmaxf(fmaxf(fmaxf(sacc[j][i][0][0], sacc[j][i][0][1]),
                                               fmaxf(sacc[j][i][0][2], sacc[j][i][0][3])),
                                         fmaxf(fmaxf(sacc[j][i][1][0], sacc[j][i][1][1]),
                                               fmaxf(sacc[j][i][1][2], sacc[j][i][1][3]))));
        lmax[i] *= c;
        grow[i] = __builtin_amdgcn_ballot_w64(lmax[i] > m_run[i] + kRescale) != 0ull;
        any_grow = any_grow || grow[i];
      }
      if (any_grow) {
#pragma unroll
        for (int i = 0; i < QT; ++i) {
          if (!grow[i]) continue;
          float tmax = fmaxf(lmax[i], partner_f32<4>(lmax[i]));  // lane l ^ 16
          tmax = fmaxf(tmax, partner_f32<5>(tmax));              // lane l ^ 32
          const float m_new = fmaxf(m_run[i], tmax);
          const float alpha =
              (m_new == -INFINITY) ? 1.0f : __builtin_amdgcn_exp2f(m_run[i] - m_new);
          l_run[i] *= alpha;
#pragma unroll
          for (int d = 0; d < DT; ++d) acc[i][d] *= alpha;
          m_run[i] = m_new;
        }
      }
#pragma unroll
      for (int i = 0; i < QT; ++i) {
        const float nmu = m_run[i] == -INFINITY ? 0.0f : -m_run[i];
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[j][i][st][e], c, nmu));
              pf[j][i][4 * st + e] = (bf16_t)pv;
              psum += pv;
            }
        l_run[i] += psum;
      }
    }
  };

  // V of the tile in LDS stage `stage`.  O^T += V^T P^T over the tile: in
  // chunk j this lane's 8 P values are the keys wkey0 + 32 j + 8 lg .. + 7 in
  // V^T column order
  auto tile_pv = [&](int stage, const Probs& pf) {
    const bf16_t* sv = smem + stage * Lds<D>::kStage + Lds<D>::kStageK;
    const unsigned char* sb = smem_raw + stage * LdsDirect::kStage;
    (void)sv; (void)sb;
#pragma unroll
    for (int j = 0; j < PV_STEPS; ++j) {
      const int ck0 = wkey0 + 32 * j;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        bf16x8 vf;
        if constexpr (DL) {
          typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
          const unsigned char* vp = sb + dl_v[d] + ck0 * LdsDirect::kRow;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 4 * LdsDirect::kRow));
          vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          const bf16_t* vrow = sv + (16 * d + l16) * Lds<D>::kPitchV;
          const int sw = Lds<D>::swz(16 * d);  // the same for rows 16d .. 16d+15
          vf = *reinterpret_cast<const bf16x8*>(vrow + ((ck0 + 8 * lg) ^ sw));
        }
#pragma unroll
        for (int i = 0; i < QT; ++i) acc[i][d] = mfma16x16x32(vf, pf[j][i], acc[i][d]);
      }
    }
  };

  auto compute_tile = [&](int stage, int kt0) {
    if (!wave_on) return;  // no live query tile in this wave (uniform)
    Scores sacc;
    Probs pf;
    tile_scores(stage, sacc);
    tile_softmax(kt0, sacc, pf);
    tile_pv(stage, pf);
  };

  // ---------------------------------------------------------------- key loop
  // LDS double buffer; PF tiles of global loads in flight.  The barrier waits
  // for this wave's LDS traffic only, so prefetched global loads stay in flight.
  const int n_tiles = (k_end - k_begin + kKeyTile - 1) / kKeyTile;
  if constexpr (DL) {
    // Two LDS stages, K one tile ahead of V.  The scores of tile it + 1 are
    // computed in the iteration that finishes tile it, beside its softmax and
    // P V, so a wave has MFMA and VALU work of two tiles to interleave.
    // Iteration it reads K of tile it + 1 (stage (it + 1) & 1) and V of tile
    // it (stage it & 1), and first loads K of tile it + 2 and V of tile it + 1
    // into the stages whose K and V the previous iteration finished reading.
    for (int t = 1; t < NS; ++t) issue_rows(kbase, t % NS, false, k_begin + t * kKeyTile, k_end);
    for (int t = 1; t < NS - 1; ++t) issue_rows(vbase, t % NS, true, k_begin + t * kKeyTile, k_end);
    wait_loads<0>();
    if (k_begin + kKeyTile > k_end) {
      // tile 0 was loaded over every cache slot: zero its rows past the range
      // (cache slots past the sequence may hold any bits, NaN included)
      lds_barrier();
      const int n_in = k_end - k_begin;
      for (int e = tid; e < (kKeyTile - n_in) * 32; e += kThreads) {
        const int row = n_in + (e >> 5), part = e & 31;  // 16 chunks of K, then 16 of V
        *reinterpret_cast<u32x4*>(smem_raw + (part >> 4) * LdsDirect::kStageK + row * LdsDirect::kRow +
                                  16 * (part & 15)) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    lds_barrier();
    Scores sacc;
    if (wave_on) tile_scores(0, sacc);
    lds_barrier();  // K of tile 0 is read before K of tile NS replaces it
    // one iteration per tile, unrolled by the two stages so that every LDS
    // address is a constant offset from a per-lane base
    auto dl_iter = [&](auto cur_c, int it) {
      constexpr int cur = decltype(cur_c)::value, nxt = 1 - cur;
      issue_rows(kbase, cur, false, k_begin + (it + NS) * kKeyTile, k_end);
      issue_rows(vbase, nxt, true, k_begin + (it + NS - 1) * kKeyTile, k_end);
      if (wave_on) {
        Probs pf;
        tile_softmax(k_begin + it * kKeyTile, sacc, pf);
        Scores snext;
        tile_scores(nxt, snext);  // past the last tile: zeros, unused
        tile_pv(cur, pf);
#pragma unroll
        for (int j = 0; j < PV_STEPS; ++j)
#pragma unroll
          for (int i = 0; i < QT; ++i)
#pragma unroll
            for (int st = 0; st < 2; ++st) sacc[j][i][st] = snext[j][i][st];
      }
      // K of tile it + 2 and V of tile it + 1 have landed
      wait_loads<0>();
      lds_barrier();
    };
    int it = 0;
#pragma unroll 1
    for (; it + 2 <= n_tiles; it += 2) {
      dl_iter(StageC<0>{}, it);
      dl_iter(StageC<1>{}, it + 1);
    }
    if (it < n_tiles) dl_iter(StageC<0>{}, it);
    wait_loads<0>();
  } else if constexpr (PF == 1) {
    store_tile(kA, vA, 0);
    lds_barrier();
#pragma unroll 1
    for (int it = 0; it < n_tiles; ++it) {
      const int kt0 = k_begin + it * kKeyTile;
      const bool more = it + 1 < n_tiles;
      if (more) load_tile(kA, vA, kt0 + kKeyTile, k_end);
      compute_tile(it & 1, kt0);
      if (more) store_tile(kA, vA, (it + 1) & 1);
      lds_barrier();
    }
  } else {
    // Two register sets (A: even tiles, B: odd tiles) alternate over the two
    // LDS stages.  Loads are unconditional (indices clamp to the last key, so
    // loads past the end fetch a resident row) and the loop body is straight
    // line, so the loads of the next two tiles stay in flight across barriers.
    bf16x8 kB[K_UNITS], vB[VK];
    load_tile(kB, vB, k_begin + kKeyTile, k_end);
    store_tile(kA, vA, 0);
    lds_barrier();
    const int n_pairs = (n_tiles + 1) >> 1;
#pragma unroll 1
    for (int it = 0; it < n_pairs; ++it) {
      const int kt0 = k_begin + 2 * it * kKeyTile;  // tile 2it in stage 0, 2it+1 in B
      load_tile(kA, vA, kt0 + 2 * kKeyTile, k_end);
      compute_tile(0, kt0);
      store_tile(kB, vB, 1);
      lds_barrier();
      load_tile(kB, vB, kt0 + 3 * kKeyTile, k_end);
      if (2 * it + 1 < n_tiles) compute_tile(1, kt0 + kKeyTile);
      store_tile(kA, vA, 0);
      lds_barrier();
    }
  }

  // ---------------------------------------------------------------- combine lanes
  // each lane holds the partial sum of its own keys; the 4 lane groups of a
  // query (lanes l, l ^ 16, l ^ 32, l ^ 48) add theirs
#pragma unroll
  for (int i = 0; i < QT; ++i) {
    l_run[i] += partner_f32<4>(l_run[i]);
    l_run[i] += partner_f32<5>(l_run[i]);
  }

  // ---------------------------------------------------------------- combine key groups
  if constexpr (KG == 2) {
    float* xs = reinterpret_cast<float*>(smem_raw);  // LDS reused after the loop
    // per row group: QT * (DT*4*64 acc floats + 64 m + 64 l)
    constexpr int PER_QT = DT * 4 * 64 + 128;
    static_assert(RG * QT * PER_QT * 4 <= Lds<D>::kBytes, "key-group exchange fits in LDS");
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
        for (int e = 0; e < 4; ++e)
          acc[i][d][e] = acc[i][d][e] * a1 + p[(d * 4 + e) * 64 + lane] * a2;
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
    const bool live = qt_on[i] && r < rows_valid;
    if (n_splits == 1) {
      bf16_t* orow = a.out + (((size_t)b * T_cap + t) * H + g_kv * G + gq) * D;
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
      float* po = a.part_o + (ubase + r) * D;
#pragma unroll
      for (int d = 0; d < DT; ++d) {
        f32x4 o = live ? acc[i][d] : f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<f32x4*>(po + 16 * d + 4 * lg) = o;
      }
      if (lg == 0) {
        a.part_m[ubase + r] = live ? m_run[i] : -INFINITY;
        a.part_l[ubase + r] = live ? l_run[i] : 0.0f;
      }
    }
  }
}

// Combine the per-split partials of one (b, kv head) and write bf16 rows.  A
// thread owns one row and 4 output dims.  Every load of every split is issued
// up front and unconditionally (one memory round trip); a split that saw no
// key for the row (m = -inf) is dropped by a select, so whatever its unwritten
// O partial holds never reaches the sum.

template <int D, int NW, int QT, int KG, int PF, int NS, bool ONCE>
int launch_main(int n_slots, const AttnArgs& args, hipStream_t s) {
  auto kern = k_attn_bf16<D, NW, QT, KG, PF, NS, ONCE>;
  const int lds = NS > 0 ? NS * LdsDirect::kStage : Lds<D>::kBytes;
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  hipLaunchKernelGGL(kern, dim3(n_slots), dim3(NW * 64), lds, s, args);
  return launch_status();
}

// The direct-to-LDS GQA plan (D = 128, 4 waves, two query tiles per wave, one
// key group, two LDS stages), defined in attn_direct.hip.
int launch_direct(bool once, int n_slots, const AttnArgs& args, hipStream_t s);

}  // namespace attn
}  // namespace spec
