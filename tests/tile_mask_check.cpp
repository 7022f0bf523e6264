// CPU check of the attention kernel's per-tile visibility bits
// (csrc/tile_mask.hpp) against a per-key brute force, meant to be built with
// the undefined-behaviour sanitizer (any shift by 64 or more aborts the run).
//
// Domain: every first-tile-key offset nctx = ctx - kt0 in [-140, 80] and range
// end nin = k_end - kt0 in [-4, 80], ancestor words of many shapes (random,
// single bits at 0, 63, 64, 127, chains, all ones, none), every lane group lg
// in 0..3, wave key offset wkey0 in {0, 32} and both key orders (the staged
// layout's and the direct-load layout's).  For each case every tile key
// p in 0..63 and every lane bit is compared with the definition: key kt0 + p is
// visible iff it lies inside the range and is a context key or a tree key
// whose ancestor bit is set.
//
// It also replays the per-element test an earlier version of the kernel used
// (word select by tree index, shift by the index modulo 64) over the same
// domain, to show what that test computed.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <initializer_list>

#define SPEC_HD
#include "../tree_attention_verification_beam_amd/csrc/tile_mask.hpp"

static bool brute(int p, int nctx, int nin, uint64_t m0, uint64_t m1) {
  if (p >= nin) return false;
  if (p < nctx) return true;
  const int a = p - nctx;  // tree index
  if (a >= 128) return false;
  return ((a < 64 ? m0 >> a : m1 >> (a - 64)) & 1ull) != 0;
}

// the earlier kernel's per-score test, written as it was: key = kt0 + p
static bool old_element(int p, int nctx, int nin, uint64_t m0, uint64_t m1) {
  const int aa = p - nctx;  // key - ctx
  const uint64_t w = aa < 64 ? m0 : m1;
  const bool tree_vis = ((w >> (aa & 63)) & 1ull) != 0ull;
  return p < nin && (aa < 0 || tree_vis);
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64() {  // xorshift64*
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return rng_state * 0x2545F4914F6CDD1Dull;
}

int main() {
  long checked = 0, old_mismatch = 0, old_mismatch_feasible = 0;
  uint64_t masks[40][2] = {{0, 0}, {~0ull, ~0ull}, {1, 0}, {1ull << 63, 0}, {0, 1},
                           {0, 1ull << 63}, {~0ull, 0}, {0, ~0ull}};
  int n_masks = 8;
  // ancestor chains: root, every node up to t (a path of a chain-shaped tree)
  for (int t : {3, 40, 63, 64, 65, 100, 126, 127}) {
    uint64_t a = 0, b = 0;
    for (int j = 0; j <= t; ++j) (j < 64 ? a : b) |= 1ull << (j & 63);
    masks[n_masks][0] = a;
    masks[n_masks][1] = b;
    ++n_masks;
  }
  while (n_masks < 40) {
    masks[n_masks][0] = next_u64() | 1ull;  // the root is always an ancestor
    masks[n_masks][1] = next_u64();
    ++n_masks;
  }
  for (int mi = 0; mi < n_masks; ++mi) {
    const uint64_t m0 = masks[mi][0], m1 = masks[mi][1];
    for (int nctx = -140; nctx <= 80; ++nctx) {
      for (int nin = -4; nin <= 80; ++nin) {
        const uint64_t bits = spec::tile_vis_bits(nctx, nin, m0, m1);
        for (int p = 0; p < 64; ++p) {
          const bool want = brute(p, nctx, nin, m0, m1);
          if ((((bits >> p) & 1ull) != 0) != want) {
            std::printf("tile bit mismatch: nctx %d nin %d p %d mask %d\n", nctx, nin, p, mi);
            return 1;
          }
          if (old_element(p, nctx, nin, m0, m1) != want) {
            ++old_mismatch;
            // a kernel range ends within 128 tree keys of the context: k_end <= ctx + T_cap
            if (nin <= nctx + 128) ++old_mismatch_feasible;
          }
          ++checked;
        }
        for (int wkey0 : {0, 32}) {
          for (int lg = 0; lg < 4; ++lg) {
            const uint64_t lv = spec::lane_vis_bits(bits, wkey0, lg);
            const int h = (lg >> 1) & 1;
            const int chunks = wkey0 == 0 ? 2 : 1;  // one key group: 64 keys; two: 32 each
            for (int j = 0; j < chunks; ++j)
              for (int st = 0; st < 2; ++st)
                for (int e = 0; e < 4; ++e) {
                  const int key = wkey0 + 32 * j + 8 * lg + 4 * (st ^ h) + e;
                  const int c = 32 * j + 4 * st + e;
                  if ((((lv >> c) & 1ull) != 0) != brute(key, nctx, nin, m0, m1)) {
                    std::printf("lane bit mismatch: nctx %d nin %d lg %d wkey0 %d c %d\n", nctx,
                                nin, lg, wkey0, c);
                    return 1;
                  }
                  ++checked;
                }
          }
        }
        for (int lg = 0; lg < 4; ++lg) {
          // direct-load layout: natural key order over the whole tile
          const uint64_t lv = spec::lane_vis_bits_direct(bits, lg);
          for (int j = 0; j < 2; ++j)
            for (int st = 0; st < 2; ++st)
              for (int e = 0; e < 4; ++e) {
                const int key = 32 * j + 8 * lg + 4 * st + e;
                const int c = 32 * j + 4 * st + e;
                if ((((lv >> c) & 1ull) != 0) != brute(key, nctx, nin, m0, m1)) {
                  std::printf("direct lane bit mismatch: nctx %d nin %d lg %d c %d\n", nctx, nin, lg, c);
                  return 1;
                }
                ++checked;
              }
        }
      }
    }
  }
  std::printf("checked %ld bits; earlier per-element test mismatches %ld (%ld with k_end <= "
              "ctx + 128)\n", checked, old_mismatch, old_mismatch_feasible);
  return 0;
}
