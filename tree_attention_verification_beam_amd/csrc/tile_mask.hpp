// tile_mask.hpp -- visibility bits of one 64-key tile of the tree-masked
// attention, for one query row.
//
// "Clover: Regressive Lightweight Speculative Decoding with Sequential
// Knowledge", causal mask construction: node i sees node j iff j is an
// ancestor of i or i = j; every node sees the whole context.  A query row's
// ancestor set is two 64-bit words (bit a: tree node a, which sits at cache
// slot ctx + a).  Plain integer code, host and device: the test suite checks
// it on the CPU against a per-key brute force under the undefined-behaviour
// sanitizer.
#pragma once

#include <stdint.h>

#ifndef SPEC_HD
#define SPEC_HD __host__ __device__
#endif

namespace spec {

// Bit p <-> key kt0 + p of a 64-key tile: visible iff the key lies inside the
// range (p < nin, nin = k_end - kt0) and is a context key (p < nctx, nctx =
// ctx - kt0) or a tree key whose ancestor bit (tree index p - nctx) is set in
// (m0, m1).  Every shift amount stays in 0..63.
SPEC_HD inline uint64_t tile_vis_bits(int nctx, int nin, uint64_t m0, uint64_t m1) {
  uint64_t bits;
  if (nctx >= 64) {
    bits = ~0ull;
  } else if (nctx >= 0) {
    // tree indices 0 .. 63 - nctx follow the nctx context keys
    bits = (nctx > 0 ? (~0ull >> (64 - nctx)) : 0ull) | (m0 << nctx);
  } else {
    const int sh = -nctx;  // tree index of the tile's first key
    bits = sh >= 128 ? 0ull
           : sh >= 64 ? (m1 >> (sh - 64))
           : sh == 0  ? m0
                      : (m0 >> sh) | (m1 << (64 - sh));
  }
  if (nin < 64) bits &= nin > 0 ? (~0ull >> (64 - nin)) : 0ull;
  return bits;
}

// The bits of one MFMA lane group's keys, in the order its scores are held.
// In each 32-key chunk j of the wave's keys (first key wkey0 of the tile) the
// lane group lg holds keys wkey0 + 32 j + 8 lg + 4 (st ^ h) + e, h = (lg >> 1)
// & 1, for sub-tile st and element e; bit 32 j + 4 st + e of the result is that
// key's visibility (the two 4-key halves of every byte swap when h = 1).
SPEC_HD inline uint64_t lane_vis_bits(uint64_t tile_bits, int wkey0, int lg) {
  const uint64_t v = tile_bits >> (wkey0 + 8 * lg);
  const uint64_t sw = ((v >> 4) & 0x0F0F0F0F0F0F0F0Full) | ((v << 4) & 0xF0F0F0F0F0F0F0F0ull);
  return ((lg >> 1) & 1) ? sw : v;
}

// The same for the direct-load layout (one key group over the whole tile,
// keys in natural order): the lane group lg holds keys 32 j + 8 lg + 4 st + e,
// and bit 32 j + 4 st + e of the result is that key's visibility.
SPEC_HD inline uint64_t lane_vis_bits_direct(uint64_t tile_bits, int lg) {
  return tile_bits >> (8 * lg);
}

}  // namespace spec
