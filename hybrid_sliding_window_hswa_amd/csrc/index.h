// Page-table index arithmetic of the kernels, as plain constexpr functions:
// the HIP compiler makes them usable on the device, and the host-side index
// checks (tests/sanitize/index_check.cpp) call the same code.
//
// Slot rules of the dual pool ("MiMo-V2.5 Series Inference Full-Link
// Optimization" sec. 2.1, "KVCache Dual Pool"; 16-token pages behind a page
// table as in "Following the Bottleneck: Optimizing MiniMax M3 on AMD
// Instinct MI355X" sec. 3): position pos of a sequence sits in entry pos / 16
// of its Full page-table row, and in entry (pos mod C) / 16 of its ring row
// of C / 16 pages.
#pragma once

#include <stdint.h>

namespace hswa {
namespace idx {

constexpr int32_t kPage = 16;
constexpr int kFull = 0;
constexpr int kSwa = 1;

// Entry of a sequence's page-table row that holds position pos: the Full
// row for Full layers, the ring row (C = ring_slots slots) for SWA layers.
constexpr int32_t table_entry(int kind, int32_t pos, int32_t ring_slots) {
  return kind == kFull ? pos / kPage : (pos % ring_slots) / kPage;
}

// Prefill: the entry of the first page a wave moves.  Keys come in 32-key
// steps of two pages starting at kstart (a multiple of 32); the waves of half
// h move page h of every step.
constexpr int32_t prefill_first_entry(int kind, int32_t kstart, int half, int32_t ring_slots) {
  return table_entry(kind, kstart + kPage * half, ring_slots);
}

// Prefill: the same wave's entry one step (two pages) later.  A ring row of
// npr pages wraps; a ring of one page wraps twice per step.
constexpr int32_t prefill_next_entry(int kind, int32_t e, int32_t npr) {
  e += 2;
  if (kind != kFull) {
    if (e >= npr) e -= npr;
    if (e >= npr) e -= npr;
  }
  return e;
}

// Decode (Full layers): keys per split of a sequence of L keys.  Its
// min(n_splits, ceil(L / split_len)) splits share the keys evenly in 64-key
// multiples, so they cover every key even when the plan's max_seq_len was
// below L; split s holds [s * len, min(L, (s + 1) * len)).
constexpr int32_t split_keys(int32_t L, int32_t n_splits, int32_t split_len) {
  const int32_t by_len = (L + split_len - 1) / split_len;
  const int32_t ns = n_splits < by_len ? n_splits : by_len;
  return ((L + ns - 1) / ns + 63) / 64 * 64;
}

// Append and transfer grids: page tiles per sequence for up to max_rows
// positions (a range of max_rows positions starting anywhere in a page
// touches at most this many pages), and the first position of tile t of a
// range that starts at p0.
constexpr int32_t tiles_for(int32_t max_rows) { return (max_rows + kPage - 2) / kPage + 1; }
constexpr int32_t tile_pos(int32_t p0, int32_t t) { return (p0 / kPage + t) * kPage; }

// Oldest position a ring of ring_slots slots can still hold at length L: an
// older position's slot belongs to a newer one.
constexpr int32_t ring_oldest(int32_t L, int32_t ring_slots) { return L - ring_slots; }

}  // namespace idx
}  // namespace hswa
