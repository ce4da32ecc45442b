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

// Decode: the first position of the page that a workgroup reads as page x
// (0-based, 16 keys each) of the step starting at kp0, over its key range
// [klo, khi).  A page holding a key of the range is itself; a page with none
// (before klo in the first step, at or past khi in the last) is replaced by
// the step's first page that holds one, so the lanes that would read it load
// lines the step reads anyway and a call reads no page outside its range.
constexpr int32_t decode_page_pos(int32_t kp0, int32_t x, int32_t klo, int32_t khi) {
  const int32_t first = kp0 + kPage * x;
  if (first + kPage > klo && first < khi) return first;
  return (klo > kp0 ? klo : kp0) / kPage * kPage;
}

// FP8 decode grid: the scales of a page live in [Hkv][16] fp32 rows of 64
// bytes, so KV heads 2j and 2j + 1 share a 128-byte line.  Workgroups go to
// the 8 XCDs (each with its own L2) round-robin by block index, so blocks b
// and b + 8 share an XCD.  With an even head count, pair p = (unit, heads
// 2j and 2j + 1), unit = (sequence, split), takes blocks 16 (p / 8) + p % 8
// and that + 8: both heads of a line on one XCD, each line fetched once.
// Returns false for the padding blocks of the last 16-block group.
constexpr bool fp8_block(int32_t b, int32_t hkv, int32_t units, int32_t* unit, int32_t* head) {
  const int32_t group = b / 16, r = b % 16;
  const int32_t pair = 8 * group + r % 8;
  *unit = pair / (hkv / 2);
  *head = 2 * (pair % (hkv / 2)) + r / 8;
  return *unit < units;
}
// Blocks of that grid: units * hkv rounded up to whole 16-block groups.
constexpr int32_t fp8_blocks(int32_t hkv, int32_t units) {
  return (units * (hkv / 2) + 7) / 8 * 16;
}

// Decode work queues (split-K calls).  A pre-pass lists the (sequence,
// split) units that hold keys; a grid of resident workgroups then takes
// (unit, KV head) items from a queue by an atomic counter, so no workgroup
// slot is spent on an empty split.  bf16/fp16 pages use one queue for the
// whole grid.  FP8 pages (paired heads) use 8 queues, queue q = block index
// mod 8 (one per XCD: blocks go to the XCDs round-robin), so that heads 2j
// and 2j + 1 of a unit, whose scales share 128-byte lines, run on one XCD.
// Queue state: the counters at kQueueStride * q, the unit count at
// kQueueCount, the unit list from kQueueList (int32 words).
constexpr int32_t kQueues = 8;
constexpr int32_t kQueueStride = 32;  // one 128-byte line per counter
constexpr int32_t kQueueCount = kQueues * kQueueStride;
constexpr int32_t kQueueList = kQueueCount + kQueueStride;

// The queue that block b takes its items from.
constexpr int32_t queue_of_block(int32_t b, bool paired) { return paired ? b % kQueues : 0; }

// Item k of queue q over `units` listed units and hkv heads.  Unpaired (one
// queue): item k is (unit, head) = (k / hkv, k % hkv), unit-major.  Paired
// (hkv even, 8 queues): heads 2j and 2j + 1 of a unit are items 2m and
// 2m + 1 of queue q, for head pairs P = 8m + q of the unit-major (unit,
// pair) order.  False once the queue is exhausted.
constexpr bool queue_item(int32_t k, int32_t q, int32_t units, int32_t hkv, bool paired,
                          int32_t* unit, int32_t* head) {
  if (paired) {
    const int32_t hp = hkv / 2;
    const int64_t P = (int64_t)kQueues * (k / 2) + q;
    if (P >= (int64_t)units * hp) return false;
    *unit = (int32_t)(P / hp);
    *head = 2 * (int32_t)(P % hp) + k % 2;
    return true;
  }
  if (q != 0 || (int64_t)k >= (int64_t)units * hkv) return false;
  *unit = k / hkv;
  *head = k % hkv;
  return true;
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
