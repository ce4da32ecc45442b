// Host check of the kernels' page-table indexing, built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_sanitized_host.py.
//
// The kernels compute every page-table index through the constexpr helpers
// of csrc/index.h; this program walks the same loops as the kernels (the
// prefill waves' page stepping, the decode splits' pages, the append and
// transfer tiles) over many pool geometries and asserts, for every index a
// kernel reads:
//   - it lies inside the sequence's row (Full: the allocated pages,
//     ceil(L / 16); SWA: the ring's C / 16 pages);
//   - it is the entry of the slot formula for the keys the page carries
//     (Full pos / 16, SWA (pos mod C) / 16);
//   - every key a kernel uses is still held by the ring (pos >= L - C), and
//     the decode splits cover [0, L) exactly once.
// Geometries: rings of 1-8 pages and larger ones, windows 1..C, row counts
// within what alloc admits (resident + new <= C), lengths across page and
// ring boundaries.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <vector>

#include "index.h"  // csrc/index.h, found through the include path

using namespace hswa::idx;

static long g_checks = 0;

#define CHECK(cond, ...)                                             \
  do {                                                               \
    ++g_checks;                                                      \
    if (!(cond)) {                                                   \
      fprintf(stderr, "FAILED %s at %s:%d: ", #cond, __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);                                  \
      fprintf(stderr, "\n");                                         \
      exit(1);                                                       \
    }                                                                \
  } while (0)

static int32_t row_len(int kind, int32_t L, int32_t C) {
  return kind == kFull ? (L + kPage - 1) / kPage : C / kPage;
}

// The prefill kernel's page walk for one sequence with n query rows (its
// last n positions of L), query blocks of QB rows.
static void prefill_walk(int kind, int32_t L, int32_t n, int32_t W, int32_t C, int32_t QB) {
  const int32_t npr = C / kPage;
  const int32_t rl = row_len(kind, L, C);
  const int32_t qblocks = (n + QB - 1) / QB;
  for (int32_t qb = 0; qb < qblocks; ++qb) {
    const int32_t P0 = L - n + qb * QB;
    const int32_t nrows = n - qb * QB < QB ? n - qb * QB : QB;
    const int32_t wg_khi = P0 + nrows - 1;
    const int32_t wg_klo = kind == kFull ? 0 : (P0 - W + 1 > 0 ? P0 - W + 1 : 0);
    const int32_t kstart = (wg_klo / 32) * 32;
    const int32_t nsteps = (wg_khi - kstart) / 32 + 1;
    if (kind == kSwa)
      CHECK(wg_klo >= ring_oldest(L, C), "prefill: key %d left the ring (L %d C %d)", wg_klo, L,
            C);
    for (int half = 0; half < 2; ++half) {
      int32_t e = prefill_first_entry(kind, kstart, half, C);
      for (int32_t s = 0; s < nsteps; ++s) {
        const int32_t kp = kstart + 32 * s + kPage * half;  // first key of this wave's page
        if (kp <= wg_khi) {  // the kernel reads the table only then
          CHECK(e >= 0 && e < rl, "prefill: entry %d outside row of %d (kind %d L %d n %d W %d "
                "C %d QB %d qb %d step %d half %d)", e, rl, kind, L, n, W, C, QB, qb, s, half);
          CHECK(e == table_entry(kind, kp, C), "prefill: entry %d, slot formula %d (kind %d L %d "
                "n %d W %d C %d QB %d qb %d step %d half %d)", e, table_entry(kind, kp, C), kind,
                L, n, W, C, QB, qb, s, half);
        }
        e = prefill_next_entry(kind, e, npr);
      }
    }
  }
}

// The decode kernels' page walk: bf16 pages and FP8 KV-head pairs in 32-key
// steps (pages kp0 and kp0 + 16), FP8 pages of one head in 64-key steps (four
// pages), over the splits of a Full layer or the window of a SWA layer; n
// rows end at position L - 1.
static void decode_walk(int kind, int32_t L, int32_t n, int32_t W, int32_t C, int32_t n_splits,
                        int32_t split_len, int step_keys) {
  const int32_t rl = row_len(kind, L, C);
  std::vector<int> cover(kind == kFull ? L : 0, 0);
  const int32_t nsplit = kind == kFull ? n_splits : 1;
  int32_t nonempty = 0;
  for (int32_t split = 0; split < nsplit; ++split) {
    int32_t klo, khi;
    if (kind == kFull) {
      const int32_t len = split_keys(L, n_splits, split_len);
      klo = split * len;
      khi = klo + len < L ? klo + len : L;
    } else {
      klo = L - n - W + 1 > 0 ? L - n - W + 1 : 0;
      khi = L;
      CHECK(klo >= ring_oldest(L, C), "decode: key %d left the ring (L %d n %d W %d C %d)", klo,
            L, n, W, C);
    }
    if (klo >= khi) continue;
    ++nonempty;
    for (int32_t k = klo; k < khi && kind == kFull; ++k) cover[k]++;
    const int32_t s0 = (klo / step_keys) * step_keys;
    const int32_t nsteps = (khi - 1 - s0) / step_keys + 1;
    for (int32_t st = 0; st < nsteps; ++st) {
      const int32_t kp0 = s0 + step_keys * st;
      for (int32_t x = 0; x < step_keys / kPage; ++x) {
        const int32_t own = kp0 + kPage * x;
        const int32_t pos = decode_page_pos(kp0, x, klo, khi);
        // the page read holds a key of the range and lies in the step; a
        // page that holds one is read itself
        CHECK(pos % kPage == 0 && pos + kPage > klo && pos < khi && pos >= kp0 &&
              pos < kp0 + step_keys && (pos == own || own + kPage <= klo || own >= khi),
              "decode: step %d page %d reads position %d (klo %d khi %d)", kp0, x, pos, klo,
              khi);
        const int32_t e = table_entry(kind, pos, C);
        CHECK(e >= 0 && e < rl, "decode: entry %d outside row of %d (kind %d L %d n %d W %d C %d "
              "splits %d/%d split %d step %d)", e, rl, kind, L, n, W, C, n_splits, split_len,
              split, st);
      }
    }
  }
  if (kind == kFull) {
    for (int32_t k = 0; k < L; ++k)
      CHECK(cover[k] == 1, "decode: key %d covered %d times (L %d splits %d/%d)", k, cover[k], L,
            n_splits, split_len);
    // the combine merges ceil(L / len) splits: exactly the non-empty ones
    const int32_t len = split_keys(L, n_splits, split_len);
    CHECK((L + len - 1) / len == nonempty && nonempty <= n_splits,
          "decode: combine count %d, non-empty splits %d (L %d splits %d/%d)",
          (L + len - 1) / len, nonempty, L, n_splits, split_len);
  }
}

// The append kernel's tiles (rows at positions [L - n, L), grid sized by
// max_rows >= n) and the transfer kernel's (positions [p0, p0 + n)).
static void tile_walk(int kind, int32_t L, int32_t p0, int32_t n, int32_t max_rows, int32_t C,
                      bool xfer) {
  const int32_t rl = row_len(kind, L, C);
  std::vector<int> cover(n, 0);
  std::vector<int> slot_of(C, -1);
  const int32_t tiles = tiles_for(max_rows);
  for (int32_t t = 0; t < tiles; ++t) {
    const int32_t tp = tile_pos(p0, t);
    if (tp >= p0 + n) continue;
    int32_t lo = tp > p0 ? tp : p0;
    if (xfer && kind == kSwa && ring_oldest(L, C) > lo) lo = ring_oldest(L, C);
    const int32_t hi = tp + kPage < p0 + n ? tp + kPage : p0 + n;
    if (lo >= hi) continue;
    const int32_t e = table_entry(kind, tp, C);
    CHECK(e >= 0 && e < rl, "%s: entry %d outside row of %d (kind %d L %d p0 %d n %d C %d)",
          xfer ? "xfer" : "append", e, rl, kind, L, p0, n, C);
    for (int32_t pos = lo; pos < hi; ++pos) {
      CHECK(table_entry(kind, pos, C) == e, "tile: position %d not on the tile's page", pos);
      cover[pos - p0]++;
      if (kind == kSwa) {  // no two written positions share a ring slot
        const int32_t sl = pos % C;
        CHECK(slot_of[sl] < 0, "%s: positions %d and %d share ring slot %d (C %d)",
              xfer ? "xfer" : "append", slot_of[sl], pos, sl, C);
        slot_of[sl] = pos;
      }
    }
  }
  const int32_t first = xfer && kind == kSwa && ring_oldest(L, C) > p0 ? ring_oldest(L, C) : p0;
  for (int32_t pos = p0; pos < p0 + n; ++pos)
    CHECK(cover[pos - p0] == (pos >= first ? 1 : 0), "%s: position %d written %d times "
          "(kind %d L %d p0 %d n %d C %d)", xfer ? "xfer" : "append", pos, cover[pos - p0], kind,
          L, p0, n, C);
}

int main() {
  const int32_t rings[] = {1, 2, 3, 4, 5, 6, 7, 8, 24, 136};
  const int32_t qbs[] = {32, 64, 128};
  for (int32_t npr : rings) {
    const int32_t C = npr * kPage;
    for (int32_t W = 1; W <= C && W <= 200; W += (npr > 8 ? 7 : (npr > 4 ? 3 : 1))) {
      // SWA: n new rows admitted when min(L - n, W - 1) + n <= C
      for (int32_t n = 1; n <= C - W + 1; n += (C > 128 ? 97 : (n < 20 ? 1 : 11))) {
        for (int32_t L = n; L <= n + 3 * C + 40; L += (C > 128 ? 61 : 7)) {
          if ((L - n < W - 1 ? L - n : W - 1) + n > C) continue;
          for (int32_t QB : qbs) prefill_walk(kSwa, L, n, W, C, QB);
          if (n <= 4) {
            decode_walk(kSwa, L, n, W, C, 1, 64, 32);
            decode_walk(kSwa, L, n, W, C, 1, 64, 64);
          }
          tile_walk(kSwa, L, L - n, n, n + (L % 5), C, false);
          if (n <= C) tile_walk(kSwa, L, L - n, n, n, C, true);
        }
      }
    }
    // transfers of ranges reaching below the ring's oldest position
    for (int32_t L = 1; L <= 5 * C; L += (C > 128 ? 97 : 5))
      for (int32_t p0 = 0; p0 < L; p0 += (C > 128 ? 89 : 3)) {
        const int32_t n = L - p0 < C ? L - p0 : C;
        tile_walk(kSwa, L, p0, n, n, C, true);
      }
  }
  // Full layers: prefill chunks of any size over any prefix
  for (int32_t L = 1; L <= 2200; L += 13)
    for (int32_t n = 1; n <= L; n += (n < 40 ? 1 : 61))
      for (int32_t QB : qbs) {
        prefill_walk(kFull, L, n, 0, 16, QB);
        tile_walk(kFull, L, L - n, n, n, 16, false);
      }
  // Full decode: every split plan, including hints below the length
  for (int32_t L = 1; L <= 9000; L += 97)
    for (int32_t ns : {1, 2, 3, 5, 8, 13, 21, 40})
      for (int32_t sl = 64; sl <= 4096; sl *= 4) {
        decode_walk(kFull, L, 1, 0, 16, ns, sl, 32);
        decode_walk(kFull, L, 1, 0, 16, ns, sl, 64);
      }
  // FP8 decode grid: a bijection onto (unit, head), heads 2j and 2j + 1 of a
  // unit on blocks of the same XCD (block index mod 8)
  for (int32_t hkv = 2; hkv <= 16; hkv += 2)
    for (int32_t units = 1; units <= 300; units += (units < 40 ? 1 : 37)) {
      const int32_t nb = fp8_blocks(hkv, units);
      CHECK(nb % 16 == 0 && nb >= units * hkv && nb < units * hkv + 16,
            "fp8 grid: %d blocks for %d x %d", nb, units, hkv);
      std::vector<int32_t> block_of(units * hkv, -1);
      for (int32_t b = 0; b < nb; ++b) {
        int32_t u = -1, h = -1;
        if (!fp8_block(b, hkv, units, &u, &h)) continue;
        CHECK(u >= 0 && u < units && h >= 0 && h < hkv, "fp8 block %d -> (%d, %d)", b, u, h);
        CHECK(block_of[u * hkv + h] < 0, "fp8 blocks %d and %d -> (%d, %d)",
              block_of[u * hkv + h], b, u, h);
        block_of[u * hkv + h] = b;
      }
      for (int32_t u = 0; u < units; ++u)
        for (int32_t h = 0; h < hkv; h += 2) {
          const int32_t b0 = block_of[u * hkv + h], b1 = block_of[u * hkv + h + 1];
          CHECK(b0 >= 0 && b1 >= 0 && b0 % 8 == b1 % 8, "fp8 heads %d, %d of unit %d on "
                "blocks %d, %d", h, h + 1, u, b0, b1);
        }
    }
  // Decode work queues: over the queues that blocks take items from (one
  // unpaired, 8 paired) every (unit, head) item comes exactly once, a queue
  // stays exhausted once it is, and paired heads 2j and 2j + 1 of a unit
  // share a queue
  for (int32_t hkv = 1; hkv <= 16; ++hkv)
    for (int paired = 0; paired <= (hkv % 2 == 0 ? 1 : 0); ++paired)
      for (int32_t units = 0; units <= 200; units += (units < 30 ? 1 : 17)) {
        std::vector<int32_t> queue_of(units * hkv, -1);
        std::vector<int32_t> used;
        for (int32_t b = 0; b < 64; ++b) {
          const int32_t q = queue_of_block(b, paired);
          CHECK(q >= 0 && q < kQueues, "block %d takes queue %d", b, q);
          if (std::find(used.begin(), used.end(), q) == used.end()) used.push_back(q);
        }
        CHECK((int)used.size() == (paired ? kQueues : 1), "%d queues in use (paired %d)",
              (int)used.size(), paired);
        for (int32_t q : used) {
          bool done = false;
          for (int32_t k = 0; k < units * hkv + 8; ++k) {
            int32_t u = -1, h = -1;
            const bool ok = queue_item(k, q, units, hkv, paired, &u, &h);
            CHECK(!(done && ok), "queue %d item %d after the end (units %d hkv %d)", q, k,
                  units, hkv);
            if (!ok) {
              done = true;
              continue;
            }
            CHECK(u >= 0 && u < units && h >= 0 && h < hkv, "queue %d item %d -> (%d, %d)", q,
                  k, u, h);
            CHECK(queue_of[u * hkv + h] < 0, "item (%d, %d) in queues %d and %d", u, h,
                  queue_of[u * hkv + h], q);
            queue_of[u * hkv + h] = q;
          }
        }
        for (int32_t x = 0; x < units * hkv; ++x)
          CHECK(queue_of[x] >= 0, "item (%d, %d) in no queue (units %d hkv %d paired %d)",
                x / hkv, x % hkv, units, hkv, paired);
        if (paired)
          for (int32_t x = 0; x < units * hkv; x += 2)
            CHECK(queue_of[x] == queue_of[x + 1], "paired heads of unit %d in queues %d, %d",
                  x / hkv, queue_of[x], queue_of[x + 1]);
      }
  printf("index checks passed: %ld\n", g_checks);
  return 0;
}
