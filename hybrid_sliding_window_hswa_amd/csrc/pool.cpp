// Dual KV pool bookkeeping: Full page allocator, per-sequence SWA rings,
// the Full-to-SWA map and window eviction.
//
// Follows "MiMo-V2.5 Series Inference Full-Link Optimization" sec. 2.1
// ("KVCache Dual Pool": Full pool O(N) and SWA pool O(W); Full index
// authoritative with a Full-to-SWA map; joint capacity check; "SWA-aware
// prefix cache tree" point 2: release out-of-window SWA entries per chunk,
// per request end and as decode advances) and the 16-token page tables of
// "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct MI355X"
// sec. 3.
//
// The host keeps the authoritative metadata.  Each operation computes its
// effect on the host, then enqueues one small kernel (a few, for very
// uneven page lists) that applies the same effect to the caller's device
// tables.  The kernel reads a compact record list (position ranges and page
// ids, not per-slot values) straight from a pinned, device-readable staging
// buffer; a ring of staging buffers, each with completion words that the
// kernel's blocks write when done reading, keeps the host from overwriting
// a buffer the device has not read yet.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <new>
#include <thread>
#include <vector>

#include "../../include/hswa.h"
#include "internal.h"

using hswa::PoolRec;

namespace {

constexpr int kPage = HSWA_PAGE_SIZE;
constexpr int kStages = 16;

struct Stage {
  void* buf = nullptr;       // pinned host memory, device-readable
  size_t cap = 0;
  // the apply kernel that last read the buffer: its blocks write `seq` into
  // done[0 .. nblk) when they no longer need the buffer
  volatile int32_t* done = nullptr;
  int32_t nblk = 0;
  int32_t seq = 0;
  bool pending = false;
};

// Waits until every block of the kernel that last read the stage is done
// with it.  After a second of polling the device is synchronised once, so a
// failed or aborted kernel surfaces as an error instead of a hang.
int wait_stage(Stage& st) {
  if (!st.pending) return HSWA_OK;
  auto all_done = [&]() {
    for (int32_t i = 0; i < st.nblk; ++i)
      if (st.done[i] != st.seq) return false;
    return true;
  };
  const auto t0 = std::chrono::steady_clock::now();
  bool synced = false;
  while (!all_done()) {
    if (!synced && std::chrono::steady_clock::now() - t0 > std::chrono::seconds(1)) {
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return hswa::hip_fail(e, "waiting for a pool staging buffer");
      synced = true;
      if (!all_done()) {
        hswa::set_error("pool table update did not report completion");
        return HSWA_E_HIP;
      }
      break;
    }
    std::this_thread::yield();
  }
  std::atomic_thread_fence(std::memory_order_acquire);
  st.pending = false;
  return HSWA_OK;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct hswa_pool {
  int32_t W = 0, C = 0, max_seqs = 0, max_pages = 0, num_pages = 0;
  int32_t ring_pages_per_seq = 0;
  // host metadata
  std::vector<int32_t> len;        // tokens per sequence
  std::vector<int32_t> res_start;  // first position still in the SWA ring
  std::vector<int32_t> npages;     // Full pages held per sequence
  std::vector<int32_t> fpt;        // [max_seqs][max_pages]
  std::vector<int32_t> rpt;        // [max_seqs][C/16]
  std::vector<int32_t> map;        // [num_pages*16]
  std::vector<int32_t> freeq;      // FIFO ring of free pages
  int64_t fhead = 0, fcount = 0;
  std::vector<int32_t> refs;       // per Full page: sequences holding it
  std::vector<uint32_t> mark;      // per-sequence epoch for duplicate checks
  uint32_t epoch = 0;
  // device mirror
  bool has_dev = false;
  hswa::PoolDev dev{};
  Stage stage[kStages];
  int next_stage = 0;
  int32_t flush_seq = 0;
  std::vector<void*> retired;      // outgrown staging buffers, freed at destroy

  int32_t pop_page() {
    int32_t p = freeq[fhead];
    fhead = (fhead + 1) % num_pages;
    --fcount;
    refs[p] = 1;
    return p;
  }
  // one holder lets go of a page; true when no sequence holds it any more
  bool drop_page(int32_t p) { return --refs[p] == 0; }
  // leading pages of sequence b that another sequence also holds (a fork
  // shares a prefix of its source's pages, so shared pages form a prefix)
  int32_t shared_pages(int32_t b) const {
    int32_t n = 0;
    const int32_t* row = &fpt[(size_t)b * max_pages];
    while (n < npages[b] && refs[row[n]] > 1) ++n;
    return n;
  }
  void push_page(int32_t p) {
    freeq[(fhead + fcount) % num_pages] = p;
    ++fcount;
  }
  void push_page_front(int32_t p) {
    fhead = (fhead + num_pages - 1) % num_pages;
    freeq[fhead] = p;
    ++fcount;
  }
  int32_t full_slot(int32_t b, int32_t pos) const {
    return fpt[(size_t)b * max_pages + pos / kPage] * kPage + pos % kPage;
  }
  int32_t swa_slot(int32_t b, int32_t pos) const {
    int32_t r = pos % C;
    return rpt[(size_t)b * ring_pages_per_seq + r / kPage] * kPage + r % kPage;
  }
};

namespace {

// Validates a list of sequence ids (range, no repeats).
int check_ids(hswa_pool* p, int32_t n, const int32_t* ids) {
  if (n < 0) {
    hswa::set_error("n_seqs must be >= 0 (got %d)", n);
    return HSWA_E_INVAL;
  }
  if (n > 0 && !ids) {
    hswa::set_error("seq_ids is NULL");
    return HSWA_E_INVAL;
  }
  if (++p->epoch == 0) {
    std::fill(p->mark.begin(), p->mark.end(), 0u);
    p->epoch = 1;
  }
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    if (b < 0 || b >= p->max_seqs) {
      hswa::set_error("sequence id %d out of range [0, %d)", b, p->max_seqs);
      return HSWA_E_INVAL;
    }
    if (p->mark[b] == p->epoch) {
      hswa::set_error("sequence id %d listed twice", b);
      return HSWA_E_INVAL;
    }
    p->mark[b] = p->epoch;
  }
  return HSWA_OK;
}

// Builds a record covering the given position ranges and fpt writes; the
// record's page list spans every logical page any of them touches.
struct RecBuilder {
  std::vector<PoolRec> recs;
  std::vector<int32_t> pages;  // records' page lists, back to back (at pg_off)
  std::vector<int32_t> rpages; // ring page of each listed logical page

  void add(const hswa_pool* p, int32_t b, int32_t new_len, int32_t clr_lo,
           int32_t clr_hi, int32_t set_lo, int32_t set_hi, int32_t fpt_lo,
           int32_t fpt_hi, int32_t fpt_clear, const int32_t* page_src) {
    PoolRec r{};
    r.seq = b;
    r.new_len = new_len;
    r.clr_lo = clr_lo;
    r.clr_hi = std::max(clr_lo, clr_hi);
    r.set_lo = set_lo;
    r.set_hi = std::max(set_lo, set_hi);
    r.fpt_lo = fpt_lo;
    r.fpt_hi = std::max(fpt_lo, fpt_hi);
    r.fpt_clear = fpt_clear;
    int64_t lo = INT64_MAX, hi = INT64_MIN;  // logical pages [lo, hi)
    if (r.clr_hi > r.clr_lo) {
      lo = std::min<int64_t>(lo, r.clr_lo / kPage);
      hi = std::max<int64_t>(hi, (r.clr_hi - 1) / kPage + 1);
    }
    if (r.set_hi > r.set_lo) {
      lo = std::min<int64_t>(lo, r.set_lo / kPage);
      hi = std::max<int64_t>(hi, (r.set_hi - 1) / kPage + 1);
    }
    if (r.fpt_hi > r.fpt_lo && !fpt_clear) {
      lo = std::min<int64_t>(lo, r.fpt_lo);
      hi = std::max<int64_t>(hi, r.fpt_hi);
    }
    if (hi <= lo) {
      lo = 0;
      hi = 0;
    }
    r.pg_lo = (int32_t)lo;
    r.pg_off = (int32_t)pages.size();
    r.npg = (int32_t)(hi - lo);
    const int32_t* ring = &p->rpt[(size_t)b * p->ring_pages_per_seq];
    for (int64_t lp = lo; lp < hi; ++lp) {
      pages.push_back(page_src[lp]);
      rpages.push_back(ring[(lp * kPage) % p->C / kPage]);
    }
    recs.push_back(r);
  }
};

// Copies a group of records (rb.recs[idx[0..n_recs)]) into a staging buffer
// and enqueues the apply kernel.  Buffer layout: records, Full page lists
// (record x's at x * stride), ring page lists (at (n_recs + x) * stride),
// then one completion word per block.
int flush_group(hswa_pool* p, const RecBuilder& rb, const int* idx, int n_recs,
                int32_t stride, hipStream_t s) {
  const int nblk = hswa::pool_apply_blocks(n_recs, stride);
  size_t rec_bytes = (size_t)n_recs * sizeof(PoolRec);
  size_t done_off = (rec_bytes + 2 * (size_t)n_recs * stride * sizeof(int32_t) + 63) / 64 * 64;
  size_t bytes = done_off + (size_t)nblk * sizeof(int32_t);
  Stage& st = p->stage[p->next_stage];
  p->next_stage = (p->next_stage + 1) % kStages;
  int rc = wait_stage(st);
  if (rc) return rc;
  if (st.cap < bytes) {
    if (st.buf) p->retired.push_back(st.buf);
    st.buf = nullptr;
    size_t cap = std::max<size_t>(bytes + bytes / 2, 64 << 10);
    hipError_t e = hipHostMalloc(&st.buf, cap, hipHostMallocCoherent | hipHostMallocMapped);
    if (e != hipSuccess) {
      st.cap = 0;
      return hswa::hip_fail(e, "hipHostMalloc of a pool staging buffer");
    }
    st.cap = cap;
  }
  PoolRec* recs = (PoolRec*)st.buf;
  int32_t* lists = (int32_t*)((char*)st.buf + rec_bytes);
  for (int x = 0; x < n_recs; ++x) {
    const PoolRec& r = rb.recs[idx[x]];
    recs[x] = r;
    if (r.npg > 0) {
      memcpy(lists + (size_t)x * stride, rb.pages.data() + r.pg_off, r.npg * sizeof(int32_t));
      memcpy(lists + (size_t)(n_recs + x) * stride, rb.rpages.data() + r.pg_off,
             r.npg * sizeof(int32_t));
    }
  }
  void* dptr = nullptr;
  hipError_t e = hipHostGetDevicePointer(&dptr, st.buf, 0);
  if (e != hipSuccess) return hswa::hip_fail(e, "hipHostGetDevicePointer");
  // positive and never a stale value; wraps to 1 before int32 overflow
  p->flush_seq = p->flush_seq == INT32_MAX ? 1 : p->flush_seq + 1;
  st.seq = p->flush_seq;
  st.nblk = nblk;
  st.done = (volatile int32_t*)((char*)st.buf + done_off);
  for (int i = 0; i < nblk; ++i) st.done[i] = 0;
  e = hswa::launch_pool_apply(p->dev, (const PoolRec*)dptr, n_recs,
                              (const int32_t*)((char*)dptr + rec_bytes), stride,
                              (int32_t*)((char*)dptr + done_off), st.seq, s);
  if (e != hipSuccess) return hswa::hip_fail(e, "pool table update launch");
  st.pending = true;
  return HSWA_OK;
}

// Enqueues the records' device-table updates.  Each record is one sequence,
// so they apply in any order.  Their page lists are padded to a common
// length per launch: records go out longest list first, in groups whose
// padded lists stay within twice their own size (plus 256 entries), which
// is one group when the lists are alike (the usual case) and a few when one
// list dwarfs the others.
int flush(hswa_pool* p, const RecBuilder& rb, void* stream) {
  if (!p->has_dev || rb.recs.empty()) return HSWA_OK;
  hipStream_t s = (hipStream_t)stream;
  const int n = (int)rb.recs.size();
  std::vector<int> order(n);
  for (int i = 0; i < n; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return rb.recs[a].npg > rb.recs[b].npg; });
  int i = 0;
  while (i < n) {
    const int32_t stride = std::max<int32_t>(1, rb.recs[order[i]].npg);
    int64_t sum = 0;
    int j = i;
    for (; j < n; ++j) {
      const int64_t npg = rb.recs[order[j]].npg;
      if (j > i && (int64_t)(j - i + 1) * stride > 2 * (sum + npg) + 256) break;
      sum += npg;
    }
    int rc = flush_group(p, rb, order.data() + i, j - i, stride, s);
    if (rc) return rc;
    i = j;
  }
  return HSWA_OK;
}

// The device effect of an eviction or an alloc on one sequence: the new
// length (-1: unchanged), map entries cleared [clr_lo, clr_hi) and set
// [set_lo, set_hi) by position, and fpt entries [fpt_lo, fpt_hi) written
// from the sequence's row.  An eviction and an alloc of one sequence touch
// disjoint positions and pages, so their effects merge into one record.
struct Eff {
  int32_t b, new_len, clr_lo, clr_hi, set_lo, set_hi, fpt_lo, fpt_hi;
};

// Records of the effects (built after the host change, which keeps every
// page id the records list), then one flush.
int flush_effs(hswa_pool* p, const std::vector<Eff>& effs, void* stream) {
  if (!p->has_dev) return HSWA_OK;
  RecBuilder rb;
  for (const Eff& e : effs)
    rb.add(p, e.b, e.new_len, e.clr_lo, e.clr_hi, e.set_lo, e.set_hi, e.fpt_lo, e.fpt_hi, 0,
           &p->fpt[(size_t)e.b * p->max_pages]);
  return flush(p, rb, stream);
}

// Checks of an eviction: ids and the capacity of evicted_out.
int evict_check(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* evicted_out,
                int64_t evicted_cap) {
  int rc = check_ids(p, n, ids);
  if (rc) return rc;
  int64_t total = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    int32_t keep_from = std::max(0, p->len[b] - p->W + 1);
    total += std::max(0, keep_from - p->res_start[b]);
  }
  if (evicted_out && total > evicted_cap) {
    hswa::set_error("evicted_out holds %lld entries, %lld needed", (long long)evicted_cap,
                    (long long)total);
    return HSWA_E_INVAL;
  }
  return HSWA_OK;
}

// The eviction's host change; its device effect goes to effs.
void evict_host(hswa_pool* p, int32_t n, const int32_t* ids, int32_t* evicted_out,
                int32_t* counts_out, std::vector<Eff>& effs) {
  int64_t o = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    int32_t keep_from = std::max(0, p->len[b] - p->W + 1);
    int32_t lo = p->res_start[b];
    int32_t cnt = std::max(0, keep_from - lo);
    for (int32_t pos = lo; pos < lo + cnt; ++pos) {
      int32_t fs = p->full_slot(b, pos);
      p->map[fs] = -1;
      if (evicted_out) evicted_out[o] = fs;
      ++o;
    }
    if (counts_out) counts_out[i] = cnt;
    p->res_start[b] = std::max(lo, keep_from);
    // the device effect is map entries only (length and fpt unwritten)
    if (cnt > 0) effs.push_back(Eff{b, -1, lo, lo + cnt, 0, 0, 0, 0});
  }
}

// Checks of an alloc (ring checked) or import (ring not checked).  res_at,
// if given, is each sequence's first resident position at the time of the
// alloc (an eviction in the same operation comes first).
int alloc_check(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* n_new,
                bool importing, const std::vector<int32_t>* res_at) {
  int rc = check_ids(p, n, ids);
  if (rc) return rc;
  if (n > 0 && !n_new) {
    hswa::set_error("n_new is NULL");
    return HSWA_E_INVAL;
  }
  // Joint capacity check before any change ([MiMo] 2.1 Scheduling
  // Constraints): Full pages for all listed sequences together, the page
  // table row of each, and (alloc only) each SWA ring.
  int64_t need_pages = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    int64_t k = n_new[i];
    if (k < 0) {
      hswa::set_error("n_new[%d] = %lld is negative", i, (long long)k);
      return HSWA_E_INVAL;
    }
    int64_t new_len = (int64_t)p->len[b] + k;
    if (new_len > (int64_t)INT32_MAX - kPage) {
      hswa::set_error("sequence %d would exceed the int32 position range", b);
      return HSWA_E_INVAL;
    }
    int64_t pages = ceil_div(new_len, kPage);
    if (pages > p->max_pages) {
      hswa::set_error("sequence %d needs %lld pages, its table row holds %d", b,
                      (long long)pages, p->max_pages);
      return HSWA_E_NOSPC;
    }
    need_pages += pages - p->npages[b];
    const int32_t res = res_at ? (*res_at)[b] : p->res_start[b];
    if (!importing && (int64_t)(p->len[b] - res) + k > p->C) {
      hswa::set_error("SWA ring of sequence %d: %d resident + %lld new > %d slots", b,
                      p->len[b] - res, (long long)k, p->C);
      return HSWA_E_NOSPC;
    }
  }
  if (need_pages > p->fcount) {
    hswa::set_error("Full pool: %lld pages needed, %lld free", (long long)need_pages,
                    (long long)p->fcount);
    return HSWA_E_NOSPC;
  }
  return HSWA_OK;
}

// The alloc's (or import's) host change; its device effect goes to effs.
void alloc_host(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* n_new,
                int32_t* full_out, int32_t* swa_out, bool importing, std::vector<Eff>& effs) {
  size_t o = 0;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    int32_t L = p->len[b];
    int32_t k = n_new[i];
    int32_t new_len = L + k;
    int32_t old_pages = p->npages[b];
    int32_t keep_from = importing ? std::max(0, new_len - p->W + 1) : 0;
    int32_t clr_lo = p->res_start[b], clr_hi = clr_lo;
    if (importing) {
      clr_hi = std::max(clr_lo, std::min(keep_from, L));
      for (int32_t pos = clr_lo; pos < clr_hi; ++pos) p->map[p->full_slot(b, pos)] = -1;
      p->res_start[b] = std::max(p->res_start[b], keep_from);
    }
    int32_t* row = &p->fpt[(size_t)b * p->max_pages];
    for (int32_t pos = L; pos < new_len; ++pos) {
      if (pos % kPage == 0) row[pos / kPage] = p->pop_page();
      int32_t fs = p->full_slot(b, pos);
      int32_t ss = -1;
      if (pos >= keep_from) {
        ss = p->swa_slot(b, pos);
        p->map[fs] = ss;
      }
      if (full_out) full_out[o] = fs;
      if (swa_out) swa_out[o] = ss;
      ++o;
    }
    p->npages[b] = (int32_t)ceil_div(new_len, kPage);
    p->len[b] = new_len;
    effs.push_back(
        Eff{b, new_len, clr_lo, clr_hi, std::max(L, keep_from), new_len, old_pages, p->npages[b]});
  }
}

// Shared body of alloc (ring checked) and import (ring not checked; only
// in-window positions get SWA slots).
int alloc_impl(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* n_new,
               int32_t* full_out, int32_t* swa_out, void* stream, bool importing) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  int rc = alloc_check(p, n, ids, n_new, importing, nullptr);
  if (rc) return rc;
  std::vector<Eff> effs;
  alloc_host(p, n, ids, n_new, full_out, swa_out, importing, effs);
  return flush_effs(p, effs, stream);
}

}  // namespace

extern "C" {

int hswa_pool_create(const hswa_pool_desc* d, hswa_pool** out) {
  hswa::clear_error();
  if (!d || !out) {
    hswa::set_error("desc and out must be non-NULL");
    return HSWA_E_INVAL;
  }
  *out = nullptr;
  if (d->page_size != kPage) {
    hswa::set_error("page_size must be 16 (got %d)", d->page_size);
    return HSWA_E_INVAL;
  }
  if (d->window < 1 || d->ring_slots < d->window || d->ring_slots % kPage != 0) {
    hswa::set_error("need window >= 1 and ring_slots >= window, a multiple of 16 "
                    "(window %d, ring_slots %d)", d->window, d->ring_slots);
    return HSWA_E_INVAL;
  }
  if (d->max_seqs < 1 || d->max_pages_per_seq < 1 || d->num_full_pages < 1) {
    hswa::set_error("max_seqs, max_pages_per_seq and num_full_pages must be >= 1");
    return HSWA_E_INVAL;
  }
  if ((int64_t)d->num_full_pages * kPage > INT32_MAX ||
      (int64_t)d->max_seqs * (d->ring_slots / kPage) * kPage > INT32_MAX ||
      (int64_t)d->max_pages_per_seq * kPage > INT32_MAX ||
      (int64_t)d->max_seqs * d->max_pages_per_seq > INT32_MAX) {
    hswa::set_error("pool too large for int32 slot ids and table indices");
    return HSWA_E_INVAL;
  }
  if (!d->full_free_order || !d->ring_pages) {
    hswa::set_error("full_free_order and ring_pages must be given");
    return HSWA_E_INVAL;
  }
  int ndev = (d->dev_seq_len != nullptr) + (d->dev_fpt != nullptr) +
             (d->dev_rpt != nullptr) + (d->dev_map != nullptr);
  if (ndev != 0 && ndev != 4) {
    hswa::set_error("give all four device tables or none");
    return HSWA_E_INVAL;
  }
  hswa_pool* p = new (std::nothrow) hswa_pool();
  if (!p) {
    hswa::set_error("out of host memory");
    return HSWA_E_INVAL;
  }
  p->W = d->window;
  p->C = d->ring_slots;
  p->max_seqs = d->max_seqs;
  p->max_pages = d->max_pages_per_seq;
  p->num_pages = d->num_full_pages;
  p->ring_pages_per_seq = d->ring_slots / kPage;
  try {
    // both page lists must be permutations
    std::vector<uint8_t> seen((size_t)p->num_pages, 0);
    for (int32_t i = 0; i < p->num_pages; ++i) {
      int32_t v = d->full_free_order[i];
      if (v < 0 || v >= p->num_pages || seen[v]) {
        hswa::set_error("full_free_order is not a permutation of 0..%d", p->num_pages - 1);
        delete p;
        return HSWA_E_INVAL;
      }
      seen[v] = 1;
    }
    int64_t nring = (int64_t)p->max_seqs * p->ring_pages_per_seq;
    std::vector<uint8_t> rseen((size_t)nring, 0);
    for (int64_t i = 0; i < nring; ++i) {
      int32_t v = d->ring_pages[i];
      if (v < 0 || v >= nring || rseen[v]) {
        hswa::set_error("ring_pages is not a permutation of 0..%lld", (long long)nring - 1);
        delete p;
        return HSWA_E_INVAL;
      }
      rseen[v] = 1;
    }
    p->len.assign(p->max_seqs, 0);
    p->res_start.assign(p->max_seqs, 0);
    p->npages.assign(p->max_seqs, 0);
    p->mark.assign(p->max_seqs, 0);
    p->fpt.assign((size_t)p->max_seqs * p->max_pages, -1);
    p->rpt.assign(d->ring_pages, d->ring_pages + nring);
    p->map.assign((size_t)p->num_pages * kPage, -1);
    p->freeq.assign(d->full_free_order, d->full_free_order + p->num_pages);
    p->refs.assign(p->num_pages, 0);
    p->fhead = 0;
    p->fcount = p->num_pages;
  } catch (const std::bad_alloc&) {
    hswa::set_error("out of host memory");
    delete p;
    return HSWA_E_INVAL;
  }
  if (ndev == 4) {
    p->has_dev = true;
    p->dev.seq_len = d->dev_seq_len;
    p->dev.fpt = d->dev_fpt;
    p->dev.rpt = d->dev_rpt;
    p->dev.map = d->dev_map;
    p->dev.max_pages = p->max_pages;
    p->dev.ring_slots = p->C;
    struct {
      void* dst;
      const void* src;
      size_t bytes;
    } copies[] = {
        {d->dev_seq_len, p->len.data(), p->len.size() * 4},
        {d->dev_fpt, p->fpt.data(), p->fpt.size() * 4},
        {d->dev_rpt, p->rpt.data(), p->rpt.size() * 4},
        {d->dev_map, p->map.data(), p->map.size() * 4},
    };
    for (auto& c : copies) {
      hipError_t e = hipMemcpy(c.dst, c.src, c.bytes, hipMemcpyHostToDevice);
      if (e != hipSuccess) {
        int rc = hswa::hip_fail(e, "initial device table copy");
        delete p;
        return rc;
      }
    }
  }
  *out = p;
  return HSWA_OK;
}

void hswa_pool_destroy(hswa_pool* p) {
  if (!p) return;
  for (auto& st : p->stage) {
    wait_stage(st);
    if (st.buf) (void)hipHostFree(st.buf);
  }
  for (void* b : p->retired) (void)hipHostFree(b);
  delete p;
}

int hswa_pool_get_view(const hswa_pool* p, hswa_pool_view* out) {
  hswa::clear_error();
  if (!p || !out) {
    hswa::set_error("pool and out must be non-NULL");
    return HSWA_E_INVAL;
  }
  if (!p->has_dev) {
    hswa::set_error("pool has no device tables");
    return HSWA_E_INVAL;
  }
  out->seq_len = p->dev.seq_len;
  out->fpt = p->dev.fpt;
  out->rpt = p->dev.rpt;
  out->map = p->dev.map;
  out->max_seqs = p->max_seqs;
  out->max_pages_per_seq = p->max_pages;
  out->ring_slots = p->C;
  out->window = p->W;
  return HSWA_OK;
}

int hswa_pool_alloc(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* n_new,
                    int32_t* full_out, int32_t* swa_out, void* stream) {
  return alloc_impl(p, n, ids, n_new, full_out, swa_out, stream, false);
}

int hswa_pool_import(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* n_new,
                     int32_t* full_out, int32_t* swa_out, void* stream) {
  return alloc_impl(p, n, ids, n_new, full_out, swa_out, stream, true);
}

int hswa_pool_evict(hswa_pool* p, int32_t n, const int32_t* ids, int32_t* evicted_out,
                    int64_t evicted_cap, int32_t* counts_out, void* stream) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  int rc = evict_check(p, n, ids, evicted_out, evicted_cap);
  if (rc) return rc;
  std::vector<Eff> effs;
  evict_host(p, n, ids, evicted_out, counts_out, effs);
  return flush_effs(p, effs, stream);
}

int hswa_pool_evict_alloc(hswa_pool* p, int32_t n_ev, const int32_t* ev_ids,
                          int32_t* evicted_out, int64_t evicted_cap, int32_t* counts_out,
                          int32_t n_al, const int32_t* al_ids, const int32_t* n_new,
                          int32_t* full_out, int32_t* swa_out, void* stream) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  // every check of both before any change; the alloc sees the rings as the
  // eviction leaves them
  int rc = evict_check(p, n_ev, ev_ids, evicted_out, evicted_cap);
  if (rc) return rc;
  std::vector<int32_t> res_at(p->res_start);
  for (int32_t i = 0; i < n_ev; ++i) {
    const int32_t b = ev_ids[i];
    res_at[b] = std::max(res_at[b], std::max(0, p->len[b] - p->W + 1));
  }
  rc = alloc_check(p, n_al, al_ids, n_new, false, &res_at);
  if (rc) return rc;
  std::vector<Eff> effs;
  evict_host(p, n_ev, ev_ids, evicted_out, counts_out, effs);
  const size_t n_evict_effs = effs.size();
  alloc_host(p, n_al, al_ids, n_new, full_out, swa_out, false, effs);
  // one record per sequence: a sequence's eviction joins its alloc
  std::vector<int32_t> ev_of(p->max_seqs, -1);
  for (size_t x = 0; x < n_evict_effs; ++x) ev_of[effs[x].b] = (int32_t)x;
  std::vector<bool> merged(n_evict_effs, false);
  std::vector<Eff> out;
  out.reserve(effs.size());
  for (size_t x = n_evict_effs; x < effs.size(); ++x) {
    Eff e = effs[x];
    const int32_t v = ev_of[e.b];
    if (v >= 0) {  // an alloc clears nothing, so the eviction's range fits
      e.clr_lo = effs[v].clr_lo;
      e.clr_hi = effs[v].clr_hi;
      merged[v] = true;
    }
    out.push_back(e);
  }
  for (size_t x = 0; x < n_evict_effs; ++x)
    if (!merged[x]) out.push_back(effs[x]);
  return flush_effs(p, out, stream);
}

int hswa_pool_release(hswa_pool* p, int32_t n, const int32_t* ids, void* stream) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  int rc = check_ids(p, n, ids);
  if (rc) return rc;
  RecBuilder rb;
  for (int32_t i = 0; i < n; ++i) {
    int32_t b = ids[i];
    int32_t* row = &p->fpt[(size_t)b * p->max_pages];
    int32_t lo = p->res_start[b], hi = p->len[b];
    for (int32_t pos = lo; pos < hi; ++pos) p->map[p->full_slot(b, pos)] = -1;
    if (p->has_dev) rb.add(p, b, 0, lo, hi, 0, 0, 0, p->npages[b], 1, row);
    for (int32_t lp = 0; lp < p->npages[b]; ++lp) {
      if (p->drop_page(row[lp])) p->push_page(row[lp]);  // last holder
      row[lp] = -1;
    }
    p->npages[b] = 0;
    p->len[b] = 0;
    p->res_start[b] = 0;
  }
  return flush(p, rb, stream);
}

int hswa_pool_truncate(hswa_pool* p, int32_t n, const int32_t* ids, const int32_t* new_len,
                       void* stream) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  int rc = check_ids(p, n, ids);
  if (rc) return rc;
  if (n > 0 && !new_len) {
    hswa::set_error("new_len is NULL");
    return HSWA_E_INVAL;
  }
  // every check before any change
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    const int32_t k = new_len[i];
    if (k < 0 || k > p->len[b]) {
      hswa::set_error("new_len[%d] = %d outside [0, %d] (sequence %d)", i, k, p->len[b], b);
      return HSWA_E_INVAL;
    }
    if (p->res_start[b] > std::max(0, k - p->W + 1)) {
      hswa::set_error("sequence %d: positions from %d are resident, the window of length %d "
                      "starts at %d (truncate before evicting)",
                      b, p->res_start[b], k, std::max(0, k - p->W + 1));
      return HSWA_E_INVAL;
    }
    // a page another sequence holds may neither be freed nor take new
    // positions (a later append would overwrite the other holder's K/V)
    const int32_t sh = p->shared_pages(b);
    if (k < p->len[b] && (int64_t)k < (int64_t)kPage * sh) {
      hswa::set_error("sequence %d: length %d cuts into its first %d pages, which another "
                      "sequence also holds", b, k, sh);
      return HSWA_E_INVAL;
    }
  }
  RecBuilder rb;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    const int32_t k = new_len[i];
    const int32_t L = p->len[b];
    if (k == L) continue;
    int32_t* row = &p->fpt[(size_t)b * p->max_pages];
    for (int32_t pos = k; pos < L; ++pos) p->map[p->full_slot(b, pos)] = -1;
    const int32_t keep = (int32_t)ceil_div(k, kPage);
    // the record copies the page ids of the cleared range before they go
    if (p->has_dev) rb.add(p, b, k, k, L, 0, 0, keep, p->npages[b], 1, row);
    for (int32_t lp = p->npages[b] - 1; lp >= keep; --lp) {
      p->drop_page(row[lp]);  // held by b alone (checked above)
      p->push_page_front(row[lp]);
      row[lp] = -1;
    }
    p->npages[b] = keep;
    p->len[b] = k;
  }
  return flush(p, rb, stream);
}

int hswa_pool_match_len(const hswa_pool* p, int32_t n, const int32_t* ids,
                        const int32_t* want, int32_t tail, int32_t* out) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  if (n < 0 || (n > 0 && (!ids || !want || !out)) || tail < 0) {
    hswa::set_error("match_len: bad arguments (n %d, tail %d)", n, tail);
    return HSWA_E_INVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->max_seqs || want[i] < 0) {
      hswa::set_error("match_len: entry %d: sequence %d / length %d out of range", i, ids[i],
                      want[i]);
      return HSWA_E_INVAL;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    int32_t k = std::min(want[i], p->len[b]);
    // A position without an SWA entry at h rules out every end in
    // (h, h + tail]; walk back from the match end to the first end whose
    // tail window has no such position.  Positions before the sequence's
    // first resident one have none of its entries (a page it shares with
    // another sequence may carry that one's).
    while (k > 0) {
      int32_t hole = -1;
      for (int32_t pos = k - 1; pos >= std::max(0, k - tail); --pos) {
        if (pos < p->res_start[b] || p->map[p->full_slot(b, pos)] < 0) {
          hole = pos;
          break;
        }
      }
      if (hole < 0) break;
      k = hole;
    }
    out[i] = k;
  }
  return HSWA_OK;
}

int hswa_pool_fork(hswa_pool* p, int32_t n, const int32_t* src_ids, const int32_t* dst_ids,
                   const int32_t* lens, int32_t* full_from, int32_t* swa_from, void* stream) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  int rc = check_ids(p, n, dst_ids);  // destinations distinct and in range
  if (rc) return rc;
  if (n > 0 && (!src_ids || !lens)) {
    hswa::set_error("fork: src_ids and lens are required");
    return HSWA_E_INVAL;
  }
  // every check before any change: sources in range and not destinations,
  // destinations empty, lengths window-safe for their sources, then the
  // Full pages of all forks together
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t a = src_ids[i], b = dst_ids[i], m = lens[i];
    if (a < 0 || a >= p->max_seqs || p->mark[a] == p->epoch) {
      hswa::set_error("fork %d: source %d out of range or also a destination", i, a);
      return HSWA_E_INVAL;
    }
    if (p->len[b] != 0) {
      hswa::set_error("fork %d: destination %d holds %d positions (must be empty)", i, b,
                      p->len[b]);
      return HSWA_E_INVAL;
    }
    if (m < 0 || m > p->len[a]) {
      hswa::set_error("fork %d: length %d outside [0, %d]", i, m, p->len[a]);
      return HSWA_E_INVAL;
    }
    for (int32_t pos = std::max(0, m - (p->W - 1)); pos < m; ++pos) {
      if (pos < p->res_start[a] || p->map[p->full_slot(a, pos)] < 0) {
        hswa::set_error("fork %d: position %d of source %d has left the SWA pool, so %d "
                        "positions are not window-safe (see hswa_pool_match_len)", i, pos, a, m);
        return HSWA_E_INVAL;
      }
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t m = lens[i];
    const int64_t pages = ceil_div(m, kPage);
    if (pages > p->max_pages) {
      hswa::set_error("fork %d: %lld pages, a table row holds %d", i, (long long)pages,
                      p->max_pages);
      return HSWA_E_NOSPC;
    }
    need += pages - std::max(0, m - p->W + 1) / kPage;
  }
  if (need > p->fcount) {
    hswa::set_error("Full pool: %lld pages needed, %lld free", (long long)need,
                    (long long)p->fcount);
    return HSWA_E_NOSPC;
  }
  RecBuilder rb;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t a = src_ids[i], b = dst_ids[i], m = lens[i];
    const int32_t start = std::max(0, m - p->W + 1);   // dst's window start
    const int32_t own = start / kPage;                 // pages shared below it
    const int32_t pages = (int32_t)ceil_div(m, kPage);
    const int32_t* srow = &p->fpt[(size_t)a * p->max_pages];
    int32_t* row = &p->fpt[(size_t)b * p->max_pages];
    for (int32_t lp = 0; lp < own; ++lp) {
      row[lp] = srow[lp];
      ++p->refs[row[lp]];
    }
    for (int32_t lp = own; lp < pages; ++lp) row[lp] = p->pop_page();
    for (int32_t pos = start; pos < m; ++pos) p->map[p->full_slot(b, pos)] = p->swa_slot(b, pos);
    p->npages[b] = pages;
    p->len[b] = m;
    p->res_start[b] = start;
    if (full_from) full_from[i] = kPage * own;
    if (swa_from) swa_from[i] = start;
    if (p->has_dev) rb.add(p, b, m, 0, 0, start, m, 0, pages, 0, row);
  }
  return flush(p, rb, stream);
}

int hswa_pool_window_counts(const hswa_pool* p, int32_t kind, int32_t n, const int32_t* ids,
                            int32_t* counts) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  if ((kind != HSWA_LAYER_FULL && kind != HSWA_LAYER_SWA) || n < 0 ||
      (n > 0 && (!ids || !counts))) {
    hswa::set_error("window_counts: bad arguments (kind %d, n %d)", kind, n);
    return HSWA_E_INVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (ids[i] < 0 || ids[i] >= p->max_seqs) {
      hswa::set_error("window_counts: sequence id %d out of range", ids[i]);
      return HSWA_E_INVAL;
    }
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t L = p->len[ids[i]];
    counts[i] = kind == HSWA_LAYER_FULL ? L : std::min(L, p->W - 1);
  }
  return HSWA_OK;
}

int hswa_pool_read_tables(const hswa_pool* p, int32_t* seq_len, int32_t* fpt,
                          int32_t* map, int32_t* free_pages, int32_t* n_free) {
  hswa::clear_error();
  if (!p) {
    hswa::set_error("pool is NULL");
    return HSWA_E_INVAL;
  }
  if (seq_len) memcpy(seq_len, p->len.data(), p->len.size() * 4);
  if (fpt) memcpy(fpt, p->fpt.data(), p->fpt.size() * 4);
  if (map) memcpy(map, p->map.data(), p->map.size() * 4);
  if (free_pages)
    for (int64_t i = 0; i < p->fcount; ++i)
      free_pages[i] = p->freeq[(p->fhead + i) % p->num_pages];
  if (n_free) *n_free = (int32_t)p->fcount;
  return HSWA_OK;
}

}  // extern "C"
