// Internal declarations shared by the host code and the HIP kernels of the
// Hybrid SWA library.  Not part of the public ABI (include/hswa.h is).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <string>

namespace hswa {

// Largest KV head count the entry points accept: the kernels address a
// page's K or V block of all KV heads (16 tokens x Hkv x d x 2 bytes) with
// 32-bit byte offsets.
constexpr int32_t kMaxKvHeads = 1024;

// ---------------------------------------------------------------------------
// Errors: thread-local text of the last failure (hswa_last_error).
void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();
int hip_fail(hipError_t e, const char* what);

// ---------------------------------------------------------------------------
// Device-table update of the dual pool.  One record per sequence touched by
// a pool operation; the kernel applies all records of one operation.
struct PoolRec {
  int32_t seq;       // sequence id
  int32_t new_len;   // seq_len after the operation; < 0 leaves it unwritten
  int32_t clr_lo;    // positions [clr_lo, clr_hi) lose their SWA entry
  int32_t clr_hi;
  int32_t set_lo;    // positions [set_lo, set_hi) get map = their SWA slot
  int32_t set_hi;
  int32_t pg_lo;     // logical page of the record's first listed page
  int32_t pg_off;    // offset of this record's pages in the page list
  int32_t fpt_lo;    // fpt entries [fpt_lo, fpt_hi) of the row are written
  int32_t fpt_hi;
  int32_t fpt_clear; // 1: write -1, 0: write the listed physical page
  int32_t npg;       // listed pages: logical pages [pg_lo, pg_lo + npg)
};

struct PoolDev {
  int32_t* seq_len;
  int32_t* fpt;
  const int32_t* rpt;
  int32_t* map;
  int32_t max_pages;
  int32_t ring_slots;
};

// recs/pages live in pinned host memory readable by the device.  Record x's
// Full pages sit at pages[x * stride ..] and the ring pages of the same
// logical pages at pages[(n_recs + x) * stride ..] (stride >= every record's
// npg), so a block can read its record and its page ids at once.  Every block of the
// launch writes `seq` into done[its index] (pinned host memory) once it has
// read everything it needs from the staging buffer, so the host knows when
// the buffer may be reused without recording an event.
int pool_apply_blocks(int n_recs, int32_t stride);
hipError_t launch_pool_apply(const PoolDev& dev, const PoolRec* recs, int n_recs,
                             const int32_t* pages, int32_t stride, int32_t* done,
                             int32_t seq, hipStream_t stream);

// ---------------------------------------------------------------------------
// Attention kernels.
struct Tables {
  const int32_t* seq_len;
  const int32_t* fpt;
  const int32_t* rpt;
  int32_t max_pages;
  int32_t ring_slots;
  int32_t max_seqs;
};

struct AttnParams {
  int32_t kind;          // 0 FULL, 1 SWA
  int32_t window;
  int32_t hq, hkv, d;
  float scale_log2;      // softmax scale * log2(e)
  int32_t num_seqs;
  const int32_t* seq_ids;
  const int32_t* cu_q;   // nullptr: one row per sequence (decode)
  const int32_t* q_pos;  // nullptr: rows end at seq_len; else first row's position
  int32_t total_q;
  int32_t max_q_len;
  int32_t max_seq_len;
  const uint16_t* q;
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache;
  uint16_t* v_cache;
  Tables t;
  void* out;             // fp32, or fp16 when out_f16
  int32_t out_f16;
  int32_t* vlen;
  // FP8 pages (kv_fp8 = 1): k_cache/v_cache hold e4m3 codes, one fp32 scale
  // per (page, KV head, token) in k_scale/v_scale ([page][Hkv][16])
  int32_t kv_fp8;
  float* k_scale;
  float* v_scale;
  // decode split-K
  int32_t n_splits;
  int32_t split_len;
  float* ws;             // [total_q][hq][n_splits][d] partial sums, then
                         // [total_q][hq][n_splits][2] (max, sum)
  int32_t* queue;        // split-K calls: work-queue state after the partial
                         // states (idx::kQueue*); nullptr: one workgroup per
                         // (sequence, split, KV head)
};

// Window-masked transfer of one layer's KV between the pages and a packed
// buffer of [token][Hkv][d] 16-bit words (K bf16, V fp16) that the device
// can address (pinned host memory or device memory).
struct XferParams {
  int32_t kind;            // 0 FULL, 1 SWA: which page table maps positions
  int32_t hkv, d;
  int32_t num_seqs;
  const int32_t* seq_ids;
  const int32_t* cu_tok;   // [num_seqs+1]: sequence i moves
                           // n_i = cu_tok[i+1]-cu_tok[i] positions from
  const int32_t* first_pos;  // [num_seqs] first_pos[i] on; nullptr: its last n_i
  int32_t max_tok;
  int32_t total_tok;       // tokens the packed buffers hold
  uint16_t* k_cache;
  uint16_t* v_cache;
  Tables t;
  uint16_t* buf_k;         // device-usable address of the packed buffers
  uint16_t* buf_v;
  // FP8 pages: codes move as bytes ([token][Hkv][d] in the buffers, V too)
  // and the fp32 scales of each (token, head) beside them
  bool kv_fp8;
  float* k_scale;          // page scales [page][Hkv][16]
  float* v_scale;
  float* buf_k_scale;      // device-usable [total_tok][Hkv]
  float* buf_v_scale;
};

// Copy of one layer's K/V between two sequences of a pool, page to page.
struct CopyParams {
  int32_t kind;
  int32_t hkv, d;
  int32_t num_seqs;
  const int32_t* src_ids;
  const int32_t* dst_ids;
  const int32_t* first_pos;
  const int32_t* end_pos;
  int32_t max_tok;
  uint16_t* k_cache;
  uint16_t* v_cache;
  Tables t;
  bool kv_fp8;             // FP8 pages: byte codes plus these fp32 scales
  float* k_scale;          // [page][Hkv][16]
  float* v_scale;
};

hipError_t launch_append(const AttnParams& p, hipStream_t stream);
hipError_t launch_copy(const CopyParams& p, hipStream_t stream);
// to_host: pages -> buffer (offload); else buffer -> pages (restore)
hipError_t launch_xfer(const XferParams& p, bool to_host, hipStream_t stream);
hipError_t launch_prefill(const AttnParams& p, hipStream_t stream);
hipError_t launch_decode(const AttnParams& p, hipStream_t stream);

// Device scratch of the allocation-free decode (hswa_decode_noalloc): the
// split-K partial states of one call live in a file-scope device array of
// this many bytes instead of a caller's workspace.
constexpr size_t kDecodeScratchBytes = (size_t)128 << 20;
// Device address of this GPU's copy of that array (the current device's),
// looked up once per device.
hipError_t decode_scratch(float** out);

// Split-K plan for decode: shared by the workspace query and the launch.
struct DecodePlan {
  int32_t n_splits;
  int32_t split_len;
  size_t ws_bytes;
  size_t queue_off;  // byte offset of the work-queue state in the workspace
};
// rows = query rows of the call (num_seqs for plain decode).
DecodePlan plan_decode(int32_t kind, int32_t num_seqs, int32_t rows, int32_t hq, int32_t hkv,
                       int32_t d, int32_t window, int32_t max_seq_len);

}  // namespace hswa
