// C ABI entry points for attention (prefill, decode, KV append), argument
// validation and the thread-local error text.  Kernels live in the .hip
// files; this file only checks arguments and dispatches.
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include <string>

#include "../../include/hswa.h"
#include "index.h"
#include "internal.h"

namespace hswa {

static thread_local std::string g_err;

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
}

void clear_error() { g_err.clear(); }

int hip_fail(hipError_t e, const char* what) {
  set_error("%s: %s", what, hipGetErrorString(e));
  return HSWA_E_HIP;
}

}  // namespace hswa

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Query rows per sequence a decode call takes: one new token plus up to
// three drafts of a multi-token verification step.
constexpr int32_t kMaxDecodeRows = 4;

// Shared validation of an attention call.  `decode` selects the decode form:
// one row per sequence when cu_q is NULL, else 1..4 rows per sequence.
int validate(const hswa_attn_args* a, bool decode, bool need_attn, hswa::AttnParams* p) {
  if (!a) {
    hswa::set_error("args is NULL");
    return HSWA_E_INVAL;
  }
  if (a->kind != HSWA_LAYER_FULL && a->kind != HSWA_LAYER_SWA) {
    hswa::set_error("kind must be HSWA_LAYER_FULL or HSWA_LAYER_SWA (got %d)", a->kind);
    return HSWA_E_INVAL;
  }
  if (a->head_dim != 64 && a->head_dim != 128) {
    hswa::set_error("head_dim must be 64 or 128 (got %d)", a->head_dim);
    return HSWA_E_INVAL;
  }
  if (a->num_q_heads < 1 || a->num_kv_heads < 1 || a->num_q_heads % a->num_kv_heads) {
    hswa::set_error("num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                    a->num_q_heads, a->num_kv_heads);
    return HSWA_E_INVAL;
  }
  if (a->num_kv_heads > hswa::kMaxKvHeads) {
    hswa::set_error("num_kv_heads (%d) must be <= %d", a->num_kv_heads, hswa::kMaxKvHeads);
    return HSWA_E_INVAL;
  }
  int g = a->num_q_heads / a->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) {
    hswa::set_error("query heads per KV head must be 1, 2, 4 or 8 (got %d)", g);
    return HSWA_E_UNSUPPORTED;
  }
  if (a->num_seqs < 0) {
    hswa::set_error("num_seqs must be >= 0");
    return HSWA_E_INVAL;
  }
  const hswa_pool_view& v = a->pool;
  if (!v.seq_len || !v.fpt || !v.rpt) {
    hswa::set_error("pool view has NULL device tables");
    return HSWA_E_INVAL;
  }
  if (v.ring_slots < 16 || v.ring_slots % 16 || v.max_pages_per_seq < 1 || v.window < 1 ||
      v.max_seqs < 1) {
    hswa::set_error("pool view geometry is invalid");
    return HSWA_E_INVAL;
  }
  if (a->kind == HSWA_LAYER_SWA && (a->window < 1 || a->window > v.window)) {
    hswa::set_error("SWA window %d must be in [1, pool window %d]", a->window, v.window);
    return HSWA_E_INVAL;
  }
  if (decode) {
    if (!a->cu_q && a->total_q != a->num_seqs) {
      hswa::set_error("decode: total_q (%d) must equal num_seqs (%d)", a->total_q,
                      a->num_seqs);
      return HSWA_E_INVAL;
    }
    if (a->cu_q && a->num_seqs > 0) {
      if (a->max_q_len > kMaxDecodeRows) {
        hswa::set_error("decode: at most %d rows per sequence (max_q_len %d)", kMaxDecodeRows,
                        a->max_q_len);
        return HSWA_E_UNSUPPORTED;
      }
      if (a->max_q_len < 1 || a->total_q < 0 ||
          (int64_t)a->total_q > (int64_t)a->num_seqs * a->max_q_len) {
        hswa::set_error("decode: need max_q_len >= 1 and 0 <= total_q <= num_seqs * max_q_len "
                        "(max_q_len %d, total_q %d, num_seqs %d)",
                        a->max_q_len, a->total_q, a->num_seqs);
        return HSWA_E_INVAL;
      }
    }
    if (need_attn && a->max_seq_len < 1 && a->num_seqs > 0) {
      hswa::set_error("decode: max_seq_len must be >= 1");
      return HSWA_E_INVAL;
    }
  } else {
    if (a->num_seqs > 0 && !a->cu_q) {
      hswa::set_error("prefill: cu_q is NULL");
      return HSWA_E_INVAL;
    }
    if (a->total_q < 0 || a->max_q_len < 0 || (a->total_q > 0 && a->max_q_len < 1)) {
      hswa::set_error("prefill: total_q and max_q_len must be >= 0 (max_q_len >= 1 "
                      "when there are rows)");
      return HSWA_E_INVAL;
    }
  }
  if (a->num_seqs > 0 && !a->seq_ids) {
    hswa::set_error("seq_ids is NULL");
    return HSWA_E_INVAL;
  }
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) {
    hswa::set_error("k_new and v_new must both be set or both be NULL");
    return HSWA_E_INVAL;
  }
  if (!a->k_cache || !a->v_cache) {
    hswa::set_error("k_cache and v_cache must be set");
    return HSWA_E_INVAL;
  }
  if (need_attn && a->total_q > 0 && (!a->q || !a->out)) {
    hswa::set_error("q and out must be set");
    return HSWA_E_INVAL;
  }
  if (a->out_dtype != HSWA_OUT_F32 && a->out_dtype != HSWA_OUT_F16) {
    hswa::set_error("out_dtype must be HSWA_OUT_F32 or HSWA_OUT_F16 (got %d)", a->out_dtype);
    return HSWA_E_INVAL;
  }
  if (a->kv_dtype != HSWA_KV_BF16 && a->kv_dtype != HSWA_KV_FP8) {
    hswa::set_error("kv_dtype must be HSWA_KV_BF16 or HSWA_KV_FP8 (got %d)", a->kv_dtype);
    return HSWA_E_INVAL;
  }
  if (a->kv_dtype == HSWA_KV_FP8 && (!a->k_scale || !a->v_scale)) {
    hswa::set_error("FP8 pages need k_scale and v_scale");
    return HSWA_E_INVAL;
  }
  const void* ptrs[] = {a->q, a->k_new, a->v_new, a->k_cache, a->v_cache, a->out,
                        a->k_scale, a->v_scale};
  for (const void* q : ptrs) {
    if (q && !aligned16(q)) {
      hswa::set_error("device buffers must be 16-byte aligned");
      return HSWA_E_INVAL;
    }
  }
  if ((int64_t)a->total_q * a->num_q_heads * a->head_dim > INT32_MAX) {
    hswa::set_error("q has more than 2^31 elements");
    return HSWA_E_UNSUPPORTED;
  }
  float scale = a->scale > 0.f ? a->scale : 1.0f / sqrtf((float)a->head_dim);
  *p = hswa::AttnParams{};
  p->kind = a->kind;
  p->window = a->kind == HSWA_LAYER_SWA ? a->window : 0;
  p->hq = a->num_q_heads;
  p->hkv = a->num_kv_heads;
  p->d = a->head_dim;
  p->scale_log2 = scale * 1.4426950408889634f;
  p->num_seqs = a->num_seqs;
  p->seq_ids = a->seq_ids;
  p->cu_q = a->cu_q;
  p->q_pos = a->q_pos;
  p->total_q = a->total_q;
  p->max_q_len = decode && !a->cu_q ? 1 : a->max_q_len;
  p->max_seq_len = a->max_seq_len;
  p->q = (const uint16_t*)a->q;
  p->k_new = (const uint16_t*)a->k_new;
  p->v_new = (const uint16_t*)a->v_new;
  p->k_cache = (uint16_t*)a->k_cache;
  p->v_cache = (uint16_t*)a->v_cache;
  p->t.seq_len = v.seq_len;
  p->t.fpt = v.fpt;
  p->t.rpt = v.rpt;
  p->t.max_pages = v.max_pages_per_seq;
  p->t.ring_slots = v.ring_slots;
  p->t.max_seqs = v.max_seqs;
  p->out = a->out;
  p->out_f16 = a->out_dtype == HSWA_OUT_F16;
  p->vlen = a->vlen_out;
  p->kv_fp8 = a->kv_dtype == HSWA_KV_FP8;
  p->k_scale = p->kv_fp8 ? (float*)a->k_scale : nullptr;
  p->v_scale = p->kv_fp8 ? (float*)a->v_scale : nullptr;
  return HSWA_OK;
}

// Body of hswa_decode and hswa_decode_noalloc.  With `noalloc` the split-K
// partial states go to the library's device scratch (refused when the plan
// needs more than it holds) instead of the caller's workspace; both use the
// same plan, hence the same kernels and bitwise the same results.
int decode_call(const hswa_attn_args* a, void* ws, size_t ws_bytes, bool noalloc,
                void* stream) {
  hswa::clear_error();
  hswa::AttnParams p;
  int rc = validate(a, true, true, &p);
  if (rc) return rc;
  if (p.num_seqs == 0 || p.total_q == 0) return HSWA_OK;
  hswa::DecodePlan pl = hswa::plan_decode(p.kind, p.num_seqs, p.total_q, p.hq, p.hkv, p.d,
                                          p.window, p.max_seq_len);
  if (noalloc) {
    if (pl.ws_bytes > hswa::kDecodeScratchBytes) {
      hswa::set_error("decode_noalloc: the split-K state needs %zu bytes, the device scratch "
                      "holds %zu; use hswa_decode with a workspace",
                      pl.ws_bytes, hswa::kDecodeScratchBytes);
      return HSWA_E_INVAL;
    }
    ws = nullptr;
    if (pl.ws_bytes > 0) {
      float* s = nullptr;
      hipError_t e = hswa::decode_scratch(&s);
      if (e != hipSuccess) return hswa::hip_fail(e, "device scratch address");
      ws = s;
    }
  } else {
    if (ws_bytes < pl.ws_bytes || (pl.ws_bytes > 0 && !ws)) {
      hswa::set_error("decode workspace: %zu bytes given, %zu needed", ws_bytes, pl.ws_bytes);
      return HSWA_E_INVAL;
    }
    if (ws && !aligned16(ws)) {
      hswa::set_error("workspace must be 16-byte aligned");
      return HSWA_E_INVAL;
    }
  }
  p.n_splits = pl.n_splits;
  p.split_len = pl.split_len;
  p.ws = (float*)ws;
  p.queue = pl.n_splits > 1 ? (int32_t*)((char*)ws + pl.queue_off) : nullptr;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (p.k_new) {
    e = hswa::launch_append(p, s);
    if (e != hipSuccess) return hswa::hip_fail(e, "append launch");
  }
  e = hswa::launch_decode(p, s);
  return e == hipSuccess ? HSWA_OK : hswa::hip_fail(e, "decode launch");
}

}  // namespace

static_assert(HSWA_DECODE_SCRATCH_BYTES == hswa::kDecodeScratchBytes,
              "header and library agree on the decode scratch size");

namespace hswa {

// Split-K plan for a decode call.  FULL layers cut each sequence's context
// into pieces of split_len keys (a multiple of 64, between 1,024 and about
// 20K): about 2K (sequence, KV head, piece) work items for 256 CUs, but no
// more, since every piece pays a Q load, a partial-state store and its share
// of the combine.  Pieces of 4K-20K keys measured fastest on 4K-256K
// contexts.  SWA layers read at most W keys and use one split.
DecodePlan plan_decode(int32_t kind, int32_t num_seqs, int32_t rows, int32_t hq, int32_t hkv,
                       int32_t d, int32_t window, int32_t max_seq_len) {
  DecodePlan pl{1, 0, 0};
  if (num_seqs <= 0) return pl;
  if (kind == HSWA_LAYER_SWA) {
    pl.split_len = ((window + 63) / 64) * 64;
    return pl;
  }
  const int64_t min_split = 1024;
  const int64_t max_split = 20480;
  const int64_t target_units = 2048;  // (sequence, kv head, split) work items
  int64_t units = (int64_t)num_seqs * hkv;
  int64_t want = (target_units + units - 1) / units;
  const int64_t by_max = (max_seq_len + max_split - 1) / max_split;
  if (want < by_max) want = by_max;
  int64_t max_by_len = (max_seq_len + min_split - 1) / min_split;
  int64_t n = want < max_by_len ? want : max_by_len;
  if (n < 1) n = 1;
  if (n > 128) n = 128;
  int64_t sl = (max_seq_len + n - 1) / n;
  sl = ((sl + 63) / 64) * 64;
  n = (max_seq_len + sl - 1) / sl;
  pl.n_splits = (int32_t)n;
  pl.split_len = (int32_t)sl;
  if (n > 1) {
    // partial states, then (256-byte aligned) the work-queue state: counters,
    // unit count and the list of up to num_seqs * n units
    const size_t partial = (size_t)rows * hq * n * (d + 2) * sizeof(float);
    pl.queue_off = (partial + 255) / 256 * 256;
    pl.ws_bytes = pl.queue_off + ((size_t)idx::kQueueList + (size_t)num_seqs * n) * 4;
  }
  return pl;
}

}  // namespace hswa

extern "C" {

const char* hswa_last_error(void) { return hswa::g_err.c_str(); }

const char* hswa_status_string(int s) {
  switch (s) {
    case HSWA_OK: return "HSWA_OK";
    case HSWA_E_INVAL: return "HSWA_E_INVAL";
    case HSWA_E_NOSPC: return "HSWA_E_NOSPC";
    case HSWA_E_HIP: return "HSWA_E_HIP";
    case HSWA_E_UNSUPPORTED: return "HSWA_E_UNSUPPORTED";
    default: return "unknown hswa status";
  }
}

int hswa_version(void) { return 100; }

int hswa_append_kv(const hswa_attn_args* a, void* stream) {
  hswa::clear_error();
  hswa::AttnParams p;
  bool decode = a && a->cu_q == nullptr;
  int rc = validate(a, decode, false, &p);
  if (rc) return rc;
  if (p.num_seqs == 0 || p.total_q == 0) return HSWA_OK;  // nothing to write
  if (!a->k_new) {
    hswa::set_error("append: k_new and v_new are required");
    return HSWA_E_INVAL;
  }
  hipError_t e = hswa::launch_append(p, (hipStream_t)stream);
  return e == hipSuccess ? HSWA_OK : hswa::hip_fail(e, "append launch");
}

int hswa_prefill_chunk(const hswa_attn_args* a, void* stream) {
  hswa::clear_error();
  hswa::AttnParams p;
  int rc = validate(a, false, true, &p);
  if (rc) return rc;
  if (p.num_seqs == 0 || p.total_q == 0) return HSWA_OK;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (p.k_new) {
    e = hswa::launch_append(p, s);
    if (e != hipSuccess) return hswa::hip_fail(e, "append launch");
  }
  e = hswa::launch_prefill(p, s);
  return e == hipSuccess ? HSWA_OK : hswa::hip_fail(e, "prefill launch");
}

size_t hswa_decode_workspace_bytes(const hswa_attn_args* a) {
  if (!a) return 0;
  // rows of the call: total_q (one per sequence without cu_q, when a caller
  // may have left total_q unset)
  const int32_t rows = a->total_q > a->num_seqs ? a->total_q : a->num_seqs;
  return hswa::plan_decode(a->kind, a->num_seqs, rows, a->num_q_heads, a->num_kv_heads,
                           a->head_dim, a->window, a->max_seq_len)
      .ws_bytes;
}

int hswa_decode(const hswa_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
  return decode_call(a, ws, ws_bytes, false, stream);
}

int hswa_decode_noalloc(const hswa_attn_args* a, void* stream) {
  return decode_call(a, nullptr, 0, true, stream);
}

}  // extern "C"

namespace {

// Address the device uses for a transfer buffer: device memory as is, pinned
// host memory through its device mapping; anything else is refused.
int device_view(const void* ptr, const char* what, void** out) {
  hipPointerAttribute_t at;
  hipError_t e = hipPointerGetAttributes(&at, ptr);
  if (e != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed query
    hswa::set_error("%s is neither device memory nor pinned host memory", what);
    return HSWA_E_INVAL;
  }
  if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
    *out = const_cast<void*>(ptr);
    return HSWA_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void* d = nullptr;
    e = hipHostGetDevicePointer(&d, const_cast<void*>(ptr), 0);
    if (e != hipSuccess || !d) {
      (void)hipGetLastError();
      hswa::set_error("%s: pinned host memory without a device mapping", what);
      return HSWA_E_INVAL;
    }
    *out = d;
    return HSWA_OK;
  }
  hswa::set_error("%s is neither device memory nor pinned host memory", what);
  return HSWA_E_INVAL;
}

int xfer(const hswa_xfer_args* a, bool to_host, void* stream) {
  hswa::clear_error();
  if (!a) {
    hswa::set_error("args is NULL");
    return HSWA_E_INVAL;
  }
  if (a->kind != HSWA_LAYER_FULL && a->kind != HSWA_LAYER_SWA) {
    hswa::set_error("kind must be HSWA_LAYER_FULL or HSWA_LAYER_SWA (got %d)", a->kind);
    return HSWA_E_INVAL;
  }
  if (a->head_dim != 64 && a->head_dim != 128) {
    hswa::set_error("head_dim must be 64 or 128 (got %d)", a->head_dim);
    return HSWA_E_INVAL;
  }
  if (a->num_kv_heads < 1 || a->num_kv_heads > hswa::kMaxKvHeads || a->num_seqs < 0 ||
      a->total_tok < 0 || a->max_tok < 0 || (a->total_tok > 0 && a->max_tok < 1)) {
    hswa::set_error("1 <= num_kv_heads <= %d; num_seqs, total_tok, max_tok >= 0 required",
                    hswa::kMaxKvHeads);
    return HSWA_E_INVAL;
  }
  if (a->num_seqs == 0 || a->total_tok == 0) return HSWA_OK;
  const hswa_pool_view& v = a->pool;
  if (!v.seq_len || !v.fpt || !v.rpt || v.ring_slots < 16 || v.ring_slots % 16 ||
      v.max_pages_per_seq < 1 || v.max_seqs < 1) {
    hswa::set_error("pool view is invalid");
    return HSWA_E_INVAL;
  }
  if (a->kind == HSWA_LAYER_SWA && a->max_tok > v.ring_slots) {
    hswa::set_error("SWA transfer of %d positions per sequence: the ring holds %d", a->max_tok,
                    v.ring_slots);
    return HSWA_E_INVAL;
  }
  if (!a->seq_ids || !a->cu_tok || !a->k_cache || !a->v_cache || !a->buf_k || !a->buf_v) {
    hswa::set_error("seq_ids, cu_tok, k_cache, v_cache, buf_k and buf_v must be set");
    return HSWA_E_INVAL;
  }
  const void* ptrs[] = {a->k_cache, a->v_cache, a->buf_k, a->buf_v};
  for (const void* q : ptrs) {
    if (!aligned16(q)) {
      hswa::set_error("buffers must be 16-byte aligned");
      return HSWA_E_INVAL;
    }
  }
  if (a->kv_dtype != HSWA_KV_BF16 && a->kv_dtype != HSWA_KV_FP8) {
    hswa::set_error("kv_dtype must be HSWA_KV_BF16 or HSWA_KV_FP8 (got %d)", a->kv_dtype);
    return HSWA_E_INVAL;
  }
  const bool fp8 = a->kv_dtype == HSWA_KV_FP8;
  if (fp8 && (!a->k_scale || !a->v_scale || !a->buf_k_scale || !a->buf_v_scale)) {
    hswa::set_error("FP8 pages need k_scale, v_scale, buf_k_scale and buf_v_scale");
    return HSWA_E_INVAL;
  }
  if (fp8 && (!aligned16(a->k_scale) || !aligned16(a->v_scale) || !aligned4(a->buf_k_scale) ||
              !aligned4(a->buf_v_scale))) {
    hswa::set_error("k_scale and v_scale must be 16-byte aligned, the buffer scales 4-byte");
    return HSWA_E_INVAL;
  }
  hswa::XferParams p{};
  p.kind = a->kind;
  p.hkv = a->num_kv_heads;
  p.d = a->head_dim;
  p.num_seqs = a->num_seqs;
  p.seq_ids = a->seq_ids;
  p.cu_tok = a->cu_tok;
  p.first_pos = a->first_pos;
  p.max_tok = a->max_tok;
  p.total_tok = a->total_tok;
  p.k_cache = (uint16_t*)a->k_cache;
  p.v_cache = (uint16_t*)a->v_cache;
  p.t.seq_len = v.seq_len;
  p.t.fpt = v.fpt;
  p.t.rpt = v.rpt;
  p.t.max_pages = v.max_pages_per_seq;
  p.t.ring_slots = v.ring_slots;
  p.t.max_seqs = v.max_seqs;
  void* dv = nullptr;
  int rc = device_view(a->buf_k, "buf_k", &dv);
  if (rc) return rc;
  p.buf_k = (uint16_t*)dv;
  rc = device_view(a->buf_v, "buf_v", &dv);
  if (rc) return rc;
  p.buf_v = (uint16_t*)dv;
  if (fp8) {
    p.kv_fp8 = true;
    p.k_scale = (float*)a->k_scale;
    p.v_scale = (float*)a->v_scale;
    rc = device_view(a->buf_k_scale, "buf_k_scale", &dv);
    if (rc) return rc;
    p.buf_k_scale = (float*)dv;
    rc = device_view(a->buf_v_scale, "buf_v_scale", &dv);
    if (rc) return rc;
    p.buf_v_scale = (float*)dv;
  }
  hipError_t e = hswa::launch_xfer(p, to_host, (hipStream_t)stream);
  return e == hipSuccess ? HSWA_OK : hswa::hip_fail(e, "transfer launch");
}

}  // namespace

extern "C" {

int hswa_kv_copy(const hswa_kv_copy_args* a, void* stream) {
  hswa::clear_error();
  if (!a) {
    hswa::set_error("args is NULL");
    return HSWA_E_INVAL;
  }
  if (a->kind != HSWA_LAYER_FULL && a->kind != HSWA_LAYER_SWA) {
    hswa::set_error("kind must be HSWA_LAYER_FULL or HSWA_LAYER_SWA (got %d)", a->kind);
    return HSWA_E_INVAL;
  }
  if (a->head_dim != 64 && a->head_dim != 128) {
    hswa::set_error("head_dim must be 64 or 128 (got %d)", a->head_dim);
    return HSWA_E_INVAL;
  }
  if (a->num_kv_heads < 1 || a->num_kv_heads > hswa::kMaxKvHeads || a->num_seqs < 0 ||
      a->max_tok < 0) {
    hswa::set_error("1 <= num_kv_heads <= %d; num_seqs, max_tok >= 0 required",
                    hswa::kMaxKvHeads);
    return HSWA_E_INVAL;
  }
  if (a->num_seqs == 0 || a->max_tok == 0) return HSWA_OK;
  const hswa_pool_view& v = a->pool;
  if (!v.seq_len || !v.fpt || !v.rpt || v.ring_slots < 16 || v.ring_slots % 16 ||
      v.max_pages_per_seq < 1 || v.max_seqs < 1) {
    hswa::set_error("pool view is invalid");
    return HSWA_E_INVAL;
  }
  if (a->kind == HSWA_LAYER_SWA && a->max_tok > v.ring_slots) {
    hswa::set_error("SWA copy of %d positions per sequence: the ring holds %d", a->max_tok,
                    v.ring_slots);
    return HSWA_E_INVAL;
  }
  if (!a->src_ids || !a->dst_ids || !a->first_pos || !a->end_pos || !a->k_cache ||
      !a->v_cache) {
    hswa::set_error("src_ids, dst_ids, first_pos, end_pos, k_cache and v_cache must be set");
    return HSWA_E_INVAL;
  }
  if (!aligned16(a->k_cache) || !aligned16(a->v_cache)) {
    hswa::set_error("k_cache and v_cache must be 16-byte aligned");
    return HSWA_E_INVAL;
  }
  if (a->kv_dtype != HSWA_KV_BF16 && a->kv_dtype != HSWA_KV_FP8) {
    hswa::set_error("kv_dtype must be HSWA_KV_BF16 or HSWA_KV_FP8 (got %d)", a->kv_dtype);
    return HSWA_E_INVAL;
  }
  const bool fp8 = a->kv_dtype == HSWA_KV_FP8;
  if (fp8 && (!a->k_scale || !a->v_scale)) {
    hswa::set_error("FP8 pages need k_scale and v_scale");
    return HSWA_E_INVAL;
  }
  if (fp8 && (!aligned16(a->k_scale) || !aligned16(a->v_scale))) {
    hswa::set_error("k_scale and v_scale must be 16-byte aligned");
    return HSWA_E_INVAL;
  }
  hswa::CopyParams p{};
  p.kv_fp8 = fp8;
  p.k_scale = fp8 ? (float*)a->k_scale : nullptr;
  p.v_scale = fp8 ? (float*)a->v_scale : nullptr;
  p.kind = a->kind;
  p.hkv = a->num_kv_heads;
  p.d = a->head_dim;
  p.num_seqs = a->num_seqs;
  p.src_ids = a->src_ids;
  p.dst_ids = a->dst_ids;
  p.first_pos = a->first_pos;
  p.end_pos = a->end_pos;
  p.max_tok = a->max_tok;
  p.k_cache = (uint16_t*)a->k_cache;
  p.v_cache = (uint16_t*)a->v_cache;
  p.t.seq_len = v.seq_len;
  p.t.fpt = v.fpt;
  p.t.rpt = v.rpt;
  p.t.max_pages = v.max_pages_per_seq;
  p.t.ring_slots = v.ring_slots;
  p.t.max_seqs = v.max_seqs;
  hipError_t e = hswa::launch_copy(p, (hipStream_t)stream);
  return e == hipSuccess ? HSWA_OK : hswa::hip_fail(e, "copy launch");
}

int hswa_kv_offload(const hswa_xfer_args* a, void* stream) { return xfer(a, true, stream); }

int hswa_kv_restore(const hswa_xfer_args* a, void* stream) { return xfer(a, false, stream); }

}  // extern "C"
