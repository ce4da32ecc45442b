/*
 * hswa.h -- C ABI of the Hybrid Sliding-Window Attention hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * What it computes (sources, cited by page title and section):
 *
 *   [MiMo]  "MiMo-V2.5 Series Inference Full-Link Optimization: Pushing
 *           Hybrid SWA Efficiency to the Extreme" (mimo.mi.com).
 *           Sec. 1.1: most layers are SWA layers that attend only to the last
 *           W = 128 tokens, a few Full layers attend to the whole prefix;
 *           chunked prefill is roughly compute-bound.  Sec. 1.2: decode is
 *           roughly bound by the bytes of KV it reads.  Sec. 2.1 "KVCache
 *           Dual Pool": a Full pool of O(N) and a SWA pool of O(W) with its
 *           own window eviction, one logical sequence view in which the Full
 *           index is authoritative plus a Full-to-SWA map, and a joint
 *           capacity check on admission.  Sec. 2.1 "SWA-aware prefix cache
 *           tree", point 2: out-of-window SWA entries are released when a
 *           prefill chunk completes and as decode advances.
 *   [vLLM]  "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct
 *           MI355X" (vLLM blog), sec. 3 "Which bytes move?": KV addressed as
 *           16-token pages through a per-sequence page table.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns HSWA_OK (0) or a negative hswa_status.  The
 *    text of the last failure on the calling thread is hswa_last_error().
 *    No C++ exception crosses this boundary.
 *  - "host" pointers are ordinary CPU memory; "device" pointers are GPU
 *    memory of the current HIP device, owned by the caller.  The library
 *    allocates no device memory.  Device pointers must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    All device work is enqueued on it, asynchronously; nothing waits for
 *    the device except where a function says so.
 *  - Outputs never alias inputs.  Calls that use one pool, or one layer's
 *    K/V buffers, from several host threads at once are not supported.
 *  - bf16 tensors are passed as raw 16-bit words (void*).
 *
 * Memory layout of a layer's K/V pool (Full pool or SWA ring alike):
 *    K: [num_pages][Hkv][16][head_dim]  bf16   (token-major in a page)
 *    V: [num_pages][Hkv][head_dim][16]  fp16   (dim-major in a page)
 *  A token's slot is page * 16 + offset.  One (page, head) block is
 *  16 * head_dim * 2 bytes contiguous for K and for V.  V is kept in fp16
 *  because the PV product runs on the fp16 MFMA: the append converts the
 *  bf16 input with round to nearest even, which is exact for every bf16
 *  value with 2^-14 <= |v| <= 65280 (65280 is the largest bf16 value below
 *  fp16's limit 65504), rounds smaller magnitudes to fp16 subnormals (error
 *  <= 2^-25) and turns |v| >= 65536 (the next bf16 value) into +-inf, which
 *  makes the attention outputs of that dimension non-finite for every query
 *  whose window holds the key.  The supported V domain is |v| <= 65280.
 *  Callers that write pages themselves write V in fp16.
 */
#ifndef HSWA_H
#define HSWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum hswa_status {
  HSWA_OK = 0,
  HSWA_E_INVAL = -1,       /* bad argument, size, alignment or shape       */
  HSWA_E_NOSPC = -2,       /* joint Full/SWA capacity check failed; the
                              pool is unchanged                             */
  HSWA_E_HIP = -3,         /* a HIP runtime call or kernel launch failed    */
  HSWA_E_UNSUPPORTED = -4  /* valid request outside what is built          */
} hswa_status;

typedef enum hswa_layer_kind {
  HSWA_LAYER_FULL = 0,     /* keys 0..i of query position i ([MiMo] 1.1)  */
  HSWA_LAYER_SWA = 1       /* keys max(0, i-W+1)..i, W keys counting the
                              query itself ([MiMo] 1.1; 2.1 prefix tree,
                              point 1 counts the window the same way)     */
} hswa_layer_kind;

#define HSWA_PAGE_SIZE 16

/* Storage of a layer's K/V pages.  HSWA_KV_FP8 follows the Baidu Day0
 * hybrid-attention article (Layered quantization, point 2: FP8 KV per
 * token, head and 128-element tile): OCP e4m3 codes, K [page][Hkv][16][d]
 * and V [page][Hkv][d][16] bytes, with one fp32 scale per (page, head,
 * token) for K and for V.  A row x of d <= 128 elements is one tile:
 * scale = amax/448, codes of x * (448/amax) rounded to nearest (ties to an
 * even fraction), saturated at 448; the value of a code times the scale is
 * what attention reads.  Appends quantize, decode and prefill read FP8
 * pages, and the copy and the tier transfer move their codes and scales
 * verbatim. */
/* Element type of attention outputs.  fp32 keeps the kernels' fp32
 * accumulation; fp16 halves the bytes written (11 significant bits: within
 * 2^-11 relative of the fp32 result, e.g. <= 2e-3 absolute for |o| < 8;
 * outputs are convex combinations of V, so |o| <= max |v|). */
typedef enum hswa_out_dtype {
  HSWA_OUT_F32 = 0,
  HSWA_OUT_F16 = 1
} hswa_out_dtype;

typedef enum hswa_kv_dtype {
  HSWA_KV_BF16 = 0,        /* K bf16, V fp16 (the layout above)             */
  HSWA_KV_FP8 = 1          /* K/V e4m3 codes plus fp32 scales               */
} hswa_kv_dtype;

/* Text of the last failure on this thread ("" if none).  Never NULL. */
const char* hswa_last_error(void);
/* Static name of a status code. */
const char* hswa_status_string(int status);
/* Library version as major*10000 + minor*100 + patch. */
int hswa_version(void);

/* ------------------------------------------------------------------------
 * Dual KV pool: slot bookkeeping ([MiMo] 2.1 "KVCache Dual Pool")
 *
 * The pool owns host metadata only.  It mirrors four caller-owned device
 * tables that the attention kernels read:
 *   seq_len [max_seqs]                       tokens stored per sequence
 *   fpt     [max_seqs * max_pages_per_seq]   Full page table, -1 = none
 *   rpt     [max_seqs * ring_slots/16]       SWA ring page table (fixed)
 *   map     [num_full_pages * 16]            Full slot -> SWA slot, -1 = no
 *                                            SWA entry (evicted or never)
 * Slot rules (integer, exact):
 *   full_slot(b, pos) = fpt[b][pos / 16] * 16 + pos % 16
 *   swa_slot(b, pos)  = rpt[b][(pos mod C) / 16] * 16 + (pos mod C) % 16
 * A sequence's Full page for position pos is taken from the head of a FIFO
 * free list when pos % 16 == 0; within a call sequences are served in the
 * order listed, positions ascending.  The SWA pool of a sequence is a ring
 * of C = ring_slots slots; after eviction at length L exactly the last
 * min(L, W-1) positions stay resident, which is what the next query needs.
 * -------------------------------------------------------------------- */

typedef struct hswa_pool hswa_pool;

typedef struct hswa_pool_desc {
  int32_t page_size;          /* must be 16                                  */
  int32_t window;             /* W >= 1                                      */
  int32_t ring_slots;         /* C: multiple of 16, C >= W                   */
  int32_t max_seqs;           /* sequence ids are 0 .. max_seqs-1            */
  int32_t max_pages_per_seq;  /* row length of fpt                           */
  int32_t num_full_pages;     /* Full pool size in pages                     */
  const int32_t* full_free_order; /* host [num_full_pages]: initial free list,
                                     a permutation of 0..num_full_pages-1   */
  const int32_t* ring_pages;  /* host [max_seqs * C/16]: ring page ids of
                                 each sequence, a permutation of
                                 0..max_seqs*C/16-1                          */
  /* Device tables (caller-owned, int32).  All four NULL gives a host-only
     pool (bookkeeping without a device mirror); otherwise all four must be
     set.  hswa_pool_create fills them synchronously.                        */
  int32_t* dev_seq_len;
  int32_t* dev_fpt;
  int32_t* dev_rpt;
  int32_t* dev_map;
} hswa_pool_desc;

/* Device-table view of a pool, read by the attention entry points. */
typedef struct hswa_pool_view {
  const int32_t* seq_len;
  const int32_t* fpt;
  const int32_t* rpt;
  const int32_t* map;
  int32_t max_seqs;
  int32_t max_pages_per_seq;
  int32_t ring_slots;
  int32_t window;
} hswa_pool_view;

/* Validates desc, copies it, writes the initial device tables (seq_len = 0,
   fpt = -1, rpt = ring_pages, map = -1) with a blocking copy.  *out owns
   host memory only; release it with hswa_pool_destroy. */
int hswa_pool_create(const hswa_pool_desc* desc, hswa_pool** out);
/* Waits for the pool's pending table updates, then frees host state.
   NULL is a no-op. */
void hswa_pool_destroy(hswa_pool* pool);
/* Fills *out with the device tables and geometry ([MiMo] 2.1). */
int hswa_pool_get_view(const hswa_pool* pool, hswa_pool_view* out);

/* Step "alloc" ([MiMo] 2.1 Dual Pool; Scheduling Constraints): gives Full
 * and SWA slots to n_new[i] >= 0 new positions of sequence seq_ids[i]
 * (host arrays of length n_seqs, ids distinct).  The joint check runs first
 * and nothing changes if it fails (HSWA_E_NOSPC): the Full free list must
 * hold every page the call needs, each sequence's page-table row must fit,
 * and each ring must hold resident_b + n_new_b <= C.
 * full_slots_out / swa_slots_out (host, nullable) receive sum(n_new)
 * entries: sequences in the order listed, positions ascending.  The device
 * tables (seq_len, fpt, map) are updated on `stream`. */
int hswa_pool_alloc(hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                    const int32_t* n_new, int32_t* full_slots_out,
                    int32_t* swa_slots_out, void* stream);

/* Step "evict" ([MiMo] 2.1 prefix tree, point 2): for each listed sequence
 * of length L, releases the SWA entry of every resident position
 * pos <= L - W (map[full_slot] = -1).  The library computes the set itself,
 * so an in-window position can never be evicted.  evicted_out (host,
 * nullable, capacity evicted_cap entries) receives the Full slots released,
 * ascending position per sequence, sequences in the order listed;
 * counts_out (host, nullable, n_seqs entries) the number per sequence.
 * HSWA_E_INVAL, with nothing changed, if evicted_cap is too small.
 * On the device the call writes only the map entries of the released
 * positions: seq_len, fpt and rpt are left alone, and no attention kernel
 * reads the map.  `stream` may therefore be a second stream on which the
 * eviction overlaps attention over the same pool, provided it is ordered
 * after the alloc that set those entries and before the next alloc,
 * import, release or truncate of the pool (which may reuse their pages). */
int hswa_pool_evict(hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                    int32_t* evicted_out, int64_t evicted_cap,
                    int32_t* counts_out, void* stream);

/* One chunk step's end and the next one's start ([MiMo] 2.1 prefix tree,
 * point 2, and Dual Pool; Scheduling Constraints): hswa_pool_evict of
 * ev_ids followed by hswa_pool_alloc of al_ids, with the same arguments and
 * outputs as those two calls, as one operation.  Every check of both runs
 * first, the alloc's ring check counting the eviction, and nothing changes
 * if one fails.  A sequence may be listed in both (each list without
 * repeats).  The device tables receive both effects in one table-update
 * launch on `stream` instead of two; the eviction's second-stream rule does
 * not apply, since the alloc's effects ride along. */
int hswa_pool_evict_alloc(hswa_pool* pool, int32_t n_ev, const int32_t* ev_ids,
                          int32_t* evicted_out, int64_t evicted_cap, int32_t* counts_out,
                          int32_t n_al, const int32_t* al_ids, const int32_t* n_new,
                          int32_t* full_slots_out, int32_t* swa_slots_out, void* stream);

/* Appends n_new[i] positions whose K/V the caller stores directly, e.g. a
 * context restored from another cache tier where only the in-window SWA KV
 * moves ([MiMo] 2.1 Dual Pool, "Data Transfer").  Every new position gets a
 * Full slot; only positions inside the window of the new length get SWA
 * slots (others report -1), and resident positions that leave the window are
 * released as by hswa_pool_evict.  The ring check does not apply; the Full
 * check does (HSWA_E_NOSPC, nothing changed). */
int hswa_pool_import(hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                     const int32_t* n_new, int32_t* full_slots_out,
                     int32_t* swa_slots_out, void* stream);

/* Ends the listed requests ([MiMo] 2.1 prefix tree, point 2, "request
 * end"): their Full pages return to the tail of the free list in logical
 * page order, their SWA entries are dropped, their length becomes 0. */
int hswa_pool_release(hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                      void* stream);

/* Cuts sequence seq_ids[i] back to new_len[i] positions, e.g. the draft
 * tokens a multi-token verification step rejected ([MiMo] 5.2 runs three
 * MTP layers, so a step appends one token plus up to three drafts).
 * Positions >= new_len lose their SWA entry (map = -1); Full pages that no
 * longer hold a position go back to the HEAD of the free list, lowest
 * logical page first, so the next alloc takes them again.  The window of
 * the new length must still be resident, so call it before the step's
 * hswa_pool_evict.  HSWA_E_INVAL, with nothing changed, if any new_len is
 * outside [0, seq_len] or below the resident window
 * (resident start > max(0, new_len - W + 1)).  Host arrays of n_seqs
 * entries; device tables updated on `stream`. */
int hswa_pool_truncate(hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                       const int32_t* new_len, void* stream);

/* Window-safe prefix-match length ([MiMo] 2.1 "SWA-aware prefix cache
 * tree", point 1): for each listed sequence, the longest m' <= min(want[i],
 * seq_len) such that the last min(m', tail) positions before m' all still
 * hold an SWA entry of that sequence (map >= 0, at or after its first
 * resident position); the rest of a token match is a miss.  The
 * query at m' attends to W keys counting itself, so tail = W - 1 is what this
 * library's attention needs (and what eviction keeps); the page asks for
 * tail = W.  Host arrays of n_seqs entries; out receives m'.  Reads the host
 * metadata only.  HSWA_E_INVAL for a bad id, a negative want or tail. */
int hswa_pool_match_len(const hswa_pool* pool, int32_t n_seqs, const int32_t* seq_ids,
                        const int32_t* want, int32_t tail, int32_t* out);

/* Prefix reuse across requests ([MiMo] 2.1 "SWA-aware prefix cache tree",
 * points 1 and 3: a matched prefix keeps its Full part shareable and its SWA
 * part usable as far as the window-safe match reaches).  Empty sequence
 * dst_ids[i] takes the first lens[i] positions of src_ids[i]; lens[i] must be
 * window-safe for the source with tail W - 1 (hswa_pool_match_len), i.e. the
 * source still holds SWA entries for the W - 1 positions before it.
 *   - The Full pages wholly below the destination's window start
 *     s = max(0, lens[i] - W + 1) are shared with the source (each page
 *     counts the sequences holding it; release frees it when the last one
 *     lets go).
 *   - The pages from the one holding s up to the one holding lens[i] - 1 are
 *     fresh (free-list head, logical order), and positions [s, lens[i]) get
 *     the destination's ring slots and map entries.  Every map entry so has
 *     one owner: shared positions stay outside the destination's window.
 *   - full_from[i] / swa_from[i] (host, nullable) receive the first position
 *     whose K/V the caller copies from source to destination with
 *     hswa_kv_copy, up to lens[i]: 16 * (s / 16) for FULL layers (the fresh
 *     pages), s for SWA layers (the window).
 * Checks come first and nothing changes on failure: HSWA_E_INVAL for a bad
 * id, a destination that is not empty or is also a source, a length outside
 * [0, source length] or not window-safe; HSWA_E_NOSPC when the Full pool
 * lacks the fresh pages of all forks together or a row is too short.  A
 * sequence may not be cut (hswa_pool_truncate) into a page another sequence
 * holds: HSWA_E_INVAL.  Device tables are updated on `stream`. */
int hswa_pool_fork(hswa_pool* pool, int32_t n, const int32_t* src_ids, const int32_t* dst_ids,
                   const int32_t* lens, int32_t* full_from, int32_t* swa_from, void* stream);

/* Host copies of the pool's metadata for inspection (each pointer nullable):
 * seq_len [max_seqs], fpt [max_seqs*max_pages_per_seq], map
 * [num_full_pages*16], free_pages [num_full_pages] (free list head first)
 * with its length in *n_free. */
int hswa_pool_read_tables(const hswa_pool* pool, int32_t* seq_len, int32_t* fpt,
                          int32_t* map, int32_t* free_pages, int32_t* n_free);

/* ------------------------------------------------------------------------
 * Attention over the dual pool
 * -------------------------------------------------------------------- */

typedef struct hswa_attn_args {
  int32_t kind;             /* hswa_layer_kind                              */
  int32_t window;           /* SWA: 1 <= window <= pool window; FULL: unused */
  int32_t num_q_heads;      /* Hq                                           */
  int32_t num_kv_heads;     /* Hkv in [1, 1024]; Hq / Hkv in {1, 2, 4, 8}    */
  int32_t head_dim;         /* 64 or 128                                    */
  float scale;              /* softmax scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t num_seqs;         /* sequences in this call                       */
  const int32_t* seq_ids;   /* device [num_seqs], distinct pool sequence ids */
  const int32_t* cu_q;      /* device [num_seqs+1], row offsets of each
                               sequence's query rows; required by prefill,
                               optional for decode (NULL: one row each)     */
  int32_t total_q;          /* rows of q / out (= cu_q[num_seqs]; decode
                               without cu_q: num_seqs).  A sequence whose
                               rows [cu_q[i], cu_q[i+1]) leave [0, total_q)
                               is skipped: nothing of it is read or written */
  int32_t max_q_len;        /* max rows of one sequence (host hint sizing
                               the grid; must be >= the true max).  Prefill
                               rows past a smaller hint are not computed:
                               they are written as NaN, with vlen_out -1.
                               Decode with cu_q: 1..4                        */
  int32_t max_seq_len;      /* decode: the longest listed sequence's length
                               (host hint sizing the split-K plan and the
                               workspace).  A smaller hint costs speed, not
                               correctness: a longer sequence is cut into
                               the planned number of (longer) splits        */
  const void* q;            /* device bf16 [total_q][Hq][head_dim]          */
  const void* k_new;        /* device bf16 [total_q][Hkv][head_dim] or NULL  */
  const void* v_new;        /* device bf16 [total_q][Hkv][head_dim] or NULL  */
  hswa_pool_view pool;      /* from hswa_pool_get_view                      */
  void* k_cache;            /* this layer's K pages: the Full pool for FULL
                               layers, the SWA ring pool for SWA layers     */
  void* v_cache;            /* this layer's V pages (layout above)          */
  void* out;                /* device [total_q][Hq][head_dim], fp32 or fp16
                               as out_dtype says                             */
  int32_t* vlen_out;        /* device int32 [total_q] or NULL: number of keys
                               each query row attended to                   */
  int32_t kv_dtype;         /* hswa_kv_dtype of k_cache/v_cache              */
  void* k_scale;            /* HSWA_KV_FP8: device fp32 [num_pages][Hkv][16],
                               one scale per token of each (page, head)      */
  void* v_scale;            /* HSWA_KV_FP8: the same for V; else NULL        */
  int32_t out_dtype;        /* hswa_out_dtype of out                         */
  const int32_t* q_pos;     /* device [num_seqs] or NULL: position of each
                               sequence's first query row.  NULL: the rows
                               are the last positions, [seq_len - n, seq_len)
                               read from the pool's seq_len table.  Given:
                               [q_pos[i], q_pos[i] + n) (they must have
                               slots), and SWA attention and appends then
                               read no table that an alloc, evict or import
                               writes (only the fixed ring table), so those
                               pool calls may run on another stream beside
                               them.  Full layers still read fpt, so their
                               alloc must precede them.                      */
} hswa_attn_args;

/* Chunked prefill of one layer ([MiMo] 1.1 chunked prefill; 2.1 prefix
 * tree, point 2).  The query rows of sequence i are its LAST
 * (cu_q[i+1]-cu_q[i]) positions, i.e. the tokens just given slots by
 * hswa_pool_alloc: row r is position seq_len - n_i + (r - cu_q[i]).  When
 * k_new/v_new are set they are first written into k_cache/v_cache at those
 * positions' slots (Full slots for FULL layers, SWA ring slots for SWA
 * layers); then each row attends to its keys through the page tables.
 * Every needed key must be resident, which holds when the caller allocates
 * the chunk after evicting the previous one.  Output fp32 or fp16
 * (out_dtype).  FP8 pages (kv_dtype HSWA_KV_FP8, k_scale/v_scale set): the
 * append quantizes the rows, and attention reads K as code values with
 * each score times its key's K scale, and V as code * scale rounded to
 * fp16. */
int hswa_prefill_chunk(const hswa_attn_args* args, void* stream);

/* Decode step of one layer ([MiMo] 1.2).  Without cu_q: one query row per
 * listed sequence, at position seq_len - 1.  With cu_q: sequence i has
 * n_i = cu_q[i+1] - cu_q[i] rows, 1 <= n_i <= max_q_len <= 4, its last n_i
 * positions (one new token plus the drafts of a multi-token verification
 * step; [MiMo] 5.2 runs three MTP layers), each row attending causally to
 * its own keys (SWA: the W keys ending at its position); all rows of a
 * sequence share every K/V byte read.  A SWA ring must then hold
 * W - 1 + n_i slots.  max_q_len > 4 is HSWA_E_UNSUPPORTED.  Appends
 * k_new/v_new when set, then attends; FULL layers split the context across
 * workgroups and merge the parts (log-sum-exp) in a second kernel.
 * `workspace` is a caller-owned device buffer of at least
 * hswa_decode_workspace_bytes(args) bytes (may be NULL when that is 0;
 * the size depends on kind, window, num_seqs, max(total_q, num_seqs), the
 * head counts, head_dim and max_seq_len, and no memory is read);
 * HSWA_E_INVAL if it is smaller.  It receives the split partial states and
 * the call's work list (which the call builds itself: the buffer needs no
 * initialisation), so calls in flight at the same time need workspaces of
 * their own. */
int hswa_decode(const hswa_attn_args* args, void* workspace, size_t ws_bytes,
                void* stream);
size_t hswa_decode_workspace_bytes(const hswa_attn_args* args);

/* Decode without allocation, for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, plan, kernels and
 * results (bitwise) as hswa_decode with a workspace of
 * hswa_decode_workspace_bytes(args) bytes; the split-K partial states and
 * work list go instead to a device array of HSWA_DECODE_SCRATCH_BYTES that the library
 * holds on each GPU it runs on until the process ends (its address is
 * looked up on the first call on a device).  No memory is allocated and
 * nothing in the array needs clearing between calls.  HSWA_E_INVAL, with
 * nothing launched, when the call needs more than the array holds
 * (hswa_decode_workspace_bytes(args) > HSWA_DECODE_SCRATCH_BYTES, e.g.
 * 1,024 rows of 64 heads at d = 128 over 128K-token contexts, 7 splits).
 * Every call on one GPU shares the array: calls whose device work overlaps
 * (other streams, other host threads) race and give undefined results, so
 * issue them in order on one stream. */
#define HSWA_DECODE_SCRATCH_BYTES ((size_t)128 << 20)
int hswa_decode_noalloc(const hswa_attn_args* args, void* stream);

/* KV append alone: writes k_new/v_new (both required when there are rows)
 * of the query rows described as for hswa_prefill_chunk (cu_q given) or
 * hswa_decode (cu_q NULL: one row per sequence) into k_cache/v_cache.  No
 * attention.  A call with no rows (num_seqs or total_q 0) does nothing. */
int hswa_append_kv(const hswa_attn_args* args, void* stream);

/* ------------------------------------------------------------------------
 * Window-masked tier transfer ([MiMo] 2.1 "KVCache Dual Pool", Data
 * Transfer: moves between cache tiers go by the SWA mask, so only the valid
 * window of a SWA layer crosses the link; "KVCache asynchronous
 * layer-by-layer pulling": the small SWA pulls hide behind compute, one
 * layer at a time).
 *
 * The mask of a sequence of length L: a SWA layer moves positions
 * [max(0, L - W + 1), L) -- the window the next query reads, which is what
 * eviction keeps resident -- and a FULL layer moves [0, L).
 * -------------------------------------------------------------------- */

/* Tokens the mask moves per listed sequence (host arrays of n_seqs entries,
 * from the pool's host metadata): FULL seq_len, SWA min(seq_len, W - 1). */
int hswa_pool_window_counts(const hswa_pool* pool, int32_t kind, int32_t n_seqs,
                            const int32_t* seq_ids, int32_t* counts_out);

typedef struct hswa_xfer_args {
  int32_t kind;             /* hswa_layer_kind of the layer whose pages move  */
  int32_t num_kv_heads;     /* Hkv in [1, 1024]                              */
  int32_t head_dim;         /* 64 or 128                                     */
  int32_t num_seqs;
  const int32_t* seq_ids;   /* device [num_seqs], distinct pool sequence ids  */
  const int32_t* cu_tok;    /* device [num_seqs+1]: sequence i moves
                               n_i = cu_tok[i+1]-cu_tok[i] positions (the
                               counts of hswa_pool_window_counts for a masked
                               move) ...                                     */
  const int32_t* first_pos; /* ... from device first_pos[i] on, or, when NULL,
                               its last n_i positions [seq_len - n_i, seq_len).
                               Explicit positions let a transfer run on one
                               stream while allocs on another grow seq_len.
                               A sequence whose range is not below seq_len is
                               skipped.                                      */
  int32_t total_tok;        /* cu_tok[num_seqs]; a sequence whose tokens
                               [cu_tok[i], cu_tok[i+1]) leave [0, total_tok)
                               is skipped                                    */
  int32_t max_tok;          /* host hint >= every per-sequence count; SWA:
                               at most ring_slots (HSWA_E_INVAL otherwise).
                               SWA positions below seq_len - ring_slots are
                               no longer in the ring (their slots hold newer
                               positions): offload leaves their buffer rows
                               unwritten and restore does not write them    */
  hswa_pool_view pool;      /* from hswa_pool_get_view                       */
  void* k_cache;            /* this layer's K pages (layout above)           */
  void* v_cache;            /* this layer's V pages                          */
  void* buf_k;              /* [total_tok][Hkv][head_dim] 16-bit words, K as
                               bf16; pinned host memory (hipHostMalloc, or a
                               torch pin_memory tensor) or device memory     */
  void* buf_v;              /* same layout, V as fp16 (the pool's format)    */
  int32_t kv_dtype;         /* hswa_kv_dtype of the pages; HSWA_KV_FP8: buf_k
                               and buf_v hold [total_tok][Hkv][head_dim] e4m3
                               code bytes (V token-major too) ...            */
  void* k_scale;            /* ... the pages' device fp32 scales
                               [num_pages][Hkv][16] of K and of V (NULL for
                               BF16 pages) ...                               */
  void* v_scale;
  void* buf_k_scale;        /* ... and [total_tok][Hkv] fp32 scales of K and
                               of V, pinned host or device memory like the
                               code buffers; 4-byte aligned (all other
                               buffers 16-byte)                              */
  void* buf_v_scale;
} hswa_xfer_args;

/* Offload: copies the listed positions' K/V from the layer's pages into
 * buf_k/buf_v (sequences in the order listed, positions ascending).  The
 * copy is asynchronous on `stream`; read the buffers after it completes.
 * FP8 pages move their code bytes and each position's K and V scales.
 * HSWA_E_INVAL for a bad argument (FP8 without all four scale arrays) or a
 * buffer that is neither device memory nor pinned host memory. */
int hswa_kv_offload(const hswa_xfer_args* args, void* stream);

/* Restore: writes buf_k/buf_v into the pages at the listed positions' slots
 * (Full slots for FULL layers, ring slots for SWA layers), typically after
 * hswa_pool_import gave the restored context its slots; other positions of a
 * page are untouched.  Asynchronous on `stream`; keep the buffers unchanged
 * until it completes.  Offload then restore gives back the same bits. */
int hswa_kv_restore(const hswa_xfer_args* args, void* stream);

/* ------------------------------------------------------------------------
 * K/V copy between sequences of one pool, for prefix reuse ([MiMo] 2.1
 * "SWA-aware prefix cache tree", point 3): after hswa_pool_fork, a FULL
 * layer copies positions [full_from, len) of each fork and a SWA layer
 * [swa_from, len) from the source's pages to the destination's.
 * -------------------------------------------------------------------- */
typedef struct hswa_kv_copy_args {
  int32_t kind;             /* hswa_layer_kind of the layer whose pages copy */
  int32_t num_kv_heads;     /* Hkv in [1, 1024]                               */
  int32_t head_dim;         /* 64 or 128                                      */
  int32_t num_seqs;         /* copies in this call                           */
  const int32_t* src_ids;   /* device [num_seqs]: source sequence ids        */
  const int32_t* dst_ids;   /* device [num_seqs]: destination sequence ids   */
  const int32_t* first_pos; /* device [num_seqs]: copy i moves positions     */
  const int32_t* end_pos;   /* [first_pos[i], end_pos[i]) (device) ...        */
  int32_t max_tok;          /* ... host hint >= every end_pos - first_pos;
                               SWA: at most ring_slots                        */
  hswa_pool_view pool;      /* from hswa_pool_get_view                        */
  void* k_cache;            /* this layer's K pages (layout above)            */
  void* v_cache;            /* this layer's V pages                           */
  int32_t kv_dtype;         /* hswa_kv_dtype of the pages                     */
  void* k_scale;            /* HSWA_KV_FP8: device fp32 [num_pages][Hkv][16]  */
  void* v_scale;            /* scales of K and V, copied with the codes; else
                               NULL                                          */
} hswa_kv_copy_args;

/* Copies, for every listed pair, the K and V of positions [first_pos,
 * end_pos) from the source's slots to the destination's slots of the same
 * positions (Full slots for FULL layers, ring slots for SWA layers); the
 * bits are copied verbatim and other positions of a page are untouched.
 * Positions at or beyond either sequence's length are not copied, nor, for
 * SWA layers, positions older than length - ring_slots of either sequence
 * (their slots hold newer positions); a pair with equal ids copies nothing.
 * Asynchronous on `stream`, ordered after the hswa_pool_fork that gave the
 * destination its slots.  FP8 pages copy each position's codes and its K
 * and V scales.  HSWA_E_INVAL for a bad argument (FP8 without both scale
 * arrays) or an SWA max_tok above ring_slots. */
int hswa_kv_copy(const hswa_kv_copy_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSWA_H */
