// Paged decode attention over the dual pool: one to four query rows per
// sequence (one new token, or one token plus the drafts of a multi-token
// verification step).
//
// "MiMo-V2.5 Series Inference Full-Link Optimization" sec. 1.2: decode is
// bound by the bytes of KV it reads.  A Full layer reads the whole prefix
// through the Full page table; a SWA layer reads at most W keys (plus the
// step's other rows) from the sequence's ring (sec. 2.1 "KVCache Dual
// Pool").  Sec. 5.2 decodes with three MTP layers, i.e. up to four rows of
// one sequence are verified at once; they share every K/V byte read here.
//
// Design (gfx950):
//  - One workgroup = 4 wavefronts works on one (sequence, KV head, split)
//    at a time.  Full layers split a context of L keys into ceil(L /
//    split_len) equal pieces (64-key multiples) of the plan's n_splits, so
//    there is work for 256 CUs without short tail pieces; pieces are merged
//    by log-sum-exp in decode_combine_kernel.  Shorter contexts leave some
//    of the n_splits empty, so split-K calls run a work queue: a pre-pass
//    lists the pieces that hold keys, longest first, and as many
//    workgroups as the device holds take (piece, KV head) items from it,
//    instead of one workgroup per (sequence, split, KV head) most of which
//    would find nothing to do and still hold back dispatch.
//  - The (row, head) pairs that share a KV head ride in the N dimension of
//    16x16x32 MFMAs: S^T[key][col] = K[key][:] . Q[col][:], column
//    col = row * G + head, in 16-column tiles.  Every K/V byte is read from
//    HBM once for all G heads and all rows of the sequence.  Past 16 columns
//    (8 heads, more than 2 rows) a wave carries two tiles' state, so two
//    waves per SIMD fit instead of three; splitting the tiles over wave
//    pairs measured slower (each pair re-reads the K/V step and has half
//    the unique bytes in flight), and so did a second V buffer issued one
//    phase earlier.
//  - K rows (token-major pages) are the A operand loaded straight from HBM,
//    16 bytes per lane.  The 32 keys of a step are dealt to the two 16-row
//    score tiles so that each lane's eight scores are eight consecutive keys
//    of one page (tile 0 row 4a+r is key 8a+r, tile 1 row 4a+r is key
//    8a+4+r); with V pages dim-major and in fp16, the PV product
//    O^T[d][col] = V^T[d][key] . P^T[key][col] then reads each lane's V
//    fragment as 16 contiguous bytes and needs no conversion.  P enters the
//    PV MFMA as fp16, keeping the weights to 11 significant bits.
//  - Each column has its own causal (and window) limit: row r of a sequence
//    with n rows sits at position L - n + r.
//  - Online softmax in fp32 in the log2 domain (exp2 of prescaled scores).
//  - FP8 pages (e4m3 codes, one fp32 scale per token and head): codes
//    convert exactly to bf16 (K) and fp16 (V); the K scale multiplies each
//    score, the V scale (times 2^8) each fp16 weight, so the MFMAs see exact
//    codes and half the bytes move.
//  - Wave w takes 32-key steps w, w+4, ...; the four partial states merge
//    through LDS in a fixed order, so results depend only on logical key
//    positions, never on where pages sit in memory.
#include <hip/hip_runtime.h>

#include <algorithm>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kDecWaves = 4;

// K/V page loads, non-temporal or plain.  A Full layer's keys are read once
// per call; on bf16 pages non-temporal loads measured 7% faster on 128K-256K
// contexts, on FP8 pages 6% slower (same box, alternating runs), so only
// bf16 Full layers use them.  A SWA window's first and last keys can share
// one ring page (a ring of W slots), which two steps of a wave then read:
// plain loads let the second read hit L2, where non-temporal ones went to
// HBM again (10% more bytes per call).
template <bool NT, typename T>
__device__ __forceinline__ T ld_kv(const T* a) {
  if constexpr (NT)
    return __builtin_nontemporal_load(a);
  else
    return *a;
}

// One output element in the caller's output type (fp32, or fp16 rounded to
// nearest).
__device__ __forceinline__ void store_out(const AttnParams& p, int64_t idx, float x) {
  if (p.out_f16)
    ((_Float16*)p.out)[idx] = (_Float16)x;
  else
    ((float*)p.out)[idx] = x;
}

// Merges the four waves' partial states of a workgroup (fixed order), one
// column tile at a time, and stores the result (one split) or the partial
// state for decode_combine_kernel (several splits).  Column 16t + c of tile
// t is (row, head) = ((16t + c) / G, (16t + c) % G) of KV head kvh; with
// NCH > 0 the columns cover KV heads 2 kvh and 2 kvh + 1, NCH each.
template <int D, int G, int NT, int CT, int NCH = 0>
__device__ __forceinline__ void merge_store(const AttnParams& p, float (&red_o)[kDecWaves][CT][D],
                                            float (&red_ml)[kDecWaves][CT][2],
                                            const f32x4 (&o)[NT][D / 16], const float (&m)[NT],
                                            const float (&lsum)[NT], int kvh, int split,
                                            int row0, int nr) {
  constexpr int NB = D / 16;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int q4 = lane >> 4;
  const int hq = p.hq;
  const int hq_base = (NCH > 0 ? 2 * kvh : kvh) * G;
  for (int t = 0; t < NT; ++t) {
    float ls = lsum[t];
    ls += xor_lane(ls, 16);
    ls += xor_lane(ls, 32);
    if (t > 0) __syncthreads();  // the previous tile's merge has read LDS
    if (col < CT) {
      for (int nb = 0; nb < NB; ++nb)
        *(f32x4*)(&red_o[wave][col][16 * nb + 4 * q4]) = o[t][nb];
      if (q4 == 0) {
        red_ml[wave][col][0] = m[t];
        red_ml[wave][col][1] = ls;
      }
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < CT * D; idx += blockDim.x) {
      const int c = idx / D;
      const int d = idx % D;
      const int g0 = 16 * t + c;
      const int mem = NCH > 0 ? g0 / NCH : 0;  // which KV head of the pair
      const int g = NCH > 0 ? g0 % NCH : g0;
      const int r = g / G;
      if (r >= nr) continue;
      float M = -INFINITY;
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_ml[w][c][0]);
      float num = 0.f, den = 0.f;
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = red_ml[w][c][0];
        const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        num += sc * red_o[w][c][d];
        den += sc * red_ml[w][c][1];
      }
      const int64_t hrow = (int64_t)(row0 + r) * hq + hq_base + mem * G + g % G;
      if (p.n_splits == 1) {
        store_out(p, hrow * D + d, num / den);
      } else {
        const int64_t slot = hrow * p.n_splits + split;
        p.ws[slot * D + d] = num;
        if (d == 0) {
          float* ml = p.ws + (int64_t)p.total_q * hq * p.n_splits * D;
          ml[2 * slot] = M;
          ml[2 * slot + 1] = den;
        }
      }
    }
  }
}

// Block -> ((sequence, split) unit, KV head).  KV heads run fastest, so
// workgroups running at the same time read all heads' slices of the pages,
// which spreads their traffic over all HBM channels.  FP8 pages with an even
// head count pair heads 2j and 2j + 1 on one XCD, whose scale rows share a
// 128-byte line (idx::fp8_block).  False for padding blocks.
template <bool F8>
__device__ __forceinline__ bool decode_block(const AttnParams& p, int* unit, int* kvh) {
  if (F8 && (p.hkv & 1) == 0)
    return idx::fp8_block(blockIdx.x, p.hkv, p.num_seqs * p.n_splits, unit, kvh);
  *kvh = blockIdx.x % p.hkv;
  *unit = blockIdx.x / p.hkv;
  return true;
}

// Lazy rescaling of the bf16/fp16 decode (scores are in the log2 domain).
constexpr float kDecLazy = 8.0f;

// Split-K calls: the workgroup takes (unit, KV head) items from its queue
// (idx::queue_of_block, idx::queue_item) until the queue is exhausted and
// runs body(unit, head) on each; the pre-pass (decode_units_kernel) has
// listed the units that hold keys and zeroed the counters.  Other calls,
// and SWA layers (one split): one item, from the block index.  Every
// workgroup ends once its queue's counter passes the item count; no
// workgroup waits on another.
template <int KIND, bool PAIRED, typename F>
__device__ __forceinline__ void for_each_item(const AttnParams& p, F&& body) {
  const bool queued = KIND == 0 && p.queue;  // uniform
  const bool paired = PAIRED && (p.hkv & 1) == 0;
  __shared__ int s_k;
  const int q = idx::queue_of_block(blockIdx.x, paired);
  for (int it = 0;; ++it) {
    int unit, kvh;
    if (!queued) {
      if (it > 0 || !decode_block<PAIRED>(p, &unit, &kvh)) return;
    } else {
      if (threadIdx.x == 0)
        s_k = __hip_atomic_fetch_add(p.queue + idx::kQueueStride * q, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const int k = s_k;
      __syncthreads();  // every wave has read s_k before it is written again
      const int units = min(p.queue[idx::kQueueCount], p.num_seqs * p.n_splits);
      int a;
      if (!idx::queue_item(k, q, units, p.hkv, paired, &a, &kvh)) return;
      unit = p.queue[idx::kQueueList + a];
    }
    body(unit, kvh);
  }
}

template <int D, int KIND, int G, int QN, bool F8>
__device__ __forceinline__ void decode_unit(const AttnParams& p, const int unit, const int kvh) {
  constexpr int NB = D / 16;                  // 16-row d blocks of O^T
  constexpr int NC = D / 32;                  // 32-wide d chunks of the QK reduction
  constexpr int NCOL = G * QN;                // (row, head) columns
  constexpr int NT = (NCOL + 15) / 16;        // 16-column tiles
  constexpr int CT = NCOL < 16 ? NCOL : 16;   // columns used per tile
  constexpr int ESZ = F8 ? 1 : 2;             // bytes per stored K/V element
  // a lane's 8 elements of a K row or V column: 16 bytes (bf16 / fp16) or
  // 8 bytes (e4m3 codes)
  typedef typename std::conditional<F8, u32x2, u32x4>::type Raw;
  __shared__ __attribute__((aligned(16))) float red_o[kDecWaves][CT][D];
  __shared__ float red_ml[kDecWaves][CT][2];

  // unit = (sequence, split)
  const int i = unit / p.n_splits;
  const int split = unit % p.n_splits;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;  // rows: positions L-n .. L-1
  const int L = call_len(p, i, sid, n);
  if (n <= 0 || n > L || row0 < 0 || row0 + n > p.total_q) return;
  const int nr = min(n, QN);                         // rows computed here
  int klo, khi;  // keys [klo, khi) of this workgroup
  if (KIND == 0) {
    const int len = idx::split_keys(L, p.n_splits, p.split_len);
    klo = split * len;
    khi = min(L, klo + len);
  } else {
    klo = max(0, L - n - p.window + 1);  // window start of the first row
    khi = L;
  }
  if (klo >= khi) return;  // whole workgroup idle: no barrier reached

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // column within a tile (N index)
  const int q4 = lane >> 4;   // which 8-wide k slice / 4-row group
  const int hq = p.hq;
  const int hkv = p.hkv;
  const int W = p.window;

  // Per column tile t: this lane's column 16t + col is (row, head) =
  // ((16t + col) / G, (16t + col) % G); its query position and whether it
  // is a real pair.
  int cpos[NT];
  bool con[NT];
  bf16x8 qf[NT][NC];  // Q^T fragments: lane holds Q[col][32c + 8*q4 .. +8]
  for (int t = 0; t < NT; ++t) {
    const int gc = 16 * t + col;
    const int r = gc / G;
    con[t] = col < CT && r < nr;
    cpos[t] = L - n + r;
    const uint16_t* qrow = p.q + ((int64_t)(row0 + (con[t] ? r : 0)) * hq + kvh * G + gc % G) * D;
    for (int c = 0; c < NC; ++c) {
      u32x4 w = con[t] ? *(const u32x4*)(qrow + 32 * c + 8 * q4) : u32x4{0, 0, 0, 0};
      qf[t][c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x4 o[NT][NB];
  float m[NT], lsum[NT];
  for (int t = 0; t < NT; ++t) {
    for (int nb = 0; nb < NB; ++nb) o[t][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[t] = -INFINITY;
    lsum[t] = 0.f;
  }
  const float sl2 = p.scale_log2;

  const int s0 = (klo / 32) * 32;
  const int nsteps = (khi - 1 - s0) / 32 + 1;
  const int64_t blk = (int64_t)kPage * D * ESZ;  // bytes per (page, head) block

  // Page-table row of the sequence, read through the constant address space
  // so the lookups are scalar loads (the tables do not change while the
  // kernel runs).
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  const ctab_t ptab = (ctab_t)(KIND == 0 ? p.t.fpt + (int64_t)sid * p.t.max_pages
                                         : p.t.rpt + (int64_t)sid * (p.t.ring_slots / kPage));
  auto page_at = [&](int pos) {
    return ptab[__builtin_amdgcn_readfirstlane(idx::table_entry(KIND, pos, p.t.ring_slots))];
  };
  // K: this lane's row `col` of score tile kt is key 8*(col/4) + 4kt + col%4,
  // on page col/8.  V: keys 8*q4 .. +8 are page q4/2, offset 8*(q4%2); the
  // lane's scores and weights are those same 8 keys, so its FP8 scales are
  // 8 consecutive floats.
  const int kpage = col >> 3;
  const int krow0 = (8 * (col >> 2) + (col & 3)) & 15;
  const int k_lane = (krow0 * D + 8 * q4) * ESZ;
  const int v_lane = (col * kPage + 8 * (q4 & 1)) * ESZ;
  const uint8_t* kbase = (const uint8_t*)p.k_cache;
  const uint8_t* vbase = (const uint8_t*)p.v_cache;
  struct Ptrs {
    const uint8_t* k;
    const uint8_t* v;
    int64_t sc;  // FP8: index of the lane's first key scale
  };
  auto step_pages = [&](int kp0) {
    // a page with no key of [klo, khi) reads the step's other page (those
    // keys are masked)
    int32_t pg0 = page_at(idx::decode_page_pos(kp0, 0, klo, khi));
    int32_t pg1 = page_at(idx::decode_page_pos(kp0, 1, klo, khi));
    // a missing page means the caller skipped alloc: read page 0 of the pool
    // instead of faulting (the result of such a call is undefined)
    pg0 = pg0 < 0 ? 0 : pg0;
    pg1 = pg1 < 0 ? 0 : pg1;
    const int64_t vblk = (int64_t)((q4 >> 1) ? pg1 : pg0) * hkv + kvh;
    return Ptrs{kbase + ((int64_t)(kpage ? pg1 : pg0) * hkv + kvh) * blk + k_lane,
                vbase + vblk * blk + v_lane, vblk * kPage + 8 * (q4 & 1)};
  };
  auto load_k = [&](const Ptrs& pt, Raw (&kr)[2][NC]) {
    for (int c = 0; c < NC; ++c) {
      kr[0][c] = ld_kv<KIND == 0 && !F8>((const Raw*)(pt.k + 32 * c * ESZ));
      kr[1][c] =
          ld_kv<KIND == 0 && !F8>((const Raw*)(pt.k + (4 * D + 32 * c) * ESZ));
    }
  };
  auto load_v = [&](const Ptrs& pt, Raw (&vr)[NB]) {
    for (int nb = 0; nb < NB; ++nb)
      vr[nb] = ld_kv<KIND == 0 && !F8>((const Raw*)(pt.v + 16 * nb * kPage * ESZ));
  };
  auto load_scales = [&](const Ptrs& pt, u32x4 (&sc)[4]) {
    if (F8) {
      sc[0] = *(const u32x4*)(p.k_scale + pt.sc);
      sc[1] = *(const u32x4*)(p.k_scale + pt.sc + 4);
      sc[2] = *(const u32x4*)(p.v_scale + pt.sc);
      sc[3] = *(const u32x4*)(p.v_scale + pt.sc + 4);
    }
  };
  auto kfrag = [&](const Raw& w) -> bf16x8 {
    if constexpr (F8) {
      const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
      return __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]});
    } else {
      return __builtin_bit_cast(bf16x8, w);
    }
  };
  auto vfrag = [&](const Raw& w, const Raw& mask) -> f16x8 {
    if constexpr (F8) {
      const u32x2 x = w & mask;
      const u32x2 a = e4m3x4_to_f16x4(x[0]), b = e4m3x4_to_f16x4(x[1]);
      return __builtin_bit_cast(f16x8, u32x4{a[0], a[1], b[0], b[1]});
    } else {
      return __builtin_bit_cast(f16x8, w & mask);
    }
  };

  // Software pipeline, register-neutral: the K loads (and FP8 scales) of
  // this wave's next step are issued as soon as the score MFMAs have
  // consumed the current K fragments, the V loads as soon as the PV MFMAs
  // have consumed V; so each wave keeps a step's worth of bytes in flight
  // through its math.
  Raw kr[2][NC], vr[NB];
  u32x4 sc[4], scn[4];  // FP8 scales of this step and of the next: K 0-1, V 2-3
  Ptrs pt;
  if (wave < nsteps) {
    pt = step_pages(s0 + 32 * wave);
    load_k(pt, kr);
    load_v(pt, vr);
    load_scales(pt, sc);
  }
  for (int st = wave; st < nsteps; st += kDecWaves) {
    const int kp0 = s0 + 32 * st;
    const bool more = st + kDecWaves < nsteps;
    Ptrs ptn = pt;
    if (more) ptn = step_pages(kp0 + 32 * kDecWaves);

    // S^T for the two 16-key tiles of every column tile, then refill K
    f32x4 s[NT][2];
    for (int t = 0; t < NT; ++t)
      for (int kt = 0; kt < 2; ++kt) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int c = 0; c < NC; ++c)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfrag(kr[kt][c]), qf[t][c], acc, 0, 0, 0);
        s[t][kt] = acc;
      }
    if (more) {
      load_k(ptn, kr);
      load_scales(ptn, scn);
    }
    // lane value (kt, r) is key kp0 + 8*q4 + 4kt + r.  Keys outside the
    // workgroup's range have their V zeroed (their slots may hold stale or
    // unwritten data); keys inside it but past a column's own position (or
    // before its window) only get a zero weight.
    unsigned valid = 0;
    for (int j = 0; j < 8; ++j) {
      const int kp = kp0 + 8 * q4 + j;
      valid |= (unsigned)(kp >= klo && kp < khi) << j;
    }
    // FP8: the K scale multiplies the score; the V scale (times 2^8, undone
    // at the end) goes into the fp16 weight of the key
    float kscale[8], vscale[8];
    for (int j = 0; j < 8; ++j) {
      kscale[j] = F8 ? __uint_as_float(sc[j >> 2][j & 3]) * sl2 : sl2;
      vscale[j] = F8 ? ((valid >> j) & 1u ? __uint_as_float(sc[2 + (j >> 2)][j & 3]) * 256.f : 0.f)
                     : 1.f;
    }
    f16x8 pf[NT];
    float alpha[NT];
    bool resc[NT];  // wave-uniform: this tile's O is rescaled in this step
    for (int t = 0; t < NT; ++t) {
      float mx = -INFINITY;
      float sv[8];
      for (int j = 0; j < 8; ++j) {
        const int kp = kp0 + 8 * q4 + j;
        bool ok = (valid >> j) & 1u;
        if (QN > 1) ok = ok && kp <= cpos[t] && (KIND == 0 || kp > cpos[t] - W);
        const float x = ok ? s[t][j >> 2][j & 3] * kscale[j] : -INFINITY;
        sv[j] = x;
        mx = fmaxf(mx, x);
      }
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      // bf16/fp16 pages: the running max moves (and O is rescaled) only when
      // a score exceeds it by more than 2^kDecLazy, so the fp16 weights stay
      // <= 2^kDecLazy.  FP8 weights carry the V scale and move every step.
      resc[t] = F8 || __builtin_amdgcn_ballot_w64(mx > m[t] + kDecLazy) != 0;
      if (resc[t]) {
        const float m_new = fmaxf(m[t], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        alpha[t] = fast_exp2(m[t] - m_use);
        m[t] = m_new;
      } else {
        alpha[t] = 1.f;
      }
      const float m_use = m[t] == -INFINITY ? 0.f : m[t];
      float ps = 0.f;
      for (int j = 0; j < 8; ++j) {
        const float e = fast_exp2(sv[j] - m_use);
        if (F8) {
          pf[t][j] = (_Float16)(e * vscale[j]);
          ps += e;
        } else {
          pf[t][j] = (_Float16)e;
          ps += (float)pf[t][j];  // sum the fp16 weights the PV product uses
        }
      }
      lsum[t] = lsum[t] * alpha[t] + ps;
    }
    Raw vmask;
    for (int x = 0; x < (int)(sizeof(Raw) / 4); ++x) vmask[x] = ~0u;
    if (valid != 0xffu) {
      for (int j = 0; j < 8; ++j)
        if (!((valid >> j) & 1u)) {
          if (F8)
            vmask[j >> 2] &= ~(0xffu << (8 * (j & 3)));
          else
            vmask[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
        }
    }
    for (int nb = 0; nb < NB; ++nb) {
      const f16x8 vf = vfrag(vr[nb], vmask);
      for (int t = 0; t < NT; ++t) {
        if (resc[t]) o[t][nb] *= alpha[t];
        o[t][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf[t], o[t][nb], 0, 0, 0);
      }
    }
    // refill V
    if (more) {
      load_v(ptn, vr);
      if (F8)
        for (int x = 0; x < 4; ++x) sc[x] = scn[x];
    }
    pt = ptn;
  }
  if (F8)  // the weights carried a factor 2^8
    for (int t = 0; t < NT; ++t)
      for (int nb = 0; nb < NB; ++nb) o[t][nb] *= 0.00390625f;

  merge_store<D, G, NT, CT>(p, red_o, red_ml, o, m, lsum, kvh, split, row0, nr);
  if (p.vlen && split == 0 && kvh == 0 && (int)threadIdx.x < nr) {
    const int pos = L - n + threadIdx.x;
    p.vlen[row0 + threadIdx.x] = KIND == 0 ? pos + 1 : min(pos + 1, W);
  }
}


template <int D, int KIND, int G, int QN, bool F8>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(G * QN > 16 ? 2 : 3, 4))) decode_kernel(AttnParams p) {
  for_each_item<KIND, F8>(p, [&](int unit, int kvh) { decode_unit<D, KIND, G, QN, F8>(p, unit, kvh); });
}

// FP8 decode with 64-key steps (one column tile: G * QN <= 16).  The step
// covers four pages; a lane's four score tiles hold all 16 keys of one page
// (tile kt row 4a + r is key 16a + 4kt + r), so its V fragment for the two
// PV products of the step is one 16-byte page row (keys 0-7, then 8-15) and
// its scales are 16 consecutive floats.  Each lane's K fragment is a
// contiguous quarter of the row (d in [q4 * D/4, (q4 + 1) * D/4)); Q takes
// the same order of the reduction.  A wave then keeps 16.5 KB in flight per
// step, as much as the bf16 path, at two waves per SIMD.
//
// PAIR (Full layers, G * QN <= 8): the unit covers KV heads 2 kvh and
// 2 kvh + 1 in 32-key steps over two pages.  Rows 4a .. 4a + 3 of a score
// tile (row group a) belong to page a >> 1 and head a & 1, so each wave
// reads the two heads' adjacent code blocks of a page, 4 KB in a run, and
// their scales as one 128-byte line.  The 16 columns are the two heads' G * QN (row, head)
// pairs; a lane whose rows belong to the other head of its column gets
// -inf scores, so it adds nothing to the column's max, sum or output.
template <int D, int KIND, int G, int QN, bool PAIR>
__device__ __forceinline__ void decode_fp8_unit(const AttnParams& p, const int unit,
                                                const int kvh) {
  constexpr int NB = D / 16;                  // 16-row d blocks of O^T
  constexpr int NC = D / 32;                  // 32-wide chunks of the QK reduction
  constexpr int DQ = D / 4;                   // contiguous K bytes of a lane per row
  constexpr int KV4 = DQ / 16;                // 16-byte loads per row and lane
  constexpr int NCH = G * QN;                 // columns per KV head
  constexpr int NCOL = PAIR ? 2 * NCH : NCH;
  constexpr int CT = NCOL;                    // one tile
  static_assert(NCOL <= 16, "one column tile");
  static_assert(!PAIR || KIND == 0, "head pairs serve Full layers");
  constexpr int SK = PAIR ? 32 : 64;          // keys per step
  constexpr int NPG = SK / kPage;             // pages per step
  __shared__ __attribute__((aligned(16))) float red_o[kDecWaves][CT][D];
  __shared__ float red_ml[kDecWaves][CT][2];

  // unit = (sequence, split)
  const int i = unit / p.n_splits;
  const int split = unit % p.n_splits;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  const int L = call_len(p, i, sid, n);
  if (n <= 0 || n > L || row0 < 0 || row0 + n > p.total_q) return;
  const int nr = min(n, QN);
  int klo, khi;
  if (KIND == 0) {
    const int len = idx::split_keys(L, p.n_splits, p.split_len);
    klo = split * len;
    khi = min(L, klo + len);
  } else {
    klo = max(0, L - n - p.window + 1);
    khi = L;
  }
  if (klo >= khi) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int q4 = lane >> 4;
  const int hq = p.hq;
  const int hkv = p.hkv;
  const int W = p.window;

  // column col: KV head h0 + mem, row crow, query head (h0 + mem) G + c2 % G
  const int h0 = PAIR ? 2 * kvh : kvh;
  const int mem = PAIR ? col / NCH : 0;
  const int c2 = PAIR ? col % NCH : col;
  const int crow = c2 / G;
  const bool con = col < CT && crow < nr;
  const int cpos = L - n + crow;
  // PAIR: this lane's score rows belong to its column's KV head
  const bool lane_head = !PAIR || (q4 & 1) == mem;
  bf16x8 qf[1][NC];  // lane holds Q[col][q4 * DQ + 8c .. +8]
  {
    const uint16_t* qrow =
        p.q + ((int64_t)(row0 + (con ? crow : 0)) * hq + (h0 + (con ? mem : 0)) * G + c2 % G) * D;
    for (int c = 0; c < NC; ++c) {
      u32x4 w = con ? *(const u32x4*)(qrow + q4 * DQ + 8 * c) : u32x4{0, 0, 0, 0};
      qf[0][c] = __builtin_bit_cast(bf16x8, w);
    }
  }
  f32x4 o[1][NB];
  float m[1] = {-INFINITY}, lsum[1] = {0.f};
  for (int nb = 0; nb < NB; ++nb) o[0][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sl2 = p.scale_log2;

  const int s0 = (klo / SK) * SK;
  const int nsteps = (khi - 1 - s0) / SK + 1;
  const int64_t blk = (int64_t)kPage * D;  // bytes per (page, head) block
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  const ctab_t ptab = (ctab_t)(KIND == 0 ? p.t.fpt + (int64_t)sid * p.t.max_pages
                                         : p.t.rpt + (int64_t)sid * (p.t.ring_slots / kPage));
  auto page_at = [&](int pos) {
    return ptab[__builtin_amdgcn_readfirstlane(idx::table_entry(KIND, pos, p.t.ring_slots))];
  };
  const uint8_t* kbase = (const uint8_t*)p.k_cache;
  const uint8_t* vbase = (const uint8_t*)p.v_cache;
  struct Ptrs {
    const uint8_t* k;  // this lane's K row (row group col/4, row col%4), its d quarter
    const uint8_t* v;  // row group q4, dim col
    int64_t sc;        // scales of row group q4
  };
  auto step_pages = [&](int kp0) {
    int32_t pg[NPG];
    for (int x = 0; x < NPG; ++x) {
      // a page with no key of [klo, khi): a page of the step that has one
      // (masked keys); a missing page (skipped alloc): page 0 of the pool
      const int32_t v = page_at(idx::decode_page_pos(kp0, x, klo, khi));
      pg[x] = v < 0 ? 0 : v;
    }
    // row group a = col >> 2 (K rows) or q4 (scores, V, scales): page a, or
    // with PAIR page a >> 1 of KV head h0 + (a & 1)
    const int ak = col >> 2;
    const int32_t pk = PAIR ? pg[ak >> 1] : pg[ak], pv = PAIR ? pg[q4 >> 1] : pg[q4];
    const int hk = PAIR ? h0 + (ak & 1) : kvh, hv = PAIR ? h0 + (q4 & 1) : kvh;
    return Ptrs{kbase + ((int64_t)pk * hkv + hk) * blk + (col & 3) * D + q4 * DQ,
                vbase + ((int64_t)pv * hkv + hv) * blk + col * kPage,
                ((int64_t)pv * hkv + hv) * kPage};
  };
  u32x4 kr[4][KV4], vr[NB], sc[8];  // sc: K scales 0-3, V scales 4-7
  auto load_k = [&](const Ptrs& pt) {
    for (int kt = 0; kt < 4; ++kt)
      for (int x = 0; x < KV4; ++x)
        kr[kt][x] = ld_kv<false>((const u32x4*)(pt.k + 4 * kt * D + 16 * x));
  };
  auto load_v = [&](const Ptrs& pt) {
    for (int nb = 0; nb < NB; ++nb)
      vr[nb] = ld_kv<false>((const u32x4*)(pt.v + 16 * nb * kPage));
    for (int x = 0; x < 4; ++x) {
      sc[x] = *(const u32x4*)(p.k_scale + pt.sc + 4 * x);
      sc[4 + x] = *(const u32x4*)(p.v_scale + pt.sc + 4 * x);
    }
  };
  Ptrs pt;
  if (wave < nsteps) {
    pt = step_pages(s0 + SK * wave);
    load_k(pt);
    load_v(pt);
  }
  for (int st = wave; st < nsteps; st += kDecWaves) {
    const int kp0 = s0 + SK * st;
    const bool more = st + kDecWaves < nsteps;
    Ptrs ptn = pt;
    if (more) ptn = step_pages(kp0 + SK * kDecWaves);
    // S^T of the four 16-key tiles
    f32x4 s4[4];
    for (int kt = 0; kt < 4; ++kt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < NC; ++c) {
        const uint32_t* w = (const uint32_t*)&kr[kt][0] + 2 * c;
        const u32x2 a = e4m3x4_to_bf16x4(w[0]), b = e4m3x4_to_bf16x4(w[1]);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, u32x4{a[0], a[1], b[0], b[1]}), qf[0][c], acc, 0, 0, 0);
      }
      s4[kt] = acc;
    }
    if (more) load_k(ptn);
    // lane value (kt, r) is key kp0 + 16*page + 4kt + r, in-page index 4kt + r,
    // page = q4 (PAIR: q4 >> 1)
    const int page16 = 16 * (PAIR ? q4 >> 1 : q4);
    unsigned valid = 0;
    for (int j = 0; j < 16; ++j) {
      const int kp = kp0 + page16 + j;
      valid |= (unsigned)(kp >= klo && kp < khi) << j;
    }
    float mx = -INFINITY;
    float sv[16];
    for (int j = 0; j < 16; ++j) {
      const int kp = kp0 + page16 + j;
      bool ok = lane_head && ((valid >> j) & 1u);
      if (QN > 1) ok = ok && kp <= cpos && (KIND == 0 || kp > cpos - W);
      const float ks = __uint_as_float(sc[j >> 2][j & 3]);
      const float x = ok ? s4[j >> 2][j & 3] * (ks * sl2) : -INFINITY;
      sv[j] = x;
      mx = fmaxf(mx, x);
    }
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m[0], mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m[0] - m_use);
    f16x8 pf[2];
    float ps = 0.f;
    for (int j = 0; j < 16; ++j) {
      const float e = fast_exp2(sv[j] - m_use);
      // V scale times 2^8 into the fp16 weight; masked keys' scales may be NaN
      const float vs = (valid >> j) & 1u ? __uint_as_float(sc[4 + (j >> 2)][j & 3]) * 256.f : 0.f;
      pf[j >> 3][j & 7] = (_Float16)(e * vs);
      ps += e;
    }
    lsum[0] = lsum[0] * alpha + ps;
    m[0] = m_new;
    u32x4 vmask = {~0u, ~0u, ~0u, ~0u};
    if (valid != 0xffffu)
      for (int j = 0; j < 16; ++j)
        if (!((valid >> j) & 1u)) vmask[j >> 2] &= ~(0xffu << (8 * (j & 3)));
    for (int nb = 0; nb < NB; ++nb) {
      const u32x4 w = vr[nb] & vmask;
      o[0][nb] *= alpha;
      for (int h = 0; h < 2; ++h) {
        const u32x2 a = e4m3x4_to_f16x4(w[2 * h]), b = e4m3x4_to_f16x4(w[2 * h + 1]);
        o[0][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(f16x8, u32x4{a[0], a[1], b[0], b[1]}), pf[h], o[0][nb], 0, 0, 0);
      }
    }
    if (more) load_v(ptn);
    pt = ptn;
  }
  for (int nb = 0; nb < NB; ++nb) o[0][nb] *= 0.00390625f;  // the weights carried 2^8
  merge_store<D, G, 1, CT, PAIR ? NCH : 0>(p, red_o, red_ml, o, m, lsum, kvh, split, row0, nr);
  if (p.vlen && split == 0 && kvh == 0 && (int)threadIdx.x < nr) {
    const int pos = L - n + threadIdx.x;
    p.vlen[row0 + threadIdx.x] = KIND == 0 ? pos + 1 : min(pos + 1, W);
  }
}


template <int D, int KIND, int G, int QN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4)))
decode_fp8_kernel(AttnParams p) {
  for_each_item<KIND, true>(p, [&](int unit, int kvh) {
    decode_fp8_unit<D, KIND, G, QN, false>(p, unit, kvh);
  });
}

// Full layers with an even KV head count and a split-K plan: items are
// (unit, KV head pair) from one queue, both heads in one workgroup.
template <int D, int G, int QN>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 4)))
decode_fp8_pair_kernel(AttnParams p) {
  __shared__ int s_k;
  const int pairs = p.hkv / 2;
  for (;;) {
    if (threadIdx.x == 0)
      s_k = __hip_atomic_fetch_add(p.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    const int k = s_k;
    __syncthreads();  // every wave has read s_k before it is written again
    const int units = min(p.queue[idx::kQueueCount], p.num_seqs * p.n_splits);
    int a, pair;
    if (!idx::queue_item(k, 0, units, pairs, false, &a, &pair)) return;
    decode_fp8_unit<D, 0, G, QN, true>(p, p.queue[idx::kQueueList + a], pair);
  }
}

// Log-sum-exp merge of the split partial states of one (query row, head).
// Block x = (sequence, row within the sequence), y = query head.  A split
// whose keys all lie past the row's position holds max = -inf and weight 0.
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(AttnParams p, int qn) {
  const int i = blockIdx.x / qn;
  const int r = blockIdx.x % qn;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  const int L = call_len(p, i, sid, n);
  if (n <= 0 || n > L || r >= n || row0 < 0 || row0 + n > p.total_q) return;
  const int len = idx::split_keys(L, p.n_splits, p.split_len);
  const int ns = (L + len - 1) / len;  // the splits that hold keys
  const int64_t hrow = (int64_t)(row0 + r) * p.hq + h;
  const float* ml = p.ws + (int64_t)p.total_q * p.hq * p.n_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * (hrow * p.n_splits + s)]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t slot = hrow * p.n_splits + s;
    const float sc = fast_exp2(ml[2 * slot] - M);
    num += sc * p.ws[slot * D + d];
    den += sc * ml[2 * slot + 1];
  }
  store_out(p, hrow * D + d, num / den);
}

// Pre-pass of a split-K call: lists the (sequence, split) units that hold
// keys (a sequence of L keys has ceil(L / len) of its n_splits pieces of
// len keys), longest pieces first, with their count, and zeroes the queue
// counters.  Longest first keeps the grid's tail short: the last items
// taken are the shortest.  Pieces are sorted by length in kLenBuckets
// classes (counting sort through LDS counters, so the order within a class
// varies; every item writes its own partial state, so results do not).
// Sequences the decode kernels skip (bad id, no rows, rows past the
// length) get no units.  One workgroup, 256 sequences at a time.
constexpr int kLenBuckets = 64;

__device__ __forceinline__ int units_of(const AttnParams& p, int i, int* bucket) {
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return 0;
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  const int L = call_len(p, i, sid, n);
  if (n <= 0 || n > L || row0 < 0 || row0 + n > p.total_q) return 0;
  const int len = idx::split_keys(L, p.n_splits, p.split_len);
  const int64_t b = (int64_t)(len - 1) * kLenBuckets / max(p.split_len, 64);
  *bucket = (int)min<int64_t>(b, kLenBuckets - 1);
  return (L + len - 1) / len;
}

__global__ void __launch_bounds__(256) decode_units_kernel(AttnParams p) {
  __shared__ int hist[kLenBuckets];
  const int tid = threadIdx.x;
  if (tid < kLenBuckets) hist[tid] = 0;
  if (tid < idx::kQueues) p.queue[idx::kQueueStride * tid] = 0;
  __syncthreads();
  for (int i = tid; i < p.num_seqs; i += 256) {
    int b = 0;
    const int ns = units_of(p, i, &b);
    if (ns > 0) atomicAdd(&hist[b], ns);
  }
  __syncthreads();
  if (tid == 0) {  // start of each class, longest class first
    int run = 0;
    for (int b = kLenBuckets - 1; b >= 0; --b) {
      const int c = hist[b];
      hist[b] = run;
      run += c;
    }
    p.queue[idx::kQueueCount] = run;
  }
  __syncthreads();
  for (int i = tid; i < p.num_seqs; i += 256) {
    int b = 0;
    const int ns = units_of(p, i, &b);
    if (ns <= 0) continue;
    const int at = atomicAdd(&hist[b], ns);
    for (int sp = 0; sp < ns; ++sp) p.queue[idx::kQueueList + at + sp] = i * p.n_splits + sp;
  }
}

// Workgroups of a queue grid: as many as the device holds at once (a
// multiple of the 8 queues), at most one per item.  The count per device
// and kernel is looked up once (`cache`, one slot per device).
constexpr int kMaxQueueDevices = 64;
template <typename K>
hipError_t queue_grid(K kernel, std::atomic<int> (&cache)[kMaxQueueDevices], int64_t items,
                      unsigned* grid) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  int slots = dev >= 0 && dev < kMaxQueueDevices ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (slots <= 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0);
    if (e != hipSuccess) return e;
    slots = std::max(cus, 1) * std::max(per_cu, 1);
    if (dev >= 0 && dev < kMaxQueueDevices) cache[dev].store(slots, std::memory_order_relaxed);
  }
  const int64_t q = idx::kQueues;
  int64_t g = (int64_t)slots / q * q;
  g = std::min<int64_t>(std::max<int64_t>(g, q), (items + q - 1) / q * q);
  *grid = (unsigned)g;
  return hipSuccess;
}

// FP8 pages with one column tile take the 64-key kernel; two tiles (8
// heads, more than two rows) keep the 32-key one, whose registers already
// hold two tiles' state.
template <int D, int KIND, int G, int QN, bool F8>
hipError_t launch_decode_one(const AttnParams& p, dim3 grid, hipStream_t s) {
  static std::atomic<int> slots[kMaxQueueDevices];  // per instantiation
  const int64_t items = (int64_t)p.num_seqs * p.n_splits * p.hkv;
  if constexpr (F8 && KIND == 0 && G * QN <= 8) {
    if (p.queue && p.hkv % 2 == 0) {
      static std::atomic<int> pair_slots[kMaxQueueDevices];
      hipError_t e = queue_grid(decode_fp8_pair_kernel<D, G, QN>, pair_slots, items / 2, &grid.x);
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((decode_fp8_pair_kernel<D, G, QN>), grid, dim3(256), 0, s, p);
      return hipGetLastError();
    }
  }
  if constexpr (F8 && G * QN <= 16) {
    if (p.queue) {
      hipError_t e = queue_grid(decode_fp8_kernel<D, KIND, G, QN>, slots, items, &grid.x);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_fp8_kernel<D, KIND, G, QN>), grid, dim3(256), 0, s, p);
  } else {
    if (p.queue) {
      hipError_t e = queue_grid(decode_kernel<D, KIND, G, QN, F8>, slots, items, &grid.x);
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_kernel<D, KIND, G, QN, F8>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

template <int D, int KIND, int QN, bool F8>
hipError_t launch_decode_q(const AttnParams& p, hipStream_t s) {
  const int units = p.num_seqs * p.n_splits;
  dim3 grid((unsigned)(F8 && p.hkv % 2 == 0 ? idx::fp8_blocks(p.hkv, units) : units * p.hkv), 1);
  if (p.queue) {
    hipLaunchKernelGGL(decode_units_kernel, dim3(1), dim3(256), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipError_t e = hipSuccess;
  switch (p.hq / p.hkv) {
    case 1: e = launch_decode_one<D, KIND, 1, QN, F8>(p, grid, s); break;
    case 2: e = launch_decode_one<D, KIND, 2, QN, F8>(p, grid, s); break;
    case 4: e = launch_decode_one<D, KIND, 4, QN, F8>(p, grid, s); break;
    default: e = launch_decode_one<D, KIND, 8, QN, F8>(p, grid, s); break;
  }
  if (e != hipSuccess || p.n_splits == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.num_seqs * QN, p.hq), dim3(D), 0, s, p,
                     QN);
  return hipGetLastError();
}

// Rows per sequence: 1 (plain decode), up to 2, up to 4; K/V pages in
// bf16/fp16 or FP8.
template <int D, int KIND, bool F8>
hipError_t launch_decode_f(const AttnParams& p, hipStream_t s) {
  if (p.max_q_len <= 1) return launch_decode_q<D, KIND, 1, F8>(p, s);
  if (p.max_q_len == 2) return launch_decode_q<D, KIND, 2, F8>(p, s);
  return launch_decode_q<D, KIND, 4, F8>(p, s);
}

template <int D, int KIND>
hipError_t launch_decode_g(const AttnParams& p, hipStream_t s) {
  return p.kv_fp8 ? launch_decode_f<D, KIND, true>(p, s) : launch_decode_f<D, KIND, false>(p, s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Split-K partial states of the allocation-free decode entry point.  Each
// GPU the library runs on holds its own copy of this array (allocated with
// the code object, kept until the process ends).  In host code its name
// stands for a host-side shadow, not a device address: kernels receive the
// address that hipGetSymbolAddress reports for the current device.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<float*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t decode_scratch(float** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  float* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    a = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!a) {
      void* ptr = nullptr;  // this device is current
      e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!ptr) return hipErrorInvalidSymbol;
      a = (float*)ptr;
      g_scratch_addr[dev].store(a, std::memory_order_release);
    }
  }
  *out = a;
  return hipSuccess;
}

hipError_t launch_decode(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_decode_g<128, 0>(p, s) : launch_decode_g<128, 1>(p, s);
  return p.kind == 0 ? launch_decode_g<64, 0>(p, s) : launch_decode_g<64, 1>(p, s);
}

}  // namespace hswa
