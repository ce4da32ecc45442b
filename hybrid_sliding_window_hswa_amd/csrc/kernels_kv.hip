// Pool table updates and the KV append (scatter of new K/V into pages).
//
// Page layout of a layer's pool (Full pool and SWA ring alike), per
// "Following the Bottleneck: Optimizing MiniMax M3 on AMD Instinct MI355X"
// sec. 3 (16-token pages behind a page table):
//   K: [page][Hkv][16][d]   bf16, token-major: a key row is d contiguous
//   V: [page][Hkv][d][16]   fp16, dim-major: the 16 tokens of one dim are
//                           contiguous, the operand order of the PV matrix
//                           product (keys are its reduction dim).  V is
//                           stored in fp16 because that product runs on the
//                           fp16 MFMA; bf16 -> fp16 is exact for
//                           2^-14 <= |v| <= 65280 (every bf16 value
//                           there), |v| >= 65536 becomes +-inf.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

// ---------------------------------------------------------------------------
// Applies one pool operation's records to the device tables.  Block x is a
// record (one sequence); blocks along y and threads stride over its listed
// pages (thread j handles logical page pg_lo + j: its fpt entry and its 16
// map entries).  Records and page lists sit in pinned host memory, read over
// the bus.  Record x's Full pages start at pages[x * stride] and the ring
// pages of the same logical pages at pages[(n_recs + x) * stride] (a logical
// page's 16 positions share one ring page, as the ring holds whole pages), so
// a thread issues the reads of its page ids together with the read of the
// record and the block pays one bus round trip.
__global__ void __launch_bounds__(256) pool_apply_kernel(PoolDev d, const PoolRec* recs,
                                                         const int32_t* pages, int32_t stride,
                                                         int32_t* done, int32_t seq) {
  const int j0 = blockIdx.y * blockDim.x + threadIdx.x;
  const int jstep = gridDim.y * blockDim.x;
  const int32_t* pg = pages + (int64_t)blockIdx.x * stride;
  const int32_t* rg = pages + (int64_t)(gridDim.x + blockIdx.x) * stride;
  const int32_t first = j0 < stride ? pg[j0] : 0;  // before the record arrives
  const int32_t rfirst = j0 < stride ? rg[j0] : 0;
  const PoolRec r = recs[blockIdx.x];
  if (j0 == 0 && r.new_len >= 0) d.seq_len[r.seq] = r.new_len;
  int32_t* row = d.fpt + (int64_t)r.seq * d.max_pages;
  if (r.fpt_clear)  // cleared entries need no page id
    for (int lp = r.fpt_lo + j0; lp < r.fpt_hi; lp += jstep) row[lp] = -1;
  for (int j = j0; j < r.npg; j += jstep) {
    const int32_t page = j == j0 ? first : pg[j];
    const int32_t rpage = j == j0 ? rfirst : rg[j];
    const int lp = r.pg_lo + j;
    if (!r.fpt_clear && lp >= r.fpt_lo && lp < r.fpt_hi) row[lp] = page;
    int32_t* m = d.map + (int64_t)page * kPage;
    for (int x = 0; x < kPage; ++x) {
      const int pos = lp * kPage + x;
      if (pos >= r.clr_lo && pos < r.clr_hi) m[x] = -1;
      if (pos >= r.set_lo && pos < r.set_hi) m[x] = rpage * kPage + x;
    }
  }
  // every read of the staging buffer by this block is complete
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_store(done + blockIdx.y * gridDim.x + blockIdx.x, seq, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_SYSTEM);
}

int pool_apply_blocks(int n_recs, int32_t stride) {
  int64_t y = ((int64_t)stride + 255) / 256;  // one listed page per thread
  if (y < 1) y = 1;
  if (y > 64) y = 64;
  return n_recs * (int)y;
}

hipError_t launch_pool_apply(const PoolDev& d, const PoolRec* recs, int n_recs,
                             const int32_t* pages, int32_t stride, int32_t* done,
                             int32_t seq, hipStream_t s) {
  if (n_recs <= 0) return hipSuccess;
  const int y = pool_apply_blocks(n_recs, stride) / n_recs;
  hipLaunchKernelGGL(pool_apply_kernel, dim3(n_recs, (unsigned)y), dim3(256), 0, s, d, recs,
                     pages, stride, done, seq);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// KV append.  One workgroup per (sequence, 16-position page tile, KV head).
// The rows of sequence i are its last n_i positions [L - n_i, L).  Full
// page tiles are written with 16-byte stores (K rows straight, V through
// an LDS transpose); tiles shared with positions outside this call are
// written element by element so those positions are untouched.
template <int D, int KIND>
__global__ void __launch_bounds__(256) append_kernel(AttnParams p, int tiles_per_seq) {
  __shared__ uint16_t vt[kPage][D + 8];
  // KV heads run fastest: the workgroups of one tile, resident together,
  // read whole token rows [Hkv][d] of the input between them
  const int h = blockIdx.x % p.hkv;
  const int i = (blockIdx.x / p.hkv) / tiles_per_seq;
  const int t = (blockIdx.x / p.hkv) % tiles_per_seq;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;  // invalid id: nothing to write
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  const int L = call_len(p, i, sid, n);
  const int p0 = L - n;
  const int tile_pos = idx::tile_pos(p0, t);
  if (n <= 0 || n > L || tile_pos >= L || row0 < 0 || row0 + n > p.total_q) return;
  const int lo = max(tile_pos, p0);
  const int hi = min(tile_pos + kPage, L);
  const bool whole = (lo == tile_pos) && (hi == tile_pos + kPage);
  const int32_t page = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile_pos, p.t.max_pages,
                                     p.t.ring_slots);
  if (page < 0) return;  // position without a page: the caller skipped alloc
  const int hkv = p.hkv;
  uint16_t* kdst = p.k_cache + ((int64_t)page * hkv + h) * kPage * D;
  uint16_t* vdst = p.v_cache + ((int64_t)page * hkv + h) * D * kPage;
  constexpr int kChunks = D / 8;  // 16-byte chunks per row
  const int tid = threadIdx.x;
  // K rows and the V tile into LDS
  if (tid < kPage * kChunks) {
    const int tok = tid / kChunks;
    const int c = tid % kChunks;
    const int pos = tile_pos + tok;
    if (pos >= lo && pos < hi) {
      const int64_t row = row0 + (pos - p0);
      const u32x4 kv = *(const u32x4*)(p.k_new + (row * hkv + h) * D + c * 8);
      *(u32x4*)(kdst + tok * D + c * 8) = kv;
      const u32x4 vv = *(const u32x4*)(p.v_new + (row * hkv + h) * D + c * 8);
      *(u32x4*)(&vt[tok][c * 8]) = vv;
    }
  }
  __syncthreads();
  // V^T: thread (e, half) owns 8 tokens of dim e
  if (tid < D * 2) {
    const int e = tid >> 1;
    const int half = tid & 1;
    uint16_t* dst = vdst + e * kPage + half * 8;
    if (whole) {
      u32x4 w;
      for (int j = 0; j < 4; ++j)
        w[j] = pack_f16x2(bf16_lo(vt[half * 8 + 2 * j][e]), bf16_lo(vt[half * 8 + 2 * j + 1][e]));
      *(u32x4*)dst = w;
    } else {
      for (int j = 0; j < 8; ++j) {
        const int pos = tile_pos + half * 8 + j;
        if (pos >= lo && pos < hi)
          dst[j] = __builtin_bit_cast(uint16_t, (_Float16)bf16_lo(vt[half * 8 + j][e]));
      }
    }
  }
}

// Quantizing KV append for FP8 pages ("Baidu Day0" hybrid-attention
// article, Layered quantization, point 2: FP8 KV per token, head and
// 128-element tile).  Same grid as append_kernel.  Each (token, head) row of
// d <= 128 elements is one tile: amax over the row, scale = amax / 448,
// codes of x * (448 / amax) in e4m3.  Pages: K [page][Hkv][16][d] codes
// (token-major), V [page][Hkv][d][16] codes (dim-major, through an LDS
// transpose), scales [page][Hkv][16] fp32.
template <int D, int KIND>
__global__ void __launch_bounds__(256) append_fp8_kernel(AttnParams p, int tiles_per_seq) {
  constexpr int CPR = D / 8;  // threads per row (8 elements each)
  __shared__ __attribute__((aligned(16))) uint8_t vt[kPage][D + 16];
  const int h = blockIdx.x % p.hkv;  // KV heads fastest, as in append_kernel
  const int i = (blockIdx.x / p.hkv) / tiles_per_seq;
  const int t = (blockIdx.x / p.hkv) % tiles_per_seq;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  const int L = call_len(p, i, sid, n);
  const int p0 = L - n;
  const int tile_pos = idx::tile_pos(p0, t);
  if (n <= 0 || n > L || tile_pos >= L || row0 < 0 || row0 + n > p.total_q) return;
  const int lo = max(tile_pos, p0);
  const int hi = min(tile_pos + kPage, L);
  const int32_t page = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile_pos, p.t.max_pages,
                                     p.t.ring_slots);
  if (page < 0) return;
  const int hkv = p.hkv;
  const int64_t blk = (int64_t)page * hkv + h;
  uint8_t* kdst = (uint8_t*)p.k_cache + blk * kPage * D;
  uint8_t* vdst = (uint8_t*)p.v_cache + blk * D * kPage;
  const int tid = threadIdx.x;
  const int tok = tid / CPR;  // rows are groups of CPR consecutive lanes
  const int c = tid % CPR;
  const int pos = tile_pos + tok;
  const bool act = tid < kPage * CPR && pos >= lo && pos < hi;
  const int64_t row = row0 + (pos - p0);
  // quantizes this thread's 8 elements of a row (src[0..7] as fp32) with the
  // row's amax, reduced over the row's CPR lanes
  auto quant = [&](const uint16_t* src, float* scale_out) -> u32x2 {
    float x[8];
    float amax = 0.f;
    if (act) {
      const u32x4 w = *(const u32x4*)src;
      for (int j = 0; j < 4; ++j) {
        x[2 * j] = bf16_lo(w[j]);
        x[2 * j + 1] = bf16_hi(w[j]);
      }
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
    }
    for (int m = 1; m < CPR; m <<= 1) amax = fmaxf(amax, xor_lane(amax, m));
    const float inv = amax > 0.f ? __fdiv_rn(448.0f, amax) : 0.f;
    *scale_out = __fdiv_rn(amax, 448.0f);
    u32x2 out = {0u, 0u};
    if (act)
      for (int j = 0; j < 8; ++j) out[j >> 2] |= e4m3_encode(x[j] * inv) << (8 * (j & 3));
    return out;
  };
  float ks, vs;
  const u32x2 kq = quant(p.k_new + (row * hkv + h) * D + c * 8, &ks);
  const u32x2 vq = quant(p.v_new + (row * hkv + h) * D + c * 8, &vs);
  if (act) {
    *(u32x2*)(kdst + tok * D + c * 8) = kq;
    *(u32x2*)(&vt[tok][c * 8]) = vq;
    if (c == 0) {
      p.k_scale[blk * kPage + tok] = ks;
      p.v_scale[blk * kPage + tok] = vs;
    }
  }
  __syncthreads();
  // V^T: thread (e, half) owns 8 tokens of dim e
  if (tid < D * 2) {
    const int e = tid >> 1;
    const int half = tid & 1;
    uint8_t* dst = vdst + e * kPage + half * 8;
    const int pos0 = tile_pos + half * 8;
    if (pos0 >= lo && pos0 + 8 <= hi) {
      u32x2 w = {0u, 0u};
      for (int j = 0; j < 8; ++j) w[j >> 2] |= (uint32_t)vt[half * 8 + j][e] << (8 * (j & 3));
      *(u32x2*)dst = w;
    } else {
      for (int j = 0; j < 8; ++j)
        if (pos0 + j >= lo && pos0 + j < hi) dst[j] = vt[half * 8 + j][e];
    }
  }
}

hipError_t launch_append(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0) return hipSuccess;
  const int tiles = idx::tiles_for(p.max_q_len);
  const int64_t blocks = (int64_t)p.num_seqs * tiles * p.hkv;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  if (p.kv_fp8) {
    if (p.d == 128) {
      if (p.kind == 0)
        hipLaunchKernelGGL((append_fp8_kernel<128, 0>), grid, dim3(256), 0, s, p, tiles);
      else
        hipLaunchKernelGGL((append_fp8_kernel<128, 1>), grid, dim3(256), 0, s, p, tiles);
    } else {
      if (p.kind == 0)
        hipLaunchKernelGGL((append_fp8_kernel<64, 0>), grid, dim3(256), 0, s, p, tiles);
      else
        hipLaunchKernelGGL((append_fp8_kernel<64, 1>), grid, dim3(256), 0, s, p, tiles);
    }
    return hipGetLastError();
  }
  if (p.d == 128) {
    if (p.kind == 0)
      hipLaunchKernelGGL((append_kernel<128, 0>), grid, dim3(256), 0, s, p, tiles);
    else
      hipLaunchKernelGGL((append_kernel<128, 1>), grid, dim3(256), 0, s, p, tiles);
  } else {
    if (p.kind == 0)
      hipLaunchKernelGGL((append_kernel<64, 0>), grid, dim3(256), 0, s, p, tiles);
    else
      hipLaunchKernelGGL((append_kernel<64, 1>), grid, dim3(256), 0, s, p, tiles);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// K/V copy between two sequences of one pool, for prefix reuse ("MiMo-V2.5
// Series Inference Full-Link Optimization" sec. 2.1, "SWA-aware prefix cache
// tree", point 3).  One workgroup per (pair, 16-position page tile) copies
// every KV head of the tile.  A position sits at the same in-page offset in
// both sequences (pos % 16 for Full pages; (pos mod C) % 16 = pos % 16 in a
// ring of C slots), so the copy moves K rows and V columns between the two
// pages at that offset: whole 16-byte pieces when the tile is whole,
// element by element otherwise.
template <int D, int KIND>
__global__ void __launch_bounds__(256) copy_kernel(CopyParams p, int tiles_per_pair) {
  constexpr int CPR = D / 8;  // 16-byte chunks per K row
  const int i = blockIdx.x / tiles_per_pair;
  const int t = blockIdx.x % tiles_per_pair;
  const int a = p.src_ids[i], b = p.dst_ids[i];
  if (a < 0 || a >= p.t.max_seqs || b < 0 || b >= p.t.max_seqs || a == b) return;
  const int La = p.t.seq_len[a], Lb = p.t.seq_len[b];
  int p0 = p.first_pos[i];
  int p1 = min(p.end_pos[i], min(La, Lb));     // stored in both sequences
  if (KIND != 0)                               // still held by both rings
    p0 = max(p0, max(idx::ring_oldest(La, p.t.ring_slots), idx::ring_oldest(Lb, p.t.ring_slots)));
  p0 = max(p0, 0);
  if (p1 - p0 > p.max_tok) p1 = p0 + p.max_tok;  // the grid covers max_tok positions
  const int tile_pos = idx::tile_pos(p0, t);
  if (p0 >= p1 || tile_pos >= p1) return;
  const int lo = max(tile_pos, p0), hi = min(tile_pos + kPage, p1);
  const int32_t pa = page_of<KIND>(p.t.fpt, p.t.rpt, a, tile_pos, p.t.max_pages, p.t.ring_slots);
  const int32_t pb = page_of<KIND>(p.t.fpt, p.t.rpt, b, tile_pos, p.t.max_pages, p.t.ring_slots);
  if (pa < 0 || pb < 0) return;  // a position without a page: the caller skipped alloc
  const int hkv = p.hkv;
  const int tid = threadIdx.x;
  const bool whole = lo == tile_pos && hi == tile_pos + kPage;
  // K rows: (head, token, chunk), chunks fastest
  for (int e = tid; e < hkv * kPage * CPR; e += blockDim.x) {
    const int h = e / (kPage * CPR);
    const int tok = (e / CPR) % kPage;
    const int c = e % CPR;
    if (tile_pos + tok < lo || tile_pos + tok >= hi) continue;
    const int64_t off = (int64_t)h * kPage * D + tok * D + c * 8;
    *(u32x4*)(p.k_cache + (int64_t)pb * hkv * kPage * D + off) =
        *(const u32x4*)(p.k_cache + (int64_t)pa * hkv * kPage * D + off);
  }
  // V columns: (head, dim, 8-token half)
  for (int e = tid; e < hkv * D * 2; e += blockDim.x) {
    const int h = e / (2 * D);
    const int dim = (e / 2) % D;
    const int half = e % 2;
    const int64_t off = (int64_t)h * D * kPage + dim * kPage + half * 8;
    const uint16_t* src = p.v_cache + (int64_t)pa * hkv * D * kPage + off;
    uint16_t* dst = p.v_cache + (int64_t)pb * hkv * D * kPage + off;
    if (whole) {
      *(u32x4*)dst = *(const u32x4*)src;
    } else {
      for (int j = 0; j < 8; ++j) {
        const int pos = tile_pos + half * 8 + j;
        if (pos >= lo && pos < hi) dst[j] = src[j];
      }
    }
  }
}

// The same copy over FP8 pages: K rows of D code bytes, V columns of 16
// code bytes (one per token), and each copied token's K and V scale.
template <int D, int KIND>
__global__ void __launch_bounds__(256) copy8_kernel(CopyParams p, int tiles_per_pair) {
  constexpr int CPR = D / 16;  // 16-byte chunks per K row
  const int i = blockIdx.x / tiles_per_pair;
  const int t = blockIdx.x % tiles_per_pair;
  const int a = p.src_ids[i], b = p.dst_ids[i];
  if (a < 0 || a >= p.t.max_seqs || b < 0 || b >= p.t.max_seqs || a == b) return;
  const int La = p.t.seq_len[a], Lb = p.t.seq_len[b];
  int p0 = p.first_pos[i];
  int p1 = min(p.end_pos[i], min(La, Lb));
  if (KIND != 0)
    p0 = max(p0, max(idx::ring_oldest(La, p.t.ring_slots), idx::ring_oldest(Lb, p.t.ring_slots)));
  p0 = max(p0, 0);
  if (p1 - p0 > p.max_tok) p1 = p0 + p.max_tok;
  const int tile_pos = idx::tile_pos(p0, t);
  if (p0 >= p1 || tile_pos >= p1) return;
  const int lo = max(tile_pos, p0), hi = min(tile_pos + kPage, p1);
  const int32_t pa = page_of<KIND>(p.t.fpt, p.t.rpt, a, tile_pos, p.t.max_pages, p.t.ring_slots);
  const int32_t pb = page_of<KIND>(p.t.fpt, p.t.rpt, b, tile_pos, p.t.max_pages, p.t.ring_slots);
  if (pa < 0 || pb < 0) return;
  const int hkv = p.hkv;
  const int tid = threadIdx.x;
  const bool whole = lo == tile_pos && hi == tile_pos + kPage;
  const int64_t bytes = (int64_t)hkv * kPage * D;  // code bytes of one page, K or V
  const uint8_t* ksrc = (const uint8_t*)p.k_cache + pa * bytes;
  uint8_t* kdst = (uint8_t*)p.k_cache + pb * bytes;
  const uint8_t* vsrc = (const uint8_t*)p.v_cache + pa * bytes;
  uint8_t* vdst = (uint8_t*)p.v_cache + pb * bytes;
  // K rows: (head, token, chunk)
  for (int e = tid; e < hkv * kPage * CPR; e += blockDim.x) {
    const int tok = (e / CPR) % kPage;
    if (tile_pos + tok < lo || tile_pos + tok >= hi) continue;
    *(u32x4*)(kdst + (int64_t)e * 16) = *(const u32x4*)(ksrc + (int64_t)e * 16);
  }
  // V columns: (head, dim), 16 tokens each
  for (int e = tid; e < hkv * D; e += blockDim.x) {
    if (whole) {
      *(u32x4*)(vdst + (int64_t)e * 16) = *(const u32x4*)(vsrc + (int64_t)e * 16);
    } else {
      for (int j = lo - tile_pos; j < hi - tile_pos; ++j)
        vdst[(int64_t)e * 16 + j] = vsrc[(int64_t)e * 16 + j];
    }
  }
  // scales: (head, token)
  for (int e = tid; e < hkv * kPage; e += blockDim.x) {
    const int tok = e % kPage;
    if (tile_pos + tok < lo || tile_pos + tok >= hi) continue;
    p.k_scale[((int64_t)pb * hkv) * kPage + e] = p.k_scale[((int64_t)pa * hkv) * kPage + e];
    p.v_scale[((int64_t)pb * hkv) * kPage + e] = p.v_scale[((int64_t)pa * hkv) * kPage + e];
  }
}

hipError_t launch_copy(const CopyParams& p, hipStream_t s) {
  if (p.num_seqs <= 0 || p.max_tok <= 0) return hipSuccess;
  const int tiles = idx::tiles_for(p.max_tok);
  const int64_t blocks = (int64_t)p.num_seqs * tiles;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  dim3 grid((unsigned)blocks);
  if (p.kv_fp8) {
    if (p.d == 128) {
      if (p.kind == 0)
        hipLaunchKernelGGL((copy8_kernel<128, 0>), grid, dim3(256), 0, s, p, tiles);
      else
        hipLaunchKernelGGL((copy8_kernel<128, 1>), grid, dim3(256), 0, s, p, tiles);
    } else {
      if (p.kind == 0)
        hipLaunchKernelGGL((copy8_kernel<64, 0>), grid, dim3(256), 0, s, p, tiles);
      else
        hipLaunchKernelGGL((copy8_kernel<64, 1>), grid, dim3(256), 0, s, p, tiles);
    }
    return hipGetLastError();
  }
  if (p.d == 128) {
    if (p.kind == 0)
      hipLaunchKernelGGL((copy_kernel<128, 0>), grid, dim3(256), 0, s, p, tiles);
    else
      hipLaunchKernelGGL((copy_kernel<128, 1>), grid, dim3(256), 0, s, p, tiles);
  } else {
    if (p.kind == 0)
      hipLaunchKernelGGL((copy_kernel<64, 0>), grid, dim3(256), 0, s, p, tiles);
    else
      hipLaunchKernelGGL((copy_kernel<64, 1>), grid, dim3(256), 0, s, p, tiles);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Window-masked transfer ("MiMo-V2.5 Series Inference Full-Link
// Optimization" sec. 2.1 "KVCache Dual Pool", Data Transfer: tiers exchange
// only the valid SWA window).  One workgroup per (sequence, 16-position page
// tile) moves every KV head of the tile.  The packed buffer holds a token's
// heads contiguously, so each wave moves contiguous runs of it (PCIe-friendly
// when the buffer is host memory).  K rows copy straight; V goes through LDS
// between the dim-major fp16 page and token-major rows.  Positions of a tile
// outside the transferred range are never written (a ring page holds other
// positions too).
constexpr int kXferHeads = 8;  // KV heads staged in LDS at a time

template <int D, int KIND, bool TO_HOST>
__global__ void __launch_bounds__(256) xfer_kernel(XferParams p, int tiles_per_seq) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint16_t vt[kPage][kXferHeads][D + 8];
  const int i = blockIdx.x / tiles_per_seq;
  const int t = blockIdx.x % tiles_per_seq;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int tok0 = p.cu_tok[i];
  const int n = p.cu_tok[i + 1] - tok0;
  const int L = p.t.seq_len[sid];
  const int p0 = p.first_pos ? p.first_pos[i] : L - n;  // positions [p0, p0 + n)
  if (n <= 0 || p0 < 0 || p0 > L - n) return;  // only stored positions move
  if (tok0 < 0 || tok0 + n > p.total_tok) return;  // tokens outside the buffers
  const int tile_pos = idx::tile_pos(p0, t);
  if (tile_pos >= p0 + n) return;
  // A SWA ring of C slots holds at most positions [L - C, L): an older
  // position's slot belongs to a newer one, so it is neither read (offload)
  // nor written (restore, which would overwrite live K/V).
  const int lo = max(max(tile_pos, p0), KIND == 0 ? 0 : idx::ring_oldest(L, p.t.ring_slots));
  const int hi = min(tile_pos + kPage, p0 + n);
  if (lo >= hi) return;
  const int32_t page = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile_pos, p.t.max_pages,
                                     p.t.ring_slots);
  if (page < 0) return;  // position without a page: the caller skipped alloc
  const int hkv = p.hkv;
  const int tid = threadIdx.x;
  // buffer row of position pos, head h
  auto brow = [&](int pos, int h) { return ((int64_t)(tok0 + pos - p0) * hkv + h) * D; };
  auto kpage = [&](int h) { return p.k_cache + ((int64_t)page * hkv + h) * kPage * D; };
  auto vpage = [&](int h) { return p.v_cache + ((int64_t)page * hkv + h) * D * kPage; };

  // K: (token, head, chunk) with the chunk fastest
  for (int idx = tid; idx < kPage * hkv * CPR; idx += blockDim.x) {
    const int tok = idx / (hkv * CPR);
    const int h = (idx / CPR) % hkv;
    const int c = idx % CPR;
    const int pos = tile_pos + tok;
    if (pos < lo || pos >= hi) continue;
    u32x4* pg = (u32x4*)(kpage(h) + tok * D + c * 8);
    u32x4* bf = (u32x4*)(p.buf_k + brow(pos, h) + c * 8);
    if (TO_HOST)
      *bf = *pg;
    else
      *pg = *bf;
  }
  // V, kXferHeads heads at a time through LDS
  for (int h0 = 0; h0 < hkv; h0 += kXferHeads) {
    const int nh = min(kXferHeads, hkv - h0);
    if (TO_HOST) {
      // page (head, dim e, 8-token half) -> LDS [token][head][dim]
      for (int idx = tid; idx < nh * D * 2; idx += blockDim.x) {
        const int hh = idx / (2 * D);
        const int e = (idx / 2) % D;
        const int half = idx % 2;
        const u32x4 w = *(const u32x4*)(vpage(h0 + hh) + e * kPage + half * 8);
        for (int j = 0; j < 8; ++j)
          vt[half * 8 + j][hh][e] = (uint16_t)(w[j >> 1] >> (16 * (j & 1)));
      }
      __syncthreads();
      for (int idx = tid; idx < kPage * nh * CPR; idx += blockDim.x) {
        const int tok = idx / (nh * CPR);
        const int hh = (idx / CPR) % nh;
        const int c = idx % CPR;
        const int pos = tile_pos + tok;
        if (pos >= lo && pos < hi)
          *(u32x4*)(p.buf_v + brow(pos, h0 + hh) + c * 8) = *(const u32x4*)(&vt[tok][hh][c * 8]);
      }
    } else {
      for (int idx = tid; idx < kPage * nh * CPR; idx += blockDim.x) {
        const int tok = idx / (nh * CPR);
        const int hh = (idx / CPR) % nh;
        const int c = idx % CPR;
        const int pos = tile_pos + tok;
        if (pos >= lo && pos < hi)
          *(u32x4*)(&vt[tok][hh][c * 8]) = *(const u32x4*)(p.buf_v + brow(pos, h0 + hh) + c * 8);
      }
      __syncthreads();
      for (int idx = tid; idx < nh * D * 2; idx += blockDim.x) {
        const int hh = idx / (2 * D);
        const int e = (idx / 2) % D;
        const int half = idx % 2;
        uint16_t* dst = vpage(h0 + hh) + e * kPage + half * 8;
        const int pos0 = tile_pos + half * 8;
        if (pos0 >= lo && pos0 + 8 <= hi) {
          u32x4 w;
          for (int j = 0; j < 4; ++j)
            w[j] = (uint32_t)vt[half * 8 + 2 * j][hh][e] |
                   ((uint32_t)vt[half * 8 + 2 * j + 1][hh][e] << 16);
          *(u32x4*)dst = w;
        } else {
          for (int j = 0; j < 8; ++j)
            if (pos0 + j >= lo && pos0 + j < hi) dst[j] = vt[half * 8 + j][hh][e];
        }
      }
    }
    __syncthreads();  // LDS free for the next head group
  }
}

// The same transfer over FP8 pages.  The buffers hold code bytes
// [token][Hkv][d] for K and for V and the fp32 scales [token][Hkv] of each;
// V goes through LDS between the page's 16-byte token columns and the
// buffer's rows.
template <int D, int KIND, bool TO_HOST>
__global__ void __launch_bounds__(256) xfer8_kernel(XferParams p, int tiles_per_seq) {
  constexpr int CPR = D / 16;  // 16-byte chunks per row
  __shared__ __attribute__((aligned(16))) uint8_t vt[kPage][kXferHeads][D + 16];
  const int i = blockIdx.x / tiles_per_seq;
  const int t = blockIdx.x % tiles_per_seq;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int tok0 = p.cu_tok[i];
  const int n = p.cu_tok[i + 1] - tok0;
  const int L = p.t.seq_len[sid];
  const int p0 = p.first_pos ? p.first_pos[i] : L - n;
  if (n <= 0 || p0 < 0 || p0 > L - n) return;
  if (tok0 < 0 || tok0 + n > p.total_tok) return;
  const int tile_pos = idx::tile_pos(p0, t);
  if (tile_pos >= p0 + n) return;
  const int lo = max(max(tile_pos, p0), KIND == 0 ? 0 : idx::ring_oldest(L, p.t.ring_slots));
  const int hi = min(tile_pos + kPage, p0 + n);
  if (lo >= hi) return;
  const int32_t page = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile_pos, p.t.max_pages,
                                     p.t.ring_slots);
  if (page < 0) return;
  const int hkv = p.hkv;
  const int tid = threadIdx.x;
  const int64_t bytes = (int64_t)hkv * kPage * D;  // code bytes of one page, K or V
  uint8_t* kpg = (uint8_t*)p.k_cache + page * bytes;
  uint8_t* vpg = (uint8_t*)p.v_cache + page * bytes;
  uint8_t* bk = (uint8_t*)p.buf_k;
  uint8_t* bv = (uint8_t*)p.buf_v;
  // buffer token index of the tile's first position
  const int64_t b0 = (int64_t)tok0 + tile_pos - p0;

  // K rows: (token, head, chunk)
  for (int e = tid; e < kPage * hkv * CPR; e += blockDim.x) {
    const int tok = e / (hkv * CPR);
    const int h = (e / CPR) % hkv;
    const int c = e % CPR;
    const int pos = tile_pos + tok;
    if (pos < lo || pos >= hi) continue;
    u32x4* pg = (u32x4*)(kpg + ((int64_t)h * kPage + tok) * D + c * 16);
    u32x4* bf = (u32x4*)(bk + ((b0 + tok) * hkv + h) * D + c * 16);
    if (TO_HOST)
      *bf = *pg;
    else
      *pg = *bf;
  }
  // scales: (token, head)
  for (int e = tid; e < kPage * hkv; e += blockDim.x) {
    const int tok = e / hkv;
    const int h = e % hkv;
    const int pos = tile_pos + tok;
    if (pos < lo || pos >= hi) continue;
    const int64_t ps = ((int64_t)page * hkv + h) * kPage + tok;
    const int64_t bs = (b0 + tok) * hkv + h;
    if (TO_HOST) {
      p.buf_k_scale[bs] = p.k_scale[ps];
      p.buf_v_scale[bs] = p.v_scale[ps];
    } else {
      p.k_scale[ps] = p.buf_k_scale[bs];
      p.v_scale[ps] = p.buf_v_scale[bs];
    }
  }
  // V, kXferHeads heads at a time through LDS
  const bool whole = lo == tile_pos && hi == tile_pos + kPage;
  for (int h0 = 0; h0 < hkv; h0 += kXferHeads) {
    const int nh = min(kXferHeads, hkv - h0);
    if (TO_HOST) {
      // page column (head, dim e) of 16 tokens -> LDS [token][head][dim]
      for (int e = tid; e < nh * D; e += blockDim.x) {
        const int hh = e / D, dim = e % D;
        const u32x4 w = *(const u32x4*)(vpg + ((int64_t)(h0 + hh) * D + dim) * kPage);
        for (int j = 0; j < kPage; ++j)
          vt[j][hh][dim] = (uint8_t)(w[j >> 2] >> (8 * (j & 3)));
      }
      __syncthreads();
      for (int e = tid; e < kPage * nh * CPR; e += blockDim.x) {
        const int tok = e / (nh * CPR);
        const int hh = (e / CPR) % nh;
        const int c = e % CPR;
        const int pos = tile_pos + tok;
        if (pos >= lo && pos < hi)
          *(u32x4*)(bv + ((b0 + tok) * hkv + h0 + hh) * D + c * 16) =
              *(const u32x4*)(&vt[tok][hh][c * 16]);
      }
    } else {
      for (int e = tid; e < kPage * nh * CPR; e += blockDim.x) {
        const int tok = e / (nh * CPR);
        const int hh = (e / CPR) % nh;
        const int c = e % CPR;
        const int pos = tile_pos + tok;
        if (pos >= lo && pos < hi)
          *(u32x4*)(&vt[tok][hh][c * 16]) =
              *(const u32x4*)(bv + ((b0 + tok) * hkv + h0 + hh) * D + c * 16);
      }
      __syncthreads();
      for (int e = tid; e < nh * D; e += blockDim.x) {
        const int hh = e / D, dim = e % D;
        uint8_t* dst = vpg + ((int64_t)(h0 + hh) * D + dim) * kPage;
        if (whole) {
          u32x4 w = {0u, 0u, 0u, 0u};
          for (int j = 0; j < kPage; ++j) w[j >> 2] |= (uint32_t)vt[j][hh][dim] << (8 * (j & 3));
          *(u32x4*)dst = w;
        } else {
          for (int j = lo - tile_pos; j < hi - tile_pos; ++j) dst[j] = vt[j][hh][dim];
        }
      }
    }
    __syncthreads();  // LDS free for the next head group
  }
}

hipError_t launch_xfer(const XferParams& p, bool to_host, hipStream_t s) {
  if (p.num_seqs <= 0) return hipSuccess;
  const int tiles = idx::tiles_for(p.max_tok);
  dim3 grid((unsigned)(p.num_seqs * tiles));
#define HSWA_XFER(D_, K_)                                                                   \
  if (p.kv_fp8 && to_host)                                                                  \
    hipLaunchKernelGGL((xfer8_kernel<D_, K_, true>), grid, dim3(256), 0, s, p, tiles);      \
  else if (p.kv_fp8)                                                                        \
    hipLaunchKernelGGL((xfer8_kernel<D_, K_, false>), grid, dim3(256), 0, s, p, tiles);     \
  else if (to_host)                                                                         \
    hipLaunchKernelGGL((xfer_kernel<D_, K_, true>), grid, dim3(256), 0, s, p, tiles);       \
  else                                                                                      \
    hipLaunchKernelGGL((xfer_kernel<D_, K_, false>), grid, dim3(256), 0, s, p, tiles);
  if (p.d == 128) {
    if (p.kind == 0) {
      HSWA_XFER(128, 0)
    } else {
      HSWA_XFER(128, 1)
    }
  } else {
    if (p.kind == 0) {
      HSWA_XFER(64, 0)
    } else {
      HSWA_XFER(64, 1)
    }
  }
#undef HSWA_XFER
  return hipGetLastError();
}

}  // namespace hswa
