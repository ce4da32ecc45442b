// Chunked-prefill attention over the dual pool (Full and SWA layers).
//
// "MiMo-V2.5 Series Inference Full-Link Optimization" sec. 1.1: SWA layers
// attend to the last W keys, Full layers to the whole prefix; prefill runs
// in chunks.  The chunk's own K/V are already in the pool (appended before
// attention), so query position i reads keys [i-W+1, i] (SWA, from the
// ring) or [0, i] (Full, through the Full page table).
//
// Design (gfx950):
//  - Workgroup = 4 wavefronts for one (sequence, query block, KV head,
//    head group).  Wave w owns 32 query positions of one query head, so up
//    to four heads sharing a KV head (and, for G < 4, several 32-position
//    groups) share every K/V tile the workgroup stages.  Small workgroups
//    let three of them share a CU, so one's loads overlap another's math.
//    The grid runs KV heads fastest: workgroups resident at the same time
//    then cover all KV heads' slices of the pages (all HBM channels).
//    Query blocks run last first, so a Full chunk's longest prefixes start
//    first.
//  - Scores use the 32x32x16 bf16 MFMA as S^T[key][row] = K . Q^T, with the
//    Q^T fragments held in registers for the whole key loop and K read from
//    LDS.  The output uses the 32x32x16 fp16 MFMA as O^T[d][row] = V^T . P^T
//    on the fp16 V pages.  K rows are placed in LDS with bits 2 and 3 of the
//    in-page key index swapped, which makes the eight scores a lane holds per
//    page eight consecutive keys: each lane's probabilities are then exactly
//    the B operand of the PV product and its V fragment is 16 contiguous
//    bytes of the page, so P never goes through LDS and V is copied verbatim.
//  - K/V move global -> LDS by DMA (global_load_lds_dwordx4: each lane's 16
//    bytes land at the LDS base + 16 * lane), in 32-key steps (two 16-token
//    pages) through three LDS buffers: the loads of steps s+1 and s+2 are in
//    flight while step s computes, and no registers hold staged data.  Each
//    wave moves one (K or V, page) block of a step, so it needs one page id
//    per step.  The K rows' 16-byte chunks are XOR-swizzled by row so that
//    the QK operand reads are free of bank conflicts without padding.
//  - Keys outside the workgroup's range (their slots can hold evicted or
//    unwritten data) get -inf scores through the per-row masks, and their V
//    is zeroed in LDS before use so that 0 * V stays 0.
//  - Online softmax in fp32, log2 domain, with lazy rescaling: the two lanes
//    of a row exchange their maxima only when the running max must move.
//    The row sum adds the fp16 weights the PV product uses.
//  - Output fp32 (or fp16 on request), passed through LDS so that stores
//    write whole row pieces.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * 64;
constexpr int kBufs = 3;  // LDS buffers: the step computed plus two in flight
// Lazy softmax rescaling: the running max is only moved when a new score
// exceeds it by more than 2^kLazy, so unnormalised weights stay <= 2^kLazy
// (exact in fp16 with the same relative precision) and the O rescale runs
// rarely.  The final division by the row sum makes the result independent
// of where the max was taken.
constexpr float kLazy = 8.0f;

// 16 bytes per lane from sbase + voff (the lane's byte offset) into LDS at
// lds_base + 16 * lane.  The transfer counts on the vector-memory counter;
// the kernel waits for it explicitly (the compiler does not see it).  M0
// (the LDS address of the transfer) is written inside the statement; the
// compiler warns that it cannot preserve a clobbered M0, and nothing else
// in these kernels uses M0 (no LDS-size or relative-addressing forms on
// gfx950), so no value of its is live across the statement.
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds_base), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}
// 4 bytes per lane from sbase + voff into LDS at lds_base + 4 * lane (the
// lanes that execute it), as dma16.
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds_base), "v"(voff),
               "s"(sbase)
               : "memory", "m0");
}
// Wait until at most N vector-memory operations of the wave are in flight
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm_at_most() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int D, int KIND, int G, bool F8>
__global__ void __launch_bounds__(kPreThreads) __attribute__((amdgpu_waves_per_eu(3, 4)))
prefill_kernel(AttnParams p, int qblocks, int total_tiles) {
  constexpr int HPW = G < kPreWaves ? G : kPreWaves;  // heads per workgroup
  constexpr int HG = G / HPW;                         // workgroups per KV head
  constexpr int PG = kPreWaves / HPW;                 // 32-position groups
  constexpr int QB = 32 * PG;                         // query positions per workgroup
  constexpr int NC = D / 16;                          // k steps of the QK product
  constexpr int NM = D / 32;                          // 32-row d blocks of O^T
  constexpr int CPR = D / 8;                          // 16-byte chunks per K row
  constexpr int KBYTES = 32 * D * 2;                  // K bytes per 32-key step
  constexpr int VPAGE = 16 * D * 2;                   // V bytes per page block
  constexpr int SBYTES = 2 * KBYTES;                  // K + V bytes per step
  constexpr int NI = SBYTES / 1024;                   // 1 KB transfers per step
  constexpr int NIW = NI / kPreWaves;                 // per wave
  static_assert(NI % kPreWaves == 0 && NIW >= 1, "a step's transfers split over the waves");
  // FP8 pages: a wave moves its page block's e4m3 codes (half the bytes)
  // into the second half of the block's bf16 / fp16 region, plus the
  // block's 16 scales, then widens the codes in place before the barrier.
  // The scales of a step sit after its V region: K of pages 0, 1, then V.
  constexpr int NT8 = kPage * D / 1024;                 // 1 KB code transfers per block
  constexpr int NWAIT = F8 ? NT8 + 1 : NIW;             // a wave's transfers per step
  constexpr int SB = SBYTES + (F8 ? 4 * kPage * 4 : 0);  // bytes per step buffer
  constexpr int OROW = 64 * 4 + 16;  // LDS bytes per row of a 64-dim output piece (padded)
  constexpr int OBYTES = kPreWaves * 32 * OROW;
  constexpr int LBYTES = kBufs * SB > OBYTES ? kBufs * SB : OBYTES;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[LBYTES];

  const int t = blockIdx.x;
  if (t >= total_tiles) return;
  const int NY = p.hkv * HG;
  const int yh = t % NY;
  const int qb = qblocks - 1 - (t / NY) % qblocks;  // longest (Full) blocks first
  const int i = (t / NY) / qblocks;
  const int kvh = yh % p.hkv;
  const int hg = yh / p.hkv;

  const int row0 = p.cu_q[i];
  const int n = p.cu_q[i + 1] - row0;
  if (qb * QB >= n) return;  // whole workgroup idle: no barrier reached
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int L = call_len(p, i, sid, n);
  if (n > L) return;         // rows without allocated positions
  if (row0 < 0 || row0 + n > p.total_q) return;  // rows outside q / out
  const int W = p.window;
  const int P0 = L - n + qb * QB;        // position of the workgroup's row 0
  const int nrows = min(QB, n - qb * QB);
  const int wg_khi = P0 + nrows - 1;     // last key any row needs
  const int wg_klo = KIND == 0 ? 0 : max(0, P0 - W + 1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int hl = hg * HPW + wave % HPW;
  const int r0 = (wave / HPW) * 32;      // first workgroup row of this wave
  const int head = kvh * G + hl;
  const int qr = lane & 31;              // query row within the wave (N index)
  const int h2 = lane >> 5;              // k half of the MFMA operands
  const int my_row = r0 + qr;
  const bool row_ok = my_row < nrows;
  const int my_pos = P0 + my_row;
  const bool wave_on = r0 < nrows;
  const int w_pos_lo = P0 + r0;
  const int w_pos_hi = P0 + min(r0 + 32, nrows) - 1;
  const int w_klo = KIND == 0 ? 0 : max(0, w_pos_lo - W + 1);
  const int hq = p.hq;
  const int hkv = p.hkv;
  const int64_t grow = (int64_t)row0 + qb * QB + (row_ok ? my_row : nrows - 1);


  bf16x8 qf[NC];  // Q^T fragments, loaded after step 0's transfers are issued
  f32x16 o[NM];
  for (int mb = 0; mb < NM; ++mb)
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m = -INFINITY;   // running max of scaled scores (log2 domain)
  float lsum = 0.f;      // this lane's share of the row sum
  const float sl2 = p.scale_log2;

  const int kstart = (wg_klo / 32) * 32;
  const int nsteps = (wg_khi - kstart) / 32 + 1;
  const uint32_t lds0 = (uint32_t)(size_t)((__attribute__((address_space(3))) uint8_t*)(lds));

  // Transfers of one step.  Transfers 0 .. NI/2-1 fill the K region: LDS row
  // r (of 32) holds key swap23(r % 16) of page r / 16, its chunk j at
  // position j ^ (r % CPR).  Transfers NI/2 .. NI-1 copy the two V page
  // blocks verbatim.  Wave w issues transfers w*NIW .. +NIW, which is the K
  // (w < 2) or V (w >= 2) block of the step's page w & 1: one page id and
  // one scalar base per wave and step, plus a per-lane offset fixed for the
  // kernel.
  static_assert(kPreWaves == 4 && NI == 4 * NIW, "one (tensor, page) block per wave");
  uint32_t voff[NIW];
  for (int ii = 0; ii < NIW; ++ii) {
    const int inst = wave * NIW + ii;
    if (inst < NI / 2) {
      const int slot = inst * 64 + lane;
      const int row = slot / CPR;
      const int rr = row & 15;
      const int kr = ((rr >> 2) & 1) * 8 + ((rr >> 3) & 1) * 4 + (rr & 3);
      const int j = (slot % CPR) ^ (row & (CPR - 1));
      voff[ii] = (kr * D + j * 8) * 2;
    } else {
      voff[ii] = ((inst - NI / 2) * 1024 + lane * 16) % VPAGE;
    }
  }
  // This wave's page: the table row of the sequence and the page index of
  // the next step to issue (for SWA a ring page, advanced with wrap-around).
  const int half = wave & 1;
  const uint16_t* tens = (wave >= 2 ? p.v_cache : p.k_cache) + (int64_t)kvh * kPage * D;
  const uint32_t pbytes = (uint32_t)hkv * kPage * D * 2;  // bytes per page (< 2^32)
  const int npr = p.t.ring_slots / kPage;             // ring pages of a sequence (SWA)
  const int32_t* prow = KIND == 0 ? p.t.fpt + (int64_t)sid * p.t.max_pages
                                  : p.t.rpt + (int64_t)sid * npr;
  int ipg = idx::prefill_first_entry(KIND, kstart, half, p.t.ring_slots);
  // a page past the range reads page 0 (present in every pool); its keys are
  // masked like any other key outside the range
  auto issue = [&](int kp0, int buf) {
    const int32_t pg = kp0 + kPage * half <= wg_khi ? scalar_load_i32(prow, ipg) : 0;
    ipg = idx::prefill_next_entry(KIND, ipg, npr);
    if constexpr (F8) {
      const int64_t blk = (int64_t)(uint32_t)pg * hkv + kvh;  // (page, KV head) block
      const uint8_t* codes = (const uint8_t*)(wave >= 2 ? p.v_cache : p.k_cache) + blk * kPage * D;
      const uint32_t region = lds0 + buf * SB + (wave >= 2 ? KBYTES + half * VPAGE : half * VPAGE);
      for (int x = 0; x < NT8; ++x) dma16(x * 1024 + 16 * lane, codes, region + kPage * D + x * 1024);
      const float* sc = (wave >= 2 ? p.v_scale : p.k_scale) + blk * kPage;
      if (lane < kPage)
        dma4(4 * lane, sc, lds0 + buf * SB + SBYTES + (wave >= 2 ? 128 : 0) + 64 * half);
      return;
    }
    const uint16_t* src =
        (const uint16_t*)((const uint8_t*)tens + (uint64_t)(uint32_t)pg * pbytes);
    const uint32_t base = lds0 + buf * SB + wave * NIW * 1024;
    for (int ii = 0; ii < NIW; ++ii) dma16(voff[ii], src, base + ii * 1024);
  };

  // FP8: this wave's block of buffer bc, codes -> the bf16 / fp16 layout the
  // bf16 pages give, in place (all of a lane's reads come before its
  // writes; the wave's LDS operations run in order, and only this wave
  // touches the block).  K: exact bf16 codes, key kr in LDS row
  // swap23(kr) with swizzled chunks; its scale multiplies the scores.  V:
  // code * scale rounded to fp16, dim-major.
  auto widen = [&](int bc) {
    uint8_t* reg = lds + bc * SB + (wave >= 2 ? KBYTES + half * VPAGE : half * VPAGE);
    const uint8_t* raw = reg + kPage * D;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed here rather than held across the loop
    if (wave < 2) {
      constexpr int CL = D / 4;  // codes per lane: a quarter of key row ln / 4
      const int kr = ln >> 2, q = ln & 3;
      u32x4 c[CL / 16];
      for (int t = 0; t < CL / 16; ++t) c[t] = *(const u32x4*)(raw + kr * D + q * CL + 16 * t);
      asm volatile("" ::: "memory");  // no write moves above the reads
      const int rr = ((kr >> 2) & 1) * 8 + ((kr >> 3) & 1) * 4 + (kr & 3);  // its LDS row
      for (int t = 0; t < CL / 16; ++t)
        for (int hh = 0; hh < 2; ++hh) {
          const u32x2 a = e4m3x4_to_bf16x4(c[t][2 * hh]), b = e4m3x4_to_bf16x4(c[t][2 * hh + 1]);
          const int j = (q * CL + 16 * t + 8 * hh) / 8;  // 16-byte chunk of the bf16 row
          *(u32x4*)(reg + rr * (CPR * 16) + (j ^ (rr & (CPR - 1))) * 16) =
              u32x4{a[0], a[1], b[0], b[1]};
        }
    } else {
      constexpr int DL = D / 64;  // dims per lane, 16 codes (keys) each
      u32x4 c[DL];
      for (int t = 0; t < DL; ++t) c[t] = *(const u32x4*)(raw + (DL * ln + t) * kPage);
      const float* vsc = (const float*)(lds + bc * SB + SBYTES + 128 + 64 * half);
      f32x4 sc[4];
      for (int x = 0; x < 4; ++x) sc[x] = *(const f32x4*)(vsc + 4 * x);
      asm volatile("" ::: "memory");
      for (int t = 0; t < DL; ++t) {
        uint32_t w[8];  // fp16 pairs of keys 2m, 2m + 1
        for (int x = 0; x < 4; ++x) {
          // keys 4x .. 4x + 3 to fp32 (exact), two codes per conversion; the
          // upper pair is shifted down rather than picked by the word select,
          // which the compiler drops when the pair is widened like this
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(c[t][x], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(c[t][x] >> 16, false);
          w[2 * x] = pack_f16x2(lo[0] * sc[x][0], lo[1] * sc[x][1]);
          w[2 * x + 1] = pack_f16x2(hi[0] * sc[x][2], hi[1] * sc[x][3]);
        }
        uint8_t* row = reg + (DL * ln + t) * (kPage * 2);
        *(u32x4*)row = u32x4{w[0], w[1], w[2], w[3]};
        *(u32x4*)(row + 16) = u32x4{w[4], w[5], w[6], w[7]};
      }
    }
  };

  // One 32-key step of scores, softmax and PV from LDS buffer `buf`.
  auto compute = [&](int buf, int kp0) {
    // does this wave have any unmasked key in the step?
    if (!(wave_on && kp0 <= w_pos_hi && kp0 + 31 >= w_klo)) return;
    const uint8_t* kb = lds + buf * SB;
    f32x16 sacc;
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    for (int c = 0; c < NC; ++c) {
      const int pos = (2 * c + h2) ^ (qr & (CPR - 1));
      bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(kb + qr * (CPR * 16) + pos * 16));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc, 0, 0, 0);
    }
    if constexpr (F8) {
      // each score times its key's K scale (value r = 4j + i is in-page key
      // 8*h2 + 4(j%2) + i of page j/2); a masked key's NaN scale is masked
      // with its score below
      const float* ksc = (const float*)(kb + SBYTES);
      for (int j = 0; j < 4; ++j) {
        const f32x4 s = *(const f32x4*)(ksc + kPage * (j >> 1) + 8 * h2 + 4 * (j & 1));
        for (int i = 0; i < 4; ++i) sacc[4 * j + i] *= s[i];
      }
    }
    // every key of the step valid for every row of the wave?
    const bool interior = kp0 + 31 <= w_pos_lo && (KIND == 0 || kp0 > w_pos_hi - W);
    float mx = -INFINITY;
    if (interior) {
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    } else {
      // lane value r = 4j + i is key kp0 + 16(j/2) + 8*h2 + 4(j%2) + i
      const int rel = kp0 + 8 * h2 - my_pos;  // key - query of value 0
      for (int r = 0; r < 16; ++r) {
        const int dk = rel + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
        const bool ok = dk <= 0 && (KIND == 0 || dk > -W);
        sacc[r] = ok ? sacc[r] : -INFINITY;
        mx = fmaxf(mx, sacc[r]);
      }
    }
    // the running max moves only when some score exceeds it by 2^kLazy;
    // then the two lanes of a row agree on the new one through one exchange
    if (__builtin_amdgcn_ballot_w64(mx * sl2 > m + kLazy) != 0) {  // wave-uniform
      const float m_new = fmaxf(m, fmaxf(mx, xor_lane(mx, 32)) * sl2);
      const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m - m_new);
      for (int mb = 0; mb < NM; ++mb) o[mb] *= alpha;
      lsum *= alpha;
      m = m_new;
    }
    const float mo = m == -INFINITY ? 0.f : m;
    f16x8 pf0, pf1;
    for (int r = 0; r < 8; ++r) {
      pf0[r] = (_Float16)fast_exp2(__builtin_fmaf(sacc[r], sl2, -mo));
      pf1[r] = (_Float16)fast_exp2(__builtin_fmaf(sacc[r + 8], sl2, -mo));
    }
    // row sum of the fp16 weights the PV product uses, two per dot2
    const f16x2 one2 = {(_Float16)1.f, (_Float16)1.f};
    for (int r = 0; r < 8; r += 2) {
      lsum = __builtin_amdgcn_fdot2(f16x2{pf0[r], pf0[r + 1]}, one2, lsum, false);
      lsum = __builtin_amdgcn_fdot2(f16x2{pf1[r], pf1[r + 1]}, one2, lsum, false);
    }
    // V fragment: dim 32mb + qr, keys 8*h2 .. +8 of each page
    const uint8_t* v0 = kb + KBYTES + qr * 32 + h2 * 16;
    for (int mb = 0; mb < NM; ++mb) {
      f16x8 va = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + mb * 1024));
      f16x8 vb = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + VPAGE + mb * 1024));
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf0, o[mb], 0, 0, 0);
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb, pf1, o[mb], 0, 0, 0);
    }
  };

  // Step 0's transfers, then the Q^T fragments (lane holds Q[row qr][16c +
  // 8*h2 .. +8]), so that Q's latency overlaps step 0's; the full wait tells
  // the compiler that Q has arrived (it does not see the transfers), then
  // step 1's transfers.  Transfers stop at the last step; each wait counts
  // what was issued after the step it waits for (memory operations complete
  // in issue order).
  issue(kstart, 0);
  {
    const uint16_t* qrow = p.q + (grow * hq + head) * D;
    for (int c = 0; c < NC; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * c + 8 * h2));
  }
  wait_vm_all();
  if (nsteps > 1) issue(kstart + 32, 1);
  // One step s over LDS buffer bc (its transfers landed), refilling buffer
  // bn (step s-1's) with step s+2.  The loop below runs three steps per
  // iteration so that the buffer indices, hence the LDS offsets, are
  // compile-time constants.
  auto step = [&](int s, int bc, int bn) __attribute__((always_inline)) {
    const int kp0 = kstart + 32 * s;
    // this wave's part of step s (and, at s = 0, Q) has landed
    if (s + 1 < nsteps)
      wait_vm_at_most<NWAIT>();
    else
      wait_vm_at_most<0>();
    if constexpr (F8) widen(bc);
    __syncthreads();         // every part has; step s-1's buffer is free
    if (!(kp0 >= wg_klo && kp0 + 31 <= wg_khi)) {
      // keys of the step outside the workgroup's range: zero their V
      uint8_t* vz = lds + bc * SB + KBYTES;
      for (int e = tid; e < 2 * D; e += kPreThreads) {  // (page block, dim) rows
        const int key0 = kp0 + 16 * (e / D);
        u32x4* rowp = (u32x4*)(vz + (e / D) * VPAGE + (e % D) * 32);
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 w = rowp[hf];
          for (int x = 0; x < 8; ++x) {
            const int k = key0 + 8 * hf + x;
            if (k < wg_klo || k > wg_khi) w[x >> 1] &= (x & 1) ? 0x0000ffffu : 0xffff0000u;
          }
          rowp[hf] = w;
        }
      }
      __syncthreads();
    }
    if (s + 2 < nsteps) issue(kp0 + 64, bn);  // into step s-1's buffer
    compute(bc, kp0);
  };
  static_assert(kBufs == 3, "three steps per iteration");
  for (int s = 0; s < nsteps; s += 3) {
    step(s, 0, 2);
    if (s + 1 < nsteps) step(s + 1, 1, 0);
    if (s + 2 < nsteps) step(s + 2, 2, 1);
  }
  wait_vm_at_most<0>();  // no transfer may land after the workgroup leaves

  // Output.  A lane holds 4 consecutive dims per (mb, j) of its row, so
  // storing straight from registers would write 32 bytes to each of 32 rows
  // per instruction.  Instead each wave passes its 32 x D tile through LDS
  // (the K/V buffers are free once every wave has left the loop), 64 dims at
  // a time, and stores whole rows: every store instruction writes 4
  // contiguous 256-byte row pieces.
  lsum += xor_lane(lsum, 32);
  const float inv = 1.0f / lsum;
  __syncthreads();
  uint8_t* ot = lds + wave * 32 * OROW;
  for (int ps = 0; ps < NM / 2; ++ps) {
    for (int mh = 0; mh < 2; ++mh) {
      const int mb = 2 * ps + mh;
      for (int j = 0; j < 4; ++j) {
        f32x4 v = {o[mb][4 * j] * inv, o[mb][4 * j + 1] * inv, o[mb][4 * j + 2] * inv,
                   o[mb][4 * j + 3] * inv};
        *(f32x4*)(ot + qr * OROW + (32 * mh + 8 * j + 4 * h2) * 4) = v;
      }
    }
    // fp32: lane l stores 16 bytes of row 4k + l / 16 (dims 64 ps + 4 (l % 16)
    // ..); fp16: 16 bytes of row 8k + l / 8 (dims 64 ps + 8 (l % 8) ..).  The
    // output is not read again here, so the stores are non-temporal.
    if (!p.out_f16) {
      for (int k = 0; k < 8; ++k) {
        const int r = 4 * k + (lane >> 4);
        const f32x4 v = *(const f32x4*)(ot + r * OROW + (lane & 15) * 16);
        if (r0 + r < nrows) {
          const int64_t gr = (int64_t)row0 + qb * QB + r0 + r;
          __builtin_nontemporal_store(v, (f32x4*)((float*)p.out + (gr * hq + head) * D +
                                                  64 * ps + 4 * (lane & 15)));
        }
      }
    } else {
      for (int k = 0; k < 4; ++k) {
        const int r = 8 * k + (lane >> 3);
        const f32x4 a = *(const f32x4*)(ot + r * OROW + (lane & 7) * 32);
        const f32x4 b = *(const f32x4*)(ot + r * OROW + (lane & 7) * 32 + 16);
        const u32x4 h = {pack_f16x2(a[0], a[1]), pack_f16x2(a[2], a[3]), pack_f16x2(b[0], b[1]),
                         pack_f16x2(b[2], b[3])};
        if (r0 + r < nrows) {
          const int64_t gr = (int64_t)row0 + qb * QB + r0 + r;
          __builtin_nontemporal_store(h, (u32x4*)((_Float16*)p.out + (gr * hq + head) * D +
                                                  64 * ps + 8 * (lane & 7)));
        }
      }
    }
  }
  if (row_ok && p.vlen && kvh == 0 && hl == 0 && h2 == 0)
    p.vlen[grow] = KIND == 0 ? my_pos + 1 : min(my_pos + 1, W);

  // The grid holds qblocks query blocks per sequence, sized by the caller's
  // max_q_len.  Rows past them (a hint below the true row count) are not
  // computed; the last block's workgroups fill them with NaN (vlen -1) so
  // the violation shows instead of leaving stale output.
  if (qb == qblocks - 1 && n > qblocks * QB) {
    const int64_t rlo = (int64_t)row0 + qblocks * QB, rhi = (int64_t)row0 + n;
    for (int64_t e = tid; e < (rhi - rlo) * HPW * D; e += kPreThreads) {
      const int64_t r = rlo + e / (HPW * D);
      const int hh = kvh * G + hg * HPW + (int)((e / D) % HPW);
      const int64_t idx = (r * hq + hh) * D + e % D;
      if (p.out_f16)
        ((_Float16*)p.out)[idx] = (_Float16)__builtin_nanf("");
      else
        ((float*)p.out)[idx] = __builtin_nanf("");
      if (p.vlen && kvh == 0 && hg == 0 && e % (HPW * D) == 0) p.vlen[r] = -1;
    }
  }
}

template <int D, int KIND, int G, bool F8>
hipError_t launch_prefill_g(const AttnParams& p, hipStream_t s) {
  constexpr int HPW = G < kPreWaves ? G : kPreWaves;
  constexpr int QB = 32 * (kPreWaves / HPW);
  const int qblocks = (p.max_q_len + QB - 1) / QB;
  const int64_t tiles = (int64_t)p.num_seqs * qblocks * p.hkv * (G / HPW);
  if (tiles > INT32_MAX - 8) return hipErrorInvalidValue;
  const int grid = (int)tiles;
  hipLaunchKernelGGL((prefill_kernel<D, KIND, G, F8>), dim3(grid), dim3(kPreThreads), 0, s, p,
                     qblocks, (int)tiles);
  return hipGetLastError();
}

template <int D, int KIND, bool F8>
hipError_t launch_prefill_f(const AttnParams& p, hipStream_t s) {
  switch (p.hq / p.hkv) {
    case 1: return launch_prefill_g<D, KIND, 1, F8>(p, s);
    case 2: return launch_prefill_g<D, KIND, 2, F8>(p, s);
    case 4: return launch_prefill_g<D, KIND, 4, F8>(p, s);
    default: return launch_prefill_g<D, KIND, 8, F8>(p, s);
  }
}

template <int D, int KIND>
hipError_t launch_prefill_k(const AttnParams& p, hipStream_t s) {
  return p.kv_fp8 ? launch_prefill_f<D, KIND, true>(p, s) : launch_prefill_f<D, KIND, false>(p, s);
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0 || p.total_q <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_prefill_k<128, 0>(p, s) : launch_prefill_k<128, 1>(p, s);
  return p.kind == 0 ? launch_prefill_k<64, 0>(p, s) : launch_prefill_k<64, 1>(p, s);
}

}  // namespace hswa
