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
//    head group); the grid runs head groups fastest (HBM channel spread).  Wave w owns 32 query positions of one query head, so up
//    to four heads sharing a KV head (and, for G < 4, several 32-position
//    groups) share every K/V tile the workgroup stages.  Small workgroups
//    let three of them share a CU, so one's loads overlap another's math.
//  - Scores use the 32x32x16 bf16 MFMA as S^T[key][row] = K . Q^T, with the
//    Q^T fragments held in registers for the whole key loop and K read from
//    LDS.  The output uses the 32x32x16 fp16 MFMA as O^T[d][row] = V^T . P^T
//    on the fp16 V pages.  K rows are staged with bits 2 and 3 of the
//    in-page key index swapped, which makes the eight scores a lane holds per
//    page eight consecutive keys: each lane's probabilities are then exactly
//    the B operand of the PV product and its V fragment is 16 contiguous
//    bytes of the page, so P never goes through LDS and V is copied verbatim.
//  - K/V move through LDS in 32-key steps (two 16-token pages), double
//    buffered: global loads of step s+1 are in flight while step s computes.
//  - Keys outside the workgroup's range are staged as zeros (their slots can
//    hold evicted or unwritten data); per-row masks select -inf scores.
//  - Online softmax in fp32, log2 domain, with lazy rescaling: the two lanes
//    of a row exchange their maxima only when the running max must move;
//    output fp32.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kPreWaves = 4;
constexpr int kPreThreads = kPreWaves * 64;
// Lazy softmax rescaling: the running max is only moved when a new score
// exceeds it by more than 2^kLazy, so unnormalised weights stay <= 2^kLazy
// (exact in fp16 with the same relative precision) and the O rescale runs
// rarely.  The final division by the row sum makes the result independent
// of where the max was taken.
constexpr float kLazy = 8.0f;

template <int D, int KIND, int G>
__global__ void __launch_bounds__(kPreThreads) __attribute__((amdgpu_waves_per_eu(3, 4)))
prefill_kernel(AttnParams p, int qblocks,
                                                              int total_tiles) {
  constexpr int HPW = G < kPreWaves ? G : kPreWaves;  // heads per workgroup
  constexpr int HG = G / HPW;                         // workgroups per KV head
  constexpr int PG = kPreWaves / HPW;                 // 32-position groups
  constexpr int QB = 32 * PG;                         // query positions per workgroup
  constexpr int KROW = D + 8;                         // LDS K row in bf16 (16-byte pad)
  constexpr int NC = D / 16;                          // k steps of the QK product
  constexpr int NM = D / 32;                          // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t kl[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vl[2][2 * D * 16];

  // Tile order: head group fastest.  Workgroups running at the same time
  // then cover every KV head's slice of the K/V pages and every head's slice
  // of the Q/O rows, which spreads their traffic over all HBM channels (one
  // head's slices alone concentrate on a few).  Neighbouring query blocks of
  // one head, whose K/V windows overlap, still run close together in time.
  const int t = blockIdx.x;
  if (t >= total_tiles) return;
  const int NY = p.hkv * HG;
  const int yh = t % NY;
  const int qb = (t / NY) % qblocks;
  const int i = (t / NY) / qblocks;
  const int kvh = yh / HG;
  const int hg = yh % HG;

  const int row0 = p.cu_q[i];
  const int n = p.cu_q[i + 1] - row0;
  if (qb * QB >= n) return;  // whole workgroup idle: no barrier reached
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int L = p.t.seq_len[sid];
  if (n > L) return;         // rows without allocated positions
  const int W = p.window;
  const int P0 = L - n + qb * QB;        // position of the workgroup's row 0
  const int nrows = min(QB, n - qb * QB);
  const int wg_khi = P0 + nrows - 1;     // last key any row needs
  const int wg_klo = KIND == 0 ? 0 : max(0, P0 - W + 1);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
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

  // Q^T fragments: lane holds Q[row qr][16c + 8*h2 .. +8]
  bf16x8 qf[NC];
  {
    const uint16_t* qrow = p.q + (grow * hq + head) * D;
    for (int c = 0; c < NC; ++c)
      qf[c] = __builtin_bit_cast(bf16x8, *(const u32x4*)(qrow + 16 * c + 8 * h2));
  }

  f32x16 o[NM];
  for (int mb = 0; mb < NM; ++mb)
    for (int r = 0; r < 16; ++r) o[mb][r] = 0.f;
  float m = -INFINITY;   // running max of scaled scores (log2 domain)
  float lsum = 0.f;      // this lane's share of the row sum
  const float sl2 = p.scale_log2;

  const int kstart = (wg_klo / 32) * 32;
  const int nsteps = (wg_khi - kstart) / 32 + 1;
  const int64_t head_stride = (int64_t)kPage * D;

  // Staging.  One 16-token page block of one head is 16*D*2 contiguous
  // bytes for K (token-major) and for V (dim-major), so thread t copies the
  // 16-byte chunk(s) at t*8 (+ j*kPreThreads*8) of each of the step's two
  // page blocks.  For K the chunk is row (t*8)/D, columns (t*8)%D; for V it
  // is dim (t*8)/16, keys 8*(t&1) .. +8.  Loads are issued one step ahead
  // and unconditionally (a tile past the range reads page 0, which every
  // pool has); masking and the LDS write happen after the step's math, when
  // the data has arrived anyway.  Page ids come by scalar loads, so waiting
  // for them never waits for the K/V loads in flight.
  constexpr int EPB = kPage * D;                    // elements per page block
  constexpr int NCH = EPB / 8;                      // 16-byte chunks per block
  constexpr int CPT = (NCH + kPreThreads - 1) / kPreThreads;
  u32x4 kreg[2][CPT], vreg[2][CPT];
  auto stage_load = [&](int kp0) {
    // both page ids first: their wait then covers no K/V load
    int32_t pgs[2];
    for (int t2 = 0; t2 < 2; ++t2) {
      const int tile = kp0 + 16 * t2;
      pgs[t2] = tile <= wg_khi ? page_of_uniform<KIND>(p.t.fpt, p.t.rpt, sid, tile,
                                                       p.t.max_pages, p.t.ring_slots)
                               : 0;
    }
    for (int t2 = 0; t2 < 2; ++t2) {
      const uint16_t* kb = p.k_cache + ((int64_t)pgs[t2] * hkv + kvh) * head_stride;
      const uint16_t* vb = p.v_cache + ((int64_t)pgs[t2] * hkv + kvh) * head_stride;
      for (int j = 0; j < CPT; ++j) {
        const int e = (tid + j * kPreThreads) * 8;  // element offset in the block
        if (NCH % kPreThreads != 0 && e >= EPB) break;
        kreg[t2][j] = *(const u32x4*)(kb + e);
        vreg[t2][j] = *(const u32x4*)(vb + e);
      }
    }
  };
  auto stage_store = [&](int buf, int kp0) {
    // wave-uniform: whether every key of the step's two page blocks lies
    // inside the workgroup's key range
    const bool inner = kp0 >= wg_klo && kp0 + 31 <= wg_khi;
    for (int t2 = 0; t2 < 2; ++t2) {
      const int tile = kp0 + 16 * t2;
      for (int j = 0; j < CPT; ++j) {
        const int e = (tid + j * kPreThreads) * 8;
        if (NCH % kPreThreads != 0 && e >= EPB) break;
        u32x4 kv = kreg[t2][j], vv = vreg[t2][j];
        if (!inner) {
          // keys outside [wg_klo, wg_khi] may hold evicted or unwritten data
          const int kk = tile + e / D;
          if (kk < wg_klo || kk > wg_khi) kv = u32x4{0, 0, 0, 0};
          const int k8 = tile + (e % 16);
          for (int x = 0; x < 8; ++x) {
            const int kp = k8 + x;
            if (kp < wg_klo || kp > wg_khi) vv[x >> 1] &= (x & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
        // key row kr of the page goes to LDS row swap23(kr) of the page half
        const int kr = e / D;
        const int rho = ((kr >> 2) & 1) * 8 + ((kr >> 3) & 1) * 4 + (kr & 3);
        *(u32x4*)(&kl[buf][(16 * t2 + rho) * KROW + e % D]) = kv;
        *(u32x4*)(&vl[buf][t2 * EPB + e]) = vv;
      }
    }
  };

  // One 32-key step of scores, softmax and PV from LDS buffer `buf`.
  auto compute = [&](int buf, int kp0) {
    // does this wave have any unmasked key in the step?
    if (!(wave_on && kp0 <= w_pos_hi && kp0 + 31 >= w_klo)) return;
    f32x16 sacc;
    for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
    const uint16_t* krow = &kl[buf][qr * KROW + 8 * h2];
    for (int c = 0; c < NC; ++c) {
      bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + 16 * c));
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc, 0, 0, 0);
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
    float ps = 0.f;
    f16x8 pf0, pf1;
    for (int r = 0; r < 8; ++r) {
      const float e0 = fast_exp2(__builtin_fmaf(sacc[r], sl2, -mo));
      const float e1 = fast_exp2(__builtin_fmaf(sacc[r + 8], sl2, -mo));
      ps += e0 + e1;
      pf0[r] = (_Float16)e0;
      pf1[r] = (_Float16)e1;
    }
    lsum += ps;
    // V fragment: dim 32mb + qr, keys 8*h2 .. +8 of each page
    const uint16_t* v0 = &vl[buf][qr * 16 + 8 * h2];
    for (int mb = 0; mb < NM; ++mb) {
      f16x8 va = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + 512 * mb));
      f16x8 vb = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + EPB + 512 * mb));
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf0, o[mb], 0, 0, 0);
      o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb, pf1, o[mb], 0, 0, 0);
    }
  };

  stage_load(kstart);
  stage_store(0, kstart);
  wait_vm_all();  // Q fragments have arrived
  __syncthreads();
  // every iteration loads and stores (the last one a masked tile past the
  // range), so the loads never merge with other values in registers
  for (int s = 0; s < nsteps; ++s) {
    const int kp0 = kstart + 32 * s;
    stage_load(kp0 + 32);
    compute(s & 1, kp0);
    stage_store((s & 1) ^ 1, kp0 + 32);
    __syncthreads();
  }

  lsum += xor_lane(lsum, 32);
  if (row_ok) {
    const float inv = 1.0f / lsum;
    float* orow = p.out + (grow * hq + head) * D;
    for (int mb = 0; mb < NM; ++mb)
      for (int j = 0; j < 4; ++j) {
        f32x4 v = {o[mb][4 * j] * inv, o[mb][4 * j + 1] * inv, o[mb][4 * j + 2] * inv,
                   o[mb][4 * j + 3] * inv};
        *(f32x4*)(orow + 32 * mb + 8 * j + 4 * h2) = v;
      }
    if (p.vlen && kvh == 0 && hl == 0 && h2 == 0)
      p.vlen[grow] = KIND == 0 ? my_pos + 1 : min(my_pos + 1, W);
  }
}

template <int D, int KIND, int G>
hipError_t launch_prefill_g(const AttnParams& p, hipStream_t s) {
  constexpr int HPW = G < kPreWaves ? G : kPreWaves;
  constexpr int QB = 32 * (kPreWaves / HPW);
  const int qblocks = (p.max_q_len + QB - 1) / QB;
  const int64_t tiles = (int64_t)p.num_seqs * qblocks * p.hkv * (G / HPW);
  if (tiles > INT32_MAX - 8) return hipErrorInvalidValue;
  const int grid = (int)tiles;
  hipLaunchKernelGGL((prefill_kernel<D, KIND, G>), dim3(grid), dim3(kPreThreads), 0, s, p,
                     qblocks, (int)tiles);
  return hipGetLastError();
}

template <int D, int KIND>
hipError_t launch_prefill_k(const AttnParams& p, hipStream_t s) {
  switch (p.hq / p.hkv) {
    case 1: return launch_prefill_g<D, KIND, 1>(p, s);
    case 2: return launch_prefill_g<D, KIND, 2>(p, s);
    case 4: return launch_prefill_g<D, KIND, 4>(p, s);
    default: return launch_prefill_g<D, KIND, 8>(p, s);
  }
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0 || p.total_q <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_prefill_k<128, 0>(p, s) : launch_prefill_k<128, 1>(p, s);
  return p.kind == 0 ? launch_prefill_k<64, 0>(p, s) : launch_prefill_k<64, 1>(p, s);
}

}  // namespace hswa
