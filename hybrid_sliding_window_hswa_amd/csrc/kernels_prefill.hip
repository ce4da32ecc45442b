// Chunked-prefill attention over the dual pool (Full and SWA layers).
//
// "MiMo-V2.5 Series Inference Full-Link Optimization" sec. 1.1: SWA layers
// attend to the last W keys, Full layers to the whole prefix; prefill runs
// in chunks.  The chunk's own K/V are already in the pool (appended before
// attention), so query position i reads keys [i-W+1, i] (SWA, from the
// ring) or [0, i] (Full, through the Full page table).
//
// Design (gfx950):
//  - Workgroup = 8 wavefronts for one (sequence, query block, KV head).
//    Wave w owns 32 query positions of one query head of the group, so the
//    G heads sharing a KV head (and, for G < 8, several 32-position groups)
//    share every K/V tile the workgroup stages.
//  - Scores use the 32x32x16 bf16 MFMA as S^T[key][row] = K . Q^T, with the
//    Q^T fragments held in registers for the whole key loop and K read from
//    LDS.  The output uses the 32x32x16 fp16 MFMA as O^T[d][row] = V^T . P^T.
//    The score layout puts each lane's probabilities exactly where the PV
//    product wants them, so P never goes through LDS.
//  - K/V move through LDS in 32-key steps (two 16-token pages), double
//    buffered: global loads of step s+1 are in flight while step s computes.
//    V is converted to fp16 once, at staging, and stored in the key order the
//    PV fragments read (16 contiguous bytes per lane).
//  - Keys outside the workgroup's range are staged as zeros (their slots can
//    hold evicted or unwritten data); per-row masks select -inf scores.
//  - Online softmax in fp32, log2 domain; output fp32.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kPreWaves = 8;
constexpr int kPreThreads = kPreWaves * 64;

template <int D, int KIND, int G>
__global__ void __launch_bounds__(kPreThreads) prefill_kernel(AttnParams p, int qblocks) {
  constexpr int QB = 32 * kPreWaves / G;  // query positions per workgroup
  constexpr int KROW = D + 8;             // LDS K row in bf16 (16-byte pad)
  constexpr int NC = D / 16;              // k steps of the QK product
  constexpr int NM = D / 32;              // 32-row d blocks of O^T
  __shared__ __attribute__((aligned(16))) uint16_t kl[2][32 * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t vl[2][2 * D * 16];

  const int i = blockIdx.x / qblocks;
  const int qb = blockIdx.x % qblocks;
  const int kvh = blockIdx.y;
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
  const int hl = wave % G;
  const int r0 = (wave / G) * 32;        // first workgroup row of this wave
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
  float m = -INFINITY;
  float lsum = 0.f;
  const float sl2 = p.scale_log2;

  const int kstart = (wg_klo / 32) * 32;
  const int nsteps = (wg_khi - kstart) / 32 + 1;
  const int64_t head_stride = (int64_t)kPage * D;

  // staging roles: K thread (key sk, 16-byte chunk sc); V thread (page st,
  // dim sd, 8-key half sh)
  constexpr int KCH = D / 8;
  const bool k_role = tid < 32 * KCH;
  const int sk = tid / KCH;
  const int sc = tid % KCH;
  const bool v_role = tid < 2 * D * 2;
  const int st = tid / (2 * D);
  const int sd = (tid / 2) % D;
  const int sh = tid & 1;

  u32x4 kreg, vreg;
  auto stage_load = [&](int kp0) {
    kreg = u32x4{0, 0, 0, 0};
    vreg = u32x4{0, 0, 0, 0};
    if (k_role) {
      const int tile = kp0 + (sk / 16) * 16;
      const int kp = kp0 + sk;
      if (tile <= wg_khi && kp >= wg_klo && kp <= wg_khi) {
        const int32_t pg = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile, p.t.max_pages,
                                         p.t.ring_slots);
        if (pg >= 0)
          kreg = *(const u32x4*)(p.k_cache + ((int64_t)pg * hkv + kvh) * head_stride +
                               (sk % 16) * D + sc * 8);
      }
    }
    if (v_role) {
      const int tile = kp0 + 16 * st;
      const int k8 = tile + 8 * sh;
      if (tile <= wg_khi && k8 + 7 >= wg_klo && k8 <= wg_khi) {
        const int32_t pg = page_of<KIND>(p.t.fpt, p.t.rpt, sid, tile, p.t.max_pages,
                                         p.t.ring_slots);
        if (pg >= 0)
          vreg = *(const u32x4*)(p.v_cache + ((int64_t)pg * hkv + kvh) * head_stride +
                                 sd * kPage + 8 * sh);
        if (k8 < wg_klo || k8 + 7 > wg_khi) {
          for (int j = 0; j < 8; ++j) {
            const int kp = k8 + j;
            if (kp < wg_klo || kp > wg_khi) vreg[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
          }
        }
      }
    }
  };
  auto stage_store = [&](int buf) {
    if (k_role) *(u32x4*)(&kl[buf][sk * KROW + sc * 8]) = kreg;
    if (v_role) {
      // page-local keys 8*sh + 0..3 go to slots 4*sh + 0..3 and keys
      // 8*sh + 4..7 to slots 8 + 4*sh + 0..3 (the PV operand order)
      uint16_t* dst = &vl[buf][(st * D + sd) * 16];
      u32x2 a = {bf16x2_to_f16x2(vreg[0]), bf16x2_to_f16x2(vreg[1])};
      u32x2 b = {bf16x2_to_f16x2(vreg[2]), bf16x2_to_f16x2(vreg[3])};
      *(u32x2*)(dst + 4 * sh) = a;
      *(u32x2*)(dst + 8 + 4 * sh) = b;
    }
  };

  stage_load(kstart);
  stage_store(0);
  __syncthreads();

  for (int s = 0; s < nsteps; ++s) {
    const int kp0 = kstart + 32 * s;
    const int buf = s & 1;
    if (s + 1 < nsteps) stage_load(kp0 + 32);
    // does this wave have any unmasked key in the step?
    if (wave_on && kp0 <= w_pos_hi && kp0 + 31 >= w_klo) {
      f32x16 sacc;
      for (int r = 0; r < 16; ++r) sacc[r] = 0.f;
      const uint16_t* krow = &kl[buf][qr * KROW + 8 * h2];
      for (int c = 0; c < NC; ++c) {
        bf16x8 kf = __builtin_bit_cast(bf16x8, *(const u32x4*)(krow + 16 * c));
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], sacc, 0, 0, 0);
      }
      // lane value r is key kp0 + 8*(r/4) + 4*h2 + r%4 for query row qr
      float sv[16];
      float mx = -INFINITY;
      for (int r = 0; r < 16; ++r) {
        const int kp = kp0 + 8 * (r >> 2) + 4 * h2 + (r & 3);
        const bool ok = kp <= my_pos && (KIND == 0 || kp > my_pos - W);
        sv[r] = ok ? sacc[r] * sl2 : -INFINITY;
        mx = fmaxf(mx, sv[r]);
      }
      mx = fmaxf(mx, xor_lane(mx, 32));
      const float m_new = fmaxf(m, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m - m_use);
      float ps = 0.f;
      f16x8 pf0, pf1;
      for (int r = 0; r < 8; ++r) {
        const float e0 = fast_exp2(sv[r] - m_use);
        const float e1 = fast_exp2(sv[r + 8] - m_use);
        ps += e0 + e1;
        pf0[r] = (_Float16)e0;
        pf1[r] = (_Float16)e1;
      }
      lsum = lsum * alpha + ps;
      m = m_new;
      const uint16_t* v0 = &vl[buf][0];
      for (int mb = 0; mb < NM; ++mb) {
        o[mb] *= alpha;
        const int d = 32 * mb + qr;
        f16x8 va = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + d * 16 + 8 * h2));
        f16x8 vb = __builtin_bit_cast(f16x8, *(const u32x4*)(v0 + (D + d) * 16 + 8 * h2));
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, pf0, o[mb], 0, 0, 0);
        o[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vb, pf1, o[mb], 0, 0, 0);
      }
    }
    if (s + 1 < nsteps) stage_store(buf ^ 1);
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

template <int D, int KIND>
hipError_t launch_prefill_g(const AttnParams& p, hipStream_t s) {
  const int g = p.hq / p.hkv;
  const int qb_pos = 32 * kPreWaves / g;
  const int qblocks = (p.max_q_len + qb_pos - 1) / qb_pos;
  dim3 grid((unsigned)(p.num_seqs * qblocks), (unsigned)p.hkv);
  switch (g) {
    case 1:
      hipLaunchKernelGGL((prefill_kernel<D, KIND, 1>), grid, dim3(kPreThreads), 0, s, p, qblocks);
      break;
    case 2:
      hipLaunchKernelGGL((prefill_kernel<D, KIND, 2>), grid, dim3(kPreThreads), 0, s, p, qblocks);
      break;
    case 4:
      hipLaunchKernelGGL((prefill_kernel<D, KIND, 4>), grid, dim3(kPreThreads), 0, s, p, qblocks);
      break;
    default:
      hipLaunchKernelGGL((prefill_kernel<D, KIND, 8>), grid, dim3(kPreThreads), 0, s, p, qblocks);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0 || p.total_q <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_prefill_g<128, 0>(p, s) : launch_prefill_g<128, 1>(p, s);
  return p.kind == 0 ? launch_prefill_g<64, 0>(p, s) : launch_prefill_g<64, 1>(p, s);
}

}  // namespace hswa
