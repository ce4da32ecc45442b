// Paged decode attention over the dual pool, one query row per sequence.
//
// "MiMo-V2.5 Series Inference Full-Link Optimization" sec. 1.2: decode is
// bound by the bytes of KV it reads.  A Full layer reads the whole prefix
// through the Full page table; a SWA layer reads at most W keys from the
// sequence's ring (sec. 2.1 "KVCache Dual Pool").
//
// Design (gfx950):
//  - One workgroup = 4 wavefronts per (sequence, KV head, split).  Full
//    layers split the context in split_len-key pieces so the grid fills 256
//    CUs; pieces are merged by log-sum-exp in decode_combine_kernel.
//  - The G query heads that share a KV head ride in the N dimension of a
//    16x16x32 MFMA: S^T[key][head] = K[key][:] . Q[head][:], so every K/V
//    byte is read from HBM once for all G heads.
//  - K rows (token-major pages) are the A operand loaded straight from HBM,
//    16 bytes per lane.  The 32 keys of a step are dealt to the two 16-row
//    score tiles so that each lane's eight scores are eight consecutive keys
//    of one page (tile 0 row 4a+r is key 8a+r, tile 1 row 4a+r is key
//    8a+4+r); with V pages dim-major and in fp16, the PV product
//    O^T[d][head] = V^T[d][key] . P^T[key][head] then reads each lane's V
//    fragment as 16 contiguous bytes and needs no conversion.  P enters the
//    PV MFMA as fp16, keeping the weights to 11 significant bits.
//  - Online softmax in fp32 in the log2 domain (exp2 of prescaled scores).
//  - Wave w takes 32-key steps w, w+4, ...; the four partial states merge
//    through LDS in a fixed order, so results depend only on logical key
//    positions, never on where pages sit in memory.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kDecWaves = 4;

template <int D, int KIND, int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 4)))
decode_kernel(AttnParams p) {
  constexpr int NB = D / 16;  // 16-row d blocks of O^T
  constexpr int NC = D / 32;  // 32-wide d chunks of the QK reduction
  __shared__ __attribute__((aligned(16))) float red_o[kDecWaves][G][D];
  __shared__ float red_ml[kDecWaves][G][2];

  // KV head fastest in the grid: workgroups running at the same time then
  // read all KV heads' slices of the pages, which spreads their traffic over
  // all HBM channels (one head's 4 KB slices alone concentrate on a few).
  const int kvh = blockIdx.x % p.hkv;
  const int i = (blockIdx.x / p.hkv) / p.n_splits;
  const int split = (blockIdx.x / p.hkv) % p.n_splits;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int L = p.t.seq_len[sid];
  int klo, khi;  // keys [klo, khi) of this workgroup
  if (KIND == 0) {
    klo = split * p.split_len;
    khi = min(L, klo + p.split_len);
  } else {
    klo = max(0, L - p.window);
    khi = L;
  }
  if (klo >= khi) return;  // whole workgroup idle: no barrier reached

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // query head within the group (N index)
  const int q4 = lane >> 4;   // which 8-wide k slice / 4-row group
  const int hq = p.hq;
  const int hkv = p.hkv;

  // Q^T fragments: lane holds Q[head col][32c + 8*q4 .. +8]
  bf16x8 qf[NC];
  {
    const bool has = col < G;
    const uint16_t* qrow = p.q + ((int64_t)i * hq + kvh * G + (has ? col : 0)) * D;
    for (int c = 0; c < NC; ++c) {
      u32x4 w = has ? *(const u32x4*)(qrow + 32 * c + 8 * q4) : u32x4{0, 0, 0, 0};
      qf[c] = __builtin_bit_cast(bf16x8, w);
    }
  }

  f32x4 o[NB];
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  float lsum = 0.f;
  const float sl2 = p.scale_log2;

  const int s0 = (klo / 32) * 32;
  const int nsteps = (khi - 1 - s0) / 32 + 1;
  const int64_t head_stride = (int64_t)kPage * D;  // elements per (page, head) block

  // Page-table row of the sequence, read through the constant address space
  // so the lookups are scalar loads (the tables do not change while the
  // kernel runs).
  typedef const __attribute__((address_space(4))) int32_t* ctab_t;
  const ctab_t ptab = (ctab_t)(KIND == 0 ? p.t.fpt + (int64_t)sid * p.t.max_pages
                                         : p.t.rpt + (int64_t)sid * (p.t.ring_slots / kPage));
  auto page_at = [&](int pos) {
    const int idx = KIND == 0 ? pos / kPage : (pos % p.t.ring_slots) / kPage;
    return ptab[__builtin_amdgcn_readfirstlane(idx)];
  };
  // K: this lane's row `col` of score tile t is key 8*(col/4) + 4t + col%4,
  // on page col/8.  V: keys 8*q4 .. +8 are page q4/2, offset 8*(q4%2).
  const int kpage = col >> 3;
  const int krow0 = (8 * (col >> 2) + (col & 3)) & 15;
  const int k_lane = krow0 * D + 8 * q4;
  const int v_lane = col * kPage + 8 * (q4 & 1);
  auto step_pages = [&](int kp0, const uint16_t*& kb, const uint16_t*& vb) {
    int32_t pg0 = page_at(kp0);
    // a page past the last key: read page 0 again (those keys are masked)
    int32_t pg1 = kp0 + 16 < khi ? page_at(kp0 + 16) : pg0;
    // a missing page means the caller skipped alloc: read page 0 of the pool
    // instead of faulting (the result of such a call is undefined)
    pg0 = pg0 < 0 ? 0 : pg0;
    pg1 = pg1 < 0 ? 0 : pg1;
    kb = p.k_cache + ((int64_t)(kpage ? pg1 : pg0) * hkv + kvh) * head_stride + k_lane;
    vb = p.v_cache + ((int64_t)((q4 >> 1) ? pg1 : pg0) * hkv + kvh) * head_stride + v_lane;
  };

  // Software pipeline, register-neutral: the K loads of this wave's next
  // step are issued as soon as the score MFMAs have consumed the current K
  // fragments, the V loads as soon as the PV MFMAs have consumed V; so each
  // wave keeps a step's worth of bytes in flight through its math.
  u32x4 kr[2][NC], vr[NB];
  const uint16_t *kb, *vb;
  if (wave < nsteps) {
    step_pages(s0 + 32 * wave, kb, vb);
    for (int c = 0; c < NC; ++c) {
      kr[0][c] = *(const u32x4*)(kb + 32 * c);
      kr[1][c] = *(const u32x4*)(kb + 4 * D + 32 * c);
    }
    for (int nb = 0; nb < NB; ++nb) vr[nb] = *(const u32x4*)(vb + 16 * nb * kPage);
  }
  for (int st = wave; st < nsteps; st += kDecWaves) {
    const int kp0 = s0 + 32 * st;
    const bool more = st + kDecWaves < nsteps;
    const uint16_t *kbn = kb, *vbn = vb;
    if (more) step_pages(kp0 + 32 * kDecWaves, kbn, vbn);

    // S^T for the two 16-key tiles, then refill K
    f32x4 s[2];
    for (int t = 0; t < 2; ++t) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int c = 0; c < NC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[t][c]), qf[c],
                                                      acc, 0, 0, 0);
      s[t] = acc;
    }
    if (more)
      for (int c = 0; c < NC; ++c) {
        kr[0][c] = *(const u32x4*)(kbn + 32 * c);
        kr[1][c] = *(const u32x4*)(kbn + 4 * D + 32 * c);
      }
    // mask: lane value (t, r) is key kp0 + 8*q4 + 4t + r
    unsigned valid = 0;
    float mx = -INFINITY;
    float sv[8];
    for (int t = 0; t < 2; ++t)
      for (int r = 0; r < 4; ++r) {
        const int kp = kp0 + 8 * q4 + 4 * t + r;
        const bool ok = kp >= klo && kp < khi;
        valid |= (unsigned)ok << (4 * t + r);
        const float x = ok ? s[t][r] * sl2 : -INFINITY;
        sv[4 * t + r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    f16x8 pf;
    float ps = 0.f;
    for (int j = 0; j < 8; ++j) {
      pf[j] = (_Float16)fast_exp2(sv[j] - m_use);
      ps += (float)pf[j];  // sum the fp16 weights the PV product uses
    }
    lsum = lsum * alpha + ps;
    m = m_new;
    u32x4 vmask = {~0u, ~0u, ~0u, ~0u};
    if (valid != 0xffu) {
      // zero V of masked keys: their slots may hold stale or unwritten data
      for (int j = 0; j < 8; ++j)
        if (!((valid >> j) & 1u)) vmask[j >> 1] &= (j & 1) ? 0x0000ffffu : 0xffff0000u;
    }
    for (int nb = 0; nb < NB; ++nb) {
      const f16x8 vf = __builtin_bit_cast(f16x8, vr[nb] & vmask);
      o[nb] *= alpha;
      o[nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pf, o[nb], 0, 0, 0);
    }
    // refill V
    if (more)
      for (int nb = 0; nb < NB; ++nb) vr[nb] = *(const u32x4*)(vbn + 16 * nb * kPage);
    kb = kbn;
    vb = vbn;
  }

  // merge the four waves' states (fixed order)
  lsum += xor_lane(lsum, 16);
  lsum += xor_lane(lsum, 32);
  if (col < G) {
    for (int nb = 0; nb < NB; ++nb)
      *(f32x4*)(&red_o[wave][col][16 * nb + 4 * q4]) = o[nb];
    if (q4 == 0) {
      red_ml[wave][col][0] = m;
      red_ml[wave][col][1] = lsum;
    }
  }
  __syncthreads();
  const int hq_base = kvh * G;
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int c = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_ml[w][c][0]);
    float num = 0.f, den = 0.f;
    for (int w = 0; w < kDecWaves; ++w) {
      const float mw = red_ml[w][c][0];
      const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
      num += sc * red_o[w][c][d];
      den += sc * red_ml[w][c][1];
    }
    const int64_t hrow = (int64_t)i * hq + hq_base + c;
    if (p.n_splits == 1) {
      p.out[hrow * D + d] = num / den;
    } else {
      const int64_t slot = hrow * p.n_splits + split;
      p.ws[slot * D + d] = num;
      if (d == 0) {
        float* ml = p.ws + (int64_t)p.num_seqs * hq * p.n_splits * D;
        ml[2 * slot] = M;
        ml[2 * slot + 1] = den;
      }
    }
  }
  if (p.vlen && split == 0 && kvh == 0 && threadIdx.x == 0)
    p.vlen[i] = KIND == 0 ? L : min(L, p.window);
}

// Log-sum-exp merge of the split partial states of one (sequence, head).
template <int D>
__global__ void __launch_bounds__(D) decode_combine_kernel(AttnParams p) {
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int L = p.t.seq_len[sid];
  const int ns = min(p.n_splits, (L + p.split_len - 1) / p.split_len);
  const int64_t hrow = (int64_t)i * p.hq + h;
  const float* ml = p.ws + (int64_t)p.num_seqs * p.hq * p.n_splits * D;
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, ml[2 * (hrow * p.n_splits + s)]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t slot = hrow * p.n_splits + s;
    const float sc = fast_exp2(ml[2 * slot] - M);
    num += sc * p.ws[slot * D + d];
    den += sc * ml[2 * slot + 1];
  }
  p.out[hrow * D + d] = num / den;
}

template <int D, int KIND>
hipError_t launch_decode_g(const AttnParams& p, hipStream_t s) {
  dim3 grid((unsigned)(p.num_seqs * p.n_splits * p.hkv), 1);
  const int g = p.hq / p.hkv;
  switch (g) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, KIND, 1>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, KIND, 2>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, KIND, 4>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_kernel<D, KIND, 8>), grid, dim3(256), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_splits == 1) return e;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.num_seqs, p.hq), dim3(D), 0, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_decode_g<128, 0>(p, s) : launch_decode_g<128, 1>(p, s);
  return p.kind == 0 ? launch_decode_g<64, 0>(p, s) : launch_decode_g<64, 1>(p, s);
}

}  // namespace hswa
