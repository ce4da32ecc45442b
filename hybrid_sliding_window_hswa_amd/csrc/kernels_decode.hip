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
//  - One workgroup = 4 wavefronts per (sequence, KV head, split).  Full
//    layers split the context in split_len-key pieces so the grid fills 256
//    CUs; pieces are merged by log-sum-exp in decode_combine_kernel.
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

#include <type_traits>

#include "device.h"
#include "internal.h"

namespace hswa {

using namespace dev;

namespace {

constexpr int kDecWaves = 4;

template <int D, int KIND, int G, int QN, bool F8>
__global__ void __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(G * QN > 16 ? 2 : 3, 4))) decode_kernel(AttnParams p) {
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

  // KV head fastest in the grid: workgroups running at the same time then
  // read all KV heads' slices of the pages, which spreads their traffic over
  // all HBM channels (one head's 4 KB slices alone concentrate on a few).
  const int kvh = blockIdx.x % p.hkv;
  const int i = (blockIdx.x / p.hkv) / p.n_splits;
  const int split = (blockIdx.x / p.hkv) % p.n_splits;
  const int sid = p.seq_ids[i];
  if (sid < 0 || sid >= p.t.max_seqs) return;
  const int L = p.t.seq_len[sid];
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;  // rows: positions L-n .. L-1
  if (n <= 0 || n > L) return;
  const int nr = min(n, QN);                         // rows computed here
  int klo, khi;  // keys [klo, khi) of this workgroup
  if (KIND == 0) {
    klo = split * p.split_len;
    khi = min(L, klo + p.split_len);
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
    const int idx = KIND == 0 ? pos / kPage : (pos % p.t.ring_slots) / kPage;
    return ptab[__builtin_amdgcn_readfirstlane(idx)];
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
    int32_t pg0 = page_at(kp0);
    // a page past the last key: read page 0 again (those keys are masked)
    int32_t pg1 = kp0 + 16 < khi ? page_at(kp0 + 16) : pg0;
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
      kr[0][c] = *(const Raw*)(pt.k + 32 * c * ESZ);
      kr[1][c] = *(const Raw*)(pt.k + (4 * D + 32 * c) * ESZ);
    }
  };
  auto load_v = [&](const Ptrs& pt, Raw (&vr)[NB]) {
    for (int nb = 0; nb < NB; ++nb) vr[nb] = *(const Raw*)(pt.v + 16 * nb * kPage * ESZ);
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
      const float m_new = fmaxf(m[t], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[t] = fast_exp2(m[t] - m_use);
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
      m[t] = m_new;
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
        o[t][nb] *= alpha[t];
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

  // merge the four waves' states (fixed order), one column tile at a time
  const int hq_base = kvh * G;
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
      const int g = 16 * t + c;
      const int r = g / G;
      if (r >= nr) continue;
      float M = -INFINITY;
      for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, red_ml[w][c][0]);
      float num = 0.f, den = 0.f;
      for (int w = 0; w < kDecWaves; ++w) {
        const float mw = red_ml[w][c][0];
        const float sc2 = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        num += sc2 * red_o[w][c][d];
        den += sc2 * red_ml[w][c][1];
      }
      const int64_t hrow = (int64_t)(row0 + r) * hq + hq_base + g % G;
      if (p.n_splits == 1) {
        p.out[hrow * D + d] = num / den;
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
  if (p.vlen && split == 0 && kvh == 0 && (int)threadIdx.x < nr) {
    const int pos = L - n + threadIdx.x;
    p.vlen[row0 + threadIdx.x] = KIND == 0 ? pos + 1 : min(pos + 1, W);
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
  const int L = p.t.seq_len[sid];
  const int row0 = p.cu_q ? p.cu_q[i] : i;
  const int n = p.cu_q ? p.cu_q[i + 1] - row0 : 1;
  if (n <= 0 || n > L || r >= n) return;
  const int ns = min(p.n_splits, (L + p.split_len - 1) / p.split_len);
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
  p.out[hrow * D + d] = num / den;
}

template <int D, int KIND, int QN, bool F8>
hipError_t launch_decode_q(const AttnParams& p, hipStream_t s) {
  dim3 grid((unsigned)(p.num_seqs * p.n_splits * p.hkv), 1);
  switch (p.hq / p.hkv) {
    case 1: hipLaunchKernelGGL((decode_kernel<D, KIND, 1, QN, F8>), grid, dim3(256), 0, s, p); break;
    case 2: hipLaunchKernelGGL((decode_kernel<D, KIND, 2, QN, F8>), grid, dim3(256), 0, s, p); break;
    case 4: hipLaunchKernelGGL((decode_kernel<D, KIND, 4, QN, F8>), grid, dim3(256), 0, s, p); break;
    default: hipLaunchKernelGGL((decode_kernel<D, KIND, 8, QN, F8>), grid, dim3(256), 0, s, p); break;
  }
  hipError_t e = hipGetLastError();
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

hipError_t launch_decode(const AttnParams& p, hipStream_t s) {
  if (p.num_seqs <= 0) return hipSuccess;
  if (p.d == 128)
    return p.kind == 0 ? launch_decode_g<128, 0>(p, s) : launch_decode_g<128, 1>(p, s);
  return p.kind == 0 ? launch_decode_g<64, 0>(p, s) : launch_decode_g<64, 1>(p, s);
}

}  // namespace hswa
