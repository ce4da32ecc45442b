// Device-side helpers for the gfx950 kernels: vector types for the MFMA
// builtins, bf16/fp16 conversions, cross-lane reductions and page lookups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "index.h"
#include "internal.h"

namespace hswa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kPage = 16;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two bf16 (packed in one dword) -> two fp16 (packed).  Exact for
// 2^-14 <= |x| <= 65280 (the largest bf16 below fp16's limit); smaller
// magnitudes round to fp16 subnormals, |x| >= 65536 rounds to +-inf.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  f16x2 h = {(_Float16)bf16_lo(w), (_Float16)bf16_hi(w)};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 h = {(_Float16)a, (_Float16)b};
  return __builtin_bit_cast(uint32_t, h);
}

// Lane exchange inside a wavefront (ds_bpermute based).
__device__ __forceinline__ float xor_lane(float v, int mask) {
  int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane ^ mask) & 63) << 2, __float_as_int(v)));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Waits until every vector memory load of the wave has returned (gfx9
// s_waitcnt encoding: vmcnt = 0, expcnt and lgkmcnt left at their maxima).
// Used once after loads whose registers stay live across a loop, so the
// compiler's wait insertion need not assume they are still in flight inside
// the loop.
__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// FP8 (OCP e4m3: 1 sign, 4 exponent bits with bias 7, 3 fraction bits,
// subnormals below 2^-6 in steps of 2^-9, largest finite 448, 0x7F NaN).

// e4m3 code of an fp32 value, rounded to nearest with ties to an even
// fraction, saturated at 448 (every |y| > 448 becomes +-448; no NaN is
// produced).  Written from the format definition with integer operations.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fminf(fabsf(y), 448.0f);
  if (a < 0.015625f)  // below 2^-6: subnormal step 2^-9 (8 steps = smallest normal)
    return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t b = __float_as_uint(a);
  const uint32_t m = b & 0x7fffffu;
  const uint32_t e = (b >> 23) - 120u;                   // (E - 127) + 7
  const uint32_t q = (m + 0x7ffffu + ((m >> 20) & 1u)) >> 20;  // 3 bits, ties to even
  return sign | ((e << 3) + q);                          // q == 8 carries into e
}

// Four e4m3 codes (one dword, byte j = code j) -> four bf16 (two dwords),
// exactly: every e4m3 value is a bf16 value.  gfx950's scaled conversion
// takes two codes (word_sel picks bytes 0-1 or 2-3) straight to a bf16
// pair; with scale 1 it equals the fp32 decode of OCP e4m3 (itself checked
// against the definition on all 256 codes) on every non-NaN code pair.
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true))};
}

// The same four codes -> four fp16, exactly (e4m3 values lie in fp16's
// normal range).
__device__ __forceinline__ u32x2 e4m3x4_to_f16x4(uint32_t w) {
  return u32x2{
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true))};
}

// Physical page holding the 16-aligned key tile that starts at `pos` for
// sequence `sid`: Full layers read the Full page table, SWA layers the ring
// page table (position taken modulo the ring size).
template <int KIND>
__device__ __forceinline__ int32_t page_of(const int32_t* __restrict__ fpt,
                                           const int32_t* __restrict__ rpt, int32_t sid,
                                           int32_t pos, int32_t max_pages, int32_t ring) {
  const int32_t e = idx::table_entry(KIND, pos, ring);
  return KIND == 0 ? fpt[(int64_t)sid * max_pages + e] : rpt[(int64_t)sid * (ring / kPage) + e];
}

// The same lookup for a wave-uniform (sid, pos), as a scalar load: the
// entry arrives in a scalar register and only the scalar-memory counter is
// waited on, so vector loads already in flight (a prefetch of K/V) are not
// waited for.  A read through the scalar cache; the pool tables hold fewer
// than 2^31 entries (pool creation checks it).
__device__ __forceinline__ int32_t scalar_load_i32(const int32_t* base, int32_t idx) {
  const int32_t* ptr = base + __builtin_amdgcn_readfirstlane(idx);
  int32_t v;
  asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(ptr) : "memory");
  return v;
}
template <int KIND>
__device__ __forceinline__ int32_t page_of_uniform(const int32_t* __restrict__ fpt,
                                                   const int32_t* __restrict__ rpt, int32_t sid,
                                                   int32_t pos, int32_t max_pages,
                                                   int32_t ring) {
  const int32_t e = idx::table_entry(KIND, pos, ring);
  return KIND == 0 ? scalar_load_i32(fpt, sid * max_pages + e)
                   : scalar_load_i32(rpt, sid * (ring / kPage) + e);
}

// Length of sequence i of an attention or append call whose n rows are its
// last positions: the caller's q_pos (first row's position) plus n when
// given, else the pool's seq_len.  With q_pos the kernels read no pool table
// that an alloc writes (for SWA layers; Full layers still read fpt).
__device__ __forceinline__ int call_len(const AttnParams& p, int i, int sid, int n) {
  return p.q_pos ? p.q_pos[i] + n : p.t.seq_len[sid];
}

}  // namespace dev
}  // namespace hswa
