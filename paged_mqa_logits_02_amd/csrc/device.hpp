// Device helpers for gfx950 (CDNA4): MFMA operand types, matrix-core
// wrappers, cross-lane reductions and small load/store helpers.  Everything
// here is wave64-specific.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pmqa {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kPage = 64;   // tokens per KV page
constexpr int kWave = 64;   // lanes per wavefront

constexpr int kFmtFp4 = 4;  // cbsz/blgp operand format: e2m1

// D[16x16] = A[16x128] * B[128x16] (+ C), e2m1 operands (32 values = 16
// bytes per lane) and one e8m0 block scale per lane and operand, applied to
// that lane's 32 values; fp32 accumulate.  Lane l holds row (l & 15) of A /
// column (l & 15) of B and 32 of the 128 K values, in the same slots for A
// and B.  Output lane l, element i is D[4*(l>>4) + i][l & 15].
__device__ __forceinline__ v4f mfma_fp4(const v4i& a, int sa, const v4i& b, int sb, const v4f& c) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 0, sa, 0,
                                                          sb);
}

// D[32x32] = A[32x64] * B[64x32] (+ C), e2m1 operands (32 values = 16 bytes
// per lane) and one e8m0 block scale per lane and operand; fp32 accumulate.
// Lane l holds row (l & 31) of A / column (l & 31) of B and 32 of the 64 K
// values, in the same slots for A and B.  Output lane l, element i is
// D[8*(i>>2) + 4*(l>>5) + (i&3)][l & 31].
__device__ __forceinline__ v16f mfma32_fp4(const v4i& a, int sa, const v4i& b, int sb,
                                           const v16f& c) {
  v8i a8 = {a[0], a[1], a[2], a[3], 0, 0, 0, 0};
  v8i b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8, b8, c, kFmtFp4, kFmtFp4, 0, sa, 0,
                                                         sb);
}

// Summation precision of the matrix instructions (measured on gfx950 with
// crafted operands, one instruction each):
//  * FP8 forms (16x16x128 / 32x32x64 f8f6f4, 16x16x32 fp8): the products of
//    each run of 8 consecutive K values of a lane are summed in fixed point
//    aligned to the run's largest product, keeping bits down to 2^-13 of that
//    product's leading bit and truncating the rest toward zero; the runs'
//    sums and C are then added at fp32 precision.  A product below 2^-13 of
//    its run's largest vanishes, so a cancelling dot product can lose its
//    whole value.
//  * FP4 operands: every e2m1 x e2m1 product is a multiple of 1/4 of at most
//    36, so a run always fits the window: exact, and 32-value blocks whose
//    scales lie 2^30 apart still add at fp32 precision.
//  * f16 / bf16 forms: products exact, sums at fp32 precision.
// The FP8 variant therefore widens its e4m3 operands exactly to f16 and
// multiplies them with the f16 forms.

// D[16x16] = A[16x32] * B[32x16] (+ C), f16 operands (8 per lane), fp32
// accumulate; output layout as mfma_fp4.
__device__ __forceinline__ v4f mfma_f16(const v8h& a, const v8h& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Eight e4m3 values (the bytes of lo, then of hi) widened to f16; exact for
// every finite code, subnormals included (checked on all 256 codes).
__device__ __forceinline__ v8h e4m3x8_to_f16(int lo, int hi) {
  const v2h a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const v2h b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const v2h c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const v2h d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return (v8h){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// A lane's 32 e4m3 K values of one FP8 operand fragment (bytes 8u .. 8u+7 in
// octet u), widened to f16.  The octets feed four f16 products of 8 K values
// per lane; query and key octets are formed the same way, so every product
// pairs matching head_dim indices.
struct Half32 {
  v8h h[4];
};
__device__ __forceinline__ Half32 widen32(const v8i& v) {
  Half32 r;
#pragma unroll
  for (int u = 0; u < 4; ++u) r.h[u] = e4m3x8_to_f16(v[2 * u], v[2 * u + 1]);
  return r;
}
// Sum over the 32 K values of one lane group (16x16 output tiles).
__device__ __forceinline__ v4f mfma_half32(const Half32& a, const Half32& b, v4f c) {
#pragma unroll
  for (int u = 0; u < 4; ++u) c = mfma_f16(a.h[u], b.h[u], c);
  return c;
}

// D[16x16] = A[16x32] * B[32x16] (+ C), bf16 operands (8 per lane), fp32 accumulate.
__device__ __forceinline__ v4f mfma_bf16(const v8bf& a, const v8bf& b, const v4f& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float relu(float x) { return __builtin_fmaxf(x, 0.0f); }

// Sum of x over lanes l, l^32: v_permlane32_swap exchanges the upper half of
// its first operand with the lower half of its second.
__device__ __forceinline__ void swap32(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}
// v_permlane16_swap exchanges the odd 16-lane rows of the first operand with
// the even rows of the second.
__device__ __forceinline__ void swap16(float& x, float& y) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  x = __uint_as_float(r[0]);
  y = __uint_as_float(r[1]);
}

// Transposing reduction over the four 16-lane rows.  Input: four values a[s]
// per lane.  Output (returned): in row g (lanes 16g..16g+15), lane l holds
// sum over rows r of a[g] at lane 16r + (l & 15).
__device__ __forceinline__ float row_transpose_reduce4(float a0, float a1, float a2, float a3) {
  swap32(a0, a2);  // a0: rows 0,1 of old a0 | rows 0,1 of old a2 (upper half)
  swap32(a1, a3);
  float x = a0 + a2;  // rows 0-1: a0 halves summed; rows 2-3: a2 halves summed
  float y = a1 + a3;  // rows 0-1: a1; rows 2-3: a3
  swap16(x, y);
  return x + y;  // row 0: a0, row 1: a1, row 2: a2, row 3: a3 (full sums)
}

// Sum over all four 16-lane rows, result in every row.
__device__ __forceinline__ float row_reduce4(float a) {
  float b = a;
  swap32(a, b);
  a += b;
  b = a;
  swap16(a, b);
  return a + b;
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
__device__ __forceinline__ T ldg(const void* p) {
  return *reinterpret_cast<const T*>(p);
}

// Wave-wide inclusive prefix sum (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d, kWave);
    if (lane >= d) v += u;
  }
  return v;
}

}  // namespace pmqa
