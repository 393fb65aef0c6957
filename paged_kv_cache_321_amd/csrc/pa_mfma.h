// Matrix-core building blocks shared by the decode and multi-query attention
// kernels: operand vector types, bf16 packing, exact E4M3 -> bf16 widening and
// the swizzled LDS page that is read back transposed as an MFMA operand.
//
// MFMA operand layouts on gfx950 (v_mfma_f32_16x16x32_bf16 and
// v_mfma_f32_16x16x16bf16_1k, checked on the hardware): A lane i holds row
// i % 16 at k = 8 * (i / 16) + j (4 * (i / 16) + j for the 16-deep form);
// B lane i holds column i % 16 at the same k; the f32 result lane i holds rows
// 4 * (i / 16) + j of column i % 16.
#ifndef PA_MFMA_H_
#define PA_MFMA_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Orders this wave's LDS writes before its later LDS reads (and the reverse)
// as seen by the compiler; the LDS unit serves one wave's requests in order.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Two finite floats -> two bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// c + the two bf16 values packed in w, in one v_dot2_f32_bf16 against (1, 1)
// (the products are exact; one float32 rounding of the sum): the softmax
// weights as the PV product sees them, so that the running sum (the
// denominator) adds exactly the weights the numerator was formed with.
__device__ __forceinline__ float bf16x2_acc(uint32_t w, float c) {
  constexpr uint32_t kOnes = 0x3f803f80u;  // bf16 1.0 in both halves
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, kOnes), c,
                                         false);
}

// Eight E4M3 codes -> eight bf16, exact (an E4M3 value has 3 mantissa bits),
// with v_cvt_scalef32_pk_bf16_fp8 at scale 1 (checked on gfx950: exact for all
// 256 codes in both halves).
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  return make_uint4(fp8x2_to_bf16x2<false>(lo), fp8x2_to_bf16x2<true>(lo), fp8x2_to_bf16x2<false>(hi),
                    fp8x2_to_bf16x2<true>(hi));
}

// V page in LDS (rows of ROWB = 128 or 256 bytes), read back transposed.
// 16-byte chunk c of row `row` is stored at chunk c ^ swz<ROWB>(row).  In a
// transposed read each 16-lane group reads 4 consecutive rows, and two such
// groups 8 consecutive rows, at the same 32-byte column segment.  The
// swizzle moves the segment by an even number of chunks so that, whether the
// LDS serves 16 lanes over 32 banks or 32 lanes over 64 banks (4-byte banks)
// per cycle, the rows served together hit distinct banks: 256-byte rows
// (a whole 64-bank line) take 8 segment positions, 128-byte rows (half a
// line, alternating halves) 4 positions spread over both parities.
template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  static_assert(ROWB == 128 || ROWB == 256, "128- or 256-byte rows");
  return ROWB == 256 ? 2 * (row & 7) : 2 * ((row & 3) ^ ((row >> 2) & 1));
}

// Four k slots of the V^T A operand from a bf16 page of ROWB-byte rows, via
// gfx950's ds_read_b64_tr_b16 (checked on the hardware): in each group of 16
// lanes, lane 4r + c receives element c of the 8-byte rows addressed by lanes
// r, r + 4, r + 8, r + 12.  Lane l16 addresses token tb + l16 / 4 at columns
// d0 + 4 (l16 % 4) .. +3, so it receives column d0 + l16 of tokens tb .. tb + 3.
template <int ROWB>
__device__ __forceinline__ s16x4_t vt4(const unsigned char* page, int l16, int tb, int d0) {
  const int t = tb + (l16 >> 2);
  const int d = d0 + 4 * (l16 & 3);
  const unsigned char* a = page + t * ROWB + (((d >> 3) ^ swz<ROWB>(t)) << 4) + ((d & 7) << 1);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4_t*)a);
}

}  // namespace pa

#endif  // PA_MFMA_H_
