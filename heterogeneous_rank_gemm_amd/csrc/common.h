// Device helpers shared by the HIP kernels of the LoRA library (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace hrg {

// 16-byte global load of 8 bf16 values (caller guarantees 16-byte alignment).
__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint16_t* p) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}

// fp32 -> bf16 bits, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// C[16x16] += A[16x32] B[32x16].  Lane l supplies A row (l%16) and B column
// (l%16), each with k in [8*(l/16), 8*(l/16)+8).  Result: lane l holds column
// (l%16), rows 4*(l/16) + i, i = 0..3.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C[32x32] += A[32x16] B[16x32].  Lane l supplies A row (l%32) and B column
// (l%32), each with k in [8*(l/32), 8*(l/32)+8).  Result register r of lane l
// is row 8*(r/4) + 4*(l/32) + (r%4), column (l%32).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Eight 4-bit weights of one 32-bit word (nibble e = bits 4e..4e+3) to bf16:
// bf16((q - z) * s), given s and -z * s in fp32.  q * s and z * s are exact
// in fp32 (a bf16 scale times a 4-bit integer), so the fma is exact and the
// only rounding is the conversion to bf16 (to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ bf16x8 dequant_q4x8(uint32_t w, float s, float nzs) {
  uint32_t lo = w & 0x0f0f0f0fu, hi = (w >> 4) & 0x0f0f0f0fu;
  // opaque to the optimizer, so that byte b converts with one
  // v_cvt_f32_ubyte<b> instead of a bit-field extract plus a conversion
  asm volatile("" : "+v"(lo), "+v"(hi));
  uint32_t p[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    // elements 2b (nibble 2b, byte b of lo) and 2b + 1 (byte b of hi): one
    // packed conversion
    const f32x2_t v = {__builtin_fmaf((float)((lo >> (8 * b)) & 0xffu), s, nzs),
                       __builtin_fmaf((float)((hi >> (8 * b)) & 0xffu), s, nzs)};
    p[b] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  }
  return __builtin_bit_cast(bf16x8, make_uint4(p[0], p[1], p[2], p[3]));
}

// {scale, -zero * scale} of a packed group word (bf16 scale bits 0..15, zero
// point bits 16..19).
__device__ __forceinline__ float2 q4_group(uint32_t sz) {
  const float s = __builtin_bit_cast(float, sz << 16);
  return make_float2(s, -(float)((sz >> 16) & 15u) * s);
}

// Entry b (0..3) of a float4 without a register array (a select chain).
__device__ __forceinline__ float pick4(float4 v, int b) {
  return b == 0 ? v.x : b == 1 ? v.y : b == 2 ? v.z : v.w;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  // DPP lane moves (register to register, no LDS round trip): shifts by
  // 1, 2, 4, 8 within each row of 16 lanes (lanes shifted in read zero),
  // then the last lane of row 0 to row 1 and of row 2 to row 3, then lane 31
  // to rows 2 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// counter[key] += 1 for every lane with `valid`, as one LDS atomic per run of
// equal keys in consecutive valid lanes (a batch whose requests each hold many
// tokens has long runs; 64 lanes adding to one address serialise).  Every
// lane of the wave must call it.
__device__ __forceinline__ void count_runs(int* counter, int key, bool valid) {
  const int lane = __lane_id();
  const uint64_t vmask = __ballot(valid);
  const int left = __shfl_up(key, 1, 64);
  const bool joins = lane > 0 && ((vmask >> (lane - 1)) & 1) && left == key;
  const uint64_t heads = __ballot(valid && !joins);
  const bool last = lane == 63 || !((vmask >> (lane + 1)) & 1) || ((heads >> (lane + 1)) & 1);
  if (valid && last) {
    const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);
    const int first = 63 - __builtin_clzll(heads & upto);
    atomicAdd(&counter[key], lane - first + 1);
  }
}

}  // namespace hrg
