// Device-side helpers shared by the gfx950 kernels of libsmlp.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smlp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// fp32 -> bf16 bits, round to nearest, ties to even; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> packed bf16x2 (lo in bits 0..15).
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// SiLU(g) * u in fp32: g * u / (1 + e^-g).  expf of a large positive -g overflows to
// +inf and gives -0, the correct limit.
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g * u / (1.0f + __expf(-g));
}

// D += A * B for one 16x16x32 bf16 tile.  Lane l holds A[l%16][8*(l/16) .. +7],
// B[8*(l/16) .. +7][l%16]; D: lane l, element j holds D[4*(l/16)+j][l%16].
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A * B for one 32x32x16 bf16 tile.  Lane l holds A[l%32][8*(l/32) .. +7],
// B[8*(l/32) .. +7][l%32]; D: lane l, element j holds
// D[8*(j/4) + 4*(l/32) + j%4][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// D += A * B for one 32x32x16 fp16 tile (same lane layout as the bf16 form).
__device__ __forceinline__ f32x16 mfma32x32x16_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}

// Eight bf16 values -> eight fp16 values, element order kept.  Every bf16 value in the
// fp16 normal range is exactly representable (8 significant bits of 11), so the
// conversion is exact there; smaller magnitudes round toward zero to a multiple of
// 2^-24 and magnitudes past 65504 saturate to 65504 (neither occurs for weights).
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(v[j] << 16),
                                                                  __uint_as_float(v[j] & 0xffff0000u)));
  return r;
}

// fp32 -> fp16 bits, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint32_t f2h(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Buffer resource over [base, base + bytes) for raw buffer loads; a load whose offset
// is at or past `bytes` returns zeros without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
// 16-byte raw buffer loads: non-temporal (read-once weights) and default policy.
__device__ __forceinline__ u32x4 buf_ld_nt(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2));
}
__device__ __forceinline__ u32x4 buf_ld(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// 16-byte buffer loads of each lane straight into LDS: lane p of the wave writes bytes
// [16p, 16p + 16) of the 1 KB block at `dst` (one block for the whole wave; the
// address must be wave-uniform).  Out-of-range offsets write zeros.  Completion is
// tracked by vmcnt like any vector memory load.  Non-temporal and default policy.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void buf_ld_lds_nt(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, 0, 0, 2);
}
__device__ __forceinline__ void buf_ld_lds(__amdgpu_buffer_rsrc_t r, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, (int)off, 0, 0, 0);
}

// s_waitcnt vmcnt(n) (expcnt and lgkmcnt not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0f70);
}

// 16-byte global loads.  Weights are read exactly once per call, so they are loaded
// non-temporally; activations are re-read by many workgroups and use normal loads.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace smlp
