// Device-side helpers shared by the gfx950 kernels of the MoE layer: storage types,
// bf16 conversion, MFMA operand types, wave-wide reductions, buffer loads and the LDS
// row swizzle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;  // CDNA wavefront width
constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, 32 CUs each

// bf16 is stored as its raw 16-bit pattern.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Monotone map of an f32 onto uint32: a < b  <=>  key(a) < key(b) (no NaNs).
__device__ __forceinline__ uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), m, kWave);
    uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), m, kWave);
    uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

// LDS tiles are rows of one 128-byte K step (64 bf16 or 32 f32 elements).
constexpr int kRowBytes = 128;

// gfx950's LDS serves a ds_read_b128 16 lanes (256 bytes, 64 banks) at a time; the
// fragment reads of one phase touch 16 consecutive rows at one chunk.  Rows 2j and 2j+1
// fall in different bank halves, and the XOR with (row / 2) % 8 spreads the 8 row pairs
// over the 8 chunk slots, so one phase hits 16 distinct bank groups.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kRowBytes + ((chunk ^ ((row >> 1) & 7)) << 4);
}

// Raw buffer resource over [base, base + bytes): loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base,
                                                              uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes,
                                           0x00020000);
}

// Cache policy of a load: kStream marks data read once (weights streamed from HBM) as
// non-temporal, so it does not push the reused rows and scales out of the L1.
constexpr int kCached = 0;
constexpr int kStream = 2;

// 16 bytes per lane from buffer offset voffset + soffset (buffer_load_dwordx4).
template <int POLICY = kCached>
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voffset,
                                        uint32_t soffset) {
  return __builtin_amdgcn_raw_buffer_load_b128(rsrc, voffset, soffset, POLICY);
}

}  // namespace moe
