// Shared device-side definitions for the SageSLA kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sagesla {

constexpr int kD = 128;         // head dimension
constexpr int kBlk = 64;        // tokens per block
constexpr int kBlkBytes = 8192; // one block of INT8/FP8 codes (64 x 128)
constexpr int kChunk = 16;      // key blocks per linear-state partial sum
constexpr int kStateElems = 129 * 128;  // one block's linear state: H^T (128 x 128) and z (1 x 128)
constexpr int kGroup = 256;     // query blocks per group in the complement kernels
constexpr int kMaskWords = kGroup / 32;  // 32-bit words of one union entry's membership mask

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef short v8s __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Two fp32 -> bf16 round-to-nearest-even conversions packed in one word (a low, b high):
// one gfx950 v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// INT8 code: round half to even of x*inv, clamped to [-127, 127]
__device__ __forceinline__ int q_int8(float x, float inv) {
  float y = __builtin_rintf(x * inv);
  y = fminf(fmaxf(y, -127.0f), 127.0f);
  return (int)y;
}

__device__ __forceinline__ int block_len(int i, int N) {
  int rem = N - i * kBlk;
  return rem < kBlk ? rem : kBlk;
}

// Byte offset of (row, channel) of a 64x128 INT8 block in MFMA operand order:
// ((t*4 + s)*64 + lane)*16 + e with t = row/32, r = row%32, g = ch/64, s = (ch%64)/16,
// e = ch%16, lane = 32*g + r.
__device__ __forceinline__ int qk_code_offset(int row, int ch) {
  int t = row >> 5, r = row & 31, g = ch >> 6, s = (ch >> 4) & 3, e = ch & 15;
  return ((t * 4 + s) * 64 + (g * 32 + r)) * 16 + e;
}

// Byte offset of (token, channel) of a 64x128 FP8 V block in MFMA operand order:
// ((dt*2 + e/16)*64 + lane)*16 + e%16 with dt = ch/32, r = ch%32, lane = 32*g + r, where
// the token is decomposed as token = 32*(e/16) + 8*((e%16)/4) + 4*g + e%4 (e in 0..31:
// the operand's 32 bytes, stored as two lane-contiguous 16-byte halves).
__device__ __forceinline__ int v_code_offset(int tok, int ch) {
  int dt = ch >> 5, r = ch & 31;
  int t = tok >> 5, rem = tok & 31, a = rem >> 3, g = (rem >> 2) & 1, b = rem & 3;
  int e = 16 * t + 4 * a + b;
  return ((dt * 2 + (e >> 4)) * 64 + (g * 32 + r)) * 16 + (e & 15);
}

// XCD-aware tile order: consecutive workgroup ids go round-robin over the 8 XCDs, so
// give each XCD a contiguous run of tiles (same head, neighbouring blocks share L2).
__device__ __forceinline__ int xcd_tile(int bid, int per_xcd) { return (bid & 7) * per_xcd + (bid >> 3); }

}  // namespace sagesla
