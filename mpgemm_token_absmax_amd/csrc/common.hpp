// Device helpers shared by the gfx950 kernels of the ternary BitLinear library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bl {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Decoding 2-bit codes with v_perm_b32 (byte select from the 8 bytes
// {S0:S1}; selector 0-7 picks a byte, 8 replicates the sign bit of byte 1,
// 12 gives 0x00). I2_S codes 00/01/10 are 0/+1/-1; the unused 11 decodes to 0.
//  * a field in bits 0-1 of each byte (mask 0x03030303) selects 0..3:
//    table bytes 0x00, 0x01, 0xFF, 0x00 in S1 (kLutLo);
//  * a field in bits 2-3 (mask 0x0C0C0C0C) selects 0, 4, 8, 12:
//    byte 0 = 0x00 (S1), byte 4 = 0x01 (S0 byte 0), sign of S1 byte 1 = 1
//    (-> 0xFF), and 12 -> 0x00 (kLutHiS1 / kLutHiS0).
constexpr uint32_t kLutLo = 0x00FF0100u;
constexpr uint32_t kLutHiS1 = 0x00008000u;
constexpr uint32_t kLutHiS0 = 0x00000001u;

// Decode one 16-weight group word into 4 dwords of int8 weights in k order
// (dword i = weights 4i .. 4i+3, held in field i of bytes 0..3): 9 VALU ops.
__device__ __forceinline__ v4i decode_word(uint32_t word) {
  const uint32_t hi = word >> 4;
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(0u, kLutLo, word & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(kLutHiS0, kLutHiS1, word & 0x0C0C0C0Cu);
  r.z = (int)__builtin_amdgcn_perm(0u, kLutLo, hi & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(kLutHiS0, kLutHiS1, hi & 0x0C0C0C0Cu);
  return r;
}

// Ternary value of weight o of a group of b bytes starting at p (generic,
// byte-wise; used only on shapes off the fast paths).
__device__ __forceinline__ int decode_one(const uint8_t* p, int b, int o) {
  const uint32_t f = (p[o % b] >> (2 * (o / b))) & 3u;
  return f == 1u ? 1 : (f == 2u ? -1 : 0);
}

// fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Dequantize an exact accumulator: fl32(fl32(acc) * c) with c = fl32(gamma*d).
__device__ __forceinline__ float dequant(int acc, float c) {
  return __fmul_rn((float)acc, c);
}

// Per-token absmax int8 quantization arithmetic, shared by bl_quantize_act and
// the fused decode kernel so both produce identical codes:
//   max of |x| taken on bf16 magnitude bits (for finite values the bit order of
//   |x| is the value order); s = fl32(127 / m); q = clamp(rne(fl32(x * s)), +-127).
__device__ __forceinline__ uint32_t absmax4_bf16(uint2 v) {
  const uint32_t a = v.x & 0x7FFF7FFFu, b = v.y & 0x7FFF7FFFu;
  return max(max(a & 0xFFFFu, a >> 16), max(b & 0xFFFFu, b >> 16));
}

__device__ __forceinline__ uint32_t quant1_bf16(uint32_t bf16bits, float s) {
  const float x = __uint_as_float(bf16bits << 16);
  float r = rintf(__fmul_rn(x, s));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)r;
}

// 4 bf16 -> 4 int8 packed little-endian in a 32-bit word.
__device__ __forceinline__ uint32_t quant4_bf16(uint2 v, float s) {
  return quant1_bf16(v.x & 0xFFFFu, s) | (quant1_bf16(v.x >> 16, s) << 8) |
         (quant1_bf16(v.y & 0xFFFFu, s) << 16) | (quant1_bf16(v.y >> 16, s) << 24);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace bl
