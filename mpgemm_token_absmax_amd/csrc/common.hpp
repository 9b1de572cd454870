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

typedef __attribute__((address_space(3))) void lds_void;

// One 16-byte direct-to-LDS load per lane (global_load_lds_dwordx4): lane l
// writes dst + 16*l, dst is wave-uniform. A plain function, so that no kernel
// template instantiates the device-only builtin itself (clang's host pass
// rejects a second template instantiation that reaches it).
__device__ __forceinline__ void lds_dma16(const void* src, int8_t* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_void*)dst, 16, 0, 0);
}

// Wait until at most n vector-memory operations of this wave are outstanding.
template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] (7 = no wait) | lgkmcnt[11:8] (15) | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
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

// Max of the 8 bf16 magnitudes of a 16-byte chunk (packed 16-bit max).
__device__ __forceinline__ uint32_t absmax8_bf16(uint4 v) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  const u16x2 a = __builtin_bit_cast(u16x2, v.x & 0x7FFF7FFFu);
  const u16x2 b = __builtin_bit_cast(u16x2, v.y & 0x7FFF7FFFu);
  const u16x2 c = __builtin_bit_cast(u16x2, v.z & 0x7FFF7FFFu);
  const u16x2 d = __builtin_bit_cast(u16x2, v.w & 0x7FFF7FFFu);
  const u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b),
                                            __builtin_elementwise_max(c, d));
  return max((uint32_t)m.x, (uint32_t)m.y);
}

// The int8 code of one bf16 value as the low byte of fl32(fl32(x*s) + 1.5*2^23):
// for |y| < 2^22, adding 1.5*2^23 rounds y to an integer with ties to even and
// leaves it in the low mantissa bits (two's complement, so the low byte is
// the int8 code). With s = fl32(127/m) and |x| <= m, |fl32(x*s)| < 127.5, so
// the clamp to +-127 of the definition never binds: identical to quant1_bf16.
__device__ __forceinline__ uint32_t qbits_bf16(uint32_t bf16_in_high_half, float s) {
  return __float_as_uint(__fadd_rn(__fmul_rn(__uint_as_float(bf16_in_high_half), s),
                                   12582912.0f));
}

// 8 bf16 (16 bytes) -> 8 int8 codes (8 bytes), same codes as quant4_bf16.
__device__ __forceinline__ uint2 quant8_bf16(uint4 v, float s) {
  uint32_t w[4];
  const uint32_t in[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t lo = qbits_bf16(in[i] << 16, s);
    const uint32_t hi = qbits_bf16(in[i] & 0xFFFF0000u, s);
    w[i] = __builtin_amdgcn_perm(hi, lo, 0x0C0C0400u);     // bytes: lo.b0, hi.b0, 0, 0
  }
  return make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                    __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
}

// Max over the wave of a value held by every lane (all lanes active): DPP
// within each row of 16 lanes, then the four row results through SGPRs.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  int x = (int)v;
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));   // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));   // row_mirror
  const int r0 = __builtin_amdgcn_readlane(x, 0), r1 = __builtin_amdgcn_readlane(x, 16);
  const int r2 = __builtin_amdgcn_readlane(x, 32), r3 = __builtin_amdgcn_readlane(x, 48);
  return (uint32_t)max(max(r0, r1), max(r2, r3));
}

// ---- residual add + RMSNorm + quantize arithmetic, shared by the fused norm
// kernel and the one-token decode kernel with the norm folded in. Per token:
//   h = bf16_rne(fl32(x + r)); ms = fl32(S / K) with S = sum h^2 exactly (one
//   rounding); rinv = fl32(1/fl32(sqrt(fl32(ms + eps)))); y = fl32(fl32(h*rinv)*g).

// Two packed bf16 sums: bf16_rne(fl32(x + r)) per half.
__device__ __forceinline__ uint32_t add2_bf16(uint32_t x, uint32_t r) {
  const float lo = __fadd_rn(__uint_as_float(x << 16), __uint_as_float(r << 16));
  const float hi = __fadd_rn(__uint_as_float(x & 0xFFFF0000u), __uint_as_float(r & 0xFFFF0000u));
  return (uint32_t)f32_to_bf16_rne(lo) | ((uint32_t)f32_to_bf16_rne(hi) << 16);
}

__device__ __forceinline__ double sumsq2_bf16(uint32_t w, double acc) {
  const double lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
  acc += lo * lo;    // exact product; one fp64 rounding per add
  acc += hi * hi;
  return acc;
}

// The mean square ms = fl32(S / K), fast path. tot is an fp64 sum of the exact
// squares in any order, so |tot - S| <= (K-1) * 2^-53 * S (every term is >= 0);
// qv = fl64(tot / K) adds one rounding, so qv is within (K+1) * 2^-53 * qv of
// S / K (to first order). When qv lies farther than (K+2) * 2^-52 * qv from
// both fp32 rounding midpoints next to fl32(qv), S / K is on the same side of
// them and rounds to the same fp32 value: returns true with *ms = fl32(qv).
// Otherwise (about K * 2^-27 of random tokens) the caller computes ms from the
// exact bins below. tot == 0 means S == 0 (no square of a nonzero bf16
// underflows fp64).
__device__ __forceinline__ bool ms_fast(double tot, int64_t K, float* ms) {
  const double qv = tot / (double)K;
  const float f = (float)qv;
  *ms = f;
  if (tot == 0.0) return true;
  const uint32_t u = __float_as_uint(f);
  const double fd = (double)f;
  const double flo = u ? (double)__uint_as_float(u - 1u) : -(double)__uint_as_float(1u);
  const double fhi = (double)__uint_as_float(u + 1u);
  const double tol = (double)(K + 2) * 0x1p-52 * qv;
  return qv - 0.5 * (fd + flo) > tol && 0.5 * (fd + fhi) - qv > tol;
}

// Exact path: bins[b] (256 uint64 in LDS, zeroed) collects s^2 of every h =
// s * 2^(b - 134) of the row, with b the bf16 exponent field (1 for
// subnormals) and s the significand with its hidden bit (s < 256), so that
// S = 2^-268 * sum_b bins[b] * 4^b exactly. Two bf16 values per call.
__device__ __forceinline__ void sq_bins_add2(uint32_t w, unsigned long long* bins) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t v = i ? (w >> 16) : (w & 0xFFFFu);
    const uint32_t e = (v >> 7) & 0xFFu, m = v & 0x7Fu;
    if (e | m) {
      const uint32_t s = e ? (m | 0x80u) : m;
      atomicAdd(&bins[e ? e : 1u], (unsigned long long)(s * s));
    }
  }
}

// The rare exact path in two parts. First every thread of the block takes
// whole bins b (tid, tid + NT, ...) and adds bins[b] * 4^b, a value below
// 2^(2b + 64), into 64-bit column sums of 32-bit words: cols[j] collects bits
// 32j .. 32j+31 of each term (at most 3 words per term, each word < 2^32, at
// most 256 terms a column: no overflow). Then one thread propagates the
// carries, so that W holds T = sum_b bins[b] * 4^b as a 640-bit integer.
__device__ __forceinline__ void bins_to_cols(const unsigned long long* bins,
                                             unsigned long long* cols, int tid, int nt) {
  for (int b = tid; b < 256; b += nt) {
    const unsigned long long v = bins[b];
    if (b == 0 || !v) continue;
    const int w = b >> 4, sh = 2 * (b & 15);           // bit offset 2b = 32w + sh
    const unsigned long long lo = v << sh;
    const uint32_t hi = sh ? (uint32_t)(v >> (64 - sh)) : 0u;
    atomicAdd(&cols[w], (unsigned long long)(uint32_t)lo);
    atomicAdd(&cols[w + 1], lo >> 32);
    if (hi) atomicAdd(&cols[w + 2], (unsigned long long)hi);
  }
}

// fl32(S / K) from the column sums (one thread). W (20 words of LDS, so the
// hot kernels keep no private array) receives T with its carries; A = the
// top 64 bits of T (T = A * 2^L + rest), X = floor(A / K); S / K = X *
// 2^(L - 268) plus a positive part below one unit of X exactly when rest or
// A mod K is nonzero (the sticky bit). X has at least 46 significant bits, so
// one round to nearest even at the fp32 position (subnormals included) with
// that sticky bit gives the correctly rounded quotient.
__device__ __forceinline__ float ms_from_cols(const unsigned long long* cols, uint32_t* W,
                                              int64_t K) {
  unsigned long long c = 0;
  for (int j = 0; j < 20; ++j) {
    c += cols[j];
    W[j] = (uint32_t)c;
    c >>= 32;
  }
  int top = 19;
  while (top >= 0 && W[top] == 0u) --top;
  if (top < 0) return 0.0f;
  const int P = 32 * top + 31 - __builtin_clz(W[top]);      // top set bit of T
  const int L = P - 63;
  unsigned long long A;
  bool sticky = false;
  if (L <= 0) {                                              // T < 2^64: exact
    const unsigned long long T = ((unsigned long long)W[1] << 32) | W[0];
    A = T << (-L);
  } else {
    const int j0 = L >> 5, sh = L & 31;
    const uint32_t w2 = j0 + 2 < 20 ? W[j0 + 2] : 0u;
    const unsigned long long lo64 = ((unsigned long long)W[j0 + 1] << 32) | W[j0];
    A = sh ? ((lo64 >> sh) | ((unsigned long long)w2 << (64 - sh))) : lo64;
    sticky = (W[j0] & ((1u << sh) - 1u)) != 0u;
    for (int j = 0; j < j0; ++j) sticky = sticky || W[j] != 0u;
  }
  // X = A / K and the remainder by binary long division (few registers: this
  // path shares its kernel's register budget)
  const unsigned long long Ku = (unsigned long long)K;
  unsigned long long X = 0, rem = 0;
  for (int i = 63; i >= 0; --i) {
    rem = (rem << 1) | ((A >> i) & 1u);
    X <<= 1;
    if (rem >= Ku) {
      rem -= Ku;
      X |= 1u;
    }
  }
  sticky = sticky || rem != 0u;
  const int ex = 63 - __builtin_clzll(X);                    // X >= 2^63 / K > 0
  int lsb = ex + L - 268 - 23;                               // fp32 unit of a normal result
  if (lsb < -149) lsb = -149;
  const int sh2 = lsb - (L - 268);                           // bits of X below that unit
  unsigned long long keep;
  if (sh2 > 64) {
    keep = 0;                                                // below half the smallest unit
  } else if (sh2 == 64) {
    const unsigned long long half = 1ull << 63;
    keep = (X > half || (X == half && sticky)) ? 1u : 0u;
  } else {
    keep = X >> sh2;
    const unsigned long long rem = X & ((1ull << sh2) - 1ull), half = 1ull << (sh2 - 1);
    if (rem > half || (rem == half && (sticky || (keep & 1u)))) ++keep;
  }
  return (float)ldexp((double)keep, lsb);
}

// LDS of the exact path: the exponent bins, the 640-bit sum and the result.
struct MsScratch {
  unsigned long long bins[256];
  unsigned long long cols[20];
  uint32_t words[20];
  float ms;
};

// ms of a row from its fp64 sum of squares tot: the fast path when it is
// certain, else the exact bins (sc: LDS; add_own(bins) adds the calling
// thread's values with sq_bins_add2). Every thread of the block must call it
// with the same tot (the branch is uniform).
template <int NT, class F>
__device__ __forceinline__ float mean_square(double tot, int64_t K, MsScratch* sc, F add_own) {
  float ms;
  if (ms_fast(tot, K, &ms)) return ms;
  for (int i = (int)threadIdx.x; i < 256; i += NT) sc->bins[i] = 0ull;
  for (int i = (int)threadIdx.x; i < 20; i += NT) sc->cols[i] = 0ull;
  __syncthreads();
  add_own(sc->bins);
  __syncthreads();
  bins_to_cols(sc->bins, sc->cols, (int)threadIdx.x, NT);
  __syncthreads();
  if (threadIdx.x == 0) sc->ms = ms_from_cols(sc->cols, sc->words, K);
  __syncthreads();
  return sc->ms;
}

// rinv = fl32(1/fl32(sqrt(fl32(ms + eps)))), 0 when ms + eps is 0. sqrt and
// 1/x run in fp64 and are rounded once to fp32, which is the correctly rounded
// fp32 result (fp64 carries more than 2*24 + 2 bits).
__device__ __forceinline__ float norm_rinv(float ms, float eps) {
  const float v = __fadd_rn(ms, eps);
  if (!(v > 0.0f)) return 0.0f;
  const float root = (float)__dsqrt_rn((double)v);
  return (float)__ddiv_rn(1.0, (double)root);
}

__device__ __forceinline__ float norm1(uint32_t h_high, float rinv, uint32_t g_high) {
  return __fmul_rn(__fmul_rn(__uint_as_float(h_high), rinv), __uint_as_float(g_high));
}

// int8 code of fp32 y: low byte of fl32(fl32(y*s) + 1.5*2^23); |y| <= m and
// s = fl32(127/m) keep |fl32(y*s)| < 127.5, so it is rne(y*s) in [-127, 127].
__device__ __forceinline__ uint32_t qbits_f32(float y, float s) {
  return __float_as_uint(__fadd_rn(__fmul_rn(y, s), 12582912.0f));
}

// Four fp32 values -> four int8 codes packed little-endian.
__device__ __forceinline__ uint32_t quant4_f32(const float* y, float s) {
  const uint32_t a = __builtin_amdgcn_perm(qbits_f32(y[1], s), qbits_f32(y[0], s), 0x0C0C0400u);
  const uint32_t b = __builtin_amdgcn_perm(qbits_f32(y[3], s), qbits_f32(y[2], s), 0x0C0C0400u);
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// y of the 8 values of a 16-byte chunk (h and g as packed bf16 pairs).
__device__ __forceinline__ void norm8(uint4 h, uint4 g, float rinv, float* y) {
  const uint32_t hw[4] = {h.x, h.y, h.z, h.w};
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    y[2 * j] = norm1(hw[j] << 16, rinv, gw[j] << 16);
    y[2 * j + 1] = norm1(hw[j] & 0xFFFF0000u, rinv, gw[j] & 0xFFFF0000u);
  }
}

__device__ __forceinline__ uint32_t absbits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// Max over a block of kThreads threads (every thread gets it); red: one word
// per wave in LDS.
template <int kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
  __syncthreads();
  uint32_t m = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) m = max(m, red[w]);
  return m;
}

// Sum over a block of per-thread int32 values (exact), one int32 slot per
// wave in LDS.
template <int kThreads>
__device__ __forceinline__ int block_sum_i32(int v, int* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
  __syncthreads();
  int t = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) t += red[w];
  return t;
}

// acc + the sum of the four int8 codes packed in w (exact).
__device__ __forceinline__ int code_sum4(uint32_t w, int acc) {
  return __builtin_amdgcn_sdot4((int)w, 0x01010101, acc, false);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

}  // namespace bl
