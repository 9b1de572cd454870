// Absmean ternarization and I2_S packing (gfx950). Offline conversion: not on
// the per-token path.
//
// Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 (I2_S: 2 bits per weight, one scale per tensor);
// FairyFuse article, "三元量化方案" (w > 0.5a -> +1, w < -0.5a -> -1, else 0)
// and "融合内核设计" (codes 00/01/10 = 0/+1/-1). The scale a is BitNet
// b1.58's absmean gamma = mean |W| over the whole matrix.
//
// gamma must be bit-reproducible because a one-ulp change flips the weights
// that sit on the threshold. It is computed from the EXACT sum of |w|:
//   1. k_absmean_bins: every |w| (fp32) is mant * 2^(e-150) with a 24-bit
//      integer mant; each workgroup adds mant into a 64-bit LDS bin per
//      exponent e (integer adds: order free, no rounding) and writes its 256
//      bins to the workspace. n < 2^39 elements cannot overflow a bin.
//   2. k_gamma_finalize: one workgroup sums the bins over workgroups, one
//      thread carries them into a 384-bit integer V (sum = V * 2^-149),
//      rounds V to the nearest fp64 (ties to even), divides by n in fp64 and
//      rounds to fp32.
//   3. k_ternarize_pack: t = 0.5f * gamma; codes; one 32-bit group word per
//      thread (K % 16 == 0) or one byte per thread (other K).
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kLimbs = 6;

__device__ __forceinline__ void add_bin(unsigned long long* bins, uint32_t bits) {
  const uint32_t u = bits & 0x7FFFFFFFu;
  if (u == 0u) return;
  const uint32_t e = u >> 23;
  const uint32_t mant = e ? ((u & 0x7FFFFFu) | 0x800000u) : u;
  atomicAdd(&bins[e ? e : 1u], (unsigned long long)mant);
}

__global__ __launch_bounds__(kBinThreads) void k_absmean_bins(const float4* __restrict__ w,
                                                              int64_t n4,
                                                              unsigned long long* __restrict__ ws) {
  __shared__ unsigned long long bins[kBins];
  bins[threadIdx.x] = 0ull;
  __syncthreads();
  const int64_t stride = (int64_t)gridDim.x * kBinThreads;
  for (int64_t c = (int64_t)blockIdx.x * kBinThreads + threadIdx.x; c < n4; c += stride) {
    const float4 v = w[c];
    add_bin(bins, __float_as_uint(v.x));
    add_bin(bins, __float_as_uint(v.y));
    add_bin(bins, __float_as_uint(v.z));
    add_bin(bins, __float_as_uint(v.w));
  }
  __syncthreads();
  ws[(int64_t)blockIdx.x * kBins + threadIdx.x] = bins[threadIdx.x];
}

__device__ void limb_add(uint64_t* limb, int i, uint64_t x) {
  while (x && i < kLimbs) {
    const uint64_t old = limb[i];
    limb[i] = old + x;
    x = limb[i] < old ? 1ull : 0ull;
    ++i;
  }
}

__global__ __launch_bounds__(kBins) void k_gamma_finalize(const unsigned long long* __restrict__ ws,
                                                          int nblk, int64_t n,
                                                          float* __restrict__ gamma) {
  __shared__ unsigned long long tot[kBins];
  unsigned long long s = 0ull;
  for (int b = 0; b < nblk; ++b) s += ws[(int64_t)b * kBins + threadIdx.x];
  tot[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint64_t limb[kLimbs] = {0, 0, 0, 0, 0, 0};
  for (int e = 1; e < kBins; ++e) {          // bin e holds mantissas scaled by 2^(e-150)
    const uint64_t v = tot[e];
    if (!v) continue;
    const int sh = e - 1;                   // V counts units of 2^-149
    const int li = sh >> 6, off = sh & 63;
    limb_add(limb, li, v << off);
    if (off) limb_add(limb, li + 1, v >> (64 - off));
  }
  int top = -1;
  for (int i = kLimbs - 1; i >= 0; --i)
    if (limb[i]) { top = i; break; }
  if (top < 0) { gamma[0] = 0.0f; return; }
  int p = 64 * top + 63 - __clzll((long long)limb[top]);   // position of the leading 1
  uint64_t mant;
  bool rb = false, st = false;
  if (p <= 52) {
    mant = limb[0];                          // exact
  } else {
    const int low = p - 63;                  // bit position of the window's lsb
    uint64_t win;
    bool below = false;
    if (low < 0) {
      win = limb[0] << (-low);
    } else {
      const int li = low >> 6, off = low & 63;
      win = limb[li] >> off;
      if (off) win |= (li + 1 < kLimbs ? limb[li + 1] : 0ull) << (64 - off);
      if (off) below = (limb[li] & ((1ull << off) - 1ull)) != 0ull;
      for (int i = 0; i < li; ++i) below = below || limb[i] != 0ull;
    }
    mant = win >> 11;                        // 53 significant bits
    rb = ((win >> 10) & 1ull) != 0ull;
    st = below || (win & 0x3FFull) != 0ull;
  }
  int e2 = (p <= 52) ? -149 : p - 52 - 149;
  if (rb && (st || (mant & 1ull))) {
    ++mant;
    if (mant >> 53) { mant >>= 1; ++e2; }
  }
  const double sum = ldexp((double)mant, e2);
  gamma[0] = (float)(sum / (double)n);
}

__device__ __forceinline__ uint32_t code_f32(float v, float t) {
  return v > t ? 1u : (v < -t ? 2u : 0u);
}
__device__ __forceinline__ uint32_t code_i8(int v) {
  return v > 0 ? 1u : (v < 0 ? 2u : 0u);
}

// K % 16 == 0: the flat packed array is a sequence of full group words.
__global__ void k_pack_f32_words(const float4* __restrict__ w, int64_t nwords,
                                 const float* __restrict__ gamma, uint32_t* __restrict__ out) {
  const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= nwords) return;
  const float t = 0.5f * gamma[0];
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {               // weights 4i .. 4i+3 -> field i of bytes 0..3
    const float4 f = w[4 * wi + i];
    word |= code_f32(f.x, t) << (2 * i);
    word |= code_f32(f.y, t) << (8 + 2 * i);
    word |= code_f32(f.z, t) << (16 + 2 * i);
    word |= code_f32(f.w, t) << (24 + 2 * i);
  }
  out[wi] = word;
}

__global__ void k_pack_i8_words(const uint4* __restrict__ w, int64_t nwords,
                                uint32_t* __restrict__ out) {
  const int64_t wi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (wi >= nwords) return;
  const uint4 v = w[wi];
  const uint32_t c[4] = {v.x, v.y, v.z, v.w};
  uint32_t word = 0u;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      word |= code_i8((int)(int8_t)(c[i] >> (8 * j))) << (8 * j + 2 * i);
  out[wi] = word;
}

// Any K % 4 == 0: one output byte per thread, weights located by the group rule.
template <bool F32>
__global__ void k_pack_bytes(const void* __restrict__ wv, int64_t N, int64_t K,
                             const float* __restrict__ gamma, uint8_t* __restrict__ out) {
  const int64_t RB = K / 4;
  const int64_t bi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (bi >= N * RB) return;
  const int64_t n = bi / RB, jb = bi % RB;
  const int64_t g = jb / 4;
  const int64_t b = min((int64_t)4, RB - 4 * g);
  const int64_t j = jb - 4 * g;
  const float t = F32 ? 0.5f * gamma[0] : 0.0f;
  uint32_t byte = 0u;
  for (int i = 0; i < 4; ++i) {
    const int64_t k = 16 * g + i * b + j;
    uint32_t c;
    if constexpr (F32) c = code_f32(static_cast<const float*>(wv)[n * K + k], t);
    else c = code_i8(static_cast<const int8_t*>(wv)[n * K + k]);
    byte |= c << (2 * i);
  }
  out[bi] = (uint8_t)byte;
}

unsigned grid_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_absmean_gamma(const float* w, int64_t N, int64_t K, float* gamma, void* ws,
                                hipStream_t s) {
  const int64_t n = N * K;
  const int64_t nblk = bin_blocks(n);
  auto* bins = static_cast<unsigned long long*>(ws);
  hipLaunchKernelGGL(k_absmean_bins, dim3((unsigned)nblk), dim3(kBinThreads), 0, s,
                     reinterpret_cast<const float4*>(w), n / 4, bins);
  hipLaunchKernelGGL(k_gamma_finalize, dim3(1), dim3(kBins), 0, s, bins, (int)nblk, n, gamma);
  return hipGetLastError();
}

hipError_t launch_pack_f32(const float* w, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           void* ws, hipStream_t s) {
  const int64_t n = N * K;
  const hipError_t e = launch_absmean_gamma(w, N, K, gamma, ws, s);
  if (e != hipSuccess) return e;
  if (K % 16 == 0) {
    const int64_t nw = n / 16;
    hipLaunchKernelGGL(k_pack_f32_words, dim3(grid_for(nw, 256)), dim3(256), 0, s,
                       reinterpret_cast<const float4*>(w), nw, gamma,
                       reinterpret_cast<uint32_t*>(packed));
  } else {
    hipLaunchKernelGGL(k_pack_bytes<true>, dim3(grid_for(N * (K / 4), 256)), dim3(256), 0, s,
                       static_cast<const void*>(w), N, K, gamma, packed);
  }
  return hipGetLastError();
}

hipError_t launch_pack_ternary(const int8_t* w, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t s) {
  if (K % 16 == 0) {
    const int64_t nw = N * K / 16;
    hipLaunchKernelGGL(k_pack_i8_words, dim3(grid_for(nw, 256)), dim3(256), 0, s,
                       reinterpret_cast<const uint4*>(w), nw, reinterpret_cast<uint32_t*>(packed));
  } else {
    hipLaunchKernelGGL(k_pack_bytes<false>, dim3(grid_for(N * (K / 4), 256)), dim3(256), 0, s,
                       static_cast<const void*>(w), N, K, static_cast<const float*>(nullptr),
                       packed);
  }
  return hipGetLastError();
}

}  // namespace bl
