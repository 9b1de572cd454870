// Per-token absmax int8 activation quantization (gfx950).
//
// Source: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 / 4.1: the ternary weights meet int8 activations that
// carry one scale per vector (not per block). Per token t (one row of x):
//   m = max |x[t][:]|, s = fl32(127/m), q = clamp(rne(fl32(x*s)), -127, 127),
//   d[t] = fl32(m/127); an all-zero row gives q = 0, d = 0.
//
// One workgroup of 256 threads per token. Each thread reads 8 bf16 (16 bytes,
// when K and ldx are multiples of 8) or 4 bf16 per chunk; up to 32768 values
// the row stays in registers between the max and the quantize pass,
// otherwise the second pass re-reads it (an L2 hit).
// The max is taken on the magnitude bits: for finite values the ordering of
// the bit patterns of |x| is the ordering of the values.
// Optionally (qs != nullptr) each row also gets the exact int32 sum of its
// codes, qs[t] = sum_k q[t][k], which lets the GEMM run on offset weights.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kQThreads = 256;

// NC > 0: row cached in registers (K <= 1024*NC). NC == 0: two passes over x.
template <int NC>
__global__ __launch_bounds__(kQThreads) void k_quant_absmax(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    float* __restrict__ d, int* __restrict__ qs) {
  __shared__ uint32_t red[kQThreads / kWave];
  __shared__ int red_q[kQThreads / kWave];
  const int64_t t = blockIdx.x;
  const uint2* xr = reinterpret_cast<const uint2*>(x + t * ldx);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + t * K);
  const int64_t nchunk = K / 4;
  uint32_t mb = 0;
  int sum = 0;
  if constexpr (NC > 0) {
    uint2 v[NC];
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * kQThreads;
      v[i] = c < nchunk ? xr[c] : make_uint2(0u, 0u);
      mb = max(mb, absmax4_bf16(v[i]));
    }
    mb = block_max_u32<kQThreads>(mb, red);
    const float m = __uint_as_float(mb << 16);
    const float s = mb ? 127.0f / m : 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int64_t c = threadIdx.x + (int64_t)i * kQThreads;
      if (c < nchunk) {
        const uint32_t w = mb ? quant4_bf16(v[i], s) : 0u;
        qr[c] = w;
        sum = code_sum4(w, sum);
      }
    }
    if (threadIdx.x == 0) d[t] = mb ? m / 127.0f : 0.0f;
  } else {
    for (int64_t c = threadIdx.x; c < nchunk; c += kQThreads) mb = max(mb, absmax4_bf16(xr[c]));
    mb = block_max_u32<kQThreads>(mb, red);
    const float m = __uint_as_float(mb << 16);
    const float s = mb ? 127.0f / m : 0.0f;
    for (int64_t c = threadIdx.x; c < nchunk; c += kQThreads) {
      const uint32_t w = mb ? quant4_bf16(xr[c], s) : 0u;
      qr[c] = w;
      sum = code_sum4(w, sum);
    }
    if (threadIdx.x == 0) d[t] = mb ? m / 127.0f : 0.0f;
  }
  if (qs) {
    sum = block_sum_i32<kQThreads>(sum, red_q);
    if (threadIdx.x == 0) qs[t] = sum;
  }
}

// 16-byte variant (K % 8 == 0, ldx % 8 == 0): 8 bf16 per chunk, the row in
// registers (K <= 2048*NC). Loads are unconditional (chunk index clamped, the
// value of a chunk past the row ignored) so they are all in flight at once.
// given_max: nullptr -> the row's own absmax (per token); else the absmax
// bits to use (per tensor, the same for every row). qst: nullptr, or where
// the sum of the row's codes goes (red_q: its reduction slots).
template <int NC>
__device__ __forceinline__ void quant_row16(const uint16_t* __restrict__ xrow, int64_t K,
                                            int8_t* __restrict__ qrow, float* __restrict__ dt,
                                            uint32_t* red, const uint32_t* given_max,
                                            int* qst, int* red_q) {
  const uint4* xr = reinterpret_cast<const uint4*>(xrow);
  uint2* qr = reinterpret_cast<uint2*>(qrow);
  const int nchunk = (int)(K / 8);
  uint4 v[NC];
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (int)threadIdx.x + i * kQThreads;
    v[i] = xr[c < nchunk ? c : nchunk - 1];
  }
  uint32_t mb = 0;
  if (given_max) {
    mb = *given_max;
  } else {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      const int c = (int)threadIdx.x + i * kQThreads;
      const uint32_t m8 = max(absmax4_bf16(make_uint2(v[i].x, v[i].y)),
                              absmax4_bf16(make_uint2(v[i].z, v[i].w)));
      mb = max(mb, c < nchunk ? m8 : 0u);
    }
    mb = block_max_u32<kQThreads>(mb, red);
  }
  const float m = __uint_as_float(mb << 16);
  const float s = mb ? 127.0f / m : 0.0f;
  int sum = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (int)threadIdx.x + i * kQThreads;
    if (c < nchunk) {
      const uint2 w = mb ? make_uint2(quant4_bf16(make_uint2(v[i].x, v[i].y), s),
                                      quant4_bf16(make_uint2(v[i].z, v[i].w), s))
                         : make_uint2(0u, 0u);
      qr[c] = w;
      sum = code_sum4(w.y, code_sum4(w.x, sum));
    }
  }
  if (threadIdx.x == 0) *dt = mb ? m / 127.0f : 0.0f;
  if (qst) {
    sum = block_sum_i32<kQThreads>(sum, red_q);
    if (threadIdx.x == 0) *qst = sum;
  }
}

template <int NC>
__global__ __launch_bounds__(kQThreads) void k_quant_absmax16(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, int8_t* __restrict__ q,
    float* __restrict__ d, int* __restrict__ qs) {
  __shared__ uint32_t red[kQThreads / kWave];
  __shared__ int red_q[kQThreads / kWave];
  const int64_t t = blockIdx.x;
  quant_row16<NC>(x + t * ldx, K, q + t * K, d + t, red, nullptr, qs ? qs + t : nullptr, red_q);
}

// Every problem of a decode group at once: grid x = token, y = problem; each
// problem's x [M][ldx] goes to its q [M][K] and d [M].
template <int NC>
__global__ __launch_bounds__(kQThreads) void k_quant_group(DecodeGroup g) {
  __shared__ uint32_t red[kQThreads / kWave];
  const DecodeProblem& P = g.p[blockIdx.y];
  const int64_t t = blockIdx.x;
  quant_row16<NC>(P.x + t * P.ldx, P.K, P.q + t * P.K, P.d + t, red, nullptr, nullptr, nullptr);
}

// ---- one scale for the whole tensor: row maxima first, then quantize -----

// Absmax bits of each row (any K % 4 == 0): maxb[t] = max_k |x[t][k]| bits.
__global__ __launch_bounds__(kQThreads) void k_row_absmax(const uint16_t* __restrict__ x,
                                                          int64_t K, int64_t ldx,
                                                          uint32_t* __restrict__ maxb) {
  __shared__ uint32_t red[kQThreads / kWave];
  const int64_t t = blockIdx.x;
  const uint2* xr = reinterpret_cast<const uint2*>(x + t * ldx);
  uint32_t mb = 0;
  for (int64_t c = threadIdx.x; c < K / 4; c += kQThreads) mb = max(mb, absmax4_bf16(xr[c]));
  mb = block_max_u32<kQThreads>(mb, red);
  if (threadIdx.x == 0) maxb[t] = mb;
}

// The tensor's absmax bits from the M row maxima (every block reads them all).
__device__ __forceinline__ uint32_t tensor_absmax(const uint32_t* __restrict__ maxb, int64_t M,
                                                  uint32_t* red) {
  uint32_t mb = 0;
  for (int64_t i = threadIdx.x; i < M; i += kQThreads) mb = max(mb, maxb[i]);
  return block_max_u32<kQThreads>(mb, red);
}

template <int NC>
__global__ __launch_bounds__(kQThreads) void k_quant_tensor16(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, const uint32_t* __restrict__ maxb,
    int64_t M, int8_t* __restrict__ q, float* __restrict__ d, int* __restrict__ qs) {
  __shared__ uint32_t red[kQThreads / kWave];
  __shared__ uint32_t red2[kQThreads / kWave];
  __shared__ int red_q[kQThreads / kWave];
  const uint32_t mb = tensor_absmax(maxb, M, red);
  const int64_t t = blockIdx.x;
  quant_row16<NC>(x + t * ldx, K, q + t * K, d + t, red2, &mb, qs ? qs + t : nullptr, red_q);
}

// Any K % 4 == 0 and row stride: 4 values per chunk, the row read once.
__global__ __launch_bounds__(kQThreads) void k_quant_tensor_any(
    const uint16_t* __restrict__ x, int64_t K, int64_t ldx, const uint32_t* __restrict__ maxb,
    int64_t M, int8_t* __restrict__ q, float* __restrict__ d, int* __restrict__ qs) {
  __shared__ uint32_t red[kQThreads / kWave];
  __shared__ int red_q[kQThreads / kWave];
  const uint32_t mb = tensor_absmax(maxb, M, red);
  const int64_t t = blockIdx.x;
  const uint2* xr = reinterpret_cast<const uint2*>(x + t * ldx);
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + t * K);
  const float m = __uint_as_float(mb << 16);
  const float s = mb ? 127.0f / m : 0.0f;
  int sum = 0;
  for (int64_t c = threadIdx.x; c < K / 4; c += kQThreads) {
    const uint32_t w = mb ? quant4_bf16(xr[c], s) : 0u;
    qr[c] = w;
    sum = code_sum4(w, sum);
  }
  if (threadIdx.x == 0) d[t] = mb ? m / 127.0f : 0.0f;
  if (qs) {
    sum = block_sum_i32<kQThreads>(sum, red_q);
    if (threadIdx.x == 0) qs[t] = sum;
  }
}

// d[:] = 0 and, when given, qs[:] = 0 (the K == 0 case).
__global__ void k_fill_zero_dq(float* __restrict__ d, int* __restrict__ qs, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    d[i] = 0.0f;
    if (qs) qs[i] = 0;
  }
}

template <int NC>
hipError_t launch_nc(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, float* d,
                     int* qs, hipStream_t s) {
  hipLaunchKernelGGL(k_quant_absmax<NC>, dim3((unsigned)M), dim3(kQThreads), 0, s, x, K, ldx, q,
                     d, qs);
  return hipGetLastError();
}

template <int NC>
hipError_t launch_nc16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, float* d,
                       int* qs, hipStream_t s) {
  hipLaunchKernelGGL(k_quant_absmax16<NC>, dim3((unsigned)M), dim3(kQThreads), 0, s, x, K, ldx,
                     q, d, qs);
  return hipGetLastError();
}

template <int NC>
hipError_t launch_group_nc(const DecodeGroup& g, hipStream_t s) {
  hipLaunchKernelGGL(k_quant_group<NC>, dim3((unsigned)g.M, (unsigned)g.count), dim3(kQThreads), 0,
                     s, g);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_group(const DecodeGroup& g, hipStream_t s) {
  int64_t kmax = 0;
  bool wide = true;
  for (int i = 0; i < g.count; ++i) {
    kmax = g.p[i].K > kmax ? g.p[i].K : kmax;
    wide = wide && g.p[i].K % 8 == 0 && g.p[i].ldx % 8 == 0;
  }
  if (wide && kmax > 0 && kmax <= 2048 * 16) {
    const int64_t per_thread = (kmax / 8 + kQThreads - 1) / kQThreads;
    if (per_thread <= 1) return launch_group_nc<1>(g, s);
    if (per_thread <= 2) return launch_group_nc<2>(g, s);
    if (per_thread <= 4) return launch_group_nc<4>(g, s);
    if (per_thread <= 8) return launch_group_nc<8>(g, s);
    return launch_group_nc<16>(g, s);
  }
  for (int i = 0; i < g.count; ++i) {
    const DecodeProblem& p = g.p[i];
    const hipError_t e = launch_quantize_act(p.x, g.M, p.K, p.ldx, p.q, p.d, nullptr, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_quantize_act_tensor(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      int8_t* q, float* d, int* qs, uint32_t* maxb, hipStream_t s) {
  if (K == 0) {
    hipLaunchKernelGGL(k_fill_zero_dq, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, d, qs, M);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(k_row_absmax, dim3((unsigned)M), dim3(kQThreads), 0, s, x, K, ldx, maxb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (K % 8 == 0 && ldx % 8 == 0 && K <= 2048 * 16) {
    const int64_t per_thread = (K / 8 + kQThreads - 1) / kQThreads;
    const dim3 g((unsigned)M), b(kQThreads);
    if (per_thread <= 1) hipLaunchKernelGGL(k_quant_tensor16<1>, g, b, 0, s, x, K, ldx, maxb, M, q, d, qs);
    else if (per_thread <= 2) hipLaunchKernelGGL(k_quant_tensor16<2>, g, b, 0, s, x, K, ldx, maxb, M, q, d, qs);
    else if (per_thread <= 4) hipLaunchKernelGGL(k_quant_tensor16<4>, g, b, 0, s, x, K, ldx, maxb, M, q, d, qs);
    else if (per_thread <= 8) hipLaunchKernelGGL(k_quant_tensor16<8>, g, b, 0, s, x, K, ldx, maxb, M, q, d, qs);
    else hipLaunchKernelGGL(k_quant_tensor16<16>, g, b, 0, s, x, K, ldx, maxb, M, q, d, qs);
  } else {
    hipLaunchKernelGGL(k_quant_tensor_any, dim3((unsigned)M), dim3(kQThreads), 0, s, x, K, ldx, maxb,
                       M, q, d, qs);
  }
  return hipGetLastError();
}

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               float* d, int* qs, hipStream_t s) {
  if (K == 0) {
    hipLaunchKernelGGL(k_fill_zero_dq, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, d, qs, M);
    return hipGetLastError();
  }
  if (K % 8 == 0 && ldx % 8 == 0 && K <= 2048 * 16) {
    const int64_t per_thread = (K / 8 + kQThreads - 1) / kQThreads;
    if (per_thread <= 1) return launch_nc16<1>(x, M, K, ldx, q, d, qs, s);
    if (per_thread <= 2) return launch_nc16<2>(x, M, K, ldx, q, d, qs, s);
    if (per_thread <= 4) return launch_nc16<4>(x, M, K, ldx, q, d, qs, s);
    if (per_thread <= 8) return launch_nc16<8>(x, M, K, ldx, q, d, qs, s);
    return launch_nc16<16>(x, M, K, ldx, q, d, qs, s);
  }
  const int64_t per_thread = (K / 4 + kQThreads - 1) / kQThreads;
  if (per_thread <= 1) return launch_nc<1>(x, M, K, ldx, q, d, qs, s);
  if (per_thread <= 2) return launch_nc<2>(x, M, K, ldx, q, d, qs, s);
  if (per_thread <= 4) return launch_nc<4>(x, M, K, ldx, q, d, qs, s);
  if (per_thread <= 8) return launch_nc<8>(x, M, K, ldx, q, d, qs, s);
  if (per_thread <= 16) return launch_nc<16>(x, M, K, ldx, q, d, qs, s);
  if (per_thread <= 32) return launch_nc<32>(x, M, K, ldx, q, d, qs, s);
  return launch_nc<0>(x, M, K, ldx, q, d, qs, s);
}

}  // namespace bl
