// Residual add + RMSNorm fused with the per-token absmax int8 quantizer (gfx950).
//
// Source: BinaryAI Engine forum post, "关键技术机制解析" §2 (the residual add and
// the RMS normalization run as one pass over the activations) feeding the
// per-token absmax quantizer of the Bitnet.cpp reading notes, Part A 2.3 / 4.1.
// Per token t (row of x, r):
//   h  = bf16_rne(fl32(x + r))            (h = x without r; written to h_out)
//   ms = fl32(sum_k h^2 / K)
//   rinv = fl32(1 / fl32(sqrt(fl32(ms + eps))))
//   y  = fl32(fl32(h * rinv) * g)         (g: bf16 norm weight, one per feature)
//   m = max |y|, s = fl32(127 / m), q = rne(fl32(y * s)), d = fl32(m / 127);
//   q = 0 and d = 0 when m = 0 or fl32(ms + eps) = 0.
// Rounding: ms is the correctly rounded fp32 value of the exact mean square.
// The fp64 sum of the exact squares settles it when its error bound keeps it
// away from every fp32 rounding midpoint (all but about K * 2^-27 of random
// tokens); otherwise the block sums the squares exactly, as integers binned by
// exponent, and rounds that sum divided by K once. sqrt and 1/x run in fp64
// and are rounded once to fp32, which gives the correctly rounded fp32 result
// (fp64 carries more than 2*24 + 2 bits).
//
// One workgroup per token. Fast path (K % 8 == 0, ldx % 8 == 0, K <= 32768):
// each thread holds NC 16-byte chunks of the row in registers, so x, r and g
// are read once and h, q written once: 2K + 2K (+ 2K h) + K bytes per token.
// Other shapes: the generic kernel makes three passes over the row, the later
// two hitting L2.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

// Sum over a block of kThreads threads. The butterfly gives every lane of a
// wave the same value (fp addition is commutative), and every thread adds the
// wave partials in the same order, so the result is uniform.
template <int kThreads>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int wid = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[wid] = v;
  __syncthreads();
  double s = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) s += red[w];
  return s;
}

// 16 bytes at a uniform base plus a 32-bit byte offset (one SGPR base and a
// single VGPR offset per load, instead of a 64-bit address per load).
__device__ __forceinline__ uint4 ld16(const void* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(base) + off);
}


// Fast path. x, r and h_out are not __restrict__: h_out may be r or x itself
// (every chunk is loaded before the same thread stores it). Registers: the x
// and r chunks, then h and g; y is recomputed from them for the codes rather
// than kept, so the kernel stays at 8 waves per SIMD.
template <int NT, int NC, bool kRes>
__global__ __launch_bounds__(NT) void k_rmsnorm_quant16(
    const uint16_t* x, const uint16_t* r, const uint16_t* __restrict__ g, float eps, int64_t K,
    int64_t ldx, uint16_t* h_out, int8_t* __restrict__ q, float* __restrict__ d,
    int* __restrict__ qs) {
  __shared__ double red_s[NT / kWave];
  __shared__ uint32_t red_m[NT / kWave];
  __shared__ int red_q[NT / kWave];
  __shared__ MsScratch msx;
  const int64_t t = blockIdx.x;
  const int nchunk = (int)(K / 8);
  const uint16_t* xrow = x + t * ldx;
  const uint16_t* rrow = r + t * ldx;
  uint32_t off[NC];                         // byte offset of each chunk (clamped)
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const uint32_t c = threadIdx.x + (uint32_t)(i * NT);
    off[i] = 16u * (c < (uint32_t)nchunk ? c : (uint32_t)nchunk - 1u);
  }
  uint4 hv[NC], gv[NC];
  // Every x and r load issued before any use (a chunk past the row is
  // ignored below).
#pragma unroll
  for (int i = 0; i < NC; ++i) hv[i] = ld16(xrow, off[i]);
  uint4 rv[kRes ? NC : 1];
  if constexpr (kRes) {
#pragma unroll
    for (int i = 0; i < NC; ++i) rv[i] = ld16(rrow, off[i]);
  }
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (int)threadIdx.x + i * NT;
    if constexpr (kRes) {
      hv[i].x = add2_bf16(hv[i].x, rv[i].x);
      hv[i].y = add2_bf16(hv[i].y, rv[i].y);
      hv[i].z = add2_bf16(hv[i].z, rv[i].z);
      hv[i].w = add2_bf16(hv[i].w, rv[i].w);
      // h as opaque values: the compiler keeps these 4 registers instead of
      // x and r (8) to recompute them later
      asm volatile("" : "+v"(hv[i].x), "+v"(hv[i].y), "+v"(hv[i].z), "+v"(hv[i].w));
    }
    if (c < nchunk) {
      ss = sumsq2_bf16(hv[i].x, ss);
      ss = sumsq2_bf16(hv[i].y, ss);
      ss = sumsq2_bf16(hv[i].z, ss);
      ss = sumsq2_bf16(hv[i].w, ss);
      if (h_out) reinterpret_cast<uint4*>(h_out + t * ldx)[c] = hv[i];
    }
  }
  const float ms = mean_square<NT>(block_sum_f64<NT>(ss, red_s), K, &msx,
                                   [&](unsigned long long* b) {
#pragma unroll
    for (int i = 0; i < NC; ++i) {
      if ((int)threadIdx.x + i * NT < nchunk) {
        sq_bins_add2(hv[i].x, b);
        sq_bins_add2(hv[i].y, b);
        sq_bins_add2(hv[i].z, b);
        sq_bins_add2(hv[i].w, b);
      }
      __builtin_amdgcn_sched_barrier(0);    // one chunk at a time: few registers
    }
  });
  // g (the same for every token: an L2 hit) is loaded once the mean square
  // is known, so it holds no registers across the sum
#pragma unroll
  for (int i = 0; i < NC; ++i) gv[i] = ld16(g, off[i]);
  const float rinv = norm_rinv(ms, eps);
  uint32_t mb = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    float y[8];
    norm8(hv[i], gv[i], rinv, y);
    uint32_t m8 = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) m8 = max(m8, absbits(y[j]));
    const int c = (int)threadIdx.x + i * NT;
    mb = max(mb, c < nchunk ? m8 : 0u);
  }
  mb = block_max_u32<NT>(mb, red_m);
  const float m = __uint_as_float(mb);
  const float s = mb ? 127.0f / m : 0.0f;
  uint2* qr = reinterpret_cast<uint2*>(q + t * K);
  int sum = 0;
#pragma unroll
  for (int i = 0; i < NC; ++i) {
    const int c = (int)threadIdx.x + i * NT;
    if (c < nchunk) {
      float y[8];
      norm8(hv[i], gv[i], rinv, y);
      const uint2 w = mb ? make_uint2(quant4_f32(&y[0], s), quant4_f32(&y[4], s))
                         : make_uint2(0u, 0u);
      qr[c] = w;
      sum = code_sum4(w.y, code_sum4(w.x, sum));
    }
  }
  if (threadIdx.x == 0) d[t] = mb ? m / 127.0f : 0.0f;
  if (qs) {
    sum = block_sum_i32<NT>(sum, red_q);
    if (threadIdx.x == 0) qs[t] = sum;
  }
}

// Generic path (K % 4 == 0, ldx % 4 == 0): three passes of 4 values per chunk.
// Passes 2 and 3 read h back from h_out when it is given (h_out may be x or r),
// else recompute it from x and r.
constexpr int kGenThreads = 256;

__device__ __forceinline__ uint2 load_h4(const uint2* xr, const uint2* rr, int64_t c) {
  uint2 v = xr[c];
  if (rr) {
    const uint2 w = rr[c];
    v = make_uint2(add2_bf16(v.x, w.x), add2_bf16(v.y, w.y));
  }
  return v;
}

__device__ __forceinline__ void norm4(uint2 h, uint2 gw, float rinv, float* y) {
  y[0] = norm1(h.x << 16, rinv, gw.x << 16);
  y[1] = norm1(h.x & 0xFFFF0000u, rinv, gw.x & 0xFFFF0000u);
  y[2] = norm1(h.y << 16, rinv, gw.y << 16);
  y[3] = norm1(h.y & 0xFFFF0000u, rinv, gw.y & 0xFFFF0000u);
}

__global__ __launch_bounds__(kGenThreads) void k_rmsnorm_quant_any(
    const uint16_t* x, const uint16_t* r, const uint16_t* __restrict__ g, float eps, int64_t K,
    int64_t ldx, uint16_t* h_out, int8_t* __restrict__ q, float* __restrict__ d,
    int* __restrict__ qs) {
  __shared__ double red_s[kGenThreads / kWave];
  __shared__ uint32_t red_m[kGenThreads / kWave];
  __shared__ int red_q[kGenThreads / kWave];
  __shared__ MsScratch msx;
  const int64_t t = blockIdx.x;
  const int64_t nchunk = K / 4;
  const uint2* xr = reinterpret_cast<const uint2*>(x + t * ldx);
  const uint2* rr = r ? reinterpret_cast<const uint2*>(r + t * ldx) : nullptr;
  uint2* hr = h_out ? reinterpret_cast<uint2*>(h_out + t * ldx) : nullptr;
  const uint2* gr = reinterpret_cast<const uint2*>(g);
  double ss = 0.0;
  for (int64_t c = threadIdx.x; c < nchunk; c += kGenThreads) {
    const uint2 h = load_h4(xr, rr, c);
    ss = sumsq2_bf16(h.y, sumsq2_bf16(h.x, ss));
    if (hr) hr[c] = h;
  }
  const float ms = mean_square<kGenThreads>(
      block_sum_f64<kGenThreads>(ss, red_s), K, &msx, [&](unsigned long long* b) {
        for (int64_t c = threadIdx.x; c < nchunk; c += kGenThreads) {
          const uint2 h = hr ? hr[c] : load_h4(xr, rr, c);
          sq_bins_add2(h.x, b);
          sq_bins_add2(h.y, b);
        }
      });
  const float rinv = norm_rinv(ms, eps);
  uint32_t mb = 0;
  for (int64_t c = threadIdx.x; c < nchunk; c += kGenThreads) {
    float y[4];
    norm4(hr ? hr[c] : load_h4(xr, rr, c), gr[c], rinv, y);
    mb = max(max(mb, max(absbits(y[0]), absbits(y[1]))), max(absbits(y[2]), absbits(y[3])));
  }
  mb = block_max_u32<kGenThreads>(mb, red_m);
  const float m = __uint_as_float(mb);
  const float s = mb ? 127.0f / m : 0.0f;
  uint32_t* qr = reinterpret_cast<uint32_t*>(q + t * K);
  int sum = 0;
  for (int64_t c = threadIdx.x; c < nchunk; c += kGenThreads) {
    float y[4];
    norm4(hr ? hr[c] : load_h4(xr, rr, c), gr[c], rinv, y);
    const uint32_t w = mb ? quant4_f32(y, s) : 0u;
    qr[c] = w;
    sum = code_sum4(w, sum);
  }
  if (threadIdx.x == 0) d[t] = mb ? m / 127.0f : 0.0f;
  if (qs) {
    sum = block_sum_i32<kGenThreads>(sum, red_q);
    if (threadIdx.x == 0) qs[t] = sum;
  }
}

// d[:] = 0 and, when given, qs[:] = 0 (the K == 0 case).
__global__ void k_zero_dq(float* __restrict__ d, int* __restrict__ qs, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    d[i] = 0.0f;
    if (qs) qs[i] = 0;
  }
}

template <int NT, int NC>
hipError_t launch16(const uint16_t* x, const uint16_t* r, const uint16_t* g, float eps, int64_t M,
                    int64_t K, int64_t ldx, uint16_t* h_out, int8_t* q, float* d, int* qs,
                    hipStream_t s) {
  if (r)
    hipLaunchKernelGGL((k_rmsnorm_quant16<NT, NC, true>), dim3((unsigned)M), dim3(NT), 0, s, x, r,
                       g, eps, K, ldx, h_out, q, d, qs);
  else
    hipLaunchKernelGGL((k_rmsnorm_quant16<NT, NC, false>), dim3((unsigned)M), dim3(NT), 0, s, x,
                       r, g, eps, K, ldx, h_out, q, d, qs);
  return hipGetLastError();
}

// Fast-path shape: NT threads, NC 16-byte chunks per thread (0 if generic).
int rmsnorm_quant_config(int64_t K, int64_t ldx, int* threads, int* chunks) {
  if (K <= 0 || K % 8 != 0 || ldx % 8 != 0 || K > kRmsNormFastMaxK) {
    *threads = kGenThreads;
    *chunks = 0;
    return 0;
  }
  const int64_t nchunk = K / 8;
  if (nchunk <= 4 * 256) {
    *threads = 256;
    *chunks = (int)((nchunk + 255) / 256);
  } else {
    *threads = 1024;
    *chunks = (int)((nchunk + 1023) / 1024);
  }
  return 1;
}

}  // namespace

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* r, const uint16_t* g,
                                float eps, int64_t M, int64_t K, int64_t ldx, uint16_t* h_out,
                                int8_t* q, float* d, int* qs, hipStream_t s) {
  if (K == 0) {
    hipLaunchKernelGGL(k_zero_dq, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s, d, qs, M);
    return hipGetLastError();
  }
  int nt = 0, nc = 0;
  if (rmsnorm_quant_config(K, ldx, &nt, &nc)) {
    if (nt == 256) {
      switch (nc) {
        case 1: return launch16<256, 1>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
        case 2: return launch16<256, 2>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
        case 3: return launch16<256, 3>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
        default: return launch16<256, 4>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
      }
    }
    switch (nc) {
      case 1: return launch16<1024, 1>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
      case 2: return launch16<1024, 2>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
      case 3: return launch16<1024, 3>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
      default: return launch16<1024, 4>(x, r, g, eps, M, K, ldx, h_out, q, d, qs, s);
    }
  }
  hipLaunchKernelGGL(k_rmsnorm_quant_any, dim3((unsigned)M), dim3(kGenThreads), 0, s, x, r, g, eps,
                     K, ldx, h_out, q, d, qs);
  return hipGetLastError();
}

}  // namespace bl
