// Decode-time ternary GEMV (1 <= M <= 16 tokens) on gfx950, plus the generic
// kernel for shapes off the fast paths.
//
// Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 / 4.1 (I2_S: element-wise multiply-add over 2-bit
// ternary codes and int8 activations, exact sums); bitnet.cpp how-to blog 1.1
// (decode streams every weight once per token: memory-bandwidth bound) and
// 1.2 (ternary weights make the products adds and subtracts); FairyFuse
// "融合内核设计" (unpack, accumulate and write in one pass, no intermediate
// stores).
//
// Design (HBM-bound): the packed weights are the only large stream. Each wave
// owns RTW tiles of 16 output rows and a K-slice; lane (r = lane%16,
// h = lane/16) streams 16 bytes (64 weights) of row r per 256-weight step with
// one 128-bit load, so the 4 lanes of a row read 64 contiguous bytes. Each
// 32-bit group word decodes in registers (shift, mask, v_perm_b32 through the
// code table) to 16 int8 weights in k order, which feed one
// v_mfma_i32_16x16x64_i8 against the matching 16 activation bytes of token r
// (zero for r >= M). The int8 x ternary products are therefore exact int32
// adds; the MFMA sums 64 of them per lane group. Waves that split K combine
// their int32 tiles through LDS (exact, order free), and the dequant epilogue
// (acc * fl32(gamma * d_t)) is fused into the store.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;

__device__ __forceinline__ void store_out(void* y, int ytype, int64_t idx, int acc, float c) {
  if (ytype == 0) {
    static_cast<int*>(y)[idx] = acc;
  } else if (ytype == 1) {
    static_cast<float*>(y)[idx] = dequant(acc, c);
  } else {
    static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(dequant(acc, c));
  }
}

// Store 4 consecutive outputs y[t][n .. n+3] of one token (vector store when
// the 4 columns exist and are aligned).
__device__ __forceinline__ void store_quad(void* y, int ytype, int64_t N, int64_t t, int64_t n,
                                           v4i acc, float c) {
  const int64_t base = t * N + n;
  if (n + 3 < N && (N & 3) == 0) {
    if (ytype == 0) {
      *reinterpret_cast<v4i*>(static_cast<int*>(y) + base) = acc;
    } else if (ytype == 1) {
      float4 f = make_float4(dequant(acc.x, c), dequant(acc.y, c), dequant(acc.z, c),
                             dequant(acc.w, c));
      *reinterpret_cast<float4*>(static_cast<float*>(y) + base) = f;
    } else {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(dequant(acc.x, c)) |
                          ((uint32_t)f32_to_bf16_rne(dequant(acc.y, c)) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(dequant(acc.z, c)) |
                          ((uint32_t)f32_to_bf16_rne(dequant(acc.w, c)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + base) = make_uint2(lo, hi);
    }
  } else {
    const int a[4] = {acc.x, acc.y, acc.z, acc.w};
    for (int v = 0; v < 4; ++v)
      if (n + v < N) store_out(y, ytype, base + v, a[v], c);
  }
}

// RTW: 16-row tiles per wave. WK: waves splitting K (the block's other
// kWavesPerBlock / WK waves take further row tiles). U: 256-weight steps whose
// loads are issued together.
template <int RTW, int WK, int U>
__global__ __launch_bounds__(kThreads) void k_gemv_i2s(
    const uint8_t* __restrict__ packed, const float* __restrict__ gamma, int64_t N, int64_t K,
    const int8_t* __restrict__ q, const float* __restrict__ d, int64_t M, void* __restrict__ y,
    int ytype) {
  constexpr int WR = kWavesPerBlock / WK;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const int wr = wv / WK, wk = wv % WK;
  const int r = lane & 15, h = lane >> 4;
  const int64_t RB = K / 4;                       // packed bytes per row
  const int64_t nss = (RB + 63) / 64;             // 256-weight steps per row
  const int64_t n0 = ((int64_t)blockIdx.x * WR + wr) * RTW * 16;

  v4i acc[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) acc[i] = v4i{0, 0, 0, 0};

  const bool tok_ok = r < M;
  const int8_t* qrow = q + (int64_t)r * K;

  for (int64_t js = wk; js < nss; js += (int64_t)WK * U) {
    uint4 wq[U][RTW];
    v4i b[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t j = js + (int64_t)u * WK;
      const int64_t off = j * 64 + 16 * h;
      const bool kv = j < nss && off < RB;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const int64_t row = n0 + rt * 16 + r;
        wq[u][rt] = (kv && row < N)
                        ? *reinterpret_cast<const uint4*>(packed + row * RB + off)
                        : make_uint4(0u, 0u, 0u, 0u);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t k = j * 256 + 64 * h + 16 * s;
        b[u][s] = (kv && tok_ok && k < K) ? *reinterpret_cast<const v4i*>(qrow + k)
                                         : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const uint32_t wds[4] = {wq[u][rt].x, wq[u][rt].y, wq[u][rt].z, wq[u][rt].w};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word(wds[s]), b[u][s], acc[rt],
                                                          0, 0, 0);
      }
    }
  }

  if constexpr (WK > 1) {
    __shared__ v4i red[WK > 1 ? WK - 1 : 1][WR][RTW][kWave];
    if (wk > 0) {
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) red[wk - 1][wr][rt][lane] = acc[rt];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WK - 1; ++w)
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) acc[rt] += red[w][wr][rt][lane];
  }

  // D[i][j] layout of the 16x16 MFMA: lane holds column j = lane%16 (token)
  // and rows i = 4*(lane/16) + v (output features), v = 0..3.
  if (!tok_ok) return;
  const float c = ytype ? gamma[0] * d[r] : 0.0f;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int64_t n = n0 + rt * 16 + 4 * h;
    if (n < N) store_quad(y, ytype, N, r, n, acc[rt], c);
  }
}

// One thread per output: any K % 4 == 0 (group rule applied byte-wise).
__global__ void k_generic(const uint8_t* __restrict__ packed, const float* __restrict__ gamma,
                          int64_t N, int64_t K, const int8_t* __restrict__ q,
                          const float* __restrict__ d, int64_t M, void* __restrict__ y,
                          int ytype) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int64_t RB = K / 4;
  const uint8_t* row = packed + n * RB;
  for (int64_t t = blockIdx.y; t < M; t += gridDim.y) {
    const int8_t* qr = q + t * K;
    int acc = 0;
    for (int64_t g = 0; 4 * g < RB; ++g) {
      const int b = (int)min((int64_t)4, RB - 4 * g);
      for (int o = 0; o < 4 * b; ++o) acc += decode_one(row + 4 * g, b, o) * (int)qr[16 * g + o];
    }
    const float c = ytype ? gamma[0] * d[t] : 0.0f;
    store_out(y, ytype, t * N + n, acc, c);
  }
}

template <int RTW, int WK, int U>
hipError_t launch_cfg(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                      const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                      hipStream_t s) {
  constexpr int WR = kWavesPerBlock / WK;
  const int64_t rows_per_block = (int64_t)WR * RTW * 16;
  const int64_t blocks = (N + rows_per_block - 1) / rows_per_block;
  hipLaunchKernelGGL((k_gemv_i2s<RTW, WK, U>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                     packed, gamma, N, K, q, d, M, y, ytype);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_generic(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                          hipStream_t s) {
  const unsigned gx = (unsigned)((N + 255) / 256);
  const unsigned gy = (unsigned)(M < 65535 ? M : 65535);
  hipLaunchKernelGGL(k_generic, dim3(gx, gy), dim3(256), 0, s, packed, gamma, N, K, q, d, M, y,
                     ytype);
  return hipGetLastError();
}

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s) {
  if (K % 64 != 0) return launch_generic(packed, gamma, N, K, q, d, M, y, ytype, s);
  const int64_t row_tiles = (N + 15) / 16;
  if (M > 4) {
    if (row_tiles >= 1024) return launch_cfg<2, 2, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
    return launch_cfg<2, 4, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
  }
  if (row_tiles >= 2048) return launch_cfg<1, 2, 4>(packed, gamma, N, K, q, d, M, y, ytype, s);
  return launch_cfg<1, 4, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
}

}  // namespace bl
