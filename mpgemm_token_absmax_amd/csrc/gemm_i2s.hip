// Prefill ternary GEMM (any M, int8 MFMA) on gfx950.
//
// Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 / 4.1 (I2_S: exact multiply-add of ternary codes with int8
// activations), 4.4 (prefill is compute bound and was left unoptimized by the
// CPU system); bitnet.cpp how-to blog 1.3 (prefill is the dense-compute phase).
//
// At M tokens the contraction acc[t][n] = sum_k q[t][k] * w[n][k] is a dense
// int8 GEMM (zeros are not skipped: I2_S is element-wise multiply-add), so it
// runs on v_mfma_i32_16x16x64_i8 with the ternary weights decoded to int8 in
// registers just before the MFMA.
//
// Block = 4 waves as 2 (rows) x 2 (tokens); wave tile = RT*16 output features
// x TT*16 tokens; K advances 256 weights per step (4 MFMA sub-steps of 64).
//   * activations (int8, the large operand per byte of work) are staged per
//     step into LDS as a [128 tokens][256 + 16 pad] byte tile, shared by the
//     two waves of each token half; the next step's tile is prefetched into
//     registers while the current one is consumed;
//   * packed weights (2 bits, 4x smaller) go straight from global memory to
//     registers: lane (r = lane%16, h = lane/16) loads 16 bytes of row r
//     covering weights 64h .. 64h+63 of the step; its 32-bit word s decodes
//     (9 VALU ops) to the 16 int8 weights 64h+16s .. +15, which the MFMA of
//     sub-step s pairs with activation bytes 64h+16s .. +15 of token r. The
//     same lane -> k assignment on both operands makes the MFMA's 64-term dot
//     exactly the sum over those k.
// Accumulation is exact int32; the dequant (acc * fl32(gamma * d_t)) is fused
// into the store.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 256;                 // weights (k) per step
constexpr int kLdsStride = kBK + 16;     // padded bytes per token row in LDS

__device__ __forceinline__ void store_quad(void* y, int ytype, int64_t N, int64_t t, int64_t n,
                                           v4i acc, float c) {
  const int64_t base = t * N + n;
  if (n + 3 < N && (N & 3) == 0) {
    if (ytype == 0) {
      *reinterpret_cast<v4i*>(static_cast<int*>(y) + base) = acc;
    } else if (ytype == 1) {
      *reinterpret_cast<float4*>(static_cast<float*>(y) + base) =
          make_float4(dequant(acc.x, c), dequant(acc.y, c), dequant(acc.z, c), dequant(acc.w, c));
    } else {
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(dequant(acc.x, c)) |
                          ((uint32_t)f32_to_bf16_rne(dequant(acc.y, c)) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(dequant(acc.z, c)) |
                          ((uint32_t)f32_to_bf16_rne(dequant(acc.w, c)) << 16);
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + base) = make_uint2(lo, hi);
    }
    return;
  }
  const int a[4] = {acc.x, acc.y, acc.z, acc.w};
  for (int v = 0; v < 4; ++v) {
    if (n + v >= N) break;
    if (ytype == 0) static_cast<int*>(y)[base + v] = a[v];
    else if (ytype == 1) static_cast<float*>(y)[base + v] = dequant(a[v], c);
    else static_cast<uint16_t*>(y)[base + v] = f32_to_bf16_rne(dequant(a[v], c));
  }
}

template <int RT, int TT>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_i2s(
    const uint8_t* __restrict__ packed, const float* __restrict__ gamma, int64_t N, int64_t K,
    const int8_t* __restrict__ q, const float* __restrict__ d, int64_t M, void* __restrict__ y,
    int ytype) {
  constexpr int BN = 2 * RT * 16;       // output features per block
  constexpr int BM = 2 * TT * 16;       // tokens per block
  constexpr int kChunks = BM * kBK / 16 / kThreads;   // 16-byte activation chunks per thread
  static_assert(kChunks * kThreads * 16 == BM * kBK, "tile/threads mismatch");
  __shared__ __attribute__((aligned(16))) int8_t bs[BM * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int wr = wv >> 1, wt = wv & 1;
  const int r = lane & 15, h = lane >> 4;
  const int64_t RB = K / 4;
  const int64_t n0 = (int64_t)blockIdx.x * BN + wr * RT * 16;
  const int64_t m0 = (int64_t)blockIdx.y * BM;
  const int64_t nks = (K + kBK - 1) / kBK;

  // activation staging: chunk c -> token c/16, 16-byte column c%16
  uint4 stage[kChunks];
  auto load_b = [&](int64_t ks) {
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = tid + u * kThreads;
      const int64_t tok = m0 + c / 16;
      const int64_t k = ks * kBK + (c % 16) * 16;
      stage[u] = (tok < M && k < K) ? *reinterpret_cast<const uint4*>(q + tok * K + k)
                                    : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto store_b = [&]() {
#pragma unroll
    for (int u = 0; u < kChunks; ++u) {
      const int c = tid + u * kThreads;
      *reinterpret_cast<uint4*>(bs + (c / 16) * kLdsStride + (c % 16) * 16) = stage[u];
    }
  };
  uint4 wa[RT];
  auto load_a = [&](int64_t ks) {
    const int64_t kw = ks * kBK + 64 * h;       // first weight of this lane's chunk
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t row = n0 + rt * 16 + r;
      wa[rt] = (row < N && kw < K) ? *reinterpret_cast<const uint4*>(packed + row * RB + kw / 4)
                                   : make_uint4(0u, 0u, 0u, 0u);
    }
  };

  v4i acc[RT][TT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  load_a(0);
  load_b(0);
  for (int64_t ks = 0; ks < nks; ++ks) {
    __syncthreads();                 // every wave is done reading the previous tile
    store_b();
    __syncthreads();
    uint4 wcur[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wcur[rt] = wa[rt];
    if (ks + 1 < nks) {              // prefetch the next step while this one computes
      load_a(ks + 1);
      load_b(ks + 1);
    }
    const int8_t* bw = bs + (wt * TT * 16 + r) * kLdsStride + 64 * h;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      v4i bf[TT];
#pragma unroll
      for (int tt = 0; tt < TT; ++tt)
        bf[tt] = *reinterpret_cast<const v4i*>(bw + tt * 16 * kLdsStride + 16 * s);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t word = s == 0 ? wcur[rt].x : s == 1 ? wcur[rt].y : s == 2 ? wcur[rt].z
                                                                                 : wcur[rt].w;
        const v4i af = decode_word(word);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[rt][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[tt], acc[rt][tt], 0, 0, 0);
      }
    }
  }

  // D layout: lane holds token (column) lane%16 and features 4*(lane/16) + v.
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int64_t tok = m0 + wt * TT * 16 + tt * 16 + r;
    if (tok >= M) continue;
    const float c = ytype ? gamma[0] * d[tok] : 0.0f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t n = n0 + rt * 16 + 4 * h;
      if (n < N) store_quad(y, ytype, N, tok, n, acc[rt][tt], c);
    }
  }
}

template <int RT, int TT>
hipError_t launch_cfg(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                      const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                      hipStream_t s) {
  constexpr int BN = 2 * RT * 16, BM = 2 * TT * 16;
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  hipLaunchKernelGGL((k_gemm_i2s<RT, TT>), grid, dim3(kThreads), 0, s, packed, gamma, N, K, q,
                     d, M, y, ytype);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s) {
  if (K % 64 != 0) return launch_generic(packed, gamma, N, K, q, d, M, y, ytype, s);
  if (M <= 16) return launch_gemv(packed, gamma, N, K, q, d, M, y, ytype, s);
  return launch_cfg<4, 4>(packed, gamma, N, K, q, d, M, y, ytype, s);
}

}  // namespace bl
