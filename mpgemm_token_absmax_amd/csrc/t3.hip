// Base-3 ternary weights, five per byte (1.6 bits per weight): packing, the
// decode GEMV over int8 activations and the one-token fused decode (bf16 x
// quantized in the kernel) (gfx950).
//
// Source: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3: the format table lists element-wise multiply-add
// formats under 2 bits per weight (TQ1_0 at 1.69, TL2 at 1.67); a ternary
// weight has three values, so five fit a byte (3^5 = 243). The contraction is
// the exact integer sum of I2_S (Part A 2.3 / 4.1), over 20% fewer bytes.
//
// Layout (include/bitlinear.h): a row is padded with zero weights to a
// multiple of 320; unit u (weights 80u .. 80u+79) is 16 bytes at row offset
// 16u; byte j of a unit holds weights j + 16i (i = 0..4) as digits d = w + 1
// of v = sum d_i 3^(4-i), stored as ceil(256 v / 243). Read as the fraction
// q/256 the byte starts with v's base-3 digits, so they come off one at a
// time: y = 3x, digit = y >> 8, x = y mod 256.
//
// GEMV (M <= 16 tokens): a block owns 16 output rows; its WPB waves split K
// into runs of 320-weight steps. Lane (r = lane%16, h = lane/16) loads the
// 16-byte unit h of its row's step (80 weights) and decodes it plane by
// plane: plane i is 16 consecutive weights (k = 80h + 16i + 0..15) in byte
// order, the A operand of one v_mfma_i32_16x16x64_i8 whose B operand is the
// 16 activation bytes of token r at the same k. A step is 1 KB of packed
// weights per wave, as for I2_S (1024 weights there, 1280 here).
// Decode per 32-bit word (4 bytes) and plane: two multiply-by-3 on the
// even/odd bytes held in 16-bit slots (3*255 < 2^16: no carry between
// slots), one v_perm_b32 to gather the four digits (bits 8..15 of each
// slot), one v_perm_b32 through the table {-1, 0, +1}, two masks for the next
// plane: 6 VALU ops per 4 weights (I2_S: 9 per 16).
// Padding weights decode to 0, so activation fragments past K only need a
// valid address (clamped into the row), not masking.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr uint32_t kT3Table = 0x000100FFu;      // digit 0, 1, 2 -> int8 -1, 0, +1

// The plane-by-plane decoder of one 16-byte unit.
struct T3Unit {
  uint32_t lo[4], hi[4];                          // even / odd bytes in 16-bit slots

  __device__ __forceinline__ explicit T3Unit(v4i u) {
    const uint32_t w[4] = {(uint32_t)u.x, (uint32_t)u.y, (uint32_t)u.z, (uint32_t)u.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      lo[k] = w[k] & 0x00FF00FFu;
      hi[k] = (w[k] >> 8) & 0x00FF00FFu;
    }
  }

  // Weights of the next plane (16 int8 in byte order); `last` skips the
  // state update after plane 4.
  __device__ __forceinline__ v4i next(bool last) {
    v4i out;
    int* o = reinterpret_cast<int*>(&out);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t yl = lo[k] + (lo[k] << 1), yh = hi[k] + (hi[k] << 1);
      const uint32_t dig = __builtin_amdgcn_perm(yh, yl, 0x07030501u);   // bytes 1, 3 of each
      o[k] = (int)__builtin_amdgcn_perm(0u, kT3Table, dig);
      if (!last) {
        lo[k] = yl & 0x00FF00FFu;
        hi[k] = yh & 0x00FF00FFu;
      }
    }
    return out;
  }
};

// Ternary value of weight k of row n (0 past K).
template <bool F32>
__device__ __forceinline__ int trit(const void* w, int64_t n, int64_t K, int64_t k, float t) {
  if (k >= K) return 0;
  if constexpr (F32) {
    const float v = static_cast<const float*>(w)[n * K + k];
    return v > t ? 1 : (v < -t ? -1 : 0);
  } else {
    const int v = static_cast<const int8_t*>(w)[n * K + k];
    return v > 0 ? 1 : (v < 0 ? -1 : 0);
  }
}

// One output byte per thread.
template <bool F32>
__global__ void k_pack_t3(const void* __restrict__ w, int64_t N, int64_t K,
                          const float* __restrict__ gamma, uint8_t* __restrict__ out) {
  const int64_t RBt = 64 * ((K + 319) / 320);
  const int64_t bi = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (bi >= N * RBt) return;
  const int64_t n = bi / RBt, jb = bi % RBt;
  const int64_t u = jb / 16, j = jb % 16;
  const float t = F32 ? 0.5f * gamma[0] : 0.0f;
  int v = 0;
#pragma unroll
  for (int i = 0; i < 5; ++i) v = 3 * v + (trit<F32>(w, n, K, 80 * u + j + 16 * i, t) + 1);
  out[bi] = (uint8_t)((256 * v + 242) / 243);     // ceil(256 v / 243)
}

__global__ void k_zero_y(void* __restrict__ y, int ytype, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  if (ytype == 0) static_cast<int*>(y)[i] = 0;
  else if (ytype == 1) static_cast<float*>(y)[i] = 0.0f;
  else static_cast<uint16_t*>(y)[i] = 0;
}

__global__ void k_zero_f32(float* __restrict__ d, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) d[i] = 0.0f;
}

__device__ __forceinline__ void t3_store_quad(void* y, int ytype, int64_t N, int64_t t, int64_t n,
                                              v4i acc, float c) {
  const int64_t base = t * N + n;
  const int a[4] = {acc.x, acc.y, acc.z, acc.w};
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    if (n + v >= N) break;
    if (ytype == 0) static_cast<int*>(y)[base + v] = a[v];
    else if (ytype == 1) static_cast<float*>(y)[base + v] = dequant(a[v], c);
    else static_cast<uint16_t*>(y)[base + v] = f32_to_bf16_rne(dequant(a[v], c));
  }
}

// WPB waves split K; U steps per load batch (two batches in flight).
template <int WPB, int U>
__global__ __launch_bounds__(WPB * kWave) void k_gemv_t3(
    const uint8_t* __restrict__ packed, const float* __restrict__ gptr, int64_t N, int K,
    const int8_t* __restrict__ qin, const float* __restrict__ din, int M, void* __restrict__ yp,
    int ytype) {
  __shared__ v4i red[WPB > 1 ? WPB - 1 : 1][kWave];
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (WPB - 1);
  const int r = lane & 15, h = lane >> 4;
  const int nsteps = (K + 319) / 320;
  const int RBt = 64 * nsteps;
  const int len = (nsteps + WPB - 1) / WPB;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int tok = r < M ? r : M - 1;
  const int8_t* qrow = qin + (int64_t)tok * K;
  int64_t row = n0 + r;
  row = row < N ? row : N - 1;
  const uint8_t* wrow = packed + row * RBt;

  v4i wa[U], wb[U], qa[U][5], qb[U][5];
  auto load = [&](v4i (&w)[U], v4i (&qf)[U][5], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = max(min(j + u, jb - 1), 0);
      w[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + step * 64 + 16 * h));
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        int kk = step * 320 + 80 * h + 16 * i;
        kk = kk < K ? kk : K - 16;              // past K: padding weights are 0
        qf[u][i] = *reinterpret_cast<const v4i*>(qrow + kk);
      }
    }
  };
  load(wa, qa, ja);
  const float dtok = ytype ? din[tok] : 0.0f;
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;

  v4i acc0 = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0};   // two chains (even / odd plane)
  auto compute = [&](const v4i (&w)[U], const v4i (&qf)[U][5], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        T3Unit dec(w[u]);
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          v4i& a = (i & 1) ? acc1 : acc0;
          a = __builtin_amdgcn_mfma_i32_16x16x64_i8(dec.next(i == 4), qf[u][i], a, 0, 0, 0);
        }
      }
    }
  };
  for (int j = ja; j < jb; j += 2 * U) {
    if (j + U < jb) load(wb, qb, j + U);
    compute(wa, qa, j);
    if (j + 2 * U < jb) load(wa, qa, j + 2 * U);
    if (j + U < jb) compute(wb, qb, j + U);
  }
  v4i acc = acc0 + acc1;
  if constexpr (WPB > 1) {
    if (wk > 0) red[wk - 1][lane] = acc;
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WPB - 1; ++w) acc += red[w][lane];
  }
  // D layout: lane holds token lane%16 and rows 4*(lane/16) + v
  if (r >= M) return;
  const int64_t n = n0 + 4 * h;
  if (n < N) t3_store_quad(yp, ytype, N, r, n, acc, gam * dtok);
}

// One-token fused decode over base-3 weights (M == 1, bf16 x, K <= 65536):
// the quantize prologue of the I2_S one-token decode (each wave loads its part
// of x, the block combines the part maxima with one barrier, each wave writes
// its codes to a wave-private LDS region), then the contraction with whole
// cache-line weight loads. A segment is two 320-weight steps, 128 bytes of a
// row: eight 16-byte units of 80 weights. A block owns 16 rows; each load
// instruction covers 8 rows x one segment (lane (r8 = lane%8, c = lane/8)
// reads unit c of row r8), two loads per segment (rows 0-7 and 8-15).
// As the A operand of v_mfma_i32_16x16x64_i8 (decoded plane by plane, 16
// weights each) the lane sits at row m = lane%16 = r8 + 8(c&1) and k-group
// h = c/2: MFMA rows m < 8 carry the even units, rows m >= 8 the odd units of
// the same 8 real rows. Column n of the B operand holds the codes of unit
// 2h + (n&1), so row r of a half is D[r][0] + D[8 + r][1] (lanes 0/16 plus
// lanes 33/49 of the result). The codes past K are zeroed in LDS up to the end
// of the wave's last segment, so units past the row (an odd step count:
// clamped loads) and the format's padding weights contribute nothing.
// WPB waves per block split the segments; XR: 16-byte x chunks per lane
// (covers len*80 chunks), U: segments per load batch; SINGLE: U >= len.
template <int WPB, int XR, int U, bool SINGLE>
__global__ __launch_bounds__(WPB * kWave) void k_decode1_t3(DecodeGroup grp, int len_max) {
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [wave][len_max*640]
  __shared__ v4i red[WPB > 1 ? WPB - 1 : 1][2][kWave];
  __shared__ uint32_t wmax[WPB];

  const DecodeProblem& P = grp.p[blockIdx.y];
  const int64_t N = P.N;
  const int K = (int)P.K;
  const uint8_t* __restrict__ packed = P.packed;
  const uint16_t* __restrict__ xg = P.x;
  const float* gptr = P.gamma;
  void* yp = P.y;
  int8_t* qp = P.q;
  float* dp = P.d;
  const int ytype = P.ytype;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  asm volatile("" ::"s"(packed), "s"(xg), "s"(K), "s"(gptr), "s"(yp), "s"(qp), "s"(dp),
               "s"(ytype), "s"(len_max));
  if (n0 >= N) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (WPB - 1);
  const int h = lane >> 4, c = lane >> 3, r8 = lane & 7;
  const int nsteps = (K + 319) / 320;
  const int RBt = 64 * nsteps;
  const bool first_block = blockIdx.x == 0;

  const int nseg = (nsteps + 1) / 2;
  const int len = (nseg + WPB - 1) / WPB;
  const int ja = min(wk * len, nseg);
  const int jb = min(ja + len, nseg);
  const int klo = min(ja * 640, K);
  const int khi = min(jb * 640, K);
  const int nch = (khi - klo) / 8;
  int8_t* wact = act + wk * len_max * 640;

  // ---- 1. loads: this wave's part of x, then the first weight batch -----
  const uint4* xs = reinterpret_cast<const uint4*>(xg) + (nch > 0 ? klo / 8 : 0);
  const int clast = nch > 0 ? nch - 1 : 0;
  uint4 xv[XR];
#pragma unroll
  for (int u = 0; u < XR; ++u) xv[u] = xs[min(lane + u * kWave, clast)];
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;
  int64_t ra = n0 + r8, rb = n0 + 8 + r8;
  ra = ra < N ? ra : N - 1;
  rb = rb < N ? rb : N - 1;
  const uint8_t* wrow0 = packed + ra * RBt;
  const uint8_t* wrow1 = packed + rb * RBt;
  v4i wa[U][2], wb[SINGLE ? 1 : U][2];
  auto load_w = [&](auto& dst, int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int seg = max(min(j + u, jb - 1), 0);
      int off = seg * 128 + 16 * c;
      off = off < RBt ? off : RBt - 16;      // past the row: its codes are zero
      dst[u][0] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow0 + off));
      dst[u][1] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow1 + off));
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. absmax of the row: part maxima, one barrier -------------------
  uint32_t m = 0u;
#pragma unroll
  for (int u = 0; u < XR; ++u) m = max(m, lane + u * kWave < nch ? absmax8_bf16(xv[u]) : 0u);
  m = wave_max_u32(m);
  if (lane == 0) wmax[wk] = m;
  __syncthreads();
#pragma unroll
  for (int w = 0; w < WPB; ++w) m = max(m, wmax[w]);
  const float mf = __uint_as_float(m << 16);
  const float sq = m ? 127.0f / mf : 0.0f;
  const float dv = m ? mf / 127.0f : 0.0f;
  if (first_block && wk == 0 && lane == 0 && dp) dp[0] = dv;

  // ---- 3. int8 codes of this part -> the wave's LDS region --------------
  const bool write_q = first_block && qp;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int cc = lane + u * kWave;
    if (cc < nch) {
      const uint2 qv = quant8_bf16(xv[u], sq);
      *reinterpret_cast<uint2*>(wact + 8 * cc) = qv;
      if (write_q) *reinterpret_cast<uint2*>(qp + klo + 8 * cc) = qv;
    }
  }
  for (int b = (khi - klo) + 16 * lane; b < (jb - ja) * 640; b += 16 * kWave)
    *reinterpret_cast<v4i*>(wact + b) = v4i{0, 0, 0, 0};
  __builtin_amdgcn_wave_barrier();

  // ---- 4. MFMA over this part's segments, plane by plane ------------------
  v4i acc[2][2];                                       // [half][chain]
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = v4i{0, 0, 0, 0};
  const int8_t* arow = wact + 80 * (2 * h + (lane & 1));
  auto compute = [&](const auto& w, int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        v4i b[5];
#pragma unroll
        for (int p = 0; p < 5; ++p)
          b[p] = *reinterpret_cast<const v4i*>(arow + (j + u - ja) * 640 + 16 * p);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          T3Unit dec(w[u][i]);
#pragma unroll
          for (int p = 0; p < 5; ++p)
            acc[i][p & 1] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(dec.next(p == 4), b[p], acc[i][p & 1], 0, 0, 0);
        }
      }
    }
  };
  if constexpr (SINGLE) {
    compute(wa, ja);
  } else {
    for (int j = ja; j < jb; j += 2 * U) {
      if (j + U < jb) load_w(wb, j + U);
      compute(wa, j);
      if (j + 2 * U < jb) load_w(wa, j + 2 * U);
      if (j + U < jb) compute(wb, j + U);
    }
  }
  v4i a2[2] = {acc[0][0] + acc[0][1], acc[1][0] + acc[1][1]};

  // ---- 5. sum of the parts, even + odd units, dequant, store ------------
  if constexpr (WPB > 1) {
    if (wk > 0) {
      red[wk - 1][0][lane] = a2[0];
      red[wk - 1][1][lane] = a2[1];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int w = 0; w < WPB - 1; ++w) {
      a2[0] += red[w][0][lane];
      a2[1] += red[w][1][lane];
    }
  }
  v4i o[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    o[i].x = a2[i].x + __shfl(a2[i].x, lane + 33, kWave);
    o[i].y = a2[i].y + __shfl(a2[i].y, lane + 33, kWave);
    o[i].z = a2[i].z + __shfl(a2[i].z, lane + 33, kWave);
    o[i].w = a2[i].w + __shfl(a2[i].w, lane + 33, kWave);
  }
  if ((lane & 15) != 0 || lane >= 32) return;          // lanes 0 and 16
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int64_t n = n0 + 8 * i + 4 * h;
    if (n < N) t3_store_quad(yp, ytype, N, 0, n, o[i], gam * dv);
  }
}

template <int WPB, int XR, int U, bool SINGLE>
hipError_t launch_one_token_t3(DecodeGroup& g, int len_max, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 15) / 16;
    blocks = b > blocks ? b : blocks;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)WPB * len_max * 640;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&k_decode1_t3<WPB, XR, U, SINGLE>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_decode1_t3<WPB, XR, U, SINGLE>), dim3((unsigned)blocks, (unsigned)g.count),
                     dim3(WPB * kWave), lds, s, g, len_max);
  return hipGetLastError();
}

// Longest per-wave run of 640-weight segments when WPB waves split K.
int t3_segs_per_wave(const DecodeGroup& g, int wpb) {
  int len = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t nseg = ((g.p[i].K + 319) / 320 + 1) / 2;
    const int l = (int)((nseg + wpb - 1) / wpb);
    len = l > len ? l : len;
  }
  return len;
}

template <int WPB, int U>
hipError_t launch_t3(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                     const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                     hipStream_t s) {
  hipLaunchKernelGGL((k_gemv_t3<WPB, U>), dim3((unsigned)((N + 15) / 16)), dim3(WPB * kWave), 0,
                     s, packed, gamma, N, (int)K, q, d, (int)M, y, ytype);
  return hipGetLastError();
}

unsigned grid256(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

int t3_steps_per_wave(int64_t K, int wpb) { return (int)((((K + 319) / 320) + wpb - 1) / wpb); }

hipError_t launch_pack_t3(const void* w, bool f32, int64_t N, int64_t K, uint8_t* packed,
                          const float* gamma, hipStream_t s) {
  const int64_t n = N * 64 * ((K + 319) / 320);
  if (f32)
    hipLaunchKernelGGL(k_pack_t3<true>, dim3(grid256(n)), dim3(256), 0, s, w, N, K, gamma, packed);
  else
    hipLaunchKernelGGL(k_pack_t3<false>, dim3(grid256(n)), dim3(256), 0, s, w, N, K, gamma,
                       packed);
  return hipGetLastError();
}

// Enough waves per block that each walks at most two steps per batch.
hipError_t launch_gemv_t3(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                          hipStream_t s) {
  if (K == 0) {
    hipLaunchKernelGGL(k_zero_y, dim3(grid256(M * N)), dim3(256), 0, s, y, ytype, M * N);
    return hipGetLastError();
  }
  const int l4 = t3_steps_per_wave(K, 4);
  if (l4 <= 1) return launch_t3<4, 1>(packed, gamma, N, K, q, d, M, y, ytype, s);
  if (l4 == 2) return launch_t3<4, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
  const int l8 = t3_steps_per_wave(K, 8);
  if (l8 <= 2) return launch_t3<8, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
  return launch_t3<16, 2>(packed, gamma, N, K, q, d, M, y, ytype, s);
}

// One token: quantize in the kernel; each wave walks at most 4 segments in
// one load batch up to 8 waves, else batches of 4. Several tokens: one launch
// quantizes every problem's x into its q and d, then one GEMV per problem.
hipError_t launch_decode_group_t3(DecodeGroup& g, hipStream_t s) {
  int kept = 0;
  for (int i = 0; i < g.count; ++i) {
    if (g.p[i].K == 0) {
      hipLaunchKernelGGL(k_zero_y, dim3(grid256(g.M * g.p[i].N)), dim3(256), 0, s, g.p[i].y,
                         g.p[i].ytype, g.M * g.p[i].N);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      if (g.p[i].d) {
        hipLaunchKernelGGL(k_zero_f32, dim3(1), dim3(64), 0, s, g.p[i].d, (int64_t)g.M);
        const hipError_t e2 = hipGetLastError();
        if (e2 != hipSuccess) return e2;
      }
    } else {
      g.p[kept++] = g.p[i];
    }
  }
  g.count = kept;
  if (g.count == 0) return hipSuccess;
  if (g.M == 1) {
    const int w4 = t3_segs_per_wave(g, 4);
    if (w4 <= 1) return launch_one_token_t3<4, 2, 1, true>(g, w4, s);
    if (w4 == 2) return launch_one_token_t3<4, 3, 2, true>(g, w4, s);
    if (w4 <= 4) return launch_one_token_t3<4, 5, 4, true>(g, w4, s);
    const int w8 = t3_segs_per_wave(g, 8);
    if (w8 <= 4) return launch_one_token_t3<8, 5, 4, true>(g, w8, s);
    if (w8 <= 8) return launch_one_token_t3<8, 10, 4, false>(g, w8, s);
    const int w16 = t3_segs_per_wave(g, 16);      // <= 7 for K <= 65536
    return launch_one_token_t3<16, 10, 4, false>(g, w16, s);
  }
  hipError_t e = launch_quantize_group(g, s);
  for (int i = 0; i < g.count && e == hipSuccess; ++i) {
    const DecodeProblem& p = g.p[i];
    e = launch_gemv_t3(p.packed, p.gamma, p.N, p.K, p.q, p.d, g.M, p.y, p.ytype, s);
  }
  return e;
}

}  // namespace bl
