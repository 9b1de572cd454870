// Decode-time ternary GEMV (1 <= M <= 16 tokens) on gfx950: the plain GEMV
// (int8 activations in) and the fused decode group (bf16 activations in:
// per-token absmax quantization, GEMV and dequant in one launch for up to
// kMaxGroup independent projections), plus the generic kernel for shapes off
// the fast paths.
//
// Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 / 4.1 (I2_S: element-wise multiply-add over 2-bit ternary
// codes and int8 activations quantized with one scale per vector, exact
// sums); bitnet.cpp how-to blog 1.1 (decode streams every weight once per
// token: memory-bandwidth bound) and 1.2 (ternary weights make the products
// adds and subtracts); FairyFuse "融合内核设计" (load activations, walk the
// 2-bit codes, accumulate and write in one pass with no intermediate stores).
//
// Design (HBM-bound: the packed weights are the only large stream):
//  * a launch covers one or more problems; blocks are dealt to problems by a
//    prefix table in the kernel arguments;
//  * each block first issues its first batch of weight loads, then builds the
//    int8 activations of all M tokens in LDS: copied from q (plain GEMV) or
//    quantized from bf16 x with the same arithmetic as bl_quantize_act
//    (fused decode; block 0 of a problem also writes q and d);
//  * each wave owns RTW tiles of 16 output rows and every WK-th 256-weight
//    step of K. Lane (r = lane%16, h = lane/16) streams 16 bytes (64 weights)
//    of row r per step with one 128-bit load (the 4 lanes of a row read 64
//    contiguous bytes); loads of the next U steps are in flight while the
//    current ones are consumed;
//  * each 32-bit group word decodes in registers (9 VALU ops: shift, masks,
//    v_perm_b32 through the code table) to 16 int8 weights in k order and
//    feeds one v_mfma_i32_16x16x64_i8 against the 16 matching activation
//    bytes of token r read from LDS (zero for r >= M): the ternary x int8
//    products are exact int32 adds;
//  * waves that split K add their int32 tiles through LDS (exact, order
//    free) and the dequant acc * fl32(gamma * d_t) is fused into the store.
#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesPerBlock = kThreads / kWave;
constexpr int kActLds = 48 * 1024;      // LDS bytes for activations (M * K chunk)
constexpr int kXReg = 8;                // bf16 x chunks (4 values) per thread kept in registers
constexpr int kQReg = 2;                // int8 q chunks (16 values) per thread kept in registers

__device__ __forceinline__ void store_out(void* y, int ytype, int64_t idx, int acc, float c) {
  if (ytype == 0) {
    static_cast<int*>(y)[idx] = acc;
  } else if (ytype == 1) {
    static_cast<float*>(y)[idx] = dequant(acc, c);
  } else {
    static_cast<uint16_t*>(y)[idx] = f32_to_bf16_rne(dequant(acc, c));
  }
}

// Store y[t][n .. n+3] of one token (vector store when the 4 columns exist and
// are aligned).
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
  } else {
    const int a[4] = {acc.x, acc.y, acc.z, acc.w};
    for (int v = 0; v < 4; ++v)
      if (n + v < N) store_out(y, ytype, base + v, a[v], c);
  }
}

template <int RTW, int WK, int U>
__global__ __launch_bounds__(kThreads) void k_gemv_i2s(DecodeGroup grp) {
  constexpr int WR = kWavesPerBlock / WK;
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [M][kc] int8
  __shared__ v4i red[WK > 1 ? WK - 1 : 1][WR][RTW][kWave];
  __shared__ uint32_t mred[kWavesPerBlock][kMaxDecodeM];
  __shared__ float sc[kMaxDecodeM];
  __shared__ float dsh[kMaxDecodeM];

  // problem of this block (uniform scan over a short prefix table)
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) pi += (i < grp.count && (int)blockIdx.x >= grp.block0[i]);
  const DecodeProblem& P = grp.p[pi];
  const int64_t N = P.N, K = P.K;
  const int M = grp.M;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int wr = wv / WK, wk = wv % WK;
  const int r = lane & 15, h = lane >> 4;
  const int64_t RB = K / 4;                       // packed bytes per row
  const int64_t n0 = ((int64_t)(blockIdx.x - grp.block0[pi]) * WR + wr) * RTW * 16;
  const bool first_block = (int)blockIdx.x == grp.block0[pi];
  const uint8_t* __restrict__ packed = P.packed;
  const uint16_t* __restrict__ xg = P.x;
  const int64_t kq = K / 4;                       // 4-element chunks per token row

  // K is processed in chunks of kc weights whose int8 activations fit in LDS.
  const int64_t kc_max = ((int64_t)(kActLds / M) / 256) * 256;
  const int64_t kc = K < kc_max ? K : kc_max;

  v4i wa[U][RTW], wb[U][RTW];   // two batches of weight loads
  // loads of the steps [j, min(j + U, jend)) of this wave into dst
  auto load_w = [&](v4i (&dst)[U][RTW], int64_t j, int64_t jend) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t off = (j + u) * 64 + 16 * h;
      const bool kv = j + u < jend && off < RB;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt) {
        const int64_t row = n0 + rt * 16 + r;
        dst[u][rt] = (kv && row < N)
                         ? __builtin_nontemporal_load(
                               reinterpret_cast<const v4i*>(packed + row * RB + off))
                         : v4i{0, 0, 0, 0};
      }
    }
  };
  // this wave's contiguous range of 256-weight steps inside a chunk
  auto wave_range = [&](int64_t k0, int64_t kn, int64_t& ja, int64_t& jb) {
    const int64_t js0 = k0 / 256, jend = (k0 + kn + 255) / 256;
    const int64_t len = (jend - js0 + WK - 1) / WK;
    ja = js0 + wk * len;
    jb = ja + len < jend ? ja + len : jend;
  };

  int64_t ja, jb;
  wave_range(0, kc, ja, jb);
  load_w(wa, ja, jb);                             // weights in flight during the prologue

  // ---- per-token scales (fused path: absmax of bf16 x, same arithmetic as
  // bl_quantize_act); rows of M*K <= kThreads*4*kXReg stay in registers.
  const bool x_in_regs = xg && M * kq <= (int64_t)kThreads * kXReg;
  uint2 xv[kXReg];
  if (xg) {
    for (int t = 0; t < M; ++t) {
      uint32_t m = 0u;
      if (x_in_regs) {
#pragma unroll
        for (int u = 0; u < kXReg; ++u) {
          const int64_t i = tid + (int64_t)u * kThreads;
          if (t == 0) {
            xv[u] = make_uint2(0u, 0u);
            if (i < M * kq) xv[u] = *reinterpret_cast<const uint2*>(xg + (i / kq) * P.ldx +
                                                                   (i % kq) * 4);
          }
          if (i < M * kq && i / kq == t) m = max(m, absmax4_bf16(xv[u]));
        }
      } else {
        const uint2* xr = reinterpret_cast<const uint2*>(xg + (int64_t)t * P.ldx);
        for (int64_t c = tid; c < kq; c += kThreads) m = max(m, absmax4_bf16(xr[c]));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
      if (lane == 0) mred[wv][t] = m;
    }
    __syncthreads();
    if (tid < M) {
      uint32_t mb = mred[0][tid];
#pragma unroll
      for (int w = 1; w < kWavesPerBlock; ++w) mb = max(mb, mred[w][tid]);
      const float m = __uint_as_float(mb << 16);
      sc[tid] = mb ? 127.0f / m : 0.0f;
      const float dd = mb ? m / 127.0f : 0.0f;
      dsh[tid] = dd;
      if (first_block && P.d) P.d[tid] = dd;
    }
    __syncthreads();
  }

  v4i acc[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) acc[i] = v4i{0, 0, 0, 0};

  for (int64_t k0 = 0; k0 < K; k0 += kc) {
    const int64_t kn = (K - k0) < kc ? (K - k0) : kc;      // multiple of 64
    if (k0 > 0) {
      wave_range(k0, kn, ja, jb);
      load_w(wa, ja, jb);
      __syncthreads();                                     // previous chunk consumed
    }
    // stage the int8 activations [M][kn] of this chunk into LDS
    if (x_in_regs) {                                       // single chunk (kn == K)
#pragma unroll
      for (int u = 0; u < kXReg; ++u) {
        const int64_t i = tid + (int64_t)u * kThreads;
        if (i < M * kq) {
          const int64_t t = i / kq;
          const float s = sc[t];
          const uint32_t v = s != 0.0f ? quant4_bf16(xv[u], s) : 0u;
          reinterpret_cast<uint32_t*>(act)[i] = v;
          if (first_block && P.q) reinterpret_cast<uint32_t*>(P.q)[i] = v;
        }
      }
    } else if (xg) {
      const int64_t nq = kn / 4;
      for (int64_t i = tid; i < M * nq; i += kThreads) {
        const int64_t t = i / nq, c = i % nq;
        const float s = sc[t];
        const uint2 v2 = *reinterpret_cast<const uint2*>(xg + t * P.ldx + k0 + 4 * c);
        const uint32_t v = s != 0.0f ? quant4_bf16(v2, s) : 0u;
        reinterpret_cast<uint32_t*>(act)[i] = v;
        if (first_block && P.q)
          *reinterpret_cast<uint32_t*>(P.q + t * K + k0 + 4 * c) = v;
      }
    } else {
      const int64_t n16 = kn / 16;
      for (int64_t i = tid; i < M * n16; i += kThreads) {
        const int64_t t = i / n16, c = i % n16;
        reinterpret_cast<v4i*>(act)[i] =
            *reinterpret_cast<const v4i*>(P.qin + t * K + k0 + 16 * c);
      }
    }
    __syncthreads();

    const int8_t* arow = act + (int64_t)r * kn + 64 * h;
    const bool tok_ok = r < M;
    const int64_t js0 = k0 / 256;
    auto compute = [&](const v4i (&w)[U][RTW], int64_t j) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u >= jb) break;
        const int64_t kk = (j + u - js0) * 256;            // offset inside the chunk
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v4i b = v4i{0, 0, 0, 0};
          if (tok_ok && kk + 64 * h + 16 * s < kn)
            b = *reinterpret_cast<const v4i*>(arow + kk + 16 * s);
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt)
            acc[rt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][rt][s]),
                                                            b, acc[rt], 0, 0, 0);
        }
      }
    };
    // two batches of U steps in flight: compute one while the next loads
    for (int64_t j = ja; j < jb; j += 2 * U) {
      if (j + U < jb) load_w(wb, j + U, jb);
      compute(wa, j);
      if (j + 2 * U < jb) load_w(wa, j + 2 * U, jb);
      if (j + U < jb) compute(wb, j + U);
    }
  }

  if constexpr (WK > 1) {
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

  // D[i][j] of the 16x16 MFMA: lane holds column j = lane%16 (token) and rows
  // i = 4*(lane/16) + v (output features), v = 0..3.
  if (r >= M) return;
  float c = 0.0f;
  if (P.ytype) c = P.gamma[0] * (xg ? dsh[r] : P.din[r]);
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int64_t n = n0 + rt * 16 + 4 * h;
    if (n < N) store_quad(P.y, P.ytype, N, r, n, acc[rt], c);
  }
}

// One-token fused decode (M == 1, bf16 x, K <= 16384): per block 16 output
// rows, the four waves split K into quarters. Each wave loads only its
// quarter of x (before its weights: vector loads retire in order), takes the
// absmax of it (packed 16-bit max, DPP), and the block combines the four
// maxima with one barrier; each wave then quantizes its own quarter into a
// wave-private LDS region (the exact add-1.5*2^23 rounding of quant8_bf16),
// runs its MFMA steps with every lane reading token 0's fragments (lanes of
// tokens 1..15 feed output columns that are never stored) and the block sums
// the four partial accumulators with a second barrier.
// Grid: x = row blocks of the largest problem, y = problem (so a block finds
// its problem without first loading a table); blocks past a problem's rows
// exit at once.
// WPB: waves per block (each takes 1/WPB of K), XR: 16-byte x chunks per lane
// (covers len*32 chunks), U: steps per load batch.
template <int WPB, int XR, int U>
__global__ __launch_bounds__(WPB * kWave) void k_decode1(DecodeGroup grp, int len_max) {
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [wave][len_max*256]
  __shared__ v4i red[WPB - 1][kWave];
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
  // Every field in one scalar round trip, before the exit test: a scalar
  // load still in flight later would make each LDS wait a full wait (they
  // share a counter and scalar loads complete out of order).
  asm volatile("" ::"s"(packed), "s"(xg), "s"(K), "s"(gptr), "s"(yp), "s"(qp), "s"(dp),
               "s"(ytype), "s"(len_max));
  if (n0 >= N) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (WPB - 1);   // K part
  const int h = lane >> 4;
  const int RB = K / 4;
  const bool first_block = blockIdx.x == 0;

  const int nsteps = (K + 255) / 256;
  const int len = (nsteps + WPB - 1) / WPB;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int klo = min(ja * 256, K);
  const int khi = min(jb * 256, K);
  const int nch = (khi - klo) / 8;                    // 8-value chunks of this part
  int8_t* wact = act + wk * len_max * 256;

  // ---- 1. loads: this quarter of x, then the first weight batch ---------
  const uint4* xs = reinterpret_cast<const uint4*>(xg) + (nch > 0 ? klo / 8 : 0);
  const int clast = nch > 0 ? nch - 1 : 0;
  uint4 xv[XR];
#pragma unroll
  for (int u = 0; u < XR; ++u) xv[u] = xs[min(lane + u * kWave, clast)];
  // gamma by a vector load, issued with x (counted with the vector loads)
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;
  int64_t row = n0 + (lane & 15);
  row = row < N ? row : N - 1;
  const uint8_t* wrow = packed + row * RB;
  v4i wa[U], wb[U];
  auto load_w = [&](v4i (&dst)[U], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = max(min(j + u, jb - 1), 0);
      int off = step * 64 + 16 * h;
      off = off < RB ? off : RB - 16;
      dst[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow + off));
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. absmax of the row: quarter maxima, one barrier ----------------
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

  // ---- 3. int8 codes of this quarter -> the wave's LDS region -----------
  const bool write_q = first_block && qp;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int c = lane + u * kWave;
    if (c < nch) {
      const uint2 qv = quant8_bf16(xv[u], sq);
      *reinterpret_cast<uint2*>(wact + 8 * c) = qv;
      if (write_q) *reinterpret_cast<uint2*>(qp + klo + 8 * c) = qv;
    }
  }
  // zeros past K in the last partial step (K % 256 != 0)
  for (int b = (khi - klo) + 16 * lane; b < (jb - ja) * 256; b += 16 * kWave)
    *reinterpret_cast<v4i*>(wact + b) = v4i{0, 0, 0, 0};
  // the region is this wave's alone and LDS serves a wave in order
  __builtin_amdgcn_wave_barrier();

  // ---- 4. MFMA over this quarter's steps --------------------------------
  v4i acc0 = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0};  // two chains (even / odd s)
  const int8_t* arow = wact + 64 * h;
  auto read_b = [&](v4i (&b)[4], int j) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
      b[s] = *reinterpret_cast<const v4i*>(arow + (j - ja) * 256 + 16 * s);
  };
  auto compute = [&](const v4i (&w)[U], int j) {
    v4i bn[4];
    read_b(bn, j);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        v4i b[4] = {bn[0], bn[1], bn[2], bn[3]};
        if (u + 1 < U && j + u + 1 < jb) read_b(bn, j + u + 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v4i& a = (s & 1) ? acc1 : acc0;
          a = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][s]), b[s], a, 0,
                                                    0, 0);
        }
      }
    }
  };
  for (int j = ja; j < jb; j += 2 * U) {
    if (j + U < jb) load_w(wb, j + U);
    compute(wa, j);
    if (j + 2 * U < jb) load_w(wa, j + 2 * U);
    if (j + U < jb) compute(wb, j + U);
  }
  v4i acc = acc0 + acc1;

  // ---- 5. sum of the quarters, dequant, store ---------------------------
  if (wk > 0) red[wk - 1][lane] = acc;
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int w = 0; w < WPB - 1; ++w) acc += red[w][lane];
  // D layout: lane holds token lane%16 and rows 4*(lane/16) + v; token 0 only
  if ((lane & 15) != 0) return;
  const int64_t n = n0 + 4 * h;
  if (n < N) store_quad(yp, ytype, N, 0, n, acc, gam * dv);
}

// Fast decode kernel (every problem's per-wave activation slice fits in LDS).
// Each wave owns a contiguous range of 256-weight steps and builds the int8
// activations of exactly that range in a wave-private LDS region.
//  * Vector loads retire in issue order, so the activation loads are issued
//    before the weight loads: waiting for them never waits for the HBM stream.
//  * XF > 0 (fused, one token, K <= XF*512): every wave reads the whole bf16
//    row and takes its absmax itself, so no block barrier precedes the MFMA
//    loop; otherwise the waves exchange per-token maxima through LDS (one
//    barrier).
//  * Wave-uniform values live in scalar registers and loads are unconditional
//    with clamped, always-valid addresses (rows past N read row N-1 and are
//    never stored; lanes past K meet zero activations), so the step loop has
//    no per-lane control flow and the compiler waits only for the loads it
//    needs.
template <int RTW, int WK, int U, int XF>
__global__ __launch_bounds__(kThreads) void k_decode_fast(DecodeGroup grp, int len_max) {
  constexpr int WR = kWavesPerBlock / WK;
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [wave][M][len_max*256]
  __shared__ v4i red[WK > 1 ? WK - 1 : 1][WR][RTW][kWave];
  __shared__ uint32_t wmax[kWavesPerBlock][kMaxDecodeM];

  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) pi += (i < grp.count && (int)blockIdx.x >= grp.block0[i]);
  const DecodeProblem& P = grp.p[pi];
  const int64_t N = P.N;
  const int K = (int)P.K;
  const int M = grp.M;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wv / WK, wk = wv % WK;
  const int r = lane & 15, h = lane >> 4;
  const int RB = K / 4;
  const int64_t n0 = ((int64_t)(blockIdx.x - grp.block0[pi]) * WR + wr) * RTW * 16;
  const bool first_block = (int)blockIdx.x == grp.block0[pi];
  const uint16_t* __restrict__ xg = P.x;
  if (K < 64) return;         // the launcher routes K == 0 problems to k_zero_outputs

  // this wave's steps [ja, jb) and weights [klo, khi)
  const int nsteps = (K + 255) / 256;
  const int len = (nsteps + WK - 1) / WK;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int klo = min(ja * 256, K);
  const int khi = min(jb * 256, K);
  const int kw = khi - klo;                           // multiple of 64 (may be 0)
  const int region = len_max * 256;                   // bytes per token row in LDS
  int8_t* wact = act + wv * M * region;

  const uint8_t* wrow[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    int64_t row = n0 + rt * 16 + r;
    row = row < N ? row : N - 1;
    wrow[rt] = P.packed + row * RB;
  }
  v4i wa[U][RTW], wb[U][RTW];
  auto load_w = [&](v4i (&dst)[U][RTW], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = max(min(j + u, jb - 1), 0);
      int off = step * 64 + 16 * h;
      off = off < RB ? off : RB - 16;
#pragma unroll
      for (int rt = 0; rt < RTW; ++rt)
        dst[u][rt] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow[rt] + off));
    }
  };

  // ---- 1. activation loads (before the weights) -------------------------
  const bool full_row = XF > 0 && xg && M == 1 && K <= XF * 512;
  const int nch8 = K / 8;                             // 8-value chunks of the row
  uint4 xf[XF > 0 ? XF : 1];
  if (full_row) {
#pragma unroll
    for (int u = 0; u < XF; ++u) {
      const int c = min(lane + u * kWave, nch8 - 1);
      xf[u] = *reinterpret_cast<const uint4*>(xg + 8 * c);
    }
  }
  const int cpt = kw / 4;                             // 4-value chunks of this wave's range
  const bool cache = xg && !full_row && M == 1 && cpt <= kXReg * kWave;
  uint2 xv[kXReg];
  if (cache && cpt > 0) {
#pragma unroll
    for (int u = 0; u < kXReg; ++u) {
      const int c = min(lane + u * kWave, cpt - 1);
      xv[u] = *reinterpret_cast<const uint2*>(xg + klo + 4 * c);
    }
  }
  const int c16 = kw / 16;
  const bool qcache = !xg && M == 1 && c16 <= kQReg * kWave;
  v4i qv[kQReg];
  if (qcache && c16 > 0) {
#pragma unroll
    for (int u = 0; u < kQReg; ++u) {
      const int c = min(lane + u * kWave, c16 - 1);
      qv[u] = *reinterpret_cast<const v4i*>(P.qin + klo + 16 * c);
    }
  }
  const float gam = P.ytype ? P.gamma[0] : 0.0f;      // epilogue operands, fetched early
  const float din_r = (!xg && P.ytype) ? P.din[r < M ? r : 0] : 0.0f;
  __builtin_amdgcn_sched_barrier(0);
  // ---- 2. weight loads --------------------------------------------------
  load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. int8 activations of this wave's range -> its LDS region -------
  float d_lane = 0.0f;                                // lane t < M: token t's d
  const bool write_q = first_block && wr == 0 && P.q;
  if (full_row) {
    uint32_t m = 0u;
#pragma unroll
    for (int u = 0; u < XF; ++u)
      if (lane + u * kWave < nch8)
        m = max(m, max(absmax4_bf16(make_uint2(xf[u].x, xf[u].y)),
                       absmax4_bf16(make_uint2(xf[u].z, xf[u].w))));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
    const float mf = __uint_as_float(m << 16);
    const float s = m ? 127.0f / mf : 0.0f;
    d_lane = m ? mf / 127.0f : 0.0f;
    if (first_block && wv == 0 && lane == 0 && P.d) P.d[0] = d_lane;
    const int c_lo = klo / 8, c_hi = khi / 8;
#pragma unroll
    for (int u = 0; u < XF; ++u) {
      const int c = lane + u * kWave;
      if (c >= c_lo && c < c_hi) {
        const uint32_t lo = s != 0.0f ? quant4_bf16(make_uint2(xf[u].x, xf[u].y), s) : 0u;
        const uint32_t hi = s != 0.0f ? quant4_bf16(make_uint2(xf[u].z, xf[u].w), s) : 0u;
        *reinterpret_cast<uint2*>(wact + 8 * (c - c_lo)) = make_uint2(lo, hi);
        if (write_q) *reinterpret_cast<uint2*>(P.q + 8 * c) = make_uint2(lo, hi);
      }
    }
  } else if (xg) {
    // per-token maxima of this wave's range, exchanged through LDS (1 barrier)
    for (int t = 0; t < M; ++t) {
      uint32_t m = 0u;
      if (cache) {
#pragma unroll
        for (int u = 0; u < kXReg; ++u)
          m = max(m, lane + u * kWave < cpt ? absmax4_bf16(xv[u]) : 0u);
      } else {
        const uint16_t* xr = xg + (int64_t)t * P.ldx + klo;
        for (int c = lane; c < cpt; c += kWave)
          m = max(m, absmax4_bf16(*reinterpret_cast<const uint2*>(xr + 4 * c)));
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off, kWave));
      if (lane == 0) wmax[wv][t] = m;
    }
    __syncthreads();
    float s_lane = 0.0f;
    if (lane < M) {
      uint32_t mb = wmax[0][lane];
#pragma unroll
      for (int w = 1; w < kWavesPerBlock; ++w) mb = max(mb, wmax[w][lane]);
      const float m = __uint_as_float(mb << 16);
      s_lane = mb ? 127.0f / m : 0.0f;
      d_lane = mb ? m / 127.0f : 0.0f;
      if (first_block && wv == 0 && P.d) P.d[lane] = d_lane;
    }
    for (int t = 0; t < M; ++t) {
      const float s = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                    __builtin_bit_cast(int, s_lane), t));
      uint32_t* dst = reinterpret_cast<uint32_t*>(wact + t * region);
      uint32_t* qo = write_q ? reinterpret_cast<uint32_t*>(P.q + (int64_t)t * K + klo) : nullptr;
      if (cache) {
#pragma unroll
        for (int u = 0; u < kXReg; ++u) {
          const int c = lane + u * kWave;
          if (c < cpt) {
            const uint32_t v = s != 0.0f ? quant4_bf16(xv[u], s) : 0u;
            dst[c] = v;
            if (qo) qo[c] = v;
          }
        }
      } else {
        const uint16_t* xr = xg + (int64_t)t * P.ldx + klo;
        for (int c = lane; c < cpt; c += kWave) {
          const uint32_t v =
              s != 0.0f ? quant4_bf16(*reinterpret_cast<const uint2*>(xr + 4 * c), s) : 0u;
          dst[c] = v;
          if (qo) qo[c] = v;
        }
      }
    }
  } else if (qcache) {
    v4i* dst = reinterpret_cast<v4i*>(wact);
#pragma unroll
    for (int u = 0; u < kQReg; ++u) {
      const int c = lane + u * kWave;
      if (c < c16) dst[c] = qv[u];
    }
  } else {
    for (int t = 0; t < M; ++t) {
      const v4i* src = reinterpret_cast<const v4i*>(P.qin + (int64_t)t * K + klo);
      v4i* dst = reinterpret_cast<v4i*>(wact + t * region);
      for (int c = lane; c < c16; c += kWave) dst[c] = src[c];
    }
  }
  // zero the region tail [kw, len*256) that the last partial step reads
  for (int t = 0; t < M; ++t) {
    v4i* dst = reinterpret_cast<v4i*>(wact + t * region);
    for (int c = kw / 16 + lane; c < len * 16; c += kWave) dst[c] = v4i{0, 0, 0, 0};
  }
  // The region is private to this wave and LDS serves a wave's accesses in
  // order, so its reads below see these writes without a fence.
  __builtin_amdgcn_wave_barrier();

  // ---- 4. MFMA over this wave's steps -----------------------------------
  v4i acc0[RTW], acc1[RTW];                           // two chains (even / odd s)
#pragma unroll
  for (int i = 0; i < RTW; ++i) acc0[i] = acc1[i] = v4i{0, 0, 0, 0};
  const bool tok_ok = r < M;
  const int8_t* arow = wact + (tok_ok ? r : 0) * region + 64 * h;
  auto read_b = [&](v4i (&b)[4], int j) {             // activation fragments of step j
    const int kk = (j - ja) * 256;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const v4i v = *reinterpret_cast<const v4i*>(arow + kk + 16 * s);
      b[s] = tok_ok ? v : v4i{0, 0, 0, 0};
    }
  };
  auto compute = [&](const v4i (&w)[U][RTW], int j) {
    v4i bn[4];
    read_b(bn, j);                                    // issued before the weights are awaited
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        v4i b[4] = {bn[0], bn[1], bn[2], bn[3]};
        if (u + 1 < U && j + u + 1 < jb) read_b(bn, j + u + 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) {
            v4i& a = (s & 1) ? acc1[rt] : acc0[rt];
            a = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][rt][s]), b[s], a,
                                                      0, 0, 0);
          }
      }
    }
  };
  for (int j = ja; j < jb; j += 2 * U) {
    if (j + U < jb) load_w(wb, j + U);
    compute(wa, j);
    if (j + 2 * U < jb) load_w(wa, j + 2 * U);
    if (j + U < jb) compute(wb, j + U);
  }
  v4i acc[RTW];
#pragma unroll
  for (int i = 0; i < RTW; ++i) acc[i] = acc0[i] + acc1[i];

  // ---- 5. K-split reduction and the fused dequant store -----------------
  if constexpr (WK > 1) {
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

  // D[i][j] of the 16x16 MFMA: lane holds column j = lane%16 (token) and rows
  // i = 4*(lane/16) + v (output features), v = 0..3.
  const float dr = xg ? (full_row ? d_lane : __shfl(d_lane, tok_ok ? r : 0, kWave)) : din_r;
  if (!tok_ok) return;
  const float c = gam * dr;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int64_t n = n0 + rt * 16 + 4 * h;
    if (n < N) store_quad(P.y, P.ytype, N, r, n, acc[rt], c);
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
hipError_t launch_cfg(DecodeGroup& g, hipStream_t s) {
  constexpr int WR = kWavesPerBlock / WK;
  constexpr int64_t rows_per_block = (int64_t)WR * RTW * 16;
  int blocks = 0;
  for (int i = 0; i < g.count; ++i) {
    g.block0[i] = blocks;
    blocks += (int)((g.p[i].N + rows_per_block - 1) / rows_per_block);
  }
  if (blocks == 0) return hipSuccess;
  // dynamic LDS: the largest [M][K chunk] activation tile of the group
  size_t lds = 16;
  for (int i = 0; i < g.count; ++i) {
    const int64_t kc_max = ((int64_t)(kActLds / g.M) / 256) * 256;
    const int64_t kc = g.p[i].K < kc_max ? g.p[i].K : kc_max;
    const size_t b = (size_t)(g.M * kc);
    if (b > lds) lds = b;
  }
  hipLaunchKernelGGL((k_gemv_i2s<RTW, WK, U>), dim3((unsigned)blocks), dim3(kThreads), lds, s, g);
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

// K == 0: nothing to contract, every output is 0 (and every token's scale 0).
__global__ void k_zero_outputs(void* __restrict__ y, int ytype, int64_t n, float* __restrict__ d,
                               int M) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) store_out(y, ytype, i, 0, 0.0f);
  if (d && i < M) d[i] = 0.0f;
}

hipError_t launch_zero_outputs(const DecodeProblem& p, int M, hipStream_t s) {
  const int64_t n = (int64_t)M * p.N;
  const int64_t cover = n > M ? n : M;
  hipLaunchKernelGGL(k_zero_outputs, dim3((unsigned)((cover + 255) / 256)), dim3(256), 0, s, p.y,
                     p.ytype, n, p.x ? p.d : nullptr, M);
  return hipGetLastError();
}

template <int RTW, int WK, int U, int XF>
hipError_t launch_fast(DecodeGroup& g, int len_max, hipStream_t s) {
  constexpr int WR = kWavesPerBlock / WK;
  constexpr int64_t rows_per_block = (int64_t)WR * RTW * 16;
  int blocks = 0;
  for (int i = 0; i < g.count; ++i) {
    g.block0[i] = blocks;
    blocks += (int)((g.p[i].N + rows_per_block - 1) / rows_per_block);
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)kWavesPerBlock * g.M * len_max * 256;
  hipLaunchKernelGGL((k_decode_fast<RTW, WK, U, XF>), dim3((unsigned)blocks), dim3(kThreads),
                     lds < 16 ? 16 : lds, s, g, len_max);
  return hipGetLastError();
}

template <int WPB, int XR, int U>
hipError_t launch_one_token(DecodeGroup& g, int len_max, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 15) / 16;
    blocks = b > blocks ? b : blocks;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)WPB * len_max * 256;
  hipLaunchKernelGGL((k_decode1<WPB, XR, U>), dim3((unsigned)blocks, (unsigned)g.count),
                     dim3(WPB * kWave), lds, s, g, len_max);
  return hipGetLastError();
}

hipError_t launch_decode_group(DecodeGroup& g, hipStream_t s) {
  // problems with K == 0 only need zero outputs; keep them away from the
  // MFMA kernels (whose loads assume at least one 64-weight group per row)
  int kept = 0;
  for (int i = 0; i < g.count; ++i) {
    if (g.p[i].K == 0) {
      const hipError_t e = launch_zero_outputs(g.p[i], g.M, s);
      if (e != hipSuccess) return e;
    } else {
      g.p[kept++] = g.p[i];
    }
  }
  g.count = kept;
  if (g.count == 0) return hipSuccess;
  int64_t row_tiles = 0;
  for (int i = 0; i < g.count; ++i) row_tiles += (g.p[i].N + 15) / 16;
  // fast path: each wave's [M][steps * 256] int8 slice fits in LDS
  constexpr int kFastWK = 4;
  int len_max = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t steps = (g.p[i].K + 255) / 256;
    const int len = (int)((steps + kFastWK - 1) / kFastWK);
    if (len > len_max) len_max = len;
  }
  bool all_x = true;
  for (int i = 0; i < g.count; ++i) all_x = all_x && g.p[i].x != nullptr;
  if (g.M == 1 && all_x && len_max <= 16) {         // one token, fused quantize
    if (len_max <= 2) return launch_one_token<4, 1, 4>(g, len_max, s);
    if (len_max <= 4) return launch_one_token<4, 2, 4>(g, len_max, s);
    // longer rows: eight waves per block, so each wave's serial step chain
    // stays at most 8 steps (up to K = 16384)
    int len8 = 0;
    for (int i = 0; i < g.count; ++i) {
      const int len = (int)(((g.p[i].K + 255) / 256 + 7) / 8);
      len8 = len > len8 ? len : len8;
    }
    if (len8 <= 4) return launch_one_token<8, 2, 4>(g, len8, s);
    return launch_one_token<8, 4, 8>(g, len8, s);
  }
  if ((int64_t)kWavesPerBlock * g.M * len_max * 256 <= kActLds) {
    int64_t kmax = 0;
    for (int i = 0; i < g.count; ++i) kmax = g.p[i].K > kmax ? g.p[i].K : kmax;
    const bool fused1 = g.M == 1 && g.p[0].x != nullptr;   // whole-row absmax per wave
    if (len_max <= 4) {
      if (fused1 && kmax <= 8 * 512) return launch_fast<1, kFastWK, 4, 8>(g, len_max, s);
      return launch_fast<1, kFastWK, 4, 0>(g, len_max, s);
    }
    if (fused1 && kmax <= 16 * 512) return launch_fast<1, kFastWK, 8, 16>(g, len_max, s);
    return launch_fast<1, kFastWK, 8, 0>(g, len_max, s);
  }
  if (row_tiles >= 2048) return launch_cfg<1, 2, 8>(g, s);
  return launch_cfg<1, 4, 8>(g, s);
}

hipError_t launch_gemv(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s) {
  if (K % 64 != 0) return launch_generic(packed, gamma, N, K, q, d, M, y, ytype, s);
  DecodeGroup g{};
  g.count = 1;
  g.M = (int)M;
  DecodeProblem& p = g.p[0];
  p.packed = packed;
  p.gamma = gamma;
  p.N = N;
  p.K = K;
  p.qin = q;
  p.din = d;
  p.y = y;
  p.ytype = ytype;
  return launch_decode_group(g, s);
}

}  // namespace bl
