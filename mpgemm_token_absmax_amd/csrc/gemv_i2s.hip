// Decode-time ternary GEMV (1 <= M <= 16 tokens) on gfx950: the fused
// one-token decode group (bf16 activations in: per-token absmax quantization,
// GEMV and dequant in one launch for up to kMaxGroup independent projections),
// the same with the quantization in the kernel for 2..4 tokens, the GEMV over
// int8 activations (bl_gemv, and larger decode groups after one grouped
// quantize launch), and the generic kernel for shapes off the fast paths.
//
// Sources: "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
// notes, Part A 2.3 / 4.1 (I2_S: element-wise multiply-add over 2-bit ternary
// codes and int8 activations quantized with one scale per vector, exact
// sums); bitnet.cpp how-to blog 1.1 (decode streams every weight once per
// token: memory-bandwidth bound) and 1.2 (ternary weights make the products
// adds and subtracts); FairyFuse "融合内核设计" (load activations, walk the
// 2-bit codes, accumulate and write in one pass with no intermediate stores).
//
// Common design (HBM bound: the packed weights are the only large stream):
//  * a block owns 16 output rows of one problem (grid y = problem) and its
//    WPB waves split K into contiguous runs of 256-weight steps;
//  * lane (r = lane%16, h = lane/16) streams 16 bytes (64 weights) of row r
//    per step with one 128-bit load (the 4 lanes of a row read 64 contiguous
//    bytes); the loads of the next U steps are in flight while the current
//    ones are consumed;
//  * each 32-bit group word decodes in registers (9 VALU ops: shift, masks,
//    v_perm_b32 through the code table) to 16 int8 weights in k order and
//    feeds one v_mfma_i32_16x16x64_i8 against the 16 activation bytes of
//    token r over the same k: the ternary x int8 products are exact int32
//    adds;
//  * the waves add their int32 tiles through LDS (exact, order free) and the
//    dequant acc * fl32(gamma * d_t) is fused into the store.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

// Problems with at least this many output rows take the whole-line decode
// kernel (k_decode1w); smaller ones k_decode1, whose shorter steps spread a
// small launch over more waves.
constexpr int64_t kWideN = 8192;

// One-token-style fused decode (quantize in the kernel) up to this many tokens.
constexpr int kFusedTokens = 4;

// One-token launches with at least this many 16-row blocks (two per compute
// unit on MI355X) issue a wave's weight loads only once the block has the
// activation row's maximum (k_decode1), or once the wave's codes are written
// (k_decode1w, from kLateWeightsAfterCodes blocks): x then reaches each
// wave ahead of the weight traffic of the blocks beside it, while those
// blocks keep HBM busy. Measured with a distinct x per launch: 28672 x 8192
// (1792 blocks) 14.8 -> 13.4 us, the 7B-class {q,k,v} (768 blocks) 5.79 ->
// 5.72 us; with one block per compute unit the delay idles the memory system
// (the 7B-class {o}: 3.54 -> 3.82 us), so those launches load the weights
// first.
constexpr int64_t kLateWeightsBlocks = 512;
constexpr int64_t kLateWeightsAfterCodes = 1024;

// Two row tiles per wave in k_gemvq from this many 32-row blocks per launch.
constexpr int64_t kGemvqTwoTileBlocks = 256;

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

// One-token fused decode (M == 1, bf16 x, K <= 65536): per block 16 output
// rows, the WPB waves split K into WPB parts. Each wave loads only its
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
// NORM: the residual add and RMSNorm of the token come first (the group's
// nr, ng, eps, nh): each wave adds its part of r to its part of x, the block
// sums the parts' fp64 sums of squares (one barrier), each wave normalizes
// its part and the block takes the absmax of y (a second barrier); the codes
// are those of y. The first block writes h (and q, d when asked).
// LATE: the first weight batch is issued after the row maximum is known
// instead of right after x (launches with several blocks per compute unit).
template <int WPB, int RTW, int XR, int U, bool NORM = false, bool LATE = false>
__global__ __launch_bounds__(WPB * kWave) void k_decode1(DecodeGroup grp, int len_max) {
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [wave][len_max*256]
  __shared__ v4i red[WPB - 1][RTW][kWave];
  __shared__ uint32_t wmax[WPB];
  __shared__ double wss[NORM ? WPB : 1];
  // LDS of the exact mean-square path (norm launches only)
  __shared__ typename std::conditional<NORM, MsScratch, char>::type msx_lds;

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
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RTW);
  // Every field in one scalar round trip, before the exit test: a scalar
  // load still in flight later would make each LDS wait a full wait (they
  // share a counter and scalar loads complete out of order).
  asm volatile("" ::"s"(packed), "s"(xg), "s"(K), "s"(gptr), "s"(yp), "s"(qp), "s"(dp),
               "s"(ytype), "s"(len_max));
  const uint16_t* nr = NORM ? grp.nr : nullptr;
  const uint16_t* ng = NORM ? grp.ng : nullptr;
  uint16_t* nh = NORM ? grp.nh : nullptr;
  const float eps = NORM ? grp.eps : 0.0f;
  if constexpr (NORM) asm volatile("" ::"s"(nr), "s"(ng), "s"(nh), "s"(eps));
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
  uint4 rv[NORM ? XR : 1], gv[NORM ? XR : 1];
  if constexpr (NORM) {
    const int cb = nch > 0 ? klo / 8 : 0;
    if (nr) {
#pragma unroll
      for (int u = 0; u < XR; ++u)
        rv[u] = reinterpret_cast<const uint4*>(nr)[cb + min(lane + u * kWave, clast)];
    }
#pragma unroll
    for (int u = 0; u < XR; ++u)
      gv[u] = reinterpret_cast<const uint4*>(ng)[cb + min(lane + u * kWave, clast)];
  }
  // gamma by a vector load, issued with x (counted with the vector loads)
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;
  const uint8_t* wrow[RTW];
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    int64_t row = n0 + rt * 16 + (lane & 15);
    row = row < N ? row : N - 1;
    wrow[rt] = packed + row * RB;
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
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!LATE) load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. absmax of the row: quarter maxima, one barrier ----------------
  float sq, dv;
  float rinv = 0.0f;
  if constexpr (NORM) {
    // h = bf16(x + r), the fp64 sum of squares of the row (parts in wave order)
    if (nr) {
#pragma unroll
      for (int u = 0; u < XR; ++u) {
        xv[u].x = add2_bf16(xv[u].x, rv[u].x);
        xv[u].y = add2_bf16(xv[u].y, rv[u].y);
        xv[u].z = add2_bf16(xv[u].z, rv[u].z);
        xv[u].w = add2_bf16(xv[u].w, rv[u].w);
        // h as opaque values (not recomputed later from x and r)
        asm volatile("" : "+v"(xv[u].x), "+v"(xv[u].y), "+v"(xv[u].z), "+v"(xv[u].w));
      }
    }
    double ss = 0.0;
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      if (lane + u * kWave < nch) {
        ss = sumsq2_bf16(xv[u].x, ss);
        ss = sumsq2_bf16(xv[u].y, ss);
        ss = sumsq2_bf16(xv[u].z, ss);
        ss = sumsq2_bf16(xv[u].w, ss);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off, kWave);
    if (lane == 0) wss[wk] = ss;
    __syncthreads();
    double tot = wss[0];
#pragma unroll
    for (int w = 1; w < WPB; ++w) tot += wss[w];
    const float ms = mean_square<WPB * kWave>(tot, K, reinterpret_cast<MsScratch*>(&msx_lds), [&](unsigned long long* b) {
#pragma unroll
      for (int u = 0; u < XR; ++u) {
        if (lane + u * kWave < nch) {
          sq_bins_add2(xv[u].x, b);
          sq_bins_add2(xv[u].y, b);
          sq_bins_add2(xv[u].z, b);
          sq_bins_add2(xv[u].w, b);
        }
        __builtin_amdgcn_sched_barrier(0);    // one chunk at a time: few registers
      }
    });
    rinv = norm_rinv(ms, eps);
    uint32_t mb = 0u;
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      float y[8];
      norm8(xv[u], gv[u], rinv, y);
      uint32_t m8 = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) m8 = max(m8, absbits(y[i]));
      mb = max(mb, lane + u * kWave < nch ? m8 : 0u);
    }
    mb = wave_max_u32(mb);
    if (lane == 0) wmax[wk] = mb;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPB; ++w) mb = max(mb, wmax[w]);
    const float mf = __uint_as_float(mb);
    sq = mb ? 127.0f / mf : 0.0f;
    dv = mb ? mf / 127.0f : 0.0f;
  } else {
    uint32_t m = 0u;
#pragma unroll
    for (int u = 0; u < XR; ++u) m = max(m, lane + u * kWave < nch ? absmax8_bf16(xv[u]) : 0u);
    m = wave_max_u32(m);
    if (lane == 0) wmax[wk] = m;
    __syncthreads();
#pragma unroll
    for (int w = 0; w < WPB; ++w) m = max(m, wmax[w]);
    const float mf = __uint_as_float(m << 16);
    sq = m ? 127.0f / mf : 0.0f;
    dv = m ? mf / 127.0f : 0.0f;
  }
  if (first_block && wk == 0 && lane == 0 && dp) dp[0] = dv;
  if constexpr (LATE) {                     // the row maximum is known: now the weights
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, ja);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 3. int8 codes of this quarter -> the wave's LDS region -----------
  const bool write_q = first_block && qp;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const int c = lane + u * kWave;
    if (c < nch) {
      uint2 qv;
      if constexpr (NORM) {
        float y[8];
        norm8(xv[u], gv[u], rinv, y);
        qv = make_uint2(quant4_f32(&y[0], sq), quant4_f32(&y[4], sq));
        if (first_block && nh) reinterpret_cast<uint4*>(nh + klo)[c] = xv[u];
      } else {
        qv = quant8_bf16(xv[u], sq);
      }
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
  v4i acc0[RTW], acc1[RTW];                           // two chains (even / odd s)
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) acc0[rt] = acc1[rt] = v4i{0, 0, 0, 0};
  const int8_t* arow = wact + 64 * h;
  // the four activation fragments of a step are read from LDS one step ahead
  // of their MFMAs (with one or two waves per SIMD nothing else hides the
  // read latency); steps past the wave's last read its last step's bytes
  auto read_b = [&](v4i (&b)[4], int j) {
    const int8_t* p = arow + (min(j, jb - 1) - ja) * 256;
#pragma unroll
    for (int s = 0; s < 4; ++s) b[s] = *reinterpret_cast<const v4i*>(p + 16 * s);
  };
  auto compute = [&](const v4i (&w)[U][RTW], int j) {
    v4i bc[4], bn[4];
    read_b(bc, j);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (u + 1 < U) read_b(bn, j + u + 1);
      if (j + u < jb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int rt = 0; rt < RTW; ++rt) {
            v4i& a = (s & 1) ? acc1[rt] : acc0[rt];
            a = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][rt][s]), bc[s],
                                                      a, 0, 0, 0);
          }
        }
      }
      if (u + 1 < U) {
#pragma unroll
        for (int s = 0; s < 4; ++s) bc[s] = bn[s];
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
  for (int rt = 0; rt < RTW; ++rt) acc[rt] = acc0[rt] + acc1[rt];

  // ---- 5. sum of the parts, dequant, store ------------------------------
  if (wk > 0) {
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) red[wk - 1][rt][lane] = acc[rt];
  }
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int w = 0; w < WPB - 1; ++w)
#pragma unroll
    for (int rt = 0; rt < RTW; ++rt) acc[rt] += red[w][rt][lane];
  // D layout: lane holds token lane%16 and rows 4*(lane/16) + v; token 0 only
  if ((lane & 15) != 0) return;
#pragma unroll
  for (int rt = 0; rt < RTW; ++rt) {
    const int64_t n = n0 + rt * 16 + 4 * h;
    if (n < N) store_quad(yp, ytype, N, 0, n, acc[rt], gam * dv);
  }
}

// Fused decode for 2..MT tokens: k_decode1 with every token's activations
// quantized in the kernel (each wave its K part of each token; the block
// combines the per-token part maxima with one barrier). The tokens' int8 rows
// sit in the wave's LDS region at a stride of len_max*256 + 16 bytes, so the
// 16 lanes of a fragment read spread over the banks; lane (n, h) reads token
// n's fragments (token MT-1 for n >= MT: those output columns are dropped).
// Tokens M..MT-1 repeat token M-1 (read, quantized, never stored).
// LATE: the first weight batch is issued after the row maxima are known, as
// in k_decode1 (on the 7B-class layer at 4 tokens: 35.5 -> 33.6 us).
template <int WPB, int XR, int U, int MT, bool LATE = false>
__global__ __launch_bounds__(WPB * kWave) void k_decodeT(DecodeGroup grp, int len_max) {
  extern __shared__ __attribute__((aligned(16))) int8_t act[];   // [wave][MT][tstride]
  __shared__ v4i red[WPB - 1][kWave];
  __shared__ uint32_t wmax[MT][WPB];

  const DecodeProblem& P = grp.p[blockIdx.y];
  const int64_t N = P.N;
  const int K = (int)P.K;
  const uint8_t* __restrict__ packed = P.packed;
  const uint16_t* __restrict__ xg = P.x;
  const int64_t ldx = P.ldx;
  const float* gptr = P.gamma;
  void* yp = P.y;
  int8_t* qp = P.q;
  float* dp = P.d;
  const int ytype = P.ytype;
  const int M = grp.M;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  asm volatile("" ::"s"(packed), "s"(xg), "s"(K), "s"(ldx), "s"(gptr), "s"(yp), "s"(qp),
               "s"(dp), "s"(ytype), "s"(M), "s"(len_max));
  if (n0 >= N) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (WPB - 1);
  const int h = lane >> 4;
  const int RB = K / 4;
  const bool first_block = blockIdx.x == 0;
  const int nsteps = (K + 255) / 256;
  const int len = (nsteps + WPB - 1) / WPB;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int klo = min(ja * 256, K);
  const int khi = min(jb * 256, K);
  const int nch = (khi - klo) / 8;
  const int tstride = len_max * 256 + 16;
  int8_t* wact = act + wk * MT * tstride;

  // ---- 1. loads: this part of every token's x, then the first weight batch
  const int cb = nch > 0 ? klo / 8 : 0;
  const int clast = nch > 0 ? nch - 1 : 0;
  uint4 xv[MT][XR];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const uint4* xs = reinterpret_cast<const uint4*>(xg + (int64_t)min(t, M - 1) * ldx) + cb;
#pragma unroll
    for (int u = 0; u < XR; ++u) xv[t][u] = xs[min(lane + u * kWave, clast)];
  }
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
  if constexpr (!LATE) load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. per-token absmax: part maxima, one barrier ---------------------
  float sq[MT], dv[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    uint32_t m = 0u;
#pragma unroll
    for (int u = 0; u < XR; ++u) m = max(m, lane + u * kWave < nch ? absmax8_bf16(xv[t][u]) : 0u);
    m = wave_max_u32(m);
    if (lane == 0) wmax[t][wk] = m;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    uint32_t m = 0u;
#pragma unroll
    for (int w = 0; w < WPB; ++w) m = max(m, wmax[t][w]);
    const float mf = __uint_as_float(m << 16);
    sq[t] = m ? 127.0f / mf : 0.0f;
    dv[t] = m ? mf / 127.0f : 0.0f;
  }
  if (first_block && wk == 0 && lane < M && dp) {
    float dl = dv[0];
#pragma unroll
    for (int t = 1; t < MT; ++t) dl = lane == t ? dv[t] : dl;
    dp[lane] = dl;
  }

  if constexpr (LATE) {                     // the row maxima are known: now the weights
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, ja);
    __builtin_amdgcn_sched_barrier(0);
  }
  // ---- 3. int8 codes of this part of every token -> LDS ------------------
  const bool write_q = first_block && qp;
#pragma unroll
  for (int t = 0; t < MT; ++t) {
#pragma unroll
    for (int u = 0; u < XR; ++u) {
      const int c = lane + u * kWave;
      if (c < nch) {
        const uint2 qv = quant8_bf16(xv[t][u], sq[t]);
        *reinterpret_cast<uint2*>(wact + t * tstride + 8 * c) = qv;
        if (write_q && t < M) *reinterpret_cast<uint2*>(qp + (int64_t)t * K + klo + 8 * c) = qv;
      }
    }
    for (int b = (khi - klo) + 16 * lane; b < (jb - ja) * 256; b += 16 * kWave)
      *reinterpret_cast<v4i*>(wact + t * tstride + b) = v4i{0, 0, 0, 0};
  }
  __builtin_amdgcn_wave_barrier();

  // ---- 4. MFMA over this part's steps ------------------------------------
  v4i acc0 = v4i{0, 0, 0, 0}, acc1 = v4i{0, 0, 0, 0};
  const int tok = min(lane & 15, MT - 1);
  const int8_t* arow = wact + tok * tstride + 64 * h;
  auto compute = [&](const v4i (&w)[U], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v4i b = *reinterpret_cast<const v4i*>(arow + (j + u - ja) * 256 + 16 * s);
          v4i& a = (s & 1) ? acc1 : acc0;
          a = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][s]), b, a, 0, 0, 0);
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

  // ---- 5. sum of the parts, dequant, store -------------------------------
  if (wk > 0) red[wk - 1][lane] = acc;
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int w = 0; w < WPB - 1; ++w) acc += red[w][lane];
  const int n = lane & 15;                              // token of this lane's column
  if (n >= M) return;
  float dn = dv[0];
#pragma unroll
  for (int t = 1; t < MT; ++t) dn = n == t ? dv[t] : dn;
  const int64_t r0 = n0 + 4 * h;
  if (r0 < N) store_quad(yp, ytype, N, n, r0, acc, gam * dn);
}

// One-token fused decode for wide problems (N >= kWideN): the same quantize
// and contraction as k_decode1, with the weight loads shaped for whole cache
// lines. Each load instruction covers 8 rows x 128 contiguous bytes (lane
// (r8 = lane%8, c = lane/8) reads row r8, bytes 16c..16c+15 of the row's
// 128-byte segment), where k_decode1's covers 16 rows x 64 bytes (half
// lines, the other half fetched by the next step). A step is 512 weights of
// the block's 16 rows: two loads (rows 0-7 and 8-15).
// MFMA mapping: lane l of a load holds row r8 + 8i and the 64-weight chunk c of
// the segment. As the A operand of v_mfma_i32_16x16x64_i8 the lane sits at
// row m = l%16 = r8 + 8(c&1) and k-group h = l/16 = c/2, so MFMA rows m < 8
// carry the even chunks and rows m >= 8 the odd chunks of the same 8 real
// rows. The B operand gives column n the activations of chunk 2h + (n&1):
// column 0 pairs with the even chunks, column 1 with the odd ones, and row r
// of half i is D[r][0] + D[8 + r][1] (lanes 0/16 and 33/49 of the result).
// The WPB waves split K into runs of 512-weight steps; SINGLE: every step of
// a wave's run is in one load batch (U >= run length), so no second buffer
// is held. XDMA: x goes to the wave's LDS region by direct-to-LDS loads (no
// registers while the weights are in flight: 7 waves per SIMD at 4 steps
// per wave, which puts the 1792 blocks of a 28672-row problem in one round),
// and each chunk's codes are written in place over the bf16 values, which by
// then are read (chunk c of step u is read before step u writes chunks below
// 32(u + 1), and every chunk below that was read at step u/2 or earlier).
// LATE: the first weight batch is issued after the wave's codes are written
// instead of right after x (launches with many blocks per compute unit).
template <int WPB, int XR, int U, bool SINGLE, bool XDMA = false, bool LATE = false>
__global__ __launch_bounds__(WPB * kWave) void k_decode1w(DecodeGroup grp, int len_max) {
  // [wave][len_max*512] codes; [wave][len_max*1024] with XDMA (the bf16 x first)
  extern __shared__ __attribute__((aligned(16))) int8_t act[];
  __shared__ v4i red[WPB - 1][2][kWave];
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
  const int RB = K / 4;
  const bool first_block = blockIdx.x == 0;

  const int nsteps = (K + 511) / 512;
  const int len = (nsteps + WPB - 1) / WPB;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int klo = min(ja * 512, K);
  const int khi = min(jb * 512, K);
  const int nch = (khi - klo) / 8;
  int8_t* wact = act + wk * len_max * (XDMA ? 1024 : 512);

  // ---- 1. loads: this wave's part of x, then the first weight batch -----
  const uint4* xs = reinterpret_cast<const uint4*>(xg) + (nch > 0 ? klo / 8 : 0);
  const int clast = nch > 0 ? nch - 1 : 0;
  uint4 xv[XDMA ? 1 : XR];
  if constexpr (XDMA) {
#pragma unroll
    for (int u = 0; u < XR; ++u) lds_dma16(xs + min(lane + u * kWave, clast), wact + 1024 * u);
  } else {
#pragma unroll
    for (int u = 0; u < XR; ++u) xv[u] = xs[min(lane + u * kWave, clast)];
  }
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;
  int64_t ra = n0 + r8, rb = n0 + 8 + r8;
  ra = ra < N ? ra : N - 1;
  rb = rb < N ? rb : N - 1;
  const uint8_t* wrow0 = packed + ra * RB;
  const uint8_t* wrow1 = packed + rb * RB;
  v4i wa[U][2], wb[SINGLE ? 1 : U][2];
  auto load_w = [&](auto& dst, int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = max(min(j + u, jb - 1), 0);
      int off = step * 128 + 16 * c;
      off = off < RB ? off : RB - 16;        // lanes past K (masked below)
      dst[u][0] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow0 + off));
      dst[u][1] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow1 + off));
    }
  };
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (!LATE) load_w(wa, ja);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 2. absmax of the row: part maxima, one barrier -------------------
  // XDMA: only the 2U weight loads are younger than the x loads (gamma's, if
  // any, sits between them), so this wait retires x and leaves the weights in
  // flight; the compiler's own wait for direct-to-LDS loads is a full one.
  // LATE: no weight load is in flight yet.
  if constexpr (XDMA) wait_vm<LATE ? 0 : 2 * U>();
  const uint4* xl = reinterpret_cast<const uint4*>(wact) + lane;   // XDMA: chunk lane + 64u
  uint32_t m = 0u;
#pragma unroll
  for (int u = 0; u < XR; ++u) {
    const uint4 v = XDMA ? xl[kWave * u] : xv[u];
    m = max(m, lane + u * kWave < nch ? absmax8_bf16(v) : 0u);
  }
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
    const uint4 v = XDMA ? xl[kWave * u] : xv[u];
    if (cc < nch) {
      const uint2 qv = quant8_bf16(v, sq);
      *reinterpret_cast<uint2*>(wact + 8 * cc) = qv;
      if (write_q) *reinterpret_cast<uint2*>(qp + klo + 8 * cc) = qv;
    }
  }
  // (activation bytes past K in a partial last step are never paired with a
  // weight: those weights are masked to 0)
  __builtin_amdgcn_wave_barrier();
  if constexpr (LATE) {                     // the wave's codes are written: now the weights
    __builtin_amdgcn_sched_barrier(0);
    load_w(wa, ja);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- 4. MFMA over this part's steps ----------------------------------
  // one accumulator per row half: the halves alternate, so an MFMA never
  // waits on the one just issued; each activation fragment is read from LDS
  // next to its two MFMAs (registers: 7 waves per SIMD at 4 steps per wave)
  v4i acc[2];
  acc[0] = acc[1] = v4i{0, 0, 0, 0};
  const int8_t* arow = wact + 64 * (2 * h + (lane & 1));
  auto compute = [&](const auto& w, int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        const uint32_t kmask = (j + u) * 512 + 64 * c < K ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const v4i b = *reinterpret_cast<const v4i*>(arow + (j + u - ja) * 512 + 16 * s);
#pragma unroll
          for (int i = 0; i < 2; ++i)
            acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                decode_word((uint32_t)w[u][i][s] & kmask), b, acc[i], 0, 0, 0);
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
  v4i a2[2] = {acc[0], acc[1]};

  // ---- 5. sum of the parts, even + odd chunks, dequant, store -----------
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
    if (n < N) store_quad(yp, ytype, N, 0, n, o[i], gam * dv);
  }
}

// Decode contraction over int8 activations q [M][K] (scales d), M <= 16.
// The activation fragments are read straight from global memory in the MFMA
// B layout (lane r, h: token r's 64 bytes at k = 256*step + 64h): every block
// of the launch reads the same q, so those loads hit L2, and they travel with
// the weight loads of the same step. No LDS staging and no barrier before the
// MFMAs. A partial last step (K % 256 != 0) zeroes the packed words of the
// lanes past K (code 00 is weight 0), whose loads were clamped into the row.
template <int WPB, int U, int RT>
__global__ __launch_bounds__(WPB * kWave) void k_gemvq(DecodeGroup grp) {
  __shared__ v4i red[WPB - 1][RT][kWave];

  const DecodeProblem& P = grp.p[blockIdx.y];
  const int64_t N = P.N;
  const int K = (int)P.K;
  const uint8_t* __restrict__ packed = P.packed;
  const int8_t* __restrict__ qin = P.qin;
  const float* __restrict__ din = P.din;
  const float* gptr = P.gamma;
  void* yp = P.y;
  const int ytype = P.ytype;
  const int M = grp.M;
  const int64_t n0 = (int64_t)blockIdx.x * (16 * RT);
  // every field in one scalar round trip (a scalar load still in flight later
  // would turn each LDS wait into a full wait)
  asm volatile("" ::"s"(packed), "s"(qin), "s"(din), "s"(gptr), "s"(yp), "s"(K), "s"(ytype),
               "s"(M));
  if (n0 >= N) return;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) & (WPB - 1);
  const int r = lane & 15, h = lane >> 4;
  const int RB = K / 4;
  const int nsteps = (K + 255) / 256;
  const int len = (nsteps + WPB - 1) / WPB;
  const int ja = min(wk * len, nsteps);
  const int jb = min(ja + len, nsteps);
  const int tok = r < M ? r : M - 1;
  const int8_t* qrow = qin + (int64_t)tok * K;
  const uint8_t* wrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    int64_t row = n0 + 16 * rt + r;
    row = row < N ? row : N - 1;
    wrow[rt] = packed + row * RB;
  }

  v4i wa[U][RT], wb[U][RT], qa[U][4], qb[U][4];
  auto load = [&](v4i (&w)[U][RT], v4i (&qf)[U][4], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int step = max(min(j + u, jb - 1), 0);
      int off = step * 64 + 16 * h;
      off = off < RB ? off : RB - 16;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        w[u][rt] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wrow[rt] + off));
      int kk = step * 256 + 64 * h;
      kk = kk < K ? kk : K - 64;
#pragma unroll
      for (int s = 0; s < 4; ++s) qf[u][s] = *reinterpret_cast<const v4i*>(qrow + kk + 16 * s);
    }
  };
  load(wa, qa, ja);
  // epilogue operands, behind the first batch
  const float dtok = ytype ? din[tok] : 0.0f;
  const float gam = ytype ? __builtin_nontemporal_load(gptr) : 0.0f;

  v4i acc0[RT], acc1[RT];                               // two chains (even / odd s)
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc0[rt] = acc1[rt] = v4i{0, 0, 0, 0};
  auto compute = [&](const v4i (&w)[U][RT], const v4i (&qf)[U][4], int j) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j + u < jb) {
        const uint32_t kmask = (j + u) * 256 + 64 * h < K ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            v4i& a = (s & 1) ? acc1[rt] : acc0[rt];
            a = __builtin_amdgcn_mfma_i32_16x16x64_i8(decode_word((uint32_t)w[u][rt][s] & kmask),
                                                      qf[u][s], a, 0, 0, 0);
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
  v4i acc[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) acc[rt] = acc0[rt] + acc1[rt];
  if (wk > 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) red[wk - 1][rt][lane] = acc[rt];
  }
  __syncthreads();
  if (wk > 0) return;
#pragma unroll
  for (int w = 0; w < WPB - 1; ++w)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) acc[rt] += red[w][rt][lane];
  // D layout: lane holds token lane%16 and rows 4*(lane/16) + v
  if (r >= M) return;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t n = n0 + 16 * rt + 4 * h;
    if (n < N) store_quad(yp, ytype, N, r, n, acc[rt], gam * dtok);
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

template <int WPB, int RTW, int XR, int U, bool NORM = false>
hipError_t launch_one_token(DecodeGroup& g, int len_max, hipStream_t s) {
  int64_t blocks = 0, total = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 16 * RTW - 1) / (16 * RTW);
    blocks = b > blocks ? b : blocks;
    total += b;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)WPB * len_max * 256;
  if (!NORM && total >= kLateWeightsBlocks)
    hipLaunchKernelGGL((k_decode1<WPB, RTW, XR, U, NORM, true>),
                       dim3((unsigned)blocks, (unsigned)g.count), dim3(WPB * kWave), lds, s, g,
                       len_max);
  else
    hipLaunchKernelGGL((k_decode1<WPB, RTW, XR, U, NORM, false>),
                       dim3((unsigned)blocks, (unsigned)g.count), dim3(WPB * kWave), lds, s, g,
                       len_max);
  return hipGetLastError();
}

template <int WPB, int XR, int U, bool SINGLE, bool XDMA = false>
hipError_t launch_one_token_w(DecodeGroup& g, int len_max, hipStream_t s) {
  static_assert(!XDMA || XR <= U, "the x staging must fit the wave's LDS region");
  int64_t blocks = 0, total = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 15) / 16;
    blocks = b > blocks ? b : blocks;
    total += b;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)WPB * len_max * (XDMA ? 1024 : 512);
  if (total >= kLateWeightsAfterCodes)
    hipLaunchKernelGGL((k_decode1w<WPB, XR, U, SINGLE, XDMA, true>),
                       dim3((unsigned)blocks, (unsigned)g.count), dim3(WPB * kWave), lds, s, g,
                       len_max);
  else
    hipLaunchKernelGGL((k_decode1w<WPB, XR, U, SINGLE, XDMA, false>),
                       dim3((unsigned)blocks, (unsigned)g.count), dim3(WPB * kWave), lds, s, g,
                       len_max);
  return hipGetLastError();
}

template <int WPB, int XR, int U>
hipError_t launch_tokens(DecodeGroup& g, int len_max, hipStream_t s) {
  constexpr int MT = kFusedTokens;
  int64_t blocks = 0, total = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 15) / 16;
    blocks = b > blocks ? b : blocks;
    total += b;
  }
  if (blocks == 0) return hipSuccess;
  const size_t lds = (size_t)WPB * MT * (len_max * 256 + 16);
  const bool late = total >= kLateWeightsBlocks;
  if (lds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        late ? reinterpret_cast<const void*>(&k_decodeT<WPB, XR, U, MT, true>)
             : reinterpret_cast<const void*>(&k_decodeT<WPB, XR, U, MT, false>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (late)
    hipLaunchKernelGGL((k_decodeT<WPB, XR, U, MT, true>), dim3((unsigned)blocks, (unsigned)g.count),
                       dim3(WPB * kWave), lds, s, g, len_max);
  else
    hipLaunchKernelGGL((k_decodeT<WPB, XR, U, MT, false>), dim3((unsigned)blocks, (unsigned)g.count),
                       dim3(WPB * kWave), lds, s, g, len_max);
  return hipGetLastError();
}

// Longest per-wave run of 512-weight steps in the group when WPB waves split K.
int wide_steps_per_wave(const DecodeGroup& g, int wpb) {
  int len = 0;
  for (int i = 0; i < g.count; ++i) {
    const int l = (int)(((g.p[i].K + 511) / 512 + wpb - 1) / wpb);
    len = l > len ? l : len;
  }
  return len;
}

// Longest per-wave run of 256-weight steps in the group when WPB waves split K.
int steps_per_wave(const DecodeGroup& g, int wpb) {
  int len = 0;
  for (int i = 0; i < g.count; ++i) {
    const int l = (int)(((g.p[i].K + 255) / 256 + wpb - 1) / wpb);
    len = l > len ? l : len;
  }
  return len;
}

template <int WPB, int U, int RT = 1>
hipError_t launch_q(DecodeGroup& g, hipStream_t s) {
  int64_t blocks = 0;
  for (int i = 0; i < g.count; ++i) {
    const int64_t b = (g.p[i].N + 16 * RT - 1) / (16 * RT);
    blocks = b > blocks ? b : blocks;
  }
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemvq<WPB, U, RT>), dim3((unsigned)blocks, (unsigned)g.count),
                     dim3(WPB * kWave), 0, s, g);
  return hipGetLastError();
}

// int8 activations in (p.qin, p.din): enough waves per block that each walks
// at most about 4 steps of K, in one load batch of exactly that many steps.
// Every block reads all M tokens' fragments of its K range (L2 hits), M/4
// times the weight bytes it streams at M = 16; when the launch has at least
// one 32-row block per CU, each wave takes two row tiles that share those
// fragments (half the L2 traffic per weight byte), in half-size load batches.
hipError_t launch_gemvq(DecodeGroup& g, hipStream_t s) {
  int64_t blocks32 = 0;
  for (int i = 0; i < g.count; ++i) blocks32 += (g.p[i].N + 31) / 32;
  const bool two = blocks32 >= kGemvqTwoTileBlocks;
  const int len4 = steps_per_wave(g, 4);
  if (len4 <= 1) return two ? launch_q<4, 1, 2>(g, s) : launch_q<4, 1>(g, s);
  if (len4 == 2) return two ? launch_q<4, 1, 2>(g, s) : launch_q<4, 2>(g, s);
  if (len4 == 3) return two ? launch_q<4, 2, 2>(g, s) : launch_q<4, 3>(g, s);
  if (len4 == 4) return two ? launch_q<4, 2, 2>(g, s) : launch_q<4, 4>(g, s);
  const int len8 = steps_per_wave(g, 8);
  if (len8 == 3) return two ? launch_q<8, 2, 2>(g, s) : launch_q<8, 3>(g, s);
  if (len8 == 4) return two ? launch_q<8, 2, 2>(g, s) : launch_q<8, 4>(g, s);
  return launch_q<16, 2>(g, s);           // 16 waves: no registers for a second tile
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
  bool fused = true;
  for (int i = 0; i < g.count; ++i) fused = fused && g.p[i].x != nullptr;
  if (fused && g.M == 1) {                          // one token: quantize in the kernel
    int64_t nmax = 0;
    for (int i = 0; i < g.count; ++i) nmax = g.p[i].N > nmax ? g.p[i].N : nmax;
    if (nmax >= kWideN) {                           // whole-line weight loads
      const int w4 = wide_steps_per_wave(g, 4);
      if (w4 <= 1) return launch_one_token_w<4, 1, 1, true>(g, w4, s);
      if (w4 == 2) return launch_one_token_w<4, 2, 2, true>(g, w4, s);
      if (w4 == 3) return launch_one_token_w<4, 3, 3, true>(g, w4, s);
      if (w4 == 4) return launch_one_token_w<4, 4, 4, true, true>(g, w4, s);
      const int w8 = wide_steps_per_wave(g, 8);
      if (w8 <= 4) return launch_one_token_w<8, 4, 4, true>(g, w8, s);
      if (w8 <= 8) return launch_one_token_w<8, 8, 2, false>(g, w8, s);   // batches of 2: measured 10% faster than 4 at K = 28672
      const int w16 = wide_steps_per_wave(g, 16);  // <= 8 for K <= 65536
      return launch_one_token_w<16, 8, 4, false>(g, w16, s);
    }
    const int len4 = steps_per_wave(g, 4);
    // one load batch of exactly the steps of the longest wave when it is
    // short (a clamped extra load still costs a request), else batches of 4
    if (len4 <= 1) return launch_one_token<4, 1, 1, 1>(g, len4, s);
    if (len4 == 2) return launch_one_token<4, 1, 1, 2>(g, len4, s);
    if (len4 == 3) return launch_one_token<4, 1, 2, 3>(g, len4, s);
    if (len4 == 4) return launch_one_token<4, 1, 2, 4>(g, len4, s);
    // up to 8 steps per wave: all of them in one load batch (a batch that
    // does not divide the steps issues clamped extra loads, which still cost
    // requests: the 7B-class {down} launch, 6 steps a wave, ran 6.35 us in
    // batches of 4 and 5.89 us in one batch of 6)
    const int len8 = steps_per_wave(g, 8);
    if (len8 == 3) return launch_one_token<8, 1, 2, 3>(g, len8, s);
    if (len8 == 4) return launch_one_token<8, 1, 2, 4>(g, len8, s);
    if (len8 == 5) return launch_one_token<8, 1, 4, 5>(g, len8, s);
    if (len8 == 6) return launch_one_token<8, 1, 4, 6>(g, len8, s);
    if (len8 == 7) return launch_one_token<8, 1, 4, 7>(g, len8, s);
    if (len8 == 8) return launch_one_token<8, 1, 4, 8>(g, len8, s);
    const int len16 = steps_per_wave(g, 16);       // <= 16 for K <= 65536
    if (len16 == 5) return launch_one_token<16, 1, 4, 5>(g, len16, s);
    if (len16 == 6) return launch_one_token<16, 1, 4, 6>(g, len16, s);
    if (len16 == 7) return launch_one_token<16, 1, 4, 7>(g, len16, s);
    if (len16 == 8) return launch_one_token<16, 1, 4, 8>(g, len16, s);
    return launch_one_token<16, 1, 8, 4>(g, len16, s);
  }
  bool tokens_ok = fused && g.M <= kFusedTokens;
  for (int i = 0; i < g.count && tokens_ok; ++i)
    tokens_ok = g.p[i].ldx % 8 == 0 && g.p[i].K <= 32768;
  if (tokens_ok) {                                  // 2..4 tokens: quantize in the kernel
    const int len4 = steps_per_wave(g, 4);
    if (len4 <= 2) return launch_tokens<4, 1, 2>(g, len4, s);
    if (len4 <= 4) return launch_tokens<4, 2, 4>(g, len4, s);
    const int len8 = steps_per_wave(g, 8);
    if (len8 <= 4) return launch_tokens<8, 2, 4>(g, len8, s);
    if (len8 <= 8) return launch_tokens<8, 4, 4>(g, len8, s);
    const int len16 = steps_per_wave(g, 16);       // <= 8 for K <= 32768
    return launch_tokens<16, 4, 4>(g, len16, s);
  }
  if (fused) {
    // several tokens: one launch quantizes every problem's x into its q and
    // d (each block of the GEMV would otherwise redo all M rows), then the
    // GEMV reads those codes
    const hipError_t e = launch_quantize_group(g, s);
    if (e != hipSuccess) return e;
    for (int i = 0; i < g.count; ++i) {
      g.p[i].qin = g.p[i].q;
      g.p[i].din = g.p[i].d;
      g.p[i].x = nullptr;
    }
  }
  return launch_gemvq(g, s);
}

hipError_t launch_decode_norm_group(DecodeGroup& g, hipStream_t s) {
  // the same configurations as the one-token decode (every problem has K)
  const int len4 = steps_per_wave(g, 4);
  if (len4 <= 1) return launch_one_token<4, 1, 1, 1, true>(g, len4, s);
  if (len4 == 2) return launch_one_token<4, 1, 1, 2, true>(g, len4, s);
  if (len4 == 3) return launch_one_token<4, 1, 2, 3, true>(g, len4, s);
  if (len4 == 4) return launch_one_token<4, 1, 2, 4, true>(g, len4, s);
  const int len8 = steps_per_wave(g, 8);
  if (len8 == 3) return launch_one_token<8, 1, 2, 3, true>(g, len8, s);
  if (len8 == 4) return launch_one_token<8, 1, 2, 4, true>(g, len8, s);
  if (len8 <= 8) return launch_one_token<8, 1, 4, 4, true>(g, len8, s);
  const int len16 = steps_per_wave(g, 16);
  if (len16 <= 8) return launch_one_token<16, 1, 4, 4, true>(g, len16, s);
  return hipErrorInvalidValue;                      // K > 32768: rejected at the boundary
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
