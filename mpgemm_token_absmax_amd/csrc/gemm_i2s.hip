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
// Block = 4 waves as WRW (feature rows) x WTW (tokens); wave tile = RT*16
// output features x TT*16 tokens; K advances 128 weights per step (two MFMA
// sub-steps of 64).
//  * Both operands of a step are staged in LDS by direct-to-LDS loads
//    (global_load_lds_dwordx4: no register staging) into two stage buffers,
//    one barrier per step: a wave reads all of step ks's fragments into
//    registers, then issues step ks+1's loads, which land while its MFMAs
//    run. LDS has 64 4-byte banks; a 64-bit read serves lanes 0-31 in one
//    cycle and 32-63 in the next, a 128-bit read serves 16 lanes a cycle,
//    the lanes of a 32-lane half being split by the parity of lane bits
//    2..4 (measured with the bank-conflict counter). Conflict-free layouts
//    for the fragment reads under that rule: chunk c of activation row t
//    (128 bytes) sits at chunk position c ^ swz(t) (swz below), and a
//    16-row group of packed weights is stored as [bytes 0-15 of rows 0..15 |
//    bytes 16-31 of rows 0..15].
//  * Lane (r = lane%16, h = lane/16) of a sub-step s covers k = 32h + 16s ..
//    +15 of the step on both operands: the 32-bit packed word of that k range
//    decodes (9 VALU ops) to 16 int8 weights that the MFMA pairs with the 16
//    activation bytes of the same k range, so the MFMA's 64-term dot is
//    exactly the sum over those k.
//  * Loads are unconditional with clamped addresses; out-of-range tokens and
//    rows only reach outputs that are never stored, and weights past K are
//    zeroed before the MFMA, so stale activations there add nothing. The
//    vector ALU work of a step is kept to the decode (it does not hide under
//    the other wave's MFMAs): load addresses are a uniform tile base plus a
//    fixed per-lane 32-bit offset, and shapes with K % 128 == 0 (the kernel
//    flag KFULL) compile no code for a partial last step.
//  * Blocks are ordered so that consecutive blocks on one XCD (blocks are
//    dealt to the 8 XCDs round robin) share a token tile, whose activations
//    then stay in that XCD's L2.
// Accumulation is exact int32; the dequant (acc * fl32(gamma * d_t)) is fused
// into the store.
//  * Offset weights (when the caller passes the token sums qs[t] = sum_k
//    q[t][k]): the matrix cores get w + 1 in {0, 1, 2} instead of w in
//    {-1, 0, +1}, so the accumulator holds acc + qs[t] exactly and the
//    epilogue subtracts qs[t]. -1 is the byte 0xFF; operands of 0..2 switch
//    far fewer multiplier bits, the matrix cores draw less power and the
//    clock (power-limited under a full matrix load) rises: measured 3-7%
//    more throughput on the 100B-class shapes. The decode is the same 9 ops
//    with other tables.
#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace bl {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = kGemmBK;             // weights (k) per step
constexpr int kXcds = 8;

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

// Chunk swizzle of activation row t: u = (t/2) % 8 with bit 1 flipped when
// bits 1 and 2 of u differ. Lanes served in one cycle of a 128-bit fragment
// read then cover all 16 16-byte slots of a 256-byte bank row.
__device__ __forceinline__ int swz(int t) {
  const int u = (t >> 1) & 7;
  return u ^ ((((u >> 1) ^ (u >> 2)) & 1) << 1);
}

// decode_word with w + 1 in place of w (code 00 -> 1, 01 -> 2, 10 -> 0): the
// same selectors into other tables (bytes 01 02 00 01 for fields 0 and 2;
// for fields 1 and 3, selector 0 -> byte 0 of the second source, 4 -> byte 0
// of the first, 8 -> the sign of byte 1 of the second, which is 0).
constexpr uint32_t kLutLoP1 = 0x01000201u;
constexpr uint32_t kLutHiP1S1 = 0x00000001u;
constexpr uint32_t kLutHiP1S0 = 0x00000002u;

__device__ __forceinline__ v4i decode_word_p1(uint32_t word) {
  const uint32_t hi = word >> 4;
  v4i r;
  r.x = (int)__builtin_amdgcn_perm(0u, kLutLoP1, word & 0x03030303u);
  r.y = (int)__builtin_amdgcn_perm(kLutHiP1S0, kLutHiP1S1, word & 0x0C0C0C0Cu);
  r.z = (int)__builtin_amdgcn_perm(0u, kLutLoP1, hi & 0x03030303u);
  r.w = (int)__builtin_amdgcn_perm(kLutHiP1S0, kLutHiP1S1, hi & 0x0C0C0C0Cu);
  return r;
}

// Kernel argument of a GEMM launch: the problems that share q, each owning
// a contiguous range of row blocks [rb0[i], rb0[i+1]). With splits > 1 the K
// steps of every tile are cut into `splits` contiguous ranges, one block per
// range, and each block stores its exact int32 partial tile at ws + wsoff[i]
// + split * M * N (layout [split][M][N]); k_gemm_finalize adds them.
struct GemmArgs {
  int count;
  int total_rb;
  int splits;
  int rb0[kMaxGroup + 1];
  int64_t wsoff[kMaxGroup];
  int* ws;
  GemmProblem p[kMaxGroup];
};

// Store 4 int32 partial sums ws[t][n .. n+3] of an [M][N] partial tile.
__device__ __forceinline__ void store_partial(int* ws, int64_t N, int64_t t, int64_t n, v4i a) {
  const int64_t base = t * N + n;
  if (n + 3 < N && (N & 3) == 0) {
    *reinterpret_cast<v4i*>(ws + base) = a;
    return;
  }
  const int v[4] = {a.x, a.y, a.z, a.w};
  for (int i = 0; i < 4 && n + i < N; ++i) ws[base + i] = v[i];
}

template <int RT, int TT, int WRW>
struct GemmCfg {
  static constexpr int WTW = 4 / WRW;
  static constexpr int BN = WRW * RT * 16;            // output features per block
  static constexpr int BM = WTW * TT * 16;            // tokens per block
  static constexpr int kBBytes = BM * kBK;            // activation tile per stage
  static constexpr int kABytes = BN * (kBK / 4);      // packed weight tile per stage
  static constexpr int kStage = kBBytes + kABytes;
  static constexpr int kLds = 2 * kStage;              // double buffered
  static constexpr int kBLoads = kBBytes / (16 * kThreads);   // per wave per stage
  static constexpr int kALoads = (kABytes + 16 * kThreads - 1) / (16 * kThreads);
  static_assert(kBBytes % (16 * kThreads) == 0, "activation tile must split over the block");
};

// Direct-to-LDS loads of step ks into its stage (see k_gemm_i2s). Each
// address is a uniform base (the block's tile origin, advanced by the step)
// plus a per-lane 32-bit offset that stays fixed for the whole loop.
// The last step when K % 128 == 64 reaches past K: there a lane's activation
// chunk is moved 64 weights back (valid memory; its weights are zeroed
// before the MFMA) and its packed half 16 bytes back (bwrap, awrap).
template <int NB, int NA, int kStage, int kBBytes, int BN, bool KFULL>
__device__ __forceinline__ void issue_step(int8_t* smem, int ks, int wv, const int8_t* bbase,
                                           const uint32_t (&boff)[NB], uint32_t bwrap,
                                           const uint8_t* abase, const uint32_t (&aoff)[NA],
                                           uint32_t awrap, int nfull) {
  int8_t* st = smem + (ks & 1) * kStage;
  const int64_t kb = (int64_t)ks * kBK;
  const int8_t* bb = bbase + kb;
  const uint8_t* ab = abase + kb / 4;
  if (KFULL || ks < nfull) {                          // a whole step
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_dma16(bb + boff[i], st + (i * 4 + wv) * 1024);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if ((i * 4 + wv) * 32 < BN)                     // wave-uniform: rows of the tile exist
        lds_dma16(ab + aoff[i], st + kBBytes + (i * 4 + wv) * 1024);
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) lds_dma16(bb + (boff[i] - bwrap), st + (i * 4 + wv) * 1024);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      if ((i * 4 + wv) * 32 < BN)
        lds_dma16(ab + (aoff[i] - awrap), st + kBBytes + (i * 4 + wv) * 1024);
  }
}

// OFF: offset weights (w + 1) and qs[t] subtracted in the epilogue.
// KFULL: K % 128 == 0, every step whole (no code for a partial last step).
template <int RT, int TT, int WRW, bool OFF, bool KFULL>
__global__ __launch_bounds__(kThreads, (RT * TT >= 64 ? 1 : 2)) void k_gemm_i2s(const GemmArgs g, int64_t K,
                                                          const int8_t* __restrict__ q,
                                                          const float* __restrict__ d,
                                                          const int* __restrict__ qs, int64_t M,
                                                          int n_tok_blocks) {
  using C = GemmCfg<RT, TT, WRW>;
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];

  // XCD-aware order: block b runs on XCD b % 8; give each XCD a contiguous run
  // of the tile sequence (token-tile major) so its blocks share activations.
  // The splits of a tile are consecutive in this order (they read the same
  // rows of packed weights and tokens, at different K).
  const int n_row_blocks = g.total_rb;
  const int S = g.splits;
  const int nb = n_row_blocks * n_tok_blocks * S;
  int lin = blockIdx.x;
  if (nb % kXcds == 0) lin = (blockIdx.x % kXcds) * (nb / kXcds) + blockIdx.x / kXcds;
  const int split = lin % S;
  lin /= S;
  const int tb = lin / n_row_blocks;
  int rb = lin % n_row_blocks;
  int pi = 0;                                         // problem of this block (uniform)
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < g.count && rb >= g.rb0[i]) pi = i;
  rb -= g.rb0[pi];
  const uint8_t* __restrict__ packed = g.p[pi].packed;
  const int64_t N = g.p[pi].N;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;   // 4 waves
  const int wr = wv % WRW, wt = wv / WRW;
  const int r = lane & 15, h = lane >> 4;
  const int64_t RB = K / 4;
  const int64_t n_blk = (int64_t)rb * C::BN;
  const int64_t m_blk = (int64_t)tb * C::BM;
  const int nks_all = (int)((K + kBK - 1) / kBK);
  const int nfull = (int)(K / kBK);                   // steps with all 128 weights
  // this block's steps [ks0, nks): split s of S takes a contiguous share
  const int ks0 = (int)((int64_t)nks_all * split / S);
  const int nks = (int)((int64_t)nks_all * (split + 1) / S);

  // ---- per-lane source addresses of the direct-to-LDS loads ---------------
  // activations: wave instruction i covers tile rows t = (i*4 + wv)*8 + l/8;
  // LDS chunk p = l%8 of row t holds global chunk p ^ swz(t), and swz(t)
  // depends on (t/2) % 8 == (4*(wv%2) + l/16) % 8 only, the same for every i
  // (offsets from the tile origin: at most 256*K and 128*K/4, below 2^32 for
  // K <= 2^24, which the launcher ensures)
  const int8_t* bbase = q + m_blk * K;
  uint32_t boff[C::kBLoads];
  const int bchunk = 16 * ((lane & 7) ^ swz(2 * (4 * (wv & 1) + (lane >> 4))));
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i) {
    const int t = (i * 4 + wv) * 8 + (lane >> 3);
    int64_t tok = m_blk + t;
    tok = tok < M ? tok : M - 1;
    boff[i] = (uint32_t)((tok - m_blk) * K + bchunk);
  }
  const uint32_t bwrap = bchunk >= 64 ? 64u : 0u;
  // packed weights: 32 bytes per row per step; wave instruction i covers rows
  // (i*4 + wv)*32 + 16*(l/32) + l%16, byte half (l/16)%2
  const uint8_t* abase = packed + n_blk * RB;
  uint32_t aoff[C::kALoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int row = (i * 4 + wv) * 32 + 16 * (lane >> 5) + (lane & 15);
    int64_t n = n_blk + (row < C::BN ? row : C::BN - 1);
    n = n < N ? n : N - 1;
    aoff[i] = (uint32_t)((n - n_blk) * RB + 16 * (lane >> 4 & 1));
  }
  const uint32_t awrap = (lane >> 4 & 1) ? 16u : 0u;
  v4i acc[RT][TT];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  if (ks0 < nks)
    issue_step<C::kBLoads, C::kALoads, C::kStage, C::kBBytes, C::BN, KFULL>(smem, ks0, wv, bbase,
                                                                     boff, bwrap, abase, aoff,
                                                                     awrap, nfull);

  for (int ks = ks0; ks < nks; ++ks) {
    wait_vm<0>();             // this wave's loads of step ks have landed
    __syncthreads();          // every wave's have; every wave is done reading step ks-1

    // All fragments of step ks go to registers before step ks+1 is issued: the
    // compiler cannot tell the two stages apart and would otherwise wait for
    // the new loads before these reads, serialising load and compute.
    const int8_t* st = smem + (ks & 1) * C::kStage;
    const int8_t* sa = st + C::kBBytes;
    const int64_t kb = (int64_t)ks * kBK;
    // packed words of the two sub-steps: row rt*16 + r, bytes 8h .. 8h+7
    uint2 aw[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      aw[rt] = *reinterpret_cast<const uint2*>(sa + (wr * RT + rt) * 512 + (h >> 1) * 256 +
                                               r * 16 + 8 * (h & 1));
    v4i bf[2][TT];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int tt = 0; tt < TT; ++tt) {
        const int t = wt * TT * 16 + tt * 16 + r;
        const int p = (2 * h + s) ^ swz(t);
        bf[s][tt] = *reinterpret_cast<const v4i*>(st + t * kBK + 16 * p);
      }

    // unconditional, so the wait counts stay exact across the loop: the last
    // step re-loads itself into the idle buffer, which nothing reads again
    issue_step<C::kBLoads, C::kALoads, C::kStage, C::kBBytes, C::BN, KFULL>(
        smem, ks + 1 < nks ? ks + 1 : ks, wv, bbase, boff, bwrap, abase, aoff, awrap, nfull);

    if (!KFULL && ks >= nfull) {    // the last step of a K % 128 == 64 shape
      const bool kin = kb + 32 * h < K;               // this lane's 32 weights exist
      constexpr uint32_t kZeroCodes = OFF ? 0xAAAAAAAAu : 0u;   // words that decode to 0
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        aw[rt].x = kin ? aw[rt].x : kZeroCodes;
        aw[rt].y = kin ? aw[rt].y : kZeroCodes;
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const uint32_t word = s == 0 ? aw[rt].x : aw[rt].y;
        const v4i af = OFF ? decode_word_p1(word) : decode_word(word);
#pragma unroll
        for (int tt = 0; tt < TT; ++tt)
          acc[rt][tt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[s][tt], acc[rt][tt], 0, 0, 0);
      }
    }
    // Schedule of the step: the fragment reads, then the next step's loads,
    // then vector ALU and MFMA groups in alternation. With these groups the
    // scheduler issues the loads right after the reads (a whole step ahead of
    // their wait) and places most of the decode ahead of an unbroken run of
    // MFMAs, so that with two waves per SIMD one wave's decode overlaps the
    // other's matrix work. Its own order sank the loads to the end of the
    // loop and spread the decode through the MFMAs: 8-11% slower on the
    // 100B-class shapes.
    __builtin_amdgcn_sched_group_barrier(0x100, RT + 2 * TT, 0);                  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x020, C::kBLoads + C::kALoads, 0);      // global loads
    __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);                           // VALU
#pragma unroll
    for (int i = 0; i < 2 * RT * TT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 1, 0);                          // VALU
    }
  }

  wait_vm<0>();                // no LDS write may still be in flight when the block ends

  // D layout: lane holds token (column) lane%16 and features 4*(lane/16) + v.
  if (S > 1) {                 // raw partial sums (offset form included): finalized later
    int* wsp = g.ws + g.wsoff[pi] + (int64_t)split * M * N;
#pragma unroll
    for (int tt = 0; tt < TT; ++tt) {
      const int64_t tok = m_blk + wt * TT * 16 + tt * 16 + r;
      if (tok >= M) continue;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int64_t n = n_blk + wr * RT * 16 + rt * 16 + 4 * h;
        if (n < N) store_partial(wsp, N, tok, n, acc[rt][tt]);
      }
    }
    return;
  }
  const int ytype = g.p[pi].ytype;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt) {
    const int64_t tok = m_blk + wt * TT * 16 + tt * 16 + r;
    if (tok >= M) continue;
    const float c = ytype ? g.p[pi].gamma[0] * d[tok] : 0.0f;
    if constexpr (OFF) {
      const int st = qs[tok];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) acc[rt][tt] -= v4i{st, st, st, st};
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int64_t n = n_blk + wr * RT * 16 + rt * 16 + 4 * h;
      if (n < N) store_quad(g.p[pi].y, ytype, N, tok, n, acc[rt][tt], c);
    }
  }
}

// The partial tiles of a split launch, added in split order (int32 sums are
// exact, so the order does not change them), the token sums subtracted for
// offset weights, and the same dequant and store as the unsplit epilogue:
// the outputs are bit-identical. Grid: x = 256-thread blocks over the
// [M][ceil(N/4)] quads of the largest problem, y = problem.
__global__ __launch_bounds__(256) void k_gemm_finalize(const GemmArgs g, const float* __restrict__ d,
                                                       const int* __restrict__ qs, int64_t M,
                                                       bool off) {
  const GemmProblem& P = g.p[blockIdx.y];
  const int64_t N = P.N;
  const int64_t qpr = (N + 3) / 4;                    // quads per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= M * qpr) return;
  const int64_t t = i / qpr, n = 4 * (i % qpr);
  const int* wsp = g.ws + g.wsoff[blockIdx.y] + t * N + n;
  const bool vec = n + 3 < N && (N & 3) == 0;
  v4i acc = v4i{0, 0, 0, 0};
  for (int sp = 0; sp < g.splits; ++sp) {
    const int* src = wsp + (int64_t)sp * M * N;
    if (vec) {
      acc += *reinterpret_cast<const v4i*>(src);
    } else {
      acc.x += src[0];
      if (n + 1 < N) acc.y += src[1];
      if (n + 2 < N) acc.z += src[2];
      if (n + 3 < N) acc.w += src[3];
    }
  }
  if (off) acc -= v4i{qs[t], qs[t], qs[t], qs[t]};
  const float c = P.ytype ? P.gamma[0] * d[t] : 0.0f;
  store_quad(P.y, P.ytype, N, t, n, acc, c);
}

template <int RT, int TT, int WRW>
GemmArgs make_args(const GemmProblem* const* p, int count, int splits, int* ws, int64_t M) {
  using C = GemmCfg<RT, TT, WRW>;
  GemmArgs a{};
  int64_t rb = 0, off = 0;
  for (int i = 0; i < count; ++i) {
    a.rb0[i] = (int)rb;
    a.p[i] = *p[i];
    a.wsoff[i] = off;
    rb += (p[i]->N + C::BN - 1) / C::BN;
    off += (int64_t)splits * M * p[i]->N;
  }
  a.count = count;
  a.rb0[count] = (int)rb;
  a.total_rb = (int)rb;
  a.splits = splits;
  a.ws = ws;
  return a;
}

template <int RT, int TT, int WRW, bool OFF, bool KFULL>
hipError_t launch_cfg(const GemmProblem* const* p, int count, int64_t K, const int8_t* q,
                      const float* d, const int* qs, int64_t M, int splits, int* ws,
                      hipStream_t s) {
  using C = GemmCfg<RT, TT, WRW>;
  const GemmArgs a = make_args<RT, TT, WRW>(p, count, splits, ws, M);
  const int64_t ntb = (M + C::BM - 1) / C::BM;
  if ((int64_t)a.total_rb * ntb * splits > INT32_MAX) return hipErrorInvalidValue;
  if (C::kLds > 64 * 1024) {
    const hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&k_gemm_i2s<RT, TT, WRW, OFF, KFULL>),
        hipFuncAttributeMaxDynamicSharedMemorySize, C::kLds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((k_gemm_i2s<RT, TT, WRW, OFF, KFULL>),
                     dim3((unsigned)(a.total_rb * ntb * splits)), dim3(kThreads), C::kLds, s, a, K,
                     q, d, qs, M, (int)ntb);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  int64_t nmax = 0;
  for (int i = 0; i < count; ++i) nmax = p[i]->N > nmax ? p[i]->N : nmax;
  const int64_t quads = M * ((nmax + 3) / 4);
  hipLaunchKernelGGL(k_gemm_finalize, dim3((unsigned)((quads + 255) / 256), (unsigned)count),
                     dim3(256), 0, s, a, d, qs, M, OFF);
  return hipGetLastError();
}

template <int RT, int TT, int WRW>
hipError_t launch_tiles(bool off, bool full, const GemmProblem* const* p, int count, int64_t K,
                        const int8_t* q, const float* d, const int* qs, int64_t M, int splits,
                        int* ws, hipStream_t s) {
  if (off)
    return full ? launch_cfg<RT, TT, WRW, true, true>(p, count, K, q, d, qs, M, splits, ws, s)
                : launch_cfg<RT, TT, WRW, true, false>(p, count, K, q, d, qs, M, splits, ws, s);
  return full ? launch_cfg<RT, TT, WRW, false, true>(p, count, K, q, d, qs, M, splits, ws, s)
              : launch_cfg<RT, TT, WRW, false, false>(p, count, K, q, d, qs, M, splits, ws, s);
}

}  // namespace

hipError_t launch_gemm_group(const GemmProblem* p, int count, int64_t K, const int8_t* q,
                             const float* d, const int* qs, int64_t M, void* ws, hipStream_t s) {
  hipError_t e = hipSuccess;
  int64_t Ns[kMaxGroup];
  for (int i = 0; i < count; ++i) Ns[i] = p[i].N;
  const GemmPlan pl = plan_gemm_group(Ns, count, K, M);
  if (!pl.mfma) {
    for (int i = 0; i < count && e == hipSuccess; ++i)
      e = K % 64 != 0 || K > kGemmMaxK ? launch_generic(p[i].packed, p[i].gamma, p[i].N, K, q, d, M, p[i].y,
                                       p[i].ytype, s)
                      : launch_gemv(p[i].packed, p[i].gamma, p[i].N, K, q, d, M, p[i].y,
                                    p[i].ytype, s);
    return e;
  }
  const GemmProblem* big[kMaxGroup];
  const GemmProblem* small[kMaxGroup];
  for (int j = 0; j < pl.nbig; ++j) big[j] = &p[pl.big[j]];
  for (int j = 0; j < pl.nsmall; ++j) small[j] = &p[pl.small[j]];
  // offset weights need the token sums and |acc + qs[t]| <= 254*K in int32
  const bool off = qs != nullptr && 254 * K <= INT32_MAX;
  const bool full = K % kBK == 0;
  if (pl.nbig) e = launch_tiles<4, 8, 2>(off, full, big, pl.nbig, K, q, d, qs, M, 1, nullptr, s);
  if (e == hipSuccess && pl.nsmall) {
    // without a workspace the launch runs unsplit (same results)
    const int sp = ws ? pl.splits : 1;
    int* w = static_cast<int*>(ws);
    e = pl.small32 ? launch_tiles<1, 4, 2>(off, full, small, pl.nsmall, K, q, d, qs, M, sp, w, s)
                   : launch_tiles<2, 4, 2>(off, full, small, pl.nsmall, K, q, d, qs, M, sp, w, s);
  }
  return e;
}

// ---- the workspace of the allocation-free grouped GEMM ----------------------
// A split plan holds at most kSplitBlocks blocks of at most 64 x 128 outputs
// (splits * blocks <= kSplitBlocks), so its partial sums never exceed
// kSplitBlocks * 64 * 128 * 4 bytes = kNoAllocScratchBytes. The array lives on
// every device the library runs on until the process ends. In host code its
// name is a host-side stand-in, never a device address: only the pointer
// hipGetSymbolAddress returns (per device) reaches kernels.
static __device__ __align__(256) int scratch[kNoAllocScratchBytes / sizeof(int)];

namespace {
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev[kMaxDevices];            // device address of `scratch`, per device
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev[dev]) {                 // first call on this device (it is current)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_dev[dev] = p;
  }
  *ptr = scratch_dev[dev];
  return hipSuccess;
}

hipError_t launch_gemm(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, const int* qs, int64_t M, void* y,
                       int ytype, void* ws, hipStream_t s) {
  const GemmProblem p{packed, gamma, y, N, ytype};
  return launch_gemm_group(&p, 1, K, q, d, qs, M, ws, s);
}

}  // namespace bl
