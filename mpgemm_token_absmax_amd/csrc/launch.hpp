// Internal launchers behind the C ABI (include/bitlinear.h). Arguments are
// already validated by api.cpp; each launcher only enqueues work on `s`.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

constexpr int kMaxGroup = 8;        // problems per decode-group launch
constexpr int kMaxDecodeM = 16;     // tokens of the decode kernels

// Prefill GEMM: weights per K step, the largest K of the MFMA path (per-lane
// load offsets stay 32-bit), and the split-K rule (plan_gemm_group).
constexpr int kGemmBK = 128;
constexpr int64_t kGemmMaxK = (int64_t)1 << 24;
constexpr int64_t kSplitBlocks = 1024;   // split-K aims at about this many blocks
constexpr int64_t kSplitMinSteps = 4;    // K steps per split, at least
constexpr int64_t kSplitMaxBlocks = 256; // launches with at least this many tiles run unsplit
constexpr int64_t kSplitMinK = 32;       // K steps of a launch worth splitting, at least
constexpr int64_t kMaxSplits = 8;

// fp32 packing: exponent bins of |w| per workgroup (kBins of them, one
// thread each) over at most kMaxBinBlocks workgroups.
constexpr int kBinThreads = 256;
constexpr int kBins = 256;
constexpr int kMaxBinBlocks = 1024;
int64_t bin_blocks(int64_t n);

// One GEMV of a decode launch. Activations come either as bf16 x (quantized
// in-kernel; q and d, when not NULL, receive the codes and scales) or as
// int8 qin with scales din.
struct DecodeProblem {
  const uint8_t* packed;
  const float* gamma;
  const uint16_t* x;
  int8_t* q;
  float* d;
  const int8_t* qin;
  const float* din;
  void* y;
  int64_t N;
  int64_t K;
  int64_t ldx;
  int ytype;
};

// Kernel argument of a decode launch. The header (count, M and each
// problem's first block) comes first so one scalar load finds the problem of
// a block.
struct DecodeGroup {
  int count;
  int M;
  int block0[kMaxGroup];      // first block of each problem (set by the launcher)
  DecodeProblem p[kMaxGroup];
  // One-token groups with the residual add and RMSNorm folded in (every
  // problem reads the same x and K): residual (or NULL), norm weight [K], h
  // out (or NULL), eps.
  const uint16_t* nr;
  const uint16_t* ng;
  uint16_t* nh;
  float eps;
};

hipError_t launch_decode_group(DecodeGroup& g, hipStream_t s);
// M == 1, every problem with the same x and K (K % 64 == 0): h = x (+ r),
// RMSNorm with g and eps, per-token quantize, then each problem's GEMV.
hipError_t launch_decode_norm_group(DecodeGroup& g, hipStream_t s);
// bf16 x -> q, d of every problem of a group (M tokens each), one launch.
hipError_t launch_quantize_group(const DecodeGroup& g, hipStream_t s);

// qs (may be NULL): qs[t] = sum_k q[t][k], exact.
hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               float* d, int* qs, hipStream_t s);
// One scale for the whole tensor; maxb: M words of workspace (row maxima).
hipError_t launch_quantize_act_tensor(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                      int8_t* q, float* d, int* qs, uint32_t* maxb,
                                      hipStream_t s);

// Residual add + RMSNorm + per-token absmax int8 (r and h_out may be NULL;
// h_out may be x or r itself). x, r, h_out share the row stride ldx.
constexpr int64_t kRmsNormFastMaxK = 32768;
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* r, const uint16_t* g,
                                float eps, int64_t M, int64_t K, int64_t ldx, uint16_t* h_out,
                                int8_t* q, float* d, int* qs, hipStream_t s);

// Base-3 weights, five per byte: rows of 64*ceil(K/320) bytes.
hipError_t launch_pack_t3(const void* w, bool f32, int64_t N, int64_t K, uint8_t* packed,
                          const float* gamma, hipStream_t s);
hipError_t launch_gemv_t3(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                          hipStream_t s);
// One token: quantize in the kernel (K % 16 == 0, K <= 65536); several tokens:
// quantize every problem's x into its q and d, then launch_gemv_t3 per problem.
hipError_t launch_decode_group_t3(DecodeGroup& g, hipStream_t s);
// Exponent bins and gamma of an fp32 matrix (the first two launches of the
// fp32 I2_S packing): gamma[0] = fl32(exact sum |w| / (N*K)).
hipError_t launch_absmean_gamma(const float* w, int64_t N, int64_t K, float* gamma, void* ws,
                                hipStream_t s);

size_t pack_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_pack_f32(const float* w, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           void* ws, hipStream_t s);
hipError_t launch_pack_ternary(const int8_t* w, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t s);

// y layout: [M][N]; ytype: 0 = int32 acc, 1 = fp32, 2 = bf16 bits.
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s);
// qs (may be NULL): the token sums of q; with them the GEMM runs on offset
// weights (w + 1) and subtracts qs[t] in the epilogue. ws (may be NULL: no
// split): int32 partial sums of a split-K launch, plan_gemm_group's
// ws_bytes at least.
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, const int* qs, int64_t M, void* y,
                       int ytype, void* ws, hipStream_t s);
// Several GEMMs over the same int8 activations q [M][K] (scales d): problem i
// has its own packed [N_i][K/4], gamma, y [M][N_i] and output type.
struct GemmProblem {
  const uint8_t* packed;
  const float* gamma;
  void* y;
  int64_t N;
  int ytype;
};
hipError_t launch_gemm_group(const GemmProblem* p, int count, int64_t K, const int8_t* q,
                             const float* d, const int* qs, int64_t M, void* ws, hipStream_t s);

// How a grouped GEMM is launched: which problems take 128x256 tiles (big),
// the tile of the rest (32x128 or 64x128), and the K split of that launch
// with the workspace it needs (0 when it does not split or mfma is false:
// then the GEMV or the generic kernel runs).
struct GemmPlan {
  bool mfma;
  int nbig, nsmall;
  int big[kMaxGroup], small[kMaxGroup];
  bool small32;
  int splits;
  size_t ws_bytes;
};
GemmPlan plan_gemm_group(const int64_t* Ns, int count, int64_t K, int64_t M);

// The allocation-free grouped GEMM's workspace: a file-scope device array of
// this many bytes (the most a split plan needs); *ptr = its address on the
// current device (looked up on the first call on each device).
constexpr size_t kNoAllocScratchBytes = (size_t)1024 * 64 * 128 * 4;
static_assert(kSplitBlocks * 64 * 128 * sizeof(int) <= kNoAllocScratchBytes,
              "a split plan's partial sums fit the allocation-free workspace");
hipError_t noalloc_scratch(void** ptr);

// Shapes off the fast paths (K % 64 != 0): one thread per output element.
hipError_t launch_generic(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                          hipStream_t s);

}  // namespace bl
