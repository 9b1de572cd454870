// Host-side planning of the library's launches, shared by the kernels'
// launchers and the C ABI's validation (workspace sizes): no device code, so
// the validation layer also builds with a host compiler alone.
#include "launch.hpp"

namespace bl {

// Workgroups of the exponent-bin pass of the fp32 packing over n weights.
int64_t bin_blocks(int64_t n) {
  int64_t b = (n + (int64_t)kBinThreads * 64 - 1) / ((int64_t)kBinThreads * 64);
  if (b < 1) b = 1;
  if (b > kMaxBinBlocks) b = kMaxBinBlocks;
  return b;
}

size_t pack_workspace_bytes(int64_t N, int64_t K) {
  return (size_t)bin_blocks(N * K) * kBins * sizeof(unsigned long long);
}

// Launch plan of a grouped GEMM over M tokens (K % 64 == 0, M > 16):
// problems big enough to fill the chip with 128x256 tiles share one launch of
// those (their blocks then fill whole rounds together); the rest share one
// launch of 64x128 tiles, or of 32x128 tiles when 64x128 would give fewer
// blocks than CUs. That second launch splits K when its tiles leave CUs
// idle (fewer than 256 blocks) and K is long (at least 32 steps of 128
// weights): S = min(8, 1024 / blocks, steps / 4) ranges of at least four
// steps, so more blocks share the K loop. Measured on MI355X: the 2B {down}
// projection (K = 6912) at 64 tokens 24.7 -> 13.4 us, at 128 tokens 25.1 ->
// 15.8 us; at K = 2560, or with 256 blocks or more, the partial sums' traffic
// and the second launch cost as much as the split saves or more (2B {q,k,v}
// at 512 tokens 14.5 -> 22.7 us with 2 splits), so those run unsplit.
GemmPlan plan_gemm_group(const int64_t* Ns, int count, int64_t K, int64_t M) {
  GemmPlan pl{};
  pl.mfma = K % 64 == 0 && M > 16 && K <= kGemmMaxK;
  pl.splits = 1;
  if (!pl.mfma) return pl;
  int64_t b64 = 0;
  for (int i = 0; i < count; ++i) {
    if (((Ns[i] + 127) / 128) * ((M + 255) / 256) >= 256) {
      pl.big[pl.nbig++] = i;
    } else {
      pl.small[pl.nsmall++] = i;
      b64 += ((Ns[i] + 63) / 64) * ((M + 127) / 128);
    }
  }
  if (pl.nsmall == 0) return pl;
  pl.small32 = b64 < 256;
  const int64_t bn = pl.small32 ? 32 : 64;
  int64_t blocks = 0, nsum = 0;
  for (int j = 0; j < pl.nsmall; ++j) {
    blocks += ((Ns[pl.small[j]] + bn - 1) / bn) * ((M + 127) / 128);
    nsum += Ns[pl.small[j]];
  }
  const int64_t steps = (K + kGemmBK - 1) / kGemmBK;
  if (blocks >= kSplitMaxBlocks || steps < kSplitMinK) return pl;
  int64_t sp = blocks > 0 ? kSplitBlocks / blocks : 1;
  sp = sp < steps / kSplitMinSteps ? sp : steps / kSplitMinSteps;
  sp = sp < kMaxSplits ? sp : kMaxSplits;
  if (sp >= 2) {
    pl.splits = (int)sp;
    pl.ws_bytes = (size_t)(sp * M * nsum) * sizeof(int);
  }
  return pl;
}

}  // namespace bl
