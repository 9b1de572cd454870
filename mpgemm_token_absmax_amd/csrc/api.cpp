// C ABI of the ternary BitLinear library: argument validation and dispatch.
// Declarations, argument meaning, layouts, ownership and errors: the public
// header bitlinear.h. Validation touches no HIP API, so every error path runs
// (and is tested) on a machine without a GPU.
#include <hip/hip_runtime_api.h>

#include "../../include/bitlinear.h"
#include "launch.hpp"

namespace {

constexpr int64_t kGemvMaxM = 16;
constexpr int64_t kFp32ExactK = ((int64_t)1 << 24) / 127;   // 127*K < 2^24
constexpr int64_t kDecodeMaxK = 65536;                       // fused decode: K per problem
static_assert(bl::kNoAllocScratchBytes == BL_GEMM_NOALLOC_SCRATCH_BYTES,
              "the header states the allocation-free workspace size");

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? BL_OK : BL_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

int check_matmul(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                 const int8_t* q, const float* d, int64_t M, const void* y, int ytype) {
  if (M < 0 || N < 0 || K < 0 || K % 4 != 0) return BL_ERR_SHAPE;
  if (ytype < BL_OUT_I32 || ytype > BL_OUT_BF16) return BL_ERR_DTYPE;
  if (M == 0 || N == 0) return BL_OK;
  if (!y) return BL_ERR_NULL;
  if (K > 0 && (!packed || !q)) return BL_ERR_NULL;
  if (ytype != BL_OUT_I32 && (!gamma || !d)) return BL_ERR_NULL;
  if (127 * K > INT32_MAX) return BL_ERR_SHAPE;
  if (ytype != BL_OUT_I32 && K > kFp32ExactK) return BL_ERR_SHAPE;
  if (!aligned(y, 16)) return BL_ERR_ALIGN;
  if (K > 0 && (!aligned(packed, 16) || !aligned(q, 16))) return BL_ERR_ALIGN;
  if ((gamma && !aligned(gamma, 4)) || (d && !aligned(d, 4))) return BL_ERR_ALIGN;
  return BL_OK;
}

}  // namespace

extern "C" {

int bl_abi_version(void) { return BL_ABI_VERSION; }

const char* bl_status_string(int status) {
  switch (status) {
    case BL_OK: return "ok";
    case BL_ERR_NULL: return "a required pointer is NULL";
    case BL_ERR_SHAPE: return "invalid shape (negative size, K % 4 != 0, ldx < K, M > 16 for gemv, or K too large)";
    case BL_ERR_ALIGN: return "misaligned pointer or stride";
    case BL_ERR_DTYPE: return "unknown weight or output type";
    case BL_ERR_WORKSPACE: return "workspace missing or too small";
    case BL_ERR_HIP: return "HIP runtime error while launching";
    case BL_ERR_ALIAS: return "an output overlaps an input it may not share";
    default: return "unknown status";
  }
}

int bl_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q, float* d,
                    int32_t* qsum, void* stream) {
  if (M < 0 || K < 0 || K % 4 != 0 || ldx < K) return BL_ERR_SHAPE;
  if (M == 0) return BL_OK;
  if (!d || (K > 0 && (!x || !q))) return BL_ERR_NULL;
  if (K > 0 && ldx % 4 != 0) return BL_ERR_ALIGN;
  if (!aligned(d, 4) || !aligned(qsum, 4)) return BL_ERR_ALIGN;
  if (K > 0 && (!aligned(x, 16) || !aligned(q, 16))) return BL_ERR_ALIGN;
  if (M > INT32_MAX || (qsum && 127 * K > INT32_MAX)) return BL_ERR_SHAPE;
  return hip_status(bl::launch_quantize_act(x, M, K, ldx, q, d, qsum, as_stream(stream)));
}

size_t bl_quantize_act_tensor_workspace(int64_t M) {
  if (M <= 0) return 0;
  return (size_t)((4 * M + 15) / 16 * 16);
}

int bl_quantize_act_tensor(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                           float* d, int32_t* qsum, void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || K < 0 || K % 4 != 0 || ldx < K) return BL_ERR_SHAPE;
  if (M == 0) return BL_OK;
  if (!d || (K > 0 && (!x || !q))) return BL_ERR_NULL;
  if (K > 0 && ldx % 4 != 0) return BL_ERR_ALIGN;
  if (!aligned(d, 4) || !aligned(qsum, 4)) return BL_ERR_ALIGN;
  if (K > 0 && (!aligned(x, 16) || !aligned(q, 16))) return BL_ERR_ALIGN;
  if (M > INT32_MAX || (qsum && 127 * K > INT32_MAX)) return BL_ERR_SHAPE;
  if (K > 0 && (!ws || ws_bytes < bl_quantize_act_tensor_workspace(M))) return BL_ERR_WORKSPACE;
  if (K > 0 && !aligned(ws, 16)) return BL_ERR_ALIGN;
  return hip_status(bl::launch_quantize_act_tensor(x, M, K, ldx, q, d, qsum,
                                                   static_cast<uint32_t*>(ws), as_stream(stream)));
}

namespace {

// Byte range [p, p + rows*ld + K) * 2 of a bf16 [rows][K] array of row stride ld.
bool overlap_bf16(const uint16_t* a, const uint16_t* b, int64_t M, int64_t K, int64_t ld) {
  const uintptr_t n = (uintptr_t)(((M - 1) * ld + K) * 2);
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + n && pb < pa + n;
}

}  // namespace

int bl_rmsnorm_quant(const uint16_t* x, const uint16_t* r, const uint16_t* g, float eps,
                     int64_t M, int64_t K, int64_t ldx, uint16_t* h_out, int8_t* q, float* d,
                     int32_t* qsum, void* stream) {
  if (M < 0 || K < 0 || K % 4 != 0 || ldx < K) return BL_ERR_SHAPE;
  if (!(eps >= 0.0f) || eps > 3.4028235e38f) return BL_ERR_SHAPE;     // NaN, inf, < 0
  if (M == 0) return BL_OK;
  if (!d || (K > 0 && (!x || !g || !q))) return BL_ERR_NULL;
  if (M > INT32_MAX || (qsum && 127 * K > INT32_MAX)) return BL_ERR_SHAPE;
  if (!aligned(d, 4) || !aligned(qsum, 4)) return BL_ERR_ALIGN;
  if (K > 0) {
    if (ldx % 4 != 0) return BL_ERR_ALIGN;
    if (!aligned(x, 16) || !aligned(g, 16) || !aligned(q, 16)) return BL_ERR_ALIGN;
    if ((r && !aligned(r, 16)) || (h_out && !aligned(h_out, 16))) return BL_ERR_ALIGN;
    if (h_out && h_out != x && overlap_bf16(h_out, x, M, K, ldx)) return BL_ERR_ALIAS;
    if (h_out && r && h_out != r && overlap_bf16(h_out, r, M, K, ldx)) return BL_ERR_ALIAS;
  }
  return hip_status(bl::launch_rmsnorm_quant(x, r, g, eps, M, K, ldx, h_out, q, d, qsum,
                                             as_stream(stream)));
}

size_t bl_pack_i2s_workspace(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0) return 0;
  return bl::pack_workspace_bytes(N, K);
}

int bl_pack_i2s(const void* w, int wtype, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                void* ws, size_t ws_bytes, void* stream) {
  if (N < 0 || K < 0 || K % 4 != 0) return BL_ERR_SHAPE;
  if (wtype != BL_W_F32 && wtype != BL_W_TERNARY_I8) return BL_ERR_DTYPE;
  if (wtype == BL_W_F32) {
    if (N == 0 || K == 0) return BL_ERR_SHAPE;     // gamma of an empty matrix is undefined
    if (N > ((int64_t)1 << 38) / K) return BL_ERR_SHAPE;   // exact-sum bins: n < 2^38
    if (!w || !packed || !gamma) return BL_ERR_NULL;
    if (!ws) return BL_ERR_WORKSPACE;
    if (ws_bytes < bl::pack_workspace_bytes(N, K)) return BL_ERR_WORKSPACE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(ws, 16))
      return BL_ERR_ALIGN;
    return hip_status(bl::launch_pack_f32(static_cast<const float*>(w), N, K, packed, gamma, ws,
                                          as_stream(stream)));
  }
  if (N == 0 || K == 0) return BL_OK;
  if (!w || !packed) return BL_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16)) return BL_ERR_ALIGN;
  return hip_status(bl::launch_pack_ternary(static_cast<const int8_t*>(w), N, K, packed,
                                            as_stream(stream)));
}

size_t bl_pack_t3_row_bytes(int64_t K) {
  if (K <= 0) return 0;
  return (size_t)(64 * ((K + 319) / 320));
}

int bl_pack_t3(const void* w, int wtype, int64_t N, int64_t K, uint8_t* packed, float* gamma,
               void* ws, size_t ws_bytes, void* stream) {
  if (N < 0 || K < 0 || K % 16 != 0) return BL_ERR_SHAPE;
  if (wtype != BL_W_F32 && wtype != BL_W_TERNARY_I8) return BL_ERR_DTYPE;
  if (wtype == BL_W_F32) {
    if (N == 0 || K == 0) return BL_ERR_SHAPE;     // gamma of an empty matrix is undefined
    if (N > ((int64_t)1 << 38) / K) return BL_ERR_SHAPE;
    if (!w || !packed || !gamma) return BL_ERR_NULL;
    if (!ws) return BL_ERR_WORKSPACE;
    if (ws_bytes < bl::pack_workspace_bytes(N, K)) return BL_ERR_WORKSPACE;
    if (!aligned(w, 16) || !aligned(packed, 16) || !aligned(gamma, 4) || !aligned(ws, 16))
      return BL_ERR_ALIGN;
    hipError_t e = bl::launch_absmean_gamma(static_cast<const float*>(w), N, K, gamma, ws,
                                            as_stream(stream));
    if (e == hipSuccess) e = bl::launch_pack_t3(w, true, N, K, packed, gamma, as_stream(stream));
    return hip_status(e);
  }
  if (N == 0 || K == 0) return BL_OK;
  if (!w || !packed) return BL_ERR_NULL;
  if (!aligned(w, 16) || !aligned(packed, 16)) return BL_ERR_ALIGN;
  return hip_status(bl::launch_pack_t3(w, false, N, K, packed, nullptr, as_stream(stream)));
}

int bl_gemv_t3(const uint8_t* packed, const float* gamma, int64_t N, int64_t K, const int8_t* q,
               const float* d, int64_t M, void* y, int ytype, void* stream) {
  if (M > kGemvMaxM || K % 16 != 0) return BL_ERR_SHAPE;
  const int st = check_matmul(packed, gamma, N, K, q, d, M, y, ytype);
  if (st != BL_OK || M == 0 || N == 0) return st;
  if (N * 64 * ((K + 319) / 320) > ((int64_t)1 << 40)) return BL_ERR_SHAPE;
  return hip_status(bl::launch_gemv_t3(packed, gamma, N, K, q, d, M, y, ytype,
                                       as_stream(stream)));
}

int bl_gemv(const uint8_t* packed, const float* gamma, int64_t N, int64_t K, const int8_t* q,
            const float* d, int64_t M, void* y, int ytype, void* stream) {
  if (M > kGemvMaxM) return BL_ERR_SHAPE;
  const int st = check_matmul(packed, gamma, N, K, q, d, M, y, ytype);
  if (st != BL_OK || M == 0 || N == 0) return st;
  return hip_status(bl::launch_gemv(packed, gamma, N, K, q, d, M, y, ytype, as_stream(stream)));
}

}  // extern "C"

namespace {

// Workspace of a grouped GEMM over the problems with these N (N == 0 ones
// left out, as the call skips them): the split-K partial sums of its plan.
size_t gemm_ws_bytes(const int64_t* Ns, int count, int64_t K, int64_t M) {
  int64_t kept[bl::kMaxGroup];
  int n = 0;
  for (int i = 0; i < count; ++i)
    if (Ns[i] > 0) kept[n++] = Ns[i];
  if (n == 0 || M <= 0 || K <= 0) return 0;
  return bl::plan_gemm_group(kept, n, K, M).ws_bytes;
}

// The workspace rule shared by bl_gemm and bl_gemm_group: NULL runs unsplit;
// otherwise it must hold `need` bytes and be 16-byte aligned.
int check_gemm_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (!ws) return BL_OK;
  if (ws_bytes < need) return BL_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return BL_ERR_ALIGN;
  return BL_OK;
}

}  // namespace

extern "C" {

size_t bl_gemm_workspace(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0 || K % 4 != 0) return 0;
  return gemm_ws_bytes(&N, 1, K, M);
}

size_t bl_gemm_group_workspace(const int64_t* Ns, int count, int64_t K, int64_t M) {
  if (!Ns || count <= 0 || count > bl::kMaxGroup || K <= 0 || K % 4 != 0 || M <= 0) return 0;
  return gemm_ws_bytes(Ns, count, K, M);
}

int bl_gemm(const uint8_t* packed, const float* gamma, int64_t N, int64_t K, const int8_t* q,
            const float* d, const int32_t* qsum, int64_t M, void* y, int ytype, void* ws,
            size_t ws_bytes, void* stream) {
  const int st = check_matmul(packed, gamma, N, K, q, d, M, y, ytype);
  if (st != BL_OK || M == 0 || N == 0) return st;
  if (!aligned(qsum, 4)) return BL_ERR_ALIGN;
  if (N > (int64_t)UINT32_MAX * 64 || M > (int64_t)65535 * 128) return BL_ERR_SHAPE;
  const int wst = check_gemm_ws(ws, ws_bytes, bl_gemm_workspace(M, N, K));
  if (wst != BL_OK) return wst;
  return hip_status(bl::launch_gemm(packed, gamma, N, K, q, d, qsum, M, y, ytype, ws,
                                    as_stream(stream)));
}

}  // extern "C"

namespace {

// Validation of a grouped GEMM (every problem, before anything is launched);
// on BL_OK, g[0..n) are the problems with N > 0 and Ns their sizes.
int check_gemm_group(const bl_gemm_problem* problems, int count, int64_t K, const int8_t* q,
                     const float* d, const int32_t* qsum, int64_t M, bl::GemmProblem* g,
                     int64_t* Ns, int* n) {
  *n = 0;
  if (count < 0 || count > bl::kMaxGroup || M < 0 || K < 0 || K % 4 != 0) return BL_ERR_SHAPE;
  if (count == 0 || M == 0) return BL_OK;
  if (!problems) return BL_ERR_NULL;
  if (!aligned(qsum, 4)) return BL_ERR_ALIGN;
  if (M > (int64_t)65535 * 256) return BL_ERR_SHAPE;
  for (int i = 0; i < count; ++i) {
    const bl_gemm_problem& p = problems[i];
    const int st = check_matmul(p.packed, p.gamma, p.N, K, q, d, M, p.y, p.ytype);
    if (st != BL_OK) return st;
    if (p.N > (int64_t)UINT32_MAX * 64) return BL_ERR_SHAPE;
    if (p.N == 0) continue;
    Ns[*n] = p.N;
    g[(*n)++] = bl::GemmProblem{p.packed, p.gamma, p.y, p.N, p.ytype};
  }
  return BL_OK;
}

}  // namespace

extern "C" {

int bl_gemm_group(const bl_gemm_problem* problems, int count, int64_t K, const int8_t* q,
                  const float* d, const int32_t* qsum, int64_t M, void* ws, size_t ws_bytes,
                  void* stream) {
  bl::GemmProblem g[bl::kMaxGroup];
  int64_t Ns[bl::kMaxGroup];
  int n = 0;
  const int st = check_gemm_group(problems, count, K, q, d, qsum, M, g, Ns, &n);
  if (st != BL_OK || n == 0) return st;
  const int wst = check_gemm_ws(ws, ws_bytes, gemm_ws_bytes(Ns, n, K, M));
  if (wst != BL_OK) return wst;
  return hip_status(bl::launch_gemm_group(g, n, K, q, d, qsum, M, ws, as_stream(stream)));
}

int bl_gemm_group_noalloc(const bl_gemm_problem* problems, int count, int64_t K, const int8_t* q,
                          const float* d, const int32_t* qsum, int64_t M, void* stream) {
  bl::GemmProblem g[bl::kMaxGroup];
  int64_t Ns[bl::kMaxGroup];
  int n = 0;
  const int st = check_gemm_group(problems, count, K, q, d, qsum, M, g, Ns, &n);
  if (st != BL_OK || n == 0) return st;
  const size_t need = gemm_ws_bytes(Ns, n, K, M);
  if (need > bl::kNoAllocScratchBytes) return BL_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0 && bl::noalloc_scratch(&ws) != hipSuccess) return BL_ERR_HIP;
  return hip_status(bl::launch_gemm_group(g, n, K, q, d, qsum, M, ws, as_stream(stream)));
}

int bl_decode_norm_group(const bl_decode_problem* problems, int count, const uint16_t* r,
                         const uint16_t* g, float eps, uint16_t* h_out, void* stream) {
  if (count < 0 || count > bl::kMaxGroup) return BL_ERR_SHAPE;
  if (!(eps >= 0.0f) || eps > 3.4028235e38f) return BL_ERR_SHAPE;
  if (count == 0) return BL_OK;
  if (!problems) return BL_ERR_NULL;
  const uint16_t* x = problems[0].x;
  const int64_t K = problems[0].K;
  if (K <= 0 || K % 64 != 0 || K > 32768) return BL_ERR_SHAPE;
  if (!x || !g) return BL_ERR_NULL;
  if (!aligned(x, 16) || !aligned(g, 16) || (r && !aligned(r, 16)) ||
      (h_out && !aligned(h_out, 16)))
    return BL_ERR_ALIGN;
  if (h_out && (overlap_bf16(h_out, x, 1, K, K) || (r && overlap_bf16(h_out, r, 1, K, K))))
    return BL_ERR_ALIAS;
  bl::DecodeGroup gr{};
  gr.M = 1;
  for (int i = 0; i < count; ++i) {
    const bl_decode_problem& p = problems[i];
    if (p.x != x || p.K != K) return BL_ERR_SHAPE;   // one normalized input per group
    if (p.N < 0) return BL_ERR_SHAPE;
    if (p.ytype < BL_OUT_I32 || p.ytype > BL_OUT_BF16) return BL_ERR_DTYPE;
    if (p.N == 0) continue;
    if (!p.y || !p.packed || (p.ytype != BL_OUT_I32 && !p.gamma)) return BL_ERR_NULL;
    if (!aligned(p.y, 16) || !aligned(p.packed, 16)) return BL_ERR_ALIGN;
    if ((p.q && !aligned(p.q, 16)) || (p.d && !aligned(p.d, 4)) ||
        (p.gamma && !aligned(p.gamma, 4)))
      return BL_ERR_ALIGN;
    bl::DecodeProblem& d = gr.p[gr.count++];
    d.packed = p.packed;
    d.gamma = p.gamma;
    d.N = p.N;
    d.K = K;
    d.x = x;
    d.ldx = K;
    d.q = p.q;
    d.d = p.d;
    d.y = p.y;
    d.ytype = p.ytype;
  }
  if (gr.count == 0) return BL_OK;
  gr.nr = r;
  gr.ng = g;
  gr.nh = h_out;
  gr.eps = eps;
  return hip_status(bl::launch_decode_norm_group(gr, as_stream(stream)));
}

}  // extern "C"

namespace {

// Validation shared by the I2_S and base-3 decode groups (kmod: required
// divisor of K; t3: base-3 row bytes); fills g on success.
int check_decode_group(const bl_decode_problem* problems, int count, int64_t M, int kmod,
                       bool t3, bl::DecodeGroup& g) {
  if (count < 0 || count > bl::kMaxGroup || M < 0 || M > kGemvMaxM) return BL_ERR_SHAPE;
  if (count == 0 || M == 0) return BL_OK;
  if (!problems) return BL_ERR_NULL;
  g.M = (int)M;
  for (int i = 0; i < count; ++i) {
    const bl_decode_problem& p = problems[i];
    if (p.N < 0 || p.K < 0 || p.K % kmod != 0 || p.ldx < p.K || p.K > kDecodeMaxK)
      return BL_ERR_SHAPE;
    if (t3 && p.N * 64 * ((p.K + 319) / 320) > ((int64_t)1 << 40)) return BL_ERR_SHAPE;
    if (p.ytype < BL_OUT_I32 || p.ytype > BL_OUT_BF16) return BL_ERR_DTYPE;
    if (p.ytype != BL_OUT_I32 && p.K > kFp32ExactK) return BL_ERR_SHAPE;
    if (127 * p.K > INT32_MAX) return BL_ERR_SHAPE;
    if (p.N == 0) continue;
    if (!p.y || (p.K > 0 && (!p.packed || !p.x)) || (p.ytype != BL_OUT_I32 && !p.gamma))
      return BL_ERR_NULL;
    if (M > 1 && p.K > 0 && (!p.q || !p.d)) return BL_ERR_NULL;   // staging of the codes
    if ((p.K > 0 && p.ldx % 4 != 0) || !aligned(p.y, 16)) return BL_ERR_ALIGN;   // K == 0 reads no x
    if (p.K > 0 && (!aligned(p.packed, 16) || !aligned(p.x, 16))) return BL_ERR_ALIGN;
    if ((p.q && !aligned(p.q, 16)) || (p.d && !aligned(p.d, 4)) ||
        (p.gamma && !aligned(p.gamma, 4)))
      return BL_ERR_ALIGN;
    bl::DecodeProblem& d = g.p[g.count++];
    d.packed = p.packed;
    d.gamma = p.gamma;
    d.N = p.N;
    d.K = p.K;
    d.x = p.x;
    d.ldx = p.ldx;
    d.q = p.q;
    d.d = p.d;
    d.y = p.y;
    d.ytype = p.ytype;
  }
  return BL_OK;
}

}  // namespace

extern "C" {

int bl_decode_group(const bl_decode_problem* problems, int count, int64_t M, void* stream) {
  bl::DecodeGroup g{};
  const int st = check_decode_group(problems, count, M, 64, false, g);
  if (st != BL_OK || g.count == 0) return st;
  return hip_status(bl::launch_decode_group(g, as_stream(stream)));
}

int bl_decode_group_t3(const bl_decode_problem* problems, int count, int64_t M, void* stream) {
  bl::DecodeGroup g{};
  const int st = check_decode_group(problems, count, M, 16, true, g);
  if (st != BL_OK || g.count == 0) return st;
  return hip_status(bl::launch_decode_group_t3(g, as_stream(stream)));
}

}  // extern "C"
