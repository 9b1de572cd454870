/*
 * bitlinear.h -- C ABI of the ternary BitLinear mpGEMM library (libbitlinear.so).
 *
 * The library computes a BitNet b1.58 linear layer on an AMD Instinct MI355X
 * (gfx950): ternary weights {-1, 0, +1} stored as 2-bit I2_S codes with one
 * per-tensor absmean scale, contracted against int8 activations quantized per
 * token by absmax, with exact int32 accumulation, then dequantized.
 *
 * Sources (web pages; cited by title and section):
 *   [BN]  "Bitnet.cpp: Efficient Edge Inference for Ternary LLMs" reading
 *         notes (arXiv 2502.11880): Part A 2.3 (I2_S: element-wise,
 *         multiply-add based, 2.0 bits per weight, ternary weights with one
 *         scale and int8 activations), 4.1 (lossless: no re-quantized partial
 *         sums), Part B "方法公式化".
 *   [FF]  FairyFuse article: "三元量化方案" (threshold at +-0.5 of a per-layer
 *         scale), "融合内核设计" (codes 00/01/10 = 0/+1/-1; add or subtract
 *         activations; fused unpack-accumulate-store).
 *   [HB]  bitnet.cpp how-to blog: 1.1 (decode streams every weight once per
 *         token, so it is memory-bandwidth bound), 1.2 (ternary weights turn
 *         multiply-adds into adds and subtracts).
 *   [BE]  "BinaryAI Engine：从零构建的CPU推理引擎如何超越llama.cpp":
 *         "关键技术机制解析" §2 (residual add and RMSNorm fused, halving the
 *         memory passes of a layer).
 *
 * Conventions (all calls):
 *   - Every array argument is a DEVICE pointer owned by the caller. The
 *     library never allocates, frees or keeps global mutable state.
 *     Outputs must not alias inputs.
 *   - Base pointers of x, q, packed, w and y must be 16-byte aligned; d and
 *     gamma 4-byte aligned (BL_ERR_ALIGN otherwise). Allocations from
 *     hipMalloc / PyTorch satisfy this.
 *   - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *     enqueues work on `stream` and returns; arguments are validated before
 *     anything is enqueued, and a rejected call enqueues nothing. A launch
 *     failure returns BL_ERR_HIP. Faults during execution surface at the
 *     caller's next synchronization of the stream. No call synchronizes.
 *   - M (tokens), N (output features) and K (input features) are counts;
 *     negative values are BL_ERR_SHAPE. K must be a multiple of 4.
 *     A call with M == 0 or N == 0 does nothing and returns BL_OK.
 *   - Calls are thread-safe (no shared state); results are deterministic and
 *     do not depend on the launch configuration.
 *
 * I2_S packed layout (the pages fix the code table [FF] and the 2-bit width
 * [BN], not the bit order; this layout is the library's choice):
 *   packed is uint8 [N][K/4], row n at byte offset n*(K/4). Each row is cut
 *   into groups of 16 weights (4 bytes); the last group of a row may hold
 *   4, 8 or 12 weights (b = 1, 2 or 3 bytes). Within a group of b bytes,
 *   weight o (0 <= o < 4b) is stored in byte (o mod b) at bits
 *   2*(o div b) .. 2*(o div b)+1. Code 00 = 0, 01 = +1, 10 = -1; 11 is never
 *   written (results over bytes that hold it are unspecified). For a full group, shifting its little-endian
 *   32-bit word right by 2i and masking 0x03030303 yields the codes of
 *   weights 4i .. 4i+3 in byte order.
 */
#ifndef BITLINEAR_H
#define BITLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BL_ABI_VERSION 4

/* Status codes returned by every call. */
enum {
  BL_OK = 0,
  BL_ERR_NULL = -1,      /* a required pointer is NULL                        */
  BL_ERR_SHAPE = -2,     /* negative size, K % 4 != 0, ldx < K, M > 16 (gemv) */
  BL_ERR_ALIGN = -3,     /* a pointer or stride breaks the alignment rules    */
  BL_ERR_DTYPE = -4,     /* unknown weight or output type enum                */
  BL_ERR_WORKSPACE = -5, /* workspace missing or smaller than required        */
  BL_ERR_HIP = -6,       /* the HIP runtime refused a launch                  */
  BL_ERR_ALIAS = -7      /* an output overlaps an input it may not share      */
};

/* Weight input type of bl_pack_i2s. */
enum {
  BL_W_F32 = 0,         /* fp32 [N][K]: absmean-ternarize, write *gamma      */
  BL_W_TERNARY_I8 = 1   /* int8 [N][K] ternary values: pack only             */
};

/* Output type of bl_gemv / bl_gemm. */
enum {
  BL_OUT_I32 = 0,   /* raw exact accumulator acc[t][n] (int32)               */
  BL_OUT_F32 = 1,   /* y = fl32(fl32(acc) * fl32(gamma * d_t))               */
  BL_OUT_BF16 = 2   /* the fp32 y rounded to nearest-even bf16 (uint16 bits) */
};

/* BL_ABI_VERSION of the loaded library. */
int bl_abi_version(void);

/* Static text for a status code; never NULL. */
const char *bl_status_string(int status);

/*
 * bl_quantize_act -- per-token absmax int8 quantization of activations.
 * Defines: [BN] Part A 2.3 / 4.1 (int8 activations with one scale per
 * vector, not per block); applied per token (row of x).
 *   m_t = max_k |x[t][k]|;   if m_t == 0: q[t][:] = 0, d[t] = 0;  else
 *   s_t = fl32(127 / m_t),   q[t][k] = clamp(rne(fl32(x[t][k] * s_t)), -127, 127),
 *   d[t] = fl32(m_t / 127)   (the dequantization multiplier).
 * x:   bf16 bit patterns, [M] rows of K values, row stride ldx elements
 *      (ldx >= K, ldx % 4 == 0).
 * q:   int8 [M][K], row stride K.     d: fp32 [M].
 * qsum: NULL, or int32 [M] (4-byte aligned) that receives the exact token
 *   sums qsum[t] = sum_k q[t][k] (needs 127*K <= INT32_MAX). Passed on to
 *   bl_gemm / bl_gemm_group they let the GEMM run on offset weights; the
 *   quantizer computes them from the codes it already holds.
 * Inputs must be finite; rows whose absmax is below 2^-120 (where 127/m
 * overflows fp32) give unspecified q. K == 0 writes d[:] = 0 (and qsum[:] = 0).
 */
int bl_quantize_act(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                    int8_t *q, float *d, int32_t *qsum, void *stream);

/*
 * bl_quantize_act_tensor_workspace -- bytes of workspace bl_quantize_act_tensor
 * needs for M tokens (4*M rounded up to 16; 0 for M <= 0).
 */
size_t bl_quantize_act_tensor_workspace(int64_t M);

/*
 * bl_quantize_act_tensor -- absmax int8 quantization with ONE scale for the
 * whole activation tensor (all M tokens).
 * Defines: [BN] Part A 2.3 / 4.1 (int8 activations with one per-tensor
 * scale), the literal setting of the pages for several tokens.
 *   m = max over every t, k of |x[t][k]|; if m == 0: q = 0 and d[:] = 0; else
 *   s = fl32(127 / m), q[t][k] = clamp(rne(fl32(x[t][k] * s)), -127, 127), and
 *   every d[t] = fl32(m / 127) (so bl_gemv / bl_gemm apply it unchanged).
 * Arguments as bl_quantize_act (qsum included), plus a workspace of ws_bytes bytes (>=
 * bl_quantize_act_tensor_workspace(M), 16-byte aligned; not needed when
 * K == 0): it receives the row maxima between the two launches the call
 * enqueues (row maxima, then quantize with the tensor's maximum).
 */
int bl_quantize_act_tensor(const uint16_t *x, int64_t M, int64_t K, int64_t ldx,
                           int8_t *q, float *d, int32_t *qsum, void *ws, size_t ws_bytes,
                           void *stream);

/*
 * bl_rmsnorm_quant -- residual add + RMSNorm fused with the per-token absmax
 * int8 quantizer, one pass over the activations.
 * Defines: [BE] "关键技术机制解析" §2 (residual add and RMS normalization
 * fused in one pass) feeding [BN] Part A 2.3 / 4.1 (per-token absmax int8).
 * The pages give no normalization formula; plain RMSNorm with a per-feature
 * weight is taken. Per token t:
 *   h[t][k] = bf16_rne(fl32(x[t][k] + r[t][k]))    (h = x when r is NULL)
 *   ms_t    = fl32(sum_k h[t][k]^2 / K)
 *   rinv_t  = fl32(1 / fl32(sqrt(fl32(ms_t + eps))))
 *   y[t][k] = fl32(fl32(h[t][k] * rinv_t) * g[k])
 *   then q, d of y exactly as bl_quantize_act (m = max|y|, s = fl32(127/m),
 *   q = rne(fl32(y*s)), d = fl32(m/127)); q = 0 and d[t] = 0 when m = 0 or
 *   fl32(ms_t + eps) = 0.
 * ms_t is the correctly rounded fp32 value of the exact mean square (an fp64
 * sum decides it when its error bound allows; otherwise the squares are
 * summed exactly as integers binned by exponent).
 * x, r: bf16 [M][K] row stride ldx (r may be NULL); g: bf16 [K];
 * h_out: bf16 [M][K] row stride ldx, or NULL (not written); it may be r or x
 * itself (in-place update of the residual stream) but must not otherwise
 * overlap them; q: int8 [M][K] (row stride K); d: fp32 [M]; qsum: NULL or the
 * token sums of q, as in bl_quantize_act. eps: finite,
 * >= 0. Inputs must be finite, and neither ms_t nor y may overflow fp32
 * (|h| below about 1.8e19; codes are unspecified otherwise). K % 4 == 0, ldx >= K, ldx % 4 == 0; x, r, g, h_out
 * and q 16-byte aligned. K == 0: d[:] = 0 (and qsum[:] = 0). One launch.
 */
int bl_rmsnorm_quant(const uint16_t *x, const uint16_t *r, const uint16_t *g, float eps,
                     int64_t M, int64_t K, int64_t ldx, uint16_t *h_out, int8_t *q,
                     float *d, int32_t *qsum, void *stream);

/*
 * bl_pack_i2s_workspace -- bytes of workspace bl_pack_i2s needs for an
 * N x K fp32 matrix (BL_W_F32). BL_W_TERNARY_I8 needs none.
 */
size_t bl_pack_i2s_workspace(int64_t N, int64_t K);

/*
 * bl_pack_i2s -- ternarize (optionally) and pack weights into I2_S.
 * Defines: [BN] Part A 2.3 (2-bit I2_S with one per-tensor scale),
 * [FF] "三元量化方案" (w > 0.5*alpha -> +1, w < -0.5*alpha -> -1, else 0),
 * with alpha read as BitNet b1.58's absmean scale gamma = mean |W|.
 *   BL_W_F32: w is fp32 [N][K] (finite). gamma = fl32(fl64(exact sum |w|) /
 *     (N*K)) is written to *gamma (device, 1 float); t = fl32(0.5*gamma);
 *     weight -> +1 if w > t, -1 if w < -t, else 0. The exact sum is order
 *     independent, so gamma and the codes are bit-reproducible.
 *     1 <= N*K < 2^38. Needs ws_bytes >= bl_pack_i2s_workspace(N, K) (16-byte aligned).
 *   BL_W_TERNARY_I8: w is int8 [N][K] ternary values; each is taken by its
 *     sign (> 0 -> +1, < 0 -> -1, 0 -> 0). *gamma is neither read nor
 *     written (the caller keeps the scale); gamma and ws may be NULL.
 * packed: uint8 [N][K/4] in the layout above.
 */
int bl_pack_i2s(const void *w, int wtype, int64_t N, int64_t K, uint8_t *packed,
                float *gamma, void *ws, size_t ws_bytes, void *stream);

/*
 * bl_gemv -- decode-time BitLinear for 1 <= M <= 16 tokens.
 * Defines: [BN] Part A 2.3 / 4.1 (I2_S multiply-add with exact sums),
 * [HB] 1.1-1.2, [FF] "融合内核设计" (unpack and accumulate in one pass).
 *   acc[t][n] = sum_k q[t][k] * w[n][k]  (exact int32; |acc| <= 127*K)
 *   y[t][n]   = acc[t][n] (BL_OUT_I32) or its dequantized value (BL_OUT_F32 /
 *               BL_OUT_BF16, see the output enum), y row stride N.
 * packed: uint8 [N][K/4]; gamma: device fp32 (1 value); q: int8 [M][K];
 * d: fp32 [M]. M > 16 is BL_ERR_SHAPE (use bl_gemm). For BL_OUT_F32 and
 * BL_OUT_BF16, K must satisfy 127*K < 2^24 (fp32-exact accumulator).
 * Results are bit-identical to bl_gemm's for the same inputs.
 */
int bl_gemv(const uint8_t *packed, const float *gamma, int64_t N, int64_t K,
            const int8_t *q, const float *d, int64_t M, void *y, int ytype,
            void *stream);

/*
 * Base-3 weights, five per byte (1.6 bits per weight).
 * Defines: [BN] Part A 2.3 (the format table's element-wise multiply-add
 * formats below 2 bits per weight, TQ1_0 at 1.69 and TL2 at 1.67 bits per
 * weight: three values per weight, so five weights fit one byte, 3^5 = 243).
 * The byte layout is the library's:
 *   - a row of K weights is padded with zero weights to a multiple of 320
 *     and takes bl_pack_t3_row_bytes(K) = 64*ceil(K/320) bytes;
 *   - unit u of a row (weights 80u .. 80u+79) is the 16 bytes at row offset
 *     16u; byte j of a unit (0..15) holds weights 80u + j + 16i, i = 0..4;
 *   - those five weights give digits d_i = w + 1 and v = sum d_i 3^(4-i)
 *     (d_0 most significant); the byte stores ceil(256 v / 243).
 * The contraction over these weights is the I2_S one, exactly.
 */
size_t bl_pack_t3_row_bytes(int64_t K);

/*
 * bl_pack_t3 -- ternarize (optionally) and pack weights into the base-3
 * format. Arguments, wtype rules, gamma and workspace exactly as bl_pack_i2s
 * (BL_W_F32 computes gamma and the same ternary values; the workspace size is
 * bl_pack_i2s_workspace(N, K)); packed: uint8 [N][bl_pack_t3_row_bytes(K)].
 * K % 16 == 0.
 */
int bl_pack_t3(const void *w, int wtype, int64_t N, int64_t K, uint8_t *packed,
               float *gamma, void *ws, size_t ws_bytes, void *stream);

/*
 * bl_gemv_t3 -- bl_gemv over base-3 packed weights.
 * Defines: as bl_gemv ([BN] Part A 2.3 / 4.1): acc[t][n] = sum_k q[t][k] *
 * w[n][k] exactly, then the same dequant and output types, so the outputs
 * equal bl_gemv's on the I2_S packing of the same weights.
 * packed: uint8 [N][bl_pack_t3_row_bytes(K)] from bl_pack_t3 (padding must
 * be the zero weights bl_pack_t3 writes); q: int8 [M][K]; d: fp32 [M];
 * 0 <= M <= 16; K % 16 == 0 (BL_ERR_SHAPE otherwise); K == 0 gives zeros.
 */
int bl_gemv_t3(const uint8_t *packed, const float *gamma, int64_t N, int64_t K,
               const int8_t *q, const float *d, int64_t M, void *y, int ytype,
               void *stream);

/*
 * bl_gemm_workspace -- bytes of workspace with which bl_gemm splits K for
 * this shape (0: the call does not split). A launch with fewer output tiles
 * than about four per compute unit splits its K steps into up to 8 ranges
 * of at least 512 weights; each range's exact int32 partial sums go to the
 * workspace ([splits][M][N] int32) and a second launch adds them, subtracts
 * the token sums and dequantizes. Integer sums are exact, so the results are
 * bit-identical with and without the split.
 */
size_t bl_gemm_workspace(int64_t M, int64_t N, int64_t K);

/*
 * bl_gemm -- prefill BitLinear for any M >= 1 (int8 MFMA path).
 * Defines: as bl_gemv ([BN] Part A 2.3 / 4.1); the pages leave prefill
 * unoptimized ([BN] 4.4), so this is the dense contraction on matrix cores.
 * Same arguments and results as bl_gemv, plus a workspace and qsum:
 *   ws: NULL (the launch runs unsplit), or device memory of ws_bytes >=
 *     bl_gemm_workspace(M, N, K), 16-byte aligned (BL_ERR_WORKSPACE /
 *     BL_ERR_ALIGN otherwise), overlapping no other argument; it receives
 *     the split-K partial sums. Calls that share a workspace must not
 *     overlap in time (it is not needed after the call's work ends).
 *   qsum: NULL, or int32 [M] (4-byte aligned) holding the token sums
 *     qsum[t] = sum_k q[t][k] of exactly this q (as bl_quantize_act or
 *     bl_rmsnorm_quant write them; they are not checked). With them the
 *     matrix cores get the weights plus one, in {0, 1, 2}, and the kernel
 *     subtracts qsum[t] from each accumulator: the same exact acc, computed
 *     with operands that switch fewer bits, which keeps the power-limited
 *     clock higher. Results are bit-identical with and without qsum.
 */
int bl_gemm(const uint8_t *packed, const float *gamma, int64_t N, int64_t K,
            const int8_t *q, const float *d, const int32_t *qsum, int64_t M, void *y,
            int ytype, void *ws, size_t ws_bytes, void *stream);

/*
 * bl_gemm_problem / bl_gemm_group -- several BitLinear GEMMs over the SAME
 * quantized activations, as few launches as the shapes allow.
 * Defines: as bl_gemm, once per problem ([BN] Part A 2.3 / 4.1). Meant for
 * the projections of a decoder layer that read one input (q/k/v; gate/up).
 *   problems: HOST array of `count` descriptors (0 <= count <= 8), read during
 *     the call only; every pointer inside is a device pointer.
 *   per problem: packed uint8 [N][K/4], gamma (device, 1 float), y [M][N] of
 *     type ytype (see the output enum), row stride N; N == 0 is skipped.
 *   shared: K (K % 4 == 0), q int8 [M][K], d fp32 [M], qsum (NULL or the
 *     token sums of q, as in bl_gemm), M >= 0 tokens; ws, ws_bytes: NULL or
 *     a workspace of >= bl_gemm_group_workspace(...) bytes, as in bl_gemm.
 * Each y is bit-identical to what bl_gemm gives for that problem alone.
 * Validation is bl_gemm's, problem by problem; nothing is launched when any
 * problem fails it. Outputs must not alias any input or each other.
 */
typedef struct bl_gemm_problem {
  const uint8_t *packed;
  const float *gamma;
  int64_t N;
  void *y;
  int ytype;
} bl_gemm_problem;

/*
 * bl_gemm_group_workspace -- bytes of workspace with which bl_gemm_group
 * splits K for problems of these output sizes (Ns: HOST array of `count`
 * N values; N == 0 problems count for nothing), as bl_gemm_workspace.
 */
size_t bl_gemm_group_workspace(const int64_t *Ns, int count, int64_t K, int64_t M);

int bl_gemm_group(const bl_gemm_problem *problems, int count, int64_t K, const int8_t *q,
                  const float *d, const int32_t *qsum, int64_t M, void *ws, size_t ws_bytes,
                  void *stream);

/*
 * bl_gemm_group_noalloc -- bl_gemm_group for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. Same arguments (minus the workspace),
 * validation and results as bl_gemm_group with a workspace of
 * bl_gemm_group_workspace(...) bytes; it calls no allocating routine.
 * The split-K partial sums go to a workspace inside the library: a
 * file-scope device array of BL_GEMM_NOALLOC_SCRATCH_BYTES (32 MiB, the
 * most any launch plan needs) that each GPU the library runs on holds until
 * the process ends; its address on a device is looked up on the first call
 * there. BL_ERR_WORKSPACE if a plan ever needed more; BL_ERR_HIP if the
 * lookup fails. Every call on one GPU shares that array: calls that overlap
 * in time on one GPU (two streams, two threads) race and may give wrong
 * results; calls ordered on one stream do not (each launch writes every
 * partial sum it later reads).
 */
#define BL_GEMM_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int bl_gemm_group_noalloc(const bl_gemm_problem *problems, int count, int64_t K,
                          const int8_t *q, const float *d, const int32_t *qsum, int64_t M,
                          void *stream);

/*
 * bl_decode_problem / bl_decode_group -- fused decode BitLinear for a group
 * of independent projections in ONE launch: per-token absmax int8
 * quantization of bf16 activations, the I2_S GEMV and the dequant.
 * Defines: the composition of bl_quantize_act and bl_gemv ([BN] Part A 2.3 /
 * 4.1, [HB] 1.1-1.2), fused as in [FF] "融合内核设计" (activations loaded,
 * codes walked, sums accumulated and written in one pass). Results (y, and q
 * and d when requested) are bit-identical to bl_quantize_act followed by
 * bl_gemv on the same inputs. Meant for the projections of one decoder layer
 * that do not depend on each other (e.g. q/k/v, or gate/up).
 *   problems: HOST array of `count` descriptors (1 <= count <= 8), read during
 *     the call only; every pointer inside is a device pointer.
 *   M: tokens, 1 <= M <= 16, shared by all problems.
 *   per problem: packed uint8 [N][K/4], gamma (device, 1 float), x bf16 [M]
 *     rows of K values with row stride ldx (ldx >= K, ldx % 4 == 0), y [M][N]
 *     of type ytype; q (int8 [M][K]) and d (fp32 [M]) receive the quantized
 *     activations. At M == 1 they are optional (NULL: not written); at M > 1
 *     they are required (BL_ERR_NULL otherwise). Up to 4 tokens (every
 *     ldx % 8 == 0, K <= 32768) the GEMV launch quantizes and writes them
 *     itself; otherwise the codes are staged there by a quantize pass inside
 *     the call, ahead of the GEMV launch.
 *     K % 64 == 0 and K <= 65536 are required (BL_ERR_SHAPE otherwise);
 *     N == 0 problems are skipped. Outputs must not alias any
 *     input or each other.
 */
typedef struct bl_decode_problem {
  const uint8_t *packed;
  const float *gamma;
  int64_t N;
  int64_t K;
  const uint16_t *x;
  int64_t ldx;
  int8_t *q;
  float *d;
  void *y;
  int ytype;
} bl_decode_problem;

int bl_decode_group(const bl_decode_problem *problems, int count, int64_t M, void *stream);

/*
 * bl_decode_group_t3 -- bl_decode_group over base-3 packed weights (five per
 * byte, 1.6 bits per weight).
 * Defines: the composition of bl_quantize_act and bl_gemv_t3 ([BN] Part A
 * 2.3 / 4.1: the same exact contraction; the format table's sub-2-bit
 * element-wise formats for the weight bytes), fused as in [FF] "融合内核设计".
 * Results (y, and q and d when requested) are bit-identical to
 * bl_quantize_act followed by bl_gemv_t3, and to bl_decode_group on the I2_S
 * packing of the same weights.
 *   problems, count, M: as bl_decode_group, except that packed is uint8
 *     [N][bl_pack_t3_row_bytes(K)] from bl_pack_t3 and K % 16 == 0
 *     (K <= 65536; BL_ERR_SHAPE otherwise). At M == 1 one launch quantizes
 *     and contracts every problem (q and d optional); at M > 1 q and d are
 *     required and receive the codes from a quantize pass inside the call,
 *     which bl_gemv_t3 then reads, one launch per problem.
 * Outputs must not alias any input or each other.
 */
int bl_decode_group_t3(const bl_decode_problem *problems, int count, int64_t M, void *stream);

/*
 * bl_decode_norm_group -- one token through the residual add, RMSNorm and the
 * per-token quantizer, then up to 8 projections of the normalized token, in
 * one launch.
 * Defines: bl_rmsnorm_quant ([BE] "关键技术机制解析" §2 with [BN] Part A 2.3 /
 * 4.1) composed with bl_gemv, fused as in [FF] "融合内核设计". Every problem
 * reads the same x (bf16 [1][K], its x field) and has the same K; r (bf16
 * [K] or NULL) is the residual, g (bf16 [K]) the norm weight, eps finite and
 * >= 0. Each problem's y is bl_gemv's output for the codes and scale of
 * y_norm = RMSNorm(h) * g, h = bf16(x + r); q and d, when given, receive those
 * codes and scale; h_out (bf16 [K] or NULL) receives h. h_out must not
 * overlap x or r (other blocks still read them while it is written).
 * M is 1. K % 64 == 0 and K <= 32768; N, ytype, gamma and alignment as in
 * bl_decode_group; g, r and h_out 16-byte aligned. The mean square is the
 * correctly rounded one, as in bl_rmsnorm_quant.
 */
int bl_decode_norm_group(const bl_decode_problem *problems, int count, const uint16_t *r,
                         const uint16_t *g, float eps, uint16_t *h_out, void *stream);


#ifdef __cplusplus
}
#endif

#endif /* BITLINEAR_H */
