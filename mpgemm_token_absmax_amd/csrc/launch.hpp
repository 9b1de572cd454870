// Internal launchers behind the C ABI (include/bitlinear.h). Arguments are
// already validated by api.cpp; each launcher only enqueues work on `s`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

hipError_t launch_quantize_act(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int8_t* q,
                               float* d, hipStream_t s);

size_t pack_workspace_bytes(int64_t N, int64_t K);
hipError_t launch_pack_f32(const float* w, int64_t N, int64_t K, uint8_t* packed, float* gamma,
                           void* ws, hipStream_t s);
hipError_t launch_pack_ternary(const int8_t* w, int64_t N, int64_t K, uint8_t* packed,
                               hipStream_t s);

// y layout: [M][N]; ytype: 0 = int32 acc, 1 = fp32, 2 = bf16 bits.
hipError_t launch_gemv(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s);
hipError_t launch_gemm(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                       const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                       hipStream_t s);
// Shapes off the fast paths (K % 64 != 0): one thread per output element.
hipError_t launch_generic(const uint8_t* packed, const float* gamma, int64_t N, int64_t K,
                          const int8_t* q, const float* d, int64_t M, void* y, int ytype,
                          hipStream_t s);

}  // namespace bl
