// Stand-ins for the library's kernel launchers (test infrastructure): the C
// ABI's validation layer (api.cpp) and its host-side planning (plan.cpp)
// link against these instead of the HIP kernels, so that a host compiler can
// build them with the address and undefined-behaviour sanitizers. Each stub
// records its name and a few arguments and returns success.
#include <cstring>

#include "../../mpgemm_token_absmax_amd/csrc/launch.hpp"

namespace {
struct LastCall {
  char name[48];
  long long M, N, K;
  const void* ws;
  int count;
};
LastCall last;
long long calls;

hipError_t record(const char* name, long long M, long long N, long long K, const void* ws,
                  int count) {
  std::strncpy(last.name, name, sizeof(last.name) - 1);
  last.M = M;
  last.N = N;
  last.K = K;
  last.ws = ws;
  last.count = count;
  ++calls;
  return hipSuccess;
}
alignas(256) int fake_scratch[64];
}  // namespace

extern "C" {
// Calls recorded since the library loaded, and the last one.
long long blstub_calls(void) { return calls; }
const char* blstub_last_name(void) { return last.name; }
void blstub_last(long long* out, const void** ws) {
  out[0] = last.M;
  out[1] = last.N;
  out[2] = last.K;
  out[3] = last.count;
  *ws = last.ws;
}
}

namespace bl {

hipError_t launch_decode_group(DecodeGroup& g, hipStream_t) {
  return record("decode_group", g.M, g.count ? g.p[0].N : 0, g.count ? g.p[0].K : 0, nullptr,
                g.count);
}
hipError_t launch_decode_norm_group(DecodeGroup& g, hipStream_t) {
  return record("decode_norm_group", g.M, g.count ? g.p[0].N : 0, g.count ? g.p[0].K : 0,
                nullptr, g.count);
}
hipError_t launch_quantize_group(const DecodeGroup& g, hipStream_t) {
  return record("quantize_group", g.M, 0, 0, nullptr, g.count);
}
hipError_t launch_quantize_act(const uint16_t*, int64_t M, int64_t K, int64_t, int8_t*, float*,
                               int*, hipStream_t) {
  return record("quantize_act", M, 0, K, nullptr, 1);
}
hipError_t launch_quantize_act_tensor(const uint16_t*, int64_t M, int64_t K, int64_t, int8_t*,
                                      float*, int*, uint32_t* ws, hipStream_t) {
  return record("quantize_act_tensor", M, 0, K, ws, 1);
}
hipError_t launch_rmsnorm_quant(const uint16_t*, const uint16_t*, const uint16_t*, float,
                                int64_t M, int64_t K, int64_t, uint16_t*, int8_t*, float*, int*,
                                hipStream_t) {
  return record("rmsnorm_quant", M, 0, K, nullptr, 1);
}
hipError_t launch_pack_t3(const void*, bool, int64_t N, int64_t K, uint8_t*, const float*,
                          hipStream_t) {
  return record("pack_t3", 0, N, K, nullptr, 1);
}
hipError_t launch_gemv_t3(const uint8_t*, const float*, int64_t N, int64_t K, const int8_t*,
                          const float*, int64_t M, void*, int, hipStream_t) {
  return record("gemv_t3", M, N, K, nullptr, 1);
}
hipError_t launch_decode_group_t3(DecodeGroup& g, hipStream_t) {
  return record("decode_group_t3", g.M, g.count ? g.p[0].N : 0, g.count ? g.p[0].K : 0, nullptr,
                g.count);
}
hipError_t launch_absmean_gamma(const float*, int64_t N, int64_t K, float*, void* ws,
                                hipStream_t) {
  return record("absmean_gamma", 0, N, K, ws, 1);
}
hipError_t launch_pack_f32(const float*, int64_t N, int64_t K, uint8_t*, float*, void* ws,
                           hipStream_t) {
  return record("pack_f32", 0, N, K, ws, 1);
}
hipError_t launch_pack_ternary(const int8_t*, int64_t N, int64_t K, uint8_t*, hipStream_t) {
  return record("pack_ternary", 0, N, K, nullptr, 1);
}
hipError_t launch_gemv(const uint8_t*, const float*, int64_t N, int64_t K, const int8_t*,
                       const float*, int64_t M, void*, int, hipStream_t) {
  return record("gemv", M, N, K, nullptr, 1);
}
hipError_t launch_gemm(const uint8_t*, const float*, int64_t N, int64_t K, const int8_t*,
                       const float*, const int*, int64_t M, void*, int, void* ws, hipStream_t) {
  return record("gemm", M, N, K, ws, 1);
}
hipError_t launch_gemm_group(const GemmProblem* p, int count, int64_t K, const int8_t*,
                             const float*, const int*, int64_t M, void* ws, hipStream_t) {
  return record("gemm_group", M, count ? p[0].N : 0, K, ws, count);
}
hipError_t launch_generic(const uint8_t*, const float*, int64_t N, int64_t K, const int8_t*,
                          const float*, int64_t M, void*, int, hipStream_t) {
  return record("generic", M, N, K, nullptr, 1);
}
hipError_t noalloc_scratch(void** ptr) {
  *ptr = fake_scratch;
  return hipSuccess;
}

}  // namespace bl
