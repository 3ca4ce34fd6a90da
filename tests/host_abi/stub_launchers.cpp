// Host-only stand-ins for the library's kernel launchers, linked with the
// real C ABI (abi.cpp) into a sanitizer build that needs no GPU and no HIP
// runtime: every launcher records its name and returns success; the one HIP
// API function the ABI calls (hipGetErrorString) is given a plain table.
// Test infrastructure only: nothing here computes any step of the layer.
#include <string>

#include "../../bit_activation_linear_amd/csrc/kernels.h"

namespace {
std::string g_calls;
hipError_t record(const char* name) {
  if (!g_calls.empty()) g_calls += ' ';
  g_calls += name;
  return hipSuccess;
}
}  // namespace

extern "C" const char* bitnet_stub_calls(void) { return g_calls.c_str(); }
extern "C" void bitnet_stub_reset(void) { g_calls.clear(); }

extern "C" const char* hipGetErrorString(hipError_t e) {
  switch (e) {
    case hipSuccess: return "hipSuccess";
    case hipErrorOutOfMemory: return "hipErrorOutOfMemory";
    case hipErrorInvalidValue: return "hipErrorInvalidValue";
    default: return "hipError (stub)";
  }
}

namespace bitnet {

hipError_t launch_absmean_partial(const float*, int64_t, double*, int* n_partials, hipStream_t) {
  *n_partials = 1;
  return record("absmean_partial");
}
hipError_t launch_ternarize_pack(const float*, int64_t, int64_t, const double*, int, uint8_t*,
                                 float*, hipStream_t) {
  return record("ternarize_pack");
}
hipError_t launch_pack_2bit(const int8_t*, int64_t, int64_t, uint8_t*, hipStream_t) {
  return record("pack_2bit");
}
hipError_t launch_quantize(const void*, int, int64_t, int, int, int, int8_t*, float*, hipStream_t,
                           const Prologue*, int32_t*, bool nibbles, bool fp8_pairs) {
  return record(fp8_pairs ? "quantize_fp8_pairs" : (nibbles ? "quantize_nibbles" : "quantize"));
}
hipError_t launch_kv_quantize(const void*, int, int64_t, int, int, int, int8_t*, float*,
                              hipStream_t, uint8_t* packed) {
  return record(packed ? "kv_quantize_packed" : "kv_quantize");
}
hipError_t launch_ternary_matmul(const int8_t*, const float*, int64_t, int, const uint8_t*, int64_t,
                                 const float*, int, float*, int32_t* acc, hipStream_t,
                                 const int32_t*, bool nibbles, bool fp8_pairs) {
  return record(acc ? "matmul_i32"
                    : (fp8_pairs ? "matmul_fp8_pairs" : (nibbles ? "matmul_nibbles" : "matmul")));
}
hipError_t launch_quantize_tl2_order(const void*, int, int64_t, int, int, int8_t*, float*, int32_t*,
                                     hipStream_t) {
  return record("quantize_tl2_order");
}
hipError_t launch_tl2_gemv(const int8_t*, const float*, const int32_t*, int64_t, int, const uint8_t*,
                           int64_t, const float*, int, float*, hipStream_t) {
  return record("tl2_gemv");
}
hipError_t launch_gemv(const int8_t*, const float*, int64_t, int, const uint8_t*, int64_t,
                       const float*, int, float*, int32_t*, hipStream_t, bool, const int32_t*) {
  return record("gemv");
}
hipError_t launch_gemm(const int8_t*, const float*, int64_t, int, const uint8_t*, int64_t,
                       const float*, int, float*, int32_t*, hipStream_t, const int32_t*, bool) {
  return record("gemm");
}
hipError_t launch_fused_decode(const void*, int, int64_t, int, const uint8_t*, int64_t,
                               const float*, int, float*, hipStream_t, const Prologue*, int) {
  return record("fused_decode");
}
hipError_t launch_bf16_gemm_nt(const uint16_t*, const uint16_t*, int64_t, const uint16_t*, int64_t,
                               int64_t, int64_t, int64_t, float*, int64_t, const float*, float,
                               hipStream_t) {
  return record("bf16_gemm_nt");
}
hipError_t launch_expand_transpose(const uint8_t*, int64_t, int64_t, uint16_t*, hipStream_t) {
  return record("expand_transpose");
}
hipError_t launch_split_rows(const float*, int64_t, uint16_t*, uint16_t*, hipStream_t) {
  return record("split_rows");
}
hipError_t launch_scale_transpose_split(const void*, int, const float*, float, int64_t, int64_t,
                                        int64_t, uint16_t*, uint16_t*, hipStream_t) {
  return record("scale_transpose_split");
}
hipError_t launch_codes_transpose(const int8_t*, int64_t, int64_t, int64_t, uint16_t*, hipStream_t) {
  return record("codes_transpose");
}
hipError_t launch_fwht_f32(const float*, int64_t, int, float*, hipStream_t) {
  return record("fwht_f32");
}
hipError_t launch_repack_tl2(const uint8_t*, int64_t, int, uint8_t*, hipStream_t) {
  return record("repack_tl2");
}
hipError_t launch_tl2_decode(const void*, int, int, const uint8_t*, int64_t, const float*, int,
                             float*, hipStream_t) {
  return record("tl2_decode");
}
hipError_t launch_stream_read(const void*, size_t, unsigned*, hipStream_t) {
  return record("stream_read");
}
hipError_t noalloc_scratch(void** ptr) {
  *ptr = reinterpret_cast<void*>(static_cast<uintptr_t>(0x100000));  // never dereferenced
  return record("noalloc_scratch");
}

}  // namespace bitnet
