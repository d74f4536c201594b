// Launchers that must never run: the C-ABI sanitizer driver links the ABI
// layer against these instead of the kernels, and only makes calls that the
// ABI must reject (or accept as empty) before anything is launched.  Any
// launch reaching here aborts the driver.
#include <stdio.h>
#include <stdlib.h>

#include "../../nvfp4_w4a4_quantized_02_amd/csrc/launch.h"

namespace nvfp4 {

[[noreturn]] static void launched(const char* what) {
  fprintf(stderr, "unexpected launch: %s\n", what);
  abort();
}

int launch_amax(const void*, bool, int64_t, int64_t, int64_t, uint32_t*, hipStream_t) { launched("amax"); }
void launch_quantize_packed(const void*, bool, int64_t, int64_t, int64_t, const uint32_t*, int, const float*,
                            uint8_t*, uint8_t*, float*, hipStream_t) {
  launched("quantize_packed");
}
void launch_quantize_f16(const void*, bool, int64_t, int64_t, int64_t, int64_t, const uint32_t*, int, const float*,
                         void*, float*, uint8_t*, uint8_t*, hipStream_t) {
  launched("quantize_f16");
}
void launch_fill_f32(float*, float, hipStream_t) { launched("fill_f32"); }
void launch_copy_f32(float*, const float*, hipStream_t) { launched("copy_f32"); }
void launch_dequant(const uint8_t*, const uint8_t*, const float*, int64_t, int64_t, void*, bool, int64_t,
                    hipStream_t) {
  launched("dequant");
}
void launch_fuse_rescale(const RescaleArgs&, hipStream_t) { launched("fuse_rescale"); }
void launch_fp8_quantize(const void*, bool, int64_t, int64_t, int64_t, const uint32_t*, int, const float*, uint8_t*,
                         float*, hipStream_t) {
  launched("fp8_quantize");
}
void launch_fp8_dequant(const uint8_t*, const float*, int64_t, int64_t, void*, bool, int64_t, hipStream_t) {
  launched("fp8_dequant");
}
void launch_gemm(bool, const void*, size_t, int64_t, int64_t, const uint8_t*, const uint8_t*, int64_t, const float*,
                 const float*, void*, bool, int64_t, float*, hipStream_t) {
  launched("gemm");
}
void launch_gemm_fp8w(bool, const void*, size_t, int64_t, int64_t, const uint8_t*, int64_t, const float*,
                      const float*, void*, bool, int64_t, float*, hipStream_t) {
  launched("gemm_fp8w");
}
void launch_gemv_fp8w(bool, const void*, size_t, int64_t, int64_t, const uint8_t*, int64_t, const float*,
                      const float*, void*, bool, int64_t, hipStream_t) {
  launched("gemv_fp8w");
}
void launch_gemv(bool, const void*, size_t, int64_t, int64_t, const uint8_t*, const uint8_t*, int64_t,
                 const float*, const float*, void*, bool, int64_t, hipStream_t) {
  launched("gemv");
}
bool launch_gemv_fp4(const void*, bool, int64_t, int64_t, size_t, const float*, const uint8_t*, const uint8_t*,
                     int64_t, const float*, void*, bool, size_t, void*, float*, uint8_t*, hipStream_t) {
  launched("gemv_fp4");
}
bool launch_gemv_fp4_prepared(const uint8_t*, int64_t, int64_t, const float*, const uint8_t*, const uint8_t*,
                              int64_t, const float*, void*, bool, size_t, hipStream_t) {
  launched("gemv_fp4_prepared");
}

}  // namespace nvfp4
