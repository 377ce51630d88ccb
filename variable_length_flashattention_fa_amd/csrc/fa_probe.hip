// Measured matrix-core ceiling: a kernel that issues nothing but independent bf16
// v_mfma_f32_32x32x16_bf16 instructions (four accumulators per wave, one or two waves
// per SIMD, one workgroup per compute unit).  Its rate is what the backward kernels can
// be held against besides the published peak (the chip's clock under a dense MFMA load
// sits below the clock that peak assumes).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "fa_internal.h"

namespace fa {
namespace {

#define FA_MFMA4 \
    "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n\t"    \
    "v_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]\n\t"  \
    "v_mfma_f32_32x32x16_bf16 a[32:47], v[0:3], v[4:7], a[32:47]\n\t"  \
    "v_mfma_f32_32x32x16_bf16 a[48:63], v[0:3], v[4:7], a[48:63]\n\t"
#define FA_ACC16(b) "a" #b "0", "a" #b "1", "a" #b "2", "a" #b "3", "a" #b "4", "a" #b "5", "a" #b "6", "a" #b "7", \
                    "a" #b "8", "a" #b "9"

// Each wave issues 8 * iters MFMAs.  Operands v0..v7 are read but never written (their
// values do not matter); the accumulators a0..a63 are declared as clobbered.
__global__ __launch_bounds__(512) void mfma_probe_kernel(int iters) {
    asm volatile("v_mov_b32 v0, 0\n\tv_mov_b32 v1, 0\n\tv_mov_b32 v2, 0\n\tv_mov_b32 v3, 0\n\t"
                 "v_mov_b32 v4, 0\n\tv_mov_b32 v5, 0\n\tv_mov_b32 v6, 0\n\tv_mov_b32 v7, 0" ::: "v0", "v1", "v2", "v3",
                 "v4", "v5", "v6", "v7");
    for (int i = 0; i < iters; ++i) {
        asm volatile(FA_MFMA4 FA_MFMA4 ::: "a0", "a1", "a2", "a3", "a4", "a5", "a6", "a7", "a8", "a9",
                     FA_ACC16(1), FA_ACC16(2), FA_ACC16(3), FA_ACC16(4), FA_ACC16(5), "a60", "a61", "a62", "a63");
    }
}

#undef FA_MFMA4
#undef FA_ACC16

}  // namespace
}  // namespace fa

extern "C" int fa_mfma_peak(int32_t waves_per_simd, double* tflops) {
    fa::clear_error();
    if (tflops == nullptr) {
        fa::set_error("fa_mfma_peak: tflops is null");
        return FA_ERR_NULLPTR;
    }
    if (waves_per_simd != 1 && waves_per_simd != 2) {
        fa::set_error("fa_mfma_peak: waves_per_simd must be 1 or 2");
        return FA_ERR_INVALID;
    }
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        fa::set_error("fa_mfma_peak: no device");
        return FA_ERR_RUNTIME;
    }
    const int cus = prop.multiProcessorCount;
    const int threads = 256 * waves_per_simd;
    const int iters = 20000;
    hipEvent_t e0 = nullptr, e1 = nullptr;
    hipError_t e = hipEventCreate(&e0);
    if (e == hipSuccess) e = hipEventCreate(&e1);
    if (e == hipSuccess) {
        fa::mfma_probe_kernel<<<dim3(cus), dim3(threads)>>>(100);  // warm the clocks up
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e0, nullptr);
    if (e == hipSuccess) {
        fa::mfma_probe_kernel<<<dim3(cus), dim3(threads)>>>(iters);
        e = hipGetLastError();
    }
    if (e == hipSuccess) e = hipEventRecord(e1, nullptr);
    if (e == hipSuccess) e = hipEventSynchronize(e1);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
    if (e0) hipEventDestroy(e0);
    if (e1) hipEventDestroy(e1);
    if (e != hipSuccess || ms <= 0.f) {
        fa::set_error(std::string("fa_mfma_peak: ") + hipGetErrorString(e));
        return FA_ERR_RUNTIME;
    }
    const double flops = static_cast<double>(cus) * threads / 64 * iters * 8 * (2.0 * 32 * 32 * 16);
    *tflops = flops / (ms * 1e-3) / 1e12;
    return FA_OK;
}
