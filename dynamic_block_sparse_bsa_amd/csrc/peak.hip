// Dense MFMA throughput probe for the benchmark: how many bf16 (or fp8) MFMA flops per
// second this card sustains when every SIMD issues nothing but independent MFMAs with
// register operands. It sets the attainable ceiling that the attention kernel's rate is
// compared with, beside the datasheet peak (the card holds a lower clock under dense MFMA
// load than the 2.4 GHz the datasheet figure assumes).
//
// Not part of libbsa's interface: built into its own library, libbsa_peak.so, and called
// only by bench.py.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

namespace {

constexpr int kChains = 4;  // independent accumulators per wave

// Each wave runs `iters` rounds of kChains x 4 MFMAs on its own registers and writes one
// value that depends on every accumulator, so nothing is optimised away.
template <bool FP8>
__global__ void __launch_bounds__(256) peak_kernel(int iters, float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) acc[c] = (f32x16){};
    if constexpr (FP8) {
        const int v = 0x38383838 ^ (lane & 7);  // E4M3 values near 1
        const i32x8 a = {v, v, v, v, v, v, v, v}, b = {v, v + 1, v, v + 1, v, v + 1, v, v + 1};
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < kChains; ++c)
                    acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
        }
    } else {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            a[e] = (__bf16)(1.0f + 0.001f * (lane + e));
            b[e] = (__bf16)(1.0f - 0.001f * (lane - e));
        }
        for (int i = 0; i < iters; ++i) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < kChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[c][e];
    sink[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Flops one launch of bsa_peak_run performs.
double bsa_peak_flops(int fp8, int workgroups, int iters) {
    const double per_mfma = fp8 ? 32.0 * 32.0 * 64.0 * 2.0 : 32.0 * 32.0 * 16.0 * 2.0;
    return per_mfma * 4.0 * kChains * (double)iters * 4.0 /* waves */ * (double)workgroups;
}

// Launches `workgroups` workgroups of four waves; sink holds workgroups * 256 floats.
int bsa_peak_run(int fp8, int workgroups, int iters, float* sink, void* stream) {
    if (workgroups < 1 || iters < 1 || !sink) return 1;
    if (fp8)
        hipLaunchKernelGGL(peak_kernel<true>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, sink);
    else
        hipLaunchKernelGGL(peak_kernel<false>, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
