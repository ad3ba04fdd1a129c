// Calibration kernels for the benchmark (libmqa_calib.so; not part of the op's
// library).  They give the two machine figures the op's timings are read
// against on the GPU that runs them:
//
//   - the launch floor: an empty kernel timed the way a short call is timed
//     (a kernel that does nothing still pays dispatch and completion);
//   - the fp8 MFMA rate: waves that only issue independent
//     v_mfma_scale_f32_32x32x64_f8f6f4 (the instruction of the op's contraction,
//     131072 flops each) with no memory traffic in the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void calib_empty_kernel() {}

constexpr int kChains = 4;  // independent accumulators per wave, so the pipe never waits

__global__ __launch_bounds__(256) void calib_mfma_fp8_kernel(int iters, float *out)
{
    const int lane = threadIdx.x & 63;
    // operands: arbitrary small fp8 codes that depend on the lane (0x38 = 1.0)
    i32x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = 0x38383838 ^ ((lane + i) & 1);
        b[i] = 0x30303030 ^ ((lane + 3 * i) & 1);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
        acc[c] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c)
            acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int r = 0; r < 16; ++r)
            s += acc[c][r];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

} // namespace

extern "C" int mqa_calib_empty(int launches, hipStream_t stream)
{
    for (int i = 0; i < launches; ++i)
        hipLaunchKernelGGL(calib_empty_kernel, dim3(1), dim3(64), 0, stream);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// blocks workgroups of 4 waves, each wave issuing iters * 4 MFMAs; out needs
// blocks * 256 floats.  Flops = blocks * 4 * iters * 4 * 131072.
extern "C" int mqa_calib_mfma_fp8(int blocks, int iters, float *out, hipStream_t stream)
{
    if (blocks <= 0 || iters <= 0 || !out)
        return -1;
    hipLaunchKernelGGL(calib_mfma_fp8_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
