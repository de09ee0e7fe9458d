// tree_mfma_peak: a measurement aid, not part of the attention path.
//
// Every wave runs a long chain of bf16 32x32x16 matrix products on register
// operands over four independent accumulators, so the matrix cores are the
// only limit.  Timing it gives the matrix-core rate this GPU sustains, which
// the benchmark reports beside the published peak as a second denominator.
#include "common.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr int kPeakAcc = 4;

__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters, float* __restrict__ sink) {
    // operands from the thread index, so the products cannot be folded at compile time
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
        b[i] = (__bf16)(float)((3 * threadIdx.x + i) & 7);
    }
    f32x16 acc[kPeakAcc];
#pragma unroll
    for (int k = 0; k < kPeakAcc; ++k) zero(acc[k]);
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int k = 0; k < kPeakAcc; ++k) acc[k] = mfma32(a, b, acc[k]);
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < kPeakAcc; ++k)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[k][r];
    if (s == -1.f) sink[threadIdx.x] = s;  // never true for these operands; keeps the products live
}

}  // namespace

}  // namespace treeattn

using namespace treeattn;

extern "C" tree_status tree_mfma_peak(int64_t blocks, int64_t iters, float* sink, double* flops, void* stream) {
    clear_error();
    if (blocks <= 0 || blocks > (1 << 24) || iters <= 0 || iters > (1 << 30))
        return fail(TREE_ERR_INVALID_ARG, "blocks %lld, iters %lld", (long long)blocks, (long long)iters);
    if (!sink || !flops) return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    // 256 threads = 4 waves per block; 32 x 32 x 16 x 2 flops per product
    *flops = (double)blocks * 4.0 * (double)iters * kPeakAcc * 32768.0;
    hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, (int)iters, sink);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TREE_ERR_DEVICE, "mfma peak launch: %s", hipGetErrorString(e));
    return TREE_OK;
}
