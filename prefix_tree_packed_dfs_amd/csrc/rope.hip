// tree_rope: rotary position embedding at tree depth, in place.
//
// [DAG "Positions"]: a token's position is its depth in the tree, so every
// parent-child step along a path is one position apart however far apart the
// two sit in the packed row.  Rotate-half pairing: x[i] and x[i + D/2] turn
// by pos * theta^(-2i/D).
//
// HBM-bound: every element is read once and written once.  A thread owns four
// (fp32) or eight (bf16: 16-byte accesses) consecutive frequencies of one slot
// and walks over the heads, so its sines and cosines are computed once and
// reused H times.  They are computed in fp64
// (the angle reaches tens of thousands of radians at depth 36K, where an fp32
// angle would already be off by ~1e-3) and rounded once to the storage type.
// A slot at depth 0 (a root, or a padding slot) turns by angle 0, which is the
// identity, so its rows are neither read nor written.
#include "common.h"
#include "device.h"

#include <cmath>

namespace treeattn {

template <int D>
__global__ __launch_bounds__(256) void rope_kernel_bf16(__bf16* __restrict__ x, const int32_t* __restrict__ pos,
                                                   int64_t BN, int H, double log2_theta) {
    constexpr int HALF = D / 2;
    constexpr int OCTS = HALF / 8;  // threads per slot: eight frequencies each
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t slot = gid / OCTS;
    const int oct = (int)(gid % OCTS);
    if (slot >= BN) return;
    const int p_i = pos[slot];
    if (p_i == 0) return;  // identity
    const double p = (double)p_i;
    float c[8], s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const int i = oct * 8 + u;
        // theta^(-2i/D) = 2^(-(2i/D) log2 theta)
        const double ang = p * exp2(-(double)(2 * i) / (double)D * log2_theta);
        double sd, cd;
        sincos(ang, &sd, &cd);
        c[u] = (float)cd;
        s[u] = (float)sd;
    }
    // fp32 products are enough for bf16 storage: one rounding of an fp32
    // expression whose error is far below half a bf16 ulp.
    __bf16* row = x + slot * (int64_t)H * D + oct * 8;
    auto rotate = [&](const bf16x8& va, const bf16x8& vb, bf16x8& ra, bf16x8& rb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float xa = (float)va[u], xb = (float)vb[u];
            ra[u] = (__bf16)(xa * c[u] - xb * s[u]);
            rb[u] = (__bf16)(xb * c[u] + xa * s[u]);
        }
    };
    // heads in groups of four: all loads of a group are in flight together
    int h = 0;
    for (; h + 4 <= H; h += 4) {
        bf16x8 va[4], vb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            va[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D);
            vb[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D + HALF);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            bf16x8 ra, rb;
            rotate(va[e], vb[e], ra, rb);
            *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D) = ra;
            *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D + HALF) = rb;
        }
    }
    for (; h < H; ++h) {
        bf16x8* a = reinterpret_cast<bf16x8*>(row + (int64_t)h * D);
        bf16x8* b = reinterpret_cast<bf16x8*>(row + (int64_t)h * D + HALF);
        bf16x8 ra, rb;
        rotate(*a, *b, ra, rb);
        *a = ra;
        *b = rb;
    }
}

// fp32 storage keeps its full 24-bit mantissa only if the rotation itself is
// done in fp64: the fp32 path rotates in double and rounds once.
template <int D>
__global__ __launch_bounds__(256) void rope_kernel_f32(float* __restrict__ x,
                                                       const int32_t* __restrict__ pos, int64_t BN,
                                                       int H, double log2_theta) {
    constexpr int HALF = D / 2;
    constexpr int QUADS = HALF / 4;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t slot = gid / QUADS;
    const int quad = (int)(gid % QUADS);
    if (slot >= BN) return;
    const int p_i = pos[slot];
    if (p_i == 0) return;  // identity
    const double p = (double)p_i;
    double c[4], s[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = quad * 4 + u;
        const double ang = p * exp2(-(double)(2 * i) / (double)D * log2_theta);
        sincos(ang, &s[u], &c[u]);
    }
    float* row = x + slot * (int64_t)H * D + quad * 4;
    for (int h = 0; h < H; ++h) {
        float4* a = reinterpret_cast<float4*>(row + (int64_t)h * D);
        float4* b = reinterpret_cast<float4*>(row + (int64_t)h * D + HALF);
        float4 va = *a, vb = *b;
        double xa[4] = {va.x, va.y, va.z, va.w}, xb[4] = {vb.x, vb.y, vb.z, vb.w};
        float ra[4], rb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ra[u] = (float)(xa[u] * c[u] - xb[u] * s[u]);
            rb[u] = (float)(xb[u] * c[u] + xa[u] * s[u]);
        }
        *a = make_float4(ra[0], ra[1], ra[2], ra[3]);
        *b = make_float4(rb[0], rb[1], rb[2], rb[3]);
    }
}

}  // namespace treeattn

using namespace treeattn;

extern "C" tree_status tree_rope(tree_dtype dt, void* x, int64_t B, int64_t N, int64_t H, int64_t D,
                                 const int32_t* pos_ids, float theta, void* stream) {
    clear_error();
    if (B < 0 || N < 0 || H < 0) return fail(TREE_ERR_INVALID_ARG, "negative size");
    if (D != 64 && D != 128) return fail(TREE_ERR_UNSUPPORTED, "head dim %lld (64 or 128)", (long long)D);
    if (dt != TREE_F32 && dt != TREE_BF16) return fail(TREE_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
    if (!(theta > 0.0f)) return fail(TREE_ERR_INVALID_ARG, "theta must be > 0");
    const int64_t BN = B * N;
    if (BN == 0 || H == 0) return TREE_OK;
    if (!x || !pos_ids) return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    if (H > (1 << 20)) return fail(TREE_ERR_INVALID_ARG, "too many heads");
    hipStream_t st = (hipStream_t)stream;
    const int64_t threads = BN * (dt == TREE_F32 ? D / 8 : D / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return fail(TREE_ERR_INVALID_ARG, "row too long");
    const double l2t = std::log2((double)theta);
    dim3 grid((unsigned)blocks), block(256);
    if (dt == TREE_F32) {
        if (D == 64) hipLaunchKernelGGL(rope_kernel_f32<64>, grid, block, 0, st, (float*)x, pos_ids, BN, (int)H, l2t);
        else hipLaunchKernelGGL(rope_kernel_f32<128>, grid, block, 0, st, (float*)x, pos_ids, BN, (int)H, l2t);
    } else {
        if (D == 64) hipLaunchKernelGGL(rope_kernel_bf16<64>, grid, block, 0, st, (__bf16*)x, pos_ids, BN, (int)H, l2t);
        else hipLaunchKernelGGL(rope_kernel_bf16<128>, grid, block, 0, st, (__bf16*)x, pos_ids, BN, (int)H, l2t);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TREE_ERR_DEVICE, "rope launch: %s", hipGetErrorString(e));
    return TREE_OK;
}
