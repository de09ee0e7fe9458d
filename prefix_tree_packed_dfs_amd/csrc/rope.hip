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
// reused H times.  The angle reaches tens of thousands of radians at depth
// 36K, where an fp32 angle would already be off by ~1e-3, so it is formed in
// fp64: for fp32 storage the whole rotation is fp64, for bf16 the fp64 angle
// is reduced to [-pi, pi] and its sine and cosine are taken in fp32.
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
    __bf16* row = x + slot * (int64_t)H * D + oct * 8;
    // the first group of heads is loaded before the angles are computed
    constexpr int HG = 4;
    bf16x8 va[HG], vb[HG];
    const int h0 = min(H, HG);
#pragma unroll
    for (int e = 0; e < HG; ++e)
        if (e < h0) {
            va[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)e * D);
            vb[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)e * D + HALF);
        }
    // Angle p * theta^(-2i/D) in fp64, reduced to [-pi, pi] in fp64 (the
    // product and the reduction are exact to ~1e-11 rad at any depth), then
    // sine and cosine of the reduced angle in fp32 (errors near 1e-7, far
    // below half a bf16 ulp).  Frequencies: one exp2 per thread, then the
    // constant ratio theta^(-2/D) between neighbours.
    const double p = (double)p_i;
    const double ratio = exp2(-2.0 / (double)D * log2_theta);
    double f = exp2(-(double)(16 * oct) / (double)D * log2_theta);
    constexpr double kTwoPi = 6.283185307179586;
    constexpr double kInvTwoPi = 0.15915494309189535;
    float c[8], s[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        const double ang = p * f;
        const double r = fma(-rint(ang * kInvTwoPi), kTwoPi, ang);
        // sine and cosine of the fp32 head of the angle, corrected to first
        // order by its fp32 tail (the tail is below 2e-7 rad)
        const float rh = (float)r, rl = (float)(r - (double)rh);
        float sh, ch;
        sincosf(rh, &sh, &ch);
        s[u] = fmaf(ch, rl, sh);
        c[u] = fmaf(-sh, rl, ch);
        f *= ratio;
    }
    // fp32 products are enough for bf16 storage: one rounding of an fp32
    // expression whose error is far below half a bf16 ulp.
    auto rotate = [&](const bf16x8& a, const bf16x8& b, bf16x8& ra, bf16x8& rb) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float xa = (float)a[u], xb = (float)b[u];
            ra[u] = (__bf16)(xa * c[u] - xb * s[u]);
            rb[u] = (__bf16)(xb * c[u] + xa * s[u]);
        }
    };
    for (int h = 0;;) {
        const int n = min(HG, H - h);
#pragma unroll
        for (int e = 0; e < HG; ++e)
            if (e < n) {
                bf16x8 ra, rb;
                rotate(va[e], vb[e], ra, rb);
                *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D) = ra;
                *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D + HALF) = rb;
            }
        h += HG;
        if (h >= H) break;
        const int m = min(HG, H - h);
#pragma unroll
        for (int e = 0; e < HG; ++e)
            if (e < m) {
                va[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D);
                vb[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D + HALF);
            }
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
