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

// Both kernels rotate the H1 heads of x1 and then the H2 heads of x2 (H2 = 0:
// one tensor) at the same slots, so q and k share one launch and one set of
// sines.
template <int D>
__global__ __launch_bounds__(256) void rope_kernel_bf16(__bf16* __restrict__ x1, int H1, __bf16* __restrict__ x2,
                                                        int H2, const int32_t* __restrict__ pos, int64_t BN,
                                                        double log2_theta) {
    constexpr int HALF = D / 2;
    constexpr int OCTS = HALF / 8;  // threads per slot: eight frequencies each
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t slot = gid / OCTS;
    const int oct = (int)(gid % OCTS);
    if (slot >= BN) return;
    const int p_i = pos[slot];
    if (p_i == 0) return;  // identity
    __bf16* row1 = x1 + slot * (int64_t)H1 * D + oct * 8;
    // the first group of heads is loaded before the angles are computed
    constexpr int HG = 4;
    bf16x8 va[HG], vb[HG];
    const int h0 = min(H1, HG);
#pragma unroll
    for (int e = 0; e < HG; ++e)
        if (e < h0) {
            va[e] = *reinterpret_cast<const bf16x8*>(row1 + (int64_t)e * D);
            vb[e] = *reinterpret_cast<const bf16x8*>(row1 + (int64_t)e * D + HALF);
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
    // heads in groups of HG, all loads of a group in flight together; the
    // first group of the first tensor is already loaded
    auto walk = [&](__bf16* row, int H, bool loaded) {
        for (int h = 0; h < H; h += HG) {
            const int n = min(HG, H - h);
            if (!loaded) {
#pragma unroll
                for (int e = 0; e < HG; ++e)
                    if (e < n) {
                        va[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D);
                        vb[e] = *reinterpret_cast<const bf16x8*>(row + (int64_t)(h + e) * D + HALF);
                    }
            }
            loaded = false;
#pragma unroll
            for (int e = 0; e < HG; ++e)
                if (e < n) {
                    bf16x8 ra, rb;
                    rotate(va[e], vb[e], ra, rb);
                    *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D) = ra;
                    *reinterpret_cast<bf16x8*>(row + (int64_t)(h + e) * D + HALF) = rb;
                }
        }
    };
    walk(row1, H1, true);
    if (H2 > 0) walk(x2 + slot * (int64_t)H2 * D + oct * 8, H2, false);
}

// fp32 storage keeps its full 24-bit mantissa only if the rotation itself is
// done in fp64: the fp32 path takes its sines and rotates in double and
// rounds once.
template <int D>
__global__ __launch_bounds__(256) void rope_kernel_f32(float* __restrict__ x1, int H1, float* __restrict__ x2, int H2,
                                                       const int32_t* __restrict__ pos, int64_t BN,
                                                       double log2_theta) {
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
    auto walk = [&](float* row, int H) {
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
    };
    walk(x1 + slot * (int64_t)H1 * D + quad * 4, H1);
    if (H2 > 0) walk(x2 + slot * (int64_t)H2 * D + quad * 4, H2);
}

}  // namespace treeattn

using namespace treeattn;

namespace {

// Shared by both entry points: x2 may be null with H2 = 0.
tree_status rope_launch(tree_dtype dt, void* x1, int64_t H1, void* x2, int64_t H2, int64_t B, int64_t N, int64_t D,
                        const int32_t* pos_ids, float theta, void* stream) {
    if (B < 0 || N < 0 || H1 < 0 || H2 < 0) return fail(TREE_ERR_INVALID_ARG, "negative size");
    if (D != 64 && D != 128) return fail(TREE_ERR_UNSUPPORTED, "head dim %lld (64 or 128)", (long long)D);
    if (dt != TREE_F32 && dt != TREE_BF16) return fail(TREE_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
    if (!(theta > 0.0f)) return fail(TREE_ERR_INVALID_ARG, "theta must be > 0");
    if (H1 > (1 << 20) || H2 > (1 << 20)) return fail(TREE_ERR_INVALID_ARG, "too many heads");
    const int64_t BN = B * N;
    if (BN == 0 || H1 + H2 == 0) return TREE_OK;
    if (H1 == 0) {  // only the second tensor: rotate it as the first
        x1 = x2;
        H1 = H2;
        x2 = nullptr;
        H2 = 0;
    }
    if (!x1 || (H2 > 0 && !x2) || !pos_ids) return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    hipStream_t st = (hipStream_t)stream;
    const int64_t threads = BN * (dt == TREE_F32 ? D / 8 : D / 16);
    const int64_t blocks = (threads + 255) / 256;
    if (blocks > 0x7fffffffLL) return fail(TREE_ERR_INVALID_ARG, "row too long");
    const double l2t = std::log2((double)theta);
    dim3 grid((unsigned)blocks), block(256);
    const int h1 = (int)H1, h2 = (int)H2;
    if (dt == TREE_F32) {
        float *a = (float*)x1, *b = (float*)x2;
        if (D == 64) hipLaunchKernelGGL(rope_kernel_f32<64>, grid, block, 0, st, a, h1, b, h2, pos_ids, BN, l2t);
        else hipLaunchKernelGGL(rope_kernel_f32<128>, grid, block, 0, st, a, h1, b, h2, pos_ids, BN, l2t);
    } else {
        __bf16 *a = (__bf16*)x1, *b = (__bf16*)x2;
        if (D == 64) hipLaunchKernelGGL(rope_kernel_bf16<64>, grid, block, 0, st, a, h1, b, h2, pos_ids, BN, l2t);
        else hipLaunchKernelGGL(rope_kernel_bf16<128>, grid, block, 0, st, a, h1, b, h2, pos_ids, BN, l2t);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(TREE_ERR_DEVICE, "rope launch: %s", hipGetErrorString(e));
    return TREE_OK;
}

}  // namespace

extern "C" tree_status tree_rope(tree_dtype dt, void* x, int64_t B, int64_t N, int64_t H, int64_t D,
                                 const int32_t* pos_ids, float theta, void* stream) {
    clear_error();
    return rope_launch(dt, x, H, nullptr, 0, B, N, D, pos_ids, theta, stream);
}

extern "C" tree_status tree_rope_qk(tree_dtype dt, void* q, void* k, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                                    int64_t D, const int32_t* pos_ids, float theta, void* stream) {
    clear_error();
    if (q && k && q == k && Hq > 0 && Hkv > 0) return fail(TREE_ERR_INVALID_ARG, "q and k are the same buffer");
    return rope_launch(dt, q, Hq, k, Hkv, B, N, D, pos_ids, theta, stream);
}
