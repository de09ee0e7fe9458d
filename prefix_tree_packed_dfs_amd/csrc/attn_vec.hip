// Vector-ALU attention kernels over a packed tree (the fp32 path).
//
// Mask: query i sees key j iff j <= i <= subtree_end[j] (the pre-order /
// exit-order interval of [ART "Token-mixing layers"]; equivalently j is i or
// one of its ancestors [DAG "The mask"]).  A 64-key tile whose largest
// subtree_end is below the first query of the block has no visible pair and
// is skipped whole.
//
// kVecLanes lanes own one query row (forward, dq) or one key row (dk/dv);
// the other side of the product is staged in LDS 64 rows at a time.  fp32
// accumulation and softmax throughout.  These kernels serve the fp32 dtype,
// whose tolerance (1e-5 relative) the bf16 matrix-core path cannot meet.
#include "attn_vec.h"
#include "device.h"

#include <cmath>

namespace treeattn {

namespace {

constexpr int TB = 64;  // threads per block = keys per staged tile
// Lanes per query (forward, dq) or key (dk/dv) row: lane c owns the
// dimensions c, c + kVecLanes, ...; dot products are summed over the row's
// lanes by log2(kVecLanes) exchanges.  An eighth of the serial work per lane
// and eight times the blocks of one lane per row (16 lanes measured the same).
constexpr int kVecLanes = 8;

template <typename T, int D>
__global__ __launch_bounds__(TB) void vec_fwd(const T* __restrict__ q, const T* __restrict__ k,
                                              const T* __restrict__ v, const int32_t* __restrict__ se,
                                              int N, int Hq, int Hkv, float scale, T* __restrict__ out,
                                              float* __restrict__ lse) {
    constexpr int QPB = TB / kVecLanes, DL = D / kVecLanes;
    __shared__ float ks[TB][D];
    __shared__ float vs[TB][D];
    __shared__ int ses[TB];
    const int b = blockIdx.z, h = blockIdx.y, i0 = blockIdx.x * QPB, t = threadIdx.x;
    const int c = t % kVecLanes, i = i0 + t / kVecLanes;
    const int g = h / (Hq / Hkv);
    const int i_last = min(i0 + QPB, N) - 1;
    float qr[DL], o[DL];
    const T* qp = q + (((int64_t)b * N + min(i, N - 1)) * Hq + h) * D + c;
#pragma unroll
    for (int x = 0; x < DL; ++x) {
        qr[x] = to_f32(qp[kVecLanes * x]) * scale;
        o[x] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    const int32_t* ser = se + (int64_t)b * N;
    for (int j0 = 0; j0 <= i_last; j0 += TB) {
        const int j = j0 + t;
        const int sej = j < N ? ser[j] : -1;
        if (wave_max_i32(sej) < i0) continue;  // no key of this tile is visible to the block
        ses[t] = sej;
        for (int e = t; e < TB * D; e += TB) {
            const int r = e / D, cc = e % D, jj = j0 + r;
            float kv = 0.f, vv = 0.f;
            if (jj < N) {
                const int64_t off = (((int64_t)b * N + jj) * Hkv + g) * D + cc;
                kv = to_f32(k[off]);
                vv = to_f32(v[off]);
            }
            ks[r][cc] = kv;
            vs[r][cc] = vv;
        }
        __syncthreads();
        if (i < N) {
            const int jn = min(TB, N - j0);
            for (int r = 0; r < jn; ++r) {
                const int jj = j0 + r;
                if (jj > i || i > ses[r]) continue;  // the same for every lane of a query
                float s = 0.f;
#pragma unroll
                for (int x = 0; x < DL; ++x) s = fmaf(qr[x], ks[r][c + kVecLanes * x], s);
#pragma unroll
                for (int w = 1; w < kVecLanes; w <<= 1) s += __shfl_xor(s, w, 64);
                const float mn = fmaxf(m, s);
                const float corr = expf(m - mn), p = expf(s - mn);
                l = l * corr + p;
#pragma unroll
                for (int x = 0; x < DL; ++x) o[x] = fmaf(p, vs[r][c + kVecLanes * x], o[x] * corr);
                m = mn;
            }
        }
        __syncthreads();
    }
    if (i < N) {
        const float inv = 1.f / l;
        T* op = out + (((int64_t)b * N + i) * Hq + h) * D + c;
#pragma unroll
        for (int x = 0; x < DL; ++x) op[kVecLanes * x] = from_f32<T>(o[x] * inv);
        if (c == 0) lse[((int64_t)b * Hq + h) * N + i] = m + logf(l);
    }
}

// delta[b,h,i] = sum_d dout * out (the row term of the softmax gradient)
template <typename T, int D>
__global__ __launch_bounds__(256) void vec_delta(const T* __restrict__ out, const T* __restrict__ dout,
                                                 int64_t rows, int N, int Hq, float* __restrict__ delta) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // r = (b*N + i)*Hq + h
    if (r >= rows) return;
    const T* a = out + r * D;
    const T* c = dout + r * D;
    float s = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; ++d) s = fmaf(to_f32(a[d]), to_f32(c[d]), s);
    const int h = (int)(r % Hq);
    const int64_t bi = r / Hq;
    const int64_t b = bi / N, i = bi % N;
    delta[(b * Hq + h) * N + i] = s;
}

template <typename T, int D>
__global__ __launch_bounds__(TB) void vec_dq(const T* __restrict__ q, const T* __restrict__ k,
                                             const T* __restrict__ v, const int32_t* __restrict__ se,
                                             const float* __restrict__ lse, const float* __restrict__ delta,
                                             const T* __restrict__ dout, int N, int Hq, int Hkv, float scale,
                                             T* __restrict__ dq) {
    constexpr int QPB = TB / kVecLanes, DL = D / kVecLanes;
    __shared__ float ks[TB][D];
    __shared__ float vs[TB][D];
    __shared__ int ses[TB];
    const int b = blockIdx.z, h = blockIdx.y, i0 = blockIdx.x * QPB, t = threadIdx.x;
    const int c = t % kVecLanes, i = i0 + t / kVecLanes;
    const int g = h / (Hq / Hkv);
    const int i_last = min(i0 + QPB, N) - 1;
    const int ic = min(i, N - 1);
    float qr[DL], dor[DL], acc[DL];
    const T* qp = q + (((int64_t)b * N + ic) * Hq + h) * D + c;
    const T* dp = dout + (((int64_t)b * N + ic) * Hq + h) * D + c;
#pragma unroll
    for (int x = 0; x < DL; ++x) {
        qr[x] = to_f32(qp[kVecLanes * x]) * scale;
        dor[x] = to_f32(dp[kVecLanes * x]);
        acc[x] = 0.f;
    }
    const float li = lse[((int64_t)b * Hq + h) * N + ic];
    const float di = delta[((int64_t)b * Hq + h) * N + ic];
    const int32_t* ser = se + (int64_t)b * N;
    for (int j0 = 0; j0 <= i_last; j0 += TB) {
        const int j = j0 + t;
        const int sej = j < N ? ser[j] : -1;
        if (wave_max_i32(sej) < i0) continue;
        ses[t] = sej;
        for (int e = t; e < TB * D; e += TB) {
            const int r = e / D, cc = e % D, jj = j0 + r;
            float kv = 0.f, vv = 0.f;
            if (jj < N) {
                const int64_t off = (((int64_t)b * N + jj) * Hkv + g) * D + cc;
                kv = to_f32(k[off]);
                vv = to_f32(v[off]);
            }
            ks[r][cc] = kv;
            vs[r][cc] = vv;
        }
        __syncthreads();
        if (i < N) {
            const int jn = min(TB, N - j0);
            for (int r = 0; r < jn; ++r) {
                const int jj = j0 + r;
                if (jj > i || i > ses[r]) continue;  // the same for every lane of a query
                float s = 0.f, dpv = 0.f;
#pragma unroll
                for (int x = 0; x < DL; ++x) {
                    s = fmaf(qr[x], ks[r][c + kVecLanes * x], s);
                    dpv = fmaf(dor[x], vs[r][c + kVecLanes * x], dpv);
                }
#pragma unroll
                for (int w = 1; w < kVecLanes; w <<= 1) {
                    s += __shfl_xor(s, w, 64);
                    dpv += __shfl_xor(dpv, w, 64);
                }
                const float ds = expf(s - li) * (dpv - di);
#pragma unroll
                for (int x = 0; x < DL; ++x) acc[x] = fmaf(ds, ks[r][c + kVecLanes * x], acc[x]);
            }
        }
        __syncthreads();
    }
    if (i < N) {
        T* o = dq + (((int64_t)b * N + i) * Hq + h) * D + c;
#pragma unroll
        for (int x = 0; x < DL; ++x) o[kVecLanes * x] = from_f32<T>(acc[x] * scale);
    }
}

// kVecLanes lanes per key row of KV head g, 64 / kVecLanes keys per block;
// loops over the query heads of the group and over the queries i in
// [j, subtree_end[j]] (exactly the queries that see key j), staged 64 at a
// time.
template <typename T, int D>
__global__ __launch_bounds__(TB) void vec_dkdv(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, const int32_t* __restrict__ se,
                                               const float* __restrict__ lse, const float* __restrict__ delta,
                                               const T* __restrict__ dout, int N, int Hq, int Hkv, float scale,
                                               T* __restrict__ dk, T* __restrict__ dv) {
    constexpr int KPB = TB / kVecLanes, DL = D / kVecLanes;
    __shared__ float qs[TB][D];
    __shared__ float dos[TB][D];
    __shared__ float ls[TB], dls[TB];
    const int b = blockIdx.z, g = blockIdx.y, t = threadIdx.x;
    const int c = t % kVecLanes;
    const int j0 = blockIdx.x * KPB, j = j0 + t / kVecLanes;
    const int G = Hq / Hkv;
    const int32_t* ser = se + (int64_t)b * N;
    const int sej = j < N ? ser[j] : -1;
    const int q_end = wave_max_i32(sej);  // last query any key of the block serves
    float kr[DL], vr[DL], adk[DL], adv[DL];
    {
        const int64_t off = (((int64_t)b * N + min(j, N - 1)) * Hkv + g) * D + c;
#pragma unroll
        for (int x = 0; x < DL; ++x) {
            kr[x] = to_f32(k[off + kVecLanes * x]);
            vr[x] = to_f32(v[off + kVecLanes * x]);
            adk[x] = adv[x] = 0.f;
        }
    }
    for (int hh = 0; hh < G; ++hh) {
        const int h = g * G + hh;
        for (int i0 = j0; i0 <= q_end; i0 += TB) {
            for (int e = t; e < TB * D; e += TB) {
                const int r = e / D, cc = e % D, ii = i0 + r;
                float qv = 0.f, dv_ = 0.f;
                if (ii < N) {
                    const int64_t off = (((int64_t)b * N + ii) * Hq + h) * D + cc;
                    qv = to_f32(q[off]) * scale;
                    dv_ = to_f32(dout[off]);
                }
                qs[r][cc] = qv;
                dos[r][cc] = dv_;
            }
            {
                const int ii = i0 + t;
                ls[t] = ii < N ? lse[((int64_t)b * Hq + h) * N + ii] : 0.f;
                dls[t] = ii < N ? delta[((int64_t)b * Hq + h) * N + ii] : 0.f;
            }
            __syncthreads();
            if (j < N) {
                const int rn = min(TB, N - i0);
                for (int r = 0; r < rn; ++r) {
                    const int ii = i0 + r;
                    if (ii < j || ii > sej) continue;  // the same for every lane of a key
                    float s = 0.f, dpv = 0.f;
#pragma unroll
                    for (int x = 0; x < DL; ++x) {
                        s = fmaf(qs[r][c + kVecLanes * x], kr[x], s);
                        dpv = fmaf(dos[r][c + kVecLanes * x], vr[x], dpv);
                    }
#pragma unroll
                    for (int o = 1; o < kVecLanes; o <<= 1) {
                        s += __shfl_xor(s, o, 64);
                        dpv += __shfl_xor(dpv, o, 64);
                    }
                    const float p = expf(s - ls[r]);
                    const float ds = p * (dpv - dls[r]);
#pragma unroll
                    for (int x = 0; x < DL; ++x) {
                        adv[x] = fmaf(p, dos[r][c + kVecLanes * x], adv[x]);
                        adk[x] = fmaf(ds, qs[r][c + kVecLanes * x], adk[x]);  // q already carries the scale
                    }
                }
            }
            __syncthreads();
        }
    }
    if (j < N) {
        T* okp = dk + (((int64_t)b * N + j) * Hkv + g) * D + c;
        T* ovp = dv + (((int64_t)b * N + j) * Hkv + g) * D + c;
#pragma unroll
        for (int x = 0; x < DL; ++x) {
            okp[kVecLanes * x] = from_f32<T>(adk[x]);
            ovp[kVecLanes * x] = from_f32<T>(adv[x]);
        }
    }
}

template <typename T, int D>
hipError_t launch_fwd(const AttnArgs& a, hipStream_t st) {
    constexpr int QPB = TB / kVecLanes;
    dim3 grid((a.N + QPB - 1) / QPB, a.Hq, a.B), block(TB);
    hipLaunchKernelGGL((vec_fwd<T, D>), grid, block, 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v,
                       a.se, a.N, a.Hq, a.Hkv, a.scale, (T*)a.out, a.lse);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd(const AttnArgs& a, float* delta, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.N * a.Hq;
    hipLaunchKernelGGL((vec_delta<T, D>), dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st,
                       (const T*)a.out, (const T*)a.dout, rows, a.N, a.Hq, delta);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    constexpr int RPB = TB / kVecLanes;  // query (dq) or key (dk/dv) rows per block
    dim3 gq((a.N + RPB - 1) / RPB, a.Hq, a.B), gk((a.N + RPB - 1) / RPB, a.Hkv, a.B), block(TB);
    hipLaunchKernelGGL((vec_dq<T, D>), gq, block, 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.se,
                       a.lse, delta, (const T*)a.dout, a.N, a.Hq, a.Hkv, a.scale, (T*)a.dq);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((vec_dkdv<T, D>), gk, block, 0, st, (const T*)a.q, (const T*)a.k, (const T*)a.v, a.se,
                       a.lse, delta, (const T*)a.dout, a.N, a.Hq, a.Hkv, a.scale, (T*)a.dk, (T*)a.dv);
    return hipGetLastError();
}

}  // namespace

hipError_t vec_attn_fwd(const AttnArgs& a, hipStream_t st) {
    if (a.dt == TREE_F32) return a.D == 64 ? launch_fwd<float, 64>(a, st) : launch_fwd<float, 128>(a, st);
    return a.D == 64 ? launch_fwd<__bf16, 64>(a, st) : launch_fwd<__bf16, 128>(a, st);
}

hipError_t vec_attn_bwd(const AttnArgs& a, float* delta, hipStream_t st) {
    if (a.dt == TREE_F32)
        return a.D == 64 ? launch_bwd<float, 64>(a, delta, st) : launch_bwd<float, 128>(a, delta, st);
    return a.D == 64 ? launch_bwd<__bf16, 64>(a, delta, st) : launch_bwd<__bf16, 128>(a, delta, st);
}

}  // namespace treeattn
