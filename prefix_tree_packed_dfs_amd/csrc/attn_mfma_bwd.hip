// bf16 attention backward over a packed tree on CDNA4 matrix cores.
//
// The pages give no backward pass; this is the exact gradient of the forward
// (same interval mask j <= i <= subtree_end[j], same tile classes).  With
// P = exp(scale * q.k - lse) and delta_i = dout_i . out_i:
//   dV = P^T dout,   dP = dout V^T,   dS = P * (dP - delta),
//   dK = scale dS^T Q,   dQ = scale dS K.
// Three kernels, no atomics (the result is bitwise reproducible):
//   bwd_prep  delta, Q^T and dout^T per query head, K^T per KV head (rows
//             permuted in 16-row groups to match the accumulator order), and
//             the per-tile subtree_end range;
//   bwd_dkdv  KV-stationary: a workgroup owns 128 keys of one KV head (32 per
//             wave, K and V held as MFMA operands in registers) and walks the
//             query blocks [j0, max subtree_end] for every query head of the
//             group.  A wave skips a 32x32 block whose keys see none of its
//             queries and drops the mask where all of them are visible.
//               S = Q K^T, dP = dout V^T     (A = Q, dout from LDS)
//               dV^T += dout^T P, dK^T += Q^T dS   (B = P, dS straight from
//               the S / dP accumulators: a lane holds one key and 16 queries)
//   bwd_dq    query-stationary, shaped like the forward: S^T = K Q^T and
//             dP^T = V dout^T with Q, dout in registers, then
//             dQ^T += K^T dS^T with dS^T taken from the accumulator.
// dK/dV and dQ recompute S and dP separately (7 products instead of 5) so
// that no partial dQ has to be summed across workgroups.
#include <climits>

#include "attn_mfma.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
    return *reinterpret_cast<const T*>(p);
}

// grid (T, Hq, B), 256 threads
template <int D>
__global__ __launch_bounds__(256) void bwd_prep(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                const __bf16* __restrict__ out, const __bf16* __restrict__ dout,
                                                const int32_t* __restrict__ se, int N, int Hq, int Hkv, int T,
                                                float* __restrict__ delta, __bf16* __restrict__ qt,
                                                __bf16* __restrict__ dot, __bf16* __restrict__ ktr,
                                                int32_t* __restrict__ tmin, int32_t* __restrict__ tmax) {
    constexpr int CPR = D / 8;
    __shared__ __attribute__((aligned(16))) __bf16 ta[KT][D + 8];
    __shared__ __attribute__((aligned(16))) __bf16 tb[KT][D + 8];
    const int t = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int j0 = t * KT;
    const int64_t row_len = (int64_t)T * KT;
    for (int e = tid; e < KT * CPR; e += 256) {
        const int r = e / CPR, c = e % CPR, j = j0 + r;
        bf16x8 vq = {}, vd = {};
        if (j < N) {
            const int64_t off = (((int64_t)b * N + j) * Hq + h) * D + c * 8;
            vq = ld16<bf16x8>(q + off);
            vd = ld16<bf16x8>(dout + off);
        }
        *reinterpret_cast<bf16x8*>(&ta[r][c * 8]) = vq;
        *reinterpret_cast<bf16x8*>(&tb[r][c * 8]) = vd;
    }
    {  // delta: four threads per row
        const int r = tid >> 2, part = tid & 3, j = j0 + r;
        float s = 0.f;
        if (j < N) {
            const int64_t off = (((int64_t)b * N + j) * Hq + h) * D + part * (D / 4);
#pragma unroll
            for (int c = 0; c < D / 4; c += 8) {
                const bf16x8 a = ld16<bf16x8>(out + off + c), d8 = ld16<bf16x8>(dout + off + c);
#pragma unroll
                for (int u = 0; u < 8; ++u) s = fmaf((float)a[u], (float)d8[u], s);
            }
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        if (part == 0 && j < N) delta[((int64_t)b * Hq + h) * N + j] = s;
    }
    __syncthreads();
    __bf16* dst_q = qt + ((int64_t)b * Hq + h) * D * row_len + j0;
    __bf16* dst_d = dot + ((int64_t)b * Hq + h) * D * row_len + j0;
    for (int e = tid; e < D * (KT / 8); e += 256) {
        const int d = e / (KT / 8), c = e % (KT / 8);
        bf16x8 oq, od;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = c * 8 + u;
            const int row = (p >> 4) * 16 + inv_phys16(p & 15);
            oq[u] = ta[row][d];
            od[u] = tb[row][d];
        }
        *reinterpret_cast<bf16x8*>(dst_q + (int64_t)d * row_len + c * 8) = oq;
        *reinterpret_cast<bf16x8*>(dst_d + (int64_t)d * row_len + c * 8) = od;
    }
    if (h < Hkv) {  // K^T of KV head h
        __syncthreads();
        for (int e = tid; e < KT * CPR; e += 256) {
            const int r = e / CPR, c = e % CPR, j = j0 + r;
            bf16x8 vk = {};
            if (j < N) vk = ld16<bf16x8>(k + (((int64_t)b * N + j) * Hkv + h) * D + c * 8);
            *reinterpret_cast<bf16x8*>(&ta[r][c * 8]) = vk;
        }
        __syncthreads();
        __bf16* dst_k = ktr + ((int64_t)b * Hkv + h) * D * row_len + j0;
        for (int e = tid; e < D * (KT / 8); e += 256) {
            const int d = e / (KT / 8), c = e % (KT / 8);
            bf16x8 ok;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int p = c * 8 + u;
                ok[u] = ta[(p >> 4) * 16 + inv_phys16(p & 15)][d];
            }
            *reinterpret_cast<bf16x8*>(dst_k + (int64_t)d * row_len + c * 8) = ok;
        }
    }
    if (h == 0 && tid < 64) {
        const int j = j0 + tid;
        const int s = j < N ? se[(int64_t)b * N + j] : -1;
        const int mn = wave_min_i32(j < N ? s : INT_MAX);
        const int mx = wave_max_i32(s);
        if (tid == 0) {
            tmin[(int64_t)b * T + t] = mn;
            tmax[(int64_t)b * T + t] = mx;
        }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: grid (ceil(N/128) * B * Hkv), 256 threads
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                   const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                                                   const float* __restrict__ lse, const float* __restrict__ delta,
                                                   const __bf16* __restrict__ qt, const __bf16* __restrict__ dot,
                                                   const int32_t* __restrict__ se, int B, int N, int Hq, int Hkv,
                                                   int T, float scale_log2, float scale, __bf16* __restrict__ dk,
                                                   __bf16* __restrict__ dv) {
    constexpr int NC = D / 16, NDB = D / 32;
    constexpr int RSTR = D * 2 + 16;     // LDS bytes per natural row (32 rows per block)
    constexpr int TSTR = 32 * 2 + 16;    // LDS bytes per transposed row (32 positions)
    constexpr int NBYTES = 32 * RSTR;
    constexpr int TBYTES = D * TSTR;
    constexpr int BUF = 2 * NBYTES + 2 * TBYTES;
    constexpr int NCH = 32 * D / 8 / 256;  // 16-byte chunks per thread per natural tile
    constexpr int TCH = D * 32 / 8 / 256;  // ... per transposed tile
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
    __shared__ float l2s[2][32], dls[2][32];
    __shared__ int qmax_s[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int GH = B * Hkv;
    const int gi = blockIdx.x % GH;
    const int kt_i = blockIdx.x / GH;  // ascending: keys early in the row have the longest query ranges
    const int g = gi % Hkv, b = gi / Hkv;
    const int G = Hq / Hkv;
    const int j0 = kt_i * 128;
    const int j0w = j0 + 32 * wave;
    const int jk = j0w + l32;
    const bool kvalid = jk < N;
    const int32_t* seb = se + (int64_t)b * N;
    const int sek = kvalid ? seb[jk] : -1;
    const int wmax = wave_max_i32(sek);
    const int wmin = wave_min_i32(kvalid ? sek : INT_MAX);

    bf16x8 kf[NC], vf[NC];
    {
        const int64_t off = (((int64_t)b * N + jk) * Hkv + g) * D + hi * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 z = {};
            kf[c] = kvalid ? ld16<bf16x8>(k + off + 16 * c) : z;
            vf[c] = kvalid ? ld16<bf16x8>(v + off + 16 * c) : z;
        }
    }
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        zero(dkt[db]);
        zero(dvt[db]);
    }
    if (lane == 0) qmax_s[wave] = wmax;
    __syncthreads();
    const int qmax = max(max(qmax_s[0], qmax_s[1]), max(qmax_s[2], qmax_s[3]));
    const int pb0 = j0 / 32, pb1 = qmax / 32;
    const int nvis = (pb1 - pb0 + 1) * G;
    const int64_t row_len = (int64_t)T * KT;

    bf16x8 sq[NCH], sd[NCH], sqt[TCH], sdt[TCH];
    float sl = 0.f, sdl = 0.f;
    auto load_vis = [&](int vi) {
        const int i0 = (pb0 + vi / G) * 32;
        const int h = g * G + vi % G;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int e = tid + 256 * u;
            const int r = e / (D / 8), c = e % (D / 8), i = i0 + r;
            const int64_t off = (((int64_t)b * N + i) * Hq + h) * D + c * 8;
            bf16x8 z = {};
            sq[u] = i < N ? ld16<bf16x8>(q + off) : z;
            sd[u] = i < N ? ld16<bf16x8>(dout + off) : z;
        }
#pragma unroll
        for (int u = 0; u < TCH; ++u) {
            const int e = tid + 256 * u;
            const int d = e / 4, c = e % 4;
            const int64_t off = ((int64_t)b * Hq + h) * D * row_len + (int64_t)d * row_len + i0 + c * 8;
            sqt[u] = ld16<bf16x8>(qt + off);
            sdt[u] = ld16<bf16x8>(dot + off);
        }
        if (tid < 32) {
            const int i = i0 + tid;
            sl = i < N ? lse[((int64_t)b * Hq + h) * N + i] * kLog2e : 0.f;
            sdl = i < N ? delta[((int64_t)b * Hq + h) * N + i] : 0.f;
        }
    };
    auto store_vis = [&](int buf) {
        char* qn = smem + buf * BUF;
        char* dn = qn + NBYTES;
        char* qtt = dn + NBYTES;
        char* dtt = qtt + TBYTES;
#pragma unroll
        for (int u = 0; u < NCH; ++u) {
            const int e = tid + 256 * u;
            const int o = (e / (D / 8)) * RSTR + (e % (D / 8)) * 16;
            *reinterpret_cast<bf16x8*>(qn + o) = sq[u];
            *reinterpret_cast<bf16x8*>(dn + o) = sd[u];
        }
#pragma unroll
        for (int u = 0; u < TCH; ++u) {
            const int e = tid + 256 * u;
            const int o = (e / 4) * TSTR + (e % 4) * 16;
            *reinterpret_cast<bf16x8*>(qtt + o) = sqt[u];
            *reinterpret_cast<bf16x8*>(dtt + o) = sdt[u];
        }
        if (tid < 32) {
            l2s[buf][tid] = sl;
            dls[buf][tid] = sdl;
        }
    };

    load_vis(0);
    store_vis(0);
    __syncthreads();
    int cur = 0;
    for (int vi = 0; vi < nvis; ++vi) {
        if (vi + 1 < nvis) load_vis(vi + 1);
        const int i_lo = (pb0 + vi / G) * 32;
        const bool skip = (j0w > i_lo + 31) || (wmax < i_lo);
        if (!skip) {
            const bool full = (j0w + 31 <= i_lo) && (wmin >= i_lo + 31);
            const char* qn = smem + cur * BUF;
            const char* dn = qn + NBYTES;
            const char* qtt = dn + NBYTES;
            const char* dtt = qtt + TBYTES;
            f32x16 s, dp;
            zero(s);
            zero(dp);
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int o = l32 * RSTR + (hi * 8 + 16 * c) * 2;
                s = mfma32(ld16<bf16x8>(qn + o), kf[c], s);
                dp = mfma32(ld16<bf16x8>(dn + o), vf[c], dp);
            }
            bf16x8 pbf[2], dsf[2];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = acc_row(r, hi);
                const int i = i_lo + m;
                float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -l2s[cur][m]));
                if (!full && !(jk <= i && i <= sek)) p = 0.f;
                const float ds = p * (dp[r] - dls[cur][m]);
                pbf[r >> 3][r & 7] = (__bf16)p;
                dsf[r >> 3][r & 7] = (__bf16)ds;
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const int o = (db * 32 + l32) * TSTR + (c2 * 16 + hi * 8) * 2;
                    dvt[db] = mfma32(ld16<bf16x8>(dtt + o), pbf[c2], dvt[db]);
                    dkt[db] = mfma32(ld16<bf16x8>(qtt + o), dsf[c2], dkt[db]);
                }
        }
        if (vi + 1 < nvis) store_vis(cur ^ 1);
        __syncthreads();
        cur ^= 1;
    }
    if (kvalid) {
        __bf16* okp = dk + (((int64_t)b * N + jk) * Hkv + g) * D;
        __bf16* ovp = dv + (((int64_t)b * N + jk) * Hkv + g) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                bf16x4 a4, b4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a4[e] = (__bf16)(dkt[db][grp * 4 + e] * scale);
                    b4[e] = (__bf16)dvt[db][grp * 4 + e];
                }
                *reinterpret_cast<bf16x4*>(okp + db * 32 + grp * 8 + hi * 4) = a4;
                *reinterpret_cast<bf16x4*>(ovp + db * 32 + grp * 8 + hi * 4) = b4;
            }
    }
}

// ---------------------------------------------------------------------------
// dQ: grid (n_qtiles * B * Hkv * n_chunks), 256 threads; same work split as
// the forward (BM positions x HB heads per workgroup, 64 rows per wave).
// ---------------------------------------------------------------------------
template <int D, int HB>
__global__ __launch_bounds__(256, 1) void bwd_dq(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                 const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                                                 const float* __restrict__ lse, const float* __restrict__ delta,
                                                 const __bf16* __restrict__ ktr, const int32_t* __restrict__ se,
                                                 const int32_t* __restrict__ tmin, const int32_t* __restrict__ tmax,
                                                 int B, int N, int Hq, int Hkv, int T, int n_qtiles, int n_chunks,
                                                 float scale_log2, float scale, __bf16* __restrict__ dq) {
    constexpr int BM = 256 / HB;
    constexpr int NC = D / 16, NDB = D / 32;
    constexpr int KSTR = D * 2 + 16;     // natural K / V rows
    constexpr int TSTR = KT * 2 + 16;    // K^T rows
    constexpr int KBYTES = KT * KSTR;
    constexpr int TBYTES = D * TSTR;
    constexpr int BUF = 2 * KBYTES + TBYTES;
    constexpr int KCH = KT * D / 8 / 256;
    constexpr int TCH = D * KT / 8 / 256;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];
    __shared__ int se_s[2][KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int GH = B * Hkv * n_chunks;
    const int gi = blockIdx.x % GH;
    const int qi = blockIdx.x / GH;
    const int qtile = n_qtiles - 1 - qi;
    const int chunk = gi % n_chunks;
    const int g = (gi / n_chunks) % Hkv;
    const int b = gi / (n_chunks * Hkv);
    const int G = Hq / Hkv;
    const int head_base = g * G + chunk * HB;
    const int i0 = qtile * BM;
    const int i_last = min(i0 + BM, N) - 1;
    const int t_last = i_last / KT;
    const int32_t* tmaxb = tmax + (int64_t)b * T;
    const int32_t* tminb = tmin + (int64_t)b * T;
    const int32_t* seb = se + (int64_t)b * N;

    int posb[2], head[2];
    bf16x8 qf[2][NC], df[2][NC];
    float l2q[2], dlq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int bi = 2 * wave + qb;
        head[qb] = head_base + bi % HB;
        posb[qb] = i0 + (bi / HB) * 32;
        const int p = posb[qb] + l32;
        const int64_t off = (((int64_t)b * N + p) * Hq + head[qb]) * D + hi * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 z = {};
            qf[qb][c] = p < N ? ld16<bf16x8>(q + off + 16 * c) : z;
            df[qb][c] = p < N ? ld16<bf16x8>(dout + off + 16 * c) : z;
        }
        l2q[qb] = p < N ? lse[((int64_t)b * Hq + head[qb]) * N + p] * kLog2e : 0.f;
        dlq[qb] = p < N ? delta[((int64_t)b * Hq + head[qb]) * N + p] : 0.f;
    }
    f32x16 acc[2][NDB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db) zero(acc[qb][db]);

    const int64_t row_len = (int64_t)T * KT;
    const __bf16* ktb = ktr + ((int64_t)b * Hkv + g) * D * row_len;
    bf16x8 rk[KCH], rv[KCH], rt[TCH];
    int rse = -1;
    auto load_tile = [&](int t) {
        const int j0 = t * KT;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int e = tid + 256 * u;
            const int row = e / (D / 8), c = e % (D / 8), j = j0 + row;
            const int64_t off = (((int64_t)b * N + j) * Hkv + g) * D + c * 8;
            bf16x8 z = {};
            rk[u] = j < N ? ld16<bf16x8>(k + off) : z;
            rv[u] = j < N ? ld16<bf16x8>(v + off) : z;
        }
#pragma unroll
        for (int u = 0; u < TCH; ++u) {
            const int e = tid + 256 * u;
            const int d = e / (KT / 8), c = e % (KT / 8);
            rt[u] = ld16<bf16x8>(ktb + (int64_t)d * row_len + j0 + c * 8);
        }
        if (tid < KT) rse = (j0 + tid < N) ? seb[j0 + tid] : -1;
    };
    auto store_tile = [&](int buf) {
        char* kb = smem + buf * BUF;
        char* vb = kb + KBYTES;
        char* tb = vb + KBYTES;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int e = tid + 256 * u;
            const int o = (e / (D / 8)) * KSTR + (e % (D / 8)) * 16;
            *reinterpret_cast<bf16x8*>(kb + o) = rk[u];
            *reinterpret_cast<bf16x8*>(vb + o) = rv[u];
        }
#pragma unroll
        for (int u = 0; u < TCH; ++u) {
            const int e = tid + 256 * u;
            *reinterpret_cast<bf16x8*>(tb + (e / (KT / 8)) * TSTR + (e % (KT / 8)) * 16) = rt[u];
        }
        if (tid < KT) se_s[buf][tid] = rse;
    };

    int t = next_visible(tmaxb, 0, t_last, i0);
    int cur = 0;
    if (t >= 0) {
        load_tile(t);
        store_tile(0);
    }
    __syncthreads();
    while (t >= 0) {
        const int tn = next_visible(tmaxb, t + 1, t_last, i0);
        if (tn >= 0) load_tile(tn);
        const int j0 = t * KT;
        const bool full = (j0 + KT - 1 <= i0) && (tminb[t] >= i_last);
        const char* kb = smem + cur * BUF;
        const char* vb = kb + KBYTES;
        const char* tb = vb + KBYTES;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            f32x16 st[2], dpt[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                zero(st[qb]);
                zero(dpt[qb]);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const int o = (x * 32 + l32) * KSTR + (hi * 8 + 16 * c) * 2;
                const bf16x8 ak = ld16<bf16x8>(kb + o), av = ld16<bf16x8>(vb + o);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    st[qb] = mfma32(ak, qf[qb][c], st[qb]);
                    dpt[qb] = mfma32(av, df[qb][c], dpt[qb]);
                }
            }
            bf16x8 dsf[2][2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int ip = posb[qb] + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jj = x * 32 + acc_row(r, hi);
                    float p = __builtin_amdgcn_exp2f(fmaf(st[qb][r], scale_log2, -l2q[qb]));
                    if (!full && !(j0 + jj <= ip && ip <= se_s[cur][jj])) p = 0.f;
                    dsf[qb][r >> 3][r & 7] = (__bf16)(p * (dpt[qb][r] - dlq[qb]));
                }
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const bf16x8 a = ld16<bf16x8>(tb + (db * 32 + l32) * TSTR + (x * 32 + c2 * 16 + hi * 8) * 2);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) acc[qb][db] = mfma32(a, dsf[qb][c2], acc[qb][db]);
                }
        }
        if (tn >= 0) store_tile(cur ^ 1);
        __syncthreads();
        cur ^= 1;
        t = tn;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int p = posb[qb] + l32;
        if (p < N) {
            __bf16* o = dq + (((int64_t)b * N + p) * Hq + head[qb]) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    bf16x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[qb][db][grp * 4 + e] * scale);
                    *reinterpret_cast<bf16x4*>(o + db * 32 + grp * 8 + hi * 4) = v4;
                }
        }
    }
}

template <int D, int HB>
hipError_t launch_dq(const AttnArgs& a, const BwdWorkspace& w, int T, hipStream_t st) {
    constexpr int BM = 256 / HB;
    const int G = a.Hq / a.Hkv;
    const int n_chunks = G / HB;
    const int n_qtiles = (a.N + BM - 1) / BM;
    const int64_t blocks = (int64_t)n_qtiles * a.B * a.Hkv * n_chunks;
    hipLaunchKernelGGL((bwd_dq<D, HB>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse, w.delta,
                       (const __bf16*)w.kt, a.se, w.tile_min, w.tile_max, a.B, a.N, a.Hq, a.Hkv, T, n_qtiles,
                       n_chunks, a.scale * kLog2e, a.scale, (__bf16*)a.dq);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd(const AttnArgs& a, const BwdWorkspace& w, hipStream_t st) {
    const int T = (a.N + KT - 1) / KT;
    hipLaunchKernelGGL((bwd_prep<D>), dim3(T, a.Hq, a.B), dim3(256), 0, st, (const __bf16*)a.q, (const __bf16*)a.k,
                       (const __bf16*)a.out, (const __bf16*)a.dout, a.se, a.N, a.Hq, a.Hkv, T, w.delta,
                       (__bf16*)w.qt, (__bf16*)w.dot, (__bf16*)w.kt, w.tile_min, w.tile_max);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_ktiles = (a.N + 127) / 128;
    hipLaunchKernelGGL((bwd_dkdv<D>), dim3((unsigned)((int64_t)n_ktiles * a.B * a.Hkv)), dim3(256), 0, st,
                       (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, a.lse,
                       w.delta, (const __bf16*)w.qt, (const __bf16*)w.dot, a.se, a.B, a.N, a.Hq, a.Hkv, T,
                       a.scale * kLog2e, a.scale, (__bf16*)a.dk, (__bf16*)a.dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (heads_per_wg(a.Hq / a.Hkv)) {
        case 1: return launch_dq<D, 1>(a, w, T, st);
        case 2: return launch_dq<D, 2>(a, w, T, st);
        case 4: return launch_dq<D, 4>(a, w, T, st);
        default: return launch_dq<D, 8>(a, w, T, st);
    }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t mfma_bwd_ws_bytes(int B, int N, int Hq, int Hkv, int D) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    const size_t Np = T * KT;
    return align256((size_t)B * Hq * N * sizeof(float)) + 2 * align256((size_t)B * Hq * D * Np * 2) +
           align256((size_t)B * Hkv * D * Np * 2) + 2 * align256((size_t)B * T * sizeof(int32_t));
}

BwdWorkspace carve_bwd_ws(void* ws, int B, int N, int Hq, int Hkv, int D) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    const size_t Np = T * KT;
    char* p = static_cast<char*>(ws);
    BwdWorkspace w;
    w.delta = reinterpret_cast<float*>(p);
    p += align256((size_t)B * Hq * N * sizeof(float));
    w.qt = reinterpret_cast<uint16_t*>(p);
    p += align256((size_t)B * Hq * D * Np * 2);
    w.dot = reinterpret_cast<uint16_t*>(p);
    p += align256((size_t)B * Hq * D * Np * 2);
    w.kt = reinterpret_cast<uint16_t*>(p);
    p += align256((size_t)B * Hkv * D * Np * 2);
    w.tile_min = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_max = reinterpret_cast<int32_t*>(p);
    return w;
}

hipError_t mfma_attn_bwd(const AttnArgs& a, const BwdWorkspace& w, hipStream_t st) {
    return a.D == 64 ? launch_bwd<64>(a, w, st) : launch_bwd<128>(a, w, st);
}

}  // namespace treeattn
