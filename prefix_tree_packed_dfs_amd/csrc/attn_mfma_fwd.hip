// bf16 attention forward over a packed tree on CDNA4 matrix cores.
//
// Mask [ART "Token-mixing layers"; DAG "The mask"]: query i sees key j iff
// j <= i <= subtree_end[j].  Per 64-key tile, the smallest and largest
// subtree_end decide the tile's class for a block of queries [i0, i1]:
//   skipped  max_se < i0                      (no key of the tile is an ancestor)
//   full     j1 <= i0 and min_se >= i1        (every key is an ancestor of every query)
//   partial  otherwise                        (the interval test runs per element)
// which is the pages' decomposition into fully visible ancestor blocks, a
// causal block on the query's own segment, and skipped blocks.
//
// Work decomposition (one workgroup = 4 waves = 256 query rows):
//   * the rows are BM positions x HB query heads that share one KV head
//     (BM * HB = 256), so a K/V tile staged once in LDS serves every head of
//     the GQA group;
//   * each wave owns two 32-row query blocks and keeps their Q fragments in
//     registers; every K or V fragment read from LDS feeds two MFMAs.
// Products are v_mfma_f32_32x32x16_bf16 in the transposed orientation:
//   S^T = K Q^T   (A = K from LDS, B = Q^T from registers)
//   O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T accumulator)
// In the 32x32 accumulator a lane holds one query (column) and 16 keys, so
// the softmax reductions stay inside the lane except one exchange with lane
// l^32, and the probabilities are already laid out as the B operand of the
// next product.  V^T comes from a prep kernel that also permutes keys inside
// each 16-key group to the order the accumulator holds them in, so each MFMA
// operand is one 16-byte LDS read.  Online softmax in fp32 with exp2 and a
// log2(e)-prescaled scale; P is rounded to bf16 for the PV product.
#include <climits>

#include "attn_mfma.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr float kLn2 = 0.69314718055994531f;

// V -> V^T (keys permuted inside 16-key groups, zero past N) and per-tile
// subtree_end range.  grid (T, Hkv, B), 256 threads.
template <int D>
__global__ __launch_bounds__(256) void fwd_prep(const __bf16* __restrict__ v, const int32_t* __restrict__ se,
                                                int N, int Hkv, int T, int32_t* __restrict__ tmin,
                                                int32_t* __restrict__ tmax, __bf16* __restrict__ vt) {
    constexpr int CPR = D / 8;  // 16-byte chunks per key row
    __shared__ __attribute__((aligned(16))) __bf16 tile[KT][D + 8];
    const int t = blockIdx.x, g = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int j0 = t * KT;
    for (int e = tid; e < KT * CPR; e += 256) {
        const int r = e / CPR, c = e % CPR, j = j0 + r;
        bf16x8 val = {};
        if (j < N) val = *reinterpret_cast<const bf16x8*>(v + (((int64_t)b * N + j) * Hkv + g) * D + c * 8);
        *reinterpret_cast<bf16x8*>(&tile[r][c * 8]) = val;
    }
    __syncthreads();
    const int64_t row_len = (int64_t)T * KT;
    __bf16* dst = vt + ((int64_t)b * Hkv + g) * D * row_len + j0;
    for (int e = tid; e < D * (KT / 8); e += 256) {
        const int d = e / (KT / 8), c = e % (KT / 8);
        bf16x8 o;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int p = c * 8 + u;
            o[u] = tile[(p >> 4) * 16 + inv_phys16(p & 15)][d];
        }
        *reinterpret_cast<bf16x8*>(dst + (int64_t)d * row_len + c * 8) = o;
    }
    if (g == 0 && tid < 64) {
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

template <int D, int HB>
__global__ __launch_bounds__(256, 1) void fwd_main(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                   const __bf16* __restrict__ vt, const int32_t* __restrict__ se,
                                                   const int32_t* __restrict__ tmin,
                                                   const int32_t* __restrict__ tmax, int B, int N, int Hq,
                                                   int Hkv, int T, int n_qtiles, int n_chunks, float scale_log2,
                                                   __bf16* __restrict__ out, float* __restrict__ lse) {
    constexpr int BM = 256 / HB;        // positions per workgroup
    constexpr int NC = D / 16;          // 16-wide chunks of the head dim
    constexpr int NDB = D / 32;         // 32-row blocks of the head dim
    constexpr int KSTR = D * 2 + 16;    // LDS bytes per K row (padded: conflict-free b128 reads)
    constexpr int VSTR = KT * 2 + 16;   // LDS bytes per V^T row
    constexpr int KBYTES = KT * KSTR;
    constexpr int VBYTES = D * VSTR;
    constexpr int KCH = KT * D / 8 / 256;  // 16-byte chunks per thread per K tile
    constexpr int VCH = D * KT / 8 / 256;  // ... per V^T tile
    __shared__ __attribute__((aligned(16))) char smem[2 * (KBYTES + VBYTES)];
    __shared__ int se_s[2][KT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // work item: consecutive blocks go to different XCDs; the head-group index
    // is the fast one so each XCD keeps to a fixed set of KV heads
    const int GH = B * Hkv * n_chunks;
    const int gi = blockIdx.x % GH;
    const int qi = blockIdx.x / GH;
    const int qt = n_qtiles - 1 - qi;  // deeper (later) query tiles first
    const int chunk = gi % n_chunks;
    const int g = (gi / n_chunks) % Hkv;
    const int b = gi / (n_chunks * Hkv);
    const int G = Hq / Hkv;
    const int head_base = g * G + chunk * HB;
    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, N) - 1;
    const int t_last = i_last / KT;
    const int32_t* tmaxb = tmax + (int64_t)b * T;
    const int32_t* tminb = tmin + (int64_t)b * T;
    const int32_t* seb = se + (int64_t)b * N;

    int posb[2], head[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int bi = 2 * wave + qb;
        head[qb] = head_base + bi % HB;
        posb[qb] = i0 + (bi / HB) * 32;
    }
    bf16x8 qf[2][NC];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int p = posb[qb] + l32;
        const __bf16* src = q + (((int64_t)b * N + p) * Hq + head[qb]) * D + hi * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 z = {};
            qf[qb][c] = p < N ? *reinterpret_cast<const bf16x8*>(src + 16 * c) : z;
        }
    }
    f32x16 acc[2][NDB];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    const int64_t vt_row = (int64_t)T * KT;
    const __bf16* vtb = vt + ((int64_t)b * Hkv + g) * D * vt_row;
    bf16x8 rk[KCH], rv[VCH];
    int rse = -1;

    auto load_tile = [&](int t) {
        const int j0 = t * KT;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int e = tid + 256 * u;
            const int row = e / (D / 8), c = e % (D / 8), j = j0 + row;
            bf16x8 z = {};
            rk[u] = j < N ? *reinterpret_cast<const bf16x8*>(k + (((int64_t)b * N + j) * Hkv + g) * D + c * 8) : z;
        }
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int e = tid + 256 * u;
            const int d = e / (KT / 8), c = e % (KT / 8);
            rv[u] = *reinterpret_cast<const bf16x8*>(vtb + (int64_t)d * vt_row + j0 + c * 8);
        }
        if (tid < KT) rse = (j0 + tid < N) ? seb[j0 + tid] : -1;
    };
    auto store_tile = [&](int buf) {
        char* kb = smem + buf * (KBYTES + VBYTES);
        char* vb = kb + KBYTES;
#pragma unroll
        for (int u = 0; u < KCH; ++u) {
            const int e = tid + 256 * u;
            *reinterpret_cast<bf16x8*>(kb + (e / (D / 8)) * KSTR + (e % (D / 8)) * 16) = rk[u];
        }
#pragma unroll
        for (int u = 0; u < VCH; ++u) {
            const int e = tid + 256 * u;
            *reinterpret_cast<bf16x8*>(vb + (e / (KT / 8)) * VSTR + (e % (KT / 8)) * 16) = rv[u];
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
        const char* kb = smem + cur * (KBYTES + VBYTES);
        const char* vb = kb + KBYTES;

        // S^T = K Q^T for 64 keys x 64 queries
        f32x16 s[2][2];
#pragma unroll
        for (int x = 0; x < 2; ++x)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[x][qb][r] = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb + (x * 32 + l32) * KSTR + (hi * 8 + 16 * c) * 2);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) s[x][qb] = mfma32(a, qf[qb][c], s[x][qb]);
            }
        }
        if (!full) {
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int jj = x * 32 + 8 * (r >> 2) + hi * 4 + (r & 3);
                    const int j = j0 + jj, sej = se_s[cur][jj];
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        const int ip = posb[qb] + l32;
                        if (!(j <= ip && ip <= sej)) s[x][qb][r] = -INFINITY;
                    }
                }
        }
        // online softmax per query (one query per lane per block)
        bf16x8 pf[2][2][2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[x][qb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[qb], mx * scale_log2);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float corr = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
            m_run[qb] = m_new;
            float rs = 0.f;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(s[x][qb][r], scale_log2, -m_use));
                    rs += p;
                    pf[qb][x][r >> 3][r & 7] = (__bf16)p;
                }
            l_run[qb] = l_run[qb] * corr + rs;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[qb][db][r] *= corr;
        }
        // O^T += V^T P^T
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(vb + (db * 32 + l32) * VSTR +
                                                                      (x * 32 + c2 * 16 + hi * 8) * 2);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) acc[qb][db] = mfma32(a, pf[qb][x][c2], acc[qb][db]);
                }
        if (tn >= 0) store_tile(cur ^ 1);
        __syncthreads();
        cur ^= 1;
        t = tn;
    }

    // epilogue: O = O^T / l, lse = (m + log2 l) ln 2
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const float lt = l_run[qb] + __shfl_xor(l_run[qb], 32, 64);
        const int p = posb[qb] + l32;
        if (p < N) {
            const float inv = 1.f / lt;
            __bf16* o = out + (((int64_t)b * N + p) * Hq + head[qb]) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int grp = 0; grp < 4; ++grp) {
                    bf16x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[qb][db][grp * 4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(o + db * 32 + grp * 8 + hi * 4) = v4;
                }
            if (hi == 0) lse[((int64_t)b * Hq + head[qb]) * N + p] = (m_run[qb] + __log2f(lt)) * kLn2;
        }
    }
}

template <int D, int HB>
hipError_t launch_main(const AttnArgs& a, const FwdWorkspace& w, int T, hipStream_t st) {
    constexpr int BM = 256 / HB;
    const int G = a.Hq / a.Hkv;
    const int n_chunks = G / HB;
    const int n_qtiles = (a.N + BM - 1) / BM;
    const int64_t blocks = (int64_t)n_qtiles * a.B * a.Hkv * n_chunks;
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((fwd_main<D, HB>), dim3((unsigned)blocks), dim3(256), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)w.vt, a.se, w.tile_min, w.tile_max, a.B, a.N, a.Hq,
                       a.Hkv, T, n_qtiles, n_chunks, scale_log2, (__bf16*)a.out, a.lse);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd(const AttnArgs& a, const FwdWorkspace& w, hipStream_t st) {
    const int T = (a.N + KT - 1) / KT;
    hipLaunchKernelGGL((fwd_prep<D>), dim3(T, a.Hkv, a.B), dim3(256), 0, st, (const __bf16*)a.v, a.se, a.N, a.Hkv,
                       T, w.tile_min, w.tile_max, (__bf16*)w.vt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (heads_per_wg(a.Hq / a.Hkv)) {
        case 1: return launch_main<D, 1>(a, w, T, st);
        case 2: return launch_main<D, 2>(a, w, T, st);
        case 4: return launch_main<D, 4>(a, w, T, st);
        default: return launch_main<D, 8>(a, w, T, st);
    }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t mfma_fwd_ws_bytes(int B, int N, int Hkv, int D) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    return 2 * align256((size_t)B * T * sizeof(int32_t)) + align256((size_t)B * Hkv * D * T * KT * 2);
}

FwdWorkspace carve_fwd_ws(void* ws, int B, int N, int Hkv, int D) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    char* p = static_cast<char*>(ws);
    FwdWorkspace w;
    w.tile_min = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_max = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.vt = reinterpret_cast<uint16_t*>(p);
    (void)Hkv;
    (void)D;
    return w;
}

hipError_t mfma_attn_fwd(const AttnArgs& a, const FwdWorkspace& w, hipStream_t st) {
    return a.D == 64 ? launch_fwd<64>(a, w, st) : launch_fwd<128>(a, w, st);
}

}  // namespace treeattn
