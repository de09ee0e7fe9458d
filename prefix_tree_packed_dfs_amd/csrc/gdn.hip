// Gated-delta-rule token mixing over a packed tree on CDNA4 (bf16 matrix cores, fp32 state).
//
// The layer (Gated DeltaNet, Yang, Kautz and Hatamizadeh 2024): a short
// depthwise causal convolution and SiLU on the q | k | v channels, q and k
// L2-normalised per head (q scaled by dk^-1/2), then per value head the state
// recurrence
//     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t.
// Over a packed tree the state runs along root-to-leaf paths, forks at branch
// points and starts from zero at roots [ART "Token-mixing layers"].
//
// Kernels of one call:
//   gdn_conv    32 slots x 2048 channels per workgroup: the convolution reads
//               each slot and its W-1 nearest ancestors through the parent
//               array (a fork's children all read the parent's inputs; roots
//               see zeros), then SiLU and the per-head normalisation; bf16 out.
//   gdn_chunk   one wave per (chunk, value head), every chunk of the row at
//               once: the chunk-local part of the chunked form (below) as
//               operand fragments for the state pass.
//   gdn_state   one launch per chain depth, one workgroup per (chain, value
//               head), one wave per 32 value columns: runs the chain's chunks
//               in order from its parent chain's final state (zero at a root),
//               writes the outputs and, for a chain with children, its final
//               state.
//
// Chunked form (H = S^T, dk x dv; a chunk of L <= 64 tokens from state H0;
// G_i = g_1 + ... + g_i inside the chunk):
//   A_ij = beta_i (k_i . k_j) e^{G_i - G_j} (j < i),  T = (I + A)^-1,
//   W = T diag(beta e^G) K,  U = T diag(beta) V,  D = U - W H0,
//   o_i = e^{G_i} q_i^T H0 + sum_{j <= i} e^{G_i - G_j} (q_i . k_j) D_j,
//   H_end = e^{G_L} H0 + sum_j e^{G_L - G_j} k_j D_j^T.
// A chunk shorter than 64 is padded with g = beta = 0 and zero q, k, v, which
// leaves the state and the outputs unchanged, so a chain's final state is
// exact at any length and children start from it directly.
#include <hip/hip_runtime.h>

#include "gdn.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float exp_f(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// ---------------------------------------------------------------------------
// gdn_conv: grid (ceil(n / kConvTokens), C / 2048), 256 threads.  A thread owns 8
// consecutive channels of a 2048-channel slab, keeps their taps in registers and
// runs over kConvTokens consecutive slots.  The channel count is a multiple of 128
// (whole heads), so a slab may end part-way: threads past C idle.
// ---------------------------------------------------------------------------
constexpr int kConvTokens = 32;

template <int W>
__global__ __launch_bounds__(256) void gdn_conv(const __bf16* __restrict__ x, const float* __restrict__ conv_w,
                                                const int32_t* __restrict__ parent, int n, int C, int qk_channels,
                                                float q_scale, __bf16* __restrict__ mixed) {
    __shared__ int s_anc[kConvTokens][4];
    const int ch = (blockIdx.y * 256 + (int)threadIdx.x) * 8;
    const bool act = ch < C;
    const int t0 = blockIdx.x * kConvTokens, cnt = min(n - t0, kConvTokens);
    // ancestors of the block's slots, one thread per slot
    if ((int)threadIdx.x < cnt) {
        int a = t0 + (int)threadIdx.x;
        s_anc[threadIdx.x][0] = a;
#pragma unroll
        for (int j = 1; j < W; ++j) {
            a = a >= 0 ? parent[a] : -1;
            s_anc[threadIdx.x][j] = a;
        }
    }
    float w[8][W];
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
        for (int j = 0; j < W; ++j) w[e][j] = act ? conv_w[(int64_t)(ch + e) * W + j] : 0.f;
    const bool qk = act && ch < 2 * qk_channels;
    const float post = ch < qk_channels ? q_scale : 1.f;
    __syncthreads();
    // Slots run in order; along a chain a slot's ancestors are the slots just
    // before it, whose inputs are still in registers (win[j-1] = slot t - j), so
    // a chain slot loads only its own row.  Other ancestors are loaded directly.
    constexpr int U = 4;  // slots whose own rows are loaded together, one batch ahead
    const bf16x8 z = {};
    bf16x8 cur[U], nxt[U], win[3] = {z, z, z};
#pragma unroll
    for (int u = 0; u < U; ++u)
        cur[u] = (act && u < cnt) ? *reinterpret_cast<const bf16x8*>(x + (int64_t)(t0 + u) * C + ch) : z;
    for (int tb = 0; tb < cnt; tb += U) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int tn = tb + U + u;
            nxt[u] = (act && tn < cnt) ? *reinterpret_cast<const bf16x8*>(x + (int64_t)(t0 + tn) * C + ch) : z;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (tb + u >= cnt) break;
            const int t = t0 + tb + u;
            bf16x8 xs[W];
            xs[0] = cur[u];
#pragma unroll
            for (int j = 1; j < W; ++j) {
                const int a = s_anc[tb + u][j];
                if (a == t - j && t - j >= t0) xs[j] = win[j - 1];
                else xs[j] = (act && a >= 0) ? *reinterpret_cast<const bf16x8*>(x + (int64_t)a * C + ch) : z;
            }
            win[2] = win[1];
            win[1] = win[0];
            win[0] = cur[u];
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < W; ++j) acc = fmaf(w[e][W - 1 - j], (float)xs[j][e], acc);
                // SiLU with the hardware exp2 and reciprocal (about 1 ulp of fp32; the result is stored as bf16)
                y[e] = acc * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-acc * kLog2e));
            }
            // q and k: L2 norm over the head's 128 channels = 16 consecutive lanes
            float ss = 0.f;
            if (qk) {
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) ss += __shfl_xor(ss, o, 64);
            if (act) {
                const float f = qk ? (ss > 0.f ? __builtin_amdgcn_rsqf(ss) : 0.f) * post : 1.f;
                bf16x8 r;
#pragma unroll
                for (int e = 0; e < 8; ++e) r[e] = (__bf16)(y[e] * f);
                *reinterpret_cast<bf16x8*>(mixed + (int64_t)t * C + ch) = r;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) cur[u] = nxt[u];
    }
}

// Two 8-byte loads give the A operand of a row-major bf16 matrix for one
// 16-wide K step in the permuted order: slots 0-3 = columns 4h + 0..3,
// slots 4-7 = columns 8 + 4h + 0..3 of the step (h = lane / 32).
__device__ __forceinline__ bf16x8 ld_perm(const __bf16* row_step, int hf) {
    const bf16x4 a = *reinterpret_cast<const bf16x4*>(row_step + 4 * hf);
    const bf16x4 b = *reinterpret_cast<const bf16x4*>(row_step + 8 + 4 * hf);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int half) {
    bf16x8 r;
#pragma unroll
    for (int t = 0; t < 8; ++t) r[t] = (__bf16)c[8 * half + t];
    return r;
}

// ---------------------------------------------------------------------------
// gdn_chunk: grid n_chunks * Hv, one wave.
// ---------------------------------------------------------------------------
constexpr int kTRow = 72;  // bf16 per LDS row of T (64 + 8 padding)
constexpr int kARow = 72;  // fp32 per LDS row of A^T

// Copy the 64 rows (256 bytes each) of one head of a chunk into LDS, 16-byte
// pieces swizzled per row, and zero the rows past the chunk's end.  Lane i of
// copy k fills row 4k + i / 16, LDS piece i % 16, which holds data piece
// (i % 16) ^ row_swizzle(row).
__device__ __forceinline__ void stage_rows(const __bf16* rows0, int C, int len, char* lds) {
    const int ln = lane_id_here();
    const uint32_t rstride = (uint32_t)C * 2u;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int r = 4 * k + (ln >> 4);
        const int piece = (ln & 15) ^ row_swizzle<128>(r);
        const uint32_t off = (uint32_t)min(r, len - 1) * rstride + (uint32_t)piece * 16u;
        dma16s(rows0, off, lds + k * 1024);
    }
}
__device__ __forceinline__ void zero_rows(int len, char* lds) {
    const int lane = threadIdx.x & 63;
    for (int r = len + (lane >> 4); r < 64; r += 4)
        *reinterpret_cast<uint4*>(lds + r * 256 + (lane & 15) * 16) = make_uint4(0, 0, 0, 0);
}
// A fragment of a staged row: row r, 16-byte data piece p
__device__ __forceinline__ bf16x8 lds_piece(const char* lds, int r, int p) {
    return *reinterpret_cast<const bf16x8*>(lds + r * 256 + ((p ^ row_swizzle<128>(r)) * 16));
}

__global__ __launch_bounds__(64) void gdn_chunk(const __bf16* __restrict__ mixed, const float* __restrict__ g,
                                               const float* __restrict__ beta, const int32_t* __restrict__ chunks,
                                               int C, int Hk, int Hv, char* __restrict__ blocks) {
    __shared__ __attribute__((aligned(1024))) float sAT[64 * kARow];  // Q rows, then A^T, then T rows
    __shared__ __attribute__((aligned(1024))) char sK[64 * 256];     // K rows, later V rows (swizzled)
    __shared__ __attribute__((aligned(16))) float sG[64], sB[64], sF[64];
    const int lane = threadIdx.x, l32 = lane & 31, hf = lane >> 5;
    const int ci = blockIdx.x / Hv, h = blockIdx.x % Hv, hk = h / (Hv / Hk);
    const int start = chunks[2 * ci], len = chunks[2 * ci + 1];
    char* blk = blocks + ((int64_t)ci * Hv + h) * kGdnBlock;
    const __bf16* qrow = mixed + (int64_t)start * C + (int64_t)hk * kGdnDim;
    const __bf16* krow = mixed + (int64_t)start * C + (int64_t)(Hk + hk) * kGdnDim;
    const __bf16* vrow = mixed + (int64_t)start * C + (int64_t)(2 * Hk + h) * kGdnDim;
    char* sQ = reinterpret_cast<char*>(sAT);

    stage_rows(krow, C, len, sK);
    stage_rows(qrow, C, len, sQ);
    // gates: inclusive scan of g over the chunk (lane = token); padding g = beta = 0
    const bool real = lane < len;
    const float gl = real ? g[(int64_t)(start + lane) * Hv + h] : 0.f;
    const float bl = real ? beta[(int64_t)(start + lane) * Hv + h] : 0.f;
    float G = gl;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const float up = __shfl_up(G, o, 64);
        if (lane >= o) G += up;
    }
    const float GL = __shfl(G, 63, 64);
    sG[lane] = G;
    sB[lane] = bl;
    sF[lane] = bl * exp_f(G);
    reinterpret_cast<float*>(blk + kGdnELG)[lane] = exp_f(GL - G);
    if (lane == 0) reinterpret_cast<float*>(blk + kGdnGL)[0] = exp_f(GL);
    wait_vmcnt<0>();
    zero_rows(len, sK);
    zero_rows(len, sQ);
    __syncthreads();

    // K and Q rows as operand fragments: row 32X + l32, columns 16s + 8hf .. +7
    bf16x8 kf[2][8], qf[2][8];
#pragma unroll
    for (int X = 0; X < 2; ++X)
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            kf[X][s] = lds_piece(sK, 32 * X + l32, 2 * s + hf);
            qf[X][s] = lds_piece(sQ, 32 * X + l32, 2 * s + hf);
        }
    // diag(e^G) Q as A fragments, K = head dim in the permuted order (columns 16s + 4hf + 0..3, 16s + 8 + 4hf + 0..3)
    {
        bf16x8* Qf = reinterpret_cast<bf16x8*>(blk + kGdnQ);
#pragma unroll
        for (int I = 0; I < 2; ++I) {
            const int r = 32 * I + l32;
            const float e = exp_f(sG[r]);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const bf16x4 a = *reinterpret_cast<const bf16x4*>(
                    sQ + r * 256 + (((2 * s) ^ row_swizzle<128>(r)) * 16) + 8 * hf);
                const bf16x4 c = *reinterpret_cast<const bf16x4*>(
                    sQ + r * 256 + (((2 * s + 1) ^ row_swizzle<128>(r)) * 16) + 8 * hf);
                bf16x8 f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    f[t] = (__bf16)((float)a[t] * e);
                    f[4 + t] = (__bf16)((float)c[t] * e);
                }
                Qf[(I * 8 + s) * 64 + lane] = f;
            }
        }
    }
    // KK = K K^T (lower tiles) and M^T = K Q^T (upper tiles), rows j = 32X + acc_row, columns 32Y + l32
    f32x16 kk00 = {}, kk10 = {}, kk11 = {}, m00 = {}, m01 = {}, m11 = {};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        kk00 = mfma32(kf[0][s], kf[0][s], kk00);
        kk10 = mfma32(kf[1][s], kf[0][s], kk10);
        kk11 = mfma32(kf[1][s], kf[1][s], kk11);
        m00 = mfma32(kf[0][s], qf[0][s], m00);
        m01 = mfma32(kf[0][s], qf[1][s], m01);
        m11 = mfma32(kf[1][s], qf[1][s], m11);
    }
    __syncthreads();  // every lane is done with the Q rows (A^T goes there next)
    // M fragments: (row tile I = Y, K step 2X + c) from the M^T tile (X, Y), masked j <= i, decayed
    {
        bf16x8* Mf = reinterpret_cast<bf16x8*>(blk + kGdnM);
        auto emit = [&](const f32x16& acc, int X, int Y) {
            const int i = 32 * Y + l32;
            const float Gi = sG[i];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                bf16x8 f;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const int r = 8 * c + t;
                    const int j = 32 * X + acc_row(r, hf);
                    f[t] = (__bf16)(j <= i ? acc[r] * exp_f(Gi - sG[j]) : 0.f);
                }
                Mf[(Y * 4 + 2 * X + c) * 64 + lane] = f;
            }
        };
        emit(m00, 0, 0);
        emit(m01, 0, 1);
        emit(m11, 1, 1);
        const bf16x8 z = {};
        Mf[(0 * 4 + 2) * 64 + lane] = z;
        Mf[(0 * 4 + 3) * 64 + lane] = z;
    }
    // A^T[c][j] = beta_j (k_j . k_c) e^{G_j - G_c} for j > c (only those entries are read)
    {
        auto put = [&](const f32x16& acc, int X, int Y) {
            const int c = 32 * Y + l32;
            const float Gc = sG[c];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const int j0 = 32 * X + 8 * q4 + 4 * hf;
                f32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + e;
                    v[e] = j > c ? sB[j] * acc[4 * q4 + e] * exp_f(sG[j] - Gc) : 0.f;
                }
                *reinterpret_cast<f32x4*>(&sAT[c * kARow + j0]) = v;
            }
        };
        put(kk00, 0, 0);
        put(kk10, 1, 0);
        put(kk11, 1, 1);
    }
    __syncthreads();

    // T = (I + A)^-1, lane i keeps row i: T[i][c] = [i == c] - sum_{j > c} A[j][c] T[i][j].
    // Column c of A is read (broadcast) while column c + 1 is being used.
    float T[64];
    f32x4 acol[2][16];
#pragma unroll
    for (int c = 63; c >= 0; --c) {
        if (c > 0) {
#pragma unroll
            for (int j4 = c / 4; j4 < 16; ++j4)
                acol[(c - 1) & 1][j4] = *reinterpret_cast<const f32x4*>(&sAT[(c - 1) * kARow + 4 * j4]);
        }
        __builtin_amdgcn_sched_barrier(0);
        float acc0 = lane == c ? 1.f : 0.f, acc1 = 0.f;
#pragma unroll
        for (int j4 = (c + 1) / 4; j4 < 16; ++j4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * j4 + e;
                if (j > c) {
                    if (e & 1) acc1 = fmaf(-acol[c & 1][j4][e], T[j], acc1);
                    else acc0 = fmaf(-acol[c & 1][j4][e], T[j], acc0);
                }
            }
        }
        T[c] = acc0 + acc1;
        __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();  // every lane is done reading A^T
    // rows of T diag(beta e^G) and T diag(beta) as bf16 (reusing the A^T space)
    __bf16* sT1 = reinterpret_cast<__bf16*>(sAT);
    __bf16* sT2 = sT1 + 64 * kTRow;
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
        bf16x8 a, b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = 8 * c8 + e;
            a[e] = (__bf16)(T[j] * sF[j]);
            b[e] = (__bf16)(T[j] * sB[j]);
        }
        *reinterpret_cast<bf16x8*>(sT1 + lane * kTRow + 8 * c8) = a;
        *reinterpret_cast<bf16x8*>(sT2 + lane * kTRow + 8 * c8) = b;
    }
    __syncthreads();

    // transposed reads of the staged rows: A operand of X^T (rows = head dim), K = rows of X
    int tr_off[4][2];
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 4 * (lane >> 5) + ((lane >> 2) & 3) + 8 * half;
            const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            tr_off[db][half] = row * 256 + ((chunk ^ row_swizzle<128>(row)) * 16) + 8 * (lane & 1);
        }
    // W^T = K^T (T diag(beta e^G))^T: accumulator tile (D', I) holds, per lane, the A fragments of W
    // for row i = 32I + l32 and K steps 2D', 2D' + 1; K^T fragments are kept for the state pass
    {
        bf16x8* Wn = reinterpret_cast<bf16x8*>(blk + kGdnWn);
        bf16x8* KT = reinterpret_cast<bf16x8*>(blk + kGdnKT);
        bf16x8 tb[2][4];
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int c = 0; c < 4; ++c) tb[I][c] = ld_perm(sT1 + (32 * I + l32) * kTRow + 16 * c, hf);
#pragma unroll
        for (int Dp = 0; Dp < 4; ++Dp) {
            f32x16 w0 = {}, w1 = {};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const char* r0 = sK + (16 * c) * 256;
                const bf16x8 kt = ld_tr(r0 + tr_off[Dp][0], r0 + tr_off[Dp][1]);
                KT[(Dp * 4 + c) * 64 + lane] = kt;
                w0 = mfma32(kt, tb[0][c], w0);
                w1 = mfma32(kt, tb[1][c], w1);
            }
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                bf16x8 f0, f1;
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    f0[t] = (__bf16)(-w0[8 * half + t]);
                    f1[t] = (__bf16)(-w1[8 * half + t]);
                }
                Wn[(0 * 8 + 2 * Dp + half) * 64 + lane] = f0;
                Wn[(1 * 8 + 2 * Dp + half) * 64 + lane] = f1;
            }
        }
    }
    __syncthreads();  // done with the K rows
    // V rows into LDS, then U = (T diag(beta)) V in accumulator layout
    stage_rows(vrow, C, len, sK);
    wait_vmcnt<0>();
    zero_rows(len, sK);
    __syncthreads();
    {
        bf16x8* Uo = reinterpret_cast<bf16x8*>(blk + kGdnU);
        bf16x8 ta[2][4];
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int c = 0; c < 4; ++c) ta[I][c] = ld_perm(sT2 + (32 * I + l32) * kTRow + 16 * c, hf);
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            f32x16 u0 = {}, u1 = {};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const char* r0 = sK + (16 * c) * 256;
                const bf16x8 vb = ld_tr(r0 + tr_off[J][0], r0 + tr_off[J][1]);
                u0 = mfma32(ta[0][c], vb, u0);
                u1 = mfma32(ta[1][c], vb, u1);
            }
            Uo[((J * 2 + 0) * 64 + lane) * 2 + 0] = pack8(u0, 0);
            Uo[((J * 2 + 0) * 64 + lane) * 2 + 1] = pack8(u0, 1);
            Uo[((J * 2 + 1) * 64 + lane) * 2 + 0] = pack8(u1, 0);
            Uo[((J * 2 + 1) * 64 + lane) * 2 + 1] = pack8(u1, 1);
        }
    }
}

// ---------------------------------------------------------------------------
// gdn_state: grid (chains of this depth) * Hv, 256 threads; wave b owns value
// columns 32b .. 32b + 31 of the state.  Each chunk's block is copied whole
// into LDS one chunk ahead (two stages); the state stays in registers.
// ---------------------------------------------------------------------------
constexpr int kStageDma = (int)((kGdnBlock + 1023) / 1024);  // 1 KB copies per stage

__global__ __launch_bounds__(256) void gdn_state(const char* __restrict__ blocks, const int32_t* __restrict__ segs,
                                                 const int32_t* __restrict__ chunks, int seg0, int Hv,
                                                 float* __restrict__ states, __bf16* __restrict__ out) {
    __shared__ __attribute__((aligned(1024))) char stage[2][kGdnBlock];
    const int lane = threadIdx.x & 63, l32 = lane & 31, hf = lane >> 5;
    const int b = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int si = seg0 + blockIdx.x / Hv, h = blockIdx.x % Hv;
    const int first = segs[4 * si], n_ch = segs[4 * si + 1], psi = segs[4 * si + 2], own = segs[4 * si + 3];

    // state tiles H[D'] (rows = key dims 32D' + acc_row, columns 32b + l32), fp32
    f32x16 H[4];
    if (psi >= 0) {
        const f32x4* src = reinterpret_cast<const f32x4*>(states) + ((((int64_t)psi * Hv + h) * 4 + b) * 4) * 64 * 4;
#pragma unroll
        for (int Dp = 0; Dp < 4; ++Dp)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 v = src[(Dp * 64 + lane) * 4 + q4];
#pragma unroll
                for (int e = 0; e < 4; ++e) H[Dp][4 * q4 + e] = v[e];
            }
    } else {
#pragma unroll
        for (int Dp = 0; Dp < 4; ++Dp) zero(H[Dp]);
    }
    wait_vmcnt<0>();  // the state is in registers before any copy is in flight

    // copy block ci into stage sidx: 1 KB per instruction, waves take every fourth KB
    auto issue = [&](int ci, int sidx) {
        const char* src = blocks + ((int64_t)ci * Hv + h) * kGdnBlock;
        const int ln = lane_id_here();
#pragma unroll
        for (int m = 0; m < (kStageDma + 3) / 4; ++m) {
            const int k = b + 4 * m;
            const uint32_t off = (uint32_t)(k * 1024 + ln * 16);
            if (k < kStageDma && off < kGdnBlock) dma16s(src, off, stage[sidx] + k * 1024);
        }
    };
    issue(first, 0);
    for (int c = 0; c < n_ch; ++c) {
        wait_vmcnt<0>();
        barrier();  // stage c % 2 is complete, and every wave is done with stage (c + 1) % 2
        if (c + 1 < n_ch) issue(first + c + 1, (c + 1) & 1);
        const int ci = first + c;
        const int start = chunks[2 * ci], len = chunks[2 * ci + 1];
        const char* st = stage[c & 1];
        const bf16x8* Wn = reinterpret_cast<const bf16x8*>(st + kGdnWn);
        const bf16x8* Mf = reinterpret_cast<const bf16x8*>(st + kGdnM);
        const bf16x8* KT = reinterpret_cast<const bf16x8*>(st + kGdnKT);
        const bf16x8* Qf = reinterpret_cast<const bf16x8*>(st + kGdnQ);
        const bf16x8* Uc = reinterpret_cast<const bf16x8*>(st + kGdnU);
        const float* eLG = reinterpret_cast<const float*>(st + kGdnELG);
        const float gL = *reinterpret_cast<const float*>(st + kGdnGL);

        // the operands of the first products from LDS first (the rest are read where used)
        bf16x8 wf[2][8], qf[2][8], uf[2][2];
#pragma unroll
        for (int I = 0; I < 2; ++I) {
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                wf[I][s] = Wn[(I * 8 + s) * 64 + lane];
                qf[I][s] = Qf[(I * 8 + s) * 64 + lane];
            }
            uf[I][0] = Uc[((b * 2 + I) * 64 + lane) * 2 + 0];
            uf[I][1] = Uc[((b * 2 + I) * 64 + lane) * 2 + 1];
        }
        __builtin_amdgcn_sched_barrier(0);

        bf16x8 Hb[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) Hb[s] = pack8(H[s >> 1], s & 1);
        // D = U - W H0 and X = diag(e^G) Q H0 (rows = tokens 32I + acc_row)
        f32x16 Dt[2], X[2];
#pragma unroll
        for (int I = 0; I < 2; ++I) {
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                Dt[I][t] = (float)uf[I][0][t];
                Dt[I][8 + t] = (float)uf[I][1][t];
            }
            zero(X[I]);
        }
#pragma unroll
        for (int s = 0; s < 8; ++s)
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                Dt[I] = mfma32(wf[I][s], Hb[s], Dt[I]);
                X[I] = mfma32(qf[I][s], Hb[s], X[I]);
            }
        // o = X + M D
        bf16x8 Db[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) Db[s] = pack8(Dt[s >> 1], s & 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int I = 0; I < 2; ++I) X[I] = mfma32(Mf[(I * 4 + s) * 64 + lane], Db[s], X[I]);
        // H_end = e^{G_L} H0 + K^T diag(e^{G_L - G}) D
#pragma unroll
        for (int I = 0; I < 2; ++I)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4 e = *reinterpret_cast<const f32x4*>(eLG + 32 * I + 8 * q4 + 4 * hf);
#pragma unroll
                for (int t = 0; t < 4; ++t) Dt[I][4 * q4 + t] *= e[t];
            }
#pragma unroll
        for (int s = 0; s < 4; ++s) Db[s] = pack8(Dt[s >> 1], s & 1);
#pragma unroll
        for (int Dp = 0; Dp < 4; ++Dp) {
#pragma unroll
            for (int r = 0; r < 16; ++r) H[Dp][r] *= gL;
#pragma unroll
            for (int s = 0; s < 4; ++s) H[Dp] = mfma32(KT[(Dp * 4 + s) * 64 + lane], Db[s], H[Dp]);
        }
        __bf16* orow = out + ((int64_t)start * Hv + h) * kGdnDim + 32 * b + l32;
        const int64_t rs = (int64_t)Hv * kGdnDim;
        if (len == 64) {
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int r = 0; r < 16; ++r) orow[(32 * I + acc_row(r, hf)) * rs] = (__bf16)X[I][r];
        } else {
#pragma unroll
            for (int I = 0; I < 2; ++I)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int i = 32 * I + acc_row(r, hf);
                    if (i < len) orow[i * rs] = (__bf16)X[I][r];
                }
        }
    }
    if (own < 0) return;  // no child reads this chain's final state
    f32x4* dst = reinterpret_cast<f32x4*>(states) + ((((int64_t)own * Hv + h) * 4 + b) * 4) * 64 * 4;
#pragma unroll
    for (int Dp = 0; Dp < 4; ++Dp)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = H[Dp][4 * q4 + e];
            dst[(Dp * 64 + lane) * 4 + q4] = v;
        }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t gdn_ws_bytes(int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv) {
    const int64_t C = (2 * Hk + Hv) * kGdnDim;
    return align256((size_t)n * C * 2) + align256((size_t)n_chunks * Hv * kGdnBlock) +
           align256((size_t)n_states * Hv * kGdnDim * kGdnDim * 4);
}

GdnWorkspace carve_gdn_ws(void* ws, int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv) {
    const int64_t C = (2 * Hk + Hv) * kGdnDim;
    char* p = static_cast<char*>(ws);
    GdnWorkspace w;
    w.mixed = p;
    p += align256((size_t)n * C * 2);
    w.blocks = p;
    p += align256((size_t)n_chunks * Hv * kGdnBlock);
    w.states = reinterpret_cast<float*>(p);
    (void)n_states;
    return w;
}

hipError_t gdn_forward(const GdnArgs& a, const GdnWorkspace& w, hipStream_t st) {
    const int C = (2 * a.Hk + a.Hv) * kGdnDim;
    const float q_scale = 1.f / sqrtf((float)kGdnDim);
    const dim3 cgrid((unsigned)((a.n + kConvTokens - 1) / kConvTokens), (unsigned)((C + 2047) / 2048));
    switch (a.W) {
        case 1: hipLaunchKernelGGL((gdn_conv<1>), cgrid, dim3(256), 0, st, (const __bf16*)a.x, a.conv_w, a.parent, a.n, C, a.Hk * kGdnDim, q_scale, (__bf16*)w.mixed); break;
        case 2: hipLaunchKernelGGL((gdn_conv<2>), cgrid, dim3(256), 0, st, (const __bf16*)a.x, a.conv_w, a.parent, a.n, C, a.Hk * kGdnDim, q_scale, (__bf16*)w.mixed); break;
        case 3: hipLaunchKernelGGL((gdn_conv<3>), cgrid, dim3(256), 0, st, (const __bf16*)a.x, a.conv_w, a.parent, a.n, C, a.Hk * kGdnDim, q_scale, (__bf16*)w.mixed); break;
        default: hipLaunchKernelGGL((gdn_conv<4>), cgrid, dim3(256), 0, st, (const __bf16*)a.x, a.conv_w, a.parent, a.n, C, a.Hk * kGdnDim, q_scale, (__bf16*)w.mixed); break;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gdn_chunk, dim3((unsigned)((int64_t)a.n_chunks * a.Hv)), dim3(64), 0, st, (const __bf16*)w.mixed, a.g,
                       a.beta, a.chunks, C, a.Hk, a.Hv, w.blocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int d = 0; d < a.n_depths; ++d) {
        const int s0 = a.depth_off[d], s1 = a.depth_off[d + 1];
        if (s1 <= s0) continue;
        hipLaunchKernelGGL(gdn_state, dim3((unsigned)((int64_t)(s1 - s0) * a.Hv)), dim3(256), 0, st, w.blocks,
                           a.segs, a.chunks, s0, a.Hv, w.states, (__bf16*)a.out);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace treeattn
