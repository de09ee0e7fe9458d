// bf16 attention backward over a packed tree on CDNA4 matrix cores.
//
// The pages give no backward pass; this is the exact gradient of the forward
// (same interval mask j <= i <= subtree_end[j], same tile classes).  With
// P = exp(scale * q.k - lse) and delta_i = dout_i . out_i:
//   dV = P^T dout,   dP = dout V^T,   dS = P * (dP - delta),
//   dK = scale dS^T Q,   dQ = scale dS K.
// Kernels, in launch order, no atomics on results (bitwise reproducible):
//   tile ranges  min / max subtree_end per 64-key tile and which tiles hold
//                isolated slots only (shared with the forward);
//   bwd_dq       query-stationary and persistent, shaped like the forward:
//                S^T = K Q^T and dP^T = V dout^T with Q, dout in registers,
//                then dQ^T += K^T dS^T with dS^T taken from the accumulator;
//                it also writes delta and lse * log2(e) for the next kernel,
//                and one of its workgroups first writes the dK/dV work plan
//                (split long KV tiles, per-XCD queues);
//   bwd_dkdv     KV-stationary and persistent: a workgroup owns 256 keys of
//                one KV head (32 per wave) and walks the query blocks its
//                keys can see, for every query head of the group:
//                  S = Q K^T, dP = dout V^T     (A = Q, dout rows from LDS)
//                  dV^T += dout^T P, dK^T += Q^T dS   (A by transposed LDS
//                  loads, B = P, dS straight from the S / dP accumulators)
//   bwd_reduce   sums the partials of split tiles in chunk order.
// Tiles whose slots are all isolated (they see and are seen only by
// themselves) get the one-key gradients from isolated-slot units, one of
// which a dQ workgroup takes after each item of matrix work: dq = dk = 0 and
// dv = the group's dout rows summed.
// dK/dV and dQ recompute S and dP separately (7 products instead of 5) so
// that no partial dQ has to be summed across workgroups.
#include <algorithm>
#include <climits>
#include <type_traits>
#include <vector>

#include "attn_mfma.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ T ld16(const void* p) {
    return *reinterpret_cast<const T*>(p);
}


// ---------------------------------------------------------------------------
// dK/dV work plan (one workgroup of the dQ kernel).  A KV tile of kKvTile keys visits every
// (32-position block, query head) pair from its first key's block to the
// block of the largest subtree_end among its keys.  Keys of a long shared
// prefix visit almost the whole row while keys near the leaves visit a few
// blocks, so a tile whose range exceeds C blocks is cut at multiples of C
// (absolute block positions, C = budget / G; the budget grows by a quarter
// until the chunks fit the partial-sum slots the workspace holds, so it stays
// within 25% of the smallest that fits; with no slots no tile is split).  Each KV head has its own queue (g mod
// NQ, so one XCD keeps one head's data), ordered longest unit first so that
// the CUs of an XCD run out of work together.  The order of units of equal
// length is arbitrary; every unit's result is the same whatever the order.
// ctrl: [0..7] queue counters, [8..15] lengths, [16..23] starts, [24] split tiles.
// tile_plan[u]: {first block, last block, chunks, first slot or -1}.
// ---------------------------------------------------------------------------
constexpr int kPlanBuckets = 4096;

// Exclusive prefix sum over the NT threads of the workgroup: inside each wave
// by shuffles, then over the NT / 64 wave totals (s_scan holds at least that
// many ints).
template <int NT>
__device__ int block_exclusive_scan(int v, int* s_scan) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) s_scan[wave] = x;
    __syncthreads();
    if (wave == 0) {
        int t = lane < NW ? s_scan[lane] : 0;
#pragma unroll
        for (int off = 1; off < NW; off <<= 1) {
            const int y = __shfl_up(t, off, 64);
            if (lane >= off) t += y;
        }
        if (lane < NW) s_scan[lane] = t;  // inclusive totals of waves 0..lane
    }
    __syncthreads();
    const int r = x - v + (wave > 0 ? s_scan[wave - 1] : 0);
    __syncthreads();
    return r;
}

// The plan, computed by the NT threads of one workgroup.  lds: at least
// kPlanLds ints of shared memory the workgroup does not otherwise use meanwhile.
constexpr int kPlanLds = 64 + kPlanBuckets;

template <int NT>
__device__ void make_plan(const int32_t* __restrict__ tmax, const int32_t* __restrict__ tiso, int B, int N, int T,
                          int G, int Hkv, int slot_cap, int* __restrict__ ctrl, int4* __restrict__ tile_plan,
                          int4* __restrict__ units, int4* __restrict__ split_tiles, int* lds) {
    static_assert(kPlanBuckets % NT == 0 && NT % 64 == 0 && NT / 64 <= 48, "bucket scan layout");
    int& s_sum = lds[0];
    int& s_budget = lds[1];
    int* s_scan = lds + 16;
    int* s_cnt = lds + 64;
    const int tid = threadIdx.x;
    const int TT = (N + kKvTile - 1) / kKvTile;  // KV tiles per row
    const int BT = B * TT;
    constexpr int SUB = kKvTile / KT, BPT = kKvTile / 32;  // 64-key tiles, 32-key blocks per KV tile
    const int NQ = Hkv < 8 ? Hkv : 8;
    // a tile of isolated keys gets no units (bwd_dq writes their gradients)
    for (int u = tid; u < BT; u += NT) {
        const int b = u / TT, t = u % TT;
        int qmax = -1, iso = 1;
        for (int x = SUB * t; x < min(SUB * t + SUB, T); ++x) {
            qmax = max(qmax, tmax[(int64_t)b * T + x]);
            iso &= tiso[(int64_t)b * T + x];
        }
        tile_plan[u] = iso ? make_int4(BPT * t, BPT * t, 0, -1) : make_int4(BPT * t, max(qmax / 32, BPT * t), 1, -1);
    }
    if (tid == 0) s_budget = kVisitBudget;
    __syncthreads();
    int C;
    for (;;) {
        if (tid == 0) s_sum = 0;
        __syncthreads();
        C = max(1, s_budget / G);
        int part = 0;
        for (int u = tid; u < BT; u += NT) {
            const int4 e = tile_plan[u];
            if (e.y - e.x + 1 > C) part += e.y / C - e.x / C + 1;
        }
        if (part) atomicAdd(&s_sum, part);
        __syncthreads();
        const bool fits = (int64_t)s_sum * Hkv <= slot_cap;
        __syncthreads();
        if (fits) break;
        if (tid == 0) s_budget += max(1, s_budget / 4);
        __syncthreads();
    }
    // chunks per tile; slots and split-tile indices by an exclusive scan in tile order
    const int per = (BT + NT - 1) / NT;
    const int u0 = min(BT, tid * per), u1 = min(BT, u0 + per);
    int my_chunks = 0, my_split = 0, my_units = 0;
    for (int u = u0; u < u1; ++u) {
        const int4 e = tile_plan[u];
        const int nc = e.z == 0 ? 0 : e.y - e.x + 1 > C ? e.y / C - e.x / C + 1 : 1;
        if (nc > 1) {
            my_chunks += nc;
            my_split += 1;
        }
        my_units += nc;
    }
    // chunk and split counts are at most slot_cap <= kSplitSlots: pack both in one scan
    const int packed = block_exclusive_scan<NT>(my_chunks | (my_split << 16), s_scan);
    const int n_units = [&] {
        const int before = block_exclusive_scan<NT>(my_units, s_scan);
        if (tid == NT - 1) s_sum = before + my_units;
        __syncthreads();
        return s_sum;
    }();
    {
        int slot = packed & 0xFFFF, z = packed >> 16;
        for (int u = u0; u < u1; ++u) {
            int4 e = tile_plan[u];
            const int nc = e.z == 0 ? 0 : e.y - e.x + 1 > C ? e.y / C - e.x / C + 1 : 1;
            if (nc > 1) {
                e.z = nc;
                e.w = slot;
                split_tiles[z] = make_int4(u / TT, u % TT, slot, nc);
                slot += nc;
                ++z;
            }
            tile_plan[u] = e;
        }
        if (tid == NT - 1) {
            ctrl[24] = z;
            int start = 0;
            for (int x = 0; x < NQ; ++x) {
                const int hg = (Hkv - x + NQ - 1) / NQ;  // heads in queue x
                ctrl[x] = 0;
                ctrl[8 + x] = n_units * hg;
                ctrl[16 + x] = start;
                start += n_units * hg;
            }
        }
    }
    // queue order: longest units first (the units of a KV head's queue run on
    // one XCD; taking the long ones first keeps its CUs finishing together).
    // The bucket of a unit is C minus its number of query blocks.
    const int64_t NKEY = C + 1;
    auto ukey = [&](const int4& e, int kk) {
        int nb = e.y - e.x + 1;
        if (e.z > 1) {
            const int k = e.x / C + kk;
            nb = min(e.y, k * C + C - 1) - max(e.x, k * C) + 1;
        }
        return C - nb;
    };
    int shift = 0;
    while (((NKEY - 1) >> shift) >= kPlanBuckets) ++shift;
    for (int x = tid; x < kPlanBuckets; x += NT) s_cnt[x] = 0;
    __syncthreads();
    for (int u = u0; u < u1; ++u) {
        const int4 e = tile_plan[u];
        for (int kk = 0; kk < e.z; ++kk) atomicAdd(&s_cnt[ukey(e, kk) >> shift], 1);
    }
    __syncthreads();
    {  // exclusive scan of the bucket counts, PB per thread
        constexpr int PB = kPlanBuckets / NT;
        int cb[PB], s = 0;
#pragma unroll
        for (int i = 0; i < PB; ++i) {
            cb[i] = s_cnt[PB * tid + i];
            s += cb[i];
        }
        int off = block_exclusive_scan<NT>(s, s_scan);
#pragma unroll
        for (int i = 0; i < PB; ++i) {
            s_cnt[PB * tid + i] = off;
            off += cb[i];
        }
    }
    __syncthreads();
    for (int u = u0; u < u1; ++u) {
        const int4 e = tile_plan[u];
        const int b = u / TT, t = u % TT;
        for (int kk = 0; kk < e.z; ++kk) {
            const int pos = atomicAdd(&s_cnt[ukey(e, kk) >> shift], 1);
            int v0 = 0, v1 = (e.y - e.x + 1) * G, slot = -1;
            if (e.z > 1) {
                const int k = e.x / C + kk;
                v0 = (max(e.x, k * C) - e.x) * G;
                v1 = (min(e.y, k * C + C - 1) - e.x + 1) * G;
                slot = e.w + kk;
            }
            for (int g = 0; g < Hkv; ++g) {
                const int x = g % NQ, r = g / NQ, hg = (Hkv - x + NQ - 1) / NQ;
                const int idx = ctrl[16 + x] + pos * hg + r;
                units[2 * idx] = make_int4(b * Hkv + g, t, v0, v1);
                units[2 * idx + 1] = make_int4(slot >= 0 ? slot * Hkv + g : -1, 0, 0, 0);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Sum the chunk partials of split tiles in chunk order and write bf16 dK, dV.
// The work is (split tile, KV head, group of kReduceKeys keys); the grid
// strides over it (the number of split tiles is known only on the device).  A
// thread owns a few float4 positions of its group and walks the chunks with
// their loads in flight together.
constexpr int kReduceKeys = 16;

template <int D>
__global__ __launch_bounds__(256) void bwd_reduce(const int* __restrict__ ctrl,
                                                 const int4* __restrict__ split_tiles,
                                                 const float* __restrict__ partial, int N, int Hkv,
                                                 __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
    constexpr int ROW4 = D / 4;                          // float4 per key row
    constexpr int PER = 2 * kReduceKeys * ROW4 / 256;   // float4 positions per thread (dK and dV)
    constexpr int SLOT = 2 * kKvTile * D;               // floats per slot
    const int n_split = ctrl[24];
    constexpr int KG = kKvTile / kReduceKeys;  // key groups per tile
    for (int wk = blockIdx.x; wk < n_split * Hkv * KG; wk += gridDim.x) {
    const int w = wk / KG;
    const int4 st = split_tiles[w / Hkv];
    const int g = w % Hkv;
    const int b = st.x, j0 = st.y * kKvTile;
    const int k0 = (wk % KG) * kReduceKeys;
    int off[PER];
    float4 acc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int which = e / (kReduceKeys * ROW4);     // 0: dK, 1: dV
        const int rem = e % (kReduceKeys * ROW4);
        off[i] = which * kKvTile * D + (k0 + rem / ROW4) * D + (rem % ROW4) * 4;
        acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const float* base = partial + (int64_t)(st.z * Hkv + g) * SLOT;
#pragma unroll 4
    for (int kk = 0; kk < st.w; ++kk) {
        const float* src = base + (int64_t)kk * Hkv * SLOT;
        float4 v[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) v[i] = *reinterpret_cast<const float4*>(src + off[i]);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            acc[i].x += v[i].x;
            acc[i].y += v[i].y;
            acc[i].z += v[i].z;
            acc[i].w += v[i].w;
        }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = threadIdx.x + 256 * i;
        const int which = e / (kReduceKeys * ROW4);
        const int rem = e % (kReduceKeys * ROW4);
        const int j = j0 + k0 + rem / ROW4;
        if (j >= N) continue;
        bf16x4 o;
        o[0] = (__bf16)acc[i].x;
        o[1] = (__bf16)acc[i].y;
        o[2] = (__bf16)acc[i].z;
        o[3] = (__bf16)acc[i].w;
        __bf16* dst = (which ? dv : dk) + (((int64_t)b * N + j) * Hkv + g) * D + (rem % ROW4) * 4;
        *reinterpret_cast<bf16x4*>(dst) = o;
    }
    }
}

// ---------------------------------------------------------------------------
// dK, dV: persistent, one 512-thread workgroup per CU (8 waves x 32 keys);
// work units come from the plan's queues.  A visit is 32 positions of one
// query head: its stage holds those Q and dout rows as they are in memory
// (16-byte chunks swizzled), lse * log2(e) and delta.  S = Q K^T and
// dP = dout V^T read Q and dout rows as the A operand; dV^T += dout^T P and
// dK^T += Q^T dS read the same rows through transposed LDS loads.  K sits in
// registers, V in this wave's own LDS rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dkdv(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                   const __bf16* __restrict__ v, const __bf16* __restrict__ dout,
                                                   const float* __restrict__ lse2, const float* __restrict__ delta,
                                                   const int32_t* __restrict__ se, int N, int Hq, int Hkv,
                                                   float scale_log2, float scale, int* __restrict__ ctrl,
                                                   const int4* __restrict__ units, float* __restrict__ partial,
                                                   __bf16* __restrict__ dk, __bf16* __restrict__ dv) {
    constexpr int NC = D / 16, NDB = D / 32;
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int NROW = D * 2;            // bytes per row
    constexpr int NBYTES = 32 * NROW;      // 32 rows
    constexpr int STAGE = 2 * NBYTES + 256;
    constexpr int NSTAGE = 4;
    // 16-byte chunks each wave loads per array and visit; below 64 a single
    // load with only the first lanes active (head dim 64)
    constexpr int NCH = NBYTES / 16 / 8;
    constexpr int NDMA = NCH >= 64 ? NCH / 64 : 1;
    constexpr int NLANES = NCH >= 64 ? 64 : NCH;
    constexpr int PER_VISIT = 2 * NDMA + 1;
    constexpr int VDMA = NBYTES / 1024;    // this wave's 32 V rows
    static_assert(NSTAGE == 4 && 2 * PER_VISIT < 16, "wait counts below assume four stages");
    __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * STAGE];
    __shared__ __attribute__((aligned(1024))) char vrows[8 * NBYTES];
    __shared__ int4 unit_s[2];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: bases stay scalar
    const int l32 = lane & 31, hi = lane >> 5;
    const int G = Hq / Hkv;
    const int NQ = Hkv < 8 ? Hkv : 8;
    const int qx = blockIdx.x % NQ;
    char* const vw = vrows + wave * NBYTES;
    // operand loads: row l32, chunk 2c + hi = 2c ^ hi, stored at 2c ^ (hi ^ swizzle)
    const int nat = l32 * NROW;
    const int nat_x = (hi ^ row_swizzle<D>(l32)) * 16;
    // transposed loads: this lane supplies row 4 (lane / 32) + (lane / 4) % 4 (+ 8 for
    // slots 4-7, + 16 per 16-row chunk) and column 32 db + 16 ((lane / 16) % 2) + 4 (lane % 4)
    int tr_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 4 * (lane >> 5) + ((lane >> 2) & 3) + 8 * half;
            const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            tr_off[db][half] = row * NROW + ((chunk ^ row_swizzle<D>(row)) * 16) + 8 * (lane & 1);
        }

    for (;;) {
    if (tid == 0) {
        const int idx = atomicAdd(&ctrl[qx], 1);
        if (idx < ctrl[8 + qx]) {
            unit_s[0] = units[2 * (ctrl[16 + qx] + idx)];
            unit_s[1] = units[2 * (ctrl[16 + qx] + idx) + 1];
        } else {
            unit_s[0] = make_int4(-1, 0, 0, 0);
        }
    }
    __syncthreads();
    // unit fields are wave-uniform: keep them (and all address bases) in SGPRs
    const int ux = __builtin_amdgcn_readfirstlane(unit_s[0].x);
    const int slot = __builtin_amdgcn_readfirstlane(unit_s[1].x);
    if (ux < 0) break;
    const int g = ux % Hkv, b = ux / Hkv;
    static_assert(kKvTile == 256, "eight waves of 32 keys");
    const int j0 = __builtin_amdgcn_readfirstlane(unit_s[0].y) * kKvTile;
    const int v_begin = __builtin_amdgcn_readfirstlane(unit_s[0].z);
    const int v_end = __builtin_amdgcn_readfirstlane(unit_s[0].w);
    const int j0w = j0 + 32 * wave;
    const int jk = j0w + l32;
    const bool kvalid = jk < N;
    const int32_t* seb = se + (int64_t)b * N;
    const int sek = kvalid ? seb[jk] : -1;
    const int wmax = wave_max_i32(sek);
    const int wmin = wave_min_i32(kvalid ? sek : INT_MAX);

    // this wave's V rows into LDS (swizzled like the stage rows)
    {
        const int r0 = min(j0w, N - 1);  // a wave past the end still loads rows in bounds
        const __bf16* vb = v + (((int64_t)b * N + r0) * Hkv + g) * D;
        const int lim = N - 1 - r0;
#pragma unroll
        for (int u = 0; u < VDMA; ++u) {
            const int e = u * 64 + lane;
            const int row = e / CPR;
            const int gch = (e % CPR) ^ row_swizzle<D>(row);
            dma16s(vb, (uint32_t)(min(row, lim) * Hkv * D + gch * 8) * 2u, vw + u * 1024);
        }
    }
    bf16x8 kf[NC];
    {
        const int64_t off = (((int64_t)b * N + min(jk, N - 1)) * Hkv + g) * D + hi * 8;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 z = {};
            kf[c] = kvalid ? ld16<bf16x8>(k + off + 16 * c) : z;
        }
    }
    // K (and the V rows) complete before any prefetch is issued: the
    // compiler's own wait for K then sits here, not inside the visit loop
    // where it would drain every prefetch
    wait_vmcnt<0>();
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        zero(dkt[db]);
        zero(dvt[db]);
    }
    const int pb0 = j0 / 32;
    const int nvis = v_end - v_begin;  // this unit's visits [v_begin, v_end) of the tile
    // per-lane part of the stage loads: row and swizzled chunk of each 16-byte piece
    int drow[NDMA], dcol[NDMA];
#pragma unroll
    for (int u = 0; u < NDMA; ++u) {
        const int e = wave * NCH + u * 64 + lane;
        drow[u] = e / CPR;
        dcol[u] = ((e % CPR) ^ row_swizzle<D>(e / CPR)) * 16;
    }
    const float* rowvec = wave < 4 ? lse2 : delta;

    // all of this wave's loads for one visit (32 positions x one query head)
    // Visit v of the unit covers positions (pb0 + (v_begin + v) / G) * 32 on
    // query head g * G + (v_begin + v) % G.  The loads and the products step
    // through the visits with a cursor each (block, head in the group, and
    // the element offsets of the rows): no division per visit.
    struct Cursor {
        int blk, hh;
        int64_t qoff, roff;  // Q / dout rows, lse2 / delta rows
    };
    auto cursor_at = [&](int vl) {
        const int vi = v_begin + vl;
        Cursor c;
        c.blk = pb0 + vi / G;
        c.hh = vi % G;
        c.qoff = (((int64_t)b * N + c.blk * 32) * Hq + g * G + c.hh) * D;
        c.roff = ((int64_t)b * Hq + g * G + c.hh) * N + c.blk * 32;
        return c;
    };
    auto advance = [&](Cursor& c) {
        if (++c.hh == G) {
            c.hh = 0;
            ++c.blk;
            c.qoff += (int64_t)(32 * Hq - (G - 1)) * D;
            c.roff += 32 - (int64_t)(G - 1) * N;
        } else {
            c.qoff += D;
            c.roff += N;
        }
    };
    auto issue = [&](const Cursor& c, int stage) {
        char* dst = smem + stage * STAGE;
        const int i0 = c.blk * 32;
        const int lim = N - 1 - i0;  // rows past the end repeat the last one
        const __bf16* qb = q + c.qoff;
        const __bf16* db = dout + c.qoff;
#pragma unroll
        for (int u = 0; u < NDMA; ++u) {
            const int e0 = wave * NCH + u * 64;  // first chunk of this load
            const uint32_t off = (uint32_t)(min(drow[u], lim) * (Hq * D * 2) + dcol[u]);
            if (lane < NLANES) {
                dma16s(qb, off, dst + e0 * 16);
                dma16s(db, off, dst + NBYTES + e0 * 16);
            }
        }
        const int ln = lane_id_here();
        if (ln < 8) {
            const float* rb = rowvec + c.roff;
            dma4s(rb, (uint32_t)min((wave & 3) * 8 + ln, lim) * 4u, dst + 2 * NBYTES + wave * 32);
        }
    };

    // one visit; FULL: every (query, key) pair of the block is visible
    auto visit = [&](auto full_tag, const char* st, int i_lo) {
        constexpr bool FULL = decltype(full_tag)::value;
        const float* l2s = reinterpret_cast<const float*>(st + 2 * NBYTES);
        const float* dls = l2s + 32;
        // S = Q K^T, dP = dout V^T: 32 queries x this wave's 32 keys
        f32x16 s, dp;
        zero(s);
        zero(dp);
        // operand loads run one chunk ahead of the products; the scheduling
        // fences stop the compiler from hoisting every load of the phase
        // (which runs out of registers)
        bf16x8 qa = ld16<bf16x8>(st + nat + nat_x), da = ld16<bf16x8>(st + NBYTES + nat + nat_x),
               va = ld16<bf16x8>(vw + nat + nat_x);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            bf16x8 qn = qa, dn = da, vn = va;
            if (c + 1 < NC) {
                const int o = nat + ((32 * (c + 1)) ^ nat_x);
                qn = ld16<bf16x8>(st + o);
                dn = ld16<bf16x8>(st + NBYTES + o);
                vn = ld16<bf16x8>(vw + o);
            }
            s = mfma32(qa, kf[c], s);
            dp = mfma32(da, va, dp);
            qa = qn;
            da = dn;
            va = vn;
            __builtin_amdgcn_sched_barrier(0);
        }
        bf16x8 pbf[2], dsf[2];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            const int m0 = 8 * gq + 4 * hi;
            const float4 l4 = *reinterpret_cast<const float4*>(l2s + m0);
            const float4 d4 = *reinterpret_cast<const float4*>(dls + m0);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dl[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = gq * 4 + e;
                float p = __builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, -lv[e]));
                if constexpr (!FULL) {
                    const int i = i_lo + m0 + e;
                    if (!(jk <= i && i <= sek)) p = 0.f;
                }
                pbf[r >> 3][r & 7] = (__bf16)p;
                dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dl[e]));
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // dV^T += dout^T P, dK^T += Q^T dS (A operands by transposed loads,
        // one (db, c2) step ahead of the products)
        auto tr_pair = [&](int step, bf16x8& a_dv, bf16x8& a_dk) {
            const int db = step >> 1, c2 = step & 1;
            const char* r0 = st + c2 * 16 * NROW;
            a_dv = ld_tr(r0 + NBYTES + tr_off[db][0], r0 + NBYTES + tr_off[db][1]);
            a_dk = ld_tr(r0 + tr_off[db][0], r0 + tr_off[db][1]);
        };
        bf16x8 tv, tk;
        tr_pair(0, tv, tk);
#pragma unroll
        for (int step = 0; step < 2 * NDB; ++step) {
            bf16x8 nv = tv, nk = tk;
            if (step + 1 < 2 * NDB) tr_pair(step + 1, nv, nk);
            const int db = step >> 1, c2 = step & 1;
            dvt[db] = mfma32(tv, pbf[c2], dvt[db]);
            dkt[db] = mfma32(tk, dsf[c2], dkt[db]);
            tv = nv;
            tk = nk;
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    Cursor ic = cursor_at(0);  // next visit to load
#pragma unroll
    for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
        if (s0 < nvis) {
            issue(ic, s0);
            advance(ic);
        }
    Cursor cc = cursor_at(0);  // visit of the products
    for (int vi = 0; vi < nvis; ++vi) {
        // visits issued after this one and possibly still in flight
        const int ahead = min(nvis - 1 - vi, NSTAGE - 2);
        if (ahead >= 2) wait_vmcnt<2 * PER_VISIT>();
        else if (ahead == 1) wait_vmcnt<PER_VISIT>();
        else wait_vmcnt<0>();
        barrier();
        if (vi + NSTAGE - 1 < nvis) {
            issue(ic, (vi + NSTAGE - 1) % NSTAGE);
            advance(ic);
        }
        const int i_lo = cc.blk * 32;
        advance(cc);
        const bool skip = (j0w > i_lo + 31) || (wmax < i_lo);
        if (skip) continue;
        const bool full = (j0w + 31 <= i_lo) && (wmin >= i_lo + 31);
        const char* st = smem + (vi % NSTAGE) * STAGE;
        if (full) visit(std::true_type{}, st, i_lo);
        else visit(std::false_type{}, st, i_lo);
    }
    if (kvalid && slot < 0) {
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
    } else if (slot >= 0) {  // a chunk of a split tile: fp32 partials, summed by bwd_reduce
        float* pk = partial + (int64_t)slot * 2 * kKvTile * D + (32 * wave + l32) * D;
        float* pv = pk + kKvTile * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d = db * 32 + grp * 8 + hi * 4;
                *reinterpret_cast<float4*>(pk + d) =
                    make_float4(dkt[db][grp * 4] * scale, dkt[db][grp * 4 + 1] * scale,
                                dkt[db][grp * 4 + 2] * scale, dkt[db][grp * 4 + 3] * scale);
                *reinterpret_cast<float4*>(pv + d) =
                    make_float4(dvt[db][grp * 4], dvt[db][grp * 4 + 1], dvt[db][grp * 4 + 2], dvt[db][grp * 4 + 3]);
            }
    }
    __syncthreads();  // unit_s is reused by the next unit
    }
}

// ---------------------------------------------------------------------------
// dQ: persistent 512-thread workgroups, one per CU, taking work items (BM
// positions x HB query heads of one KV head, 32 rows per wave) as the forward
// does: n_qblocks x B x Hkv x n_chunks items, deepest query block first.
// ---------------------------------------------------------------------------
// One work item of dQ: BM positions x HB query heads of one KV head.
template <int D, int HB>
__device__ __forceinline__ bool dq_item(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                        const __bf16* __restrict__ v, const __bf16* __restrict__ out,
                                        const __bf16* __restrict__ dout, const float* __restrict__ lse,
                                        float* __restrict__ delta, float* __restrict__ lse2,
                                        const int32_t* __restrict__ se, const int32_t* __restrict__ tmin,
                                        const int32_t* __restrict__ tmax, const int32_t* __restrict__ tiso, int B,
                                        int N, int Hq, int Hkv, int T, int n_qblocks, int n_chunks, float scale_log2,
                                        float scale, __bf16* __restrict__ dq, int item, char* smem, int* list,
                                        int* list_meta) {
    constexpr int BM = 256 / HB;
    constexpr int NC = D / 16, NDB = D / 32;
    constexpr int CPR = D / 8;
    constexpr int KROW = D * 2;            // K / V rows as in memory, chunks swizzled by row_swizzle
    constexpr int KBYTES = KT * KROW;
    constexpr int STAGE = 2 * KBYTES + KT * 4;
    constexpr int NSTAGE = 4;
    constexpr int KDMA = KBYTES / 1024 / 8;
    constexpr int PER_TILE = 2 * KDMA + 1;
    static_assert(2 * PER_TILE < 16, "wait counts");
    constexpr int LCAP = 1024;
    constexpr int FULL = 1 << 30;
    // LDS operand loads in flight ahead of the products that read them
    constexpr int PF_KV = 2, PF_TR = 3;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: load bases stay scalar
    const int l32 = lane & 31, hi = lane >> 5;
    const int GH = B * Hkv * n_chunks;
    const int gi = item % GH;
    const int qi = item / GH;
    const int qtile = n_qblocks - 1 - qi;
    const int chunk = gi % n_chunks;
    const int g = (gi / n_chunks) % Hkv;
    const int b = gi / (n_chunks * Hkv);
    const int G = Hq / Hkv;
    const int head = g * G + chunk * HB + wave % HB;
    const int i0 = qtile * BM;
    const int i_last = min(i0 + BM, N) - 1;
    const int t_last = i_last / KT;
    const int32_t* tmaxb = tmax + (int64_t)b * T;
    const int32_t* tminb = tmin + (int64_t)b * T;
    const int32_t* seb = se + (int64_t)b * N;
    const int ip = i0 + (wave / HB) * 32 + l32;

    // Q and dout of this lane's query in registers (lane halves hold the two
    // halves of each 16-wide chunk of the head dim); delta = dout . out of the
    // query is a dot over both halves, and it and lse * log2(e) are stored
    // for the dK/dV kernel, which runs after this one.  (The out rows are
    // read per lane: the stages hold the Q and dout rows of every wave only.)
    bf16x8 qf[NC], df[NC];
    float l2q, dlq;
    {
        // The wave's Q and dout rows arrive by DMA in whole rows (16 lanes per
        // 256-byte row, chunks swizzled as the stages' rows) into its part of
        // the idle stages; the fragments are then LDS reads.  Every wave is
        // past them at the tile-list barrier, before any tile overwrites them.
        constexpr int ROWB = D * 2, CH = D / 8, RPI = 64 / CH;
        const int p0 = i0 + (wave / HB) * 32;
        const int pr = min(p0, N - 1);   // base row in bounds; rows past the end repeat the last one
        const int lim = N - 1 - pr;
        char* sq = smem + wave * 2 * 32 * ROWB;
        const __bf16* qb = q + (((int64_t)b * N + pr) * Hq + head) * D;
        const __bf16* dob = dout + (((int64_t)b * N + pr) * Hq + head) * D;
#pragma unroll
        for (int u = 0; u < 32 * ROWB / 1024; ++u) {
            const int r = u * RPI + lane / CH;
            const uint32_t o = (uint32_t)(min(r, lim) * Hq * D * 2 + ((lane % CH) ^ row_swizzle<D>(r)) * 16);
            dma16s(qb, o, sq + u * 1024);
            dma16s(dob, o, sq + 32 * ROWB + u * 1024);
        }
        const int pc = min(ip, N - 1);
        const int64_t off = (((int64_t)b * N + pc) * Hq + head) * D + hi * 8;
        bf16x8 ofr[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) ofr[c] = ld16<bf16x8>(out + off + 16 * c);
        const int64_t ro = ((int64_t)b * Hq + head) * N + pc;
        const float lsev = lse[ro];
        // every load of the item's start lands at this one wait, so none is
        // left for the compiler to wait on inside the tile loop (where it
        // would drain the prefetches of later tiles)
        wait_vmcnt<0>();
        const uint32_t qa = lds_off(sq) + (uint32_t)(l32 * ROWB + ((hi ^ row_swizzle<D>(l32)) * 16));
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qf[c] = lds_ld16(qa ^ (32u * c));
            df[c] = lds_ld16((qa ^ (32u * c)) + 32 * ROWB);
        }
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const bf16x8 of = ofr[c];
            const bf16x8 d8 = df[c];
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 0, 1),
                                                  __builtin_shufflevector(d8, d8, 0, 1), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 2, 3),
                                                  __builtin_shufflevector(d8, d8, 2, 3), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 4, 5),
                                                  __builtin_shufflevector(d8, d8, 4, 5), dot, false);
            dot = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 6, 7),
                                                  __builtin_shufflevector(d8, d8, 6, 7), dot, false);
        }
        l2q = lsev * kLog2e;
        dlq = add_xor32(dot);
        if (ip < N && hi == 0) {
            delta[ro] = dlq;
            lse2[ro] = l2q;
        }
    }
    {
        // a block of isolated slots only: its gradients are written by the
        // isolated-slot units
        int iso = 1;
        for (int t = i0 / KT; t <= t_last; ++t) iso &= tiso[(int64_t)b * T + t];
        if (iso) return false;
    }
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) zero(acc[db]);

    const __bf16* kb_ = k + ((int64_t)b * N * Hkv + g) * D;
    const __bf16* vb_ = v + ((int64_t)b * N * Hkv + g) * D;
    int koff[KDMA], krow[KDMA];
#pragma unroll
    for (int u = 0; u < KDMA; ++u) {
        const int kk = wave * KDMA + u;
        krow[u] = kk * (64 / CPR) + lane / CPR;
        koff[u] = ((lane % CPR) ^ row_swizzle<D>(krow[u])) * 16;
    }
    const int kstride = Hkv * D * 2;  // bytes between consecutive keys
    auto issue = [&](int t, int stage) {
        char* dst = smem + stage * STAGE;
        const int j0 = t * KT;
        const int lim = N - 1 - j0;
        const __bf16* kt = kb_ + (int64_t)j0 * Hkv * D;
        const __bf16* vt = vb_ + (int64_t)j0 * Hkv * D;
#pragma unroll
        for (int u = 0; u < KDMA; ++u) {
            const uint32_t off = (uint32_t)(min(krow[u], lim) * kstride + koff[u]);
            dma16s(kt, off, dst + (wave * KDMA + u) * 1024);
            dma16s(vt, off, dst + KBYTES + (wave * KDMA + u) * 1024);
        }
        const int ln = lane_id_here();
        if (ln < 8) dma4s(seb + j0, (uint32_t)min(wave * 8 + ln, lim) * 4u, dst + 2 * KBYTES + wave * 32);
    };
    // operand loads of K / V rows: row x * 32 + l32, chunk 2c + hi (chunk 0's
    // offset here; chunk c is that XOR 32 c), and the transposed loads of K rows
    // for the K^T operand
    const uint32_t o_nat = (uint32_t)(l32 * KROW + ((hi ^ row_swizzle<D>(l32)) * 16));
    const uint32_t o_tr = tr_offset0<D>(lane);

    int resume = 0;
    while (resume >= 0) {
        if (wave == 0) {
            int cnt = 0, next = -1;
            for (int base = resume; base <= t_last; base += 64) {
                const int t = base + lane;
                const bool vis = t <= t_last && tmaxb[t] >= i0;
                const bool full = vis && (t * KT + KT - 1 <= i0) && tminb[t] >= i_last;
                const unsigned long long m = __ballot(vis);
                const int n_m = __popcll(m);
                if (cnt + n_m > LCAP) {
                    next = base;
                    break;
                }
                const int pos = cnt + __popcll(m & ((1ull << lane) - 1ull));
                if (vis) list[pos] = t | (full ? FULL : 0);
                cnt += n_m;
            }
            if (lane == 0) {
                list_meta[0] = cnt;
                list_meta[1] = next;
            }
        }
        __syncthreads();
        const int cnt = list_meta[0];
        resume = list_meta[1];

#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (s0 < cnt) issue(list[s0] & (FULL - 1), s0);
        for (int it = 0; it < cnt; ++it) {
            // tiles issued after this one and possibly still in flight
            const int ahead = min(cnt - 1 - it, NSTAGE - 2);
            if (ahead >= 2) wait_vmcnt<2 * PER_TILE>();
            else if (ahead == 1) wait_vmcnt<PER_TILE>();
            else wait_vmcnt<0>();
            barrier();
            if (it + NSTAGE - 1 < cnt) issue(list[it + NSTAGE - 1] & (FULL - 1), (it + NSTAGE - 1) % NSTAGE);
            const int e = list[it];
            const int t = e & (FULL - 1);
            const bool full = __builtin_amdgcn_readfirstlane(e & FULL) != 0;
            const int j0 = t * KT;
            const char* st = smem + (it % NSTAGE) * STAGE;
            const int* ses = reinterpret_cast<const int*>(st + 2 * KBYTES);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                f32x16 sacc, dpt;
                zero(sacc);
                zero(dpt);
                // K and V chunks of rows x * 32 + l32, PF_KV chunks ahead of the products
                const uint32_t kv = lds_off(st) + (uint32_t)(x * 32 * KROW) + o_nat;
                // the matrix-core phases run at raised wave priority: where both
                // waves of a SIMD can issue, the one feeding the matrix core goes
                // first and the other's vector work fills its gaps
                prio(1);
                bf16x8 kq[PF_KV], vq[PF_KV];
#pragma unroll
                for (int i = 0; i < PF_KV; ++i) {
                    kq[i] = lds_ld16(kv ^ (32u * i));
                    vq[i] = lds_ld16((kv ^ (32u * i)) + KBYTES);
                }
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    const bf16x8 ka = kq[c % PF_KV], va = vq[c % PF_KV];
                    if (c + PF_KV < NC) {
                        const uint32_t a = kv ^ (32u * (c + PF_KV));
                        kq[c % PF_KV] = lds_ld16(a);
                        vq[c % PF_KV] = lds_ld16(a + KBYTES);
                    }
                    sacc = mfma32(ka, qf[c], sacc);
                    dpt = mfma32(va, df[c], dpt);
                    __builtin_amdgcn_sched_barrier(0);
                }
                prio(0);
                float p[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, -l2q));
                if (!full) {  // the interval test, only on tiles that are not fully visible
                    asm volatile("");  // keep this a branch (not selects run on every tile)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int jj = x * 32 + 8 * gq + 4 * hi;
                        const int4 s4 = *reinterpret_cast<const int4*>(ses + jj);
                        const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4)
                            if (!(j0 + jj + e4 <= ip && ip <= sv[e4])) p[gq * 4 + e4] = 0.f;
                    }
                }
                bf16x8 dsf[2];
#pragma unroll
                for (int r = 0; r < 16; ++r) dsf[r >> 3][r & 7] = (__bf16)(p[r] * (dpt[r] - dlq));
                prio(1);
                // dQ^T += K^T dS^T (K^T by transposed loads of the K rows, PF_TR steps ahead)
                const uint32_t tk = lds_off(st) + (uint32_t)(x * 32 * KROW) + o_tr;
                bf16x8 tq[PF_TR];
#pragma unroll
                for (int i = 0; i < PF_TR; ++i) tq[i] = lds_tr_block<D>(tk, i >> 1, 16 * (i & 1));
#pragma unroll
                for (int step = 0; step < 2 * NDB; ++step) {
                    const int db = step >> 1, c2 = step & 1;
                    const bf16x8 ta = tq[step % PF_TR];
                    if (step + PF_TR < 2 * NDB)
                        tq[step % PF_TR] = lds_tr_block<D>(tk, (step + PF_TR) >> 1, 16 * ((step + PF_TR) & 1));
                    acc[db] = mfma32(ta, dsf[c2], acc[db]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                prio(0);
                // keep the two key halves apart: interleaving them needs more
                // registers than a wave has
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();
    }
    // The wave's 32 rows go out through its own LDS rows (idle now, chunks
    // swizzled as the stages' rows): each store then writes 16 contiguous
    // bytes and a row is 16 lanes of one store.  Rows of isolated tiles belong
    // to the isolated-slot units (the wave's rows lie in one 64-slot tile).
    {
        constexpr int ROWB = D * 2, CH = D / 8;
        char* stg = smem + wave * 32 * ROWB;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][grp * 4 + e] * scale);
                *reinterpret_cast<bf16x4*>(stg + l32 * ROWB + (((db * 4 + grp) ^ row_swizzle<D>(l32)) * 16) +
                                           hi * 8) = v4;
            }
        const int p0 = i0 + (wave / HB) * 32;
        if (p0 < N && !tiso[(int64_t)b * T + p0 / KT]) {
            __bf16* o = dq + (((int64_t)b * N + p0) * Hq + head) * D;
#pragma unroll
            for (int kk = 0; kk < 32 * CH / 64; ++kk) {
                const int e = kk * 64 + lane, r = e / CH, c = e % CH;
                const bf16x8 val = *reinterpret_cast<const bf16x8*>(stg + r * ROWB + ((c ^ row_swizzle<D>(r)) * 16));
                if (p0 + r < N) *reinterpret_cast<bf16x8*>(o + (int64_t)r * Hq * D + c * 8) = val;
            }
        }
    }
    return true;
}

// Persistent dQ: one 512-thread workgroup per CU takes work items from NQ
// queues, numbered and assigned as in the persistent forward.
// Arguments of the dK/dV plan, passed through the dQ kernel that computes it.
struct PlanArgs {
    const int32_t* tmax;
    const int32_t* tiso;
    int B, N, T, G, Hkv, slot_cap;
    int* ctrl;
    int4* tile_plan;
    int4* units;
    int4* split_tiles;
};

// The plan by one 512-thread workgroup of the dQ kernel; out of line, so the
// dQ items' registers are allocated without it.
__device__ __attribute__((noinline)) void plan_in_wg(const int32_t* tmax, const int32_t* tiso, int B, int N, int T,
                                                     int G, int Hkv, int slot_cap, int* ctrl, int4* tile_plan,
                                                     int4* units, int4* split_tiles, int* lds) {
    make_plan<512>(tmax, tiso, B, N, T, G, Hkv, slot_cap, ctrl, tile_plan, units, split_tiles, lds);
}

// One unit of isolated-slot work of the backward: part `unit % kIsoSplit` of
// listed tile `unit / kIsoSplit`.  P = 1 on the diagonal and nothing else, so
// dS = P (dP - delta) = dout.v - dout.out = 0: dq = dk = 0, and dv of a key is
// the sum of the dout rows of the query heads sharing its KV head.  The dK/dV
// kernel runs later and rewrites the keys of every 256-key tile it owns (the
// same values up to rounding), so a key of an isolated 64-key tile inside a
// mixed 256-key tile ends with its values.  Out of line, so that the main
// item's registers are allocated without it.
template <int D>
__device__ __attribute__((noinline)) void dq_iso_unit(const __bf16* __restrict__ dout,
                                                      const int32_t* __restrict__ iso_list, int N, int Hq, int Hkv,
                                                      int T, __bf16* __restrict__ dq, __bf16* __restrict__ dk,
                                                      __bf16* __restrict__ dv, int unit) {
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = Hq / Hkv;
    const int e = (lane % LPR) * 8;
    const bf16x8 z = {};
    const int bt = iso_list[unit / kIsoSplit];
    const int t = bt % T, b = bt / T;
    const int part = unit % kIsoSplit;
    const int qrows = KT * Hq / kIsoSplit, qbase = part * qrows;
#pragma unroll 4
    for (int r0 = qbase + wave * RPW; r0 < qbase + qrows; r0 += 8 * RPW) {  // dq rows
        const int r = r0 + lane / LPR;
        const int slot = t * KT + r / Hq;
        if (slot < N) *reinterpret_cast<bf16x8*>(dq + (((int64_t)b * N + slot) * Hq + r % Hq) * D + e) = z;
    }
    const int kvrows = KT * Hkv / kIsoSplit, kvbase = part * kvrows;
    for (int r0 = kvbase + wave * RPW; r0 < kvbase + kvrows; r0 += 8 * RPW) {  // dk, dv rows
        const int r = r0 + lane / LPR;
        const int slot = t * KT + r / Hkv, g = r % Hkv;
        if (slot >= N) continue;
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        const __bf16* src = dout + (((int64_t)b * N + slot) * Hq + (int64_t)g * G) * D + e;
        for (int h = 0; h < G; ++h) {
            const bf16x8 d8 = *reinterpret_cast<const bf16x8*>(src + (int64_t)h * D);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] += (float)d8[i];
        }
        bf16x8 o;
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (__bf16)acc[i];
        const int64_t kv = (((int64_t)b * N + slot) * Hkv + g) * D + e;
        *reinterpret_cast<bf16x8*>(dk + kv) = z;
        *reinterpret_cast<bf16x8*>(dv + kv) = o;
    }
}

template <int D, int HB>
__global__ __launch_bounds__(512, 1) void bwd_dq(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                 const __bf16* __restrict__ v, const __bf16* __restrict__ out,
                                                 const __bf16* __restrict__ dout, const float* __restrict__ lse,
                                                 float* __restrict__ delta, float* __restrict__ lse2,
                                                 const int32_t* __restrict__ se,
                                                 const int32_t* __restrict__ tmin, const int32_t* __restrict__ tmax,
                                                 const int32_t* __restrict__ tiso,
                                                 int B, int N, int Hq, int Hkv, int T, int n_qtiles, int n_chunks,
                                                 float scale_log2, float scale, __bf16* __restrict__ dq,
                                                 __bf16* __restrict__ dk, __bf16* __restrict__ dv,
                                                 const int32_t* __restrict__ iso_list, int* __restrict__ qctr,
                                                 int NQ, int n_items, PlanArgs plan) {
    constexpr int STAGE = 2 * KT * D * 2 + KT * 4;
    __shared__ __attribute__((aligned(1024))) char smem[4 * STAGE];
    __shared__ int list[1024];
    __shared__ int list_meta[2];
    __shared__ int s_item;
    const int qx = blockIdx.x % NQ;
    // the last workgroup first writes the dK/dV plan (read only by the next
    // kernel); the others meanwhile take its share of the items
    if (blockIdx.x == gridDim.x - 1) {
        static_assert(kPlanLds * 4 <= 4 * STAGE, "plan scratch fits the stages");
        plan_in_wg(plan.tmax, plan.tiso, plan.B, plan.N, plan.T, plan.G, plan.Hkv, plan.slot_cap, plan.ctrl,
                   plan.tile_plan, plan.units, plan.split_tiles, reinterpret_cast<int*>(smem));
        __syncthreads();
    }
    const int n_units = qctr[kIsoCount] * kIsoSplit;  // isolated-slot units
    bool iso_left = n_units > 0;
    auto claim = [&](int* ctr) {
        if (threadIdx.x == 0) s_item = atomicAdd(ctr, 1);
        __syncthreads();
        const int x = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        return x;
    };
    // Items cover the query blocks up to the end of the last 256-key tile with
    // a slot that is not isolated (in any row): the dK/dV kernel reads delta
    // and lse of every row such a tile reaches, padding rows after its real
    // keys included.  The blocks after it are left to the isolated-slot units.
    constexpr int BM = 256 / HB;
    constexpr int TPK = kKvTile / KT;
    const int real_keys = (qctr[kRealTiles] + TPK - 1) / TPK * kKvTile;
    const int n_qblocks = min(n_qtiles, (real_keys + BM - 1) / BM);
    const int n_work = n_qblocks * (n_items / n_qtiles);
    for (;;) {
        const int item = qx + NQ * claim(&qctr[qx]);
        if (item >= n_work) break;
        const bool worked = dq_item<D, HB>(q, k, v, out, dout, lse, delta, lse2, se, tmin, tmax, tiso, B, N, Hq,
                                           Hkv, T, n_qblocks, n_chunks, scale_log2, scale, dq, item, smem, list,
                                           list_meta);
        __syncthreads();  // the stages and the list are reused by the next item
        // one unit of the (HBM-bound) isolated-slot work after each item of
        // matrix work, spread over the kernel as in the forward
        if (worked && iso_left) {
            const int u = claim(&qctr[kIsoQueue]);
            if (u < n_units) dq_iso_unit<D>(dout, iso_list, N, Hq, Hkv, T, dq, dk, dv, u);
            else iso_left = false;  // the queue is empty: no more claims
        }
    }
    while (iso_left) {  // what is left of it
        const int u = claim(&qctr[kIsoQueue]);
        if (u >= n_units) break;
        dq_iso_unit<D>(dout, iso_list, N, Hq, Hkv, T, dq, dk, dv, u);
    }
}

template <int D, int HB>
hipError_t launch_dq(const AttnArgs& a, const BwdWorkspace& w, int T, hipStream_t st) {
    constexpr int BM = 256 / HB;
    const int G = a.Hq / a.Hkv;
    const int n_chunks = G / HB;
    const int n_qtiles = (a.N + BM - 1) / BM;
    const int64_t items = (int64_t)n_qtiles * a.B * a.Hkv * n_chunks;
    const int grid = (int)std::min<int64_t>(items, mfma_num_cus());
    const int NQ = std::min(kItemQueues, grid);
    hipLaunchKernelGGL((bwd_dq<D, HB>), dim3((unsigned)grid), dim3(512), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.out, (const __bf16*)a.dout, a.lse,
                       w.delta, w.lse2, a.se, w.tile_min, w.tile_max, w.tile_iso, a.B, a.N, a.Hq, a.Hkv, T,
                       n_qtiles, n_chunks, a.scale * kLog2e, a.scale, (__bf16*)a.dq, (__bf16*)a.dk, (__bf16*)a.dv,
                       w.iso_list, w.qctr, NQ, (int)items,
                       PlanArgs{w.tile_max, w.tile_iso, a.B, a.N, T, a.Hq / a.Hkv, a.Hkv, w.slot_cap, w.ctrl,
                                w.tile_plan, w.units, w.split_tiles});
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd(const AttnArgs& a, const BwdWorkspace& w, hipStream_t st) {
    const int T = (a.N + KT - 1) / KT;
    hipError_t e = launch_tile_ranges(a.se, a.B, a.N, w.tile_min, w.tile_max, w.tile_iso, w.iso_list, w.qctr, st);
    if (e != hipSuccess) return e;
    // dQ first: it also writes delta and lse * log2(e), which dK/dV reads
    switch (heads_per_wg(a.Hq / a.Hkv)) {
        case 1: e = launch_dq<D, 1>(a, w, T, st); break;
        case 2: e = launch_dq<D, 2>(a, w, T, st); break;
        case 4: e = launch_dq<D, 4>(a, w, T, st); break;
        default: e = launch_dq<D, 8>(a, w, T, st); break;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkdv<D>), dim3((unsigned)mfma_num_cus()), dim3(512), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.dout, w.lse2, w.delta, a.se, a.N,
                       a.Hq, a.Hkv, a.scale * kLog2e, a.scale, w.ctrl, w.units, w.partial, (__bf16*)a.dk,
                       (__bf16*)a.dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_reduce<D>), dim3(4 * mfma_num_cus()), dim3(256), 0, st, w.ctrl,
                       w.split_tiles, w.partial, a.N, a.Hkv, (__bf16*)a.dk, (__bf16*)a.dv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Plan tables (queue control, per-tile plan, unit queues, split-tile table)
// sized for the largest partial-sum capacity, and the bytes of one slot.
size_t plan_table_bytes(int B, int N, int Hkv) {
    const size_t TT = (size_t)(N + kKvTile - 1) / kKvTile;
    const size_t ucap = (size_t)kSplitSlots + (size_t)B * TT * Hkv;
    return align256(32 * sizeof(int)) + align256((size_t)B * TT * sizeof(int4)) +
           align256(ucap * 2 * sizeof(int4)) + align256((size_t)(kSplitSlots / 2) * sizeof(int4));
}
size_t slot_bytes(int D) { return (size_t)2 * kKvTile * D * sizeof(float); }

}  // namespace

size_t mfma_bwd_ws_bytes(int B, int N, int Hq, int Hkv, int D, int slots) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    return 2 * align256((size_t)B * Hq * N * sizeof(float)) + 4 * align256((size_t)B * T * sizeof(int32_t)) +
           align256(kQueueCounters * sizeof(int32_t)) + plan_table_bytes(B, N, Hkv) +
           (size_t)std::min(std::max(slots, 0), kSplitSlots) * slot_bytes(D);
}

int mfma_bwd_plan_slots(const int32_t* se, int B, int N, int Hq, int Hkv) {
    // the device plan's first budget on the device's tile ranges: the tile
    // ranges kernels (smallest / largest subtree_end per 64-key tile, isolated
    // tiles) and make_plan's chunk count, recomputed here from the host row
    const int T = (N + KT - 1) / KT, TT = (N + kKvTile - 1) / kKvTile;
    const int G = Hq / Hkv, C = std::max(1, kVisitBudget / G);
    constexpr int SUB = kKvTile / KT, BPT = kKvTile / 32;
    std::vector<int> tmax(T), tiso(T);
    int64_t chunks = 0;
    for (int b = 0; b < B; ++b) {
        const int32_t* row = se + (int64_t)b * N;
        int before = -1;  // largest subtree_end of the keys before tile t
        for (int t = 0; t < T; ++t) {
            int mx = -1;
            bool self_only = true;
            for (int j = t * KT; j < std::min(N, t * KT + KT); ++j) {
                mx = std::max(mx, row[j]);
                self_only = self_only && row[j] == j;
            }
            tmax[t] = mx;
            tiso[t] = self_only && before < t * KT;
            before = std::max(before, mx);
        }
        for (int tt = 0; tt < TT; ++tt) {
            int qmax = -1;
            bool iso = true;
            for (int x = SUB * tt; x < std::min(SUB * tt + SUB, T); ++x) {
                qmax = std::max(qmax, tmax[x]);
                iso = iso && tiso[x];
            }
            if (iso) continue;
            const int first = BPT * tt, last = std::max(qmax / 32, BPT * tt);
            if (last - first + 1 > C) chunks += last / C - first / C + 1;
        }
    }
    return (int)std::min<int64_t>(kSplitSlots, chunks * Hkv);
}

BwdWorkspace carve_bwd_ws(void* ws, size_t ws_bytes, int B, int N, int Hq, int Hkv, int D) {
    const size_t T = (size_t)(N + KT - 1) / KT;
    char* p = static_cast<char*>(ws);
    BwdWorkspace w;
    w.delta = reinterpret_cast<float*>(p);
    p += align256((size_t)B * Hq * N * sizeof(float));
    w.lse2 = reinterpret_cast<float*>(p);
    p += align256((size_t)B * Hq * N * sizeof(float));
    w.tile_min = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_max = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_iso = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.iso_list = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.qctr = reinterpret_cast<int32_t*>(p);
    p += align256(kQueueCounters * sizeof(int32_t));
    const size_t TT = (size_t)(N + kKvTile - 1) / kKvTile;
    const size_t ucap = (size_t)kSplitSlots + (size_t)B * TT * Hkv;
    w.ctrl = reinterpret_cast<int32_t*>(p);
    p += align256(32 * sizeof(int));
    w.tile_plan = reinterpret_cast<int4*>(p);
    p += align256((size_t)B * TT * sizeof(int4));
    w.units = reinterpret_cast<int4*>(p);
    p += align256(ucap * 2 * sizeof(int4));
    w.split_tiles = reinterpret_cast<int4*>(p);
    p += align256((size_t)(kSplitSlots / 2) * sizeof(int4));
    w.partial = reinterpret_cast<float*>(p);
    // the partial-sum slots are what the workspace holds beyond the fixed part
    const size_t fixed = mfma_bwd_ws_bytes(B, N, Hq, Hkv, D, 0);
    w.slot_cap = ws_bytes > fixed ? (int)std::min<size_t>(kSplitSlots, (ws_bytes - fixed) / slot_bytes(D)) : 0;
    return w;
}

hipError_t mfma_attn_bwd(const AttnArgs& a, const BwdWorkspace& w, hipStream_t st) {
    return a.D == 64 ? launch_bwd<64>(a, w, st) : launch_bwd<128>(a, w, st);
}

}  // namespace treeattn
