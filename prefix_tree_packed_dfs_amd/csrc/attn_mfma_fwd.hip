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
// Work decomposition (one work item = 8 waves = 256 query rows):
//   * the rows are BM positions x HB query heads that share one KV head
//     (BM * HB = 256), so a K/V tile staged once in LDS serves every head of
//     the GQA group;
//   * each wave owns one 32-row query block (32 positions of one head) and
//     keeps its Q fragments in registers;
//   * the kernel is persistent: one workgroup per CU takes items from
//     per-XCD queues, deepest query block first.
// Tiles whose slots all see and are seen only by themselves (padding,
// one-token sequences) get the one-key result from isolated-slot units, one
// of which a workgroup takes after each item of matrix work.
// Products are v_mfma_f32_32x32x16_bf16 in the transposed orientation:
//   S^T = K Q^T   (A = K from LDS, B = Q^T from registers)
//   O^T += V^T P^T (A = V^T from LDS, B = P^T straight from the S^T accumulator)
// In the 32x32 accumulator a lane holds one query (column) and 16 keys, so
// the softmax reductions stay inside the lane except one exchange with lane
// l^32, and the probabilities are already laid out as the B operand of the
// next product.  K and V tiles are staged in LDS as they are in memory
// (16-byte chunks swizzled); the V^T operand comes from transposed LDS loads
// (ds_read_b64_tr_b16) that also put the keys of each 16-key group in the
// order the accumulator holds them.  Online softmax in fp32 with exp2 and a
// log2(e)-prescaled scale; P is rounded to bf16 for the PV product.
#include <algorithm>
#include <atomic>
#include <climits>

#include "attn_mfma.h"
#include "mfma_common.h"

namespace treeattn {

namespace {

constexpr float kLn2 = 0.69314718055994531f;

// Smallest and largest subtree_end of every 64-key tile, and whether every key
// of the tile is seen by itself only (subtree_end[j] == j): grid (ceil(T / 4),
// B), 256 threads, one wave per tile.
__global__ __launch_bounds__(256) void fwd_prep(const int32_t* __restrict__ se, int N, int T,
                                                int32_t* __restrict__ tmin, int32_t* __restrict__ tmax,
                                                int32_t* __restrict__ tiso, int32_t* __restrict__ qctr) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6), b = blockIdx.y, lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x < kQueueCounters) qctr[threadIdx.x] = 0;  // work queues
    if (t >= T) return;
    const int j = t * KT + lane;
    const int s = j < N ? se[(int64_t)b * N + j] : -1;
    const int mn = wave_min_i32(j < N ? s : INT_MAX);
    const int mx = wave_max_i32(s);
    const bool self_only = __ballot(j < N && s != j) == 0;
    if (lane == 0) {
        tmin[(int64_t)b * T + t] = mn;
        tmax[(int64_t)b * T + t] = mx;
        tiso[(int64_t)b * T + t] = self_only ? 1 : 0;
    }
}

// A slot is isolated when it is a root without descendants: no interval
// [j, subtree_end[j]] other than its own contains it, so as a query it sees only
// itself and as a key it is seen only by itself (the padding after the packed
// tokens of a row, one-token sequences).  A tile of keys seen by themselves
// only is isolated when no key before the tile reaches into it, i.e. the
// largest subtree_end before the tile is below its first slot.  Grid (B), 1024
// threads; a running maximum over the tiles, 1024 per step.
// The isolated tiles are also listed (as b * T + t, in no particular order) in
// iso_list, their number in qctr[kIsoCount].
__global__ __launch_bounds__(1024) void iso_scan(const int32_t* __restrict__ tmax, int T,
                                                 int32_t* __restrict__ tiso, int32_t* __restrict__ iso_list,
                                                 int32_t* __restrict__ qctr) {
    __shared__ int s_wave[16];
    __shared__ int s_cnt[16];
    __shared__ int s_base;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = -1;  // largest subtree_end of the tiles before this step's
    int real_end = 0;  // one past this thread's last tile that is not isolated
    for (int c0 = 0; c0 < T; c0 += 1024) {
        const int t = c0 + tid;
        int v = t < T ? tmax[(int64_t)b * T + t] : -1;
        // inclusive running maximum: inside the wave, then over the waves
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int y = __shfl_up(v, off, 64);
            if (lane >= off) v = max(v, y);
        }
        if (lane == 63) s_wave[wave] = v;
        __syncthreads();
        if (wave == 0) {
            int w = lane < 16 ? s_wave[lane] : -1;
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) {
                const int y = __shfl_up(w, off, 64);
                if (lane >= off) w = max(w, y);
            }
            if (lane < 16) s_wave[lane] = w;
        }
        __syncthreads();
        const int incl = max(v, wave > 0 ? s_wave[wave - 1] : -1);
        const int prev = __shfl_up(incl, 1, 64);
        const int before = max(carry, lane > 0 ? prev : (wave > 0 ? s_wave[wave - 1] : -1));
        int flag = 0;
        if (t < T) {
            int* f = tiso + (int64_t)b * T + t;
            flag = (*f && before < t * KT) ? 1 : 0;
            *f = flag;
            if (!flag) real_end = t + 1;
        }
        // append the isolated tiles of this step: rank inside the wave by a
        // ballot, then wave offsets, one atomic per step for the base
        const unsigned long long m = __ballot(flag);
        if (lane == 0) s_cnt[wave] = __popcll(m);
        carry = max(carry, s_wave[15]);
        __syncthreads();
        if (tid == 0) {
            int run = 0;
            for (int w = 0; w < 16; ++w) {
                const int c = s_cnt[w];
                s_cnt[w] = run;
                run += c;
            }
            s_base = run ? atomicAdd(&qctr[kIsoCount], run) : 0;
        }
        __syncthreads();
        if (flag) iso_list[s_base + s_cnt[wave] + __popcll(m & ((1ull << lane) - 1ull))] = b * T + t;
        __syncthreads();
    }
    // the tiles past the last non-isolated one of every row (the padding at
    // the end of the rows) need no work items: their slots are isolated
    real_end = wave_max_i32(real_end);
    if (lane == 0 && real_end > 0) atomicMax(&qctr[kRealTiles], real_end);
}

// One unit of isolated-slot work of the forward: part `unit % kIsoSplit` of
// the (slot, head) rows of listed tile `unit / kIsoSplit`: a query that sees
// only itself has a one-term softmax, so out = v and lse = scale q.k; D / 8
// lanes per row.  Out of line, so that the main item's registers are
// allocated without it.
template <int D>
__device__ __attribute__((noinline)) void fwd_iso_unit(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                       const __bf16* __restrict__ v,
                                                       const int32_t* __restrict__ iso_list, int N, int Hq, int Hkv,
                                                       int T, float scale, __bf16* __restrict__ out,
                                                       float* __restrict__ lse, int unit) {
    constexpr int LPR = D / 8, RPW = 64 / LPR;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int G = Hq / Hkv, rows = KT * Hq / kIsoSplit;
    const int e = (lane % LPR) * 8;
    const int bt = iso_list[unit / kIsoSplit];
    const int t = bt % T, b = bt / T;
    const int rbase = (unit % kIsoSplit) * rows;
#pragma unroll 4
    for (int r0 = rbase + wave * RPW; r0 < rbase + rows; r0 += 8 * RPW) {
        const int r = r0 + lane / LPR;
        const int slot = t * KT + r / Hq, h = r % Hq;
        const int sc = min(slot, N - 1);
        const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(q + (((int64_t)b * N + sc) * Hq + h) * D + e);
        const int64_t kv = (((int64_t)b * N + sc) * Hkv + h / G) * D + e;
        const bf16x8 k8 = *reinterpret_cast<const bf16x8*>(k + kv);
        const bf16x8 v8 = *reinterpret_cast<const bf16x8*>(v + kv);
        float dot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) dot = fmaf((float)q8[i], (float)k8[i], dot);
#pragma unroll
        for (int o = 1; o < LPR; o <<= 1) dot += __shfl_xor(dot, o, 64);
        if (slot < N) {
            *reinterpret_cast<bf16x8*>(out + (((int64_t)b * N + slot) * Hq + h) * D + e) = v8;
            if (lane % LPR == 0) lse[((int64_t)b * Hq + h) * N + slot] = dot * scale;
        }
    }
}

// Loads this lane's Q fragments of work item `item` (rows decoded as in
// fwd_item; rows past the end of the row are zero).
template <int D, int HB>
__device__ __forceinline__ void fwd_load_q(const __bf16* __restrict__ q, int B, int N, int Hq, int Hkv,
                                           int n_qblocks, int n_chunks, int item, bf16x8 (&qf)[D / 16]) {
    constexpr int BM = 256 / HB;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int GH = B * Hkv * n_chunks;
    const int gi = item % GH, qi = item / GH;
    const int chunk = gi % n_chunks, g = (gi / n_chunks) % Hkv, b = gi / (n_chunks * Hkv);
    const int head = g * (Hq / Hkv) + chunk * HB + wave % HB;
    const int ip = (n_qblocks - 1 - qi) * BM + (wave / HB) * 32 + (lane & 31);
    const __bf16* src = q + (((int64_t)b * N + min(ip, N - 1)) * Hq + head) * D + (lane >> 5) * 8;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
        bf16x8 z = {};
        qf[c] = ip < N ? *reinterpret_cast<const bf16x8*>(src + 16 * c) : z;
    }
}

// One work item of the forward: BM positions x HB query heads of one KV head.
// Q is loaded here unless q_ready (the previous item loaded it).  After its
// last tile the item claims the next item of its queue and loads that item's
// Q, so the load runs during this item's epilogue; next_item returns the
// claimed item (-1 if none was claimed: an item of isolated slots only).
template <int D, int HB>
__device__ __forceinline__ bool fwd_item(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                         const __bf16* __restrict__ v, const int32_t* __restrict__ se,
                                         const int32_t* __restrict__ tmin, const int32_t* __restrict__ tmax,
                                         const int32_t* __restrict__ tiso, int B, int N, int Hq, int Hkv, int T,
                                         int n_qblocks, int n_chunks, float scale_log2, __bf16* __restrict__ out,
                                         float* __restrict__ lse, int item, char* smem, int* list, int* list_meta,
                                         bf16x8 (&qf)[D / 16], bool q_ready, int* qctr, int qx, int NQ, int n_work,
                                         int* s_next, int& next_item) {
    constexpr int BM = 256 / HB;          // positions per workgroup (8 waves x 32 rows = BM x HB)
    constexpr int NC = D / 16;            // 16-wide chunks of the head dim
    constexpr int NDB = D / 32;           // 32-row blocks of the head dim
    constexpr int CPR = D / 8;            // 16-byte chunks per K / V row
    constexpr int KROW = D * 2;           // LDS bytes per row (chunks swizzled by row_swizzle)
    constexpr int KBYTES = KT * KROW;
    constexpr int STAGE = 2 * KBYTES + KT * 4;
    constexpr int NSTAGE = 4;
    constexpr int KDMA = KBYTES / 1024 / 8;   // 1 KB loads per wave per K (and per V) tile
    constexpr int PER_TILE = 2 * KDMA + 1;    // vector memory ops per wave per tile
    constexpr int LCAP = 1024;                // visible tiles listed per pass
    constexpr int FULL = 1 << 30;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: load bases stay scalar
    const int l32 = lane & 31, hi = lane >> 5;
    const int GH = B * Hkv * n_chunks;
    const int gi = item % GH;
    const int qi = item / GH;
    const int qt = n_qblocks - 1 - qi;  // deeper (later) query tiles first
    const int chunk = gi % n_chunks;
    const int g = (gi / n_chunks) % Hkv;
    const int b = gi / (n_chunks * Hkv);
    const int G = Hq / Hkv;
    const int head = g * G + chunk * HB + wave % HB;
    const int i0 = qt * BM;
    const int i_last = min(i0 + BM, N) - 1;
    const int t_last = i_last / KT;
    {
        // a block of isolated slots only is left to the isolated-slot units
        int iso = 1;
        for (int t = i0 / KT; t <= t_last; ++t) iso &= tiso[(int64_t)b * T + t];
        if (iso) return false;
    }
    const int32_t* tmaxb = tmax + (int64_t)b * T;
    const int32_t* tminb = tmin + (int64_t)b * T;
    const int32_t* seb = se + (int64_t)b * N;
    const int posb = i0 + (wave / HB) * 32;
    const int ip = posb + l32;  // this lane's query position

    if (!q_ready) fwd_load_q<D, HB>(q, B, N, Hq, Hkv, n_qblocks, n_chunks, item, qf);
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) zero(acc[db]);
    float m_run = -INFINITY, l_run = 0.f;

    const __bf16* kb_ = k + ((int64_t)b * N * Hkv + g) * D;
    const __bf16* vb_ = v + ((int64_t)b * N * Hkv + g) * D;

    // all of this wave's loads of one tile: K and V rows (swizzled) and
    // subtree_end.  Per-lane source offsets inside a tile are fixed, so they
    // are computed once; rows past the end of the row are clamped (last tile).
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
    // operand loads of K rows: row x * 32 + l32, chunk 2c + hi
    const int nat_x = (hi ^ row_swizzle<D>(l32)) * 16;
    // transposed loads of V rows (see the dK/dV kernel for the lane mapping)
    int tr_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int row = 4 * (lane >> 5) + ((lane >> 2) & 3) + 8 * half;
            const int chunk = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
            tr_off[db][half] = row * KROW + ((chunk ^ row_swizzle<D>(row)) * 16) + 8 * (lane & 1);
        }

    int resume = 0;
    while (resume >= 0) {
        // visible tiles of this query block, in order, with their class
        if (wave == 0) {
            int cnt = 0, next = -1;
            // the tile bounds of LPF chunks of 64 tiles are loaded together,
            // so the list costs one memory latency per LPF chunks
            constexpr int LPF = 4;
            for (int base0 = resume; base0 <= t_last && next < 0; base0 += 64 * LPF) {
                int tmx[LPF], tmn[LPF];
#pragma unroll
                for (int c = 0; c < LPF; ++c) {
                    const int t = min(base0 + 64 * c + lane, t_last);
                    tmx[c] = tmaxb[t];
                    tmn[c] = tminb[t];
                }
#pragma unroll
                for (int c = 0; c < LPF; ++c) {
                    const int base = base0 + 64 * c;
                    if (base > t_last) break;
                    const int t = base + lane;
                    const bool vis = t <= t_last && tmx[c] >= i0;
                    const bool full = vis && (t * KT + KT - 1 <= i0) && tmn[c] >= i_last;
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
            }
            if (lane == 0) {
                list_meta[0] = cnt;
                list_meta[1] = next;
            }
        }
        __syncthreads();
        const int cnt = list_meta[0];
        resume = list_meta[1];
        // Q (loaded while the list was built) completes before any prefetch is
        // issued: the compiler's wait for it then does not drain the first
        // tiles' prefetches
        wait_vmcnt<0>();

        // Software pipeline: S for tile it+1 is issued next to the softmax and
        // PV product of tile it, so the matrix core has work while the VALU
        // computes probabilities.  Stage it % 4 holds tile it (its V^T and
        // subtree_end are still read), stage (it+1) % 4 tile it+1 (its K is
        // read), and up to two more tiles are in flight.
        // Wait until this wave's loads of a tile have landed, given how many
        // tiles were issued after it, then publish every wave's share.
        auto wait_tile = [&](int ahead) {
            if (ahead >= 2) wait_vmcnt<2 * PER_TILE>();
            else if (ahead == 1) wait_vmcnt<PER_TILE>();
            else wait_vmcnt<0>();
            barrier();
        };
        auto s_product = [&](const char* st, f32x16 (&sacc)[2]) {  // S^T = K Q^T for one tile
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
                for (int x = 0; x < 2; ++x) {
                    bf16x8 a;
                    // Up to two heads per item: one base register per lane, the chunk XORed in and the
                    // row block as an immediate offset. At four and eight heads (more live registers)
                    // per-load offsets measured faster.
                    if constexpr (HB <= 2) {
                        a = lds_ld16(((lds_off(st) + (uint32_t)(l32 * KROW + nat_x)) ^ (32u * c)) +
                                     (uint32_t)(x * 32 * KROW));
                    } else {
                        a = *reinterpret_cast<const bf16x8*>(st + (x * 32 + l32) * KROW + ((32 * c) ^ nat_x));
                    }
                    sacc[x] = c == 0 ? mfma32(a, qf[c], f32x16{}) : mfma32(a, qf[c], sacc[x]);
                }
        };
#pragma unroll
        for (int s0 = 0; s0 < NSTAGE - 1; ++s0)
            if (s0 < cnt) issue(list[s0] & (FULL - 1), s0);
        f32x16 scur[2], snext[2];
        wait_tile(min(NSTAGE - 2, cnt - 1));  // tiles 1 and 2 may still be in flight
        s_product(smem, snext);
        for (int it = 0; it < cnt; ++it) {
            const int e = list[it];
            const int t = e & (FULL - 1);
            const bool full = (e & FULL) != 0;
            const int j0 = t * KT;
            const char* st = smem + (it % NSTAGE) * STAGE;
            scur[0] = snext[0];
            scur[1] = snext[1];
            const bool more = it + 1 < cnt;
            if (more) {
                // issued so far: tiles up to it + 2, so at most one after tile it + 1
                wait_tile(min(1, cnt - 2 - it));
                if (it + NSTAGE - 1 < cnt) issue(list[it + NSTAGE - 1] & (FULL - 1), (it + NSTAGE - 1) % NSTAGE);
            }
            if (!full) {
                const int* ses = reinterpret_cast<const int*>(st + 2 * KBYTES);
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int gq = 0; gq < 4; ++gq) {
                        const int jj = x * 32 + 8 * gq + 4 * hi;
                        const int4 s4 = *reinterpret_cast<const int4*>(ses + jj);
                        const int sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                        for (int e4 = 0; e4 < 4; ++e4) {
                            // a select, not a branch: both tests on every lane
                            const bool vis = (j0 + jj + e4 <= ip) & (ip <= sv[e4]);
                            scur[x][gq * 4 + e4] = vis ? scur[x][gq * 4 + e4] : -INFINITY;
                        }
                    }
            }
            // online softmax; the running max is only raised (and the output
            // rescaled) when a new score exceeds it by more than 2^8
            float mx = -INFINITY;
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, scur[x][r]);
            mx = max_xor32(mx);
            const float mxs = mx * scale_log2;
            if (__ballot(mxs > m_run + 8.f)) {
                const float m_new = fmaxf(m_run, mxs);
                const float corr = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= corr;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[db][r] *= corr;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            // From here on one straight-line block: the next tile's S product
            // (on the last tile it re-reads this stage and is discarded), the
            // probabilities of this tile, and its PV product.
            s_product(smem + ((more ? it + 1 : it) % NSTAGE) * STAGE, snext);
            bf16x8 pf[2][2];
            float rs = 0.f;  // fp32 row sum of the unrounded probabilities
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(scur[x][r], scale_log2, -m_use));
                    rs += p;
                    pf[x][r >> 3][r & 7] = (__bf16)p;
                }
            l_run += rs;
            // O^T += V^T P^T (V^T by transposed loads of the V rows)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int x = 0; x < 2; ++x)
#pragma unroll
                    for (int c2 = 0; c2 < 2; ++c2) {
                        bf16x8 a;
                        if constexpr (HB <= 2) {  // same split as for the K fragments above
                            a = lds_tr_block<D>(lds_off(st) + (uint32_t)(KBYTES + x * 32 * KROW) + tr_offset0<D>(lane),
                                                db, 16 * c2);
                        } else {
                            const char* r0 = st + KBYTES + (x * 32 + c2 * 16) * KROW;
                            a = ld_tr(r0 + tr_off[db][0], r0 + tr_off[db][1]);
                        }
                        acc[db] = mfma32(a, pf[x][c2], acc[db]);
                    }
        }
        if (resume < 0) {
            // the last pass: claim the next item now and load its Q, in flight during the epilogue
            if (tid == 0) *s_next = atomicAdd(&qctr[qx], 1);
            __syncthreads();
            next_item = qx + NQ * s_next[0];
            if (next_item < n_work) fwd_load_q<D, HB>(q, B, N, Hq, Hkv, n_qblocks, n_chunks, next_item, qf);
        }
        __syncthreads();  // the list is rebuilt only after every wave is done with it
    }

    // epilogue: O = O^T / l, lse = (m + log2 l) ln 2
    const float lt = add_xor32(l_run);
    // The wave's 32 rows go out through its own LDS rows (idle now, chunks
    // swizzled as the stages' rows): each store then writes 16 contiguous
    // bytes and a row is 16 lanes of one store.  Rows of isolated tiles belong
    // to the isolated-slot units (the wave's rows lie in one 64-slot tile).
    {
        constexpr int ROWB = D * 2, CH = D / 8;
        char* stg = smem + wave * 32 * ROWB;
        const float inv = 1.f / lt;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                bf16x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = (__bf16)(acc[db][grp * 4 + e] * inv);
                *reinterpret_cast<bf16x4*>(stg + l32 * ROWB + (((db * 4 + grp) ^ row_swizzle<D>(l32)) * 16) +
                                           hi * 8) = v4;
            }
        if (posb < N && !tiso[(int64_t)b * T + posb / KT]) {
            __bf16* o = out + (((int64_t)b * N + posb) * Hq + head) * D;
#pragma unroll
            for (int kk = 0; kk < 32 * CH / 64; ++kk) {
                const int e = kk * 64 + lane, r = e / CH, c = e % CH;
                const bf16x8 val = *reinterpret_cast<const bf16x8*>(stg + r * ROWB + ((c ^ row_swizzle<D>(r)) * 16));
                if (posb + r < N) *reinterpret_cast<bf16x8*>(o + (int64_t)r * Hq * D + c * 8) = val;
            }
            if (hi == 0 && ip < N) lse[((int64_t)b * Hq + head) * N + ip] = (m_run + __log2f(lt)) * kLn2;
        }
    }
    return true;
}

// Persistent forward: one 512-thread workgroup per CU takes work items from
// NQ queues (workgroup w serves queue w mod NQ; queue x holds items x, x + NQ,
// ...).  Items are numbered deepest query block first, with the KV head
// fastest, so the longest items go first and a queue keeps to one KV head
// whenever the heads are a multiple of NQ (its K and V stay in one XCD's L2).
template <int D, int HB>
__global__ __launch_bounds__(512, 1) void fwd_main(const __bf16* __restrict__ q, const __bf16* __restrict__ k,
                                                   const __bf16* __restrict__ v, const int32_t* __restrict__ se,
                                                   const int32_t* __restrict__ tmin,
                                                   const int32_t* __restrict__ tmax,
                                                   const int32_t* __restrict__ tiso, int B, int N, int Hq,
                                                   int Hkv, int T, int n_qtiles, int n_chunks, float scale_log2,
                                                   float scale, __bf16* __restrict__ out, float* __restrict__ lse,
                                                   const int32_t* __restrict__ iso_list, int* __restrict__ qctr,
                                                   int NQ, int n_items) {
    constexpr int STAGE = 2 * KT * D * 2 + KT * 4;
    __shared__ __attribute__((aligned(1024))) char smem[4 * STAGE];
    __shared__ int list[1024];
    __shared__ int list_meta[2];
    __shared__ int s_item, s_next;
    const int qx = blockIdx.x % NQ;
    const int n_units = qctr[kIsoCount] * kIsoSplit;  // isolated-slot units
    bool iso_left = n_units > 0;
    auto claim = [&](int* ctr) {
        if (threadIdx.x == 0) s_item = atomicAdd(ctr, 1);
        __syncthreads();
        const int x = __builtin_amdgcn_readfirstlane(s_item);
        __syncthreads();
        return x;
    };
    // Items cover the query blocks up to the last one with a slot that is not
    // isolated (in any row); the blocks after it (the padding at the end of the
    // rows) are left to the isolated-slot units.
    constexpr int BM = 256 / HB;
    const int n_qblocks = min(n_qtiles, (qctr[kRealTiles] * KT + BM - 1) / BM);
    const int n_work = n_qblocks * (n_items / n_qtiles);
    bf16x8 qf[D / 16];
    int item = qx + NQ * claim(&qctr[qx]);
    bool q_ready = false;
    while (item < n_work) {
        int next_item = -1;
        const bool worked = fwd_item<D, HB>(q, k, v, se, tmin, tmax, tiso, B, N, Hq, Hkv, T, n_qblocks, n_chunks,
                                            scale_log2, out, lse, item, smem, list, list_meta, qf, q_ready, qctr,
                                            qx, NQ, n_work, &s_next, next_item);
        __syncthreads();  // the stages and the list are reused by the next item
        // one unit of the (HBM-bound) isolated-slot work after each item of
        // matrix work, so that it is spread over the kernel instead of
        // saturating HBM on every CU at once
        if (worked && iso_left) {
            const int u = claim(&qctr[kIsoQueue]);
            if (u < n_units) fwd_iso_unit<D>(q, k, v, iso_list, N, Hq, Hkv, T, scale, out, lse, u);
            else iso_left = false;  // the queue is empty: no more claims
        }
        // the item the last one claimed (its Q already loaded), else a claim now
        q_ready = next_item >= 0;
        item = q_ready ? next_item : qx + NQ * claim(&qctr[qx]);
    }
    while (iso_left) {  // what is left of it
        const int u = claim(&qctr[kIsoQueue]);
        if (u >= n_units) break;
        fwd_iso_unit<D>(q, k, v, iso_list, N, Hq, Hkv, T, scale, out, lse, u);
    }
}

template <int D, int HB>
hipError_t launch_main(const AttnArgs& a, const FwdWorkspace& w, int T, hipStream_t st) {
    constexpr int BM = 256 / HB;
    const int G = a.Hq / a.Hkv;
    const int n_chunks = G / HB;
    const int n_qtiles = (a.N + BM - 1) / BM;
    const int64_t items = (int64_t)n_qtiles * a.B * a.Hkv * n_chunks;
    const int grid = (int)std::min<int64_t>(items, mfma_num_cus());
    const int NQ = std::min(kItemQueues, grid);
    const float scale_log2 = a.scale * 1.4426950408889634f;
    hipLaunchKernelGGL((fwd_main<D, HB>), dim3((unsigned)grid), dim3(512), 0, st, (const __bf16*)a.q,
                       (const __bf16*)a.k, (const __bf16*)a.v, a.se, w.tile_min, w.tile_max, w.tile_iso, a.B,
                       a.N, a.Hq, a.Hkv, T, n_qtiles, n_chunks, scale_log2, a.scale, (__bf16*)a.out, a.lse,
                       w.iso_list, w.qctr, NQ, (int)items);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fwd(const AttnArgs& a, const FwdWorkspace& w, hipStream_t st) {
    const int T = (a.N + KT - 1) / KT;
    hipError_t e = launch_tile_ranges(a.se, a.B, a.N, w.tile_min, w.tile_max, w.tile_iso, w.iso_list, w.qctr, st);
    if (e != hipSuccess) return e;
    switch (heads_per_wg(a.Hq / a.Hkv)) {
        case 1: e = launch_main<D, 1>(a, w, T, st); break;
        case 2: e = launch_main<D, 2>(a, w, T, st); break;
        case 4: e = launch_main<D, 4>(a, w, T, st); break;
        default: e = launch_main<D, 8>(a, w, T, st); break;
    }
    if (e != hipSuccess) return e;
    return hipSuccess;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t mfma_fwd_ws_bytes(int B, int N, int Hkv, int D) {
    (void)Hkv;
    (void)D;
    const size_t T = (size_t)(N + KT - 1) / KT;
    return 4 * align256((size_t)B * T * sizeof(int32_t)) + align256(kQueueCounters * sizeof(int32_t));
}

FwdWorkspace carve_fwd_ws(void* ws, int B, int N, int Hkv, int D) {
    (void)Hkv;
    (void)D;
    const size_t T = (size_t)(N + KT - 1) / KT;
    char* p = static_cast<char*>(ws);
    FwdWorkspace w;
    w.tile_min = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_max = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.tile_iso = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.iso_list = reinterpret_cast<int32_t*>(p);
    p += align256((size_t)B * T * sizeof(int32_t));
    w.qctr = reinterpret_cast<int32_t*>(p);
    return w;
}

hipError_t launch_tile_ranges(const int32_t* se, int B, int N, int32_t* tmin, int32_t* tmax, int32_t* tiso,
                              int32_t* iso_list, int32_t* qctr, hipStream_t st) {
    const int T = (N + KT - 1) / KT;
    hipLaunchKernelGGL(fwd_prep, dim3((T + 3) / 4, B), dim3(256), 0, st, se, N, T, tmin, tmax, tiso, qctr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(iso_scan, dim3(B), dim3(1024), 0, st, tmax, T, tiso, iso_list, qctr);
    return hipGetLastError();
}

int mfma_num_cus() {
    // A per-device value written once: racing first calls store the same
    // number, and the atomics make the sharing between threads well defined.
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n <= 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t mfma_attn_fwd(const AttnArgs& a, const FwdWorkspace& w, hipStream_t st) {
    return a.D == 64 ? launch_fwd<64>(a, w, st) : launch_fwd<128>(a, w, st);
}

}  // namespace treeattn
