// Matrix-core (MFMA) attention path for bf16: shared constants and launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "attn_vec.h"

namespace treeattn {

// Keys per KV tile and rows per MFMA block.
constexpr int KT = 64;
// Work queues of the persistent query-stationary kernels (one per XCD).
constexpr int kItemQueues = 8;
// Work-queue counters after the item queues: the isolated-slot unit queue,
// the number of isolated tiles listed, and the number of KT-key tiles up to
// the last one (over all rows) that holds a slot that is not isolated.  An
// isolated tile is kIsoSplit units.
constexpr int kIsoQueue = kItemQueues;
constexpr int kIsoCount = kItemQueues + 1;
constexpr int kRealTiles = kItemQueues + 2;
constexpr int kQueueCounters = kItemQueues + 3;
constexpr int kIsoSplit = 8;

// Query heads one workgroup serves (all heads sharing a KV head, up to 8).
inline int heads_per_wg(int G) { return G >= 8 ? 8 : G; }
// Whether the MFMA path covers this shape (else the vector path runs).
inline bool mfma_supported(int D, int G) {
    return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G % 8 == 0);
}

// Workspace carved by the forward: per-tile subtree_end range.
struct FwdWorkspace {
    int32_t* tile_min;   // [B, T]
    int32_t* tile_max;   // [B, T]
    int32_t* tile_iso;   // [B, T] 1 if every slot of the tile is isolated (sees and is seen by itself only)
    int32_t* iso_list;   // [B * T] the isolated tiles, b * T + t, in no particular order
    int32_t* qctr;       // [kQueueCounters] work-queue counters of the persistent forward
};

// Workspace carved by the backward.
struct BwdWorkspace {
    float* delta;        // [B, Hq, N]  rowsum(dout * out)
    float* lse2;         // [B, Hq, N]  lse * log2(e)
    int32_t* tile_min;   // [B, T]
    int32_t* tile_max;   // [B, T]
    int32_t* tile_iso;   // [B, T]
    int32_t* iso_list;   // [B * T]
    int32_t* qctr;       // [kQueueCounters] work-queue counters of the persistent dQ kernel
    // dK/dV work plan: KV tiles of 256 keys whose query range is long are split
    // into chunks of visits; chunks write fp32 partials that a reduce pass sums
    int32_t* ctrl;       // queue counters / lengths / starts, split-tile count
    int4* tile_plan;     // [B * TT] {first query block, last query block, chunks, first slot or -1}
    int4* units;         // [unit capacity][2] {b*Hkv+g, tile, first visit, end visit}, {slot, 0, 0, 0}
    int4* split_tiles;   // [kSplitSlots/2] {b, tile, first slot, splits}
    float* partial;      // [slot_cap][2][kKvTile][D] fp32 dK, dV partial sums
    int slot_cap;        // partial-sum slots the workspace holds (0 .. kSplitSlots)
};

// Keys per dK/dV workgroup tile, partial-sum slots for split tiles, and the
// initial visit budget per chunk.
constexpr int kKvTile = 256;
constexpr int kSplitSlots = 1536 * 256 / kKvTile;
constexpr int kVisitBudget = 320;

// Smallest and largest subtree_end of every KT-key tile of each row ([B, T]),
// and whether every slot of the tile is isolated; the isolated tiles listed
// in iso_list, their number in qctr[kIsoCount]; qctr[kRealTiles] = one past
// the last tile of any row with a slot that is not isolated.
// (Also zeroes the kQueueCounters work-queue counters at qctr first.)
hipError_t launch_tile_ranges(const int32_t* se, int B, int N, int32_t* tmin, int32_t* tmax, int32_t* tiso,
                              int32_t* iso_list, int32_t* qctr, hipStream_t st);
// Compute units of the current device (cached per device).
int mfma_num_cus();
size_t mfma_fwd_ws_bytes(int B, int N, int Hkv, int D);
FwdWorkspace carve_fwd_ws(void* ws, int B, int N, int Hkv, int D);
hipError_t mfma_attn_fwd(const AttnArgs& a, const FwdWorkspace& w, hipStream_t st);
// Backward workspace with `slots` partial-sum slots (0 = the fixed part only).
size_t mfma_bwd_ws_bytes(int B, int N, int Hq, int Hkv, int D, int slots);
// Partial-sum slots the dK/dV plan of these rows uses at its first budget
// (capped at kSplitSlots), from subtree_end [B, N] in host memory.
int mfma_bwd_plan_slots(const int32_t* se, int B, int N, int Hq, int Hkv);
BwdWorkspace carve_bwd_ws(void* ws, size_t ws_bytes, int B, int N, int Hq, int Hkv, int D);
hipError_t mfma_attn_bwd(const AttnArgs& a, const BwdWorkspace& w, hipStream_t st);

}  // namespace treeattn
