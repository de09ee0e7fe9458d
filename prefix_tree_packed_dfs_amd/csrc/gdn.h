// Gated-delta-rule mixing over a packed row: launchers and workspace layout (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace treeattn {

constexpr int kGdnChunk = 64;   // tokens per chunk of the chunked recurrence
constexpr int kGdnDim = 128;    // key and value head dim

// Per (chunk, value head) block written by the chunk kernel and copied whole into
// LDS by the state pass: operand fragments in the lane order the matrix core reads.
//   Wn  [2 row tiles][8 K-steps][64 lanes][8]  bf16   -W, A operand of W H
//   M   [2 row tiles][4 K-steps][64][8]        bf16   decayed, masked Q K^T, A operand
//   KT  [4 row tiles][4 K-steps][64][8]        bf16   K^T, A operand of the state update
//   Q   [2 row tiles][8 K-steps][64][8]        bf16   diag(e^G) Q, A operand of Q H
//   U   [4 col tiles][2 row tiles][64][16]     bf16   U, accumulator layout
//   eLG [64] fp32 e^{G_last - G_j}; gL fp32 e^{G_last}
constexpr size_t kGdnWn = 0;
constexpr size_t kGdnM = kGdnWn + 2 * 8 * 64 * 8 * 2;
constexpr size_t kGdnKT = kGdnM + 2 * 4 * 64 * 8 * 2;
constexpr size_t kGdnQ = kGdnKT + 4 * 4 * 64 * 8 * 2;
constexpr size_t kGdnU = kGdnQ + 2 * 8 * 64 * 8 * 2;
constexpr size_t kGdnELG = kGdnU + 4 * 2 * 64 * 16 * 2;
constexpr size_t kGdnGL = kGdnELG + 64 * 4;
constexpr size_t kGdnBlock = kGdnGL + 256;  // 74,240 bytes

struct GdnArgs {
    const void* x;            // [n, C] bf16 mixing input, channels q | k | v
    const float* conv_w;      // [C, W]
    int W;
    const float* g;           // [n, Hv] log decay
    const float* beta;        // [n, Hv]
    const int32_t* parent;    // [n] parent slot, -1 at roots
    const int32_t* segs;      // [n_seg][4] first chunk, chunk count, parent state slot, own state slot
    const int32_t* chunks;    // [n_chunks][2] first slot, length
    const int32_t* depth_off; // host [n_depths + 1]
    int n, n_seg, n_chunks, n_depths, Hk, Hv;
    void* out;                // [n, Hv, 128] bf16
};

struct GdnWorkspace {
    void* mixed;              // [n, C] bf16 after convolution, SiLU and normalisation
    char* blocks;             // [n_chunks][Hv] blocks of kGdnBlock bytes
    float* states;            // [n_states][Hv][4][4][64][16] final state of every chain with children
};

size_t gdn_ws_bytes(int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv);
GdnWorkspace carve_gdn_ws(void* ws, int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv);
hipError_t gdn_forward(const GdnArgs& a, const GdnWorkspace& w, hipStream_t st);

}  // namespace treeattn
