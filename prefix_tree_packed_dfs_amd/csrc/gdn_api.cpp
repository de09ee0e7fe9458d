// Device entry points of the C ABI for gated-delta-rule mixing: argument checks, workspace, dispatch.
#include <hip/hip_runtime.h>

#include "common.h"
#include "gdn.h"

using namespace treeattn;

namespace {

tree_status check_gdn(int64_t n, int64_t n_seg, int64_t n_chunks, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv) {
    if (n < 0 || n_seg < 0 || n_chunks < 0 || Hk < 1 || Hv < 1)
        return fail(TREE_ERR_INVALID_ARG, "bad sizes n=%lld chains=%lld chunks=%lld Hk=%lld Hv=%lld", (long long)n,
                    (long long)n_seg, (long long)n_chunks, (long long)Hk, (long long)Hv);
    if (Hv % Hk) return fail(TREE_ERR_INVALID_ARG, "Hv %lld not a multiple of Hk %lld", (long long)Hv, (long long)Hk);
    if (dk != kGdnDim || dv != kGdnDim)
        return fail(TREE_ERR_UNSUPPORTED, "head dims %lld x %lld (128 x 128)", (long long)dk, (long long)dv);
    if (n > INT32_MAX || n_seg > n || n_chunks > n || Hv > 65535 || Hk > 65535)
        return fail(TREE_ERR_UNSUPPORTED, "sizes beyond the launch grid");
    if (n_chunks * Hv > INT32_MAX || n_seg * Hv > INT32_MAX)
        return fail(TREE_ERR_UNSUPPORTED, "sizes beyond the launch grid");
    return TREE_OK;
}

}  // namespace

extern "C" size_t tree_gdn_workspace_bytes(int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv,
                                           int64_t dk, int64_t dv) {
    if (check_gdn(n, n_states, n_chunks, Hk, Hv, dk, dv) != TREE_OK) return 0;
    return gdn_ws_bytes(n, n_states, n_chunks, Hk, Hv);
}

extern "C" tree_status tree_gdn_fwd(tree_dtype dt, const void* x, const float* conv_w, int64_t conv_width,
                                    const float* g, const float* beta, const int32_t* parent_slot,
                                    const int32_t* segments, int64_t n_segments, const int32_t* chunks,
                                    int64_t n_chunks, const int32_t* depth_offsets, int64_t n_depths,
                                    int64_t n_states, int64_t n, int64_t Hk, int64_t Hv, int64_t dk, int64_t dv,
                                    void* out, void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    if (dt != TREE_BF16) return fail(TREE_ERR_UNSUPPORTED, "dtype %d (bf16 only)", (int)dt);
    tree_status s = check_gdn(n, n_segments, n_chunks, Hk, Hv, dk, dv);
    if (s != TREE_OK) return s;
    if (conv_width < 1 || conv_width > 4) return fail(TREE_ERR_UNSUPPORTED, "conv width %lld (1..4)", (long long)conv_width);
    if (n == 0) return TREE_OK;
    if (!x || !conv_w || !g || !beta || !parent_slot || !segments || !chunks || !depth_offsets || !out)
        return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    if (n_states < 0 || (n_segments > 0 && n_states >= n_segments))
        return fail(TREE_ERR_INVALID_ARG, "n_states %lld for %lld chains", (long long)n_states, (long long)n_segments);
    if (n_segments < 1 || n_chunks < n_segments || n_depths < 1 || n_depths > n_segments)
        return fail(TREE_ERR_INVALID_ARG, "plan sizes %lld chains, %lld chunks, %lld depths do not fit %lld slots",
                    (long long)n_segments, (long long)n_chunks, (long long)n_depths, (long long)n);
    // the host half of the plan: depth buckets must tile [0, n_segments) in order
    if (depth_offsets[0] != 0 || depth_offsets[n_depths] != n_segments)
        return fail(TREE_ERR_INVALID_ARG, "depth_offsets do not cover the chains");
    for (int64_t d = 0; d < n_depths; ++d)
        if (depth_offsets[d + 1] <= depth_offsets[d])
            return fail(TREE_ERR_INVALID_ARG, "depth_offsets not increasing at %lld", (long long)d);
    const size_t need = gdn_ws_bytes(n, n_states, n_chunks, Hk, Hv);
    if (ws_bytes < need || !ws) return fail(TREE_ERR_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
    GdnArgs a{x, conv_w, (int)conv_width, g, beta, parent_slot, segments, chunks,
              depth_offsets, (int)n, (int)n_segments, (int)n_chunks, (int)n_depths, (int)Hk, (int)Hv,
              out};
    const hipError_t e = gdn_forward(a, carve_gdn_ws(ws, n, n_states, n_chunks, Hk, Hv), (hipStream_t)stream);
    if (e != hipSuccess) return fail(TREE_ERR_DEVICE, "tree_gdn_fwd launch: %s", hipGetErrorString(e));
    return TREE_OK;
}
