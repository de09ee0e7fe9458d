// Device entry points of the C ABI: argument checks, workspace carving, dispatch.
#include <hip/hip_runtime.h>

#include <cmath>

#include "attn_mfma.h"
#include "attn_vec.h"
#include "common.h"

using namespace treeattn;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

tree_status check_shapes(tree_dtype dt, int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t D) {
    if (dt != TREE_F32 && dt != TREE_BF16) return fail(TREE_ERR_INVALID_ARG, "bad dtype %d", (int)dt);
    if (B < 0 || N < 0 || Hq < 1 || Hkv < 1)
        return fail(TREE_ERR_INVALID_ARG, "bad sizes B=%lld N=%lld Hq=%lld Hkv=%lld", (long long)B,
                    (long long)N, (long long)Hq, (long long)Hkv);
    if (Hq % Hkv) return fail(TREE_ERR_INVALID_ARG, "Hq %lld not a multiple of Hkv %lld", (long long)Hq, (long long)Hkv);
    if (D != 64 && D != 128) return fail(TREE_ERR_UNSUPPORTED, "head dim %lld (64 or 128)", (long long)D);
    if (B > 65535 || N > (1LL << 30) || Hq > 65535)
        return fail(TREE_ERR_UNSUPPORTED, "sizes beyond the launch grid");
    if (B * N * Hq * D >= (1LL << 40)) return fail(TREE_ERR_UNSUPPORTED, "tensor too large");
    return TREE_OK;
}

bool use_mfma(tree_dtype dt, int64_t Hq, int64_t Hkv, int64_t D) {
    return dt == TREE_BF16 && mfma_supported((int)D, (int)(Hq / Hkv));
}

size_t fwd_ws(tree_dtype dt, int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t D) {
    return use_mfma(dt, Hq, Hkv, D) ? mfma_fwd_ws_bytes((int)B, (int)N, (int)Hkv, (int)D) : 0;
}

// Backward workspace with `slots` partial-sum slots (the vector path needs only delta).
size_t bwd_ws(tree_dtype dt, int64_t B, int64_t N, int64_t Hq, int64_t Hkv, int64_t D, int slots) {
    if (use_mfma(dt, Hq, Hkv, D)) return mfma_bwd_ws_bytes((int)B, (int)N, (int)Hq, (int)Hkv, (int)D, slots);
    return align_up((size_t)B * Hq * N * sizeof(float));  // delta
}

tree_status device_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return TREE_OK;
    return fail(TREE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" size_t tree_attn_workspace_bytes(tree_dtype dt, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                                            int64_t D, int bwd) {
    if (check_shapes(dt, B, N, Hq, Hkv, D) != TREE_OK) return 0;
    return bwd ? bwd_ws(dt, B, N, Hq, Hkv, D, kSplitSlots) : fwd_ws(dt, B, N, Hq, Hkv, D);
}

extern "C" size_t tree_attn_bwd_workspace_bytes_for(tree_dtype dt, const int32_t* subtree_end, int64_t B,
                                                    int64_t N, int64_t Hq, int64_t Hkv, int64_t D) {
    if (check_shapes(dt, B, N, Hq, Hkv, D) != TREE_OK) return 0;
    if (!use_mfma(dt, Hq, Hkv, D)) return bwd_ws(dt, B, N, Hq, Hkv, D, 0);
    if (B * N > 0 && !subtree_end) return 0;
    const int slots = B * N > 0 ? mfma_bwd_plan_slots(subtree_end, (int)B, (int)N, (int)Hq, (int)Hkv) : 0;
    return bwd_ws(dt, B, N, Hq, Hkv, D, slots);
}

extern "C" tree_status tree_attn_fwd(tree_dtype dt, const void* q, const void* k, const void* v,
                                     const int32_t* subtree_end, int64_t B, int64_t N, int64_t Hq,
                                     int64_t Hkv, int64_t D, float softmax_scale, void* out, float* lse,
                                     void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    tree_status s = check_shapes(dt, B, N, Hq, Hkv, D);
    if (s != TREE_OK) return s;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
        return fail(TREE_ERR_INVALID_ARG, "softmax_scale %g must be finite and positive", (double)softmax_scale);
    if (B == 0 || N == 0) return TREE_OK;
    if (!q || !k || !v || !subtree_end || !out || !lse) return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    const size_t need = fwd_ws(dt, B, N, Hq, Hkv, D);
    if (ws_bytes < need || (need && !ws))
        return fail(TREE_ERR_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnArgs a{dt, q, k, v, subtree_end, (int)B, (int)N, (int)Hq, (int)Hkv, (int)D, softmax_scale,
               out, lse, nullptr, nullptr, nullptr, nullptr};
    if (use_mfma(dt, Hq, Hkv, D))
        return device_status(mfma_attn_fwd(a, carve_fwd_ws(ws, (int)B, (int)N, (int)Hkv, (int)D), (hipStream_t)stream),
                             "tree_attn_fwd launch");
    return device_status(vec_attn_fwd(a, (hipStream_t)stream), "tree_attn_fwd launch");
}

extern "C" tree_status tree_attn_bwd(tree_dtype dt, const void* q, const void* k, const void* v,
                                     const int32_t* subtree_end, const void* out, const float* lse,
                                     const void* dout, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                                     int64_t D, float softmax_scale, void* dq, void* dk, void* dv,
                                     void* ws, size_t ws_bytes, void* stream) {
    clear_error();
    tree_status s = check_shapes(dt, B, N, Hq, Hkv, D);
    if (s != TREE_OK) return s;
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
        return fail(TREE_ERR_INVALID_ARG, "softmax_scale %g must be finite and positive", (double)softmax_scale);
    if (B == 0 || N == 0) return TREE_OK;
    if (!q || !k || !v || !subtree_end || !out || !lse || !dout || !dq || !dk || !dv)
        return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    const size_t need = bwd_ws(dt, B, N, Hq, Hkv, D, 0);  // fixed part; partial-sum slots are what is beyond
    if (ws_bytes < need || !ws) return fail(TREE_ERR_CAPACITY, "workspace %zu < %zu bytes", ws_bytes, need);
    AttnArgs a{dt, q, k, v, subtree_end, (int)B, (int)N, (int)Hq, (int)Hkv, (int)D, softmax_scale,
               const_cast<void*>(out), const_cast<float*>(lse), dout, dq, dk, dv};
    if (use_mfma(dt, Hq, Hkv, D))
        return device_status(
            mfma_attn_bwd(a, carve_bwd_ws(ws, ws_bytes, (int)B, (int)N, (int)Hq, (int)Hkv, (int)D),
                          (hipStream_t)stream),
            "tree_attn_bwd launch");
    return device_status(vec_attn_bwd(a, (float*)ws, (hipStream_t)stream), "tree_attn_bwd launch");
}
