// Arguments of one attention call, shared by the kernel families.
#pragma once

#include <hip/hip_runtime.h>

#include "common.h"

namespace treeattn {

struct AttnArgs {
    tree_dtype dt;
    const void* q;
    const void* k;
    const void* v;
    const int32_t* se;  // subtree_end [B, N]
    int B, N, Hq, Hkv, D;
    float scale;
    void* out;
    float* lse;
    // backward only
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
};

hipError_t vec_attn_fwd(const AttnArgs& a, hipStream_t st);
hipError_t vec_attn_bwd(const AttnArgs& a, float* delta, hipStream_t st);

}  // namespace treeattn
