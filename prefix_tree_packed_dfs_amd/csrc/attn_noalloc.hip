// tree_attn_fwd_noalloc: the forward for callers that cannot allocate device
// memory.  Its per-call tables (per-tile subtree_end ranges, isolated-tile
// list, work-queue counters) live in a fixed array of this library's device
// code instead of a caller workspace; the kernels are tree_attn_fwd's.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/tree_attn.h"
#include "common.h"

namespace {

// Room for the forward's tables: four int32 tables of B x ceil(N / 64)
// entries (each 256-byte aligned) and the queue counters, for up to 65,536
// tiles of 64 slots.
constexpr int64_t kMaxTiles = 65536;
constexpr size_t kScratchBytes = 4 * kMaxTiles * sizeof(int32_t) + 65536;

// One copy per GPU, held until the process ends.  Host code never uses this
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device (g_ptr).
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device: looked up on the first
// call on that device (with it current), then kept.
tree_status scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return treeattn::fail(TREE_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return treeattn::fail(TREE_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return treeattn::fail(TREE_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return TREE_OK;
}

}  // namespace

extern "C" tree_status tree_attn_fwd_noalloc(tree_dtype dt, const void* q, const void* k, const void* v,
                                             const int32_t* subtree_end, int64_t B, int64_t N, int64_t Hq,
                                             int64_t Hkv, int64_t D, float softmax_scale, void* out, float* lse,
                                             void* stream) {
    treeattn::clear_error();
    // sizes first: a call beyond the array is refused before any device call
    const size_t need = tree_attn_workspace_bytes(dt, B, N, Hq, Hkv, D, 0);
    if (B >= 0 && N >= 0 && B <= 65535 && N <= (int64_t(1) << 30) && B * ((N + 63) / 64) > kMaxTiles)
        return treeattn::fail(TREE_ERR_CAPACITY, "%lld rows x %lld slots exceed the %lld tiles of 64 slots "
                              "tree_attn_fwd_noalloc holds tables for",
                              (long long)B, (long long)N, (long long)kMaxTiles);
    if (need > kScratchBytes)
        return treeattn::fail(TREE_ERR_CAPACITY, "tables of %zu bytes exceed the %zu-byte array", need,
                              kScratchBytes);
    if (need == 0)  // bad sizes (reported by the checks of tree_attn_fwd), or the vector path: no tables
        return tree_attn_fwd(dt, q, k, v, subtree_end, B, N, Hq, Hkv, D, softmax_scale, out, lse, nullptr, 0,
                             stream);
    void* ws = nullptr;
    const tree_status s = scratch_on_current_device(&ws);
    if (s != TREE_OK) return s;
    return tree_attn_fwd(dt, q, k, v, subtree_end, B, N, Hq, Hkv, D, softmax_scale, out, lse, ws, kScratchBytes,
                         stream);
}
