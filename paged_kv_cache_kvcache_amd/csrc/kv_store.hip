// store_kvcache for gfx950: scatter new K/V rows into the paged cache by slot
// ("Nano-vLLM性能调优实战", §2.2 缓存复用策略 names the store_kvcache kernel that writes the cache).
//
// One thread moves one 16-byte piece of one row.  Consecutive threads walk the pieces of
// consecutive (token, head) rows, so both the read of the packed [n][Hkv][D] input and the
// write of each destination row (contiguous in the [block][head][256][D] layout) are fully
// coalesced.  K and V pieces share one launch.  The copy is bit-exact: no arithmetic.
#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace {

struct StoreArgs {
    const uint4* k_new;
    const uint4* v_new;
    const float* k_scale_new;
    const float* v_scale_new;
    const int32_t* slots;
    uint4* k_cache;
    uint4* v_cache;
    float* k_scale;
    float* v_scale;
    int32_t pieces;          // n * Hkv * pieces_per_row, per tensor
    int32_t row_shift;       // log2(pieces_per_row); rows are 64..512 bytes, a power of two
    int32_t num_kv_heads;
};

// grid.y selects K (0) or V (1).
__global__ __launch_bounds__(256) void kv_store_kernel(StoreArgs a) {
    const int32_t p = int32_t(blockIdx.x) * 256 + int32_t(threadIdx.x);
    if (p >= a.pieces) return;
    const bool is_v = blockIdx.y != 0;
    const int32_t row = p >> a.row_shift;  // (token, head)
    const int32_t piece = p & ((1 << a.row_shift) - 1);
    const int32_t t = row / a.num_kv_heads;
    const int32_t h = row - t * a.num_kv_heads;
    const int32_t slot = a.slots[t];
    if (slot < 0) return;
    const int64_t blk = slot / pkv::kBlock, off = slot % pkv::kBlock;
    const int64_t dst_row = (blk * a.num_kv_heads + h) * pkv::kBlock + off;
    const uint4 val = (is_v ? a.v_new : a.k_new)[p];
    (is_v ? a.v_cache : a.k_cache)[(dst_row << a.row_shift) + piece] = val;
    if (a.k_scale != nullptr && piece == 0) {
        float* dst = is_v ? a.v_scale : a.k_scale;
        const float* src = is_v ? a.v_scale_new : a.k_scale_new;
        dst[blk * a.num_kv_heads + h] = src[row];
    }
}

}  // namespace

extern "C" int pkv_kv_store(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                            const float* k_scale_new, const float* v_scale_new, const int32_t* slot_mapping,
                            int32_t n, void* k_cache, void* v_cache, float* k_scale, float* v_scale,
                            void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    const bool i8 = desc->kv_dtype == PKV_I8;
    if (i8) {
        PKV_REQUIRE(k_scale_new && v_scale_new && k_scale && v_scale, PKV_ERR_INVALID,
                    "int8 cache: all four scale pointers are required");
    } else {
        PKV_REQUIRE(!k_scale_new && !v_scale_new && !k_scale && !v_scale, PKV_ERR_INVALID,
                    "scale pointers are only accepted for int8 caches");
    }
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(k_new && v_new && slot_mapping && k_cache && v_cache, PKV_ERR_INVALID, "NULL pointer");
    const uintptr_t mis = uintptr_t(k_new) | uintptr_t(v_new) | uintptr_t(k_cache) | uintptr_t(v_cache);
    PKV_REQUIRE((mis & 15) == 0, PKV_ERR_INVALID, "K/V pointers must be 16-byte aligned");
    const int row_bytes = desc->head_dim * pkv::dtype_bytes(desc->kv_dtype);
    StoreArgs a;
    a.k_new = static_cast<const uint4*>(k_new);
    a.v_new = static_cast<const uint4*>(v_new);
    a.k_scale_new = k_scale_new;
    a.v_scale_new = v_scale_new;
    a.slots = slot_mapping;
    a.k_cache = static_cast<uint4*>(k_cache);
    a.v_cache = static_cast<uint4*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    const int ppr = row_bytes / 16;
    a.row_shift = 0;
    while ((1 << a.row_shift) < ppr) ++a.row_shift;
    a.num_kv_heads = desc->num_kv_heads;
    const int64_t pieces = int64_t(n) * desc->num_kv_heads * ppr;
    PKV_REQUIRE(pieces <= INT32_MAX - 256, PKV_ERR_INVALID, "n = %d too large for one launch", n);
    a.pieces = int32_t(pieces);
    const unsigned grid = unsigned((pieces + 255) / 256);
    hipLaunchKernelGGL(kv_store_kernel, dim3(grid, 2), dim3(256), 0, static_cast<hipStream_t>(stream), a);
    hipError_t e = hipGetLastError();
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "kv_store launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}
