// Copy-on-write block copies for forked sequences (ocdem.com nano-vllm article, §2.1: the sequences
// of one request, as in parallel sampling or beam search, share physical blocks; a sequence that
// appends into a shared, partially filled block first moves to its own copy).
//
// The 256 rows of one (block, KV head) tile are contiguous, so the rows in use, 0..rows-1, are one
// flat range per head: a shared block half full costs half a block of traffic.  grid = (pair x KV
// head, 4 KiB chunks of the tile, K/V), one 16-byte piece per thread; chunks past the rows in use
// exit at once.  Many small workgroups beat fewer that keep several loads in flight per thread
// (measured on 83 pairs of bf16 8 x 128 tiles: 4 KiB per workgroup 24.5 us, 16 KiB 32 us, 32 KiB
// 43 us), since a step's copies are few and the launch must spread them over every CU.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

struct CopyArgs {
    const int32_t* src;
    const int32_t* dst;
    const int32_t* rows;  // NULL: whole blocks
    uint4* k_cache;
    uint4* v_cache;
    float* k_scale;
    float* v_scale;
    int32_t row_pieces;  // 16-byte pieces per row
    int32_t num_kv_heads;
    int32_t num_blocks;
    int32_t check;       // validate block ids and row counts (device-data checks)
};

constexpr int kCopyThreads = 256, kCopyUnroll = 1;

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyArgs a) {
    const bool is_v = blockIdx.z != 0;
    const int32_t pair = int32_t(blockIdx.x) / a.num_kv_heads;
    const int32_t h = int32_t(blockIdx.x) - pair * a.num_kv_heads;
    const int64_t s = a.src[pair], d = a.dst[pair];
    if (a.check) {  // the same in every thread: a bad pair's workgroups copy nothing
        const int32_t r = a.rows != nullptr ? a.rows[pair] : pkv::kBlock;
        const bool s_bad = s < 0 || s >= a.num_blocks, d_bad = d < 0 || d >= a.num_blocks;
        const bool r_bad = r < 0 || r > pkv::kBlock;
        if (s_bad || d_bad || r_bad) {
            if (threadIdx.x == 0 && h == 0 && blockIdx.y == 0 && blockIdx.z == 0)
                record_error(s_bad || d_bad ? pkv::kErrBlock : pkv::kErrRows, pair,
                             s_bad ? int32_t(s) : d_bad ? int32_t(d) : r);
            return;
        }
    }
    if (a.k_scale != nullptr && blockIdx.y == 0 && threadIdx.x == 0) {
        float* sc = is_v ? a.v_scale : a.k_scale;
        sc[d * a.num_kv_heads + h] = sc[s * a.num_kv_heads + h];
    }
    const int32_t limit = (a.rows != nullptr ? a.rows[pair] : pkv::kBlock) * a.row_pieces;
    const int32_t p0 = int32_t(blockIdx.y) * (kCopyThreads * kCopyUnroll) + int32_t(threadIdx.x);
    if (int32_t(blockIdx.y) * (kCopyThreads * kCopyUnroll) >= limit) return;
    const int64_t tile = int64_t(pkv::kBlock) * a.row_pieces;
    uint4* c = is_v ? a.v_cache : a.k_cache;
    const uint4* from = c + (s * a.num_kv_heads + h) * tile;
    uint4* to = c + (d * a.num_kv_heads + h) * tile;
    uint4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
        if (p0 + kCopyThreads * u < limit) v[u] = from[p0 + kCopyThreads * u];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u)
        if (p0 + kCopyThreads * u < limit) to[p0 + kCopyThreads * u] = v[u];
}

}  // namespace

extern "C" int pkv_copy_blocks(const pkv_cache_desc* desc, const int32_t* src, const int32_t* dst,
                               const int32_t* rows, int32_t n, void* k_cache, void* v_cache, float* k_scale,
                               float* v_scale, void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(n >= 0, PKV_ERR_INVALID, "n = %d", n);
    const bool i8 = desc->kv_dtype == PKV_I8;
    PKV_REQUIRE(i8 == (k_scale != nullptr) && i8 == (v_scale != nullptr), PKV_ERR_INVALID,
                i8 ? "int8 cache: k_scale and v_scale are required"
                   : "scale pointers are only accepted for int8 caches");
    if (n == 0) return PKV_OK;
    PKV_REQUIRE(src && dst && k_cache && v_cache, PKV_ERR_INVALID, "NULL pointer");
    PKV_REQUIRE(((uintptr_t(k_cache) | uintptr_t(v_cache)) & 15) == 0, PKV_ERR_INVALID,
                "cache pointers must be 16-byte aligned");
    PKV_REQUIRE(int64_t(n) * desc->num_kv_heads <= INT32_MAX, PKV_ERR_INVALID, "n = %d too large for one launch",
                n);
    CopyArgs a;
    a.src = src;
    a.dst = dst;
    a.rows = rows;
    a.k_cache = static_cast<uint4*>(k_cache);
    a.v_cache = static_cast<uint4*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.row_pieces = desc->head_dim * pkv::dtype_bytes(desc->kv_dtype) / 16;
    a.num_kv_heads = desc->num_kv_heads;
    a.num_blocks = desc->num_blocks;
    a.check = pkv::device_checks();
    const int per_wg = kCopyThreads * kCopyUnroll;
    const int chunks = (pkv::kBlock * a.row_pieces + per_wg - 1) / per_wg;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(unsigned(n) * unsigned(desc->num_kv_heads), unsigned(chunks), 2),
                       dim3(kCopyThreads), 0, static_cast<hipStream_t>(stream), a);
    hipError_t e = hipGetLastError();
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "copy_blocks launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

int pkv::read_error_copy_blocks(void* stream, int32_t* out) { return read_clear_error(stream, out); }
