// store_kvcache for gfx950: scatter new K/V rows into the paged cache by slot
// ("Nano-vLLM性能调优实战", §2.2 缓存复用策略 names the store_kvcache kernel that writes the cache).
//
// One thread moves one 16-byte piece of one row.  Consecutive threads walk the pieces of
// consecutive (token, head) rows, so both the read of the packed [n][Hkv][D] input and the
// write of each destination row (contiguous in the [block][head][256][D] layout) are fully
// coalesced.  K and V pieces share one launch.  The copy is bit-exact: no arithmetic.
#include <hip/hip_runtime.h>

#include "pkv_device.h"
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
    int64_t pool_slots;      // num_blocks * 256
    int32_t check;           // validate slots (device-data checks)
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
    if (a.check && slot >= a.pool_slots) {  // a row outside the pool is skipped and reported
        if (h == 0 && piece == 0 && !is_v) record_error(pkv::kErrSlot, t, slot);
        return;
    }
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
    a.pool_slots = int64_t(desc->num_blocks) * pkv::kBlock;
    a.check = pkv::device_checks();
    const int64_t pieces = int64_t(n) * desc->num_kv_heads * ppr;
    PKV_REQUIRE(pieces <= INT32_MAX - 256, PKV_ERR_INVALID, "n = %d too large for one launch", n);
    a.pieces = int32_t(pieces);
    const unsigned grid = unsigned((pieces + 255) / 256);
    hipLaunchKernelGGL(kv_store_kernel, dim3(grid, 2), dim3(256), 0, static_cast<hipStream_t>(stream), a);
    hipError_t e = hipGetLastError();
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "kv_store launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

// ------------------------------------------------------------------------------------------
// Quantising store into int8 caches.  The pages name INT8 KV as an engine option
// (intelliparadigm.com Nano-vLLM article, §2.2 混合精度计算流水线) without an encoding; this
// library's encoding keeps one fp32 scale per (physical block, KV head):
//   * the new rows of one call that land in one block form a run of consecutive slots (the
//     allocator hands out a prompt's tokens and a decode append this way);
//   * candidate = fl32(absmax of the run's new values / 127) (the quotient in fp64);
//   * old = the block's scale when the run starts at offset o0 > 0, else 0 (a fresh block);
//   * new = max(old, candidate); when new > old, rows 0..o0-1 are re-quantised,
//     code -> rint(code * old / new);
//   * the run's rows become clamp(rint(x / new), -127, 127) (0 when new = 0); scale = new.
// rint rounds half to even, on the exact quotient.  A quotient of an 8..32-bit value by a
// 24-bit scale is never within 2^-33 (relative) of a half-integer unless it is one, so rounding
// the fp64 quotient and rounding the exact quotient agree.
//
// One workgroup per (run, KV head, K or V), from a run list the host builds with the slot
// mapping (pkv_store_runs).  Short runs (decode appends) take one wavefront, long ones eight.
// Rounding takes one FMA per value (see quant8); on the prefill workload's chunks this took a
// chunk's store from 13.5 to 12.3 us.  Cutting long runs into 64-row pieces spread over more
// workgroups did not pay: with a second launch for the absmax (4.7 + 9.3 us) or with every piece
// reducing its whole run from L2 (14.7 us).
namespace {

struct QuantArgs {
    const char* k_new;
    const char* v_new;
    const int32_t* slots;
    const int32_t* runs;   // (first row, length) per run
    int8_t* k_cache;
    int8_t* v_cache;
    float* k_scale;
    float* v_scale;
    int32_t num_kv_heads;
    int32_t n;            // batch rows
    int32_t wide;         // runs of more than 16 rows: eight wavefronts per run
    int64_t pool_slots;   // num_blocks * 256
    int32_t check;        // validate the run list and slots (device-data checks)
};

// The fp32 estimate x * fl(1/s) of x / s has relative error below 2^-23 + 2^-48 (below 3 * 2^-24
// when x itself was rounded to fp32 first), so it is within 2.3e-5 of x / s for |x / s| <= 128:
// its rounding agrees with that of x / s unless it lies within kNearHalf of a half-integer.  Only
// then the exact fp64 residual 2 (x - k s) decides.
constexpr float kNearHalf = 6e-5f;
// fma(x, rcp, kRound) rounds x * rcp (exact inside the fma) to an integer k, ties to even, and
// leaves k in the low bits: the bit pattern is that of kRound plus k, whose low byte is k as an
// int8 for |k| <= 128
constexpr float kRound = 12582912.0f;  // 1.5 * 2^23

__device__ __forceinline__ int fix_rint(int k, double x, double s) {
    const double r2 = 2.0 * __builtin_fma(-double(k), s, x);  // exact
    const bool odd = (k & 1) != 0;
    return k + int(r2 > s || (r2 == s && odd)) - int(r2 < -s || (r2 == -s && odd));
}

// Code bytes of eight values: clamp(rint(x[e] / s), -127, 127) (s > 0, or s = 0 with rcp = 0,
// which gives zeros), with x[e] * rcp first.  |x[e]| <= 127 s holds for the run's own values (s
// is at least their absmax / 127, up to fp32 rounding that keeps the quotient below 127.5), so
// their codes need no clamp; re-quantised rows (CLAMP) are clamped, which matters only when
// rows 0..o0-1 were not written by this store (c old / s with old <= s is otherwise in range).
// xd[e] is the exact value when it differs from x[e] (a product code * old); nullptr when x[e]
// is exact.
template <bool CLAMP>
__device__ __forceinline__ uint2 quant8(const float (&x)[8], const double* xd, float s, float rcp) {
    float t[8];
    bool near = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        t[e] = __builtin_fmaf(x[e], rcp, kRound);
        const float r = __builtin_fmaf(x[e], rcp, -(t[e] - kRound));  // x rcp - k
        near |= fabsf(r) > 0.5f - kNearHalf;
    }
    uint32_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        b[e] = CLAMP ? uint32_t(min(max(int(t[e] - kRound), -127), 127)) : __float_as_uint(t[e]);
    if (near) {  // rare: the exact quotient decides
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int k = fix_rint(int(t[e] - kRound), xd != nullptr ? xd[e] : double(x[e]), double(s));
            b[e] = uint32_t(min(max(k, -127), 127));
        }
    }
    return make_uint2(__builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u) | (__builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u) << 16),
                      __builtin_amdgcn_perm(b[5], b[4], 0x0c0c0400u) | (__builtin_amdgcn_perm(b[7], b[6], 0x0c0c0400u) << 16));
}

// Eight values 8 pc .. 8 pc + 7 of head h of batch row t, as fp32.
template <int D, bool F32>
__device__ __forceinline__ void load8(const char* src, size_t row_stride, int t, int h, int pc, float (&x)[8]) {
    const char* p = src + size_t(t) * row_stride + (size_t(h) * D + 8 * pc) * (F32 ? 4 : 2);
    if constexpr (F32) {
        const uint4 u0 = reinterpret_cast<const uint4*>(p)[0], u1 = reinterpret_cast<const uint4*>(p)[1];
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e]);
    } else {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = __uint_as_float(w[e] << 16);
            x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
        }
    }
}

// The run's checks (device-data checks on): it lies in the batch and its rows in one block of
// the pool.  The same in every thread, so a failing workgroup leaves as a whole.
__device__ __forceinline__ bool run_ok(const QuantArgs& a, int run, int t0, int len, bool report) {
    const bool in_batch = t0 >= 0 && len >= 1 && len <= pkv::kBlock && t0 <= a.n - len;
    const int32_t sc = in_batch ? a.slots[t0] : 0;
    const bool slot_ok = sc >= 0 && sc < a.pool_slots && sc % pkv::kBlock + len <= pkv::kBlock;
    if ((!in_batch || !slot_ok) && report && threadIdx.x == 0)
        record_error(in_batch ? pkv::kErrSlot : pkv::kErrRun, in_batch ? t0 : run, in_batch ? sc : t0);
    return in_batch && slot_ok;
}

// Re-quantise cache rows r (of D codes) to scale sn from scale old: code -> rint(code old / sn).
template <int D>
__device__ __forceinline__ void requant_row_piece(int8_t* cache, int r, int cp, float old, float sn, float rcp) {
    uint2* p = reinterpret_cast<uint2*>(cache + size_t(r) * D + 8 * cp);
    const uint2 u = *p;
    float x[8];
    double xd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int c = int(int8_t((e < 4 ? u.x : u.y) >> (8 * (e & 3))));
        xd[e] = double(c) * double(old);  // exact
        x[e] = float(xd[e]);
    }
    *p = quant8<true>(x, xd, sn, rcp);
}

// ---- one workgroup per run: absmax, re-quantisation, codes and scale.  NT = 64 threads for
// runs of at most 16 rows (decode appends), 512 for longer ones.
template <int D, bool F32, int NT>
__global__ __launch_bounds__(NT) void kv_store_quant_kernel(QuantArgs a) {
    constexpr int PR = D / 8;    // 8-value pieces per row
    constexpr int RS = NT / PR;  // rows per pass
    constexpr int MR = (NT == 64 ? 16 : pkv::kBlock) / RS;  // passes for the longest run
    constexpr int NWAVE = NT / 64;
    const int h = blockIdx.y;
    const bool is_v = blockIdx.z != 0;
    const int t0 = a.runs[2 * blockIdx.x], len = a.runs[2 * blockIdx.x + 1];
    if (a.check && !run_ok(a, int(blockIdx.x), t0, len, h == 0 && !is_v)) return;
    const int32_t s0 = a.slots[t0];
    const int64_t blk = s0 / pkv::kBlock;
    const int o0 = s0 % pkv::kBlock;
    float* scale = (is_v ? a.v_scale : a.k_scale) + blk * a.num_kv_heads + h;
    const float old = o0 > 0 ? *scale : 0.f;  // requested early: its latency overlaps the row loads

    const char* src = is_v ? a.v_new : a.k_new;
    const size_t row_stride = size_t(a.num_kv_heads) * D * (F32 ? 4 : 2);
    const int pc = threadIdx.x % PR, r0 = threadIdx.x / PR;
    // the run's rows, all loaded at once: thread (r0, pc) holds rows r0 + u RS (slots past the
    // run re-read its last row)
    float x[MR][8];
#pragma unroll
    for (int u = 0; u < MR; ++u) load8<D, F32>(src, row_stride, t0 + min(r0 + u * RS, len - 1), h, pc, x[u]);
    float amax = 0.f;
#pragma unroll
    for (int u = 0; u < MR; ++u)
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(x[u][e]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if constexpr (NWAVE > 1) {
        __shared__ float s_red[NWAVE];
        if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = amax;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < NWAVE; ++i) amax = fmaxf(amax, s_red[i]);
    }
    const float sn = fmaxf(old, float(double(amax) / 127.0));  // the same value in every thread
    const float rcp = sn > 0.f ? 1.f / sn : 0.f;
    int8_t* cache = (is_v ? a.v_cache : a.k_cache) + ((blk * a.num_kv_heads + h) * pkv::kBlock) * D;
    if (o0 > 0 && sn > old) {  // re-quantise the block's earlier rows when the scale grows
        for (int r = r0; r < o0; r += RS) requant_row_piece<D>(cache, r, pc, old, sn, rcp);
    }
#pragma unroll
    for (int u = 0; u < MR; ++u) {
        const int r = r0 + u * RS;
        if (r < len)
            *reinterpret_cast<uint2*>(cache + size_t(o0 + r) * D + 8 * pc) = quant8<false>(x[u], nullptr, sn, rcp);
    }
    if (threadIdx.x == 0) *scale = sn;
}

template <int D, bool F32>
void launch_quant(const QuantArgs& a, int n_runs, hipStream_t st) {
    const dim3 grid(unsigned(n_runs), unsigned(a.num_kv_heads), 2);
    if (!a.wide) hipLaunchKernelGGL((kv_store_quant_kernel<D, F32, 64>), grid, dim3(64), 0, st, a);
    else hipLaunchKernelGGL((kv_store_quant_kernel<D, F32, 512>), grid, dim3(512), 0, st, a);
}

}  // namespace

extern "C" int pkv_kv_store_quant(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                                  int32_t new_dtype, const int32_t* slot_mapping, int32_t n, const int32_t* runs,
                                  int32_t n_runs, int32_t max_run, void* k_cache, void* v_cache, float* k_scale,
                                  float* v_scale, void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(desc->kv_dtype == PKV_I8, PKV_ERR_UNSUPPORTED, "the quantising store writes int8 caches only");
    PKV_REQUIRE(new_dtype == PKV_BF16 || new_dtype == PKV_F32, PKV_ERR_UNSUPPORTED,
                "new rows must be bf16 or f32 (dtype %d)", new_dtype);
    PKV_REQUIRE(n >= 0 && n_runs >= 0 && n_runs <= n, PKV_ERR_INVALID, "n = %d, n_runs = %d", n, n_runs);
    PKV_REQUIRE(desc->num_kv_heads <= 65535, PKV_ERR_UNSUPPORTED, "num_kv_heads must be at most 65535");
    if (n_runs == 0) return PKV_OK;
    PKV_REQUIRE(max_run >= 1 && max_run <= pkv::kBlock, PKV_ERR_INVALID, "max_run = %d (1..256)", max_run);
    PKV_REQUIRE(k_new && v_new && slot_mapping && runs && k_cache && v_cache && k_scale && v_scale,
                PKV_ERR_INVALID, "NULL pointer");
    const uintptr_t mis = uintptr_t(k_new) | uintptr_t(v_new) | uintptr_t(k_cache) | uintptr_t(v_cache);
    PKV_REQUIRE((mis & 15) == 0, PKV_ERR_INVALID, "K/V pointers must be 16-byte aligned");
    QuantArgs a{};
    a.wide = max_run > 16;  // eight wavefronts per run once a run has more than 16 rows
    a.k_new = static_cast<const char*>(k_new);
    a.v_new = static_cast<const char*>(v_new);
    a.slots = slot_mapping;
    a.runs = runs;
    a.k_cache = static_cast<int8_t*>(k_cache);
    a.v_cache = static_cast<int8_t*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.num_kv_heads = desc->num_kv_heads;
    a.n = n;
    a.pool_slots = int64_t(desc->num_blocks) * pkv::kBlock;
    a.check = pkv::device_checks();
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool f32 = new_dtype == PKV_F32;
    if (desc->head_dim == 64) f32 ? launch_quant<64, true>(a, n_runs, st) : launch_quant<64, false>(a, n_runs, st);
    else f32 ? launch_quant<128, true>(a, n_runs, st) : launch_quant<128, false>(a, n_runs, st);
    hipError_t e = hipGetLastError();
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "quantising store launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

int pkv::read_error_kv_store(void* stream, int32_t* out) { return read_clear_error(stream, out); }
