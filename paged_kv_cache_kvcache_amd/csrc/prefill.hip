// Varlen paged prefill attention for gfx950 on bf16 MFMA.
//
// The pages describe the full-computation (prefill) phase running FlashAttention-2 style attention
// (intelliparadigm.com Nano-vLLM article, §7.2 关键优化点) over varlen sequences in the paged cache
// ("Nano-vLLM性能调优实战", §2.2 缓存复用策略), with new tokens batched up to a token budget
// ("Nano-vLLM性能调优实战", §3.2 关键调度参数) and cached prefixes reused (ocdem.com nano-vllm
// article, §2.1).  The kernel below is this library's own design for CDNA4.
//
// Work decomposition
//   One workgroup (4 wavefronts) per (sequence, query tile, KV head).  The G = Hq/Hkv query heads
//   that read one KV head are stacked into 128 MFMA rows: a query tile holds QT = 128/G new tokens
//   of all G heads, so every K/V tile staged in LDS serves all of them.  Wavefront w owns rows
//   32w..32w+31 (row rho -> head rho / QT, token rho % QT).  Tiles are visited last-first within a
//   sequence so the longest causal rows start first.
//
// Per 64-key tile (double-buffered in LDS, next tile's global loads in flight during compute):
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T kept in registers.
//                   The accumulator layout puts one query per lane column, 16 keys per lane, and
//                   the other 16 keys of that query in lane ^ 32: the softmax max/sum of a query
//                   needs a single cross-lane swap.
//   online softmax  log2 domain, causal mask by absolute position (bottom-right aligned).
//   O^T += V^T P^T  A = V^T from LDS, B = P^T converted to bf16 straight from the S accumulators.
//                   V is stored transposed in LDS with the keys of each 16-key group permuted
//                   (bits 2 and 3 of the key index swapped) so that the 8 keys a lane needs for the
//                   MFMA operand are contiguous and match the keys its S values belong to.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>

#include "pkv_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kRows = 128;  // MFMA query rows per workgroup (tokens x heads)
constexpr int kKT = 64;     // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;

struct PrefillArgs {
    const uint16_t* q;
    const char* k_cache;
    const char* v_cache;
    const int32_t* cu_seqlens_q;
    const int32_t* seqlens_k;
    const int32_t* block_tables;
    uint16_t* out;
    int32_t B;
    int32_t max_blocks;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t causal;
    float scale_log2;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// Position of key i (0..63) of a tile in the transposed V rows: bits 2 and 3 swapped.
__device__ __forceinline__ int vpos(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int D, int G>
__global__ __launch_bounds__(kThreads, 2) void prefill_kernel(PrefillArgs a) {
    constexpr int QT = kRows / G;       // new tokens per workgroup
    constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;          // 32-row tiles of O^T
    constexpr int KP = D * 2 + 16;      // LDS pitch of a K row (bytes)
    constexpr int VP = kKT * 2 + 16;    // LDS pitch of a transposed V row (bytes)
    constexpr int KBYTES = kKT * KP;
    constexpr int BUF = KBYTES + D * VP;
    constexpr int CPR = D / 8;          // 16-byte pieces per K/V row
    constexpr int KLOADS = kKT * CPR / kThreads;  // K pieces per thread
    __shared__ __attribute__((aligned(16))) char lds[2][BUF];

    // ---- which (sequence, query tile) this workgroup owns
    const int g = blockIdx.y;
    const int x = blockIdx.x;
    int b = -1, tile = 0, nq = 0, start = 0;
    for (int s = 0; s < a.B; ++s) {
        const int n = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
        const int T = (n + QT - 1) / QT;
        if (x < start + T) {
            b = s;
            tile = T - 1 - (x - start);
            nq = n;
            break;
        }
        start += T;
    }
    if (b < 0) return;

    const int Lk = a.seqlens_k[b];
    const int qrow0 = a.cu_seqlens_q[b];
    const int q0 = tile * QT;
    const int nqt = min(QT, nq - q0);
    const int pos0 = Lk - nq + q0;  // absolute position of token q0
    const int kv_len = a.causal ? min(Lk, pos0 + nqt) : Lk;
    const int ntiles = (kv_len + kKT - 1) / kKT;

    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, col = lane & 31, h = lane >> 5;
    const int rho = 32 * w + col;
    const int j = rho / QT, t = rho % QT;
    const bool col_ok = t < nqt;
    const int P = a.causal ? min(pos0 + t, kv_len - 1) : kv_len - 1;  // last key this column sees
    // last key any column of this wavefront sees (for skipping fully masked tiles)
    int pw = P;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) pw = max(pw, __shfl_xor(pw, o, 64));
    const int pw_max = __builtin_amdgcn_readfirstlane(pw);

    // ---- Q^T operand: column col = query row, 8 consecutive d per k-step
    bf16x8_t qb[KS];
    {
        const int tq = min(t, nqt - 1);
        const uint16_t* qp = a.q + (size_t(qrow0 + q0 + tq) * a.num_q_heads + g * G + j) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 v = col_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
            qb[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks;
    const size_t head_off = size_t(g) * pkv::kBlock;

    // ---- global -> register staging of one K/V tile
    uint4 kreg[KLOADS], vreg[4];
    const bool v_thread = tid < 16 * CPR;   // threads that move a 4-key x 8-d piece of V
    const int vkg = tid / CPR, vc = tid % CPR;
    auto gload = [&](int kt) {
        const int key0 = kt * kKT;
        const int64_t phys = bt[key0 / pkv::kBlock];
        const size_t row0 = (size_t(phys) * a.num_kv_heads) * pkv::kBlock + head_off + key0 % pkv::kBlock;
        const uint4* kg = reinterpret_cast<const uint4*>(a.k_cache + row0 * D * 2);
        const uint4* vg = reinterpret_cast<const uint4*>(a.v_cache + row0 * D * 2);
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int p = tid + kThreads * r;
            const int row = p / CPR;
            kreg[r] = (key0 + row < kv_len) ? kg[p] : make_uint4(0, 0, 0, 0);
        }
        if (v_thread) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int row = 4 * vkg + k;
                vreg[k] = (key0 + row < kv_len) ? vg[row * CPR + vc] : make_uint4(0, 0, 0, 0);
            }
        }
    };
    // ---- register -> LDS (K row-major, V transposed with permuted keys)
    auto lstore = [&](int buf) {
        char* Ks = lds[buf];
        char* Vt = lds[buf] + KBYTES;
#pragma unroll
        for (int r = 0; r < KLOADS; ++r) {
            const int p = tid + kThreads * r;
            *reinterpret_cast<uint4*>(Ks + (p / CPR) * KP + (p % CPR) * 16) = kreg[r];
        }
        if (v_thread) {
            const int pos = vpos(4 * vkg);
            const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
            const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
            const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
            const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int s = 0; s < 2; ++s) {
                    const uint32_t sel = s ? 0x07060302u : 0x05040100u;
                    uint2 pr;
                    pr.x = __builtin_amdgcn_perm(w1[m], w0[m], sel);
                    pr.y = __builtin_amdgcn_perm(w3[m], w2[m], sel);
                    *reinterpret_cast<uint2*>(Vt + (8 * vc + 2 * m + s) * VP + pos * 2) = pr;
                }
            }
        }
    };

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    if (ntiles > 0) gload(0);
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        lstore(buf);
        __syncthreads();
        if (kt + 1 < ntiles) gload(kt + 1);
        if (kt * kKT > pw_max) continue;  // every key of this tile is masked for this wavefront

        const char* Ks = lds[buf];
        const char* Vt = lds[buf] + KBYTES;
        // S^T = K Q^T for keys 32mt..32mt+31
        f32x16_t s[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mt][i] = 0.f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8_t ka =
                    *reinterpret_cast<const bf16x8_t*>(Ks + (32 * mt + col) * KP + (16 * ks + 8 * h) * 2);
                s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qb[ks], s[mt], 0, 0, 0);
            }
        }
        // scale, mask, tile max
        float tmax = kNegInf;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = kt * kKT + 32 * mt + 8 * (i / 4) + 4 * h + (i % 4);
                const float v = key <= P ? s[mt][i] * a.scale_log2 : kNegInf;
                s[mt][i] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float mn = fmaxf(m_run, tmax);  // finite: key 0 is visible to every column
        const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
        m_run = mn;
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = __builtin_amdgcn_exp2f(s[mt][i] - mn);
                s[mt][i] = p;
                psum += p;
            }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
        // O^T += V^T P^T
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                uint4 pw4;
                pw4.x = pack_bf16x2(s[mt][8 * kk + 0], s[mt][8 * kk + 1]);
                pw4.y = pack_bf16x2(s[mt][8 * kk + 2], s[mt][8 * kk + 3]);
                pw4.z = pack_bf16x2(s[mt][8 * kk + 4], s[mt][8 * kk + 5]);
                pw4.w = pack_bf16x2(s[mt][8 * kk + 6], s[mt][8 * kk + 7]);
                const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pw4);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(
                        Vt + (32 * dt + col) * VP + (32 * mt + 16 * kk + 8 * h) * 2);
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, o[dt], 0, 0, 0);
                }
            }
        }
    }

    // ---- normalise and write this column's row: d = 32dt + 8(i/4) + 4h + i%4
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (!col_ok) return;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* op = a.out + (size_t(qrow0 + q0 + t) * a.num_q_heads + g * G + j) * D + 4 * h;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            uint2 v;
            v.x = pack_bf16x2(o[dt][4 * i4 + 0] * inv, o[dt][4 * i4 + 1] * inv);
            v.y = pack_bf16x2(o[dt][4 * i4 + 2] * inv, o[dt][4 * i4 + 3] * inv);
            *reinterpret_cast<uint2*>(op + 32 * dt + 8 * i4) = v;
        }
}

template <int D, int G>
hipError_t launch(const PrefillArgs& a, int total_q, hipStream_t st) {
    constexpr int QT = kRows / G;
    const long tiles = (long(total_q) + QT - 1) / QT + a.B;
    hipLaunchKernelGGL((prefill_kernel<D, G>), dim3(unsigned(tiles), a.num_kv_heads), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_g(const PrefillArgs& a, int total_q, int G, hipStream_t st) {
    switch (G) {
        case 1: return launch<D, 1>(a, total_q, st);
        case 2: return launch<D, 2>(a, total_q, st);
        case 4: return launch<D, 4>(a, total_q, st);
        case 8: return launch<D, 8>(a, total_q, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

extern "C" int pkv_paged_attn_prefill(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                      const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                      int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks, float softmax_scale, int32_t causal, void* out,
                                      void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(desc->kv_dtype == PKV_BF16, PKV_ERR_UNSUPPORTED, "prefill supports bf16 caches only");
    const int Hkv = desc->num_kv_heads, D = desc->head_dim;
    PKV_REQUIRE(B >= 0 && Hq > 0 && total_q >= 0 && max_seqlen_q >= 0 && max_seqlen_k >= 0 && max_blocks >= 0,
                PKV_ERR_INVALID, "bad shape (B=%d, Hq=%d, total_q=%d, max_seqlen_q=%d, max_seqlen_k=%d)", B, Hq,
                total_q, max_seqlen_q, max_seqlen_k);
    PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
    const int G = Hq / Hkv;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, PKV_ERR_UNSUPPORTED,
                "query group size %d (Hq/Hkv): supported 1, 2, 4, 8", G);
    PKV_REQUIRE(int64_t(max_blocks) * pkv::kBlock >= max_seqlen_k, PKV_ERR_INVALID,
                "max_blocks %d cannot hold max_seqlen_k %d", max_blocks, max_seqlen_k);
    PKV_REQUIRE(max_seqlen_q <= max_seqlen_k || !causal, PKV_ERR_INVALID,
                "causal prefill needs max_seqlen_q (%d) <= max_seqlen_k (%d)", max_seqlen_q, max_seqlen_k);
    PKV_REQUIRE(Hkv <= 65535, PKV_ERR_UNSUPPORTED, "Hkv must be at most 65535");
    PKV_REQUIRE(std::isfinite(softmax_scale), PKV_ERR_INVALID, "softmax_scale is not finite");
    if (B == 0 || total_q == 0) return PKV_OK;
    PKV_REQUIRE(q && cu_seqlens_q && seqlens_k && k_cache && v_cache && block_tables && out, PKV_ERR_INVALID,
                "NULL pointer");
    const uintptr_t mis = uintptr_t(q) | uintptr_t(k_cache) | uintptr_t(v_cache) | uintptr_t(out);
    PKV_REQUIRE((mis & 15) == 0, PKV_ERR_INVALID, "q, caches and out must be 16-byte aligned");
    PrefillArgs a{};
    a.q = static_cast<const uint16_t*>(q);
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.cu_seqlens_q = cu_seqlens_q;
    a.seqlens_k = seqlens_k;
    a.block_tables = block_tables;
    a.out = static_cast<uint16_t*>(out);
    a.B = B;
    a.max_blocks = max_blocks;
    a.num_kv_heads = Hkv;
    a.num_q_heads = Hq;
    a.causal = causal != 0;
    a.scale_log2 = softmax_scale * kLog2e;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const hipError_t e = D == 64 ? launch_g<64>(a, total_q, G, st) : launch_g<128>(a, total_q, G, st);
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}
