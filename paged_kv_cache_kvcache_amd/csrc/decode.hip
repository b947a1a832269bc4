// Paged decode attention for gfx950 (one query token per sequence).
//
// The pages name flash_attn_with_kvcache as the attention over the cache ("Nano-vLLM性能调优实战",
// §2.2 缓存复用策略) and a max_splits knob that trades latency for throughput (intelliparadigm.com
// Nano-vLLM article, closing paragraph after §8).  Everything below is this library's own design
// for CDNA4; decode streams every KV byte once, so it is an HBM-bandwidth problem and uses no MFMA.
//
// Work decomposition
//   One workgroup (4 wavefronts of 64 lanes) per (sequence, KV head, split), launched in the
//   caller's sequence order (pkv_decode_launch_order: longest contexts first, or balanced per CU
//   when the whole launch is resident at once).  A split is a run of
//   blocks_per_split 256-token blocks.  Inside a block, wavefront w owns tokens 64w..64w+63 (a
//   "tile"), so every wavefront walks the split's blocks with its own independent online-softmax
//   state and no barrier until the end.
//
// Lane layout inside a wavefront (for all dtypes and head_dim 64/128)
//   lane = 16 r + c.  Lane group r (16 lanes) reads rows 4i + r of the tile (i = 0..15), lane c
//   holds elements c*E .. c*E+E-1 of each row, E = head_dim / 16.  Load i of the four groups thus
//   covers four consecutive rows: one contiguous run of 4 * row_bytes per instruction.
//   The G query heads that share the KV head live in registers (E elements per head per lane).
//   Tiles are read through a buffer descriptor per tile whose range ends at the last valid row
//   (rows past the context end read as zeros).  The next block's K tile is requested as soon as
//   the current scores are formed, and each block's V tile at the top of its step, so a
//   wavefront has loads in flight during its own arithmetic.
//
// Scores
//   Each lane forms 16 partial dot products per head (one per row it read).  A 4-step
//   transpose-reduction over the 16 lanes of a group (DPP row_mirror, row_half_mirror, quad
//   permutes) halves the number of live values per step and leaves lane c holding the full score
//   of row 4c + r: 15 exchanges per head instead of 64 for row-by-row butterflies.
//
// Softmax
//   Log2 domain (scale * log2 e folded in, v_exp_f32).  Each 16-lane group keeps its own running
//   max m (group-uniform), a per-lane partial denominator l and an accumulator acc[G][E] for its
//   rows.  P * V broadcasts each row's probability from its owner lane with DPP row_newbcast.
//   At the end the 16 (group, wavefront) states are merged through LDS; a multi-split sequence
//   writes (m, l, acc) to the workspace and the reduce kernel merges the splits by log-sum-exp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <type_traits>
#include <vector>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 64;  // tokens per wavefront per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------- DPP helpers
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowMirror = 0x140;     // lane j <-> 15 - j within a row of 16
constexpr int kRowHalfMirror = 0x141; // lane j <-> 7 - j within each half row
constexpr int kRowNewBcast = 0x150;   // + n: broadcast lane n of each row (gfx90a and later)

// Max over the 16 lanes of a row, result in every lane of the row.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<kQuadXor1>(x));
    x = fmaxf(x, dpp<kQuadXor2>(x));
    x = fmaxf(x, dpp<kRowHalfMirror>(x));
    x = fmaxf(x, dpp<kRowMirror>(x));
    return x;
}

// One transpose-reduction step: partners differ in bit BIT of the lane's row position; each keeps
// the half of the values whose index bit matches its own and adds its partner's copy of that half.
template <int CTRL, int HALF>
__device__ __forceinline__ void treduce_step(float* x, bool upper) {
#pragma unroll
    for (int k = 0; k < HALF; ++k) {
        const float send = upper ? x[k] : x[k + HALF];
        const float keep = upper ? x[k + HALF] : x[k];
        x[k] = keep + dpp<CTRL>(send);
    }
}

// x[0..15] are per-lane partial sums of rows 0..15; returns the full sum of row c (c = lane % 16).
__device__ __forceinline__ float transpose_reduce16(float* x, int c) {
    treduce_step<kRowMirror, 8>(x, (c >> 3) & 1);
    treduce_step<kRowHalfMirror, 4>(x, (c >> 2) & 1);
    treduce_step<kQuadXor2, 2>(x, (c >> 1) & 1);
    treduce_step<kQuadXor1, 1>(x, c & 1);
    return x[0];
}

template <int N>
__device__ __forceinline__ float bcast_row(float x) {
    return dpp<kRowNewBcast + N>(x);
}

// x of lane 2u of each row of 16, in every lane of the row (u uniform and unrolled: DPP lane selects
// are immediates).
__device__ __forceinline__ uint32_t bcast_row_even(uint32_t x, int u) {
    const float f = __uint_as_float(x);
    switch (u) {
        case 0: return __float_as_uint(bcast_row<0>(f));
        case 1: return __float_as_uint(bcast_row<2>(f));
        case 2: return __float_as_uint(bcast_row<4>(f));
        case 3: return __float_as_uint(bcast_row<6>(f));
        case 4: return __float_as_uint(bcast_row<8>(f));
        case 5: return __float_as_uint(bcast_row<10>(f));
        case 6: return __float_as_uint(bcast_row<12>(f));
        default: return __float_as_uint(bcast_row<14>(f));
    }
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// f rounded to the nearest bf16 value (ties to even), as fp32.
__device__ __forceinline__ float round_bf16(float f) { return bf16_lo(pack_bf16x2(f, 0.f)); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t((u >> 16) | 0x40);  // quiet NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}

// ------------------------------------------------------------------------------ dtype traits
// A lane's E-element piece of one row is W dwords.
template <int DT, int D>
struct Traits;

template <int D>
struct Traits<PKV_F32, D> {
    static constexpr int E = D / 16;
    static constexpr int W = E;
    static constexpr int kRowBytes = D * 4;
    using QReg = float[E];
    __device__ static void load_q(QReg& q, const void* qp, size_t off) {
        const float* p = static_cast<const float*>(qp) + off;
#pragma unroll
        for (int e = 0; e < E; ++e) q[e] = p[e];
    }
    __device__ static float dot(const QReg& q, const uint32_t* w) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(q[e], __uint_as_float(w[e]), s);
        return s;
    }
    __device__ static void unpack(const uint32_t* w, float* v) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = __uint_as_float(w[e]);
    }
};

template <int D>
struct Traits<PKV_BF16, D> {
    static constexpr int E = D / 16;
    static constexpr int W = E / 2;
    static constexpr int kRowBytes = D * 2;
    using QReg = uint32_t[W];  // packed bf16 pairs
    __device__ static void load_q(QReg& q, const void* qp, size_t off) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(qp) + off);
#pragma unroll
        for (int k = 0; k < W; ++k) q[k] = p[k];
    }
    __device__ static float dot(const QReg& q, const uint32_t* w) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < W; ++k)
            s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q[k]),
                                                __builtin_bit_cast(bf16x2_t, w[k]), s, false);
        return s;
    }
    __device__ static void unpack(const uint32_t* w, float* v) {
#pragma unroll
        for (int k = 0; k < W; ++k) {
            v[2 * k] = bf16_lo(w[k]);
            v[2 * k + 1] = bf16_hi(w[k]);
        }
    }
};

template <int D>
struct Traits<PKV_I8, D> {
    static constexpr int E = D / 16;
    static constexpr int W = E / 4;
    static constexpr int kRowBytes = D;
    using QReg = float[E];  // bf16 query widened to fp32
    __device__ static void load_q(QReg& q, const void* qp, size_t off) {
        const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(qp) + off);
#pragma unroll
        for (int k = 0; k < E / 2; ++k) {
            q[2 * k] = bf16_lo(p[k]);
            q[2 * k + 1] = bf16_hi(p[k]);
        }
    }
    __device__ static float code(uint32_t w, int byte) {
        return float(int32_t(w << (24 - 8 * byte)) >> 24);
    }
    __device__ static float dot(const QReg& q, const uint32_t* w) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) s = fmaf(q[e], code(w[e / 4], e % 4), s);
        return s;
    }
    __device__ static void unpack(const uint32_t* w, float* v) {
#pragma unroll
        for (int e = 0; e < E; ++e) v[e] = code(w[e / 4], e % 4);
    }
};

// acc[j] += sum_i p_j(row i) v(row i) over the 16 rows of a lane group, for bf16 V: rows 2u and
// 2u + 1 go together through v_dot2_f32_bf16, whose operands are the two rows' bf16
// probabilities (p holds each lane's own row, already bf16 values) and the two rows' values of one
// d, gathered by one byte permute.  The fp32 path spends two FMAs and the widening of both values
// on the same pair.
template <int G, int E, int W>
__device__ __forceinline__ void pv_bf16_pairs(float (&acc)[G][E], const uint32_t (&vw)[16][W], const float (&p)[G]) {
    uint32_t pp[G];
#pragma unroll
    for (int j = 0; j < G; ++j) pp[j] = pack_bf16x2(p[j], dpp<kQuadXor1>(p[j]));  // even lane c: rows c, c + 1
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        uint32_t lo[W], hi[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            lo[k] = __builtin_amdgcn_perm(vw[2 * u + 1][k], vw[2 * u][k], 0x05040100u);  // d = 2k of both rows
            hi[k] = __builtin_amdgcn_perm(vw[2 * u + 1][k], vw[2 * u][k], 0x07060302u);  // d = 2k + 1
        }
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const bf16x2_t pu = __builtin_bit_cast(bf16x2_t, bcast_row_even(pp[j], u));
#pragma unroll
            for (int k = 0; k < W; ++k) {
                acc[j][2 * k] = __builtin_amdgcn_fdot2_f32_bf16(pu, __builtin_bit_cast(bf16x2_t, lo[k]),
                                                               acc[j][2 * k], false);
                acc[j][2 * k + 1] = __builtin_amdgcn_fdot2_f32_bf16(pu, __builtin_bit_cast(bf16x2_t, hi[k]),
                                                                   acc[j][2 * k + 1], false);
            }
        }
    }
}

template <int W>
__device__ __forceinline__ void load_piece(const char* p, uint32_t* w) {
    // K/V is streamed once: nontemporal loads (measured ~12% more read bandwidth on MI355X)
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    if constexpr (W == 1) {
        w[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    } else if constexpr (W == 2) {
        const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
        for (int k = 0; k < W; k += 4) {
            const u32x4_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p) + k / 4);
            w[k] = x.x; w[k + 1] = x.y; w[k + 2] = x.z; w[k + 3] = x.w;
        }
    }
}

// Buffer-descriptor form of load_piece: W dwords at byte offset off of the descriptor's range,
// zeros where the range ends before them; nontemporal like load_piece.  Word 3 of a gfx9 buffer
// descriptor: 32-bit data format, no swizzle, no index stride.
constexpr int kBufferWord3 = 0x00020000;
constexpr int kNontemporal = 2;  // cache-policy bit of the buffer-load builtins: nt
constexpr int kWaitVm0 = 0x0F70;  // s_waitcnt vmcnt(0), expcnt and lgkmcnt left alone
template <int W>
__device__ __forceinline__ void load_piece_buf(__amdgpu_buffer_rsrc_t rs, int off, uint32_t* w) {
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    if constexpr (W == 1) {
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kNontemporal);
    } else if constexpr (W == 2) {
        const u32x2_t x = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNontemporal);
        w[0] = x.x; w[1] = x.y;
    } else {
#pragma unroll
        for (int k = 0; k < W; k += 4) {
            const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 4 * k, 0, kNontemporal);
            w[k] = x.x; w[k + 1] = x.y; w[k + 2] = x.z; w[k + 3] = x.w;
        }
    }
}

struct DecodeArgs {
    const void* q;
    const char* k_cache;
    const char* v_cache;
    const float* k_scale;
    const float* v_scale;
    const int32_t* block_tables;
    const int32_t* context_lens;
    const int32_t* seq_order;  // optional launch order of the sequences (a permutation of 0..B-1)
    void* out;
    float* ws_acc;  // [B][Hq][S][D]
    float* ws_ml;   // [B][Hq][S][2]  (max in log2 units, denominator)
    // optional store of each sequence's new token before attending (pkv_decode_store_attend)
    const int32_t* new_slots;  // [B], -1: nothing to store
    const char* k_new;         // [B][Hkv][D] in the cache dtype
    const char* v_new;
    const float* k_scale_new;  // int8: [B][Hkv]
    const float* v_scale_new;
    char* k_store;             // writable views of the caches and (int8) scales
    char* v_store;
    float* k_scale_store;
    float* v_scale_store;
    int32_t max_blocks;
    int32_t max_context_len;  // the host's bound on every context length (the split plan covers it)
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t splits;
    int32_t blocks_per_split;
    int32_t window;    // > 0: sliding window, the last `window` keys of each sequence
    float scale_log2;  // softmax_scale * log2(e)
    int32_t B;
    int32_t num_blocks;
    int64_t pool_slots;  // num_blocks * 256
    int32_t check;       // launch the instantiation that validates order, lengths, block ids, new slots
    // grouped decode (decode_group_kernel): groups of group_size consecutive sequences whose first
    // shared_lens[group] keys sit in the same physical blocks
    int32_t group_size;
    const int32_t* shared_lens;
    int32_t max_shared_len;  // grouped decode over splits: the bound on every shared_lens entry
    int32_t reduce_all;      // the reduce merges every split slot of a row (grouped decode over splits)
};

// Device-data checks of one (sequence, split): every block id it reads is in the pool, and so is
// the new token's slot when this split stores it.  Wavefront-uniform (every wavefront of the
// workgroup computes the same), so a workgroup that fails leaves as a whole.
__device__ bool decode_split_inputs_ok(const DecodeArgs& a, int b, int blk0, int blk1, int ctx) {
    const int lane = threadIdx.x & 63;
    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks;
    for (int e0 = blk0; e0 < blk1; e0 += 64) {
        const int e = e0 + lane;
        const int v = bt[min(e, blk1 - 1)];  // clamped, so the load needs no exec mask
        const uint64_t bad = __ballot(e < blk1 && (v < 0 || v >= a.num_blocks));
        if (bad != 0) {
            const int first = __shfl(v, __ffsll(static_cast<unsigned long long>(bad)) - 1, 64);
            if (threadIdx.x == 0) record_error(pkv::kErrBlock, b, first);
            return false;
        }
    }
    if (a.new_slots != nullptr && ctx > 0) {
        const int bn = (ctx - 1) / pkv::kBlock;
        if (bn >= blk0 && bn < blk1) {
            const int32_t slot = a.new_slots[b];
            if (slot >= a.pool_slots) {
                if (threadIdx.x == 0) record_error(pkv::kErrSlot, b, slot);
                return false;
            }
        }
    }
    return true;
}

// --------------------------------------------------------------------------- split kernel
template <int DT, int D, int G, bool CHECK>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a) {
    using T = Traits<DT, D>;
    constexpr int E = T::E, W = T::W, RB = T::kRowBytes, PB = W * 4;

    const int s = blockIdx.x, g = blockIdx.y;
    const int b = a.seq_order != nullptr ? a.seq_order[blockIdx.z] : int(blockIdx.z);
    if (CHECK && (b < 0 || b >= a.B)) {  // uniform in the workgroup
        if (threadIdx.x == 0 && s == 0 && g == 0) record_error(pkv::kErrSequence, int(blockIdx.z), b);
        return;
    }
    const int ctx = a.context_lens[b];
    if (CHECK && (ctx < 0 || ctx > a.max_context_len)) {
        if (threadIdx.x == 0 && s == 0 && g == 0) record_error(pkv::kErrLength, b, ctx);
        return;
    }
    const int nblk = (ctx + pkv::kBlock - 1) / pkv::kBlock;
    // keys lo..ctx-1 are attended: all of them, or the last `window` (splits start at lo's block)
    const int lo = a.window > 0 ? max(0, ctx - a.window) : 0;
    const int blk0 = lo / pkv::kBlock + s * a.blocks_per_split;
    const int blk1 = min(nblk, blk0 + a.blocks_per_split);
    if (a.splits > 1 && blk0 >= blk1) return;  // empty split: the reduce kernel skips it
    if (CHECK && !decode_split_inputs_ok(a, b, blk0, blk1, ctx)) {
        // a rejected split's partial state is marked (denominator -1), so the reduce leaves this
        // sequence's output unwritten instead of merging whatever the workspace held
        if (a.splits > 1 && threadIdx.x < G)
            a.ws_ml[2 * ((size_t(b) * a.num_q_heads + g * G + threadIdx.x) * a.splits + s) + 1] = -1.f;
        return;
    }

    // ---- the new token of this sequence (position ctx - 1), stored by the workgroup whose split
    // holds its block before any wavefront reads that block; no other workgroup reads it
    if (a.new_slots != nullptr) {
        const int bn = (ctx - 1) / pkv::kBlock;
        const int slot = ctx > 0 && bn >= blk0 && bn < blk1 ? a.new_slots[b] : -1;
        if (slot >= 0) {
            const int64_t pblk = slot / pkv::kBlock, off = slot % pkv::kBlock;
            const size_t dst = ((size_t(pblk) * a.num_kv_heads + g) * pkv::kBlock + off) * RB;
            const size_t src = (size_t(b) * a.num_kv_heads + g) * RB;
            constexpr int NP = RB / 16;  // 16-byte pieces per row
            for (int p = threadIdx.x; p < 2 * NP; p += kThreads) {
                const bool is_v = p >= NP;
                const int pp = is_v ? p - NP : p;
                const uint4 val = reinterpret_cast<const uint4*>((is_v ? a.v_new : a.k_new) + src)[pp];
                reinterpret_cast<uint4*>((is_v ? a.v_store : a.k_store) + dst)[pp] = val;
            }
            if constexpr (DT == PKV_I8) {
                if (threadIdx.x == 0) {
                    a.k_scale_store[pblk * a.num_kv_heads + g] = a.k_scale_new[size_t(b) * a.num_kv_heads + g];
                    a.v_scale_store[pblk * a.num_kv_heads + g] = a.v_scale_new[size_t(b) * a.num_kv_heads + g];
                }
            }
        }
        __syncthreads();  // the stores are complete before any wavefront loads the block
    }

    // the wavefront index is uniform per wavefront: keep it (and the loop bounds) in scalar registers
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane >> 4, c = lane & 15;

    typename T::QReg qr[G];
#pragma unroll
    for (int j = 0; j < G; ++j)
        T::load_q(qr[j], a.q, (size_t(b) * a.num_q_heads + g * G + j) * D + c * E);

    float m[G], l[G], acc[G][E];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        m[j] = kNegInf;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] = 0.f;
    }

    // this split's block table, 64 entries at a time in one VGPR (lane i: entry blk0 + 64 win + i);
    // a block's physical index comes by readlane, with no dependent load per block
    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks;
    int bt_win = 0;
    int btv = blk0 + lane < blk1 ? bt[blk0 + lane] : 0;
    auto phys_block = [&](int blk) {  // blk is uniform
        const int win = (blk - blk0) >> 6;
        if (win != bt_win) {
            bt_win = win;
            const int e = blk0 + 64 * win + lane;
            btv = e < blk1 ? bt[e] : 0;
            // wait here, on the rare reload: a wait at the join would hold every lookup (and the
            // next block's loads behind it) until all loads in flight had landed
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        return __builtin_amdgcn_readlane(btv, (blk - blk0) & 63);
    };

    // Blocks whose quarter w holds valid tokens: blk0 .. blk_end-1 (only the last may be partial).
    const int blk_end = min(blk1, max(blk0, (ctx - w * kTile + pkv::kBlock - 1) / pkv::kBlock));
    // A wavefront's tile of one block: rows 64w..64w+63 of (block, KV head), read through a buffer
    // descriptor whose range ends at the tile's last valid row, so rows past the context end read
    // as zeros with no exec-masked loads.  The per-lane offsets are the same for every tile: only
    // the descriptor (scalar registers) changes, and no load needs a 64-bit address of its own.
    auto tile_rsrc = [&](const char* cache, int64_t phys, int valid) {
        const char* base = cache + ((size_t(phys) * a.num_kv_heads + g) * pkv::kBlock + w * kTile) * RB;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, valid * RB, kBufferWord3);
    };
    const int lane_off = r * RB + c * PB;
    auto load_tile = [&](uint32_t (&dst)[16][W], __amdgpu_buffer_rsrc_t rs) {
        // Opaque copy of the lane offset, so that the compiler folds each row's constant into the
        // load's immediate offset instead of keeping one register per row across the loop.
        int off = lane_off;
        asm volatile("" : "+v"(off));
#pragma unroll
        for (int i = 0; i < 16; ++i) load_piece_buf<W>(rs, off + 4 * i * RB, dst[i]);
    };

    // Block t + 1's K tile is requested as soon as block t's scores are formed (the K registers
    // are free then), and block t's V tile at the top of its step, right after block t - 1's P.V:
    // a wavefront keeps loads in flight through its own arithmetic while holding one K tile and one
    // V tile, as before.  Only K is carried from one step to the next.
    uint32_t kw[16][W], vw[16][W];
    auto tile_valid = [&](int blk) { return min(kTile, ctx - (blk * pkv::kBlock + w * kTile)); };
    int64_t phys = 0;
    int valid = 0;
    // int8: the scales of the block whose K tile is in flight, requested before that tile so that
    // waiting for them never waits for a tile
    float ksn = 1.f, vsn = 1.f;
    auto load_scales = [&](int64_t ph) {
        if constexpr (DT == PKV_I8) {
            ksn = a.k_scale[ph * a.num_kv_heads + g];
            vsn = a.v_scale[ph * a.num_kv_heads + g];
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (blk0 < blk_end) {
        phys = phys_block(blk0);
        valid = tile_valid(blk0);
        load_scales(phys);
        load_tile(kw, tile_rsrc(a.k_cache, phys, valid));
    }
    // One step per block; PF: this step also requests the next block's K tile.  The last step is
    // its own instantiation, so that the wait counts on every path know exactly which loads are in
    // flight.
    auto step = [&](int blk, auto prefetch) __attribute__((always_inline)) {
        constexpr bool PF = decltype(prefetch)::value;
        load_tile(vw, tile_rsrc(a.v_cache, phys, valid));
        float ks = a.scale_log2, vs = 1.f;
        if constexpr (DT == PKV_I8) {
            ks *= ksn;
            vs = vsn;
        }
        const bool row_ok = 4 * c + r < valid && blk * pkv::kBlock + w * kTile + 4 * c + r >= lo;

        float tot[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            float part[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) part[i] = T::dot(qr[j], kw[i]);
            // every lane must take part in the DPP exchanges: reduce first, mask afterwards
            tot[j] = transpose_reduce16(part, c);
            __builtin_amdgcn_sched_barrier(0);  // one head's 16 partial sums live at a time
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (PF) {
            phys = phys_block(blk + 1);
            valid = tile_valid(blk + 1);
            load_scales(phys);
            load_tile(kw, tile_rsrc(a.k_cache, phys, valid));
        }

        float p[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            const float sc = row_ok ? tot[j] * ks : kNegInf;
            const float mn = fmaxf(m[j], row_max16(sc));
            const bool none = mn == kNegInf;
            const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m[j] - mn);
            p[j] = none ? 0.f : __builtin_amdgcn_exp2f(sc - mn);
            if constexpr (DT == PKV_BF16) p[j] = round_bf16(p[j]);  // the probability P.V multiplies
            m[j] = mn;
            l[j] = l[j] * alpha + p[j];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] *= alpha;
            p[j] *= vs;
        }

        if constexpr (DT == PKV_BF16) pv_bf16_pairs(acc, vw, p);
        else
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v[E];
            T::unpack(vw[i], v);
#pragma unroll
            for (int j = 0; j < G; ++j) {
                float pi;
                switch (i) {  // DPP lane selects must be immediates
                    case 0: pi = bcast_row<0>(p[j]); break;
                    case 1: pi = bcast_row<1>(p[j]); break;
                    case 2: pi = bcast_row<2>(p[j]); break;
                    case 3: pi = bcast_row<3>(p[j]); break;
                    case 4: pi = bcast_row<4>(p[j]); break;
                    case 5: pi = bcast_row<5>(p[j]); break;
                    case 6: pi = bcast_row<6>(p[j]); break;
                    case 7: pi = bcast_row<7>(p[j]); break;
                    case 8: pi = bcast_row<8>(p[j]); break;
                    case 9: pi = bcast_row<9>(p[j]); break;
                    case 10: pi = bcast_row<10>(p[j]); break;
                    case 11: pi = bcast_row<11>(p[j]); break;
                    case 12: pi = bcast_row<12>(p[j]); break;
                    case 13: pi = bcast_row<13>(p[j]); break;
                    case 14: pi = bcast_row<14>(p[j]); break;
                    default: pi = bcast_row<15>(p[j]); break;
                }
#pragma unroll
                for (int e = 0; e < E; ++e) acc[j][e] = fmaf(pi, v[e], acc[j][e]);
            }
        }
    };
    for (int blk = blk0; blk + 1 < blk_end; ++blk) step(blk, std::true_type{});
    if (blk0 < blk_end) step(blk_end - 1, std::false_type{});

    // ---- merge the four lane groups of this wavefront, then the four wavefronts through LDS
    __shared__ float s_m[kWaves][G], s_l[kWaves][G];
    __shared__ float s_acc[kWaves][G][D];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float M = fmaxf(m[j], __shfl_xor(m[j], 16, 64));
        M = fmaxf(M, __shfl_xor(M, 32, 64));
        const float f = m[j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[j] - M);
        const float L = wave_sum(l[j] * f);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float x = acc[j][e] * f;
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[j][e] = x;
        }
        if (lane == 0) {
            s_m[w][j] = M;
            s_l[w][j] = L;
        }
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[w][j][c * E + e] = acc[j][e];
        }
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
        const int j = idx / D, d = idx - j * D;
        float M = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, s_m[ww][j]);
        float num = 0.f, den = 0.f;
        if (M != kNegInf) {
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = s_m[ww][j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(s_m[ww][j] - M);
                num += f * s_acc[ww][j][d];
                den += f * s_l[ww][j];
            }
        }
        const int h = g * G + j;
        if (a.splits == 1) {
            const float o = den > 0.f ? num / den : 0.f;
            const size_t oi = (size_t(b) * a.num_q_heads + h) * D + d;
            if constexpr (DT == PKV_F32) static_cast<float*>(a.out)[oi] = o;
            else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
        } else {
            const size_t part = (size_t(b) * a.num_q_heads + h) * a.splits + s;
            a.ws_acc[part * D + d] = num;
            if (d == 0) {
                a.ws_ml[2 * part] = M;
                a.ws_ml[2 * part + 1] = den;
            }
        }
    }
}

// --------------------------------------------------------------------------- split reduce
// out[b][h] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s over the non-empty splits.
// CHECK: a sequence whose length the split kernel rejected, or one of whose splits it rejected,
// keeps its output unwritten (every test below is uniform in the workgroup).
template <int D, bool F32_OUT, bool CHECK>
__global__ __launch_bounds__(D) void decode_reduce_kernel(DecodeArgs a) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int ctx = a.context_lens[b];
    if (CHECK && (ctx < 0 || ctx > a.max_context_len)) return;
    const int nblk = (ctx + pkv::kBlock - 1) / pkv::kBlock;
    const int lo_blk = (a.window > 0 ? max(0, ctx - a.window) : 0) / pkv::kBlock;
    const int active = a.reduce_all ? a.splits
                                    : min(a.splits, (nblk - lo_blk + a.blocks_per_split - 1) / a.blocks_per_split);
    const size_t base = (size_t(b) * a.num_q_heads + h) * a.splits;
    if constexpr (CHECK) {
        for (int s = 0; s < active; ++s)
            if (a.ws_ml[2 * (base + s) + 1] < 0.f) return;
    }
    float M = kNegInf;
    for (int s = 0; s < active; ++s) M = fmaxf(M, a.ws_ml[2 * (base + s)]);
    float num = 0.f, den = 0.f;
    for (int s = 0; s < active; ++s) {
        const float f = __builtin_amdgcn_exp2f(a.ws_ml[2 * (base + s)] - M);
        num += f * a.ws_acc[(base + s) * D + d];
        den += f * a.ws_ml[2 * (base + s) + 1];
    }
    const float o = den > 0.f ? num / den : 0.f;
    const size_t oi = (size_t(b) * a.num_q_heads + h) * D + d;
    if constexpr (F32_OUT) static_cast<float*>(a.out)[oi] = o;
    else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
}

// --------------------------------------------------------------------------- grouped decode
// Forked sequences (parallel sampling, beam search) share every block of their parent (ocdem.com
// nano-vllm article, §2.1).  Group k is the group_size consecutive sequences k*M .. k*M + M - 1,
// whose first shared_lens[k] keys sit in the same physical blocks.  One workgroup per (group, KV
// head) reads those blocks once for all GM = M x Gq query rows (Gq query heads per KV head), then
// each member's remaining keys for its own Gq rows only, and writes the members' outputs: the
// shared keys cross HBM once per group instead of once per member.  The per-block work is that of
// decode_split_kernel (same lane layout, reductions and online softmax), with rows outside the
// member skipped while its own keys are read.  Over splits (blockIdx.x, pkv_paged_attn_decode_
// grouped_split), split s walks shared blocks s*bps .. s*bps + bps - 1, the last split also the
// members' own keys, and each writes its partial state for the split reduce.
template <int DT, int D, int GM, bool CHECK>
__global__ __launch_bounds__(kThreads) void decode_group_kernel(DecodeArgs a) {
    using T = Traits<DT, D>;
    constexpr int E = T::E, W = T::W, RB = T::kRowBytes, PB = W * 4;

    const int g = blockIdx.y, grp = blockIdx.z, split = blockIdx.x;
    const int M = a.group_size, gq = a.num_q_heads / a.num_kv_heads;  // GM == M * gq
    const int b0 = grp * M;
    const int shared = a.shared_lens[grp];
    // partial slot of query row j of this group and split (grouped decode over splits)
    auto part_of = [&](int j) {
        return (size_t(b0 + j / gq) * a.num_q_heads + g * gq + j % gq) * a.splits + split;
    };
    if (CHECK) {  // uniform in the workgroup
        // a rejected group's partial states are marked (denominator -1), so the reduce leaves its
        // outputs unwritten instead of merging whatever the workspace held
        if (a.splits > 1 && threadIdx.x < GM) a.ws_ml[2 * part_of(threadIdx.x) + 1] = -1.f;
        bool ok = shared >= 0 && (a.splits == 1 || shared <= a.max_shared_len);
        int bad = 0, val = shared;
        for (int m = 0; ok && m < M; ++m) {
            const int ctx = a.context_lens[b0 + m];
            if (ctx < shared || ctx > a.max_context_len) {
                ok = false;
                bad = b0 + m;
                val = ctx;
            }
        }
        if (!ok) {
            if (threadIdx.x == 0 && g == 0 && split == 0) record_error(pkv::kErrLength, bad, val);
            return;
        }
        // the shared blocks are one set for every member, and every block read is in the pool
        const int nsh = (shared + pkv::kBlock - 1) / pkv::kBlock;
        const int lane = threadIdx.x & 63;
        for (int m = 0; m < M; ++m) {
            const int32_t* bt = a.block_tables + size_t(b0 + m) * a.max_blocks;
            const int32_t* bt0 = a.block_tables + size_t(b0) * a.max_blocks;
            const int nblk = (a.context_lens[b0 + m] + pkv::kBlock - 1) / pkv::kBlock;
            for (int e0 = 0; e0 < nblk; e0 += 64) {
                const int e = min(e0 + lane, nblk - 1);
                const int v = bt[e];
                const bool differs = e < nsh && v != bt0[e];
                const uint64_t bad_blk = __ballot(v < 0 || v >= a.num_blocks);
                const uint64_t bad_sh = __ballot(differs);
                if (bad_blk != 0 || bad_sh != 0) {
                    const bool blk = bad_blk != 0;
                    const int at = __ffsll(static_cast<unsigned long long>(blk ? bad_blk : bad_sh)) - 1;
                    const int first = __shfl(v, at, 64);
                    if (threadIdx.x == 0 && g == 0 && split == 0)
                        record_error(blk ? pkv::kErrBlock : pkv::kErrShared, b0 + m, blk ? first : e0 + at);
                    return;
                }
            }
        }
    }

    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane >> 4, c = lane & 15;

    // query row j: member j / gq, head g * gq + j % gq
    typename T::QReg qr[GM];
#pragma unroll
    for (int j = 0; j < GM; ++j)
        T::load_q(qr[j], a.q, (size_t(b0 + j / gq) * a.num_q_heads + g * gq + j % gq) * D + c * E);

    float m[GM], l[GM], acc[GM][E];
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        m[j] = kNegInf;
        l[j] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[j][e] = 0.f;
    }

    const size_t lane_off = size_t(r) * RB + size_t(c) * PB;
    // One block of this wavefront's walk: its quarter of keys blk*256 .. blk*256 + 255 below ctx and
    // from lo on, for the rows of member `only` (-1: every row).
    struct Unit {
        int64_t phys;
        int blk, ctx, lo, only;
        bool ok;
    };
    auto load_unit = [&](const Unit& u, uint32_t (&kw)[16][W], uint32_t (&vw)[16][W]) __attribute__((always_inline)) {
        const int valid = min(kTile, u.ctx - (u.blk * pkv::kBlock + w * kTile));
        const size_t tile = ((size_t(u.phys) * a.num_kv_heads + g) * pkv::kBlock + w * kTile) * RB + lane_off;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (4 * i + r < valid) {
                load_piece<W>(a.k_cache + tile + size_t(4 * i) * RB, kw[i]);
            } else {
#pragma unroll
                for (int k = 0; k < W; ++k) kw[i][k] = 0u;
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (4 * i + r < valid) {
                load_piece<W>(a.v_cache + tile + size_t(4 * i) * RB, vw[i]);
            } else {
#pragma unroll
                for (int k = 0; k < W; ++k) vw[i][k] = 0u;
            }
        }
    };
    // Rows of other members take the block's work with every score masked, which leaves their state
    // unchanged: skipping them instead made the compiler spill at eight rows.
    auto attend_unit = [&](const Unit& u, const uint32_t (&kw)[16][W], const uint32_t (&vw)[16][W])
        __attribute__((always_inline)) {
        const int64_t phys = u.phys;
        const int only = u.only;
        const int valid = min(kTile, u.ctx - (u.blk * pkv::kBlock + w * kTile));
        float ks = a.scale_log2, vs = 1.f;
        if constexpr (DT == PKV_I8) {
            ks *= a.k_scale[phys * a.num_kv_heads + g];
            vs = a.v_scale[phys * a.num_kv_heads + g];
        }
        const bool row_ok = 4 * c + r < valid && u.blk * pkv::kBlock + w * kTile + 4 * c + r >= u.lo;
        float p[GM];
#pragma unroll
        for (int j = 0; j < GM; ++j) {
            float part[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) part[i] = T::dot(qr[j], kw[i]);
            const float tot = transpose_reduce16(part, c);
            const bool mine = only < 0 || j / gq == only;
            const float sc = row_ok && mine ? tot * ks : kNegInf;
            const float mn = fmaxf(m[j], row_max16(sc));
            const bool none = mn == kNegInf;
            const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(m[j] - mn);
            p[j] = none ? 0.f : __builtin_amdgcn_exp2f(sc - mn);
            if constexpr (DT == PKV_BF16) p[j] = round_bf16(p[j]);  // the probability P.V multiplies
            m[j] = mn;
            l[j] = l[j] * alpha + p[j];
#pragma unroll
            for (int e = 0; e < E; ++e) acc[j][e] *= alpha;
            p[j] *= vs;
        }
        if constexpr (DT == PKV_BF16) pv_bf16_pairs(acc, vw, p);
        else
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float v[E];
            T::unpack(vw[i], v);
#pragma unroll
            for (int j = 0; j < GM; ++j) {
                float pi;
                switch (i) {  // DPP lane selects must be immediates
                    case 0: pi = bcast_row<0>(p[j]); break;
                    case 1: pi = bcast_row<1>(p[j]); break;
                    case 2: pi = bcast_row<2>(p[j]); break;
                    case 3: pi = bcast_row<3>(p[j]); break;
                    case 4: pi = bcast_row<4>(p[j]); break;
                    case 5: pi = bcast_row<5>(p[j]); break;
                    case 6: pi = bcast_row<6>(p[j]); break;
                    case 7: pi = bcast_row<7>(p[j]); break;
                    case 8: pi = bcast_row<8>(p[j]); break;
                    case 9: pi = bcast_row<9>(p[j]); break;
                    case 10: pi = bcast_row<10>(p[j]); break;
                    case 11: pi = bcast_row<11>(p[j]); break;
                    case 12: pi = bcast_row<12>(p[j]); break;
                    case 13: pi = bcast_row<13>(p[j]); break;
                    case 14: pi = bcast_row<14>(p[j]); break;
                    default: pi = bcast_row<15>(p[j]); break;
                }
#pragma unroll
                for (int e = 0; e < E; ++e) acc[j][e] = fmaf(pi, v[e], acc[j][e]);
            }
        }
    };

    // ---- one walk over this wavefront's blocks: first the shared keys 0 .. shared-1 from member
    // 0's table (64 entries per VGPR, by readlane), then each member's own keys shared .. ctx-1 (a
    // few blocks, one scalar load each)
    const int32_t* bt0 = a.block_tables + size_t(b0) * a.max_blocks;
    const int nsh = (shared + pkv::kBlock - 1) / pkv::kBlock;
    const int first = shared / pkv::kBlock;
    // over splits: split s walks shared blocks s bps .. s bps + bps - 1, and only the last split
    // walks the members' own keys
    const int sb0 = split * a.blocks_per_split;
    const int sb1 = a.splits > 1 ? min(nsh, sb0 + a.blocks_per_split) : nsh;
    int bt_win = sb0 >> 6;
    int btv = 64 * bt_win + lane < nsh ? bt0[64 * bt_win + lane] : 0;
    int mm = -1, nblk = sb0, blk_end = min(sb1, max(sb0, (shared - w * kTile + pkv::kBlock - 1) / pkv::kBlock));
    int wctx = shared, wlo = 0;
    const int32_t* bt = bt0;
    auto next_unit = [&]() __attribute__((always_inline)) {
        Unit u{0, 0, 0, 0, 0, false};
        while (nblk >= blk_end) {  // next member with blocks for this wavefront
            if (mm + 1 >= M || split + 1 < a.splits) return u;
            ++mm;
            wctx = a.context_lens[b0 + mm];
            bt = a.block_tables + size_t(b0 + mm) * a.max_blocks;
            nblk = first;
            blk_end = min((wctx + pkv::kBlock - 1) / pkv::kBlock,
                          max(first, (wctx - w * kTile + pkv::kBlock - 1) / pkv::kBlock));
            wlo = shared;
        }
        if (mm < 0) {
            const int win = nblk >> 6;
            if (win != bt_win) {
                bt_win = win;
                const int e = 64 * win + lane;
                btv = e < nsh ? bt0[e] : 0;
            }
            u.phys = __builtin_amdgcn_readlane(btv, nblk & 63);
        } else {
            u.phys = __builtin_amdgcn_readfirstlane(bt[nblk]);
        }
        u.blk = nblk++;
        u.ctx = wctx;
        u.lo = wlo;
        u.only = mm;
        u.ok = true;
        return u;
    };
    // The next block's K/V loads are issued before this block's arithmetic, so they overlap it:
    // with at most eight rows per group, one workgroup per (group, KV head) often leaves a single
    // wavefront per SIMD, and nothing else would hide the load latency.  Two buffers fit below the
    // register file when a lane's piece of a row is at most 4 dwords.
    constexpr bool kDouble = W <= 4;
    uint32_t ka[16][W], va[16][W];
    Unit cur = next_unit();
    if constexpr (kDouble) {
        uint32_t kb[16][W], vb[16][W];
        if (cur.ok) load_unit(cur, ka, va);
        while (cur.ok) {
            const Unit nxt = next_unit();
            if (nxt.ok) load_unit(nxt, kb, vb);
            attend_unit(cur, ka, va);
            if (!nxt.ok) break;
            cur = next_unit();
            if (cur.ok) load_unit(cur, ka, va);
            attend_unit(nxt, kb, vb);
        }
    } else {
        for (; cur.ok; cur = next_unit()) {
            load_unit(cur, ka, va);
            attend_unit(cur, ka, va);
        }
    }

    // ---- merge the four lane groups of each wavefront, then the four wavefronts through LDS
    __shared__ float s_m[kWaves][GM], s_l[kWaves][GM];
    __shared__ float s_acc[kWaves][GM][D];
#pragma unroll
    for (int j = 0; j < GM; ++j) {
        float Mx = fmaxf(m[j], __shfl_xor(m[j], 16, 64));
        Mx = fmaxf(Mx, __shfl_xor(Mx, 32, 64));
        const float f = m[j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m[j] - Mx);
        const float L = wave_sum(l[j] * f);
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float x = acc[j][e] * f;
            x += __shfl_xor(x, 16, 64);
            x += __shfl_xor(x, 32, 64);
            acc[j][e] = x;
        }
        if (lane == 0) {
            s_m[w][j] = Mx;
            s_l[w][j] = L;
        }
        if (r == 0) {
#pragma unroll
            for (int e = 0; e < E; ++e) s_acc[w][j][c * E + e] = acc[j][e];
        }
    }
    __syncthreads();

    for (int idx = threadIdx.x; idx < GM * D; idx += kThreads) {
        const int j = idx / D, d = idx - j * D;
        float Mx = kNegInf;
#pragma unroll
        for (int ww = 0; ww < kWaves; ++ww) Mx = fmaxf(Mx, s_m[ww][j]);
        float num = 0.f, den = 0.f;
        if (Mx != kNegInf) {
#pragma unroll
            for (int ww = 0; ww < kWaves; ++ww) {
                const float f = s_m[ww][j] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(s_m[ww][j] - Mx);
                num += f * s_acc[ww][j][d];
                den += f * s_l[ww][j];
            }
        }
        if (a.splits > 1) {  // this split's partial state: O and row sum relative to 2^Mx
            const size_t part = part_of(j);
            a.ws_acc[part * D + d] = num;
            if (d == 0) {
                a.ws_ml[2 * part] = Mx;
                a.ws_ml[2 * part + 1] = den;
            }
            continue;
        }
        const float o = den > 0.f ? num / den : 0.f;
        const size_t oi = (size_t(b0 + j / gq) * a.num_q_heads + g * gq + j % gq) * D + d;
        if constexpr (DT == PKV_F32) static_cast<float*>(a.out)[oi] = o;
        else static_cast<uint16_t*>(a.out)[oi] = f32_to_bf16_rne(o);
    }
}

// ------------------------------------------------------------------------------ planning
// Automatic plan: split only until the launch has two workgroups per CU.  Measured on MI355X, a
// launch that already fills the chip twice over (e.g. 64 long sequences x 8 KV heads) runs fastest
// unsplit: splits add partial-state traffic and a second launch, and the longest-first order
// already balances the tail.
int num_cus() {
    constexpr int kDevices = 16;
    static std::atomic<int> cache[kDevices];  // per device, filled on first use
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();  // no device here: plan for MI355X's 256 CUs
        return 256;
    }
    if (dev < kDevices && (n = cache[dev].load(std::memory_order_relaxed)) > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 256;
    }
    if (dev < kDevices) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

void plan(int B, int Hkv, int max_ctx, int max_splits, int* splits, int* bps) {
    const int nblk = std::max(1, (max_ctx + pkv::kBlock - 1) / pkv::kBlock);
    int S;
    if (max_splits > 0) {
        S = std::min(max_splits, nblk);
    } else {
        const long base = std::max(1L, long(B) * Hkv);
        const long target = 2L * num_cus();
        S = int(std::min<long>(nblk, std::max<long>(1, (target + base - 1) / base)));
    }
    *bps = (nblk + S - 1) / S;
    *splits = (nblk + *bps - 1) / *bps;
}

template <int DT, int D, int G>
hipError_t launch(const DecodeArgs& a, int B, hipStream_t st) {
    // device-data checks run in their own instantiation, so the production one is unchanged by them
    const dim3 grid(a.splits, a.num_kv_heads, B);
    if (a.check) hipLaunchKernelGGL((decode_split_kernel<DT, D, G, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((decode_split_kernel<DT, D, G, false>), grid, dim3(kThreads), 0, st, a);
    if (a.splits > 1) {
        if (a.check)
            hipLaunchKernelGGL((decode_reduce_kernel<D, DT == PKV_F32, true>), dim3(a.num_q_heads, B), dim3(D), 0, st, a);
        else
            hipLaunchKernelGGL((decode_reduce_kernel<D, DT == PKV_F32, false>), dim3(a.num_q_heads, B), dim3(D), 0, st,
                               a);
    }
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_g(const DecodeArgs& a, int B, int G, hipStream_t st) {
    switch (G) {
        case 1: return launch<DT, D, 1>(a, B, st);
        case 2: return launch<DT, D, 2>(a, B, st);
        case 4: return launch<DT, D, 4>(a, B, st);
        case 8: return launch<DT, D, 8>(a, B, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch_d(const DecodeArgs& a, int B, int G, int D, hipStream_t st) {
    return D == 64 ? launch_g<DT, 64>(a, B, G, st) : launch_g<DT, 128>(a, B, G, st);
}

// ------------------------------------------------------------------------------ launch order
template <int DT, int D>
const void* split_kernel_g(int G) {
    switch (G) {
        case 1: return reinterpret_cast<const void*>(&decode_split_kernel<DT, D, 1, false>);
        case 2: return reinterpret_cast<const void*>(&decode_split_kernel<DT, D, 2, false>);
        case 4: return reinterpret_cast<const void*>(&decode_split_kernel<DT, D, 4, false>);
        default: return reinterpret_cast<const void*>(&decode_split_kernel<DT, D, 8, false>);
    }
}

template <int DT>
const void* split_kernel_d(int D, int G) {
    return D == 64 ? split_kernel_g<DT, 64>(G) : split_kernel_g<DT, 128>(G);
}

// Workgroups of the production split kernel for (dtype, D, G) that one CU of the current device
// holds at once; 0 when there is no device to ask.  Cached per (device, instantiation).
int resident_per_cu(int dt, int D, int G) {
    constexpr int kDevices = 16;
    static std::atomic<int> cache[kDevices][3][2][4];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int gi = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : 3;
    std::atomic<int>* slot = dev < kDevices ? &cache[dev][dt][D == 128][gi] : nullptr;
    if (slot != nullptr && slot->load() > 0) return slot->load();
    const void* k = dt == PKV_F32 ? split_kernel_d<PKV_F32>(D, G)
                  : dt == PKV_BF16 ? split_kernel_d<PKV_BF16>(D, G) : split_kernel_d<PKV_I8>(D, G);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, kThreads, 0) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        return 0;
    }
    if (slot != nullptr) slot->store(n);
    return n;
}

}  // namespace

extern "C" int pkv_decode_launch_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                                       const int32_t* context_lens, int32_t max_context_len, int32_t max_splits,
                                       int32_t window, int32_t compute_units, int32_t workgroups_per_cu,
                                       int32_t* order) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    const int Hkv = desc->num_kv_heads, D = desc->head_dim;
    PKV_REQUIRE(B >= 0 && Hq > 0 && max_context_len >= 0 && max_splits >= 0 && window >= 0, PKV_ERR_INVALID,
                "bad shape (B=%d, Hq=%d, max_context_len=%d, max_splits=%d, window=%d)", B, Hq, max_context_len,
                max_splits, window);
    PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
    const int G = Hq / Hkv;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, PKV_ERR_UNSUPPORTED,
                "query group size %d (Hq/Hkv): supported 1, 2, 4, 8", G);
    if (B == 0) return PKV_OK;
    PKV_REQUIRE(context_lens && order, PKV_ERR_INVALID, "NULL pointer");
    // one sort key per sequence: work descending in the high half, the index ascending in the low
    // half (so ties keep sequence order)
    std::vector<uint64_t> key(B);
    for (int b = 0; b < B; ++b) {
        PKV_REQUIRE(context_lens[b] >= 0, PKV_ERR_INVALID, "context_lens[%d] = %d", b, context_lens[b]);
        const uint32_t work = uint32_t(window > 0 ? std::min(context_lens[b], window) : context_lens[b]);
        key[b] = (uint64_t(~work) << 32) | uint32_t(b);
    }
    std::sort(key.begin(), key.end());
    std::vector<int32_t> d(B);
    for (int b = 0; b < B; ++b) d[b] = int32_t(key[b] & 0xffffffffu);

    const int cus = compute_units > 0 ? compute_units : num_cus();
    const int per_cu = workgroups_per_cu > 0 ? workgroups_per_cu : resident_per_cu(desc->kv_dtype, D, G);
    PKV_REQUIRE(per_cu > 0, PKV_ERR_HIP, "no device to query the decode kernel's occupancy on");
    const int span = window > 0 ? int(std::min<int64_t>(max_context_len, int64_t(window) + pkv::kBlock - 1))
                                : max_context_len;
    int S, bps;
    plan(B, Hkv, span, max_splits, &S, &bps);
    const int64_t per_seq = int64_t(Hkv) * S;  // a sequence's workgroups are consecutive in the launch
    const int64_t round = std::max<int64_t>(1, cus / per_seq);  // sequences per round of one workgroup per CU
    if (int64_t(B) * per_seq <= int64_t(cus) * per_cu && B > round) {
        // every workgroup is resident from the start, and workgroup i shares its CU with i + cus,
        // i + 2 cus, ...: alternate the direction of successive rounds so that the long contexts of
        // one round share CUs with the short ones of the next
        for (int64_t r = 0; r * round < B; ++r) {
            const int64_t lo = r * round, hi = std::min<int64_t>(B, lo + round);
            if (r & 1) std::reverse(d.begin() + lo, d.begin() + hi);
        }
    }
    std::copy(d.begin(), d.end(), order);
    return PKV_OK;
}

extern "C" int pkv_decode_plan(int32_t B, int32_t num_kv_heads, int32_t max_context_len, int32_t max_splits,
                               int32_t* splits, int32_t* blocks_per_split) {
    PKV_REQUIRE(splits && blocks_per_split, PKV_ERR_INVALID, "NULL argument");
    PKV_REQUIRE(B >= 0 && num_kv_heads > 0 && max_context_len >= 0 && max_splits >= 0, PKV_ERR_INVALID,
                "bad shape (B=%d, Hkv=%d, max_context_len=%d, max_splits=%d)", B, num_kv_heads,
                max_context_len, max_splits);
    plan(B, num_kv_heads, max_context_len, max_splits, splits, blocks_per_split);
    return PKV_OK;
}

extern "C" size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim, int32_t num_kv_heads,
                                             int32_t max_context_len, int32_t max_splits) {
    if (B <= 0 || Hq <= 0 || head_dim <= 0 || num_kv_heads <= 0 || max_context_len < 0 || max_splits < 0)
        return 0;
    int S, bps;
    plan(B, num_kv_heads, max_context_len, max_splits, &S, &bps);
    if (S <= 1) return 0;
    return size_t(B) * Hq * S * (size_t(head_dim) + 2) * sizeof(float);
}

namespace {

struct NewTokens {
    const void* k_new = nullptr;
    const void* v_new = nullptr;
    const float* k_scale_new = nullptr;
    const float* v_scale_new = nullptr;
    const int32_t* slot_mapping = nullptr;
    void* k_cache = nullptr;
    void* v_cache = nullptr;
    float* k_scale = nullptr;
    float* v_scale = nullptr;
};

int decode_impl(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq, const void* k_cache,
                const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* block_tables,
                int32_t max_blocks, const int32_t* context_lens, const int32_t* seq_order, int32_t max_context_len,
                int32_t max_splits, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                const NewTokens* nt, int32_t window, void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    const int Hkv = desc->num_kv_heads, D = desc->head_dim;
    PKV_REQUIRE(B >= 0 && Hq > 0 && max_blocks >= 0 && max_context_len >= 0 && max_splits >= 0,
                PKV_ERR_INVALID, "bad shape (B=%d, Hq=%d, max_blocks=%d, max_context_len=%d, max_splits=%d)",
                B, Hq, max_blocks, max_context_len, max_splits);
    PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
    const int G = Hq / Hkv;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, PKV_ERR_UNSUPPORTED,
                "query group size %d (Hq/Hkv): supported 1, 2, 4, 8", G);
    PKV_REQUIRE(int64_t(max_blocks) * pkv::kBlock >= max_context_len, PKV_ERR_INVALID,
                "max_blocks %d cannot hold max_context_len %d", max_blocks, max_context_len);
    PKV_REQUIRE(B <= 65535 && Hkv <= 65535, PKV_ERR_UNSUPPORTED, "B and Hkv must be at most 65535");
    PKV_REQUIRE(std::isfinite(softmax_scale), PKV_ERR_INVALID, "softmax_scale is not finite");
    PKV_REQUIRE(window >= 0, PKV_ERR_INVALID, "window = %d", window);
    const bool i8 = desc->kv_dtype == PKV_I8;
    PKV_REQUIRE(i8 == (k_scale != nullptr) && i8 == (v_scale != nullptr), PKV_ERR_INVALID,
                "k_scale / v_scale are required for int8 caches and rejected otherwise");
    if (nt != nullptr) {
        PKV_REQUIRE(i8 == (nt->k_scale_new != nullptr) && i8 == (nt->v_scale_new != nullptr), PKV_ERR_INVALID,
                    "k_scale_new / v_scale_new are required for int8 caches and rejected otherwise");
    }
    if (B == 0) return PKV_OK;
    PKV_REQUIRE(q && k_cache && v_cache && block_tables && context_lens && out, PKV_ERR_INVALID, "NULL pointer");
    uintptr_t mis = uintptr_t(q) | uintptr_t(k_cache) | uintptr_t(v_cache) | uintptr_t(out);
    if (nt != nullptr) {
        PKV_REQUIRE(nt->k_new && nt->v_new && nt->slot_mapping, PKV_ERR_INVALID, "NULL new-token pointer");
        mis |= uintptr_t(nt->k_new) | uintptr_t(nt->v_new);
    }
    PKV_REQUIRE((mis & 15) == 0, PKV_ERR_INVALID, "q, caches, new rows and out must be 16-byte aligned");

    DecodeArgs a{};
    a.q = q;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.seq_order = seq_order;
    a.out = out;
    a.max_blocks = max_blocks;
    a.max_context_len = max_context_len;
    a.num_kv_heads = Hkv;
    a.num_q_heads = Hq;
    a.scale_log2 = softmax_scale * kLog2e;
    a.window = window;
    a.B = B;
    a.num_blocks = desc->num_blocks;
    a.pool_slots = int64_t(desc->num_blocks) * pkv::kBlock;
    a.check = pkv::device_checks();
    if (nt != nullptr) {
        a.new_slots = nt->slot_mapping;
        a.k_new = static_cast<const char*>(nt->k_new);
        a.v_new = static_cast<const char*>(nt->v_new);
        a.k_scale_new = nt->k_scale_new;
        a.v_scale_new = nt->v_scale_new;
        a.k_store = static_cast<char*>(nt->k_cache);
        a.v_store = static_cast<char*>(nt->v_cache);
        a.k_scale_store = nt->k_scale;
        a.v_scale_store = nt->v_scale;
    }
    // a window of W keys spans at most ceil((W + 255) / 256) blocks
    const int span = window > 0 ? int(std::min<int64_t>(max_context_len, int64_t(window) + pkv::kBlock - 1))
                                : max_context_len;
    plan(B, Hkv, span, max_splits, &a.splits, &a.blocks_per_split);
    if (a.splits > 1) {
        const size_t need = size_t(B) * Hq * a.splits * (size_t(D) + 2) * sizeof(float);
        PKV_REQUIRE(workspace != nullptr && workspace_bytes >= need, PKV_ERR_SMALL_BUFFER,
                    "decode needs %zu workspace bytes for %d splits, got %zu", need, a.splits, workspace_bytes);
        PKV_REQUIRE((uintptr_t(workspace) & 15) == 0, PKV_ERR_INVALID, "workspace must be 16-byte aligned");
        a.ws_acc = static_cast<float*>(workspace);
        a.ws_ml = a.ws_acc + size_t(B) * Hq * a.splits * D;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (desc->kv_dtype) {
        case PKV_F32: e = launch_d<PKV_F32>(a, B, G, D, st); break;
        case PKV_BF16: e = launch_d<PKV_BF16>(a, B, G, D, st); break;
        default: e = launch_d<PKV_I8>(a, B, G, D, st); break;
    }
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "decode launch failed: %s", hipGetErrorString(e));
    return PKV_OK;
}

template <int DT, int D, int GM>
hipError_t launch_group_gm(const DecodeArgs& a, int n_groups, hipStream_t st) {
    const dim3 grid(unsigned(a.splits), unsigned(a.num_kv_heads), unsigned(n_groups));
    if (a.check) hipLaunchKernelGGL((decode_group_kernel<DT, D, GM, true>), grid, dim3(kThreads), 0, st, a);
    else hipLaunchKernelGGL((decode_group_kernel<DT, D, GM, false>), grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_group_d(const DecodeArgs& a, int n_groups, int GM, hipStream_t st) {
    switch (GM) {
        case 1: return launch_group_gm<DT, D, 1>(a, n_groups, st);
        case 2: return launch_group_gm<DT, D, 2>(a, n_groups, st);
        case 4: return launch_group_gm<DT, D, 4>(a, n_groups, st);
        case 8: return launch_group_gm<DT, D, 8>(a, n_groups, st);
        default: return hipErrorInvalidValue;
    }
}

template <int DT>
hipError_t launch_group(const DecodeArgs& a, int n_groups, int GM, int D, hipStream_t st) {
    return D == 64 ? launch_group_d<DT, 64>(a, n_groups, GM, st) : launch_group_d<DT, 128>(a, n_groups, GM, st);
}

}  // namespace

extern "C" int pkv_paged_attn_decode(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                     const void* k_cache, const void* v_cache, const float* k_scale,
                                     const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                                     const int32_t* context_lens, const int32_t* seq_order,
                                     int32_t max_context_len, int32_t max_splits, float softmax_scale, void* out,
                                     void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                       seq_order, max_context_len, max_splits, softmax_scale, out, workspace, workspace_bytes,
                       nullptr, 0, stream);
}

extern "C" int pkv_paged_attn_decode_window(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                            const void* k_cache, const void* v_cache, const float* k_scale,
                                            const float* v_scale, const int32_t* block_tables,
                                            int32_t max_blocks, const int32_t* context_lens,
                                            const int32_t* seq_order, int32_t max_context_len,
                                            int32_t max_splits, float softmax_scale, int32_t window, void* out,
                                            void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                       seq_order, max_context_len, max_splits, softmax_scale, out, workspace, workspace_bytes,
                       nullptr, window, stream);
}

extern "C" int pkv_decode_store_attend(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                       const void* k_new, const void* v_new, const float* k_scale_new,
                                       const float* v_scale_new, const int32_t* slot_mapping, void* k_cache,
                                       void* v_cache, float* k_scale, float* v_scale, const int32_t* block_tables,
                                       int32_t max_blocks, const int32_t* context_lens, const int32_t* seq_order,
                                       int32_t max_context_len, int32_t max_splits, float softmax_scale, void* out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    NewTokens nt;
    nt.k_new = k_new;
    nt.v_new = v_new;
    nt.k_scale_new = k_scale_new;
    nt.v_scale_new = v_scale_new;
    nt.slot_mapping = slot_mapping;
    nt.k_cache = k_cache;
    nt.v_cache = v_cache;
    nt.k_scale = k_scale;
    nt.v_scale = v_scale;
    return decode_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                       seq_order, max_context_len, max_splits, softmax_scale, out, workspace, workspace_bytes, &nt,
                       0, stream);
}

// ------------------------------------------------------------------ allocation-free decode
// The split partials of pkv_paged_attn_decode_noalloc live in this file-scope array: one copy per
// device, held until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so kernels are given the device address that hipGetSymbolAddress returns for
// the current device, looked up once per device and kept below.
namespace {

constexpr size_t kScratchBytes = size_t(PKV_DECODE_SCRATCH_BYTES);
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];

// *out = the device address of `scratch` on the current device; PKV_OK, or the failure recorded.
int scratch_on_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return pkv::fail(PKV_ERR_HIP, "no current HIP device");
    }
    PKV_REQUIRE(dev >= 0 && dev < kScratchDevices, PKV_ERR_UNSUPPORTED,
                "device %d: the decode scratch is kept for devices 0..%d", dev, kScratchDevices - 1);
    void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (ptr == nullptr) {
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) {
            (void)hipGetLastError();
            return pkv::fail(PKV_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                             hipGetErrorString(e));
        }
        g_scratch_ptr[dev].store(ptr, std::memory_order_release);  // every thread finds the same address
    }
    *out = ptr;
    return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attn_decode_noalloc(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                             const void* k_cache, const void* v_cache, const float* k_scale,
                                             const float* v_scale, const int32_t* block_tables,
                                             int32_t max_blocks, const int32_t* context_lens,
                                             const int32_t* seq_order, int32_t max_context_len,
                                             int32_t max_splits, float softmax_scale, void* out, void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(B >= 0 && Hq > 0 && max_context_len >= 0 && max_splits >= 0, PKV_ERR_INVALID,
                "bad shape (B=%d, Hq=%d, max_context_len=%d, max_splits=%d)", B, Hq, max_context_len, max_splits);
    const size_t need = pkv_decode_workspace_bytes(B, Hq, desc->head_dim, desc->num_kv_heads, max_context_len,
                                                   max_splits);
    PKV_REQUIRE(need <= kScratchBytes, PKV_ERR_SMALL_BUFFER,
                "this decode plan needs %zu bytes of split workspace; the library's fixed scratch holds %zu "
                "(lower max_splits, or call pkv_paged_attn_decode with a workspace)", need, kScratchBytes);
    void* ws = nullptr;
    if (need > 0 && (rc = scratch_on_current_device(&ws)) != PKV_OK) return rc;
    return decode_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                       seq_order, max_context_len, max_splits, softmax_scale, out, ws, need, nullptr, 0, stream);
}

extern "C" int pkv_decode_group_shared_lens(const int32_t* block_tables, int32_t max_blocks,
                                            const int32_t* context_lens, int32_t B, int32_t group_size,
                                            int32_t* shared_lens) {
    PKV_REQUIRE(B >= 0 && max_blocks >= 0 && group_size >= 1, PKV_ERR_INVALID,
                "bad shape (B=%d, max_blocks=%d, group_size=%d)", B, max_blocks, group_size);
    PKV_REQUIRE(B % group_size == 0, PKV_ERR_INVALID, "B %d is not a multiple of group_size %d", B, group_size);
    if (B == 0) return PKV_OK;
    PKV_REQUIRE(block_tables && context_lens && shared_lens, PKV_ERR_INVALID, "NULL pointer");
    for (int b = 0; b < B; ++b)
        PKV_REQUIRE(context_lens[b] >= 0 && int64_t(context_lens[b]) <= int64_t(max_blocks) * pkv::kBlock,
                    PKV_ERR_INVALID, "context_lens[%d] = %d outside 0..%lld", b, context_lens[b],
                    (long long)max_blocks * pkv::kBlock);
    for (int k = 0; k < B / group_size; ++k) {
        const int b0 = k * group_size;
        int len = context_lens[b0];
        for (int m = 1; m < group_size; ++m) len = std::min(len, context_lens[b0 + m]);
        // leading blocks of the shortest context that every member holds at the same entry
        const int nblk = (len + pkv::kBlock - 1) / pkv::kBlock;
        int n = 0;
        for (; n < nblk; ++n) {
            const int32_t blk = block_tables[size_t(b0) * max_blocks + n];
            bool same = true;
            for (int m = 1; m < group_size && same; ++m) same = block_tables[size_t(b0 + m) * max_blocks + n] == blk;
            if (!same) break;
        }
        shared_lens[k] = std::min(len, n * pkv::kBlock);
    }
    return PKV_OK;
}

namespace {

template <int D, bool F32_OUT>
void reduce_all_splits(const DecodeArgs& a, int B, int Hq, bool check, hipStream_t st) {
    if (check) hipLaunchKernelGGL((decode_reduce_kernel<D, F32_OUT, true>), dim3(Hq, B), dim3(D), 0, st, a);
    else hipLaunchKernelGGL((decode_reduce_kernel<D, F32_OUT, false>), dim3(Hq, B), dim3(D), 0, st, a);
}

// Splits of a grouped launch: the shared blocks of the longest shared prefix in at most
// max_splits runs of bps blocks (S = 1: no split).
void group_plan(int32_t max_shared_len, int32_t max_splits, int* S, int* bps) {
    const int nsh = (std::max(0, max_shared_len) + pkv::kBlock - 1) / pkv::kBlock;
    const int want = std::max(1, std::min(max_splits, std::max(1, nsh)));
    *bps = std::max(1, (nsh + want - 1) / want);
    *S = std::max(1, (nsh + *bps - 1) / *bps);
    if (*S == 1) *bps = 0;
}

int grouped_impl(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq, const void* k_cache,
                 const void* v_cache, const float* k_scale, const float* v_scale, const int32_t* block_tables,
                 int32_t max_blocks, const int32_t* context_lens, int32_t max_context_len, int32_t group_size,
                 const int32_t* shared_lens, int32_t max_shared_len, int32_t max_splits, float softmax_scale,
                 void* out, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    const int Hkv = desc->num_kv_heads, D = desc->head_dim;
    PKV_REQUIRE(B >= 0 && Hq > 0 && max_blocks >= 0 && max_context_len >= 0 && group_size >= 1, PKV_ERR_INVALID,
                "bad shape (B=%d, Hq=%d, max_blocks=%d, max_context_len=%d, group_size=%d)", B, Hq, max_blocks,
                max_context_len, group_size);
    PKV_REQUIRE(Hq % Hkv == 0, PKV_ERR_INVALID, "Hq %d is not a multiple of Hkv %d", Hq, Hkv);
    PKV_REQUIRE(B % group_size == 0, PKV_ERR_INVALID, "B %d is not a multiple of group_size %d", B, group_size);
    const int GM = group_size * (Hq / Hkv);
    PKV_REQUIRE(GM == 1 || GM == 2 || GM == 4 || GM == 8, PKV_ERR_UNSUPPORTED,
                "group_size x Hq / Hkv = %d query rows per KV head: supported 1, 2, 4, 8", GM);
    PKV_REQUIRE(int64_t(max_blocks) * pkv::kBlock >= max_context_len, PKV_ERR_INVALID,
                "max_blocks %d cannot hold max_context_len %d", max_blocks, max_context_len);
    PKV_REQUIRE(B / group_size <= 65535 && Hkv <= 65535, PKV_ERR_UNSUPPORTED,
                "at most 65535 groups and 65535 KV heads");
    PKV_REQUIRE(std::isfinite(softmax_scale), PKV_ERR_INVALID, "softmax_scale is not finite");
    const bool i8 = desc->kv_dtype == PKV_I8;
    PKV_REQUIRE(i8 == (k_scale != nullptr) && i8 == (v_scale != nullptr), PKV_ERR_INVALID,
                "k_scale / v_scale are required for int8 caches and rejected otherwise");
    if (B == 0) return PKV_OK;
    PKV_REQUIRE(q && k_cache && v_cache && block_tables && context_lens && shared_lens && out, PKV_ERR_INVALID,
                "NULL pointer");
    const uintptr_t mis = uintptr_t(q) | uintptr_t(k_cache) | uintptr_t(v_cache) | uintptr_t(out);
    PKV_REQUIRE((mis & 15) == 0, PKV_ERR_INVALID, "q, caches and out must be 16-byte aligned");
    DecodeArgs a{};
    a.q = q;
    a.k_cache = static_cast<const char*>(k_cache);
    a.v_cache = static_cast<const char*>(v_cache);
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    a.out = out;
    a.max_blocks = max_blocks;
    a.max_context_len = max_context_len;
    a.num_kv_heads = Hkv;
    a.num_q_heads = Hq;
    a.splits = 1;
    a.scale_log2 = softmax_scale * kLog2e;
    a.B = B;
    a.num_blocks = desc->num_blocks;
    a.pool_slots = int64_t(desc->num_blocks) * pkv::kBlock;
    a.check = pkv::device_checks();
    a.group_size = group_size;
    a.shared_lens = shared_lens;
    int S = 1, bps = 0;
    group_plan(max_shared_len, max_splits, &S, &bps);
    if (S > 1) {
        const size_t need = size_t(B) * Hq * S * (size_t(D) + 2) * sizeof(float);
        PKV_REQUIRE(workspace != nullptr && workspace_bytes >= need, PKV_ERR_SMALL_BUFFER,
                    "%d splits need %zu bytes of workspace, %zu given", S, need, workspace_bytes);
        PKV_REQUIRE((uintptr_t(workspace) & 15) == 0, PKV_ERR_INVALID, "workspace must be 16-byte aligned");
        a.splits = S;
        a.blocks_per_split = bps;
        a.max_shared_len = max_shared_len;
        a.reduce_all = 1;
        a.ws_acc = static_cast<float*>(workspace);
        a.ws_ml = a.ws_acc + size_t(B) * Hq * S * D;
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int ng = B / group_size;
    hipError_t e;
    switch (desc->kv_dtype) {
        case PKV_F32: e = launch_group<PKV_F32>(a, ng, GM, D, st); break;
        case PKV_BF16: e = launch_group<PKV_BF16>(a, ng, GM, D, st); break;
        default: e = launch_group<PKV_I8>(a, ng, GM, D, st); break;
    }
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "grouped decode launch failed: %s", hipGetErrorString(e));
    if (S > 1) {
        const bool f32 = desc->kv_dtype == PKV_F32, chk = a.check != 0;
        if (D == 64) f32 ? reduce_all_splits<64, true>(a, B, Hq, chk, st) : reduce_all_splits<64, false>(a, B, Hq, chk, st);
        else f32 ? reduce_all_splits<128, true>(a, B, Hq, chk, st) : reduce_all_splits<128, false>(a, B, Hq, chk, st);
        e = hipGetLastError();
        PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "grouped decode reduce launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attn_decode_grouped(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                             const void* k_cache, const void* v_cache, const float* k_scale,
                                             const float* v_scale, const int32_t* block_tables,
                                             int32_t max_blocks, const int32_t* context_lens,
                                             int32_t max_context_len, int32_t group_size,
                                             const int32_t* shared_lens, float softmax_scale, void* out,
                                             void* stream) {
    return grouped_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                        max_context_len, group_size, shared_lens, 0, 1, softmax_scale, out, nullptr, 0, stream);
}

extern "C" size_t pkv_decode_grouped_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim,
                                                     int32_t max_shared_len, int32_t max_splits) {
    if (B <= 0 || Hq <= 0 || head_dim <= 0 || max_shared_len < 0 || max_splits < 0) return 0;
    int S, bps;
    group_plan(max_shared_len, max_splits, &S, &bps);
    return S > 1 ? size_t(B) * Hq * S * (size_t(head_dim) + 2) * sizeof(float) : 0;
}

extern "C" int pkv_paged_attn_decode_grouped_split(const pkv_cache_desc* desc, const void* q, int32_t B,
                                                   int32_t Hq, const void* k_cache, const void* v_cache,
                                                   const float* k_scale, const float* v_scale,
                                                   const int32_t* block_tables, int32_t max_blocks,
                                                   const int32_t* context_lens, int32_t max_context_len,
                                                   int32_t group_size, const int32_t* shared_lens,
                                                   int32_t max_shared_len, int32_t max_splits, float softmax_scale,
                                                   void* out, void* workspace, size_t workspace_bytes,
                                                   void* stream) {
    PKV_REQUIRE(max_shared_len >= 0 && max_shared_len <= max_context_len && max_splits >= 1, PKV_ERR_INVALID,
                "max_shared_len = %d (0..max_context_len %d), max_splits = %d (>= 1)", max_shared_len,
                max_context_len, max_splits);
    return grouped_impl(desc, q, B, Hq, k_cache, v_cache, k_scale, v_scale, block_tables, max_blocks, context_lens,
                        max_context_len, group_size, shared_lens, max_shared_len, max_splits, softmax_scale, out,
                        workspace, workspace_bytes, stream);
}

int pkv::read_error_decode(void* stream, int32_t* out) { return read_clear_error(stream, out); }
