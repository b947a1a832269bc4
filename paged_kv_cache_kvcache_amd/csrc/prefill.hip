// Varlen paged prefill attention for gfx950 on bf16 MFMA.
//
// The pages describe the full-computation (prefill) phase running FlashAttention-2 style attention
// (intelliparadigm.com Nano-vLLM article, §7.2 关键优化点) over varlen sequences in the paged cache
// ("Nano-vLLM性能调优实战", §2.2 缓存复用策略), with new tokens batched up to a token budget
// ("Nano-vLLM性能调优实战", §3.2 关键调度参数) and cached prefixes reused (ocdem.com nano-vllm
// article, §2.1).  The kernel below is this library's own design for CDNA4.
//
// Work decomposition
//   One workgroup (NW = 4 or 8 wavefronts) per (sequence, query tile, KV head).  The G = Hq/Hkv
//   query heads that read one KV head are stacked into 32 NW MFMA rows: a query tile holds
//   QT = 32 NW / G new tokens of all G heads, so every K/V tile staged in LDS serves all of them.
//   Wavefront w owns rows 32w..32w+31 (row rho -> head rho / QT, token rho % QT).  Work items are
//   ordered so that the tiles with the longest causal rows (each sequence's last) start first.
//   Large launches take eight wavefronts (half the K/V staging per row), small ones four (twice
//   the workgroups, a shorter tail).
//
// Per 64-key tile (two LDS stages; the next tile's DMA is in flight during compute):
//   staging         K and V rows go from HBM straight into LDS (global_load_lds_dwordx4, no
//                   registers), row-major with XOR-swizzled 16-byte chunks.
//   S^T = K Q^T     v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q^T kept in registers.
//                   The accumulator layout puts one query per lane column, 16 keys per lane, and
//                   the other 16 keys of that query in lane ^ 32: the softmax max/sum of a query
//                   needs a single cross-lane swap.
//   online softmax  log2 domain, one FMA folds the scale into the exponent, causal mask by
//                   absolute position (bottom-right aligned) on diagonal tiles only, lazy rescale.
//   O^T += V^T P^T  A = V^T read from the row-major V tile with LDS transpose reads
//                   (ds_read_b64_tr_b16), B = P^T converted to bf16 straight from the S
//                   accumulators; the transpose reads fetch V for exactly the keys each lane's P
//                   values belong to.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <atomic>
#include <vector>
#include <cmath>
#include <type_traits>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaveRows = 32;  // MFMA query rows (tokens x heads) per wavefront
constexpr int kKT = 64;     // keys per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;
constexpr bf16x2_t kOnes2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};

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
    int32_t window;  // > 0 (causal only): a query at position P sees keys P - window + 1 .. P
    float scale_log2;
    int32_t total_q;
    int32_t num_blocks;
    int32_t check;   // launch the instantiation that validates cu_seqlens_q, key lengths and block ids
    const int32_t* items;  // NULL: the built-in order; else item i = (sequence << 16) | query tile
    int32_t n_items;
    // split launches: piece i = {(sequence << 16) | query tile, first key tile, end key tile, slot}
    // (items == NULL); a piece with slot >= 0 writes its partial state to slot `slot` of `part`
    const int4* pieces;
    float* part;
    int32_t n_slots;
};

// Device-data checks (uniform in the workgroup, so a workgroup that fails leaves as a whole).
// cu_seqlens_q non-decreasing within 0..total_q:
__device__ bool prefill_cu_ok(const PrefillArgs& a) {
    bool ok = a.cu_seqlens_q[0] >= 0 && a.cu_seqlens_q[a.B] <= a.total_q;
    int bad = ok ? 0 : (a.cu_seqlens_q[0] < 0 ? 0 : a.B);
    for (int s = 0; ok && s < a.B; ++s)
        if (a.cu_seqlens_q[s + 1] < a.cu_seqlens_q[s]) {
            ok = false;
            bad = s + 1;
        }
    if (!ok && threadIdx.x == 0 && blockIdx.x == 0) record_error(pkv::kErrCuSeqlens, bad, a.cu_seqlens_q[bad]);
    return ok;
}
// every block id of keys key0..key1-1 of sequence b is in the pool:
__device__ bool prefill_blocks_ok(const PrefillArgs& a, int b, int key0, int key1) {
    const int lane = threadIdx.x & 63;
    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks;
    const int e_end = (key1 + pkv::kBlock - 1) / pkv::kBlock;
    for (int e0 = key0 / pkv::kBlock; e0 < e_end; e0 += 64) {
        const int e = e0 + lane;
        const int v = bt[min(e, e_end - 1)];  // clamped, so the load needs no exec mask
        const uint64_t bad = __ballot(e < e_end && (v < 0 || v >= a.num_blocks));
        if (bad != 0) {
            const int first = __shfl(v, __ffsll(static_cast<unsigned long long>(bad)) - 1, 64);
            if (threadIdx.x == 0) record_error(pkv::kErrBlock, b, first);
            return false;
        }
    }
    return true;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v;
    v.x = static_cast<__bf16>(lo);
    v.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, v);
}

// LDS holds 64 banks of 4 bytes: a 16-byte chunk position p of a row sits on bank group
// (row * RB / 16 + p) % 16.  Chunk c of a K or V row is stored at position c ^ swz(row), with one
// swizzle per tile so that each operand read pattern is free of bank conflicts:
//   K (ds_read_b128, 16 lanes per cycle on 16 consecutive rows, one chunk): the 16 rows must land
//     on 16 distinct bank groups;
//   V (ds_read_b64_tr_b16, 32 lanes per cycle on 4 consecutive rows x 4 consecutive chunks): the
//     16 (row, chunk) pairs must land on 16 distinct bank groups.
// The V swizzle depends only on row bits that are constant across the rows one lane reads.
template <int D>
__device__ __forceinline__ int swz_k(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int row) { return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

__device__ __forceinline__ i16x4_t read_tr(const char* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4_t*)((lds_char*)(const_cast<char*>(p))));
}

__device__ __forceinline__ void dma16(const char* src, char* lds_dst) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src, (lds_char*)lds_dst, 16,
                                     0, 0);
}

// every DMA this wavefront issued has landed in LDS (vmcnt(0); expcnt and lgkmcnt left alone)
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// v_permlane32_swap exchanges the upper half of one operand with the lower half of the other;
// swapping v with itself leaves every lane holding its own value and that of lane ^ 32.  It does
// not go through the LDS queue, so (unlike a bpermute) it does not wait for LDS reads in flight.
__device__ __forceinline__ float max_across_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// NW = wavefronts per workgroup (4 or 8): all of them share each staged K/V tile.
template <int D, int G, int NW, bool CHECK>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 2 : 1) void prefill_kernel(PrefillArgs a) {
    constexpr int kThreads = 64 * NW;
    constexpr int kRows = kWaveRows * NW;  // MFMA query rows per workgroup
    constexpr int QT = kRows / G;       // new tokens per workgroup
    constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
    constexpr int DT = D / 32;          // 32-row tiles of O^T
    constexpr int RB = D * 2;           // bytes per K/V row in LDS (chunks swizzled, no padding)
    constexpr int CPR = D / 8;          // 16-byte chunks per row
    constexpr int TB = kKT * RB;        // bytes of one K (or V) tile
    constexpr int NLD = TB / (kThreads * 16);  // DMA instructions per wavefront per tile, K and V each
    static_assert(NLD >= 1 && NLD * kThreads * 16 == TB, "a tile is a whole number of wavefront DMAs");
    // Two stages of (K tile, V tile), as two distinct arrays: the compiler then sees that reads of
    // one stage cannot alias the DMA in flight into the other and adds no wait for it.
    __shared__ __attribute__((aligned(1024))) char lds0[2 * TB];
    __shared__ __attribute__((aligned(1024))) char lds1[2 * TB];
    char* const lds[2] = {lds0, lds1};

    // ---- which (sequence, query tile, KV head) this workgroup owns.  Work items are ordered by
    // distance from the end of their sequence (every sequence's last tile first, then every
    // second-to-last tile, ...), so the tiles with the longest causal rows start first; the KV
    // head varies fastest.
    if (CHECK && !prefill_cu_ok(a)) return;
    const int g = blockIdx.x % a.num_kv_heads;
    int item = blockIdx.x / a.num_kv_heads;
    int b = -1, tile = 0, nq = 0;
    int kt_begin = 0, kt_end = INT_MAX, slot = -1;  // the key tiles this workgroup walks, its partial slot
    if (a.pieces != nullptr) {  // a split launch (the grid has exactly n_items x Hkv workgroups)
        const int4 pc = a.pieces[item];
        b = pc.x >> 16;
        tile = pc.x & 0xffff;
        kt_begin = pc.y;
        kt_end = pc.z;
        slot = pc.w;
        if (CHECK) {
            const bool seq_ok = pc.x >= 0 && b < a.B;
            const int n = seq_ok ? a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b] : 0;
            if (!seq_ok || tile >= (n + QT - 1) / QT || kt_begin < 0 || kt_end < kt_begin || slot < -1 ||
                slot >= a.n_slots) {
                if (threadIdx.x == 0 && g == 0) record_error(pkv::kErrRun, item, pc.x);
                return;
            }
        }
    } else if (a.items != nullptr) {  // the caller's order (the grid has exactly n_items x Hkv workgroups)
        const int it = a.items[item];
        b = it >> 16;
        tile = it & 0xffff;
        if (CHECK) {
            const bool seq_ok = it >= 0 && b < a.B;
            const int n = seq_ok ? a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b] : 0;
            if (!seq_ok || tile >= (n + QT - 1) / QT) {
                if (threadIdx.x == 0 && g == 0) record_error(pkv::kErrRun, item, it);
                return;
            }
        }
    }
    for (int r = 0; b < 0 && a.items == nullptr && a.pieces == nullptr; ++r) {
        int live = 0;
        for (int s = 0; s < a.B; ++s) {
            const int n = a.cu_seqlens_q[s + 1] - a.cu_seqlens_q[s];
            const int T = (n + QT - 1) / QT;
            if (T > r) {
                if (item == 0) {
                    b = s;
                    tile = T - 1 - r;
                    nq = n;
                    break;
                }
                --item;
                ++live;
            }
        }
        if (b < 0 && live == 0) break;  // past the last work item
    }
    if (b < 0) return;

    // The sequence's lengths and the first window of its block table (below) are requested
    // together, so that a workgroup's start waits for one memory round trip after its work item.
    const int lane = threadIdx.x & 63, col = lane & 31, h = lane >> 5;
    const int32_t* bt = a.block_tables + size_t(b) * a.max_blocks;
    int btv = lane < a.max_blocks ? bt[lane] : 0;
    const int Lk = a.seqlens_k[b];
    const int qrow0 = a.cu_seqlens_q[b];
    if (a.items != nullptr || a.pieces != nullptr) nq = a.cu_seqlens_q[b + 1] - qrow0;
    if (CHECK && (Lk < 0 || Lk > int64_t(a.max_blocks) * pkv::kBlock || (a.causal && Lk < nq))) {
        if (threadIdx.x == 0 && g == 0) record_error(pkv::kErrLength, b, Lk);
        return;
    }
    const int q0 = tile * QT;
    const int nqt = min(QT, nq - q0);
    const int pos0 = Lk - nq + q0;  // absolute position of token q0
    const int kv_len = a.causal ? min(Lk, pos0 + nqt) : Lk;
    const int ntiles = (kv_len + kKT - 1) / kKT;
    if (CHECK && !prefill_blocks_ok(a, b, a.window > 0 ? max(0, pos0 - a.window + 1) / kKT * kKT : 0, kv_len))
        return;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int rho = 32 * w + col;
    const int j = rho / QT, t = rho % QT;
    const bool col_ok = t < nqt;
    // last key the column of token t sees (non-decreasing in t)
    auto last_key = [&](int tt) { return a.causal ? min(pos0 + tt, kv_len - 1) : kv_len - 1; };
    // first key the column whose last key is p sees, under a sliding window (non-decreasing in p)
    auto first_key = [&](int p) { return a.window > 0 ? max(0, p - a.window + 1) : 0; };
    const int P = last_key(t), Lo = first_key(P);
    // The wavefront's columns hold tokens t_lo..t_hi of the tile: 32 consecutive tokens of one
    // head when a tile has 32 or more tokens, else every token of the tile.  Both key bounds are
    // monotone in t, so their extremes over the wavefront come from its end tokens: the last key
    // any column sees (tiles past it are skipped), the last key every column sees (tiles up to it
    // need no mask), and the same pair for the first keys of a sliding window (tiles wholly below
    // the smallest are skipped, tiles from the largest on need no lower mask).
    const int t_lo = QT >= 32 ? (32 * w) % QT : 0, t_hi = QT >= 32 ? t_lo + 31 : QT - 1;
    const int pw_max = last_key(t_hi), pw_min = last_key(t_lo);
    const int lw_min = first_key(pw_min), lw_max = first_key(pw_max);
    // the workgroup's first tile holds the first key of its first token; a piece walks its own
    // range of those tiles
    const int kt0 = a.window > 0 ? max(0, pos0 - a.window + 1) / kKT : 0;
    const int kt_lo = max(kt0, kt_begin), kt_hi = min(ntiles, kt_end);

    // ---- this sequence's block table, 64 entries at a time: lane i holds entry 64 win + i, and a
    // tile reads its physical block with readlane (no memory access per tile).  btv, requested
    // above, holds the first window.
    int bt_win = 0;
    auto phys_block = [&](int blk) {  // blk is uniform
        const int win = blk >> 6;
        if (win != bt_win) {  // a new window every 16384 keys
            bt_win = win;
            const int e = 64 * win + lane;
            btv = e < a.max_blocks ? bt[e] : 0;
        }
        return __builtin_amdgcn_readlane(btv, blk & 63);
    };

    const size_t head_off = size_t(g) * pkv::kBlock;

    // ---- global -> LDS DMA of one K/V tile.  Instruction r of wavefront w fills LDS bytes
    // [(NLD w + r) KiB, +1 KiB) of the tile, lane l the 16 bytes at +16 l: row L / CPR, position
    // L % CPR, which holds chunk (L % CPR) ^ swz_k(row) (K) or ^ swz_v(row) (V) of that key row.  Rows past the sequence end
    // are read from its last key (finite data; their scores are masked, their probabilities zero).
    int drow[NLD];
    uint32_t kcol[NLD], vcol[NLD];
#pragma unroll
    for (int r = 0; r < NLD; ++r) {
        const int L = (NLD * w + r) * 64 + lane;
        drow[r] = L / CPR;
        kcol[r] = ((L % CPR) ^ swz_k<D>(L / CPR)) * 16;
        vcol[r] = ((L % CPR) ^ swz_v<D>(L / CPR)) * 16;
    }
    auto dma = [&](int kt, char* stage) {
        const int key0 = kt * kKT;
        const int64_t phys = phys_block(key0 / pkv::kBlock);
        const size_t row0 = (size_t(phys) * a.num_kv_heads) * pkv::kBlock + head_off + key0 % pkv::kBlock;
        const char* kg = a.k_cache + row0 * RB;
        const char* vg = a.v_cache + row0 * RB;
        const int last = kv_len - 1 - key0;
#pragma unroll
        for (int r = 0; r < NLD; ++r) {
            const uint32_t row = uint32_t(min(drow[r], last) * RB);  // 32-bit offsets from a uniform base
            dma16(kg + (row + kcol[r]), stage + (NLD * w + r) * 1024);
            dma16(vg + (row + vcol[r]), stage + TB + (NLD * w + r) * 1024);
        }
    };

    // ---- per-lane LDS read offsets.  K operand (S^T = K Q^T): lane reads key row 32mt + col,
    // chunk 2ks + h; the swizzle of that row depends on col only.
    int koff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) koff[ks] = col * RB + (((2 * ks + h) ^ swz_k<D>(col)) << 4);
    // V^T operand (O^T += V^T P^T) by transpose reads: in each 16-lane group, lane i of the result
    // takes element i % 4 of the 8 bytes addressed by lane 4e + i / 4, for e = 0..3.  Lane l
    // addresses key row 4h + (l & 15) / 4 (+ a multiple of 8) and the four d from
    // 32dt + 16((l >> 4) & 1) + 4(l & 3), so result lane l holds d = 32dt + (l & 31) for four
    // consecutive keys.  The chunk of those four d is 4dt + 2((l >> 4) & 1) + ((l >> 1) & 1).
    int voff[DT];
    {
        const int vr = 4 * h + ((lane & 15) >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int c = 4 * dt + 2 * ((lane >> 4) & 1) + ((lane >> 1) & 1);
            voff[dt] = vr * RB + ((c ^ swz_v<D>(vr)) << 4) + 8 * (lane & 1);
        }
    }

    f32x16_t o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;
    float m_run = kNegInf, l_run = 0.f;

    if (kt_lo < kt_hi) dma(kt_lo, lds[0]);

    // ---- Q^T operand: column col = query row, 8 consecutive d per k-step.  Q is multiplied by
    // softmax_scale * log2(e) (fp32, rounded once to bf16), so S comes out in log2 units.  Loaded
    // once the first tile's DMA is in flight, so the two latencies overlap.
    bf16x8_t qb[KS];
    {
        const int tq = min(t, nqt - 1);
        const uint16_t* qp = a.q + (size_t(qrow0 + q0 + tq) * a.num_q_heads + g * G + j) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 v = col_ok ? *reinterpret_cast<const uint4*>(qp + 16 * ks) : make_uint4(0, 0, 0, 0);
            uint32_t* u = reinterpret_cast<uint32_t*>(&v);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                u[e] = pack_bf16x2(__uint_as_float(u[e] << 16) * a.scale_log2,
                                   __uint_as_float(u[e] & 0xffff0000u) * a.scale_log2);
            qb[ks] = __builtin_bit_cast(bf16x8_t, v);
        }
    }

    // One step per key tile: wait for its DMA, barrier (the other stage is then free: every
    // wavefront finished the previous tile), launch the next tile's DMA, compute.  The step is
    // instantiated for each LDS stage so that every LDS address offset is an immediate.
    auto step = [&](int kt, auto stage) {
        constexpr int buf = decltype(stage)::value;
        wait_dma();
        __syncthreads();
        if (kt + 1 < kt_hi) dma(kt + 1, lds[buf ^ 1]);
        // every key of this tile is masked for this wavefront (past its last key, or before its window)
        if (kt * kKT > pw_max || kt * kKT + kKT - 1 < lw_min) return;

        const char* Ks = lds[buf];
        const char* Vs = lds[buf] + TB;
        // S^T = K Q^T - base for keys 32mt..32mt+31 (log2 units, relative to this column's running
        // max; the first k-step starts from the accumulator -base), two interleaved chains
        const float base = m_run == kNegInf ? 0.f : m_run;
        f32x16_t s[2];
        {
            // all K operand reads first, so their LDS latency overlaps instead of stalling each MFMA
            bf16x8_t ka[KS][2];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    ka[ks][mt] = *reinterpret_cast<const bf16x8_t*>(Ks + koff[ks] + 32 * mt * RB);
            __builtin_amdgcn_sched_barrier(0);
            f32x16_t c0;
#pragma unroll
            for (int i = 0; i < 16; ++i) c0[i] = -base;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
                    s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks][mt], qb[ks], ks == 0 ? c0 : s[mt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // V^T operands of this tile: issued before the softmax, which hides their latency.  va
        // [mt][kk][dt] covers keys 32mt + 16kk + {4h..4h+3, 8+4h..8+4h+3}, d = 32dt + (lane & 31).
        bf16x8_t va[2][2][DT];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const char* vp = Vs + voff[dt] + (32 * mt + 16 * kk) * RB;
                    const i16x4_t lo = read_tr(vp);
                    const i16x4_t hi = read_tr(vp + 8 * RB);
                    va[mt][kk][dt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
        __builtin_amdgcn_sched_barrier(0);
        // mask (diagonal and window-edge tiles only) and tile max
        float tmax = kNegInf;
        if (kt * kKT + kKT - 1 > pw_min || kt * kKT < lw_max) {
            const uint32_t span = uint32_t(P - Lo);
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    // key kt*64 + 4h + c (c = 32mt + 8(i/4) + i%4) is visible when Lo <= key <= P:
                    // one unsigned comparison of key - Lo against P - Lo
                    const uint32_t rel = uint32_t(kt * kKT + 4 * h - Lo + 32 * mt + 8 * (i / 4) + (i % 4));
                    s[mt][i] = rel <= span ? s[mt][i] : kNegInf;
                    tmax = fmaxf(tmax, s[mt][i]);
                }
        } else {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[mt][i]);
        }
        tmax = max_across_halves(tmax);
        // Lazy rescaling: the running max only moves on a column's first tile or when its max grew
        // by more than 2^8, so most tiles skip rescaling O and take p = exp2(s) directly;
        // probabilities then stay below 2^8, well inside bf16.
        if (__any(tmax > 8.f || m_run == kNegInf)) {
            const float mn = fmaxf(m_run, base + tmax);
            const float alpha = m_run == kNegInf ? 0.f : __builtin_amdgcn_exp2f(m_run - mn);
            const float shift = mn == kNegInf ? 0.f : mn - base;
            m_run = mn;
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[dt][i] *= alpha;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[mt][i] -= shift;
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[mt][i] = __builtin_amdgcn_exp2f(s[mt][i]);
        // O^T += V^T P^T over keys 32mt + 16kk + [0, 16).  This lane's P values are keys
        // 16kk + 4h + {0..3} (elements 8kk..8kk+3 of s[mt]) and 16kk + 8 + 4h + {0..3} (8kk+4..8kk+7):
        // the keys, in that order, of the V operand va[mt][kk].
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
                // the row sum takes the same bf16 probabilities that multiply V
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw4.x), kOnes2, l_run, false);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw4.y), kOnes2, l_run, false);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw4.z), kOnes2, l_run, false);
                l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pw4.w), kOnes2, l_run, false);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mt][kk][dt], pb, o[dt], 0, 0, 0);
            }
        }
    };
    for (int kt = kt_lo; kt < kt_hi; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        if (kt + 1 < kt_hi) step(kt + 1, std::integral_constant<int, 1>{});
    }

    // ---- normalise and write this column's row: d = 32dt + 8(i/4) + 4h + i%4
    const float l_tot = sum_across_halves(l_run);
    if (slot >= 0) {
        // partial state of this piece, every row of the tile: O unnormalised and the row sum, both
        // relative to 2^m_run (m_run in log2 units; -inf with l = 0 when no key was visible).  One
        // record of D + 4 floats per row (O, m, l, padding), rows of a (slot, KV head) consecutive.
        float* pr = a.part + ((size_t(slot) * a.num_kv_heads + g) * kRows + rho) * size_t(D + 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                *reinterpret_cast<float4*>(pr + 32 * dt + 8 * i4 + 4 * h) =
                    make_float4(o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]);
        if (h == 0) *reinterpret_cast<float2*>(pr + D) = make_float2(m_run, l_tot);
        return;
    }
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

// ---- merge of a split launch's pieces: the pieces' partial states (O, l relative to 2^m) of each
// row combine by log-sum-exp, out = sum_p 2^(m_p - M) O_p / sum_p 2^(m_p - M) l_p with
// M = max_p m_p.
constexpr int kMaxPieces = 8;  // pieces per split item

struct MergeArgs {
    const int4* merges;  // {(sequence << 16) | query tile, first slot, pieces, 0}
    const float* part;
    const int32_t* cu_seqlens_q;
    uint16_t* out;
    int32_t B;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t n_slots;
    int32_t check;
};

// A (split item, KV head) takes kRows / (kMergeThreads / (D / 8)) workgroups, each a run of its
// rows; a thread owns 8 consecutive d of one row, so the threads of a row read its pieces' records
// and write its output row side by side.
constexpr int kMergeThreads = 256;

template <int D, int G, int NW>
__global__ __launch_bounds__(kMergeThreads) void prefill_merge_kernel(MergeArgs a) {
    constexpr int kRows = kWaveRows * NW, QT = kRows / G;
    constexpr int DC = D / 8, RPB = kMergeThreads / DC, PARTS = kRows / RPB;  // rows per workgroup, workgroups per tile
    const int run = blockIdx.x % PARTS, gm = blockIdx.x / PARTS;
    const int g = gm % a.num_kv_heads, mi = gm / a.num_kv_heads;
    const int4 rec = a.merges[mi];
    const int b = rec.x >> 16, tile = rec.x & 0xffff, s0 = rec.y, np = rec.z;
    if (a.check) {  // uniform in the workgroup
        const bool seq_ok = rec.x >= 0 && b < a.B;
        const int n = seq_ok ? a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b] : 0;
        if (!seq_ok || tile >= (n + QT - 1) / QT || np < 1 || np > kMaxPieces || s0 < 0 || s0 > a.n_slots - np) {
            if (threadIdx.x == 0 && g == 0 && run == 0) record_error(pkv::kErrRun, mi, rec.x);
            return;
        }
    }
    const int rho = run * RPB + threadIdx.x / DC, dc = threadIdx.x % DC;
    const int j = rho / QT, t = rho % QT;
    const int q = tile * QT + t;
    if (q >= a.cu_seqlens_q[b + 1] - a.cu_seqlens_q[b]) return;
    constexpr size_t RS = D + 4;  // floats per row record
    const float* p0 = a.part + ((size_t(s0) * a.num_kv_heads + g) * kRows + rho) * RS;
    const size_t pstep = size_t(a.num_kv_heads) * kRows * RS;  // next slot, same KV head and row
    float2 ml[kMaxPieces];
    float M = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p) {
        ml[p] = p < np ? *reinterpret_cast<const float2*>(p0 + p * pstep + D) : make_float2(-INFINITY, 0.f);
        M = fmaxf(M, ml[p].x);
    }
    float L = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int p = 0; p < kMaxPieces; ++p) {
        if (p < np && ml[p].x != -INFINITY) {
            const float wgt = __builtin_amdgcn_exp2f(ml[p].x - M);
            L += wgt * ml[p].y;
            const float4 lo = *reinterpret_cast<const float4*>(p0 + p * pstep + 8 * dc);
            const float4 hi = *reinterpret_cast<const float4*>(p0 + p * pstep + 8 * dc + 4);
            acc[0] += wgt * lo.x; acc[1] += wgt * lo.y; acc[2] += wgt * lo.z; acc[3] += wgt * lo.w;
            acc[4] += wgt * hi.x; acc[5] += wgt * hi.y; acc[6] += wgt * hi.z; acc[7] += wgt * hi.w;
        }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    uint4 v;
    v.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    v.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    v.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
    v.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
    *reinterpret_cast<uint4*>(a.out + (size_t(a.cu_seqlens_q[b] + q) * a.num_q_heads + g * G + j) * D + 8 * dc) = v;
}

template <int D, int G, int NW>
hipError_t launch_nw(const PrefillArgs& a, long items, hipStream_t st) {
    // device-data checks run in their own instantiation, so the production one is unchanged by them
    if (a.check) hipLaunchKernelGGL((prefill_kernel<D, G, NW, true>), dim3(unsigned(items)), dim3(64 * NW), 0, st, a);
    else hipLaunchKernelGGL((prefill_kernel<D, G, NW, false>), dim3(unsigned(items)), dim3(64 * NW), 0, st, a);
    return hipGetLastError();
}

// Eight-wavefront workgroups halve the K/V staging per query row; four-wavefront ones give twice as
// many workgroups, which shortens the tail of a small launch (its longest causal rows).  Eight are
// used once a launch has at least two workgroups per CU of them.
int choose_nw(long total_q, int B, int Hkv, int G, int num_cus) {
    const int QT8 = 8 * kWaveRows / G;
    const long items8 = ((total_q + QT8 - 1) / QT8 + B) * long(Hkv);
    return items8 >= 2L * num_cus ? 8 : 4;
}

template <int D, int G>
hipError_t launch(const PrefillArgs& a, int total_q, int num_cus, int nw_given, hipStream_t st) {
    const int nw = nw_given > 0 ? nw_given : choose_nw(total_q, a.B, a.num_kv_heads, G, num_cus);
    const int QT = nw * kWaveRows / G;
    const long items = a.items != nullptr || a.pieces != nullptr
                           ? long(a.n_items) * a.num_kv_heads
                           : ((long(total_q) + QT - 1) / QT + a.B) * a.num_kv_heads;
    if (items > INT32_MAX) return hipErrorInvalidValue;
    return nw == 8 ? launch_nw<D, G, 8>(a, items, st) : launch_nw<D, G, 4>(a, items, st);
}

template <int D, int G>
hipError_t launch_merge(const MergeArgs& m, int n_merges, int nw, hipStream_t st) {
    const int parts = kWaveRows * nw / (kMergeThreads / (D / 8));  // workgroups per (item, KV head)
    const dim3 grid(unsigned(long(n_merges) * m.num_kv_heads * parts));
    if (nw == 8) hipLaunchKernelGGL((prefill_merge_kernel<D, G, 8>), grid, dim3(kMergeThreads), 0, st, m);
    else hipLaunchKernelGGL((prefill_merge_kernel<D, G, 4>), grid, dim3(kMergeThreads), 0, st, m);
    return hipGetLastError();
}

template <int D>
hipError_t launch_merge_g(const MergeArgs& m, int n_merges, int G, int nw, hipStream_t st) {
    switch (G) {
        case 1: return launch_merge<D, 1>(m, n_merges, nw, st);
        case 2: return launch_merge<D, 2>(m, n_merges, nw, st);
        case 4: return launch_merge<D, 4>(m, n_merges, nw, st);
        case 8: return launch_merge<D, 8>(m, n_merges, nw, st);
        default: return hipErrorInvalidValue;
    }
}

template <int D>
hipError_t launch_g(const PrefillArgs& a, int total_q, int G, int num_cus, int nw, hipStream_t st) {
    switch (G) {
        case 1: return launch<D, 1>(a, total_q, num_cus, nw, st);
        case 2: return launch<D, 2>(a, total_q, num_cus, nw, st);
        case 4: return launch<D, 4>(a, total_q, num_cus, nw, st);
        case 8: return launch<D, 8>(a, total_q, num_cus, nw, st);
        default: return hipErrorInvalidValue;
    }
}

// compute units of the current device (queried once per device; callers may be on any thread)
int current_num_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
            (void)hipGetLastError();
            n = 256;
        }
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

}  // namespace

namespace {

int prefill_impl(const pkv_cache_desc* desc, const void* q, int32_t Hq, const int32_t* cu_seqlens_q,
                 const int32_t* seqlens_k, int32_t B, int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                 const void* k_cache, const void* v_cache, const int32_t* block_tables, int32_t max_blocks,
                 float softmax_scale, int32_t causal, int32_t window, void* out, void* stream,
                 const int32_t* items = nullptr, int32_t n_items = 0, int32_t tile_rows = 0,
                 const int32_t* pieces = nullptr, const int32_t* merges = nullptr, int32_t n_merges = 0,
                 int32_t n_slots = 0, float* part = nullptr) {
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
    PKV_REQUIRE(std::isfinite(softmax_scale) && softmax_scale > 0.f, PKV_ERR_INVALID,
                "softmax_scale must be finite and positive");
    PKV_REQUIRE(window >= 0 && (window == 0 || causal), PKV_ERR_INVALID,
                "window = %d: a sliding window needs causal attention and window >= 0", window);
    // a work list fixes the query tile: the launch must cut tiles exactly as the list did
    int nw = 0;
    if (items != nullptr || pieces != nullptr) {
        nw = tile_rows > 0 && tile_rows * G % kWaveRows == 0 ? tile_rows * G / kWaveRows : 0;
        PKV_REQUIRE(nw == 4 || nw == 8, PKV_ERR_INVALID,
                    "tile_rows %d is not a query tile of this kernel for group size %d (%d or %d)", tile_rows, G,
                    4 * kWaveRows / G, 8 * kWaveRows / G);
    }
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
    a.window = window;
    a.scale_log2 = softmax_scale * kLog2e;
    a.total_q = total_q;
    a.num_blocks = desc->num_blocks;
    a.check = pkv::device_checks();
    a.items = items;
    a.n_items = n_items;
    a.pieces = reinterpret_cast<const int4*>(pieces);
    a.part = part;
    a.n_slots = n_slots;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int cus = current_num_cus();
    hipError_t e = D == 64 ? launch_g<64>(a, total_q, G, cus, nw, st) : launch_g<128>(a, total_q, G, cus, nw, st);
    PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "prefill launch failed: %s", hipGetErrorString(e));
    if (n_merges > 0) {
        MergeArgs m{};
        m.merges = reinterpret_cast<const int4*>(merges);
        m.part = part;
        m.cu_seqlens_q = cu_seqlens_q;
        m.out = static_cast<uint16_t*>(out);
        m.B = B;
        m.num_kv_heads = Hkv;
        m.num_q_heads = Hq;
        m.n_slots = n_slots;
        m.check = a.check;
        e = D == 64 ? launch_merge_g<64>(m, n_merges, G, nw, st) : launch_merge_g<128>(m, n_merges, G, nw, st);
        PKV_REQUIRE(e == hipSuccess, PKV_ERR_HIP, "prefill merge launch failed: %s", hipGetErrorString(e));
    }
    return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attn_prefill(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                      const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                      int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                      const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                      int32_t max_blocks, float softmax_scale, int32_t causal, void* out,
                                      void* stream) {
    return prefill_impl(desc, q, Hq, cu_seqlens_q, seqlens_k, B, total_q, max_seqlen_q, max_seqlen_k, k_cache,
                        v_cache, block_tables, max_blocks, softmax_scale, causal, 0, out, stream);
}

extern "C" int pkv_paged_attn_prefill_window(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                             const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                             int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                             const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, int32_t max_blocks,
                                             float softmax_scale, int32_t window, void* out, void* stream) {
    return prefill_impl(desc, q, Hq, cu_seqlens_q, seqlens_k, B, total_q, max_seqlen_q, max_seqlen_k, k_cache,
                        v_cache, block_tables, max_blocks, softmax_scale, 1, window, out, stream);
}

extern "C" int pkv_paged_attn_prefill_ordered(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                              const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                              int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                              const void* k_cache, const void* v_cache,
                                              const int32_t* block_tables, int32_t max_blocks,
                                              float softmax_scale, int32_t causal, int32_t window,
                                              const int32_t* work_items, int32_t n_items, int32_t tile_rows,
                                              void* out, void* stream) {
    PKV_REQUIRE(n_items >= 0, PKV_ERR_INVALID, "n_items = %d", n_items);
    PKV_REQUIRE(work_items != nullptr || n_items == 0, PKV_ERR_INVALID, "NULL work_items");
    if (n_items == 0) return PKV_OK;
    return prefill_impl(desc, q, Hq, cu_seqlens_q, seqlens_k, B, total_q, max_seqlen_q, max_seqlen_k, k_cache,
                        v_cache, block_tables, max_blocks, softmax_scale, causal, window, out, stream, work_items,
                        n_items, tile_rows);
}

namespace {

// One (sequence, query tile) work item of a prefill launch: code = (sequence << 16) | tile, and
// the key tiles kt0 .. kt1 - 1 it walks (from the tile holding its first token's first key).
struct PlanItem {
    int32_t code;
    int32_t kt0, kt1;
};

// The items of a prefill call cut into query tiles of *QT tokens (the tile the launch will use), in
// sequence and tile order; PKV_OK or the failure recorded.
int plan_items(const pkv_cache_desc* desc, int32_t Hq, int32_t B, const int32_t* cu_seqlens_q,
               const int32_t* seqlens_k, int32_t causal, int32_t window, std::vector<PlanItem>& items, int* QT) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(B >= 0 && B <= 32767 && Hq > 0 && window >= 0, PKV_ERR_INVALID,
                "bad shape (B=%d, Hq=%d, window=%d)", B, Hq, window);
    PKV_REQUIRE(Hq % desc->num_kv_heads == 0, PKV_ERR_INVALID, "Hq %d is not a multiple of Hkv %d", Hq,
                desc->num_kv_heads);
    const int G = Hq / desc->num_kv_heads;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, PKV_ERR_UNSUPPORTED, "query group size %d", G);
    items.clear();
    *QT = 4 * kWaveRows / G;
    if (B == 0) return PKV_OK;
    PKV_REQUIRE(cu_seqlens_q && seqlens_k, PKV_ERR_INVALID, "NULL pointer");
    PKV_REQUIRE(cu_seqlens_q[0] == 0, PKV_ERR_INVALID, "cu_seqlens_q[0] = %d", cu_seqlens_q[0]);
    for (int b = 0; b < B; ++b) {
        const int nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        PKV_REQUIRE(nq >= 0, PKV_ERR_INVALID, "cu_seqlens_q decreases at %d", b + 1);
        PKV_REQUIRE(seqlens_k[b] >= 0 && (!causal || seqlens_k[b] >= nq), PKV_ERR_INVALID,
                    "seqlens_k[%d] = %d for %d new tokens", b, seqlens_k[b], nq);
    }
    *QT = choose_nw(cu_seqlens_q[B], B, desc->num_kv_heads, G, current_num_cus()) * kWaveRows / G;
    for (int b = 0; b < B; ++b) {
        const int nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b], L = seqlens_k[b];
        for (int t = 0; t * *QT < nq; ++t) {
            PKV_REQUIRE(t <= 0xffff, PKV_ERR_UNSUPPORTED, "sequence %d has more than 65536 query tiles", b);
            const int pos0 = L - nq + t * *QT, nqt = std::min(*QT, nq - t * *QT);
            const int kv_len = causal ? std::min(L, pos0 + nqt) : L;
            const int kt0 = window > 0 ? std::max(0, pos0 - window + 1) / kKT : 0;
            items.push_back({(b << 16) | t, kt0, std::max(kt0, (kv_len + kKT - 1) / kKT)});
        }
    }
    return PKV_OK;
}

// Launch order of work with the given weights: heaviest first (ties in index order), cut into
// rounds of one workgroup per CU (`round` items), every odd round reversed so that the heavy items
// of one round share CUs with the light ones of the next.
std::vector<int> heaviest_first_rounds(const std::vector<uint32_t>& weight, int round) {
    const int n = int(weight.size());
    std::vector<uint64_t> key(n);
    for (int i = 0; i < n; ++i) key[i] = (uint64_t(~weight[i]) << 32) | uint32_t(i);
    std::sort(key.begin(), key.end());
    round = std::max(1, round);
    for (int r0 = round; r0 < n; r0 += 2 * round)
        std::reverse(key.begin() + r0, key.begin() + std::min(n, r0 + round));
    std::vector<int> order(n);
    for (int i = 0; i < n; ++i) order[i] = int(key[i] & 0xffffffffu);
    return order;
}

}  // namespace

extern "C" int pkv_prefill_work_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                                      const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t causal,
                                      int32_t window, int32_t* work_items, int32_t capacity, int32_t* n_items,
                                      int32_t* tile_rows) {
    PKV_REQUIRE(n_items != nullptr, PKV_ERR_INVALID, "NULL n_items");
    *n_items = 0;
    PKV_REQUIRE(capacity >= 0, PKV_ERR_INVALID, "capacity = %d", capacity);
    std::vector<PlanItem> items;
    int QT = 0;
    const int rc = plan_items(desc, Hq, B, cu_seqlens_q, seqlens_k, causal, window, items, &QT);
    if (rc != PKV_OK) return rc;
    if (tile_rows != nullptr) *tile_rows = QT;
    const int n = int(items.size());
    PKV_REQUIRE(n <= capacity && (work_items != nullptr || n == 0), PKV_ERR_SMALL_BUFFER,
                "%d work items, capacity %d", n, capacity);
    // weight: the key tiles an item walks, +1 for a workgroup's fixed cost
    std::vector<uint32_t> weight(n);
    for (int i = 0; i < n; ++i) weight[i] = uint32_t(items[i].kt1 - items[i].kt0 + 1);
    const std::vector<int> order = heaviest_first_rounds(weight, current_num_cus() / desc->num_kv_heads);
    for (int i = 0; i < n; ++i) work_items[i] = items[order[i]].code;
    *n_items = n;
    return PKV_OK;
}

// Split order for launches that leave CUs idle.  A launch of fewer workgroups than the device has
// CUs is bound by its longest item (the last query tile of the longest prompt walks every key
// tile alone on a CU).  Such a launch cuts the key range of every item longer than T tiles into
// up to kMaxPieces pieces of nearly equal length, each run by its own workgroups and written as a
// partial state, and a merge launch combines the pieces by log-sum-exp (split-K, as decode does
// over its context).  T starts at kMinPieceTiles (a piece also pays a workgroup's start) and grows
// until the launch fits two workgroups per CU.  Launches that fill the device are not split.
constexpr int kMinPieceTiles = 4;

extern "C" int pkv_prefill_split_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                                       const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t causal,
                                       int32_t window, int32_t* pieces, int32_t pieces_capacity, int32_t* n_pieces,
                                       int32_t* merges, int32_t merges_capacity, int32_t* n_merges,
                                       int32_t* n_slots, int32_t* tile_rows) {
    PKV_REQUIRE(n_pieces && n_merges && n_slots && tile_rows, PKV_ERR_INVALID, "NULL output count");
    *n_pieces = *n_merges = *n_slots = 0;
    PKV_REQUIRE(pieces_capacity >= 0 && merges_capacity >= 0, PKV_ERR_INVALID, "capacity %d, %d",
                pieces_capacity, merges_capacity);
    std::vector<PlanItem> items;
    int QT = 0;
    const int rc = plan_items(desc, Hq, B, cu_seqlens_q, seqlens_k, causal, window, items, &QT);
    if (rc != PKV_OK) return rc;
    *tile_rows = QT;
    const int n = int(items.size()), Hkv = desc->num_kv_heads, cus = current_num_cus();
    // pieces per item: 1 when the launch fills the device, else ceil(tiles / T) up to kMaxPieces
    std::vector<int> np(n, 1);
    if (long(n) * Hkv < cus) {
        for (int T = kMinPieceTiles;; ++T) {
            long wgs = 0;
            for (int i = 0; i < n; ++i) {
                const int tiles = items[i].kt1 - items[i].kt0;
                np[i] = std::max(1, std::min(kMaxPieces, (tiles + T - 1) / T));
                wgs += long(np[i]) * Hkv;
            }
            if (wgs <= cus) break;
        }
    }
    struct Piece {
        int32_t code, kt0, kt1, slot;
    };
    std::vector<Piece> list;
    std::vector<int32_t> merge_list;
    int slots = 0;
    for (int i = 0; i < n; ++i) {
        const PlanItem& it = items[i];
        if (np[i] == 1) {
            list.push_back({it.code, 0, INT_MAX, -1});
            continue;
        }
        const int tiles = it.kt1 - it.kt0;
        for (int p = 0; p < np[i]; ++p)
            list.push_back({it.code, it.kt0 + tiles * p / np[i], it.kt0 + tiles * (p + 1) / np[i], slots + p});
        merge_list.insert(merge_list.end(), {it.code, slots, np[i], 0});
        slots += np[i];
    }
    const int npc = int(list.size()), nm = int(merge_list.size() / 4);
    PKV_REQUIRE(npc <= pieces_capacity && (pieces != nullptr || npc == 0), PKV_ERR_SMALL_BUFFER,
                "%d pieces, capacity %d", npc, pieces_capacity);
    PKV_REQUIRE(nm <= merges_capacity && (merges != nullptr || nm == 0), PKV_ERR_SMALL_BUFFER,
                "%d merges, capacity %d", nm, merges_capacity);
    std::vector<uint32_t> weight(npc);
    // weight: the key tiles a piece walks (a whole item: all of its tiles), +1 for the start
    for (int i = 0, k = 0; i < n; ++i)
        for (int p = 0; p < np[i]; ++p, ++k)
            weight[k] = uint32_t(np[i] == 1 ? items[i].kt1 - items[i].kt0 + 1 : list[k].kt1 - list[k].kt0 + 1);
    const std::vector<int> order = heaviest_first_rounds(weight, cus / Hkv);
    for (int i = 0; i < npc; ++i) {
        const Piece& pc = list[order[i]];
        pieces[4 * i + 0] = pc.code;
        pieces[4 * i + 1] = pc.kt0;
        pieces[4 * i + 2] = pc.kt1;
        pieces[4 * i + 3] = pc.slot;
    }
    std::copy(merge_list.begin(), merge_list.end(), merges);
    *n_pieces = npc;
    *n_merges = nm;
    *n_slots = slots;
    return PKV_OK;
}

extern "C" size_t pkv_prefill_split_workspace_bytes(const pkv_cache_desc* desc, int32_t Hq, int32_t n_slots,
                                                    int32_t tile_rows) {
    if (desc == nullptr || desc->num_kv_heads <= 0 || Hq <= 0 || Hq % desc->num_kv_heads != 0 || n_slots < 0 ||
        tile_rows <= 0)
        return 0;
    const size_t rows = size_t(tile_rows) * size_t(Hq / desc->num_kv_heads);  // MFMA rows of a query tile
    return size_t(n_slots) * size_t(desc->num_kv_heads) * size_t(desc->head_dim + 4) * rows * sizeof(float);
}

extern "C" int pkv_paged_attn_prefill_split(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                            const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                            int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                            const void* k_cache, const void* v_cache, const int32_t* block_tables,
                                            int32_t max_blocks, float softmax_scale, int32_t causal,
                                            int32_t window, const int32_t* pieces, int32_t n_pieces,
                                            const int32_t* merges, int32_t n_merges, int32_t n_slots,
                                            int32_t tile_rows, void* workspace, size_t workspace_bytes, void* out,
                                            void* stream) {
    PKV_REQUIRE(n_pieces >= 0 && n_merges >= 0 && n_slots >= 0, PKV_ERR_INVALID,
                "n_pieces = %d, n_merges = %d, n_slots = %d", n_pieces, n_merges, n_slots);
    PKV_REQUIRE(pieces != nullptr || n_pieces == 0, PKV_ERR_INVALID, "NULL pieces");
    PKV_REQUIRE(merges != nullptr || n_merges == 0, PKV_ERR_INVALID, "NULL merges");
    PKV_REQUIRE((n_merges == 0) == (n_slots == 0), PKV_ERR_INVALID,
                "%d merges over %d partial slots: both are zero or neither", n_merges, n_slots);
    if (n_pieces == 0) return PKV_OK;
    const size_t need = pkv_prefill_split_workspace_bytes(desc, Hq, n_slots, tile_rows);
    PKV_REQUIRE(n_slots == 0 || (workspace != nullptr && workspace_bytes >= need), PKV_ERR_SMALL_BUFFER,
                "%d partial slots need %zu bytes of workspace, %zu given", n_slots, need, workspace_bytes);
    PKV_REQUIRE((uintptr_t(workspace) & 15) == 0, PKV_ERR_INVALID, "workspace must be 16-byte aligned");
    return prefill_impl(desc, q, Hq, cu_seqlens_q, seqlens_k, B, total_q, max_seqlen_q, max_seqlen_k, k_cache,
                        v_cache, block_tables, max_blocks, softmax_scale, causal, window, out, stream, nullptr,
                        n_pieces, tile_rows, pieces, merges, n_merges, n_slots, static_cast<float*>(workspace));
}

extern "C" int pkv_prefill_tile_rows(const pkv_cache_desc* desc, int32_t Hq, int32_t B, int32_t total_q,
                                     int32_t* tile_rows) {
    int rc = pkv::check_desc(desc);
    if (rc != PKV_OK) return rc;
    PKV_REQUIRE(tile_rows != nullptr, PKV_ERR_INVALID, "NULL tile_rows");
    PKV_REQUIRE(B >= 0 && Hq > 0 && total_q >= 0 && Hq % desc->num_kv_heads == 0, PKV_ERR_INVALID,
                "bad shape (B=%d, Hq=%d, total_q=%d)", B, Hq, total_q);
    const int G = Hq / desc->num_kv_heads;
    PKV_REQUIRE(G == 1 || G == 2 || G == 4 || G == 8, PKV_ERR_UNSUPPORTED, "query group size %d", G);
    *tile_rows = choose_nw(total_q, B, desc->num_kv_heads, G, current_num_cus()) * kWaveRows / G;
    return PKV_OK;
}

int pkv::read_error_prefill(void* stream, int32_t* out) { return read_clear_error(stream, out); }
