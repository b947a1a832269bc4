/*
 * pkv.h -- C ABI of libpkv: attention over a paged KV cache on AMD Instinct MI355X (gfx950).
 *
 * The KV cache is cut into fixed blocks of 256 tokens; a per-sequence block
 * table maps a sequence's logical blocks onto physically scattered blocks
 * (ocdem.com nano-vllm article, §2.1 PagedAttention; block size 256 as in
 * "Nano-vLLM性能调优实战", §1.1 KV缓存块配置, and the intelliparadigm.com
 * Nano-vLLM article, §2.1 动态分块内存管理).  The library provides:
 *
 *   - a host block manager (pkv_alloc_*) producing block tables, slot
 *     mappings and prefix-hash reuse;
 *   - pkv_kv_store: the store_kvcache scatter of new K/V rows by slot;
 *   - pkv_paged_attn_decode: one query token per sequence, split-K over the
 *     context with a log-sum-exp merge;
 *   - pkv_paged_attn_prefill: varlen causal attention of new prompt tokens
 *     over cached + new keys (flash_attn_with_kvcache's role in
 *     "Nano-vLLM性能调优实战", §2.2 缓存复用策略).
 *
 * Conventions for every function:
 *   - Return 0 (PKV_OK) on success, a negative pkv_status on failure; the
 *     failure text is available from pkv_last_error() on the same thread.
 *     Nothing throws, aborts or synchronises a stream.
 *   - Device functions take device pointers owned by the caller and enqueue
 *     work on `stream` (a hipStream_t; NULL = the default stream).  Buffers
 *     must stay alive until the stream has passed the work.  The library
 *     never allocates device memory.
 *   - Arguments that can be checked on the host are checked before anything
 *     is enqueued; a rejected call enqueues nothing.  Device data (slots, block
 *     ids, lengths) is trusted: out-of-range values there are undefined, unless
 *     device-data checks are on (pkv_set_device_checks, PKV_CHECK=1), which turn
 *     them into an entry in a device error word instead.
 *
 * Cache layout (all dtypes): K and V are each
 *     [num_blocks][num_kv_heads][256][head_dim]
 * row-major, so the 256 x head_dim tile of one (block, KV head) is contiguous.
 * Token slot s lives in block s / 256 at row s % 256.  Int8 caches carry one
 * fp32 scale per (block, KV head): k_scale, v_scale are [num_blocks][num_kv_heads]
 * and a stored code c means c * scale.
 *
 * Attention semantics (the pages give no formula; the plain reading):
 *   out[h] = sum_j softmax_j(softmax_scale * q[h] . k_j) v_j, fp32 accumulation;
 *   query head h reads KV head h / (Hq / Hkv).
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 256
/* Size of the split workspace held inside the library for pkv_paged_attn_decode_noalloc. */
#define PKV_DECODE_SCRATCH_BYTES (16u << 20)

enum pkv_status {
    PKV_OK = 0,
    PKV_ERR_INVALID = -1,      /* bad argument (null pointer, negative size, inconsistent shapes) */
    PKV_ERR_UNSUPPORTED = -2,  /* valid but not implemented (head_dim, dtype combination) */
    PKV_ERR_NO_BLOCKS = -3,    /* block pool exhausted; allocator state unchanged */
    PKV_ERR_UNKNOWN_SEQ = -4,  /* sequence id not admitted (or already freed) */
    PKV_ERR_DUP_SEQ = -5,      /* sequence id already admitted */
    PKV_ERR_SMALL_BUFFER = -6, /* caller buffer (table width, slot capacity, workspace) too small */
    PKV_ERR_HIP = -7           /* a HIP runtime call or kernel launch failed */
};

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_I8 = 2 } pkv_dtype;

typedef struct {
    int32_t num_blocks;   /* physical blocks in the pool */
    int32_t block_size;   /* must be 256 */
    int32_t num_kv_heads; /* Hkv */
    int32_t head_dim;     /* 64 or 128 */
    int32_t kv_dtype;     /* pkv_dtype of the cache */
} pkv_cache_desc;

/* Text of the last failure on the calling thread ("" if none).  Owned by the library. */
const char* pkv_last_error(void);
const char* pkv_version(void);

/* Device-data checks.  Kernels normally trust the indices they read from device memory (slots,
 * block ids, context and key lengths, launch order, run lists, cu_seqlens_q): an out-of-range
 * value there is undefined.  With checks on (pkv_set_device_checks(1), or PKV_CHECK=1 in the
 * environment when the library first launches a kernel), each kernel validates those values
 * before using them and records the first bad one in a device error word instead: a bad slot's
 * row is skipped; a workgroup whose sequence, run or block pair is bad computes nothing and leaves
 * its outputs unwritten.  Checks cost one test per workgroup (per row for stores).
 * pkv_device_error reads and clears the error word on `stream` and waits for the stream:
 * *code = 0 (no error) or 1 slot, 2 block id, 3 length, 4 launch-order entry, 5 run, 6
 * cu_seqlens_q, 7 copy row count, 8 a group member's block table differing within the group's
 * shared keys; *where = the batch row, sequence or pair; *value = the bad value, or for 8 the
 * block-table entry (where and value may be NULL).  The word is per device and shared by every
 * caller. */
int pkv_set_device_checks(int32_t enable);
int pkv_device_error(int32_t* code, int32_t* where, int32_t* value, void* stream);

/* ------------------------------------------------------------------------------------------
 * Host block manager.
 *
 * Blocks come from a FIFO free pool (intelliparadigm.com Nano-vLLM article, §2.1
 * 动态分块内存管理: ceil(len / 256) blocks, taken from the head of a free deque),
 * are shared through reference counts ("1200行代码挑战vLLM", §2 内存管理策略), and
 * full blocks of a prompt are reused through a hash of the prompt prefix
 * ("1200行代码挑战vLLM", §性能优化 1. 前缀缓存).  Freed blocks keep their contents
 * and hash until they are handed out again (lazy release; intelliparadigm.com
 * article, §7.2 关键优化点).
 *
 * Exact rules (fixed so that results are reproducible bit for bit):
 *   - The free deque starts as initial_order (a permutation of 0..num_blocks-1,
 *     e.g. a seeded shuffle for random physical placement; NULL = 0,1,2,...).
 *   - Full block i of a prompt (tokens 256i..256i+255) hashes as
 *     h_i = FNV-1a-64( le64(h_{i-1}) || le32(token) x 256 ), h_{-1} = 0.
 *   - add_seq: block i is reused ("hit") only if prefix caching is on, all
 *     earlier blocks were hits, the table maps h_i to a block holding exactly
 *     these tokens, and the prompt continues past the block ((i+1)*256 < n).
 *     A hit takes a reference (and leaves the free deque if it sat there).
 *     Every other block pops the head of the free deque, drops its old hash
 *     entry, and -- if full -- is registered under h_i (last writer wins).
 *   - append: a new block is popped when the position is a multiple of 256;
 *     a block is hashed and registered when it becomes full.
 *   - free_seq: references are dropped in reverse block order; a block whose
 *     count reaches 0 goes to the tail of the free deque.
 *   - fork: the child takes the parent's tokens, blocks and hash chain; every block
 *     gains a reference, and the child's whole length counts as cached.
 *   - append_batch_cow: before a token lands in a partially filled block whose
 *     count exceeds 1, the sequence drops that reference and takes the head of
 *     the free deque instead (the caller copies the old block into it); plain
 *     append and append_batch refuse such a token (PKV_ERR_INVALID).
 *   - add_seq, append, append_batch and append_batch_cow are atomic: on failure
 *     nothing changes.
 *   - With prefix_cache = 0 nothing is hashed.
 *
 * A handle is not thread-safe: use one thread per handle.
 * ------------------------------------------------------------------------------------------ */
typedef struct pkv_allocator pkv_allocator;

/* Creates a manager over num_blocks blocks of block_size (must be 256) tokens.
 * initial_order: host int32[num_blocks] permutation or NULL.  *out receives the handle. */
int pkv_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order,
                     int32_t prefix_cache, pkv_allocator** out);
void pkv_alloc_destroy(pkv_allocator* a);

/* Admits prompt `tokens[n]` (host) as sequence seq_id; *n_cached receives how many leading
 * tokens (a multiple of 256) already have their KV in the cache through prefix hits. */
int pkv_alloc_add_seq(pkv_allocator* a, int64_t seq_id, const int32_t* tokens, int32_t n,
                      int32_t* n_cached);

/* Appends one generated token to seq_id; *slot receives the cache slot of its K/V row. */
int pkv_alloc_append(pkv_allocator* a, int64_t seq_id, int32_t token, int32_t* slot);

/* Appends tokens[i] to seq_ids[i] for i < n, in order, atomically; slots[i] receives each slot. */
int pkv_alloc_append_batch(pkv_allocator* a, const int64_t* seq_ids, const int32_t* tokens,
                           int32_t n, int32_t* slots);

/* Parallel sampling and beam search (ocdem.com nano-vllm article, §2.1: the sequences of one
 * request share physical blocks through reference counts).  pkv_alloc_fork admits child_id as
 * a copy of parent_id that shares all of its blocks (PKV_ERR_DUP_SEQ for an existing child,
 * checked first, PKV_ERR_UNKNOWN_SEQ for a missing parent).  pkv_alloc_append_batch_cow is
 * pkv_alloc_append_batch with copy-on-write: copy_src[k], copy_dst[k] (host int32[n], k <
 * *n_copies) receive the block pairs whose contents the caller must copy (pkv_copy_blocks)
 * before storing the batch's new rows, and copy_rows[k] the rows of the source in use (the
 * appending sequence's offset in the block, 1..255); a pair appears in the order the batch
 * reached it, and no destination is a source of another pair.  PKV_ERR_NO_BLOCKS when the fresh blocks for new
 * block starts and copies exceed the free deque. */
int pkv_alloc_fork(pkv_allocator* a, int64_t parent_id, int64_t child_id);
/* A beam search step's forks in one call: pkv_alloc_fork(parent_ids[i], child_ids[i]) for i < n
 * in order (a child may be the parent of a later entry), atomically. */
int pkv_alloc_fork_batch(pkv_allocator* a, const int64_t* parent_ids, const int64_t* child_ids, int32_t n);
int pkv_alloc_append_batch_cow(pkv_allocator* a, const int64_t* seq_ids, const int32_t* tokens,
                               int32_t n, int32_t* slots, int32_t* copy_src, int32_t* copy_dst,
                               int32_t* copy_rows, int32_t* n_copies);

int pkv_alloc_free_seq(pkv_allocator* a, int64_t seq_id);
/* pkv_alloc_free_seq(seq_ids[i]) for i < n in order, atomically (PKV_ERR_UNKNOWN_SEQ when an id is
 * unknown or repeated). */
int pkv_alloc_free_batch(pkv_allocator* a, const int64_t* seq_ids, int32_t n);
int pkv_alloc_num_free(const pkv_allocator* a, int32_t* out);

/* Rows of int32[n][max_blocks] (host): each sequence's physical blocks, padded with -1.
 * context_lens (host int32[n], may be NULL) receives each sequence's current length.
 * PKV_ERR_SMALL_BUFFER if a sequence holds more than max_blocks blocks. */
int pkv_alloc_block_tables(const pkv_allocator* a, const int64_t* seq_ids, int32_t n,
                           int32_t max_blocks, int32_t* out, int32_t* context_lens);

/* Metadata for prefilling sequences seq_ids[n] (host buffers): positions n_cached..len-1
 * of each sequence are the new tokens.  cu_seqlens_q[n+1] = prefix sums of new-token
 * counts, seqlens_k[n] = total lengths (cached prefix included), slot_mapping[cap] the
 * slots of the new tokens in order; *n_slots = cu_seqlens_q[n]. */
int pkv_alloc_prefill_slots(const pkv_allocator* a, const int64_t* seq_ids, int32_t n,
                            int32_t* cu_seqlens_q, int32_t* seqlens_k, int32_t* slot_mapping,
                            int32_t cap, int32_t* n_slots);

/* Chunked prefill of long prompts ("Nano-vLLM性能调优实战", §3.2 关键调度参数 caps the new tokens
 * of one step): a prompt's new tokens may be computed over several steps.  Like
 * pkv_alloc_prefill_slots, for segments [starts[i], ends[i]) of each sequence's new tokens
 * (0 <= start <= end <= new-token count): cu_seqlens_q[n+1] = prefix sums of the segment
 * lengths, seqlens_k[n] = n_cached + ends[i] (keys visible to the segment: its cached prefix,
 * earlier segments and itself), slot_mapping[cap] the segments' slots in order. */
int pkv_alloc_prefill_segment_slots(const pkv_allocator* a, const int64_t* seq_ids,
                                    const int32_t* starts, const int32_t* ends, int32_t n,
                                    int32_t* cu_seqlens_q, int32_t* seqlens_k,
                                    int32_t* slot_mapping, int32_t cap, int32_t* n_slots);

/* Test hook: when enable != 0 every block hashes to `value`, forcing collisions so that
 * the token-comparison guard can be exercised. */
int pkv_alloc_debug_constant_hash(pkv_allocator* a, int32_t enable, uint64_t value);

/* ------------------------------------------------------------------------------------------
 * store_kvcache ("Nano-vLLM性能调优实战", §2.2 缓存复用策略): for t < n with
 * slot_mapping[t] >= 0, copy k_new[t][h][:] and v_new[t][h][:] (h < Hkv) into
 * k_cache / v_cache at that slot.  An exact copy: the rows must already be in the
 * cache dtype (f32, bf16 or int8 codes).  For int8 caches k_scale_new / v_scale_new
 * ([n][Hkv] fp32, device) are written to k_scale / v_scale at [slot / 256][h]; for
 * other dtypes all four scale pointers must be NULL.  A block holds one scale per KV
 * head, so rows of one call that land in one block must carry equal scales, and slots
 * must be distinct; otherwise which value is kept is unspecified.
 * k_new, v_new: device [n][Hkv][head_dim]; slot_mapping: device int32[n]; n may be 0.
 * ------------------------------------------------------------------------------------------ */
int pkv_kv_store(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                 const float* k_scale_new, const float* v_scale_new,
                 const int32_t* slot_mapping, int32_t n, void* k_cache, void* v_cache,
                 float* k_scale, float* v_scale, void* stream);

/* ------------------------------------------------------------------------------------------
 * Quantising store into int8 caches.  The pages name INT8 KV as an engine option
 * (intelliparadigm.com Nano-vLLM article, §2.2 混合精度计算流水线) and give no encoding;
 * this one keeps one fp32 scale per (physical block, KV head), k_scale / v_scale
 * [num_blocks][num_kv_heads], and a code c stands for c * scale.
 *
 * The new rows of one call that land in one block must form one run of consecutive batch
 * rows with consecutive slots (as pkv_alloc_prefill_slots and decode appends produce); a run
 * starting at offset o0 > 0 of its block treats rows 0..o0-1 of that block and the block's
 * scale as earlier output of this function.  Per run, KV head, and K / V separately:
 *   candidate = absmax of the run's values / 127 (fp64 quotient rounded to fp32);
 *   old = the block's scale if o0 > 0, else 0;  new = max(old, candidate);
 *   if new > old the rows 0..o0-1 are re-quantised: code = rint(code * old / new);
 *   the run's rows become clamp(rint(x / new), -127, 127) (all 0 when new == 0);
 *   the block's scale becomes new.
 * rint rounds the exact quotient half to even.  Rows with slot < 0 are skipped.
 *
 * k_new, v_new: device [n][num_kv_heads][head_dim] of new_dtype (PKV_BF16 or PKV_F32),
 * finite values; slot_mapping: device int32[n]; runs: device int32[2 * n_runs], the runs of
 * slot_mapping as pkv_store_runs gives them (first row, length); max_run: host, the longest
 * run's length (1..256; it selects the launch shape); k_cache, v_cache: device int8 caches
 * (desc->kv_dtype must be PKV_I8); k_scale, v_scale: device fp32 [num_blocks][num_kv_heads].
 * Two runs in one call must not share a block (the result is then undefined).  n_runs may be 0.
 * ------------------------------------------------------------------------------------------ */
int pkv_kv_store_quant(const pkv_cache_desc* desc, const void* k_new, const void* v_new,
                       int32_t new_dtype, const int32_t* slot_mapping, int32_t n, const int32_t* runs,
                       int32_t n_runs, int32_t max_run, void* k_cache, void* v_cache, float* k_scale,
                       float* v_scale, void* stream);

/* Copy-on-write block copies (ocdem.com nano-vllm article, §2.1): for k < n, rows 0..rows[k]-1
 * of every KV head of physical block dst[k] in both caches become copies of those of block
 * src[k] (the other rows are left as they are), and for int8 caches the block's k_scale / v_scale
 * entries are copied.  src, dst: device int32[n], valid block ids, with no dst equal to any src
 * or to another dst (pkv_alloc_append_batch_cow's pairs are such); rows: device int32[n] with
 * values in 0..256, or NULL for whole blocks.  k_scale, v_scale: int8 caches only, else NULL.
 * n may be 0. */
int pkv_copy_blocks(const pkv_cache_desc* desc, const int32_t* src, const int32_t* dst, const int32_t* rows,
                    int32_t n, void* k_cache, void* v_cache, float* k_scale, float* v_scale, void* stream);

/* The runs of a slot mapping for pkv_kv_store_quant (host): maximal groups of consecutive batch
 * rows whose slots are consecutive and in one block; rows with slot < 0 belong to none.
 * slot_mapping: host int32[n]; runs: host int32[2 * cap], filled with (first row, length) per
 * run in batch order; *n_runs = the number of runs, *max_run = the longest (0 when none).
 * PKV_ERR_SMALL_BUFFER when there are more than cap runs (cap = n always suffices). */
int pkv_store_runs(const int32_t* slot_mapping, int32_t n, int32_t* runs, int32_t cap,
                   int32_t* n_runs, int32_t* max_run);

/* ------------------------------------------------------------------------------------------
 * Paged decode attention: one query token per sequence.
 *
 * The context of each sequence is cut into splits of blocks_per_split blocks; one
 * workgroup handles one (sequence, KV head, split) and, when a sequence has more than
 * one split, a second kernel merges the partial softmax states by their
 * log-sum-exp (the max_splits knob of the intelliparadigm.com Nano-vLLM article,
 * §8: more splits for throughput at some latency cost).
 *
 * pkv_decode_plan: the split count and split width the decode call will use for this
 * shape.  max_splits = 0 picks automatically (split only until there are two workgroups per
 * CU of the current device; 256 CUs are assumed when no device is visible); > 0 caps the
 * split count.
 * pkv_decode_workspace_bytes: device workspace the decode call needs (0 when the
 * plan has a single split).
 * ------------------------------------------------------------------------------------------ */
int pkv_decode_plan(int32_t B, int32_t num_kv_heads, int32_t max_context_len, int32_t max_splits,
                    int32_t* splits, int32_t* blocks_per_split);
size_t pkv_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim, int32_t num_kv_heads,
                                  int32_t max_context_len, int32_t max_splits);

/* pkv_decode_launch_order: a seq_order (below) for a decode call of this shape.
 * context_lens: host int32[B], each >= 0; with window > 0 a sequence's work is
 * min(context_lens[b], window) keys, as in pkv_paged_attn_decode_window.  order: host
 * int32[B], written with a permutation of 0..B-1.  Host-only; nothing is launched.
 * Ordering is by work, longest first, with ties kept in sequence order.
 * When every workgroup of the launch fits on the device at once (B x num_kv_heads x splits
 * <= compute_units x workgroups_per_cu), workgroup i shares its CU with workgroups
 * i + compute_units, i + 2 compute_units, ...  The longest-first order is then cut into rounds
 * of compute_units / (num_kv_heads x splits) sequences, and every odd round is reversed.  The
 * longest contexts of one round thus share CUs with the shortest of the next, which evens out
 * the per-CU work.  Otherwise workgroups wait for free slots, and longest-first keeps the
 * launch's tail short.
 * compute_units <= 0 takes the current device's CU count (256 without a device, as in
 * pkv_decode_plan).  workgroups_per_cu <= 0 asks the current device for the occupancy of the
 * decode kernel of this dtype, head_dim and group size.  Without a device that query fails
 * with PKV_ERR_HIP.  Bad shapes, a negative length, NULL pointers (B > 0) or an unsupported
 * group size are PKV_ERR_INVALID / PKV_ERR_UNSUPPORTED. */
int pkv_decode_launch_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                            const int32_t* context_lens, int32_t max_context_len,
                            int32_t max_splits, int32_t window, int32_t compute_units,
                            int32_t workgroups_per_cu, int32_t* order);

/* q: device [B][Hq][head_dim], f32 when the cache is f32, bf16 otherwise.
 * k_cache, v_cache: device, layout above.  k_scale, v_scale: int8 caches only, else NULL.
 * block_tables: device int32[B][max_blocks]; context_lens: device int32[B] -- the number
 * of tokens to attend, including the one just stored; 0 gives a zero output.
 * seq_order: NULL, or device int32[B], a permutation of 0..B-1 giving the order in which the
 * sequences' workgroups are launched (pkv_decode_launch_order computes a good one); the output
 * stays indexed by sequence.
 * max_context_len: host upper bound of context_lens (sizes the split plan).  A larger entry is
 * undefined (its tail would fall outside the plan); with device-data checks on it is recorded as
 * error 3 and that sequence's output is left unwritten.
 * out: device [B][Hq][head_dim] in the dtype of q.  workspace: device, at least
 * pkv_decode_workspace_bytes(...) bytes (may be NULL when that is 0). */
int pkv_paged_attn_decode(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                          const void* k_cache, const void* v_cache, const float* k_scale,
                          const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* context_lens, const int32_t* seq_order,
                          int32_t max_context_len, int32_t max_splits, float softmax_scale,
                          void* out, void* workspace, size_t workspace_bytes, void* stream);

/* pkv_paged_attn_decode_noalloc: pkv_paged_attn_decode for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments and results, minus the workspace: when the plan splits contexts, the partial
 * states go to a split workspace inside the library, one PKV_DECODE_SCRATCH_BYTES (16 MiB) array
 * per device, kept until the process ends.  Nothing is allocated: no hipMalloc, hipFree or
 * allocating library call.  A plan needing more than PKV_DECODE_SCRATCH_BYTES
 * (pkv_decode_workspace_bytes) is refused with PKV_ERR_SMALL_BUFFER before anything is launched;
 * lower max_splits, or call pkv_paged_attn_decode with a workspace.  Every call on one device
 * shares that device's array, and each call's partials are written before they are read, so
 * nothing needs clearing between calls; calls that may overlap on one device (different
 * streams, or different threads) race on it and must be ordered by the caller. */
int pkv_paged_attn_decode_noalloc(const pkv_cache_desc* desc, const void* q, int32_t B,
                                  int32_t Hq, const void* k_cache, const void* v_cache,
                                  const float* k_scale, const float* v_scale,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  const int32_t* context_lens, const int32_t* seq_order,
                                  int32_t max_context_len, int32_t max_splits,
                                  float softmax_scale, void* out, void* stream);

/* Sliding-window decode (intelliparadigm.com Nano-vLLM article, §7.2 关键优化点 lists sliding-
 * window attention): as pkv_paged_attn_decode, but sequence b attends only its last `window`
 * keys, positions max(0, context_lens[b] - window) .. context_lens[b] - 1; window = 0 attends
 * every key.  The split plan covers the window's blocks only (a workspace sized by
 * pkv_decode_workspace_bytes for max_context_len is always enough).  window < 0 is
 * PKV_ERR_INVALID. */
int pkv_paged_attn_decode_window(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                 const void* k_cache, const void* v_cache, const float* k_scale,
                                 const float* v_scale, const int32_t* block_tables,
                                 int32_t max_blocks, const int32_t* context_lens,
                                 const int32_t* seq_order, int32_t max_context_len,
                                 int32_t max_splits, float softmax_scale, int32_t window, void* out,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* pkv_decode_store_attend: one decode step's store and attention in one launch -- the
 * engine's store_kvcache write of each step's new token followed by attention over the cache
 * ("Nano-vLLM性能调优实战", §2.2 缓存复用策略), fused.
 * k_new, v_new: device [B][num_kv_heads][head_dim] in the cache dtype, row b the new token
 * of sequence b; k_scale_new, v_scale_new: int8 caches only, device float[B][num_kv_heads],
 * written as the scale of the token's (block, head) as pkv_kv_store does; slot_mapping:
 * device int32[B], the new token's slot, which must be the slot of position
 * context_lens[b] - 1 of sequence b in block_tables (-1: nothing stored for b).  The store
 * happens before any read of that block, by the one workgroup that reads it.  All other
 * arguments and rules are those of pkv_paged_attn_decode; k_cache, v_cache, k_scale and
 * v_scale are written.  The result equals pkv_kv_store followed by pkv_paged_attn_decode. */
int pkv_decode_store_attend(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                            const void* k_new, const void* v_new, const float* k_scale_new,
                            const float* v_scale_new, const int32_t* slot_mapping, void* k_cache,
                            void* v_cache, float* k_scale, float* v_scale,
                            const int32_t* block_tables, int32_t max_blocks,
                            const int32_t* context_lens, const int32_t* seq_order,
                            int32_t max_context_len, int32_t max_splits, float softmax_scale,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/* Grouped decode for forked sequences.  Parallel sampling and beam search keep several
 * sequences per request that share blocks (ocdem.com nano-vllm article, §2.1; a fork shares every
 * block of its parent, pkv_alloc_fork).  Group k is the group_size consecutive sequences
 * k*group_size .. k*group_size + group_size - 1 of the batch; its first shared_lens[k] keys must
 * sit in the same physical blocks for every member.  The call reads those blocks once per group
 * and KV head for all members' query heads, then each member's remaining keys for its own heads,
 * so the shared keys cross HBM once per group instead of once per member.  The output is that of
 * pkv_paged_attn_decode on the same batch up to fp32 rounding order.
 *
 * pkv_decode_group_shared_lens (host-only): shared_lens[k] = min over the members of
 * context_lens, capped at 256 x the number of leading block-table entries equal across the
 * members.  block_tables: host int32[B][max_blocks]; context_lens: host int32[B], each within
 * 0..256 x max_blocks; shared_lens: host int32[B / group_size], written.  B not a multiple of
 * group_size, group_size < 1, a bad length or a NULL pointer (B > 0) is PKV_ERR_INVALID.
 *
 * pkv_paged_attn_decode_grouped: q, k_cache, v_cache, k_scale, v_scale, block_tables,
 * context_lens, max_context_len, softmax_scale and out as in pkv_paged_attn_decode (no split, no
 * launch order, no workspace).  shared_lens: device int32[B / group_size], each at most every
 * member's context length (pkv_decode_group_shared_lens computes them).  group_size x Hq /
 * num_kv_heads must be 1, 2, 4 or 8 (query rows per KV head and group), else
 * PKV_ERR_UNSUPPORTED; B must be a multiple of group_size, else PKV_ERR_INVALID.  With
 * device-data checks on, a shared length above a member's context (or a context above
 * max_context_len) is recorded as error 3, a block id outside the pool as error 2 and a member
 * whose table differs within the shared keys as error 8; that group's output is then left
 * unwritten. */
int pkv_decode_group_shared_lens(const int32_t* block_tables, int32_t max_blocks,
                                 const int32_t* context_lens, int32_t B, int32_t group_size,
                                 int32_t* shared_lens);
int pkv_paged_attn_decode_grouped(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                  const void* k_cache, const void* v_cache, const float* k_scale,
                                  const float* v_scale, const int32_t* block_tables,
                                  int32_t max_blocks, const int32_t* context_lens,
                                  int32_t max_context_len, int32_t group_size,
                                  const int32_t* shared_lens, float softmax_scale, void* out,
                                  void* stream);

/* Grouped decode over splits.  With one workgroup per (group, KV head), a launch lasts as long as
 * its longest group while the CUs of shorter groups idle; as decode splits a context and merges the
 * pieces by log-sum-exp (the max_splits knob, intelliparadigm.com Nano-vLLM article, closing
 * paragraph), each group's shared keys are cut into splits of bps blocks, each walked by its own
 * workgroups, and a second launch merges every (member, query head)'s splits.
 *
 * pkv_decode_grouped_workspace_bytes: the workspace a call with these arguments needs, 0 when it
 * does not split (bad arguments also give 0): B x Hq x S x (head_dim + 2) floats, with S the
 * number of splits below.
 *
 * pkv_paged_attn_decode_grouped_split: arguments as pkv_paged_attn_decode_grouped, plus
 *   - max_shared_len: at least every shared_lens entry (device data) and at most
 *     max_context_len; the splits cover ceil(max_shared_len / 256) blocks;
 *   - max_splits >= 1: S = ceil(nsh / bps) splits of bps = ceil(nsh / min(max_splits, nsh))
 *     blocks, nsh = ceil(max_shared_len / 256); only the last split walks the members' own keys
 *     (those past the shared prefix); S = 1 is the unsplit call;
 *   - workspace (device, 16-byte aligned, caller-owned, at least
 *     pkv_decode_grouped_workspace_bytes bytes when that is nonzero; contents on entry ignored).
 * A bad max_shared_len or max_splits is PKV_ERR_INVALID, a short workspace PKV_ERR_SMALL_BUFFER;
 * other errors as pkv_paged_attn_decode_grouped.  With device-data checks on, a shared length above
 * max_shared_len is recorded as error 3 and that group's outputs are left unwritten.  The output
 * equals that of pkv_paged_attn_decode_grouped up to fp32 rounding order. */
size_t pkv_decode_grouped_workspace_bytes(int32_t B, int32_t Hq, int32_t head_dim, int32_t max_shared_len,
                                          int32_t max_splits);
int pkv_paged_attn_decode_grouped_split(const pkv_cache_desc* desc, const void* q, int32_t B, int32_t Hq,
                                        const void* k_cache, const void* v_cache, const float* k_scale,
                                        const float* v_scale, const int32_t* block_tables, int32_t max_blocks,
                                        const int32_t* context_lens, int32_t max_context_len,
                                        int32_t group_size, const int32_t* shared_lens, int32_t max_shared_len,
                                        int32_t max_splits, float softmax_scale, void* out, void* workspace,
                                        size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Varlen paged prefill attention (bf16 cache, bf16 q/out, fp32 accumulation): the engine's
 * full-computation phase, attention over the whole prompt with FlashAttention-2 named as the
 * kernel for it (intelliparadigm.com Nano-vLLM article, §7.2 关键优化点), reading a cache that
 * the store has just written ("Nano-vLLM性能调优实战", §2.2 缓存复用策略), for varlen batches of
 * new tokens whose cached prefix blocks are reused (ocdem.com nano-vllm article, §2.1).
 *
 * q: device bf16 [total_q][Hq][head_dim], the new tokens of B sequences back to back;
 * sequence b owns rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (device int32[B+1]).
 * seqlens_k: device int32[B], all keys of sequence b (cached prefix included), read
 * through block_tables (device int32[B][max_blocks]).  With causal != 0, new token i
 * of sequence b sits at position seqlens_k[b] - n_q(b) + i and attends keys 0..that
 * position (bottom-right alignment); otherwise it attends all seqlens_k[b] keys.
 * The new tokens' K/V must already be stored (pkv_kv_store earlier on the stream).
 * max_seqlen_q, max_seqlen_k: host upper bounds.  softmax_scale must be positive.
 * out: device bf16 [total_q][Hq][head_dim].
 * ------------------------------------------------------------------------------------------ */
int pkv_paged_attn_prefill(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                           const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                           int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                           const void* k_cache, const void* v_cache, const int32_t* block_tables,
                           int32_t max_blocks, float softmax_scale, int32_t causal, void* out,
                           void* stream);

/* Sliding-window prefill (intelliparadigm.com Nano-vLLM article, §7.2 关键优化点 lists
 * sliding-window attention): pkv_paged_attn_prefill with causal = 1, where the query at position
 * P sees keys max(0, P - window + 1) .. P; window = 0 sees every key up to P.  Key tiles before
 * a query tile's window are not read.  window < 0 is PKV_ERR_INVALID. */
int pkv_paged_attn_prefill_window(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                  const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                  int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                  const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks,
                                  float softmax_scale, int32_t window, void* out, void* stream);

/* Prefill in a caller-given work order.  A work item is one (sequence, query tile) of a launch;
 * its workgroups cover every KV head.  Items run in the order they are listed.
 * pkv_paged_attn_prefill finds each workgroup's item on the device instead: every sequence's last
 * tile first, then every second-to-last, and so on.
 *
 * pkv_prefill_work_order: host-only, nothing is launched.  It writes the launch's items into
 * work_items (host int32[capacity]), each (sequence << 16) | query tile, and their count into
 * *n_items.  cu_seqlens_q (host int32[B+1], starting at 0) and seqlens_k (host int32[B]) are
 * those of the call; causal and window are as in that call.  Order:
 *   - by work, heaviest first: key tiles of 64 keys the item attends, plus one;
 *   - cut into rounds of (CUs of the current device) / num_kv_heads items;
 *   - every odd round reversed, so the heavy items of one round share CUs with the light items of
 *     the next.
 * Ties keep sequence and tile order.  Query tiles hold *tile_rows tokens (tile_rows may be
 * NULL), the pkv_prefill_tile_rows of total_q = cu_seqlens_q[B], B, the group size and the
 * device.
 * Errors:
 *   - more items than capacity: PKV_ERR_SMALL_BUFFER;
 *   - B above 32767: PKV_ERR_INVALID;
 *   - decreasing cu_seqlens_q, or seqlens_k shorter than the new tokens of a causal call:
 *     PKV_ERR_INVALID.
 *
 * pkv_paged_attn_prefill_ordered: pkv_paged_attn_prefill / _window (window = 0: every key) with
 * work_items (device int32[n_items]) cut into query tiles of tile_rows tokens.  work_items and
 * tile_rows must be what pkv_prefill_work_order gave for the same cu_seqlens_q, seqlens_k,
 * shapes and device, whatever total_q the call passes (it may exceed cu_seqlens_q[B]); a
 * tile_rows that is not one of this kernel's tiles for the group size is PKV_ERR_INVALID.
 * Outputs are bitwise those of the unordered call with the same tile.  n_items = 0 does nothing.  The items are
 * device data: with device-data checks on, an item whose sequence or tile does not exist is
 * recorded as error 5 (where = its index, value = the item).
 *
 * pkv_prefill_tile_rows: query tokens per work item of a launch of this shape. */
int pkv_prefill_work_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                           const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t causal,
                           int32_t window, int32_t* work_items, int32_t capacity, int32_t* n_items,
                           int32_t* tile_rows);
int pkv_paged_attn_prefill_ordered(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                   const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                   int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                   const void* k_cache, const void* v_cache,
                                   const int32_t* block_tables, int32_t max_blocks,
                                   float softmax_scale, int32_t causal, int32_t window,
                                   const int32_t* work_items, int32_t n_items, int32_t tile_rows,
                                   void* out, void* stream);
int pkv_prefill_tile_rows(const pkv_cache_desc* desc, int32_t Hq, int32_t B, int32_t total_q,
                          int32_t* tile_rows);

/* Split-K prefill for launches that leave CUs idle.  The pages cap a step at a budget of new
 * tokens ("Nano-vLLM性能调优实战", §3.2 关键调度参数), so a chunk can hold few prompts; with
 * fewer workgroups than the device has CUs, the launch lasts as long as its longest item (the
 * last query tile of its longest prompt, which walks every key tile alone).  As decode splits its
 * context, such a launch splits the key range of long items into pieces, each run by its own
 * workgroups and kept as a partial state (output and row sum relative to the running maximum),
 * and a second launch merges each item's pieces by log-sum-exp (the full-computation phase's
 * FlashAttention-2 style attention, intelliparadigm.com Nano-vLLM article, §7.2 关键优化点).
 *
 * pkv_prefill_split_order: host-only, nothing is launched.  Inputs as pkv_prefill_work_order.
 * When the launch has at least as many workgroups (items x num_kv_heads) as the device has CUs,
 * no item is split: the pieces are the items of pkv_prefill_work_order, in its order, and there
 * are no merges.  Otherwise every item longer than T key tiles is cut into up to 8 pieces of
 * nearly equal length, T being the smallest value from 4 up that keeps the launch within one
 * workgroup per CU (two workgroups sharing a CU each take more than twice as long per key tile as
 * one alone).  Outputs:
 *   - pieces (host int32[pieces_capacity][4]), *n_pieces records {(sequence << 16) | query tile,
 *     first key tile, end key tile, slot}: a piece walks key tiles first .. end-1 of its item
 *     (0 .. INT32_MAX: all of them) and, with slot >= 0, writes its partial state to that slot;
 *     heaviest first in rounds as pkv_prefill_work_order orders items;
 *   - merges (host int32[merges_capacity][4]), *n_merges records {(sequence << 16) | query tile,
 *     first slot, pieces, 0}: the pieces of a split item hold consecutive slots;
 *   - *n_slots partial slots, *tile_rows tokens per query tile.
 * Errors as pkv_prefill_work_order; PKV_ERR_SMALL_BUFFER when either list exceeds its capacity
 * ((total new tokens + B) x 8 pieces and (total new tokens + B) merges always suffice).
 *
 * pkv_prefill_split_workspace_bytes: the workspace that n_slots slots need (0 for bad arguments):
 * n_slots x num_kv_heads x (head_dim + 4) x tile_rows x (Hq / num_kv_heads) floats.
 *
 * pkv_paged_attn_prefill_split: pkv_paged_attn_prefill_ordered over the pieces (device
 * int32[n_pieces][4]) and then, when n_merges > 0, the merge of the split items (device
 * int32[n_merges][4]), both enqueued on `stream`.  workspace: caller-owned device memory of at
 * least pkv_prefill_split_workspace_bytes(desc, Hq, n_slots, tile_rows) bytes, 16-byte aligned,
 * needed only when n_slots > 0; its contents before the call do not matter, and it must stay
 * alive until the stream has passed the merge.  The lists, n_slots and tile_rows must be what
 * pkv_prefill_split_order gave for the same cu_seqlens_q, seqlens_k, shapes and device; unsplit
 * items give bitwise the outputs of pkv_paged_attn_prefill_ordered, split items the same
 * attention within rounding.  Errors: those of the ordered call; a workspace too small:
 * PKV_ERR_SMALL_BUFFER; n_merges and n_slots not both zero or both positive: PKV_ERR_INVALID.
 * With device-data checks on, a piece or merge record outside the call's sequences, tiles or
 * slots is recorded as error 5 (where = its index, value = its first field). */
int pkv_prefill_split_order(const pkv_cache_desc* desc, int32_t Hq, int32_t B,
                            const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t causal,
                            int32_t window, int32_t* pieces, int32_t pieces_capacity,
                            int32_t* n_pieces, int32_t* merges, int32_t merges_capacity,
                            int32_t* n_merges, int32_t* n_slots, int32_t* tile_rows);
size_t pkv_prefill_split_workspace_bytes(const pkv_cache_desc* desc, int32_t Hq, int32_t n_slots,
                                         int32_t tile_rows);
int pkv_paged_attn_prefill_split(const pkv_cache_desc* desc, const void* q, int32_t Hq,
                                 const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t B,
                                 int32_t total_q, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks,
                                 float softmax_scale, int32_t causal, int32_t window,
                                 const int32_t* pieces, int32_t n_pieces, const int32_t* merges,
                                 int32_t n_merges, int32_t n_slots, int32_t tile_rows,
                                 void* workspace, size_t workspace_bytes, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
