"""Drives the hot path on one GPU: admit prompts, store their KV, run decode steps and prefill chunks.

This is the engine-side glue around the library, the way a scheduler would call it: the block
manager hands out blocks and slots (host), the metadata goes to the device in one pinned copy, the
store kernel writes the new K/V rows, then the attention kernel runs.  Every computation happens in
libpkv; this module only moves arrays.
"""

import ctypes

import numpy as np
import torch

from . import (BF16, BLOCK, F32, I8, Allocator, _check, copy_blocks, decode_group_shared_lens, decode_plan,
               decode_grouped_workspace_bytes, decode_store_attend, paged_attn_decode_grouped,
               paged_attn_decode_grouped_split,
               decode_workspace_bytes, desc_of, kv_store, kv_store_quant, lib, paged_attn_decode,
               paged_attn_prefill_split, prefill_split_order, prefill_split_workspace_bytes)

TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8}
# grouped decode over splits (DecodeBatch(group_splits=0)): splits ~ CUs / (groups x KV heads), at
# most this many; measured on MI355X, bf16, 16 / 8 heads, 4 beams over 8k-32k-token prompts: 1, 2, 4
# and 8 requests run best at 16, 16, 4 and 4 splits, 32 requests unsplit
GROUP_MAX_SPLITS = 16

# mean shared keys per group from which DecodeBatch reads a group's shared blocks once
# (pkv_paged_attn_decode_grouped); measured crossover on MI355X, bf16, 16 / 8 heads, D 128
GROUP_MIN_SHARED = 1536
# ... and whose shared keys hold more K/V bytes than this (the 256 MB MALL): below it the
# per-sequence kernel's re-reads of the shared blocks hit the MALL, and it wins the step (measured
# on MI355X, 4 beams over 16k-32k-token prompts: 1 and 2 requests, about 100 and 200 MB, per
# sequence 0.089-0.099 ms against 0.109-0.113 ms grouped; 4 requests, about 400 MB, 0.193 against
# 0.146 ms)
GROUP_MIN_SHARED_BYTES = 256 << 20


def _to_dev(a, device, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.to(device)


def bf16_tensor(bits_u16, device):
    """Device bf16 tensor from bf16 bit patterns held in a uint16 numpy array."""
    return _to_dev(np.asarray(bits_u16, dtype=np.uint16).view(np.int16), device, torch.bfloat16)


class PagedKV:
    """A paged KV cache pool plus its block manager."""

    def __init__(self, num_blocks, num_kv_heads, head_dim, kv_dtype, free_order=None, prefix_cache=True,
                 device="cuda", fill=None):
        self.num_blocks, self.Hkv, self.D, self.dtype = int(num_blocks), int(num_kv_heads), int(head_dim), kv_dtype
        self.device = torch.device(device)
        self.alloc = Allocator(num_blocks, free_order, prefix_cache)
        shape = (self.num_blocks, self.Hkv, BLOCK, self.D)
        tdt = TORCH_DTYPE[kv_dtype]
        self.k_cache = torch.empty(shape, dtype=tdt, device=self.device)
        self.v_cache = torch.empty(shape, dtype=tdt, device=self.device)
        if fill is not None:
            self.k_cache.fill_(fill)
            self.v_cache.fill_(fill)
        self.k_scale = self.v_scale = None
        if kv_dtype == I8:
            self.k_scale = torch.zeros((self.num_blocks, self.Hkv), dtype=torch.float32, device=self.device)
            self.v_scale = torch.zeros_like(self.k_scale)

    def store(self, slots, k_rows, v_rows, k_scale_rows=None, v_scale_rows=None):
        """Scatter device rows [n][Hkv][D] to device int32 slots[n]."""
        kv_store(k_rows, v_rows, slots, self.k_cache, self.v_cache, k_scale_rows, v_scale_rows,
                 self.k_scale, self.v_scale)

    def store_quant(self, slots, k_rows, v_rows, runs=None):
        """int8 pools: quantise bf16/fp32 device rows [n][Hkv][D] into the cache at slots[n]; ``runs`` as
        :func:`store_runs` gives them, uploaded (built from a host copy of ``slots`` when None)."""
        kv_store_quant(k_rows, v_rows, slots, self.k_cache, self.v_cache, self.k_scale, self.v_scale, runs=runs)

    def split_workspace(self, nbytes):
        """Device scratch for split prefill partials, grown on demand and reused by later chunks
        (calls on one stream never overlap); None when nothing is split."""
        if nbytes <= 0:
            return None
        ws = getattr(self, "_split_ws", None)
        if ws is None or ws.numel() < nbytes:
            ws = self._split_ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return ws

    def copy_on_write(self, src, dst, rows):
        """Enqueue the block copies src[i] -> dst[i] of rows 0..rows[i]-1 (host int32, from
        append_batch_cow) on the current stream; they must precede the store of the batch's rows."""
        n = len(src)
        if n:
            t = _to_dev(np.concatenate([src, dst, rows]).astype(np.int32), self.device)
            copy_blocks(t[:n], t[n:2 * n], self.k_cache, self.v_cache, t[2 * n:], self.k_scale, self.v_scale)


class DecodeBatch:
    """A batch of sequences in decode: history admitted and stored, then one token per step
    (``fused``: the step's store and attention in one launch, pkv_decode_store_attend)."""

    def __init__(self, kv, Hq, seq_ids, max_context_len, max_splits=0, fused=False, window=0, cow=False,
                 group_size=0, group_min_shared=GROUP_MIN_SHARED, group_splits=0):
        self.kv = kv
        self.Hq = int(Hq)
        self.ids = np.asarray(seq_ids, dtype=np.int64)
        self.B = len(self.ids)
        self.max_blocks = max(1, -(-int(max_context_len) // BLOCK))
        self.max_context_len = int(max_context_len)
        self.max_splits = max_splits
        self.fused = fused
        self.window = int(window)  # > 0: sliding-window attention over the last `window` keys
        self.cow = bool(cow)  # sequences share blocks (forks): appends copy shared partial blocks
        # > 0: sequences k*group_size .. k*group_size + group_size - 1 are forks of one request.  A step
        # whose groups share at least group_min_shared keys on average, and more than
        # GROUP_MIN_SHARED_BYTES of K/V in all, reads them once per group
        # (pkv_paged_attn_decode_grouped); shorter or fewer shared prefixes stay in the caches when
        # every sequence reads them, and the per-sequence kernel is faster there.  group_min_shared
        # = 0 takes the grouped kernel every step.
        self.group_size = int(group_size)
        self.group_min_shared = int(group_min_shared)
        # > 1: a grouped step cuts each group's shared keys into up to group_splits splits, merged
        # by log-sum-exp (pkv_paged_attn_decode_grouped_split), so that a launch of few groups does
        # not leave CUs idle; 0: about one workgroup per CU, at most GROUP_MAX_SPLITS splits
        if group_splits <= 0 and group_size:
            cus = torch.cuda.get_device_properties(kv.device).multi_processor_count
            group_splits = max(1, min(GROUP_MAX_SPLITS, cus // max(1, len(seq_ids) // group_size * kv.Hkv)))
        self.group_splits = max(1, int(group_splits))
        self.max_shared = 0
        self.grouped = False  # the path the last uploaded step takes
        if self.fused and self.window:
            raise ValueError("the fused store+attend step has no sliding window")
        if self.group_size and (self.fused or self.window or self.B % self.group_size):
            raise ValueError("grouped attention needs B a multiple of group_size, no window and no fused step")
        dev = kv.device
        self._desc = desc_of(kv.k_cache)
        # pinned staging for the per-step metadata: slots[B] | lens[B] | order[B] | tables[B][max_blocks]
        # and, with cow, the step's block copies: src[B] | dst[B] | rows[B]
        nmeta = 3 * self.B + self.B * self.max_blocks
        ncow = 3 * self.B if self.cow else 0
        ngroups = self.B // self.group_size if self.group_size else 0
        self._pin = torch.empty(nmeta + ncow + ngroups, dtype=torch.int32).pin_memory()
        self._meta = torch.empty_like(self._pin, device=dev)
        self._copied = torch.cuda.Event()
        self._copied.record()
        self.slots = self._meta[:self.B]
        self.context_lens = self._meta[self.B:2 * self.B]
        self.seq_order = self._meta[2 * self.B:3 * self.B]
        self.block_tables = self._meta[3 * self.B:nmeta].view(self.B, self.max_blocks)
        pin = self._pin.numpy()
        p32 = ctypes.POINTER(ctypes.c_int32)
        self._order_args = (ctypes.byref(self._desc), self.Hq, self.B, pin[self.B:].ctypes.data_as(p32),
                            self.max_context_len, int(max_splits), self.window, 0, 0,
                            pin[2 * self.B:].ctypes.data_as(p32))
        self._cow = self._meta[nmeta:nmeta + ncow]
        self._groups_at = nmeta + ncow
        self.shared_lens = self._meta[self._groups_at:self._groups_at + ngroups]  # per group
        self._group_ws = None
        self.n_copies = 0
        # the split plan the library uses: a window of W keys spans at most ceil((W + 255) / 256) blocks
        span = min(self.max_context_len, self.window + BLOCK - 1) if self.window else self.max_context_len
        self.splits, self.blocks_per_split = decode_plan(self.B, kv.Hkv, span, max_splits)
        nbytes = decode_workspace_bytes(self.B, self.Hq, kv.D, kv.Hkv, self.max_context_len, max_splits)
        self.workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)

    def set_sequences(self, seq_ids):
        """Point the batch at another set of B admitted sequences (e.g. the next step's beams)."""
        ids = np.asarray(seq_ids, dtype=np.int64)
        if len(ids) != self.B:
            raise ValueError(f"the batch holds {self.B} sequences, got {len(ids)}")
        self.ids = ids

    def upload_step_metadata(self, slots, copies=None):
        """Block tables and lengths of every sequence plus the new tokens' slots (and, with cow, the
        step's block copies (src, dst, rows)): one pinned H2D copy."""
        self.fill_step_metadata(slots, copies)
        self._meta.copy_(self._pin, non_blocking=True)
        self._copied.record()

    def fill_step_metadata(self, slots, copies=None):
        """The host half of :meth:`upload_step_metadata`: fill the pinned staging buffer."""
        self._copied.synchronize()  # the previous copy has left the staging buffer
        pin = self._pin.numpy()
        B, mb = self.B, self.max_blocks
        pin[:B] = slots
        if copies is not None:
            n = self.n_copies = len(copies[0])
            cow = pin[3 * B + B * mb:]
            for i, c in enumerate(copies):
                cow[i * B:i * B + n] = c
        tab = pin[3 * B:3 * B + B * mb].reshape(B, mb)
        lens = pin[B:2 * B]
        self.kv.alloc.block_tables(self.ids, mb, out=tab, context_lens=lens)
        self.host_context_lens, self.host_block_tables = lens, tab  # valid until the next upload
        if self.group_size:
            ng = B // self.group_size
            sh = pin[self._groups_at:self._groups_at + ng]
            decode_group_shared_lens(tab, lens, self.group_size, out=sh)
            self.host_shared_lens = sh
            self.max_shared = int(sh.max()) if ng else 0
            shared_bytes = int(sh.sum()) * self.kv.Hkv * self.kv.D * self.kv.k_cache.element_size() * 2
            self.grouped = self.group_min_shared == 0 or bool(
                sh.mean() >= self.group_min_shared and shared_bytes >= GROUP_MIN_SHARED_BYTES)
            if self.grouped:
                return
        # longest contexts first; when the whole launch is resident at once, balanced per CU
        # (pkv_decode_launch_order, called with pointers bound once: it runs every step)
        _check(lib().pkv_decode_launch_order(*self._order_args), "pkv_decode_launch_order")

    def step(self, tokens, q, k_new, v_new, softmax_scale, out=None, k_scale_new=None, v_scale_new=None):
        """One decode step: append one token per sequence, store its K/V, attend.  Returns out [B][Hq][D]."""
        if self.cow:
            slots, src, dst, rows = self.kv.alloc.append_batch_cow(self.ids, tokens)
            self.upload_step_metadata(slots, (src, dst, rows))
            self.copy_on_write()
        else:
            self.upload_step_metadata(self.kv.alloc.append_batch(self.ids, tokens))
        if self.fused:
            return self.store_attend(q, k_new, v_new, softmax_scale, out, k_scale_new, v_scale_new)
        self.kv.store(self.slots, k_new, v_new, k_scale_new, v_scale_new)
        return self.attend(q, softmax_scale, out)

    def copy_on_write(self):
        """The uploaded step's copy-on-write block copies (must precede the store)."""
        n, B, kv = self.n_copies, self.B, self.kv
        if n:
            c = self._cow
            copy_blocks(c[:n], c[B:B + n], kv.k_cache, kv.v_cache, c[2 * B:2 * B + n], kv.k_scale, kv.v_scale)

    def store_attend(self, q, k_new, v_new, softmax_scale, out=None, k_scale_new=None, v_scale_new=None):
        """The step's store of the new tokens and its attention, in one launch."""
        kv = self.kv
        return decode_store_attend(q, k_new, v_new, self.slots, kv.k_cache, kv.v_cache, self.block_tables,
                                  self.context_lens, self.max_context_len, softmax_scale, out=out,
                                  workspace=self.workspace, max_splits=self.max_splits, k_scale=kv.k_scale,
                                  v_scale=kv.v_scale, k_scale_new=k_scale_new, v_scale_new=v_scale_new,
                                  seq_order=self.seq_order)

    def attend(self, q, softmax_scale, out=None):
        if self.grouped and self.group_splits > 1:
            if self._group_ws is None:  # sized for the largest plan: group_splits splits
                nb = decode_grouped_workspace_bytes(self.B, self.Hq, self.kv.D, BLOCK * self.group_splits,
                                                    self.group_splits)
                self._group_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=self.kv.device)
            return paged_attn_decode_grouped_split(q, self.kv.k_cache, self.kv.v_cache, self.block_tables,
                                                   self.context_lens, self.max_context_len, softmax_scale,
                                                   self.group_size, self.shared_lens, self.max_shared,
                                                   self.group_splits, workspace=self._group_ws, out=out,
                                                   k_scale=self.kv.k_scale, v_scale=self.kv.v_scale)
        if self.grouped:
            return paged_attn_decode_grouped(q, self.kv.k_cache, self.kv.v_cache, self.block_tables,
                                             self.context_lens, self.max_context_len, softmax_scale, self.group_size,
                                             self.shared_lens, out=out, k_scale=self.kv.k_scale,
                                             v_scale=self.kv.v_scale)
        return paged_attn_decode(q, self.kv.k_cache, self.kv.v_cache, self.block_tables, self.context_lens,
                                self.max_context_len, softmax_scale, out=out, workspace=self.workspace,
                                max_splits=self.max_splits, k_scale=self.kv.k_scale, v_scale=self.kv.v_scale,
                                seq_order=self.seq_order, window=self.window)


class GraphedDecodeBatch:
    """A :class:`DecodeBatch` whose device work is replayed from HIP graphs ("1200行代码挑战vLLM",
    性能优化 §4 CUDA图支持: captured graphs cut per-launch overhead), captured on first use:
    graph 1 holds the pinned metadata upload and the store (or the fused store + attend), graph 2
    the attention (none when fused).  Two staging sets alternate, each with its own graphs, so the
    host fills step i+1's metadata while step i runs.  The captured kernels read fixed device
    buffers: the caller writes each step's inputs into ``q``, ``k_new``, ``v_new`` (int8 pools:
    ``k_scale_new``, ``v_scale_new`` too) before :meth:`step`; the result lands in ``out``.  The
    input buffers are views of one byte buffer, ``inputs``, so one copy can fill them all
    (:meth:`pack_inputs` lays out such a copy source).  B, the context capacity and the split
    plan are fixed at construction."""

    def __init__(self, kv, Hq, seq_ids, max_context_len, softmax_scale, max_splits=0, fused=False):
        self.kv = kv
        self.fused = bool(fused)
        self.scale = float(softmax_scale)
        self.sets = [DecodeBatch(kv, Hq, seq_ids, max_context_len, max_splits, fused=fused) for _ in range(2)]
        self.sets[1].workspace = self.sets[0].workspace  # one stream: the steps never overlap
        self.B, dev = self.sets[0].B, kv.device
        qdt = torch.float32 if kv.dtype == F32 else torch.bfloat16
        self._layout = [("q", (self.B, Hq, kv.D), qdt), ("k_new", (self.B, kv.Hkv, kv.D), TORCH_DTYPE[kv.dtype]),
                        ("v_new", (self.B, kv.Hkv, kv.D), TORCH_DTYPE[kv.dtype])]
        if kv.dtype == I8:
            self._layout += [("k_scale_new", (self.B, kv.Hkv), torch.float32),
                             ("v_scale_new", (self.B, kv.Hkv), torch.float32)]
        self.inputs = torch.zeros(self._offsets()[-1], dtype=torch.uint8, device=dev)
        self.k_scale_new = self.v_scale_new = None
        for name, t in zip([x[0] for x in self._layout], self.unpack(self.inputs)):
            setattr(self, name, t)
        self.out = torch.empty_like(self.q)
        self.graphs = [None, None]
        self.steps = 0

    @property
    def ids(self):
        return self.sets[0].ids

    def _offsets(self):
        off = [0]
        for _, shape, dt in self._layout:
            n = int(np.prod(shape)) * torch.empty((), dtype=dt).element_size()
            off.append(off[-1] + -(-n // 256) * 256)
        return off

    def unpack(self, buf):
        """Typed views (q, k_new, v_new[, k_scale_new, v_scale_new]) of a byte buffer laid out like
        ``inputs``."""
        off = self._offsets()
        return [buf[off[i]:off[i + 1]][:int(np.prod(shape)) * torch.empty((), dtype=dt).element_size()]
                .view(dt).view(shape) for i, (_, shape, dt) in enumerate(self._layout)]

    def pack_inputs(self, *tensors):
        """A byte buffer laid out like ``inputs`` holding the given step inputs (same order)."""
        buf = torch.zeros_like(self.inputs)
        for view, t in zip(self.unpack(buf), tensors):
            view.copy_(t)
        return buf

    def _capture(self, j):
        b = self.sets[j]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1, stream=side):
            b._meta.copy_(b._pin, non_blocking=True)
            if self.fused:
                b.store_attend(self.q, self.k_new, self.v_new, self.scale, self.out, self.k_scale_new,
                               self.v_scale_new)
            else:
                self.kv.store(b.slots, self.k_new, self.v_new, self.k_scale_new, self.v_scale_new)
        g2 = None
        if not self.fused:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2, stream=side):
                b.attend(self.q, self.scale, self.out)
        torch.cuda.current_stream().wait_stream(side)
        self.graphs[j] = (g1, g2)

    def step(self, tokens, events=None):
        """Append one token per sequence (host), then replay the step's graphs on the current
        stream.  ``events`` = (start, end) are recorded around the attention.  Returns ``out``."""
        j = self.steps % 2
        b = self.sets[j]
        b.fill_step_metadata(self.kv.alloc.append_batch(b.ids, tokens))
        if self.graphs[j] is None:
            self._capture(j)
        g1, g2 = self.graphs[j]
        if events is not None and g2 is None:
            events[0].record()
        g1.replay()
        b._copied.record()  # the staging buffer may be refilled once graph 1 has run
        if g2 is not None:
            if events is not None:
                events[0].record()
            g2.replay()
        if events is not None:
            events[1].record()
        self.steps += 1
        return self.out


def admit_and_store(kv, seq_ids, token_lists, k_rows, v_rows, k_scale_rows=None, v_scale_rows=None):
    """Admit prompts and store the KV rows of their uncached tokens (as a prefill would).

    k_rows[i], v_rows[i]: numpy [len_i][Hkv][D] per prompt (float32, bf16 bits as uint16, or int8);
    scale rows [len_i][Hkv] float32 for int8 caches.  Returns the cached-prefix length per prompt.
    """
    ncached = [kv.alloc.add_seq(s, t) for s, t in zip(seq_ids, token_lists)]
    total = sum(len(t) - c for t, c in zip(token_lists, ncached))
    cu, lk, slots = kv.alloc.prefill_slots(seq_ids, total)
    if total == 0:
        return ncached
    dev = kv.device
    sel = [slice(c, None) for c in ncached]
    def rows(arrs):
        a = np.concatenate([r[s] for r, s in zip(arrs, sel)])
        return bf16_tensor(a, dev) if kv.dtype == BF16 else _to_dev(a, dev)

    ks = vs = None
    if kv.dtype == I8:
        ks = _to_dev(np.concatenate([r[s] for r, s in zip(k_scale_rows, sel)]), dev)
        vs = _to_dev(np.concatenate([r[s] for r, s in zip(v_scale_rows, sel)]), dev)
    kv.store(_to_dev(slots, dev), rows(k_rows), rows(v_rows), ks, vs)
    return ncached


def _attend_chunk(kv, q_new, k_new, v_new, cu, lk, slots, tab, softmax_scale, causal, out):
    """Upload a chunk's metadata and its split work order (pkv_prefill_split_order: the work order,
    with long items cut into key-range pieces when the launch would leave CUs idle) in one copy,
    store the new rows, and attend in that order."""
    dev = kv.device
    B, n_new, mb = len(lk), len(slots), tab.shape[1]
    Hq = q_new.shape[1]
    desc = desc_of(kv.k_cache)
    pieces, merges, n_slots, tile_rows = prefill_split_order(desc, Hq, cu, lk, causal)
    meta = _to_dev(np.concatenate([cu, lk, slots, tab.ravel(), pieces.ravel(), merges.ravel()]).astype(np.int32),
                   dev)
    d_cu, d_lk = meta[:B + 1], meta[B + 1:2 * B + 1]
    d_slots = meta[2 * B + 1:2 * B + 1 + n_new]
    o = 2 * B + 1 + n_new
    d_tab = meta[o:o + B * mb].view(B, mb)
    o += B * mb
    d_pieces = meta[o:o + pieces.size].view(-1, 4)
    d_merges = meta[o + pieces.size:].view(-1, 4)
    kv.store(d_slots, k_new, v_new)
    n_q = np.diff(cu)
    return paged_attn_prefill_split(q_new, d_cu, d_lk, int(n_q.max()), int(lk.max()), kv.k_cache, kv.v_cache,
                                    d_tab, softmax_scale, d_pieces, d_merges, n_slots, tile_rows,
                                    kv.split_workspace(prefill_split_workspace_bytes(desc, Hq, n_slots, tile_rows)),
                                    causal, out=out)


def prefill_segments(kv, segments, q_new, k_new, v_new, softmax_scale, causal=True, out=None):
    """One prefill chunk made of segments (seq_id, start, end) of admitted sequences' new tokens, so
    that a prompt longer than the chunk's token budget is computed over several chunks: store the
    segments' K/V, then attend (each segment sees its cached prefix, earlier segments and itself).

    q_new [n][Hq][D], k_new/v_new [n][Hkv][D] (device bf16, segments in order).
    """
    n_new = int(q_new.shape[0])
    ids = [s[0] for s in segments]
    cu, lk, slots = kv.alloc.prefill_segment_slots(ids, [s[1] for s in segments], [s[2] for s in segments], n_new)
    # a table row holds all of the sequence's blocks, including those of later segments
    tab, lens = kv.alloc.block_tables(ids, kv.num_blocks)
    mb = max(1, -(-int(lens.max()) // BLOCK))
    tab = np.ascontiguousarray(tab[:, :mb])
    return _attend_chunk(kv, q_new, k_new, v_new, cu, lk, slots, tab, softmax_scale, causal, out)


def prefill_chunk(kv, seq_ids, q_new, k_new, v_new, softmax_scale, causal=True, out=None):
    """One prefill chunk over already-admitted sequences: store the new tokens' K/V, then attend.

    q_new [n_new][Hq][D], k_new/v_new [n_new][Hkv][D] (device bf16, in sequence order).
    """
    n_new = int(q_new.shape[0])
    cu, lk, slots = kv.alloc.prefill_slots(seq_ids, n_new)
    mb = max(1, -(-int(lk.max()) // BLOCK))
    tab, _ = kv.alloc.block_tables(seq_ids, mb)
    return _attend_chunk(kv, q_new, k_new, v_new, cu, lk, slots, tab, softmax_scale, causal, out)
