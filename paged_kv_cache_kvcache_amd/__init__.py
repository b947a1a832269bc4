"""Python binding of libpkv (ctypes): attention over a paged KV cache on MI355X (gfx950).

Argument marshalling only.  Every step of the path -- block management, the KV store, decode and
prefill attention -- runs inside libpkv.so (host C++ and HIP kernels); PyTorch supplies device
memory and the stream.  The names follow the C ABI in ``include/pkv.h`` without the ``pkv_``
prefix.  Importing this module does not load the library; the first call does, and fails loudly
when ``libpkv.so`` has not been built (``python -m paged_kv_cache_kvcache_amd.build``).
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
BLOCK = 256

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_NO_BLOCKS, ERR_UNKNOWN_SEQ, ERR_DUP_SEQ, ERR_SMALL_BUFFER, ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6, -7)
STATUS_NAMES = {OK: "OK", ERR_INVALID: "INVALID", ERR_UNSUPPORTED: "UNSUPPORTED", ERR_NO_BLOCKS: "NO_BLOCKS",
                ERR_UNKNOWN_SEQ: "UNKNOWN_SEQ", ERR_DUP_SEQ: "DUP_SEQ", ERR_SMALL_BUFFER: "SMALL_BUFFER",
                ERR_HIP: "HIP"}
F32, BF16, I8 = 0, 1, 2
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16, I8: torch.int8}


class PkvError(RuntimeError):
    def __init__(self, code, func, text):
        self.code = code
        self.kind = STATUS_NAMES.get(code, str(code))
        super().__init__(f"{func}: {self.kind}: {text}")


class CacheDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("kv_dtype", ctypes.c_int32)]


_i32, _i64, _u64, _f32, _vp, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_size_t)
_p32 = ctypes.POINTER(ctypes.c_int32)
_p64 = ctypes.POINTER(ctypes.c_int64)
_pdesc = ctypes.POINTER(CacheDesc)

# name -> (restype, argtypes); mirrors include/pkv.h
SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "pkv_version": (ctypes.c_char_p, []),
    "pkv_set_device_checks": (_i32, [_i32]),
    "pkv_device_error": (_i32, [_p32, _p32, _p32, _vp]),
    "pkv_alloc_create": (_i32, [_i32, _i32, _p32, _i32, ctypes.POINTER(_vp)]),
    "pkv_alloc_destroy": (None, [_vp]),
    "pkv_alloc_add_seq": (_i32, [_vp, _i64, _p32, _i32, _p32]),
    "pkv_alloc_append": (_i32, [_vp, _i64, _i32, _p32]),
    "pkv_alloc_append_batch": (_i32, [_vp, _p64, _p32, _i32, _p32]),
    "pkv_alloc_fork": (_i32, [_vp, _i64, _i64]),
    "pkv_alloc_fork_batch": (_i32, [_vp, _p64, _p64, _i32]),
    "pkv_alloc_free_batch": (_i32, [_vp, _p64, _i32]),
    "pkv_alloc_append_batch_cow": (_i32, [_vp, _p64, _p32, _i32, _p32, _p32, _p32, _p32, _p32]),
    "pkv_alloc_free_seq": (_i32, [_vp, _i64]),
    "pkv_alloc_num_free": (_i32, [_vp, _p32]),
    "pkv_alloc_block_tables": (_i32, [_vp, _p64, _i32, _i32, _p32, _p32]),
    "pkv_alloc_prefill_slots": (_i32, [_vp, _p64, _i32, _p32, _p32, _p32, _i32, _p32]),
    "pkv_alloc_debug_constant_hash": (_i32, [_vp, _i32, _u64]),
    "pkv_kv_store": (_i32, [_pdesc, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "pkv_kv_store_quant": (_i32, [_pdesc, _vp, _vp, _i32, _vp, _i32, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "pkv_alloc_prefill_segment_slots": (_i32, [_vp, ctypes.POINTER(ctypes.c_int64), _p32, _p32, _i32, _p32, _p32, _p32,
                                                _i32, ctypes.POINTER(ctypes.c_int32)]),
    "pkv_copy_blocks": (_i32, [_pdesc, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]),
    "pkv_store_runs": (_i32, [_p32, _i32, _p32, _i32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]),
    "pkv_decode_plan": (_i32, [_i32, _i32, _i32, _i32, _p32, _p32]),
    "pkv_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pkv_decode_launch_order": (_i32, [_pdesc, _i32, _i32, _p32, _i32, _i32, _i32, _i32, _i32, _p32]),
    "pkv_paged_attn_decode": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                     _i32, _f32, _vp, _vp, _sz, _vp]),
    "pkv_paged_attn_decode_noalloc": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                             _i32, _f32, _vp, _vp]),
    "pkv_paged_attn_decode_window": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _i32,
                                            _i32, _f32, _i32, _vp, _vp, _sz, _vp]),
    "pkv_decode_group_shared_lens": (_i32, [_p32, _i32, _p32, _i32, _i32, _p32]),
    "pkv_paged_attn_decode_grouped": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                             _i32, _vp, _f32, _vp, _vp]),
    "pkv_decode_grouped_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pkv_paged_attn_decode_grouped_split": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                                   _i32, _i32, _vp, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    "pkv_decode_store_attend": (_i32, [_pdesc, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i32, _vp, _vp, _i32, _i32, _f32, _vp, _vp, _sz, _vp]),
    "pkv_paged_attn_prefill": (_i32, [_pdesc, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _i32,
                                      _f32, _i32, _vp, _vp]),
    "pkv_paged_attn_prefill_window": (_i32, [_pdesc, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                             _i32, _f32, _i32, _vp, _vp]),
    "pkv_paged_attn_prefill_ordered": (_i32, [_pdesc, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                              _i32, _f32, _i32, _i32, _vp, _i32, _i32, _vp, _vp]),
    "pkv_prefill_tile_rows": (_i32, [_pdesc, _i32, _i32, _i32, _p32]),
    "pkv_prefill_work_order": (_i32, [_pdesc, _i32, _i32, _p32, _p32, _i32, _i32, _p32, _i32, _p32, _p32]),
    "pkv_prefill_split_order": (_i32, [_pdesc, _i32, _i32, _p32, _p32, _i32, _i32, _p32, _i32, _p32, _p32, _i32,
                                       _p32, _p32, _p32]),
    "pkv_prefill_split_workspace_bytes": (_sz, [_pdesc, _i32, _i32, _i32]),
    "pkv_paged_attn_prefill_split": (_i32, [_pdesc, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp,
                                            _i32, _f32, _i32, _i32, _vp, _i32, _vp, _i32, _i32, _i32, _vp, _sz,
                                            _vp, _vp]),
}

_lib = None


def lib():
    """The loaded libpkv.so (loaded after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_kvcache_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error():
    return lib().pkv_last_error().decode()


def _check(rc, func):
    if rc != OK:
        raise PkvError(rc, func, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _host_i32(values):
    import numpy as np
    a = np.ascontiguousarray(values, dtype=np.int32)
    return a, a.ctypes.data_as(_p32)


def _host_i64(values):
    import numpy as np
    a = np.ascontiguousarray(values, dtype=np.int64)
    return a, a.ctypes.data_as(_p64)


def cache_desc(num_blocks, num_kv_heads, head_dim, kv_dtype):
    return CacheDesc(int(num_blocks), BLOCK, int(num_kv_heads), int(head_dim), int(kv_dtype))


def _dtype_code(t):
    return {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8}[t.dtype]


def desc_of(k_cache):
    """Descriptor of a cache tensor laid out [num_blocks][num_kv_heads][256][head_dim]."""
    dt = {torch.float32: F32, torch.bfloat16: BF16, torch.int8: I8}[k_cache.dtype]
    nb, hkv, bs, d = k_cache.shape
    if bs != BLOCK:
        raise ValueError(f"cache block dimension is {bs}, expected {BLOCK}")
    return cache_desc(nb, hkv, d, dt)


# ------------------------------------------------------------------------------ block manager
class Allocator:
    """Host block manager (pkv_alloc_*): block tables, slot mappings, prefix reuse."""

    def __init__(self, num_blocks, initial_order=None, prefix_cache=True):
        self._h = ctypes.c_void_p()
        order = None
        if initial_order is not None:
            arr, order = _host_i32(initial_order)
            self._order = arr
        _check(lib().pkv_alloc_create(int(num_blocks), BLOCK, order, int(bool(prefix_cache)), ctypes.byref(self._h)),
               "pkv_alloc_create")
        self.num_blocks = int(num_blocks)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and h.value and _lib is not None:
            _lib.pkv_alloc_destroy(h)
            self._h = ctypes.c_void_p()

    def add_seq(self, seq_id, tokens):
        arr, p = _host_i32(tokens)
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_add_seq(self._h, int(seq_id), p, len(arr), ctypes.byref(out)), "pkv_alloc_add_seq")
        return out.value

    def append(self, seq_id, token):
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_append(self._h, int(seq_id), int(token), ctypes.byref(out)), "pkv_alloc_append")
        return out.value

    def append_batch(self, seq_ids, tokens):
        import numpy as np
        ids, pi = _host_i64(seq_ids)
        toks, pt = _host_i32(tokens)
        slots = np.empty(len(ids), dtype=np.int32)
        _check(lib().pkv_alloc_append_batch(self._h, pi, pt, len(ids), slots.ctypes.data_as(_p32)),
               "pkv_alloc_append_batch")
        return slots

    def fork(self, parent_id, child_id):
        """Admit ``child_id`` sharing every block of ``parent_id`` (parallel sampling, beam search)."""
        _check(lib().pkv_alloc_fork(self._h, int(parent_id), int(child_id)), "pkv_alloc_fork")

    def fork_batch(self, parent_ids, child_ids):
        """:meth:`fork` for each (parent, child) pair in order, atomically."""
        par, pp = _host_i64(parent_ids)
        chi, pc = _host_i64(child_ids)
        if len(par) != len(chi):
            raise ValueError("parent_ids and child_ids must have the same length")
        _check(lib().pkv_alloc_fork_batch(self._h, pp, pc, len(par)), "pkv_alloc_fork_batch")

    def free_batch(self, seq_ids):
        """:meth:`free_seq` for each id in order, atomically."""
        ids, pi = _host_i64(seq_ids)
        _check(lib().pkv_alloc_free_batch(self._h, pi, len(ids)), "pkv_alloc_free_batch")

    def append_batch_cow(self, seq_ids, tokens):
        """:meth:`append_batch` with copy-on-write: (slots, copy_src, copy_dst, copy_rows) as int32
        numpy arrays; the caller copies the rows in use of each block pair (:func:`copy_blocks`)
        before storing the batch's rows."""
        import numpy as np
        ids, pi = _host_i64(seq_ids)
        toks, pt = _host_i32(tokens)
        n = len(ids)
        slots = np.empty(n, dtype=np.int32)
        src = np.empty(max(n, 1), dtype=np.int32)
        dst = np.empty(max(n, 1), dtype=np.int32)
        rows = np.empty(max(n, 1), dtype=np.int32)
        nc = ctypes.c_int32()
        _check(lib().pkv_alloc_append_batch_cow(self._h, pi, pt, n, slots.ctypes.data_as(_p32),
                                                src.ctypes.data_as(_p32), dst.ctypes.data_as(_p32),
                                                rows.ctypes.data_as(_p32), ctypes.byref(nc)),
               "pkv_alloc_append_batch_cow")
        k = nc.value
        return slots, src[:k].copy(), dst[:k].copy(), rows[:k].copy()

    def free_seq(self, seq_id):
        _check(lib().pkv_alloc_free_seq(self._h, int(seq_id)), "pkv_alloc_free_seq")

    def num_free(self):
        out = ctypes.c_int32()
        _check(lib().pkv_alloc_num_free(self._h, ctypes.byref(out)), "pkv_alloc_num_free")
        return out.value

    def block_tables(self, seq_ids, max_blocks, out=None, context_lens=None):
        """int32 [n][max_blocks] (numpy, or fills ``out``), plus the sequences' lengths."""
        import numpy as np
        ids, pi = _host_i64(seq_ids)
        n = len(ids)
        tab = np.empty((n, max_blocks), dtype=np.int32) if out is None else out
        lens = np.empty(n, dtype=np.int32) if context_lens is None else context_lens
        _check(lib().pkv_alloc_block_tables(self._h, pi, n, int(max_blocks), tab.ctypes.data_as(_p32),
                                            lens.ctypes.data_as(_p32)), "pkv_alloc_block_tables")
        return tab, lens

    def prefill_slots(self, seq_ids, cap):
        import numpy as np
        ids, pi = _host_i64(seq_ids)
        n = len(ids)
        cu = np.empty(n + 1, dtype=np.int32)
        lk = np.empty(max(n, 1), dtype=np.int32)
        slots = np.empty(max(int(cap), 1), dtype=np.int32)
        ns = ctypes.c_int32()
        _check(lib().pkv_alloc_prefill_slots(self._h, pi, n, cu.ctypes.data_as(_p32), lk.ctypes.data_as(_p32),
                                             slots.ctypes.data_as(_p32), int(cap), ctypes.byref(ns)),
               "pkv_alloc_prefill_slots")
        return cu, lk[:n], slots[:ns.value]

    def prefill_segment_slots(self, seq_ids, starts, ends, cap):
        """As :meth:`prefill_slots` for segments [starts[i], ends[i]) of each sequence's new tokens."""
        import numpy as np
        ids, pi = _host_i64(seq_ids)
        st, ps = _host_i32(starts)
        en, pe = _host_i32(ends)
        n = len(ids)
        cu = np.empty(n + 1, dtype=np.int32)
        lk = np.empty(max(n, 1), dtype=np.int32)
        slots = np.empty(max(int(cap), 1), dtype=np.int32)
        ns = ctypes.c_int32()
        _check(lib().pkv_alloc_prefill_segment_slots(self._h, pi, ps, pe, n, cu.ctypes.data_as(_p32),
                                                     lk.ctypes.data_as(_p32), slots.ctypes.data_as(_p32), int(cap),
                                                     ctypes.byref(ns)), "pkv_alloc_prefill_segment_slots")
        return cu, lk[:n], slots[:ns.value]

    def debug_constant_hash(self, enable, value=0):
        _check(lib().pkv_alloc_debug_constant_hash(self._h, int(bool(enable)), int(value)),
               "pkv_alloc_debug_constant_hash")


# ------------------------------------------------------------------------------ device ops
def kv_store(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale_new=None, v_scale_new=None,
             k_scale=None, v_scale=None, stream=None):
    """store_kvcache: scatter k_new/v_new [n][Hkv][D] into the caches at slot_mapping[n] (int32, -1 skips)."""
    desc = desc_of(k_cache)
    n = int(slot_mapping.shape[0])
    _check(lib().pkv_kv_store(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), _ptr(k_scale_new), _ptr(v_scale_new),
                              _ptr(slot_mapping), n, _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                              _stream(stream)), "pkv_kv_store")


def set_device_checks(enable):
    """Device-data checks on or off: with them on, kernels validate the slots, block ids, lengths,
    launch order and run lists they read and report the first bad one (see :func:`device_error`)."""
    _check(lib().pkv_set_device_checks(1 if enable else 0), "pkv_set_device_checks")


def device_error(stream=None):
    """(code, where, value) of the first bad index the kernels met since the last call (code 0: none);
    clears it.  Waits for ``stream``."""
    code, where, value = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pkv_device_error(ctypes.byref(code), ctypes.byref(where), ctypes.byref(value), _stream(stream)),
           "pkv_device_error")
    return code.value, where.value, value.value


def copy_blocks(src, dst, k_cache, v_cache, rows=None, k_scale=None, v_scale=None, stream=None):
    """Copy-on-write: rows 0..rows[i]-1 (all 256 when ``rows`` is None) of every KV head of physical
    block dst[i] in both caches, and its int8 scales, become copies of block src[i]'s; src, dst,
    rows device int32 [n]."""
    desc = desc_of(k_cache)
    n = int(src.shape[0])
    if int(dst.shape[0]) != n or (rows is not None and int(rows.shape[0]) != n):
        raise ValueError("src, dst and rows must have the same length")
    _check(lib().pkv_copy_blocks(ctypes.byref(desc), _ptr(src), _ptr(dst), _ptr(rows), n, _ptr(k_cache),
                                 _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _stream(stream)), "pkv_copy_blocks")


def store_runs(slot_mapping):
    """Runs of a host int32 slot mapping for :func:`kv_store_quant`: (runs int32 [2 n_runs] as
    (first row, length) pairs, n_runs, longest run)."""
    import numpy as np
    slots, ps = _host_i32(slot_mapping)
    n = len(slots)
    runs = np.empty(2 * max(n, 1), dtype=np.int32)
    nr, mx = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pkv_store_runs(ps, n, runs.ctypes.data_as(_p32), n, ctypes.byref(nr), ctypes.byref(mx)),
           "pkv_store_runs")
    return runs[:2 * nr.value], nr.value, mx.value


def kv_store_quant(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, runs=None, stream=None):
    """Quantising store: bf16/fp32 rows k_new/v_new [n][Hkv][D] into int8 caches with one fp32 scale per
    (block, KV head), re-quantising a block's earlier rows when its scale grows.  ``runs`` = (device int32
    [2 n_runs], n_runs, longest run) from :func:`store_runs`; when None it is built from a host copy of
    ``slot_mapping``."""
    desc = desc_of(k_cache)
    n = int(slot_mapping.shape[0])
    new_dt = _dtype_code(k_new)
    if _dtype_code(v_new) != new_dt:
        raise ValueError("k_new and v_new must have the same dtype")
    if runs is None:
        r, nr, mx = store_runs(slot_mapping.cpu().numpy() if isinstance(slot_mapping, torch.Tensor) else slot_mapping)
        runs = (torch.from_numpy(r).to(k_cache.device), nr, mx)
    rt, nr, mx = runs
    _check(lib().pkv_kv_store_quant(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), new_dt, _ptr(slot_mapping), n,
                                    _ptr(rt), int(nr), int(mx), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
                                    _ptr(v_scale), _stream(stream)), "pkv_kv_store_quant")


def decode_plan(B, num_kv_heads, max_context_len, max_splits=0):
    s, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pkv_decode_plan(int(B), int(num_kv_heads), int(max_context_len), int(max_splits),
                                 ctypes.byref(s), ctypes.byref(b)), "pkv_decode_plan")
    return s.value, b.value


def decode_launch_order(desc, Hq, context_lens, max_context_len, max_splits=0, window=0, compute_units=0,
                        workgroups_per_cu=0, out=None):
    """pkv_decode_launch_order: a launch order (host int32 [B]) for a decode call of this shape.
    ``desc``: a cache descriptor (:func:`cache_desc` / :func:`desc_of`); ``context_lens``: host
    int32 [B]; ``out``: optional host int32 [B] array to fill (e.g. a view of pinned staging)."""
    import numpy as np
    lens, plens = _host_i32(context_lens)
    B = len(lens)
    if out is None:
        out = np.empty(B, dtype=np.int32)
    if out.dtype != np.int32 or out.shape != (B,) or not out.flags.c_contiguous:
        raise ValueError("out must be a contiguous int32 array of B entries")
    _check(lib().pkv_decode_launch_order(ctypes.byref(desc), int(Hq), B, plens, int(max_context_len),
                                         int(max_splits), int(window), int(compute_units), int(workgroups_per_cu),
                                         out.ctypes.data_as(_p32)), "pkv_decode_launch_order")
    return out


def decode_workspace_bytes(B, Hq, head_dim, num_kv_heads, max_context_len, max_splits=0):
    return int(lib().pkv_decode_workspace_bytes(int(B), int(Hq), int(head_dim), int(num_kv_heads),
                                                int(max_context_len), int(max_splits)))


def paged_attn_decode(q, k_cache, v_cache, block_tables, context_lens, max_context_len, softmax_scale,
                      out=None, workspace=None, max_splits=0, k_scale=None, v_scale=None, seq_order=None,
                      stream=None, window=0):
    """Decode attention; q [B][Hq][D].  Allocates ``out`` / ``workspace`` with torch when not given.
    ``seq_order`` (device int32 [B], optional): launch order of the sequences, e.g. longest first.
    ``window`` > 0: sliding window, each sequence attends its last ``window`` keys."""
    desc = desc_of(k_cache)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(B, Hq, D, desc.num_kv_heads, max_context_len, max_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if window:
        _check(lib().pkv_paged_attn_decode_window(
            ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), _ptr(seq_order),
            int(max_context_len), int(max_splits), float(softmax_scale), int(window), _ptr(out), _ptr(workspace),
            ws_bytes, _stream(stream)), "pkv_paged_attn_decode_window")
        return out
    _check(lib().pkv_paged_attn_decode(ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_cache), _ptr(v_cache),
                                       _ptr(k_scale), _ptr(v_scale), _ptr(block_tables), int(block_tables.shape[1]),
                                       _ptr(context_lens), _ptr(seq_order), int(max_context_len), int(max_splits),
                                       float(softmax_scale), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)),
           "pkv_paged_attn_decode")
    return out


def decode_group_shared_lens(block_tables, context_lens, group_size, out=None):
    """pkv_decode_group_shared_lens on host arrays: for each group of ``group_size`` consecutive
    sequences, the leading keys every member holds in the same physical blocks (int32 numpy)."""
    import numpy as np
    tab, pt = _host_i32(block_tables)
    lens, pl = _host_i32(context_lens)
    B = len(lens)
    mb = int(tab.shape[1]) if tab.ndim == 2 else 0
    res = np.empty(max(B // max(int(group_size), 1), 1), dtype=np.int32) if out is None else out
    _check(lib().pkv_decode_group_shared_lens(pt, mb, pl, B, int(group_size), res.ctypes.data_as(_p32)),
           "pkv_decode_group_shared_lens")
    return res[:B // max(int(group_size), 1)] if out is None else res


def paged_attn_decode_grouped(q, k_cache, v_cache, block_tables, context_lens, max_context_len, softmax_scale,
                              group_size, shared_lens, out=None, k_scale=None, v_scale=None, stream=None):
    """pkv_paged_attn_decode_grouped: decode for groups of ``group_size`` consecutive forked sequences
    that share their first ``shared_lens[k]`` keys (device int32 per group); q [B][Hq][D]."""
    desc = desc_of(k_cache)
    B, Hq, _ = q.shape
    if out is None:
        out = torch.empty_like(q)
    _check(lib().pkv_paged_attn_decode_grouped(
        ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), int(group_size),
        _ptr(shared_lens), float(softmax_scale), _ptr(out), _stream(stream)), "pkv_paged_attn_decode_grouped")
    return out


def decode_grouped_workspace_bytes(B, Hq, head_dim, max_shared_len, max_splits):
    """pkv_decode_grouped_workspace_bytes: the workspace of a grouped decode over splits (0: no split)."""
    return int(lib().pkv_decode_grouped_workspace_bytes(int(B), int(Hq), int(head_dim), int(max_shared_len),
                                                        int(max_splits)))


def paged_attn_decode_grouped_split(q, k_cache, v_cache, block_tables, context_lens, max_context_len, softmax_scale,
                                    group_size, shared_lens, max_shared_len, max_splits, workspace=None, out=None,
                                    k_scale=None, v_scale=None, stream=None):
    """pkv_paged_attn_decode_grouped_split: grouped decode with each group's shared keys split over up
    to ``max_splits`` workgroups per KV head and merged by log-sum-exp; ``max_shared_len`` bounds
    every entry of ``shared_lens``; ``workspace`` (device memory) of at least
    :func:`decode_grouped_workspace_bytes` bytes when that is nonzero."""
    desc = desc_of(k_cache)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = decode_grouped_workspace_bytes(B, Hq, D, max_shared_len, max_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_decode_grouped_split(
        ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), int(max_context_len), int(group_size),
        _ptr(shared_lens), int(max_shared_len), int(max_splits), float(softmax_scale), _ptr(out), _ptr(workspace),
        nbytes, _stream(stream)), "pkv_paged_attn_decode_grouped_split")
    return out


def paged_attn_decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, max_context_len, softmax_scale, out,
                              max_splits=0, k_scale=None, v_scale=None, seq_order=None, stream=None):
    """pkv_paged_attn_decode_noalloc: decode attention with the split partials in the library's own
    per-device scratch; the caller passes every input and the output ``out`` [B][Hq][D]."""
    desc = desc_of(k_cache)
    B, Hq, _ = q.shape
    _check(lib().pkv_paged_attn_decode_noalloc(
        ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), int(block_tables.shape[1]), _ptr(context_lens), _ptr(seq_order), int(max_context_len),
        int(max_splits), float(softmax_scale), _ptr(out), _stream(stream)), "pkv_paged_attn_decode_noalloc")
    return out


def decode_store_attend(q, k_new, v_new, slot_mapping, k_cache, v_cache, block_tables, context_lens, max_context_len,
                        softmax_scale, out=None, workspace=None, max_splits=0, k_scale=None, v_scale=None,
                        k_scale_new=None, v_scale_new=None, seq_order=None, stream=None):
    """One decode step's store of each sequence's new token (k_new/v_new [B][Hkv][D] in the cache
    dtype, slot_mapping [B]) and its attention, in one launch; otherwise as :func:`paged_attn_decode`."""
    desc = desc_of(k_cache)
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty_like(q)
    need = decode_workspace_bytes(B, Hq, D, desc.num_kv_heads, max_context_len, max_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_decode_store_attend(ctypes.byref(desc), _ptr(q), int(B), int(Hq), _ptr(k_new), _ptr(v_new),
                                         _ptr(k_scale_new), _ptr(v_scale_new), _ptr(slot_mapping), _ptr(k_cache),
                                         _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), _ptr(block_tables),
                                         int(block_tables.shape[1]), _ptr(context_lens), _ptr(seq_order),
                                         int(max_context_len), int(max_splits), float(softmax_scale), _ptr(out),
                                         _ptr(workspace), ws_bytes, _stream(stream)),
           "pkv_decode_store_attend")
    return out


def prefill_tile_rows(desc, Hq, B, total_q):
    """pkv_prefill_tile_rows: query tokens per work item of a prefill launch of this shape."""
    t = ctypes.c_int32()
    _check(lib().pkv_prefill_tile_rows(ctypes.byref(desc), int(Hq), int(B), int(total_q), ctypes.byref(t)),
           "pkv_prefill_tile_rows")
    return t.value


def prefill_work_order(desc, Hq, cu_seqlens_q, seqlens_k, causal=True, window=0):
    """pkv_prefill_work_order: the work items of a prefill call (host int32 array) and the query
    tile (tokens per item) they were cut with, which the ordered call must be given."""
    import numpy as np
    cu, pcu = _host_i32(cu_seqlens_q)
    lk, plk = _host_i32(seqlens_k)
    B = len(lk)
    if len(cu) != B + 1:
        raise ValueError("cu_seqlens_q must have B + 1 entries")
    cap = int(cu[-1]) + B if B else 0  # at least one query token per item
    items = np.empty(max(cap, 1), dtype=np.int32)
    n, rows = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pkv_prefill_work_order(ctypes.byref(desc), int(Hq), B, pcu, plk, int(bool(causal)), int(window),
                                        items.ctypes.data_as(_p32), cap, ctypes.byref(n), ctypes.byref(rows)),
           "pkv_prefill_work_order")
    return items[:n.value], rows.value


def paged_attn_prefill_ordered(q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache,
                               block_tables, softmax_scale, work_items, tile_rows, causal=True, window=0, out=None,
                               stream=None):
    """Varlen prefill whose work items run in the order of ``work_items`` (device int32, each
    ``(sequence << 16) | query tile``, every item of the launch exactly once), cut into query tiles
    of ``tile_rows`` tokens (both as :func:`prefill_work_order` returns them)."""
    desc = desc_of(k_cache)
    total_q, Hq, _ = q.shape
    B = int(seqlens_k.shape[0])
    if out is None:
        out = torch.empty_like(q)
    _check(lib().pkv_paged_attn_prefill_ordered(
        ctypes.byref(desc), _ptr(q), int(Hq), _ptr(cu_seqlens_q), _ptr(seqlens_k), B, int(total_q),
        int(max_seqlen_q), int(max_seqlen_k), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), float(softmax_scale), int(bool(causal)), int(window), _ptr(work_items),
        int(work_items.shape[0]), int(tile_rows), _ptr(out), _stream(stream)), "pkv_paged_attn_prefill_ordered")
    return out


def prefill_split_order(desc, Hq, cu_seqlens_q, seqlens_k, causal=True, window=0):
    """pkv_prefill_split_order: (pieces int32[n][4], merges int32[m][4], n_slots, tile_rows), host
    arrays; a launch that fills the device gets its work items unsplit and no merges."""
    import numpy as np
    cu, pcu = _host_i32(cu_seqlens_q)
    lk, plk = _host_i32(seqlens_k)
    B = len(lk)
    if len(cu) != B + 1:
        raise ValueError("cu_seqlens_q must have B + 1 entries")
    items = int(cu[-1]) + B if B else 0
    pieces = np.empty((max(8 * items, 1), 4), dtype=np.int32)
    merges = np.empty((max(items, 1), 4), dtype=np.int32)
    n, m, slots, rows = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().pkv_prefill_split_order(ctypes.byref(desc), int(Hq), B, pcu, plk, int(bool(causal)), int(window),
                                         pieces.ctypes.data_as(_p32), pieces.shape[0], ctypes.byref(n),
                                         merges.ctypes.data_as(_p32), merges.shape[0], ctypes.byref(m),
                                         ctypes.byref(slots), ctypes.byref(rows)), "pkv_prefill_split_order")
    return pieces[:n.value], merges[:m.value], slots.value, rows.value


def prefill_split_workspace_bytes(desc, Hq, n_slots, tile_rows):
    """pkv_prefill_split_workspace_bytes: the workspace of a split prefill call."""
    return int(lib().pkv_prefill_split_workspace_bytes(ctypes.byref(desc), int(Hq), int(n_slots), int(tile_rows)))


def paged_attn_prefill_split(q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache, block_tables,
                             softmax_scale, pieces, merges, n_slots, tile_rows, workspace=None, causal=True, window=0,
                             out=None, stream=None):
    """Split-K varlen prefill over ``pieces`` (device int32[n][4]) then the merge of ``merges``
    (device int32[m][4]), as :func:`prefill_split_order` gives them; ``workspace`` (device memory,
    e.g. a uint8 tensor) of at least :func:`prefill_split_workspace_bytes` bytes when n_slots > 0."""
    desc = desc_of(k_cache)
    total_q, Hq, _ = q.shape
    B = int(seqlens_k.shape[0])
    if out is None:
        out = torch.empty_like(q)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().pkv_paged_attn_prefill_split(
        ctypes.byref(desc), _ptr(q), int(Hq), _ptr(cu_seqlens_q), _ptr(seqlens_k), B, int(total_q),
        int(max_seqlen_q), int(max_seqlen_k), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        int(block_tables.shape[1]), float(softmax_scale), int(bool(causal)), int(window), _ptr(pieces),
        int(pieces.shape[0]), _ptr(merges), int(merges.shape[0]), int(n_slots), int(tile_rows), _ptr(workspace),
        wbytes, _ptr(out), _stream(stream)), "pkv_paged_attn_prefill_split")
    return out


def paged_attn_prefill(q, cu_seqlens_q, seqlens_k, max_seqlen_q, max_seqlen_k, k_cache, v_cache, block_tables,
                       softmax_scale, causal=True, out=None, stream=None, window=0):
    """Varlen prefill; q [total_q][Hq][D] bf16, cu_seqlens_q [B+1], seqlens_k [B] (device int32).
    ``window`` > 0 (causal): sliding window, the query at position P sees keys P-window+1..P."""
    desc = desc_of(k_cache)
    total_q, Hq, _ = q.shape
    B = int(seqlens_k.shape[0])
    if out is None:
        out = torch.empty_like(q)
    if window:
        if not causal:
            raise ValueError("a sliding window needs causal attention")
        _check(lib().pkv_paged_attn_prefill_window(
            ctypes.byref(desc), _ptr(q), int(Hq), _ptr(cu_seqlens_q), _ptr(seqlens_k), B, int(total_q),
            int(max_seqlen_q), int(max_seqlen_k), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
            int(block_tables.shape[1]), float(softmax_scale), int(window), _ptr(out), _stream(stream)),
            "pkv_paged_attn_prefill_window")
        return out
    _check(lib().pkv_paged_attn_prefill(ctypes.byref(desc), _ptr(q), int(Hq), _ptr(cu_seqlens_q), _ptr(seqlens_k),
                                        B, int(total_q), int(max_seqlen_q), int(max_seqlen_k), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(block_tables), int(block_tables.shape[1]),
                                        float(softmax_scale), int(bool(causal)), _ptr(out), _stream(stream)),
           "pkv_paged_attn_prefill")
    return out
