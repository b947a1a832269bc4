"""Planted mistakes in the oracle (CPU only): each must make at least one pin fail.

This shows the pins in test_oracle.py are strong enough to catch the plausible
slips -- a dropped term, a wrong index or sign, a swapped operand -- in the
oracle they pin.  Mutants are patched into the oracle modules for the duration
of one check and restored afterwards.
"""

from collections import deque

import numpy as np
import pytest

from oracle import allocator as OA
from oracle import attention as OT
from oracle import steps as OS
from tests import test_oracle as P

BLOCK = 256


def _attend_no_scale(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1])
    s = k @ q
    p = np.exp(s - s.max())
    return (p / p.sum()) @ v


def _attend_unnormalised(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1])
    s = scale * (k @ q)
    return np.exp(s - s.max()) @ v


def _attend_keys_as_values(q, k, v, scale):
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1])
    s = scale * (k @ q)
    p = np.exp(s - s.max())
    return (p / p.sum()) @ k


def _attend_drop_last_key(q, k, v, scale):
    return OT_attend_orig(q, k[:-1], v[:-1], scale) if k.shape[0] > 1 else OT_attend_orig(q, k, v, scale)


def _slot_offset_shift(row, pos):
    return int(row[pos // BLOCK]) * BLOCK + (pos + 1) % BLOCK


def _slot_wrong_block(row, pos):
    return int(row[(pos // BLOCK + 1) % len(row)]) * BLOCK + pos % BLOCK if row[-1] >= 0 else int(row[0]) * BLOCK + pos % BLOCK


def _decode_gqa_modulo(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None, v_scale=None):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        for h in range(Hq):
            g = h % Hkv
            k = OT.gather(k_cache, block_tables[b], L, g, k_scale)
            v = OT.gather(v_cache, block_tables[b], L, g, v_scale)
            out[b, h] = OT.attend(q[b, h], k, v, scale)
    return out


def _prefill_causal_off_by_one(q, k_cache, v_cache, block_tables, cu, lk, scale, causal=True):
    q = np.asarray(q, dtype=np.float64)
    Nq, Hq, D = q.shape
    G = Hq // k_cache.shape[1]
    out = np.zeros((Nq, Hq, D))
    for b in range(len(lk)):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        n_q, L = q1 - q0, int(lk[b])
        for h in range(Hq):
            k = OT.gather(k_cache, block_tables[b], L, h // G)
            v = OT.gather(v_cache, block_tables[b], L, h // G)
            for i in range(n_q):
                vis = max(1, L - n_q + i) if causal else L
                out[q0 + i, h] = OT.attend(q[q0 + i, h], k[:vis], v[:vis], scale)
    return out


def _prefill_top_left(q, k_cache, v_cache, block_tables, cu, lk, scale, causal=True):
    q = np.asarray(q, dtype=np.float64)
    Nq, Hq, D = q.shape
    G = Hq // k_cache.shape[1]
    out = np.zeros((Nq, Hq, D))
    for b in range(len(lk)):
        q0, q1 = int(cu[b]), int(cu[b + 1])
        L = int(lk[b])
        for h in range(Hq):
            k = OT.gather(k_cache, block_tables[b], L, h // G)
            v = OT.gather(v_cache, block_tables[b], L, h // G)
            for i in range(q1 - q0):
                vis = i + 1 if causal else L
                out[q0 + i, h] = OT.attend(q[q0 + i, h], k[:vis], v[:vis], scale)
    return out


def _gather_scale_ignored(cache, row, length, head, scale=None):
    return OT_gather_orig(cache, row, length, head, None)


def _fnv1(data):  # FNV-1 (multiply before xor) instead of FNV-1a
    h = 0xCBF29CE484222325
    for byte in data:
        h = (h * 0x100000001B3) & ((1 << 64) - 1)
        h ^= byte
    return h


def _block_hash_big_endian(prev, tokens):
    data = bytearray(int(prev).to_bytes(8, "big"))
    for t in tokens:
        data += int(t).to_bytes(4, "big", signed=True)
    return OA.fnv1a64(bytes(data))


def _block_hash_unchained(prev, tokens):
    return OA_block_hash_orig(0, tokens)


def _pop_lifo(self):
    b = self.free.pop()
    old = self.bhash[b]
    if old is not None and self.table.get(old) == b:
        del self.table[old]
    self.bhash[b] = None
    self.btokens[b] = None
    self.ref[b] = 1
    return b


def _free_forward(self, seq_id):
    s = self.seqs.pop(seq_id, None)
    if s is None:
        raise OA.AllocError("UNKNOWN_SEQ", str(seq_id))
    for b in s.blocks:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)


def _pop_keeps_hash(self):
    b = self.free.popleft()
    self.ref[b] = 1
    return b


def _codes_half_away(x, scale):  # rint rounding half away from zero instead of half to even
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int8)
    q = x / float(scale)
    return np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -127, 127).astype(np.int8)


def _codes_truncate(x, scale):  # truncation instead of rounding
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int8)
    return np.clip(np.trunc(x / float(scale)), -127, 127).astype(np.int8)


def _store_quant_variant(requant=True, fresh_resets=True, keep_old=True):
    def store(k_cache, v_cache, k_scale, v_scale, k_new, v_new, slot_mapping):
        kc, vc, ks, vs = k_cache.copy(), v_cache.copy(), k_scale.copy(), v_scale.copy()
        slots = [int(x) for x in slot_mapping]
        t = 0
        while t < len(slots):
            if slots[t] < 0:
                t += 1
                continue
            blk, o0 = divmod(slots[t], BLOCK)
            t1 = t + 1
            while t1 < len(slots) and slots[t1] == slots[t] + (t1 - t) and o0 + (t1 - t) < BLOCK:
                t1 += 1
            for cache, scale, new in ((kc, ks, k_new), (vc, vs, v_new)):
                for g in range(cache.shape[1]):
                    x = np.asarray(new[t:t1, g], dtype=np.float64)
                    cand = np.float32(np.abs(x).max() / 127.0)
                    old = np.float32(scale[blk, g]) if (o0 > 0 or not fresh_resets) else np.float32(0.0)
                    s_new = max(old, cand) if keep_old else cand
                    if requant and o0 > 0 and s_new > old:
                        c = cache[blk, g, :o0].astype(np.float64)
                        cache[blk, g, :o0] = np.clip(np.rint(c * float(old) / float(s_new)), -127, 127).astype(np.int8)
                    cache[blk, g, o0:o0 + (t1 - t)] = OT._int8_codes(x, s_new)
                    scale[blk, g] = s_new
            t = t1
        return kc, vc, ks, vs
    return store


def _decode_window_short(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None, v_scale=None,
                         window=0):
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    G = Hq // k_cache.shape[1]
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        for h in range(Hq):
            k = OT.gather(k_cache, block_tables[b], L, h // G, k_scale)
            v = OT.gather(v_cache, block_tables[b], L, h // G, v_scale)
            lo = max(0, L - window + 1) if window > 0 else 0   # one key short
            out[b, h] = OT.attend(q[b, h], k[lo:], v[lo:], scale)
    return out


def _prefill_window_variant(shift=0, from_start=False):
    def prefill(q, k_cache, v_cache, block_tables, cu, lk, scale, causal=True, window=0):
        q = np.asarray(q, dtype=np.float64)
        Nq, Hq, D = q.shape
        G = Hq // k_cache.shape[1]
        out = np.zeros((Nq, Hq, D))
        for b in range(len(lk)):
            q0, q1 = int(cu[b]), int(cu[b + 1])
            n_q, L = q1 - q0, int(lk[b])
            for h in range(Hq):
                k = OT.gather(k_cache, block_tables[b], L, h // G)
                v = OT.gather(v_cache, block_tables[b], L, h // G)
                for i in range(n_q):
                    vis = L - n_q + i + 1 if causal else L
                    lo = max(0, vis - window + shift) if window > 0 else 0
                    hi = vis
                    if from_start and window > 0:
                        lo, hi = 0, min(window, vis)
                    out[q0 + i, h] = OT.attend(q[q0 + i, h], k[lo:hi], v[lo:hi], scale)
        return out
    return prefill


def _append_cow_never_copies(self, seq_id, token):
    s = self.seqs[seq_id]
    pos = len(s.tokens)
    if pos % BLOCK != 0:
        self.ref[s.blocks[pos // BLOCK]] = 1   # pretend it is private: writes into the shared block
    return OA_append_orig(self, seq_id, token), -1, -1


def _append_cow_keeps_ref(self, seq_id, token):
    s = self.seqs.get(seq_id)
    pos = len(s.tokens)
    src = dst = -1
    if pos % BLOCK != 0 and self.ref[s.blocks[pos // BLOCK]] > 1:
        src = s.blocks[pos // BLOCK]
        dst = self._pop_fresh()
        s.blocks[pos // BLOCK] = dst            # the shared block keeps its old count
        self.ref[src] += 0
        saved, self.ref[src] = self.ref[src], 1
        slot = OA_append_orig(self, seq_id, token)
        self.ref[src] = saved
        return slot, src, dst
    return OA_append_orig(self, seq_id, token), src, dst


def _fork_no_refs(self, parent_id, child_id):
    p = self.seqs[parent_id]
    c = OA._Seq()
    c.blocks, c.tokens, c.n_cached, c.last_hash = list(p.blocks), list(p.tokens), len(p.tokens), p.last_hash
    self.seqs[child_id] = c


def _copy_one_row_short(caches, src, dst, rows=None):
    return OT_copy_blocks_orig(caches, src, dst, None if rows is None else [max(0, int(r) - 1) for r in rows])


def _decode_step_new_slot_late(wl, window=0):
    """decode_step with the new token's row stored one slot past the one the allocator gave it."""
    orig = OA.Allocator.append
    OA.Allocator.append = lambda self, sid, tok: orig(self, sid, tok) + 1
    try:
        return OS_decode_step_orig(wl, window)
    finally:
        OA.Allocator.append = orig


def _decode_step_context_short(wl, window=0):
    """decode_step attending the history only (context not counting the token just stored)."""
    orig = OT.decode
    OT.decode = lambda q, kc, vc, bt, lens, *a, **k: orig(q, kc, vc, bt, [max(0, L - 1) for L in lens], *a, **k)
    try:
        return OS_decode_step_orig(wl, window)
    finally:
        OT.decode = orig


def _decode_one_window_long(cfg, seq, L, window=0):
    return OS_decode_one_orig(cfg, seq, L, window + 1 if window > 0 else 0)


def _prefill_run_variant(q_from_start=False, attend_first=False, no_budget=False):
    """prefill_run with one glue slip: queries taken from the prompt's start instead of its first
    uncached token, a chunk attended before its rows are stored, or the chunk budget ignored."""
    def run(wl, causal=True, prefix_cache=True):
        cfg = wl["cfg"]
        Hkv, D = cfg["Hkv"], cfg["D"]
        prompts = wl["prompts"]
        a = OA.Allocator(wl["num_blocks"], wl["free_order"], prefix_cache=prefix_cache)
        ncached = [a.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
        n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
        budget = 1 << 30 if no_budget else cfg["chunk"]
        chunks, cur, tot = [], [], 0
        for i, n in enumerate(n_new):
            if cur and tot + n > budget:
                chunks.append(cur)
                cur, tot = [], 0
            cur.append(i)
            tot += n
        if cur:
            chunks.append(cur)
        kc = np.zeros((wl["num_blocks"], Hkv, 256, D))
        vc = np.zeros_like(kc)
        outs = []
        for ch in chunks:
            cu, lk, slots = a.prefill_slots(ch)
            kn = np.concatenate([OS._f64(prompts[i]["k"][ncached[i]:]) for i in ch])
            vn = np.concatenate([OS._f64(prompts[i]["v"][ncached[i]:]) for i in ch])
            qn = np.concatenate([OS._f64(prompts[i]["q"][0 if q_from_start else ncached[i]:]
                                         [:len(prompts[i]["tokens"]) - ncached[i]]) for i in ch])
            tables = a.block_tables(ch, max(1, -(-max(lk) // 256)))
            if attend_first:
                outs.append(OT.prefill(qn, kc, vc, tables, cu, lk, 1.0 / np.sqrt(D), causal))
            kc, vc = OT.kv_store(kc, vc, kn, vn, slots)
            if not attend_first:
                outs.append(OT.prefill(qn, kc, vc, tables, cu, lk, 1.0 / np.sqrt(D), causal))
        return np.concatenate(outs), ncached, chunks
    return run


def _segment_keys_without_prefix(self, seq_ids, starts, ends):
    cu, lk, slots = OA_segment_orig(self, seq_ids, starts, ends)
    return cu, [L - self.seqs[s].n_cached for L, s in zip(lk, seq_ids)], slots


def _segment_slots_from_sequence_start(self, seq_ids, starts, ends):
    cu, lk, _ = OA_segment_orig(self, seq_ids, starts, ends)
    slots = []
    for sid, a, b in zip(seq_ids, starts, ends):
        s = self.seqs[sid]
        slots += [s.blocks[p // BLOCK] * BLOCK + p % BLOCK for p in range(a, b)]
    return cu, lk, slots


OT_copy_blocks_orig = OT.copy_blocks
OS_decode_step_orig = OS.decode_step
OS_decode_one_orig = OS.decode_one_sequence
OA_segment_orig = OA.Allocator.prefill_segment_slots
OT_attend_orig = OT.attend
OT_gather_orig = OT.gather
OA_block_hash_orig = OA.block_hash
OA_append_orig = OA.Allocator.append

ATTN_PINS = [
    P.test_hand_worked_example,
    P.test_context_one_returns_the_new_value_exactly,
    P.test_zero_query_or_equal_keys_average_the_values,
    lambda: P.test_paged_decode_equals_torch_sdpa_on_contiguous(4, 2),
    P.test_decode_matches_pure_python_brute_force,
    P.test_int8_dequantised_decode,
    P.test_prefill_equals_sdpa_with_bottom_right_causal_mask,
]
ALLOC_PINS = [
    P.test_tiny_workload_needs_six_blocks,
    P.test_slot_is_block_times_256_plus_offset,
    P.test_prefix_hit_shares_blocks_and_counts_refs,
    P.test_block_holding_last_prompt_token_never_hits,
    P.test_lazy_release_and_fifo_reuse,
    P.test_popped_block_forgets_its_hash,
    P.test_append_hashes_full_block_for_later_reuse,
    P.test_shared_prefix_outputs_identical_and_prefix_cache_transparent,
]
QUANT_PINS = [
    P.test_int8_store_hand_example,
    P.test_int8_store_matches_exact_rational_brute_force,
    P.test_int8_store_one_shot_bounds_and_full_code_range,
    P.test_int8_store_appends_that_keep_the_absmax_equal_one_shot,
    P.test_int8_store_requantises_by_the_scale_ratio_with_ties_to_even,
]
WINDOW_PINS = [
    P.test_window_one_returns_the_newest_value,
    P.test_window_covering_every_key_is_full_attention,
    P.test_windowed_decode_matches_pure_python_brute_force,
    P.test_windowed_prefill_equals_sdpa_with_band_mask,
    P.test_windowed_prefill_last_row_equals_windowed_decode,
]
FORK_PINS = [
    P.test_fork_shares_every_block_and_copies_on_write,
    P.test_random_ops_with_forks_keep_invariants,
    P.test_copy_on_write_keeps_each_sequence_its_own_keys,
]
HASH_PINS = [lambda: [P.test_fnv1a64_published_vectors(d, e) for d, e in P._golden_fnv()],
             P.test_block_hash_closed_forms]

STEP_PINS = [
    lambda: [P.test_decode_step_equals_sdpa_on_the_drawn_rows(n, o) for n, o in P.DECODE_GLUE_CASES],
    lambda: [P.test_windowed_decode_step_equals_sdpa_on_the_last_rows(w) for w in (1, 257, 600)],
    lambda: [P.test_prefill_run_equals_sdpa_per_prompt(o) for o in P.PREFILL_GLUE_CASES],
    P.test_prefill_segment_slots_hand_worked,
]

MUTANTS = {
    "attend without the softmax scale": (OT, "attend", _attend_no_scale, ATTN_PINS),
    "attend without normalisation": (OT, "attend", _attend_unnormalised, ATTN_PINS),
    "attend weights the keys, not the values": (OT, "attend", _attend_keys_as_values, ATTN_PINS),
    "attend drops the newest key": (OT, "attend", _attend_drop_last_key, ATTN_PINS),
    "slot offset shifted by one": (OT, "slot_of", _slot_offset_shift, ATTN_PINS),
    "slot reads the wrong table entry": (OT, "slot_of", _slot_wrong_block, ATTN_PINS),
    "GQA head mapping h % Hkv": (OT, "decode", _decode_gqa_modulo, ATTN_PINS),
    "int8 scale ignored": (OT, "gather", _gather_scale_ignored, ATTN_PINS),
    "causal window one short": (OT, "prefill", _prefill_causal_off_by_one, ATTN_PINS),
    "causal mask aligned top-left": (OT, "prefill", _prefill_top_left, ATTN_PINS),
    "FNV-1 instead of FNV-1a": (OA, "fnv1a64", _fnv1, HASH_PINS),
    "block hash big-endian": (OA, "block_hash", _block_hash_big_endian, HASH_PINS),
    "block hash not chained": (OA, "block_hash", _block_hash_unchained, HASH_PINS + ALLOC_PINS),
    "free list popped LIFO": (OA.Allocator, "_pop_fresh", _pop_lifo, ALLOC_PINS),
    "free_seq in forward order": (OA.Allocator, "free_seq", _free_forward, ALLOC_PINS),
    "popped block keeps its hash": (OA.Allocator, "_pop_fresh", _pop_keeps_hash, ALLOC_PINS),
    "int8 codes round half away from zero": (OT, "_int8_codes", _codes_half_away, QUANT_PINS),
    "int8 codes truncate": (OT, "_int8_codes", _codes_truncate, QUANT_PINS),
    "int8 store never re-quantises": (OT, "kv_store_quant", _store_quant_variant(requant=False), QUANT_PINS),
    "int8 store keeps a fresh block's old scale": (OT, "kv_store_quant", _store_quant_variant(fresh_resets=False),
                                                   QUANT_PINS),
    "int8 scale from the new rows only": (OT, "kv_store_quant", _store_quant_variant(keep_old=False), QUANT_PINS),
    "decode window one key short": (OT, "decode", _decode_window_short, WINDOW_PINS),
    "copy-on-write never copies": (OA.Allocator, "append_cow", _append_cow_never_copies, FORK_PINS),
    "copy-on-write keeps the shared block's count": (OA.Allocator, "append_cow", _append_cow_keeps_ref, FORK_PINS),
    "fork takes no references": (OA.Allocator, "fork", _fork_no_refs, FORK_PINS),
    "copy-on-write copies one row short": (OT, "copy_blocks", _copy_one_row_short, FORK_PINS),
    "prefill window one key long": (OT, "prefill", _prefill_window_variant(shift=-1), WINDOW_PINS),
    "prefill window one key short": (OT, "prefill", _prefill_window_variant(shift=1), WINDOW_PINS),
    "prefill window counted from the first key": (OT, "prefill", _prefill_window_variant(from_start=True),
                                                  WINDOW_PINS),
    "decode step stores the new token one slot late": (OS, "decode_step", _decode_step_new_slot_late, STEP_PINS),
    "decode step context misses the new token": (OS, "decode_step", _decode_step_context_short, STEP_PINS),
    "one-sequence decode window one key long": (OS, "decode_one_sequence", _decode_one_window_long, STEP_PINS),
    "prefill run takes queries from the prompt start": (OS, "prefill_run", _prefill_run_variant(q_from_start=True),
                                                        STEP_PINS),
    "prefill run attends before storing the chunk": (OS, "prefill_run", _prefill_run_variant(attend_first=True),
                                                     STEP_PINS),
    "prefill run ignores the chunk budget": (OS, "prefill_run", _prefill_run_variant(no_budget=True), STEP_PINS),
    "segment key count omits the cached prefix": (OA.Allocator, "prefill_segment_slots",
                                                  _segment_keys_without_prefix, STEP_PINS),
    "segment slots counted from the sequence start": (OA.Allocator, "prefill_segment_slots",
                                                      _segment_slots_from_sequence_start, STEP_PINS),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    owner, attr, mutant, pins = MUTANTS[name]
    monkeypatch.setattr(owner, attr, mutant)
    if owner is OA and attr == "block_hash":
        # the allocator captured the module function at construction time through its default
        monkeypatch.setattr(OA.Allocator, "__init__", _init_with(OA.Allocator.__init__, mutant))
    caught = 0
    for pin in pins:
        try:
            pin()
        except (AssertionError, OA.AllocError, ValueError, IndexError):
            caught += 1
    assert caught > 0, f"no pin caught the planted mistake: {name}"


def _init_with(init, h):
    def wrapped(self, *a, **kw):
        if kw.get("hash_fn") is None:
            kw["hash_fn"] = h
        init(self, *a, **kw)
    return wrapped
