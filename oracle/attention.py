"""Oracle attention over a paged KV cache (NumPy, float64).  TEST INFRASTRUCTURE ONLY.

Paging changes only *where* the K/V rows of a sequence live, never what is
computed (ocdem.com nano-vllm article, §2.1 PagedAttention: logical blocks of a
sequence are mapped through a block table onto physically scattered blocks).
So every function below first gathers a sequence's rows through its block
table and then applies plain softmax attention: scores are scale * q·k (the
Q·Kᵀ product of the intelliparadigm.com Nano-vLLM article, §2.2 混合精度计算流水线),
probabilities are the softmax of the scores, the output is the probability-
weighted sum of the value rows.

Readings (the pages state no formula, layout or head mapping):

* cache layout: K and V are each ``[num_blocks][num_kv_heads][256][head_dim]``;
  the row of token slot ``s`` for KV head ``g`` is ``cache[s // 256, g, s % 256]``
  (all indexing goes through :func:`kv_row` / :func:`gather`);
* slot of logical position j of a sequence: ``table[j // 256] * 256 + j % 256``;
* query head h reads KV head ``h // (Hq // Hkv)``;
* decode: the context length includes the token just stored; length 0 gives a
  zero output;
* prefill (varlen, causal): query i of a sequence with n_q new tokens and
  Lk keys in total sits at position ``Lk - n_q + i`` and sees keys 0..that
  position (bottom-right alignment, so a cached prefix is visible to all
  new tokens);
* int8 caches are dequantised as ``q * scale[block, g]`` in float64 with one
  scale per (physical block, KV head).

All inputs are converted to float64 before any arithmetic.
"""

import numpy as np

BLOCK = 256


def kv_row(cache, slot, head):
    """The cache row holding token slot ``slot`` for KV head ``head``."""
    return cache[slot // BLOCK, head, slot % BLOCK]


def slot_of(table_row, pos):
    """Physical slot of logical position ``pos`` under a block-table row."""
    return int(table_row[pos // BLOCK]) * BLOCK + pos % BLOCK


def kv_store(k_cache, v_cache, k_new, v_new, slot_mapping, k_scale=None, v_scale=None,
             k_scale_new=None, v_scale_new=None):
    """store_kvcache: write each new token's K/V rows at its slot ("Nano-vLLM性能调优实战", §2.2 缓存复用策略).

    Returns new arrays; rows with slot < 0 are skipped.  For int8 caches the
    per-row scales of the new tokens are written to their block's scale entry.
    """
    k_cache = k_cache.copy()
    v_cache = v_cache.copy()
    if k_scale is not None:
        k_scale = k_scale.copy()
        v_scale = v_scale.copy()
    for t, s in enumerate(slot_mapping):
        s = int(s)
        if s < 0:
            continue
        for g in range(k_cache.shape[1]):
            k_cache[s // BLOCK, g, s % BLOCK] = k_new[t, g]
            v_cache[s // BLOCK, g, s % BLOCK] = v_new[t, g]
            if k_scale is not None:
                k_scale[s // BLOCK, g] = k_scale_new[t, g]
                v_scale[s // BLOCK, g] = v_scale_new[t, g]
    if k_scale is not None:
        return k_cache, v_cache, k_scale, v_scale
    return k_cache, v_cache


def _int8_codes(x, scale):
    """clamp(rint(x / scale), -127, 127) with the quotient in float64, ties to even; scale 0 -> 0."""
    if scale == 0:
        return np.zeros(x.shape, dtype=np.int8)
    return np.clip(np.rint(x / float(scale)), -127, 127).astype(np.int8)


def kv_store_quant(k_cache, v_cache, k_scale, v_scale, k_new, v_new, slot_mapping):
    """Quantising store_kvcache into int8 caches (INT8 KV is an engine option: intelliparadigm.com
    Nano-vLLM article, §2.2 混合精度计算流水线; the pages give no encoding, so the rule below is a
    reading).

    One fp32 scale per (physical block, KV head).  The new rows of one call that land in the same
    block form a run of consecutive slots (this is what the allocator hands out for a prompt's
    tokens and for a decode append).  For a run starting at offset o0 of block b, per KV head and
    separately for K and V:

    * candidate = absmax of the run's new values / 127, the quotient in float64 rounded to float32;
    * old = the block's scale if o0 > 0 (rows 0..o0-1 hold earlier codes), else 0 (a fresh block);
    * new = max(old, candidate); if new > old the earlier rows are re-quantised,
      code -> rint(code * old / new) (float64, ties to even);
    * the run's rows become clamp(rint(x / new), -127, 127) (float64 quotient, ties to even), all
      zero when new == 0, and the block's scale becomes new.

    Rows with slot < 0 are skipped.  Inputs are the float values (bf16-representable or float32);
    returns new (k_cache, v_cache, k_scale, v_scale).
    """
    kc, vc = k_cache.copy(), v_cache.copy()
    ks, vs = k_scale.copy(), v_scale.copy()
    slots = [int(x) for x in slot_mapping]
    n = len(slots)
    t = 0
    while t < n:
        if slots[t] < 0:
            t += 1
            continue
        blk, o0 = divmod(slots[t], BLOCK)
        t1 = t + 1
        while t1 < n and slots[t1] == slots[t] + (t1 - t) and o0 + (t1 - t) < BLOCK:
            t1 += 1
        for cache, scale, new in ((kc, ks, k_new), (vc, vs, v_new)):
            for g in range(cache.shape[1]):
                x = np.asarray(new[t:t1, g], dtype=np.float64)
                cand = np.float32(np.abs(x).max() / 127.0)
                old = np.float32(scale[blk, g]) if o0 > 0 else np.float32(0.0)
                s_new = max(old, cand)
                if o0 > 0 and s_new > old:
                    c = cache[blk, g, :o0].astype(np.float64)
                    cache[blk, g, :o0] = np.clip(np.rint(c * float(old) / float(s_new)), -127, 127).astype(np.int8)
                cache[blk, g, o0:o0 + (t1 - t)] = _int8_codes(x, s_new)
                scale[blk, g] = s_new
        t = t1
    return kc, vc, ks, vs


def copy_blocks(caches, src, dst, rows=None):
    """Copy-on-write of shared blocks (ocdem.com nano-vllm article, §2.1): block dst[i] of every
    cache array (K, V and, for int8, the per-(block, head) scales) becomes a copy of block src[i].
    With ``rows``, only rows 0..rows[i]-1 of each KV head's K/V tile are copied: the rows the
    shared block holds when a sequence leaves it (its later rows are written before anything reads
    them); per-block arrays such as scales are copied whole.  Returns new arrays."""
    out = [c.copy() for c in caches]
    for i, (a, b) in enumerate(zip(src, dst)):
        for c in out:
            if rows is not None and c.ndim == 4:
                r = int(rows[i])
                c[int(b), :, :r] = c[int(a), :, :r]
            else:
                c[int(b)] = c[int(a)]
    return out


def gather(cache, table_row, length, head, scale=None):
    """Rows 0..length-1 of one sequence for one KV head, as float64 ``[length][D]``."""
    rows = np.empty((length, cache.shape[-1]), dtype=np.float64)
    for j in range(length):
        s = slot_of(table_row, j)
        r = np.asarray(kv_row(cache, s, head), dtype=np.float64)
        if scale is not None:
            r = r * np.float64(scale[s // BLOCK, head])
        rows[j] = r
    return rows


def attend(q, k, v, scale):
    """Softmax attention of one query vector over rows ``k``/``v`` (all float64)."""
    if k.shape[0] == 0:
        return np.zeros(v.shape[-1], dtype=np.float64)
    s = scale * (k @ q)
    s = s - s.max()
    p = np.exp(s)
    p = p / p.sum()
    return p @ v


def decode(q, k_cache, v_cache, block_tables, context_lens, scale, k_scale=None, v_scale=None, window=0):
    """Paged decode attention: one query token per sequence.

    q ``[B][Hq][D]``; caches ``[nb][Hkv][256][D]``; block_tables ``[B][max_blocks]``;
    context_lens ``[B]``.  ``window`` > 0: sliding-window attention (intelliparadigm.com Nano-vLLM
    article, §7.2 关键优化点), the query at position L-1 sees only its last ``window`` keys
    L-window..L-1.  Returns float64 ``[B][Hq][D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        for g in range(Hkv):
            k = gather(k_cache, block_tables[b], L, g, k_scale)
            v = gather(v_cache, block_tables[b], L, g, v_scale)
            lo = max(0, L - window) if window > 0 else 0
            for h in range(g * group, (g + 1) * group):
                out[b, h] = attend(q[b, h], k[lo:], v[lo:], scale)
    return out


def prefill(q, k_cache, v_cache, block_tables, cu_seqlens_q, seqlens_k, scale, causal=True, window=0):
    """Varlen paged prefill attention.

    q ``[Nq][Hq][D]`` holds the new tokens of all sequences back to back
    (sequence b owns rows cu_seqlens_q[b]..cu_seqlens_q[b+1]-1); seqlens_k[b]
    counts all keys of sequence b, cached prefix included.  ``window`` > 0 (causal
    only): sliding-window attention, the query at position P sees keys
    P-window+1..P.  Returns float64 ``[Nq][Hq][D]``.
    """
    q = np.asarray(q, dtype=np.float64)
    Nq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    out = np.zeros((Nq, Hq, D), dtype=np.float64)
    for b in range(len(seqlens_k)):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        n_q, Lk = q1 - q0, int(seqlens_k[b])
        for g in range(Hkv):
            k = gather(k_cache, block_tables[b], Lk, g)
            v = gather(v_cache, block_tables[b], Lk, g)
            for i in range(n_q):
                visible = Lk - n_q + i + 1 if causal else Lk
                lo = max(0, visible - window) if window > 0 else 0
                for h in range(g * group, (g + 1) * group):
                    out[q0 + i, h] = attend(q[q0 + i, h], k[lo:visible], v[lo:visible], scale)
    return out
