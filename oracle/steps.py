"""The oracle's whole hot path on a generated workload (TEST INFRASTRUCTURE ONLY).

Takes the seeded inputs drawn by ``workloads`` (plain dicts of NumPy arrays) and runs them through
the oracle's own block manager, store and attention, in the order an engine step would: admit the
prompts (history), store their rows, append the new token, store it, attend.  Imports nothing
but the oracle and NumPy.
"""

import numpy as np

from . import allocator as OA
from . import attention as OT


def _f64(a):
    """float64 values of float32 arrays or of bf16 bit patterns held in uint16 arrays."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _rows(seq, dtype):
    if dtype == "i8":
        return seq["kq"], seq["vq"], seq["k_tok_scale"], seq["v_tok_scale"]
    return seq["k"], seq["v"], None, None


def decode_step(wl, window=0):
    """One decode step of a decode workload; returns float64 outputs [B][Hq][D].  ``window`` > 0:
    sliding-window attention over each sequence's last ``window`` keys."""
    cfg = wl["cfg"]
    dtype = cfg["dtype"]
    B, Hkv, D = len(wl["lens"]), cfg["Hkv"], cfg["D"]
    a = OA.Allocator(wl["num_blocks"], wl["free_order"])
    ids = list(range(B))
    for b, s in enumerate(wl["seqs"]):
        a.add_seq(b, s["tokens"][:-1])
    _, _, slots = a.prefill_slots(ids)
    new_slots = [a.append(b, int(s["tokens"][-1])) for b, s in enumerate(wl["seqs"])]
    shape = (wl["num_blocks"], Hkv, 256, D)
    rows = [_rows(s, dtype) for s in wl["seqs"]]

    def cat(i, sl):  # i: 0 K rows, 1 V rows, 2 K scales, 3 V scales
        xs = [r[i][sl] for r in rows]
        if i < 2 and dtype != "i8":
            xs = [_f64(x) for x in xs]
        return np.concatenate(xs)

    hist, new = slice(0, -1), slice(-1, None)
    if dtype == "i8":
        kc, vc = np.zeros(shape, np.int8), np.zeros(shape, np.int8)
        ksc = np.zeros((wl["num_blocks"], Hkv), np.float32)
        vsc = np.zeros_like(ksc)
        kc, vc, ksc, vsc = OT.kv_store(kc, vc, cat(0, hist), cat(1, hist), slots, ksc, vsc, cat(2, hist), cat(3, hist))
        kc, vc, ksc, vsc = OT.kv_store(kc, vc, cat(0, new), cat(1, new), new_slots, ksc, vsc, cat(2, new), cat(3, new))
    else:
        kc, vc = np.zeros(shape), np.zeros(shape)
        ksc = vsc = None
        kc, vc = OT.kv_store(kc, vc, cat(0, hist), cat(1, hist), slots)
        kc, vc = OT.kv_store(kc, vc, cat(0, new), cat(1, new), new_slots)
    mb = max(1, -(-max(wl["lens"]) // 256))
    tables = a.block_tables(ids, mb)
    q = np.stack([_f64(s["q"]) for s in wl["seqs"]])
    return OT.decode(q, kc, vc, tables, wl["lens"], 1.0 / np.sqrt(D), ksc, vsc, window=window)


def decode_one_sequence(cfg, seq, L, window=0):
    """Attention of one sequence's query over its own contiguous rows (sampled full-size checks);
    ``window`` > 0: over its last ``window`` rows only."""
    G = cfg["Hq"] // cfg["Hkv"]
    D = cfg["D"]
    lo = max(0, L - window) if window > 0 else 0
    if cfg["dtype"] == "i8":
        k = seq["kq"][lo:L].astype(np.float64) * seq["k_tok_scale"][lo:L, :, None].astype(np.float64)
        v = seq["vq"][lo:L].astype(np.float64) * seq["v_tok_scale"][lo:L, :, None].astype(np.float64)
    else:
        k, v = _f64(seq["k"][lo:L]), _f64(seq["v"][lo:L])
    q = _f64(seq["q"])
    return np.stack([OT.attend(q[h], k[:, h // G], v[:, h // G], 1.0 / np.sqrt(D)) for h in range(cfg["Hq"])])


def prefill_run(wl, causal=True, prefix_cache=True):
    """The whole chunked prefill workload on the oracle.

    Admits every prompt in order (prefix hits included), packs them into chunks of at most
    cfg["chunk"] new tokens, and per chunk stores the new rows then attends.  Returns
    (outputs float64 [total_new][Hq][D] in prompt order, n_cached per prompt, chunks).
    """
    cfg = wl["cfg"]
    Hkv, D = cfg["Hkv"], cfg["D"]
    prompts = wl["prompts"]
    a = OA.Allocator(wl["num_blocks"], wl["free_order"], prefix_cache=prefix_cache)
    ncached = [a.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
    chunks, cur, tot = [], [], 0
    for i, n in enumerate(n_new):
        if cur and tot + n > cfg["chunk"]:
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
        kn = np.concatenate([_f64(prompts[i]["k"][ncached[i]:]) for i in ch])
        vn = np.concatenate([_f64(prompts[i]["v"][ncached[i]:]) for i in ch])
        qn = np.concatenate([_f64(prompts[i]["q"][ncached[i]:]) for i in ch])
        kc, vc = OT.kv_store(kc, vc, kn, vn, slots)
        tables = a.block_tables(ch, max(1, -(-max(lk) // 256)))
        outs.append(OT.prefill(qn, kc, vc, tables, cu, lk, 1.0 / np.sqrt(D), causal))
    return np.concatenate(outs), ncached, chunks
