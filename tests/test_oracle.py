"""Pins of the oracle (CPU only): each test checks the oracle against something other than itself.

* published FNV-1a vectors and closed forms for the block hash;
* hand-derived block-manager outcomes;
* closed forms and a hand-worked example for attention;
* PyTorch's fp64 scaled_dot_product_attention on the CPU (a library special case);
* pure-Python brute force (math.exp, no NumPy) on tiny shapes;
* invariances: physical block permutation, shared prefixes.
"""

import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import allocator as OA
from oracle import attention as OT

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLOCK = 256


# ----------------------------------------------------------------------------- hash
def _golden_fnv():
    rows = []
    for line in open(os.path.join(GOLDEN, "fnv1a64.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        data, h = line.split()
        rows.append((b"" if data == "-" else bytes.fromhex(data), int(h, 16)))
    return rows


@pytest.mark.parametrize("data,expected", _golden_fnv())
def test_fnv1a64_published_vectors(data, expected):
    assert OA.fnv1a64(data) == expected


def test_block_hash_closed_forms():
    prime, off, m = 0x100000001B3, 0xCBF29CE484222325, 1 << 64
    # all-zero input: xor with 0 is a no-op, so the hash is offset * prime^(8 + 4*256)
    assert OA.block_hash(0, [0] * 256) == off * pow(prime, 1032, m) % m
    # prev = 1 sets only the first byte (little-endian u64)
    assert OA.block_hash(1, [0] * 256) == ((off ^ 1) * pow(prime, 1032, m)) % m
    # token 1 in the first slot sets byte 8 (little-endian i32 after the 8 prev bytes)
    h = off * pow(prime, 8, m) % m
    h = ((h ^ 1) * prime) % m
    assert OA.block_hash(0, [1] + [0] * 255) == h * pow(prime, 1023, m) % m
    # token -1 is 0xffffffff (two's complement)
    assert OA.block_hash(0, [-1] + [0] * 255) == OA.fnv1a64(bytes(8) + b"\xff" * 4 + bytes(1020))


# ------------------------------------------------------------------------ allocator
def _alloc(n, order=None, prefix=True, **kw):
    return OA.Allocator(n, list(range(n)) if order is None else order, prefix_cache=prefix, **kw)


def test_tiny_workload_needs_six_blocks():
    cfg = W.config("tiny_fp32")
    a = _alloc(8, order=[5, 2, 7, 0, 3, 6, 1, 4])
    for b, L in enumerate(cfg["ctx"]):
        a.add_seq(b, list(range(1000 * b, 1000 * b + L - 1)))
        a.append(b, 99)
    assert a.num_free() == 2
    tables = a.block_tables(range(4), 3)
    # FIFO: ctx 1 -> 0 prompt blocks, append pops 5; ctx 255 -> 2; ctx 256 -> 7; ctx 600 -> 0, 3, 6
    assert tables == [[5, -1, -1], [2, -1, -1], [7, -1, -1], [0, 3, 6]]
    a.check_invariants()


def test_slot_is_block_times_256_plus_offset():
    a = _alloc(4, order=[3, 1, 0, 2])
    a.add_seq(7, list(range(300)))
    cu, lk, slots = a.prefill_slots([7])
    assert cu == [0, 300] and lk == [300]
    assert slots == [3 * 256 + p for p in range(256)] + [1 * 256 + p for p in range(44)]
    assert a.append(7, 5) == 1 * 256 + 44


def test_prefix_hit_shares_blocks_and_counts_refs():
    base = list(range(512))
    a = _alloc(10)
    assert a.add_seq(0, base + [1, 2, 3]) == 0
    assert a.add_seq(1, base + [9] * 100) == 512
    t = a.block_tables([0, 1], 3)
    assert t[0][:2] == t[1][:2] and t[0][2] != t[1][2]
    assert a.ref[t[0][0]] == 2 and a.ref[t[0][1]] == 2 and a.ref[t[1][2]] == 1
    cu, lk, slots = a.prefill_slots([1])
    assert cu == [0, 100] and lk == [612] and slots[0] == t[1][2] * 256
    a.check_invariants()


def test_block_holding_last_prompt_token_never_hits():
    base = list(range(512))
    a = _alloc(10)
    a.add_seq(0, base)
    # identical 512-token prompt: block 1 holds the last token, so only block 0 hits
    assert a.add_seq(1, base) == 256
    a.check_invariants()


def test_hits_must_be_a_contiguous_prefix():
    const = lambda prev, toks: 42  # every full block collides on one hash value
    a = _alloc(10, hash_fn=const)
    a.add_seq(0, [1] * 256 + [2] * 256 + [3])
    # block 0 differs (guard rejects), so block 1 may not hit even though its tokens match
    assert a.add_seq(1, [7] * 256 + [2] * 256 + [3]) == 0
    a.check_invariants()


def test_collision_guard_compares_tokens():
    const = lambda prev, toks: 42
    a = _alloc(10, hash_fn=const)
    a.add_seq(0, [1] * 256 + [5])
    assert a.add_seq(1, [2] * 256 + [5]) == 0     # same hash, other tokens: miss
    assert a.add_seq(2, [2] * 256 + [6]) == 256   # last writer (seq 1's block) wins
    a.check_invariants()


def test_lazy_release_and_fifo_reuse():
    a = _alloc(6, order=[4, 1, 5, 0, 2, 3])
    a.add_seq(0, list(range(600)))          # blocks 4, 1, 5
    a.free_seq(0)                            # back to the tail in reverse: 5, 1, 4
    assert list(a.free) == [0, 2, 3, 5, 1, 4]
    # a prompt with the same first 512 tokens hits the freed (still hashed) blocks 4 and 1
    assert a.add_seq(1, list(range(512)) + [7]) == 512
    assert a.block_tables([1], 3) == [[4, 1, 0]]
    assert list(a.free) == [2, 3, 5]
    a.check_invariants()


def test_popped_block_forgets_its_hash():
    a = _alloc(2, order=[0, 1])
    a.add_seq(0, list(range(256)) + [1])      # block 0 hashed, block 1 partial
    a.free_seq(0)                              # free: 1, 0
    a.add_seq(1, [9] * 300)                    # pops 1, then 0 (its old entry is dropped)
    a.free_seq(1)
    assert a.add_seq(2, list(range(256)) + [1]) == 0
    a.check_invariants()


def test_no_blocks_is_atomic():
    a = _alloc(3)
    a.add_seq(0, list(range(300)))
    snap = (list(a.free), list(a.ref), dict(a.table), set(a.seqs))
    with pytest.raises(OA.AllocError) as e:
        a.add_seq(1, list(range(1000, 1600)))
    assert e.value.kind == "NO_BLOCKS"
    assert (list(a.free), list(a.ref), dict(a.table), set(a.seqs)) == snap


def test_no_blocks_counts_hit_blocks_taken_from_the_free_list():
    a = _alloc(3)
    a.add_seq(0, list(range(512)) + [1])  # uses all 3 blocks
    a.free_seq(0)
    # needs blocks 0,1 as hits (taken from the free list) + 2 misses: 4 > 3
    with pytest.raises(OA.AllocError):
        a.add_seq(1, list(range(512)) + [2] * 300)
    a.check_invariants()


def test_error_kinds():
    a = _alloc(4)
    a.add_seq(0, [1, 2])
    with pytest.raises(OA.AllocError) as e:
        a.add_seq(0, [1])
    assert e.value.kind == "DUP_SEQ"
    a.free_seq(0)
    with pytest.raises(OA.AllocError) as e:
        a.free_seq(0)
    assert e.value.kind == "UNKNOWN_SEQ"
    with pytest.raises(OA.AllocError) as e:
        a.append(5, 1)
    assert e.value.kind == "UNKNOWN_SEQ"
    a.add_seq(1, list(range(600)))
    with pytest.raises(OA.AllocError) as e:
        a.block_tables([1], 2)
    assert e.value.kind == "SMALL_BUFFER"


def test_append_hashes_full_block_for_later_reuse():
    a = _alloc(8)
    a.add_seq(0, list(range(255)))
    a.append(0, 255)                          # block 0 now full -> registered
    a.append(0, 256)                          # pops a new block
    assert a.add_seq(1, list(range(256)) + [5]) == 256
    a.check_invariants()


def test_random_ops_keep_invariants():
    rnd = random.Random(3)
    a = _alloc(64, order=list(np.random.default_rng(3).permutation(64)))
    live, nid = [], 0
    for _ in range(400):
        op = rnd.random()
        try:
            if op < 0.35:
                n = rnd.randint(0, 900)
                toks = [rnd.randint(0, 3) for _ in range(min(n, 512))] + [rnd.randint(0, 99) for _ in range(max(0, n - 512))]
                a.add_seq(nid, toks)
                live.append(nid)
                nid += 1
            elif op < 0.8 and live:
                a.append(rnd.choice(live), rnd.randint(0, 99))
            elif live:
                a.free_seq(live.pop(rnd.randrange(len(live))))
        except OA.AllocError as e:
            assert e.kind == "NO_BLOCKS"
        a.check_invariants()


def test_fork_shares_every_block_and_copies_on_write():
    a = _alloc(10)
    a.add_seq(0, list(range(300)))            # blocks 0 (full) and 1 (44 tokens)
    a.fork(0, 1)
    assert a.seqs[1].blocks == [0, 1] and a.ref[:2] == [2, 2] and a.seq_len(1) == 300
    with pytest.raises(OA.AllocError) as e:
        a.append(1, 7)                        # shared partial block: only with copy-on-write
    assert e.value.kind == "INVALID"
    slot, src, dst = a.append_cow(1, 7)       # the child moves to the next fresh block
    assert (src, dst) == (1, 2) and slot == 2 * 256 + 44
    assert a.seqs[1].blocks == [0, 2] and a.ref[:3] == [2, 1, 1]
    slot, src, dst = a.append_cow(0, 8)       # the parent now owns block 1 alone: no copy
    assert (src, dst) == (-1, -1) and slot == 1 * 256 + 44
    a.fork(1, 2)
    for t in range(211):                      # child 2 fills the shared block's copy; the first append copies
        slot, src, dst = a.append_cow(2, t)
        assert (src, dst) == ((2, 3) if t == 0 else (-1, -1))
    assert a.seqs[2].blocks == [0, 3] and a.seq_len(2) == 512
    slot, src, dst = a.append_cow(2, 0)       # a full last block: a fresh one, nothing to copy
    assert (src, dst) == (-1, -1) and a.seqs[2].blocks == [0, 3, 4]
    for sid in (0, 1, 2):
        a.free_seq(sid)
    a.check_invariants()
    assert a.num_free() == 10


def test_random_ops_with_forks_keep_invariants():
    rnd = random.Random(4)
    a = _alloc(48, order=list(np.random.default_rng(4).permutation(48)))
    live, nid = [], 0
    for _ in range(600):
        op = rnd.random()
        try:
            if op < 0.2:
                n = rnd.randint(1, 700)
                a.add_seq(nid, [rnd.randint(0, 3) for _ in range(n)])
                live.append(nid)
                nid += 1
            elif op < 0.35 and live:
                a.fork(rnd.choice(live), nid)
                live.append(nid)
                nid += 1
            elif op < 0.85 and live:
                a.append_cow(rnd.choice(live), rnd.randint(0, 3))
            elif live:
                a.free_seq(live.pop(rnd.randrange(len(live))))
        except OA.AllocError as e:
            assert e.kind == "NO_BLOCKS"
        a.check_invariants()


def test_copy_on_write_keeps_each_sequence_its_own_keys():
    """A forked sequence attends exactly what its parent did until they diverge; after each
    appends its own token, each sees its own (the copy holds the shared rows, the original block
    keeps the other owner's row)."""
    rng = np.random.default_rng(5)
    Hkv, D, nb = 2, 4, 8
    a = _alloc(nb)
    kc = rng.standard_normal((nb, Hkv, 256, D))
    vc = rng.standard_normal((nb, Hkv, 256, D))
    a.add_seq(0, list(range(300)))
    a.fork(0, 1)
    q = rng.standard_normal((2, 2, D))
    bt = np.array(a.block_tables([0, 1], 3))
    before = OT.decode(q, kc, vc, bt, [300, 300], 0.5)
    assert np.array_equal(before[0], OT.decode(q[:1], kc, vc, bt[:1], [300], 0.5)[0])
    assert np.array_equal(OT.decode(q[1:], kc, vc, bt[1:], [300], 0.5)[0], OT.decode(q[1:], kc, vc, bt[:1], [300], 0.5)[0])
    new = rng.standard_normal((2, Hkv, D))
    slots = []
    for sid in (1, 0):
        slot, src, dst = a.append_cow(sid, 9)
        if src >= 0:  # the rows in use: the appended token's offset
            kc, vc = OT.copy_blocks([kc, vc], [src], [dst], [slot % 256])
        slots.append(slot)
    kc, vc = OT.kv_store(kc, vc, new[[1, 0]], new[[1, 0]], slots)
    bt = np.array(a.block_tables([0, 1], 3))
    assert bt[0, 1] != bt[1, 1] and bt[0, 0] == bt[1, 0]
    for b in (0, 1):
        k_seq = OT.gather(kc, bt[b], 301, 0)
        k_par = OT.gather(kc, np.array(a.block_tables([0], 3))[0], 300, 0)
        assert np.array_equal(k_seq[:300], k_par)            # shared history, bit for bit
        assert np.array_equal(k_seq[300], new[b, 0])         # its own new token
    a.check_invariants()


# ------------------------------------------------------------------------- attention
def _rand_paged(rng, B, Hq, Hkv, D, lens, nb=None):
    """Random contiguous per-sequence K/V plus a random paged placement of them."""
    need = sum(-(-L // 256) for L in lens)
    nb = nb or need + 3
    perm = rng.permutation(nb)
    kc = rng.standard_normal((nb, Hkv, 256, D))
    vc = rng.standard_normal((nb, Hkv, 256, D))
    maxb = max(1, max(-(-L // 256) for L in lens))
    bt = -np.ones((B, maxb), dtype=np.int64)
    k_seq, v_seq, used = [], [], 0
    for b, L in enumerate(lens):
        nbk = -(-L // 256)
        bt[b, :nbk] = perm[used:used + nbk]
        used += nbk
        k = rng.standard_normal((L, Hkv, D))
        v = rng.standard_normal((L, Hkv, D))
        for j in range(L):
            blk, off = bt[b, j // 256], j % 256
            kc[blk, :, off] = k[j]
            vc[blk, :, off] = v[j]
        k_seq.append(k)
        v_seq.append(v)
    q = rng.standard_normal((B, Hq, D))
    return q, kc, vc, bt, k_seq, v_seq


def _sdpa(q, k, v, scale, mask=None):
    """torch SDPA in fp64 on the CPU: q [Hq][Nq][D], k/v [Hq][L][D]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None], scale=scale)[0].numpy()


def _golden_hand():
    vals = {}
    for line in open(os.path.join(GOLDEN, "hand_attention.txt")):
        if line.strip() and not line.startswith("#"):
            name, *xs = line.split()
            vals[name] = [math.sqrt(2.0) * math.log(3.0) if x == "sqrt2ln3" else float(x) for x in xs]
    return vals


def test_hand_worked_example():
    g = _golden_hand()
    kc = np.zeros((1, 1, 256, 2))
    vc = np.zeros((1, 1, 256, 2))
    kc[0, 0, 0], kc[0, 0, 1] = g["k0"], g["k1"]
    vc[0, 0, 0], vc[0, 0, 1] = g["v0"], g["v1"]
    out = OT.decode(np.array([[g["q"]]]), kc, vc, [[0]], [2], 1.0 / math.sqrt(2.0))
    assert np.allclose(out[0, 0], g["o"], atol=1e-14)
    # the probabilities themselves: o = p0 v0 + p1 v1 with v0, v1 on separate axes
    assert np.allclose(out[0, 0] / 4.0, [g["p"][0], g["p"][1]], atol=1e-14)


def test_context_one_returns_the_new_value_exactly():
    rng = np.random.default_rng(0)
    q, kc, vc, bt, _, v_seq = _rand_paged(rng, 3, 4, 2, 8, [1, 1, 1])
    out = OT.decode(q, kc, vc, bt, [1, 1, 1], 0.3)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], v_seq[b][0, h // 2])


def test_zero_query_or_equal_keys_average_the_values():
    rng = np.random.default_rng(1)
    q, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, 2, 2, 1, 4, [300, 7])
    out = OT.decode(np.zeros_like(q), kc, vc, bt, [300, 7], 0.5)
    for b in range(2):
        assert np.allclose(out[b, 0], v_seq[b][:, 0].mean(axis=0), atol=1e-13)
    kc2 = np.broadcast_to(kc[:1, :, :1], kc.shape).copy()  # every key row identical
    out2 = OT.decode(q, kc2, vc, bt, [300, 7], 0.5)
    for b in range(2):
        assert np.allclose(out2[b, 1], v_seq[b][:, 0].mean(axis=0), atol=1e-13)


def test_zero_context_gives_zero_output():
    rng = np.random.default_rng(2)
    q, kc, vc, bt, _, _ = _rand_paged(rng, 2, 2, 2, 4, [0, 3])
    out = OT.decode(q, kc, vc, bt, [0, 3], 0.5)
    assert np.all(out[0] == 0)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 4), (8, 1)])
def test_paged_decode_equals_torch_sdpa_on_contiguous(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    lens = [1, 255, 256, 257, 600]
    D = 16
    q, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, len(lens), Hq, Hkv, D, lens)
    scale = 1.0 / math.sqrt(D)
    out = OT.decode(q, kc, vc, bt, lens, scale)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        k = np.repeat(k_seq[b].transpose(1, 0, 2), G, axis=0)  # [Hq][L][D], head h reads h // G
        v = np.repeat(v_seq[b].transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(q[b][:, None, :], k, v, scale)[:, 0]
        assert np.max(np.abs(out[b] - ref)) < 1e-12


def test_decode_invariant_under_block_permutation():
    rng = np.random.default_rng(5)
    lens = [40, 513, 256]
    q, kc, vc, bt, _, _ = _rand_paged(rng, 3, 4, 2, 8, lens)
    out = OT.decode(q, kc, vc, bt, lens, 0.35)
    pi = rng.permutation(kc.shape[0])
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi], vc2[pi] = kc, vc
    bt2 = np.where(bt >= 0, pi[np.maximum(bt, 0)], -1)
    assert np.array_equal(OT.decode(q, kc2, vc2, bt2, lens, 0.35), out)


def _brute(qv, keys, vals, scale):
    """Pure Python: softmax attention of one query with math.exp and explicit sums."""
    s = [scale * sum(a * b for a, b in zip(qv, k)) for k in keys]
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    return [sum(e[j] * vals[j][d] for j in range(len(keys))) / z for d in range(len(vals[0]))]


def test_decode_matches_pure_python_brute_force():
    rng = np.random.default_rng(7)
    for trial in range(20):
        B = rng.integers(1, 3)
        D = int(rng.integers(1, 5))
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * int(rng.integers(1, 3))
        lens = [int(x) for x in rng.integers(1, 6, size=B)]
        q, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, B, Hq, Hkv, D, lens)
        out = OT.decode(q, kc, vc, bt, lens, 0.7)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                ref = _brute(q[b, h].tolist(), k_seq[b][:, g].tolist(), v_seq[b][:, g].tolist(), 0.7)
                assert np.allclose(out[b, h], ref, rtol=0, atol=1e-13)


def test_int8_dequantised_decode():
    rng = np.random.default_rng(9)
    lens = [300, 20]
    nb, Hkv, D = 4, 2, 8
    kq = rng.integers(-127, 128, size=(nb, Hkv, 256, D)).astype(np.int8)
    vq = rng.integers(-127, 128, size=(nb, Hkv, 256, D)).astype(np.int8)
    ks = rng.random((nb, Hkv)).astype(np.float32)
    vs = rng.random((nb, Hkv)).astype(np.float32)
    bt = [[2, 0], [3, -1]]
    q = rng.standard_normal((2, 4, D))
    out = OT.decode(q, kq, vq, bt, lens, 0.3, ks, vs)
    kd = kq.astype(np.float64) * ks.astype(np.float64)[:, :, None, None]
    vd = vq.astype(np.float64) * vs.astype(np.float64)[:, :, None, None]
    for b, L in enumerate(lens):
        rows = [bt[b][j // 256] for j in range(L)]
        offs = [j % 256 for j in range(L)]
        for h in range(4):
            k = kd[rows, h // 2, offs]
            v = vd[rows, h // 2, offs]
            ref = _sdpa(q[b, h][None, None], k[None], v[None], 0.3)[0, 0]
            assert np.max(np.abs(out[b, h] - ref)) < 1e-12


def _bottom_right_mask(n_q, Lk):
    i = np.arange(n_q)[:, None]
    j = np.arange(Lk)[None, :]
    return np.where(j <= Lk - n_q + i, 0.0, -np.inf)


def test_prefill_equals_sdpa_with_bottom_right_causal_mask():
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 4, 2, 8
    lens_k = [300, 5, 520]
    n_q = [45, 5, 264]  # first and last have a cached prefix
    q_all, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, 3, Hq, Hkv, D, lens_k)
    cu = np.concatenate([[0], np.cumsum(n_q)])
    q = rng.standard_normal((cu[-1], Hq, D))
    out = OT.prefill(q, kc, vc, bt, cu, lens_k, 0.4)
    for b in range(3):
        k = np.repeat(k_seq[b].transpose(1, 0, 2), 2, axis=0)
        v = np.repeat(v_seq[b].transpose(1, 0, 2), 2, axis=0)
        qb = q[cu[b]:cu[b + 1]].transpose(1, 0, 2)
        ref = _sdpa(qb, k, v, 0.4, _bottom_right_mask(n_q[b], lens_k[b])).transpose(1, 0, 2)
        assert np.max(np.abs(out[cu[b]:cu[b + 1]] - ref)) < 1e-12
    # with no cached prefix the mask is torch's own is_causal
    qb = q[cu[1]:cu[2]].transpose(1, 0, 2)
    k = np.repeat(k_seq[1].transpose(1, 0, 2), 2, axis=0)
    v = np.repeat(v_seq[1].transpose(1, 0, 2), 2, axis=0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(qb)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        is_causal=True, scale=0.4)[0].numpy().transpose(1, 0, 2)
    assert np.max(np.abs(out[cu[1]:cu[2]] - ref)) < 1e-12
    # non-causal sees every key
    out_nc = OT.prefill(q, kc, vc, bt, cu, lens_k, 0.4, causal=False)
    qb = q[cu[0]:cu[1]].transpose(1, 0, 2)
    k = np.repeat(k_seq[0].transpose(1, 0, 2), 2, axis=0)
    v = np.repeat(v_seq[0].transpose(1, 0, 2), 2, axis=0)
    assert np.max(np.abs(out_nc[cu[0]:cu[1]] - _sdpa(qb, k, v, 0.4).transpose(1, 0, 2))) < 1e-12


def test_prefill_last_row_equals_decode():
    rng = np.random.default_rng(12)
    lens = [77, 600]
    q_dec, kc, vc, bt, _, _ = _rand_paged(rng, 2, 4, 2, 8, lens)
    q = np.concatenate([np.zeros((76, 4, 8)), q_dec[0][None], np.zeros((599, 4, 8)), q_dec[1][None]])
    cu = [0, 77, 677]
    pre = OT.prefill(q, kc, vc, bt, cu, lens, 0.25)
    dec = OT.decode(q_dec, kc, vc, bt, lens, 0.25)
    assert np.max(np.abs(pre[76] - dec[0])) < 1e-13 and np.max(np.abs(pre[676] - dec[1])) < 1e-13


def test_kv_store_copies_rows_and_skips_negative_slots():
    rng = np.random.default_rng(13)
    kc = np.full((3, 2, 256, 4), 7.5)
    vc = np.full((3, 2, 256, 4), -7.5)
    kn = rng.standard_normal((4, 2, 4))
    vn = rng.standard_normal((4, 2, 4))
    slots = [2 * 256 + 5, -1, 0, 256 + 255]
    k2, v2 = OT.kv_store(kc, vc, kn, vn, slots)
    assert np.array_equal(k2[2, :, 5], kn[0]) and np.array_equal(v2[0, :, 0], vn[2])
    assert np.array_equal(k2[1, :, 255], kn[3])
    touched = np.zeros((3, 256), bool)
    for s in slots:
        if s >= 0:
            touched[s // 256, s % 256] = True
    assert np.all(k2.transpose(0, 2, 1, 3)[~touched] == 7.5)
    assert np.all(v2.transpose(0, 2, 1, 3)[~touched] == -7.5)
    assert np.all(kc == 7.5)  # input untouched


def test_shared_prefix_outputs_identical_and_prefix_cache_transparent():
    """Group members agree on their first 512 positions; a cached prefix changes no suffix output."""
    cfg = W.config("prefill_prefix", B=3, ctx=[700, 530, 600], Hq=2, Hkv=1, D=8, group=8)
    wl = W.prefill_workload(cfg, 0)
    res = {}
    for prefix in (False, True):
        a = OA.Allocator(wl["num_blocks"], wl["free_order"], prefix_cache=prefix)
        ncached = [a.add_seq(i, p["tokens"]) for i, p in enumerate(wl["prompts"])]
        cu, lk, slots = a.prefill_slots(range(3))
        kn = np.concatenate([W.bf16_bits_to_f32(p["k"][c:]) for p, c in zip(wl["prompts"], ncached)])
        vn = np.concatenate([W.bf16_bits_to_f32(p["v"][c:]) for p, c in zip(wl["prompts"], ncached)])
        qn = np.concatenate([W.bf16_bits_to_f32(p["q"][c:]) for p, c in zip(wl["prompts"], ncached)])
        kc = np.zeros((wl["num_blocks"], 1, 256, 8))
        vc = np.zeros_like(kc)
        kc, vc = OT.kv_store(kc, vc, kn, vn, slots)
        out = OT.prefill(qn, kc, vc, a.block_tables(range(3), 3), cu, lk, 0.3)
        res[prefix] = (ncached, cu, out)
    nc, cu, out = res[False]
    assert nc == [0, 0, 0]
    for i in (1, 2):
        assert np.array_equal(out[cu[i]:cu[i] + 512], out[cu[0]:cu[0] + 512])
    nc1, cu1, out1 = res[True]
    assert nc1 == [0, 512, 512]
    for i in (1, 2):
        n = cu[i + 1] - cu[i]
        assert np.allclose(out1[cu1[i]:cu1[i + 1]], out[cu[i] + 512:cu[i] + n], atol=1e-13, rtol=0)


# -------------------------------------------------------------------- sliding-window attention
def test_window_one_returns_the_newest_value():
    rng = np.random.default_rng(21)
    q, kc, vc, bt, _, v_seq = _rand_paged(rng, 3, 4, 2, 8, [1, 300, 513])
    out = OT.decode(q, kc, vc, bt, [1, 300, 513], 0.3, window=1)
    for b, L in enumerate([1, 300, 513]):
        for h in range(4):
            assert np.array_equal(out[b, h], v_seq[b][L - 1, h // 2])
    cu = [0, 1, 41, 141]
    qn = rng.standard_normal((141, 4, 8))
    outp = OT.prefill(qn, kc, vc, bt, cu, [1, 300, 513], 0.3, window=1)
    for b, (L, nq) in enumerate(zip([1, 300, 513], [1, 40, 100])):
        for i in range(nq):
            for h in range(4):
                assert np.array_equal(outp[cu[b] + i, h], v_seq[b][L - nq + i, h // 2])


def test_window_covering_every_key_is_full_attention():
    rng = np.random.default_rng(22)
    lens = [300, 7, 600]
    q, kc, vc, bt, _, _ = _rand_paged(rng, 3, 4, 2, 8, lens)
    assert np.array_equal(OT.decode(q, kc, vc, bt, lens, 0.3, window=600), OT.decode(q, kc, vc, bt, lens, 0.3))
    cu = [0, 50, 57, 157]
    qn = rng.standard_normal((157, 4, 8))
    full = OT.prefill(qn, kc, vc, bt, cu, lens, 0.3)
    assert np.array_equal(OT.prefill(qn, kc, vc, bt, cu, lens, 0.3, window=600), full)
    assert not np.allclose(OT.prefill(qn, kc, vc, bt, cu, lens, 0.3, window=599), full)


def test_windowed_decode_matches_pure_python_brute_force():
    rng = np.random.default_rng(23)
    for trial in range(20):
        B = int(rng.integers(1, 3))
        D = int(rng.integers(1, 5))
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * int(rng.integers(1, 3))
        lens = [int(x) for x in rng.integers(1, 9, size=B)]
        w = int(rng.integers(1, 6))
        q, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, B, Hq, Hkv, D, lens)
        out = OT.decode(q, kc, vc, bt, lens, 0.7, window=w)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                keys = k_seq[b][:, g].tolist()[-w:]
                vals = v_seq[b][:, g].tolist()[-w:]
                assert np.allclose(out[b, h], _brute(q[b, h].tolist(), keys, vals, 0.7), rtol=0, atol=1e-13)


def _band_mask(n_q, L, window):
    """Bottom-right causal mask limited to the last ``window`` keys of each query."""
    m = np.full((n_q, L), -np.inf)
    for i in range(n_q):
        p = L - n_q + i
        m[i, max(0, p - window + 1):p + 1] = 0.0
    return m


def test_windowed_prefill_equals_sdpa_with_band_mask():
    rng = np.random.default_rng(24)
    Hq, Hkv, D = 4, 2, 8
    lens_k = [300, 5, 520]
    n_q = [45, 5, 264]
    q_all, kc, vc, bt, k_seq, v_seq = _rand_paged(rng, 3, Hq, Hkv, D, lens_k)
    cu = np.concatenate([[0], np.cumsum(n_q)])
    q = rng.standard_normal((cu[-1], Hq, D))
    for window in (1, 3, 64, 100, 257):
        out = OT.prefill(q, kc, vc, bt, cu, lens_k, 0.4, window=window)
        for b in range(3):
            k = np.repeat(k_seq[b].transpose(1, 0, 2), 2, axis=0)
            v = np.repeat(v_seq[b].transpose(1, 0, 2), 2, axis=0)
            qb = q[cu[b]:cu[b + 1]].transpose(1, 0, 2)
            ref = _sdpa(qb, k, v, 0.4, _band_mask(n_q[b], lens_k[b], window)).transpose(1, 0, 2)
            assert np.max(np.abs(out[cu[b]:cu[b + 1]] - ref)) < 1e-12, (window, b)


def test_windowed_prefill_last_row_equals_windowed_decode():
    rng = np.random.default_rng(25)
    lens = [300, 600]
    q, kc, vc, bt, _, _ = _rand_paged(rng, 2, 4, 2, 8, lens)
    cu = [0, 20, 70]
    qn = rng.standard_normal((70, 4, 8))
    qn[19], qn[69] = q[0], q[1]
    outp = OT.prefill(qn, kc, vc, bt, cu, lens, 0.3, window=130)
    outd = OT.decode(q, kc, vc, bt, lens, 0.3, window=130)
    assert np.allclose(outp[[19, 69]], outd, rtol=0, atol=1e-13)


# ------------------------------------------------------------------- int8 quantising store
def _golden_int8_store():
    vals = {}
    for line in open(os.path.join(GOLDEN, "int8_store.txt")):
        if line.strip() and not line.startswith("#"):
            name, *xs = line.split()
            vals[name] = [float(x) for x in xs]
    return vals


def _quant_cache(nb, hkv, d):
    return (np.zeros((nb, hkv, BLOCK, d), dtype=np.int8), np.zeros((nb, hkv, BLOCK, d), dtype=np.int8),
            np.zeros((nb, hkv), dtype=np.float32), np.zeros((nb, hkv), dtype=np.float32))


def test_int8_store_hand_example():
    g = _golden_int8_store()
    kc, vc, ks, vs = _quant_cache(1, 1, 2)
    for c in (1, 2, 3):
        off = int(g[f"call{c}_offset"][0])
        rows = np.array(g[f"call{c}_rows"], dtype=np.float32).reshape(-1, 1, 2)
        slots = np.arange(off, off + rows.shape[0])
        kc, vc, ks, vs = OT.kv_store_quant(kc, vc, ks, vs, rows, -rows, slots)
        codes = np.array(g[f"call{c}_codes"], dtype=np.int8).reshape(-1, 2)
        m, e = g[f"call{c}_scale"]
        assert ks[0, 0] == np.float32(math.ldexp(m, int(e))) and vs[0, 0] == ks[0, 0]
        assert np.array_equal(kc[0, 0, :codes.shape[0]], codes)
        assert np.array_equal(vc[0, 0, :codes.shape[0]], -codes)  # V took the negated rows


def _rint_even(fr):
    fl = math.floor(fr)
    rem = fr - fl
    if rem != Fraction(1, 2):
        return fl + (1 if rem > Fraction(1, 2) else 0)
    return fl if fl % 2 == 0 else fl + 1


def _store_quant_exact(cache, scale, new, slots):
    """The quantising store in exact rational arithmetic, pure Python (no NumPy arithmetic):
    quotients are exact and rounded half to even; the scale is absmax/127 rounded to fp64 and
    then to fp32, as the rule states."""
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
        for h in range(len(scale[blk])):
            amax = max(abs(Fraction(float(new[r][h][d]))) for r in range(t, t1) for d in range(len(new[r][h])))
            cand = Fraction(float(np.float32(float(amax / 127))))
            old = Fraction(float(scale[blk][h])) if o0 > 0 else Fraction(0)
            s_new = max(old, cand)
            if o0 > 0 and s_new > old:
                for r in range(o0):
                    cache[blk][h][r] = [max(-127, min(127, _rint_even(c * old / s_new))) for c in cache[blk][h][r]]
            for r in range(t, t1):
                cache[blk][h][o0 + r - t] = [0 if s_new == 0 else max(-127, min(127, _rint_even(Fraction(float(x)) / s_new)))
                                             for x in new[r][h]]
            scale[blk][h] = float(s_new)
        t = t1


def test_int8_store_matches_exact_rational_brute_force():
    rng = np.random.default_rng(7)
    nb, hkv, d = 3, 2, 4
    kc, vc, ks, vs = _quant_cache(nb, hkv, d)
    ex_cache = [[[[0] * d for _ in range(BLOCK)] for _ in range(hkv)] for _ in range(nb)]
    ex_scale = [[0.0] * hkv for _ in range(nb)]
    # a prompt store (run from offset 0, a skipped row, a second block), then appends whose
    # values sometimes raise the block's absmax, a zero row, and a store into a reused block
    calls = [
        [0, 1, 2, -1, 256, 257],
        [3], [4], [258], [5], [6], [259],
        [512, 513, 514, 515], [516], [0, 1],
    ]
    for i, slots in enumerate(calls):
        x = rng.standard_normal((len(slots), hkv, d)).astype(np.float32) * np.float32(2.0 ** rng.integers(-3, 4))
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
        if i == 4:
            x[:] = 0.0
        kc, vc, ks, vs = OT.kv_store_quant(kc, vc, ks, vs, x, x, np.array(slots))
        _store_quant_exact(ex_cache, ex_scale, x.tolist(), slots)
        assert np.array_equal(kc, np.array(ex_cache, dtype=np.int8)), f"call {i}"
        assert np.array_equal(ks, np.array(ex_scale, dtype=np.float32)), f"call {i}"
        assert np.array_equal(vc, kc) and np.array_equal(vs, ks)


def test_int8_store_one_shot_bounds_and_full_code_range():
    rng = np.random.default_rng(8)
    kc, vc, ks, vs = _quant_cache(2, 3, 16)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((300, 3, 16)).astype(np.float32)))
    x[256:, 2] = 0.0
    slots = np.concatenate([np.arange(256, 512), np.arange(0, 44)])  # block 1 full, block 0 partial
    kc, vc, ks, vs = OT.kv_store_quant(kc, vc, ks, vs, x, x * 3, slots)
    for blk, (lo, hi) in ((1, (0, 256)), (0, (256, 300))):
        for h in range(3):
            for cache, scale, mul in ((kc, ks, 1), (vc, vs, 3)):
                vals = x[lo:hi, h].astype(np.float64) * mul
                s = float(scale[blk, h])
                codes = cache[blk, h, :hi - lo].astype(np.float64)
                if not vals.any():
                    assert s == 0 and not codes.any()
                    continue
                assert s == np.float32(np.abs(vals).max() / 127.0)
                assert np.abs(codes).max() == 127
                assert np.abs(codes * s - vals).max() <= s / 2 * (1 + 1e-6)


def test_int8_store_appends_that_keep_the_absmax_equal_one_shot():
    rng = np.random.default_rng(9)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((40, 2, 8)).astype(np.float32)))
    x[0, :, 0] = 8.0  # the first token holds every head's absmax, so no later append re-quantises
    one = OT.kv_store_quant(*_quant_cache(1, 2, 8), x, x, np.arange(40))
    inc = _quant_cache(1, 2, 8)
    for t in range(40):
        inc = OT.kv_store_quant(*inc, x[t:t + 1], x[t:t + 1], np.array([t]))
    for a, b in zip(one, inc):
        assert np.array_equal(a, b)


def test_int8_store_requantises_by_the_scale_ratio_with_ties_to_even():
    kc, vc, ks, vs = _quant_cache(1, 1, 8)
    kc[0, 0, 0] = [1, 2, 3, -3, 5, -5, 127, -127]
    ks[0, 0] = np.float32(0.5)
    # a new row whose absmax is 127 gives scale 1.0 = twice the old one: codes halve, ties to even;
    # the new row's own quotients x / 1.0 include exact ties too
    row = np.array([[[127.0, 2.5, -2.5, 0.5, 1.5, -0.5, 3.5, 0.0]]], dtype=np.float32)
    kc, vc, ks, vs = OT.kv_store_quant(kc, vc, ks, vs, row, row, np.array([1]))
    assert ks[0, 0] == 1.0
    assert list(kc[0, 0, 0]) == [0, 1, 2, -2, 2, -2, 64, -64]
    assert list(kc[0, 0, 1]) == [127, 2, -2, 0, 2, 0, 4, 0]
    # a store at offset 0 starts a fresh block: the old scale is ignored
    small = np.zeros((1, 1, 8), dtype=np.float32)
    small[0, 0, 0] = 1.0
    kc, vc, ks, vs = OT.kv_store_quant(kc, vc, ks, vs, small, small, np.array([0]))
    assert ks[0, 0] == np.float32(1.0 / 127.0) and kc[0, 0, 0, 0] == 127


# ------------------------------------------------------------------------ generators
def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact ties round to even
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_int8_encoding_rules():
    rng = np.random.default_rng(1)
    x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((300, 2, 16)).astype(np.float32)))
    x[256:, 1] = 0.0  # second block of head 1 is all zero
    codes, tok_s, blk_s = W.int8_encode(x, 300)
    assert codes.min() >= -127 and codes.max() <= 127
    assert blk_s[1, 1] == 0 and np.all(codes[256:, 1] == 0)
    for i, (lo, hi) in enumerate([(0, 256), (256, 300)]):
        for g in range(2):
            s = blk_s[i, g]
            if s == 0:
                continue
            assert s == np.float32(np.abs(x[lo:hi, g]).max() / 127.0)
            assert np.all(tok_s[lo:hi, g] == s)
            err = np.abs(codes[lo:hi, g].astype(np.float64) * s - x[lo:hi, g])
            assert err.max() <= s / 2 * (1 + 1e-6)
            assert np.abs(codes[lo:hi, g]).max() == 127


def test_pack_chunks_greedy():
    assert W.pack_chunks([1000, 3000, 200, 4096, 1], 4096) == [[0, 1], [2], [3], [4]]


# ------------------------------------------------------ the oracle's whole-step glue (steps.py)
# These pin oracle/steps.py and Allocator.prefill_segment_slots against things that do not come
# from the oracle: torch's fp64 SDPA over each sequence's *contiguous* rows as drawn by workloads
# (no block manager, no cache, no table), hand-derived prefix-cache counts and hand-worked slots.
from oracle import steps as OS  # noqa: E402


def _seq_rows_f64(cfg, seq, lo, hi):
    """K, V rows lo..hi-1 of one drawn sequence as float64 [Hkv][n][D] (int8: codes x token scale)."""
    if cfg["dtype"] == "i8":
        k = seq["kq"][lo:hi].astype(np.float64) * seq["k_tok_scale"][lo:hi, :, None].astype(np.float64)
        v = seq["vq"][lo:hi].astype(np.float64) * seq["v_tok_scale"][lo:hi, :, None].astype(np.float64)
    elif cfg["dtype"] == "bf16":
        k = W.bf16_bits_to_f32(seq["k"][lo:hi]).astype(np.float64)
        v = W.bf16_bits_to_f32(seq["v"][lo:hi]).astype(np.float64)
    else:
        k, v = seq["k"][lo:hi].astype(np.float64), seq["v"][lo:hi].astype(np.float64)
    return k.transpose(1, 0, 2), v.transpose(1, 0, 2)


def _q_f64(cfg, x):
    return x.astype(np.float64) if cfg["dtype"] == "f32" else W.bf16_bits_to_f32(x).astype(np.float64)


def _sdpa_decode_ref(cfg, seq, L, window=0):
    """One decode query per head over the sequence's last min(L, window) contiguous rows."""
    G, D = cfg["Hq"] // cfg["Hkv"], cfg["D"]
    lo = max(0, L - window) if window > 0 else 0
    k, v = _seq_rows_f64(cfg, seq, lo, L)
    q = _q_f64(cfg, seq["q"])
    return _sdpa(q[:, None, :], np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), 1.0 / math.sqrt(D))[:, 0]


DECODE_GLUE_CASES = [
    ("tiny_fp32", {}),
    ("qwen3_decode", dict(B=3, ctx=[1, 257, 700], Hq=4, Hkv=2, D=16)),
    ("int8_decode", dict(B=3, ctx=[255, 256, 530], Hq=4, Hkv=4, D=16)),
    ("long_decode", dict(B=2, ctx=[513, 300], Hq=8, Hkv=1, D=8)),
]


@pytest.mark.parametrize("name,over", DECODE_GLUE_CASES, ids=[c[0] for c in DECODE_GLUE_CASES])
def test_decode_step_equals_sdpa_on_the_drawn_rows(name, over):
    """decode_step (admit the history, store it, append and store the new token, attend) gives, for
    every sequence, attention of its query over all of its drawn rows, the new one included: the
    store-then-attend order of "Nano-vLLM性能调优实战" §2.2 缓存复用策略, context counting the
    token just stored."""
    cfg = W.config(name, **over)
    wl = W.decode_workload(cfg, 0)
    out = OS.decode_step(wl)
    for b, (seq, L) in enumerate(zip(wl["seqs"], wl["lens"])):
        ref = _sdpa_decode_ref(cfg, seq, L)
        assert np.max(np.abs(out[b] - ref)) < 1e-12, (name, b)
        one = OS.decode_one_sequence(cfg, seq, L)
        assert np.max(np.abs(one - ref)) < 1e-12, (name, b)


@pytest.mark.parametrize("window", [1, 2, 255, 256, 257, 600])
def test_windowed_decode_step_equals_sdpa_on_the_last_rows(window):
    cfg = W.config("qwen3_decode", B=3, ctx=[1, 300, 700], Hq=4, Hkv=2, D=8)
    wl = W.decode_workload(cfg, 1)
    out = OS.decode_step(wl, window=window)
    for b, (seq, L) in enumerate(zip(wl["seqs"], wl["lens"])):
        ref = _sdpa_decode_ref(cfg, seq, L, window)
        assert np.max(np.abs(out[b] - ref)) < 1e-12, b
        assert np.max(np.abs(OS.decode_one_sequence(cfg, seq, L, window) - ref)) < 1e-12, b


def _expected_n_cached(lens, group, shared):
    """Tokens each prompt finds cached, derived by hand from the prefix-cache rules: only full
    blocks inside the group's shared tokens can match; the block holding a prompt's last token never
    hits; a block hits only if an earlier prompt of the group held it in full (it was registered
    then) and every earlier block hit too.  Nothing is freed during admission, so nothing registered
    is lost."""
    out = []
    for i, n in enumerate(lens):
        earlier = lens[(i // group) * group:i]
        k = 0
        while ((k + 1) * BLOCK <= shared and (k + 1) * BLOCK < n
               and any(m >= (k + 1) * BLOCK for m in earlier)):
            k += 1
        out.append(k * BLOCK)
    return out


PREFILL_GLUE_CASES = [
    # lengths chosen so prefixes of 0, 1 and 2 blocks hit, with prompts shorter than the shared part
    dict(B=10, ctx=[300, 700, 512, 513, 257, 256, 900, 520, 600, 1000], group=4, chunk=1500),
    dict(B=6, ctx=[1000, 100, 530, 515, 1024, 260], group=8, chunk=4096),
]


@pytest.mark.parametrize("over", PREFILL_GLUE_CASES, ids=["several_chunks", "one_chunk"])
def test_prefill_run_equals_sdpa_per_prompt(over):
    """prefill_run: every prompt's new tokens attend its whole drawn prefix with a bottom-right
    causal mask ("Nano-vLLM性能调优实战" §2.2: the cache is written, then read), whatever the
    prefix cache hit and however the prompts were packed into chunks of at most ``chunk`` new
    tokens (§3.2 关键调度参数: whole prompts, in order, each chunk filled greedily)."""
    cfg = W.config("prefill_prefix", Hq=4, Hkv=2, D=8, **over)
    wl = W.prefill_workload(cfg, 0)
    out, ncached, chunks = OS.prefill_run(wl)
    assert ncached == _expected_n_cached(wl["lens"], cfg["group"], cfg["shared"])
    n_new = [L - c for L, c in zip(wl["lens"], ncached)]
    assert [i for ch in chunks for i in ch] == list(range(len(n_new)))
    for c, ch in enumerate(chunks):
        assert sum(n_new[i] for i in ch) <= cfg["chunk"]
        if c + 1 < len(chunks):  # greedy: the next prompt did not fit
            assert sum(n_new[i] for i in ch) + n_new[chunks[c + 1][0]] > cfg["chunk"]
    assert out.shape == (sum(n_new), cfg["Hq"], cfg["D"])
    G, r = cfg["Hq"] // cfg["Hkv"], 0
    for p, L, nc in zip(wl["prompts"], wl["lens"], ncached):
        k, v = _seq_rows_f64(cfg, p, 0, L)
        q = _q_f64(cfg, p["q"][nc:L]).transpose(1, 0, 2)
        ref = _sdpa(q, np.repeat(k, G, axis=0), np.repeat(v, G, axis=0), 1.0 / math.sqrt(cfg["D"]),
                    _bottom_right_mask(L - nc, L)).transpose(1, 0, 2)
        assert np.max(np.abs(out[r:r + L - nc] - ref)) < 1e-12
        r += L - nc
    assert r == out.shape[0]
    # with the prefix cache off every token is new, and the outputs of the shared tokens repeat
    out0, nc0, _ = OS.prefill_run(wl, prefix_cache=False)
    assert nc0 == [0] * len(wl["lens"])
    assert out0.shape[0] == sum(wl["lens"])


def test_prefill_segment_slots_hand_worked():
    """A 556-token prompt whose first block is cached has 300 new tokens, computed as segments
    [0, 256) and [256, 300) in two steps ("Nano-vLLM性能调优实战" §3.2: at most a fixed number of new
    tokens per step).  Each segment's keys are the cached prefix plus the new tokens up to its end."""
    a = _alloc(10)  # FIFO pool 0, 1, 2, ...
    base = list(range(1000, 1512))
    assert a.add_seq(0, base + [1, 2, 3]) == 0  # 515 tokens: blocks 0, 1, 2
    assert a.add_seq(1, base[:256] + list(range(5000, 5300))) == 256  # block 0 hits; pops 3, 4
    assert a.block_tables([1], 3) == [[0, 3, 4]]
    cu, lk, slots = a.prefill_segment_slots([1], [0], [256])
    assert cu == [0, 256] and lk == [512] and slots == list(range(3 * 256, 4 * 256))
    cu, lk, slots = a.prefill_segment_slots([1], [256], [300])
    assert cu == [0, 44] and lk == [556] and slots == list(range(4 * 256, 4 * 256 + 44))
    # several sequences in one call, one of them an empty segment
    cu, lk, slots = a.prefill_segment_slots([0, 1, 0], [510, 100, 0], [515, 101, 0])
    assert cu == [0, 5, 6, 6] and lk == [515, 357, 0]
    assert slots == [1 * 256 + 254, 1 * 256 + 255, 2 * 256 + 0, 2 * 256 + 1, 2 * 256 + 2, 3 * 256 + 100]
    # the whole new range as one segment is prefill_slots
    assert a.prefill_segment_slots([0, 1], [0, 0], [515, 300]) == tuple(a.prefill_slots([0, 1]))
    for bad in ([(-1, 5)], [(5, 4)], [(0, 301)]):
        with pytest.raises(OA.AllocError):
            a.prefill_segment_slots([1], [bad[0][0]], [bad[0][1]])
