"""The native block manager (libpkv, C++) against the oracle's (pure Python), bit for bit (CPU only)."""

import random

import numpy as np
import pytest
import torch  # noqa: F401

import paged_kv_cache_kvcache_amd as P
import workloads as W
from oracle import allocator as OA


def _pair(n, seed=0, prefix=True):
    order = np.random.default_rng(seed).permutation(n).astype(np.int32)
    return P.Allocator(n, order, prefix), OA.Allocator(n, order, prefix_cache=prefix)


def _same_state(native, oracle, ids, max_blocks):
    assert native.num_free() == oracle.num_free()
    if not ids:
        return
    tab, lens = native.block_tables(ids, max_blocks)
    assert tab.tolist() == oracle.block_tables(ids, max_blocks)
    assert lens.tolist() == [oracle.seq_len(i) for i in ids]


def _call(native_fn, oracle_fn):
    """Run the same operation on both; they must agree on the result or on the error kind."""
    try:
        expect = oracle_fn()
    except OA.AllocError as e:
        with pytest.raises(P.PkvError) as ne:
            native_fn()
        assert ne.value.kind == e.kind
        return None
    got = native_fn()
    if isinstance(got, np.ndarray):
        got = got.tolist()
    assert got == expect
    return got


@pytest.mark.parametrize("seed,prefix", [(0, True), (1, True), (2, False), (3, True)])
def test_random_operation_sequences_match_bit_for_bit(seed, prefix):
    rnd = random.Random(seed)
    native, oracle = _pair(48, seed, prefix)
    live, nid = [], 0
    shared = [rnd.randint(0, 50) for _ in range(768)]
    for _ in range(300):
        op = rnd.random()
        if op < 0.3:
            n = rnd.randint(0, 1000)
            share = rnd.choice([0, 256, 512, 700])
            toks = shared[:min(n, share)] + [rnd.randint(0, 10 ** 6) for _ in range(max(0, n - share))]
            if _call(lambda: native.add_seq(nid, toks), lambda: oracle.add_seq(nid, toks)) is not None:
                live.append(nid)
            nid += 1
        elif op < 0.55 and live:
            sid = rnd.choice(live)
            tok = rnd.randint(0, 9)
            _call(lambda: native.append(sid, tok), lambda: oracle.append(sid, tok))
        elif op < 0.75 and live:
            ids = [rnd.choice(live) for _ in range(rnd.randint(1, 6))]
            toks = [rnd.randint(0, 9) for _ in ids]
            # the oracle has no batch call: appending one by one is its definition, applied atomically
            snap_free = oracle.num_free()
            need = 0
            lens = {}
            for i in ids:
                lens.setdefault(i, oracle.seq_len(i))
                need += lens[i] % 256 == 0
                lens[i] += 1
            if need > snap_free:
                with pytest.raises(P.PkvError) as e:
                    native.append_batch(ids, toks)
                assert e.value.kind == "NO_BLOCKS"
            else:
                expect = [oracle.append(i, t) for i, t in zip(ids, toks)]
                assert native.append_batch(ids, toks).tolist() == expect
        elif op < 0.9 and live:
            sid = live.pop(rnd.randrange(len(live)))
            _call(lambda: native.free_seq(sid), lambda: oracle.free_seq(sid))
        else:
            sid = rnd.randint(0, nid + 2)
            _call(lambda: native.free_seq(sid), lambda: oracle.free_seq(sid))
            if sid in live:
                live.remove(sid)
        _same_state(native, oracle, live, 64)
        if live:
            cu, lk, slots = native.prefill_slots(live, 100000)
            ocu, olk, oslots = oracle.prefill_slots(live)
            assert cu.tolist() == ocu and lk.tolist() == olk and slots.tolist() == oslots
        oracle.check_invariants()


def test_forced_hash_collisions_match():
    native, oracle = _pair(10)
    native.debug_constant_hash(True, 42)
    oracle._hash = lambda prev, toks: 42
    live = []
    for sid, toks in enumerate([[1] * 256 + [5], [2] * 256 + [5], [2] * 256 + [6], [1] * 512 + [3],
                                [7] * 256 + [2] * 256 + [3], [2] * 256 + [1] * 256 + [9]]):
        if _call(lambda: native.add_seq(sid, toks), lambda: oracle.add_seq(sid, toks)) is not None:
            live.append(sid)
        _same_state(native, oracle, live, 4)
    assert len(live) >= 4


def test_errors_leave_state_unchanged():
    native, oracle = _pair(4)
    native.add_seq(0, list(range(700)))
    with pytest.raises(P.PkvError) as e:
        native.add_seq(1, list(range(1000, 1600)))
    assert e.value.kind == "NO_BLOCKS"
    with pytest.raises(P.PkvError) as e:
        native.add_seq(0, [1])
    assert e.value.kind == "DUP_SEQ"
    with pytest.raises(P.PkvError) as e:
        native.block_tables([0], 2)
    assert e.value.kind == "SMALL_BUFFER"
    with pytest.raises(P.PkvError) as e:
        native.prefill_slots([0], 10)
    assert e.value.kind == "SMALL_BUFFER"
    with pytest.raises(P.PkvError) as e:
        native.append_batch([0, 5], [1, 1])
    assert e.value.kind == "UNKNOWN_SEQ"
    assert native.num_free() == 1
    oracle.add_seq(0, list(range(700)))
    _same_state(native, oracle, [0], 3)


def test_bad_initial_order_is_rejected():
    with pytest.raises(P.PkvError):
        P.Allocator(4, [0, 1, 1, 2])
    with pytest.raises(P.PkvError):
        P.Allocator(4, [0, 1, 2, 4])


@pytest.mark.parametrize("name", ["tiny_fp32", "qwen3_decode", "long_decode", "int8_decode"])
def test_decode_workload_tables_match(name):
    """The block tables every decode workload runs on (full size), native vs oracle."""
    cfg = W.config(name)
    lens = W.lengths(cfg, 0)
    nb = W.pool_blocks(cfg, lens)
    order = W.free_order(cfg, 0, nb)
    native, oracle = P.Allocator(nb, order), OA.Allocator(nb, order)
    rng = np.random.default_rng(0)
    for b, L in enumerate(lens):
        toks = rng.integers(0, W.VOCAB, size=L - 1).tolist()
        assert native.add_seq(b, toks) == oracle.add_seq(b, toks)
    ids = list(range(len(lens)))
    assert native.append_batch(ids, [7] * len(ids)).tolist() == [oracle.append(i, 7) for i in ids]
    mb = -(-max(lens) // 256)
    _same_state(native, oracle, ids, mb)
    if name == "tiny_fp32":
        assert nb - native.num_free() == 6


def test_prefill_workload_prefix_sharing_matches():
    cfg = W.config("prefill_prefix")
    for seed in (0, 1, 2):
        wl = W.prefill_workload(cfg, seed)
        native = P.Allocator(wl["num_blocks"], wl["free_order"])
        oracle = OA.Allocator(wl["num_blocks"], wl["free_order"])
        nc = [native.add_seq(i, p["tokens"]) for i, p in enumerate(wl["prompts"])]
        assert nc == [oracle.add_seq(i, p["tokens"]) for i, p in enumerate(wl["prompts"])]
        # block k < 2 of the shared 512 tokens is reused when an earlier group member holds it full and
        # this prompt continues past it
        for i, n in enumerate(wl["lens"]):
            earlier = wl["lens"][i - i % 8:i]
            k = 0
            while k < 2 and any(m >= 256 * (k + 1) for m in earlier) and 256 * (k + 1) < n:
                k += 1
            assert nc[i] == 256 * k, (seed, i, n, nc[i])
        assert sum(nc) > 0
        ids = list(range(32))
        _same_state(native, oracle, ids, 4)
        cu, lk, slots = native.prefill_slots(ids, 40000)
        ocu, olk, oslots = oracle.prefill_slots(ids)
        assert (cu.tolist(), lk.tolist(), slots.tolist()) == (ocu, olk, oslots)


def test_long_prompts_split_into_chunks_match():
    """Chunked prefill of prompts longer than a chunk: the segments of every chunk (native vs
    oracle, bit for bit), and over all chunks they give exactly the whole-prompt slots."""
    cfg = W.config("prefill_long")
    for seed in (0, 1):
        wl = W.prefill_workload(cfg, seed)
        native = P.Allocator(wl["num_blocks"], wl["free_order"])
        oracle = OA.Allocator(wl["num_blocks"], wl["free_order"])
        nc = [native.add_seq(i, p["tokens"]) for i, p in enumerate(wl["prompts"])]
        assert nc == [oracle.add_seq(i, p["tokens"]) for i, p in enumerate(wl["prompts"])]
        assert nc[1] > 0 and nc[3] > 0   # the second of each pair reuses the shared prefix
        n_new = [len(p["tokens"]) - c for p, c in zip(wl["prompts"], nc)]
        chunks = W.pack_chunks_split(n_new, cfg["chunk"])
        assert all(sum(b - a for _, a, b in ch) == cfg["chunk"] for ch in chunks[:-1])
        assert 0 < sum(b - a for _, a, b in chunks[-1]) <= cfg["chunk"]
        got = {i: [] for i in range(len(n_new))}
        for ch in chunks:
            ids, st, en = [s[0] for s in ch], [s[1] for s in ch], [s[2] for s in ch]
            cu, lk, slots = native.prefill_segment_slots(ids, st, en, cfg["chunk"])
            ocu, olk, oslots = oracle.prefill_segment_slots(ids, st, en)
            assert (cu.tolist(), lk.tolist(), slots.tolist()) == (ocu, olk, oslots)
            for k, (i, a, b) in enumerate(ch):
                assert lk[k] == nc[i] + b
                got[i] += slots[cu[k]:cu[k + 1]].tolist()
        _, _, whole = native.prefill_slots(list(range(len(n_new))), sum(n_new))
        assert sum((got[i] for i in range(len(n_new))), []) == whole.tolist()


def test_segment_slots_reject_bad_segments():
    native = P.Allocator(8, list(range(8)))
    native.add_seq(0, list(range(300)))
    with pytest.raises(P.PkvError):
        native.prefill_segment_slots([0], [10], [5], 100)      # start after end
    with pytest.raises(P.PkvError):
        native.prefill_segment_slots([0], [0], [301], 400)     # past the new tokens
    with pytest.raises(P.PkvError):
        native.prefill_segment_slots([7], [0], [1], 10)        # unknown sequence
    with pytest.raises(P.PkvError):
        native.prefill_segment_slots([0], [0], [300], 100)     # capacity
    cu, lk, slots = native.prefill_segment_slots([0, 0], [0, 256], [256, 300], 300)
    assert cu.tolist() == [0, 256, 300] and lk.tolist() == [256, 300] and slots.tolist() == list(range(300))
