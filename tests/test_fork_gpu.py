"""Forked sequences (parallel sampling, beam search) on the GPU against the oracle.

The sequences of one request share physical blocks (ocdem.com nano-vllm article, §2.1): a fork
shares every block of its parent, and an append into a shared, partially filled block first moves
the appending sequence to a fresh copy of that block (copy-on-write).  One side runs the native
block manager, pkv_copy_blocks and the store / decode kernels; the other the oracle's block
manager, block copy, store and decode.  After every step the whole caches (codes and scales for
int8) must be equal bit for bit and the decode outputs within the dtype's tolerance.
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
import workloads as W
from oracle import allocator as OA
from oracle import attention as OT
from paged_kv_cache_kvcache_amd import runner as R
from tests.gpu_cases import check_tol, say

pytestmark = pytest.mark.gpu
NB, HKV, HQ, D = 40, 2, 8, 128
SCALE = 1.0 / math.sqrt(D)
CODE_FILL = 85


def _dev(a, device):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class Both:
    """One block pool on the GPU (native allocator) and in the oracle.

    mode "bf16": bf16 cache; "i8": int8 cache fed pre-quantised rows with per-token scales;
    "i8q": int8 cache fed bf16 rows through the quantising store."""

    def __init__(self, mode, device, seed, hkv=HKV, d=D, nb=NB):
        self.mode, self.device, self.hkv, self.d = mode, device, hkv, d
        self.rng = np.random.default_rng(seed)
        order = np.random.default_rng(seed + 100).permutation(nb).astype(np.int32)
        shape = (nb, hkv, 256, d)
        if mode == "bf16":
            self.kv = R.PagedKV(nb, hkv, d, P.BF16, order, device=device, fill=float("nan"))
            self.oc = [np.full(shape, np.nan, dtype=np.float32) for _ in range(2)]
        else:
            self.kv = R.PagedKV(nb, hkv, d, P.I8, order, device=device, fill=CODE_FILL)
            self.oc = [np.full(shape, CODE_FILL, dtype=np.int8) for _ in range(2)]
            self.oc += [np.zeros((nb, hkv), dtype=np.float32) for _ in range(2)]
        self.oa = OA.Allocator(nb, order, prefix_cache=True)

    # --- both sides --------------------------------------------------------------------------
    def add(self, sid, toks):
        nc = self.kv.alloc.add_seq(sid, toks)
        assert nc == self.oa.add_seq(sid, toks)
        _, _, slots = self.kv.alloc.prefill_slots([sid], len(toks) - nc)
        assert slots.tolist() == self.oa.prefill_slots([sid])[2]
        self.store(slots)

    def fork(self, parent, child):
        self.kv.alloc.fork(parent, child)
        self.oa.fork(parent, child)

    def free(self, sid):
        self.kv.alloc.free_seq(sid)
        self.oa.free_seq(sid)

    def store(self, slots):
        """New K/V rows for ``slots`` (host int32), written on both sides."""
        rows = [self._rows(slots) for _ in range(2)]
        sm = _dev(np.asarray(slots, dtype=np.int32), self.device)
        if self.mode == "bf16":
            self.kv.store(sm, rows[0][1], rows[1][1])
            self.oc = list(OT.kv_store(*self.oc, rows[0][0], rows[1][0], slots))
        elif self.mode == "i8":
            self.kv.store(sm, rows[0][1], rows[1][1], rows[0][3], rows[1][3])
            self.oc = list(OT.kv_store(self.oc[0], self.oc[1], rows[0][0], rows[1][0], slots, self.oc[2],
                                       self.oc[3], rows[0][2], rows[1][2]))
        else:
            self.kv.store_quant(sm, rows[0][1], rows[1][1])
            self.oc = list(OT.kv_store_quant(*self.oc, rows[0][0], rows[1][0], slots))

    def _rows(self, slots):
        """(oracle rows, device rows, oracle scales, device scales) of new tokens at ``slots``."""
        n = len(slots)
        if self.mode == "i8":
            codes = self.rng.integers(-127, 128, size=(n, self.hkv, self.d)).astype(np.int8)
            # a block keeps one scale per KV head: rows bound for one block carry the same one
            blk = np.asarray(slots, dtype=np.float32)[:, None] // 256
            sc = (0.005 + 0.0003 * blk + 0.002 * np.arange(self.hkv, dtype=np.float32)).astype(np.float32)
            return codes, _dev(codes, self.device), sc, _dev(sc, self.device)
        bits = W.f32_to_bf16_bits(self.rng.standard_normal((n, self.hkv, self.d)).astype(np.float32))
        return W.bf16_bits_to_f32(bits), R.bf16_tensor(bits, self.device), None, None

    def oracle_append(self, ids, toks):
        """The oracle's copy-on-write appends and block copies (the rows in use: each copying
        token's offset); returns (slots, src, dst, rows)."""
        res = [self.oa.append_cow(i, t) for i, t in zip(ids, toks)]
        cop = [r for r in res if r[1] >= 0]
        src, dst, rows = [r[1] for r in cop], [r[2] for r in cop], [r[0] % 256 for r in cop]
        self.oc = OT.copy_blocks(self.oc, src, dst, rows)
        return [r[0] for r in res], src, dst, rows

    def step(self, ids):
        """One token per sequence with copy-on-write, on both sides; returns the copy count."""
        toks = self.rng.integers(0, 1000, size=len(ids)).tolist()
        got = self.kv.alloc.append_batch_cow(ids, toks)
        assert [g.tolist() for g in got] == list(self.oracle_append(ids, toks))
        slots, src, dst, rows = got
        self.kv.copy_on_write(src, dst, rows)
        self.store(slots)
        return len(src)

    # --- checks ------------------------------------------------------------------------------
    def check_caches(self, what):
        torch.cuda.synchronize()
        dev = [self.kv.k_cache, self.kv.v_cache] + ([self.kv.k_scale, self.kv.v_scale] if self.mode != "bf16" else [])
        for g, ref, name in zip(dev, self.oc, ("K", "V", "K scales", "V scales")):
            got = g.float().cpu().numpy() if g.dtype == torch.bfloat16 else g.cpu().numpy()
            if not np.array_equal(got, ref, equal_nan=got.dtype.kind == "f"):
                bad = np.argwhere(~((got == ref) | (np.isnan(got) & np.isnan(ref)))) if got.dtype.kind == "f" \
                    else np.argwhere(got != ref)
                raise AssertionError(f"{what}: {name} cache differs at {len(bad)} places, first {bad[:4].tolist()}")

    def decode(self, ids, what):
        lens = [self.oa.seq_len(i) for i in ids]
        mb = -(-max(lens) // 256)
        tab, dlens = self.kv.alloc.block_tables(ids, mb)
        assert dlens.tolist() == lens and tab.tolist() == self.oa.block_tables(ids, mb)
        bits = W.f32_to_bf16_bits(self.rng.standard_normal((len(ids), HQ, D)).astype(np.float32))
        q = R.bf16_tensor(bits, self.device)
        ks, vs = (self.kv.k_scale, self.kv.v_scale) if self.mode != "bf16" else (None, None)
        out = P.paged_attn_decode(q, self.kv.k_cache, self.kv.v_cache, _dev(tab, self.device),
                                  _dev(dlens, self.device), max(lens), SCALE, k_scale=ks, v_scale=vs)
        ref = OT.decode(W.bf16_bits_to_f32(bits), *self.oc[:2], tab.tolist(), lens, SCALE,
                        *(self.oc[2:] if self.mode != "bf16" else (None, None)))
        check_tol(out.float().cpu().numpy().astype(np.float64), ref, "bf16" if self.mode == "bf16" else "i8", what)


    def decode_grouped(self, ids, group_size, hq, what, splits=()):
        """pkv_paged_attn_decode_grouped over groups of ``group_size`` consecutive ``ids`` against
        the oracle's plain decode of every sequence; returns the groups' shared lengths."""
        lens = [self.oa.seq_len(i) for i in ids]
        mb = -(-max(lens) // 256)
        tab, dlens = self.kv.alloc.block_tables(ids, mb)
        assert dlens.tolist() == lens and tab.tolist() == self.oa.block_tables(ids, mb)
        shared = P.decode_group_shared_lens(tab, dlens, group_size)
        # the definition, entry by entry: the shortest member's length, cut at the first block
        # entry where the members' tables differ
        for k, sl in enumerate(shared.tolist()):
            rows = tab[k * group_size:(k + 1) * group_size]
            n = min(lens[k * group_size:(k + 1) * group_size])
            first_diff = next((e for e in range(-(-n // 256)) if len(set(rows[:, e].tolist())) > 1), None)
            assert sl == (n if first_diff is None else min(n, 256 * first_diff)), (k, sl)
        bits = W.f32_to_bf16_bits(self.rng.standard_normal((len(ids), hq, self.d)).astype(np.float32))
        q = R.bf16_tensor(bits, self.device)
        ks, vs = (self.kv.k_scale, self.kv.v_scale) if self.mode != "bf16" else (None, None)
        out = P.paged_attn_decode_grouped(q, self.kv.k_cache, self.kv.v_cache, _dev(tab, self.device),
                                          _dev(dlens, self.device), max(lens), 1.0 / math.sqrt(self.d), group_size,
                                          _dev(shared, self.device), k_scale=ks, v_scale=vs)
        ref = OT.decode(W.bf16_bits_to_f32(bits), *self.oc[:2], tab.tolist(), lens, 1.0 / math.sqrt(self.d),
                        *(self.oc[2:] if self.mode != "bf16" else (None, None)))
        check_tol(out.float().cpu().numpy().astype(np.float64), ref, "bf16" if self.mode == "bf16" else "i8", what)
        # the same groups over splits of their shared keys (pkv_paged_attn_decode_grouped_split),
        # with every split count up to more splits than shared blocks; max_shared_len above the
        # longest shared length, so trailing splits of every group are empty
        for ms in splits:
            max_sh = min(max(lens), int(shared.max()) + 300)
            need = P.decode_grouped_workspace_bytes(len(ids), hq, self.d, max_sh, ms)
            ws = torch.full((max(need, 16),), 0xFF, dtype=torch.uint8, device=self.device)  # NaN bytes
            got = P.paged_attn_decode_grouped_split(q, self.kv.k_cache, self.kv.v_cache, _dev(tab, self.device),
                                                    _dev(dlens, self.device), max(lens), 1.0 / math.sqrt(self.d),
                                                    group_size, _dev(shared, self.device), max_sh, ms,
                                                    workspace=ws, k_scale=ks, v_scale=vs)
            check_tol(got.float().cpu().numpy().astype(np.float64), ref, "bf16" if self.mode == "bf16" else "i8",
                      f"{what} split {ms} (workspace {need} bytes)")
        return shared.tolist()


@pytest.mark.parametrize("mode,hq,hkv,d,m", [("bf16", 8, 2, 128, 2), ("bf16", 4, 2, 128, 4), ("bf16", 2, 2, 64, 8),
                                             ("bf16", 2, 2, 128, 1), ("i8", 8, 4, 128, 2), ("i8q", 4, 4, 64, 4)])
def test_grouped_decode_matches_oracle(gpu, mode, hq, hkv, d, m):
    """Groups of m forks per request, read through pkv_paged_attn_decode_grouped, against the oracle:
    prompts ending inside a block, on a block boundary and one token short of one; members whose
    lengths differ inside a group; a member re-forked from another after a prune; appends that
    cross into new blocks, so members differ in full blocks too."""
    both = Both(mode, gpu, seed=20 + m, hkv=hkv, d=d, nb=72)
    rnd = np.random.default_rng(m)
    prompts = [300, 512, 255]
    groups = []
    for r, n in enumerate(prompts):
        both.add(100 * r, rnd.integers(0, 1000, size=n).tolist())
        for k in range(1, m):
            both.fork(100 * r, 100 * r + k)
        groups.append([100 * r + k for k in range(m)])
    flat = lambda: [i for g in groups for i in g]
    seen_partial = False
    for step in range(5):
        if step == 1:  # the first member of every group runs two tokens ahead of the others
            both.step([g[0] for g in groups])
            both.step([g[0] for g in groups])
        if step == 3 and m > 1:  # prune each group's last member, re-fork it from the first
            for g in groups:
                both.free(g[-1])
                both.fork(g[0], g[-1])
        both.step(flat())
        shared = both.decode_grouped(flat(), m, hq, f"{mode} m={m} step {step}")
        lens = [both.oa.seq_len(i) for i in flat()]
        seen_partial |= any(sl < max(lens[k * m:(k + 1) * m]) for k, sl in enumerate(shared))
        say(f"  {mode} hq={hq} hkv={hkv} d={d} m={m} step {step}: shared {shared}, lengths {lens}")
        both.oa.check_invariants()
    assert seen_partial or m == 1  # some member read keys beyond its group's shared ones


@pytest.mark.parametrize("mode,hq,hkv,d,m", [("bf16", 8, 4, 128, 4), ("bf16", 2, 2, 64, 8), ("i8", 8, 8, 128, 1),
                                             ("i8q", 4, 2, 128, 2)])
def test_grouped_split_decode_matches_oracle(gpu, mode, hq, hkv, d, m):
    """pkv_paged_attn_decode_grouped_split against the oracle: groups of m forks over prompts of
    different lengths (2,000-4,700 tokens, 8-19 blocks), members that diverge inside a group, and
    1, 2, 3, 7 and 64 splits of the shared keys (the short groups' last splits are empty)."""
    both = Both(mode, gpu, seed=40 + m, hkv=hkv, d=d, nb=260)
    rnd = np.random.default_rng(100 + m)
    groups = []
    for r, n in enumerate([4700, 2000, 3333]):
        both.add(100 * r, rnd.integers(0, 1000, size=n).tolist())
        for k in range(1, m):
            both.fork(100 * r, 100 * r + k)
        groups.append([100 * r + k for k in range(m)])
    flat = lambda: [i for g in groups for i in g]
    for step in range(3):
        if step == 1:  # the first member of every group runs ahead of the others
            both.step([g[0] for g in groups])
        both.step(flat())
        shared = both.decode_grouped(flat(), m, hq, f"{mode} m={m} step {step}", splits=(1, 2, 3, 7, 64))
        say(f"  {mode} hq={hq} hkv={hkv} d={d} m={m} step {step}: shared {shared}")


@pytest.mark.parametrize("mode", ["bf16", "i8", "i8q"])
def test_beam_search_with_forks_and_pruning(gpu, mode):
    both = Both(mode, gpu, seed=7)
    rnd = np.random.default_rng(3)
    shared = rnd.integers(0, 1000, size=256).tolist()
    # partial last blocks (300, 517 tokens), a prefix-cache hit (seq 1 reuses seq 0's first block)
    # and a prompt one token short of a full block (255 tokens)
    both.add(0, shared + rnd.integers(0, 1000, size=44).tolist())
    both.add(1, shared + rnd.integers(0, 1000, size=261).tolist())
    both.add(2, rnd.integers(0, 1000, size=255).tolist())
    for p, c in ((0, 10), (0, 11), (1, 12), (2, 15)):
        both.fork(p, c)
    both.check_caches("after prompts and forks")
    live = [0, 10, 11, 1, 12, 2, 15]
    total = 0
    for step in range(6):
        if step == 2:  # prune a beam, fork a survivor twice (a fork of a fork)
            both.free(11)
            both.fork(10, 13)
            both.fork(13, 14)
            live = [0, 10, 13, 14, 1, 12, 2, 15]
        if step == 4:  # the parent ends; its children keep the shared blocks
            both.free(0)
            live.remove(0)
        n = both.step(live)
        total += n
        say(f"  {mode} step {step}: {len(live)} sequences, {n} block copies")
        both.check_caches(f"step {step}")
        both.decode(live, f"{mode} step {step} decode")
        both.oa.check_invariants()
    assert total == 6  # step 0: seqs 10, 11, 1, 2; step 2: seqs 10, 13
    assert both.kv.alloc.num_free() == both.oa.num_free()


@pytest.mark.parametrize("fused", [False, True])
def test_decode_batch_with_copy_on_write(gpu, fused):
    """The runner's decode step (DecodeBatch with cow=True): copies, store (or fused store and
    attend) and attention in order on one stream; at step 2 a beam is replaced by a fork of
    another (set_sequences)."""
    both = Both("bf16", gpu, seed=11)
    rnd = np.random.default_rng(5)
    both.add(0, rnd.integers(0, 1000, size=383).tolist())
    both.add(1, rnd.integers(0, 1000, size=128).tolist())
    for p, c in ((0, 1000), (0, 1001), (1, 1002)):
        both.fork(p, c)
    ids = [0, 1000, 1001, 1, 1002]
    batch = R.DecodeBatch(both.kv, HQ, ids, 400, fused=fused, cow=True)
    for step in range(4):
        if step == 2:
            both.free(1001)
            both.fork(1000, 1003)
            ids = [0, 1000, 1003, 1, 1002]
            batch.set_sequences(ids)
        toks = both.rng.integers(0, 1000, size=len(ids)).tolist()
        slots, src, dst, _ = both.oracle_append(ids, toks)  # the native append runs inside batch.step
        rows = [both._rows(slots) for _ in range(2)]
        both.oc = list(OT.kv_store(*both.oc, rows[0][0], rows[1][0], slots))
        bits = W.f32_to_bf16_bits(both.rng.standard_normal((len(ids), HQ, D)).astype(np.float32))
        out = batch.step(toks, R.bf16_tensor(bits, gpu), rows[0][1], rows[1][1], SCALE)
        assert batch.slots.cpu().numpy().tolist() == slots
        lens = [both.oa.seq_len(i) for i in ids]
        ref = OT.decode(W.bf16_bits_to_f32(bits), *both.oc[:2], both.oa.block_tables(ids, 2), lens, SCALE)
        say(f"  fused={fused} step {step}: {len(src)} block copies")
        check_tol(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"fused={fused} step {step}")
        both.check_caches(f"fused={fused} step {step}")


@pytest.mark.parametrize("min_shared,group_splits", [(0, 0), (0, 1), (1 << 30, 0)])
def test_decode_batch_grouped(gpu, min_shared, group_splits):
    """DecodeBatch with group_size: two requests of two beams each, steps with copy-on-write and a
    re-fork; min_shared 0 takes the grouped kernel every step, a huge one the per-sequence one;
    group_splits 0 lets the runner split the two groups' shared keys (few groups: many splits), 1
    keeps one workgroup per group and KV head."""
    both = Both("bf16", gpu, seed=13)
    rnd = np.random.default_rng(8)
    both.add(0, rnd.integers(0, 1000, size=700).tolist())
    both.add(1, rnd.integers(0, 1000, size=511).tolist())
    both.fork(0, 1000)
    both.fork(1, 1001)
    ids = [0, 1000, 1, 1001]
    batch = R.DecodeBatch(both.kv, HQ, ids, 800, cow=True, group_size=2, group_min_shared=min_shared,
                          group_splits=group_splits)
    assert (batch.group_splits > 1) == (group_splits == 0)  # two groups leave most CUs idle unsplit
    for step in range(4):
        if step == 2:  # the second beam of request 0 is replaced by a fork of the first
            both.free(1000)
            both.fork(0, 1002)
            ids = [0, 1002, 1, 1001]
            batch.set_sequences(ids)
        toks = both.rng.integers(0, 1000, size=len(ids)).tolist()
        slots, src, dst, _ = both.oracle_append(ids, toks)
        rows = [both._rows(slots) for _ in range(2)]
        both.oc = list(OT.kv_store(*both.oc, rows[0][0], rows[1][0], slots))
        bits = W.f32_to_bf16_bits(both.rng.standard_normal((len(ids), HQ, D)).astype(np.float32))
        out = batch.step(toks, R.bf16_tensor(bits, gpu), rows[0][1], rows[1][1], SCALE)
        assert batch.grouped == (min_shared == 0)
        lens = [both.oa.seq_len(i) for i in ids]
        ref = OT.decode(W.bf16_bits_to_f32(bits), *both.oc[:2], both.oa.block_tables(ids, 4), lens, SCALE)
        say(f"  min_shared={min_shared} step {step}: shared {batch.host_shared_lens.tolist()}, lengths {lens}")
        check_tol(out.float().cpu().numpy().astype(np.float64), ref, "bf16", f"grouped batch step {step}")
        both.check_caches(f"grouped batch step {step}")


@pytest.mark.parametrize("dtype,hkv,d", [(P.F32, 1, 64), (P.BF16, 8, 128), (P.BF16, 3, 64), (P.I8, 2, 128),
                                          (P.I8, 5, 64)])
@pytest.mark.parametrize("with_rows", [True, False])
def test_copy_blocks_matches_oracle_bit_for_bit(gpu, dtype, hkv, d, with_rows):
    """pkv_copy_blocks on random caches: row counts 0, 1, 255, 256 and random ones, or whole blocks."""
    rng = np.random.default_rng(hkv * 1000 + d)
    nb, n = 24, 9
    shape = (nb, hkv, 256, d)
    if dtype == P.I8:
        caches = [rng.integers(-127, 128, size=shape).astype(np.int8) for _ in range(2)]
        caches += [rng.uniform(0.01, 1, size=(nb, hkv)).astype(np.float32) for _ in range(2)]
    else:
        x = [rng.standard_normal(shape).astype(np.float32) for _ in range(2)]
        caches = [W.bf16_bits_to_f32(W.f32_to_bf16_bits(a)) for a in x] if dtype == P.BF16 else x
    perm = rng.permutation(nb)
    src, dst = perm[:n].astype(np.int32), perm[n:2 * n].astype(np.int32)
    rows = np.array([0, 1, 255, 256] + rng.integers(1, 256, size=n - 4).tolist(), dtype=np.int32)
    tdt = {P.F32: torch.float32, P.BF16: torch.bfloat16, P.I8: torch.int8}[dtype]
    g = [_dev(c, gpu).to(tdt) for c in caches[:2]] + [_dev(c, gpu) for c in caches[2:]]
    P.copy_blocks(_dev(src, gpu), _dev(dst, gpu), g[0], g[1], _dev(rows, gpu) if with_rows else None,
                  *(g[2:] if dtype == P.I8 else (None, None)))
    ref = OT.copy_blocks(caches, src, dst, rows if with_rows else None)
    torch.cuda.synchronize()
    for t, r in zip(g, ref):
        got = t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()
        assert np.array_equal(got, r)
