"""The C ABI library (CPU only): it loads, exports what include/pkv.h declares, and rejects bad
arguments on the host before anything is enqueued.  No test here launches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest
import torch  # noqa: F401  (loaded first, so libpkv binds to torch's HIP runtime)

import paged_kv_cache_kvcache_amd as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_\w+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_function():
    lib = P.lib()
    declared = _header_functions()
    assert len(declared) >= 17
    for name in declared:
        assert hasattr(lib, name), f"{name} declared in pkv.h but not exported"
    assert sorted(P.SIGNATURES) == declared, "binding signatures drift from pkv.h"
    assert P.lib().pkv_version().decode().startswith("pkv")


def test_library_has_gfx950_code_object():
    data = open(P.LIB_PATH, "rb").read()
    assert b"gfx950" in data


FAKE = ctypes.c_void_p(1 << 20)  # never dereferenced: every call below is rejected on the host


def _desc(**kw):
    d = dict(num_blocks=8, num_kv_heads=2, head_dim=64, kv_dtype=P.F32)
    d.update(kw)
    return P.cache_desc(**d)


def _store(desc, n=1, scales=(None, None, None, None), ptr=FAKE):
    return P.lib().pkv_kv_store(ctypes.byref(desc), ptr, ptr, *scales[:2], ptr, n, ptr, ptr, *scales[2:], None)


@pytest.mark.parametrize("kw,code", [
    (dict(head_dim=96), P.ERR_UNSUPPORTED),
    (dict(kv_dtype=7), P.ERR_UNSUPPORTED),
    (dict(num_kv_heads=0), P.ERR_INVALID),
    (dict(num_blocks=0), P.ERR_INVALID),
])
def test_kv_store_rejects_bad_descriptors(kw, code):
    assert _store(_desc(**kw)) == code
    assert P.last_error()


def test_kv_store_rejects_block_size_other_than_256():
    d = _desc()
    d.block_size = 128
    assert _store(d) == P.ERR_UNSUPPORTED


def test_kv_store_scale_pointer_rules():
    assert _store(_desc(kv_dtype=P.I8)) == P.ERR_INVALID  # int8 needs scales
    assert _store(_desc(), scales=(FAKE, FAKE, FAKE, FAKE)) == P.ERR_INVALID  # f32 rejects them
    assert _store(_desc(), n=-1) == P.ERR_INVALID
    assert _store(_desc(), ptr=ctypes.c_void_p(8)) == P.ERR_INVALID  # misaligned
    assert _store(_desc(), n=0) == P.OK  # empty store enqueues nothing


def test_quantising_store_rejects_bad_arguments():
    i8 = _desc(kv_dtype=P.I8)

    def call(desc, new_dt=P.BF16, n=4, n_runs=1, max_run=4, runs=FAKE, ptr=FAKE, scales=FAKE):
        return P.lib().pkv_kv_store_quant(ctypes.byref(desc), ptr, ptr, new_dt, FAKE, n, runs, n_runs, max_run, ptr,
                                          ptr, scales, scales, None)
    assert call(_desc(kv_dtype=P.BF16)) == P.ERR_UNSUPPORTED   # writes int8 caches only
    assert call(i8, new_dt=P.I8) == P.ERR_UNSUPPORTED           # rows must be bf16 or f32
    assert call(i8, n=-1) == P.ERR_INVALID
    assert call(i8, n_runs=5) == P.ERR_INVALID                  # more runs than rows
    assert call(i8, max_run=0) == P.ERR_INVALID
    assert call(i8, max_run=257) == P.ERR_INVALID
    assert call(i8, runs=None) == P.ERR_INVALID                 # run list required
    assert call(i8, scales=None) == P.ERR_INVALID               # scales required
    assert call(i8, ptr=ctypes.c_void_p(8)) == P.ERR_INVALID    # misaligned
    assert call(i8, n_runs=0) == P.OK


def test_store_runs():
    runs, nr, mx = P.store_runs([5, 6, 7, -1, 8, 255, 256, 257, 1000, 1002, -1])
    # 5..7 (run), -1 breaks it, 8 alone, 255 is a block's last slot, 256..257 open the next block,
    # 1000 and 1002 are not consecutive
    assert nr == 6 and mx == 3
    assert runs.reshape(-1, 2).tolist() == [[0, 3], [4, 1], [5, 1], [6, 2], [8, 1], [9, 1]]
    assert P.store_runs([])[1:] == (0, 0)
    assert P.store_runs([-1, -1])[1:] == (0, 0)
    full = P.store_runs(list(range(512, 1024)))
    assert full[1:] == (2, 256) and full[0].tolist() == [0, 256, 256, 256]
    rng = np.random.default_rng(3)
    for _ in range(20):   # the runs cover exactly the rows with a slot, each maximal
        slots = []
        for _ in range(rng.integers(1, 8)):
            start = int(rng.integers(0, 4 * 256))
            slots += list(range(start, start + int(rng.integers(1, 300)))) + ([-1] if rng.random() < 0.3 else [])
        runs, nr, mx = P.store_runs(slots)
        rows = []
        for t, ln in runs.reshape(-1, 2):
            assert all(slots[t + i] == slots[t] + i for i in range(ln)) and slots[t] % 256 + ln <= 256
            end = t + ln
            assert not (end < len(slots) and slots[end] == slots[end - 1] + 1 and slots[end] % 256 != 0)
            rows += range(t, t + ln)
        assert rows == [t for t, s in enumerate(slots) if s >= 0]
        assert mx == max(runs[1::2], default=0)


def _decode(desc, B=2, Hq=4, max_blocks=3, max_ctx=600, splits=0, ks=None, vs=None, ws=None, ws_bytes=0,
            scale=0.125):
    return P.lib().pkv_paged_attn_decode(ctypes.byref(desc), FAKE, B, Hq, FAKE, FAKE, ks, vs, FAKE, max_blocks,
                                         FAKE, None, max_ctx, splits, scale, FAKE, ws, ws_bytes, None)


def test_decode_rejects_bad_arguments():
    d = _desc()
    assert _decode(d, Hq=3) == P.ERR_INVALID                       # Hq % Hkv
    assert _decode(d, Hq=2 * 16) == P.ERR_UNSUPPORTED               # group 16
    assert _decode(d, max_blocks=2, max_ctx=600) == P.ERR_INVALID   # table too narrow
    assert _decode(d, scale=float("nan")) == P.ERR_INVALID
    assert _decode(d, ks=FAKE, vs=FAKE) == P.ERR_INVALID            # scales on a float cache
    assert _decode(_desc(kv_dtype=P.I8)) == P.ERR_INVALID           # int8 without scales
    assert _decode(d, B=0) == P.OK


def _grouped(desc, B=4, Hq=4, group_size=2, max_blocks=3, max_ctx=600, ks=None, vs=None, scale=0.125):
    return P.lib().pkv_paged_attn_decode_grouped(ctypes.byref(desc), FAKE, B, Hq, FAKE, FAKE, ks, vs, FAKE,
                                                 max_blocks, FAKE, max_ctx, group_size, FAKE, scale, FAKE, None)


def test_grouped_decode_rejects_bad_arguments():
    d = _desc()  # 2 KV heads: Hq 4 gives two query heads per KV head
    assert _grouped(d, B=3) == P.ERR_INVALID                       # B % group_size
    assert _grouped(d, group_size=0) == P.ERR_INVALID
    assert _grouped(d, group_size=8, B=8) == P.ERR_UNSUPPORTED     # 8 members x 2 heads = 16 rows
    assert _grouped(d, group_size=3, B=6) == P.ERR_UNSUPPORTED     # 6 rows
    assert _grouped(d, Hq=3) == P.ERR_INVALID
    assert _grouped(d, max_blocks=2) == P.ERR_INVALID               # table too narrow
    assert _grouped(d, ks=FAKE, vs=FAKE) == P.ERR_INVALID
    assert _grouped(_desc(kv_dtype=P.I8)) == P.ERR_INVALID
    assert _grouped(d, B=0) == P.OK


def test_grouped_split_workspace_and_rejections():
    """pkv_decode_grouped_workspace_bytes: B x Hq x S x (D + 2) floats with S = ceil(nsh / bps),
    bps = ceil(nsh / min(max_splits, nsh)), nsh = ceil(max_shared_len / 256); 0 without a split.
    pkv_paged_attn_decode_grouped_split rejects bad bounds and a short workspace on the host."""
    for B, Hq, D, msl, ms in [(8, 16, 128, 20000, 4), (4, 8, 64, 300, 8), (4, 8, 64, 256, 8), (2, 4, 128, 9000, 5),
                              (2, 4, 128, 9000, 1), (2, 4, 128, 0, 3)]:
        nsh = -(-msl // 256)
        want = max(1, min(ms, max(1, nsh)))
        bps = max(1, -(-nsh // want))
        S = max(1, -(-nsh // bps))
        assert P.decode_grouped_workspace_bytes(B, Hq, D, msl, ms) == (B * Hq * S * (D + 2) * 4 if S > 1 else 0)
    assert P.decode_grouped_workspace_bytes(8, 16, 128, 20000, 4) == 8 * 16 * 4 * 130 * 4  # 79 blocks: 4 x 20
    assert P.decode_grouped_workspace_bytes(0, 16, 128, 20000, 4) == 0

    d = _desc()  # 2 KV heads, D 64

    def call(max_shared=500, max_splits=2, ws=FAKE, ws_bytes=1 << 30, max_ctx=600):
        return P.lib().pkv_paged_attn_decode_grouped_split(ctypes.byref(d), FAKE, 4, 4, FAKE, FAKE, None, None, FAKE,
                                                           3, FAKE, max_ctx, 2, FAKE, max_shared, max_splits, 0.125,
                                                           FAKE, ws, ws_bytes, None)
    assert call(max_shared=700) == P.ERR_INVALID      # above max_context_len
    assert call(max_shared=-1) == P.ERR_INVALID
    assert call(max_splits=0) == P.ERR_INVALID
    assert call(ws=None, ws_bytes=0) == P.ERR_SMALL_BUFFER   # two splits of the 2 shared blocks need one
    assert call(ws_bytes=16) == P.ERR_SMALL_BUFFER
    assert call(ws=ctypes.c_void_p((1 << 20) + 4)) == P.ERR_INVALID  # misaligned workspace


def _shared_lens_by_definition(tab, lens, m):
    """Per group: the shortest member's length, cut at 256 x the first block entry where the
    members' tables differ (only entries below that length count)."""
    res = []
    for k in range(len(lens) // m):
        rows, n = tab[k * m:(k + 1) * m], min(lens[k * m:(k + 1) * m])
        e = 0
        while e < -(-n // 256) and len(set(int(x) for x in rows[:, e])) == 1:
            e += 1
        res.append(min(n, 256 * e))
    return res


@pytest.mark.parametrize("seed", range(6))
def test_group_shared_lens_match_the_definition(seed):
    """pkv_decode_group_shared_lens against a brute-force reading of its definition on random
    fork structures: members copied from one table, then diverging from a random block on."""
    rng = np.random.default_rng(seed)
    m = [1, 2, 3, 4, 8, 5][seed]
    ng, mb = 7, 6
    tab = np.full((ng * m, mb), -1, dtype=np.int32)
    lens = np.zeros(ng * m, dtype=np.int32)
    nxt = 0
    for k in range(ng):
        base = rng.integers(0, 1000, size=mb).astype(np.int32)
        for j in range(m):
            i = k * m + j
            n = int(rng.integers(0, mb * 256 + 1)) if k != 0 else 256 * int(rng.integers(0, mb + 1))
            nb = -(-n // 256)
            row = base.copy()
            cut = int(rng.integers(0, mb + 1))  # from this block on the member has its own
            row[cut:] = 2000 + nxt + np.arange(mb - cut)
            nxt += mb
            tab[i, :nb] = row[:nb]
            lens[i] = n
    got = P.decode_group_shared_lens(tab, lens, m).tolist()
    assert got == _shared_lens_by_definition(tab, lens.tolist(), m)
    # a group whose members are identical shares everything; one whose first entries differ nothing
    same = np.tile(np.array([[5, 6, -1]], np.int32), (m, 1))
    assert P.decode_group_shared_lens(same, np.full(m, 300, np.int32), m).tolist() == [300]
    if m > 1:
        diff = same.copy()
        diff[1, 0] = 9
        assert P.decode_group_shared_lens(diff, np.full(m, 300, np.int32), m).tolist() == [0]


def test_group_shared_lens_errors():
    tab = np.zeros((4, 2), np.int32)
    with pytest.raises(RuntimeError):
        P.decode_group_shared_lens(tab, np.full(4, 10, np.int32), 3)      # B % group_size
    with pytest.raises(RuntimeError):
        P.decode_group_shared_lens(tab, np.array([10, -1, 5, 5], np.int32), 2)  # negative length
    with pytest.raises(RuntimeError):
        P.decode_group_shared_lens(tab, np.array([10, 513, 5, 5], np.int32), 2)  # past the table


def test_fused_store_decode_rejects_bad_arguments():
    d = _desc()
    i8 = _desc(kv_dtype=P.I8)

    def call(desc, k_new=FAKE, slots=FAKE, ksn=None, vsn=None, ks=None, vs=None):
        return P.lib().pkv_decode_store_attend(ctypes.byref(desc), FAKE, 2, 4, k_new, FAKE, ksn, vsn, slots, FAKE,
                                               FAKE, ks, vs, FAKE, 3, FAKE, None, 600, 0, 0.125, FAKE, None, 0, None)
    assert call(d, k_new=None) == P.ERR_INVALID                  # new rows required
    assert call(d, slots=None) == P.ERR_INVALID                  # slots required
    assert call(d, k_new=ctypes.c_void_p((1 << 20) + 4)) == P.ERR_INVALID  # misaligned rows
    assert call(d, ksn=FAKE, vsn=FAKE) == P.ERR_INVALID          # scales on a float cache
    assert call(i8, ks=FAKE, vs=FAKE) == P.ERR_INVALID           # int8 without the new tokens' scales


def test_decode_needs_its_workspace():
    d = _desc()
    need = P.decode_workspace_bytes(2, 4, 64, 2, 600, 3)
    assert need == 2 * 4 * 3 * (64 + 2) * 4
    assert _decode(d, splits=3) == P.ERR_SMALL_BUFFER
    assert _decode(d, splits=3, ws=FAKE, ws_bytes=need - 4) == P.ERR_SMALL_BUFFER


def test_decode_plan():
    assert P.decode_plan(4, 2, 600, 1) == (1, 3)
    assert P.decode_plan(4, 2, 600, 2) == (2, 2)
    assert P.decode_plan(4, 2, 600, 9) == (3, 1)       # at most one split per block
    assert P.decode_plan(4, 2, 0, 0) == (1, 1)
    s, bps = P.decode_plan(16, 8, 8192, 0)             # 128 workgroups: split the long contexts
    assert s == 4 and s * bps >= 32 and (s - 1) * bps < 32   # up to 2 per CU of 256 CUs
    assert P.decode_plan(64, 8, 8192, 0)[0] == 1        # 512 workgroups already fill 256 CUs twice
    assert P.decode_plan(256, 8, 2048, 0)[0] == 1
    assert P.decode_workspace_bytes(256, 16, 128, 8, 2048, 0) == 0


def _cu_work(order, lens, per_seq, cus):
    """Keys per CU when workgroup i of the launch (sequence order[i // per_seq]) runs on CU i % cus."""
    work = np.zeros(cus, dtype=np.int64)
    for i in range(len(order) * per_seq):
        work[i % cus] += lens[order[i // per_seq]]
    return work


def test_decode_launch_order_longest_first_when_workgroups_queue():
    rng = np.random.default_rng(3)
    d = _desc(num_kv_heads=8, head_dim=128, kv_dtype=P.BF16)
    lens = rng.integers(100, 2049, size=256).astype(np.int32)
    lens[10] = lens[11] = lens[200]  # ties keep sequence order
    # 256 x 8 workgroups, 2 per CU of 256 CUs: they queue, so longest context first
    order = P.decode_launch_order(d, 16, lens, 2048, compute_units=256, workgroups_per_cu=2)
    assert sorted(order) == list(range(256))
    assert np.all(np.diff(lens[order]) <= 0)
    for i, j in zip(order, order[1:]):
        assert lens[i] != lens[j] or i < j
    assert list(P.decode_launch_order(d, 16, np.full(300, 7), 7, compute_units=256, workgroups_per_cu=2)) == \
        list(range(300))


def test_decode_launch_order_balances_a_resident_launch():
    d = _desc(num_kv_heads=8, head_dim=128, kv_dtype=P.BF16)
    # 64 sequences x 8 KV heads = 512 workgroups, exactly 2 per CU: the two sequences on each CU
    # of an evenly spaced length mix sum to the same number of keys
    lens = (8192 - 64 * np.random.default_rng(0).permutation(64)).astype(np.int32)
    order = P.decode_launch_order(d, 32, lens, 8192, compute_units=256, workgroups_per_cu=2)
    assert sorted(order) == list(range(64))
    work = _cu_work(order, lens, 8, 256)
    assert work.min() == work.max() == 8192 + 8192 - 63 * 64
    first = _cu_work(np.argsort(-lens, kind="stable"), lens, 8, 256)
    assert first.max() > work.max()
    # random lengths, a partial last round and three workgroups per CU: never worse than longest first
    rng = np.random.default_rng(5)
    for B, per_cu in ((48, 2), (64, 2), (80, 3), (96, 3)):
        lens = rng.integers(4096, 8193, size=B).astype(np.int32)
        order = P.decode_launch_order(d, 32, lens, 8192, compute_units=256, workgroups_per_cu=per_cu)
        assert sorted(order) == list(range(B))
        assert _cu_work(order, lens, 8, 256).max() <= _cu_work(np.argsort(-lens, kind="stable"), lens, 8, 256).max()
    # a window caps each sequence's work: every context longer than the window is a tie
    lens = np.array([9000, 300, 5000, 700, 8000], dtype=np.int32)
    order = P.decode_launch_order(d, 16, lens, 9000, window=1000, compute_units=256, workgroups_per_cu=1)
    assert list(order) == [0, 2, 4, 3, 1]


def test_decode_launch_order_errors():
    d = _desc()
    assert list(P.decode_launch_order(d, 4, np.zeros(0, np.int32), 0, compute_units=4, workgroups_per_cu=1)) == []
    with pytest.raises(RuntimeError):
        P.decode_launch_order(d, 4, [5, -1], 5, compute_units=4, workgroups_per_cu=1)
    with pytest.raises(RuntimeError):
        P.decode_launch_order(d, 3, [5, 1], 5, compute_units=4, workgroups_per_cu=1)  # Hq not a multiple of Hkv
    lens = np.array([5, 1], dtype=np.int32)
    out = np.empty(2, dtype=np.int32)
    rc = P.lib().pkv_decode_launch_order(ctypes.byref(d), 4, 2, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         5, 0, 0, 4, 1, None)
    assert rc == P.ERR_INVALID
    rc = P.lib().pkv_decode_launch_order(ctypes.byref(d), 32, 2, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                         5, 0, 0, 4, 1, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
    assert rc == P.ERR_UNSUPPORTED  # group size 16
    if not torch.cuda.is_available():
        # the occupancy query needs a device
        rc = P.lib().pkv_decode_launch_order(ctypes.byref(d), 4, 2, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                             5, 0, 0, 4, 0, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)))
        assert rc == P.ERR_HIP


def _item_work(it, cu, lk, qt, causal=True, window=0):
    """Key tiles (of 64) a prefill work item attends, from the kernel's causal rule."""
    b, t = it >> 16, it & 0xFFFF
    nq, L = int(cu[b + 1] - cu[b]), int(lk[b])
    pos0 = L - nq + t * qt
    kv_len = min(L, pos0 + min(qt, nq - t * qt)) if causal else L
    first = max(0, pos0 - window + 1) // 64 if window else 0
    return -(-kv_len // 64) - first


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 200)])
def test_prefill_work_order(causal, window):
    rng = np.random.default_rng(11)
    d = _desc(num_kv_heads=8, head_dim=128, kv_dtype=P.BF16)
    nq = rng.integers(1, 900, size=13)
    nq[3] = 64  # exactly one tile
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    lk = (nq + rng.integers(0, 600, size=13)).astype(np.int32)
    qt = P.prefill_tile_rows(d, 16, 13, int(cu[-1]))
    assert qt in (64, 128)
    items, rows = P.prefill_work_order(d, 16, cu, lk, causal, window)
    assert rows == qt
    # every (sequence, tile) of the call exactly once
    assert sorted(items.tolist()) == sorted((b << 16) | t for b in range(13) for t in range(-(-int(nq[b]) // qt)))
    work = [_item_work(int(i), cu, lk, qt, causal, window) for i in items]
    R = 256 // 8  # items per round of one workgroup per CU (256 CUs without a device)
    rounds = [work[r:r + R] for r in range(0, len(work), R)]
    assert len(rounds) >= 3
    assert min(rounds[0]) >= max(w for r in rounds[1:] for w in r)  # the heaviest items first
    for i, r in enumerate(rounds):
        assert r == sorted(r, reverse=(i % 2 == 0))  # heaviest first, lightest first, ...
    # rounds hold consecutive ranks of the heaviest-first order
    assert sorted(work, reverse=True) == [w for i, r in enumerate(rounds) for w in (r if i % 2 == 0 else r[::-1])]


def test_prefill_work_order_errors():
    d = _desc(num_kv_heads=2, head_dim=64, kv_dtype=P.BF16)
    assert len(P.prefill_work_order(d, 4, [0], [])[0]) == 0
    with pytest.raises(RuntimeError):
        P.prefill_work_order(d, 4, [0, 10, 5], [10, 10])  # decreasing cu_seqlens_q
    with pytest.raises(RuntimeError):
        P.prefill_work_order(d, 4, [0, 10], [9])  # causal: fewer keys than new tokens
    assert len(P.prefill_work_order(d, 4, [0, 10], [9], causal=False)[0]) == 1
    with pytest.raises(RuntimeError):
        P.prefill_work_order(d, 3, [0, 10], [10])  # Hq not a multiple of Hkv
    cu, lk = np.array([0, 200], np.int32), np.array([200], np.int32)
    out, n = np.empty(2, np.int32), ctypes.c_int32()
    p32 = ctypes.POINTER(ctypes.c_int32)
    rc = P.lib().pkv_prefill_work_order(ctypes.byref(d), 4, 1, cu.ctypes.data_as(p32), lk.ctypes.data_as(p32), 1, 0,
                                        out.ctypes.data_as(p32), 2, ctypes.byref(n), None)
    assert rc == P.ERR_SMALL_BUFFER and n.value == 0  # 200 tokens in tiles of 64: four items
    rc = P.lib().pkv_paged_attn_prefill_ordered(ctypes.byref(d), FAKE, 4, FAKE, FAKE, 1, 1, 1, 1, FAKE, FAKE, FAKE,
                                                1, 0.1, 1, 0, None, 1, 64, FAKE, None)
    assert rc == P.ERR_INVALID  # items missing
    for bad in (0, 48, 96, 512):  # G = 2: tiles of 64 or 128 tokens only
        rc = P.lib().pkv_paged_attn_prefill_ordered(ctypes.byref(d), FAKE, 4, FAKE, FAKE, 1, 1, 1, 1, FAKE, FAKE,
                                                    FAKE, 1, 0.1, 1, 0, FAKE, 1, bad, FAKE, None)
        assert rc == P.ERR_INVALID, bad


def test_prefill_rejects_bad_descriptor():
    d = _desc(head_dim=80)
    rc = P.lib().pkv_paged_attn_prefill(ctypes.byref(d), FAKE, 4, FAKE, FAKE, 1, 1, 1, 1, FAKE, FAKE, FAKE, 1,
                                        0.1, 1, FAKE, None)
    assert rc == P.ERR_UNSUPPORTED


def test_copy_blocks_rejects_bad_arguments():
    def call(desc, n=2, ptr=FAKE, scales=(None, None)):
        return P.lib().pkv_copy_blocks(ctypes.byref(desc), ptr, ptr, None, n, ptr, ptr, scales[0], scales[1], None)

    assert call(_desc(), n=-1) == P.ERR_INVALID
    assert call(_desc(), ptr=None) == P.ERR_INVALID
    assert call(_desc(), scales=(FAKE, FAKE)) == P.ERR_INVALID          # only int8 takes scales
    assert call(_desc(kv_dtype=P.I8)) == P.ERR_INVALID                  # int8 needs them
    assert call(_desc(kv_dtype=P.I8), scales=(FAKE, None)) == P.ERR_INVALID
    assert call(_desc(head_dim=80)) == P.ERR_UNSUPPORTED
    assert call(_desc(), n=0, ptr=None) == P.OK                         # nothing to copy


def test_device_check_switch_and_error_word_arguments():
    assert P.lib().pkv_set_device_checks(1) == P.OK
    assert P.lib().pkv_set_device_checks(0) == P.OK
    assert P.lib().pkv_device_error(None, None, None, None) == P.ERR_INVALID  # code is required


@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 300)])
def test_prefill_split_order(causal, window):
    """pkv_prefill_split_order on a launch with fewer workgroups than CUs: every item's key tiles
    are covered once, by its pieces in key order (consecutive slots, one merge record) or whole;
    the pieces per item are min(8, ceil(tiles / T)) for the smallest T from 4 up that fits the launch
    in one workgroup per CU (256 CUs without a device); the workspace formula; and a launch that
    fills the device stays the work order."""
    d = _desc(num_kv_heads=8, head_dim=128, kv_dtype=P.BF16)
    nq = np.array([300, 5, 190, 64], np.int32)
    lk = np.array([1900, 2000, 1300, 64], np.int32)
    cu = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    pieces, merges, n_slots, qt = P.prefill_split_order(d, 16, cu, lk, causal, window)
    assert qt == P.prefill_tile_rows(d, 16, 4, int(cu[-1]))
    items = {(b << 16) | t for b in range(4) for t in range(-(-int(nq[b]) // qt))}
    assert len(items) * 8 < 256  # underfilled: the case must split
    assert len(merges) > 0 and len(pieces) * 8 <= 256
    works = {code: _item_work(code, cu, lk, qt, causal, window) for code in items}
    T = next(T for T in range(4, 10**6) if sum(max(1, min(8, -(-w // T))) for w in works.values()) * 8 <= 256)
    by_item = {}
    for code, a, b, slot in pieces.tolist():
        by_item.setdefault(code, []).append((a, b, slot))
    assert set(by_item) == items
    split = {int(m[0]): (int(m[1]), int(m[2])) for m in merges}
    for code, ps in by_item.items():
        work = _item_work(code, cu, lk, qt, causal, window)
        first = max(0, (int(lk[code >> 16]) - int(nq[code >> 16]) + (code & 0xffff) * qt) - window + 1) // 64 \
            if window else 0
        if code not in split:
            assert ps == [(0, 2**31 - 1, -1)]
            assert work <= T
            continue
        s0, npc = split[code]
        ps = sorted(ps)
        assert len(ps) == npc == min(8, -(-work // T)) and npc >= 2
        assert [p[2] for p in ps] == list(range(s0, s0 + npc))
        assert ps[0][0] == first and ps[-1][1] == first + work
        assert all(ps[i][1] == ps[i + 1][0] for i in range(npc - 1))
        assert all(b - a >= min(4, work // npc) for a, b, _ in ps)
    assert sorted(s for m in merges for s in range(m[1], m[1] + m[2])) == list(range(n_slots))
    G = 2
    assert P.prefill_split_workspace_bytes(d, 16, n_slots, qt) == n_slots * 8 * (128 + 4) * qt * G * 4
    assert P.prefill_split_workspace_bytes(d, 16, 0, qt) == 0
    # a launch that fills the device: the work order itself, nothing split
    rng = np.random.default_rng(5)
    nq2 = rng.integers(100, 900, size=13).astype(np.int32)
    cu2 = np.concatenate([[0], np.cumsum(nq2)]).astype(np.int32)
    lk2 = (nq2 + 300).astype(np.int32)
    p2, m2, s2, qt2 = P.prefill_split_order(d, 16, cu2, lk2, causal, window)
    order, qt3 = P.prefill_work_order(d, 16, cu2, lk2, causal, window)
    assert qt2 == qt3 and len(m2) == 0 and s2 == 0
    assert (p2[:, 0] == order).all() and (p2[:, 1] == 0).all() and (p2[:, 2] == 2**31 - 1).all()
    assert (p2[:, 3] == -1).all()


def test_prefill_split_errors():
    d = _desc(num_kv_heads=2, head_dim=64, kv_dtype=P.BF16)
    p32 = ctypes.POINTER(ctypes.c_int32)
    cu, lk = np.array([0, 200], np.int32), np.array([2000], np.int32)
    pieces, merges = np.empty((1, 4), np.int32), np.empty((4, 4), np.int32)
    n, m, s, t = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    rc = P.lib().pkv_prefill_split_order(ctypes.byref(d), 4, 1, cu.ctypes.data_as(p32), lk.ctypes.data_as(p32), 1, 0,
                                         pieces.ctypes.data_as(p32), 1, ctypes.byref(n), merges.ctypes.data_as(p32),
                                         4, ctypes.byref(m), ctypes.byref(s), ctypes.byref(t))
    assert rc == P.ERR_SMALL_BUFFER and n.value == 0  # four items of which some are split: more than one piece
    args = lambda pc, npc, mg, nm, ns, ws, wb: P.lib().pkv_paged_attn_prefill_split(
        ctypes.byref(d), FAKE, 4, FAKE, FAKE, 1, 200, 200, 2000, FAKE, FAKE, FAKE, 8, 0.1, 1, 0, pc, npc, mg, nm, ns,
        64, ws, wb, FAKE, None)
    assert args(None, 1, FAKE, 1, 2, FAKE, 1 << 30) == P.ERR_INVALID  # pieces missing
    assert args(FAKE, 1, None, 1, 2, FAKE, 1 << 30) == P.ERR_INVALID  # merges missing
    assert args(FAKE, 1, FAKE, 1, 0, FAKE, 1 << 30) == P.ERR_INVALID  # merges without slots
    assert args(FAKE, 1, FAKE, 1, 2, FAKE, 16) == P.ERR_SMALL_BUFFER  # workspace too small
    assert args(FAKE, 1, FAKE, 1, 2, None, 0) == P.ERR_SMALL_BUFFER  # no workspace
    assert args(FAKE, 0, None, 0, 0, None, 0) == P.OK  # nothing to do
