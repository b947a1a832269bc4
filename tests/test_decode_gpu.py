"""GPU parity of kv_store and paged decode against the oracle (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
import workloads as W
from oracle import attention as OT
from tests.gpu_cases import (check_tol, dev_rows, gpu_decode, host_out, oracle_decode, say, to_f64)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------------------------ kv_store
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 128), ("bf16", 64), ("i8", 128), ("f32", 128)])
def test_kv_store_is_an_exact_scatter(gpu, dtype, D):
    say(f"kv_store {dtype} D={D}")
    rng = np.random.default_rng(D)
    nb, Hkv, n = 5, 3, 700
    slots = rng.permutation(nb * 256)[:n].astype(np.int32)
    slots[::97] = -1
    kdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i8": torch.int8}[dtype]
    if dtype == "i8":
        kn = rng.integers(-127, 128, size=(n, Hkv, D)).astype(np.int8)
        vn = rng.integers(-127, 128, size=(n, Hkv, D)).astype(np.int8)
        sentinel = 99
    else:
        kn = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        vn = rng.standard_normal((n, Hkv, D)).astype(np.float32)
        sentinel = 7.25
    k_cache = torch.full((nb, Hkv, 256, D), sentinel, dtype=kdt, device=gpu)
    v_cache = torch.full_like(k_cache, sentinel)
    kt = torch.from_numpy(kn).to(gpu).to(kdt)
    vt = torch.from_numpy(vn).to(gpu).to(kdt)
    scales = [None] * 4
    if dtype == "i8":
        ksn = rng.random((n, Hkv)).astype(np.float32)
        vsn = rng.random((n, Hkv)).astype(np.float32)
        scales = [torch.from_numpy(ksn).to(gpu), torch.from_numpy(vsn).to(gpu),
                  torch.full((nb, Hkv), -1.0, device=gpu), torch.full((nb, Hkv), -1.0, device=gpu)]
    P.kv_store(kt, vt, torch.from_numpy(slots).to(gpu), k_cache, v_cache, *scales)
    torch.cuda.synchronize()
    # oracle on the exact values the device received
    ref_k = np.full((nb, Hkv, 256, D), sentinel, dtype=np.float64)
    ref_v = ref_k.copy()
    kin, vin = kt.double().cpu().numpy(), vt.double().cpu().numpy()
    if dtype == "i8":
        rks, rvs = np.full((nb, Hkv), -1.0), np.full((nb, Hkv), -1.0)
        ref_k, ref_v, rks, rvs = OT.kv_store(ref_k, ref_v, kin, vin, slots, rks, rvs, ksn, vsn)
        # several tokens of one block may carry different scales here: the last writer is not
        # ordered between threads, so check each written entry equals one of its writers' values
        got_ks = scales[2].cpu().numpy()
        for blk in range(nb):
            for h in range(Hkv):
                writers = [ksn[t, h] for t in range(n) if slots[t] >= 0 and slots[t] // 256 == blk]
                if writers:
                    assert got_ks[blk, h] in writers
                else:
                    assert got_ks[blk, h] == -1.0
    else:
        ref_k, ref_v = OT.kv_store(ref_k, ref_v, kin, vin, slots)
    assert np.array_equal(k_cache.double().cpu().numpy(), ref_k)
    assert np.array_equal(v_cache.double().cpu().numpy(), ref_v)
    if dtype == "bf16":  # bit patterns, not just values
        t = int(np.flatnonzero(slots >= 0)[0])
        s0 = int(slots[t])
        assert torch.equal(k_cache.view(torch.int16)[s0 // 256, :, s0 % 256], kt.view(torch.int16)[t])


def test_kv_store_empty_is_a_no_op(gpu):
    k = torch.zeros((2, 1, 256, 64), device=gpu)
    v = torch.zeros_like(k)
    e = torch.empty((0, 1, 64), device=gpu)
    P.kv_store(e, e, torch.empty(0, dtype=torch.int32, device=gpu), k, v)
    torch.cuda.synchronize()
    assert k.abs().sum().item() == 0


# ------------------------------------------------------------------------------------ decode
SMALL = {
    "tiny_fp32": dict(),
    "tiny_fp32_257": dict(base="tiny_fp32", ctx=[1, 255, 256, 257, 600, 513], B=6, pool=12),
    "qwen3_decode": dict(B=6),
    "long_decode": dict(B=3),
    "int8_decode": dict(B=3),
    # every query-group size and head_dim the C ABI accepts, in every cache dtype
    "g8_bf16": dict(base="qwen3_decode", B=4, Hq=64, Hkv=8),
    "g8_i8": dict(base="int8_decode", B=3, ctx=(100, 1500), Hq=64, Hkv=8),
    "g8_f32": dict(base="tiny_fp32", Hq=16, Hkv=2),
    "g1_f32": dict(base="tiny_fp32", Hq=2, Hkv=2),
    "bf16_d64": dict(base="qwen3_decode", B=5, D=64),
    "g8_bf16_d64": dict(base="qwen3_decode", B=3, D=64, Hq=32, Hkv=4),
    "i8_d64": dict(base="int8_decode", B=3, ctx=(100, 1500), D=64, Hq=8, Hkv=4),
}


def _cfg(name):
    over = dict(SMALL[name])
    base = over.pop("base", name)
    return W.config(base, **over)


_REF = {}


def _oracle(name, seed, wl):
    """The oracle's answer for a workload, computed once per (workload, seed)."""
    if (name, seed) not in _REF:
        _REF[(name, seed)] = oracle_decode(wl)
    return _REF[(name, seed)]


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("max_splits", [0, 1, 3])
def test_decode_matches_oracle(gpu, name, max_splits):
    cfg = _cfg(name)
    wl = W.decode_workload(cfg, 0)
    say(f"decode {name} splits={max_splits} lens={wl['lens']}")
    out, _, _ = gpu_decode(wl, gpu, max_splits=max_splits, fill=float("nan") if cfg["dtype"] != "i8" else None)
    check_tol(host_out(out), _oracle(name, 0, wl), cfg["dtype"], f"{name}/splits={max_splits}")


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("max_splits", [0, 3])
def test_fused_store_equals_store_then_attend(gpu, name, max_splits):
    """pkv_decode_store_attend leaves the same cache (rows and int8 scales) and the same output,
    bit for bit, as pkv_kv_store followed by pkv_paged_attn_decode."""
    cfg = _cfg(name)
    wl = W.decode_workload(cfg, 0)
    fill = float("nan") if cfg["dtype"] != "i8" else -128  # rows nobody writes compare equal too
    a, kva, _ = gpu_decode(wl, gpu, max_splits=max_splits, fill=fill, fused=True)
    b, kvb, _ = gpu_decode(wl, gpu, max_splits=max_splits, fill=fill, fused=False)
    bits = lambda t: t.contiguous().view(torch.uint8)
    assert torch.equal(bits(a), bits(b))
    assert torch.equal(bits(kva.k_cache), bits(kvb.k_cache)) and torch.equal(bits(kva.v_cache), bits(kvb.v_cache))
    if cfg["dtype"] == "i8":
        assert torch.equal(bits(kva.k_scale), bits(kvb.k_scale)) and torch.equal(bits(kva.v_scale), bits(kvb.v_scale))


@pytest.mark.parametrize("seed", [1, 2])
def test_decode_other_seeds(gpu, seed):
    cfg = _cfg("qwen3_decode")
    wl = W.decode_workload(cfg, seed)
    out, _, _ = gpu_decode(wl, gpu)
    check_tol(host_out(out), oracle_decode(wl), "bf16", f"qwen3 seed {seed}")


def test_decode_is_deterministic_and_placement_invariant(gpu):
    cfg = _cfg("qwen3_decode")
    wl = W.decode_workload(cfg, 0)
    a, _, _ = gpu_decode(wl, gpu)
    b, _, _ = gpu_decode(wl, gpu)
    other = np.random.default_rng(5).permutation(wl["num_blocks"]).astype(np.int32)
    c, _, _ = gpu_decode(wl, gpu, free_order=other)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_decode_split_count_changes_little(gpu):
    cfg = _cfg("long_decode")
    wl = W.decode_workload(cfg, 0)
    outs = [host_out(gpu_decode(wl, gpu, max_splits=s)[0]) for s in (1, 2, 5, 32)]
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() < 1e-2


def test_decode_zero_context_gives_zero(gpu):
    Hkv, D = 2, 64
    k = torch.randn((3, Hkv, 256, D), device=gpu)
    v = torch.randn_like(k)
    q = torch.randn((2, 4, D), device=gpu)
    bt = torch.tensor([[0, 1], [2, 1]], dtype=torch.int32, device=gpu)  # every row valid for its length
    for splits in (1, 2):
        lens = torch.tensor([0, 300 if splits == 1 else 10], dtype=torch.int32, device=gpu)
        out = P.paged_attn_decode(q, k, v, bt, lens, 512, 0.125, max_splits=splits)
        torch.cuda.synchronize()
        assert torch.all(out[0] == 0)
        assert torch.all(torch.isfinite(out[1]))


# --------------------------------------------------------------------- full-size workloads
@pytest.mark.parametrize("name", ["qwen3_decode", "long_decode", "int8_decode"])
def test_decode_full_size_every_sequence(gpu, name):
    """Full-size workload on the path the bench times: kv_store then pkv_paged_attn_decode (not the
    fused launch), the automatic split plan for the bench's max_context_len, and its launch order.
    Every sequence and every head is checked element by element against the oracle's attention
    over that sequence's rows, and every stored cache row bit for bit through the oracle's own
    block manager."""
    import bench
    from oracle import allocator as OA
    from oracle import steps as OS
    cfg = W.config(name)
    wl = W.decode_workload(cfg, 0)
    say(f"full-size {name}: B={len(wl['lens'])} sum ctx={sum(wl['lens'])}")
    max_ctx = bench.decode_max_context(wl["lens"], bench.DEFAULT_WARMUP, bench.DEFAULT_STEPS)
    out, kv, batch = gpu_decode(wl, gpu, max_context_len=max_ctx, fused=False)
    say(f"  plan: splits={batch.splits} blocks/split={batch.blocks_per_split}")
    got = host_out(out)
    ref = np.stack([OS.decode_one_sequence(cfg, s, L) for s, L in zip(wl["seqs"], wl["lens"])])
    check_tol(got, ref, cfg["dtype"], f"{name} full size, all {len(wl['lens'])} sequences")
    # every sequence's cache rows, located through the oracle's own block manager
    a = OA.Allocator(wl["num_blocks"], wl["free_order"])
    for b, s in enumerate(wl["seqs"]):
        a.add_seq(b, s["tokens"][:-1])
    for b, s in enumerate(wl["seqs"]):
        a.append(b, int(s["tokens"][-1]))
    i8 = cfg["dtype"] == "i8"
    view = torch.int8 if i8 else torch.int16
    kc, vc = kv.k_cache.view(view), kv.v_cache.view(view)
    mb = max(-(-L // 256) for L in wl["lens"])
    tables = np.array(a.block_tables(range(len(wl["lens"])), mb), dtype=np.int64)
    for b, (s, L) in enumerate(zip(wl["seqs"], wl["lens"])):
        j = np.arange(L)
        idx = torch.from_numpy(tables[b][j // 256]).to(gpu)
        off = torch.from_numpy(j % 256).to(gpu)
        gk, gv = kc[idx, :, off].cpu().numpy(), vc[idx, :, off].cpu().numpy()
        ek, ev = (s["kq"], s["vq"]) if i8 else (s["k"], s["v"])
        assert np.array_equal(gk.view(ek.dtype), ek) and np.array_equal(gv.view(ev.dtype), ev), b
        if i8:
            blocks = torch.from_numpy(tables[b][:-(-L // 256)]).to(gpu)
            assert np.array_equal(kv.k_scale[blocks].cpu().numpy(), s["k_blk_scale"]), b
            assert np.array_equal(kv.v_scale[blocks].cpu().numpy(), s["v_blk_scale"]), b


def test_launch_order_from_the_device(gpu):
    """pkv_decode_launch_order with the device's CU count and the decode kernel's occupancy: a
    permutation; longest first when the workgroups queue (B=256 x 8 KV heads), balanced rounds when
    every workgroup is resident at once (B=64 x 8 KV heads, G=4)."""
    rng = np.random.default_rng(2)
    d = P.cache_desc(16, 8, 128, P.BF16)
    lens = rng.integers(100, 2049, size=256).astype(np.int32)
    order = P.decode_launch_order(d, 16, lens, 2048)
    assert sorted(order) == list(range(256)) and np.all(np.diff(lens[order]) <= 0)
    lens = rng.integers(4096, 8193, size=64).astype(np.int32)
    order = P.decode_launch_order(d, 32, lens, 8192)
    say(f"  B=64 G=4 order head {list(order[:4])} ... tail {list(order[-4:])}")
    assert sorted(order) == list(range(64))
    assert not np.all(np.diff(lens[order]) <= 0)  # 512 workgroups fit the device at once
