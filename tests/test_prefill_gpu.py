"""GPU parity of chunked varlen paged prefill against the oracle (needs an MI355X)."""

import numpy as np
import pytest

import workloads as W
from oracle import steps as OS
from tests.gpu_cases import check_tol, gpu_prefill, say

pytestmark = pytest.mark.gpu


def _run(cfg, seed=0, causal=True, prefix_cache=True):
    wl = W.prefill_workload(cfg, seed)
    say(f"prefill {cfg['name']} B={cfg['B']} Hq={cfg['Hq']} Hkv={cfg['Hkv']} D={cfg['D']} lens={wl['lens'][:8]}... "
        f"causal={causal} prefix={prefix_cache}")
    got = gpu_prefill(wl, "cuda", causal, prefix_cache)
    ref, ncached, chunks = OS.prefill_run(wl, causal, prefix_cache)
    say(f"  cached={ncached[:8]}... chunks={[len(c) for c in chunks]}")
    return got, ref, ncached


@pytest.mark.parametrize("Hq,Hkv,D", [(16, 8, 128), (4, 4, 128), (8, 2, 64), (16, 2, 128), (4, 1, 64)])
def test_prefill_small_chunks(Hq, Hkv, D):
    """Several chunks, shared prefixes, ragged tails; every query-group size and both head dims."""
    cfg = W.config("prefill_prefix", B=7, Hq=Hq, Hkv=Hkv, D=D, group=3, chunk=1500)
    got, ref, ncached = _run(cfg)
    assert sum(ncached) > 0
    check_tol(got, ref, "bf16", f"prefill Hq={Hq} Hkv={Hkv} D={D}")


def test_prefill_non_causal():
    cfg = W.config("prefill_prefix", B=5, group=2, chunk=2000)
    got, ref, _ = _run(cfg, causal=False)
    check_tol(got, ref, "bf16", "prefill non-causal")


def test_prefill_short_and_single_token_prompts():
    cfg = W.config("prefill_prefix", B=6, ctx=[1, 2, 63, 64, 65, 300], group=8, chunk=4096)
    got, ref, _ = _run(cfg)
    check_tol(got, ref, "bf16", "prefill short prompts")


@pytest.mark.parametrize("D,causal", [(128, True), (64, False)])
def test_prefill_wide_workgroups(D, causal):
    """One chunk of ~8K new tokens with ragged tails: enough query tiles that the kernel runs with
    eight-wavefront workgroups (at least two per CU of them)."""
    import torch
    lens = [1000, 1100, 900, 1050, 1023, 977, 1100, 1040]
    cfg = W.config("prefill_prefix", B=8, ctx=lens, D=D, group=1, shared=0, chunk=9000)
    qt8 = 8 * 32 // (cfg["Hq"] // cfg["Hkv"])
    items8 = (-(-sum(lens) // qt8) + cfg["B"]) * cfg["Hkv"]
    assert items8 >= 2 * torch.cuda.get_device_properties(0).multi_processor_count
    got, ref, _ = _run(cfg, causal=causal)
    check_tol(got, ref, "bf16", f"prefill wide workgroups D={D} causal={causal}")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_full_workload(seed):
    """The full 32-prompt workload: chunks of at most 4096 new tokens, groups of 8 sharing 512 tokens."""
    cfg = W.config("prefill_prefix")
    got, ref, ncached = _run(cfg, seed)
    assert got.shape == ref.shape
    check_tol(got, ref, "bf16", f"prefill full seed {seed}")


def test_prefix_cache_changes_no_suffix_output():
    cfg = W.config("prefill_prefix", B=8, group=4, chunk=4096)
    wl = W.prefill_workload(cfg, 0)
    on = gpu_prefill(wl, "cuda", True, True)
    off = gpu_prefill(wl, "cuda", True, False)
    _, ncached, _ = OS.prefill_run(wl, True, True)
    # rows of prompt i: with the cache on they start at its cached length
    r_on = r_off = 0
    for i, n in enumerate(wl["lens"]):
        c = ncached[i]
        a = on[r_on:r_on + n - c]
        b = off[r_off + c:r_off + n]
        assert np.abs(a - b).max() < 2e-2
        r_on += n - c
        r_off += n


def test_prefill_is_deterministic_and_placement_invariant():
    """Reruns give bitwise the same outputs, and so does another physical placement of the blocks:
    the kernel reads the same values in the same order wherever the blocks sit."""
    cfg = W.config("prefill_prefix")
    wl = W.prefill_workload(cfg, 0)
    a = gpu_prefill(wl, "cuda")
    b = gpu_prefill(wl, "cuda")
    other = dict(wl, free_order=np.random.default_rng(9).permutation(wl["num_blocks"]).astype(np.int32))
    c = gpu_prefill(other, "cuda")
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


@pytest.mark.parametrize("name,over,causal,window", [
    ("prefill_prefix", {}, True, 0),
    ("prefill_prefix", dict(B=8, ctx=[1000, 1100, 900, 1050, 1023, 977, 1100, 1040], group=1, shared=0, chunk=9000),
     True, 0),
    ("prefill_prefix", dict(B=5, group=2, chunk=2000), False, 0),
    ("prefill_prefix", dict(B=9, group=3, chunk=3000), True, 300),
])
def test_work_order_gives_bitwise_the_built_in_order(name, over, causal, window):
    """pkv_paged_attn_prefill_ordered with pkv_prefill_work_order's items against the built-in
    order of pkv_paged_attn_prefill(_window): the same outputs bit for bit, chunk by chunk."""
    import math
    import torch
    import paged_kv_cache_kvcache_amd as P
    from paged_kv_cache_kvcache_amd import runner as R
    from tests.gpu_cases import dev_rows
    cfg = W.config(name, **over)
    wl = W.prefill_workload(cfg, 0)
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    prompts = wl["prompts"]
    kv = R.PagedKV(wl["num_blocks"], Hkv, D, P.BF16, wl["free_order"], device="cuda", fill=0)
    ncached = [kv.alloc.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    for ch in W.pack_chunks(n_new, cfg["chunk"]):
        rows = lambda key: dev_rows(np.concatenate([prompts[i][key][ncached[i]:] for i in ch]), "cuda")
        q, k, v = rows("q"), rows("k"), rows("v")
        cu, lk, slots = kv.alloc.prefill_slots(ch, int(q.shape[0]))
        tab, _ = kv.alloc.block_tables(ch, max(1, -(-int(lk.max()) // 256)))
        kv.store(to(slots), k, v)
        items, qt = P.prefill_work_order(P.desc_of(kv.k_cache), Hq, cu, lk, causal, window)
        assert qt == P.prefill_tile_rows(P.desc_of(kv.k_cache), Hq, len(ch), int(cu[-1]))
        assert len(items) == sum(-(-int(n) // qt) for n in np.diff(cu))
        args = (q, to(cu), to(lk), int(np.diff(cu).max()), int(lk.max()), kv.k_cache, kv.v_cache, to(tab),
                1.0 / math.sqrt(D))
        ref = P.paged_attn_prefill(*args, causal, window=window)
        got = P.paged_attn_prefill_ordered(*args, to(items), qt, causal, window)
        torch.cuda.synchronize()
        say(f"  chunk of {len(ch)} prompts: {len(items)} items of {qt} tokens")
        assert torch.equal(ref, got)


def test_ordered_prefill_with_padded_q_keeps_the_list_tile():
    """A caller may pass q with more rows than cu_seqlens_q[B] (padding).  The launch then still
    cuts query tiles as the work list did, even where the padded total_q alone would choose the
    other workgroup shape: outputs equal the unpadded call bit for bit and the padding rows of out
    stay untouched."""
    import math
    import torch
    import paged_kv_cache_kvcache_amd as P
    from paged_kv_cache_kvcache_amd import runner as R
    from tests.gpu_cases import dev_rows
    cfg = W.config("prefill_prefix", B=8, group=4)  # small enough for four-wavefront tiles
    wl = W.prefill_workload(cfg, 1)
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    prompts = wl["prompts"]
    kv = R.PagedKV(wl["num_blocks"], Hkv, D, P.BF16, wl["free_order"], device="cuda", fill=0)
    ncached = [kv.alloc.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    ch = list(range(len(prompts)))
    rows = lambda key: dev_rows(np.concatenate([prompts[i][key][ncached[i]:] for i in ch]), "cuda")
    q, k, v = rows("q"), rows("k"), rows("v")
    n = int(q.shape[0])
    cu, lk, slots = kv.alloc.prefill_slots(ch, n)
    tab, _ = kv.alloc.block_tables(ch, max(1, -(-int(lk.max()) // 256)))
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    kv.store(to(slots), k, v)
    d = P.desc_of(kv.k_cache)
    items, qt = P.prefill_work_order(d, Hq, cu, lk, True)
    assert qt == 4 * 32 // (Hq // Hkv)
    # pad well past the real rows (where the kernel has a choice of tile, past the size that would
    # choose the other one)
    pad = next((p for p in range(0, 64 * n, 64) if P.prefill_tile_rows(d, Hq, len(ch), n + p) != qt), 2 * n)
    say(f"  {n} tokens in tiles of {qt}; with {pad} rows of padding the size alone gives tiles of "
        f"{P.prefill_tile_rows(d, Hq, len(ch), n + pad)}")
    qp = torch.cat([q, torch.zeros((pad, Hq, D), dtype=q.dtype, device=q.device)])
    out = torch.full_like(qp, 3.0)
    args = (to(cu), to(lk), int(np.diff(cu).max()), int(lk.max()), kv.k_cache, kv.v_cache, to(tab),
            1.0 / math.sqrt(D), to(items), qt)
    ref = P.paged_attn_prefill_ordered(q, *args)
    P.paged_attn_prefill_ordered(qp, *args, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out[:n], ref)
    assert bool((out[n:] == 3.0).all())
