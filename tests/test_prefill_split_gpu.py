"""GPU parity of split-K prefill (pkv_prefill_split_order + pkv_paged_attn_prefill_split) for
launches that would leave CUs idle: long items cut into key-range pieces, merged by log-sum-exp."""

import math

import numpy as np
import pytest

import workloads as W
from oracle import attention as OA
from tests.gpu_cases import check_tol, dev_rows, host_out, say

pytestmark = pytest.mark.gpu


def _chunk_case(cfg, seed, causal, window, chunk_index=None):
    """Admit the workload, store one chunk (the last by default) and return what a split call needs."""
    import torch
    import paged_kv_cache_kvcache_amd as P
    from paged_kv_cache_kvcache_amd import runner as R
    wl = W.prefill_workload(cfg, seed)
    Hq, Hkv, D = cfg["Hq"], cfg["Hkv"], cfg["D"]
    prompts = wl["prompts"]
    kv = R.PagedKV(wl["num_blocks"], Hkv, D, P.BF16, wl["free_order"], device="cuda", fill=0)
    ncached = [kv.alloc.add_seq(i, p["tokens"]) for i, p in enumerate(prompts)]
    n_new = [len(p["tokens"]) - c for p, c in zip(prompts, ncached)]
    chunks = W.pack_chunks(n_new, cfg["chunk"])
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()
    # every chunk's rows are stored (a later chunk's prompts may reuse blocks an earlier one stored)
    for c, ch in enumerate(chunks):
        rows = lambda key: dev_rows(np.concatenate([prompts[i][key][ncached[i]:] for i in ch]), "cuda")
        cu, lk, slots = kv.alloc.prefill_slots(ch, sum(n_new[i] for i in ch))
        kv.store(to(slots), rows("k"), rows("v"))
    ch = chunks[-1 if chunk_index is None else chunk_index]
    q = dev_rows(np.concatenate([prompts[i]["q"][ncached[i]:] for i in ch]), "cuda")
    cu, lk, _ = kv.alloc.prefill_slots(ch, int(q.shape[0]))
    tab, _ = kv.alloc.block_tables(ch, max(1, -(-int(lk.max()) // 256)))
    d = P.desc_of(kv.k_cache)
    pieces, merges, n_slots, qt = P.prefill_split_order(d, Hq, cu, lk, causal, window)
    args = (q, to(cu), to(lk), int(np.diff(cu).max()), int(lk.max()), kv.k_cache, kv.v_cache, to(tab),
            1.0 / math.sqrt(D))
    return dict(wl=wl, ch=ch, ncached=ncached, kv=kv, cu=cu, lk=lk, tab=tab, q=q, args=args, d=d, to=to,
                pieces=pieces, merges=merges, n_slots=n_slots, qt=qt)


def _split(c, causal, window, workspace=None):
    import torch
    import paged_kv_cache_kvcache_amd as P
    Hq = c["q"].shape[1]
    if workspace is None:
        nb = P.prefill_split_workspace_bytes(c["d"], Hq, c["n_slots"], c["qt"])
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda").fill_(0xFF)  # NaN bytes
    return P.paged_attn_prefill_split(*c["args"], c["to"](c["pieces"]), c["to"](c["merges"]), c["n_slots"], c["qt"],
                                      workspace, causal, window)


def _oracle_rows(c, causal, window):
    """The oracle's paged prefill (float64) over the chunk's prompts, their K/V rows laid out in a
    cache of their own (consecutive blocks) straight from the workload's draws."""
    wl = c["wl"]
    cfg = wl["cfg"]
    Hkv, D = cfg["Hkv"], cfg["D"]
    prompts = [wl["prompts"][i] for i in c["ch"]]

    def f64(a):  # the workload holds bf16 values as their bit patterns
        a = np.asarray(a)
        return (W.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a).astype(np.float64)

    lens = [len(p["tokens"]) for p in prompts]
    nblk = [-(-L // 256) for L in lens]
    kc = np.zeros((sum(nblk), Hkv, 256, D))
    vc = np.zeros_like(kc)
    tab = np.full((len(prompts), max(nblk)), -1, dtype=np.int64)
    off = 0
    for b, (p, L) in enumerate(zip(prompts, lens)):
        for j in range(nblk[b]):
            r0, r1 = 256 * j, min(L, 256 * (j + 1))
            kc[off + j, :, :r1 - r0] = f64(p["k"][r0:r1]).transpose(1, 0, 2)
            vc[off + j, :, :r1 - r0] = f64(p["v"][r0:r1]).transpose(1, 0, 2)
            tab[b, j] = off + j
        off += nblk[b]
    q = np.concatenate([f64(p["q"][n0:]) for p, n0 in zip(prompts, [c["ncached"][i] for i in c["ch"]])])
    return OA.prefill(q, kc, vc, tab, c["cu"], lens, 1.0 / math.sqrt(D), causal, window)


@pytest.mark.parametrize("over,causal,window", [
    ({}, True, 0),                                         # the 32-prompt workload's last chunk (6 prompts)
    (dict(B=3, ctx=[1900, 2000, 1300], group=1, shared=0, chunk=4096), True, 0),
    (dict(B=3, ctx=[1900, 2000, 1300], group=1, shared=0, chunk=4096), True, 700),
    (dict(B=2, ctx=[700, 400], group=1, shared=0, chunk=4096), False, 0),
    (dict(B=2, ctx=[1500, 900], Hq=8, Hkv=8, D=64, group=1, shared=0, chunk=4096), True, 0),
    (dict(B=2, ctx=[700, 400], Hq=16, Hkv=2, group=1, shared=0, chunk=4096), True, 0),
])
def test_split_prefill_matches_the_definition(over, causal, window):
    cfg = W.config("prefill_prefix", **over)
    c = _chunk_case(cfg, 0, causal, window)
    say(f"split prefill {over} causal={causal} window={window}: {len(c['pieces'])} pieces, "
        f"{len(c['merges'])} merges, {c['n_slots']} slots, tiles of {c['qt']}")
    assert len(c["merges"]) > 0, "the case must split"
    got = host_out(_split(c, causal, window))
    check_tol(got, _oracle_rows(c, causal, window), "bf16", "split prefill")


def test_split_prefill_is_deterministic_and_keeps_unsplit_items_bitwise():
    """Two calls (workspace filled differently before each) give the same bits; rows of items that
    are not split equal the ordered call bit for bit, and split rows agree with it to rounding."""
    import torch
    import paged_kv_cache_kvcache_amd as P
    cfg = W.config("prefill_prefix")
    c = _chunk_case(cfg, 0, True, 0)  # its last chunk splits 10 of its 18 items
    a = _split(c, True, 0)
    nb = P.prefill_split_workspace_bytes(c["d"], c["q"].shape[1], c["n_slots"], c["qt"])
    b = _split(c, True, 0, torch.zeros(nb, dtype=torch.uint8, device="cuda"))
    items, qt = P.prefill_work_order(c["d"], c["q"].shape[1], c["cu"], c["lk"], True)
    ref = P.paged_attn_prefill_ordered(*c["args"], c["to"](items), qt, True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert qt == c["qt"]
    split_codes = set(int(m) for m in c["merges"][:, 0])
    seq_of = np.repeat(np.arange(len(c["lk"])), np.diff(c["cu"]))
    tile_of = np.concatenate([np.arange(n) // qt for n in np.diff(c["cu"])])
    is_split = np.array([(int(s) << 16 | int(t)) in split_codes for s, t in zip(seq_of, tile_of)])
    assert is_split.any() and (~is_split).any()
    same = torch.from_numpy(~is_split).cuda()
    assert torch.equal(a[same], ref[same])
    err = (a.float() - ref.float()).abs().max().item()
    say(f"  split rows differ from the unsplit call by at most {err:.3e}")
    assert err <= 2e-2


def test_full_launch_is_not_split():
    """A chunk that fills the device keeps its work items whole, in the work order, with no merge,
    and the split call gives bitwise the ordered call."""
    import torch
    import paged_kv_cache_kvcache_amd as P
    cfg = W.config("prefill_prefix")
    c = _chunk_case(cfg, 0, True, 0, chunk_index=0)
    items, qt = P.prefill_work_order(c["d"], c["q"].shape[1], c["cu"], c["lk"], True)
    assert len(c["merges"]) == 0 and c["n_slots"] == 0
    assert (c["pieces"][:, 0] == items).all() and (c["pieces"][:, 3] == -1).all()
    got = P.paged_attn_prefill_split(*c["args"], c["to"](c["pieces"]), c["to"](c["merges"].reshape(-1, 4)), 0, qt,
                                     None, True, 0)
    ref = P.paged_attn_prefill_ordered(*c["args"], c["to"](items), qt, True)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
