"""pkv_paged_attn_decode_noalloc against pkv_paged_attn_decode (needs an MI355X).

The allocation-free entry point keeps its split partials in the library's per-device scratch.  Its
output must equal, bit for bit, the workspace entry point's on the same inputs and plan, on two
calls in a row (the second smaller, so stale partials of the first would show), and a plan larger
than the scratch must be refused before anything is launched.
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
import workloads as W
from tests.gpu_cases import DT, check_tol, dev_rows, say

pytestmark = pytest.mark.gpu


def _setup(gpu, name, seed, **over):
    """A decode workload admitted and stored through the native block manager (new token included)."""
    from paged_kv_cache_kvcache_amd import runner as R
    from tests.gpu_cases import kv_arrays
    cfg = W.config(name, **over)
    wl = W.decode_workload(cfg, seed)
    kv = R.PagedKV(wl["num_blocks"], cfg["Hkv"], cfg["D"], DT[cfg["dtype"]], wl["free_order"], device=gpu)
    parts = [kv_arrays(s, cfg["dtype"]) for s in wl["seqs"]]
    R.admit_and_store(kv, list(range(len(wl["lens"]))), [s["tokens"] for s in wl["seqs"]], [p[0] for p in parts],
                      [p[1] for p in parts], [p[2] for p in parts], [p[3] for p in parts])
    mb = max(1, -(-max(wl["lens"]) // 256))
    tab, lens = kv.alloc.block_tables(list(range(len(wl["lens"]))), mb)
    q = dev_rows(np.stack([s["q"] for s in wl["seqs"]]), gpu)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(gpu)
    return cfg, wl, kv, q, to(tab), to(lens)


@pytest.mark.parametrize("name,over,splits", [
    ("long_decode", dict(B=6), 0),  # the automatic plan splits these contexts
    ("int8_decode", dict(B=4, ctx=(2000, 6000)), 5),
    ("tiny_fp32", {}, 3),
])
def test_noalloc_equals_workspace_decode_on_two_calls(gpu, name, over, splits):
    from oracle import steps as OS
    big = _setup(gpu, name, 0, **over)
    small_over = dict(over, B=max(1, over.get("B", 4) - 2)) if name != "tiny_fp32" else dict(ctx=[3, 300], B=2)
    small = _setup(gpu, name, 1, **small_over)
    for tag, (cfg, wl, kv, q, tab, lens) in (("first", big), ("second, smaller", small)):
        max_ctx = max(wl["lens"])
        plan = P.decode_plan(len(wl["lens"]), cfg["Hkv"], max_ctx, splits)
        need = P.decode_workspace_bytes(len(wl["lens"]), cfg["Hq"], cfg["D"], cfg["Hkv"], max_ctx, splits)
        say(f"noalloc {name} ({tag}): B={len(wl['lens'])} plan={plan} workspace={need} bytes")
        assert plan[0] > 1 and need > 0, "the case must use the split workspace"
        scale = 1.0 / math.sqrt(cfg["D"])
        ref = P.paged_attn_decode(q, kv.k_cache, kv.v_cache, tab, lens, max_ctx, scale, max_splits=splits,
                                  k_scale=kv.k_scale, v_scale=kv.v_scale)
        out = torch.full_like(ref, float("nan") if cfg["dtype"] != "i8" else 7.0)
        P.paged_attn_decode_noalloc(q, kv.k_cache, kv.v_cache, tab, lens, max_ctx, scale, out, max_splits=splits,
                                    k_scale=kv.k_scale, v_scale=kv.v_scale)
        torch.cuda.synchronize()
        bits = lambda t: t.contiguous().view(torch.uint8)
        assert torch.equal(bits(out), bits(ref)), "noalloc output differs from the workspace call's"
        # and against the oracle, to the workload's tolerance
        got = out.float().cpu().numpy().astype(np.float64)
        exp = np.stack([OS.decode_one_sequence(cfg, s, L) for s, L in zip(wl["seqs"], wl["lens"])])
        check_tol(got, exp, cfg["dtype"], f"noalloc {name} {tag}")


def test_noalloc_refuses_a_plan_larger_than_its_scratch(gpu):
    """B x Hq x splits x (D + 2) x 4 bytes over PKV_DECODE_SCRATCH_BYTES: refused on the host with
    PKV_ERR_SMALL_BUFFER, and the output is not touched."""
    B, Hq, Hkv, D, ctx = 64, 32, 8, 128, 8192
    need = P.decode_workspace_bytes(B, Hq, D, Hkv, ctx, 32)
    assert need > (16 << 20)
    kc = torch.zeros((4, Hkv, 256, D), dtype=torch.bfloat16, device=gpu)
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=gpu)
    tab = torch.zeros((B, 32), dtype=torch.int32, device=gpu)
    lens = torch.ones(B, dtype=torch.int32, device=gpu)
    out = torch.full_like(q, 5.0)
    with pytest.raises(P.PkvError) as e:
        P.paged_attn_decode_noalloc(q, kc, kc, tab, lens, ctx, 0.1, out, max_splits=32)
    assert e.value.code == P.ERR_SMALL_BUFFER
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())
