"""Decode steps replayed from HIP graphs (runner.GraphedDecodeBatch) against the same steps run
eagerly (runner.DecodeBatch), on two pools that receive identical histories and inputs.

Each graph replay must give bitwise the eager step's output; between the replays the test runs the
eager step and synchronises, and after the last step both caches must be bitwise equal.  Two staging
sets alternate, so every captured graph is replayed three times.  The last step's outputs are also
checked against the oracle's attention over the graphed pool's caches.
"""

import math

import numpy as np
import pytest
import torch

import workloads as W
from oracle import attention as OT
from paged_kv_cache_kvcache_amd import runner as R
from tests.gpu_cases import DT, check_tol, dev_rows, kv_arrays, say

pytestmark = pytest.mark.gpu
STEPS = 6

CASES = [
    ("qwen3_decode", dict(B=24, ctx=(100, 1400)), False, 0),
    ("qwen3_decode", dict(B=24, ctx=(100, 1400)), True, 0),
    ("qwen3_decode", dict(B=24, ctx=(300, 1400)), False, 3),
    ("int8_decode", dict(B=12, ctx=(100, 1500), Hq=16, Hkv=8), False, 0),
    ("int8_decode", dict(B=12, ctx=(100, 1500), Hq=16, Hkv=8), True, 3),
    ("tiny_fp32", dict(pool=None), False, 0),
]


def _pool(wl, device, nb):
    cfg = wl["cfg"]
    # the same fill in both pools, so that rows no step writes compare equal too
    kv = R.PagedKV(nb, cfg["Hkv"], cfg["D"], DT[cfg["dtype"]], W.free_order(cfg, 0, nb), device=device, fill=0)
    parts = [kv_arrays(s, cfg["dtype"]) for s in wl["seqs"]]
    R.admit_and_store(kv, list(range(len(parts))), [s["tokens"] for s in wl["seqs"]], [p[0] for p in parts],
                      [p[1] for p in parts], [p[2] for p in parts], [p[3] for p in parts])
    return kv


def _step_inputs(cfg, s, B, rng, device):
    inp = W.decode_step_inputs(cfg, 0, s, B)
    out = dict(tokens=inp["tokens"], q=dev_rows(inp["q"], device))
    if cfg["dtype"] == "i8":
        # pre-quantised codes and per-(token, head) scales; the eager and graphed pools get the same
        for x in ("k", "v"):
            out[x] = dev_rows(rng.integers(-127, 128, size=(B, cfg["Hkv"], cfg["D"])).astype(np.int8), device)
            out[x + "s"] = dev_rows(rng.uniform(0.005, 0.02, size=(B, cfg["Hkv"])).astype(np.float32), device)
    else:
        out["k"], out["v"] = dev_rows(inp["k"], device), dev_rows(inp["v"], device)
        out["ks"] = out["vs"] = None
    return out


@pytest.mark.parametrize("name,over,fused,splits", CASES)
def test_graph_replays_match_eager_steps(gpu, name, over, fused, splits):
    cfg = W.config(name, **over)
    wl = W.decode_workload(cfg, 0)
    B, Hq, D = len(wl["lens"]), cfg["Hq"], cfg["D"]
    nb = W.pool_blocks(dict(cfg, pool=None), [L + STEPS for L in wl["lens"]])
    max_ctx = max(wl["lens"]) + STEPS
    scale = 1.0 / math.sqrt(D)
    say(f"  {name} B={B} fused={fused} max_splits={splits}: {nb} blocks")
    kv_e, kv_g = _pool(wl, gpu, nb), _pool(wl, gpu, nb)
    eager = R.DecodeBatch(kv_e, Hq, list(range(B)), max_ctx, splits, fused=fused)
    graphed = R.GraphedDecodeBatch(kv_g, Hq, list(range(B)), max_ctx, scale, splits, fused=fused)
    rng = np.random.default_rng(1)
    for s in range(STEPS):
        x = _step_inputs(cfg, s, B, rng, gpu)
        out_e = eager.step(x["tokens"], x["q"], x["k"], x["v"], scale, k_scale_new=x["ks"],
                           v_scale_new=x["vs"]).clone()
        torch.cuda.synchronize()
        graphed.q.copy_(x["q"])
        graphed.k_new.copy_(x["k"])
        graphed.v_new.copy_(x["v"])
        if x["ks"] is not None:
            graphed.k_scale_new.copy_(x["ks"])
            graphed.v_scale_new.copy_(x["vs"])
        out_g = graphed.step(x["tokens"])
        torch.cuda.synchronize()
        assert torch.equal(out_e, out_g), f"step {s}: graph replay differs from the eager step"
    for a, b in ((kv_e.k_cache, kv_g.k_cache), (kv_e.v_cache, kv_g.v_cache), (kv_e.k_scale, kv_g.k_scale)):
        assert a is None or torch.equal(a, b)
    # the last step against the oracle, over the graphed pool's caches
    ids = list(range(B))
    tab, lens = kv_g.alloc.block_tables(ids, -(-max_ctx // 256))
    host = lambda t: None if t is None else t.float().cpu().numpy()
    ref = OT.decode(host(graphed.q), host(kv_g.k_cache), host(kv_g.v_cache), tab, lens, scale,
                    host(kv_g.k_scale), host(kv_g.v_scale))
    check_tol(host(graphed.out).astype(np.float64), ref, cfg["dtype"], f"{name} last graphed step")
