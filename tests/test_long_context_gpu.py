"""Contexts longer than 64 blocks (16,384 tokens) on the GPU: the attention kernels hold a
sequence's block table 64 entries at a time and load the next window when a sequence crosses
one.  Both kernels are checked against the oracle across such a crossing."""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
import workloads as W
from oracle import attention as OT
from tests.gpu_cases import check_tol, gpu_decode, host_out, oracle_decode, say, to_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("max_splits", [1, 0])
def test_decode_crosses_block_table_window(max_splits):
    """17,000- and 20,000-token contexts: one split walks 67 and 79 blocks (two windows)."""
    cfg = W.config("qwen3_decode", B=3, ctx=[20000, 17000, 300])
    wl = W.decode_workload(cfg, 0)
    say(f"long decode lens={wl['lens']} max_splits={max_splits}")
    out, _, _ = gpu_decode(wl, "cuda", max_splits=max_splits)
    check_tol(host_out(out), oracle_decode(wl), "bf16", f"long decode max_splits={max_splits}")


@pytest.mark.parametrize("name,dtype,fused", [("long_decode", "bf16", False), ("long_decode", "bf16", True),
                                              ("int8_decode", "i8", False), ("tiny_fp32", "f32", False)])
def test_decode_next_block_loads_across_window(name, dtype, fused):
    """The split kernel requests each block's K tile while the previous block is still being
    attended; across a block-table window reload (67 and 79 blocks in one split) and partial last
    tiles, with rows nobody writes holding NaN (int8: -128), the result still matches the oracle."""
    cfg = W.config(name, B=3, ctx=[20000, 17000, 300], pool=None)  # pool sized from the lengths
    assert cfg["dtype"] == dtype
    wl = W.decode_workload(cfg, 1)
    fill = -128 if dtype == "i8" else float("nan")
    say(f"long decode {name} lens={wl['lens']} fused={fused}")
    out, _, _ = gpu_decode(wl, "cuda", max_splits=1, fill=fill, fused=fused)
    check_tol(host_out(out), oracle_decode(wl), dtype, f"long decode {name} fused={fused}")


def test_prefill_crosses_block_table_window():
    """96 new tokens after a 16,904-token cached prefix (67 blocks, two windows), next to a short
    prompt; physical blocks shuffled over the pool."""
    rng = np.random.default_rng(11)
    Hq, Hkv, D = 16, 8, 128
    n_keys, n_new = [17000, 700], [96, 700]
    nblk = [-(-L // 256) for L in n_keys]
    pool = sum(nblk) + 7
    perm = rng.permutation(pool).astype(np.int32)
    tables = np.full((2, max(nblk)), -1, np.int32)
    tables[0, :nblk[0]] = perm[:nblk[0]]
    tables[1, :nblk[1]] = perm[nblk[0]:nblk[0] + nblk[1]]
    kc = W.f32_to_bf16_bits(rng.standard_normal((pool, Hkv, 256, D), dtype=np.float32))
    vc = W.f32_to_bf16_bits(rng.standard_normal((pool, Hkv, 256, D), dtype=np.float32))
    q = W.f32_to_bf16_bits(rng.standard_normal((sum(n_new), Hq, D), dtype=np.float32))
    cu = np.array([0, n_new[0], sum(n_new)], np.int32)
    lk = np.array(n_keys, np.int32)
    scale = 1.0 / math.sqrt(D)

    dev = torch.device("cuda")
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    got = P.paged_attn_prefill(bf(q), i32(cu), i32(lk), max(n_new), max(n_keys), bf(kc), bf(vc), i32(tables),
                               scale, True)
    torch.cuda.synchronize()
    ref = OT.prefill(to_f64(q), to_f64(kc), to_f64(vc), tables, cu, lk, scale, causal=True)
    check_tol(host_out(got), ref, "bf16", "long prefill")
