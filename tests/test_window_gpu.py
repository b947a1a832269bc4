"""Sliding-window decode and prefill on the GPU against the oracle.

Random paged caches (a random permutation of physical blocks), windows that are shorter than one
block, cross block edges, cover the whole context or exceed it; decode with the split planner's
choice and forced splits; prefill with cached prefixes, both workgroup shapes (the eight-wavefront
one on a large launch, checked on sampled rows), and several query-group sizes.
"""

import math

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
import workloads as W
from oracle import attention as OT
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu
TOL = {P.F32: (1e-5, 1e-6), P.BF16: (2e-2, 2e-3), P.I8: (5e-2, 5e-3)}


def _paged(rng, lens, Hkv, D, dt, device):
    """Caches holding each sequence's rows at a random placement: (device caches, host float64 copies
    as the cache stores them, block table, int8 scales)."""
    nblk = [-(-L // 256) for L in lens]
    nb = sum(nblk) + 2
    perm = rng.permutation(nb)
    bt = np.full((len(lens), max(1, max(nblk))), -1, dtype=np.int32)
    o = 0
    for b, k in enumerate(nblk):
        bt[b, :k] = perm[o:o + k]
        o += k
    x = rng.standard_normal((2, nb, Hkv, 256, D)).astype(np.float32)
    if dt == P.I8:
        codes = rng.integers(-127, 128, size=x.shape).astype(np.int8)
        scales = (rng.random((2, nb, Hkv)) * 0.05 + 0.001).astype(np.float32)
        host = [codes[i].astype(np.float64) for i in range(2)]
        dev = [torch.from_numpy(codes[i]).to(device) for i in range(2)]
        return dev, host, bt, scales
    if dt == P.BF16:
        x = W.bf16_bits_to_f32(W.f32_to_bf16_bits(x))
        dev = [torch.from_numpy(x[i]).to(device).to(torch.bfloat16) for i in range(2)]
    else:
        dev = [torch.from_numpy(x[i]).to(device) for i in range(2)]
    return dev, [x[i].astype(np.float64) for i in range(2)], bt, None


def _check(got, ref, dt, what):
    err = np.abs(got - ref)
    say(f"  {what}: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")
    assert err.max() < TOL[dt][0] and err.mean() < TOL[dt][1], what


@pytest.mark.parametrize("dt,D,Hq,Hkv", [(P.BF16, 128, 16, 8), (P.F32, 64, 4, 2), (P.I8, 128, 32, 32)])
def test_windowed_decode(gpu, dt, D, Hq, Hkv):
    rng = np.random.default_rng(31)
    lens = [1, 255, 256, 257, 600, 1000, 2000, 3333]
    dev, host, bt, scales = _paged(rng, lens, Hkv, D, dt, gpu)
    q = rng.standard_normal((len(lens), Hq, D)).astype(np.float32)
    if dt != P.F32:
        q = W.bf16_bits_to_f32(W.f32_to_bf16_bits(q))
    qd = torch.from_numpy(q).to(gpu)
    if dt != P.F32:
        qd = qd.to(torch.bfloat16)
    ks = vs = None
    if scales is not None:
        ks, vs = (torch.from_numpy(scales[i]).to(gpu) for i in range(2))
    btd = torch.from_numpy(bt).to(gpu)
    cl = torch.tensor(lens, dtype=torch.int32, device=gpu)
    scale = 1.0 / math.sqrt(D)
    for window in (1, 100, 256, 257, 1000, 5000):
        ref = OT.decode(q, host[0], host[1], bt, lens, scale, None if scales is None else scales[0],
                        None if scales is None else scales[1], window=window)
        for splits in (0, 1, 3):
            out = P.paged_attn_decode(qd, dev[0], dev[1], btd, cl, max(lens), scale, max_splits=splits,
                                      k_scale=ks, v_scale=vs, window=window)
            _check(out.float().cpu().numpy(), ref, dt, f"window {window}, splits {splits}")


def _prefill_case(gpu, rng, Hq, Hkv, D, lens_k, n_q, window, sample=None):
    dev, host, bt, _ = _paged(rng, lens_k, Hkv, D, P.BF16, gpu)
    cu = np.concatenate([[0], np.cumsum(n_q)]).astype(np.int32)
    q = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32)))
    scale = 1.0 / math.sqrt(D)
    out = P.paged_attn_prefill(torch.from_numpy(q).to(gpu).to(torch.bfloat16), torch.from_numpy(cu).to(gpu),
                               torch.tensor(lens_k, dtype=torch.int32, device=gpu), max(n_q), max(lens_k), dev[0],
                               dev[1], torch.from_numpy(bt).to(gpu), scale, True, window=window)
    got = out.float().cpu().numpy()
    if sample is None:
        return got, OT.prefill(q, host[0], host[1], bt, cu, lens_k, scale, window=window)
    # sampled rows against the plain definition on each sequence's own rows
    G = Hq // Hkv
    rows, refs = [], []
    for b in range(len(lens_k)):
        pick = sorted(set([0, n_q[b] - 1] + rng.integers(0, n_q[b], size=sample).tolist()))
        for i in pick:
            pos = lens_k[b] - n_q[b] + i
            lo = max(0, pos - window + 1)
            r = np.zeros((Hq, D))
            for g in range(Hkv):
                kk = OT.gather(host[0], bt[b], pos + 1, g)[lo:]
                vv = OT.gather(host[1], bt[b], pos + 1, g)[lo:]
                for h in range(g * G, (g + 1) * G):
                    r[h] = OT.attend(q[cu[b] + i, h].astype(np.float64), kk, vv, scale)
            rows.append(cu[b] + i)
            refs.append(r)
    return got[rows], np.stack(refs)


@pytest.mark.parametrize("G,D", [(1, 128), (2, 128), (8, 128), (2, 64)])
def test_windowed_prefill(gpu, G, D):
    rng = np.random.default_rng(32 + G + D)
    Hkv = 2
    lens_k = [300, 5, 700, 1100]
    n_q = [45, 5, 700, 400]   # cached prefixes on the first and the last
    for window in (1, 64, 100, 257, 1000):
        got, ref = _prefill_case(gpu, rng, G * Hkv, Hkv, D, lens_k, n_q, window)
        _check(got, ref, P.BF16, f"G {G} D {D} window {window}")


def test_windowed_prefill_wide_workgroups(gpu):
    """A launch large enough for eight-wavefront workgroups (G = 1: 256 tokens per workgroup)."""
    rng = np.random.default_rng(40)
    Hkv, D = 8, 128
    lens_k = [5000, 4000, 5000, 5000]
    n_q = [5000, 3000, 4500, 5000]
    QT8 = 256
    items8 = (sum(n_q) // QT8 + len(n_q)) * Hkv
    assert items8 >= 2 * 256
    for window in (200, 1500):
        got, ref = _prefill_case(gpu, rng, Hkv, Hkv, D, lens_k, n_q, window, sample=6)
        _check(got, ref, P.BF16, f"wide, window {window}")


@pytest.mark.parametrize("name,window", [("long_decode", 1024), ("qwen3_decode", 512), ("int8_decode", 700)])
def test_windowed_decode_full_size_sampled(gpu, name, window):
    """The full-size workloads with the window the bench measures, in its launch configuration
    (automatic split plan over the window's span): eight sampled sequences against the plain
    definition over their own last ``window`` rows."""
    from oracle import steps as OS
    from tests.gpu_cases import check_tol, gpu_decode, host_out
    cfg = W.config(name)
    wl = W.decode_workload(cfg, 0)
    say(f"full-size {name}, window {window}: B={len(wl['lens'])}")
    out, _, _ = gpu_decode(wl, gpu, max_context_len=max(wl["lens"]) + 23, window=window)
    got = host_out(out)
    sample = np.random.default_rng(11).choice(len(wl["lens"]), size=8, replace=False)
    ref = np.stack([OS.decode_one_sequence(cfg, wl["seqs"][b], wl["lens"][b], window) for b in sample])
    check_tol(got[sample], ref, cfg["dtype"], f"{name} window {window}, 8 sampled sequences")
