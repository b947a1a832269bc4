"""Device-data checks on the GPU: with checks on, every kernel turns an out-of-range index it reads
from device memory into an entry in the error word instead of using it.

Every bad value here is chosen so that even an unchecked kernel would stay inside memory the test
owns: caches, tables, lengths, queries and outputs are views of buffers one block, row or entry
larger than the view the kernel is told about.  Each case checks the reported (code, where, value),
that the word is cleared by reading it, and that the valid part of the call still did its work.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_kvcache_amd as P
from tests.gpu_cases import say

pytestmark = pytest.mark.gpu
NB, HKV, HQ, D = 6, 2, 4, 128
SLOT, BLOCK_ID, LENGTH, SEQUENCE, RUN, CU_SEQLENS, ROWS = 1, 2, 3, 4, 5, 6, 7


@pytest.fixture
def checks(gpu):
    P.set_device_checks(True)
    assert P.device_error() == (0, 0, 0)
    yield gpu
    P.set_device_checks(False)
    P.device_error()


def _caches(dev, dtype=torch.bfloat16, fill=0):
    """K and V caches of NB blocks as views of NB + 1 blocks (an unchecked access to block NB stays
    inside the allocation)."""
    full = [torch.full((NB + 1, HKV, 256, D), fill, dtype=dtype, device=dev) for _ in range(2)]
    return full, [f[:NB] for f in full]


def _i32(x, dev):
    return torch.tensor(x, dtype=torch.int32, device=dev)


def _expect(code, where, value):
    got = P.device_error()
    say(f"  device error {got}")
    assert got == (code, where, value)
    assert P.device_error() == (0, 0, 0)  # reading cleared it


def test_no_error_with_valid_inputs(checks):
    dev = checks
    _, (kc, vc) = _caches(dev)
    rows = torch.randn(3, HKV, D, device=dev).to(torch.bfloat16)
    P.kv_store(rows, rows, _i32([0, 300, NB * 256 - 1], dev), kc, vc)
    _expect(0, 0, 0)


def test_store_skips_a_slot_outside_the_pool(checks):
    dev = checks
    full, (kc, vc) = _caches(dev)
    rows = torch.randn(3, HKV, D, device=dev).to(torch.bfloat16)
    P.kv_store(rows, rows, _i32([5, NB * 256 + 7, 600], dev), kc, vc)
    _expect(SLOT, 1, NB * 256 + 7)
    assert torch.equal(kc[0, :, 5], rows[0]) and torch.equal(kc[2, :, 600 - 512], rows[2])
    assert not full[0][NB].any()  # the block past the pool was not written


def test_quantising_store_rejects_a_bad_run(checks):
    dev = checks
    full, (kc, vc) = _caches(dev, torch.int8)
    ks = torch.zeros((NB, HKV), device=dev)
    vs = torch.zeros_like(ks)
    rows = torch.randn(4, HKV, D, device=dev).to(torch.bfloat16)
    slots = _i32([256, 257, 258, 259], dev)
    # run 1 claims no rows (length 0); run 0 is valid and still stored
    runs = (_i32([0, 1, 1, 0], dev), 2, 1)
    P.kv_store_quant(rows, rows, slots, kc, vc, ks, vs, runs=runs)
    _expect(RUN, 1, 1)
    assert ks[1].abs().sum() > 0 and kc[1, :, 0].abs().sum() > 0


def test_quantising_store_rejects_a_run_leaving_its_block(checks):
    dev = checks
    _, (kc, vc) = _caches(dev, torch.int8)
    ks = torch.zeros((NB, HKV), device=dev)
    rows = torch.randn(3, HKV, D, device=dev).to(torch.bfloat16)
    slots = _i32([254, 255, 256], dev)  # three rows from offset 254 would cross into the next block
    P.kv_store_quant(rows, rows, slots, kc, vc, ks, ks.clone(), runs=(_i32([0, 3], dev), 1, 3))
    _expect(SLOT, 0, 254)
    assert not kc.any()


def test_block_copy_rejects_bad_pairs(checks):
    dev = checks
    full, (kc, vc) = _caches(dev, fill=1)
    kc[3].fill_(2)
    P.copy_blocks(_i32([3, NB], dev), _i32([4, 5], dev), kc, vc, _i32([256, 10], dev))
    _expect(BLOCK_ID, 1, NB)
    assert torch.equal(kc[4], kc[3]) and bool((kc[5] == 1).all())
    P.copy_blocks(_i32([3], dev), _i32([4], dev), kc, vc, _i32([300], dev))
    _expect(ROWS, 0, 300)


def _decode(dev, tables, lens, order=None, B=2, max_ctx=512, rows=3, max_splits=0):
    """Decode over views: q/out/lens/order/tables one row or entry larger than the kernel is told."""
    _, (kc, vc) = _caches(dev)
    kc.normal_()
    vc.normal_()
    q_full = torch.randn(B + 1, HQ, D, device=dev).to(torch.bfloat16)
    out_full = torch.zeros_like(q_full)
    tab_full = _i32(tables, dev)
    lens_full = _i32(lens, dev)
    order_t = None if order is None else _i32(order, dev)[:B]
    P.paged_attn_decode(q_full[:B], kc, vc, tab_full[:B], lens_full[:B], max_ctx, 0.088, out=out_full[:B],
                        seq_order=order_t, max_splits=max_splits)
    return out_full


@pytest.mark.parametrize("splits", [1, 2])
def test_decode_rejects_a_block_id_outside_the_pool(checks, splits):
    """With one split the rejected workgroup writes nothing; with two, its split is marked and the
    reduce leaves the sequence's output unwritten rather than merge a stale partial."""
    out = _decode(checks, [[0, NB], [2, 3], [1, 1]], [300, 400, 1], max_splits=splits)
    _expect(BLOCK_ID, 0, NB)
    assert out[1].abs().sum() > 0  # the valid sequence was attended
    assert not out[0].any()


def test_decode_rejects_a_length_the_table_cannot_hold(checks):
    out = _decode(checks, [[0, 1], [2, 3], [4, 5]], [513, 200, 1])
    _expect(LENGTH, 0, 513)
    assert out[1].abs().sum() > 0 and not out[0].any()


def test_decode_rejects_a_length_above_max_context_len(checks):
    """The table could hold it, but the split plan covers only max_context_len keys: without the
    check the tail of the context would be silently left out."""
    out = _decode(checks, [[0, 1], [2, 3], [4, 5]], [301, 200, 1], max_ctx=300)
    _expect(LENGTH, 0, 301)
    assert out[1].abs().sum() > 0 and not out[0].any()


def test_decode_rejects_a_launch_order_entry_outside_the_batch(checks):
    out = _decode(checks, [[0, 1], [2, 3], [4, 5]], [100, 200, 1], order=[2, 1, 0])
    _expect(SEQUENCE, 0, 2)
    assert out[1].abs().sum() > 0


def test_fused_store_rejects_a_slot_outside_the_pool(checks):
    dev = checks
    _, (kc, vc) = _caches(dev)
    q = torch.randn(2, HQ, D, device=dev).to(torch.bfloat16)
    new = torch.randn(2, HKV, D, device=dev).to(torch.bfloat16)
    tab = _i32([[0, 1], [2, 3]], dev)
    P.decode_store_attend(q, new, new, _i32([NB * 256 + 3, 2 * 256 + 9], dev), kc, vc, tab, _i32([300, 10], dev),
                          512, 0.088)
    _expect(SLOT, 0, NB * 256 + 3)
    assert torch.equal(kc[2, :, 9], new[1])


def _prefill(dev, cu, lk, tables, total_q=96, max_q=64, max_k=512):
    _, (kc, vc) = _caches(dev)
    kc.normal_()
    vc.normal_()
    q = torch.randn(total_q, HQ, D, device=dev).to(torch.bfloat16)
    out = torch.zeros_like(q)
    P.paged_attn_prefill(q, _i32(cu, dev), _i32(lk, dev), max_q, max_k, kc, vc, _i32(tables, dev), 0.088, True,
                         out=out)
    return out


def test_prefill_rejects_a_block_id_outside_the_pool(checks):
    out = _prefill(checks, [0, 64, 96], [300, 32], [[0, NB], [2, 3]])
    _expect(BLOCK_ID, 0, NB)
    assert out[64:].abs().sum() > 0 and not out[:64].any()


def test_prefill_rejects_a_key_length_the_table_cannot_hold(checks):
    out = _prefill(checks, [0, 64, 96], [64, 600], [[0, 1], [2, 3]])
    _expect(LENGTH, 1, 600)
    assert out[:64].abs().sum() > 0


def test_prefill_rejects_decreasing_cu_seqlens(checks):
    _prefill(checks, [0, 64, 32], [64, 64], [[0, 1], [2, 3]])
    code, where, value = P.device_error()
    assert (code, where, value) == (CU_SEQLENS, 2, 32)


def test_ordered_prefill_rejects_an_item_outside_the_call(checks):
    dev = checks
    _, (kc, vc) = _caches(dev)
    kc.normal_()
    vc.normal_()
    q = torch.randn(96, HQ, D, device=dev).to(torch.bfloat16)
    out = torch.zeros_like(q)
    # items of sequence 0 (tile 0) and sequence 1 (tile 0), then a sequence that does not exist
    items = _i32([0, 1 << 16, 2 << 16], dev)
    P.paged_attn_prefill_ordered(q, _i32([0, 64, 96], dev), _i32([64, 32], dev), 64, 64, kc, vc,
                                 _i32([[0, 1], [2, 3]], dev), 0.088, items, 64, True, out=out)
    _expect(RUN, 2, 2 << 16)
    assert out[:64].abs().sum() > 0 and out[64:].abs().sum() > 0


SHARED = 8


@pytest.mark.parametrize("case,split", [("tables differ", False), ("shared past a context", False),
                                        ("block outside the pool", False), ("tables differ", True),
                                        ("shared past a context", True), ("block outside the pool", True),
                                        ("shared past its bound", True)])
def test_grouped_decode_rejects_a_bad_group(checks, case, split):
    """pkv_paged_attn_decode_grouped (split: pkv_paged_attn_decode_grouped_split over two splits, the
    workspace filled with NaN bytes), two groups of two sequences: group 0 is bad in one way, group 1
    is valid.  Group 0's outputs stay unwritten, group 1's match the plain decode."""
    dev = checks
    _, (kc, vc) = _caches(dev)
    kc.copy_(torch.randn_like(kc, dtype=torch.float32).to(kc.dtype))
    vc.copy_(torch.randn_like(vc, dtype=torch.float32).to(vc.dtype))
    tab = [[0, 1, -1], [0, 1, -1], [3, 4, -1], [3, 5, -1]]
    lens, shared = [400, 400, 300, 300], [400, 256]
    expect = None
    if case == "tables differ":  # member 1 has its own block at entry 1, inside the claimed 400 keys
        tab[1][1] = 2
        expect = (SHARED, 1, 1)
    elif case == "shared past a context":
        shared[0] = 500
        expect = (LENGTH, 0, 500 if split else 400)  # over splits, the bound (400) is checked first
    elif case == "shared past its bound":  # 400 shared keys, but the call's bound is 300
        expect = (LENGTH, 0, 400)
    else:
        tab[1][1] = tab[0][1] = NB  # shared, but outside the pool
        expect = (BLOCK_ID, 0, NB)
    q = torch.randn(4, HQ, D, device=dev).to(torch.bfloat16)
    out = torch.full_like(q, 7.0)
    t, ln = _i32(tab, dev), _i32(lens, dev)
    if split:
        bound = 300 if case == "shared past its bound" else 400
        ws = torch.full((P.decode_grouped_workspace_bytes(4, HQ, D, bound, 2),), 0xFF, dtype=torch.uint8, device=dev)
        assert ws.numel() > 0  # the call splits
        P.paged_attn_decode_grouped_split(q, kc, vc, t, ln, 400, 0.088, 2, _i32(shared, dev), bound, 2, workspace=ws,
                                          out=out)
    else:
        P.paged_attn_decode_grouped(q, kc, vc, t, ln, 400, 0.088, 2, _i32(shared, dev), out=out)
    _expect(*expect)
    assert bool((out[:2] == 7.0).all())
    ref = P.paged_attn_decode(q[2:], kc, vc, t[2:], ln[2:], 400, 0.088)
    torch.cuda.synchronize()
    assert (out[2:].float() - ref.float()).abs().max().item() < 2e-2


def test_split_prefill_rejects_a_piece_slot_outside_the_workspace(checks):
    """Pieces of sequence 0's tile split over slots 0 and 1, then a piece of sequence 1 that names
    slot 2 of a call with 2 slots (the workspace holds a third slot, so even an unchecked write
    would stay in memory the test owns): error 5 for that piece, sequence 0 still merged."""
    dev = checks
    _, (kc, vc) = _caches(dev)
    kc.normal_()
    vc.normal_()
    q = torch.randn(96, HQ, D, device=dev).to(torch.bfloat16)
    out = torch.zeros_like(q)
    desc = P.desc_of(kc)
    ws = torch.zeros(P.prefill_split_workspace_bytes(desc, HQ, 3, 64), dtype=torch.uint8, device=dev)
    pieces = _i32([[0, 0, 2, 0], [0, 2, 4, 1], [1 << 16, 0, 2**31 - 1, 2]], dev)
    merges = _i32([[0, 0, 2, 0]], dev)
    P.paged_attn_prefill_split(q, _i32([0, 64, 96], dev), _i32([256, 32], dev), 64, 256, kc, vc,
                               _i32([[0, 1], [2, 3]], dev), 0.088, pieces, merges, 2, 64, ws, True, out=out)
    _expect(RUN, 2, 1 << 16)
    assert out[:64].abs().sum() > 0 and not out[64:].any()
