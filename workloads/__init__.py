"""Seeded synthetic inputs for paged-KV attention, shared by the GPU path's tests and the oracle.

This module only *draws* inputs: sequence lengths, token ids, Q/K/V values,
the initial order of the free block pool, and the int8 encoding of the int8
workload's KV.  It holds none of the attention arithmetic and none of the block
manager's logic, so neither side of a parity test can borrow the other's
mistakes through it.

Every draw comes from a NumPy ``default_rng`` stream keyed by
``(seed, workload id, purpose, index)``, so any single sequence can be
regenerated on its own (the oracle checks sampled sequences of the full-size
workloads that way).

Workloads (the shapes of the Qwen3-0.6B / 7B engines the pages benchmark;
"1200行代码挑战vLLM", §性能对比; intelliparadigm.com Nano-vLLM article, §4):

* ``tiny_fp32``  -- 4 sequences of context {1, 255, 256, 600}; 4 Q / 2 KV heads,
  head_dim 64, fp32, pool of 8 blocks, N(0,1).
* ``qwen3_decode`` -- batch 256, context U[100, 2048], 16 Q / 8 KV heads,
  head_dim 128, bf16 KV, N(0,1) * 0.5.
* ``prefill_prefix`` -- 32 prompts of length U[100, 1024] in groups of 8 that
  share their first 512 tokens (ids and Q/K/V), 16 Q / 8 KV heads, head_dim
  128, bf16, N(0,1), packed greedily into chunks of at most 4096 new tokens.
* ``long_decode`` -- batch 64, context U[4096, 8192], 32 Q / 8 KV heads,
  head_dim 128, bf16, N(0,1).
* ``int8_decode`` -- batch 128, context U[512, 8192], 32 Q / 32 KV heads,
  head_dim 128; K/V drawn N(0,1), rounded to bf16, then stored as int8 with one
  fp32 absmax/127 scale per (block, KV head); bf16 query.
* ``prefill_long`` -- 4 prompts of length U[4096, 12288] in pairs that share
  their first 2048 tokens, 16 Q / 8 KV heads, head_dim 128, bf16, N(0,1); each
  chunk is filled to 4096 new tokens, splitting prompts across chunks.
* ``int8_store`` -- the prompts of ``prefill_prefix``, for the quantising store.

Pool size (the Qwen3 workload asks for "total tokens x 1.1", which does not fit
once every sequence rounds up to whole blocks): ceil(1.1 * sum(ceil(L/256)))
blocks, except the tiny workload's fixed 8.
"""

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BLOCK = 256
VOCAB = 32000

CONFIGS = {
    "tiny_fp32": dict(id=1, kind="decode", B=4, ctx=[1, 255, 256, 600], Hq=4, Hkv=2, D=64,
                      dtype="f32", value_scale=1.0, pool=8),
    "qwen3_decode": dict(id=2, kind="decode", B=256, ctx=(100, 2048), Hq=16, Hkv=8, D=128,
                         dtype="bf16", value_scale=0.5, pool=None),
    "prefill_prefix": dict(id=3, kind="prefill", B=32, ctx=(100, 1024), Hq=16, Hkv=8, D=128,
                           dtype="bf16", value_scale=1.0, pool=None, group=8, shared=512, chunk=4096),
    "long_decode": dict(id=4, kind="decode", B=64, ctx=(4096, 8192), Hq=32, Hkv=8, D=128,
                        dtype="bf16", value_scale=1.0, pool=None),
    "int8_decode": dict(id=5, kind="decode", B=128, ctx=(512, 8192), Hq=32, Hkv=32, D=128,
                        dtype="i8", value_scale=1.0, pool=None),
    # prompts longer than one step's token budget, computed over several chunks
    "prefill_long": dict(id=7, kind="prefill", B=4, ctx=(4096, 12288), Hq=16, Hkv=8, D=128,
                         dtype="bf16", value_scale=1.0, pool=None, group=2, shared=2048, chunk=4096,
                         split=True),
    # beam search over decode prompts: B requests x `beams` beams that re-fork every step
    "beam_decode": dict(id=8, kind="beam", B=64, beams=4, ctx=(100, 2048), Hq=16, Hkv=8, D=128,
                        dtype="bf16", value_scale=0.5, pool=None),
    # the same beam search over long prompts, whose shared blocks no cache holds
    "beam_long": dict(id=9, kind="beam", B=32, beams=4, ctx=(16384, 32768), Hq=16, Hkv=8, D=128,
                      dtype="bf16", value_scale=0.5, pool=None),
    # the prompts of prefill_prefix (same seeds, same draws), stored by the quantising store into
    # int8 caches; dtype is that of the new rows
    "int8_store": dict(id=3, kind="store", B=32, ctx=(100, 1024), Hq=16, Hkv=8, D=128,
                       dtype="bf16", value_scale=1.0, pool=None, group=8, shared=512, chunk=4096),
}

_P_LEN, _P_SEQ, _P_GROUP, _P_POOL, _P_STEP, _P_BEAM = 0, 1, 2, 3, 4, 5


def _rng(seed, cfg, purpose, index=0):
    return np.random.default_rng([int(seed), int(cfg["id"]), purpose, int(index)])


def config(name, **overrides):
    cfg = dict(CONFIGS[name])
    cfg["name"] = name
    cfg.update(overrides)
    return cfg


# -- bf16 encoding (round to nearest even, as torch.bfloat16 does) -----------
def f32_to_bf16_bits(x):
    """Round float32 values to bf16, nearest-even; returns the bf16 bit patterns as uint16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(u16):
    return (np.asarray(u16, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# -- int8 encoding of one sequence's KV (data preparation for int8_decode) ---
def int8_encode(x_f32, length):
    """Per (logical block, KV head) absmax/127 scale over the block's valid tokens.

    x_f32: ``[L][Hkv][D]`` float32 values (already bf16-representable).
    Returns (codes int8 ``[L][Hkv][D]``, scale per token ``[L][Hkv]`` float32,
    scale per logical block ``[nblk][Hkv]`` float32).  Codes are
    clamp(rint(x / scale), -127, 127) with rint rounding half to even, computed
    in float64; an all-zero block has scale 0 and codes 0.
    """
    L, Hkv, D = x_f32.shape
    nblk = -(-L // BLOCK)
    codes = np.zeros((L, Hkv, D), dtype=np.int8)
    tok_scale = np.zeros((L, Hkv), dtype=np.float32)
    blk_scale = np.zeros((nblk, Hkv), dtype=np.float32)
    for i in range(nblk):
        lo, hi = i * BLOCK, min(L, (i + 1) * BLOCK)
        x = x_f32[lo:hi].astype(np.float64)
        amax = np.abs(x).max(axis=(0, 2))  # [Hkv]
        s = (amax / 127.0).astype(np.float32)
        blk_scale[i] = s
        tok_scale[lo:hi] = s[None, :]
        s64 = s.astype(np.float64)
        safe = np.where(s64 > 0, s64, 1.0)
        c = np.rint(x / safe[None, :, None])
        c = np.clip(c, -127, 127)
        c[:, s64 == 0, :] = 0
        codes[lo:hi] = c.astype(np.int8)
    return codes, tok_scale, blk_scale


# -- lengths, pool ------------------------------------------------------------
def lengths(cfg, seed):
    if isinstance(cfg["ctx"], list):
        return list(cfg["ctx"])
    lo, hi = cfg["ctx"]
    return [int(x) for x in _rng(seed, cfg, _P_LEN).integers(lo, hi, size=cfg["B"], endpoint=True)]


def pool_blocks(cfg, lens):
    if cfg.get("pool"):
        return int(cfg["pool"])
    need = sum(-(-L // BLOCK) for L in lens)
    return int(math.ceil(1.1 * need - 1e-9))


def free_order(cfg, seed, num_blocks):
    """Initial order of the free block pool: a seeded random permutation (random physical placement)."""
    return _rng(seed, cfg, _P_POOL).permutation(num_blocks).astype(np.int32)


def _normal(rng, shape, scale, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x = x * np.float32(scale)
    if dtype == "f32":
        return x
    return f32_to_bf16_bits(x)  # bf16 and the int8 source


# -- decode workloads -----------------------------------------------------------
def decode_sequence(cfg, seed, b, L):
    """All data of decode sequence ``b`` with context length ``L`` (the last token is the new one).

    Keys: tokens ``[L]`` int32; k, v ``[L][Hkv][D]`` (float32, or bf16 bits as uint16);
    q ``[Hq][D]``; for int8 also kq, vq (int8), k_tok_scale, v_tok_scale ``[L][Hkv]``,
    k_blk_scale, v_blk_scale ``[nblk][Hkv]``.
    """
    rng = _rng(seed, cfg, _P_SEQ, b)
    Hq, Hkv, D, dt, vs = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["dtype"], cfg["value_scale"]
    out = {"tokens": rng.integers(0, VOCAB, size=L, dtype=np.int32)}
    out["k"] = _normal(rng, (L, Hkv, D), vs, dt)
    out["v"] = _normal(rng, (L, Hkv, D), vs, dt)
    out["q"] = _normal(rng, (Hq, D), vs, dt)
    if dt == "i8":
        out["kq"], out["k_tok_scale"], out["k_blk_scale"] = int8_encode(bf16_bits_to_f32(out["k"]), L)
        out["vq"], out["v_tok_scale"], out["v_blk_scale"] = int8_encode(bf16_bits_to_f32(out["v"]), L)
    return out


def decode_workload(cfg, seed, threads=16):
    """Lengths, pool, free order and per-sequence data of a decode workload."""
    lens = lengths(cfg, seed)
    nb = pool_blocks(cfg, lens)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        seqs = list(ex.map(lambda a: decode_sequence(cfg, seed, a[0], a[1]), enumerate(lens)))
    return dict(cfg=cfg, seed=seed, lens=lens, num_blocks=nb, free_order=free_order(cfg, seed, nb), seqs=seqs)


def decode_step_inputs(cfg, seed, step, B):
    """New-token inputs of decode step ``step`` (after the workload's own step) for all B sequences.

    Returns tokens ``[B]``, q ``[B][Hq][D]``, k, v ``[B][Hkv][D]`` drawn like the workload's values.
    (int8 workloads: k, v are the bf16 source; see :func:`int8_encode_token`.)
    """
    rng = _rng(seed, cfg, _P_STEP, step)
    Hq, Hkv, D, dt, vs = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["dtype"], cfg["value_scale"]
    return dict(tokens=rng.integers(0, VOCAB, size=B, dtype=np.int32), q=_normal(rng, (B, Hq, D), vs, dt),
                k=_normal(rng, (B, Hkv, D), vs, dt), v=_normal(rng, (B, Hkv, D), vs, dt))


def beam_parents(cfg, seed, step):
    """Beam search step ``step``: for each request and each of its new beams, the index of the
    current beam it continues (uniform draws; a beam picked twice is forked twice, one not picked
    ends).  Returns int ``[B][beams]``."""
    return _rng(seed, cfg, _P_BEAM, step).integers(0, cfg["beams"], size=(cfg["B"], cfg["beams"]))


def int8_encode_token(x_f32, block_scale):
    """int8 codes of decode tokens ``[B][Hkv][D]``: a token that opens a new block (block_scale row
    is NaN) sets the block's scale from its own absmax; otherwise it reuses the block's scale and
    its codes are clamped to +-127.  Returns (codes, scale ``[B][Hkv]``)."""
    x = x_f32.astype(np.float64)
    own = (np.abs(x).max(axis=2) / 127.0).astype(np.float32)
    s = np.where(np.isnan(block_scale), own, block_scale).astype(np.float32)
    s64 = s.astype(np.float64)
    safe = np.where(s64 > 0, s64, 1.0)
    c = np.clip(np.rint(x / safe[:, :, None]), -127, 127)
    c[s64 == 0] = 0
    return c.astype(np.int8), s


# -- prefill workload -------------------------------------------------------------
def prefill_prompt(cfg, seed, i, n):
    """Prompt ``i`` of length ``n``: positions < shared come from its group's stream."""
    Hq, Hkv, D, dt, vs = cfg["Hq"], cfg["Hkv"], cfg["D"], cfg["dtype"], cfg["value_scale"]
    shared = cfg["shared"]
    g = _rng(seed, cfg, _P_GROUP, i // cfg["group"])
    gt = g.integers(0, VOCAB, size=shared, dtype=np.int32)
    gk = _normal(g, (shared, Hkv, D), vs, dt)
    gv = _normal(g, (shared, Hkv, D), vs, dt)
    gq = _normal(g, (shared, Hq, D), vs, dt)
    own = max(0, n - shared)
    r = _rng(seed, cfg, _P_SEQ, i)
    ot = r.integers(0, VOCAB, size=own, dtype=np.int32)
    ok = _normal(r, (own, Hkv, D), vs, dt)
    ov = _normal(r, (own, Hkv, D), vs, dt)
    oq = _normal(r, (own, Hq, D), vs, dt)
    m = min(n, shared)
    return dict(tokens=np.concatenate([gt[:m], ot]), k=np.concatenate([gk[:m], ok]),
                v=np.concatenate([gv[:m], ov]), q=np.concatenate([gq[:m], oq]))


def prefill_workload(cfg, seed):
    lens = lengths(cfg, seed)
    prompts = [prefill_prompt(cfg, seed, i, n) for i, n in enumerate(lens)]
    nb = pool_blocks(cfg, lens)
    return dict(cfg=cfg, seed=seed, lens=lens, num_blocks=nb, free_order=free_order(cfg, seed, nb),
                prompts=prompts)


def pack_chunks_split(n_new, budget):
    """Prompts in order, each chunk filled to ``budget`` new tokens: a prompt that does not fit is
    split, its first part ending the chunk and the rest continuing in the next.  Returns chunks as
    lists of (prompt, start, end) segments of the prompts' new tokens."""
    chunks, cur, room = [], [], budget
    for i, n in enumerate(n_new):
        a = 0
        while a < n:
            b = min(n, a + room)
            cur.append((i, a, b))
            room -= b - a
            a = b
            if room == 0:
                chunks.append(cur)
                cur, room = [], budget
    if cur:
        chunks.append(cur)
    return chunks


def pack_chunks(n_new, budget):
    """Whole prompts, in order, greedily packed so that each chunk's new tokens total at most ``budget``."""
    chunks, cur, tot = [], [], 0
    for i, n in enumerate(n_new):
        if n > budget:
            raise ValueError(f"prompt {i} has {n} new tokens, more than one chunk ({budget})")
        if cur and tot + n > budget:
            chunks.append(cur)
            cur, tot = [], 0
        cur.append(i)
        tot += n
    if cur:
        chunks.append(cur)
    return chunks
