"""Oracle block manager (pure Python).  TEST INFRASTRUCTURE ONLY.

The pages describe the pieces but print no complete algorithm:

* a pool of fixed-size blocks (256 tokens), a sequence of length n takes
  ceil(n / 256) of them, handed out first-in first-out from a free deque
  (intelliparadigm.com Nano-vLLM article, §2.1 动态分块内存管理; block size 256 and
  "a multiple of 256" in "Nano-vLLM性能调优实战", §1.1 KV缓存块配置);
* reclamation by plain reference counts ("1200行代码挑战vLLM", §2 内存管理策略);
* prefix reuse: a prompt hash maps to stored KV ("1200行代码挑战vLLM",
  §性能优化 1. 前缀缓存), which at block granularity lets sequences share the
  physical blocks of a common prefix (ocdem.com nano-vllm article, §2.1);
* lazy release (intelliparadigm.com article, §7.2 关键优化点 -- 延迟释放策略).

Readings taken where the pages are silent (each is a choice, written down so
that a second implementation can match it bit for bit):

1. The free deque starts in a caller-given order (the seeded permutation is an
   input, not drawn here).  Refcounts start at 0, the hash table is empty.
2. add_seq: block i of the prompt is *full* when (i+1)*256 <= n.  A full block
   gets the chained hash h_i = FNV-1a-64(le64(h_{i-1}) || le32(tokens of block
   i)), h_{-1} = 0.  Block i is a *hit* when prefix caching is on, every earlier
   block was a hit, h_i is in the table, the table's block stores exactly these
   256 tokens, and (i+1)*256 < n (the block holding the last prompt token is
   never reused, so at least one token is always computed).  A hit takes a
   reference (removing the block from the free deque if its count was 0).  A
   miss pops the head of the free deque, drops that block's old table entry if
   the table still points at it, forgets its old hash, and -- if block i is
   full -- records h_i, the tokens, and table[h_i] = block (last writer wins).
   If the misses do not fit in the free deque the call fails and nothing
   changes.
3. append: position pos = len; a new block is popped (as a miss, no hash) when
   pos % 256 == 0; slot = table[pos // 256] * 256 + pos % 256; when the block
   becomes full it is hashed (chained on the sequence's previous full block)
   and registered.
4. free_seq: walk the sequence's blocks in reverse, decrement, and append a
   block to the free deque when its count reaches 0; it keeps its hash and
   tokens until it is popped again (lazy release).
5. With prefix caching off nothing is hashed or registered.
"""

from collections import deque

BLOCK = 256
_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK64 = (1 << 64) - 1


class AllocError(Exception):
    """Raised with ``kind`` one of NO_BLOCKS, UNKNOWN_SEQ, DUP_SEQ, SMALL_BUFFER, INVALID."""

    def __init__(self, kind, msg=""):
        super().__init__(f"{kind}: {msg}")
        self.kind = kind


def fnv1a64(data):
    """FNV-1a, 64-bit: for each byte, xor it in, then multiply by the FNV prime."""
    h = _FNV_OFFSET
    for byte in data:
        h ^= byte
        h = (h * _FNV_PRIME) & _MASK64
    return h


def block_hash(prev_hash, tokens):
    """Chained hash of one full block: FNV-1a-64 over le64(prev) followed by le32 of each token."""
    data = bytearray(int(prev_hash).to_bytes(8, "little"))
    for t in tokens:
        data += int(t).to_bytes(4, "little", signed=True)
    return fnv1a64(bytes(data))


class _Seq:
    __slots__ = ("blocks", "tokens", "n_cached", "last_hash")

    def __init__(self):
        self.blocks = []
        self.tokens = []
        self.n_cached = 0
        self.last_hash = 0


class Allocator:
    def __init__(self, num_blocks, initial_order, prefix_cache=True, block_size=BLOCK, hash_fn=None):
        if block_size != BLOCK:
            raise AllocError("INVALID", "block size must be 256")
        order = [int(b) for b in initial_order]
        if sorted(order) != list(range(num_blocks)):
            raise AllocError("INVALID", "initial order must be a permutation of the pool")
        self.num_blocks = num_blocks
        self.prefix_cache = bool(prefix_cache)
        self.free = deque(order)
        self.ref = [0] * num_blocks
        self.bhash = [None] * num_blocks
        self.btokens = [None] * num_blocks
        self.table = {}
        self.seqs = {}
        # test hook: a replacement for block_hash(prev, tokens), e.g. a constant to force collisions
        self._hash = hash_fn if hash_fn is not None else block_hash

    # -- helpers ---------------------------------------------------------
    def _pop_fresh(self):
        b = self.free.popleft()
        old = self.bhash[b]
        if old is not None and self.table.get(old) == b:
            del self.table[old]
        self.bhash[b] = None
        self.btokens[b] = None
        self.ref[b] = 1
        return b

    def _register(self, b, h, chunk):
        self.bhash[b] = h
        self.btokens[b] = tuple(chunk)
        self.table[h] = b

    # -- API ---------------------------------------------------------------
    def add_seq(self, seq_id, tokens):
        """Admit a prompt; returns the number of leading tokens whose KV is already cached."""
        if seq_id in self.seqs:
            raise AllocError("DUP_SEQ", str(seq_id))
        tokens = [int(t) for t in tokens]
        n = len(tokens)
        nb = -(-n // BLOCK)
        plan = []
        prev = 0
        hit_ok = self.prefix_cache
        for i in range(nb):
            chunk = tokens[i * BLOCK:(i + 1) * BLOCK]
            full = (i + 1) * BLOCK <= n
            h = self._hash(prev, chunk) if (full and self.prefix_cache) else None
            hit = None
            if hit_ok and h is not None and (i + 1) * BLOCK < n and h in self.table:
                cand = self.table[h]
                if self.btokens[cand] == tuple(chunk):
                    hit = cand
            if hit is None:
                hit_ok = False
            plan.append((hit, h, chunk))
            prev = h if h is not None else 0
        n_miss = sum(1 for hit, _, _ in plan if hit is None)
        freed_hits = {hit for hit, _, _ in plan if hit is not None and self.ref[hit] == 0}
        if n_miss > len(self.free) - len(freed_hits):
            raise AllocError("NO_BLOCKS", f"need {n_miss} fresh blocks")
        s = _Seq()
        for hit, h, chunk in plan:
            if hit is not None:
                if self.ref[hit] == 0:
                    self.free.remove(hit)
                self.ref[hit] += 1
                s.blocks.append(hit)
                s.n_cached += BLOCK
            else:
                b = self._pop_fresh()
                if h is not None:
                    self._register(b, h, chunk)
                s.blocks.append(b)
            if h is not None:
                s.last_hash = h
        s.tokens = tokens
        self.seqs[seq_id] = s
        return s.n_cached

    def fork(self, parent_id, child_id):
        """Parallel sampling / beam search (ocdem.com nano-vllm article, §2.1: sequences of one
        request share physical blocks): the child takes the parent's tokens and every one of its
        blocks, each block's reference count growing by one.  A partially filled last block stays
        shared until one of its owners appends (:meth:`append_cow`)."""
        if child_id in self.seqs:
            raise AllocError("DUP_SEQ", str(child_id))
        p = self.seqs.get(parent_id)
        if p is None:
            raise AllocError("UNKNOWN_SEQ", str(parent_id))
        c = _Seq()
        c.blocks = list(p.blocks)
        c.tokens = list(p.tokens)
        c.n_cached = len(p.tokens)
        c.last_hash = p.last_hash
        for b in c.blocks:
            self.ref[b] += 1
        self.seqs[child_id] = c

    def append_cow(self, seq_id, token):
        """:meth:`append` with copy-on-write: when the token lands in a partially filled block that
        other sequences still hold, the sequence first moves to a fresh block, into which the caller
        copies the shared block's contents.  Returns (slot, src, dst), src = dst = -1 without a copy."""
        s = self.seqs.get(seq_id)
        if s is None:
            raise AllocError("UNKNOWN_SEQ", str(seq_id))
        pos = len(s.tokens)
        src = dst = -1
        if pos % BLOCK != 0 and self.ref[s.blocks[pos // BLOCK]] > 1:
            if not self.free:
                raise AllocError("NO_BLOCKS", "copy-on-write")
            src = s.blocks[pos // BLOCK]
            dst = self._pop_fresh()
            self.ref[src] -= 1
            s.blocks[pos // BLOCK] = dst
        return self.append(seq_id, token), src, dst

    def append(self, seq_id, token):
        """Add one decoded token; returns its cache slot.  A partially filled block shared with a
        fork must go through :meth:`append_cow`."""
        s = self.seqs.get(seq_id)
        if s is None:
            raise AllocError("UNKNOWN_SEQ", str(seq_id))
        pos = len(s.tokens)
        if pos % BLOCK != 0 and self.ref[s.blocks[pos // BLOCK]] > 1:
            raise AllocError("INVALID", "the block is shared with a fork: append with copy-on-write")
        if pos % BLOCK == 0:
            if not self.free:
                raise AllocError("NO_BLOCKS", "append")
            s.blocks.append(self._pop_fresh())
        s.tokens.append(int(token))
        slot = s.blocks[pos // BLOCK] * BLOCK + pos % BLOCK
        if self.prefix_cache and len(s.tokens) % BLOCK == 0:
            i = len(s.tokens) // BLOCK - 1
            chunk = s.tokens[i * BLOCK:(i + 1) * BLOCK]
            h = self._hash(s.last_hash, chunk)
            self._register(s.blocks[i], h, chunk)
            s.last_hash = h
        return slot

    def free_seq(self, seq_id):
        s = self.seqs.pop(seq_id, None)
        if s is None:
            raise AllocError("UNKNOWN_SEQ", str(seq_id))
        for b in reversed(s.blocks):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    def num_free(self):
        return len(self.free)

    def seq_len(self, seq_id):
        return len(self.seqs[seq_id].tokens)

    def block_tables(self, seq_ids, max_blocks):
        rows = []
        for sid in seq_ids:
            s = self.seqs.get(sid)
            if s is None:
                raise AllocError("UNKNOWN_SEQ", str(sid))
            if len(s.blocks) > max_blocks:
                raise AllocError("SMALL_BUFFER", f"{len(s.blocks)} blocks > {max_blocks}")
            rows.append(list(s.blocks) + [-1] * (max_blocks - len(s.blocks)))
        return rows

    def prefill_slots(self, seq_ids):
        """cu_seqlens_q, seqlens_k and slots of the tokens not yet in the cache (positions n_cached..len-1)."""
        cu = [0]
        lens_k = []
        slots = []
        for sid in seq_ids:
            s = self.seqs.get(sid)
            if s is None:
                raise AllocError("UNKNOWN_SEQ", str(sid))
            n = len(s.tokens)
            for pos in range(s.n_cached, n):
                slots.append(s.blocks[pos // BLOCK] * BLOCK + pos % BLOCK)
            cu.append(cu[-1] + n - s.n_cached)
            lens_k.append(n)
        return cu, lens_k, slots

    def prefill_segment_slots(self, seq_ids, starts, ends):
        """Segments [start, end) of each sequence's new tokens, computed over several steps when a
        prompt exceeds one step's token budget ("Nano-vLLM性能调优实战", §3.2 关键调度参数): the
        segment's queries see the cached prefix, the earlier segments and themselves, so its key
        count is n_cached + end."""
        cu = [0]
        lens_k = []
        slots = []
        for sid, a, b in zip(seq_ids, starts, ends):
            s = self.seqs.get(sid)
            if s is None:
                raise AllocError("UNKNOWN_SEQ", str(sid))
            if not 0 <= a <= b <= len(s.tokens) - s.n_cached:
                raise AllocError("INVALID", f"segment [{a}, {b})")
            for pos in range(s.n_cached + a, s.n_cached + b):
                slots.append(s.blocks[pos // BLOCK] * BLOCK + pos % BLOCK)
            cu.append(cu[-1] + b - a)
            lens_k.append(s.n_cached + b)
        return cu, lens_k, slots

    # -- introspection for invariant tests --------------------------------
    def check_invariants(self):
        owners = [0] * self.num_blocks
        for s in self.seqs.values():
            for b in s.blocks:
                owners[b] += 1
        assert owners == self.ref, "refcount != number of owning sequences"
        assert len(set(self.free)) == len(self.free), "block twice in the free deque"
        assert all(self.ref[b] == 0 for b in self.free), "free block with references"
        in_use = sum(1 for r in self.ref if r > 0)
        assert len(self.free) + in_use == self.num_blocks, "blocks lost or duplicated"
        for h, b in self.table.items():
            assert self.bhash[b] == h, "table entry does not match its block's hash"
