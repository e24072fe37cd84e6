"""Reference model of the physical block pool that feeds the kernels their
block tables and slot mappings.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/`` may import this module.
It is plain Python over lists and dicts, written to be read against the pages;
the product's allocator is C++ behind the C ABI and shares nothing with it.

What the pages fix:
- The cache is cut into uniform blocks of a fixed number of tokens; one global
  pool of such physical blocks serves every request.  A request takes free
  blocks as it needs more room and gives them back when it ends; the request's
  block table maps its logical blocks to physical ones, which need not be
  contiguous ("Nano-vLLM engine deep-dive", section 2.2; "LLM basics primer"
  part 4, section 17.7).
- Requests with a common prefix (a shared system prompt) may point at the same
  physical blocks, so the prefix is held once; writes to a shared block go
  through copy-on-write; prefix caching is named as a benefit of paging
  (deep-dive section 2.2; primer part 4, sections 17.6 and 17.7).
- One block id covers every layer's pool ("Nano-vLLM Part 2", section 05.2).

Where the pages stop, this model takes these readings:
- A block is shared by reference counting: ref[b] is the number of live
  sequences whose table holds b; b is free when ref[b] is 0.
- The free list is first-in first-out: allocation takes the block freed
  longest ago (initially 0, 1, 2, ...); a finished sequence returns its blocks
  last block first.
- Prefix caching covers full blocks only.  A full block is identified by its
  tokens and by the identity of the block before it (its physical id and how
  many times that id has been handed out), so a hit means the whole prefix up
  to the end of the block is the same.  A freed block keeps its identity until
  it is handed out again, so a later request can still hit it.
- A prompt never hits its final token: at most (n - 1) // block_size blocks of
  an n-token prompt come from the cache, so at least one token is computed.
- Copy-on-write happens when a sequence appends into a partly filled block that
  another sequence also holds (after fork): the appender gets a fresh block and
  the pair (old, new) is reported for the caller to copy before storing.
"""
from __future__ import annotations


class PoolError(Exception):
    """An operation the pool refuses (no state changes)."""


class CapacityError(PoolError):
    """Not enough free blocks (no state changes)."""


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int = 16, prefix_caching: bool = False):
        if num_blocks <= 0 or block_size <= 0:
            raise PoolError("num_blocks and block_size must be positive")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.prefix_caching = prefix_caching
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks          # times each id has been handed out
        self.free = list(range(num_blocks))  # FIFO: index 0 is taken next
        self.cache = {}                      # identity -> block id (full blocks)
        self.identity = [None] * num_blocks  # block id -> identity it is cached under
        self.seqs = {}                       # seq id -> {"blocks": [...], "tokens": [...]}

    # -- helpers --------------------------------------------------------------
    def _key(self, prev_block, block_tokens):
        if prev_block is None:
            return (-1, 0, tuple(block_tokens))
        return (prev_block, self.gen[prev_block], tuple(block_tokens))

    def _take_free(self):
        b = self.free.pop(0)
        if self.identity[b] is not None:     # its old content is overwritten: forget it
            del self.cache[self.identity[b]]
            self.identity[b] = None
        self.gen[b] += 1
        self.ref[b] = 1
        return b

    def _register(self, seq, index):
        """Cache block `index` of `seq` (now full) under its identity, unless
        an equal block is already cached."""
        if not self.prefix_caching:
            return
        bs = self.block_size
        blocks = seq["blocks"]
        prev = blocks[index - 1] if index > 0 else None
        key = self._key(prev, seq["tokens"][index * bs:(index + 1) * bs])
        b = blocks[index]
        if key not in self.cache and self.identity[b] is None:
            self.cache[key] = b
            self.identity[b] = key

    # -- operations -------------------------------------------------------------
    def add_seq(self, seq_id, tokens):
        """Admit a prompt.  Returns (slots, num_cached): the cache slot of each
        prompt token (-1 for tokens whose block came from the prefix cache, so
        a store skips them) and how many leading tokens are already cached."""
        if seq_id in self.seqs:
            raise PoolError(f"sequence {seq_id} exists")
        n = len(tokens)
        bs = self.block_size
        if n <= 0:
            raise PoolError("a prompt has at least one token")
        # look the leading full blocks up first, without changing anything
        hits = []
        if self.prefix_caching:
            prev = None
            for i in range((n - 1) // bs):
                b = self.cache.get(self._key(prev, tokens[i * bs:(i + 1) * bs]))
                if b is None:
                    break
                hits.append(b)
                prev = b
        need = -(-n // bs) - len(hits)
        revived = sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free) - revived:
            raise CapacityError(f"{need} blocks needed, {len(self.free) - revived} free")
        blocks = []
        for b in hits:
            if self.ref[b] == 0:
                self.free.remove(b)
            self.ref[b] += 1
            blocks.append(b)
        for _ in range(need):
            blocks.append(self._take_free())
        seq = {"blocks": blocks, "tokens": list(tokens)}
        self.seqs[seq_id] = seq
        for i in range(len(hits), n // bs):
            self._register(seq, i)
        num_cached = len(hits) * bs
        slots = [-1 if t < num_cached else blocks[t // bs] * bs + t % bs for t in range(n)]
        return slots, num_cached

    def append(self, seq_id, token):
        """One decode token.  Returns (slot, copy): copy is (src, dst) when the
        append forced a copy-on-write of the partly filled last block, else
        None."""
        seq = self._seq(seq_id)
        bs = self.block_size
        blocks = seq["blocks"]
        p = len(seq["tokens"])
        copy = None
        if p % bs == 0:
            if not self.free:
                raise CapacityError("no free block")
            blocks.append(self._take_free())
        elif self.ref[blocks[-1]] > 1:
            if not self.free:
                raise CapacityError("no free block for copy-on-write")
            old = blocks[-1]
            new = self._take_free()
            self.ref[old] -= 1
            blocks[-1] = new
            copy = (old, new)
        seq["tokens"].append(token)
        if (p + 1) % bs == 0:
            self._register(seq, p // bs)
        return blocks[p // bs] * bs + p % bs, copy

    def fork(self, parent_id, child_id):
        """The child shares every block of the parent (parallel sampling)."""
        parent = self._seq(parent_id)
        if child_id in self.seqs:
            raise PoolError(f"sequence {child_id} exists")
        for b in parent["blocks"]:
            self.ref[b] += 1
        self.seqs[child_id] = {"blocks": list(parent["blocks"]), "tokens": list(parent["tokens"])}

    def free_seq(self, seq_id):
        seq = self.seqs.pop(seq_id, None)
        if seq is None:
            raise PoolError(f"unknown sequence {seq_id}")
        for b in reversed(seq["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free.append(b)

    # -- queries ----------------------------------------------------------------
    def _seq(self, seq_id):
        if seq_id not in self.seqs:
            raise PoolError(f"unknown sequence {seq_id}")
        return self.seqs[seq_id]

    def block_table(self, seq_id):
        return list(self._seq(seq_id)["blocks"])

    def seq_len(self, seq_id):
        return len(self._seq(seq_id)["tokens"])

    def num_free(self):
        return len(self.free)

    def refcount(self, b):
        return self.ref[b]
