"""Host-side block manager of a paged KV cache, as a plain Python model.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it does, and where it is stated:

* The cache is a pool of fixed 16-token blocks; a sequence owns a list of
  physical blocks (its block table) that grows on demand: a new block is
  taken only when the last one is full, so at most one block per sequence is
  partly empty ([d7kj] section 三; [qingdujian] section 二 appends at the next
  offset of the last block and opens a block when it is full; [freetools]
  section on PagedAttention).
* When a request ends its blocks are released at once for other requests
  ([freetools] section on PagedAttention).
* Several sequences may share physical blocks: branches of one request (beam
  search) and requests with the same prefix ([d7kj] section 三; [k1-blog]
  section on PagedAttention and vLLM).  A block is shared by reference
  count; a shared block that must still receive tokens is copied first
  (copy-on-write), so a sequence never writes into a block another sequence
  reads.
* Prefix caching ([d7kj] section 五): full blocks are found again by a hash
  of their content; the hash of a block covers every token before it as
  well, so one different token early in a prompt changes every later block's
  hash and nothing after it is reused ([d7kj] section 七).

Readings where the pages are silent (the C++ manager follows the same):

* Free blocks form a first-in first-out queue, initially 0 .. N-1; a block
  whose last reference goes away returns to its back.
* With prefix caching, a full block whose content is registered is not
  freed when its last reference goes: it stays cached (its K/V remain valid)
  in a least-recently-released list, and is evicted (its hash forgotten) only
  when a block is needed and the free queue is empty.  A sequence releases its
  blocks from its last block to its first, so the oldest prefix blocks are
  evicted last.
* A block's content is registered (hash -> block) when it becomes full, if
  no other block is registered under that content.  Matches compare the
  tokens themselves, so a hash collision can never share wrong data.
* A new sequence shares cached blocks only for full blocks lying entirely
  in its first n - 1 tokens: the block holding its last prompt token is
  always private (that token's query is computed, and its K/V written).
* Running out of blocks is an error that leaves the manager unchanged.
"""

from typing import Dict, List, Tuple

BLOCK = 16
_FNV_OFFSET = 0xCBF29CE484222325
_FNV_PRIME = 0x100000001B3
_MASK = (1 << 64) - 1


def block_hash(parent: int, tokens) -> int:
    """FNV-1a (64-bit) over the parent block's hash and the block's 16 token
    ids, each as 8 / 4 little-endian bytes."""
    h = _FNV_OFFSET
    data = parent.to_bytes(8, "little") + b"".join(
        (int(t) & 0xFFFFFFFF).to_bytes(4, "little") for t in tokens)
    for byte in data:
        h = ((h ^ byte) * _FNV_PRIME) & _MASK
    return h


class OutOfBlocks(RuntimeError):
    pass


class BlockManager:
    def __init__(self, num_blocks: int, prefix_caching: bool):
        self.n = num_blocks
        self.caching = prefix_caching
        self.free: List[int] = list(range(num_blocks))
        self.ref = [0] * num_blocks
        self.cached_lru: List[int] = []              # unreferenced cached blocks, oldest first
        self.by_hash: Dict[int, List[Tuple[Tuple[int, ...], int]]] = {}  # hash -> [(tokens, block)]
        self.block_key: Dict[int, Tuple[int, Tuple[int, ...]]] = {}  # block -> (hash, tokens)
        self.tables: Dict[int, List[int]] = {}
        self.tokens: Dict[int, List[int]] = {}

    # -- helpers
    def _lookup(self, h, toks):
        for t, b in self.by_hash.get(h, []):
            if t == toks:
                return b
        return None

    def _available(self) -> int:
        return len(self.free) + len(self.cached_lru)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop(0)
        elif self.cached_lru:
            b = self.cached_lru.pop(0)
            h, toks = self.block_key.pop(b)
            self.by_hash[h] = [(t, x) for t, x in self.by_hash[h] if x != b]
            if not self.by_hash[h]:
                del self.by_hash[h]
        else:
            raise OutOfBlocks("no free block")
        self.ref[b] = 1
        return b

    def _release(self, b: int) -> None:
        self.ref[b] -= 1
        if self.ref[b] == 0:
            (self.cached_lru if b in self.block_key else self.free).append(b)

    def _chain(self, toks: List[int], nblocks: int) -> List[int]:
        hs, h = [], 0
        for j in range(nblocks):
            h = block_hash(h, toks[BLOCK * j: BLOCK * (j + 1)])
            hs.append(h)
        return hs

    def _register_full(self, seq: int, j: int) -> None:
        toks = self.tokens[seq]
        blk = self.tables[seq][j]
        if not self.caching or blk in self.block_key:
            return
        key = tuple(toks[BLOCK * j: BLOCK * (j + 1)])
        h = self._chain(toks, j + 1)[j]
        if self._lookup(h, key) is None:
            self.by_hash.setdefault(h, []).append((key, blk))
            self.block_key[blk] = (h, key)

    # -- operations
    def add(self, seq: int, prompt) -> int:
        """New sequence with its prompt tokens; returns how many leading
        tokens already have their K/V in shared cached blocks."""
        if seq in self.tables:
            raise KeyError(f"sequence {seq} exists")
        prompt = [int(t) for t in prompt]
        n = len(prompt)
        need = -(-n // BLOCK)
        matched = []
        if self.caching and n > 0:
            hs = self._chain(prompt, (n - 1) // BLOCK)
            for j, h in enumerate(hs):
                b = self._lookup(h, tuple(prompt[BLOCK * j: BLOCK * (j + 1)]))
                if b is None:
                    break
                matched.append(b)
        revived = sum(1 for b in matched if self.ref[b] == 0)
        if need - len(matched) > self._available() - revived:
            raise OutOfBlocks("not enough blocks for the prompt")
        for b in matched:
            if self.ref[b] == 0:
                self.cached_lru.remove(b)
            self.ref[b] += 1
        table = list(matched)
        for _ in range(need - len(matched)):
            table.append(self._take())
        self.tables[seq] = table
        self.tokens[seq] = prompt
        for j in range(len(matched), n // BLOCK):
            self._register_full(seq, j)
        return BLOCK * len(matched)

    def append(self, seq: int, token: int) -> List[Tuple[int, int]]:
        """Reserve the slot of one more token; returns the block copies
        (src, dst) to perform before writing it (copy-on-write)."""
        table, toks = self.tables[seq], self.tokens[seq]
        t = len(toks)
        copies = []
        if t % BLOCK == 0:
            if self._available() < 1:
                raise OutOfBlocks("no block for the new token")
            table.append(self._take())
        else:
            last = table[-1]
            if self.ref[last] > 1:
                if self._available() < 1:
                    raise OutOfBlocks("no block for the copy")
                new = self._take()
                self._release(last)
                table[-1] = new
                copies.append((last, new))
        toks.append(int(token))
        if (t + 1) % BLOCK == 0:
            self._register_full(seq, t // BLOCK)
        return copies

    def fork(self, parent: int, child: int) -> None:
        if child in self.tables:
            raise KeyError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.tokens[child] = list(self.tokens[parent])
        for b in self.tables[child]:
            self.ref[b] += 1

    def free_seq(self, seq: int) -> None:
        table = self.tables.pop(seq)
        del self.tokens[seq]
        for b in reversed(table):
            self._release(b)

    def table(self, seqs, max_blocks: int):
        rows, lens = [], []
        for s in seqs:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            rows.append(t + [-1] * (max_blocks - len(t)))
            lens.append(len(self.tokens[s]))
        return rows, lens

    def stats(self) -> Tuple[int, int]:
        return len(self.free), len(self.cached_lru)
