"""Plain reference for the host block pool with hash-chained prefix reuse.

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline may use this module; the product path never does.

What is modelled: the block manager of a paged KV cache ("rvLLM:
High-performance LLM inference in Rust", architecture diagram: "Block Manager
(paged KV)") with prefix caching as "Litellama" describes it (section
"Features", Prefix Caching): every full 16-token block is identified by a
hash chained from the previous block's hash and its own tokens, so a request
whose leading blocks match an earlier one's reuses those physical blocks, and
blocks no sequence uses any more stay cached until capacity pressure evicts
the least recently released one.

The steps, in the order the pool takes them (the page gives the idea in one
sentence; these are the readings taken, each listed in the design notes):
  * hash(block i) = FNV-1a-64 over the 8 little-endian bytes of the parent
    hash (the seed for block 0) followed by the 16 token ids as 4-byte
    little-endian integers;
  * add_sequence: the longest run of leading full blocks found in the cache
    (same hash, same parent and same tokens) is reused; the remaining full
    blocks and a trailing partial block take blocks from the free queue, and
    the new full blocks are registered in the cache. The call fails without
    changing anything when the free queue cannot supply what it needs;
  * the free queue holds the blocks no sequence uses, least recently
    released first; taking a block from it evicts the cache entry it carries;
  * append_token: a token that starts a new block takes one from the free
    queue; a token that completes a block registers that block's hash (unless
    the cache already holds another block with that hash);
  * free_sequence releases the sequence's blocks last block first, so a
    sequence's tail is evicted before its head;
  * initially every block is free, in id order.
"""
import struct
from collections import OrderedDict

BLOCK = 16
FNV_OFFSET = 0xCBF29CE484222325
FNV_PRIME = 0x100000001B3
MASK = (1 << 64) - 1


def fnv1a64(data, h=FNV_OFFSET):
    for byte in data:
        h ^= byte
        h = (h * FNV_PRIME) & MASK
    return h


def chain_hash(parent, tokens):
    data = struct.pack("<Q", parent) + b"".join(struct.pack("<i", int(t)) for t in tokens)
    return fnv1a64(data)


class PoolError(Exception):
    pass


class BlockPoolRef:
    def __init__(self, num_blocks, seed):
        self.n = num_blocks
        self.seed = seed
        self.ref = [0] * num_blocks
        self.key = [None] * num_blocks          # (hash, parent, tokens) of a registered full block
        self.free = OrderedDict((b, None) for b in range(num_blocks))
        self.cached = {}                        # hash -> block
        self.seqs = {}                          # id -> dict(tokens, blocks, parent)

    # -- the free queue
    def _take_free(self):
        blk, _ = self.free.popitem(last=False)
        k = self.key[blk]
        if k is not None:                       # evict its cache entry
            if self.cached.get(k[0]) == blk:
                del self.cached[k[0]]
            self.key[blk] = None
        return blk

    def _lookup(self, h, parent, tokens):
        blk = self.cached.get(h)
        if blk is None:
            return None
        k = self.key[blk]
        return blk if k == (h, parent, tuple(tokens)) else None

    def _register(self, blk, h, parent, tokens):
        self.key[blk] = (h, parent, tuple(tokens))
        if h not in self.cached:
            self.cached[h] = blk

    # -- operations
    def add_sequence(self, sid, tokens):
        """Returns the number of leading tokens found in the cache."""
        if sid in self.seqs:
            raise PoolError("sequence exists")
        tokens = [int(t) for t in tokens]
        nfull = len(tokens) // BLOCK
        parent, hits = self.seed, []
        hashes = []
        for i in range(nfull):
            blk_tokens = tokens[BLOCK * i: BLOCK * (i + 1)]
            h = chain_hash(parent, blk_tokens)
            hashes.append((h, parent, blk_tokens))
            if len(hits) == i:
                blk = self._lookup(h, parent, blk_tokens)
                if blk is not None:
                    hits.append(blk)
            parent = h
        need = (nfull - len(hits)) + (1 if len(tokens) % BLOCK else 0)
        need += sum(1 for b in hits if self.ref[b] == 0)
        if need > len(self.free):
            raise PoolError("out of blocks")
        blocks = []
        for b in hits:
            if self.ref[b] == 0:
                del self.free[b]
            self.ref[b] += 1
            blocks.append(b)
        for i in range(len(hits), nfull):
            b = self._take_free()
            self.ref[b] = 1
            self._register(b, *hashes[i])
            blocks.append(b)
        if len(tokens) % BLOCK:
            b = self._take_free()
            self.ref[b] = 1
            blocks.append(b)
        self.seqs[sid] = {"tokens": tokens, "blocks": blocks,
                          "parent": hashes[-1][0] if nfull else self.seed}
        return BLOCK * len(hits)

    def append_token(self, sid, token):
        s = self.seqs.get(sid)
        if s is None:
            raise PoolError("no such sequence")
        if len(s["tokens"]) % BLOCK == 0:
            if not self.free:
                raise PoolError("out of blocks")
            b = self._take_free()
            self.ref[b] = 1
            s["blocks"].append(b)
        s["tokens"].append(int(token))
        if len(s["tokens"]) % BLOCK == 0:
            blk_tokens = s["tokens"][-BLOCK:]
            h = chain_hash(s["parent"], blk_tokens)
            self._register(s["blocks"][-1], h, s["parent"], blk_tokens)
            s["parent"] = h

    def free_sequence(self, sid):
        s = self.seqs.pop(sid, None)
        if s is None:
            raise PoolError("no such sequence")
        for b in reversed(s["blocks"]):
            self.ref[b] -= 1
            if self.ref[b] == 0:
                self.free[b] = None

    def num_free(self):
        return len(self.free)

    def block_table(self, sids, max_blocks, pad):
        rows, lens = [], []
        for sid in sids:
            s = self.seqs.get(sid)
            if s is None or len(s["blocks"]) > max_blocks:
                raise PoolError("no such sequence or table too narrow")
            rows.append(s["blocks"] + [pad] * (max_blocks - len(s["blocks"])))
            lens.append(len(s["tokens"]))
        return rows, lens


__all__ = ["BLOCK", "BlockPoolRef", "PoolError", "chain_hash", "fnv1a64"]
