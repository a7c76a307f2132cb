"""Plain Python model of the host block manager (TEST INFRASTRUCTURE ONLY).

Written from the pages, with the policies the library documents in include/pa.h, as
slowly and directly as possible: the tests run the same operations on this model and on
the C++ manager and compare every result.

  [P3] "内存优化：KV Cache管理、PagedAttention原理与内存池配置": blocks of a global pool are
       allocated on demand and appended as a request grows, returned when it ends; shared
       by reference counting; free blocks kept in a list (O(1) allocation and release);
       prefix caching indexes prefix blocks by hash and reuses them only for an exactly
       identical prefix.
  [P1] "突破GPU内存瓶颈：vLLM与PagedAttention技术深度解析" §2 (block tables, shared blocks)
       and §5 (beam search candidates share blocks).

Policies: free blocks are a stack (the most recently freed block is handed out first,
initially 0, 1, 2, ...); a full block is indexed under (parent block, parent generation,
token ids); released indexed blocks wait in a queue and are evicted oldest first when the
stack is empty; appending to a partly filled shared block copies it first.
"""
from __future__ import annotations

OK, ERR_INVALID, ERR_NO_BLOCK = 0, -1, -3


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = False):
        self.nb = num_blocks
        self.bs = block_size
        self.pc = prefix_caching
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks
        self.free = list(range(num_blocks - 1, -1, -1))  # top = end
        self.evictable = []                               # oldest first
        self.key_of = {}                                  # block -> key
        self.index = {}                                   # key -> block
        self.seqs = []                                    # None once freed, else dict

    # ---- pool ----
    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        elif self.evictable:
            b = self.evictable.pop(0)
            self._unindex(b)
        else:
            raise RuntimeError("no block")
        self.ref[b] = 1
        self.gen[b] += 1
        return b

    def _unindex(self, b):
        if b in self.key_of:
            del self.index[self.key_of.pop(b)]

    def _release(self, b):
        self.ref[b] -= 1
        if self.ref[b] > 0:
            return
        if self.pc and b in self.key_of:
            self.evictable.append(b)
        else:
            self._unindex(b)
            self.free.append(b)

    def _key(self, parent, tokens):
        return (parent, 0 if parent < 0 else self.gen[parent], tuple(tokens))

    def _index_full(self, sq, j):
        if not self.pc:
            return
        b = sq["blocks"][j]
        if b in self.key_of:
            return
        parent = -1 if j == 0 else sq["blocks"][j - 1]
        k = self._key(parent, sq["tokens"][j * self.bs:(j + 1) * self.bs])
        if k in self.index:
            return
        self.index[k] = b
        self.key_of[b] = k

    def _live(self, s):
        return 0 <= s < len(self.seqs) and self.seqs[s] is not None

    # ---- operations (return codes as the library) ----
    def add_sequence(self, tokens):
        n = len(tokens)
        nblk = (n + self.bs - 1) // self.bs
        hit = []
        if self.pc:
            parent = -1
            for j in range(n // self.bs):
                k = self._key(parent, tokens[j * self.bs:(j + 1) * self.bs])
                if k not in self.index:
                    break
                hit.append(self.index[k])
                parent = hit[-1]
        evictable_hits = sum(1 for b in hit if b in self.evictable)
        if self.available() - evictable_hits < nblk - len(hit):
            return ERR_NO_BLOCK, 0
        sq = {"blocks": [], "tokens": list(tokens)}
        for b in hit:
            if b in self.evictable:
                self.evictable.remove(b)
            self.ref[b] += 1
            sq["blocks"].append(b)
        for _ in range(len(hit), nblk):
            sq["blocks"].append(self._take())
        for j in range(len(hit), n // self.bs):
            self._index_full(sq, j)
        self.seqs.append(sq)
        return len(self.seqs) - 1, len(hit) * self.bs

    def append_token(self, s, token):
        if not self._live(s):
            return ERR_INVALID, -1, -1, -1
        sq = self.seqs[s]
        pos = len(sq["tokens"])
        src = dst = -1
        if pos % self.bs == 0:
            if self.available() < 1:
                return ERR_NO_BLOCK, -1, -1, -1
            sq["blocks"].append(self._take())
        else:
            last = sq["blocks"][-1]
            if self.ref[last] > 1:
                if self.available() < 1:
                    return ERR_NO_BLOCK, -1, -1, -1
                fresh = self._take()
                self._release(last)
                sq["blocks"][-1] = fresh
                src, dst = last, fresh
        sq["tokens"].append(token)
        slot = sq["blocks"][-1] * self.bs + pos % self.bs
        if (pos + 1) % self.bs == 0:
            self._index_full(sq, len(sq["blocks"]) - 1)
        return OK, slot, src, dst

    def fork(self, parent):
        if not self._live(parent):
            return ERR_INVALID
        p = self.seqs[parent]
        for b in p["blocks"]:
            self.ref[b] += 1
        self.seqs.append({"blocks": list(p["blocks"]), "tokens": list(p["tokens"])})
        return len(self.seqs) - 1

    def free_sequence(self, s):
        if not self._live(s):
            return ERR_INVALID
        for b in reversed(self.seqs[s]["blocks"]):
            self._release(b)
        self.seqs[s] = None
        return OK

    def block_table(self, s):
        return list(self.seqs[s]["blocks"])

    def context_len(self, s):
        return len(self.seqs[s]["tokens"])
