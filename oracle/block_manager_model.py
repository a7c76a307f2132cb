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
  [P2] vLLM architecture deep-dive §2.3: with no free block, evict the block whose K-th
       most recent access is furthest back (LRU-K, K = 2 named).

Policies: free blocks are a stack (the most recently freed block is handed out first,
initially 0, 1, 2, ...); a full block is indexed under (parent block, parent generation,
token ids); released indexed blocks stay cached and, when the stack is empty, the one
with the oldest K-th most recent access is evicted (a clock ticks once per add, append
or fork; gaining a reference to a block or writing into it is an access, once per
operation; fewer than K accesses = oldest; ties: older last access, then deeper in its
chain, then lower id); appending to a partly filled shared block copies it first.
"""
from __future__ import annotations

OK, ERR_INVALID, ERR_NO_BLOCK = 0, -1, -3


class BlockManagerModel:
    def __init__(self, num_blocks: int, block_size: int, prefix_caching: bool = False, lru_k: int = 2):
        self.nb = num_blocks
        self.bs = block_size
        self.pc = prefix_caching
        self.k = lru_k
        self.clock = 0
        self.ref = [0] * num_blocks
        self.gen = [0] * num_blocks
        self.times = [[] for _ in range(num_blocks)]     # access times, most recent first
        self.depth = [0] * num_blocks
        self.free = list(range(num_blocks - 1, -1, -1))  # top = end
        self.evictable = []                               # unordered
        self.key_of = {}                                  # block -> key
        self.index = {}                                   # key -> block
        self.seqs = []                                    # None once freed, else dict

    def _access(self, b):
        if not self.times[b] or self.times[b][0] != self.clock:
            self.times[b].insert(0, self.clock)

    def _victim(self):
        def kth(b):
            return self.times[b][self.k - 1] if len(self.times[b]) >= self.k else -1

        def last(b):
            return self.times[b][0] if self.times[b] else -1

        return min(self.evictable, key=lambda b: (kth(b), last(b), -self.depth[b], b))

    # ---- pool ----
    def available(self) -> int:
        return len(self.free) + len(self.evictable)

    def _take(self) -> int:
        if self.free:
            b = self.free.pop()
        elif self.evictable:
            b = self._victim()
            self.evictable.remove(b)
            self._unindex(b)
        else:
            raise RuntimeError("no block")
        self.ref[b] = 1
        self.gen[b] += 1
        self._access(b)
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
        self.depth[b] = j

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
        self.clock += 1
        sq = {"blocks": [], "tokens": list(tokens)}
        for b in hit:
            if b in self.evictable:
                self.evictable.remove(b)
            self.ref[b] += 1
            self._access(b)
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
        need_new = pos % self.bs == 0
        need_copy = not need_new and self.ref[sq["blocks"][-1]] > 1
        if (need_new or need_copy) and self.available() < 1:
            return ERR_NO_BLOCK, -1, -1, -1
        self.clock += 1
        if need_new:
            sq["blocks"].append(self._take())
        elif need_copy:
            last = sq["blocks"][-1]
            fresh = self._take()
            self._release(last)
            sq["blocks"][-1] = fresh
            src, dst = last, fresh
        sq["tokens"].append(token)
        self._access(sq["blocks"][-1])
        slot = sq["blocks"][-1] * self.bs + pos % self.bs
        if (pos + 1) % self.bs == 0:
            self._index_full(sq, len(sq["blocks"]) - 1)
        return OK, slot, src, dst

    def fork(self, parent):
        if not self._live(parent):
            return ERR_INVALID
        p = self.seqs[parent]
        self.clock += 1
        for b in p["blocks"]:
            self.ref[b] += 1
            self._access(b)
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
