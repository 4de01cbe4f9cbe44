"""Reference semantics of Feather's batch-forming structure, by brute force.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). It shares no code with
the library's C++ implementation.

Feather page ("Requests of a Feather Must Flock Together"), Metodologia, 1:
requests are represented by cumulative hashes over fixed-size token blocks;
the structure keeps a working set of the active batch's hashes and a min-heap
of waiting requests keyed by their missing count (blocks not yet covered by
the active batch), so the best request to add next is found in O(log W).
It supports insert, find-best, add-to-batch and remove-finished.

What that computes, written out plainly here (readings of points the page
leaves open):
  * only a request's full blocks count (a trailing partial block is not
    hashed); block i of request w is covered when some active request has
    the same tokens over blocks 0..i (cumulative hashes identify prefixes);
  * missing(w) = w's full blocks - the longest run of leading blocks w
    shares with any active request;
  * the best waiting request has the smallest missing count, ties going to
    the earliest inserted;
  * forming a batch (a static stand-in for the page's learned stopping
    policy, which is out of scope): if nothing is active, admit the earliest
    waiting request; then keep admitting the best one while its missing
    count is at most max_missing and the batch holds fewer than max_batch.
"""
from __future__ import annotations


class BruteCht:
    def __init__(self, block_size: int):
        self.bs = int(block_size)
        self.tokens = {}     # id -> list of tokens
        self.seq = {}        # id -> insertion order
        self.waiting = set()
        self.active = set()
        self._next = 0

    def insert(self, rid: int, tokens) -> None:
        if rid in self.tokens:
            raise ValueError("duplicate request id")
        self.tokens[rid] = [int(t) for t in tokens]
        self.seq[rid] = self._next
        self._next += 1
        self.waiting.add(rid)

    def nblocks(self, rid: int) -> int:
        return len(self.tokens[rid]) // self.bs

    def shared_blocks(self, a: int, b: int) -> int:
        ta, tb = self.tokens[a], self.tokens[b]
        n = min(len(ta), len(tb)) // self.bs
        k = 0
        while k < n and ta[k * self.bs:(k + 1) * self.bs] == tb[k * self.bs:(k + 1) * self.bs]:
            k += 1
        return k

    def missing(self, rid: int) -> int:
        best = 0
        for a in self.active:
            best = max(best, self.shared_blocks(rid, a))
        return self.nblocks(rid) - best

    def best(self):
        """(id, missing) of the best waiting request, or (-1, -1)."""
        if not self.waiting:
            return -1, -1
        rid = min(self.waiting, key=lambda w: (self.missing(w), self.seq[w]))
        return rid, self.missing(rid)

    def admit(self, rid: int) -> None:
        self.waiting.remove(rid)
        self.active.add(rid)

    def complete(self, rid: int) -> None:
        self.active.remove(rid)
        del self.tokens[rid]
        del self.seq[rid]

    def form_batch(self, max_batch: int, max_missing: int):
        out = []
        if not self.active and self.waiting and max_batch > 0:
            first = min(self.waiting, key=lambda w: self.seq[w])
            self.admit(first)
            out.append(first)
        while len(self.active) < max_batch:
            rid, m = self.best()
            if rid < 0 or m > max_missing:
                break
            self.admit(rid)
            out.append(rid)
        return out
