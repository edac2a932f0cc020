"""Lookahead cache, written out plainly (TEST INFRASTRUCTURE).

Design talk "大模型倍速推理引擎 TACO-LLM 的设计与实践", section "优化方案设计思路",
part "1.基于批处理的 Lookahead Cache" (and "优化策略总结" item 1): each sequence of
a batch keeps a local cache, all share a global cache; a query is answered by
the longest match of the sequence's latest tokens; the answer is a
multi-branch forest; each sequence's candidate length adapts to its hit rate
and to the batch size.

The talk fixes no data structure or formula; this module takes these
readings (the library header restates them):
  * count_local(s, p) = occurrences of the token string p inside sequence s's
    history; count_global(p) = the sum over every history ever appended
    (released sequences included); only strings of length <= window count;
  * a query takes the longest suffix p of the history, len(p) <= max_match,
    with at least one continuation p + x of positive count; candidates are
    extensions of p, scored count_local + count_global, picked best first
    (score descending, then parent index, then token id), each pick making
    its own one-token extensions eligible, until the budget is spent;
  * hit rate h (16.16 fixed point, starts at 1.0): after a step that proposed
    n > 0 candidates of which a were accepted, h = (h + 65536 * a // n) // 2;
    budget = clamp((max_len * h + 32768) // 65536, min_len, max_len); when a
    batch's budgets sum past batch_cap > 0, each becomes
    max(min_len, budget * batch_cap // total).

Nothing here is shared with the library: counts are found by scanning the
histories, not from a trie.
"""
from __future__ import annotations


class LookaheadOracle:
    def __init__(self, window: int, max_match: int):
        assert 2 <= window <= 64 and 1 <= max_match <= window - 1
        self.window, self.max_match = window, max_match
        self.hist = {}        # live sequence -> list of tokens
        self.retired = []     # histories of released sequences (still in the global counts)
        self.hit = {}         # sequence -> hit rate, 16.16 fixed point

    # ------------------------------------------------------------------ history
    def append(self, seq: int, tokens) -> None:
        self.hist.setdefault(seq, []).extend(int(t) for t in tokens)

    def release(self, seq: int) -> None:
        if seq in self.hist:
            self.retired.append(self.hist.pop(seq))
        self.hit.pop(seq, None)

    # ------------------------------------------------------------------ counts
    @staticmethod
    def occurrences(h, p) -> int:
        """How many times the string p occurs inside history h."""
        n = len(p)
        return sum(1 for i in range(len(h) - n + 1) if h[i:i + n] == p)

    def count_local(self, seq: int, p) -> int:
        if len(p) > self.window:
            return 0
        return self.occurrences(self.hist.get(seq, []), list(p))

    def count_global(self, p) -> int:
        if len(p) > self.window:
            return 0
        return sum(self.occurrences(h, list(p)) for h in list(self.hist.values()) + self.retired)

    def score(self, seq: int, p) -> int:
        return self.count_local(seq, p) + self.count_global(p)

    def continuations(self, seq: int, p):
        """Tokens x with p + x counted somewhere, ascending."""
        if len(p) + 1 > self.window:
            return []
        xs = set()
        for h in list(self.hist.values()) + self.retired:
            n = len(p)
            for i in range(len(h) - n):
                if h[i:i + n] == list(p):
                    xs.add(h[i + n])
        return sorted(xs)

    # ------------------------------------------------------------------ query
    def match(self, seq: int):
        """The longest suffix of the history with a continuation, or None."""
        h = self.hist.get(seq, [])
        for k in range(min(self.max_match, len(h)), 0, -1):
            p = h[len(h) - k:]
            if self.continuations(seq, p):
                return p
        return None

    def propose(self, seq: int, budget: int):
        """(tokens, parents) of at most budget candidates, parents before children."""
        p = self.match(seq)
        if p is None or budget <= 0:
            return [], []
        frontier = [(self.score(seq, p + [x]), -1, x, p + [x]) for x in self.continuations(seq, p)]
        tokens, parents = [], []
        while frontier and len(tokens) < budget:
            best = min(frontier, key=lambda c: (-c[0], c[1], c[2]))
            frontier.remove(best)
            _, parent, x, s = best
            tokens.append(x)
            parents.append(parent)
            me = len(tokens) - 1
            frontier += [(self.score(seq, s + [y]), me, y, s + [y]) for y in self.continuations(seq, s)]
        return tokens, parents

    # ------------------------------------------------------------------ budgets
    def update_budgets(self, seqs, proposed, accepted, min_len: int, max_len: int, batch_cap: int = 0):
        out = []
        for s, n, a in zip(seqs, proposed, accepted):
            h = self.hit.get(s, 1 << 16)
            if n > 0:
                h = (h + (a << 16) // n) >> 1
            self.hit[s] = h
            out.append(min(max((max_len * h + (1 << 15)) >> 16, min_len), max_len))
        total = sum(out)
        if batch_cap > 0 and total > batch_cap:
            out = [max(min_len, b * batch_cap // total) for b in out]
        return out


def tree_mask_from_parents(parents, count: int, max_q: int):
    """Ancestor-or-self mask [max_q][max_q] (lists of 0/1) of one candidate forest."""
    m = [[0] * max_q for _ in range(max_q)]
    for i in range(count):
        j = i
        while j >= 0:
            m[i][j] = 1
            j = parents[j]
    return m
