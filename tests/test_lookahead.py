"""Lookahead cache (host C++ in libpta, include/pta_lookahead.h) against the plain oracle
(oracle/lookahead.py), and the oracle against a hand-worked example and the properties its
definition fixes.  CPU only."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import paged_speculative_verify_amd as psv
from oracle.lookahead import LookaheadOracle, tree_mask_from_parents
from workload.tokens import synthetic_streams

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lookahead_worked_example.txt")


def golden():
    out = {}
    with open(GOLDEN, encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = (p.strip() for p in line.split("=", 1))
                out[k] = [int(x) for x in v.split()]
    return out


# ---------------------------------------------------------------- oracle pins
@pytest.mark.parametrize("mm,budget,key", [(2, 5, "mm2_budget5"), (4, 6, "mm4_budget6")])
def test_oracle_worked_example(mm, budget, key):
    g = golden()
    o = LookaheadOracle(g["window"][0], mm)
    o.append(0, g["history"])
    tok, par = o.propose(0, budget)
    assert tok == g[key + "_tokens"] and par == g[key + "_parents"]


def pin_budgets(cls=LookaheadOracle):
    """Budget arithmetic of the oracle class against the hand-worked golden values: hit-rate
    steps, a capped batch where flooring bites and one where the min_len floor keeps the total
    above the cap."""
    g = golden()
    o = cls(8, 4)
    assert o.update_budgets([0], [8], [2], 1, 8) == g["budget_after_2_of_8"]
    o = cls(8, 4)
    assert o.update_budgets([0, 1, 2], [0, 0, 8], [0, 0, 0], 1, 8, 10) == g["batch_cap_10_budgets"]
    o = cls(8, 4)
    assert o.update_budgets([0, 1, 2, 3], [0, 0, 8, 8], [0, 0, 0, 0], 1, 8, 11) == g["cap11_min1_budgets"]
    o = cls(8, 4)
    assert o.update_budgets([0, 1, 2, 3], [0, 0, 8, 8], [0, 0, 0, 0], 3, 8, 8) == g["cap8_min3_budgets"]
    o = cls(8, 4)
    steps = [o.update_budgets([0], [n], [a], 1, 8)[0] for n, a in ((8, 2), (4, 4), (0, 0), (3, 1))]
    assert steps == g["hit_steps_budgets"] and o.hit[0] == g["hit_steps_final_rate"][0]
    o = cls(8, 4)
    assert o.update_budgets([0, 1, 2], [0, 0, 0], [0, 0, 0], 1, 8, 0) == [8, 8, 8]   # no cap


def pin_released(cls=LookaheadOracle):
    """Global counts keep a released sequence's history (golden, worked by hand)."""
    g = golden()
    o = cls(4, 2)
    o.append(0, [1, 2, 3, 1, 2])
    o.append(1, [1, 2, 4] * 3)
    o.release(1)
    assert o.propose(0, 2) == (g["released_query_tokens"], g["released_query_parents"])
    assert o.propose(1, 2) == ([], [])
    o.append(1, [1, 2])
    assert o.propose(1, 2) == (g["reused_query_tokens"], g["reused_query_parents"])


def test_oracle_budgets_worked_example():
    pin_budgets()


def test_oracle_released_history_worked_example():
    pin_released()


class _RoundedCap(LookaheadOracle):
    """Planted mistake: the batch cap rounds to nearest instead of flooring."""
    def update_budgets(self, seqs, proposed, accepted, min_len, max_len, batch_cap=0):
        out = LookaheadOracle.update_budgets(self, seqs, proposed, accepted, min_len, max_len, 0)
        total = sum(out)
        if batch_cap > 0 and total > batch_cap:
            out = [max(min_len, (2 * b * batch_cap + total) // (2 * total)) for b in out]
        return out


class _NoMinFloorUnderCap(LookaheadOracle):
    """Planted mistake: the capped budgets lose their min_len floor."""
    def update_budgets(self, seqs, proposed, accepted, min_len, max_len, batch_cap=0):
        out = LookaheadOracle.update_budgets(self, seqs, proposed, accepted, min_len, max_len, 0)
        total = sum(out)
        if batch_cap > 0 and total > batch_cap:
            out = [b * batch_cap // total for b in out]
        return out


class _RoundedHitRate(LookaheadOracle):
    """Planted mistake: the accepted fraction is rounded up instead of floored."""
    def update_budgets(self, seqs, proposed, accepted, min_len, max_len, batch_cap=0):
        out = []
        for s, n, a in zip(seqs, proposed, accepted):
            h = self.hit.get(s, 1 << 16)
            if n > 0:
                h = (h + -(-(a << 16) // n)) >> 1
            self.hit[s] = h
            out.append(min(max((max_len * h + (1 << 15)) >> 16, min_len), max_len))
        total = sum(out)
        if batch_cap > 0 and total > batch_cap:
            out = [max(min_len, b * batch_cap // total) for b in out]
        return out


class _ForgetsReleased(LookaheadOracle):
    """Planted mistake: a released sequence's history leaves the global counts."""
    def release(self, seq):
        self.hist.pop(seq, None)
        self.hit.pop(seq, None)


class _KeepsReleasedLive(LookaheadOracle):
    """Planted mistake: release keeps the history live and also files it as retired (counted
    twice), and a re-used sequence id continues the old history."""
    def release(self, seq):
        if seq in self.hist:
            self.retired.append(list(self.hist[seq]))
        self.hit.pop(seq, None)


@pytest.mark.parametrize("mutant,pin", [(_RoundedCap, pin_budgets), (_NoMinFloorUnderCap, pin_budgets),
                                        (_RoundedHitRate, pin_budgets), (_ForgetsReleased, pin_released),
                                        (_KeepsReleasedLive, pin_released)])
def test_planted_mistakes_fail_a_pin(mutant, pin):
    with pytest.raises(AssertionError):
        pin(mutant)


def test_oracle_properties():
    """Best-first picks never raise the score (a string occurs at most as often as its prefix),
    a smaller budget gives a prefix of a larger one's answer, every candidate string occurs in
    some history, and no longer suffix than the match has a continuation."""
    streams = synthetic_streams(3, 300, vocab=40, seed=3)
    o = LookaheadOracle(6, 4)
    for s, t in enumerate(streams):
        o.append(s, t)
    for s in range(3):
        p = o.match(s)
        assert p is not None
        h = o.hist[s]
        for k in range(len(p) + 1, min(o.max_match, len(h)) + 1):
            assert not o.continuations(s, h[len(h) - k:])
        tok, par = o.propose(s, 12)
        strings = []
        for i, (x, q) in enumerate(zip(tok, par)):
            strings.append((p if q < 0 else strings[q]) + [x])
        scores = [o.score(s, st) for st in strings]
        assert all(a >= b for a, b in zip(scores, scores[1:]))
        assert all(o.count_global(st) > 0 for st in strings)
        assert all(len(st) <= o.window for st in strings)
        for b in range(13):
            tb, pb = o.propose(s, b)
            assert tb == tok[:b] and pb == par[:b]


def test_oracle_no_match_and_distinct_tokens():
    o = LookaheadOracle(8, 4)
    o.append(0, list(range(50)))            # every token once: nothing ever continues the suffix
    assert o.propose(0, 8) == ([], [])
    assert o.propose(7, 8) == ([], [])       # unknown sequence
    o.append(1, [49, 100])                   # another sequence continues 49 with 100 (global cache)
    assert o.propose(0, 8) == ([100], [-1])


def test_tree_mask_round_trip_with_accept_oracle():
    """The mask built from a proposal gives back the same parents under the acceptance
    oracle's own reading of the mask."""
    streams = synthetic_streams(2, 400, vocab=30, seed=4)
    o = LookaheadOracle(8, 4)
    for s, t in enumerate(streams):
        o.append(s, t)
    for s in range(2):
        tok, par = o.propose(s, 16)
        m = np.array(tree_mask_from_parents(par, len(tok), 16), np.uint8)
        assert list(oracle.tree_parents(m, len(tok))) == par


# ---------------------------------------------------------------- library parity
def run_both(window, mm, streams, queries, budget, max_q):
    c = psv.LookaheadCache(window, mm)
    o = LookaheadOracle(window, mm)
    for s, t in enumerate(streams):
        c.append(s, t)
        o.append(s, t)
    tok, par, cnt = c.propose(queries, [budget] * len(queries), max_q)
    for i, s in enumerate(queries):
        et, ep = o.propose(s, budget)
        assert cnt[i] == len(et), (s, cnt[i], len(et))
        assert list(tok[i, :cnt[i]]) == et and list(par[i, :cnt[i]]) == ep
        assert (tok[i, cnt[i]:] == -1).all() and (par[i, cnt[i]:] == -1).all()
    return c, o


@pytest.mark.parametrize("window,mm,vocab,n,seed", [
    (8, 4, 50, 400, 11), (4, 3, 20, 300, 12), (16, 8, 200, 600, 13), (2, 1, 10, 200, 14), (12, 2, 30, 500, 15),
])
def test_propose_matches_oracle(window, mm, vocab, n, seed):
    streams = synthetic_streams(4, n, vocab=vocab, seed=seed)
    run_both(window, mm, streams, [0, 1, 2, 3, 9], 10, 16)


def test_incremental_appends_release_and_budgets():
    streams = synthetic_streams(3, 240, vocab=25, seed=21)
    c = psv.LookaheadCache(6, 3)
    o = LookaheadOracle(6, 3)
    rng = np.random.default_rng(22)
    pos = [0, 0, 0]
    budgets = [8, 8, 8]
    for step in range(30):
        for s in range(3):
            k = int(rng.integers(0, 9))              # a step commits 0..8 tokens
            chunk = streams[s][pos[s]:pos[s] + k]
            pos[s] += k
            c.append(s, chunk)
            o.append(s, chunk)
        if step == 15:
            c.release(1)
            o.release(1)
        tok, par, cnt = c.propose([0, 1, 2], budgets, 8)
        for i in range(3):
            et, ep = o.propose(i, budgets[i])
            assert list(tok[i, :cnt[i]]) == et and list(par[i, :cnt[i]]) == ep
        acc = [int(rng.integers(0, x + 1)) for x in cnt]
        got = c.update_budgets([0, 1, 2], cnt, acc, 1, 8, 16)
        want = o.update_budgets([0, 1, 2], [int(x) for x in cnt], acc, 1, 8, 16)
        assert list(got) == want
        budgets = list(got)


def test_tree_mask_matches_oracle():
    streams = synthetic_streams(4, 300, vocab=20, seed=31)
    c, o = run_both(8, 4, streams, [0, 1, 2, 3], 12, 12)
    tok, par, cnt = c.propose([0, 1, 2, 3], [12, 5, 0, 12], 12)
    mask = psv.taco_la_tree_mask(par, cnt)
    for i in range(4):
        assert np.array_equal(mask[i], np.array(tree_mask_from_parents(list(par[i]), int(cnt[i]), 12), np.uint8))


def test_host_argument_checks():
    lib = psv.load()
    assert not lib.taco_la_create(1, 1) and not lib.taco_la_create(8, 8) and not lib.taco_la_create(65, 4)
    c = psv.LookaheadCache(8, 4)
    with pytest.raises(psv.PtaError):
        c.append(-1, [1, 2])
    with pytest.raises(psv.PtaError):
        c.append(0, [1, -2])
    with pytest.raises(psv.PtaError):
        c.propose([0], [9], 8)                      # budget above max_q
    with pytest.raises(psv.PtaError):
        c.update_budgets([0], [2], [3], 1, 8)       # more accepted than proposed
    with pytest.raises(psv.PtaError):
        psv.taco_la_tree_mask(np.array([[0, -1]], np.int32), [1])   # a node its own parent
    c.append(0, [])
    assert c.propose([0], [4], 8)[2][0] == 0


def test_append_batch_equals_single_appends():
    streams = synthetic_streams(5, 200, vocab=15, seed=41)
    a = psv.LookaheadCache(6, 4)
    b = psv.LookaheadCache(6, 4)
    pos = [0] * 5
    rng = np.random.default_rng(42)
    for _ in range(25):
        chunks = []
        for s in range(5):
            k = int(rng.integers(0, 7))
            chunks.append(streams[s][pos[s]:pos[s] + k])
            pos[s] += k
        a.append_batch([4, 3, 2, 1, 0], chunks[::-1])
        for s in range(5):
            b.append(s, chunks[s])
        ra, rb = a.propose(range(5), [6] * 5, 6), b.propose(range(5), [6] * 5, 6)
        assert all(np.array_equal(x, y) for x, y in zip(ra, rb))
    with pytest.raises(psv.PtaError):
        a.append_batch([0, 1], [[1, 2], [3, -1]])      # a negative token: nothing appended
    assert all(np.array_equal(x, y) for x, y in zip(a.propose(range(5), [6] * 5, 6),
                                                      b.propose(range(5), [6] * 5, 6)))


def test_library_matches_budget_and_release_goldens():
    """The C++ cache against the hand-worked values themselves (not only against the oracle)."""
    g = golden()
    c = psv.LookaheadCache(8, 4)
    assert list(c.update_budgets([0, 1, 2, 3], [0, 0, 8, 8], [0, 0, 0, 0], 1, 8, 11)) == g["cap11_min1_budgets"]
    c = psv.LookaheadCache(8, 4)
    assert list(c.update_budgets([0, 1, 2, 3], [0, 0, 8, 8], [0, 0, 0, 0], 3, 8, 8)) == g["cap8_min3_budgets"]
    c = psv.LookaheadCache(8, 4)
    steps = [int(c.update_budgets([0], [n], [a], 1, 8)[0]) for n, a in ((8, 2), (4, 4), (0, 0), (3, 1))]
    assert steps == g["hit_steps_budgets"]
    c = psv.LookaheadCache(4, 2)
    c.append(0, [1, 2, 3, 1, 2])
    c.append(1, [1, 2, 4] * 3)
    c.release(1)
    tok, par, cnt = c.propose([0, 1], [2, 2], 4)
    assert list(tok[0, :cnt[0]]) == g["released_query_tokens"] and list(par[0, :cnt[0]]) == g["released_query_parents"]
    assert cnt[1] == 0
    c.append(1, [1, 2])
    tok, par, cnt = c.propose([1], [2], 4)
    assert list(tok[0, :cnt[0]]) == g["reused_query_tokens"] and list(par[0, :cnt[0]]) == g["reused_query_parents"]


# ---------------------------------------------------------------- worker threads
def replay(threads, streams, window, mm, plan, budget, max_q):
    """Run an append/propose plan on a cache with the given thread count; every proposal."""
    c = psv.LookaheadCache(window, mm, threads=threads)
    assert c.threads == threads
    out = []
    for kind, arg in plan:
        if kind == "append":
            c.append_batch([s for s, _ in arg], [ch for _, ch in arg])
        elif kind == "release":
            c.release(arg)
        else:
            tok, par, cnt = c.propose(arg, [budget] * len(arg), max_q)
            out.append((tok.copy(), par.copy(), cnt.copy()))
    return out


def make_plan(streams, seed, steps, long_every=0):
    rng = np.random.default_rng(seed)
    n = len(streams)
    pos = [0] * n
    plan = []
    for step in range(steps):
        batch = []
        for s in rng.permutation(n):
            k = int(rng.integers(0, 9))
            if long_every and step % long_every == long_every - 1 and s % 2 == 0:
                k = int(rng.integers(40, 140))           # a chunk longer than the ring
            batch.append((int(s), streams[s][pos[s]:pos[s] + k]))
            pos[s] += k
        if step % 5 == 2:                                 # one sequence named twice in a batch
            s = int(rng.integers(0, n))
            batch.append((s, streams[s][pos[s]:pos[s] + 3]))
            pos[s] += 3
        plan.append(("append", batch))
        if step == steps // 2:
            plan.append(("release", 1))
        plan.append(("propose", list(range(n)) + [n + 5]))
    return plan


@pytest.mark.parametrize("window,mm", [(16, 8), (6, 3), (64, 63)])
def test_thread_count_does_not_change_results(window, mm):
    """The same appends and queries on 1, 3 and 8 threads give identical proposals: the global
    counts split by first token and the local ones by sequence count the same strings."""
    streams = synthetic_streams(12, 1200, vocab=60, seed=51)
    plan = make_plan(streams, 52, 40, long_every=7)
    ref = replay(1, streams, window, mm, plan, 10, 12)
    for t in (3, 8):
        got = replay(t, streams, window, mm, plan, 10, 12)
        for (a, b, c), (x, y, z) in zip(ref, got):
            assert np.array_equal(a, x) and np.array_equal(b, y) and np.array_equal(c, z)


@pytest.mark.parametrize("threads", [1, 4])
@pytest.mark.parametrize("chunk", [1, 40, 57, 70, 75, 130])
def test_long_chunks_match_oracle(threads, chunk):
    """Appends to an existing history in chunks around the ring length (64 tracked starts):
    a chunk of 50 .. 78 tokens makes a start read before the append share its ring slot with a
    start written by it."""
    window, mm = 16, 8
    streams = synthetic_streams(3, 700, vocab=25, seed=61 + chunk)
    c = psv.LookaheadCache(window, mm, threads=threads)
    o = LookaheadOracle(window, mm)
    pos = [0, 0, 0]
    for _ in range(4):
        batch = []
        for s in range(3):
            ch = streams[s][pos[s]:pos[s] + chunk + 3 * s]
            pos[s] += len(ch)
            batch.append(ch)
            o.append(s, ch)
        c.append_batch([0, 1, 2], batch)
        tok, par, cnt = c.propose([0, 1, 2], [9, 9, 9], 9)
        for s in range(3):
            et, ep = o.propose(s, 9)
            assert list(tok[s, :cnt[s]]) == et and list(par[s, :cnt[s]]) == ep


def test_set_threads_checks():
    lib = psv.load()
    c = psv.LookaheadCache(8, 4)
    assert c.threads == 1
    for bad in (0, -1, 65):
        with pytest.raises(psv.PtaError):
            c.set_threads(bad)
    assert c.threads == 1
    c.set_threads(5)
    assert c.threads == 5
    c.append(0, [1, 2, 3, 1, 2])
    c.set_threads(2)                                   # resized with history in place
    assert c.threads == 2 and list(c.propose([0], [2], 4)[0][0, :1]) == [3]
    c.set_threads(1)
    assert c.threads == 1
    assert lib.taco_la_set_threads(None, 2) == 1      # PTA_ERR_NULL_PTR
    assert lib.taco_la_threads(None) == 0


def test_bench_lookahead_line(capsys):
    """bench.py's lookahead-cache line on a small batch: it checks that 1 and 3 threads propose
    the same trees, and reports the back-to-back and in-loop rates."""
    import argparse
    import json
    import bench
    assert bench.lookahead_cache_bench(argparse.Namespace(la_threads=3), B=6, prompt=64, steps=10) == 0
    line = json.loads(capsys.readouterr().out.strip().splitlines()[-1])
    assert line["threads"] == 3 and line["value"] > 0 and line["unit"] == "trees/s"
    for k in ("back_to_back", "back_to_back_one_thread", "in_loop", "in_loop_one_thread"):
        assert line[k]["value"] > 0


def test_threaded_cache_in_a_forked_child():
    """A child process after fork() has none of the cache's workers: its calls run on the calling
    thread, give the parent's results, and taco_la_set_threads can start new workers there."""
    import multiprocessing as mp
    streams = synthetic_streams(4, 300, vocab=20, seed=71)
    c = psv.LookaheadCache(8, 4, threads=4)
    c.append_batch(range(4), streams)
    want = c.propose(range(4), [6] * 4, 6)
    ctx = mp.get_context("fork")
    q = ctx.Queue()

    def child():
        try:
            n0 = c.threads
            got = c.propose(range(4), [6] * 4, 6)
            c.append_batch(range(4), [s[:5] for s in streams])
            c.set_threads(3)
            again = c.propose(range(4), [6] * 4, 6)
            q.put((n0, c.threads, [x.tolist() for x in got], [x.tolist() for x in again]))
        except Exception as e:          # reported to the parent
            q.put(repr(e))

    p = ctx.Process(target=child)
    p.start()
    out = q.get(timeout=60)
    p.join(timeout=60)
    assert not isinstance(out, str), out
    n0, n1, got, again = out
    assert n0 == 1 and n1 == 3
    assert all(np.array_equal(np.array(g), w) for g, w in zip(got, want))
    assert p.exitcode == 0
    assert c.threads == 4                            # the parent keeps its workers
