#!/usr/bin/env python3
"""Benchmark of the paged tree attention hot path on one MI355X.

One step = the whole hot path over one batch: append the candidates' K/V rows
into their paged slots, then paged tree attention over every sequence's
context (on the decode workloads the append runs inside the attention launch).
Inputs are synthetic, seeded and resident in HBM before the timed region;
R independent input sets are rotated step to step so the 256 MB last-level
cache cannot serve the KV stream of a previous step.

The default run measures the widest-tree, largest single-GPU workload
(long_splitk_verify: 4 sequences of 32K-128K tokens, 64/8 heads, a 32-node
candidate tree each) and prints ONE JSON line.  `value` is KV HBM bytes
(algorithmic: every K/V byte of every sequence's context counted once) per
second of whole-step wall time (append + attention, K steps between two
synchronisations with no timing events inside), in GB/s.  `roofline` holds the
attention call's HBM and matrix-core fractions: HIP events on the launch
stream bracket K back-to-back attention calls in a pass of their own.  The
same line carries the measured streaming-read and matrix-core ceilings of the
device, the fp64 CPU oracle timed on the host's cores and compared with the
timed call's output, and the other Llama-shaped workloads measured the same
way (fewer steps) under `workloads`.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "KV HBM GB/s (% of peak) + verified candidate tokens/s, paged tree attn, 1 GPU"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
HEADLINE = "long_splitk_verify"
# measured in the same run as the headline (attention call, parity on sampled sequences)
EXTRA_WORKLOADS = ("llama3_8b_decode", "llama31_70b_verify", "fp8_kv_chain")
# max |GPU - oracle| bound per KV dtype
TOLERANCE = {"f32": 1e-5, "bf16": 1e-2, "fp8": 3e-2}
SETTLE_S = 0.3                 # untimed steps after the warm-up, before any measurement

# launch configuration of each workload: entry point ("whole": one pass per
# sequence, "split": split-K partitions of `split` tokens, "balanced": equal
# page slices per wave of a persistent grid) and kernel family (auto picks by
# rows per KV head); fuse_append: the step's KV append runs inside the
# attention launch (taco_paged_tree_attn_append for the whole-context entry,
# taco_paged_tree_attn_balanced_append for the balanced one) instead of as
# taco_kv_append before it.  Fused where that measured faster; on the fp8 chain
# workload (1024 workgroups, each encoding 8 candidates) the in-kernel append
# costs what the separate launch does.
LAUNCH = {
    "tiny_decode": dict(mode="whole", split=None, path="auto"),
    "llama3_8b_decode": dict(mode="whole", split=None, path="auto", fuse_append=True),
    "llama31_70b_verify": dict(mode="balanced", split=None, path="auto", fuse_append=True),
    "long_splitk_verify": dict(mode="balanced", split=None, path="auto", fuse_append=True),
    "fp8_kv_chain": dict(mode="whole", split=None, path="auto"),
    "shared_prefix_decode": dict(mode="whole", split=None, path="auto", fuse_append=True),
}



def launch_config(name: str) -> dict:
    cfg = dict(LAUNCH[name])
    if cfg["mode"] == "shared":
        # the shared-prefix entry works split-K with the shared prefix as partition 0
        from workload.gen import CONFIGS
        cfg["split"] = CONFIGS[name].shared_prefix_pages * 16
    return cfg




# ------------------------------------------------------------------ accounting
def kv_bytes(w) -> int:
    """Algorithmic KV bytes of one attention pass: each K and V element of every
    sequence's context once, plus the per-(page, KV head) scales for fp8."""
    s = w.spec
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[s.kv_dtype]
    Hkv, D = w.k_cache.shape[1], w.k_cache.shape[3]
    n = int(w.ctx_lens.astype(np.int64).sum()) * Hkv * D * 2 * elem
    if s.kv_dtype == "fp8":
        n += int(w.pages_used.astype(np.int64).sum()) * Hkv * 2 * 4
    return n


def unique_kv_bytes(w) -> int:
    """KV bytes of the distinct (page, KV head) rows a pass must read at least once: with
    shared-prefix pages every group's prefix counts once, not once per member."""
    s = w.spec
    n = kv_bytes(w)
    if s.shared_prefix_pages > 0 and s.share_group > 1:
        elem = {"f32": 4, "bf16": 2, "fp8": 1}[s.kv_dtype]
        Hkv, D = w.k_cache.shape[1], w.k_cache.shape[3]
        B = w.q.shape[0]
        groups = (B + s.share_group - 1) // s.share_group
        n -= (B - groups) * s.shared_prefix_pages * 16 * Hkv * D * 2 * elem
    return n


def attn_flops(w) -> int:
    """Algorithmic flops: 4 * D per (q-head, candidate, visible key) pair."""
    D = w.q.shape[3]
    Hq = w.q.shape[2]
    tot = 0
    for b in range(w.q.shape[0]):
        C, qb = int(w.ctx_lens[b]), int(w.q_lens[b])
        L = C - qb
        vis = L * qb + int((w.tree_mask[b, :qb, :qb] != 0).sum())
        tot += vis
    return 4 * D * Hq * tot


# ------------------------------------------------------------------ device setup
class DeviceSet:
    """One input set on the device plus its KV-append operands."""

    def __init__(self, w, torch):
        from workload.device import to_device
        self.w = w
        self.d = to_device(w)
        s = w.spec
        B, Qmax, Hq, D = w.q.shape
        Hkv = w.k_cache.shape[1]
        # the candidates' slots: logical positions L..C-1 of every sequence
        pos = [(b, t) for b in range(B) for t in range(int(w.ctx_lens[b]) - int(w.q_lens[b]), int(w.ctx_lens[b]))]
        slots = np.array([int(w.block_tables[b, t // 16]) * 16 + t % 16 for b, t in pos], dtype=np.int64)
        # new rows equal to what the slots already hold, so re-appending every step is idempotent
        # (fp8: the rows are code * scale in float32, which re-encode to the same codes)
        if s.kv_dtype == "fp8":
            import torch as _t
            ks = np.empty((len(pos), Hkv, D), np.float32)
            vs = np.empty_like(ks)
            for n, (b, t) in enumerate(pos):
                page, off = int(w.block_tables[b, t // 16]), t % 16
                kc = _t.from_numpy(w.k_cache[page, :, off].copy()).view(_t.float8_e4m3fn).float().numpy()
                vc = _t.from_numpy(w.v_cache[page, :, off].copy()).view(_t.float8_e4m3fn).float().numpy()
                ks[n] = kc * w.k_scale[page][:, None]
                vs[n] = vc * w.v_scale[page][:, None]
            self.k_new = torch.from_numpy(ks).cuda()
            self.v_new = torch.from_numpy(vs).cuda()
        else:
            kn = np.stack([w.k_cache[int(w.block_tables[b, t // 16]), :, t % 16] for b, t in pos])
            vn = np.stack([w.v_cache[int(w.block_tables[b, t // 16]), :, t % 16] for b, t in pos])
            self.k_new = torch.from_numpy(kn).cuda()
            self.v_new = torch.from_numpy(vn).cuda()
            if s.kv_dtype == "bf16":
                self.k_new = self.k_new.view(torch.bfloat16)
                self.v_new = self.v_new.view(torch.bfloat16)
        self.slots = torch.from_numpy(slots).cuda()
        # the same rows laid out [B, Qmax, Hkv, D] for the append fused into the attention launch
        full = torch.zeros((B, Qmax, Hkv, D), dtype=self.k_new.dtype, device=self.k_new.device)
        fullv = torch.zeros_like(full)
        n = 0
        for b in range(B):
            qb = int(w.q_lens[b])
            full[b, :qb] = self.k_new[n:n + qb]
            fullv[b, :qb] = self.v_new[n:n + qb]
            n += qb
        self.k_new_full, self.v_new_full = full, fullv
        self.out = torch.empty_like(self.d.q)
        # shared-prefix groups: the first sequence of each run of share_group sequences leads it
        G = max(1, s.share_group) if s.shared_prefix_pages > 0 else 1
        self.max_group = G
        self.prefix_leader = torch.from_numpy(
            np.array([(b // G) * G for b in range(B)], dtype=np.int32)).to(self.d.q.device)
        self.lse = torch.empty((B, Hq, Qmax), dtype=torch.float32, device=self.d.q.device)
        self.workspace = None


# ------------------------------------------------------------------ CPU baseline (oracle)
def accepted_walk(tok, par, cnt, truth):
    """Greedy acceptance against the stream's true next tokens: the deepest candidate whose path
    spells truth[0..d-1]; returns d."""
    best, depth = 0, {}
    for i in range(cnt):
        d = 1 if par[i] < 0 else (depth.get(par[i], -1) + 1 if depth.get(par[i], -1) > 0 else -1)
        if d > 0 and d <= len(truth) and tok[i] == truth[d - 1]:
            depth[i] = d
            best = max(best, d)
        else:
            depth[i] = -1
    return best


def lookahead_cache_bench(args, B=64, prompt=1024, steps=200, window=16, max_match=8, max_len=8,
                          batch_cap=256):
    """Host lookahead cache over a decode batch: every step proposes each sequence's candidate
    tree, scores it against the synthetic stream's true continuation (greedy acceptance), feeds
    the hit back into the budgets and appends the accepted tokens plus one.  Timed: the library
    calls only (through the Python binding).  Run once on one thread and once on
    --la-threads threads; the proposals must agree."""
    import paged_speculative_verify_amd as psv
    from workload.tokens import synthetic_streams
    streams = synthetic_streams(B, prompt + steps * (max_len + 1) + 16, vocab=1000, seed=7)
    seq_arr = np.arange(B, dtype=np.int32)
    prompts = np.concatenate([np.asarray(streams[s][:prompt], np.int32) for s in range(B)])

    def run(threads, plan=None):
        """The decode loop; with plan (the per-step budgets and appended tokens of an earlier
        run) the calls are replayed back to back without the acceptance walk in between."""
        cache = psv.LookaheadCache(window, max_match, threads=threads)
        pos = [prompt] * B
        t0 = time.perf_counter()
        cache.append_packed(seq_arr, np.full(B, prompt, np.int32), prompts)
        t_ingest = time.perf_counter() - t0
        budgets = np.full(B, max_len, np.int32)
        made = cand = 0
        t_prop = t_rest = 0.0
        digest = 0
        record = []
        for step in range(steps):
            if plan is not None:
                budgets = plan[step][0]
            t0 = time.perf_counter()
            tok, par, cnt = cache.propose(seq_arr, budgets, max_len)
            t_prop += time.perf_counter() - t0
            if plan is None:
                digest = hash((digest, tok.tobytes(), par.tobytes()))
                acc = [accepted_walk(tok[i], par[i], int(cnt[i]), streams[i][pos[i]:pos[i] + max_len])
                       for i in range(B)]
                lens = np.array([a + 1 for a in acc], np.int32)      # accepted tokens plus the bonus token
                packed = np.concatenate([np.asarray(streams[i][pos[i]:pos[i] + acc[i] + 1], np.int32)
                                         for i in range(B)])
                acc = np.asarray(acc, np.int32)
                record.append((budgets, cnt, acc, lens, packed))
            else:
                _, cnt, acc, lens, packed = plan[step]
            t0 = time.perf_counter()
            budgets = cache.update_budgets(seq_arr, cnt, acc, 1, max_len, batch_cap)
            cache.append_packed(seq_arr, lens, packed)
            t_rest += time.perf_counter() - t0
            if plan is None:
                for i in range(B):
                    pos[i] += acc[i] + 1
                made += int(acc.sum()) + B
                cand += int(np.sum(cnt))
            else:
                digest = hash((digest, tok.tobytes(), par.tobytes()))
        t_lib = t_prop + t_rest
        return {"rate": B * steps / t_lib, "ms_step": 1e3 * t_lib / steps, "ms_propose": 1e3 * t_prop / steps,
                "ms_budgets_append": 1e3 * t_rest / steps, "ingest": B * prompt / t_ingest,
                "made": made, "cand": cand, "digest": digest, "record": record}

    def summary(r):
        return {"value": round(r["rate"], 1), "ms_per_batch_step": round(r["ms_step"], 4),
                "ms_propose": round(r["ms_propose"], 4), "ms_budgets_append": round(r["ms_budgets_append"], 4),
                "prompt_ingest_tokens_per_s": round(r["ingest"], 1)}

    loop1 = run(1)
    plan = loop1["record"]
    loopn = run(args.la_threads)
    back1 = run(1, plan)
    backn = run(args.la_threads, plan)
    if not (loop1["digest"] == loopn["digest"] and back1["digest"] == backn["digest"]):
        print("lookahead cache: proposals differ between 1 and %d threads" % args.la_threads, file=sys.stderr)
        return 1
    # the oracle on a bounded sample: 2 sequences, 10 steps
    import oracle
    o = oracle.LookaheadOracle(window, max_match)
    t0 = time.perf_counter()
    for s in range(2):
        o.append(s, streams[s][:prompt])
    for _ in range(10):
        for s in range(2):
            o.propose(s, max_len)
    t_or = time.perf_counter() - t0
    print(json.dumps({
        "metric": "lookahead cache: candidate trees proposed per second (host)",
        "value": round(backn["rate"], 1), "unit": "trees/s", "higher_is_better": True, "data": "synthetic",
        "threads": args.la_threads,
        "config": {"workload": "lookahead_cache_decode_batch", "batch": B, "prompt_tokens": prompt,
                   "steps": steps, "window": window, "max_match": max_match, "max_len": max_len,
                   "batch_cap": batch_cap},
        "back_to_back": summary(backn), "back_to_back_one_thread": summary(back1),
        "in_loop": summary(loopn), "in_loop_one_thread": summary(loop1),
        "tokens_per_step_mean": round(loop1["made"] / (B * steps), 3),
        "candidates_per_step_mean": round(loop1["cand"] / (B * steps), 3),
        "cpu_baseline": {"value": round(20 / t_or, 2), "unit": "trees/s", "cores": 1, "kind": "oracle",
                         "sample": f"2 sequences, {prompt}-token prompts, 10 proposals each, in {t_or:.1f} s"},
        "note": "value: the calls of the decode loop (propose, budgets, append) replayed back to back "
                "on the cache's threads; in_loop: the same calls with the Python acceptance walk "
                "(about a millisecond) between them, long enough for idle workers to sleep. Times "
                "include the Python binding's argument handling. tokens_per_step depends on the "
                "synthetic streams' repetition, not on real text"}))
    return 0


def blas_description() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{x.get('internal_api')} {x.get('version')} ({x.get('threading_layer')})"
                for x in threadpool_info() if x.get("user_api") == "blas"]
        return ", ".join(libs) if libs else "unknown"
    except Exception:                      # pragma: no cover - diagnostic only
        return "unknown"


def oracle_rows(w, sel):
    """fp64 oracle output of sequences `sel` (index array) of workload w."""
    import oracle
    s = w.spec
    ref, _ = oracle.paged_tree_attn(w.q[sel], w.k_cache, w.v_cache, w.block_tables[sel], w.ctx_lens[sel],
                                    w.q_lens[sel], w.tree_mask[sel], w.scale, q_dtype=s.q_dtype,
                                    kv_dtype=s.kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale)
    return ref


def max_diff(gpu_rows, ref) -> float:
    v = ~np.isnan(ref)                     # padding rows (i >= q_b) are NaN in the oracle
    return float(np.abs(gpu_rows[v] - ref[v]).max()) if v.any() else 0.0


def cpu_baseline(w, gpu_out, budget_s=12.0):
    """Time the fp64 oracle on whole sequences of the same workload, BLAS on every core of this
    process's affinity set, until the time budget is spent; report its KV GB/s and its max
    |difference| from the GPU output (of the timed call) on that sample."""
    from threadpoolctl import threadpool_limits
    s = w.spec
    elem = {"f32": 4, "bf16": 2, "fp8": 1}[s.kv_dtype]
    Hkv, D = w.k_cache.shape[1], w.k_cache.shape[3]
    cores = len(os.sched_getaffinity(0))
    done, kvb, err = [], 0, 0.0
    t_total = 0.0
    with threadpool_limits(limits=cores, user_api="blas"):
        for b in range(w.q.shape[0]):
            t0 = time.perf_counter()
            ref = oracle_rows(w, np.array([b]))
            t_total += time.perf_counter() - t0
            done.append(b)
            kvb += int(w.ctx_lens[b]) * Hkv * D * 2 * elem
            err = max(err, max_diff(gpu_out[b], ref[0]))
            if t_total >= budget_s:
                break
    return {"value": round(kvb / t_total / 1e9, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(done)} of {w.q.shape[0]} sequences (whole contexts, {kvb / 1e6:.0f} MB of KV) "
                      f"in {t_total:.1f} s, fp64 numpy; matrix products on {cores} BLAS threads "
                      f"({blas_description()}), element-wise steps on one thread",
            "sequences": done, "max_abs_diff_vs_gpu": err}


def load_traffic(config_name: str, src_hash: str):
    """HBM bytes per launch from the committed counter summary, if it matches the kernels."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != src_hash:
        return None
    return t.get("hbm_bytes_per_launch")


# ------------------------------------------------------------------ device ceilings
def calibrate(psv, torch, read_bytes=2 << 30, reps=5):
    """Measured ceilings of this device with the library's own kernels: a streaming read of a
    2 GiB buffer (far beyond the caches) and a bf16 matrix-core loop."""
    dev = torch.device("cuda")
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    buf = torch.empty(read_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    sink = torch.zeros(65535, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    res = {}
    for wg_per_cu in (4, 8):
        wgs = cus * wg_per_cu
        for _ in range(2):
            psv.taco_pta_calib_stream_read(buf, sink, wgs)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            psv.taco_pta_calib_stream_read(buf, sink, wgs)
        e1.record(stream)
        torch.cuda.synchronize()
        res[wgs] = read_bytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    best_wgs = max(res, key=res.get)
    del buf
    fsink = torch.zeros(65535, dtype=torch.float32, device=dev)
    wgs, iters = cus * 2, 4096
    for _ in range(2):
        psv.taco_pta_calib_mfma_bf16(wgs, iters, fsink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    flops = 0
    for _ in range(reps):
        flops += psv.taco_pta_calib_mfma_bf16(wgs, iters, fsink)
    e1.record(stream)
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) / 1e3) / 1e12
    return {"stream_read_gbs": round(res[best_wgs], 1),
            "stream_read": f"{read_bytes >> 30} GiB read once per launch with 16-byte loads, {best_wgs} "
                           f"workgroups of 256 lanes (best of {sorted(res)}), {reps} launches",
            "mfma_bf16_tflops": round(tflops, 1),
            "mfma_bf16": f"v_mfma_f32_32x32x16_bf16, 4 independent chains per wave, {wgs} workgroups of "
                         f"4 waves, {iters} rounds, {reps} launches",
            "compute_units": cus}


# ------------------------------------------------------------------ one workload
def resolve_cfg(name, args):
    """The workload's launch configuration with the command-line overrides applied."""
    cfg = launch_config(name)
    if args.path is not None:
        cfg["path"] = args.path
    if args.split is not None:
        cfg["mode"] = "split" if args.split > 0 else ("whole" if args.split == 0 else "balanced")
        cfg["split"] = args.split if args.split > 0 else None
    if args.shared_entry:
        from workload.gen import CONFIGS
        if CONFIGS[name].shared_prefix_pages <= 0 or args.private_pages:
            raise SystemExit("--shared-entry needs a shared-prefix workload on shared pages")
        cfg["mode"], cfg["split"] = "shared", CONFIGS[name].shared_prefix_pages * 16
    # the fused appends live in the whole-context stream grid and the wide balanced grid, as each
    # workload's own launch configuration uses them; any entry or path override runs the append apart
    if (cfg["mode"] != launch_config(name)["mode"] or args.path not in (None, "auto") or args.separate_append):
        cfg.pop("fuse_append", None)
    return cfg


def build_sets(psv, torch, name, cfg, nsets, private_pages=False):
    """Generate, upload and prepare `nsets` independent input sets of workload `name`."""
    from workload import make
    sets = []
    for r in range(nsets):
        w = make(name, seed=None if r == 0 else 1000 + r, **({"share_group": 1} if private_pages else {}))
        sets.append(DeviceSet(w, torch))
        print(f"[bench] {name} set {r}: ctx sum {int(w.ctx_lens.sum())}, KV {kv_bytes(w) / 1e6:.1f} MB",
              file=sys.stderr, flush=True)
    for ds in sets:
        d = ds.d
        if cfg["mode"] in ("split", "shared"):
            nbytes = psv.taco_paged_tree_attn_splitk_workspace_size(
                d.q, d.k_cache, d.block_tables, cfg["split"], max_ctx_len=d.max_ctx_len)
        elif cfg["mode"] == "balanced":
            nbytes = psv.taco_paged_tree_attn_balanced_workspace_size(
                d.q, d.k_cache, d.block_tables, max_ctx_len=d.max_ctx_len)
        else:
            nbytes = 0
        if nbytes:
            ds.workspace = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        # validated once, then re-issued with no per-call Python checks so the host stays ahead
        if cfg.get("fuse_append"):
            ds.append_call = lambda: None        # the append runs inside the attention launch
        else:
            ds.append_call = psv.prepare_kv_append(ds.k_new, ds.v_new, ds.slots, d.k_cache, d.v_cache,
                                                   k_scale=d.k_scale, v_scale=d.v_scale)
        # block tables that alias a shared prefix's pages say so (they keep the default cache policy)
        shared = ds.w.spec.shared_prefix_pages > 0 and ds.w.spec.share_group > 1
        ds.attn_call = psv.prepare_paged_tree_attn(
            cfg["mode"] + "_append" if cfg.get("fuse_append") else cfg["mode"],
            d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens, d.tree_mask,
            d.scale, ds.out, lse=ds.lse, k_scale=d.k_scale, v_scale=d.v_scale,
            partition_tokens=cfg["split"], workspace=ds.workspace, max_ctx_len=d.max_ctx_len,
            prefix_leader=ds.prefix_leader, max_group=ds.max_group, k_new=ds.k_new_full, v_new=ds.v_new_full,
            path=cfg["path"], shared_pages=shared)
    torch.cuda.synchronize()
    return sets


def measure(torch, sets, cfg, K, warmup, per_call=True):
    """Timings of one workload: warm-up, clock settling, the attention calls bracketed by HIP
    events on the launch stream (rotating sets: no cache reuse across calls), the same set
    repeated (warm), one event pair per call (percentiles), the append calls, and the whole
    steps between two synchronisations with nothing else in between."""
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        ds = sets[i % len(sets)]
        ds.append_call()
        ds.attn_call()
    torch.cuda.synchronize()
    # clock settling: a few warm-up steps are over in about a millisecond, well before the GPU
    # clock has ramped up; untimed steps continue for at least SETTLE_S of wall time so that
    # no measurement below sees the ramp
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < SETTLE_S:
        for _ in range(8):
            ds = sets[n_settle % len(sets)]
            ds.append_call()
            ds.attn_call()
            n_settle += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    order = [(warmup + n_settle + i) % len(sets) for i in range(K)]

    def bracketed(fn, idx):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(K):
            fn(sets[idx[i]])
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    # K attention calls back to back between two events (an event pair around every single
    # call adds its own overhead to each call)
    attn_ms = bracketed(lambda ds: ds.attn_call(), order)
    warm_ms = bracketed(lambda ds: ds.attn_call(), [order[0]] * K)
    pct = None
    if per_call:
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        torch.cuda.synchronize()
        for i in range(K):
            evs[i][0].record(stream)
            sets[order[i]].attn_call()
            evs[i][1].record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs]) * 1e3
        pct = {"p10": round(float(np.percentile(t, 10)), 2), "p50": round(float(np.percentile(t, 50)), 2),
               "p90": round(float(np.percentile(t, 90)), 2)}
    append_ms = None if cfg.get("fuse_append") else bracketed(lambda ds: ds.append_call(), order)
    # the timed steps: nothing but the step's own launches between the two synchronisations
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for i in range(K):
        ds = sets[order[i]]
        ds.append_call()
        ds.attn_call()
    t_enqueue = time.perf_counter() - t_wall
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    return {"order": order, "attn_ms": attn_ms, "warm_ms": warm_ms, "pct_us": pct, "append_ms": append_ms,
            "ms_per_step": wall / K * 1e3, "enqueue_ms": t_enqueue / K * 1e3, "n_settle": n_settle,
            "settle_ms": settle_ms}


def accounting(sets, order):
    """Per-launch means over the timed order: KV bytes (every sequence), distinct KV bytes,
    candidates and algorithmic flops."""
    K = len(order)
    flops = {r: attn_flops(sets[r].w) for r in set(order)}
    return {"kv": sum(kv_bytes(sets[o].w) for o in order) / K,
            "unique_kv": sum(unique_kv_bytes(sets[o].w) for o in order) / K,
            "cands": sum(int(sets[o].w.q_lens.sum()) for o in order) / K,
            "flops": sum(flops[o] for o in order) / K}


def timed_output(torch, ds):
    """The output of the prepared (timed) call on set ds, as float64 on the host."""
    ds.append_call()
    ds.attn_call()
    torch.cuda.synchronize()
    return ds.out.to(torch.float64).cpu().numpy()


def ceilings(acc, attn_ms):
    """Both roofline fractions of one attention call and the bound its intensity implies."""
    s = attn_ms / 1e3
    gbs = acc["unique_kv"] / s / 1e9
    tfl = acc["flops"] / s / 1e12
    intensity = acc["flops"] / acc["unique_kv"]
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    floor_s = max(acc["unique_kv"] / (HBM_PEAK_GBS * 1e9), acc["flops"] / (BF16_PEAK_TFLOPS * 1e12))
    return {"gbs": gbs, "tflops": tfl, "intensity": intensity, "ridge": ridge,
            "bound": "mfma" if intensity > ridge else "hbm", "floor_us": floor_s * 1e6,
            "frac_of_floor": floor_s / s}


def extra_workload(psv, torch, name, args):
    """One more Llama-shaped workload in the same run: fewer steps, parity of the timed call on
    sampled sequences."""
    cfg = resolve_cfg(name, argparse.Namespace(path=None, split=None, shared_entry=False, private_pages=False,
                                               separate_append=False))
    nsets = 1 if name == "fp8_kv_chain" else 2          # fp8: 2.4 GB of KV per set, ten times the LLC
    sets = build_sets(psv, torch, name, cfg, nsets)
    K = min(args.steps, 20)
    m = measure(torch, sets, cfg, K, args.warmup, per_call=False)
    acc = accounting(sets, m["order"])
    c = ceilings(acc, m["attn_ms"])
    w = sets[0].w
    gpu = timed_output(torch, sets[0])
    B = w.q.shape[0]
    sel = sorted(set([0, B // 3, (2 * B) // 3, B - 1]))
    ref = oracle_rows(w, np.array(sel))
    err = max(max_diff(gpu[b], ref[i]) for i, b in enumerate(sel))
    tol = TOLERANCE[w.spec.kv_dtype]
    res = {"entry": cfg["mode"] + (" (KV append fused)" if cfg.get("fuse_append") else ""),
           "attention_us": round(m["attn_ms"] * 1e3, 2), "attention_us_warm": round(m["warm_ms"] * 1e3, 2),
           "ms_per_step": round(m["ms_per_step"], 5), "kv_bytes_per_step": int(acc["kv"]),
           "hbm_gbs": round(c["gbs"], 1), "hbm_frac": round(c["gbs"] / HBM_PEAK_GBS, 4),
           "mfma_tflops": round(c["tflops"], 1), "mfma_frac": round(c["tflops"] / BF16_PEAK_TFLOPS, 4),
           "bound": c["bound"], "frac_of_roofline_time": round(c["frac_of_floor"], 4),
           "candidates_per_s": round(acc["cands"] / (m["ms_per_step"] / 1e3), 1), "steps": K,
           "input_sets_rotated": nsets, "parity_sequences": sel, "max_abs_diff_vs_oracle": err,
           "tolerance": tol, "parity_ok": bool(err <= tol)}
    del sets
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ quantized GEMM
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 MFMA
W4_GROUP = 128
GEMM_SHAPES = {
    # Llama-3.1-70B MLP gate + up projections (N = 2 x 28672, K = 8192) over the verify step's
    # 512 candidate tokens (32 sequences x 16), and over a 64-sequence decode step; W8A8 (fp8
    # activations and weights), W4A16 (bf16 activations, int4 weights in groups of 128) and W8A16
    # (bf16 activations, fp8 weights with per-channel scales)
    "llama70b_gate_up_verify512": ("w8a8", 512, 57344, 8192),
    "llama70b_gate_up_decode64": ("w8a8", 64, 57344, 8192),
    "w4a16_llama70b_gate_up_verify512": ("w4a16", 512, 57344, 8192),
    "w4a16_llama70b_gate_up_decode64": ("w4a16", 64, 57344, 8192),
    "w8a16_llama70b_gate_up_verify512": ("w8a16", 512, 57344, 8192),
    "w8a16_llama70b_gate_up_decode64": ("w8a16", 64, 57344, 8192),
    "w4a8_llama70b_gate_up_verify512": ("w4a8", 512, 57344, 8192),
    "w4a8_llama70b_gate_up_decode64": ("w4a8", 64, 57344, 8192),
}
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA (POP/s x 1000)


def w4a8_oracle_rows(oracle, a_codes, a_scale, w_packed, w_scale, group, with_bound=True):
    """(fp64 reference, bound 2^-8 |ref| + 2^-14 a_scale sum|a||q|s) of a few rows, column chunk by
    column chunk."""
    K = a_codes.shape[1]
    ref = np.empty((a_codes.shape[0], w_packed.shape[0]))
    S = np.empty_like(ref)
    A = np.abs(a_codes.view(np.int8).astype(np.float64)) * a_scale.astype(np.float64)[:, None]
    for c0 in range(0, w_packed.shape[0], 4096):
        c1 = min(c0 + 4096, w_packed.shape[0])
        ref[:, c0:c1] = oracle.w4a8_gemm(a_codes, a_scale, w_packed[c0:c1], w_scale[c0:c1], group)
        if with_bound:
            q = np.abs(oracle.decode_int4_packed(w_packed[c0:c1], K)).astype(np.float64)
            S[:, c0:c1] = A @ (q * np.repeat(w_scale[c0:c1].astype(np.float64), group, axis=1)).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def w8a16_oracle_rows(oracle, a_bits, w_codes, w_scale, with_bound=True):
    """(fp64 reference, bound 2^-8 |ref| + 2^-14 w_scale sum|a||w|) of a few rows, column chunk by
    column chunk."""
    from oracle.formats import decode_bf16, decode_fp8_e4m3fn
    ref = np.empty((a_bits.shape[0], w_codes.shape[0]))
    S = np.empty_like(ref)
    A = np.abs(decode_bf16(a_bits))
    for c0 in range(0, w_codes.shape[0], 4096):
        c1 = min(c0 + 4096, w_codes.shape[0])
        ref[:, c0:c1] = oracle.w8a16_gemm(a_bits, w_codes[c0:c1], w_scale[c0:c1])
        if with_bound:
            S[:, c0:c1] = A @ (np.abs(decode_fp8_e4m3fn(w_codes[c0:c1])) *
                               w_scale[c0:c1].astype(np.float64)[:, None]).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def w4a16_oracle_rows(oracle, a_bits, w_packed, w_scale, group, with_bound=True):
    """(fp64 reference, bound 2^-8 |ref| + 2^-14 sum|a||q|s) of a few rows, column chunk by column
    chunk (the decoded weights of the whole matrix would not fit in host memory at once)."""
    from oracle.formats import decode_bf16
    K = a_bits.shape[1]
    ref = np.empty((a_bits.shape[0], w_packed.shape[0]))
    S = np.empty_like(ref)
    A = np.abs(decode_bf16(a_bits))
    for c0 in range(0, w_packed.shape[0], 4096):
        c1 = min(c0 + 4096, w_packed.shape[0])
        ref[:, c0:c1] = oracle.w4a16_gemm(a_bits, w_packed[c0:c1], w_scale[c0:c1], group)
        if with_bound:
            q = np.abs(oracle.decode_int4_packed(w_packed[c0:c1], K)).astype(np.float64)
            S[:, c0:c1] = A @ (q * np.repeat(w_scale[c0:c1].astype(np.float64), group, axis=1)).T
    return ref, 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S


def gemm_bench(psv, torch, name, steps=30, warmup=5, cpu_rows=2, parity_rows=(0, 1, 255, 511)):
    """A quantized GEMM on one Llama-70B-shaped projection: timed calls (HIP events around
    back-to-back calls), roofline against the matrix-core peak of the operand type or HBM
    (whichever the shape's intensity says bounds it), parity of sampled output rows against the
    fp64 oracle, the oracle timed on a few rows."""
    import oracle
    from workload.gemm import make_w4a8_device, make_w4a16_device, make_w8a8_device, make_w8a16_device
    op, M, N, K = GEMM_SHAPES[name]
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    if op == "w8a8":
        a, sa, w, sw = make_w8a8_device(M, N, K, seed=11, torch=torch)
        # up to 256 rows the weights rearranged once (taco_gemm_w8a16_pack, untimed, as at model
        # load) are faster; past 256 rows the 128-byte k-step kernel on row-major weights is
        w8_tiled = M <= 256
        wt = psv.taco_gemm_w8a16_pack(w) if w8_tiled else None
        call = ((lambda: psv.taco_gemm_w8a8(a, sa, wt, sw, y, tiled=(N, K))) if w8_tiled
                else (lambda: psv.taco_gemm_w8a8(a, sa, w, sw, y)))
        peak = FP8_PEAK_TFLOPS
        kernel = "gemm_w8a8_k128_kernel" if M > 256 and K % 128 == 0 else "gemm_w8a8_kernel"
        nbytes = M * K + N * K + 2 * M * N + 4 * (M + N)
    elif op == "w8a16":
        a, w, sw = make_w8a16_device(M, N, K, seed=11, torch=torch)
        # weights rearranged into the kernel's load order once, as at model load (untimed)
        wt = psv.taco_gemm_w8a16_pack(w)
        call = lambda: psv.taco_gemm_w8a16(a, wt, sw, y, tiled=(N, K))
        peak, kernel = BF16_PEAK_TFLOPS, "gemm_w8a16_kernel"
        nbytes = 2 * M * K + N * K + 4 * N + 2 * M * N
    elif op == "w4a8":
        G = W4_GROUP
        a, sa, w, sw = make_w4a8_device(M, N, K, G, seed=11, torch=torch)
        # weights rearranged into the kernel's load order once, as at model load (untimed)
        wt = psv.taco_gemm_w4a16_pack(w)
        call = lambda: psv.taco_gemm_w4a8(a, sa, wt, sw, G, y, tiled=(N, K))
        peak, kernel = INT8_PEAK_TOPS, "gemm_w4a8_kernel"
        nbytes = M * K + 4 * M + N * K // 2 + 4 * N * (K // G) + 2 * M * N
    else:
        G = W4_GROUP
        a, w, sw = make_w4a16_device(M, N, K, G, seed=11, torch=torch)
        # weights rearranged into the kernel's load order once, as at model load (untimed)
        wt = psv.taco_gemm_w4a16_pack(w)
        call = lambda: psv.taco_gemm_w4a16(a, wt, sw, G, y, tiled=(N, K))
        peak, kernel = BF16_PEAK_TFLOPS, "gemm_w4a16_kernel"
        nbytes = 2 * M * K + N * K // 2 + 4 * N * (K // G) + 2 * M * N
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SETTLE_S:
        for _ in range(8):
            call()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        call()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * M * N * K
    tflops = flops / (ms / 1e3) / 1e12
    gbs = nbytes / (ms / 1e3) / 1e9
    intensity = flops / nbytes
    ridge = peak * 1e12 / (HBM_PEAK_GBS * 1e9)
    bound = "mfma" if intensity > ridge else "hbm"
    # parity: sampled rows of the timed call's output against the oracle; the oracle on a few
    # rows, all cores
    rows = np.array([r for r in parity_rows if r < M])
    sel = torch.from_numpy(rows).cuda()
    got = y[sel].float().cpu().numpy().astype(np.float64)
    from threadpoolctl import threadpool_limits
    cores = len(os.sched_getaffinity(0))
    if op == "w8a8":
        wc, wsc = w.cpu().numpy(), sw.cpu().numpy()
        ac, asc = a[sel].cpu().numpy(), sa.cpu().numpy()[rows]
        ref = oracle.w8a8_gemm(ac, asc, wc, wsc)
        from oracle.formats import decode_fp8_e4m3fn
        S = (np.abs(decode_fp8_e4m3fn(ac)) * asc.astype(np.float64)[:, None]) @ \
            (np.abs(decode_fp8_e4m3fn(wc)) * wsc.astype(np.float64)[:, None]).T
        bnd = 2.0 ** -8 * np.abs(ref) + 2.0 ** -14 * S
        with threadpool_limits(limits=cores, user_api="blas"):
            t0 = time.perf_counter()
            oracle.w8a8_gemm(ac[:cpu_rows], asc[:cpu_rows], wc, wsc)
            t_cpu = time.perf_counter() - t0
        dtype = "fp8-e4m3 x fp8-e4m3 -> f32 -> bf16"
        metric = "W8A8 GEMM TFLOP/s (fp8 e4m3fn operands, per-row scales, bf16 out), 1 GPU"
        bound_text = "2^-8 |y_ref| + 2^-14 a_scale w_scale sum|a||w| per output"
        config = {"workload": name, "M": M, "N": N, "K": K,
                  "weights": ("rearranged by taco_gemm_w8a16_pack before timing (taco_gemm_w8a8_tiled)"
                              if w8_tiled else "row-major")}
    elif op == "w8a16":
        a_bits = a[sel].view(torch.int16).cpu().numpy().view(np.uint16)
        wc, wsc = w.cpu().numpy(), sw.cpu().numpy()
        ref, bnd = w8a16_oracle_rows(oracle, a_bits, wc, wsc)
        with threadpool_limits(limits=cores, user_api="blas"):
            t0 = time.perf_counter()
            w8a16_oracle_rows(oracle, a_bits[:cpu_rows], wc, wsc, with_bound=False)
            t_cpu = time.perf_counter() - t0
        dtype = "bf16 x fp8-e4m3 (exact to bf16) -> f32, channel scale in f32 -> bf16"
        metric = "W8A16 GEMM TFLOP/s (bf16 activations, fp8 e4m3fn weights, per-channel scales, bf16 out), 1 GPU"
        bound_text = "2^-8 |y_ref| + 2^-14 w_scale sum_k |a||w| per output"
        config = {"workload": name, "M": M, "N": N, "K": K,
                  "weights": "rearranged by taco_gemm_w8a16_pack before timing (taco_gemm_w8a16_tiled)"}
    elif op == "w4a8":
        ac, asc = a[sel].cpu().numpy().view(np.uint8), sa.cpu().numpy()[rows]
        wp, wsc = w.cpu().numpy(), sw.cpu().numpy()
        ref, bnd = w4a8_oracle_rows(oracle, ac, asc, wp, wsc, W4_GROUP)
        with threadpool_limits(limits=cores, user_api="blas"):
            t0 = time.perf_counter()
            w4a8_oracle_rows(oracle, ac[:cpu_rows], asc[:cpu_rows], wp, wsc, W4_GROUP, with_bound=False)
            t_cpu = time.perf_counter() - t0
        dtype = "int8 x int4 (exact to int8) -> i32 per group, group scales in f32 -> bf16"
        metric = ("W4A8 GEMM TOP/s (int8 activations with row scales, int4 weights, group-128 scales, "
                  "bf16 out), 1 GPU")
        bound_text = "2^-8 |y_ref| + 2^-14 a_scale sum_k |a||q| w_scale per output"
        config = {"workload": name, "M": M, "N": N, "K": K, "group": W4_GROUP,
                  "weights": "rearranged by taco_gemm_w4a16_pack before timing (taco_gemm_w4a8_tiled)"}
    else:
        a_bits = a[sel].view(torch.int16).cpu().numpy().view(np.uint16)
        wp, wsc = w.cpu().numpy(), sw.cpu().numpy()
        ref, bnd = w4a16_oracle_rows(oracle, a_bits, wp, wsc, W4_GROUP)
        with threadpool_limits(limits=cores, user_api="blas"):
            t0 = time.perf_counter()
            w4a16_oracle_rows(oracle, a_bits[:cpu_rows], wp, wsc, W4_GROUP, with_bound=False)
            t_cpu = time.perf_counter() - t0
        dtype = "bf16 x int4 (exact to bf16) -> f32, group scales in f32 -> bf16"
        metric = "W4A16 GEMM TFLOP/s (bf16 activations, int4 weights, group-128 scales, bf16 out), 1 GPU"
        bound_text = "2^-8 |y_ref| + 2^-14 sum_k |a||q| w_scale per output"
        config = {"workload": name, "M": M, "N": N, "K": K, "group": W4_GROUP,
                  "weights": "rearranged by taco_gemm_w4a16_pack before timing (taco_gemm_w4a16_tiled)"}
    excess = float((np.abs(got - ref) - bnd).max())
    ops = "TOP/s" if op == "w4a8" else "TFLOP/s"          # integer products count as operations
    res = {
        "metric": metric,
        "value": round(tflops, 2), "unit": ops, "higher_is_better": True, "data": "synthetic",
        "dtype": dtype, "config": config,
        "us_per_call": round(ms * 1e3, 2), "steps": steps, "warmup": warmup,
        "roofline": {"bound": bound, "achieved": round(tflops if bound == "mfma" else gbs, 2),
                     "peak": peak if bound == "mfma" else HBM_PEAK_GBS,
                     "unit": ops if bound == "mfma" else "GB/s",
                     "frac": round(tflops / peak if bound == "mfma" else gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "mfma_frac": round(tflops / peak, 4),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes_per_launch": nbytes, "algorithmic_flops_per_launch": int(flops),
                     "arithmetic_intensity_flop_per_byte": round(intensity, 1),
                     "ridge_flop_per_byte": round(ridge, 1), "kernel": kernel,
                     "timing": f"HIP events on the launch stream around {steps} back-to-back calls"},
        "parity": {"rows": rows.tolist(), "max_excess_over_bound": excess, "parity_ok": bool(excess <= 0),
                   "bound": bound_text},
        "cpu_baseline": {"value": round(2.0 * cpu_rows * N * K / t_cpu / 1e12, 6), "unit": ops,
                         "cores": cores, "kind": "oracle",
                         "sample": f"{cpu_rows} output rows x {N} columns, fp64 numpy, {t_cpu:.1f} s"},
    }
    del a, w, y, call
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ main
def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE, choices=sorted(LAUNCH))
    ap.add_argument("--sets", type=int, default=2, help="input sets rotated step to step")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --config (no calibration kernels, no other workloads)")
    ap.add_argument("--path", choices=["auto", "valu", "mfma", "tile", "tile16"], default=None,
                    help="override the kernel family of the workload's launch configuration")
    ap.add_argument("--split", type=int, default=None,
                    help="override the entry point: split-K partition length, 0 = one pass per "
                         "sequence, -1 = balanced page slices")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--separate-append", action="store_true",
                    help="launch the KV append (taco_kv_append) apart from attention even where the "
                         "workload fuses it into the attention call")
    ap.add_argument("--shared-entry", action="store_true",
                    help="shared-prefix workload only: run taco_paged_tree_attn_shared_prefix (each "
                         "group's prefix partition worked once) instead of the whole-context grid")
    ap.add_argument("--private-pages", action="store_true",
                    help="shared-prefix workload only: the same batch with every sequence on pages of "
                         "its own (the reference the shared pages are compared with)")
    ap.add_argument("--lookahead-cache", action="store_true",
                    help="instead of the bench line: the host lookahead cache (propose, budgets, append) "
                         "over a decode batch of synthetic token streams, one JSON line; needs no GPU")
    ap.add_argument("--la-threads", type=int, default=8,
                    help="with --lookahead-cache: threads of the cache's batch calls (also timed on one)")
    ap.add_argument("--gemm", choices=sorted(GEMM_SHAPES), default=None,
                    help="instead of the bench line: one quantized GEMM (W8A8, W4A16, W8A16 or W4A8) on a Llama-70B-shaped projection")
    ap.add_argument("--qlen-floor", action="store_true",
                    help="instead of the bench line: attention time against the number of candidates "
                         "per sequence at the decode shape, T(q_len) / T(1)")
    args = ap.parse_args(argv)

    if args.lookahead_cache:
        return lookahead_cache_bench(args)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    import paged_speculative_verify_amd as psv
    psv.load()

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch_each_way": n, "launches": 5}))
        return 0

    if args.qlen_floor:
        return qlen_floor(psv, torch, args)

    if args.gemm:
        r = gemm_bench(psv, torch, args.gemm, steps=args.steps, warmup=args.warmup)
        print(json.dumps(r), flush=True)
        return 0 if r["parity"]["parity_ok"] else 3

    name = args.config
    cfg = resolve_cfg(name, args)
    extras = not args.no_extra and name == HEADLINE
    calib = None
    if extras:
        print("[bench] device ceilings (streaming read, matrix-core loop)", file=sys.stderr, flush=True)
        calib = calibrate(psv, torch)
    print(f"[bench] generating {args.sets} input set(s) for {name}", file=sys.stderr, flush=True)
    sets = build_sets(psv, torch, name, cfg, args.sets, private_pages=args.private_pages)
    K = args.steps
    m = measure(torch, sets, cfg, K, args.warmup)
    acc = accounting(sets, m["order"])
    c = ceilings(acc, m["attn_ms"])
    ms_per_step = m["ms_per_step"]
    value = acc["kv"] / (ms_per_step / 1e3) / 1e9          # whole-step throughput, every sequence's KV
    cand_per_s = acc["cands"] / (ms_per_step / 1e3)

    from paged_speculative_verify_amd.profsum import kernel_source_hash
    src_hash = kernel_source_hash()
    traffic = load_traffic(name + ("_private_pages" if args.private_pages else ""), src_hash)
    spec0 = sets[0].w.spec
    kernel = {"balanced": "paged tree attention grid + slice merge launch (balanced entry; one call = "
                          "both launches)",
              "split": "paged tree attention kernel (split-K entry, partition merge fused)",
              "whole": "paged tree attention kernel (whole-context entry"
                       + (", KV append fused)" if cfg.get("fuse_append") else ")"),
              "shared": "paged tree attention kernel (shared-prefix entry: each group's prefix partition once, "
                        "partition merge fused)"}[cfg["mode"]]
    hbm_frac = c["gbs"] / HBM_PEAK_GBS
    mfma_frac = c["tflops"] / BF16_PEAK_TFLOPS
    roofline = {
        "bound": c["bound"],
        "achieved": round(c["gbs"] if c["bound"] == "hbm" else c["tflops"], 2),
        "peak": HBM_PEAK_GBS if c["bound"] == "hbm" else BF16_PEAK_TFLOPS,
        "unit": "GB/s" if c["bound"] == "hbm" else "TFLOP/s",
        "frac": round(hbm_frac if c["bound"] == "hbm" else mfma_frac, 4),
        "traffic": traffic,
        "hbm": {"achieved_gbs": round(c["gbs"], 2), "peak_gbs": HBM_PEAK_GBS, "frac": round(hbm_frac, 4)},
        "mfma": {"achieved_tflops": round(c["tflops"], 2), "peak_tflops": BF16_PEAK_TFLOPS,
                 "frac": round(mfma_frac, 4), "flops": "4 * head_dim per visible (q-head, candidate, key) pair"},
        "arithmetic_intensity_flop_per_byte": round(c["intensity"], 2),
        "ridge_flop_per_byte": round(c["ridge"], 2),
        "roofline_time_us": round(c["floor_us"], 2),
        "frac_of_roofline_time": round(c["frac_of_floor"], 4),
        "kernel": kernel,
        "algorithmic_bytes_per_launch": int(acc["unique_kv"]),
        "algorithmic_flops_per_launch": int(acc["flops"]),
        "timing": f"HIP events on the launch stream around {K} back-to-back attention calls "
                  f"(input sets rotated), run before the timed steps",
    }
    if calib is not None:
        roofline["hbm"]["frac_of_measured_stream_read"] = round(c["gbs"] / calib["stream_read_gbs"], 4)
        roofline["mfma"]["frac_of_measured_mfma_loop"] = round(c["tflops"] / calib["mfma_bf16_tflops"], 4)
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "fp8": "fp8-e4m3 KV, bf16 Q"}[spec0.kv_dtype],
        "data": "synthetic",
        "config": {"workload": name + (" (private pages)" if args.private_pages else ""),
                   "batch": sets[0].w.q.shape[0], "q_heads": sets[0].w.q.shape[2],
                   "kv_heads": sets[0].w.k_cache.shape[1], "head_dim": sets[0].w.q.shape[3],
                   "max_q_len": sets[0].w.q.shape[1], "page": 16, "entry": cfg["mode"],
                   "kv_append": "fused into the attention call" if cfg.get("fuse_append") else "taco_kv_append",
                   "split_tokens": cfg["split"],
                   "path": cfg["path"], "input_sets_rotated": len(sets)},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        **({"shared_prefix": {"kv_bytes_all_sequences_per_step": int(acc["kv"]),
                              "distinct_kv_bytes_per_step": int(acc["unique_kv"]),
                              "note": "value counts every sequence's context; roofline counts distinct pages"}}
           if acc["unique_kv"] != acc["kv"] else {}),
        "candidates_per_s": round(cand_per_s, 1),
        "attention_ms": round(m["attn_ms"], 5),
        "attention_us_warm": round(m["warm_ms"] * 1e3, 2),
        "attention_us_per_call_events": m["pct_us"],
        "kv_append_ms": None if m["append_ms"] is None else round(m["append_ms"], 5),
        "host_enqueue_ms_per_step": round(m["enqueue_ms"], 5),
        "clock_settle": {"untimed_steps": m["n_settle"], "ms": round(m["settle_ms"], 1)},
        "attention_tflops": round(c["tflops"], 3),
        "roofline": roofline,
        "kernel_source_hash": src_hash,
    }
    if calib is not None:
        result["device_ceilings"] = calib
    parity_ok = True
    if not args.no_cpu_baseline:
        ds = sets[m["order"][-1]]
        gpu_out = timed_output(torch, ds)
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cb = cpu_baseline(ds.w, gpu_out)
        tol = TOLERANCE[ds.w.spec.kv_dtype]
        cb["compared_with"] = "output of the timed call (" + kernel + ")"
        cb["tolerance"] = tol
        parity_ok = cb["max_abs_diff_vs_gpu"] <= tol
        cb["parity_ok"] = bool(parity_ok)
        result["cpu_baseline"] = cb
    if sets[0].w.q.shape[1] > 1:
        result["accept_commit"] = time_accept_commit(psv, torch, sets[m["order"][-1]], K)
    if extras:
        del sets
        torch.cuda.empty_cache()
        result["workloads"] = {}
        for other in EXTRA_WORKLOADS:
            print(f"[bench] extra workload {other}", file=sys.stderr, flush=True)
            r = extra_workload(psv, torch, other, args)
            parity_ok = parity_ok and r["parity_ok"]
            result["workloads"][other] = r
        result["quantized_gemm"] = {}
        for g in sorted(GEMM_SHAPES):
            print(f"[bench] quantized GEMM {g}", file=sys.stderr, flush=True)
            r = gemm_bench(psv, torch, g, steps=min(args.steps, 20), warmup=args.warmup, cpu_rows=1)
            parity_ok = parity_ok and r["parity"]["parity_ok"]
            result["quantized_gemm"][g] = {k: r[k] for k in ("value", "unit", "us_per_call", "roofline", "parity",
                                                             "cpu_baseline", "config")}
    result["parity_ok"] = bool(parity_ok)
    print(json.dumps(result), flush=True)
    if not parity_ok:
        print("[bench] a timed call's output is outside the parity tolerance against the oracle",
              file=sys.stderr, flush=True)
        return 3
    return 0


def qlen_floor(psv, torch, args):
    """Verification cost against candidates per sequence (the pages' claim: checking several
    candidates in one pass costs about one decode step).  The decode workload's batch, heads and
    context draws are kept; each sequence carries q random-tree candidates (ctx_lens include
    them, so the KV bytes are the same for every q).  One JSON line with the mean attention
    time per q and its ratio to q = 1."""
    from workload import make
    stream = torch.cuda.current_stream()
    rows, t1 = [], None
    for q in (1, 2, 4, 8, 16, 32):
        entries = ["whole", "balanced"]
        sets = [DeviceSet(make("llama3_8b_decode", seed=None if r == 0 else 2000 + r, q_len=q,
                               tree="chain" if q == 1 else "random"), torch) for r in range(2)]
        for mode in entries:
            calls = []
            for ds in sets:
                d = ds.d
                if mode == "balanced":
                    ds.workspace = torch.zeros(psv.taco_paged_tree_attn_balanced_workspace_size(
                        d.q, d.k_cache, d.block_tables, max_ctx_len=d.max_ctx_len), dtype=torch.uint8,
                        device="cuda")
                calls.append(psv.prepare_paged_tree_attn(
                    mode, d.q, d.k_cache, d.v_cache, d.block_tables, d.ctx_lens, d.q_lens, d.tree_mask,
                    d.scale, ds.out, lse=ds.lse, workspace=ds.workspace if mode == "balanced" else None,
                    max_ctx_len=d.max_ctx_len))
            for i in range(args.warmup):
                calls[i % 2]()
            torch.cuda.synchronize()
            t_settle, n = time.perf_counter(), 0
            while time.perf_counter() - t_settle < SETTLE_S:      # clock settling, untimed
                for _ in range(8):
                    calls[n % 2]()
                    n += 1
                torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(args.steps):
                calls[i % 2]()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.steps
            kvb = sum(kv_bytes(sets[i % 2].w) for i in range(args.steps)) / args.steps
            fl = sum(attn_flops(sets[i % 2].w) for i in range(args.steps)) / args.steps
            if q == 1 and mode == "whole":
                t1 = ms
            rows.append({"q_len": q, "rows_per_kv_head": 4 * q, "entry": mode, "attention_ms": round(ms, 5),
                         "ratio_to_q1": round(ms / t1, 3), "kv_gbs": round(kvb / (ms / 1e3) / 1e9, 1),
                         "tflops": round(fl / (ms / 1e3) / 1e12, 1)})
            print(f"[bench] q_len {q} {mode}: {ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del sets
        torch.cuda.empty_cache()
    best = {}
    for x in rows:
        if x["q_len"] not in best or x["attention_ms"] < best[x["q_len"]]["attention_ms"]:
            best[x["q_len"]] = x
    print(json.dumps({"qlen_floor": rows,
                      "best_entry_ratio_to_q1": {q: {"entry": x["entry"], "ratio_to_q1": x["ratio_to_q1"]}
                                                 for q, x in sorted(best.items())},
                      "workload": "llama3_8b_decode shape (B 64, 32/8 heads, D 128, "
                      "ctx U[512, 4096]) with q_len random-tree candidates", "steps": args.steps,
                      "warmup": args.warmup, "timing": "HIP events on the launch stream around the back-to-back calls, 2 input sets "
                      "rotated"}),
          flush=True)
    return 0


def time_accept_commit(psv, torch, ds, K):
    """The step after verification: greedy acceptance over each candidate tree and
    compaction of the accepted rows' K/V (synthetic token ids: every node copies its
    parent's prediction with probability 0.7).  Runs last: it rewrites cache rows."""
    from workload import make_tokens
    w, d = ds.w, ds.d
    cand, target, tprev = make_tokens(w, 11, p_match=0.7)
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d.q.device)
    cand, target, tprev = T(cand), T(target), T(tprev)
    B, Qmax = cand.shape
    outs = [torch.empty(B, dtype=torch.int32, device=d.q.device),
            torch.empty(B, Qmax, dtype=torch.int32, device=d.q.device),
            torch.empty(B, dtype=torch.int32, device=d.q.device),
            torch.empty(B, dtype=torch.int32, device=d.q.device)]
    call = lambda: psv.taco_accept_commit(cand, target, tprev, d.ctx_lens, d.q_lens, d.tree_mask,
                                          d.block_tables, d.k_cache, d.v_cache, k_scale=d.k_scale,
                                          v_scale=d.v_scale, n_accepted=outs[0], accepted_path=outs[1],
                                          bonus_tokens=outs[2], new_ctx_lens=outs[3])
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        call()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / K * 1e3
    n = outs[0].cpu().numpy()
    return {"us_per_call": round(us, 2), "sequences": int(B), "mean_accepted": round(float(n.mean()), 3),
            "candidates": int(w.q_lens.sum()), "token_match_prob": 0.7}


if __name__ == "__main__":
    sys.exit(main())
