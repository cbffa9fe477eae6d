"""Benchmark of the learned top-k sparse attention hot path on one MI355X.

Headline: decode tok/s at 128K context, k = 2048 (64 sequences, 131072 cached
tokens + the new one each; one query per sequence per step).  A step is one
pass of the whole decode path over the batch: int8 indexer scan of every
cached index key -> exact top-k -> split-KV sparse attention.  The same JSON
line also carries the 128K prefill figure (the final 8192-query chunk of a
131072-token context through the two-stage path: block reps -> block
prefilter -> token scores in kept blocks -> top-k -> sparse attention).

Each step is one lsa_forward call; every tenth timed step also records a HIP event
on its launch stream after every stage (lsa_forward_stages lists them), so every
stage's kernels are timed live inside the timed region without an event gap in
every step.

The line also carries the other configurations of the path (the 1K, 32K and 256K-chunk
prefills, decode over paged caches, the pooled 4:1 indexer, the semantic search), each
with its dominant kernel against its roofline and the step against T_roof, and the
machine's measured ceilings (lsa_peak_*), which every fraction is also given against.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
       [--no-cpu-baseline] [--no-peaks] [--peaks] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill queries/s & decode tok/s at 128K ctx, k=2048; % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense int8 MFMA, published (5.0 POPS)
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def _describe(wl):
    s = (f"{wl.name}: B={wl.B} x n_q={wl.n_q} queries at positions {wl.q_pos0}..{wl.q_pos0 + wl.n_q - 1}, "
         f"{wl.L} cached keys, indexer H_I={wl.H_I} d_I={wl.d_I} int8, k={wl.k}, "
         f"attention {wl.H_q} bf16 query heads / 1 KV head d={wl.d}")
    if wl.pooled:
        s += (f", pooled indexer: one key per {wl.block_size} keys (block-key cache resident), "
              f"keep {wl.n_keep} blocks")
    elif wl.two_stage:
        s += f", two-stage blocks of {wl.block_size} keep {wl.n_keep}"
    if wl.page_size:
        s += f", paged caches (pages of {wl.page_size} tokens in a shared pool, {wl.spare_pages} spare pages)"
    return s


def _describe_sem(wl):
    return (f"{wl.name}: B={wl.B} x n_q={wl.n_q} queries at positions {wl.q_pos0}..{wl.q_pos0 + wl.n_q - 1}, "
            f"{wl.L} cached keys, flat semantic search over bf16 index keys of 64 dims: cluster blocks of "
            f"{wl.n_cluster} keys pooled {wl.n_pool}:1 into {wl.n_cluster // wl.n_bavg} Ward buckets "
            f"(cap {wl.n_bmax} keys), top {wl.p_top} buckets -> k={wl.k} long-range keys + {wl.n_sink} sinks + "
            f"a {wl.n_cluster}-key window; attention {wl.H_q} bf16 query heads / 1 KV head d={wl.d}; "
            f"bucket cache built before timing"
            + (f"; paged storage: keys, K and V in pools of {wl.page_size}-token pages ({wl.spare_pages} spare), "
               f"the bucket cache in a pool of entries behind a block table" if wl.page_size else ""))


# Stage events are recorded on every EVENTS_EVERY-th timed step only: an event recorded
# between two kernels holds the next launch back by ~5-6 us on this GPU (measured in a
# kernel trace), which would otherwise inflate every step by about one such gap per stage.
EVENTS_EVERY = 10


class Step:
    """One pass of the path: one lsa_forward call; with record=True it also records a
    HIP event on its launch stream after every stage (lsa_forward_stages names them),
    so every stage's kernels are timed live."""

    def __init__(self, lsa, torch, wl, inp):
        self.lsa, self.torch, self.wl, self.inp = lsa, torch, wl, inp
        dev = inp["q_idx"].device
        B, n_q = wl.B, wl.n_q
        self.kw = dict(two_stage="pooled" if wl.pooled else wl.two_stage, block_size=wl.block_size,
                       n_keep=wl.n_keep)
        ws_bytes = lsa.lsa_forward_workspace_size(inp, wl.k, **self.kw)
        self.ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
        self.stages = lsa.lsa_forward_stages(inp, wl.k, self.ws.numel(), **self.kw)
        self.names = list(dict.fromkeys(self.stages))
        self.out = {
            "idx": torch.empty((B, n_q, wl.k), dtype=torch.int32, device=dev),
            "count": torch.empty((B, n_q), dtype=torch.int32, device=dev),
            "out": torch.empty_like(inp["q"]),
            "lse": torch.empty((B, n_q, wl.H_q), dtype=torch.float32, device=dev),
        }
        if wl.two_stage:
            self.out["kept"] = torch.empty((B, n_q, wl.n_keep), dtype=torch.int32, device=dev)
        self.pool = []    # event sets for recorded steps, created (recorded once) ahead of time
        self.steps = []   # per recorded step: list of (stage, start_event, end_event)

    def make_events(self, n_steps):
        torch = self.torch
        stream = torch.cuda.current_stream()
        for _ in range(n_steps):
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(self.stages) + 1)]
            for e in evs:
                e.record(stream)   # creates the HIP event
            self.pool.append(evs)
        torch.cuda.synchronize()

    def run(self, record: bool):
        evs = self.pool[len(self.steps)] if record else None
        self.lsa.lsa_forward(self.inp, k_top=self.wl.k, out=self.out, ws=self.ws, stage_events=evs, **self.kw)
        if record:
            self.steps.append([(name, evs[i], evs[i + 1]) for i, name in enumerate(self.stages)])


    def kernel_ms(self):
        """Per stage: mean total ms per step, launches per step, mean ms per launch."""
        tot = {n: 0.0 for n in self.names}
        cnt = {n: 0 for n in self.names}
        for ev in self.steps:
            for name, a, b in ev:
                tot[name] += a.elapsed_time(b)
                cnt[name] += 1
        n_steps = max(1, len(self.steps))
        return {n: {"ms_per_step": tot[n] / n_steps, "launches_per_step": cnt[n] / n_steps,
                    "ms_per_launch": tot[n] / max(1, cnt[n])} for n in self.names}


def algorithmic(wl):
    """Algorithmic work of one step (what the method must compute / move), per kernel."""
    B, n_q, H_I, d_I, H_q, d, k = wl.B, wl.n_q, wl.H_I, wl.d_I, wl.H_q, wl.d, wl.k
    pos = [wl.q_pos0 + i for i in range(n_q)]
    vis = [min(p, wl.L - 1) + 1 for p in pos]
    if wl.pooled:
        bs, nk = wl.block_size, wl.n_keep
        nbl = wl.L // bs
        blk_pairs = B * sum(min(p // bs, nbl) for p in pos)
        att_pairs = B * sum(min(nk - 1, p // bs) * bs + (p - (p // bs) * bs + 1) for p in pos)
        return {
            "block_ops": 2 * H_I * d_I * blk_pairs * 2,           # two int8 parts per block key
            "block_bytes": B * (nbl * 2 * d_I + n_q * H_I * d_I),  # the block-key cache + index queries
            "attn_flops": 4 * H_q * d * att_pairs,
            "attn_gather_bytes": att_pairs * 2 * d * 2,
        }
    if wl.two_stage:
        bs, nk = wl.block_size, wl.n_keep
        blk_pairs = sum(p // bs for p in pos) * B
        tok_pairs = 0
        for p in pos:
            own = p // bs
            n_full = min(nk - 1, own)
            tok_pairs += n_full * bs + (p - own * bs + 1)
        tok_pairs *= B
        att_pairs = B * sum(min(k, c) for c in [min(nk - 1, p // bs) * bs + (p - (p // bs) * bs + 1) for p in pos])
        return {
            "index_ops": 2 * H_I * d_I * tok_pairs,
            "block_ops": 2 * H_I * d_I * blk_pairs,
            "attn_flops": 4 * H_q * d * att_pairs,
            "attn_gather_bytes": att_pairs * 2 * d * 2,
            "tok_pairs": tok_pairs,
        }
    pairs = B * sum(vis)
    att_pairs = B * sum(min(k, c) for c in vis)
    return {
        "index_ops": 2 * H_I * d_I * pairs,
        "index_bytes": B * (wl.L * d_I + n_q * H_I * d_I),   # every index key + the index queries, read once
        "topk_bytes": 4 * pairs,                             # every score read once
        "attn_flops": 4 * H_q * d * att_pairs,
        "attn_gather_bytes": att_pairs * 2 * d * 2,          # one K and one V bf16 row per listed key
        "pairs": pairs,
    }


def t_roof_ms(wl):
    """End-to-end lower bound of one step: max(sum of each contraction's ops at its dense
    peak, compulsory HBM bytes at peak bandwidth).  Compulsory bytes: the index queries
    and index keys read once, Q read and O written once, the K/V rows the lists touch
    (at most the whole visible cache) and the lists written once."""
    alg = algorithmic(wl)
    ops_ms = ((alg.get("index_ops", 0) + alg.get("block_ops", 0)) / (INT8_PEAK_TOPS * 1e12)
              + alg["attn_flops"] / (BF16_PEAK_TFLOPS * 1e12)) * 1e3
    B, n_q = wl.B, wl.n_q
    idx_keys = B * wl.L * wl.d_I if not wl.pooled else alg["block_bytes"]
    kv = min(B * wl.L * wl.d * 2 * 2, alg["attn_gather_bytes"])
    nbytes = B * n_q * wl.H_I * wl.d_I + idx_keys + B * n_q * wl.H_q * wl.d * 2 * 2 + kv + B * n_q * wl.k * 4
    return max(ops_ms, nbytes / (HBM_PEAK_GBS * 1e9) * 1e3)


def _cpu_threads():
    """Threads the oracle's BLAS uses (the CPU baselines' core count)."""
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(wl, inp, budget_s=10.0):
    """The oracle as it stands, on a bounded sample of the same workload's rows."""
    import numpy as np
    import oracle
    import synthetic
    rows = synthetic.checked_rows(wl, n_random=56)
    done = 0
    t_work = 0.0
    batches = {}
    # cycle over the seeded rows until about budget_s of oracle time has been spent
    order = [rows[t % len(rows)] for t in range(100000)]
    for (b, i) in order:
        if b not in batches:
            batches[b] = {
                "k_idx": inp["k_idx"][b].cpu().numpy(),
                "k": inp["k"][b].float().cpu().numpy().astype(np.float64),
                "v": inp["v"][b].float().cpu().numpy().astype(np.float64),
            }
            if len(batches) > 3:
                batches.pop(next(iter(batches)))
        hb = batches[b]
        qi = inp["q_idx"][b, i].cpu().numpy()
        q = inp["q"][b, i].float().cpu().numpy().astype(np.float64)
        w = inp["w"].cpu().numpy()
        p = int(inp["q_pos"][b, i])
        t0 = time.perf_counter()
        oracle.forward_row(qi, hb["k_idx"], w, p, wl.k, q_row=q, k_cache=hb["k"], v_cache=hb["v"],
                           scale=wl.scale, two_stage=wl.two_stage, block_size=wl.block_size, n_keep=wl.n_keep)
        t_work += time.perf_counter() - t0
        done += 1
        if t_work > budget_s:
            break
    rate = done / t_work
    cores = _cpu_threads()
    unit = "tok/s" if wl.n_q == 1 else "queries/s"
    return {"value": rate, "unit": unit, "cores": cores, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{done} row evaluations cycling over {len(rows)} seeded rows of {wl.name} (incl. boundary "
                      f"rows), {t_work:.1f}s of oracle time "
                      f"(numpy fp64 BLAS, int64 scores); rate = rows / time"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_128k_index_traffic.md")
TRAFFIC_SOURCES = ["learned_top_sparse_amd/csrc/lsa_indexer.hip", "learned_top_sparse_amd/csrc/lsa_device.h",
                   "learned_top_sparse_amd/csrc/lsa_select.h", "learned_top_sparse_amd/csrc/lsa_idx_tiles.h"]


def measured_traffic():
    """HBM bytes per launch of the decode indexer from the committed rocprofv3 counter
    runs (FETCH_SIZE + WRITE_SIZE, each scaled by a 1 GiB copy's reading), or None if the
    kernel's sources changed since the counters were taken."""
    import hashlib
    import re
    try:
        txt = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    m = re.search(r"^traffic_bytes_per_launch: (\d+)$", txt, re.M)
    h = re.search(r"^kernel_sources_sha256: ([0-9a-f]{64})$", txt, re.M)
    if not (m and h):
        return None
    d = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        d.update(open(os.path.join(ROOT, f), "rb").read())
    return int(m.group(1)) if d.hexdigest() == h.group(1) else None


COUNTER_FILE = os.path.join(ROOT, "profiles", "compute_counters.md")
COUNTER_SOURCES = ["learned_top_sparse_amd/csrc/lsa_topk.hip", "learned_top_sparse_amd/csrc/lsa_indexer.hip",
                   "learned_top_sparse_amd/csrc/lsa_attn.hip", "learned_top_sparse_amd/csrc/lsa_device.h",
                   "learned_top_sparse_amd/csrc/lsa_select.h", "learned_top_sparse_amd/csrc/lsa_idx_tiles.h",
                   "learned_top_sparse_amd/csrc/lsa_internal.h"]


def counter_mfma_busy(workload, stage):
    """Matrix-core busy share (SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs' cycles) of a stage's
    kernel from the committed rocprofv3 counter runs, or None if the kernel sources
    changed since they were taken (or the stage was not profiled)."""
    import hashlib
    import re
    try:
        txt = open(COUNTER_FILE).read()
    except OSError:
        return None
    h = re.search(r"^kernel_sources_sha256: ([0-9a-f]{64})$", txt, re.M)
    m = re.search(rf"^counter_mfma_busy: {re.escape(workload)} {re.escape(stage)} ([0-9.]+)$", txt, re.M)
    if not (h and m):
        return None
    d = hashlib.sha256()
    for f in COUNTER_SOURCES:
        d.update(open(os.path.join(ROOT, f), "rb").read())
    return float(m.group(1)) if d.hexdigest() == h.group(1) else None


SEM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_128k_lsa_scan_traffic.md")
SEM_TRAFFIC_SOURCES = ["learned_top_sparse_amd/csrc/lsa_semantic.hip"]


def sem_measured_traffic():
    """HBM bytes per launch of the semantic decode scan from its committed counter runs,
    or None if its source changed since they were taken."""
    import hashlib
    import re
    try:
        txt = open(SEM_TRAFFIC_FILE).read()
    except OSError:
        return None
    f = re.search(r"^\| FETCH_SIZE \|.*\| (\d+) \|$", txt, re.M)
    w = re.search(r"^\| WRITE_SIZE \|.*\| (\d+) \|$", txt, re.M)
    h = re.search(r"kernel_sources_sha256: ([0-9a-f]{64})", txt)
    if not (f and w and h):
        return None
    d = hashlib.sha256()
    for fn in SEM_TRAFFIC_SOURCES:
        d.update(open(os.path.join(ROOT, fn), "rb").read())
    return int(f.group(1)) + int(w.group(1)) if d.hexdigest() == h.group(1) else None


def cpu_baseline_sem(wl, inp, budget_s=10.0):
    """The oracle as it stands on a bounded sample of the semantic decode: one sequence's
    bucket cache clustered by the oracle (its cost spread over the n_cluster tokens a
    block takes to complete), then that sequence's query selected and attended to
    repeatedly for about budget_s seconds."""
    import numpy as np
    import oracle
    kb = inp["k_sem"][0].float().cpu().numpy()
    q_row = inp["q_sem"][0, 0].float().cpu().numpy()
    qa = inp["q"][0, 0].float().cpu().numpy().astype(np.float64)
    kc = inp["k"][0].float().cpu().numpy().astype(np.float64)
    vc = inp["v"][0].float().cpu().numpy().astype(np.float64)
    p = int(inp["q_pos"][0, 0])
    t0 = time.perf_counter()
    cache = oracle.bucket_cache(kb, wl.n_cluster, wl.n_pool, wl.n_bavg, wl.n_bmax)
    t_cluster = time.perf_counter() - t0
    per_block = t_cluster / cache["table"].shape[0]
    n, t1 = 0, time.perf_counter()
    while True:
        oracle.semantic_forward_row(q_row, cache, p, wl.k, wl.p_top, wl.n_sink, wl.n_cluster, q_row=qa, k_cache=kc,
                                    v_cache=vc, scale=wl.scale)
        n += 1
        if time.perf_counter() - t1 > budget_s:
            break
    per_token = (time.perf_counter() - t1) / n + per_block / wl.n_cluster
    return {"value": 1.0 / per_token, "unit": "tok/s", "cores": _cpu_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"sequence 0 of {wl.name}: its {cache['table'].shape[0]} cluster blocks clustered by the oracle "
                      f"in {t_cluster:.1f}s (one block per {wl.n_cluster} tokens), then {n} selections + attentions "
                      f"of its query in {budget_s:.0f}s; rate = 1 / (time per token + clustering per token)"}


def copy_calibration(torch, nbytes=1 << 30, reps=5):
    """Plain device copy of a known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    a = torch.empty((nbytes,), dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or the platform's processor string."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _time_launches(torch, launch, reps=5, warm=2):
    """Best of `reps` timed launches (ms), events on the current stream."""
    for _ in range(warm):
        launch()
    best = float("inf")
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        launch()
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    return best


RESIDENT_POOLS_MIB = (16, 64, 128)


def resident_pool_mib(wl):
    """The smallest measured cache-resident pool (MiB) that holds the workload's K and V caches."""
    kv_mib = wl.B * wl.L * 128 * 2 * 2 / (1 << 20)
    fits = [m for m in RESIDENT_POOLS_MIB if m >= kv_mib] or [RESIDENT_POOLS_MIB[-1]]
    return fits[0]


def attention_object(alg, at_ms, wl):
    """Prefill attention: bf16 utilisation beside its gather rate and the measured
    cache-resident gather ceiling for a pool of its K+V size."""
    gb = alg["attn_gather_bytes"] / (at_ms * 1e-3) / 1e9
    tf = alg["attn_flops"] / (at_ms * 1e-3) / 1e12
    obj = {"bf16_TFLOPs": tf, "frac_bf16_peak": tf / BF16_PEAK_TFLOPS, "gather_GBs": gb,
           "gather_bytes": alg["attn_gather_bytes"], "resident_pool_MiB": resident_pool_mib(wl),
           "frac_of_measured_resident_gather": None, "frac_of_measured_l2_gather": None}
    obj["counter_mfma_busy"] = counter_mfma_busy(wl.name, "sparse_attn")
    return obj


def fill_measured_fractions(res, peaks):
    """Every fraction of a measured ceiling in the line, once the ceilings are measured:
    the decode scan against the streaming read, decode attention against the cold gather,
    int8 rooflines against the MFMA loop, prefill attention against the cache-resident
    gather over its K+V size and the L2-resident one."""
    res["measured_peaks"] = peaks
    res["roofline"]["frac_of_measured_peak"] = res["roofline"]["achieved"] / peaks["hbm_read_GBs"]
    res["decode_attn"]["frac_of_measured_cold_gather"] = res["decode_attn"]["achieved_GBs"] / peaks["gather_cold_GBs"]
    for obj in res.values():
        if not isinstance(obj, dict):
            continue
        roof = obj.get("roofline")
        if isinstance(roof, dict) and roof.get("unit") == "TOP/s":
            roof["frac_of_measured_peak"] = roof["achieved"] / peaks["int8_mfma_TOPs"]
        at = obj.get("attention")
        if isinstance(at, dict) and "resident_pool_MiB" in at:
            at["frac_of_measured_resident_gather"] = (at["gather_GBs"]
                                                      / peaks["gather_resident_GBs"][str(at["resident_pool_MiB"])])
            at["frac_of_measured_l2_gather"] = at["gather_GBs"] / peaks["gather_l2_GBs"]


def measure_peaks(lsa, torch):
    """The machine's reachable ceilings (lsa_peak_* microbenchmarks): int8 and bf16 MFMA
    issue, HBM streaming read over 2 GiB, random 256-byte row gathers over a 2 GiB pool
    after a 1 GiB read that evicts the caches (cold: the decode step's 67 MB, one
    launch timed with events like the step's stages), and steady-state gathers of 4.3 GB
    from a 64 MiB pool (Infinity Cache resident) and from a 2 MiB pool (L2 resident).
    Best of 5 launches each."""
    import ctypes as C
    L = lsa.lib()
    dev = torch.device("cuda:0")
    st = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"compute_units": n_cu}

    def sink_for(nb):
        return torch.empty((L.lsa_peak_sink_ints(nb),), dtype=torch.int32, device=dev)

    def check(rc, name):
        if rc != 0:
            raise RuntimeError(f"{name} failed: {rc}")

    nb, iters = 8 * n_cu, 2048
    sk = sink_for(nb)
    for kind, key, ops in ((0, "int8_mfma_TOPs", 32768), (1, "bf16_mfma_TFLOPs", 16384)):
        ms = _time_launches(torch, lambda: check(L.lsa_peak_mfma(kind, iters, nb, C.c_void_p(sk.data_ptr()), st),
                                                 "lsa_peak_mfma"))
        res[key] = nb * 4 * iters * 4 * ops / (ms * 1e-3) / 1e12
    big = torch.ones((2 << 30,), dtype=torch.uint8, device=dev)
    flush = torch.ones((1 << 30,), dtype=torch.uint8, device=dev)
    nb = 16 * n_cu
    sk = sink_for(nb)
    ms = _time_launches(torch, lambda: check(L.lsa_peak_read(C.c_void_p(big.data_ptr()), big.numel(), nb,
                                                             C.c_void_p(sk.data_ptr()), st), "lsa_peak_read"))
    res["hbm_read_GBs"] = big.numel() / (ms * 1e-3) / 1e9
    n_idx = 1 << 18  # 67 MB of 256-byte rows, the decode step's gather volume
    g = torch.Generator(device=dev).manual_seed(0)
    nbg = 8 * n_cu  # many waves with few rows in flight each: the fastest launch shape for random rows
    sk = sink_for(max(nb, nbg))

    def gather_ms(pool, n_rows, evict, n):
        idx = torch.randint(0, n_rows, (n,), dtype=torch.int32, device=dev, generator=g)
        best = float("inf")
        for _ in range(5):
            if evict:
                # a 1 GiB read with ordinary loads displaces the caches and leaves them clean
                # (the streaming probe's non-temporal loads would leave them as they were)
                flush.sum()
            else:
                check(L.lsa_peak_gather(C.c_void_p(pool.data_ptr()), n_rows, C.c_void_p(idx.data_ptr()), n, nbg,
                                        C.c_void_p(sk.data_ptr()), st), "lsa_peak_gather")
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            check(L.lsa_peak_gather(C.c_void_p(pool.data_ptr()), n_rows, C.c_void_p(idx.data_ptr()), n, nbg,
                                    C.c_void_p(sk.data_ptr()), st), "lsa_peak_gather")
            b.record()
            b.synchronize()
            best = min(best, a.elapsed_time(b))
        del idx
        return best

    res["gather_cold_GBs"] = n_idx * 256 / (gather_ms(big, big.numel() // 256, True, n_idx) * 1e-3) / 1e9
    n_steady = 1 << 24  # 4.3 GB of rows: long enough that launch and ramp do not count
    # cache-resident pools the size of the prefill workloads' K and V caches (the share
    # an XCD's L2 holds decides the rate); gather_warm_GBs is the 64 MiB one
    res["gather_resident_GBs"] = {}
    for mib in RESIDENT_POOLS_MIB:
        pool = big[: mib << 20]
        res["gather_resident_GBs"][str(mib)] = (n_steady * 256 / (gather_ms(pool, pool.numel() // 256, False, n_steady)
                                                                  * 1e-3) / 1e9)
    res["gather_warm_GBs"] = res["gather_resident_GBs"]["64"]
    l2 = big[: 2 << 20]
    res["gather_l2_GBs"] = n_steady * 256 / (gather_ms(l2, l2.numel() // 256, False, n_steady) * 1e-3) / 1e9
    res["method"] = ("lsa_peak_* kernels (include/lsa_peaks.h): MFMA loops of 4 independent chains per wave over "
                     f"{8 * n_cu} workgroups of 4 waves; 2 GiB streaming read (one contiguous span per workgroup, non-temporal loads); random 256-byte rows over {nbg} "
                     f"workgroups: {n_idx} rows from a 2 GiB pool after a 1 GiB read with ordinary loads (cold, the decode step's volume), "
                     f"{n_steady} rows from pools of {', '.join(str(m) for m in RESIDENT_POOLS_MIB)} MiB (the "
                     "prefill workloads' K+V sizes, Infinity Cache resident) and from a 2 MiB pool (L2 resident), "
                     "the warm pools read just before; best of 5")
    del big, flush
    torch.cuda.empty_cache()
    return res


class SemStep:
    """One pass of flat semantic search over the batch: for a prefill chunk, the clustering
    of the cluster blocks its keys complete; lsa_semantic_select (index-query
    normalisation, centroid scores, top-p and expansion); lsa_sparse_attn over the lists.
    With record=True a HIP event is recorded around each call on the stream they run on.
    The cache of the blocks before the chunk is built beforehand (a serving loop
    clusters each block once, when it completes)."""

    def __init__(self, lsa, torch, wl, inp, cache):
        self.lsa, self.torch, self.wl, self.inp, self.cache = lsa, torch, wl, inp, cache
        dev = inp["q_sem"].device
        W = wl.n_sink + wl.k + wl.n_cluster
        self.idx = torch.empty((wl.B, wl.n_q, W), dtype=torch.int32, device=dev)
        self.count = torch.empty((wl.B, wl.n_q), dtype=torch.int32, device=dev)
        self.ws = torch.empty((max(16, lsa.lsa_semantic_workspace_size(wl.B, wl.n_q, cache)),), dtype=torch.uint8,
                              device=dev)
        # a prefill chunk first clusters the blocks its own keys complete (its later
        # queries score them); decode clusters one block per n_cluster tokens, reported
        # apart as an amortised cost
        self.chunk_blocks = None
        if wl.n_q > 1:
            first = wl.q_pos0 // wl.n_cluster
            last = min(wl.L, wl.q_pos0 + wl.n_q) // wl.n_cluster
            if last > first:
                self.chunk_blocks = (first, last - first)
        # with contiguous caches the selection call records its own events around the
        # centroid scan (lsa_semantic_select_timed)
        self.timed = "paged" not in inp
        sel = ["centroid_scan", "select_expand"] if self.timed else ["semantic_select"]
        self.names = (["cluster"] if self.chunk_blocks else []) + sel + ["sparse_attn"]
        self.pool, self.steps = [], []

    make_events = Step.make_events
    kernel_ms = Step.kernel_ms

    @property
    def stages(self):
        return self.names

    def run(self, record: bool):
        evs = self.pool[len(self.steps)] if record else None
        st = self.torch.cuda.current_stream()
        wl = self.wl
        e = 0
        if record:
            evs[e].record(st)
        if self.chunk_blocks:
            self.lsa.lsa_semantic_cache(self.inp["k_sem"], cache=self.cache, first_block=self.chunk_blocks[0],
                                        n_update=self.chunk_blocks[1], paged=self.inp.get("paged"))
            if record:
                e += 1
                evs[e].record(st)
        if record and self.timed:
            self.lsa.lsa_semantic_select(self.inp["q_sem"], self.inp["q_pos"], self.cache, wl.k, wl.p_top,
                                         wl.n_sink, wl.n_cluster, idx=self.idx, count=self.count, ws=self.ws,
                                         stage_events=(evs[e], evs[e + 1], evs[e + 2]))
            e += 2
        else:
            self.lsa.lsa_semantic_select(self.inp["q_sem"], self.inp["q_pos"], self.cache, wl.k, wl.p_top,
                                         wl.n_sink, wl.n_cluster, idx=self.idx, count=self.count, ws=self.ws,
                                         paged=self.inp.get("paged"))
            if record:
                e += 1
                evs[e].record(st)
        self.out, _ = self.lsa.lsa_sparse_attn(self.inp["q"], self.inp["k"], self.inp["v"], self.idx,
                                               scale=wl.scale, return_lse=False)
        if record:
            evs[e + 1].record(st)
            self.steps.append([(n, evs[i], evs[i + 1]) for i, n in enumerate(self.names)])


def sem_algorithmic(wl):
    """Algorithmic work of one semantic step: centroids read (8 KB per cluster block
    before each query's own), centroid scores, attention over the lists."""
    pos = [wl.q_pos0 + i for i in range(wl.n_q)]
    nbl = wl.L // wl.n_cluster
    m = wl.n_cluster // wl.n_bavg
    blocks = [min(p // wl.n_cluster, nbl) for p in pos]
    lists = [min(wl.n_sink, p + 1) + (min(p, wl.n_cluster - 1) + 1) + min(wl.k, b * wl.n_cluster) for p, b in
             zip(pos, blocks)]
    att_pairs = wl.B * sum(lists)
    return {
        "centroid_bytes": wl.B * max(blocks) * m * 64 * 2 if wl.n_q == 1 else wl.B * nbl * m * 64 * 2,
        "score_flops": wl.B * sum(blocks) * m * 64 * 2,
        "attn_flops": 4 * wl.H_q * wl.d * att_pairs,
        "attn_gather_bytes": att_pairs * 2 * wl.d * 2,
    }


def measure_sem(lsa, torch, wl, steps, warmup):
    import synthetic
    dev = torch.device("cuda:0")
    inp = synthetic.make_inputs(wl.replace(page_size=0), dev)
    inp.update(synthetic.semantic_inputs(wl, dev))
    del inp["q_idx"], inp["k_idx"]
    prm = (wl.n_cluster, wl.n_pool, wl.n_bavg, wl.n_bmax)
    if wl.page_size:
        inp = synthetic.semantic_paged(inp, wl.page_size, wl.spare_pages, wl.L // wl.n_cluster)
    paged = inp.get("paged")
    torch.cuda.synchronize()
    # the whole bucket cache once (every complete block of every sequence), then the
    # launch a decode step pays every n_cluster tokens: one new block per sequence
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record()
    cache = lsa.lsa_semantic_cache(inp["k_sem"], *prm, paged=paged, n_bslots=inp.get("n_bslots"))
    e[1].record()
    nb = cache.get("NB", cache["table"].shape[1])
    lsa.lsa_semantic_cache(inp["k_sem"], cache=cache, first_block=nb - 1, n_update=1, paged=paged)
    e[2].record()
    torch.cuda.synchronize()
    cluster = {"full_cache_ms": e[0].elapsed_time(e[1]), "blocks": wl.B * nb,
               "one_block_per_sequence_ms": e[1].elapsed_time(e[2]),
               "amortised_ms_per_decode_step": e[1].elapsed_time(e[2]) / wl.n_cluster}
    step = SemStep(lsa, torch, wl, inp, cache)
    step.make_events((steps + EVENTS_EVERY - 1) // EVENTS_EVERY)
    for _ in range(warmup):
        step.run(record=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(record=(i % EVENTS_EVERY == 0))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    return inp, step, ms, cluster


def prefill_object(lsa, torch, name, steps, warmup, with_cpu):
    """One flat prefill configuration: throughput, the indexer scan's int8 MFMA roofline,
    the step against T_roof, prefill attention's bf16 utilisation beside its gather rate,
    and the oracle on a sample of its rows."""
    import synthetic
    wl = synthetic.WORKLOADS[name]
    inp, step, ms = measure(lsa, torch, wl, steps, warmup)
    km = step.kernel_ms()
    alg = algorithmic(wl)
    tr = t_roof_ms(wl)
    obj = {"workload": _describe(wl), "value": wl.B * wl.n_q / (ms * 1e-3), "unit": "queries/s", "ms_per_step": ms,
           "kernel_ms": km, "t_roof_ms": tr, "step_roofline_frac": tr / ms, "roofline": None}
    stage = "index_select" if "index_select" in km else "index_scores"
    scan_ms = km[stage]["ms_per_step"]
    if wl.L > 4096:  # the tiny case is launch-bound: its time is reported, not a roofline
        ach = alg["index_ops"] / (scan_ms * 1e-3) / 1e12
        obj["roofline"] = {"bound": "mfma", "kernel": f"{stage} (flat indexer scan, idx_flat_kernel)",
                           "achieved": ach, "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": ach / INT8_PEAK_TOPS,
                           "frac_of_measured_peak": None,
                           "counter_mfma_busy": counter_mfma_busy(wl.name, stage),
                           "algorithmic_ops_per_step": alg["index_ops"], "launch_ms_per_step": scan_ms}
    obj["attention"] = attention_object(alg, km["sparse_attn"]["ms_per_step"], wl)
    if with_cpu:
        obj["cpu_baseline"] = cpu_baseline(wl, inp)
    del inp, step
    torch.cuda.empty_cache()
    return obj


def measure(lsa, torch, wl, steps, warmup):
    import synthetic
    inp = synthetic.make_inputs(wl, torch.device("cuda:0"))
    if wl.pooled:
        # the block-key cache is kept with the caches (a serving loop updates one block per
        # block_size tokens), so it is built before the timed steps
        inp["block_keys"] = lsa.lsa_block_cache(inp["k_idx"], wl.block_size, page_table=inp.get("page_table"),
                                                page_size=wl.page_size)
    torch.cuda.synchronize()
    step = Step(lsa, torch, wl, inp)
    step.make_events((steps + EVENTS_EVERY - 1) // EVENTS_EVERY)
    for _ in range(warmup):
        step.run(record=False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step.run(record=(i % EVENTS_EVERY == 0))
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    return inp, step, ms


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None, help="time only this workload (no headline line)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--peaks", action="store_true", help="only measure the machine's ceilings")
    ap.add_argument("--no-peaks", action="store_true", help="skip the ceilings in the default run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); sharding the path "
              "across GPUs is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    import learned_top_sparse_amd as lsa
    import synthetic
    lsa.lib()
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.peaks:
        print(json.dumps({"measured_peaks": measure_peaks(lsa, torch)}), flush=True)
        return

    if args.workload:
        names = list(synthetic.WORKLOADS) if args.workload == "all" else [args.workload]
        for name in names:
            wl = synthetic.WORKLOADS[name]
            if wl.semantic:
                inp, step, ms, cluster = measure_sem(lsa, torch, wl, args.steps, args.warmup)
                print(json.dumps({"workload": wl.name, "ms_per_step": ms, "stage_events_every": EVENTS_EVERY,
                                  "kernel_ms": step.kernel_ms(), "cluster": cluster,
                                  "algorithmic": sem_algorithmic(wl)}), flush=True)
                del inp, step
                torch.cuda.empty_cache()
                continue
            inp, step, ms = measure(lsa, torch, wl, args.steps, args.warmup)
            print(json.dumps({"workload": wl.name, "ms_per_step": ms, "stage_events_every": EVENTS_EVERY,
                              "kernel_ms": step.kernel_ms(),
                              "algorithmic": algorithmic(wl)}), flush=True)
            del inp, step
            torch.cuda.empty_cache()
        return

    # The machine's ceilings are measured after every workload: their probes (a 6.7 TB/s
    # stream, dense MFMA loops) leave the chip in a state that slowed a decode step timed
    # right after them by about 3 % (242.6-244.8 against 236.6-236.8 us on one box).

    # ---- headline: decode at 128K
    wl = synthetic.WORKLOADS["decode_128k"]
    inp, step, ms = measure(lsa, torch, wl, args.steps, args.warmup)
    kms = step.kernel_ms()
    alg = algorithmic(wl)
    tok_s = wl.B * wl.n_q / (ms * 1e-3)
    idx_stage = "index_select" if "index_select" in kms else "index_scores"
    idx_ms = kms[idx_stage]["ms_per_launch"]
    launches = kms[idx_stage]["launches_per_step"]
    achieved = alg["index_bytes"] / launches / (idx_ms * 1e-3) / 1e9
    roof_t_ms = t_roof_ms(wl)
    res = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "stage_events_every": EVENTS_EVERY,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8+bf16",
        "data": "synthetic",
        "config": {"workload": _describe(wl), "global_batch": wl.B, "seq_len": wl.L, "parallelism": "none"},
        "roofline": {
            "bound": "hbm", "kernel": f"{idx_stage} (decode scan, idx_decode_kernel)",
            "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "frac_of_measured_peak": None,
            "algorithmic_bytes_per_launch": alg["index_bytes"] / launches, "launch_ms": idx_ms,
        },
        "kernel_ms": kms,
        "t_roof_ms": roof_t_ms,
        "step_roofline_frac": roof_t_ms / ms,
        "decode_attn": {
            "achieved_GBs": alg["attn_gather_bytes"] / (kms["sparse_attn"]["ms_per_step"] * 1e-3) / 1e9,
            "frac_hbm": alg["attn_gather_bytes"] / (kms["sparse_attn"]["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "frac_of_measured_cold_gather": None,
            "gather_bytes": alg["attn_gather_bytes"],
        },
        "measured_peaks": None,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inp)
    del inp, step
    torch.cuda.empty_cache()

    # ---- the same decode step over paged caches
    wpg = synthetic.WORKLOADS["decode_128k_paged"]
    inp, step, ms_g = measure(lsa, torch, wpg, args.steps, args.warmup)
    res["decode_128k_paged"] = {
        "workload": _describe(wpg), "value": wpg.B * wpg.n_q / (ms_g * 1e-3), "unit": "tok/s",
        "ms_per_step": ms_g, "kernel_ms": step.kernel_ms(),
    }
    del inp, step
    torch.cuda.empty_cache()

    # ---- decode at 128K with the pooled (4:1) indexer, block-key cache resident
    wpo = synthetic.WORKLOADS["decode_128k_pool4"]
    inp, step, ms_o = measure(lsa, torch, wpo, args.steps, args.warmup)
    ko = step.kernel_ms()
    ao = algorithmic(wpo)
    res["decode_128k_pool4"] = {
        "workload": _describe(wpo), "value": wpo.B * wpo.n_q / (ms_o * 1e-3), "unit": "tok/s",
        "ms_per_step": ms_o, "kernel_ms": ko,
        "block_scan": {
            "bound": "hbm", "kernel": "block_prefilter (blk_decode_kernel + blk_keep_merge_kernel)",
            "bytes_per_step": ao["block_bytes"],
            "achieved_GBs": ao["block_bytes"] / (ko["block_prefilter"]["ms_per_step"] * 1e-3) / 1e9,
        },
    }
    del inp, step
    torch.cuda.empty_cache()

    # ---- the pooled (4:1) indexer on the prefill configurations (block-key cache resident)
    for name in ("prefill_32k_pool4", "chunk_256k_pool4"):
        wx = synthetic.WORKLOADS[name]
        inp, step, ms_x = measure(lsa, torch, wx, args.steps if wx.L <= 32768 else max(1, args.steps // 5),
                                  args.warmup)
        kx = step.kernel_ms()
        ax = algorithmic(wx)
        ach = ax["block_ops"] / (kx["block_prefilter"]["ms_per_step"] * 1e-3) / 1e12
        res[name] = {
            "workload": _describe(wx), "value": wx.B * wx.n_q / (ms_x * 1e-3), "unit": "queries/s",
            "ms_per_step": ms_x, "kernel_ms": kx, "t_roof_ms": t_roof_ms(wx),
            "step_roofline_frac": t_roof_ms(wx) / ms_x,
            "roofline": {"bound": "mfma",
                         "kernel": "block_prefilter (blk_scores_kernel and the block keep: the score table and "
                                   "blk_select_long_kernel for rows up to 16384 blocks; a sampled threshold, the "
                                   "thresholded scan and blk_list_keep_kernel above)",
                         "achieved": ach, "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": ach / INT8_PEAK_TOPS,
                         "frac_of_measured_peak": None,
                         "counter_mfma_busy": counter_mfma_busy(name, "block_prefilter"),
                         "ops": "pooled-key scores, two int8 parts per block key"},
        }
        del inp, step
        torch.cuda.empty_cache()

    # ---- the block modes over paged caches (pools of 64-token pages, seeded page order)
    for name, unit in (("decode_128k_pool4_paged", "tok/s"), ("two_stage_128k_paged", "queries/s")):
        wx = synthetic.WORKLOADS[name]
        inp, step, ms_x = measure(lsa, torch, wx, args.steps, args.warmup)
        res[name] = {"workload": _describe(wx), "value": wx.B * wx.n_q / (ms_x * 1e-3), "unit": unit,
                     "ms_per_step": ms_x, "kernel_ms": step.kernel_ms()}
        del inp, step
        torch.cuda.empty_cache()

    # ---- prefill at 128K (two-stage chunk)
    wp = synthetic.WORKLOADS["two_stage_128k"]
    inp, step, ms_p = measure(lsa, torch, wp, args.steps, args.warmup)
    kp = step.kernel_ms()
    ap_ = algorithmic(wp)
    # With few enough kept slots the token stage scores and selects in one kernel
    # ("index_select"); otherwise it writes a score table ("index_scores") for the top-k.
    ts_stage = "index_select" if "index_select" in kp else "index_scores"
    ts_desc = ("index_select (token-stage scores in kept blocks + exact top-k, one kernel)"
               if ts_stage == "index_select" else "index_scores (token stage in kept blocks)")
    ach_p = ap_["index_ops"] / (kp[ts_stage]["ms_per_step"] * 1e-3) / 1e12
    at_p = kp["sparse_attn"]["ms_per_step"]
    res["prefill_128k"] = {
        "workload": _describe(wp),
        "value": wp.n_q / (ms_p * 1e-3), "unit": "queries/s", "ms_per_step": ms_p,
        "kernel_ms": kp,
        "roofline": {
            "bound": "mfma", "kernel": ts_desc,
            "achieved": ach_p, "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": ach_p / INT8_PEAK_TOPS,
            "frac_of_measured_peak": None,
            "counter_mfma_busy": counter_mfma_busy(wp.name, ts_stage),
        },
        "t_roof_ms": t_roof_ms(wp),
        "step_roofline_frac": t_roof_ms(wp) / ms_p,
        "attention": attention_object(ap_, at_p, wp),
    }
    if not args.no_cpu_baseline:
        res["prefill_128k"]["cpu_baseline"] = cpu_baseline(wp, inp, budget_s=10.0)
    del inp, step
    torch.cuda.empty_cache()

    # ---- the flat prefill configurations: tiny (parity size), 32K from position 0, and
    # one GPU's 16384-query chunk of a 256K context
    for name in ("tiny_prefill_1k", "prefill_32k", "chunk_256k"):
        res[name] = prefill_object(lsa, torch, name, args.steps if name != "chunk_256k" else max(1, args.steps // 5),
                                   args.warmup, not args.no_cpu_baseline)

    # ---- the pages' own method: flat semantic search at 128K, decode and a prefill chunk
    for name, unit in (("decode_128k_lsa", "tok/s"), ("decode_128k_lsa_paged", "tok/s"),
                       ("prefill_128k_lsa", "queries/s"), ("decode_1m_lsa", "tok/s")):
        ws_ = synthetic.WORKLOADS[name]
        inp, step, ms_s, cluster = measure_sem(lsa, torch, ws_, args.steps, args.warmup)
        res[name] = {
            "workload": _describe_sem(ws_), "value": ws_.B * ws_.n_q / (ms_s * 1e-3), "unit": unit,
            "ms_per_step": ms_s, "kernel_ms": step.kernel_ms(), "cluster": cluster,
            "algorithmic": sem_algorithmic(ws_),
        }
        if name == "decode_128k_lsa":
            km = res[name]["kernel_ms"]
            alg_b = res[name]["algorithmic"]["centroid_bytes"]
            ach = alg_b / (km["centroid_scan"]["ms_per_step"] * 1e-3) / 1e9
            res[name]["roofline"] = {"bound": "hbm", "kernel": "centroid scan (sem_score_decode_kernel)",
                                     "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": ach / HBM_PEAK_GBS, "traffic": sem_measured_traffic(),
                                     "algorithmic_bytes_per_launch": alg_b}
            if not args.no_cpu_baseline:
                res[name]["cpu_baseline"] = cpu_baseline_sem(ws_, inp)
        del inp, step
        torch.cuda.empty_cache()
    if not args.no_peaks:
        fill_measured_fractions(res, measure_peaks(lsa, torch))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
