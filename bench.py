#!/usr/bin/env python3
"""Benchmark of the indexer hot path on one MI355X.

A step is one call of the hot path over one batch of synthetic input that is
already resident in HBM. The timed steps are captured once into a HIP graph and
replayed, so the GPU runs them back to back; the host-launched (eager) time per
call is reported beside it. By default the workload is the variable-length decode
batch (B=4 requests, 4 bf16 query heads, 128 dims, 8192-block padded tables,
seq_len 4096..131072 tokens at 16 tokens per block, K=256) through the fused
idx_select. The timed steps rotate over enough copies of the inputs (over
512 MiB) that every step reads its centroids from HBM, not from L2 or the
256 MiB last-level cache.

Prints one JSON line:
  value         valid blocks scored + selected per second (whole job, 1 GPU)
  ms_per_step   HIP-event time per step over the timed region
  roofline      the dominant kernel: algorithmic bytes (or flops) per launch /
                average launch time, against the MI355X peak
  cpu_baseline  the CPU oracle on the host cores, on a bounded sample
  steady_us_per_call    median / min over five replays of the timed graph
  cold_us_per_call      32 single calls, each after a 1 GiB overwrite that evicts
                        L2 and the last-level cache (HIP events around the call)
  host_e2e_us_per_call  host wall clock of one call plus a stream synchronise
  sorted_us_per_call    the score-ordered output (workloads 2-4 headline the
                        id-ordered one)
  floor                 an empty launch and a streaming read of the same bytes
                        (alone, and followed by one arrival counter) on this GPU

Other modes:
  --workload N         1..7 (1: tiny fp32, 2: default, 3: top-K stress,
                       4: large GQA batch, 5: k-means assignment, 6: paged pool,
                       7: prompt tokens, 8: pooled keys)
  --pmc-calibrate      also run a plain 1 GiB device copy (for byte counters)
  --parse-pmc DIR      turn rocprofv3 --pmc output into a traffic summary
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "blocks scored+selected/sec and µs per indexer call; % of MI355X HBM peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
ROTATE_BYTES = 512 << 20
CALIB_BYTES = 1 << 30

KERNEL = {1: "select_fused_kernel", 2: "select_fused_kernel", 3: "topk_split_kernel",
          4: "select_fused_kernel", 5: "assign_kernel", 6: "select_fused_kernel",
          7: "topk_kernel", 8: "pool_keys_kernel"}
SOURCES = ["block_scoring_top_amd/csrc/" + f for f in
           ("common.hpp", "score.hpp", "select.hpp", "indexer.hip", "assign.hip", "prefill.hip",
            "pool.hip", "api.cpp")]


def source_digest() -> str:
    h = hashlib.sha256()
    for s in SOURCES:
        with open(os.path.join(ROOT, s), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(a):
    """numpy -> torch on cuda:0; bf16 bit patterns (uint16) become bfloat16 tensors."""
    import numpy as np
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(
            torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


# ----------------------------------------------------------------------------------------
# workloads: device inputs, one step, algorithmic bytes
# ----------------------------------------------------------------------------------------
class Indexer:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        q, c, sl = to_dev(x.q), to_dev(x.c), to_dev(x.seq_len)
        self.inputs = [(q, c, sl)] + [(q.clone(), c.clone(), sl.clone()) for _ in range(copies - 1)]
        dev = q.device
        self.ids = torch.empty(x.B, x.K, dtype=torch.int32, device=dev)
        self.counts = torch.empty(x.B, dtype=torch.int32, device=dev)
        nbytes = idx.idx_workspace_bytes(x.B, x.N_pad, x.H, x.K, 0)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        # blocks holding tokens: ceil(seq_len / page_size), at most N_pad
        self.nv = [min(x.N_pad, -(-int(v) // x.page_size)) for v in x.seq_len]
        elem = 2 if x.dtype == "bf16" else 4
        self.units = int(sum(self.nv))
        self.row_bytes = x.D * elem
        # centroid rows that hold tokens + query heads + seq_len + ids written
        self.alg_bytes = (self.units * self.row_bytes + x.q.size * elem + 4 * x.B + 4 * x.B * x.K)
        self.alg_flops = 2 * self.units * x.D  # after summing the heads once per request

    def step(self, i, sorted=None):
        q, c, sl = self.inputs[i % len(self.inputs)]
        self.idx.idx_select(q, c, sl, self.x.K, page_size=self.x.page_size,
                            sorted=self.x.sorted if sorted is None else sorted,
                            ids=self.ids, counts=self.counts, ws=self.ws)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][1]

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select", "B": x.B, "H": x.H, "D": x.D,
                "N_pad": x.N_pad, "page_size": x.page_size, "K": x.K, "sorted": x.sorted,
                "inputs": x.dtype, "accumulate": "f32", "seq_len": [int(v) for v in x.seq_len]
                if x.B <= 8 else f"{int(x.seq_len.min())}..{int(x.seq_len.max())}",
                "valid_blocks": self.units, "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import oracle
        x = self.x
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            S, _ = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
            oracle.select(S, self.nv, x.K, x.sorted)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return self.units / med, f"the whole batch ({self.units} valid blocks), {len(times)} " \
                                 f"calls, median {med * 1e3:.1f} ms per call"


class Paged:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        q, c = to_dev(x.q), to_dev(x.c_pool)
        ip, ix = to_dev(x.indptr), to_dev(x.indices)
        self.inputs = [(q, c, ip, ix)] + [(q.clone(), c.clone(), ip.clone(), ix.clone())
                                          for _ in range(copies - 1)]
        dev = q.device
        self.ids = torch.empty(x.B, x.K, dtype=torch.int32, device=dev)
        self.counts = torch.empty(x.B, dtype=torch.int32, device=dev)
        nbytes = idx.idx_workspace_bytes(x.B, x.max_pages, x.H, x.K, 0)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        import numpy as np
        n = np.minimum(np.diff(x.indptr.astype(np.int64)), x.max_pages)
        self.nv = [int(v) for v in n]
        self.units = int(n.sum())                      # page slots scored
        elem = 2 if x.dtype == "bf16" else 4
        unique_rows = int(np.unique(x.indices).size)   # pool rows the lists name
        # pool rows named (each read from HBM at least once) + the page lists +
        # query heads + ids written
        self.alg_bytes = (unique_rows * 128 * elem + 4 * x.indices.size + 4 * (x.B + 1)
                          + x.q.size * elem + 4 * x.B * x.K)
        self.alg_flops = 2 * self.units * 128

    def step(self, i, sorted=None):
        q, c, ip, ix = self.inputs[i % len(self.inputs)]
        self.idx.idx_select_paged(q, c, ip, ix, self.x.K, self.x.max_pages,
                                  sorted=self.x.sorted if sorted is None else sorted,
                                  ids=self.ids, counts=self.counts, ws=self.ws)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][1]

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select_paged", "B": x.B, "H": x.H, "D": 128,
                "pool_rows": int(x.c_pool.shape[0]), "max_pages": x.max_pages,
                "page_slots": self.units, "K": x.K, "sorted": x.sorted, "inputs": x.dtype,
                "accumulate": "f32", "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import oracle
        x = self.x
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            S, _, n = oracle.score_paged(x.q, x.c_pool, x.indptr, x.indices, x.max_pages, x.dtype)
            oracle.select(S, n, x.K, x.sorted)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return self.units / med, f"the whole batch ({self.units} page slots), {len(times)} " \
                                 f"calls, median {med * 1e3:.1f} ms per call"


class Prefill:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        q, c, p0 = to_dev(x.q), to_dev(x.c), to_dev(x.pos0)
        self.inputs = [(q, c, p0)] + [(q.clone(), c.clone(), p0.clone()) for _ in range(copies - 1)]
        dev = q.device
        self.ids = torch.empty(x.B, x.T, x.K, dtype=torch.int32, device=dev)
        self.counts = torch.empty(x.B, x.T, dtype=torch.int32, device=dev)
        self.ws = torch.empty(idx.idx_prefill_workspace_bytes(x.B, x.T, x.N_pad, x.K, 0),
                              dtype=torch.uint8, device=dev)
        import numpy as np
        ps = x.page_size
        nv = [np.minimum(x.N_pad, (max(int(p), 0) + np.arange(x.T) + 1 + ps - 1) // ps)
              for p in x.pos0]
        self.units = int(sum(int(v.sum()) for v in nv))        # (token, visible block) pairs
        rows = sum(int(v.max()) for v in nv)                    # centroid rows any token sees
        # centroid rows read + query heads + pos0 + ids written (the per-token
        # score rows are an intermediate and are not credited)
        self.alg_bytes = rows * 256 + x.q.size * 2 + 4 * x.B + 4 * x.B * x.T * x.K
        self.alg_flops = 2 * self.units * 128

    def step(self, i, sorted=None):
        q, c, p0 = self.inputs[i % len(self.inputs)]
        self.idx.idx_select_prefill(q, c, p0, self.x.K, page_size=self.x.page_size,
                                    sorted=self.x.sorted if sorted is None else sorted,
                                    ids=self.ids, counts=self.counts, ws=self.ws)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][1]

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select_prefill", "B": x.B, "T": x.T, "H": x.H,
                "D": 128, "N_pad": x.N_pad, "pos0": [int(v) for v in x.pos0],
                "page_size": x.page_size, "K": x.K, "sorted": x.sorted, "inputs": x.dtype,
                "accumulate": "f32 (MFMA)", "token_block_pairs": self.units,
                "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import oracle
        x = self.x
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            S, _, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
            R = x.B * x.T
            oracle.select(S.reshape(R, -1), NV.reshape(R), x.K, x.sorted)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return self.units / med, f"the whole batch ({self.units} token-block pairs), " \
                                 f"{len(times)} calls, median {med * 1e3:.1f} ms per call"


class Pool:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        k, sl = to_dev(x.k), to_dev(x.seq_len)
        self.inputs = [(k, sl)] + [(k.clone(), sl.clone()) for _ in range(copies - 1)]
        self.c = torch.zeros(x.B, x.N_pad, 128, dtype=k.dtype, device=k.device)
        import numpy as np
        S_pad = x.k.shape[1]
        sl_np = np.clip(x.seq_len.astype(np.int64), 0, S_pad)
        nv = np.minimum(x.N_pad, (sl_np + x.page_size - 1) // x.page_size)
        tokens = int(np.minimum(sl_np, nv * x.page_size).sum())
        elem = 2 if x.dtype == "bf16" else 4
        self.units = int(nv.sum())                               # blocks pooled
        # keys of the tokens held + one centroid row per block + seq_len
        self.alg_bytes = tokens * 128 * elem + self.units * 128 * elem + 4 * x.B
        self.alg_flops = tokens * 128

    def step(self, i, sorted=None):
        k, sl = self.inputs[i % len(self.inputs)]
        self.idx.idx_pool_keys(k, sl, self.x.N_pad, self.x.page_size, c=self.c)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][0]

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_pool_keys", "B": x.B, "S_pad": int(x.k.shape[1]),
                "D": 128, "N_pad": x.N_pad, "page_size": x.page_size, "inputs": x.dtype,
                "seq_len": [int(v) for v in x.seq_len], "blocks": self.units,
                "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import oracle
        x = self.x
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            oracle.pool_keys(x.k, x.seq_len, x.N_pad, x.page_size, x.dtype)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return self.units / med, f"the whole batch ({self.units} blocks), {len(times)} calls, " \
                                 f"median {med * 1e3:.1f} ms per call"


class Topk:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        s = to_dev(x.scores)
        self.inputs = [s] + [s.clone() for _ in range(copies - 1)]
        B, N = x.scores.shape
        self.ids = torch.empty(B, x.K, dtype=torch.int32, device=s.device)
        self.counts = torch.empty(B, dtype=torch.int32, device=s.device)
        self.units = B * N
        self.alg_bytes = B * N * 4 + B * x.K * 4
        self.alg_flops = 0

    def step(self, i, sorted=None):
        self.idx.idx_topk(self.inputs[i % len(self.inputs)], self.x.K, None, bool(sorted),
                          ids=self.ids, counts=self.counts)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)]

    def describe(self):
        B, N = self.x.scores.shape
        return {"workload": self.x.name, "call": "idx_topk", "rows": B, "N": N, "K": self.x.K,
                "sorted": False, "inputs": "f32", "distributions": 9,
                "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import oracle
        x = self.x
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            oracle.select(x.scores, None, x.K, False)
            times.append(time.perf_counter() - t0)
        med = statistics.median(times)
        return self.units / med, f"all {x.scores.shape[0]} rows, {len(times)} calls, " \
                                 f"median {med * 1e3:.1f} ms per call"


class Assign:
    def __init__(self, x, torch, idx, copies):
        self.x, self.torch, self.idx = x, torch, idx
        xd, cd = to_dev(x.x), to_dev(x.c)
        self.inputs = [(xd, cd)] + [(xd.clone(), cd.clone()) for _ in range(copies - 1)]
        N, D = x.x.shape
        C = x.c.shape[0]
        self.assign = torch.empty(N, dtype=torch.int32, device=xd.device)
        self.ws = torch.zeros(idx.idx_assign_workspace_bytes(C, D), dtype=torch.uint8,
                              device=xd.device)
        self.units = N
        self.alg_bytes = N * D * 2 + C * D * 2 + N * 4
        self.alg_flops = 2 * N * C * D

    def step(self, i, sorted=None):
        xd, cd = self.inputs[i % len(self.inputs)]
        self.idx.idx_assign(xd, cd, assign=self.assign, ws=self.ws)

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][0]

    def describe(self):
        N, D = self.x.x.shape
        return {"workload": self.x.name, "call": "idx_assign", "N": N, "C": self.x.c.shape[0],
                "D": D, "inputs": "bf16", "accumulate": "f32 (MFMA)",
                "input_copies": len(self.inputs)}

    def cpu_oracle(self, budget_s):
        import numpy as np
        import oracle
        x = self.x
        n = 2048
        times = []
        t_end = time.perf_counter() + budget_s
        i = 0
        while time.perf_counter() < t_end or len(times) < 3:
            rows = slice((i * n) % x.x.shape[0], (i * n) % x.x.shape[0] + n)
            t0 = time.perf_counter()
            oracle.assign(x.x[rows], x.c)
            times.append(time.perf_counter() - t0)
            i += 1
        med = statistics.median(times)
        return n / med, f"{n} of the {x.x.shape[0]} points per call, {len(times)} calls, " \
                        f"median {med * 1e3:.1f} ms per call"


def make(w, torch, idx, copies):
    import synth
    x = synth.workload(w)
    if w in (1, 2, 4):
        return Indexer(x, torch, idx, copies)
    if w == 3:
        return Topk(x, torch, idx, copies)
    if w == 6:
        return Paged(x, torch, idx, copies)
    if w == 7:
        return Prefill(x, torch, idx, copies)
    if w == 8:
        return Pool(x, torch, idx, copies)
    return Assign(x, torch, idx, copies)


def input_bytes(w, x):
    if w in (1, 2, 4):
        return x.q.nbytes + x.c.nbytes
    if w == 3:
        return x.scores.nbytes
    if w == 6:
        return x.q.nbytes + x.c_pool.nbytes + x.indptr.nbytes + x.indices.nbytes
    if w == 7:
        return x.q.nbytes + x.c.nbytes
    if w == 8:
        return x.k.nbytes
    return x.x.nbytes + x.c.nbytes


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


# ----------------------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------------------
def graph_time(torch, fn, steps, reps=1):
    """Capture `steps` calls fn(i) into one HIP graph; per-call ms of each of `reps`
    replays (HIP events on the replaying stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / steps)
    del g
    return out


def floors(torch, idx, wl, steps):
    """Attainable floor at this size: an empty launch, and a streaming read of the
    call's algorithmic bytes (rotating over the input copies, so from HBM), alone
    and followed by one arrival counter; the read takes the best of a small sweep
    of launch shapes."""
    src0 = wl.read_src(0)
    nbytes = min(wl.alg_bytes, src0.numel() * src0.element_size()) // 16 * 16
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    ticket = torch.zeros(64, dtype=torch.int32, device="cuda")
    res = {"bytes": nbytes,
           "empty_us": min(graph_time(torch, lambda i: idx.idx_floor_empty(1), steps, 3)) * 1e3}
    for key, tk in (("read", None), ("read_handoff", ticket)):
        best = None
        for threads in (256, 1024):
            for blocks in (64, 128, 256, 512, 1024, 2048):
                t = min(graph_time(torch, lambda i: idx.idx_floor_read(
                    wl.read_src(i), nbytes, sink, tk, blocks, threads), steps, 3)) * 1e3
                if best is None or t < best[0]:
                    best = (t, blocks, threads)
        res[key + "_us"] = best[0]
        res[key + "_launch"] = f"{best[1]} x {best[2]}"
    res["read_GBps"] = nbytes / (res["read_us"] * 1e-6) / 1e9
    return res


def cold_times(torch, wl, n):
    """Per-call GPU time with L2 and the last-level cache flushed before each call
    (a 1 GiB buffer is overwritten first)."""
    flush = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
    out = []
    for i in range(n):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        wl.step(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del flush
    return out


def host_e2e_times(torch, wl, n):
    """Wall clock of one host call plus a stream synchronise."""
    out = []
    for i in range(n):
        t0 = time.perf_counter()
        wl.step(i)
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3)
    return out


def stats_us(ms_list):
    return {"median": statistics.median(ms_list) * 1e3, "min": min(ms_list) * 1e3,
            "n": len(ms_list)}


# ----------------------------------------------------------------------------------------
# rocprofv3 --pmc output -> traffic summary
# ----------------------------------------------------------------------------------------
def parse_pmc(dirs, out_path, workload):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the benchmarked kernel, scaled
    by what the same counter reads for the 1 GiB calibration copy."""
    import csv
    rows = []
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += list(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {dirs}")
    per = {}  # (counter, kernel) -> {dispatch: value summed over counter instances}
    for r in rows:
        name = r.get("Kernel_Name", "")
        ctr = r.get("Counter_Name", "")
        val = float(r.get("Counter_Value", 0))
        disp = r.get("Dispatch_Id", "")
        per.setdefault((ctr, name), {}).setdefault(disp, 0.0)
        per[(ctr, name)][disp] += val
    kern = KERNEL[workload]

    def values(ctr, match):
        return [v for (c, n), d in per.items() if c == ctr and match(n) for v in d.values()]

    def avg(ctr, match):
        vals = values(ctr, match)
        return (sum(vals) / len(vals), len(vals)) if vals else (None, 0)

    def calib(ctr):
        # the 1 GiB copy is the largest copy dispatch of the run
        vals = values(ctr, lambda n: "copy" in n.lower() and kern not in n)
        return (max(vals), 1) if vals else (None, 0)

    is_kern = lambda n: kern in n
    res = {"kernel": kern, "workload": workload, "source_sha256": source_digest()}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        k, nk = avg(ctr, is_kern)
        cal, nc = calib(ctr)
        if k is None:
            continue
        res[ctr + "_kib_per_dispatch"] = k
        res[ctr + "_dispatches"] = nk
        if cal:
            scale = CALIB_BYTES / (cal * 1024.0)
            res[ctr + "_calib_scale"] = scale
            res[ctr.split("_")[0].lower() + "_bytes_per_launch"] = k * 1024.0 * scale
    with open(out_path, "w") as f:
        f.write(f"# HBM traffic of {kern} (workload {workload}) from rocprofv3 --pmc\n")
        f.write("# byte counters scaled by (1 GiB) / (counter for a plain 1 GiB device copy)\n")
        f.write("# commands (run from /tmp, repository at /root/repo):\n")
        for ctr, d in zip(("FETCH_SIZE", "WRITE_SIZE"), dirs):
            f.write(f"#   rocprofv3 --pmc {ctr} --output-format csv -d /root/repo/{d} -o pmc -- "
                    f"python3 /root/repo/bench.py --workload {workload} --steps 20 --warmup 5 "
                    "--no-cpu-baseline --no-graph --no-extras --pmc-calibrate\n")
        f.write(f"#   python3 bench.py --workload {workload} --parse-pmc {' '.join(dirs)}\n")
        for k_, v in res.items():
            f.write(f"{k_}={v}\n")
    print(json.dumps(res))


def read_traffic(workload):
    p = os.path.join(ROOT, "profiles", f"traffic_w{workload}_{KERNEL[workload]}.txt")
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k] = v
    if kv.get("source_sha256") != source_digest():
        return None  # the kernel changed since the counters were taken
    try:
        return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])
    except KeyError:
        return None


# ----------------------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="time host-launched steps instead of a replayed HIP graph")
    ap.add_argument("--pmc-calibrate", action="store_true")
    ap.add_argument("--parse-pmc", nargs="+", default=None)
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the floor, cold, host end-to-end and sorted measurements")
    ap.add_argument("--out", default=None)
    a = ap.parse_args()

    if a.parse_pmc:
        out = a.out or os.path.join(ROOT, "profiles",
                                    f"traffic_w{a.workload}_{KERNEL[a.workload]}.txt")
        parse_pmc(a.parse_pmc, out, a.workload)
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}); the indexer's "
              "requests, rows and points are independent, so a multi-GPU run is G copies of "
              "this one on disjoint slices", file=sys.stderr)
        return 2

    import torch
    import block_scoring_top_amd as idx
    idx.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    import synth
    x0 = synth.workload(a.workload)
    copies = max(1, min(256, -(-ROTATE_BYTES // input_bytes(a.workload, x0))))
    del x0
    log(f"[bench] workload {a.workload}: building inputs ({copies} copies)")
    wl = make(a.workload, torch, idx, copies)

    if a.pmc_calibrate:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # eager: one host call per step (Python binding -> C ABI -> launch)
    for i in range(a.warmup):
        wl.step(i)
    torch.cuda.synchronize()
    n_eager = min(a.steps, 500)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(n_eager):
        wl.step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / n_eager

    # timed region: the K steps captured once into a HIP graph and replayed, so
    # the GPU runs the steps back to back without waiting on the host
    graph = None
    if not a.no_graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                wl.step(i)
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(a.steps):
                wl.step(a.warmup + i)
        graph.replay()  # untimed warm replay
        torch.cuda.synchronize()
    log(f"[bench] warmup {a.warmup} done; timing {a.steps} steps "
        f"({'graph replay' if graph else 'eager'})")
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(a.steps):
            wl.step(a.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = ev0.elapsed_time(ev1) / a.steps
    log(f"[bench] {ms * 1e3:.2f} us per step (events), {wall / a.steps * 1e6:.2f} us wall, "
        f"eager {eager_ms * 1e3:.2f} us per step")

    launch_desc = "eager" if graph is None else f"hipGraph of {a.steps} steps"
    extras = {}
    if not a.no_extras:
        # the same graph replayed again: spread of the steady-state figure
        if graph is not None:
            reps = []
            for _ in range(4):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                graph.replay()
                e1.record()
                torch.cuda.synchronize()
                reps.append(e0.elapsed_time(e1) / a.steps)
            extras["steady_us_per_call"] = stats_us([ms] + reps)
        graph = None
        log("[bench] cold calls, host end-to-end, floors")
        extras["cold_us_per_call"] = stats_us(cold_times(torch, wl, 32))
        extras["host_e2e_us_per_call"] = stats_us(host_e2e_times(torch, wl, 32))
        if a.workload in (2, 3, 4, 6, 7):  # headline unsorted; the score-ordered output beside it
            extras["sorted_us_per_call"] = min(graph_time(
                torch, lambda i: wl.step(i, sorted=True), min(a.steps, 1000), 3)) * 1e3
        extras["floor"] = floors(torch, idx, wl, min(a.steps, 200))
        log(f"[bench] floors: {json.dumps(extras['floor'])}")

    per_s = 1e3 / ms
    if a.workload == 5:
        bound, unit = "mfma", "TFLOP/s"
        achieved = wl.alg_flops / (ms * 1e-3) / 1e12
        peak = MFMA_BF16_PEAK_TFLOPS
    else:
        bound, unit = "hbm", "GB/s"
        achieved = wl.alg_bytes / (ms * 1e-3) / 1e9
        peak = HBM_PEAK_GBS
    traffic = read_traffic(a.workload)
    out = {
        "metric": METRIC,
        "value": wl.units * per_s,
        "unit": {5: "points/s", 3: "entries/s", 6: "page slots/s",
                 7: "token-block pairs/s", 8: "blocks pooled/s"}.get(a.workload, "blocks/s"),
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "us_per_call": ms * 1e3, "eager_us_per_call": eager_ms * 1e3,
        "launch": launch_desc,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": wl.describe(),
        "roofline": {"bound": bound, "kernel": KERNEL[a.workload], "achieved": achieved,
                     "peak": peak, "unit": unit, "frac": achieved / peak, "traffic": traffic,
                     "alg_bytes_per_launch": wl.alg_bytes, "alg_flops_per_launch": wl.alg_flops},
    }
    if a.workload == 5:
        out["roofline"]["hbm_frac"] = wl.alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    out.update(extras)
    if not a.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle (~{a.cpu_seconds:.0f} s)")
        v, sample = wl.cpu_oracle(a.cpu_seconds)
        out["cpu_baseline"] = {"value": v, "unit": out["unit"], "cores": blas_threads(),
                               "kind": "oracle", "sample": sample}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
