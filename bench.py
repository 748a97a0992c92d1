#!/usr/bin/env python3
"""Benchmark of the indexer hot path on one MI355X.

A step is one call of the hot path over one batch of synthetic input that is
already resident in HBM. By default one run measures the five named workloads:

  1  tiny fp32 indexer: B=1, H=4, 1024 blocks, K=256, score order   (idx_select)
  2  variable-length decode batch: B=4, H=4, bf16, N_pad=8192, K=256 (idx_select)
  3  top-K stress: 64 rows x 30000 fp32, nine distributions, K=2048  (idx_topk)
  4  large GQA decode batch: B=128, H=16, bf16, N_pad=2048, K=256     (idx_select)
  5  k-means assignment: 2^20 bf16 points x 1024 centroids, D=128     (idx_assign)
  9  the top-K stress rows of workload 3 rounded to bf16               (idx_topk_bf16)
 10  clustered rows: 64 x 8000, tight cluster + wide outliers, K=1024 (idx_topk)

The headline line is workload 4, the largest single-GPU indexer batch; the
others are reported under "workloads", each with its own roofline.

How a workload is timed ("hbm_cold"):
  - the inputs are replicated into enough copies that the bytes a call really
    reads (its algorithmic bytes, not the padded allocation) add up to at least
    twice the 256 MiB last-level cache between two reads of the same copy;
  - the timed steps (step i reads copy i mod copies) are captured once into a
    HIP graph; the graph is replayed untimed for at least 20 ms (clocks ramp
    up after the host's pauses);
  - then a 1 GiB streaming read evicts L2 and the last-level cache (a read, so
    that no dirty lines are left whose write-back would be charged to the call);
  - then the graph is replayed between HIP events on the replaying stream, with
    a synchronise on each side: every step reads its inputs from HBM, and the
    GPU runs the steps back to back without host launch gaps;
  - the outputs of the timed steps are then checked against the CPU oracle (the
    cpu_baseline leg); a mismatch makes the run exit non-zero.

Beside it, per workload: steady_us_per_call (the same graph replayed again
without a flush), isolated_call_us (one call after a flush, HIP events around
that call alone; isolated_empty_us is an empty launch timed the same way, the
events' own overhead), host_e2e_us_per_call (host wall clock of one call plus a
synchronise), sorted_us_per_call (score-ordered output where the headline is
id-ordered), plan_host_e2e_us and plan_graph_host_e2e_us (the same through a
resolved plan, and through a one-call graph of it), radix8_us_per_call (the
same steps with IDX_RADIX8: four 8-bit radix passes and no linear-bin pass,
timed like the headline; radix8_same_outputs must hold, or the run fails), and
floor (an empty launch, and a streaming read of the call's algorithmic bytes,
alone and followed by one cross-workgroup arrival counter, timed like the
call).

Other modes:
  --workload N         one workload only (1..10; 6: paged pool, 7: prompt tokens,
                       8: pooled keys), printed as the headline
  --pmc-calibrate      also run a plain 1 GiB device copy (for byte counters)
  --parse-pmc DIR...   turn rocprofv3 --pmc output into a traffic summary
  --parse-trace DIR    per-workload kernel statistics of the timed regions from a
                       rocprofv3 --kernel-trace run of this script (the regions
                       are bracketed by empty marker launches)
  --paged-sweep        idx_select_paged over the five page-count regimes x five
                       batch sizes of the centroid-scorer sweep: steady and
                       cold-isolated time per cell, ids checked (one JSON line)
  --decode-shapes      idx_select on the decode shapes the pages time (one request,
                       4 fp32 heads, 751 / 2049 / 7501 blocks of 4 tokens, K = 256)
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
LLC_BYTES = 256 << 20           # MI355X last-level cache (Infinity Cache)
ROTATE_BYTES = 2 * LLC_BYTES    # distinct bytes read between two reads of one copy
FLUSH_BYTES = 1 << 30
CALIB_BYTES = 1 << 30
HEADLINE = 4
DEFAULT_SET = (1, 2, 3, 4, 5, 9, 10)
# empty launches with these workgroup counts bracket a workload's timed region
MARK_BEGIN, MARK_END = 1000, 2000
RADIX8_MARK = 50   # marker offset of a workload's IDX_RADIX8 region

KERNEL = {1: "select_fused_kernel", 2: "select_fused_kernel", 3: "topk_split_kernel",
          4: "select_fused_kernel", 5: "assign_kernel", 6: "select_fused_kernel",
          7: "topk_kernel", 8: "pool_keys_kernel", 9: "topk_split_kernel", 10: "topk_kernel"}
SOURCES = ["block_scoring_top_amd/csrc/" + f for f in
           ("common.hpp", "score.hpp", "select.hpp", "indexer_kernels.hpp", "indexer.hip",
            "indexer_radix8.hip", "assign.hip", "prefill.hip", "pool.hip", "api.cpp")]


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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [p["num_threads"] for p in threadpool_info() if p.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:
        return 1


# ----------------------------------------------------------------------------------------
# workloads: device inputs (copy 0, replicated later), one step, algorithmic bytes, the
# outputs of the timed steps, and the oracle side (cpu_baseline leg only)
# ----------------------------------------------------------------------------------------
class Workload:
    unit = "blocks/s"
    sorted_variant = False      # headline id-ordered, score order reported beside it
    radix8_variant = False      # the select with four 8-bit radix passes timed beside it
    dtype = "f32"

    def replicate(self, copies):
        self.inputs += [tuple(t.clone() for t in self.inputs[0]) for _ in range(copies - 1)]

    def read_src(self, i):
        return self.inputs[i % len(self.inputs)][self.read_index]

    def poison_outputs(self):
        for t in self.out_tensors():
            t.fill_(-1515870811)  # 0xa5a5a5a5

    def timed_outputs(self):
        return [t.cpu().numpy() for t in self.out_tensors()]

    def oracle_time(self, budget_s):
        times = []
        t_end = time.perf_counter() + budget_s
        while time.perf_counter() < t_end or len(times) < 3:
            t0 = time.perf_counter()
            self.oracle_call(len(times))
            times.append(time.perf_counter() - t0)
        return statistics.median(times), len(times)


class Indexer(Workload):
    read_index = 1

    def __init__(self, x, torch, idx):
        self.x, self.torch, self.idx = x, torch, idx
        self.dtype = x.dtype
        self.inputs = [(to_dev(x.q), to_dev(x.c), to_dev(x.seq_len))]
        self.sorted_variant = not x.sorted
        self.radix8_variant = True
        self.ids = torch.empty(x.B, x.K, dtype=torch.int32, device="cuda")
        self.counts = torch.empty(x.B, dtype=torch.int32, device="cuda")
        nbytes = idx.idx_workspace_bytes(x.B, x.N_pad, x.H, x.K, 0)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        # blocks holding tokens: ceil(seq_len / page_size), at most N_pad
        self.nv = [min(x.N_pad, -(-int(v) // x.page_size)) for v in x.seq_len]
        elem = 2 if x.dtype == "bf16" else 4
        self.units = int(sum(self.nv))
        # centroid rows that hold tokens + query heads + seq_len + ids written
        self.alg_bytes = self.units * x.D * elem + x.q.size * elem + 4 * x.B + 4 * x.B * x.K
        self.alg_flops = 2 * self.units * x.D  # after summing the heads once per request

    def step(self, i, sorted=None, radix8=False):
        q, c, sl = self.inputs[i % len(self.inputs)]
        self.idx.idx_select(q, c, sl, self.x.K, page_size=self.x.page_size,
                            sorted=self.x.sorted if sorted is None else sorted,
                            ids=self.ids, counts=self.counts, ws=self.ws, radix8=radix8)

    def out_tensors(self):
        return [self.ids, self.counts]

    def plan_e2e(self, n):
        """Host end-to-end of one call through a plan (idx_plan_select), and of
        one replay of a graph holding one plan call, each plus a synchronise."""
        torch, x = self.torch, self.x
        dt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
        plan = self.idx.plan_for(x.B, x.H, x.N_pad, x.K, dt, x.page_size, x.sorted)
        q, c, sl = self.inputs[0]
        g = plan.capture(q, c, sl, self.ids, self.counts)
        out = {}
        for key, fn in (("plan_host_e2e_us", lambda: plan(q, c, sl, self.ids, self.counts)),
                        ("plan_graph_host_e2e_us", g.replay)):
            fn()
            torch.cuda.synchronize()
            ts = []
            for _ in range(n):
                t0 = time.perf_counter()
                fn()
                torch.cuda.synchronize()
                ts.append((time.perf_counter() - t0) * 1e3)
            out[key] = stats_us(ts)
        del g
        return out

    def gpu_scores(self):
        """One more call that also writes the scores: the GPU's own fp32 scores
        (the ids are not taken from it)."""
        q, c, sl = self.inputs[0]
        _, _, s = self.idx.idx_select(q, c, sl, self.x.K, page_size=self.x.page_size,
                                      sorted=self.x.sorted, return_scores=True)
        self.torch.cuda.synchronize()
        return s.cpu().numpy()

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select", "B": x.B, "H": x.H, "D": x.D,
                "N_pad": x.N_pad, "page_size": x.page_size, "K": x.K, "sorted": x.sorted,
                "inputs": x.dtype, "accumulate": "f32", "seq_len": [int(v) for v in x.seq_len]
                if x.B <= 8 else f"{int(x.seq_len.min())}..{int(x.seq_len.max())}",
                "valid_blocks": self.units}

    def oracle_call(self, i):
        import oracle
        x = self.x
        S, _ = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
        oracle.select(S, self.nv, x.K, x.sorted)

    def sample_text(self, med, n):
        return f"the whole batch ({self.units} valid blocks), {n} calls, median " \
               f"{med * 1e3:.1f} ms per call"

    def parity(self, outs, gpu_scores):
        """C1: the timed ids are the oracle's selection from the GPU's scores;
        C2: those scores within rtol * A of fp64; C3: the ids against the fp64
        selection, inside the band."""
        import oracle
        from tests.helpers import RTOL, check_ids_band, check_ids_exact, check_scores
        x = self.x
        ids, counts = outs
        S, A = oracle.score(x.q, x.c, x.seq_len, x.page_size, x.dtype)
        nv = oracle.n_valid(x.seq_len, x.page_size, x.N_pad)
        rel = check_scores(gpu_scores, S, A, RTOL[x.dtype])
        check_ids_exact(ids, counts, gpu_scores, nv, x.K, x.sorted)
        check_ids_band(ids, S, A, nv, x.K, RTOL[x.dtype])
        return {"C1_ids_exact": True, "C2_max_err_over_A": rel, "C3_band": True,
                "rows": int(x.B)}


class Topk(Workload):
    unit = "entries/s"
    read_index = 0
    sorted_variant = True

    def __init__(self, x, torch, idx):
        import numpy as np
        self.x, self.torch, self.idx = x, torch, idx
        self.bf16 = x.scores.dtype == np.uint16   # bf16 rows go to idx_topk_bf16
        self.dtype = "bf16" if self.bf16 else "f32"
        self.radix8_variant = not self.bf16
        self.inputs = [(to_dev(x.scores),)]
        B, N = x.scores.shape
        self.ids = torch.empty(B, x.K, dtype=torch.int32, device="cuda")
        self.counts = torch.empty(B, dtype=torch.int32, device="cuda")
        self.ws = torch.zeros(max(256, idx.idx_topk_workspace_bytes(B, N, x.K, 1)),
                              dtype=torch.uint8, device="cuda")
        self.units = B * N
        self.alg_bytes = B * N * (2 if self.bf16 else 4) + B * x.K * 4
        self.alg_flops = 0

    def step(self, i, sorted=None, radix8=False):
        self.idx.idx_topk(self.inputs[i % len(self.inputs)][0], self.x.K, None, bool(sorted),
                          ids=self.ids, counts=self.counts, ws=self.ws, radix8=radix8)

    def out_tensors(self):
        return [self.ids, self.counts]

    def gpu_scores(self):
        return None

    def describe(self):
        B, N = self.x.scores.shape
        return {"workload": self.x.name, "call": "idx_topk_bf16" if self.bf16 else "idx_topk",
                "rows": B, "N": N, "K": self.x.K, "sorted": False, "inputs": self.dtype,
                "distributions": sorted(set(self.x.dists))}

    def values(self):
        import oracle
        return oracle.bf16_decode(self.x.scores) if self.bf16 else self.x.scores

    def oracle_call(self, i):
        import oracle
        oracle.select(self.values(), None, self.x.K, False)

    def sample_text(self, med, n):
        return f"all {self.x.scores.shape[0]} rows, {n} calls, median {med * 1e3:.1f} ms per call"

    def parity(self, outs, gpu_scores):
        """C1 directly: the input scores are the GPU's own."""
        from tests.helpers import check_ids_exact
        ids, counts = outs
        check_ids_exact(ids, counts, self.values(), None, self.x.K, False)
        return {"C1_ids_exact": True, "rows": int(self.x.scores.shape[0])}


class Assign(Workload):
    unit = "points/s"
    read_index = 0
    dtype = "bf16"
    SAMPLE = 2048         # points per oracle call of the CPU baseline
    PARITY_ROWS = 8192    # sampled points checked against the oracle

    def __init__(self, x, torch, idx):
        self.x, self.torch, self.idx = x, torch, idx
        self.inputs = [(to_dev(x.x), to_dev(x.c))]
        N, D = x.x.shape
        C = x.c.shape[0]
        self.assign = torch.empty(N, dtype=torch.int32, device="cuda")
        self.ws = torch.zeros(idx.idx_assign_workspace_bytes(C, D), dtype=torch.uint8,
                              device="cuda")
        self.units = N
        self.alg_bytes = N * D * 2 + C * D * 2 + N * 4
        self.alg_flops = 2 * N * C * D

    def step(self, i, sorted=None):
        xd, cd = self.inputs[i % len(self.inputs)]
        self.idx.idx_assign(xd, cd, assign=self.assign, ws=self.ws)

    def out_tensors(self):
        return [self.assign]

    def gpu_scores(self):
        return None

    def describe(self):
        N, D = self.x.x.shape
        return {"workload": self.x.name, "call": "idx_assign", "N": N, "C": self.x.c.shape[0],
                "D": D, "inputs": "bf16", "accumulate": "f32 (MFMA)"}

    def mfma_floor_shape(self):
        """The assignment kernel's grid (256 points per workgroup) and its products
        per wave (32 per tile of 64 centroids), as rounds of four."""
        N, C = self.x.x.shape[0], self.x.c.shape[0]
        return -(-N // 256), -(-C // 64) * 8

    def oracle_call(self, i):
        import oracle
        n, N = self.SAMPLE, self.x.x.shape[0]
        lo = (i * n) % N
        oracle.assign(self.x.x[lo:lo + n], self.x.c)

    def sample_text(self, med, n):
        return f"{self.SAMPLE} of the {self.x.x.shape[0]} points per call, {n} calls, " \
               f"median {med * 1e3:.1f} ms per call"

    def oracle_units(self):
        return self.SAMPLE

    def parity(self, outs, gpu_scores):
        """Every point's generating component is its nearest centroid (holds at any
        size); sampled points against the oracle's argmax, inside the band."""
        import numpy as np
        from tests.helpers import check_assign
        (a,) = outs
        np.testing.assert_array_equal(a, self.x.comp)
        rng = np.random.default_rng(5)
        N = self.x.x.shape[0]
        rows = np.concatenate([np.arange(64), rng.choice(N, self.PARITY_ROWS, replace=False),
                               np.arange(N - 64, N)])
        off = check_assign(a, None, self.x.x, self.x.c, rows)
        return {"components_recovered": int(N), "sampled_points": int(rows.size),
                "differ_inside_band": int(off)}


class Paged(Workload):
    unit = "page slots/s"
    read_index = 1

    def __init__(self, x, torch, idx):
        import numpy as np
        self.x, self.torch, self.idx = x, torch, idx
        self.dtype = x.dtype
        self.inputs = [(to_dev(x.q), to_dev(x.c_pool), to_dev(x.indptr), to_dev(x.indices))]
        self.sorted_variant = not x.sorted
        self.ids = torch.empty(x.B, x.K, dtype=torch.int32, device="cuda")
        self.counts = torch.empty(x.B, dtype=torch.int32, device="cuda")
        nbytes = idx.idx_workspace_bytes(x.B, x.max_pages, x.H, x.K, 0)
        self.ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
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

    def out_tensors(self):
        return [self.ids, self.counts]

    def gpu_scores(self):
        q, c, ip, ix = self.inputs[0]
        _, _, s = self.idx.idx_select_paged(q, c, ip, ix, self.x.K, self.x.max_pages,
                                            sorted=self.x.sorted, return_scores=True)
        self.torch.cuda.synchronize()
        return s.cpu().numpy()

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select_paged", "B": x.B, "H": x.H, "D": 128,
                "pool_rows": int(x.c_pool.shape[0]), "max_pages": x.max_pages,
                "page_slots": self.units, "K": x.K, "sorted": x.sorted, "inputs": x.dtype,
                "accumulate": "f32"}

    def oracle_call(self, i):
        import oracle
        x = self.x
        S, _, n = oracle.score_paged(x.q, x.c_pool, x.indptr, x.indices, x.max_pages, x.dtype)
        oracle.select(S, n, x.K, x.sorted)

    def sample_text(self, med, n):
        return f"the whole batch ({self.units} page slots), {n} calls, median " \
               f"{med * 1e3:.1f} ms per call"

    def parity(self, outs, gpu_scores):
        import oracle
        from tests.helpers import RTOL, check_ids_band, check_ids_exact, check_scores
        x = self.x
        ids, counts = outs
        S, A, n = oracle.score_paged(x.q, x.c_pool, x.indptr, x.indices, x.max_pages, x.dtype)
        rel = check_scores(gpu_scores, S, A, RTOL[x.dtype])
        check_ids_exact(ids, counts, gpu_scores, n, x.K, x.sorted)
        check_ids_band(ids, S, A, n, x.K, RTOL[x.dtype])
        return {"C1_ids_exact": True, "C2_max_err_over_A": rel, "C3_band": True}


class Prefill(Workload):
    unit = "token-block pairs/s"
    read_index = 1

    def __init__(self, x, torch, idx):
        import numpy as np
        self.x, self.torch, self.idx = x, torch, idx
        self.dtype = x.dtype
        self.inputs = [(to_dev(x.q), to_dev(x.c), to_dev(x.pos0))]
        self.sorted_variant = not x.sorted
        self.ids = torch.empty(x.B, x.T, x.K, dtype=torch.int32, device="cuda")
        self.counts = torch.empty(x.B, x.T, dtype=torch.int32, device="cuda")
        self.ws = torch.zeros(idx.idx_prefill_workspace_bytes(x.B, x.T, x.N_pad, x.K, 0),
                              dtype=torch.uint8, device="cuda")
        ps = x.page_size
        nv = [np.minimum(x.N_pad, (max(int(p), 0) + np.arange(x.T) + 1 + ps - 1) // ps)
              for p in x.pos0]
        self.units = int(sum(int(v.sum()) for v in nv))        # (token, visible block) pairs
        rows = sum(int(v.max()) for v in nv)                    # centroid rows any token sees
        # centroid rows read + query heads + pos0 + ids written (the per-token
        # score rows are an intermediate and are not credited)
        esz = 4 if x.dtype == "f32" else 2
        self.alg_bytes = rows * 128 * esz + x.q.size * esz + 4 * x.B + 4 * x.B * x.T * x.K
        self.alg_flops = 2 * self.units * 128

    def step(self, i, sorted=None):
        q, c, p0 = self.inputs[i % len(self.inputs)]
        self.idx.idx_select_prefill(q, c, p0, self.x.K, page_size=self.x.page_size,
                                    sorted=self.x.sorted if sorted is None else sorted,
                                    ids=self.ids, counts=self.counts, ws=self.ws)

    def out_tensors(self):
        return [self.ids, self.counts]

    def gpu_scores(self):
        q, c, p0 = self.inputs[0]
        _, _, s = self.idx.idx_select_prefill(q, c, p0, self.x.K, page_size=self.x.page_size,
                                              sorted=self.x.sorted, return_scores=True)
        self.torch.cuda.synchronize()
        return s.cpu().numpy()

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_select_prefill", "B": x.B, "T": x.T, "H": x.H,
                "D": 128, "N_pad": x.N_pad, "pos0": [int(v) for v in x.pos0],
                "page_size": x.page_size, "K": x.K, "sorted": x.sorted, "inputs": x.dtype,
                "accumulate": "f32" if self.fused_route() else "f32 (MFMA)",
                "token_block_pairs": self.units}

    def fused_route(self):
        """Calls of at most 8 tokens and 256 token rows: one fused select."""
        x = self.x
        return x.T <= 8 and x.B * x.T <= 256 and x.B * x.T * x.N_pad < 2 ** 31

    def oracle_call(self, i):
        import oracle
        x = self.x
        S, _, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
        R = x.B * x.T
        oracle.select(S.reshape(R, -1), NV.reshape(R), x.K, x.sorted)

    def sample_text(self, med, n):
        return f"the whole batch ({self.units} token-block pairs), {n} calls, median " \
               f"{med * 1e3:.1f} ms per call"

    def parity(self, outs, gpu_scores):
        import oracle
        from tests.helpers import RTOL, check_ids_band, check_ids_exact, check_scores
        x = self.x
        ids, counts = outs
        R = x.B * x.T
        S, A, NV = oracle.score_prefill(x.q, x.c, x.pos0, x.page_size, x.dtype)
        s = gpu_scores.reshape(R, -1)
        rel = check_scores(s, S.reshape(R, -1), A.reshape(R, -1), RTOL[x.dtype])
        check_ids_exact(ids.reshape(R, -1), counts.reshape(R), s, NV.reshape(R), x.K, x.sorted)
        check_ids_band(ids.reshape(R, -1), S.reshape(R, -1), A.reshape(R, -1), NV.reshape(R),
                       x.K, RTOL[x.dtype])
        return {"C1_ids_exact": True, "C2_max_err_over_A": rel, "C3_band": True}


class Pool(Workload):
    unit = "blocks pooled/s"
    read_index = 0

    def __init__(self, x, torch, idx):
        import numpy as np
        self.x, self.torch, self.idx = x, torch, idx
        self.dtype = x.dtype
        self.inputs = [(to_dev(x.k), to_dev(x.seq_len))]
        self.c = torch.zeros(x.B, x.N_pad, 128, dtype=self.inputs[0][0].dtype, device="cuda")
        S_pad = x.k.shape[1]
        sl_np = np.clip(x.seq_len.astype(np.int64), 0, S_pad)
        nv = np.minimum(x.N_pad, (sl_np + x.page_size - 1) // x.page_size)
        self.nv = nv
        tokens = int(np.minimum(sl_np, nv * x.page_size).sum())
        elem = 2 if x.dtype == "bf16" else 4
        self.units = int(nv.sum())                               # blocks pooled
        # keys of the tokens held + one centroid row per block + seq_len
        self.alg_bytes = tokens * 128 * elem + self.units * 128 * elem + 4 * x.B
        self.alg_flops = tokens * 128

    def step(self, i, sorted=None):
        k, sl = self.inputs[i % len(self.inputs)]
        self.idx.idx_pool_keys(k, sl, self.x.N_pad, self.x.page_size, c=self.c)

    def out_tensors(self):
        return []

    def poison_outputs(self):
        self.c.fill_(float("nan"))

    def timed_outputs(self):
        import numpy as np
        return [self.c.view(self.torch.int16).cpu().numpy().view(np.uint16)]

    def gpu_scores(self):
        return None

    def describe(self):
        x = self.x
        return {"workload": x.name, "call": "idx_pool_keys", "B": x.B, "S_pad": int(x.k.shape[1]),
                "D": 128, "N_pad": x.N_pad, "page_size": x.page_size, "inputs": x.dtype,
                "seq_len": [int(v) for v in x.seq_len], "blocks": self.units}

    def oracle_call(self, i):
        import oracle
        oracle.pool_keys(self.x.k, self.x.seq_len, self.x.N_pad, self.x.page_size, self.x.dtype)

    def sample_text(self, med, n):
        return f"the whole batch ({self.units} blocks), {n} calls, median {med * 1e3:.1f} ms " \
               "per call"

    def parity(self, outs, gpu_scores):
        """Every pooled value within the fp32-sum bound plus the bf16 output
        rounding of the fp64 mean."""
        import numpy as np
        import oracle
        import synth
        (bits,) = outs
        got = synth.bf16_bits_to_f32(bits).astype(np.float64)
        C, M, nv = oracle.pool_keys(self.x.k, self.x.seq_len, self.x.N_pad, self.x.page_size,
                                    self.x.dtype)
        for b in range(self.x.B):
            m = int(nv[b])
            err = np.abs(got[b, :m] - C[b, :m])
            tol = 2.0 ** -8 * np.abs(C[b, :m]) + 2.0 ** -17 * M[b, :m]
            assert not (err > tol).any(), f"request {b}: pooled values out of tolerance"
        return {"blocks_in_tolerance": int(self.units)}


def make(w, torch, idx):
    import synth
    x = synth.workload(w)
    cls = {1: Indexer, 2: Indexer, 3: Topk, 4: Indexer, 5: Assign, 6: Paged, 7: Prefill,
           8: Pool, 9: Topk, 10: Topk}[w]
    wl = cls(x, torch, idx)
    wl.w = w
    return wl


# ----------------------------------------------------------------------------------------
# timing
# ----------------------------------------------------------------------------------------
class Flusher:
    """Evicts L2 and the last-level cache with a 1 GiB streaming read (the
    library's floor read launch: reads only, so no dirty lines are left)."""

    def __init__(self, torch, idx):
        self.torch, self.idx = torch, idx
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda")
        self.sink = torch.empty(65536, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.idx.idx_floor_read(self.buf, FLUSH_BYTES, self.sink, None, 2048, 256)


def capture(torch, fn, steps, warm=3):
    """Capture `steps` calls fn(i) into one HIP graph (after a few eager calls on
    the capturing stream, so that nothing is first touched inside the capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(warm):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(steps):
            fn(i)
    return g


def replay_ms(torch, g, steps, flush=None, mark=None, idx=None):
    """Per-step ms of one replay of g, HIP events on the replaying stream, with a
    synchronise on each side; optionally after a flush, and bracketed by marker
    launches that a kernel trace can find."""
    stream = torch.cuda.current_stream()
    if flush is not None:
        flush()
    if mark is not None:
        idx.idx_floor_empty(MARK_BEGIN + mark)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    if mark is not None:
        idx.idx_floor_empty(MARK_END + mark)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def isolated_ms(torch, fn, flush, n):
    """One call after a flush, HIP events around that call alone."""
    out = []
    for i in range(n):
        flush()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn(i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def host_e2e_ms(torch, fn, n):
    """Wall clock of one host call plus a stream synchronise."""
    out = []
    for i in range(n):
        t0 = time.perf_counter()
        fn(i)
        torch.cuda.synchronize()
        out.append((time.perf_counter() - t0) * 1e3)
    return out


def stats_us(ms_list):
    return {"median": statistics.median(ms_list) * 1e3, "min": min(ms_list) * 1e3,
            "n": len(ms_list)}


def floors(torch, idx, wl, steps, flush):
    """Attainable floor at this size, timed like the call: an empty launch, and a
    streaming read of the call's algorithmic bytes over the same rotating copies
    after a flush, alone and followed by one arrival counter; the read takes the
    best of a small sweep of launch shapes."""
    src0 = wl.read_src(0)
    nbytes = min(wl.alg_bytes, src0.numel() * src0.element_size()) // 16 * 16
    sink = torch.empty(65536, dtype=torch.float32, device="cuda")
    ticket = torch.zeros(64, dtype=torch.int32, device="cuda")
    g = capture(torch, lambda i: idx.idx_floor_empty(1), steps)
    g.replay()
    res = {"bytes": nbytes, "empty_us": min(replay_ms(torch, g, steps) for _ in range(3)) * 1e3}
    del g
    for key, tk in (("read", None), ("read_handoff", ticket)):
        best = None
        for threads in (256, 1024):
            for blocks in (128, 256, 512, 1024, 2048):
                g = capture(torch, lambda i: idx.idx_floor_read(
                    wl.read_src(i), nbytes, sink, tk, blocks, threads), steps)
                g.replay()
                t = replay_ms(torch, g, steps, flush) * 1e3
                del g
                if best is None or t < best[0]:
                    best = (t, blocks, threads)
        res[key + "_us"] = best[0]
        res[key + "_launch"] = f"{best[1]} x {best[2]}"
    res["read_GBps"] = nbytes / (res["read_us"] * 1e-6) / 1e9
    if hasattr(wl, "mfma_floor_shape"):
        # the same number of bf16 products as the call, on the same grid, with
        # register operands: the matrix rate the chip sustains at its clock under
        # load (the operand data sets the power draw and so the clock)
        import numpy as np
        from synth import f32_to_bf16_bits
        blocks, iters = wl.mfma_floor_shape()
        msink = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
        # operands like the call's: normal values in bf16 (the rate depends on the data)
        frags = to_dev(f32_to_bf16_bits(np.random.default_rng(55).standard_normal(8192)
                                        .astype(np.float32)))
        g = capture(torch, lambda i: idx.idx_floor_mfma(frags, blocks, iters, msink), steps)
        g.replay()
        t = min(replay_ms(torch, g, steps) for _ in range(3))
        del g
        flops = 2 * 32 * 32 * 16 * 4 * iters * 4 * blocks
        res["mfma_us"] = t * 1e3
        res["mfma_launch"] = f"{blocks} x 256, {4 * iters} products per wave"
        res["mfma_TFLOPs"] = flops / (t * 1e-3) / 1e12
    return res


def roofline(wl, ms, traffic, floor=None):
    if wl.w == 5:
        achieved = wl.alg_flops / (ms * 1e-3) / 1e12
        r = {"bound": "mfma", "kernel": KERNEL[wl.w], "achieved": achieved,
             "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
             "frac": achieved / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic,
             "alg_flops_per_launch": wl.alg_flops, "alg_bytes_per_launch": wl.alg_bytes,
             "hbm_frac": wl.alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if floor and "mfma_TFLOPs" in floor:
            # context, not the peak: back-to-back products on register operands
            r["sustained_mfma_TFLOPs"] = floor["mfma_TFLOPs"]
            r["frac_of_sustained"] = achieved / floor["mfma_TFLOPs"]
    else:
        achieved = wl.alg_bytes / (ms * 1e-3) / 1e9
        r = {"bound": "hbm", "kernel": KERNEL[wl.w], "achieved": achieved,
             "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
             "traffic": traffic, "alg_bytes_per_launch": wl.alg_bytes}
    return r


def measure(torch, idx, wl, steps, warmup, extras, flush):
    """Time one workload as the module docstring describes; returns its result
    dict (without the oracle side) and the host copies of the timed outputs."""
    import math
    copies = max(1, math.ceil(ROTATE_BYTES / wl.alg_bytes) + 1)
    if steps is None:  # a workload beside the headline: every copy read, at least 32 steps
        steps = max(copies, 32)
    copies = min(copies, steps)
    wl.replicate(copies)
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    g = capture(torch, wl.step, steps)
    # untimed: first touch of code, page tables and every copy, then replays for
    # at least 20 ms so that the GPU clocks have ramped up after the host's pause
    t_end = time.perf_counter() + 0.02
    while True:
        g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            break
    wl.poison_outputs()
    ms = replay_ms(torch, g, steps, flush, mark=wl.w, idx=idx)
    outs = wl.timed_outputs()
    distinct = min(copies, steps) * wl.alg_bytes
    log(f"[bench] w{wl.w}: {ms * 1e3:.2f} us per call over {steps} steps "
        f"({copies} input copies, {distinct / 2**20:.0f} MiB of distinct reads)")
    res = {"us_per_call": ms * 1e3, "ms_per_step": ms, "steps": steps,
           "value": wl.units / (ms * 1e-3), "unit": wl.unit,
           "timing": "hbm_cold", "input_copies": copies,
           "distinct_read_bytes": distinct, "config": wl.describe()}
    if extras:
        res["steady_us_per_call"] = stats_us([replay_ms(torch, g, steps) for _ in range(3)])
        del g
        res["isolated_call_us"] = stats_us(isolated_ms(torch, wl.step, flush, 16))
        res["isolated_empty_us"] = stats_us(isolated_ms(
            torch, lambda i: idx.idx_floor_empty(1), flush, 8))
        res["host_e2e_us_per_call"] = stats_us(host_e2e_ms(torch, wl.step, 16))
        if hasattr(wl, "plan_e2e"):
            res.update(wl.plan_e2e(16))
        if wl.sorted_variant:
            gs = capture(torch, lambda i: wl.step(i, sorted=True), steps)
            gs.replay()
            res["sorted_us_per_call"] = replay_ms(torch, gs, steps, flush) * 1e3
            del gs
        if wl.radix8_variant:
            # the same steps with four 8-bit radix passes (IDX_RADIX8): timed the
            # same way, in a marked region, and its outputs must equal the
            # headline's (which the CPU leg checks against the oracle)
            import numpy as np
            gr = capture(torch, lambda i: wl.step(i, radix8=True), steps)
            gr.replay()
            torch.cuda.synchronize()
            wl.poison_outputs()
            res["radix8_us_per_call"] = replay_ms(torch, gr, steps, flush, mark=RADIX8_MARK + wl.w,
                                                  idx=idx) * 1e3
            res["radix8_same_outputs"] = all(
                np.array_equal(a, b) for a, b in zip(wl.timed_outputs(), outs))
            del gr
            log(f"[bench] w{wl.w} radix8: {res['radix8_us_per_call']:.2f} us per call, outputs "
                f"{'equal' if res['radix8_same_outputs'] else 'DIFFERENT'}")
        res["floor"] = floors(torch, idx, wl, steps, flush)
        log(f"[bench] w{wl.w} floors: read {res['floor']['read_us']:.2f} us, read + hand-off "
            f"{res['floor']['read_handoff_us']:.2f} us, empty {res['floor']['empty_us']:.2f} us")
        if "mfma_us" in res["floor"]:
            log(f"[bench] w{wl.w} floor: the call's products on register operands "
                f"{res['floor']['mfma_us']:.1f} us, {res['floor']['mfma_TFLOPs']:.0f} TFLOP/s")
    else:
        del g
    res["roofline"] = roofline(wl, ms, read_traffic(wl.w), res.get("floor"))
    return res, outs


def cpu_baseline_leg(wl, outs, gpu_scores, seconds):
    """The CPU oracle beside the GPU: checks the timed outputs against it (the
    run fails on a mismatch), then times it on a bounded sample."""
    parity = {"ok": True}
    try:
        parity.update(wl.parity(outs, gpu_scores))
    except AssertionError as e:
        parity = {"ok": False, "error": str(e)[:400]}
    med, n = wl.oracle_time(seconds)
    units = wl.oracle_units() if hasattr(wl, "oracle_units") else wl.units
    base = {"value": units / med, "unit": wl.unit, "cores": blas_threads(), "kind": "oracle",
            "sample": wl.sample_text(med, n) + "; numpy fp64 (BLAS threads for the products, "
                      "the selection on one thread)", "cpu_model": cpu_model()}
    return parity, base


# ----------------------------------------------------------------------------------------
# rocprofv3 output -> summaries
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
                    "--no-cpu-baseline --no-extras --pmc-calibrate\n")
        f.write(f"#   python3 bench.py --workload {workload} --parse-pmc {' '.join(dirs)}\n")
        for k_, v in res.items():
            f.write(f"{k_}={v}\n")
    print(json.dumps(res))


def parse_trace(d, out_path, command):
    """Kernel statistics of each workload's timed region in a rocprofv3 kernel
    trace of this script: the dispatches between the region's two marker
    launches, grouped by kernel name."""
    import csv
    files = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))

    def grid_wgs(r):
        gx = int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
        wx = int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 1)) or 1)
        return gx // max(wx, 1)

    regions = {}
    open_w = None
    for r in rows:
        name = r["Kernel_Name"]
        if "floor_empty_kernel" in name:
            n = grid_wgs(r)
            if MARK_BEGIN < n < MARK_BEGIN + 100:
                open_w = n - MARK_BEGIN
                regions[open_w] = []
                continue
            if MARK_END < n < MARK_END + 100:
                open_w = None
                continue
        if open_w is not None:
            regions[open_w].append(r)
    lines = [f"# Kernels of each workload's timed region (rocprofv3 kernel trace)", "",
             "Command (run from /tmp on one MI355X, repository at /root/repo):", "", "```",
             command, f"python3 bench.py --parse-trace {d}", "```", "",
             "| workload | kernel | dispatches | average (us) | min (us) | max (us) |",
             "|---|---|---|---|---|---|"]
    for w in sorted(regions):
        label = f"{w - RADIX8_MARK} (IDX_RADIX8)" if w > RADIX8_MARK else str(w)
        per = {}
        for r in regions[w]:
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per.setdefault(r["Kernel_Name"].split("(")[0], []).append(dur)
        for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"| {label} | `{k}` | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} "
                         f"| {max(v):.2f} |")
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


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
def paged_sweep(torch, idx, flush, steps=20):
    """idx_select_paged over the scorer sweep of the centroid pages: five
    page-count regimes x five batch sizes over one pool of 16384 rows, H = 4,
    K = 256, bf16. Per cell: the steady per-call time (a graph of `steps` calls
    on the same inputs, replayed; the pool stays cached, as it would across a
    serving loop's calls) and one isolated call after the 1 GiB flush; ids
    checked against the oracle's selection from the GPU's scores."""
    import numpy as np
    import synth
    from tests.helpers import check_ids_exact
    cells = []
    for r, regime in enumerate(synth.PAGE_REGIMES):
        for B in synth.PAGED_BATCHES:
            x = synth.make_paged(B, 4, 128, synth.POOL_BLOCKS, regime, 256, "bf16",
                                 600 + 10 * r + B, name=f"sweep_r{r}_b{B}")
            wl = Paged(x, torch, idx)
            g = capture(torch, wl.step, steps)
            g.replay()
            steady = min(replay_ms(torch, g, steps) for _ in range(3)) * 1e3
            del g
            iso = statistics.median(isolated_ms(torch, wl.step, flush, 8)) * 1e3
            wl.poison_outputs()
            wl.step(0)
            torch.cuda.synchronize()
            ids, counts = wl.timed_outputs()
            check_ids_exact(ids, counts, wl.gpu_scores(), np.asarray(wl.nv), x.K, x.sorted)
            cells.append({"regime": f"N({regime[0]},{regime[1]})", "B": B,
                          "page_slots": wl.units, "steady_us": steady,
                          "isolated_cold_us": iso,
                          "page_slots_per_s": wl.units / (steady * 1e-6)})
            log(f"[sweep] N{regime} B={B}: {wl.units} slots, steady {steady:.2f} us, "
                f"isolated cold {iso:.2f} us")
    return cells


def decode_shapes(torch, idx, flush, steps=20):
    """idx_select on the decode shapes the pages time their Metal score + top-K
    kernels at ("Round 18 Track C", section 3: pos0 3000, 8192 and 30000, one
    query token): one request, 4 fp32 heads of 128 dims, 4-token blocks, so
    751, 2049 and 7501 blocks; K = 256 (the pages do not state K; the tiny
    fp32 configuration's). Steady and cold-isolated time, both output orders,
    ids checked against the oracle's selection from the GPU's scores."""
    import numpy as np
    import synth
    from tests.helpers import check_ids_exact
    cells = []
    for pos0 in (3000, 8192, 30000):
        n_pad = -(-(pos0 + 1) // 4)
        for srt in (False, True):
            x = synth.make_indexer(1, 4, 128, n_pad, [pos0 + 1], 256, "f32", pos0 + int(srt),
                                   sorted_out=srt, page_size=4, name=f"decode_pos{pos0}")
            wl = Indexer(x, torch, idx)
            g = capture(torch, wl.step, steps)
            g.replay()
            steady = min(replay_ms(torch, g, steps) for _ in range(3)) * 1e3
            del g
            iso = statistics.median(isolated_ms(torch, wl.step, flush, 8)) * 1e3
            wl.poison_outputs()
            wl.step(0)
            torch.cuda.synchronize()
            ids, counts = wl.timed_outputs()
            check_ids_exact(ids, counts, wl.gpu_scores(), np.asarray(wl.nv), x.K, srt)
            cells.append({"pos0": pos0, "blocks": n_pad, "sorted": srt, "steady_us": steady,
                          "isolated_cold_us": iso})
            log(f"[decode] pos0={pos0} ({n_pad} blocks) sorted={srt}: steady {steady:.2f} us, "
                f"isolated cold {iso:.2f} us")
        # two and four query tokens (the page's ntok) and eight (the most one
        # fused launch takes): idx_select_prefill, fp32 like the page's
        for ntok in (2, 4, 8):
            n_pad = -(-(pos0 + ntok) // 4)
            x = synth.make_prefill(1, ntok, 4, 128, n_pad, [pos0], 256, pos0 + ntok, dtype="f32",
                                   page_size=4, name=f"prompt_pos{pos0}_ntok{ntok}")
            wl = Prefill(x, torch, idx)
            g = capture(torch, wl.step, steps)
            g.replay()
            steady = min(replay_ms(torch, g, steps) for _ in range(3)) * 1e3
            del g
            iso = statistics.median(isolated_ms(torch, wl.step, flush, 8)) * 1e3
            wl.poison_outputs()
            wl.step(0)
            torch.cuda.synchronize()
            outs = wl.timed_outputs()
            wl.parity(outs, wl.gpu_scores())
            cells.append({"pos0": pos0, "blocks": n_pad, "ntok": ntok, "inputs": "f32",
                          "steady_us": steady, "isolated_cold_us": iso})
            log(f"[decode] pos0={pos0} ntok={ntok}: steady {steady:.2f} us, "
                f"isolated cold {iso:.2f} us")
    return cells


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=None, choices=list(range(1, 11)))
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="CPU oracle timing budget per workload")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the CPU leg (oracle timing and the parity check)")
    ap.add_argument("--pmc-calibrate", action="store_true")
    ap.add_argument("--parse-pmc", nargs="+", default=None)
    ap.add_argument("--parse-trace", default=None)
    ap.add_argument("--trace-command", default="")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the steady, isolated, host end-to-end, sorted and floor figures")
    ap.add_argument("--out", default=None)
    ap.add_argument("--paged-sweep", action="store_true",
                    help="time idx_select_paged over the 5 page-count regimes x 5 batch sizes")
    ap.add_argument("--decode-shapes", action="store_true",
                    help="time idx_select on the pages' decode shapes (pos0 3000/8192/30000)")
    a = ap.parse_args()

    if a.parse_pmc:
        out = a.out or os.path.join(ROOT, "profiles",
                                    f"traffic_w{a.workload}_{KERNEL[a.workload]}.txt")
        parse_pmc(a.parse_pmc, out, a.workload)
        return 0
    if a.parse_trace:
        parse_trace(a.parse_trace, a.out or os.path.join(a.parse_trace, "regions.md"),
                    a.trace_command)
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
    flush = Flusher(torch, idx)
    if a.paged_sweep:
        print(json.dumps({"paged_sweep": paged_sweep(torch, idx, flush)}))
        return 0
    if a.decode_shapes:
        print(json.dumps({"decode_shapes": decode_shapes(torch, idx, flush)}))
        return 0
    if a.pmc_calibrate:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    head = a.workload if a.workload is not None else HEADLINE
    order = [head] if a.workload is not None else [w for w in DEFAULT_SET if w != head] + [head]
    results, failed = {}, []
    for w in order:
        log(f"[bench] workload {w}: building inputs")
        wl = make(w, torch, idx)
        res, outs = measure(torch, idx, wl, a.steps if w == head else None, a.warmup,
                            not a.no_extras, flush)
        if not a.no_cpu_baseline:
            log(f"[bench] w{w}: CPU leg (oracle parity check, ~{a.cpu_seconds:.0f} s timing)")
            res["parity"], res["cpu_baseline"] = cpu_baseline_leg(wl, outs, wl.gpu_scores(),
                                                                  a.cpu_seconds)
            if not res["parity"]["ok"]:
                failed.append(w)
                log(f"[bench] w{w}: PARITY FAILED: {res['parity']['error']}")
        else:
            res["parity"] = {"ok": None, "note": "not checked (--no-cpu-baseline)"}
        if res.get("radix8_same_outputs") is False:
            failed.append(w)
            log(f"[bench] w{w}: the IDX_RADIX8 select returned other outputs")
        res["dtype"] = wl.dtype
        results[w] = res
        del wl, outs
        torch.cuda.empty_cache()

    h = results[head]
    out = {
        "metric": METRIC,
        "value": h["value"], "unit": h["unit"],
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": h["ms_per_step"], "us_per_call": h["us_per_call"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": h["dtype"], "data": "synthetic",
        "config": h["config"],
        "timing": "hbm_cold: a HIP graph of the timed steps, replayed after a 1 GiB read "
                  "that evicts L2 and the last-level cache; every step reads input copies "
                  "no earlier step of the region touched",
        "roofline": h["roofline"],
    }
    for k in ("parity", "cpu_baseline", "steady_us_per_call", "isolated_call_us",
              "isolated_empty_us", "host_e2e_us_per_call", "plan_host_e2e_us",
              "plan_graph_host_e2e_us", "sorted_us_per_call", "radix8_us_per_call",
              "radix8_same_outputs", "floor",
              "input_copies", "distinct_read_bytes"):
        if k in h:
            out[k] = h[k]
    if len(results) > 1:
        out["workloads"] = {results[w]["config"]["workload"]: results[w]
                            for w in order if w != head}
    out["parity_all_ok"] = not failed if not a.no_cpu_baseline else None
    print(json.dumps(out), flush=True)
    return 3 if failed else 0


if __name__ == "__main__":
    sys.exit(main())
