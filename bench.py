#!/usr/bin/env python3
"""Benchmark of the paged GQA attention path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input.  The default workload
is the mixed scheduler step: one 4096-token prefill chunk of request A at prefix 32,768 plus one
decode token for each of 31 other requests (KV lengths log-uniform in [2000, 68000]), all in one
shared pool of 64-token pages.  Per step:
    mtd_kv_append           4096 chunk tokens of A + 31 decode tokens, one call
    mtd_attn_prefill_chunk  A's chunk over its 36,864 keys
    mtd_attn_decode         31 requests (split-K + merge)
Other workloads (--workload): decode16 (16 requests, L in [27000, 30000]), prefill90min (17 chunks
of a 67,500-token request), fulldepth_decode (28 layers x 64 requests, 128K cap), and the same
steps as whole attention blocks with the QKV and output projections around the attention
(mixed_block, fulldepth_block, decode_graph_block), besides mixed_step_overlap, decode_graph and
decode16_seqsplit (one GPU's share of decode16 split by sequence over 8 GPUs, with the merge).

Prints one JSON line.  `value` is decode-attention HBM throughput (algorithmic bytes / time) and
`prefill` carries the chunked-prefill TFLOP/s; `roofline` is for the kernel that takes the most
time in the step, timed with HIP events on the stream the library launches on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "decode-attn HBM GB/s + chunked-prefill TFLOP/s on 1 MI355X, % of roofline"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA

# Algorithmic byte / flop counts (per call).
KV_BYTES_PER_TOKEN = 2 * W.HKV * W.HEAD_DIM * 2          # K + V, all KV heads, bf16
Q_BYTES = W.HQ * W.HEAD_DIM * 2                          # one query token, all heads
OUT_BYTES = W.HQ * W.HEAD_DIM * 4 + W.HQ * 4              # fp32 O + LSE per query token


# HBM traffic per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE (scaled by the same
# counters on a copy kernel of known size) is recorded in profiles/traffic.md together with a digest
# of the kernel's sources; it is reported only while the sources still match.
TRAFFIC_TABLE = os.path.join(ROOT, "profiles", "traffic.md")
KERNEL_SOURCES = {
    "prefill_kernel+prefill_merge_kernel": ["prefill.hip"],
    "decode_split_kernel+decode_merge_kernel": ["decode.hip"],
    "proj_wide_kernel": ["proj.hip"],
    "proj_ksplit_kernel": ["proj.hip"],
}
COMMON_SOURCES = ["device_util.h", "mtd_internal.h"]


def _code_only(text: str) -> str:
    """Source text without comments and blank space, so that comment edits keep the digest."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES.get(kernel, []) + COMMON_SOURCES:
        with open(os.path.join(ROOT, "gqa_kv_cache_qwen3_amd", "csrc", name)) as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic.md if recorded for these exact sources, else None."""
    if not os.path.exists(TRAFFIC_TABLE):
        return None
    digest = source_digest(kernel)
    for line in open(TRAFFIC_TABLE):
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) >= 4 and cells[0] == kernel and cells[1] == workload and cells[2] == digest:
            try:
                return float(cells[3])
            except ValueError:
                return None
    return None


def decode_bytes(lens) -> int:
    lens = np.asarray(lens, dtype=np.int64)
    table = 4 * ((lens + W.PAGE - 1) // W.PAGE)
    return int((KV_BYTES_PER_TOKEN * lens + Q_BYTES + OUT_BYTES + table + 4).sum())


def prefill_flops(prefix: int, chunk: int) -> float:
    """4 * Hq * d flops per attended (query, key) pair; causal pairs only."""
    pairs = chunk * prefix + chunk * (chunk + 1) / 2
    return 4.0 * W.HQ * W.HEAD_DIM * pairs


def fill_normal_(t, seed, slab=1 << 28):
    import torch
    gen = torch.Generator(device=t.device)
    gen.manual_seed(seed)
    flat = t.view(-1)
    for lo in range(0, flat.numel(), slab):
        hi = min(lo + slab, flat.numel())
        flat[lo:hi] = torch.randn(hi - lo, generator=gen, device=t.device, dtype=torch.float32).to(torch.bfloat16)
    return t


def parity(o_gpu, l_gpu, o_ref, l_ref):
    """The parity metrics of one comparison: max |dO|, max |dLSE|, relative Frobenius error, max |O|."""
    o = o_gpu.detach().double().cpu().numpy().reshape(o_ref.shape)
    l = l_gpu.detach().double().cpu().numpy().reshape(l_ref.shape)
    return {"max_abs_dO": float(np.abs(o - o_ref).max()), "max_abs_dLSE": float(np.abs(l - l_ref).max()),
            "rel_frobenius": float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30)),
            "max_abs_O": float(np.abs(o_ref).max()), "within_gates": bool(np.abs(o - o_ref).max() <= 1e-2 and
                                                                         np.abs(l - l_ref).max() <= 1e-3)}


class Timer:
    """HIP events recorded on the library's stream (torch's current stream)."""

    def __init__(self, names):
        import torch
        self.torch = torch
        self.names = names
        self.samples = {n: [] for n in names}

    def step_events(self):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(len(self.names) + 1)]

    def collect(self, events):
        for i, n in enumerate(self.names):
            self.samples[n].append(events[i].elapsed_time(events[i + 1]))

    def mean_ms(self, name):
        return float(np.mean(self.samples[name]))


# --------------------------------------------------------------------------------------------
# mixed scheduler step
# --------------------------------------------------------------------------------------------

class MixedStep:
    name = "mixed_step"

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch = mtd, torch
        p = W.MIXED.params
        self.prefix, self.chunk = p["prefix"], p["chunk"]
        self.lens = W.loguniform_lengths(p["batch"], p["lo"], p["hi"], W.MIXED.tag, 0)
        final = np.concatenate([[self.prefix + self.chunk], self.lens])
        tables, n_pages, _ = W.place_pages(final, W.MIXED.tag, 0)
        self.n_pages = n_pages
        self.k = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty_like(self.k)
        fill_normal_(self.k, W.torch_seed(W.MIXED.tag, 1))
        fill_normal_(self.v, W.torch_seed(W.MIXED.tag, 2))
        self.bt_all = torch.as_tensor(tables, device=dev)
        self.bt_a = self.bt_all[0].contiguous()
        self.bt_dec = self.bt_all[1:].contiguous()
        n_new = self.chunk + len(self.lens)
        self.k_new = torch.empty((n_new, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v_new = torch.empty_like(self.k_new)
        fill_normal_(self.k_new, W.torch_seed(W.MIXED.tag, 3))
        fill_normal_(self.v_new, W.torch_seed(W.MIXED.tag, 4))
        cu = np.concatenate([[0, self.chunk], self.chunk + np.arange(1, len(self.lens) + 1)]).astype(np.int32)
        start = np.concatenate([[self.prefix], self.lens - 1]).astype(np.int32)
        self.cu = torch.as_tensor(cu, device=dev)
        self.start = torch.as_tensor(start, device=dev)
        self.q_a = torch.empty((self.chunk, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.q_d = torch.empty((len(self.lens), W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        fill_normal_(self.q_a, W.torch_seed(W.MIXED.tag, 5))
        fill_normal_(self.q_d, W.torch_seed(W.MIXED.tag, 6))
        self.kv_lens = torch.as_tensor(self.lens.astype(np.int32), device=dev)
        self.max_len = int(self.lens.max())
        self.ws = torch.empty(mtd.decode_workspace_bytes(len(self.lens), self.max_len), dtype=torch.uint8, device=dev)
        # prefill workspace: the library rebalances the causal work over the CUs and merges split tiles
        self.ws_p = torch.empty(mtd.prefill_workspace_bytes(self.chunk), dtype=torch.uint8, device=dev)
        self.o_a = torch.empty((self.chunk, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l_a = torch.empty((self.chunk, W.HQ), dtype=torch.float32, device=dev)
        self.o_d = torch.empty((len(self.lens), W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l_d = torch.empty((len(self.lens), W.HQ), dtype=torch.float32, device=dev)
        self.timer = Timer(["append", "prefill", "decode"])
        self.work = {
            "append_bytes": 2 * n_new * W.HKV * W.HEAD_DIM * 2 * 2,
            "prefill_flops": prefill_flops(self.prefix, self.chunk),
            "decode_bytes": decode_bytes(self.lens),
        }

    def step(self, events=None):
        mtd = self.mtd
        if events: events[0].record()
        mtd.mtd_kv_append(self.k, self.v, self.k_new, self.v_new, self.cu, self.start, self.bt_all)
        if events: events[1].record()
        mtd.mtd_attn_prefill_chunk(self.k, self.v, self.q_a, self.prefix, self.bt_a, W.SCALE, self.o_a, self.l_a,
                                   self.ws_p)
        if events: events[2].record()
        mtd.mtd_attn_decode(self.k, self.v, self.q_d, self.kv_lens, self.bt_dec, self.max_len, W.SCALE,
                            self.ws, self.o_d, self.l_d)
        if events: events[3].record()

    def config(self):
        return {"workload": "mixed_step: one 4096-token prefill chunk at prefix 32768 + decode of 31 requests "
                            "(KV lengths log-uniform in [2000, 68000]), shared pool of 64-token pages",
                "num_q_heads": W.HQ, "num_kv_heads": W.HKV, "head_dim": W.HEAD_DIM, "page_size": W.PAGE,
                "chunk": self.chunk, "prefix": self.prefix, "decode_batch": len(self.lens),
                "decode_kv_tokens": int(self.lens.sum()), "pool_pages": self.n_pages}

    def results(self):
        t = self.timer
        dec_ms, pre_ms, app_ms = t.mean_ms("decode"), t.mean_ms("prefill"), t.mean_ms("append")
        dec_gbs = self.work["decode_bytes"] / (dec_ms * 1e-3) / 1e9
        pre_tfs = self.work["prefill_flops"] / (pre_ms * 1e-3) / 1e12
        return {
            "decode": {"value": dec_gbs, "unit": "GB/s", "frac": dec_gbs / HBM_PEAK_GBS, "ms": dec_ms,
                       "bytes": self.work["decode_bytes"], "kernels": "decode_split_kernel + decode_merge_kernel"},
            "prefill": {"value": pre_tfs, "unit": "TFLOP/s", "frac": pre_tfs / MFMA_BF16_PEAK_TFLOPS, "ms": pre_ms,
                        "flops": self.work["prefill_flops"], "kernels": "prefill_kernel + prefill_merge_kernel"},
            "append": {"ms": app_ms, "bytes": self.work["append_bytes"], "kernels": "kv_append_kernel"},
        }

    def dominant(self, res):
        if res["prefill"]["ms"] >= res["decode"]["ms"]:
            return {"kernel": "prefill_kernel+prefill_merge_kernel", "bound": "mfma", "achieved": res["prefill"]["value"],
                    "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "per_launch": res["prefill"]["flops"],
                    "ms": res["prefill"]["ms"]}
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": res["decode"]["bytes"], "ms": res["decode"]["ms"]}

    def record(self, pool):
        """Seeds, lengths and the parity of the last timed step's outputs against the oracle: 256 prefill
        rows (every 16th) and all decode requests."""
        import torch
        from oracle.parallel import decode_problem, prefill_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        kb, vb = host(self.k), host(self.v)
        tables = self.bt_all.cpu().numpy()
        rows = np.arange(0, self.chunk, 16)
        qa, qd = host(self.q_a), host(self.q_d)
        probs = [{"q": qa[rows], "k_pages": kb, "v_pages": vb, "table": tables[0], "n_keys": self.prefix + self.chunk,
                  "q_pos": self.prefix + rows}]
        probs += [decode_problem(qd[b:b + 1], kb, vb, tables[1 + b], int(self.lens[b])) for b in range(len(self.lens))]
        ref = pool.attention(probs, W.SCALE)
        o_ref = np.concatenate([r[0] for r in ref[1:]])
        l_ref = np.concatenate([r[1] for r in ref[1:]])
        return {"seeds": {"base": W.BASE_SEED, "tag": W.MIXED.tag},
                "lengths": {"chunk": self.chunk, "prefix": self.prefix, "decode_requests": len(self.lens),
                            "decode_min": int(self.lens.min()), "decode_mean": float(self.lens.mean()),
                            "decode_max": int(self.lens.max()), "decode_sum": int(self.lens.sum())},
                "parity": {"prefill, 256 rows (every 16th)": parity(self.o_a[rows], self.l_a[rows], ref[0][0], ref[0][1]),
                           "decode, all 31 requests": parity(self.o_d, self.l_d, o_ref, l_ref)}}

    # ---- CPU baseline: the fp64 oracle on the same step ----
    def cpu_baseline(self):
        """The fp64 oracle on this step's whole input: all 4096 prefill rows and all 31 decode
        requests, over a process pool (one BLAS thread per worker) on the host's cores.  Timed:
        the oracle's compute only (page walk included); copying the pool to the host and staging
        it for the workers are not."""
        import torch
        from oracle.parallel import OraclePool, cpu_model, decode_problem, prefill_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        kb, vb = host(self.k), host(self.v)
        tables = self.bt_all.cpu().numpy()
        qa, qd = host(self.q_a), host(self.q_d)
        with OraclePool() as pool:
            staged = pool.stage([prefill_problem(qa, kb, vb, tables[0], self.prefix)])
            t0 = time.perf_counter()
            pool.run(staged, W.SCALE)
            t_pre = time.perf_counter() - t0
            staged = pool.stage([decode_problem(qd[b:b + 1], kb, vb, tables[1 + b], int(self.lens[b]))
                                 for b in range(len(self.lens))])
            t0 = time.perf_counter()
            pool.run(staged, W.SCALE)
            t_dec = time.perf_counter() - t0
            workers = pool.workers
        dec_bytes = KV_BYTES_PER_TOKEN * float(self.lens.sum())
        return {
            "value": dec_bytes / t_dec / 1e9, "unit": "GB/s",
            "prefill_tflops": self.work["prefill_flops"] / t_pre / 1e12,
            "cores": workers, "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": (f"the whole step: decode of all {len(self.lens)} requests ({int(self.lens.sum())} KV tokens, "
                       f"{t_dec:.1f} s) and all {self.chunk} prefill rows ({t_pre:.1f} s); fp64 numpy in {workers} "
                       "worker processes with one BLAS thread each"),
        }


# --------------------------------------------------------------------------------------------
# decode16 and prefill90min as standalone steps (secondary workloads)
# --------------------------------------------------------------------------------------------

class Decode16:
    name = "decode16"

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd = mtd
        p = W.DECODE16.params
        self.lens = W.uniform_lengths(p["batch"], p["lo"], p["hi"], W.DECODE16.tag, 0)
        tables, n_pages, _ = W.place_pages(self.lens, W.DECODE16.tag, 0)
        self.k = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty_like(self.k)
        fill_normal_(self.k, W.torch_seed(W.DECODE16.tag, 1))
        fill_normal_(self.v, W.torch_seed(W.DECODE16.tag, 2))
        b = len(self.lens)
        self.bt = torch.as_tensor(tables, device=dev)
        self.q = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        fill_normal_(self.q, W.torch_seed(W.DECODE16.tag, 3))
        self.k_new = torch.empty((b, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v_new = torch.empty_like(self.k_new)
        fill_normal_(self.k_new, 5)
        fill_normal_(self.v_new, 6)
        self.cu = torch.arange(b + 1, dtype=torch.int32, device=dev)
        self.start = torch.as_tensor((self.lens - 1).astype(np.int32), device=dev)
        self.kv_lens = torch.as_tensor(self.lens.astype(np.int32), device=dev)
        self.max_len = int(self.lens.max())
        self.ws = torch.empty(mtd.decode_workspace_bytes(b, self.max_len), dtype=torch.uint8, device=dev)
        self.o = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l = torch.empty((b, W.HQ), dtype=torch.float32, device=dev)
        self.timer = Timer(["append", "decode"])
        self.bytes = decode_bytes(self.lens)

    def step(self, events=None):
        mtd = self.mtd
        if events: events[0].record()
        mtd.mtd_kv_append(self.k, self.v, self.k_new, self.v_new, self.cu, self.start, self.bt)
        if events: events[1].record()
        mtd.mtd_attn_decode(self.k, self.v, self.q, self.kv_lens, self.bt, self.max_len, W.SCALE, self.ws, self.o, self.l)
        if events: events[2].record()

    def config(self):
        return {"workload": "decode16: batched decode of 16 requests, KV lengths uniform in [27000, 30000]",
                "decode_kv_tokens": int(self.lens.sum())}

    def results(self):
        ms = self.timer.mean_ms("decode")
        gbs = self.bytes / (ms * 1e-3) / 1e9
        return {"decode": {"value": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "ms": ms, "bytes": self.bytes},
                "append": {"ms": self.timer.mean_ms("append")}}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": self.bytes, "ms": res["decode"]["ms"]}

    def record(self, pool):
        """Seeds, lengths and the parity of the last timed step's outputs: all 16 requests."""
        import torch
        from oracle.parallel import decode_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        kb, vb, qb = host(self.k), host(self.v), host(self.q)
        tables = self.bt.cpu().numpy()
        ref = pool.attention([decode_problem(qb[b:b + 1], kb, vb, tables[b], int(self.lens[b]))
                              for b in range(len(self.lens))], W.SCALE)
        return {"seeds": {"base": W.BASE_SEED, "tag": W.DECODE16.tag},
                "lengths": {"requests": len(self.lens), "min": int(self.lens.min()), "mean": float(self.lens.mean()),
                            "max": int(self.lens.max()), "sum": int(self.lens.sum())},
                "parity": {"decode, all 16 requests": parity(self.o, self.l, np.concatenate([r[0] for r in ref]),
                                                             np.concatenate([r[1] for r in ref]))}}


class Tiny:
    """The tiny configuration as a step: one request's 439-token prompt appended and prefilled in one
    shot, then 32 decode steps of (append one token, decode).  Launch-bound and cache-resident: its
    figures are for parity and latency, not a roofline (the appends rewrite the same slots, so every
    step sees the same inputs).  The timed steps replay two captured HIP graphs (the prompt part and
    the 32-step decode loop), so the figures are the device's; the same calls issued eagerly are
    timed after the timed region and reported as `eager` (those depend on the host's launch rate)."""
    name = "tiny"

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch = mtd, torch
        p = W.TINY.params
        self.prompt, self.steps = p["prompt"], p["decode_steps"]
        total = self.prompt + self.steps
        tables, n_pages, _ = W.place_pages([total], W.TINY.tag, 0)
        self.table_np = tables[0]
        self.bt = torch.as_tensor(tables, device=dev)
        self.k = torch.zeros((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros_like(self.k)
        self.k_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(1, 1), dev)
        self.v_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(1, 2), dev)
        self.q_log = W.normal_bf16((total, W.HQ, W.HEAD_DIM), W.torch_seed(1, 3), dev)
        self.cu_p = torch.tensor([0, self.prompt], dtype=torch.int32, device=dev)
        self.cu_1 = torch.tensor([0, 1], dtype=torch.int32, device=dev)
        self.starts = [torch.tensor([x], dtype=torch.int32, device=dev) for x in range(total)]
        self.lens = [torch.tensor([x], dtype=torch.int32, device=dev) for x in range(total + 1)]
        self.ws = torch.empty(mtd.decode_workspace_bytes(1, total), dtype=torch.uint8, device=dev)
        self.o_p = torch.empty((self.prompt, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l_p = torch.empty((self.prompt, W.HQ), dtype=torch.float32, device=dev)
        self.o_d = torch.empty((self.steps, 1, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l_d = torch.empty((self.steps, 1, W.HQ), dtype=torch.float32, device=dev)
        self.timer = Timer(["prefill", "decode"])
        self._prompt_calls()   # one eager pass before capture (code objects loaded, same outputs)
        self._decode_calls()
        torch.cuda.synchronize()
        self.g_prompt, self.g_decode = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g_prompt):
            self._prompt_calls()
        with torch.cuda.graph(self.g_decode):
            self._decode_calls()
        torch.cuda.synchronize()
        self.eager = None

    def _prompt_calls(self):
        mtd, P = self.mtd, self.prompt
        mtd.mtd_kv_append(self.k, self.v, self.k_log[:P], self.v_log[:P], self.cu_p, self.starts[0], self.bt)
        mtd.mtd_attn_prefill_chunk(self.k, self.v, self.q_log[:P], 0, self.bt[0], W.SCALE, self.o_p, self.l_p)

    def _decode_calls(self):
        mtd, P = self.mtd, self.prompt
        for s in range(self.steps):
            n = P + s
            mtd.mtd_kv_append(self.k, self.v, self.k_log[n:n + 1], self.v_log[n:n + 1], self.cu_1, self.starts[n], self.bt)
            mtd.mtd_attn_decode(self.k, self.v, self.q_log[n:n + 1], self.lens[n + 1], self.bt, P + self.steps, W.SCALE,
                                self.ws, self.o_d[s], self.l_d[s])

    def step(self, events=None):
        if events: events[0].record()
        self.g_prompt.replay()
        if events: events[1].record()
        self.g_decode.replay()
        if events: events[2].record()

    def eager_pass(self, n=20):
        """The same step as eager library calls, n times with events (after the timed region)."""
        t = Timer(["prefill", "decode"])
        evs = []
        for _ in range(n):
            e = t.step_events()
            e[0].record()
            self._prompt_calls()
            e[1].record()
            self._decode_calls()
            e[2].record()
            evs.append(e)
        self.torch.cuda.synchronize()
        for e in evs:
            t.collect(e)
        return {"prefill_ms": t.mean_ms("prefill"), "decode_ms_per_step": t.mean_ms("decode") / self.steps,
                "note": "eager library calls: bound by the host's launch rate, which varies between runs and hosts"}

    def config(self):
        return {"workload": "tiny: one 439-token one-shot prefill (30 s of audio + 64 prompt tokens), then 32 decode "
                            "steps of (append 1 token, decode)", "prompt": self.prompt, "decode_steps": self.steps}

    def results(self):
        pre, dec = self.timer.mean_ms("prefill"), self.timer.mean_ms("decode")
        fl = prefill_flops(0, self.prompt)
        by = sum(decode_bytes([self.prompt + s + 1]) for s in range(self.steps))
        return {"prefill": {"value": fl / (pre * 1e-3) / 1e12, "unit": "TFLOP/s",
                            "frac": fl / (pre * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, "ms": pre, "flops": fl,
                            "kernels": "kv_append_kernel + prefill_kernel (one pass)"},
                "decode": {"value": by / (dec * 1e-3) / 1e9, "unit": "GB/s", "frac": by / (dec * 1e-3) / 1e9 / HBM_PEAK_GBS,
                           "ms": dec / self.steps, "bytes": by / self.steps,
                           "kernels": "32 x (kv_append_kernel + decode_split_kernel + decode_merge_kernel)"},
                "eager": self.eager_pass()}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": res["decode"]["bytes"], "ms": res["decode"]["ms"]}

    def record(self, pool):
        import oracle
        host = lambda t: t.contiguous().view(self.torch.int16).cpu().numpy().view(np.uint16)
        self.torch.cuda.synchronize()
        used = (self.prompt + self.steps + W.PAGE - 1) // W.PAGE
        idx = self.torch.as_tensor(self.table_np[:used].astype(np.int64), device=self.k.device)
        kc, vc = host(self.k.index_select(0, idx)), host(self.v.index_select(0, idx))
        ident = np.arange(used)
        qb = host(self.q_log)
        o_ref, l_ref = oracle.prefill_chunk(qb[:self.prompt], kc, vc, ident, 0, W.SCALE)
        par = {"prefill, all 439 rows": parity(self.o_p, self.l_p, o_ref, l_ref)}
        od, ld = [], []
        for s in range(self.steps):
            n = self.prompt + s + 1
            o, l = oracle.decode(qb[n - 1:n], kc, vc, [n], [ident], W.SCALE)
            od.append(o[0])
            ld.append(l[0])
        par["decode, all 32 steps"] = parity(self.o_d[:, 0], self.l_d[:, 0], np.stack(od), np.stack(ld))
        return {"seeds": {"base": W.BASE_SEED, "tag": W.TINY.tag}, "lengths": {"prompt": self.prompt,
                "decode_kv_lengths": [self.prompt + 1, self.prompt + self.steps]}, "parity": par}


class Decode16SeqSplit:
    """One GPU's share of decode16 with each request's KV split by sequence over 8 GPUs: this GPU
    holds the first eighth of every request's tokens (whole pages), decodes them (the library's
    decode over a block table that starts at the shard's first page), and merges the 8 gathered
    (O, LSE) partials with mtd_attn_merge.  The gather itself (8 x 16 heads x 129 floats per
    request) is the one step a single GPU cannot show; the other shards are the same kernels."""
    name = "decode16_seqsplit"
    GPUS = 8

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch = mtd, torch
        p = W.DECODE16.params
        self.lens = W.uniform_lengths(p["batch"], p["lo"], p["hi"], W.DECODE16.tag, 0)
        # shard 0 of each request: its first ceil(L / 8) tokens, rounded up to whole pages
        per_gpu = -(-self.lens // self.GPUS)
        self.shard = np.minimum(-(-per_gpu // W.PAGE) * W.PAGE, self.lens)
        tables, n_pages, _ = W.place_pages(self.shard, W.DECODE16.tag, 3)
        b = len(self.lens)
        self.k = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v = torch.empty_like(self.k)
        fill_normal_(self.k, W.torch_seed(W.DECODE16.tag, 31))
        fill_normal_(self.v, W.torch_seed(W.DECODE16.tag, 32))
        self.bt = torch.as_tensor(tables, device=dev)
        self.q = W.normal_bf16((b, W.HQ, W.HEAD_DIM), W.torch_seed(W.DECODE16.tag, 33), dev)
        self.kv_lens = torch.as_tensor(self.shard.astype(np.int32), device=dev)
        self.max_len = int(self.shard.max())
        self.ws = torch.empty(mtd.decode_workspace_bytes(b, self.max_len), dtype=torch.uint8, device=dev)
        # the gathered partials: this GPU's in slot 0, the other shards' as seeded stand-ins
        self.o_parts = torch.randn((self.GPUS, b, W.HQ, W.HEAD_DIM), device=dev) * 0.1
        self.l_parts = torch.randn((self.GPUS, b, W.HQ), device=dev) + 8.0
        self.out = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.lse = torch.empty((b, W.HQ), dtype=torch.float32, device=dev)
        self.timer = Timer(["decode", "merge"])
        self.work = {"decode_bytes": decode_bytes(self.shard)}

    def step(self, events=None):
        mtd = self.mtd
        if events: events[0].record()
        mtd.mtd_attn_decode(self.k, self.v, self.q, self.kv_lens, self.bt, self.max_len, W.SCALE, self.ws,
                            self.o_parts[0], self.l_parts[0])
        if events: events[1].record()
        mtd.mtd_attn_merge(self.o_parts, self.l_parts, self.out, self.lse)
        if events: events[2].record()

    def config(self):
        return {"workload": "decode16_seqsplit: one GPU's share of decode16 with each request's KV split by "
                            "sequence over 8 GPUs (the first eighth of each request's tokens), then the merge of "
                            "the 8 gathered partials", "gpus_in_split": self.GPUS, "batch": len(self.lens),
                "shard_kv_tokens": int(self.shard.sum()), "request_kv_tokens": int(self.lens.sum())}

    def results(self):
        dec_ms, mrg_ms = self.timer.mean_ms("decode"), self.timer.mean_ms("merge")
        gbs = self.work["decode_bytes"] / (dec_ms * 1e-3) / 1e9
        return {"decode": {"value": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "ms": dec_ms,
                           "bytes": self.work["decode_bytes"], "kernels": "decode_split_kernel + decode_merge_kernel (shard)"},
                "step": {"shard_decode_ms": dec_ms, "merge_ms": mrg_ms, "per_gpu_ms": dec_ms + mrg_ms,
                         "gathered_bytes_per_request": self.GPUS * W.HQ * (W.HEAD_DIM + 1) * 4}}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": res["decode"]["bytes"], "ms": res["decode"]["ms"]}


class Prefill90:
    name = "prefill90min"

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd = mtd
        p = W.PREFILL90.params
        self.total, self.chunk = p["total"], p["chunk"]
        tables, n_pages, _ = W.place_pages([self.total], W.PREFILL90.tag, 0)
        self.k = torch.zeros((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.v = torch.zeros_like(self.k)
        self.bt = torch.as_tensor(tables, device=dev)
        self.k_log = W.lowrank_keys(self.total, W.torch_seed(W.PREFILL90.tag, 1), dev)
        self.v_log = torch.empty((self.total, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        fill_normal_(self.v_log, W.torch_seed(W.PREFILL90.tag, 2))
        self.q = torch.empty((self.total, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        fill_normal_(self.q, W.torch_seed(W.PREFILL90.tag, 3))
        self.o = torch.empty((self.chunk, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l = torch.empty((self.chunk, W.HQ), dtype=torch.float32, device=dev)
        self.ws_p = torch.empty(mtd.prefill_workspace_bytes(self.chunk), dtype=torch.uint8, device=dev)
        self.chunks = [(s, min(self.chunk, self.total - s)) for s in range(0, self.total, self.chunk)]
        self.cu = [torch.tensor([0, c], dtype=torch.int32, device=dev) for _, c in self.chunks]
        self.st = [torch.tensor([s], dtype=torch.int32, device=dev) for s, _ in self.chunks]
        self.timer = Timer(["append", "prefill"])
        self.flops = sum(prefill_flops(s, c) for s, c in self.chunks)

    def step(self, events=None):
        mtd = self.mtd
        for i, (s, c) in enumerate(self.chunks):
            mtd.mtd_kv_append(self.k, self.v, self.k_log[s:s + c], self.v_log[s:s + c], self.cu[i], self.st[i], self.bt)
            mtd.mtd_attn_prefill_chunk(self.k, self.v, self.q[s:s + c], s, self.bt[0], W.SCALE, self.o[:c], self.l[:c],
                                       self.ws_p)

    def timed_step(self):
        """Per-chunk events (append and prefill separately)."""
        import torch
        mtd = self.mtd
        evs = []
        for i, (s, c) in enumerate(self.chunks):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            mtd.mtd_kv_append(self.k, self.v, self.k_log[s:s + c], self.v_log[s:s + c], self.cu[i], self.st[i], self.bt)
            e[1].record()
            mtd.mtd_attn_prefill_chunk(self.k, self.v, self.q[s:s + c], s, self.bt[0], W.SCALE, self.o[:c], self.l[:c],
                                       self.ws_p)
            e[2].record()
            evs.append(e)
        return evs

    def config(self):
        return {"workload": "prefill90min: 67,500-token request as 17 chunks of 4096 (last 1,964), K with a rank-4 "
                            "per-head component", "flops_causal": self.flops}

    def results(self):
        ms = self.timer.mean_ms("prefill")
        tfs = self.flops / (ms * 1e-3) / 1e12
        return {"prefill": {"value": tfs, "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFLOPS, "ms": ms, "flops": self.flops},
                "append": {"ms": self.timer.mean_ms("append")}}

    def dominant(self, res):
        return {"kernel": "prefill_kernel+prefill_merge_kernel", "bound": "mfma", "achieved": res["prefill"]["value"],
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "per_launch": self.flops / len(self.chunks),
                "ms": res["prefill"]["ms"] / len(self.chunks)}

    def record(self, pool):
        """Seeds, lengths and the parity of the last chunk's outputs (every row of the 1,964) after the timed
        passes (the output buffer holds the last chunk)."""
        import torch
        from oracle.parallel import prefill_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        s0, c = self.chunks[-1]
        [(o_ref, l_ref)] = pool.attention([prefill_problem(host(self.q[s0:s0 + c]), host(self.k), host(self.v),
                                                           self.bt[0].cpu().numpy(), s0)], W.SCALE)
        return {"seeds": {"base": W.BASE_SEED, "tag": W.PREFILL90.tag},
                "lengths": {"total": self.total, "chunk": self.chunk, "chunks": len(self.chunks)},
                "parity": {f"last chunk (prefix {s0}), all {c} rows": parity(self.o[:c], self.l[:c], o_ref, l_ref)}}


class FullDepth:
    """28 layers x 64 requests, all layers resident; a step appends one token per request and
    runs decode attention, layer after layer (128 steps in a full pass)."""
    name = "fulldepth_decode"

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch = mtd, torch
        free, _ = torch.cuda.mem_get_info(dev)
        self.lens0, self.seeds_tried, self.need_bytes = W.fulldepth_draw(free)
        self.inp = W.build_fulldepth(dev, self.lens0)
        self.layers, self.steps = self.inp["layers"], self.inp["steps"]
        b = len(self.lens0)
        self.bt = torch.as_tensor(self.inp["tables"], device=dev)
        self.cu = torch.arange(b + 1, dtype=torch.int32, device=dev)
        self.start = [torch.as_tensor((self.lens0 + s).astype(np.int32), device=dev) for s in range(self.steps)]
        self.kv_lens = [torch.as_tensor((self.lens0 + s + 1).astype(np.int32), device=dev) for s in range(self.steps)]
        self.max_len = int(self.lens0.max()) + self.steps
        self.ws = torch.empty(mtd.decode_workspace_bytes(b, self.max_len), dtype=torch.uint8, device=dev)
        self.o = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.l = torch.empty((b, W.HQ), dtype=torch.float32, device=dev)
        self.step_idx = 0
        self.timer = Timer(["append", "decode"])
        self.bytes_per_step = [self.layers * decode_bytes(self.lens0 + s + 1) for s in range(self.steps)]
        self.timed_bytes = 0

    def step(self, events=None):
        mtd, inp = self.mtd, self.inp
        s = self.step_idx % self.steps
        self.step_idx += 1
        app = dec = 0.0
        evs = []
        for layer in range(self.layers):
            kp, vp = inp["k_pools"][layer], inp["v_pools"][layer]
            e = [self.torch.cuda.Event(enable_timing=True) for _ in range(3)] if events is not None else None
            if e: e[0].record()
            mtd.mtd_kv_append(kp, vp, inp["k_new"][s, layer], inp["v_new"][s, layer], self.cu, self.start[s], self.bt)
            if e: e[1].record()
            mtd.mtd_attn_decode(kp, vp, inp["q"][s, layer], self.kv_lens[s], self.bt, self.max_len, W.SCALE,
                                self.ws, self.o, self.l)
            if e: e[2].record()
            if e: evs.append(e)
        if events is not None:
            events.append(evs)
            self.timed_bytes += self.bytes_per_step[s]

    def collect(self, step_events):
        for evs in step_events:
            self.timer.samples["append"].append(sum(e[0].elapsed_time(e[1]) for e in evs))
            self.timer.samples["decode"].append(sum(e[1].elapsed_time(e[2]) for e in evs))

    def config(self):
        return {"workload": "fulldepth_decode: 28 layers x 64 requests, initial KV lengths log-uniform in "
                            "[4000, 131072-128], all layers resident; per step and layer: append 1 token per "
                            "request, then decode", "layers": self.layers, "batch": len(self.lens0),
                "initial_kv_tokens": int(self.lens0.sum()), "pool_pages_per_layer": int(self.inp["num_pages"]),
                "hbm_input_bytes": int(self.need_bytes), "seeds_tried": self.seeds_tried}

    def results(self):
        dec_ms = float(np.sum(self.timer.samples["decode"]))
        calls = len(self.timer.samples["decode"]) * self.layers
        gbs = self.timed_bytes / (dec_ms * 1e-3) / 1e9
        return {"decode": {"value": gbs, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
                           "ms": dec_ms / calls, "bytes": self.timed_bytes / calls,
                           "kernels": "decode_split_kernel + decode_merge_kernel (per layer call)"},
                "append": {"ms": float(np.sum(self.timer.samples["append"])) / calls}}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": res["decode"]["bytes"], "ms": res["decode"]["ms"]}

    def record(self, pool):
        """Seeds, lengths and the parity of the last layer's decode at the last timed step: 8 requests (seeded)."""
        import torch
        from oracle.parallel import decode_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        s = (self.step_idx - 1) % self.steps
        layer = self.layers - 1
        kp, vp = self.inp["k_pools"][layer], self.inp["v_pools"][layer]
        q = host(self.inp["q"][s, layer])
        lens = self.lens0 + s + 1
        sample = np.sort(W.rng(5, 78).permutation(len(lens))[:8])
        probs = []
        for b in sample:
            used = (int(lens[b]) + W.PAGE - 1) // W.PAGE
            idx = torch.as_tensor(self.inp["tables"][b][:used].astype(np.int64), device=kp.device)
            probs.append(decode_problem(q[b:b + 1], host(kp.index_select(0, idx)), host(vp.index_select(0, idx)),
                                        np.arange(used), int(lens[b])))
        ref = pool.attention(probs, W.SCALE)
        o_ref = np.concatenate([r[0] for r in ref])
        l_ref = np.concatenate([r[1] for r in ref])
        idx = torch.as_tensor(sample, device=self.o.device)
        return {"seeds": {"base": W.BASE_SEED, "tag": W.FULLDEPTH.tag, "tried": self.seeds_tried},
                "lengths": {"layers": self.layers, "requests": len(self.lens0), "initial_min": int(self.lens0.min()),
                            "initial_mean": float(self.lens0.mean()), "initial_max": int(self.lens0.max()),
                            "steps": self.steps},
                "parity": {f"layer {layer}, step {s}, 8 requests": parity(self.o[idx], self.l[idx], o_ref, l_ref)}}

    def cpu_baseline(self):
        """The fp64 oracle on 16 of the 64 requests (seeded choice) of the layer-0 decode call of the
        last timed step, over a process pool with one BLAS thread per worker; the oracle's compute
        only is timed (the requests' pages are copied to the host and staged beforehand)."""
        import torch
        from oracle.parallel import OraclePool, cpu_model, decode_problem
        torch.cuda.synchronize()
        host = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        s = (self.step_idx - 1) % self.steps
        kp, vp = self.inp["k_pools"][0], self.inp["v_pools"][0]
        q = host(self.inp["q"][s, 0])
        lens = self.lens0 + s + 1
        sample = np.sort(W.rng(5, 77).permutation(len(lens))[:16])
        probs = []
        for b in sample:
            used = (int(lens[b]) + W.PAGE - 1) // W.PAGE
            idx = torch.as_tensor(self.inp["tables"][b][:used].astype(np.int64), device=kp.device)
            probs.append(decode_problem(q[b:b + 1], host(kp.index_select(0, idx)), host(vp.index_select(0, idx)),
                                        np.arange(used), int(lens[b])))
        with OraclePool() as pool:
            staged = pool.stage(probs)
            t0 = time.perf_counter()
            pool.run(staged, W.SCALE)
            t_dec = time.perf_counter() - t0
            workers = pool.workers
        n_tok = int(lens[sample].sum())
        return {"value": KV_BYTES_PER_TOKEN * n_tok / t_dec / 1e9, "unit": "GB/s", "cores": workers,
                "affinity_cores": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(), "kind": "oracle",
                "sample": f"16 of the 64 requests of one layer's decode call ({n_tok} KV tokens, {t_dec:.1f} s); "
                          f"fp64 numpy in {workers} worker processes with one BLAS thread each"}


def proj_work(n_tok: int):
    """Algorithmic flops and HBM bytes of one QKV projection and one output projection call:
    weights once, activations in and out once (bf16, the float32 attention output for o_proj)."""
    n_qkv, n_o = (W.HQ + 2 * W.HKV) * W.HEAD_DIM, W.HQ * W.HEAD_DIM
    qkv = {"flops": 2.0 * n_tok * W.HIDDEN * n_qkv, "bytes": 2 * (n_qkv * W.HIDDEN + n_tok * W.HIDDEN + n_tok * n_qkv)}
    o = {"flops": 2.0 * n_tok * n_o * W.HIDDEN, "bytes": 2 * W.HIDDEN * n_o + 4 * n_tok * n_o + 2 * n_tok * W.HIDDEN}
    return qkv, o


def proj_results(samples_qkv, samples_o, n_tok, calls_per_sample=1, workload=None):
    qkv_w, o_w = proj_work(n_tok)
    out = {}
    kernels = {"qkv_proj": "proj_wide_kernel", "o_proj": "proj_ksplit_kernel"}
    for name, samples, wk in (("qkv_proj", samples_qkv, qkv_w), ("o_proj", samples_o, o_w)):
        ms = float(np.sum(samples)) / (len(samples) * calls_per_sample)
        tfs = wk["flops"] / (ms * 1e-3) / 1e12
        gbs = wk["bytes"] / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "tokens": n_tok, "tflops": tfs, "mfma_frac": tfs / MFMA_BF16_PEAK_TFLOPS,
                     "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS, "flops": wk["flops"], "bytes": wk["bytes"]}
        if workload is not None:
            out[name]["traffic"] = recorded_traffic(kernels[name], workload)
    return out


class MixedBlock(MixedStep):
    """The mixed scheduler step as a whole attention block: the QKV projection of all 4127 new tokens
    (the chunk's 4096 and one per decode request) feeds the append, the prefill and the decode, and
    the output projection maps all their attention outputs back to hidden size."""
    name = "mixed_block"

    record = None  # the attention's inputs come from the projections; parity is in the tests
    def __init__(self, dev):
        super().__init__(dev)
        torch, mtd = self.torch, self.mtd
        n_new = self.chunk + len(self.lens)
        self.w_qkv, self.w_o = W.projection_weights(W.torch_seed(W.MIXED.tag, 7), dev)
        self.x = W.normal_bf16((n_new, W.HIDDEN), W.torch_seed(W.MIXED.tag, 8), dev)
        self.q_all = torch.empty((n_new, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.q_a, self.q_d = self.q_all[:self.chunk], self.q_all[self.chunk:]
        self.o_all = torch.empty((n_new, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.o_a, self.o_d = self.o_all[:self.chunk], self.o_all[self.chunk:]
        self.y = torch.empty((n_new, W.HIDDEN), dtype=torch.bfloat16, device=dev)
        self.n_new = n_new
        self.timer = Timer(["qkv_proj", "append", "prefill", "decode", "o_proj"])

    def step(self, events=None):
        mtd = self.mtd
        if events: events[0].record()
        mtd.mtd_qkv_proj(self.x, self.w_qkv, self.q_all, self.k_new, self.v_new)
        if events: events[1].record()
        mtd.mtd_kv_append(self.k, self.v, self.k_new, self.v_new, self.cu, self.start, self.bt_all)
        if events: events[2].record()
        mtd.mtd_attn_prefill_chunk(self.k, self.v, self.q_a, self.prefix, self.bt_a, W.SCALE, self.o_a, self.l_a,
                                   self.ws_p)
        if events: events[3].record()
        mtd.mtd_attn_decode(self.k, self.v, self.q_d, self.kv_lens, self.bt_dec, self.max_len, W.SCALE,
                            self.ws, self.o_d, self.l_d)
        if events: events[4].record()
        mtd.mtd_o_proj(self.o_all, self.w_o, self.y)
        if events: events[5].record()

    def config(self):
        c = super().config()
        c["workload"] = ("mixed_block: the mixed step as an attention block: QKV projection of the 4127 new "
                         "tokens (hidden 1024 -> 16+8+8 heads x 128, random bf16 weights) -> append -> "
                         "prefill chunk 4096 at prefix 32768 + decode of 31 requests -> output projection")
        c["hidden"] = W.HIDDEN
        return c

    def results(self):
        res = super().results()
        res["proj"] = proj_results(self.timer.samples["qkv_proj"], self.timer.samples["o_proj"], self.n_new,
                                   workload=self.name)
        return res

    cpu_baseline = None


class FullDepthBlock(FullDepth):
    """Full-depth decode with the projections around each layer's attention: per step and layer,
    the QKV projection of the 64 requests' hidden states, the append of the new K/V, decode
    attention, and the output projection whose result is the next layer's input."""
    name = "fulldepth_block"

    record = None  # the attention's inputs come from the projections; parity is in the tests
    def __init__(self, dev):
        import torch
        p = W.FULLDEPTH.params
        # the weights first, so that the pools are sized to the memory that is left
        self.w = [W.projection_weights(W.torch_seed(W.FULLDEPTH.tag, 50, l), dev) for l in range(p["layers"])]
        super().__init__(dev)
        b = len(self.lens0)
        self.x0 = [W.normal_bf16((b, W.HIDDEN), W.torch_seed(W.FULLDEPTH.tag, 51, s), dev) for s in range(4)]
        self.x = torch.empty((b, W.HIDDEN), dtype=torch.bfloat16, device=dev)
        self.q = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.kn = torch.empty((b, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.vn = torch.empty_like(self.kn)
        self.timer = Timer(["qkv_proj", "append", "decode", "o_proj"])

    def step(self, events=None):
        mtd, inp = self.mtd, self.inp
        s = self.step_idx % self.steps
        self.step_idx += 1
        evs = []
        x = self.x0[s % len(self.x0)]
        for layer in range(self.layers):
            kp, vp = inp["k_pools"][layer], inp["v_pools"][layer]
            w_qkv, w_o = self.w[layer]
            e = [self.torch.cuda.Event(enable_timing=True) for _ in range(5)] if events is not None else None
            if e: e[0].record()
            mtd.mtd_qkv_proj(x, w_qkv, self.q, self.kn, self.vn)
            if e: e[1].record()
            mtd.mtd_kv_append(kp, vp, self.kn, self.vn, self.cu, self.start[s], self.bt)
            if e: e[2].record()
            mtd.mtd_attn_decode(kp, vp, self.q, self.kv_lens[s], self.bt, self.max_len, W.SCALE,
                                self.ws, self.o, self.l)
            if e: e[3].record()
            mtd.mtd_o_proj(self.o, w_o, self.x)
            if e: e[4].record()
            if e: evs.append(e)
            x = self.x
        if events is not None:
            events.append(evs)
            self.timed_bytes += self.bytes_per_step[s]

    def collect(self, step_events):
        for evs in step_events:
            for i, n in enumerate(("qkv_proj", "append", "decode", "o_proj")):
                self.timer.samples[n].append(sum(e[i].elapsed_time(e[i + 1]) for e in evs))

    def config(self):
        c = super().config()
        c["workload"] = ("fulldepth_block: 28 layers x 64 requests, initial KV lengths log-uniform in "
                         "[4000, 131072-128], all layers resident; per step and layer: QKV projection of the "
                         "64 hidden states (random bf16 weights) -> append -> decode -> output projection "
                         "(the next layer's input)")
        c["hidden"] = W.HIDDEN
        return c

    def results(self):
        res = super().results()
        res["proj"] = proj_results(self.timer.samples["qkv_proj"], self.timer.samples["o_proj"], len(self.lens0),
                                   calls_per_sample=self.layers)
        calls = len(self.timer.samples["decode"]) * self.layers
        res["step"] = {"layer_ms": sum(float(np.sum(self.timer.samples[n])) for n in self.timer.names) / calls}
        return res


class MixedStepOverlap(MixedStep):
    """The mixed step with its prefill and decode running at the same time on separate compute
    units: after the append, the prefill runs on the library's stream on a budget of CU_BUDGET
    compute units (mtd_attn_prefill_chunk_cus: the chunk's causal work spread evenly over that
    many workgroups, tiles cut at range boundaries merged), and the decode on a second stream
    (default priority), whose waves take the CUs the prefill leaves free; the two are joined
    before the next step.  Prefill is bound by the matrix units and decode by HBM, so the step
    tends to max(prefill on fewer CUs, decode on the rest) instead of their sum.  Per-kernel
    times here include the contention between the two; the step time is the figure of merit."""
    name = "mixed_step_overlap"
    CU_BUDGET = 224

    def __init__(self, dev):
        super().__init__(dev)
        torch = self.torch
        self.side = torch.cuda.Stream(device=dev)
        self.appended, self.decoded = torch.cuda.Event(), torch.cuda.Event()
        self.timer = OverlapTimer()
        self.cu_budget = int(os.environ.get("MTD_BENCH_CU_BUDGET", self.CU_BUDGET))

    def step(self, events=None):
        mtd, torch = self.mtd, self.torch
        main = torch.cuda.current_stream()
        if events: events[0].record()
        mtd.mtd_kv_append(self.k, self.v, self.k_new, self.v_new, self.cu, self.start, self.bt_all)
        if events: events[1].record()
        self.appended.record(main)
        mtd.mtd_attn_prefill_chunk_cus(self.k, self.v, self.q_a, self.prefix, self.bt_a, W.SCALE, self.ws_p,
                                       self.cu_budget, self.o_a, self.l_a)
        if events: events[2].record()
        self.side.wait_event(self.appended)
        with torch.cuda.stream(self.side):
            if events: events[3].record()
            mtd.mtd_attn_decode(self.k, self.v, self.q_d, self.kv_lens, self.bt_dec, self.max_len, W.SCALE,
                                self.ws, self.o_d, self.l_d)
            if events: events[4].record()
            self.decoded.record()
        main.wait_event(self.decoded)
        if events: events[5].record()

    def config(self):
        c = super().config()
        c["workload"] = ("mixed_step_overlap: " + c["workload"].split(": ", 1)[1] +
                         f"; prefill on {self.cu_budget} CUs beside the decode on a second stream")
        c["prefill_cu_budget"] = self.cu_budget
        return c

    def results(self):
        res = super().results()
        res["step"] = {"overlapped_ms": self.timer.mean_ms("step"), "append_ms": self.timer.mean_ms("append")}
        return res

    cpu_baseline = None


class OverlapTimer(Timer):
    """append and prefill events on the library's stream, decode events on the second stream, and
    the whole step (append start to the join of both streams)."""

    def __init__(self):
        super().__init__(["append", "prefill", "decode", "step"])

    def step_events(self):
        return [self.torch.cuda.Event(enable_timing=True) for _ in range(6)]

    def collect(self, events):
        self.samples["append"].append(events[0].elapsed_time(events[1]))
        self.samples["prefill"].append(events[1].elapsed_time(events[2]))
        self.samples["decode"].append(events[3].elapsed_time(events[4]))
        self.samples["step"].append(events[0].elapsed_time(events[5]))


class DecodeGraph:
    """Launch-bound decode: one request with the tiny workload's context (439 tokens and growing)
    through 28 layers; a step is 28 x (append its new token, decode).  The same step is timed as
    eager library calls and as one replay of a captured HIP graph (decode at concurrency 1 is where
    graph capture pays off), each both as mtd_kv_append + mtd_attn_decode (3 launches per layer) and
    as mtd_attn_decode_append (2 launches per layer, same bits)."""
    name = "decode_graph"
    SLOTS = 8      # rotating input sets; one captured graph per set
    LAYERS = 28
    ROOM = 4096    # tokens the request may grow by during one timed pass

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch = mtd, torch
        self.l0 = W.TINY.params["prompt"]
        tables, n_pages, _ = W.place_pages([self.l0 + self.ROOM], W.TINY.tag, 1)
        self.bt = torch.as_tensor(tables, device=dev)
        self.k = [torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
                  for _ in range(self.LAYERS)]
        self.v = [torch.empty_like(t) for t in self.k]
        for l in range(self.LAYERS):
            fill_normal_(self.k[l], W.torch_seed(W.TINY.tag, 60, l))
            fill_normal_(self.v[l], W.torch_seed(W.TINY.tag, 61, l))
        shape_q, shape_kv = (self.SLOTS, self.LAYERS, 1, W.HQ, W.HEAD_DIM), (self.SLOTS, self.LAYERS, 1, W.HKV, W.HEAD_DIM)
        self.q = W.normal_bf16(shape_q, W.torch_seed(W.TINY.tag, 62), dev)
        self.k_new = W.normal_bf16(shape_kv, W.torch_seed(W.TINY.tag, 63), dev)
        self.v_new = W.normal_bf16(shape_kv, W.torch_seed(W.TINY.tag, 64), dev)
        self.cu = torch.arange(2, dtype=torch.int32, device=dev)
        self.pos = torch.zeros(1, dtype=torch.int32, device=dev)   # where this step's token goes
        self.len = torch.zeros(1, dtype=torch.int32, device=dev)   # KV length after the append
        self.max_len = self.l0 + self.ROOM
        self.ws = torch.empty(mtd.decode_workspace_bytes(1, self.max_len), dtype=torch.uint8, device=dev)
        self.o = torch.empty((self.LAYERS, 1, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        self.lse = torch.empty((self.LAYERS, 1, W.HQ), dtype=torch.float32, device=dev)
        self.graphs = {False: [], True: []}
        torch.cuda.synchronize()
        for fused in (False, True):
            for r in range(self.SLOTS):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    self._calls(r, fused=fused)
                self.graphs[fused].append(g)
        torch.cuda.synchronize()
        self.samples = {"eager_ms": None, "graph_ms": None, "eager_fused_ms": None, "graph_fused_ms": None,
                        "decode_call_ms": []}
        self.n_steps = 0

    def _calls(self, r, events=None, fused=False):
        mtd = self.mtd
        for l in range(self.LAYERS):
            if fused:
                mtd.mtd_attn_decode_append(self.k[l], self.v[l], self.q[r, l], self.k_new[r, l], self.v_new[r, l],
                                           self.len, self.bt, self.max_len, W.SCALE, self.ws, self.o[l], self.lse[l])
                continue
            mtd.mtd_kv_append(self.k[l], self.v[l], self.k_new[r, l], self.v_new[r, l], self.cu, self.pos, self.bt)
            if events is not None: events[l][0].record()
            mtd.mtd_attn_decode(self.k[l], self.v[l], self.q[r, l], self.len, self.bt, self.max_len, W.SCALE,
                                self.ws, self.o[l], self.lse[l])
            if events is not None: events[l][1].record()
        self.pos.add_(1)
        self.len.add_(1)

    def _reset(self):
        self.pos.fill_(self.l0)
        self.len.fill_(self.l0 + 1)

    def _pass(self, n, graph, events=None, fused=False):
        for s in range(n):
            if graph:
                self.graphs[fused][s % self.SLOTS].replay()
            else:
                ev = None
                if events is not None:
                    ev = [[self.torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(self.LAYERS)]
                    events.append(ev)
                self._calls(s % self.SLOTS, ev, fused=fused)

    def run(self, steps, warmup):
        """Eager and graph passes of `steps` steps each, after `warmup` untimed steps of each mode.
        Returns the graph pass's wall seconds; the eager wall time and per-call decode kernel times
        (HIP events, from a third, eager pass) go into the results."""
        torch = self.torch
        if steps > self.ROOM:
            raise SystemExit(f"--steps {steps} exceeds the {self.ROOM} tokens of room per pass")
        walls = {}
        for fused in (False, True):
            for graph in (False, True):
                self._reset()
                self._pass(min(warmup, self.ROOM), graph, fused=fused)
                self._reset()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                self._pass(steps, graph, fused=fused)
                torch.cuda.synchronize()
                walls[(fused, graph)] = time.perf_counter() - t0
        self._reset()
        events = []
        self._pass(steps, False, events)
        torch.cuda.synchronize()
        self.samples["decode_call_ms"] = [e[0].elapsed_time(e[1]) for ev in events for e in ev]
        self.samples["eager_ms"] = walls[(False, False)] * 1e3 / steps
        self.samples["graph_ms"] = walls[(False, True)] * 1e3 / steps
        self.samples["eager_fused_ms"] = walls[(True, False)] * 1e3 / steps
        self.samples["graph_fused_ms"] = walls[(True, True)] * 1e3 / steps
        self.n_steps = steps
        return walls[(False, True)]

    def config(self):
        return {"workload": "decode_graph: 1 request (439-token context growing by one token per step) through "
                            "28 layers; step = 28 x (append 1 token, decode); eager calls vs one HIP-graph replay",
                "layers": self.LAYERS, "batch": 1, "initial_kv_tokens": self.l0}

    def results(self):
        n = self.n_steps
        lens = self.l0 + 1 + np.arange(n)
        step_bytes = float(np.mean([self.LAYERS * decode_bytes([x]) for x in lens]))
        call_ms = float(np.mean(self.samples["decode_call_ms"]))
        call_gbs = (step_bytes / self.LAYERS) / (call_ms * 1e-3) / 1e9
        g, e = self.samples["graph_ms"], self.samples["eager_ms"]
        return {"decode": {"value": call_gbs, "unit": "GB/s", "frac": call_gbs / HBM_PEAK_GBS, "ms": call_ms,
                           "bytes": step_bytes / self.LAYERS,
                           "kernels": "decode_split_kernel + decode_merge_kernel (per layer call, eager pass)"},
                "step": {"eager_ms": e, "graph_ms": g, "graph_speedup": e / g,
                         "graph_step_gbs": step_bytes / (g * 1e-3) / 1e9, "launches_per_step": 3 * self.LAYERS + 2},
                "step_fused": {"eager_ms": self.samples["eager_fused_ms"], "graph_ms": self.samples["graph_fused_ms"],
                               "graph_speedup_vs_unfused_graph": g / self.samples["graph_fused_ms"],
                               "launches_per_step": 2 * self.LAYERS + 2,
                               "calls": "mtd_attn_decode_append (store + decode split, merge) per layer"}}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": res["decode"]["bytes"], "ms": res["decode"]["ms"]}


class DecodeGraphBuckets:
    """Decode batches padded to buckets (1, 2, 4, .., 64 requests), one captured graph per bucket,
    as a serving loop replays one graph per token: a step is 28 x (append one token per request,
    decode) with the batch's requests first and padding requests (no token, zero keys) after them.
    Cases: every bucket full at the tiny workload's short context (launch-bound), 12 requests in
    the 16-bucket and 48 in the 64-bucket (padded), decode16's 16 requests of 27,000-30,000 tokens,
    and the full-depth batch (64 requests, log-uniform up to the 128K cap).  Each case is timed as
    eager calls and as graph replays.  The 28 layers of a case share one pool (timing only: each
    layer's KV is larger than the caches, so the bytes moved are those of 28 separate layers)."""
    name = "decode_graph_buckets"
    LAYERS = 28

    def __init__(self, dev):
        import torch
        import gqa_kv_cache_qwen3_amd as mtd
        self.mtd, self.torch, self.dev = mtd, torch, dev
        tiny = W.TINY.params["prompt"]
        p16, pf = W.DECODE16.params, W.FULLDEPTH.params
        self.cases = [(f"{b} x {tiny} tokens", b, np.full(b, tiny)) for b in (1, 2, 4, 8, 16, 32, 64)]
        self.cases += [("12 x 439 tokens (padded to 16)", 16, np.full(12, tiny)),
                       ("48 x 439 tokens (padded to 64)", 64, np.full(48, tiny)),
                       ("decode16: 16 x 27k-30k tokens", 16,
                        W.uniform_lengths(p16["batch"], p16["lo"], p16["hi"], W.DECODE16.tag, 0)),
                       ("full-depth batch: 64 x 4k-128k tokens", 64,
                        W.loguniform_lengths(pf["batch"], pf["lo"], W.CONTEXT_CAP - pf["steps"], W.FULLDEPTH.tag, 0))]
        self.rows = []

    def _case(self, label, bucket, lens0, steps, warmup):
        torch, mtd, dev = self.torch, self.mtd, self.dev
        b = len(lens0)
        room = steps + warmup + 1
        tables, n_pages, _ = W.place_pages(lens0 + room, 70, bucket)
        bound = int(lens0.max()) + room
        stride = (bound + W.PAGE - 1) // W.PAGE
        bt = torch.zeros((bucket, stride), dtype=torch.int32, device=dev)
        bt[:b, : tables.shape[1]] = torch.as_tensor(tables, device=dev)
        k = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        v = torch.empty_like(k)
        fill_normal_(k, W.torch_seed(70, bucket, 1))
        fill_normal_(v, W.torch_seed(70, bucket, 2))
        q = W.normal_bf16((self.LAYERS, bucket, W.HQ, W.HEAD_DIM), W.torch_seed(70, bucket, 3), dev)
        kn = W.normal_bf16((self.LAYERS, bucket, W.HKV, W.HEAD_DIM), W.torch_seed(70, bucket, 4), dev)
        vn = W.normal_bf16((self.LAYERS, bucket, W.HKV, W.HEAD_DIM), W.torch_seed(70, bucket, 5), dev)
        cu = torch.as_tensor(np.minimum(np.arange(bucket + 1), b).astype(np.int32), device=dev)
        pos = torch.as_tensor(np.concatenate([lens0, np.zeros(bucket - b)]).astype(np.int32), device=dev)
        lens = torch.as_tensor(np.concatenate([lens0 + 1, np.zeros(bucket - b)]).astype(np.int32), device=dev)
        step_add = torch.as_tensor((np.arange(bucket) < b).astype(np.int32), device=dev)
        ws = torch.empty(mtd.decode_workspace_bytes(bucket, bound), dtype=torch.uint8, device=dev)
        o = torch.empty((self.LAYERS, bucket, W.HQ, W.HEAD_DIM), dtype=torch.float32, device=dev)
        lse = torch.empty((self.LAYERS, bucket, W.HQ), dtype=torch.float32, device=dev)

        def calls(fused=False):
            for l in range(self.LAYERS):
                if fused:  # padding requests (length 0) store nothing, as with the two calls
                    mtd.mtd_attn_decode_append(k, v, q[l], kn[l], vn[l], lens, bt, bound, W.SCALE, ws, o[l], lse[l])
                    continue
                mtd.mtd_kv_append(k, v, kn[l], vn[l], cu, pos, bt)
                mtd.mtd_attn_decode(k, v, q[l], lens, bt, bound, W.SCALE, ws, o[l], lse[l])
            pos.add_(step_add)
            lens.add_(step_add)

        def reset():
            pos.copy_(torch.as_tensor(np.concatenate([lens0, np.zeros(bucket - b)]).astype(np.int32), device=dev))
            lens.copy_(torch.as_tensor(np.concatenate([lens0 + 1, np.zeros(bucket - b)]).astype(np.int32),
                                       device=dev))

        torch.cuda.synchronize()
        graphs = {}
        for fused in (False, True):
            graphs[fused] = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graphs[fused]):
                calls(fused)
        out = {}
        for name, use_graph, fused in (("eager_ms", False, False), ("graph_ms", True, False),
                                       ("graph_fused_ms", True, True)):
            reset()
            for _ in range(warmup):
                graphs[fused].replay() if use_graph else calls(fused)
            reset()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                graphs[fused].replay() if use_graph else calls(fused)
            torch.cuda.synchronize()
            out[name] = (time.perf_counter() - t0) * 1e3 / steps
        step_bytes = self.LAYERS * decode_bytes(lens0 + 1 + steps // 2)
        del graphs, k, v
        torch.cuda.empty_cache()
        return {"case": label, "bucket": bucket, "requests": b, "kv_tokens": int(lens0.sum()),
                "eager_ms": out["eager_ms"], "graph_ms": out["graph_ms"], "speedup": out["eager_ms"] / out["graph_ms"],
                "graph_gbs": step_bytes / (out["graph_ms"] * 1e-3) / 1e9, "graph_fused_ms": out["graph_fused_ms"],
                "fused_speedup": out["graph_ms"] / out["graph_fused_ms"]}

    def run(self, steps, warmup):
        t0 = time.perf_counter()
        for label, bucket, lens0 in self.cases:
            n = steps if int(lens0.max()) < 10000 else max(3, steps // 50)
            self.rows.append(self._case(label, bucket, np.asarray(lens0, dtype=np.int64), n, min(warmup, n)))
            print(f"[decode_graph_buckets] {self.rows[-1]}", file=sys.stderr, flush=True)
        return time.perf_counter() - t0

    def config(self):
        return {"workload": "decode_graph_buckets: decode batches padded to buckets 1..64, one HIP graph per bucket, "
                            "28 x (append, decode) per step; eager calls vs graph replays, and graph replays of "
                            "28 x mtd_attn_decode_append",
                "layers": self.LAYERS, "cases": [c[0] for c in self.cases]}

    def results(self):
        d16 = [r for r in self.rows if r["case"].startswith("decode16")][0]
        return {"decode": {"value": d16["graph_gbs"], "unit": "GB/s", "frac": d16["graph_gbs"] / HBM_PEAK_GBS,
                           "ms": d16["graph_ms"] / self.LAYERS, "bytes": None,
                           "kernels": "decode_split_kernel + decode_merge_kernel (decode16 in its bucket, graph)"},
                "buckets": self.rows}

    def dominant(self, res):
        return {"kernel": "decode_split_kernel+decode_merge_kernel", "bound": "hbm", "achieved": res["decode"]["value"],
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "per_launch": None, "ms": res["decode"]["ms"]}


class DecodeGraphBlock(DecodeGraph):
    """decode_graph with the projections: per layer the QKV projection of the request's hidden state,
    the append of its new K/V, decode attention and the output projection, whose result is the next
    layer's input; eager calls against one HIP-graph replay per step."""
    name = "decode_graph_block"

    def __init__(self, dev):
        import torch
        self.w = [W.projection_weights(W.torch_seed(W.TINY.tag, 70, l), dev) for l in range(self.LAYERS)]
        self.x0 = W.normal_bf16((self.SLOTS, 1, W.HIDDEN), W.torch_seed(W.TINY.tag, 71), dev)
        self.qb = torch.empty((1, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.kb = torch.empty((1, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device=dev)
        self.vb = torch.empty_like(self.kb)
        self.xb = torch.empty((1, W.HIDDEN), dtype=torch.bfloat16, device=dev)
        super().__init__(dev)

    def _calls(self, r, events=None, fused=False):
        mtd = self.mtd
        x = self.x0[r]
        for l in range(self.LAYERS):
            w_qkv, w_o = self.w[l]
            mtd.mtd_qkv_proj(x, w_qkv, self.qb, self.kb, self.vb)
            if fused:
                mtd.mtd_attn_decode_append(self.k[l], self.v[l], self.qb, self.kb, self.vb, self.len, self.bt,
                                           self.max_len, W.SCALE, self.ws, self.o[l], self.lse[l])
            else:
                mtd.mtd_kv_append(self.k[l], self.v[l], self.kb, self.vb, self.cu, self.pos, self.bt)
                if events is not None: events[l][0].record()
                mtd.mtd_attn_decode(self.k[l], self.v[l], self.qb, self.len, self.bt, self.max_len, W.SCALE,
                                    self.ws, self.o[l], self.lse[l])
                if events is not None: events[l][1].record()
            mtd.mtd_o_proj(self.o[l], w_o, self.xb)
            x = self.xb
        self.pos.add_(1)
        self.len.add_(1)

    def config(self):
        c = super().config()
        c["workload"] = ("decode_graph_block: 1 request (439-token context growing by one token per step) through "
                         "28 attention blocks; step = 28 x (QKV projection, append, decode, output projection; "
                         "random bf16 weights); eager calls vs one HIP-graph replay, with append and decode as "
                         "two calls and as mtd_attn_decode_append")
        c["hidden"] = W.HIDDEN
        return c

    def results(self):
        res = super().results()
        res["step"]["launches_per_step"] = 5 * self.LAYERS + 2
        res["step_fused"]["launches_per_step"] = 4 * self.LAYERS + 2
        return res


WORKLOAD_CLASSES = {c.name: c for c in (Tiny, MixedStep, MixedStepOverlap, MixedBlock, Decode16, Decode16SeqSplit, Prefill90,
                                         FullDepth, FullDepthBlock, DecodeGraph, DecodeGraphBlock,
                                         DecodeGraphBuckets)}


def calibrate_copy():
    """A plain copy kernel of known size: 1 GiB read + 1 GiB written per launch, 5 launches."""
    import torch
    n = 1 << 28  # float32 elements = 1 GiB
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy": {"read_bytes_per_launch": 4 * n, "write_bytes_per_launch": 4 * n,
                                         "launches": 5, "kernel": "vectorized_elementwise_kernel (mul)"}}))


# --------------------------------------------------------------------------------------------
# the other target configurations and the practical ceiling, reported beside the default line
# --------------------------------------------------------------------------------------------

def _mean_event_ms(pairs):
    return float(np.mean([a.elapsed_time(b) for a, b in pairs]))


def extra_prefill90(dev, passes=5, warmup=3):
    """The 90-minute prompt (17 chunks, 67,500 tokens, peaked keys): aggregate prefill TFLOP/s."""
    import torch
    wl = Prefill90(dev)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    evs = [wl.timed_step() for _ in range(passes)]
    torch.cuda.synchronize()
    ms = float(np.mean([sum(e[1].elapsed_time(e[2]) for e in ev) for ev in evs]))
    tfs = wl.flops / (ms * 1e-3) / 1e12
    out = {"value": tfs, "unit": "TFLOP/s", "frac": tfs / MFMA_BF16_PEAK_TFLOPS, "ms_per_pass": ms,
           "flops": wl.flops, "passes": passes, "chunks": len(wl.chunks),
           "kernels": "prefill_kernel + prefill_merge_kernel (17 calls)"}
    del wl
    return out


def extra_decode16(dev, steps=20, warmup=500):
    """16 requests of 27,000-30,000 tokens: decode GB/s.  Returns (line object, workload)."""
    import torch
    wl = Decode16(dev)
    for _ in range(warmup):
        wl.step()
    torch.cuda.synchronize()
    all_evs = []
    for _ in range(steps):
        evs = wl.timer.step_events()
        wl.step(evs)
        all_evs.append(evs)
    torch.cuda.synchronize()
    for evs in all_evs:
        wl.timer.collect(evs)
    res = wl.results()["decode"]
    return {"value": res["value"], "unit": "GB/s", "frac": res["frac"], "ms": res["ms"], "bytes": res["bytes"],
            "steps": steps, "kernels": "decode_split_kernel + decode_merge_kernel"}, wl


def ceiling(dev, dec16, copy_bytes=4 << 30, reps=10):
    """What HBM gives on this device, measured here: a device-to-device copy of 4 GiB (bytes read +
    bytes written per second) and mtd_measure_page_read over decode16's pages (the decode's own
    access pattern: K and V page blocks in table order, 8 pages per wave, no arithmetic)."""
    import torch
    mtd = dec16.mtd
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    pairs = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    copy_ms = _mean_event_ms(pairs)
    del src, dst
    tables = dec16.bt.cpu().numpy()
    ids = np.concatenate([tables[b][: (int(n) + W.PAGE - 1) // W.PAGE] for b, n in enumerate(dec16.lens)])
    ids_t = torch.as_tensor(ids.astype(np.int32), device=dev)
    sink = mtd.mtd_measure_page_read(dec16.k, dec16.v, ids_t, 8)
    for _ in range(20):
        mtd.mtd_measure_page_read(dec16.k, dec16.v, ids_t, 8, sink)
    pairs = []
    for _ in range(reps * 5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mtd.mtd_measure_page_read(dec16.k, dec16.v, ids_t, 8, sink)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    read_ms = _mean_event_ms(pairs)
    read_bytes = len(ids) * KV_BYTES_PER_TOKEN * W.PAGE
    copy_gbs = 2 * copy_bytes / (copy_ms * 1e-3) / 1e9
    read_gbs = read_bytes / (read_ms * 1e-3) / 1e9
    return {"copy_gbs": copy_gbs, "copy_bytes_each_way": copy_bytes, "copy_ms": copy_ms,
            "page_read_gbs": read_gbs, "page_read_bytes": read_bytes, "page_read_ms": read_ms,
            "page_read_frac": read_gbs / HBM_PEAK_GBS, "unit": "GB/s",
            "kernels": "hipMemcpy D2D (torch copy_); page_read_kernel (mtd_measure_page_read)"}


# Untimed steps per workload, each about 50 ms of GPU work or more.
WARMUP_DEFAULT = {"tiny": 20, "decode_graph_buckets": 20, "mixed_step": 40, "mixed_step_overlap": 40, "mixed_block": 40, "decode16": 500,
                  "prefill90min": 3, "fulldepth_decode": 5, "fulldepth_block": 5, "decode_graph": 200,
                  "decode_graph_block": 200, "decode16_seqsplit": 2000}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 20; 128 for fulldepth_decode)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed steps (default: enough for ~50 ms of GPU work, past the clock ramp)")
    ap.add_argument("--workload", default="mixed_step", choices=sorted(WORKLOAD_CLASSES))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing on the host")
    ap.add_argument("--results-json", default=None,
                    help="also write a results record (the line, device, seeds, lengths, parity of this run's "
                         "outputs against the oracle) to this path")
    ap.add_argument("--no-extras", action="store_true",
                    help="default workload only: skip the 90-minute prefill, decode16 and ceiling objects")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 1 GiB elementwise copy 5 times (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.calibrate_copy:
        calibrate_copy()
        return

    if args.steps is None:
        args.steps = {"fulldepth_decode": 128, "fulldepth_block": 128, "decode_graph": 500,
                      "decode_graph_block": 500, "decode_graph_buckets": 200}.get(args.workload, 20)
    if args.warmup is None:
        # From idle the shader clock needs about 20 ms of sustained work to reach its steady level
        # (measured on MI355X); the default warmup covers that with margin.
        args.warmup = WARMUP_DEFAULT[args.workload]
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: this path runs on one GPU; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    import torch
    import gqa_kv_cache_qwen3_amd as mtd
    mtd.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    wl = WORKLOAD_CLASSES[args.workload](dev)
    torch.cuda.synchronize()
    if not isinstance(wl, (DecodeGraph, DecodeGraphBuckets)):
        evented = not isinstance(wl, (FullDepth, Prefill90))
        for _ in range(args.warmup):
            # The timed steps record HIP events; the warm-up records them too, since the first few dozen
            # timing events of a process have been seen to slow the launches around them (about 3x for
            # the launch-bound tiny workload) when they fell in the timed region.
            wl.step(wl.timer.step_events() if evented else None)
    torch.cuda.synchronize()
    if isinstance(wl, FullDepth):
        wl.step_idx = 0  # the timed pass starts again at step 0 (appends rewrite the same slots)

    # timed region: exactly K steps between synchronisations; per-call events inside
    t0 = time.perf_counter()
    if isinstance(wl, (DecodeGraph, DecodeGraphBuckets)):
        wall = wl.run(args.steps, args.warmup)  # warm-up and the eager passes happen inside; graph pass timed
    elif isinstance(wl, FullDepth):
        step_events = []
        for _ in range(args.steps):
            wl.step(step_events)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        wl.collect(step_events)
    elif isinstance(wl, Prefill90):
        all_evs = []
        for _ in range(args.steps):
            all_evs.append(wl.timed_step())
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for evs in all_evs:
            app = sum(e[0].elapsed_time(e[1]) for e in evs)
            pre = sum(e[1].elapsed_time(e[2]) for e in evs)
            wl.timer.samples["append"].append(app)
            wl.timer.samples["prefill"].append(pre)
    else:
        all_evs = []
        for _ in range(args.steps):
            evs = wl.timer.step_events()
            wl.step(evs)
            all_evs.append(evs)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        for evs in all_evs:
            wl.timer.collect(evs)
    ms_per_step = wall * 1e3 / args.steps

    res = wl.results()
    dom = wl.dominant(res)
    if "decode" in res:
        value, unit = res["decode"]["value"], "GB/s"
    else:
        value, unit = res["prefill"]["value"], "TFLOP/s"
    line = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 Q/K/V, seeded page placement; no trained weights)",
        "config": wl.config(),
        "roofline": {
            "kernel": dom["kernel"], "bound": dom["bound"], "achieved": round(dom["achieved"], 3),
            "peak": dom["peak"], "unit": dom["unit"], "frac": round(dom["achieved"] / dom["peak"], 4),
            "traffic": recorded_traffic(dom["kernel"], wl.name), "avg_ms": round(dom["ms"], 5),
            "per_launch": dom["per_launch"], "source_digest": source_digest(dom["kernel"]),
        },
    }
    for k in ("decode", "prefill", "append", "step", "step_fused", "eager"):
        if k in res:
            line[k] = {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in res[k].items()}
    if "buckets" in res:
        line["buckets"] = [{kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in r.items()}
                           for r in res["buckets"]]
    if "proj" in res:
        line["proj"] = {name: {kk: (round(vv, 5) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                        for name, d in res["proj"].items()}
    if type(wl) is MixedStep and not args.no_extras:
        # the other configurations that carry the targets, and the measured ceiling
        line["prefill90min"] = {k: (round(v, 5) if isinstance(v, float) else v)
                                for k, v in extra_prefill90(dev).items()}
        d16, dec16 = extra_decode16(dev)
        line["decode16"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in d16.items()}
        ceil = ceiling(dev, dec16)
        ceil["decode_frac_of_page_read"] = res["decode"]["value"] / ceil["page_read_gbs"]
        ceil["decode16_frac_of_page_read"] = d16["value"] / ceil["page_read_gbs"]
        line["ceiling"] = {k: (round(v, 5) if isinstance(v, float) else v) for k, v in ceil.items()}
        del dec16
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline and getattr(wl, "cpu_baseline", None) is not None:
        line["cpu_baseline"] = wl.cpu_baseline()
    print(json.dumps(line), flush=True)
    if args.results_json:
        write_record(args.results_json, line, wl, dev)


def write_record(path, line, wl, dev):
    """The per-configuration results record: the bench line, the device, and (where the workload has
    one) its seeds, length summary and the parity of this run's outputs against the fp64 oracle."""
    import platform
    import torch
    from oracle.parallel import OraclePool, cpu_model
    prop = torch.cuda.get_device_properties(dev)
    free, total = torch.cuda.mem_get_info(dev)
    rec = {"line": line,
           "device": {"name": prop.name, "arch": getattr(prop, "gcnArchName", ""), "compute_units": prop.multi_processor_count,
                      "memory_total": int(total), "memory_free_at_end": int(free), "torch": torch.__version__,
                      "hip": torch.version.hip, "host": platform.node(), "cpu_model": cpu_model()},
           "gates": {"max_abs_dO": 1e-2, "max_abs_dLSE": 1e-3}}
    if getattr(wl, "record", None) is not None:
        with OraclePool() as pool:
            rec.update(wl.record(pool))
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(f"bench.py: results record written to {path}", file=sys.stderr)


if __name__ == "__main__":
    main()
