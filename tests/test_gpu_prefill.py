"""mtd_attn_prefill_chunk on the GPU against the fp64 oracle: one-shot and chunked prefill over
pages written by mtd_kv_append, at small ragged shapes in full; the mixed step's 4096-token chunk
and the 90-minute prompt's chunks 0, 8 and 16 on every row (the oracle spread over a process
pool), its other chunks and the 128K-cap chunks on sampled rows; plus chunked == one-shot and
decode == 1-row prefill.  The
checks run both without a workspace (one pass per position tile) and with one (the causal work
rebalanced over the compute units: tiles t and T-1-t paired into two equal workgroups, or each
tile's keys in two halves for short chunks; split tiles merged by log-sum-exp)."""

import hashlib

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import bits, compare, log, new_pool, request_pages_host
from oracle.parallel import prefill_problem

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


class Request:
    """One request's paged KV, filled through mtd_kv_append (the path under test)."""

    def __init__(self, total: int, tag: int, lowrank: bool = False, spare: int = 2, split: bool = False,
                 cu_budget: int = 0):
        self.total = total
        self.split = split or cu_budget > 0
        self.cu_budget = cu_budget
        tables, self.num_pages, self.spare = W.place_pages([total], tag, 0, spare=spare)
        self.table_np = tables[0]
        self.table = torch.as_tensor(self.table_np, device="cuda")
        self.k = new_pool(self.num_pages, "cuda")
        self.v = new_pool(self.num_pages, "cuda")
        if lowrank:
            self.k_log = W.lowrank_keys(total, W.torch_seed(tag, 1), "cuda")
        else:
            self.k_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 1), "cuda")
        self.v_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 2), "cuda")
        self.q_log = W.normal_bf16((total, W.HQ, W.HEAD_DIM), W.torch_seed(tag, 3), "cuda")
        self.filled = 0

    def append_to(self, end: int):
        start = self.filled
        if end <= start:
            return
        mtd.mtd_kv_append(self.k, self.v, self.k_log[start:end].contiguous(),
                          self.v_log[start:end].contiguous(),
                          torch.tensor([0, end - start], dtype=torch.int32, device="cuda"),
                          torch.tensor([start], dtype=torch.int32, device="cuda"),
                          self.table[None, :].contiguous())
        self.filled = end

    def prefill(self, prefix: int, chunk: int):
        self.append_to(prefix + chunk)
        ws = None
        if self.split:
            ws = torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda")
        q = self.q_log[prefix:prefix + chunk].contiguous()
        if self.cu_budget:
            out, lse = mtd.mtd_attn_prefill_chunk_cus(self.k, self.v, q, prefix, self.table, W.SCALE, ws,
                                                      self.cu_budget)
        else:
            out, lse = mtd.mtd_attn_prefill_chunk(self.k, self.v, q, prefix, self.table, W.SCALE, workspace=ws)
        torch.cuda.synchronize()
        return out, lse

    def reference(self, prefix: int, chunk: int, rows=None):
        """Oracle over the request's pages as they sit on the device (rows: chunk-local indices)."""
        kc, vc, ident = request_pages_host(self.k, self.v, self.table_np, prefix + chunk)
        q = bits(self.q_log[prefix:prefix + chunk])
        if rows is None:
            return oracle.prefill_chunk(q, kc, vc, ident, prefix, W.SCALE)
        rows = np.asarray(rows)
        k = oracle.gather_logical(kc, ident, prefix + chunk)
        v = oracle.gather_logical(vc, ident, prefix + chunk)
        return oracle.attention(oracle.bf16_to_f64(q[rows]), k, v, prefix + rows, W.SCALE)


SPLIT = pytest.mark.parametrize("split", [False, True], ids=["one-pass", "split"])


@SPLIT
@pytest.mark.parametrize("prefix,chunk", [(0, 1), (0, 64), (0, 65), (5, 1), (63, 2), (50, 37), (100, 37),
                                          (64, 64), (500, 300), (1000, 300), (0, 439), (4096, 4096),
                                          (100, 4200), (0, 8192)])
def test_prefill_small_full_compare(prefix, chunk, split):
    log(f"prefill prefix={prefix} chunk={chunk} split={split}")
    req = Request(prefix + chunk, 200 + prefix + 7 * chunk, split=split)
    out, lse = req.prefill(prefix, chunk)
    o_ref, l_ref = req.reference(prefix, chunk)
    compare(out, lse, o_ref, l_ref, f"prefill P={prefix} C={chunk}{' split' if split else ''}")


def test_tiny_one_shot_then_decode_steps():
    """30 s of audio + 64 prompt tokens: one-shot 439-token prefill, then 32 decode steps, each
    appending its token first; every step against the oracle."""
    prompt, steps = W.TINY.params["prompt"], W.TINY.params["decode_steps"]
    req = Request(prompt + steps, W.TINY.tag)
    log("tiny one-shot prefill")
    out, lse = req.prefill(0, prompt)
    o_ref, l_ref = req.reference(0, prompt)
    compare(out, lse, o_ref, l_ref, "tiny one-shot")
    for s in range(steps):
        n = prompt + s + 1
        req.append_to(n)
        q = req.q_log[n - 1:n].contiguous()
        log(f"tiny decode step {s}")
        o, l = mtd.mtd_attn_decode(req.k, req.v, q, torch.tensor([n], dtype=torch.int32, device="cuda"),
                                   req.table[None, :].contiguous(), n, W.SCALE)
        torch.cuda.synchronize()
        kc, vc, ident = request_pages_host(req.k, req.v, req.table_np, n)
        o_ref, l_ref = oracle.decode(bits(q), kc, vc, [n], [ident], W.SCALE)
        compare(o, l, o_ref, l_ref, f"tiny decode step {s}")


@SPLIT
def test_gpu_chunked_matches_gpu_one_shot(split):
    """The tiny prompt as chunks of 128 + 128 + 128 + 55 against one 439-token call."""
    req = Request(439, 301, split=split)
    one_o, one_l = req.prefill(0, 439)
    parts_o, parts_l = [], []
    for start, c in [(0, 128), (128, 128), (256, 128), (384, 55)]:
        o, l = req.prefill(start, c)
        parts_o.append(o)
        parts_l.append(l)
    o = torch.cat(parts_o)
    l = torch.cat(parts_l)
    assert float((o - one_o).abs().max()) <= 1e-2 * 0.1
    assert float((l - one_l).abs().max()) <= 1e-3 * 0.1


def test_decode_equals_one_row_prefill():
    req = Request(3000, 302)
    o_p, l_p = req.prefill(2999, 1)
    q = req.q_log[2999:3000].contiguous()
    o_d, l_d = mtd.mtd_attn_decode(req.k, req.v, q, torch.tensor([3000], dtype=torch.int32, device="cuda"),
                                   req.table[None, :].contiguous(), 3000, W.SCALE)
    torch.cuda.synchronize()
    assert float((o_p - o_d).abs().max()) <= 1e-3
    assert float((l_p - l_d).abs().max()) <= 1e-4


def sample_rows(chunk: int, tag: int, n: int = 40) -> np.ndarray:
    """First, last, a few around the 64-row tile edges, and seeded random rows."""
    fixed = [0, 1, 15, 16, 63, 64, chunk // 2, chunk - 2, chunk - 1]
    rnd = W.rng(9, tag).choice(chunk, size=min(n, chunk), replace=False).tolist()
    return np.array(sorted({r for r in fixed + rnd if 0 <= r < chunk}))


# Oracle results of full chunks, shared by the one-pass and split runs of the same inputs (keyed
# by a digest of the exact bits the oracle read).
_FULL_REF = {}


def full_reference(pool, q_bits, kc, vc, table, prefix):
    h = hashlib.blake2b(digest_size=16)
    for a in (q_bits, kc, vc, np.asarray(table, dtype=np.int64)):
        h.update(np.ascontiguousarray(a).view(np.uint8))
    h.update(str(prefix).encode())
    key = h.hexdigest()
    if key not in _FULL_REF:
        [_FULL_REF[key]] = pool.attention([prefill_problem(q_bits, kc, vc, table, prefix)], W.SCALE)
    return _FULL_REF[key]


P90_FULL_CHUNKS = (0, 8, 16)  # first chunk, the middle one (prefix 32,768) and the partial last one


@SPLIT
def test_prefill_90_minutes_chunked(split, oracle_pool):
    """67,500 tokens in 17 chunks of 4096 (last 1,964), K with a rank-4 per-head component so the
    softmax is peaked.  Chunks 0, 8 and 16 are compared with the oracle on every row; the other 14
    on 40 sampled rows each (first, last, tile edges and seeded random rows)."""
    p = W.PREFILL90.params
    total, chunk = p["total"], p["chunk"]
    req = Request(total, W.PREFILL90.tag, lowrank=True, split=split)
    req.append_to(total)
    torch.cuda.synchronize()
    kc, vc, ident = request_pages_host(req.k, req.v, req.table_np, total)
    k = oracle.gather_logical(kc, ident, total)
    v = oracle.gather_logical(vc, ident, total)
    qb = bits(req.q_log)
    for ci, start in enumerate(range(0, total, chunk)):
        c = min(chunk, total - start)
        log(f"prefill90 chunk {ci} prefix={start} len={c} split={split}")
        out, lse = req.prefill(start, c)
        if ci in P90_FULL_CHUNKS:
            used = (start + c + W.PAGE - 1) // W.PAGE
            o_ref, l_ref = full_reference(oracle_pool, qb[start:start + c], kc[:used], vc[:used], ident[:used], start)
            compare(out, lse, o_ref, l_ref, f"prefill90 chunk {ci}, all {c} rows{' split' if split else ''}")
        else:
            rows = sample_rows(c, ci)
            o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(qb[start + rows]), k, v, start + rows, W.SCALE)
            compare(out[rows], lse[rows], o_ref, l_ref, f"prefill90 chunk {ci}{' split' if split else ''}")


@SPLIT
def test_mixed_step_prefill_part_all_rows(split, oracle_pool):
    """The mixed step's chunk: 4096 tokens of request A at prefix 32,768, every row."""
    p = W.MIXED.params
    prefix, chunk = p["prefix"], p["chunk"]
    req = Request(prefix + chunk, W.MIXED.tag, split=split)
    log(f"mixed prefill part split={split}")
    out, lse = req.prefill(prefix, chunk)
    kc, vc, ident = request_pages_host(req.k, req.v, req.table_np, prefix + chunk)
    o_ref, l_ref = full_reference(oracle_pool, bits(req.q_log[prefix:prefix + chunk]), kc, vc, ident, prefix)
    compare(out, lse, o_ref, l_ref, f"mixed prefill part, all rows{' split' if split else ''}")


@SPLIT
@pytest.mark.parametrize("chunk", [4096, 1000])
def test_prefill_at_the_context_cap(chunk, split):
    """The last chunk of a 131,072-token context (the 128K cap): a full 4096-token chunk and a
    1000-token one (fewer tiles than CUs, so the workspace path splits it), sampled rows."""
    total = W.CONTEXT_CAP
    prefix = total - chunk
    req = Request(total, 310 + chunk, split=split)
    log(f"prefill at the cap: prefix={prefix} chunk={chunk} split={split}")
    out, lse = req.prefill(prefix, chunk)
    rows = sample_rows(chunk, 311, 24)
    o_ref, l_ref = req.reference(prefix, chunk, rows)
    compare(out[rows], lse[rows], o_ref, l_ref, f"prefill cap C={chunk}{' split' if split else ''}")


@SPLIT
def test_prefill_deterministic_and_placement_invariant(split):
    a = Request(5000, 303, split=split)
    o1, l1 = a.prefill(1000, 4000)
    o2, l2 = a.prefill(1000, 4000)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # same logical data, different page placement
    b = Request(5000, 303, split=split)
    tables, _, _ = W.place_pages([5000], 304, 0, spare=2)
    b.table_np = tables[0]
    b.table = torch.as_tensor(b.table_np, device="cuda")
    o3, l3 = b.prefill(1000, 4000)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("cu_budget", [8, 64, 120, 240, 248])
@pytest.mark.parametrize("prefix,chunk", [(0, 439), (4096, 4096), (100, 4200), (0, 8192), (32768, 4096),
                                          (65536, 1964)])
def test_prefill_on_a_cu_budget(prefix, chunk, cu_budget, oracle_pool):
    """The spread schedule (mtd_attn_prefill_chunk_cus): each KV head's key tiles cut into
    cu_budget / 8 equal ranges, tiles cut by a range boundary merged; every row against the
    oracle, and the same bits on a second call."""
    log(f"prefill on a budget of {cu_budget} CUs: prefix={prefix} chunk={chunk}")
    req = Request(prefix + chunk, 500 + prefix % 997 + chunk, cu_budget=cu_budget)
    out, lse = req.prefill(prefix, chunk)
    out2, lse2 = req.prefill(prefix, chunk)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    kc, vc, ident = request_pages_host(req.k, req.v, req.table_np, prefix + chunk)
    o_ref, l_ref = full_reference(oracle_pool, bits(req.q_log[prefix:prefix + chunk]), kc, vc, ident, prefix)
    compare(out, lse, o_ref, l_ref, f"prefill P={prefix} C={chunk} on {cu_budget} CUs")
