"""Seeded synthetic inputs for the paged GQA attention path.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()``, and by both
sides of every parity check (the HIP library and the fp64 oracle).  It holds no
attention arithmetic and no paging arithmetic: only random draws, request
lengths and the seeded placement of pages in the pool.

Shapes follow the Qwen3 decoder of the pages (GQA 16/8, "Optimizing ASR Models
to Transcribe 90-Minute Multi-Speaker Audio", §ASR Model Primer component
table) with head_dim 128 and 64-token pages.  Lengths follow the pages'
workloads: about 12.5 decoder tokens per second of audio after the 4x time
merge ("MOSS-Transcribe-Diarize" cookbook, §Inference Pipeline, step 1), so
30 s of audio is 375 tokens, a 38-minute meeting about 28,500 and 90 minutes
67,500; prefill runs in 4096-token chunks (§Chunked Prefill for Long Audio);
16 concurrent requests (the benchmark setup's max_running_requests,
§Benchmark Results); 128K context cap (cookbook, §Model Architecture).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

HQ = 16          # query heads
HKV = 8          # key/value heads
HEAD_DIM = 128
HIDDEN = 1024    # decoder hidden size (input of the QKV projection, output of o_proj)
PAGE = 64        # tokens per page
SCALE = 1.0 / math.sqrt(HEAD_DIM)
CHUNK = 4096     # prefill chunk length
CONTEXT_CAP = 131072
BASE_SEED = 20261202


def rng(*tags: int) -> np.random.Generator:
    """Independent numpy stream for a (config, tensor, layer, step, ...) tag tuple."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([BASE_SEED, *tags])))


def torch_seed(*tags: int) -> int:
    """63-bit seed for a torch generator, derived from the same tag tuple."""
    return int(rng(*tags).integers(0, 2**63 - 1))


def uniform_lengths(n: int, lo: int, hi: int, *tags: int) -> np.ndarray:
    """Integers uniform on [lo, hi], both ends included."""
    return rng(*tags).integers(lo, hi + 1, size=n).astype(np.int64)


def loguniform_lengths(n: int, lo: int, hi: int, *tags: int) -> np.ndarray:
    """round(exp(U(ln lo, ln hi))), clipped to [lo, hi]."""
    u = rng(*tags).uniform(math.log(lo), math.log(hi), size=n)
    return np.clip(np.rint(np.exp(u)), lo, hi).astype(np.int64)


def pages_needed(n_tokens) -> np.ndarray:
    return (np.asarray(n_tokens, dtype=np.int64) + PAGE - 1) // PAGE


def place_pages(final_lengths, *tags: int, spare: int = 1):
    """Seeded page placement.

    The pool holds exactly the pages the requests need at their final lengths
    plus ``spare`` extra pages.  Physical page ids come from one seeded
    permutation of the pool, handed out in request order; the first ``spare``
    ids of the permutation are the spare pages.  Unused table entries point at
    the first spare page.

    Returns (block_tables int32 [R][stride], num_pages, spare_ids).
    """
    need = pages_needed(final_lengths)
    total = int(need.sum()) + spare
    perm = rng(*tags).permutation(total).astype(np.int64)
    spare_ids = perm[:spare]
    stride = max(1, int(need.max()) if len(need) else 1)
    tables = np.full((len(need), stride), spare_ids[0] if spare else 0, dtype=np.int32)
    cursor = spare
    for r, n in enumerate(need):
        tables[r, :n] = perm[cursor:cursor + n]
        cursor += int(n)
    return tables, total, spare_ids


def normal_bf16(shape, seed: int, device="cpu"):
    """fp32 N(0,1) cast to bf16 with round-to-nearest-even."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def normal_bf16_std(shape, std: float, seed: int, device="cpu"):
    """fp32 N(0, std^2) cast to bf16 with round-to-nearest-even (random projection weights use
    std = 1/sqrt(fan_in), so outputs keep the inputs' scale)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return (torch.randn(*shape, generator=gen, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def projection_weights(seed: int, device="cpu"):
    """Random bf16 weights of one layer's projections: W_qkv [(16 + 8 + 8) * 128][1024] (rows Wq,
    Wk, Wv) and W_o [1024][16 * 128], both in the [out][in] layout."""
    n_qkv = (HQ + 2 * HKV) * HEAD_DIM
    w_qkv = normal_bf16_std((n_qkv, HIDDEN), 1.0 / math.sqrt(HIDDEN), seed, device)
    w_o = normal_bf16_std((HIDDEN, HQ * HEAD_DIM), 1.0 / math.sqrt(HQ * HEAD_DIM), seed + 1, device)
    return w_qkv, w_o


def lowrank_keys(n_tokens: int, seed: int, device="cpu", rank: int = 4, weight: float = 2.0):
    """Keys with a per-KV-head low-rank component: K_g = Z + weight * A_g B_g.

    Z ~ N(0,1) [n][Hkv][D]; A ~ N(0,1) [n][Hkv][rank] are per-token coefficients;
    B ~ N(0,1) [Hkv][rank][D] are per-head directions.  Computed in fp32 and cast
    to bf16, so the scaled logits have a spread of about 4 instead of 1 and the
    softmax is peaked rather than near-uniform.
    """
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    z = torch.randn(n_tokens, HKV, HEAD_DIM, generator=gen, device=device, dtype=torch.float32)
    a = torch.randn(n_tokens, HKV, rank, generator=gen, device=device, dtype=torch.float32)
    b = torch.randn(HKV, rank, HEAD_DIM, generator=gen, device=device, dtype=torch.float32)
    # per head: [n][rank] @ [rank][D]
    low = torch.bmm(a.transpose(0, 1).contiguous(), b).transpose(0, 1)
    return (z + weight * low).to(torch.bfloat16)


# --------------------------------------------------------------------------------------
# The five workloads.  Each describes sizes and seeds only; tests and the bench build
# tensors from them.
# --------------------------------------------------------------------------------------

@dataclass
class Workload:
    name: str
    tag: int
    description: str
    params: dict = field(default_factory=dict)


TINY = Workload(
    "tiny", 1,
    "1 request: 30 s of audio (375 tokens) + 64 prompt tokens = 439-token one-shot "
    "causal prefill, then 32 decode steps; N(0,1) bf16; page 64, seeded random placement",
    dict(prompt=439, decode_steps=32),
)
DECODE16 = Workload(
    "decode16", 2,
    "batched decode, 1 layer: 16 requests (38-minute meetings), KV lengths uniform in "
    "[27000, 30000], one query token each; N(0,1) bf16; page 64, shuffled tables",
    dict(batch=16, lo=27000, hi=30000),
)
PREFILL90 = Workload(
    "prefill90min", 3,
    "chunked prefill, 1 layer: one 90-minute request of 67,500 tokens as 17 sequential "
    "4096-token chunks (last partial); K with a per-head rank-4 component of weight 2",
    dict(total=67500, chunk=CHUNK),
)
MIXED = Workload(
    "mixed_step", 4,
    "mixed scheduler step, 1 layer: one 4096-token prefill chunk at prefix 32,768 plus "
    "decode for 31 other requests with KV lengths log-uniform in [2000, 68000]; one "
    "shared pool of 64-token pages; N(0,1) bf16",
    dict(chunk=CHUNK, prefix=32768, batch=31, lo=2000, hi=68000),
)
FULLDEPTH = Workload(
    "fulldepth_decode", 5,
    "full-depth decode: 28 layers x 64 requests, KV lengths log-uniform in [4000, 131072] "
    "(128K cap; drawn in [4000, 131072-128] so 128 appended steps stay under the cap), "
    "all layers resident; each step appends 1 token per request, then decodes; 128 steps",
    dict(layers=28, batch=64, lo=4000, hi=CONTEXT_CAP, steps=128),
)

WORKLOADS = {w.name: w for w in (TINY, DECODE16, PREFILL90, MIXED, FULLDEPTH)}


# --------------------------------------------------------------------------------------
# Full-depth decode inputs (28 layers x 64 requests, all layers resident in HBM)
# --------------------------------------------------------------------------------------

def fulldepth_bytes(lens0, steps: int, layers: int) -> int:
    """Exact HBM bytes of the full-depth inputs: every layer's K+V pools, the per-step queries and
    new K/V rows, and one decode workspace."""
    b = len(lens0)
    pages = int(pages_needed(np.asarray(lens0) + steps).sum()) + 1
    pools = layers * pages * 2 * HKV * PAGE * HEAD_DIM * 2
    qs = steps * layers * b * HQ * HEAD_DIM * 2
    new = steps * layers * b * HKV * HEAD_DIM * 2 * 2
    max_len = int(np.max(lens0)) + steps
    ws = b * ((max_len + 511) // 512) * HQ * (HEAD_DIM + 1) * 4
    return pools + qs + new + ws


def fulldepth_draw(free_bytes: int, fraction: float = 0.95, max_tries: int = 8):
    """Draw initial KV lengths log-uniform in [4000, 131072 - steps]; if the inputs would not fit
    in fraction * free_bytes, redraw with the next seed (never truncating lengths).
    Returns (lens0, seeds_tried, bytes_needed)."""
    p = FULLDEPTH.params
    tried = []
    for t in range(max_tries):
        lens0 = loguniform_lengths(p["batch"], p["lo"], p["hi"] - p["steps"], FULLDEPTH.tag, t)
        need = fulldepth_bytes(lens0, p["steps"], p["layers"])
        tried.append(t)
        if need <= fraction * free_bytes:
            return lens0, tried, need
    raise MemoryError(f"full-depth inputs do not fit in {fraction} x {free_bytes} bytes after seeds {tried}")


def build_fulldepth(device, lens0, steps: int | None = None, layers: int | None = None):
    """Seeded full-depth tensors on `device`.

    Layer 0's pools are N(0,1) bf16 in every slot; layer l's pools are layer 0's rolled by l pages
    (so every layer holds different data at the cost of a copy instead of fresh draws).  All
    layers share one block table (same page ids, separate pools).  Queries and new K/V rows for
    every (step, layer) are drawn up front.
    """
    import torch
    p = FULLDEPTH.params
    steps = p["steps"] if steps is None else steps
    layers = p["layers"] if layers is None else layers
    b = len(lens0)
    tables, num_pages, spare = place_pages(np.asarray(lens0) + steps, FULLDEPTH.tag, 1)
    base_k = normal_bf16((num_pages, HKV, PAGE, HEAD_DIM), torch_seed(FULLDEPTH.tag, 1), device)
    base_v = normal_bf16((num_pages, HKV, PAGE, HEAD_DIM), torch_seed(FULLDEPTH.tag, 2), device)
    k_pools, v_pools = [base_k], [base_v]
    for layer in range(1, layers):
        k_pools.append(torch.roll(base_k, shifts=layer, dims=0))
        v_pools.append(torch.roll(base_v, shifts=layer, dims=0))
    q = normal_bf16((steps, layers, b, HQ, HEAD_DIM), torch_seed(FULLDEPTH.tag, 3), device)
    k_new = normal_bf16((steps, layers, b, HKV, HEAD_DIM), torch_seed(FULLDEPTH.tag, 4), device)
    v_new = normal_bf16((steps, layers, b, HKV, HEAD_DIM), torch_seed(FULLDEPTH.tag, 5), device)
    return dict(tables=tables, num_pages=num_pages, spare=spare, k_pools=k_pools, v_pools=v_pools,
                q=q, k_new=k_new, v_new=v_new, steps=steps, layers=layers)
