"""mtd_kv_append on the GPU: the whole pool after each call must equal the oracle's expected pool
bit for bit, untouched (NaN-poisoned) slots included."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import bits, log, new_pool

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def run_append(kp, vp, k_new, v_new, cu, start, tables):
    mtd.mtd_kv_append(kp, vp, k_new, v_new,
                      torch.as_tensor(np.asarray(cu, dtype=np.int32), device=kp.device),
                      torch.as_tensor(np.asarray(start, dtype=np.int32), device=kp.device),
                      torch.as_tensor(np.asarray(tables, dtype=np.int32), device=kp.device))


def check_append(kp, vp, counts, start, tables, tag):
    """One append call checked against oracle.kv_append on the pool's previous bits."""
    counts = np.asarray(counts)
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    n = int(cu[-1])
    k_new = torch.empty((n, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    v_new = torch.empty_like(k_new)
    if n:
        k_new.copy_(W.normal_bf16((n, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 10), "cuda"))
        v_new.copy_(W.normal_bf16((n, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 11), "cuda"))
    k_before, v_before = bits(kp), bits(vp)
    log(f"append tag={tag} n_req={len(counts)} n_new={n}")
    run_append(kp, vp, k_new, v_new, cu, start, tables)
    torch.cuda.synchronize()
    k_want, v_want = oracle.kv_append(k_before, v_before, bits(k_new), bits(v_new), cu, start, tables)
    assert np.array_equal(bits(kp), k_want)
    assert np.array_equal(bits(vp), v_want)


def test_append_tiny_prompt_then_decode_steps():
    """30 s of audio + prompt: 439-token prompt, then 32 one-token decode appends."""
    final = 439 + 32
    tables, n_pages, _ = W.place_pages([final], W.TINY.tag, 0)
    kp, vp = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")
    check_append(kp, vp, [439], [0], tables, 500)
    for step in range(32):
        check_append(kp, vp, [1], [439 + step], tables, 501 + step)


def test_append_ragged_requests():
    """Several requests: empty, single token, page-boundary starts and multi-page spans."""
    starts = np.array([0, 63, 64, 130, 7, 0, 4000])
    counts = np.array([1, 1, 65, 200, 0, 64, 129])
    final = starts + counts
    tables, n_pages, _ = W.place_pages(np.maximum(final, 1), 77, 0)
    kp, vp = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")
    check_append(kp, vp, counts, starts, tables, 600)


def test_append_chunks_of_a_90_minute_request():
    """4096-token chunk appends of the 67,500-token request (first two and the ragged last one)."""
    total, chunk = W.PREFILL90.params["total"], W.CHUNK
    tables, n_pages, _ = W.place_pages([total], W.PREFILL90.tag, 0)
    kp, vp = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")
    for k in (0, 1, 16):
        start = k * chunk
        c = min(chunk, total - start)
        check_append(kp, vp, [c], [start], tables, 700 + k)


def test_append_one_token_per_request_batch():
    """A full-depth decode step's append: one token for each of 64 requests at ragged positions."""
    lens = W.loguniform_lengths(64, 4000, W.CONTEXT_CAP - 128, 5, 0)
    # Only the page each new token lands in is backed by a real page; every other entry points at
    # a spare page, which must stay untouched.
    stride = W.CONTEXT_CAP // W.PAGE
    perm = W.rng(5, 99).permutation(65)
    tables = np.full((64, stride), perm[64], dtype=np.int32)
    for b in range(64):
        tables[b, lens[b] // W.PAGE] = perm[b]
    kp, vp = new_pool(65, "cuda"), new_pool(65, "cuda")
    check_append(kp, vp, np.ones(64, dtype=np.int64), lens, tables, 800)


def test_append_many_requests():
    """150 requests of 0 to 3 tokens each: the owning request of a token is found by binary search
    over cu_new, across more than two wavefronts' worth of requests."""
    rng = W.rng(6, 1)
    counts = rng.integers(0, 4, size=150)
    starts = rng.integers(0, 5000, size=150)
    final = np.maximum(starts + counts, 1)
    tables, n_pages, _ = W.place_pages(final, 78, 0)
    kp, vp = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")
    check_append(kp, vp, counts, starts, tables, 900)


def test_append_padded_batch_writes_only_owned_rows():
    """A batch padded to 16 rows for 11 real requests (one token each, then four padding requests
    with no token): rows 11..15 of k_new / v_new belong to no request and must not be written; the
    pool equals the oracle's, which writes only the rows cu_new assigns."""
    lens = W.loguniform_lengths(11, 10, 3000, 91, 0)
    tables, n_pages, _ = W.place_pages(lens + 1, 91, 1)
    tb = np.zeros((16, tables.shape[1]), dtype=np.int32)
    tb[:11] = tables                       # padding rows point at page 0, which holds real tokens
    kp, vp = new_pool(n_pages, "cuda", W.torch_seed(91, 2)), new_pool(n_pages, "cuda", W.torch_seed(91, 3))
    k_new = W.normal_bf16((16, W.HKV, W.HEAD_DIM), W.torch_seed(91, 4), "cuda")
    v_new = W.normal_bf16((16, W.HKV, W.HEAD_DIM), W.torch_seed(91, 5), "cuda")
    cu = np.minimum(np.arange(17), 11).astype(np.int32)
    start = np.concatenate([lens, np.zeros(5)]).astype(np.int32)
    k_before, v_before = bits(kp), bits(vp)
    log("append, 11 requests padded to 16 rows")
    run_append(kp, vp, k_new, v_new, cu, start, tb)
    torch.cuda.synchronize()
    k_want, v_want = oracle.kv_append(k_before, v_before, bits(k_new), bits(v_new), cu, start, tb)
    assert np.array_equal(bits(kp), k_want)
    assert np.array_equal(bits(vp), v_want)
