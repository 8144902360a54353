"""The oracle's process-pool driver (oracle/parallel.py) returns what the serial oracle returns.

The driver adds no arithmetic: it cuts a problem into (KV head, block of query rows) units and runs
``oracle.attention`` on each in a worker process.  These CPU tests pin that cutting: prefill chunks
and decode batches on randomly placed pages, several problems over one shared pool (each with its
own table), ragged row blocks, and a layout where a swapped head or row would show."""

import numpy as np
import pytest

import oracle
from oracle.parallel import OraclePool, decode_problem, prefill_problem, usable_cores

from workloads import place_pages

HQ, HKV, D, PAGE = 16, 8, 32, 16


def _bf16_bits(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


@pytest.fixture(scope="module")
def pool():
    with OraclePool(workers=min(4, usable_cores()), rows_per_unit=24) as p:
        yield p


def test_prefill_chunk_matches_serial(pool):
    rng = np.random.default_rng(7)
    prefix, chunk = 37, 101
    total = prefix + chunk
    tables, n_pages, _ = place_pages([total], 91, 0, spare=2)
    n_pages_alloc = max(n_pages, int(tables.max()) + 1)
    k = _bf16_bits(rng, (n_pages_alloc * 4, HKV, PAGE, D))  # more pages than the table uses
    v = _bf16_bits(rng, k.shape)
    q = _bf16_bits(rng, (chunk, HQ, D))
    table = rng.permutation(k.shape[0])[: (total + PAGE - 1) // PAGE]
    scale = 1.0 / np.sqrt(D)
    [(o, lse)] = pool.attention([prefill_problem(q, k, v, table, prefix)], scale)
    o_ref, lse_ref = oracle.prefill_chunk(q, k, v, table, prefix, scale)
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_decode_batch_on_one_shared_pool(pool):
    """Several requests over the same pool object (written once), each with its own table."""
    rng = np.random.default_rng(8)
    lens = [1, 15, 16, 17, 70, 133]
    need = [(n + PAGE - 1) // PAGE for n in lens]
    n_pages = sum(need) + 3
    k = _bf16_bits(rng, (n_pages, HKV, PAGE, D))
    v = _bf16_bits(rng, k.shape)
    perm = rng.permutation(n_pages)
    tables, cur = [], 0
    for n in need:
        tables.append(perm[cur:cur + n])
        cur += n
    q = _bf16_bits(rng, (len(lens), HQ, D))
    scale = 0.3
    probs = [decode_problem(q[b:b + 1], k, v, tables[b], lens[b]) for b in range(len(lens))]
    got = pool.attention(probs, scale)
    width = max(need)
    tb = np.zeros((len(lens), width), dtype=np.int64)
    for b, t in enumerate(tables):
        tb[b, : len(t)] = t
    o_ref, lse_ref = oracle.decode(q, k, v, lens, tb, scale)
    for b in range(len(lens)):
        np.testing.assert_allclose(got[b][0][0], o_ref[b], rtol=0, atol=1e-12)
        np.testing.assert_allclose(got[b][1][0], lse_ref[b], rtol=0, atol=1e-12)


def test_heads_and_rows_land_in_place(pool):
    """Values that name their own KV head: with identical keys each row of head h averages V of
    KV head h // 2 over its visible keys, so a misplaced head or row block changes the result."""
    n = 40
    k = np.zeros((3, HKV, PAGE, D), dtype=np.uint16)  # all-zero keys: uniform softmax
    vals = np.zeros((3, HKV, PAGE, D), dtype=np.float32)
    for g in range(HKV):
        vals[:, g] = g + 1
    v = (vals.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    q = _bf16_bits(np.random.default_rng(9), (n, HQ, D))
    [(o, lse)] = pool.attention([prefill_problem(q, k, v, np.arange(3), 0)], 0.5)
    for h in range(HQ):
        np.testing.assert_allclose(o[:, h, :], np.full((n, D), h // 2 + 1.0), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, np.log(np.arange(1, n + 1))[:, None] * np.ones((1, HQ)), atol=1e-12)
