"""Pins for the fp64 oracle, independent of the oracle's own code path.

Each pin checks the oracle against something other than itself: hand-derived
closed forms (tests/golden), brute force on tiny inputs with the textbook
softmax (no max shift, Python floats), closed-form special cases, invariants of
the definition, and torch's scaled_dot_product_attention in float64.  The last
test plants plausible mistakes in copies of the oracle and shows that some pin
catches each one.
"""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import place_pages

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64_to_bf16_bits(x):
    """Round-to-nearest-even float64 -> bf16 bits (test helper for building inputs)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def random_bf16(rs, shape, scale=1.0):
    return f64_to_bf16_bits(rs.standard_normal(shape) * scale)


def paged(logical_bits, rs, page_size, extra_pages=2):
    """Scatter logical rows [L][Hkv][D] into a randomly placed pool (test-side layout)."""
    n, hkv, d = logical_bits.shape
    n_pages = (n + page_size - 1) // page_size
    total = n_pages + extra_pages
    perm = rs.permutation(total)
    table = perm[:n_pages]
    pool = np.full((total, hkv, page_size, d), 0x7FC0, dtype=np.uint16)  # NaN poison
    for j in range(n):
        pool[table[j // page_size], :, j % page_size, :] = logical_bits[j]
    return pool, table


# ----------------------------------------------------------------------------------
# brute force: textbook softmax with Python floats, no max shift, logical arrays
# ----------------------------------------------------------------------------------

def brute_force(q, k, v, q_pos, scale):
    n_q, hq, d = q.shape
    hkv = k.shape[1]
    out = np.zeros((n_q, hq, d))
    lse = np.zeros((n_q, hq))
    for i in range(n_q):
        for h in range(hq):
            g = (h * hkv) // hq
            weights = []
            for j in range(int(q_pos[i]) + 1):
                dot = 0.0
                for c in range(d):
                    dot += float(q[i, h, c]) * float(k[j, g, c])
                weights.append(math.exp(scale * dot))
            z = sum(weights)
            lse[i, h] = math.log(z)
            for c in range(d):
                out[i, h, c] = sum(w * float(v[j, g, c]) for j, w in enumerate(weights)) / z
    return out, lse


# ----------------------------------------------------------------------------------
# pins as functions of an attention implementation (so planted mistakes can be run)
# ----------------------------------------------------------------------------------

def pin_golden(attn):
    fx = json.load(open(os.path.join(GOLDEN, "closed_form_three_keys.json")))
    q = np.array(fx["q"], dtype=np.float64)
    k = np.array(fx["k"], dtype=np.float64)
    v = np.array(fx["v"], dtype=np.float64)
    o, lse = attn(q, k, v, np.arange(3), math.log(2.0))
    exp_o = np.array([[[float(Fraction(x)) for x in row] for row in pos] for pos in fx["expected_o"]])
    exp_l = np.array([[math.log(int(s[3:-1])) for s in pos] for pos in fx["expected_lse"]])
    return np.allclose(o, exp_o, atol=1e-13, rtol=0) and np.allclose(lse, exp_l, atol=1e-13, rtol=0)


def pin_brute_force(attn, seed=0):
    rs = np.random.default_rng(seed)
    ok = True
    for hq, hkv, d, n_keys, n_q in [(2, 1, 3, 5, 5), (4, 2, 8, 12, 4), (4, 1, 4, 9, 1), (4, 4, 2, 7, 3)]:
        q = oracle.bf16_to_f64(random_bf16(rs, (n_q, hq, d)))
        k = oracle.bf16_to_f64(random_bf16(rs, (n_keys, hkv, d)))
        v = oracle.bf16_to_f64(random_bf16(rs, (n_keys, hkv, d)))
        pos = np.sort(rs.choice(n_keys, size=n_q, replace=False))
        o, lse = attn(q, k, v, pos, 0.37)
        bo, bl = brute_force(q, k, v, pos, 0.37)
        ok &= np.allclose(o, bo, rtol=1e-12, atol=1e-13) and np.allclose(lse, bl, rtol=1e-12, atol=1e-13)
    return bool(ok)


def pin_single_key(attn, seed=1):
    rs = np.random.default_rng(seed)
    q = oracle.bf16_to_f64(random_bf16(rs, (1, 4, 16)))
    k = oracle.bf16_to_f64(random_bf16(rs, (1, 2, 16)))
    v = oracle.bf16_to_f64(random_bf16(rs, (1, 2, 16)))
    scale = 1 / math.sqrt(16)
    o, lse = attn(q, k, v, [0], scale)
    ok = True
    for h in range(4):
        g = h // 2
        ok &= np.allclose(o[0, h], v[0, g], atol=1e-15)
        ok &= abs(lse[0, h] - scale * float(np.dot(q[0, h], k[0, g]))) < 1e-13
    return bool(ok)


def pin_identical_keys(attn, seed=2):
    rs = np.random.default_rng(seed)
    n = 40
    q = oracle.bf16_to_f64(random_bf16(rs, (n, 4, 8)))
    k1 = oracle.bf16_to_f64(random_bf16(rs, (1, 2, 8)))
    k = np.repeat(k1, n, axis=0)
    v = oracle.bf16_to_f64(random_bf16(rs, (n, 2, 8)))
    scale = 0.25
    o, lse = attn(q, k, v, np.arange(n), scale)
    ok = True
    for i in range(n):
        for h in range(4):
            g = h // 2
            ok &= np.allclose(o[i, h], v[: i + 1, g].mean(axis=0), atol=1e-13)
            s = scale * float(np.dot(q[i, h], k1[0, g]))
            ok &= abs(lse[i, h] - (s + math.log(i + 1))) < 1e-12
    return bool(ok)


def pin_sdpa(attn, seed=3):
    import torch
    rs = np.random.default_rng(seed)
    hq, hkv, d, n_keys, n_q = 16, 8, 32, 70, 23
    q = oracle.bf16_to_f64(random_bf16(rs, (n_q, hq, d)))
    k = oracle.bf16_to_f64(random_bf16(rs, (n_keys, hkv, d)))
    v = oracle.bf16_to_f64(random_bf16(rs, (n_keys, hkv, d)))
    prefix = n_keys - n_q                      # bottom-right: query i at position prefix + i
    o, _ = attn(q, k, v, prefix + np.arange(n_q), 1 / math.sqrt(d))
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]                 # [1][Hq][Nq][D]
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)[None]
    mask = torch.arange(n_keys)[None, :] <= (prefix + torch.arange(n_q))[:, None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=1 / math.sqrt(d))
    ref = ref[0].permute(1, 0, 2).numpy()
    return bool(np.allclose(o, ref, atol=1e-12, rtol=1e-10))


def pin_shift_scale(attn, seed=4):
    """Adding u with <q,u> = c to every key shifts LSE by scale*c and leaves O; scaling V scales O."""
    rs = np.random.default_rng(seed)
    n, d = 30, 8
    q = rs.standard_normal((n, 2, d))
    k = rs.standard_normal((n, 1, d))
    v = rs.standard_normal((n, 1, d))
    scale = 0.5
    pos = np.arange(n)
    o, lse = attn(q, k, v, pos, scale)
    ok = True
    u = rs.standard_normal(d)
    o3, lse3 = attn(q, k + u[None, None, :], v, pos, scale)
    c = q @ u                                   # [n][2]: <q_i,h , u>
    ok &= np.allclose(o3, o, atol=1e-12)
    ok &= np.allclose(lse3, lse + scale * c, atol=1e-12)
    o4, lse4 = attn(q, k, 3.5 * v, pos, scale)
    ok &= np.allclose(o4, 3.5 * o, atol=1e-12) and np.allclose(lse4, lse, atol=1e-14)
    return bool(ok)


PINS = [pin_golden, pin_brute_force, pin_single_key, pin_identical_keys, pin_sdpa, pin_shift_scale]


# ----------------------------------------------------------------------------------
# the oracle passes every pin
# ----------------------------------------------------------------------------------

@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    assert pin(oracle.attention)


def test_golden_paged_chunked():
    """The worked example again, through paged storage and a prefix + chunk split."""
    fx = json.load(open(os.path.join(GOLDEN, "closed_form_three_keys.json")))
    q = f64_to_bf16_bits(np.array(fx["q"], dtype=np.float64))
    k = f64_to_bf16_bits(np.array(fx["k"], dtype=np.float64))
    v = f64_to_bf16_bits(np.array(fx["v"], dtype=np.float64))
    rs = np.random.default_rng(0)
    kp, table = paged(k, rs, page_size=2)
    vp = np.full_like(kp, 0x7FC0)
    for j in range(3):
        vp[table[j // 2], :, j % 2, :] = v[j]
    o, lse = oracle.prefill_chunk(q[1:], kp, vp, table, 1, math.log(2.0))
    assert np.allclose(o[1, 0], [13 / 7, -2 / 7], atol=1e-13)
    assert np.allclose(lse[:, 0], [math.log(3), math.log(7)], atol=1e-13)
    assert np.allclose(o[0, 1], [0.5, 0.5], atol=1e-13)


def test_golden_page_walk_and_append():
    fx = json.load(open(os.path.join(GOLDEN, "page_walk_append_tiny.json")))
    ps, n_pages = fx["page_size"], fx["num_pages"]
    pool = np.zeros((n_pages, 1, ps, 1), dtype=np.uint16)
    for p in range(n_pages):
        for s in range(ps):
            pool[p, 0, s, 0] = 100 * p + s
    tables = np.array(fx["block_tables"])
    ap = fx["append"]
    new = np.array(ap["new_bits"], dtype=np.uint16).reshape(-1, 1, 1)
    k_out, v_out = oracle.kv_append(pool, pool, new, new, ap["cu_new"], ap["start_pos"], tables)
    expect = pool.copy()
    for page, slot, bits in fx["expected_changed"]:
        expect[page, 0, slot, 0] = bits
    assert np.array_equal(k_out, expect) and np.array_equal(v_out, expect)
    for r, rows in fx["expected_logical_after"].items():
        got = oracle.gather_logical(k_out, tables[int(r)], len(rows))
        want = oracle.bf16_to_f64(np.array(rows, dtype=np.uint16).reshape(-1, 1, 1))
        assert np.array_equal(got, want)


def test_page_of_known_values():
    assert oracle.page_of(0, 64) == (0, 0)
    assert oracle.page_of(63, 64) == (0, 63)
    assert oracle.page_of(64, 64) == (1, 0)
    assert oracle.page_of(67499, 64) == (1054, 43)


def test_page_walker_random_placement():
    """S8: gather from a randomly placed pool returns the logical rows bit for bit."""
    rs = np.random.default_rng(5)
    for n, ps in [(1, 64), (63, 64), (64, 64), (65, 64), (439, 64), (1000, 16)]:
        logical = random_bf16(rs, (n, 8, 16))
        pool, table = paged(logical, rs, ps)
        got = oracle.gather_logical(pool, table, n)
        assert np.array_equal(got, oracle.bf16_to_f64(logical))


def test_bf16_conversion_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0x0000, 0x8000], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, 2.0 ** -133, 3.3895313892515355e38, 0.0, -0.0]
    assert list(oracle.bf16_to_f64(bits)) == want


def test_chunked_equals_one_shot():
    """S4: prefix + chunk over paged KV equals one causal pass, for many chunk sizes."""
    rs = np.random.default_rng(6)
    hq, hkv, d, n = 4, 2, 16, 300
    q = random_bf16(rs, (n, hq, d))
    k = random_bf16(rs, (n, hkv, d))
    v = random_bf16(rs, (n, hkv, d))
    kp, table = paged(k, rs, 64)
    vp = np.full_like(kp, 0x7FC0)
    for j in range(n):
        vp[table[j // 64], :, j % 64, :] = v[j]
    o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(q), oracle.bf16_to_f64(k),
                                    oracle.bf16_to_f64(v), np.arange(n), 0.3)
    for chunk in (1, 7, 64, 100, 4096):
        outs, lses = [], []
        for start in range(0, n, chunk):
            c = min(chunk, n - start)
            o, l = oracle.prefill_chunk(q[start:start + c], kp, vp, table, start, 0.3)
            outs.append(o)
            lses.append(l)
        assert np.allclose(np.concatenate(outs), o_ref, atol=1e-12)
        assert np.allclose(np.concatenate(lses), l_ref, atol=1e-12)


def test_chunked_equals_one_shot_4096():
    """S4 at the pages' chunk size: 4096 + a ragged 300-token tail."""
    rs = np.random.default_rng(7)
    n = 4396
    q = random_bf16(rs, (n, 2, 8))
    k = random_bf16(rs, (n, 1, 8))
    v = random_bf16(rs, (n, 1, 8))
    kp, table = paged(k, rs, 64)
    vp = np.full_like(kp, 0x7FC0)
    for j in range(n):
        vp[table[j // 64], :, j % 64, :] = v[j]
    o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(q), oracle.bf16_to_f64(k),
                                    oracle.bf16_to_f64(v), np.arange(n), 0.35)
    o1, l1 = oracle.prefill_chunk(q[:4096], kp, vp, table, 0, 0.35)
    o2, l2 = oracle.prefill_chunk(q[4096:], kp, vp, table, 4096, 0.35)
    assert np.allclose(np.concatenate([o1, o2]), o_ref, atol=1e-12)
    assert np.allclose(np.concatenate([l1, l2]), l_ref, atol=1e-12)


def test_split_merge_equals_one_shot():
    """S5: attention over disjoint key ranges, merged by LSE, equals one pass (incl. an empty range)."""
    rs = np.random.default_rng(8)
    n, d = 500, 16
    q = rs.standard_normal((1, 4, d))
    k = rs.standard_normal((n, 2, d))
    v = rs.standard_normal((n, 2, d))
    o_ref, l_ref = oracle.attention(q, k, v, [n - 1], 0.2)
    for bounds in ([0, 100, 101, 400, 500], [0, 64, 128, 192, 256, 320, 384, 448, 500], [0, 250, 250, 500]):
        o_parts, l_parts = [], []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            if hi == lo:
                o_parts.append(np.zeros((1, 4, d)))
                l_parts.append(np.full((1, 4), -np.inf))
                continue
            # keys lo..hi-1 only: a query placed after all of them sees the whole range
            o, l = oracle.attention(q, k[lo:hi], v[lo:hi], [hi - lo - 1], 0.2)
            o_parts.append(o)
            l_parts.append(l)
        o, l = oracle.lse_merge(o_parts, l_parts)
        assert np.allclose(o, o_ref, atol=1e-12) and np.allclose(l, l_ref, atol=1e-12)


def test_decode_matches_definition():
    """Decode query sits at kv_len - 1 and sees every key; equals a 1-row prefill chunk."""
    rs = np.random.default_rng(9)
    lens = np.array([1, 63, 64, 65, 200])
    tables, n_pages, _ = place_pages(lens, 99)
    kp = np.full((n_pages, 2, 64, 8), 0x7FC0, dtype=np.uint16)
    vp = kp.copy()
    logical = []
    for b, n in enumerate(lens):
        k = random_bf16(rs, (n, 2, 8))
        v = random_bf16(rs, (n, 2, 8))
        for j in range(n):
            kp[tables[b][j // 64], :, j % 64, :] = k[j]
            vp[tables[b][j // 64], :, j % 64, :] = v[j]
        logical.append((k, v))
    q = random_bf16(rs, (len(lens), 4, 8))
    o, lse = oracle.decode(q, kp, vp, lens, tables, 0.4)
    for b, n in enumerate(lens):
        k, v = logical[b]
        bo, bl = brute_force(oracle.bf16_to_f64(q[b:b + 1]), oracle.bf16_to_f64(k), oracle.bf16_to_f64(v), [n - 1], 0.4)
        assert np.allclose(o[b], bo[0], atol=1e-12) and np.allclose(lse[b], bl[0], atol=1e-12)
        po, pl = oracle.prefill_chunk(q[b:b + 1], kp, vp, tables[b], n - 1, 0.4)
        assert np.array_equal(po[0], o[b]) and np.array_equal(pl[0], lse[b])


def test_append_then_walk_roundtrip():
    """Append of several requests and start positions, read back through the page walker."""
    rs = np.random.default_rng(10)
    final = np.array([130, 64, 1, 77])
    start = np.array([0, 63, 0, 70])
    tables, n_pages, _ = place_pages(final, 11)
    base = random_bf16(rs, (n_pages, 2, 64, 4))
    counts = final - start
    cu = np.concatenate([[0], np.cumsum(counts)])
    kn = random_bf16(rs, (int(cu[-1]), 2, 4))
    vn = random_bf16(rs, (int(cu[-1]), 2, 4))
    k_out, v_out = oracle.kv_append(base, base, kn, vn, cu, start, tables)
    touched = np.zeros(base.shape[:3], dtype=bool)
    for r in range(len(final)):
        got = oracle.gather_logical(k_out, tables[r], int(final[r]))
        assert np.array_equal(got[start[r]:], oracle.bf16_to_f64(kn[cu[r]:cu[r + 1]]))
        for p in range(start[r], final[r]):
            touched[tables[r][p // 64], :, p % 64] = True
    assert np.array_equal(k_out[~touched], base[~touched])
    assert np.array_equal(v_out[~touched], base[~touched])


# ----------------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------------

def _mut_no_scale(q, k, v, pos, scale):
    return oracle.attention(q, k, v, pos, 1.0)


def _mut_log2_lse(q, k, v, pos, scale):
    o, l = oracle.attention(q, k, v, pos, scale)
    return o, l / math.log(2.0)


def _mut_head_map_modulo(q, k, v, pos, scale):
    """Query head h reads KV head h % Hkv instead of h // (Hq/Hkv)."""
    hq, hkv = q.shape[1], k.shape[1]
    group = hq // hkv
    # the correct oracle maps h -> h // group; feed it a head order where that equals h % hkv
    order = [(h % hkv) * group + (h // hkv) for h in range(hq)]
    o, l = oracle.attention(q[:, np.argsort(order)], k, v, pos, scale)
    return o[:, order], l[:, order]


def _mut_exclusive_causal(q, k, v, pos, scale):
    """Keys j < p instead of j <= p (row p = 0 then has no keys)."""
    pos = np.asarray(pos)
    o = np.full(q.shape[:2] + (v.shape[2],), np.nan)
    l = np.full(q.shape[:2], np.nan)
    keep = pos > 0
    if keep.any():
        o[keep], l[keep] = oracle.attention(q[keep], k, v, pos[keep] - 1, scale)
    return o, l


def _mut_transposed_v(q, k, v, pos, scale):
    """PV product taken against V with its head and token axes confused (uses K as V)."""
    return oracle.attention(q, k, k, pos, scale)


def _mut_top_left(q, k, v, pos, scale):
    """Chunk rows aligned to the first key instead of the chunk's own positions."""
    pos = np.asarray(pos)
    return oracle.attention(q, k, v, pos - pos.min(), scale)


MUTANTS = [_mut_no_scale, _mut_log2_lse, _mut_head_map_modulo, _mut_exclusive_causal,
           _mut_transposed_v, _mut_top_left]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutant):
    import warnings
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        results = []
        for pin in PINS:
            try:
                results.append(pin(mutant))
            except Exception:
                results.append(False)
    assert not all(results), f"{mutant.__name__} passed every pin"
