"""Pins for the projection oracle (oracle/projection.py), independent of its own code path.

Each pin checks it against something other than itself: torch's float32 -> bf16 conversion
(round to nearest even) on ties, overflow, subnormals and NaN; brute-force sums over Python
fractions on tiny hidden sizes; weights whose rows carry their own index, so that the split into
q, k and v and the head-major feature order are read off in closed form; one-hot attention
outputs that return one column of Wo; and attention outputs placed on bf16 ties, which show
whether O is rounded before the product.  The last test plants plausible mistakes in copies of
the oracle and shows that some pin catches each one.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import projection as P

HQ, HKV, D = 16, 8, 128
NQ, NKV = HQ * D, HKV * D


def bf16_bits_exact(values):
    """bf16 bits of values that are exactly representable (test-side input builder)."""
    f = np.asarray(values, dtype=np.float32)
    bits = f.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def random_bf16(rs, shape, scale=1.0):
    """Random bf16 bits by truncating float32 patterns (any bf16 value is fine as an input)."""
    f = (rs.standard_normal(shape) * scale).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


IMPL = dict(round=P.round_to_bf16_bits, qkv=P.qkv_proj, o=P.o_proj)


# ----------------------------------------------------------------------------------
# pins as functions of an implementation (so planted mistakes can be run)
# ----------------------------------------------------------------------------------

def pin_round_matches_torch(impl, seed=0):
    rs = np.random.default_rng(seed)
    kept = rs.integers(0, 1 << 16, size=4000, dtype=np.uint64)
    low = rs.integers(0, 1 << 16, size=4000, dtype=np.uint64)
    low[:1000] = 0x8000                      # exact ties, both parities of the kept half
    low[1000:1200] = 0x7FFF                  # just below a tie
    low[1200:1400] = 0x8001                  # just above a tie
    bits = ((kept << np.uint64(16)) | low).astype(np.uint32)
    special = np.array([0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7FFFFF, 0x00000001, 0x80008000,
                        0x00018000, 0x7F800000, 0xFF800000, 0x00000000, 0x80000000, 0x3F808000,
                        0x3F818000], dtype=np.uint32)
    bits = np.concatenate([bits, special])
    x = bits.view(np.float32)
    got = impl["round"](x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    same = np.array_equal(got[~nan], want[~nan])
    nan_ok = bool(np.all(np.isnan(oracle.bf16_to_f64(got[nan])))) if nan.any() else True
    return bool(same and nan_ok)


def pin_round_nan_stays_nan(impl):
    x = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
    got = oracle.bf16_to_f64(impl["round"](x))
    return bool(np.all(np.isnan(got)))


def _brute_linear(x_bits, w_bits):
    """sum_i W[n][i] x[t][i] with exact rational arithmetic (bf16 values are dyadic)."""
    xf = [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f64(x_bits)]
    wf = [[Fraction(float(v)) for v in row] for row in oracle.bf16_to_f64(w_bits)]
    return np.array([[float(sum(a * b for a, b in zip(xr, wr))) for wr in wf] for xr in xf])


def pin_qkv_brute_force(impl, seed=1):
    rs = np.random.default_rng(seed)
    ok = True
    for t, hidden in [(1, 3), (2, 5)]:
        x = random_bf16(rs, (t, hidden))
        w = random_bf16(rs, (NQ + 2 * NKV, hidden))
        y = _brute_linear(x, w)
        q, k, v = impl["qkv"](x, w)
        ok &= np.array_equal(np.asarray(q).reshape(t, -1), y[:, :NQ])
        ok &= np.array_equal(np.asarray(k).reshape(t, -1), y[:, NQ:NQ + NKV])
        ok &= np.array_equal(np.asarray(v).reshape(t, -1), y[:, NQ + NKV:])
    return bool(ok)


def pin_qkv_labelled_rows(impl):
    """Row n of W_qkv is (n // 64, n % 64): token e_0 reads n // 64 and e_1 reads n % 64, so every
    output element names the weight row that made it."""
    n = np.arange(NQ + 2 * NKV)
    w = bf16_bits_exact(np.stack([n // 64, n % 64], axis=1).astype(np.float32))
    x = bf16_bits_exact(np.array([[1.0, 0.0], [0.0, 1.0]], dtype=np.float32))
    q, k, v = impl["qkv"](x, w)
    ok = True
    for part, heads, base in ((q, HQ, 0), (k, HKV, NQ), (v, HKV, NQ + NKV)):
        part = np.asarray(part)
        if part.shape != (2, heads, D):
            return False
        row = base + np.arange(heads)[:, None] * D + np.arange(D)[None, :]
        ok &= np.array_equal(part[0], (row // 64).astype(np.float64))
        ok &= np.array_equal(part[1], (row % 64).astype(np.float64))
    return bool(ok)


def pin_o_one_hot(impl, seed=2):
    """O with a single 1 at (head h, dim d) returns column h*128 + d of Wo."""
    rs = np.random.default_rng(seed)
    hidden = 16
    w = random_bf16(rs, (hidden, NQ))
    picks = [(0, 0), (3, 5), (15, 127), (7, 64)]
    o = np.zeros((len(picks), HQ, D), dtype=np.float32)
    for t, (h, d) in enumerate(picks):
        o[t, h, d] = 1.0
    y = np.asarray(impl["o"](o, w))
    wf = oracle.bf16_to_f64(w)
    return bool(all(np.array_equal(y[t], wf[:, h * D + d]) for t, (h, d) in enumerate(picks)))


def pin_o_rounds_input(impl):
    """O values on bf16 ties: 1 + 2^-8 rounds to 1 (even) and 1 + 3*2^-8 up to 1 + 2^-6; the
    product with a one-hot Wo row returns the rounded value."""
    hidden = 4
    w = np.zeros((hidden, NQ), dtype=np.float32)
    w[0, 0] = 1.0
    w[1, 1] = 1.0
    w[2, 2] = 1.0
    w[3, 3] = 1.0
    o = np.zeros((1, HQ, D), dtype=np.float32)
    o[0, 0, :4] = [1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 1 + 2.0 ** -8 + 2.0 ** -20]
    y = np.asarray(impl["o"](o, bf16_bits_exact(w)))
    return bool(np.array_equal(y[0], [1.0, 1 + 2.0 ** -6, -1.0, 1 + 2.0 ** -7]))


def pin_o_brute_force(impl, seed=3):
    rs = np.random.default_rng(seed)
    hidden = 3
    o = rs.standard_normal((2, HQ, D)).astype(np.float32)
    w = random_bf16(rs, (hidden, NQ))
    # the rounding is pinned on its own above; here the rounded O comes from torch
    o_bits = torch.from_numpy(o.reshape(2, -1).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = _brute_linear(o_bits, w)
    return bool(np.array_equal(np.asarray(impl["o"](o, w)), want))


PINS = [pin_round_matches_torch, pin_round_nan_stays_nan, pin_qkv_brute_force,
        pin_qkv_labelled_rows, pin_o_one_hot, pin_o_rounds_input, pin_o_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    assert pin(IMPL)


def test_qkv_full_shape():
    """hidden 1024, a few tokens: shapes and agreement with torch's float64 linear."""
    rs = np.random.default_rng(4)
    x = random_bf16(rs, (3, 1024))
    w = random_bf16(rs, (NQ + 2 * NKV, 1024), 1 / 32)
    q, k, v = P.qkv_proj(x, w)
    assert q.shape == (3, HQ, D) and k.shape == (3, HKV, D) and v.shape == (3, HKV, D)
    y = torch.nn.functional.linear(torch.from_numpy(oracle.bf16_to_f64(x)), torch.from_numpy(oracle.bf16_to_f64(w)))
    got = np.concatenate([q.reshape(3, -1), k.reshape(3, -1), v.reshape(3, -1)], axis=1)
    np.testing.assert_allclose(got, y.numpy(), rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ----------------------------------------------------------------------------------

def _mut_truncating_round(impl):
    return dict(impl, round=lambda x: (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16))


def _mut_ties_away(impl):
    def rnd(x):
        b = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
        return ((b + 0x8000) >> 16).astype(np.uint16)
    return dict(impl, round=rnd)


def _mut_w_as_in_out(impl):
    """W_qkv read as [in][out] memory (reshape instead of transpose)."""
    def qkv(x_bits, w_bits):
        w = np.asarray(w_bits)
        y = oracle.bf16_to_f64(x_bits) @ oracle.bf16_to_f64(w.reshape(w.shape[1], w.shape[0]))
        t = y.shape[0]
        return y[:, :NQ].reshape(t, HQ, D), y[:, NQ:NQ + NKV].reshape(t, HKV, D), y[:, NQ + NKV:].reshape(t, HKV, D)
    return dict(impl, qkv=qkv)


def _mut_k_v_swapped(impl):
    def qkv(x_bits, w_bits):
        q, k, v = P.qkv_proj(x_bits, w_bits)
        return q, v, k
    return dict(impl, qkv=qkv)


def _mut_dim_major_heads(impl):
    """Feature f read as (dim f // 16, head f % 16)."""
    def qkv(x_bits, w_bits):
        q, k, v = P.qkv_proj(x_bits, w_bits)
        t = q.shape[0]
        return (q.reshape(t, D, HQ).transpose(0, 2, 1), k.reshape(t, D, HKV).transpose(0, 2, 1),
                v.reshape(t, D, HKV).transpose(0, 2, 1))
    return dict(impl, qkv=qkv)


def _mut_dropped_last_term(impl):
    def qkv(x_bits, w_bits):
        x = np.asarray(x_bits).copy()
        x[:, -1] = 0
        return P.qkv_proj(x, w_bits)
    return dict(impl, qkv=qkv)


def _mut_o_unrounded(impl):
    def o(attn, w_bits):
        a = np.asarray(attn, dtype=np.float64)
        return a.reshape(a.shape[0], -1) @ oracle.bf16_to_f64(w_bits).T
    return dict(impl, o=o)


def _mut_o_wo_not_transposed(impl):
    def o(attn, w_bits):
        a = oracle.bf16_to_f64(P.round_to_bf16_bits(np.asarray(attn, np.float32).reshape(len(attn), -1)))
        w = np.asarray(w_bits)
        return a @ oracle.bf16_to_f64(w.reshape(w.shape[1], w.shape[0]))
    return dict(impl, o=o)


MUTANTS = [_mut_truncating_round, _mut_ties_away, _mut_w_as_in_out, _mut_k_v_swapped,
           _mut_dim_major_heads, _mut_dropped_last_term, _mut_o_unrounded, _mut_o_wo_not_transposed]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_planted_mistake_is_caught(mutant):
    import warnings
    impl = mutant(IMPL)
    with warnings.catch_warnings():
        warnings.simplefilter("ignore")
        results = []
        for pin in PINS:
            try:
                results.append(pin(impl))
            except Exception:
                results.append(False)
    assert not all(results), f"{mutant.__name__} passed every pin"
