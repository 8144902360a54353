"""The projections around the attention (mtd_qkv_proj, mtd_o_proj) against the fp64 oracle.

Every output element must lie within a bound derived from the arithmetic: the device sums K
bf16 x bf16 products in float32 (products exact, each addition off by at most 2^-24 of the
running sum's magnitude), then rounds to bf16 (at most 2^-8 of the value, ties to even).  With
S = sum |x_i w_i| the accumulated error is at most K 2^-24 S, so

    |y_gpu - y| <= K 2^-24 S + 2^-8 (|y| + K 2^-24 S).

The output projection rounds its float32 input to bf16 first; the oracle takes the same
decision in the same precision (float32 -> bf16, nearest even), so both multiply the same bf16
values.  Sizes: single tokens; counts around the tile heights (256 rows for QKV, 128 for the
output map) that leave a partial tile, or a tail of exactly 64 or 65 rows (a tail of at most 64
rows goes to the few-token kernel); the tiny workload's 439-token prompt; the full-depth decode
batch (64); and the mixed step's 4127 new tokens.
"""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import bits, log

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")

TAG = 6


def _bound(x64, w64, y_ref, k):
    s = np.abs(x64) @ np.abs(w64).T
    acc = k * 2.0 ** -24 * s
    return acc + 2.0 ** -8 * (np.abs(y_ref) + acc)


def _check(name, got_bf16, y_ref, bound):
    got = oracle.bf16_to_f64(bits(got_bf16)).reshape(y_ref.shape)
    err = np.abs(got - y_ref)
    worst = float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0
    exact = float(np.mean(got == oracle.bf16_to_f64(oracle.round_to_bf16_bits(y_ref.astype(np.float32))))) if err.size else 1.0
    print(f"  {name}: max err {err.max() if err.size else 0:.3g}, max err/bound {worst:.3f}, "
          f"equal to the rounded reference {100 * exact:.2f} %", flush=True)
    assert np.all(np.isfinite(got))
    assert np.all(err <= bound), f"{name}: {int((err > bound).sum())} elements beyond the bound"


def _weights(dev):
    return W.projection_weights(W.torch_seed(TAG, 0), dev)


@pytest.mark.parametrize("n_tok", [1, 8, 9, 37, 64, 65, 128, 255, 256, 257, 300, 320, 321, 439, 1000])
def test_qkv_proj_matches_oracle(n_tok):
    log(f"qkv projection n_tok={n_tok}")
    w_qkv, _ = _weights("cuda")
    x = W.normal_bf16((n_tok, W.HIDDEN), W.torch_seed(TAG, 1, n_tok), "cuda")
    q, k, v = mtd.mtd_qkv_proj(x, w_qkv)
    torch.cuda.synchronize()
    xb, wb = bits(x), bits(w_qkv)
    q_ref, k_ref, v_ref = oracle.qkv_proj(xb, wb)
    y_ref = np.concatenate([q_ref.reshape(n_tok, -1), k_ref.reshape(n_tok, -1), v_ref.reshape(n_tok, -1)], 1)
    bound = _bound(oracle.bf16_to_f64(xb), oracle.bf16_to_f64(wb), y_ref, W.HIDDEN)
    nq, nkv = W.HQ * W.HEAD_DIM, W.HKV * W.HEAD_DIM
    _check("q", q, q_ref, bound[:, :nq].reshape(q_ref.shape))
    _check("k", k, k_ref, bound[:, nq:nq + nkv].reshape(k_ref.shape))
    _check("v", v, v_ref, bound[:, nq + nkv:].reshape(v_ref.shape))


@pytest.mark.parametrize("n_tok", [1, 8, 9, 37, 64, 65, 128, 129, 192, 193, 255, 300, 439, 1000])
def test_o_proj_matches_oracle(n_tok):
    log(f"output projection n_tok={n_tok}")
    _, w_o = _weights("cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(W.torch_seed(TAG, 2, n_tok))
    attn = torch.randn((n_tok, W.HQ, W.HEAD_DIM), generator=gen, device="cuda", dtype=torch.float32) * 0.3
    y = mtd.mtd_o_proj(attn, w_o)
    torch.cuda.synchronize()
    a32, wb = attn.cpu().numpy(), bits(w_o)
    y_ref = oracle.o_proj(a32, wb)
    a64 = oracle.bf16_to_f64(oracle.round_to_bf16_bits(a32.reshape(n_tok, -1)))
    _check("o_proj", y, y_ref, _bound(a64, oracle.bf16_to_f64(wb), y_ref, W.HQ * W.HEAD_DIM))


def test_projections_full_chunk():
    """The mixed step's new tokens through both maps: a whole 4096-token prefill chunk plus 31
    decode tokens (4127 rows: every tile of both grids, a ragged last row of tiles and a row
    count that does not split evenly over the 8 XCDs)."""
    n_tok = W.CHUNK + W.MIXED.params["batch"]
    log(f"projections, full chunk n_tok={n_tok}")
    w_qkv, w_o = _weights("cuda")
    x = W.normal_bf16((n_tok, W.HIDDEN), W.torch_seed(TAG, 3), "cuda")
    q, k, v = mtd.mtd_qkv_proj(x, w_qkv)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(W.torch_seed(TAG, 4))
    attn = torch.randn((n_tok, W.HQ, W.HEAD_DIM), generator=gen, device="cuda", dtype=torch.float32) * 0.3
    y = mtd.mtd_o_proj(attn, w_o)
    torch.cuda.synchronize()
    xb, wb = bits(x), bits(w_qkv)
    q_ref, k_ref, v_ref = oracle.qkv_proj(xb, wb)
    y_ref = np.concatenate([q_ref.reshape(n_tok, -1), k_ref.reshape(n_tok, -1), v_ref.reshape(n_tok, -1)], 1)
    got = np.concatenate([bits(q).reshape(n_tok, -1), bits(k).reshape(n_tok, -1), bits(v).reshape(n_tok, -1)], 1)
    bound = _bound(oracle.bf16_to_f64(xb), oracle.bf16_to_f64(wb), y_ref, W.HIDDEN)
    _check("qkv", torch.from_numpy(got.view(np.int16)).view(torch.bfloat16), y_ref, bound)
    a32, wob = attn.cpu().numpy(), bits(w_o)
    yo_ref = oracle.o_proj(a32, wob)
    a64 = oracle.bf16_to_f64(oracle.round_to_bf16_bits(a32.reshape(n_tok, -1)))
    _check("o_proj", y, yo_ref, _bound(a64, oracle.bf16_to_f64(wob), yo_ref, W.HQ * W.HEAD_DIM))


def test_token_results_do_not_depend_on_the_batch():
    """Rows of an 1100-token call equal, bit for bit, the same tokens projected alone or in a
    different-sized call, whichever kernel serves the rows (at most 64 tokens, or a tail of at
    most 64 rows: K split over the waves of one workgroup; more: 256 x 128 tiles for QKV, 128 x 128
    tiles with K split in halves for the output map): all of them sum each 128-wide K slice with
    one MFMA chain from zero, add the slice sums of each 1024-wide group in order, and add the
    group sums in order."""
    log("projections: batch invariance")
    w_qkv, w_o = _weights("cuda")
    x = W.normal_bf16((1100, W.HIDDEN), W.torch_seed(TAG, 5), "cuda")
    attn = W.normal_bf16((1100, W.HQ, W.HEAD_DIM), W.torch_seed(TAG, 6), "cuda").float()
    full = mtd.mtd_qkv_proj(x, w_qkv)
    y_full = mtd.mtd_o_proj(attn, w_o)
    for lo, hi in [(0, 37), (128, 129), (0, 64), (0, 65), (200, 300), (0, 1000), (1024, 1100), (1088, 1100)]:
        part = mtd.mtd_qkv_proj(x[lo:hi].contiguous(), w_qkv)
        y_part = mtd.mtd_o_proj(attn[lo:hi].contiguous(), w_o)
        for a, b in zip(full, part):
            assert torch.equal(a[lo:hi], b)
        assert torch.equal(y_full[lo:hi], y_part)


def test_outputs_written_in_place_and_nothing_else():
    """Given output buffers are filled exactly: a guard row after each stays untouched."""
    log("projections: in-place outputs with guard rows")
    w_qkv, w_o = _weights("cuda")
    n = 70
    x = W.normal_bf16((n, W.HIDDEN), W.torch_seed(TAG, 7), "cuda")
    q_buf = torch.full((n + 1, W.HQ, W.HEAD_DIM), 7.0, dtype=torch.bfloat16, device="cuda")
    k_buf = torch.full((n + 1, W.HKV, W.HEAD_DIM), 7.0, dtype=torch.bfloat16, device="cuda")
    v_buf = torch.full((n + 1, W.HKV, W.HEAD_DIM), 7.0, dtype=torch.bfloat16, device="cuda")
    q, k, v = mtd.mtd_qkv_proj(x, w_qkv, q_buf[:n], k_buf[:n], v_buf[:n])
    ref = mtd.mtd_qkv_proj(x, w_qkv)
    attn = torch.randn((n, W.HQ, W.HEAD_DIM), device="cuda")
    o_buf = torch.full((n + 1, W.HIDDEN), 7.0, dtype=torch.bfloat16, device="cuda")
    mtd.mtd_o_proj(attn, w_o, o_buf[:n])
    o_ref = mtd.mtd_o_proj(attn, w_o)
    torch.cuda.synchronize()
    for buf, r in ((q_buf, ref[0]), (k_buf, ref[1]), (v_buf, ref[2]), (o_buf, o_ref)):
        assert torch.equal(buf[:n], r)
        assert bool((buf[n] == 7.0).all())
