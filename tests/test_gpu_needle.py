"""Structural probes on the GPU.  Needle probes: one key per KV head is aligned with that group's
queries so that its logit exceeds every other by about 40 (natural-log units).  Every other weight is then below
e^-40 (about 1e-12 summed over 131,072 keys), the needle's weight is exactly 1, and the output is
that key's V up to fp32 rounding.  Needles sit at the first key, on both sides of a page boundary
(slots 63 and 64), at the last key, and, in a prefill chunk, at the last prefix key, the chunk's
first key and inside the chunk; rows before a needle's position must not see it (causality).  Each
call is also held to the oracle's gate on the same bits.  Position-coded probe: identical keys and
index-coded values make every prefill row's output a closed-form mean.
"""

import numpy as np
import pytest
import torch

import gqa_kv_cache_qwen3_amd as mtd
import oracle
import workloads as W
from gpu_common import bits, compare, log, request_pages_host

pytestmark = pytest.mark.gpu

Q_NORM = 4.0       # |q| for every head
K_NEEDLE = 120.0   # |k| of the needle key; scale * 4 * 120 = 42.4 against about N(0, 0.35^2) elsewhere
O_CLOSE = 1e-4     # |O - V_needle| bound: fp32 rounding only (the rest of the softmax is < 1e-12)


def _directions(seed: int) -> torch.Tensor:
    """One unit direction per KV head, float32 [Hkv][D]."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    u = torch.randn((W.HKV, W.HEAD_DIM), generator=gen, dtype=torch.float64)
    return (u / u.norm(dim=1, keepdim=True)).float()


def _needle_request(n_tokens: int, needles, seed: int, n_q: int):
    """Random K/V for n_tokens logical positions with K[needles[g], g] = K_NEEDLE * u_g, placed in
    seeded random pages; queries [n_q][Hq][D] all along u_{h/2} with norm Q_NORM."""
    u = _directions(seed)
    k_log = W.normal_bf16((n_tokens, W.HKV, W.HEAD_DIM), seed + 1, "cuda")
    v_log = W.normal_bf16((n_tokens, W.HKV, W.HEAD_DIM), seed + 2, "cuda")
    for g, t in enumerate(needles):
        k_log[t, g] = (K_NEEDLE * u[g]).to(torch.bfloat16).cuda()
    q_one = (Q_NORM * u.repeat_interleave(W.HQ // W.HKV, dim=0)).to(torch.bfloat16)
    q = q_one[None].expand(n_q, W.HQ, W.HEAD_DIM).contiguous().cuda()
    tables, n_pages, _ = W.place_pages([n_tokens], seed, 0)
    table = tables[0]
    kp = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp.view(torch.int16).fill_(0x7FC0)
    vp.view(torch.int16).fill_(0x7FC0)
    j = torch.arange(n_tokens, device="cuda")
    pages = torch.as_tensor(table.astype(np.int64), device="cuda")[j // W.PAGE]
    kp[pages, :, j % W.PAGE, :] = k_log
    vp[pages, :, j % W.PAGE, :] = v_log
    return kp, vp, q, v_log, table


@pytest.mark.parametrize("n_tokens", [65, 200, 4097, 28500, 131072])
def test_decode_needles(n_tokens):
    L = n_tokens
    needles = [0, 63, min(64, L - 1), L - 1, L - 2, L // 2, min(127, L - 1), min(128, L - 1)]
    kp, vp, q, v_log, table = _needle_request(L, needles, 500 + L % 97, 1)
    log(f"decode needles L={L} at {needles}")
    out, lse = mtd.mtd_attn_decode(kp, vp, q, torch.tensor([L], dtype=torch.int32, device="cuda"),
                                   torch.as_tensor(table.astype(np.int32)[None, :], device="cuda"), L, W.SCALE)
    torch.cuda.synchronize()
    vh = v_log.float().cpu()
    for h in range(W.HQ):
        t = needles[h // (W.HQ // W.HKV)]
        err = (out[0, h].cpu() - vh[t, h // (W.HQ // W.HKV)]).abs().max().item()
        assert err <= O_CLOSE, (L, h, t, err)
    kc, vc, ident = request_pages_host(kp, vp, table, L)
    o_ref, l_ref = oracle.decode(bits(q), kc, vc, [L], [ident], W.SCALE)
    compare(out, lse, o_ref, l_ref, f"decode needles L={L}")


@pytest.mark.parametrize("prefix,chunk,split", [(4133, 300, False), (4133, 300, True), (4133, 4096, True)],
                         ids=["one-pass", "halves", "pairs"])
def test_prefill_needles_and_causality(prefix, chunk, split):
    total = prefix + chunk
    needles = [0, 63, 64, prefix - 1, prefix, prefix + chunk // 2, prefix + chunk - 1, 4096]
    kp, vp, q, v_log, table = _needle_request(total, needles, 700 + chunk, chunk)
    ws = torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda") if split else None
    log(f"prefill needles P={prefix} C={chunk} split={split} at {needles}")
    out, lse = mtd.mtd_attn_prefill_chunk(kp, vp, q, prefix, torch.as_tensor(table.astype(np.int32), device="cuda"),
                                          W.SCALE, workspace=ws)
    torch.cuda.synchronize()
    o = out.cpu()
    vh = v_log.float().cpu()
    group = W.HQ // W.HKV
    for g, t in enumerate(needles):
        first = max(t - prefix, 0)  # first chunk row whose position reaches the needle
        if first < chunk:
            err = (o[first:, group * g:group * (g + 1)] - vh[t, g]).abs().max().item()
            assert err <= O_CLOSE, (g, t, err)
        if first > 0:
            # rows before the needle: nowhere near its V (the needle is not visible to them)
            gap = (o[:first, group * g:group * (g + 1)] - vh[t, g]).abs().amax(dim=-1).min().item()
            assert gap > 0.1, (g, t, gap)
    # the oracle on rows around every needle boundary and the chunk's ends
    rows = sorted({r for t in needles for r in (t - prefix - 1, t - prefix, t - prefix + 1)
                   if 0 <= r < chunk} | {0, chunk - 1})
    kc, vc, ident = request_pages_host(kp, vp, table, total)
    k = oracle.gather_logical(kc, ident, total)
    v = oracle.gather_logical(vc, ident, total)
    qb = bits(q)
    o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(qb[rows]), k, v, prefix + np.asarray(rows), W.SCALE)
    compare(out[rows], lse[rows], o_ref, l_ref, f"prefill needles P={prefix} C={chunk}{' split' if split else ''}")


@pytest.mark.parametrize("split", [False, True], ids=["one-pass", "pairs"])
def test_prefill_position_coded_probe(split):
    """All keys of a KV head identical, so every row's softmax is uniform over the keys it may see;
    V carries the token index in exact bf16 integers.  Row i then outputs the mean of those integers
    over keys 0 .. P + i (closed form; the integer sums stay below 2^24, exact in fp32) and
    LSE - s = ln(P + i + 1).  A key missed or seen past the diagonal shifts the mean by about 1/n."""
    prefix, chunk = 28500, 4096
    total = prefix + chunk
    tables, n_pages, _ = W.place_pages([total], 33, 0)
    table = tables[0]
    kp = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    kp.view(torch.int16).fill_(0x7FC0)
    vp.view(torch.int16).fill_(0x7FC0)
    key = W.normal_bf16((W.HKV, W.HEAD_DIM), 34, "cuda")
    j = torch.arange(total, device="cuda")
    pages = torch.as_tensor(table.astype(np.int64), device="cuda")[j // W.PAGE]
    vals = torch.zeros((total, W.HKV, W.HEAD_DIM), dtype=torch.float32, device="cuda")
    vals[:, :, 0] = (j % 64).float()[:, None]
    vals[:, :, 1] = ((j >> 6) % 256).float()[:, None]
    vals[:, :, 2] = (j >> 14).float()[:, None]
    kp[pages, :, j % W.PAGE, :] = key
    vp[pages, :, j % W.PAGE, :] = vals.to(torch.bfloat16)
    q = W.normal_bf16((chunk, W.HQ, W.HEAD_DIM), 35, "cuda")
    ws = torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda") if split else None
    log(f"prefill position-coded probe P={prefix} C={chunk} split={split}")
    out, lse = mtd.mtd_attn_prefill_chunk(kp, vp, q, prefix, torch.as_tensor(table.astype(np.int32), device="cuda"),
                                          W.SCALE, workspace=ws)
    torch.cuda.synchronize()
    o = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    n = prefix + np.arange(chunk) + 1  # keys row i sees
    # closed-form means of the three codes over keys 0 .. n-1
    jj = np.arange(total)
    means = [np.cumsum(jj % 64)[n - 1] / n, np.cumsum((jj >> 6) % 256)[n - 1] / n, np.cumsum(jj >> 14)[n - 1] / n]
    s = W.SCALE * np.einsum("chd,hd->ch", q.double().cpu().numpy(),
                            np.repeat(key.double().cpu().numpy(), W.HQ // W.HKV, axis=0))
    assert np.abs(lse - (s + np.log(n)[:, None])).max() < 1e-4
    for c in range(3):
        err = np.abs(o[:, :, c] - means[c][:, None]) / np.maximum(1.0, means[c][:, None])
        assert err.max() < 1e-6, (c, float(err.max()))
    assert np.abs(o[:, :, 3:]).max() == 0.0
