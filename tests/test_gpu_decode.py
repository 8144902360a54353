"""mtd_attn_decode on the GPU against the fp64 oracle, plus the bitwise invariants of the
page-table read path (placement, batch, run to run) and closed-form probes at full length."""

import math

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import DecodeBatch, bits, compare, log, new_pool

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def run(batch: DecodeBatch, max_len=None, ws=None):
    max_len = batch.max_len if max_len is None else max_len
    out, lse = mtd.mtd_attn_decode(batch.k, batch.v, batch.q, batch.kv_lens, batch.bt, max_len,
                                   W.SCALE, workspace=ws)
    torch.cuda.synchronize()
    return out, lse


def test_decode_ragged_small():
    """Lengths around page (64) and split boundaries, one token, several pages."""
    lens = [1, 2, 63, 64, 65, 127, 511, 512, 513, 1000, 1025, 1536, 2049]
    log(f"decode ragged small lens={lens}")
    batch = DecodeBatch(lens, 101)
    out, lse = run(batch)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode ragged small")


def test_decode_split_bands():
    """Lengths on both sides of each change of split size (64, 128, 256 and 512 tokens at 1024, 2048
    and 4096 tokens) and of split boundaries within each band, in one batch."""
    lens = [960, 1023, 1024, 1025, 1152, 1153, 1300, 1536, 1537, 2048, 2049, 2304, 2305, 3000, 4095, 4096,
            4097, 4609, 9000]
    log(f"decode split bands lens={lens}")
    batch = DecodeBatch(lens, 104)
    out, lse = run(batch)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode split bands")
    # a request's split depends on its own length only: a sub-batch (other order, other bound)
    # gives the same bits
    sub = [18, 0, 8, 11, 15]
    idx = torch.tensor(sub, device="cuda")
    out2, lse2 = mtd.mtd_attn_decode(batch.k, batch.v, batch.q[idx].contiguous(), batch.kv_lens[idx].contiguous(),
                                     batch.bt[idx].contiguous(), int(max(lens[i] for i in sub)), W.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out2, out[idx]) and torch.equal(lse2, lse[idx])


def test_decode_batch_beyond_one_wavefront_scan():
    """130 requests: the split and merge kernels locate a request's splits by scanning kv_lens 64
    requests at a time, so batches above 64 cross that boundary twice."""
    lens = W.loguniform_lengths(130, 1, 3000, 2, 77)
    log(f"decode batch 130, lens sum {int(lens.sum())}")
    batch = DecodeBatch(lens, 105)
    out, lse = run(batch)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode batch 130")
    sub = [129, 64, 63, 0, 100]
    idx = torch.tensor(sub, device="cuda")
    out2, lse2 = mtd.mtd_attn_decode(batch.k, batch.v, batch.q[idx].contiguous(), batch.kv_lens[idx].contiguous(),
                                     batch.bt[idx].contiguous(), batch.max_len, W.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out2, out[idx]) and torch.equal(lse2, lse[idx])


def test_decode_max_len_above_longest():
    """A loose host bound (max_kv_len > every kv_len) gives the same bits as the tight one."""
    batch = DecodeBatch([700, 5, 3000], 102)
    log("decode loose max_kv_len")
    out1, lse1 = run(batch)
    big = 131072
    stride = big // W.PAGE
    bt = torch.full((3, stride), int(batch.spare[0]), dtype=torch.int32, device="cuda")
    bt[:, : batch.bt.shape[1]] = batch.bt
    out2, lse2 = mtd.mtd_attn_decode(batch.k, batch.v, batch.q, batch.kv_lens, bt, big, W.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_decode16_full_size():
    """16 concurrent 38-minute meetings: KV lengths uniform in [27000, 30000]."""
    p = W.DECODE16.params
    lens = W.uniform_lengths(p["batch"], p["lo"], p["hi"], W.DECODE16.tag, 0)
    log(f"decode16 full size lens={lens.tolist()}")
    batch = DecodeBatch(lens, W.DECODE16.tag)
    out, lse = run(batch)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode16")


def test_mixed_step_decode_part_full_size():
    """The 31 decode requests of the mixed step: KV lengths log-uniform in [2000, 68000]."""
    p = W.MIXED.params
    lens = W.loguniform_lengths(p["batch"], p["lo"], p["hi"], W.MIXED.tag, 0)
    log(f"mixed decode part lens={lens.tolist()}")
    batch = DecodeBatch(lens, W.MIXED.tag + 1000)
    out, lse = run(batch)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "mixed decode part")


def test_fulldepth_call_shape_sampled():
    """One full-depth decode call: 64 requests, log-uniform lengths up to the 128K cap;
    the oracle checks a sample of requests (shortest, longest and four seeded picks)."""
    p = W.FULLDEPTH.params
    lens = W.loguniform_lengths(p["batch"], p["lo"], p["hi"] - p["steps"], W.FULLDEPTH.tag, 0)
    log(f"fulldepth call shape: 64 requests, sum L = {int(lens.sum())}")
    batch = DecodeBatch(lens, W.FULLDEPTH.tag + 2000)
    out, lse = run(batch)
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)),
                   *W.rng(5, 7).choice(64, size=4, replace=False).tolist()})
    o_ref, l_ref = batch.reference(pick)
    compare(out[pick], lse[pick], o_ref, l_ref, f"fulldepth sampled {pick}")


def test_decode_deterministic_and_batch_invariant():
    lens = W.uniform_lengths(16, 27000, 30000, W.DECODE16.tag, 0)
    batch = DecodeBatch(lens, 103)
    log("decode determinism + batch invariance")
    out1, lse1 = run(batch)
    out2, lse2 = run(batch)
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    # the same requests in a sub-batch (and in another order) give identical bits
    sub = [9, 2, 14]
    idx = torch.tensor(sub, device="cuda")
    out3, lse3 = mtd.mtd_attn_decode(batch.k, batch.v, batch.q[idx].contiguous(),
                                     batch.kv_lens[idx].contiguous(), batch.bt[idx].contiguous(),
                                     batch.max_len, W.SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out3, out1[idx]) and torch.equal(lse3, lse1[idx])


def scatter_logical(k_log, v_log, table, n_pages, device="cuda"):
    """Test-side page placement of logical rows [L][Hkv][D] (poison elsewhere)."""
    kp, vp = new_pool(n_pages, device), new_pool(n_pages, device)
    n = k_log.shape[0]
    j = torch.arange(n, device=device)
    pages = torch.as_tensor(np.asarray(table, dtype=np.int64), device=device)[j // W.PAGE]
    kp[pages, :, j % W.PAGE, :] = k_log
    vp[pages, :, j % W.PAGE, :] = v_log
    return kp, vp


def test_page_placement_invariance_bitwise():
    """The same logical K/V under two seeded placements and the identity placement: same bits."""
    n = 5000
    k_log = W.normal_bf16((n, W.HKV, W.HEAD_DIM), 11, "cuda")
    v_log = W.normal_bf16((n, W.HKV, W.HEAD_DIM), 12, "cuda")
    q = W.normal_bf16((1, W.HQ, W.HEAD_DIM), 13, "cuda")
    used = (n + W.PAGE - 1) // W.PAGE
    results = []
    for tag in (None, 1, 2):
        table = np.arange(used) if tag is None else W.rng(42, tag).permutation(used + 3)[:used]
        kp, vp = scatter_logical(k_log, v_log, table, used + 3)
        bt = torch.as_tensor(table.astype(np.int32)[None, :], device="cuda")
        log(f"placement invariance tag={tag}")
        out, lse = mtd.mtd_attn_decode(kp, vp, q, torch.tensor([n], dtype=torch.int32, device="cuda"),
                                       bt, n, W.SCALE)
        torch.cuda.synchronize()
        results.append((out, lse))
    for out, lse in results[1:]:
        assert torch.equal(out, results[0][0]) and torch.equal(lse, results[0][1])


def test_position_coded_probe():
    """All keys identical, so every softmax is uniform over the attended tokens; V carries the
    token index in exact bf16 integers.  O is then the closed-form mean of those integers and
    LSE - s = ln(L): a missing, repeated or misplaced token shifts the mean by about 1/L."""
    lens = np.array([1, 64, 65, 4097, 28500, 67501, 131072])
    b = len(lens)
    tables, n_pages, spare = W.place_pages(lens, 31, 0)
    stride = tables.shape[1]
    kp, vp = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")
    key = W.normal_bf16((W.HKV, W.HEAD_DIM), 14, "cuda")
    for r, n in enumerate(lens):
        j = torch.arange(int(n), device="cuda")
        pages = torch.as_tensor(tables[r].astype(np.int64), device="cuda")[j // W.PAGE]
        vals = torch.zeros((int(n), W.HKV, W.HEAD_DIM), dtype=torch.float32, device="cuda")
        vals[:, :, 0] = (j % 64).float()[:, None]
        vals[:, :, 1] = ((j >> 6) % 256).float()[:, None]
        vals[:, :, 2] = (j >> 14).float()[:, None]
        kp[pages, :, j % W.PAGE, :] = key
        vp[pages, :, j % W.PAGE, :] = vals.to(torch.bfloat16)
    q = W.normal_bf16((b, W.HQ, W.HEAD_DIM), 15, "cuda")
    log(f"position-coded probe lens={lens.tolist()}")
    out, lse = mtd.mtd_attn_decode(kp, vp, q, torch.as_tensor(lens.astype(np.int32), device="cuda"),
                                   torch.as_tensor(tables, device="cuda"), int(lens.max()), W.SCALE)
    torch.cuda.synchronize()
    out = out.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    qh = q.double().cpu().numpy()
    kh = key.double().cpu().numpy()
    for r, n in enumerate(lens):
        j = np.arange(int(n))
        means = [np.mean(j % 64), np.mean((j >> 6) % 256), np.mean(j >> 14)]
        for h in range(W.HQ):
            s = W.SCALE * float(qh[r, h] @ kh[h // 2])
            assert abs(lse[r, h] - (s + math.log(n))) < 1e-5, (r, h)
            for c in range(3):
                # uniform weights are exactly 1 in bf16; only fp32 rounding of the merge remains
                assert abs(out[r, h, c] - means[c]) < 4e-6 * max(1.0, means[c]) + 1e-6, (r, h, c, out[r, h, c], means[c])
            assert np.abs(out[r, h, 3:]).max() == 0.0
