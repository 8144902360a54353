"""Device-resident block-table entries outside [0, num_pages) are trusted, not checked on the host;
the header fixes what the kernels do with them: mtd_kv_append skips the token (every other byte of
the pools is unchanged), mtd_attn_decode skips the page (the result is attention over the keys of
the valid pages), and mtd_attn_prefill_chunk reads page 0 in its place (unspecified but finite
values, no access outside the pools)."""

import numpy as np
import pytest
import torch

import gqa_kv_cache_qwen3_amd as mtd
import oracle
import workloads as W
from gpu_common import bits, compare, log, new_pool

pytestmark = pytest.mark.gpu


def _i32(values):
    return torch.as_tensor(np.asarray(values, dtype=np.int32), device="cuda")


def test_append_skips_out_of_pool_pages():
    n_pages = 6
    kp, vp = new_pool(n_pages, "cuda", seed=71), new_pool(n_pages, "cuda", seed=72)
    k0, v0 = kp.clone(), vp.clone()
    table = _i32([[3, -1, n_pages + 2, 1]])  # logical pages 1 and 2 are out of the pool
    n = 256
    k_new = W.normal_bf16((n, W.HKV, W.HEAD_DIM), 73, "cuda")
    v_new = W.normal_bf16((n, W.HKV, W.HEAD_DIM), 74, "cuda")
    log("append with out-of-pool page ids")
    mtd.mtd_kv_append(kp, vp, k_new, v_new, _i32([0, n]), _i32([0]), table)
    torch.cuda.synchronize()
    ek, ev = k0.clone(), v0.clone()
    for pos in range(n):
        page = int(table[0, pos // W.PAGE])
        if 0 <= page < n_pages:
            ek[page, :, pos % W.PAGE] = k_new[pos]
            ev[page, :, pos % W.PAGE] = v_new[pos]
    assert torch.equal(kp.view(torch.int16), ek.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), ev.view(torch.int16))


def test_decode_skips_out_of_pool_pages():
    n_pages = 8
    kp, vp = new_pool(n_pages, "cuda", seed=75), new_pool(n_pages, "cuda", seed=76)
    L = 5 * W.PAGE - 7
    pages = [4, 1, -3, 6, n_pages]  # logical pages 2 and 4 are out of the pool
    q = W.normal_bf16((1, W.HQ, W.HEAD_DIM), 77, "cuda")
    log("decode with out-of-pool page ids")
    out, lse = mtd.mtd_attn_decode(kp, vp, q, _i32([L]), _i32([pages]), L, W.SCALE)
    torch.cuda.synchronize()
    # expected: attention over the keys of the valid pages only
    kh, vh = bits(kp), bits(vp)
    keep = [(e, p) for e, p in enumerate(pages) if 0 <= p < n_pages]
    k_rows, v_rows = [], []
    for e, p in keep:
        n_valid = min(W.PAGE, L - e * W.PAGE)
        k_rows.append(oracle.bf16_to_f64(kh[p, :, :n_valid].transpose(1, 0, 2)))
        v_rows.append(oracle.bf16_to_f64(vh[p, :, :n_valid].transpose(1, 0, 2)))
    k = np.concatenate(k_rows)
    v = np.concatenate(v_rows)
    o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(bits(q)), k, v, np.array([k.shape[0] - 1]), W.SCALE)
    compare(out, lse, o_ref, l_ref, "decode over the valid pages")


def test_prefill_reads_page_zero_for_out_of_pool_pages():
    n_pages = 8
    kp, vp = new_pool(n_pages, "cuda", seed=78), new_pool(n_pages, "cuda", seed=79)
    prefix, chunk = 3 * W.PAGE, 2 * W.PAGE - 5
    table = _i32([2, n_pages + 1, 5, -2, 7])
    q = W.normal_bf16((chunk, W.HQ, W.HEAD_DIM), 80, "cuda")
    for ws in (None, torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda")):
        log(f"prefill with out-of-pool page ids, workspace={ws is not None}")
        out, lse = mtd.mtd_attn_prefill_chunk(kp, vp, q, prefix, table, W.SCALE, workspace=ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all() and torch.isfinite(lse).all()
