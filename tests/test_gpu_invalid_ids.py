"""Device-resident block-table entries outside [0, num_pages) are trusted, not checked on the host;
the header fixes what the kernels do with them: mtd_kv_append skips the token (every other byte of
the pools is unchanged), mtd_attn_decode skips the page (the result is attention over the keys of
the valid pages), and mtd_attn_prefill_chunk gives every query row attention over the keys of the
valid pages it may see (a row that sees none gets O = 0 and LSE = -inf); no access outside the
pools."""

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


def _prefill_valid_reference(kh, vh, q_bits, prefix, table, n_pages):
    """Oracle over the keys of the valid pages: row i sees the valid keys at positions <= prefix + i.
    Returns (O, LSE, rows with no valid key)."""
    total = prefix + q_bits.shape[0]
    keep = [j for j in range(total) if 0 <= table[j // W.PAGE] < n_pages]
    k = np.stack([oracle.bf16_to_f64(kh[table[j // W.PAGE], :, j % W.PAGE]) for j in keep])
    v = np.stack([oracle.bf16_to_f64(vh[table[j // W.PAGE], :, j % W.PAGE]) for j in keep])
    seen = np.searchsorted(np.asarray(keep), prefix + np.arange(q_bits.shape[0]), side="right")
    rows = np.nonzero(seen > 0)[0]
    o = np.zeros((q_bits.shape[0], W.HQ, W.HEAD_DIM))
    lse = np.full((q_bits.shape[0], W.HQ), -np.inf)
    o[rows], lse[rows] = oracle.attention(oracle.bf16_to_f64(q_bits[rows]), k, v, seen[rows] - 1, W.SCALE)
    return o, lse, np.nonzero(seen == 0)[0]


@pytest.mark.parametrize("prefix,chunk,table", [
    (3 * W.PAGE, 2 * W.PAGE - 5, [2, 9, 5, -2, 7]),          # prefix and chunk pages out of the pool
    (0, 300, [-1, 3, 100, 6, 1]),                             # the first rows see no valid key
    (4000, 4096, None),                                       # many tiles (pair schedule), a few bad ids
])
def test_prefill_skips_out_of_pool_pages(prefix, chunk, table):
    total = prefix + chunk
    n_used = (total + W.PAGE - 1) // W.PAGE
    if table is None:
        rng = np.random.default_rng(81)
        table = rng.permutation(n_used + 4)[:n_used].astype(np.int64)
        table[[3, 40, n_used - 70, n_used - 2]] = [-5, n_used + 4, 1 << 30, -1]
        n_pages = n_used + 4
    else:
        n_pages = 8
    kp, vp = new_pool(n_pages, "cuda", seed=78), new_pool(n_pages, "cuda", seed=79)
    q = W.normal_bf16((chunk, W.HQ, W.HEAD_DIM), 80, "cuda")
    o_ref, l_ref, empty = _prefill_valid_reference(bits(kp), bits(vp), bits(q), prefix, np.asarray(table), n_pages)
    full = [r for r in range(chunk) if r not in set(empty.tolist())]
    for ws in (None, torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda")):
        log(f"prefill with out-of-pool page ids, P={prefix} C={chunk}, workspace={ws is not None}")
        out, lse = mtd.mtd_attn_prefill_chunk(kp, vp, q, prefix, _i32(table), W.SCALE, workspace=ws)
        torch.cuda.synchronize()
        if len(empty):
            e = torch.as_tensor(empty, device="cuda")
            assert torch.equal(out[e], torch.zeros_like(out[e]))
            assert bool((lse[e] == -float("inf")).all())
        idx = torch.as_tensor(full, device="cuda")
        compare(out[idx], lse[idx], o_ref[full], l_ref[full],
                f"prefill over the valid pages, P={prefix} C={chunk}{' split' if ws is not None else ''}")
