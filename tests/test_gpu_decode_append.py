"""mtd_attn_decode_append on the GPU: one launch pair that stores each request's new K/V row and
decodes.  Its pools and outputs must be bit for bit those of mtd_kv_append followed by
mtd_attn_decode (ragged lengths, padding rows, out-of-pool pages, graph replay), and its outputs
must match the fp64 oracle over the pool it leaves behind."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import NAN_BF16, DecodeBatch, compare, log

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def new_rows(batch: DecodeBatch, tag: int):
    b = len(batch.lens)
    k_new = W.normal_bf16((b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 11), "cuda")
    v_new = W.normal_bf16((b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 12), "cuda")
    return k_new, v_new


def poison_new_slots(batch: DecodeBatch) -> None:
    """NaN the slot each request's new token goes to, so that a missing store shows."""
    for b, n in enumerate(batch.lens):
        n = int(n)
        if n < 1:
            continue
        page = int(batch.tables[b][(n - 1) // W.PAGE])
        if 0 <= page < batch.num_pages:
            batch.k.view(torch.int16)[page, :, (n - 1) % W.PAGE, :] = NAN_BF16
            batch.v.view(torch.int16)[page, :, (n - 1) % W.PAGE, :] = NAN_BF16


def two_calls(k, v, batch: DecodeBatch, k_new, v_new, max_len):
    b = len(batch.lens)
    cu = torch.arange(b + 1, dtype=torch.int32, device="cuda")
    start = (batch.kv_lens - 1).contiguous()
    mtd.mtd_kv_append(k, v, k_new, v_new, cu, start, batch.bt)
    return mtd.mtd_attn_decode(k, v, batch.q, batch.kv_lens, batch.bt, max_len, W.SCALE)


def same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def check_against_two_calls(batch: DecodeBatch, k_new, v_new, max_len, what):
    k2, v2 = batch.k.clone(), batch.v.clone()
    out, lse = mtd.mtd_attn_decode_append(batch.k, batch.v, batch.q, k_new, v_new, batch.kv_lens, batch.bt,
                                          max_len, W.SCALE)
    out2, lse2 = two_calls(k2, v2, batch, k_new, v_new, max_len)
    torch.cuda.synchronize()
    assert same_bits(batch.k, k2) and same_bits(batch.v, v2), f"{what}: pools differ from append + decode"
    assert torch.equal(out, out2) and torch.equal(lse, lse2), f"{what}: outputs differ from append + decode"
    return out, lse


def test_decode_append_equals_append_then_decode():
    """Ragged lengths around page (64) and split (64 to 512 tokens) boundaries; the pool after the call
    and the outputs equal the two-call sequence bit for bit, and match the oracle over that pool."""
    lens = [1, 2, 63, 64, 65, 127, 511, 512, 513, 1000, 1025, 1153, 1536, 2049, 2305, 4096, 4097, 9000]
    log(f"decode_append ragged lens={lens}")
    batch = DecodeBatch(lens, 301)
    poison_new_slots(batch)
    k_new, v_new = new_rows(batch, 301)
    out, lse = check_against_two_calls(batch, k_new, v_new, batch.max_len, "decode_append ragged")
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode_append ragged")


def test_decode_append_padding_rows_store_nothing():
    """Requests of length 0 (a batch padded to a captured size) store nothing and give O = 0,
    LSE = -inf; a length above max_kv_len stores nothing either.  The pools equal the two-call path's."""
    lens = [700, 0, 65, 0, 3000]
    log(f"decode_append padding lens={lens}")
    batch = DecodeBatch([max(n, 1) for n in lens], 302)
    batch.lens = np.asarray(lens, dtype=np.int64)
    batch.kv_lens = torch.as_tensor(batch.lens.astype(np.int32), device="cuda")
    poison_new_slots(batch)
    k_new, v_new = new_rows(batch, 302)
    before_k, before_v = batch.k.clone(), batch.v.clone()
    out, lse = check_against_two_calls(batch, k_new, v_new, 3000, "decode_append padding")
    for b in (1, 3):
        assert torch.all(out[b] == 0) and torch.all(torch.isneginf(lse[b]))
    # the padding rows' would-be slot (position -1) does not exist; every change to the pools is one of
    # the three real requests' new slots
    for pool, before in ((batch.k, before_k), (batch.v, before_v)):
        changed = (pool.view(torch.int16) != before.view(torch.int16)).any(dim=3).any(dim=1).nonzero().tolist()
        want = {(int(batch.tables[b][(n - 1) // W.PAGE]), (n - 1) % W.PAGE) for b, n in enumerate(lens) if n >= 1}
        assert {tuple(c) for c in changed} == want
    # a length beyond max_kv_len: decode clamps it, and nothing is stored
    k3, v3 = batch.k.clone(), batch.v.clone()
    mtd.mtd_attn_decode_append(batch.k, batch.v, batch.q[:1].contiguous(), k_new[:1].contiguous(),
                               v_new[:1].contiguous(), torch.tensor([701], dtype=torch.int32, device="cuda"),
                               batch.bt[:1].contiguous(), 700, W.SCALE)
    torch.cuda.synchronize()
    assert same_bits(batch.k, k3) and same_bits(batch.v, v3)


def test_decode_append_out_of_pool_page():
    """A new token whose page id lies outside the pool is neither stored nor attended to, exactly as
    with mtd_kv_append + mtd_attn_decode."""
    lens = [130, 64, 1000]
    log(f"decode_append out-of-pool page lens={lens}")
    batch = DecodeBatch(lens, 303)
    tb = batch.tables.copy()
    tb[0, (130 - 1) // W.PAGE] = -1                 # request 0's new token's page
    tb[2, (1000 - 1) // W.PAGE] = batch.num_pages   # request 2's, one past the pool
    batch.tables = tb
    batch.bt = torch.as_tensor(tb, device="cuda")
    k_new, v_new = new_rows(batch, 303)
    out, lse = check_against_two_calls(batch, k_new, v_new, batch.max_len, "decode_append out-of-pool page")
    assert torch.isfinite(out).all() and torch.isfinite(lse).all()


def test_decode_append_graph_replay():
    """One decode step (store + attend) captured as a HIP graph and replayed three times, each replay
    with fresh rows and queries and the lengths advanced by one: every replay's pools and outputs equal
    eager calls on a copy of the pools, and the last replay matches the oracle."""
    lens0 = [439, 64, 1500, 2048]
    log(f"decode_append graph replay lens0={lens0}")
    batch = DecodeBatch([n + 3 for n in lens0], 304)   # pages for three more tokens each
    lens = torch.as_tensor(np.asarray(lens0, dtype=np.int32), device="cuda")
    batch.kv_lens = lens
    max_len = max(lens0) + 3
    k_new, v_new = new_rows(batch, 304)
    out = torch.empty((len(lens0), W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda")
    lse = torch.empty((len(lens0), W.HQ), dtype=torch.float32, device="cuda")
    ws = torch.empty(mtd.decode_workspace_bytes(len(lens0), max_len), dtype=torch.uint8, device="cuda")
    k_eager, v_eager = batch.k.clone(), batch.v.clone()
    g = torch.cuda.CUDAGraph()
    lens.add_(1)
    k_graph, v_graph = batch.k.clone(), batch.v.clone()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mtd.mtd_attn_decode_append(k_graph, v_graph, batch.q, k_new, v_new, lens, batch.bt, max_len, W.SCALE,
                                   workspace=ws, out=out, lse=lse)
    for step in range(3):
        # fresh inputs for this step, written in place into the captured tensors
        k_new.copy_(W.normal_bf16(tuple(k_new.shape), W.torch_seed(304, 20, step), "cuda"))
        v_new.copy_(W.normal_bf16(tuple(v_new.shape), W.torch_seed(304, 21, step), "cuda"))
        batch.q.copy_(W.normal_bf16(tuple(batch.q.shape), W.torch_seed(304, 22, step), "cuda"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, l_e = mtd.mtd_attn_decode_append(k_eager, v_eager, batch.q, k_new, v_new, lens, batch.bt, max_len,
                                              W.SCALE)
        torch.cuda.synchronize()
        assert same_bits(k_graph, k_eager) and same_bits(v_graph, v_eager), f"replay {step}: pools differ"
        assert torch.equal(out, o_e) and torch.equal(lse, l_e), f"replay {step}: outputs differ"
        if step < 2:
            lens.add_(1)
            torch.cuda.synchronize()
    batch.k, batch.v = k_graph, v_graph
    batch.lens = lens.cpu().numpy().astype(np.int64)
    o_ref, l_ref = batch.reference()
    compare(out, lse, o_ref, l_ref, "decode_append graph replay (last step)")
