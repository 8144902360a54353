"""mtd_attn_decode_noalloc (the split partials in the library's static device scratch, nothing
allocated) against mtd_attn_decode with a caller workspace: the same kernels, so the same bits.
Two calls in a row, the second smaller (fewer and shorter requests), so stale partials of the
first would show; the smaller call is also held to the fp64 oracle."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import DecodeBatch, compare, log

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def _both(batch: DecodeBatch):
    ref_o, ref_l = mtd.mtd_attn_decode(batch.k, batch.v, batch.q, batch.kv_lens, batch.bt, batch.max_len, W.SCALE)
    out = torch.full_like(ref_o, float("nan"))
    lse = torch.full_like(ref_l, float("nan"))
    mtd.mtd_attn_decode_noalloc(batch.k, batch.v, batch.q, batch.kv_lens, batch.bt, batch.max_len, W.SCALE, out, lse)
    torch.cuda.synchronize()
    return ref_o, ref_l, out, lse


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    p = W.DECODE16.params
    big = DecodeBatch(W.uniform_lengths(p["batch"], p["lo"], p["hi"], W.DECODE16.tag, 0), 401)
    small = DecodeBatch([5, 64, 700, 1025, 3000, 9000], 402)
    for name, batch in (("16 requests of 27k-30k tokens", big), ("6 requests of 5-9000 tokens", small)):
        log(f"decode_noalloc: {name}")
        ref_o, ref_l, out, lse = _both(batch)
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), name
    o_ref, l_ref = small.reference()
    compare(out, lse, o_ref, l_ref, "decode_noalloc, second (smaller) call")


def test_noalloc_at_the_scratch_limit_and_beyond():
    """31 requests at the 128K cap fill 7936 of the 8128 partials the scratch holds; one more
    request's worth is refused on the host with MTD_ERR_WORKSPACE before anything is enqueued."""
    lens = np.full(31, 2000)
    lens[[0, 30]] = W.CONTEXT_CAP
    batch = DecodeBatch(lens, 403, poison=False)
    log("decode_noalloc at max_kv_len 131072, 31 requests")
    ref_o, ref_l, out, lse = _both(batch)
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
    need = mtd.decode_workspace_bytes(33, W.CONTEXT_CAP)
    assert need > mtd.MTD_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((33, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    kv_lens = torch.ones(33, dtype=torch.int32, device="cuda")
    bt = torch.zeros((33, W.CONTEXT_CAP // W.PAGE), dtype=torch.int32, device="cuda")
    o = torch.empty((33, W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda")
    l = torch.empty((33, W.HQ), dtype=torch.float32, device="cuda")
    with pytest.raises(mtd.MtdError) as err:
        mtd.mtd_attn_decode_noalloc(batch.k, batch.v, q, kv_lens, bt, W.CONTEXT_CAP, W.SCALE, o, l)
    assert err.value.status == mtd.MTD_ERR_WORKSPACE
