"""The mixed scheduler step with its decode on a second stream: the prefill (library's stream) and
the decode (second stream, default priority) both read the pool the append just wrote, so running
them concurrently must give exactly the bits of the sequential step."""

import numpy as np
import pytest
import torch

import workloads as W
from gpu_common import fill_normal_, log

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def _mixed_inputs(prefix, chunk, lens, tag):
    final = np.concatenate([[prefix + chunk], lens])
    tables, n_pages, _ = W.place_pages(final, tag, 0)
    k = torch.empty((n_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    fill_normal_(k, W.torch_seed(tag, 1))
    fill_normal_(v, W.torch_seed(tag, 2))
    n_new = chunk + len(lens)
    k_new = W.normal_bf16((n_new, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 3), "cuda")
    v_new = W.normal_bf16((n_new, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 4), "cuda")
    q_a = W.normal_bf16((chunk, W.HQ, W.HEAD_DIM), W.torch_seed(tag, 5), "cuda")
    q_d = W.normal_bf16((len(lens), W.HQ, W.HEAD_DIM), W.torch_seed(tag, 6), "cuda")
    cu = np.concatenate([[0, chunk], chunk + np.arange(1, len(lens) + 1)]).astype(np.int32)
    start = np.concatenate([[prefix], lens - 1]).astype(np.int32)
    bt = torch.as_tensor(tables, device="cuda")
    return dict(k=k, v=v, k_new=k_new, v_new=v_new, q_a=q_a, q_d=q_d, bt=bt,
                cu=torch.as_tensor(cu, device="cuda"), start=torch.as_tensor(start, device="cuda"),
                kv_lens=torch.as_tensor(lens.astype(np.int32), device="cuda"), max_len=int(lens.max()))


def _step(m, prefix, side=None):
    """append; prefill; decode (on `side` when given, joined back before returning)."""
    main = torch.cuda.current_stream()
    mtd.mtd_kv_append(m["k"], m["v"], m["k_new"], m["v_new"], m["cu"], m["start"], m["bt"])
    o_a, l_a = mtd.mtd_attn_prefill_chunk(m["k"], m["v"], m["q_a"], prefix, m["bt"][0].contiguous(), W.SCALE)
    bt_dec = m["bt"][1:].contiguous()
    if side is None:
        o_d, l_d = mtd.mtd_attn_decode(m["k"], m["v"], m["q_d"], m["kv_lens"], bt_dec, m["max_len"], W.SCALE)
    else:
        appended = torch.cuda.Event()
        appended.record(main)
        side.wait_event(appended)
        with torch.cuda.stream(side):
            o_d, l_d = mtd.mtd_attn_decode(m["k"], m["v"], m["q_d"], m["kv_lens"], bt_dec, m["max_len"], W.SCALE)
            done = torch.cuda.Event()
            done.record()
        main.wait_event(done)
    return o_a, l_a, o_d, l_d


def test_mixed_step_overlap_matches_sequential():
    """The full-size mixed step (chunk 4096 at prefix 32,768 + 31 decodes), twice on twin pools:
    sequential, then with the decode on a second stream; three overlapped steps in a row."""
    p = W.MIXED.params
    lens = W.loguniform_lengths(p["batch"], p["lo"], p["hi"], W.MIXED.tag, 0)
    log("mixed step: sequential vs decode on a second stream")
    seq = _mixed_inputs(p["prefix"], p["chunk"], lens, W.MIXED.tag)
    ovl = _mixed_inputs(p["prefix"], p["chunk"], lens, W.MIXED.tag)
    want = _step(seq, p["prefix"])
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for rep in range(3):
        got = _step(ovl, p["prefix"], side)
        torch.cuda.synchronize()
        for name, a, b in zip(("prefill O", "prefill LSE", "decode O", "decode LSE"), want, got):
            assert torch.equal(a, b), (rep, name)
    assert torch.equal(seq["k"], ovl["k"]) and torch.equal(seq["v"], ovl["v"])
