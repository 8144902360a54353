"""Full-depth decode at full size: 28 layers x 64 requests with all layers' KV resident in HBM,
128 steps of (append one token per request, decode) per layer.  Appends are checked bit for bit
on layers 0 and 27 at every step; decode is checked against the fp64 oracle at steps
{0, 63, 127} x layers {0, 13, 27} on eight requests per call (shortest, longest, six seeded)."""

import gc

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import bits, compare, log

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")

SAMPLE_STEPS = (0, 63, 127)
SAMPLE_LAYERS = (0, 13, 27)
APPEND_LAYERS = (0, 27)


def test_fulldepth_full_size_sampled():
    gc.collect()
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info()
    lens0, tried, need = W.fulldepth_draw(free)
    log(f"fulldepth: seeds tried {tried}, {need / 2**30:.1f} GiB of inputs, sum L0 = {int(lens0.sum())}")
    inp = W.build_fulldepth("cuda", lens0)
    steps, layers, b = inp["steps"], inp["layers"], len(lens0)
    tables = inp["tables"]
    bt = torch.as_tensor(tables, device="cuda")
    cu = torch.arange(b + 1, dtype=torch.int32, device="cuda")
    max_len = int(lens0.max()) + steps
    ws = torch.empty(mtd.decode_workspace_bytes(b, max_len), dtype=torch.uint8, device="cuda")
    picks = sorted({int(np.argmin(lens0)), int(np.argmax(lens0)),
                    *W.rng(5, 8).choice(b, size=6, replace=False).tolist()})
    checked = 0
    for s in range(steps):
        start = torch.as_tensor((lens0 + s).astype(np.int32), device="cuda")
        kv_lens = torch.as_tensor((lens0 + s + 1).astype(np.int32), device="cuda")
        for layer in range(layers):
            kp, vp = inp["k_pools"][layer], inp["v_pools"][layer]
            mtd.mtd_kv_append(kp, vp, inp["k_new"][s, layer], inp["v_new"][s, layer], cu, start, bt)
            out, lse = mtd.mtd_attn_decode(kp, vp, inp["q"][s, layer], kv_lens, bt, max_len, W.SCALE, ws)
            if layer in APPEND_LAYERS:
                entry, slot = oracle.page_of(lens0 + s, W.PAGE)
                pages = torch.as_tensor(tables[np.arange(b), entry].astype(np.int64), device="cuda")
                slots = torch.as_tensor(slot.astype(np.int64), device="cuda")
                assert torch.equal(kp[pages, :, slots, :], inp["k_new"][s, layer]), (s, layer)
                assert torch.equal(vp[pages, :, slots, :], inp["v_new"][s, layer]), (s, layer)
            if s in SAMPLE_STEPS and layer in SAMPLE_LAYERS:
                torch.cuda.synchronize()
                qb = bits(inp["q"][s, layer])
                o_ref, l_ref = [], []
                for r in picks:
                    n = int(lens0[r]) + s + 1
                    used = (n + W.PAGE - 1) // W.PAGE
                    idx = torch.as_tensor(tables[r][:used].astype(np.int64), device="cuda")
                    o, l = oracle.decode(qb[r:r + 1], bits(kp.index_select(0, idx)), bits(vp.index_select(0, idx)),
                                         [n], [np.arange(used)], W.SCALE)
                    o_ref.append(o[0])
                    l_ref.append(l[0])
                compare(out[picks], lse[picks], np.stack(o_ref), np.stack(l_ref), f"fulldepth step {s} layer {layer}")
                checked += 1
        if s % 32 == 0:
            log(f"fulldepth step {s} done")
    torch.cuda.synchronize()
    assert checked == len(SAMPLE_STEPS) * len(SAMPLE_LAYERS)
    del inp, ws
    gc.collect()
    torch.cuda.empty_cache()
