"""The mixed scheduler step as one step on one shared pool, against the fp64 oracle.

Long prompts are prefilled one 4096-token chunk per scheduler step while other requests' decode
steps are interleaved ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker Audio",
section Chunked Prefill for Long Audio).  One step here: one mtd_kv_append of the chunk's 4096
tokens (request A at prefix 32,768) and one new token for each of 31 decode requests (lengths
log-uniform in [2000, 68000]); then mtd_attn_prefill_chunk of A's chunk with the workspace (the
balanced pair schedule and its merge, as the bench times it); then mtd_attn_decode of the 31
requests.  The step runs sequentially, again on a twin pool with the decode on a second stream
beside the prefill, and once more with the prefill held to 240 compute units
(mtd_attn_prefill_chunk_cus) so that the decode runs on the other 16 at the same time.  Each run is checked against the oracle: the whole pool after the
append bit for bit, every one of the 4096 x 16 prefill rows and all 31 decode rows within the
tolerances; and the two runs must agree bit for bit."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import MixedInputs, bits, compare, log
from oracle.parallel import decode_problem, prefill_problem

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def _step(m: MixedInputs, ws_p, ws_d, side=None, cu_budget=0):
    """append; prefill (workspace, on a CU budget when given); decode, on `side` when given
    (joined before returning)."""
    main = torch.cuda.current_stream()
    mtd.mtd_kv_append(m.k, m.v, m.k_new, m.v_new, m.cu, m.start, m.bt)
    if side is not None:
        appended = torch.cuda.Event()
        appended.record(main)
    o_a, l_a = mtd.mtd_attn_prefill_chunk_cus(m.k, m.v, m.q_a, m.prefix, m.bt_a, W.SCALE, ws_p, cu_budget)
    if side is None:
        o_d, l_d = mtd.mtd_attn_decode(m.k, m.v, m.q_d, m.kv_lens, m.bt_dec, m.max_len, W.SCALE, workspace=ws_d)
    else:
        side.wait_event(appended)
        with torch.cuda.stream(side):
            o_d, l_d = mtd.mtd_attn_decode(m.k, m.v, m.q_d, m.kv_lens, m.bt_dec, m.max_len, W.SCALE,
                                           workspace=ws_d)
            done = torch.cuda.Event()
            done.record()
        main.wait_event(done)
    return o_a, l_a, o_d, l_d


def test_mixed_step_one_pool_against_oracle(oracle_pool):
    p = W.MIXED.params
    prefix, chunk = p["prefix"], p["chunk"]
    lens = W.loguniform_lengths(p["batch"], p["lo"], p["hi"], W.MIXED.tag, 0)
    log(f"mixed step on one pool: chunk {chunk} at {prefix} + decode of {len(lens)} ({int(lens.sum())} keys)")
    seq = MixedInputs(prefix, chunk, lens, W.MIXED.tag)
    ovl = MixedInputs(prefix, chunk, lens, W.MIXED.tag)
    torch.cuda.synchronize()
    k_before, v_before = bits(seq.k), bits(seq.v)
    ws_p = torch.empty(mtd.prefill_workspace_bytes(chunk), dtype=torch.uint8, device="cuda")
    ws_d = torch.empty(mtd.decode_workspace_bytes(len(lens), seq.max_len), dtype=torch.uint8, device="cuda")
    ws_p2, ws_d2 = torch.empty_like(ws_p), torch.empty_like(ws_d)

    log("mixed step: sequential")
    want = _step(seq, ws_p, ws_d)
    torch.cuda.synchronize()
    log("mixed step: decode on a second stream")
    side = torch.cuda.Stream()
    got = _step(ovl, ws_p2, ws_d2, side)
    torch.cuda.synchronize()
    for name, a, b in zip(("prefill O", "prefill LSE", "decode O", "decode LSE"), want, got):
        assert torch.equal(a, b), name
    # the overlapped step as the bench runs it: prefill on 240 of the CUs, decode beside it on a
    # second stream (a third twin pool, so that its append starts from the same bits)
    log("mixed step: prefill on a 240-CU budget, decode on a second stream")
    ovl2 = MixedInputs(prefix, chunk, lens, W.MIXED.tag)
    spread = _step(ovl2, torch.empty_like(ws_p), torch.empty_like(ws_d), side, cu_budget=240)
    torch.cuda.synchronize()
    assert torch.equal(spread[2], want[2]) and torch.equal(spread[3], want[3])  # decode: same kernels

    # the append, bit for bit over both whole pools
    k_after, v_after = bits(seq.k), bits(seq.v)
    k_exp, v_exp = oracle.kv_append(k_before, v_before, bits(seq.k_new), bits(seq.v_new), seq.cu_np,
                                    seq.start_np, seq.tables)
    del k_before, v_before
    assert np.array_equal(k_after, k_exp) and np.array_equal(v_after, v_exp)
    assert np.array_equal(bits(ovl.k), k_exp) and np.array_equal(bits(ovl.v), v_exp)
    assert np.array_equal(bits(ovl2.k), k_exp) and np.array_equal(bits(ovl2.v), v_exp)
    del k_exp, v_exp, ovl2

    # the attention outputs against the oracle over the pool as it sits on the device
    probs = [prefill_problem(bits(seq.q_a), k_after, v_after, seq.tables[0], prefix)]
    qd = bits(seq.q_d)
    probs += [decode_problem(qd[b:b + 1], k_after, v_after, seq.tables[1 + b], int(lens[b]))
              for b in range(len(lens))]
    log("mixed step: oracle (every prefill row, every decode request)")
    ref = oracle_pool.attention(probs, W.SCALE)
    o_ref = np.concatenate([r[0] for r in ref[1:]])
    l_ref = np.concatenate([r[1] for r in ref[1:]])
    for tag, (o_a, l_a, o_d, l_d) in (("sequential", want), ("second stream", got),
                                      ("240-CU prefill beside the decode", spread)):
        compare(o_a, l_a, ref[0][0], ref[0][1], f"mixed step prefill, all 4096 rows ({tag})")
        compare(o_d, l_d, o_ref, l_ref, f"mixed step decode, all 31 requests ({tag})")
