"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph, on the capture stream torch
makes current) and replayed: decode steps over several layers, and a whole chunked prompt.

Every replay must reproduce the same calls made eagerly on a twin pool bit for bit, with eager
work (the copies that stage each step's inputs) and synchronisations between replays; the last
step is also checked against the fp64 oracle.  Capture records only kernel launches: the calls
allocate nothing, set no memory and never synchronise, so the graph holds the same kernels the
eager calls run."""

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_common import bits, compare, log, new_pool, request_pages_host

pytestmark = pytest.mark.gpu

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


def _i32(values):
    return torch.as_tensor(np.asarray(values, dtype=np.int32), device="cuda")


class StepGraph:
    """Fixed input/output buffers for `layers` x (append one token per request, decode) over one
    block table, the graph that reads them, and an eager twin of the same pools."""

    def __init__(self, lens0, steps, layers, tag):
        self.lens0 = np.asarray(lens0, dtype=np.int64)
        self.steps, self.layers = steps, layers
        b = len(self.lens0)
        self.tables, n_pages, _ = W.place_pages(self.lens0 + steps, tag, 0)
        self.bt = torch.as_tensor(self.tables, device="cuda")
        self.max_len = int(self.lens0.max()) + steps
        # every slot holds N(0,1) data, so positions below lens0 act as the prompt already cached
        self.kg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 40, l)) for l in range(layers)]
        self.vg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 41, l)) for l in range(layers)]
        self.ke = [p.clone() for p in self.kg]
        self.ve = [p.clone() for p in self.vg]
        self.q_all = W.normal_bf16((steps, layers, b, W.HQ, W.HEAD_DIM), W.torch_seed(tag, 42), "cuda")
        self.k_all = W.normal_bf16((steps, layers, b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 43), "cuda")
        self.v_all = W.normal_bf16((steps, layers, b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 44), "cuda")
        self.cu = _i32(np.arange(b + 1))
        self.ws = torch.empty(mtd.decode_workspace_bytes(b, self.max_len), dtype=torch.uint8, device="cuda")
        self.ws_e = torch.empty_like(self.ws)
        # the buffers the graph reads and writes
        self.q_buf = torch.empty_like(self.q_all[0])
        self.k_buf = torch.empty_like(self.k_all[0])
        self.v_buf = torch.empty_like(self.v_all[0])
        self.start_buf = torch.zeros(b, dtype=torch.int32, device="cuda")
        self.len_buf = torch.zeros(b, dtype=torch.int32, device="cuda")
        self.o_buf = torch.empty((layers, b, W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda")
        self.l_buf = torch.empty((layers, b, W.HQ), dtype=torch.float32, device="cuda")
        self.graph = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(self.graph):
            for l in range(layers):
                mtd.mtd_kv_append(self.kg[l], self.vg[l], self.k_buf[l], self.v_buf[l], self.cu,
                                  self.start_buf, self.bt)
                mtd.mtd_attn_decode(self.kg[l], self.vg[l], self.q_buf[l], self.len_buf, self.bt,
                                    self.max_len, W.SCALE, self.ws, self.o_buf[l], self.l_buf[l])
        torch.cuda.synchronize()

    def replay_step(self, s):
        """Stage step s's inputs into the fixed buffers (eager copies), replay the graph."""
        self.q_buf.copy_(self.q_all[s])
        self.k_buf.copy_(self.k_all[s])
        self.v_buf.copy_(self.v_all[s])
        self.start_buf.copy_(_i32(self.lens0 + s))
        self.len_buf.copy_(_i32(self.lens0 + s + 1))
        self.graph.replay()

    def eager_step(self, s):
        start, kv_lens = _i32(self.lens0 + s), _i32(self.lens0 + s + 1)
        outs = []
        for l in range(self.layers):
            mtd.mtd_kv_append(self.ke[l], self.ve[l], self.k_all[s, l], self.v_all[s, l], self.cu, start, self.bt)
            outs.append(mtd.mtd_attn_decode(self.ke[l], self.ve[l], self.q_all[s, l], kv_lens, self.bt,
                                            self.max_len, W.SCALE, self.ws_e))
        return outs

    def run_and_check(self, what):
        for s in range(self.steps):
            log(f"{what}: step {s}")
            self.replay_step(s)
            eager = self.eager_step(s)
            torch.cuda.synchronize()
            for l, (o, lse) in enumerate(eager):
                assert torch.equal(self.o_buf[l], o), (what, s, l)
                assert torch.equal(self.l_buf[l], lse), (what, s, l)
        for l in range(self.layers):
            assert torch.equal(self.kg[l], self.ke[l]) and torch.equal(self.vg[l], self.ve[l]), (what, l)
        # the last step against the oracle, on layer 0 and the last layer
        s = self.steps - 1
        for l in sorted({0, self.layers - 1}):
            qb = bits(self.q_all[s, l])
            o_ref, l_ref = [], []
            for r in range(len(self.lens0)):
                n = int(self.lens0[r]) + s + 1
                kc, vc, ident = request_pages_host(self.kg[l], self.vg[l], self.tables[r], n)
                o, lse = oracle.decode(qb[r:r + 1], kc, vc, [n], [ident], W.SCALE)
                o_ref.append(o[0])
                l_ref.append(lse[0])
            compare(self.o_buf[l], self.l_buf[l], np.stack(o_ref), np.stack(l_ref), f"{what} layer {l} last step")


def test_graph_decode_loop_one_request():
    """The tiny workload's decode phase: one request with a 439-token prompt, 32 steps of
    (append its new token, decode), each step one replay of the same graph."""
    p = W.TINY.params
    log("graph: tiny decode loop, 1 request, 32 steps")
    StepGraph([p["prompt"]], p["decode_steps"], 1, W.TINY.tag).run_and_check("graph tiny")


def test_graph_multilayer_decode_step():
    """A full-depth-style step in miniature: 4 layers x 8 requests (KV 1000-9000 tokens) per graph,
    6 steps."""
    lens0 = W.loguniform_lengths(8, 1000, 9000, W.FULLDEPTH.tag, 9)
    log(f"graph: 4 layers x 8 requests, lens0={lens0.tolist()}")
    StepGraph(lens0, 6, 4, W.FULLDEPTH.tag).run_and_check("graph 4x8")


def test_graph_attention_block_step():
    """Whole attention blocks in one graph: 3 layers x (QKV projection -> append -> decode -> output
    projection, whose result feeds the next layer) for 5 requests, 4 steps; every replay bit-identical
    to the same calls made eagerly on twin pools."""
    lens0 = W.loguniform_lengths(5, 100, 3000, W.FULLDEPTH.tag, 11)
    layers, steps, b = 3, 4, len(lens0)
    log(f"graph: attention blocks, {layers} layers x {b} requests, lens0={lens0.tolist()}")
    tables, n_pages, _ = W.place_pages(lens0 + steps, W.FULLDEPTH.tag, 12)
    bt = torch.as_tensor(tables, device="cuda")
    max_len = int(lens0.max()) + steps
    tag = W.FULLDEPTH.tag
    kg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 80, l)) for l in range(layers)]
    vg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 81, l)) for l in range(layers)]
    ke, ve = [p.clone() for p in kg], [p.clone() for p in vg]
    weights = [W.projection_weights(W.torch_seed(tag, 82, l), "cuda") for l in range(layers)]
    x_all = W.normal_bf16((steps, b, W.HIDDEN), W.torch_seed(tag, 83), "cuda")
    cu = _i32(np.arange(b + 1))
    ws_g = torch.empty(mtd.decode_workspace_bytes(b, max_len), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws_g)
    x_buf = torch.empty((b, W.HIDDEN), dtype=torch.bfloat16, device="cuda")
    start_buf = torch.zeros(b, dtype=torch.int32, device="cuda")
    len_buf = torch.zeros(b, dtype=torch.int32, device="cuda")
    q_b = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    k_b = torch.empty((b, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    v_b = torch.empty_like(k_b)
    o_b = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda")
    l_b = torch.empty((b, W.HQ), dtype=torch.float32, device="cuda")
    y_g = torch.empty((layers, b, W.HIDDEN), dtype=torch.bfloat16, device="cuda")

    def block_calls(kp, vp, x, start, kv_lens, ws, y_out, o, lse, q, k, v):
        for l in range(layers):
            w_qkv, w_o = weights[l]
            mtd.mtd_qkv_proj(x, w_qkv, q, k, v)
            mtd.mtd_kv_append(kp[l], vp[l], k, v, cu, start, bt)
            mtd.mtd_attn_decode(kp[l], vp[l], q, kv_lens, bt, max_len, W.SCALE, ws, o, lse)
            mtd.mtd_o_proj(o, w_o, y_out[l])
            x = y_out[l]

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        block_calls(kg, vg, x_buf, start_buf, len_buf, ws_g, y_g, o_b, l_b, q_b, k_b, v_b)
    torch.cuda.synchronize()
    for s in range(steps):
        log(f"graph blocks: step {s}")
        x_buf.copy_(x_all[s])
        start_buf.copy_(_i32(lens0 + s))
        len_buf.copy_(_i32(lens0 + s + 1))
        graph.replay()
        y_e = torch.empty_like(y_g)
        block_calls(ke, ve, x_all[s], _i32(lens0 + s), _i32(lens0 + s + 1), ws_e, y_e,
                    torch.empty_like(o_b), torch.empty_like(l_b), torch.empty_like(q_b),
                    torch.empty_like(k_b), torch.empty_like(v_b))
        torch.cuda.synchronize()
        assert torch.equal(y_g, y_e), s
    for l in range(layers):
        assert torch.equal(kg[l], ke[l]) and torch.equal(vg[l], ve[l]), l


def test_chunked_prefill_graph_replays():
    """A whole chunked prompt in one graph: for each chunk, append its K/V, then prefill it with a
    workspace (4096-token chunks on the pair schedule, the ragged last chunk as halves).  Three
    replays, with eager work between them, each equal the eager calls bit for bit (outputs and
    pools); the last chunk is also checked against the oracle on sampled rows."""
    chunks = [4096, 4096, 1500]
    starts = np.concatenate([[0], np.cumsum(chunks)[:-1]]).astype(np.int64)
    total = int(sum(chunks))
    tables, n_pages, _ = W.place_pages([total], 57, 0)
    bt = torch.as_tensor(tables, device="cuda")
    kg, vg = new_pool(n_pages, "cuda"), new_pool(n_pages, "cuda")  # NaN-poisoned
    ke, ve = kg.clone(), vg.clone()
    k_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(57, 1), "cuda")
    v_log = W.normal_bf16((total, W.HKV, W.HEAD_DIM), W.torch_seed(57, 2), "cuda")
    q_log = W.normal_bf16((total, W.HQ, W.HEAD_DIM), W.torch_seed(57, 3), "cuda")
    ws = torch.empty(mtd.prefill_workspace_bytes(max(chunks)), dtype=torch.uint8, device="cuda")
    ws_e = torch.empty_like(ws)
    cus = [_i32([0, c]) for c in chunks]
    sps = [_i32([s]) for s in starts]
    outs = [torch.empty((c, W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda") for c in chunks]
    lses = [torch.empty((c, W.HQ), dtype=torch.float32, device="cuda") for c in chunks]

    def calls(kp, vp, work, o_list, l_list):
        for c, s, cu, sp, o, l in zip(chunks, starts, cus, sps, o_list, l_list):
            lo, hi = int(s), int(s) + c
            mtd.mtd_kv_append(kp, vp, k_log[lo:hi], v_log[lo:hi], cu, sp, bt)
            mtd.mtd_attn_prefill_chunk(kp, vp, q_log[lo:hi], lo, bt[0], W.SCALE, out=o, lse=l, workspace=work)

    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        calls(kg, vg, ws, outs, lses)
    torch.cuda.synchronize()
    log("prefill graph: eager twin")
    oe = [torch.empty_like(o) for o in outs]
    le = [torch.empty_like(l) for l in lses]
    calls(ke, ve, ws_e, oe, le)
    torch.cuda.synchronize()
    for rep in range(3):
        for o, l in zip(outs, lses):
            o.fill_(float("nan"))
            l.fill_(float("nan"))
        log(f"prefill graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for i in range(len(chunks)):
            assert torch.equal(outs[i], oe[i]) and torch.equal(lses[i], le[i]), (rep, i)
        assert torch.equal(kg.view(torch.int16), ke.view(torch.int16))
        assert torch.equal(vg.view(torch.int16), ve.view(torch.int16))
    c, s = chunks[-1], int(starts[-1])
    rows = np.unique(np.linspace(0, c - 1, 24).astype(np.int64))
    kc, vc, ident = request_pages_host(kg, vg, tables[0], total)
    k = oracle.gather_logical(kc, ident, total)
    v = oracle.gather_logical(vc, ident, total)
    o_ref, l_ref = oracle.attention(oracle.bf16_to_f64(bits(q_log[s:s + c])[rows]), k, v, s + rows, W.SCALE)
    compare(outs[-1][rows], lses[-1][rows], o_ref, l_ref, "prefill graph: last chunk")


def test_graph_batch_bucket_padding():
    """Decode batches padded to a bucket, one captured graph per bucket: the graph for 16 requests
    (4 layers of append + decode, max_kv_len bound 20,000) serves a batch of 12 and then a batch of
    9 other requests.  Padding requests append no token (their cu_new entries repeat) and decode
    zero keys (O = 0, LSE = -inf).  Every replay of the real requests equals the eager calls on
    exactly those requests bit for bit, with eager work between replays; the last step of each
    batch is also checked against the oracle."""
    bucket, layers, bound, tag = 16, 4, 20000, 77
    lens_a = W.loguniform_lengths(12, 500, 16000, tag, 1)
    lens_b = W.loguniform_lengths(9, 64, 9000, tag, 2)
    steps = 3
    tables, n_pages, _ = W.place_pages(np.concatenate([lens_a, lens_b]) + steps, tag, 3)
    stride = (bound + W.PAGE - 1) // W.PAGE
    tb = np.zeros((len(tables), stride), dtype=np.int32)
    tb[:, : tables.shape[1]] = tables
    kg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 40, l)) for l in range(layers)]
    vg = [new_pool(n_pages, "cuda", W.torch_seed(tag, 41, l)) for l in range(layers)]
    ke, ve = [p.clone() for p in kg], [p.clone() for p in vg]
    q_buf = torch.empty((layers, bucket, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    k_buf = torch.empty((layers, bucket, W.HKV, W.HEAD_DIM), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.empty_like(k_buf)
    cu_buf = torch.zeros(bucket + 1, dtype=torch.int32, device="cuda")
    start_buf = torch.zeros(bucket, dtype=torch.int32, device="cuda")
    len_buf = torch.zeros(bucket, dtype=torch.int32, device="cuda")
    bt_buf = torch.zeros((bucket, stride), dtype=torch.int32, device="cuda")
    o_buf = torch.empty((layers, bucket, W.HQ, W.HEAD_DIM), dtype=torch.float32, device="cuda")
    l_buf = torch.empty((layers, bucket, W.HQ), dtype=torch.float32, device="cuda")
    ws = torch.empty(mtd.decode_workspace_bytes(bucket, bound), dtype=torch.uint8, device="cuda")
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        for l in range(layers):
            mtd.mtd_kv_append(kg[l], vg[l], k_buf[l], v_buf[l], cu_buf, start_buf, bt_buf)
            mtd.mtd_attn_decode(kg[l], vg[l], q_buf[l], len_buf, bt_buf, bound, W.SCALE, ws, o_buf[l], l_buf[l])
    torch.cuda.synchronize()

    for name, rows, lens0 in (("batch of 12", np.arange(12), lens_a), ("batch of 9", 12 + np.arange(9), lens_b)):
        b = len(rows)
        bt_real = torch.as_tensor(tb[rows], device="cuda")
        cu_real = _i32(np.arange(b + 1))
        ws_e = torch.empty(mtd.decode_workspace_bytes(b, int(lens0.max()) + steps), dtype=torch.uint8,
                           device="cuda")
        for s in range(steps):
            log(f"bucket graph, {name}: step {s}")
            q = W.normal_bf16((layers, b, W.HQ, W.HEAD_DIM), W.torch_seed(tag, 50 + s, b), "cuda")
            kn = W.normal_bf16((layers, b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 60 + s, b), "cuda")
            vn = W.normal_bf16((layers, b, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 70 + s, b), "cuda")
            # stage the real requests into the bucket's buffers; the rest is padding
            q_buf.zero_()
            k_buf.zero_()
            v_buf.zero_()
            q_buf[:, :b] = q
            k_buf[:, :b] = kn
            v_buf[:, :b] = vn
            cu_buf.copy_(_i32(np.minimum(np.arange(bucket + 1), b)))
            start_buf.copy_(_i32(np.concatenate([lens0 + s, np.zeros(bucket - b)])))
            len_buf.copy_(_i32(np.concatenate([lens0 + s + 1, np.zeros(bucket - b)])))
            bt_buf.zero_()
            bt_buf[:b] = bt_real
            o_buf.fill_(float("nan"))
            l_buf.fill_(float("nan"))
            graph.replay()
            eager = []
            for l in range(layers):
                mtd.mtd_kv_append(ke[l], ve[l], kn[l], vn[l], cu_real, _i32(lens0 + s), bt_real)
                eager.append(mtd.mtd_attn_decode(ke[l], ve[l], q[l], _i32(lens0 + s + 1), bt_real,
                                                 int(lens0.max()) + steps, W.SCALE, ws_e))
            torch.cuda.synchronize()
            for l, (o, lse) in enumerate(eager):
                assert torch.equal(o_buf[l, :b], o) and torch.equal(l_buf[l, :b], lse), (name, s, l)
                assert torch.equal(o_buf[l, b:], torch.zeros_like(o_buf[l, b:])), (name, s, l)
                assert bool((l_buf[l, b:] == -float("inf")).all()), (name, s, l)
        for l in range(layers):
            assert torch.equal(kg[l], ke[l]) and torch.equal(vg[l], ve[l]), (name, l)
        qb = bits(q[0])
        o_ref, l_ref = [], []
        for i, r in enumerate(rows):
            n = int(lens0[i]) + steps
            kc, vc, ident = request_pages_host(kg[0], vg[0], tb[r], n)
            o, lse = oracle.decode(qb[i:i + 1], kc, vc, [n], [ident], W.SCALE)
            o_ref.append(o[0])
            l_ref.append(lse[0])
        compare(o_buf[0, :b], l_buf[0, :b], np.stack(o_ref), np.stack(l_ref), f"bucket graph, {name}, last step")
