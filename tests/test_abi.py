"""C-ABI library checks that need no GPU: the library loads, exports every declared symbol, binds
to the one HIP runtime torch loaded, and rejects every invalid host-side argument with the
documented status before anything is enqueued (so no kernel is ever launched here)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mtd.h")

mtd = pytest.importorskip("gqa_kv_cache_qwen3_amd")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mtd.LIB_PATH):
        pytest.skip("libmtd.so not built")
    return mtd.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtd_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("mtd_kv_append", "mtd_attn_prefill_chunk", "mtd_attn_prefill_workspace_bytes",
              "mtd_attn_decode", "mtd_attn_decode_workspace_bytes", "mtd_status_string",
              "mtd_last_error", "mtd_abi_version", "mtd_qkv_proj", "mtd_o_proj", "mtd_attn_merge"):
        assert n in names


def test_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in mtd.h but not exported"


def test_abi_version(lib):
    text = open(HEADER).read()
    want = int(re.search(r"#define MTD_ABI_VERSION (\d+)", text).group(1))
    assert lib.mtd_abi_version() == want


def test_single_hip_runtime(lib):
    maps = open("/proc/self/maps").read().splitlines()
    paths = {line.split()[-1] for line in maps if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        s = lib.mtd_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.mtd_status_string(7).decode() == "unknown status"


FAKE = 0x1000  # non-null placeholder; every call below fails validation before using it


def layer(**kw):
    base = dict(k_pages=FAKE, v_pages=FAKE, num_pages=10, page_size=64, num_kv_heads=8, head_dim=128)
    base.update(kw)
    return mtd.KvLayer(**base)


def append(lib, kv, **kw):
    a = dict(k_new=FAKE, v_new=FAKE, cu_new=FAKE, start_pos=FAKE, bt=FAKE, bt_stride=4, n_req=1, n_new=3)
    a.update(kw)
    return lib.mtd_kv_append(ctypes.byref(kv) if kv is not None else None, a["k_new"], a["v_new"],
                             a["cu_new"], a["start_pos"], a["bt"], a["bt_stride"], a["n_req"],
                             a["n_new"], None)


def prefill(lib, kv, **kw):
    a = dict(q=FAKE, chunk=10, prefix=0, bt=FAKE, bt_len=4, hq=16, scale=0.088, ws=None, ws_bytes=0,
             out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mtd_attn_prefill_chunk(ctypes.byref(kv) if kv is not None else None, a["q"],
                                      a["chunk"], a["prefix"], a["bt"], a["bt_len"], a["hq"],
                                      a["scale"], a["ws"], a["ws_bytes"], a["out"], a["lse"], None)


def decode(lib, kv, **kw):
    a = dict(q=FAKE, lens=FAKE, bt=FAKE, stride=16, batch=2, max_len=1000, hq=16, scale=0.088,
             ws=FAKE, ws_bytes=None, out=FAKE, lse=FAKE)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.mtd_attn_decode_workspace_bytes(max(a["batch"], 1), 16, max(min(a["max_len"], 131072), 1), 128)
    return lib.mtd_attn_decode(ctypes.byref(kv) if kv is not None else None, a["q"], a["lens"],
                               a["bt"], a["stride"], a["batch"], a["max_len"], a["hq"], a["scale"],
                               a["ws"], a["ws_bytes"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k_pages=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(v_pages=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(num_pages=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(page_size=32), mtd.MTD_ERR_UNSUPPORTED),
    (dict(num_kv_heads=4), mtd.MTD_ERR_UNSUPPORTED),
    (dict(head_dim=64), mtd.MTD_ERR_UNSUPPORTED),
])
def test_layer_validation(lib, kw, code):
    kv = layer(**kw)
    assert append(lib, kv) == code
    assert prefill(lib, kv) == code
    assert decode(lib, kv) == code
    assert lib.mtd_last_error().decode() != ""


MIS = FAKE + 4  # non-null, 4-byte aligned, not 16-byte aligned


def test_alignment_validation(lib):
    """Pools, token rows, O and workspaces must be 16-byte aligned (checked before any launch)."""
    for kw in (dict(k_pages=MIS), dict(v_pages=MIS)):
        kv = layer(**kw)
        assert append(lib, kv) == mtd.MTD_ERR_INVALID_ARG
        assert prefill(lib, kv) == mtd.MTD_ERR_INVALID_ARG
        assert decode(lib, kv) == mtd.MTD_ERR_INVALID_ARG
    for kw in (dict(k_new=MIS), dict(v_new=MIS)):
        assert append(lib, layer(), **kw) == mtd.MTD_ERR_INVALID_ARG
    ws = lib.mtd_attn_prefill_workspace_bytes(10, 16, 128)
    for kw in (dict(q=MIS), dict(out=MIS), dict(ws=MIS, ws_bytes=ws)):
        assert prefill(lib, layer(), **kw) == mtd.MTD_ERR_INVALID_ARG
    for kw in (dict(q=MIS), dict(out=MIS), dict(ws=MIS)):
        assert decode(lib, layer(), **kw) == mtd.MTD_ERR_INVALID_ARG
    assert "16-byte" in lib.mtd_last_error().decode()


def test_null_layer(lib):
    assert append(lib, None) == mtd.MTD_ERR_INVALID_ARG
    assert prefill(lib, None) == mtd.MTD_ERR_INVALID_ARG
    assert decode(lib, None) == mtd.MTD_ERR_INVALID_ARG


@pytest.mark.parametrize("kw,code", [
    (dict(n_req=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(n_new=-1), mtd.MTD_ERR_INVALID_ARG),
    (dict(bt_stride=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(k_new=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(v_new=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(cu_new=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(start_pos=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(bt=None), mtd.MTD_ERR_INVALID_ARG),
])
def test_append_validation(lib, kw, code):
    assert append(lib, layer(), **kw) == code


def test_append_empty_is_noop(lib):
    # n_new = 0 enqueues nothing (and needs no k_new / v_new)
    assert append(lib, layer(), n_new=0, k_new=None, v_new=None) == mtd.MTD_OK


@pytest.mark.parametrize("kw,code", [
    (dict(hq=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(hq=12), mtd.MTD_ERR_UNSUPPORTED),
    (dict(hq=32), mtd.MTD_ERR_UNSUPPORTED),
    (dict(scale=0.0), mtd.MTD_ERR_INVALID_ARG),
    (dict(scale=-1.0), mtd.MTD_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mtd.MTD_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mtd.MTD_ERR_INVALID_ARG),
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(bt=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lse=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(chunk=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(prefix=-1), mtd.MTD_ERR_INVALID_ARG),
    (dict(prefix=131072 - 9, chunk=10, bt_len=2048), mtd.MTD_ERR_CAPACITY),
    (dict(prefix=200, chunk=57, bt_len=4), mtd.MTD_ERR_CAPACITY),   # 257 tokens need 5 pages
    (dict(ws=FAKE, ws_bytes=0), mtd.MTD_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=10 * 16 * 129 * 4 - 1), mtd.MTD_ERR_WORKSPACE),
    (dict(ws=FAKE, ws_bytes=10 * 16 * 129 * 4, hq=12), mtd.MTD_ERR_UNSUPPORTED),
])
def test_prefill_validation(lib, kw, code):
    assert prefill(lib, layer(), **kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(hq=8), mtd.MTD_ERR_UNSUPPORTED),
    (dict(scale=float("nan")), mtd.MTD_ERR_INVALID_ARG),
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lens=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(bt=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lse=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(batch=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(max_len=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(max_len=131073, stride=4096), mtd.MTD_ERR_CAPACITY),
    (dict(max_len=1025, stride=16), mtd.MTD_ERR_CAPACITY),           # 1025 tokens need 17 pages
    (dict(ws=None), mtd.MTD_ERR_WORKSPACE),
    (dict(ws_bytes=100), mtd.MTD_ERR_WORKSPACE),
])
def test_decode_validation(lib, kw, code):
    assert decode(lib, layer(), **kw) == code


def decode_append(lib, kv, **kw):
    a = dict(q=FAKE, k_new=FAKE, v_new=FAKE, lens=FAKE, bt=FAKE, stride=16, batch=2, max_len=1000, hq=16,
             scale=0.088, ws=FAKE, ws_bytes=None, out=FAKE, lse=FAKE)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = lib.mtd_attn_decode_workspace_bytes(max(a["batch"], 1), 16, max(min(a["max_len"], 131072), 1), 128)
    return lib.mtd_attn_decode_append(ctypes.byref(kv) if kv is not None else None, a["q"], a["k_new"], a["v_new"],
                                      a["lens"], a["bt"], a["stride"], a["batch"], a["max_len"], a["hq"], a["scale"],
                                      a["ws"], a["ws_bytes"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k_new=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(v_new=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(k_new=FAKE + 8), mtd.MTD_ERR_INVALID_ARG),                 # not 16-byte aligned
    (dict(v_new=FAKE + 4), mtd.MTD_ERR_INVALID_ARG),
    (dict(hq=8), mtd.MTD_ERR_UNSUPPORTED),
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(batch=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(max_len=1025, stride=16), mtd.MTD_ERR_CAPACITY),
    (dict(ws=None), mtd.MTD_ERR_WORKSPACE),
])
def test_decode_append_validation(lib, kw, code):
    assert decode_append(lib, layer(), **kw) == code


def test_decode_append_checks_the_layer(lib):
    assert decode_append(lib, None) == mtd.MTD_ERR_INVALID_ARG
    assert decode_append(lib, layer(num_pages=0)) == mtd.MTD_ERR_INVALID_ARG


def test_prefill_workspace_size_formula(lib):
    # one part of every split item, partial O and LSE: chunk_len rows of 16 heads x (128 + 1) floats
    for c in (1, 2, 127, 128, 129, 4096, 131072):
        assert lib.mtd_attn_prefill_workspace_bytes(c, 16, 128) == c * 16 * 129 * 4
    assert lib.mtd_attn_prefill_workspace_bytes(0, 16, 128) == 0
    assert lib.mtd_attn_prefill_workspace_bytes(131073, 16, 128) == 0
    assert lib.mtd_attn_prefill_workspace_bytes(10, 8, 128) == 0
    assert lib.mtd_attn_prefill_workspace_bytes(10, 16, 64) == 0


def _split_tokens(n):
    # the documented partition: 64-token runs up to 1024 tokens, 128 up to 2048, 256 up to 4096,
    # else 512
    return 64 if n <= 1024 else 128 if n <= 2048 else 256 if n <= 4096 else 512


# most partials of any length 1..M, by brute force over every length
_RUNS = np.array([0] + [-(-n // _split_tokens(n)) for n in range(1, 131073)])
_MAX_RUNS = np.maximum.accumulate(_RUNS)


def test_workspace_size_formula(lib):
    # partials: batch * (most runs of any request of <= max_kv_len tokens), 16 heads x (128 + 1) floats
    for batch, max_len in [(1, 1), (1, 64), (1, 65), (1, 439), (1, 1024), (1, 1025), (1, 2048), (2, 2049),
                           (1, 4096), (1, 4097), (3, 6000), (1, 8192), (2, 8193), (1, 8705), (16, 30000),
                           (31, 68000), (64, 131072)]:
        parts = batch * int(_MAX_RUNS[max_len])
        assert lib.mtd_attn_decode_workspace_bytes(batch, 16, max_len, 128) == parts * 16 * 129 * 4, (batch, max_len)
    # every bound from 1 to 131072 tokens, at batch 1
    got = np.array([lib.mtd_attn_decode_workspace_bytes(1, 16, m, 128) for m in range(1, 131073, 7)])
    assert np.array_equal(got, _MAX_RUNS[1:131073:7] * 16 * 129 * 4)
    assert lib.mtd_attn_decode_workspace_bytes(0, 16, 100, 128) == 0
    assert lib.mtd_attn_decode_workspace_bytes(1, 16, 0, 128) == 0
    assert lib.mtd_attn_decode_workspace_bytes(1, 16, 131073, 128) == 0
    assert lib.mtd_attn_decode_workspace_bytes(1, 8, 100, 128) == 0


def test_binding_rejects_cpu_tensors():
    import torch
    cpu = torch.zeros((2, 8, 64, 128), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mtd.kv_layer(cpu, cpu)
    with pytest.raises(TypeError):
        mtd.kv_layer(cpu.float(), cpu.float())


def qkv(lib, **kw):
    a = dict(x=FAKE, w=FAKE, n_tok=5, hidden=1024, hq=16, hkv=8, d=128, q=FAKE, k=FAKE, v=FAKE)
    a.update(kw)
    return lib.mtd_qkv_proj(a["x"], a["w"], a["n_tok"], a["hidden"], a["hq"], a["hkv"], a["d"],
                            a["q"], a["k"], a["v"], None)


def oproj(lib, **kw):
    a = dict(attn=FAKE, w=FAKE, n_tok=5, hq=16, d=128, hidden=1024, out=FAKE)
    a.update(kw)
    return lib.mtd_o_proj(a["attn"], a["w"], a["n_tok"], a["hq"], a["d"], a["hidden"], a["out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_tok=-1), mtd.MTD_ERR_INVALID_ARG),
    (dict(hidden=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(hidden=2048), mtd.MTD_ERR_UNSUPPORTED),
    (dict(hq=32), mtd.MTD_ERR_UNSUPPORTED),
    (dict(d=64), mtd.MTD_ERR_UNSUPPORTED),
    (dict(x=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(w=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(k=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(v=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), mtd.MTD_ERR_INVALID_ARG),
    (dict(w=FAKE + 2), mtd.MTD_ERR_INVALID_ARG),
    (dict(v=FAKE + 4), mtd.MTD_ERR_INVALID_ARG),
])
def test_qkv_proj_validation(lib, kw, code):
    assert qkv(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def test_qkv_proj_kv_heads_checked(lib):
    assert qkv(lib, hkv=4) == mtd.MTD_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(n_tok=-3), mtd.MTD_ERR_INVALID_ARG),
    (dict(hidden=512), mtd.MTD_ERR_UNSUPPORTED),
    (dict(hq=8), mtd.MTD_ERR_UNSUPPORTED),
    (dict(d=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(attn=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(w=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(attn=FAKE + 4), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=FAKE + 2), mtd.MTD_ERR_INVALID_ARG),
])
def test_o_proj_validation(lib, kw, code):
    assert oproj(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def test_projections_of_no_tokens_enqueue_nothing(lib):
    """n_tok = 0 is valid and returns before any HIP call (so it runs without a GPU)."""
    assert qkv(lib, n_tok=0) == mtd.MTD_OK
    assert oproj(lib, n_tok=0) == mtd.MTD_OK


def merge(lib, **kw):
    a = dict(o=FAKE, l=FAKE, n_parts=3, n_rows=10, d=128, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mtd_attn_merge(a["o"], a["l"], a["n_parts"], a["n_rows"], a["d"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(n_parts=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(n_parts=mtd.MTD_MAX_MERGE_PARTS + 1), mtd.MTD_ERR_INVALID_ARG),
    (dict(n_rows=-1), mtd.MTD_ERR_INVALID_ARG),
    (dict(d=64), mtd.MTD_ERR_UNSUPPORTED),
    (dict(o=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(l=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lse=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(o=FAKE + 4), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=FAKE + 8), mtd.MTD_ERR_INVALID_ARG),
])
def test_merge_validation(lib, kw, code):
    assert merge(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def prefill_cus(lib, kv=None, **kw):
    a = dict(q=FAKE, chunk=10, prefix=0, bt=FAKE, bt_len=4, hq=16, scale=0.088, ws=FAKE, ws_bytes=1 << 30,
             cus=64, out=FAKE, lse=FAKE)
    a.update(kw)
    return lib.mtd_attn_prefill_chunk_cus(ctypes.byref(kv or layer()), a["q"], a["chunk"], a["prefix"], a["bt"],
                                          a["bt_len"], a["hq"], a["scale"], a["ws"], a["ws_bytes"], a["cus"],
                                          a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(cus=-1), mtd.MTD_ERR_INVALID_ARG),
    (dict(ws=None, ws_bytes=0), mtd.MTD_ERR_WORKSPACE),            # a budget needs the workspace
    (dict(ws_bytes=100), mtd.MTD_ERR_WORKSPACE),
    (dict(chunk=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(prefix=131072), mtd.MTD_ERR_CAPACITY),
    (dict(bt_len=0), mtd.MTD_ERR_CAPACITY),
    (dict(hq=8), mtd.MTD_ERR_UNSUPPORTED),
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
])
def test_prefill_cus_validation(lib, kw, code):
    assert prefill_cus(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def decode_noalloc(lib, kv=None, **kw):
    a = dict(q=FAKE, lens=FAKE, bt=FAKE, stride=2048, batch=2, max_len=1000, hq=16, scale=0.088, out=FAKE,
             lse=FAKE)
    a.update(kw)
    return lib.mtd_attn_decode_noalloc(ctypes.byref(kv or layer()), a["q"], a["lens"], a["bt"], a["stride"],
                                       a["batch"], a["max_len"], a["hq"], a["scale"], a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lens=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(bt=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(lse=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(out=FAKE + 4), mtd.MTD_ERR_INVALID_ARG),
    (dict(batch=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(max_len=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(max_len=131073), mtd.MTD_ERR_CAPACITY),
    (dict(stride=15), mtd.MTD_ERR_CAPACITY),
    (dict(hq=8), mtd.MTD_ERR_UNSUPPORTED),
    (dict(scale=0.0), mtd.MTD_ERR_INVALID_ARG),
    # 33 requests at the 128K cap need more partials than the static scratch holds
    (dict(batch=33, max_len=131072), mtd.MTD_ERR_WORKSPACE),
])
def test_decode_noalloc_validation(lib, kw, code):
    assert decode_noalloc(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def test_decode_noalloc_scratch_limit_matches_the_header(lib):
    text = open(HEADER).read()
    assert "#define MTD_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    assert mtd.MTD_DECODE_NOALLOC_SCRATCH_BYTES == 64 << 20
    # the largest batch at the cap that fits: 31 requests (7936 partials); 32 do not (8192 > 8128)
    assert lib.mtd_attn_decode_workspace_bytes(31, 16, 131072, 128) <= mtd.MTD_DECODE_NOALLOC_SCRATCH_BYTES
    assert lib.mtd_attn_decode_workspace_bytes(32, 16, 131072, 128) > mtd.MTD_DECODE_NOALLOC_SCRATCH_BYTES


def page_read(lib, kv=None, **kw):
    a = dict(ids=FAKE, n=100, ppw=8, sink=FAKE, words=None)
    a.update(kw)
    words = a["words"] if a["words"] is not None else lib.mtd_measure_page_read_sink_words(a["n"], a["ppw"])
    return lib.mtd_measure_page_read(ctypes.byref(kv or layer()), a["ids"], a["n"], a["ppw"], a["sink"], words, None)


@pytest.mark.parametrize("kw,code", [
    (dict(n=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(ppw=0), mtd.MTD_ERR_INVALID_ARG),
    (dict(ppw=65), mtd.MTD_ERR_INVALID_ARG),
    (dict(ids=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(sink=None), mtd.MTD_ERR_INVALID_ARG),
    (dict(words=13 * 8 * 64 - 1), mtd.MTD_ERR_WORKSPACE),
])
def test_page_read_validation(lib, kw, code):
    assert page_read(lib, **kw) == code
    assert lib.mtd_last_error().decode() != ""


def test_page_read_sink_words(lib):
    assert lib.mtd_measure_page_read_sink_words(100, 8) == 13 * 8 * 64
    assert lib.mtd_measure_page_read_sink_words(0, 8) == 0
    assert lib.mtd_measure_page_read_sink_words(10, 0) == 0


def test_page_read_checks_the_layer(lib):
    assert page_read(lib, kv=layer(head_dim=64)) == mtd.MTD_ERR_UNSUPPORTED


def test_merge_of_no_rows_enqueues_nothing(lib):
    assert merge(lib, n_rows=0) == mtd.MTD_OK
    assert merge(lib, n_rows=0, n_parts=mtd.MTD_MAX_MERGE_PARTS) == mtd.MTD_OK
