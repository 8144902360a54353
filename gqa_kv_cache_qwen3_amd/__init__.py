"""Python binding of libmtd: paged causal GQA attention kernels for MI355X (gfx950).

Argument marshalling only: every function checks dtypes, devices, shapes and contiguity of torch
tensors, then passes raw device pointers and the current HIP stream to the C-ABI library
(include/mtd.h).  All arithmetic runs in the library's HIP kernels; there is no fallback.  The
library must be built first (``python -m gqa_kv_cache_qwen3_amd.build``); importing a function
without it raises.

Names match the C entry points:
    mtd_kv_append(k_pages, v_pages, k_new, v_new, cu_new, start_pos, block_tables)
    mtd_attn_prefill_chunk(k_pages, v_pages, q, prefix_len, block_table, scale, out=None, lse=None,
                           workspace=None)
    mtd_attn_prefill_chunk_cus(k_pages, v_pages, q, prefix_len, block_table, scale, workspace, cu_budget,
                               out=None, lse=None)
    mtd_attn_decode(k_pages, v_pages, q, kv_lens, block_tables, max_kv_len, scale,
                    workspace=None, out=None, lse=None)
    mtd_qkv_proj(x, w_qkv, q=None, k_new=None, v_new=None)
    mtd_o_proj(attn, w_o, out=None)
    mtd_attn_merge(o_parts, lse_parts, out=None, lse=None)
    mtd_attn_decode_noalloc(k_pages, v_pages, q, kv_lens, block_tables, max_kv_len, scale, out, lse)
    mtd_attn_decode_append(k_pages, v_pages, q, k_new, v_new, kv_lens, block_tables, max_kv_len, scale,
                           workspace=None, out=None, lse=None)
    mtd_measure_page_read(k_pages, v_pages, page_ids, pages_per_wave=8, sink=None)   (measurement aid)
"""

from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libmtd binds to (one runtime per process)

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libmtd.so")

MTD_OK = 0
MTD_ERR_INVALID_ARG = -1
MTD_ERR_UNSUPPORTED = -2
MTD_ERR_CAPACITY = -3
MTD_ERR_WORKSPACE = -4
MTD_ERR_HIP = -5
MTD_MAX_CONTEXT = 131072
MTD_MAX_MERGE_PARTS = 1024
MTD_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20

NUM_Q_HEADS = 16
NUM_KV_HEADS = 8
HEAD_DIM = 128
PAGE_SIZE = 64
HIDDEN = 1024


class MtdError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"libmtd status {status}: {detail}")
        self.status = status
        self.detail = detail


class KvLayer(ctypes.Structure):
    """mtd_kv_layer_t"""
    _fields_ = [
        ("k_pages", ctypes.c_void_p),
        ("v_pages", ctypes.c_void_p),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
    ]


_LIB = None
_P = ctypes.c_void_p
_I = ctypes.c_int32


def lib() -> ctypes.CDLL:
    """The loaded libmtd (raises if it was never built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m gqa_kv_cache_qwen3_amd.build`")
        cdll = ctypes.CDLL(LIB_PATH)
        kvp = ctypes.POINTER(KvLayer)
        cdll.mtd_kv_append.argtypes = [kvp, _P, _P, _P, _P, _P, _I, _I, _I, _P]
        cdll.mtd_kv_append.restype = ctypes.c_int
        cdll.mtd_attn_prefill_chunk.argtypes = [kvp, _P, _I, _I, _P, _I, _I, ctypes.c_float, _P,
                                                ctypes.c_size_t, _P, _P, _P]
        cdll.mtd_attn_prefill_chunk.restype = ctypes.c_int
        cdll.mtd_attn_prefill_workspace_bytes.argtypes = [_I, _I, _I]
        cdll.mtd_attn_prefill_workspace_bytes.restype = ctypes.c_size_t
        cdll.mtd_attn_decode_workspace_bytes.argtypes = [_I, _I, _I, _I]
        cdll.mtd_attn_decode_workspace_bytes.restype = ctypes.c_size_t
        cdll.mtd_attn_decode.argtypes = [kvp, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P,
                                         ctypes.c_size_t, _P, _P, _P]
        cdll.mtd_attn_decode.restype = ctypes.c_int
        cdll.mtd_attn_decode_append.argtypes = [kvp, _P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P,
                                                ctypes.c_size_t, _P, _P, _P]
        cdll.mtd_attn_decode_append.restype = ctypes.c_int
        cdll.mtd_qkv_proj.argtypes = [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]
        cdll.mtd_qkv_proj.restype = ctypes.c_int
        cdll.mtd_o_proj.argtypes = [_P, _P, _I, _I, _I, _I, _P, _P]
        cdll.mtd_o_proj.restype = ctypes.c_int
        cdll.mtd_attn_merge.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
        cdll.mtd_attn_merge.restype = ctypes.c_int
        cdll.mtd_attn_prefill_chunk_cus.argtypes = [kvp, _P, _I, _I, _P, _I, _I, ctypes.c_float, _P,
                                                    ctypes.c_size_t, _I, _P, _P, _P]
        cdll.mtd_attn_prefill_chunk_cus.restype = ctypes.c_int
        cdll.mtd_attn_decode_noalloc.argtypes = [kvp, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _P, _P, _P]
        cdll.mtd_attn_decode_noalloc.restype = ctypes.c_int
        cdll.mtd_measure_page_read.argtypes = [kvp, _P, _I, _I, _P, ctypes.c_size_t, _P]
        cdll.mtd_measure_page_read.restype = ctypes.c_int
        cdll.mtd_measure_page_read_sink_words.argtypes = [_I, _I]
        cdll.mtd_measure_page_read_sink_words.restype = ctypes.c_size_t
        cdll.mtd_status_string.argtypes = [ctypes.c_int]
        cdll.mtd_status_string.restype = ctypes.c_char_p
        cdll.mtd_last_error.argtypes = []
        cdll.mtd_last_error.restype = ctypes.c_char_p
        cdll.mtd_abi_version.argtypes = []
        cdll.mtd_abi_version.restype = ctypes.c_int
        _LIB = cdll
    return _LIB


def _check(status: int) -> None:
    if status != MTD_OK:
        detail = lib().mtd_last_error().decode()
        raise MtdError(status, f"{lib().mtd_status_string(status).decode()}: {detail}")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")


def kv_layer(k_pages: torch.Tensor, v_pages: torch.Tensor) -> KvLayer:
    """Describe one layer's pools: bf16 [num_pages][num_kv_heads][page_size][head_dim]."""
    _need(k_pages, "k_pages", torch.bfloat16, 4)
    _need(v_pages, "v_pages", torch.bfloat16, 4)
    if k_pages.shape != v_pages.shape:
        raise ValueError("k_pages and v_pages differ in shape")
    if k_pages.device != v_pages.device:
        raise ValueError("k_pages and v_pages are on different devices")
    n, hkv, ps, d = k_pages.shape
    return KvLayer(k_pages.data_ptr(), v_pages.data_ptr(), n, ps, hkv, d)


def mtd_kv_append(k_pages, v_pages, k_new, v_new, cu_new, start_pos, block_tables) -> None:
    """Write new K/V rows ([n_new][Hkv][D] bf16) into their pages; see include/mtd.h."""
    layer = kv_layer(k_pages, v_pages)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(cu_new, "cu_new", torch.int32, 1)
    _need(start_pos, "start_pos", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    if k_new.shape != v_new.shape or tuple(k_new.shape[1:]) != (layer.num_kv_heads, layer.head_dim):
        raise ValueError(f"k_new/v_new must be [n_new][{layer.num_kv_heads}][{layer.head_dim}]")
    n_req = start_pos.shape[0]
    if cu_new.shape[0] != n_req + 1 or block_tables.shape[0] != n_req:
        raise ValueError("cu_new must have n_req + 1 entries and block_tables n_req rows")
    _check(lib().mtd_kv_append(ctypes.byref(layer), k_new.data_ptr(), v_new.data_ptr(),
                               cu_new.data_ptr(), start_pos.data_ptr(), block_tables.data_ptr(),
                               block_tables.shape[1], n_req, k_new.shape[0], _stream()))


def prefill_workspace_bytes(chunk_len: int, num_q_heads: int = NUM_Q_HEADS, head_dim: int = HEAD_DIM) -> int:
    return int(lib().mtd_attn_prefill_workspace_bytes(chunk_len, num_q_heads, head_dim))


def mtd_attn_prefill_chunk(k_pages, v_pages, q, prefix_len: int, block_table, scale: float,
                           out=None, lse=None, workspace=None):
    """Causal attention of a chunk q ([C][Hq][D] bf16) at prefix_len over the pages.

    workspace: None (one pass per position tile) or a uint8 device tensor of at least
    prefill_workspace_bytes(C) bytes (causal work rebalanced over the CUs, split items merged).
    Returns (out float32 [C][Hq][D], lse float32 [C][Hq]).
    """
    layer = kv_layer(k_pages, v_pages)
    _need(q, "q", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 1)
    c, hq, d = q.shape
    if out is None:
        out = torch.empty((c, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((c, hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (c, hq, d) or tuple(lse.shape) != (c, hq):
        raise ValueError("out must be [C][Hq][D] and lse [C][Hq]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().mtd_attn_prefill_chunk(ctypes.byref(layer), q.data_ptr(), c, int(prefix_len),
                                        block_table.data_ptr(), block_table.shape[0], hq,
                                        float(scale), ws_ptr, ws_bytes, out.data_ptr(),
                                        lse.data_ptr(), _stream()))
    return out, lse


def mtd_attn_prefill_chunk_cus(k_pages, v_pages, q, prefix_len: int, block_table, scale: float, workspace,
                               cu_budget: int, out=None, lse=None):
    """mtd_attn_prefill_chunk on a budget of cu_budget compute units (0 = all; > 0 needs the
    workspace), leaving the device's other CUs free for work on another stream."""
    layer = kv_layer(k_pages, v_pages)
    _need(q, "q", torch.bfloat16, 3)
    _need(block_table, "block_table", torch.int32, 1)
    c, hq, d = q.shape
    if out is None:
        out = torch.empty((c, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((c, hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (c, hq, d) or tuple(lse.shape) != (c, hq):
        raise ValueError("out must be [C][Hq][D] and lse [C][Hq]")
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel()
    _check(lib().mtd_attn_prefill_chunk_cus(ctypes.byref(layer), q.data_ptr(), c, int(prefix_len),
                                            block_table.data_ptr(), block_table.shape[0], hq, float(scale),
                                            ws_ptr, ws_bytes, int(cu_budget), out.data_ptr(), lse.data_ptr(),
                                            _stream()))
    return out, lse


def decode_workspace_bytes(batch: int, max_kv_len: int, num_q_heads: int = NUM_Q_HEADS,
                           head_dim: int = HEAD_DIM) -> int:
    return int(lib().mtd_attn_decode_workspace_bytes(batch, num_q_heads, max_kv_len, head_dim))


def mtd_attn_decode(k_pages, v_pages, q, kv_lens, block_tables, max_kv_len: int, scale: float,
                    workspace=None, out=None, lse=None):
    """One query token per request ([B][Hq][D] bf16) over each request's kv_lens[b] keys.

    Returns (out float32 [B][Hq][D], lse float32 [B][Hq]).
    """
    layer = kv_layer(k_pages, v_pages)
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    b, hq, d = q.shape
    if kv_lens.shape[0] != b or block_tables.shape[0] != b:
        raise ValueError("kv_lens and block_tables must have one entry/row per request")
    need = decode_workspace_bytes(b, int(max_kv_len), hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (b, hq, d) or tuple(lse.shape) != (b, hq):
        raise ValueError("out must be [B][Hq][D] and lse [B][Hq]")
    _check(lib().mtd_attn_decode(ctypes.byref(layer), q.data_ptr(), kv_lens.data_ptr(),
                                 block_tables.data_ptr(), block_tables.shape[1], b,
                                 int(max_kv_len), hq, float(scale), workspace.data_ptr(),
                                 workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream()))
    return out, lse


def mtd_attn_decode_append(k_pages, v_pages, q, k_new, v_new, kv_lens, block_tables, max_kv_len: int,
                           scale: float, workspace=None, out=None, lse=None):
    """One decode step: store each request's new K/V row ([B][Hkv][D] bf16) at position kv_lens[b] - 1,
    then attend as mtd_attn_decode.  Returns (out float32 [B][Hq][D], lse float32 [B][Hq])."""
    layer = kv_layer(k_pages, v_pages)
    _need(q, "q", torch.bfloat16, 3)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    b, hq, d = q.shape
    if kv_lens.shape[0] != b or block_tables.shape[0] != b:
        raise ValueError("kv_lens and block_tables must have one entry/row per request")
    if k_new.shape != v_new.shape or tuple(k_new.shape) != (b, layer.num_kv_heads, layer.head_dim):
        raise ValueError(f"k_new/v_new must be [{b}][{layer.num_kv_heads}][{layer.head_dim}]")
    need = decode_workspace_bytes(b, int(max_kv_len), hq, d)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8, 1)
    if out is None:
        out = torch.empty((b, hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    if tuple(out.shape) != (b, hq, d) or tuple(lse.shape) != (b, hq):
        raise ValueError("out must be [B][Hq][D] and lse [B][Hq]")
    _check(lib().mtd_attn_decode_append(ctypes.byref(layer), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                        kv_lens.data_ptr(), block_tables.data_ptr(), block_tables.shape[1], b,
                                        int(max_kv_len), hq, float(scale), workspace.data_ptr(),
                                        workspace.numel(), out.data_ptr(), lse.data_ptr(), _stream()))
    return out, lse


def mtd_measure_page_read(k_pages, v_pages, page_ids, pages_per_wave: int = 8, sink=None):
    """Measurement aid: read the K/V blocks of page_ids (int32 [n] on the device) with the decode's
    access pattern and nothing else.  Returns the sink (uint8 view of the folded words)."""
    layer = kv_layer(k_pages, v_pages)
    _need(page_ids, "page_ids", torch.int32, 1)
    words = int(lib().mtd_measure_page_read_sink_words(page_ids.shape[0], pages_per_wave))
    if sink is None:
        sink = torch.empty(max(4 * words, 4), dtype=torch.uint8, device=page_ids.device)
    _need(sink, "sink", torch.uint8, 1)
    _check(lib().mtd_measure_page_read(ctypes.byref(layer), page_ids.data_ptr(), page_ids.shape[0],
                                       int(pages_per_wave), sink.data_ptr(), sink.numel() // 4, _stream()))
    return sink


def mtd_attn_decode_noalloc(k_pages, v_pages, q, kv_lens, block_tables, max_kv_len: int, scale: float,
                            out, lse):
    """mtd_attn_decode with the library's static scratch instead of a workspace: allocates nothing,
    so out (float32 [B][Hq][D]) and lse (float32 [B][Hq]) must be given."""
    layer = kv_layer(k_pages, v_pages)
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_lens, "kv_lens", torch.int32, 1)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(out, "out", torch.float32, 3)
    _need(lse, "lse", torch.float32, 2)
    b, hq, d = q.shape
    if kv_lens.shape[0] != b or block_tables.shape[0] != b:
        raise ValueError("kv_lens and block_tables must have one entry/row per request")
    if tuple(out.shape) != (b, hq, d) or tuple(lse.shape) != (b, hq):
        raise ValueError("out must be [B][Hq][D] and lse [B][Hq]")
    _check(lib().mtd_attn_decode_noalloc(ctypes.byref(layer), q.data_ptr(), kv_lens.data_ptr(),
                                         block_tables.data_ptr(), block_tables.shape[1], b, int(max_kv_len),
                                         hq, float(scale), out.data_ptr(), lse.data_ptr(), _stream()))
    return out, lse


def _out(t, name, shape, dtype, like):
    if t is None:
        t = torch.empty(shape, dtype=dtype, device=like.device)
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be {list(shape)}, got {tuple(t.shape)}")
    return t


def mtd_qkv_proj(x, w_qkv, q=None, k_new=None, v_new=None):
    """q, k, v of n_tok tokens from their hidden states x (bf16 [n_tok][1024]) and the stacked
    weights w_qkv (bf16 [(16 + 8 + 8) * 128][1024], rows Wq, Wk, Wv).

    Returns (q bf16 [n_tok][16][128], k_new bf16 [n_tok][8][128], v_new bf16 [n_tok][8][128]).
    """
    _need(x, "x", torch.bfloat16, 2)
    _need(w_qkv, "w_qkv", torch.bfloat16, 2)
    n_tok, hidden = x.shape
    n_feat = (NUM_Q_HEADS + 2 * NUM_KV_HEADS) * HEAD_DIM
    if tuple(w_qkv.shape) != (n_feat, hidden):
        raise ValueError(f"w_qkv must be [{n_feat}][{hidden}], got {tuple(w_qkv.shape)}")
    q = _out(q, "q", (n_tok, NUM_Q_HEADS, HEAD_DIM), torch.bfloat16, x)
    k_new = _out(k_new, "k_new", (n_tok, NUM_KV_HEADS, HEAD_DIM), torch.bfloat16, x)
    v_new = _out(v_new, "v_new", (n_tok, NUM_KV_HEADS, HEAD_DIM), torch.bfloat16, x)
    _check(lib().mtd_qkv_proj(x.data_ptr(), w_qkv.data_ptr(), n_tok, hidden, NUM_Q_HEADS,
                              NUM_KV_HEADS, HEAD_DIM, q.data_ptr(), k_new.data_ptr(),
                              v_new.data_ptr(), _stream()))
    return q, k_new, v_new


def mtd_o_proj(attn, w_o, out=None):
    """Hidden states from the attention output attn (float32 [n_tok][16][128], rounded to bf16
    on the way in) and w_o (bf16 [1024][16 * 128]).  Returns out bf16 [n_tok][1024]."""
    _need(attn, "attn", torch.float32, 3)
    _need(w_o, "w_o", torch.bfloat16, 2)
    n_tok, hq, d = attn.shape
    hidden = w_o.shape[0]
    if w_o.shape[1] != hq * d:
        raise ValueError(f"w_o must be [hidden][{hq * d}], got {tuple(w_o.shape)}")
    out = _out(out, "out", (n_tok, hidden), torch.bfloat16, attn)
    _check(lib().mtd_o_proj(attn.data_ptr(), w_o.data_ptr(), n_tok, hq, d, hidden, out.data_ptr(),
                            _stream()))
    return out


def mtd_attn_merge(o_parts, lse_parts, out=None, lse=None):
    """Combine attention results over disjoint key sets: o_parts float32 [S][..., D] and
    lse_parts float32 [S][...] (natural log; -inf = no keys) -> (out [..., D], lse [...])."""
    _need(o_parts, "o_parts", torch.float32)
    _need(lse_parts, "lse_parts", torch.float32)
    if o_parts.dim() < 2 or tuple(o_parts.shape[:-1]) != tuple(lse_parts.shape):
        raise ValueError("o_parts must be [S][..., D] with lse_parts [S][...]")
    n_parts, d = o_parts.shape[0], o_parts.shape[-1]
    rows_shape = tuple(lse_parts.shape[1:])
    n_rows = lse_parts[0].numel() if n_parts else 0
    out = _out(out, "out", rows_shape + (d,), torch.float32, o_parts)
    lse = _out(lse, "lse", rows_shape, torch.float32, o_parts)
    _check(lib().mtd_attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), n_parts, n_rows, d,
                                out.data_ptr(), lse.data_ptr(), _stream()))
    return out, lse


__all__ = [
    "MtdError", "KvLayer", "lib", "kv_layer", "mtd_kv_append", "mtd_attn_prefill_chunk",
    "mtd_attn_decode", "decode_workspace_bytes", "prefill_workspace_bytes", "mtd_qkv_proj",
    "mtd_o_proj", "mtd_attn_merge",
]
