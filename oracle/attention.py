"""fp64 CPU oracle for paged, causal, grouped-query attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The HIP library
and its Python binding never import or call it, and it shares no code, header,
table or helper with them.  It is plain numpy in float64, written so that a
reader can check it against the attention definition by eye.

What is computed, and where the pages say so
--------------------------------------------
* The text decoder is Qwen3 with 28 layers, hidden size 1024 and grouped-query
  attention with 16 query heads over 8 key/value heads
  ("Optimizing ASR Models to Transcribe 90-Minute Multi-Speaker Audio",
  §ASR Model Primer, component table; "MOSS-Transcribe-Diarize" cookbook,
  §Model Architecture table).  The README ("MOSS-Transcribe-Diarize 0.9B",
  §Model Architecture) calls it a Qwen3-0.6B style causal decoder.
* Prefill runs the whole prompt through the decoder to build the KV cache;
  for long audio the prompt is cut into 4096-token pieces, one per scheduler
  step, each piece attending to all keys before it plus itself causally
  ("Optimizing ASR Models ...", §ASR Model Primer and §Chunked Prefill for
  Long Audio; cookbook §Inference Pipeline).
* Autoregressive decode produces one token per request per step over that
  request's whole KV ("Optimizing ASR Models ...", §ASR Model Primer,
  "Autoregressive Decode"; cookbook §Inference Pipeline, step 3).

Paging, chunking and split-K are only ways of reaching the same numbers, so
the oracle is the textbook definition of causal softmax attention.  For query
row ``i`` at absolute position ``p_i`` of query head ``h`` (KV head
``g = h // (Hq // Hkv)``)::

    s_j  = scale * <q_i,h , k_j,g>          for j = 0 .. p_i (inclusive)
    LSE  = ln(sum_j exp(s_j))               natural log of the scaled logits
    O    = sum_j exp(s_j - LSE) * v_j,g

Readings where the pages are silent (each also listed in the design notes):
head_dim 128; the softmax scale 1/sqrt(head_dim); query head h reads KV head
h // (Hq/Hkv) (consecutive pairs share a KV head); chunk query i sits at
absolute position prefix + i (bottom-right causal alignment); decode sees the
token appended in the same step (its query sits at position kv_len - 1);
pages are laid out [page][kv_head][slot][dim] with K and V in separate pools;
outputs O and LSE are float64 here (float32 on the device).

Storage convention: bf16 tensors arrive as numpy ``uint16`` bit patterns so
the oracle reads exactly the bits the device consumed; the bf16 -> float64
conversion below is exact.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_to_f64",
    "page_of",
    "gather_logical",
    "attention",
    "prefill_chunk",
    "decode",
    "kv_append",
    "lse_merge",
]

# Query rows handled per matrix product; bounds the score block to
# QUERY_BLOCK x L doubles.  Pure memory bound, no effect on the result.
QUERY_BLOCK = 256


def bf16_to_f64(bits) -> np.ndarray:
    """Exact bf16 -> float64: a bf16 value is the top half of a float32."""
    b = np.asarray(bits)
    if b.dtype != np.uint16:
        b = b.astype(np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def page_of(pos, page_size: int):
    """Logical token ``pos`` of a request lives in table entry ``pos // page_size``,
    slot ``pos % page_size`` of that page."""
    pos = np.asarray(pos)
    return pos // page_size, pos % page_size


def gather_logical(pool, block_table, n_tokens: int) -> np.ndarray:
    """Page walk: logical rows 0 .. n_tokens-1 of one request, as float64.

    ``pool`` holds bf16 bits shaped [num_pages][Hkv][page_size][D];
    ``block_table`` lists the request's physical page ids in logical order.
    Returns [n_tokens][Hkv][D].
    """
    pool = np.asarray(pool)
    page_size = pool.shape[2]
    pos = np.arange(n_tokens)
    entry, slot = page_of(pos, page_size)
    pages = np.asarray(block_table, dtype=np.int64)[entry]
    # pool[pages[j], :, slot[j], :] for every j -> [n_tokens][Hkv][D]
    rows = pool[pages, :, slot, :]
    return bf16_to_f64(rows)


def attention(q, k, v, q_pos, scale: float):
    """Exact causal grouped-query attention in float64.

    q: [Nq][Hq][D]; k, v: [L][Hkv][D]; q_pos: [Nq] absolute positions (< L).
    Query row i of head h attends keys j <= q_pos[i] of KV head h // (Hq // Hkv).
    Returns (O [Nq][Hq][D], LSE [Nq][Hq]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n_q, n_qh, _ = q.shape
    n_kv, n_kvh, _ = k.shape
    if n_qh % n_kvh != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    if n_q and (q_pos.min() < 0 or q_pos.max() >= n_kv):
        raise ValueError("query position outside the key range")
    group = n_qh // n_kvh
    out = np.zeros((n_q, n_qh, v.shape[2]), dtype=np.float64)
    lse = np.zeros((n_q, n_qh), dtype=np.float64)
    key_idx = np.arange(n_kv)
    for h in range(n_qh):
        g = h // group
        for lo in range(0, n_q, QUERY_BLOCK):
            hi = min(lo + QUERY_BLOCK, n_q)
            pos = q_pos[lo:hi]
            n_keys = int(pos.max()) + 1           # keys beyond the last row are never attended
            s = scale * (q[lo:hi, h, :] @ k[:n_keys, g, :].T)
            s = np.where(key_idx[None, :n_keys] <= pos[:, None], s, -np.inf)
            m = s.max(axis=1, keepdims=True)      # finite: key 0 is always attended
            e = np.exp(s - m)
            denom = e.sum(axis=1, keepdims=True)
            lse[lo:hi, h] = m[:, 0] + np.log(denom[:, 0])
            out[lo:hi, h, :] = (e / denom) @ v[:n_keys, g, :]
    return out, lse


def prefill_chunk(q_bits, k_pool, v_pool, block_table, prefix_len: int, scale: float):
    """One prefill chunk over paged KV.

    q_bits: bf16 bits [C][Hq][D] for chunk positions prefix_len .. prefix_len+C-1.
    The chunk's own K/V must already sit in the pages (the caller appends first).
    Query i sits at absolute position prefix_len + i and sees keys 0 .. prefix_len + i.
    Returns (O [C][Hq][D], LSE [C][Hq]) in float64.
    """
    q = bf16_to_f64(q_bits)
    c = q.shape[0]
    total = prefix_len + c
    k = gather_logical(k_pool, block_table, total)
    v = gather_logical(v_pool, block_table, total)
    return attention(q, k, v, prefix_len + np.arange(c), scale)


def decode(q_bits, k_pool, v_pool, kv_lens, block_tables, scale: float):
    """Batched single-token decode over paged KV.

    q_bits: bf16 bits [B][Hq][D]; kv_lens[b] counts request b's tokens including
    the one appended this step, so its query sits at position kv_lens[b] - 1.
    Returns (O [B][Hq][D], LSE [B][Hq]) in float64.
    """
    q = bf16_to_f64(q_bits)
    n_b, n_qh, d = q.shape
    out = np.zeros((n_b, n_qh, d))
    lse = np.zeros((n_b, n_qh))
    for b in range(n_b):
        n = int(kv_lens[b])
        k = gather_logical(k_pool, block_tables[b], n)
        v = gather_logical(v_pool, block_tables[b], n)
        o_b, l_b = attention(q[b:b + 1], k, v, [n - 1], scale)
        out[b], lse[b] = o_b[0], l_b[0]
    return out, lse


def kv_append(k_pool, v_pool, k_new, v_new, cu_new, start_pos, block_tables):
    """Expected pools after writing new K/V rows into their page slots.

    Token t of request r (cu_new[r] <= t < cu_new[r+1]) has logical position
    start_pos[r] + (t - cu_new[r]) and is stored, for every KV head, at
    (block_tables[r][pos // page_size], head, pos % page_size).  Every other
    byte of the pools is unchanged.  Works on bit patterns, so the copy is exact.
    """
    k_out = np.array(k_pool, copy=True)
    v_out = np.array(v_pool, copy=True)
    page_size = k_out.shape[2]
    for r in range(len(start_pos)):
        for t in range(int(cu_new[r]), int(cu_new[r + 1])):
            pos = int(start_pos[r]) + (t - int(cu_new[r]))
            entry, slot = page_of(pos, page_size)
            page = int(block_tables[r][entry])
            k_out[page, :, slot, :] = k_new[t]
            v_out[page, :, slot, :] = v_new[t]
    return k_out, v_out


def lse_merge(o_parts, lse_parts):
    """Combine attention results over disjoint key sets.

    o_parts[s] / lse_parts[s] are attention output and LSE over key set s.  The
    union's LSE is the log-sum-exp of the parts; its output is the parts'
    outputs weighted by exp(lse_s - LSE).  Parts with LSE = -inf (no keys)
    carry zero weight.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)
    w = np.exp(lse_parts - m)
    total = w.sum(axis=0)
    lse = m + np.log(total)
    o = (w[..., None] * o_parts).sum(axis=0) / total[..., None]
    return o, lse
