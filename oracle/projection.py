"""fp64 CPU oracle for the attention block's input and output projections.

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import
it, and it shares no code with the HIP library.

What is computed, and where the pages say so
--------------------------------------------
The text decoder is Qwen3 with 28 layers, hidden size 1024 and grouped-query
attention with 16 query heads over 8 key/value heads ("Optimizing ASR Models
to Transcribe 90-Minute Multi-Speaker Audio", §ASR Model Primer, component
table; "MOSS-Transcribe-Diarize" cookbook, §Model Architecture table).  Around
the attention of each layer sit the linear maps that make its inputs and
consume its output.  The pages give their sizes only through those numbers;
the plainest reading, taken here:

* QKV projection: for token t with hidden state x_t (1024 values),
  q_t = Wq x_t (16 heads x 128 = 2048 values), k_t = Wk x_t and v_t = Wv x_t
  (8 heads x 128 = 1024 values each), no bias.  The three weight matrices are
  stacked row-wise into one [4096][1024] matrix W_qkv = [Wq; Wk; Wv] in the
  usual [out][in] layout, so row n of W_qkv makes output feature n, and output
  feature f of each part is (head f // 128, dim f % 128).
* Output projection: y_t = Wo o_t, Wo [1024][2048], o_t the 16 heads' attention
  outputs concatenated head-major (feature h*128 + d), no bias.

Readings where the pages are silent (each also listed in the design notes):
no biases; the per-head q/k normalisation and rotary embedding Qwen3 applies
between the projection and attention are not part of these maps; the model
carries activations in bf16, so the attention output (float32 from the
attention kernels) is rounded to bf16, to nearest with ties to even, before the
output projection, and the projections' own results are returned here in
float64 (the device rounds them to bf16).

bf16 tensors arrive as numpy ``uint16`` bit patterns, as in ``attention.py``.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_to_f64

__all__ = ["round_to_bf16_bits", "linear", "qkv_proj", "o_proj"]

NUM_Q_HEADS = 16
NUM_KV_HEADS = 8
HEAD_DIM = 128


def round_to_bf16_bits(x_f32) -> np.ndarray:
    """float32 values -> bf16 bit patterns, rounding to nearest, ties to even.

    A bf16 value keeps the upper 16 bits of a float32.  Adding 0x7FFF plus the
    lowest kept bit to the 32-bit pattern carries into the kept half exactly
    when the dropped half is above one half, or equal to it with an odd kept
    half; the carry also walks up into the exponent where the mantissa
    overflows, and reaches infinity only from above the largest bf16.  NaNs
    are kept quiet NaNs of the same sign.
    """
    x = np.ascontiguousarray(np.asarray(x_f32, dtype=np.float32))
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    quiet = ((bits >> np.uint64(16)).astype(np.uint16)) | np.uint16(0x0040)
    return np.where(nan, quiet, rounded).astype(np.uint16)


def linear(x, w_bits) -> np.ndarray:
    """y[t][n] = sum_i W[n][i] x[t][i] in float64.

    x: float64 values [T][K] (already exact bf16 values); w_bits: bf16 bits
    [N][K] in the [out][in] layout.  Returns float64 [T][N].
    """
    x = np.asarray(x, dtype=np.float64)
    w = bf16_to_f64(w_bits)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[1]:
        raise ValueError(f"shapes {x.shape} and {w.shape} do not chain")
    return x @ w.T


def qkv_proj(x_bits, w_qkv_bits):
    """The QKV projection of T tokens.

    x_bits: bf16 bits [T][hidden]; w_qkv_bits: bf16 bits
    [(16 + 8 + 8) * 128][hidden], rows Wq then Wk then Wv.
    Returns float64 q [T][16][128], k [T][8][128], v [T][8][128].
    """
    x = bf16_to_f64(x_bits)
    n_q = NUM_Q_HEADS * HEAD_DIM
    n_kv = NUM_KV_HEADS * HEAD_DIM
    if np.asarray(w_qkv_bits).shape[0] != n_q + 2 * n_kv:
        raise ValueError("W_qkv must have (16 + 8 + 8) * 128 rows")
    y = linear(x, w_qkv_bits)
    t = x.shape[0]
    q = y[:, :n_q].reshape(t, NUM_Q_HEADS, HEAD_DIM)
    k = y[:, n_q:n_q + n_kv].reshape(t, NUM_KV_HEADS, HEAD_DIM)
    v = y[:, n_q + n_kv:].reshape(t, NUM_KV_HEADS, HEAD_DIM)
    return q, k, v


def o_proj(attn_f32, w_o_bits) -> np.ndarray:
    """The output projection of T tokens' attention outputs.

    attn_f32: float32 [T][16][128] (the attention kernels' O); w_o_bits: bf16
    bits [hidden][16 * 128].  O is rounded to bf16 first (the model's
    activation type), then y = Wo o in float64.  Returns float64 [T][hidden].
    """
    o = np.asarray(attn_f32, dtype=np.float32)
    t = o.shape[0]
    o_bf16 = bf16_to_f64(round_to_bf16_bits(o.reshape(t, -1)))
    return linear(o_bf16, w_o_bits)
