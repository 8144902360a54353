"""Shared setup for the GPU parity tests: seeded pools, poisoning of unused slots, host copies of
one request's pages for the oracle, and the comparison gate.

The expected values always come from ``oracle`` (float64, CPU) applied to the exact bf16 bits the
device consumed; nothing here computes attention.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import workloads as W

NAN_BF16 = 0x7FC0          # quiet NaN as bf16 bits: poison for slots no request owns
O_TOL = 1e-2               # max |O_gpu - O_ref|
LSE_TOL = 1e-3             # max |LSE_gpu - LSE_ref|


def log(msg: str) -> None:
    """Name the case on stdout before each GPU step (flushed, so a crash still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> numpy uint16 bit patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def fill_normal_(t: torch.Tensor, seed: int, slab: int = 1 << 28) -> torch.Tensor:
    """Fill a bf16 tensor with N(0,1) values (fp32 draws, RNE cast), in slabs to bound temporaries."""
    gen = torch.Generator(device=t.device)
    gen.manual_seed(seed)
    flat = t.view(-1)
    for lo in range(0, flat.numel(), slab):
        hi = min(lo + slab, flat.numel())
        flat[lo:hi] = torch.randn(hi - lo, generator=gen, device=t.device, dtype=torch.float32).to(torch.bfloat16)
    return t


def new_pool(num_pages: int, device, seed: int | None = None) -> torch.Tensor:
    pool = torch.empty((num_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=device)
    if seed is None:
        pool.view(torch.int16).fill_(NAN_BF16)
    else:
        fill_normal_(pool, seed)
    return pool


def poison_unused(pool: torch.Tensor, tables: np.ndarray, lens, spare_ids) -> None:
    """NaN every slot that holds no token: the tail of each request's last page and spare pages."""
    as_int = pool.view(torch.int16)
    for b, n in enumerate(lens):
        n = int(n)
        used = (n + W.PAGE - 1) // W.PAGE
        tail = n - (used - 1) * W.PAGE
        if tail < W.PAGE:
            as_int[int(tables[b][used - 1]), :, tail:, :] = NAN_BF16
    for s in spare_ids:
        as_int[int(s)] = NAN_BF16


def request_pages_host(k_pool: torch.Tensor, v_pool: torch.Tensor, table_row, n_tokens: int):
    """Copy the pages one request uses to the host; returns (k_bits, v_bits, identity table)."""
    used = (n_tokens + W.PAGE - 1) // W.PAGE
    idx = torch.as_tensor(np.asarray(table_row[:used], dtype=np.int64), device=k_pool.device)
    kc = bits(k_pool.index_select(0, idx))
    vc = bits(v_pool.index_select(0, idx))
    return kc, vc, np.arange(used)


def compare(o_gpu: torch.Tensor, lse_gpu: torch.Tensor, o_ref: np.ndarray, lse_ref: np.ndarray, what: str):
    """The parity gate: max-abs O error <= 1e-2 and max-abs LSE error <= 1e-3, no NaN."""
    o = o_gpu.detach().double().cpu().numpy()
    lse = lse_gpu.detach().double().cpu().numpy()
    assert o.shape == o_ref.shape and lse.shape == lse_ref.shape, (o.shape, o_ref.shape)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), f"{what}: non-finite output"
    err_o = float(np.abs(o - o_ref).max())
    err_l = float(np.abs(lse - lse_ref).max())
    rel = float(np.linalg.norm(o - o_ref) / max(np.linalg.norm(o_ref), 1e-30))
    print(f"[parity] {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e} rel={rel:.2e} "
          f"max|O|={np.abs(o_ref).max():.3e}", flush=True)
    assert err_o <= O_TOL, f"{what}: max|dO| = {err_o}"
    assert err_l <= LSE_TOL, f"{what}: max|dLSE| = {err_l}"
    return err_o, err_l


def host_pool_of(pool: torch.Tensor) -> np.ndarray:
    """The whole pool as host bf16 bits (for the oracle, which reads the exact bits on the device)."""
    return bits(pool)


class MixedInputs:
    """The mixed scheduler step's inputs on one shared pool of 64-token pages: a chunk of request
    A (C tokens at prefix P) and one new token for each decode request, appended in one call;
    request A first in the block table, then the decode requests.  ``lens`` are the decode
    requests' lengths including the appended token.  The same tag gives the same bits."""

    def __init__(self, prefix: int, chunk: int, lens, tag: int, device="cuda"):
        self.prefix, self.chunk = prefix, chunk
        self.lens = np.asarray(lens, dtype=np.int64)
        final = np.concatenate([[prefix + chunk], self.lens])
        self.tables, self.num_pages, _ = W.place_pages(final, tag, 0)
        self.k = torch.empty((self.num_pages, W.HKV, W.PAGE, W.HEAD_DIM), dtype=torch.bfloat16, device=device)
        self.v = torch.empty_like(self.k)
        fill_normal_(self.k, W.torch_seed(tag, 1))
        fill_normal_(self.v, W.torch_seed(tag, 2))
        n_new = chunk + len(self.lens)
        self.k_new = W.normal_bf16((n_new, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 3), device)
        self.v_new = W.normal_bf16((n_new, W.HKV, W.HEAD_DIM), W.torch_seed(tag, 4), device)
        self.q_a = W.normal_bf16((chunk, W.HQ, W.HEAD_DIM), W.torch_seed(tag, 5), device)
        self.q_d = W.normal_bf16((len(self.lens), W.HQ, W.HEAD_DIM), W.torch_seed(tag, 6), device)
        self.cu_np = np.concatenate([[0, chunk], chunk + np.arange(1, len(self.lens) + 1)]).astype(np.int32)
        self.start_np = np.concatenate([[prefix], self.lens - 1]).astype(np.int32)
        self.bt = torch.as_tensor(self.tables, device=device)
        self.bt_a = self.bt[0].contiguous()
        self.bt_dec = self.bt[1:].contiguous()
        self.cu = torch.as_tensor(self.cu_np, device=device)
        self.start = torch.as_tensor(self.start_np, device=device)
        self.kv_lens = torch.as_tensor(self.lens.astype(np.int32), device=device)
        self.max_len = int(self.lens.max())


class DecodeBatch:
    """Decode-only pool: random K/V in every slot, unused slots poisoned, seeded placement."""

    def __init__(self, lens, tag: int, device="cuda", poison=True, spare=1):
        self.lens = np.asarray(lens, dtype=np.int64)
        self.tables, self.num_pages, self.spare = W.place_pages(self.lens, tag, 0, spare=spare)
        self.k = new_pool(self.num_pages, device, W.torch_seed(tag, 1))
        self.v = new_pool(self.num_pages, device, W.torch_seed(tag, 2))
        if poison:
            poison_unused(self.k, self.tables, self.lens, self.spare)
            poison_unused(self.v, self.tables, self.lens, self.spare)
        b = len(self.lens)
        self.q = torch.empty((b, W.HQ, W.HEAD_DIM), dtype=torch.bfloat16, device=device)
        fill_normal_(self.q, W.torch_seed(tag, 3))
        self.max_len = int(self.lens.max())
        stride = max(self.tables.shape[1], (self.max_len + W.PAGE - 1) // W.PAGE)
        tb = np.full((b, stride), self.spare[0], dtype=np.int32)
        tb[:, : self.tables.shape[1]] = self.tables
        self.tables = tb
        self.bt = torch.as_tensor(tb, device=device)
        self.kv_lens = torch.as_tensor(self.lens.astype(np.int32), device=device)

    def reference(self, rows=None):
        """Oracle (O, LSE) for the given request indices (default: all)."""
        rows = range(len(self.lens)) if rows is None else rows
        qb = bits(self.q)
        outs, lses = [], []
        for b in rows:
            kc, vc, ident = request_pages_host(self.k, self.v, self.tables[b], int(self.lens[b]))
            o, l = oracle.decode(qb[b:b + 1], kc, vc, [int(self.lens[b])], [ident], W.SCALE)
            outs.append(o[0])
            lses.append(l[0])
        return np.stack(outs), np.stack(lses)
