"""Device set-up for one synthetic decode step (used by the tests, the smoke check
and the benchmark).

It uploads a drawn workload, packs the weights with mla_absorb_weights, fills
the latent cache with mla_append_latent (contiguous or paged) and runs
mla_decode / mla_decode_paged. PyTorch provides memory and the stream only.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

from . import mla
from .synth import Workload


def to_device(a: Optional[np.ndarray], device="cuda"):
    if a is None:
        return None
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


class GpuStep:
    """One layer's decode step on the GPU for workload `w` and drawn tensors `t`."""

    def __init__(self, w: Workload, t: dict, device="cuda", poison: bool = True,
                 t_max: Optional[int] = None, pool_blocks: Optional[int] = None):
        self.w = w
        self.device = device
        dt = mla.MLA_F32 if w.dtype == "f32" else mla.MLA_BF16
        self.dims = mla.dims(w.h, w.d_c, w.d_r, w.d_n, w.d_v, dt, rope_base=w.rope_base)
        self.tdtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
        B = w.batch
        # weights
        w_uk, w_uv = to_device(t["w_uk"], device), to_device(t["w_uv"], device)
        nbytes = mla.mla_absorb_weights(self.dims)
        self.packed = torch.empty(nbytes, dtype=torch.uint8, device=device)
        mla.mla_absorb_weights(self.dims, w_uk, w_uv, self.packed)
        del w_uk, w_uv
        # queries
        self.q_nope = to_device(t["q_nope"], device)
        self.q_rope = to_device(t["q_r"], device)
        self.gate_x = to_device(t.get("x"), device)
        self.w_gate = to_device(t.get("w_g"), device)
        self.kv_lens = torch.from_numpy(w.kv_lens.astype(np.int32)).to(device)
        self.kv_lens_host = [int(v) for v in w.kv_lens]
        # cache
        fill = float("nan") if poison else 0.0
        if w.paged:
            self.n_blocks = int(pool_blocks or w.pool_blocks)
            self.pool = torch.full((self.n_blocks, w.block_size, w.row), fill, dtype=self.tdtype, device=device)
            self.block_table = torch.from_numpy(w.block_table.astype(np.int32)).to(device)
            self.cache = self.pool
        else:
            self.t_max = int(t_max or w.kv_max)
            self.cache = torch.full((B, self.t_max, w.row), fill, dtype=self.tdtype, device=device)
            self.block_table = None
        self._append(t)
        self.out = torch.empty((B, w.n_q, w.h * w.d_v), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, w.n_q, w.h), dtype=torch.float32, device=device)
        self.workspace = None
        self._ws_key = None

    def _append(self, t: dict):
        """Append every sequence's tokens 0 .. kv_len-1 (one call per sequence, since
        ragged batches end at different slots)."""
        w = self.w
        c_kv = to_device(t["c_kv"], self.device)
        k_r = to_device(t["k_r"], self.device)
        zero = torch.zeros(1, dtype=torch.int32, device=self.device)
        for b in range(w.batch):
            n = int(w.kv_lens[b])
            ck = c_kv[b:b + 1, :n].contiguous()
            kr = k_r[b:b + 1, :n].contiguous() if k_r is not None else None
            if w.paged:
                mla.mla_append_latent(self.dims, self.pool, c_kv=ck, k_r=kr, pos0=zero,
                                      block_table=self.block_table[b:b + 1].contiguous(),
                                      block_size=w.block_size, max_blocks=w.max_blocks,
                                      n_blocks=self.n_blocks)
            else:
                view = self.cache[b:b + 1]
                mla.mla_append_latent(self.dims, view, c_kv=ck, k_r=kr, pos0=zero, t_max=self.t_max)
        torch.cuda.synchronize()

    def cache_rows(self, b: int, n: int) -> torch.Tensor:
        """Logical rows 0..n-1 of sequence b, gathered (for checks)."""
        w = self.w
        if not w.paged:
            return self.cache[b, :n]
        blocks = self.block_table[b, :(n + w.block_size - 1) // w.block_size].long()
        return self.pool[blocks].reshape(-1, w.row)[:n]

    def decode(self, num_splits: int = 0, events=None, use_host_lens: bool = True, stream=None,
               out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None):
        w = self.w
        out = self.out if out is None else out
        lse = self.lse if lse is None else lse
        kw = dict(kv_lens=self.kv_lens, max_kv_len=w.kv_max, q_nope=self.q_nope, q_rope=self.q_rope,
                  packed_w=self.packed, out=out, lse=lse,
                  kv_lens_host=self.kv_lens_host if use_host_lens else None,
                  gate_x=self.gate_x, w_gate=self.w_gate, num_splits=num_splits, events=events,
                  stream=stream)
        key = (num_splits, use_host_lens)
        if self.workspace is None or key != self._ws_key:
            nbytes = self.workspace_bytes(num_splits, use_host_lens)
            if self.workspace is None or self.workspace.numel() < nbytes:
                self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
            self._ws_key = key
        kw["workspace"] = self.workspace
        if w.paged:
            mla.mla_decode_paged(self.dims, self.pool, self.block_table, w.block_size, w.max_blocks,
                                 self.n_blocks, **kw)
        else:
            mla.mla_decode(self.dims, self.cache, self.t_max, **kw)
        return out

    def workspace_bytes(self, num_splits: int = 0, use_host_lens: bool = True) -> int:
        w = self.w
        return mla.decode_workspace_bytes(self.dims, batch=w.batch, n_q=w.n_q, max_kv_len=w.kv_max,
                                          kv_lens_host=self.kv_lens_host if use_host_lens else None,
                                          gated=w.gated, num_splits=num_splits, paged=w.paged,
                                          block_size=w.block_size)
