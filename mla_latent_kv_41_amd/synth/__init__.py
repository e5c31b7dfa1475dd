"""Seeded synthetic workloads for absorbed-MLA decode.

Holds random draws and shape bookkeeping only: none of the attention
arithmetic lives here. The oracle and the HIP path both take their inputs from
this module, so they compute on bit-identical data.

bf16 tensors are returned as ``numpy.uint16`` arrays holding the bf16 bit
patterns; fp32 tensors as ``numpy.float32``.

The five workloads are the MLA decode shapes of the DeepSeek-V2 attention
block described on the source pages ("MLA多头潜在注意力机制" §2.2 and §5;
"解耦 RoPE" cache row of 512 + 64 on the linear-algebra page), plus the
gated, position-free variant of the Gated-MLA page (§2.6, §3.3).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the generator with gcc into ``libsynth.so`` next to its source."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    u64, i32, i64 = ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64
    vp, dbl = ctypes.c_void_p, ctypes.c_double
    lib.synth_key.restype = u64
    lib.synth_key.argtypes = [u64, ctypes.c_char_p]
    for name in ("synth_normal_f64", "synth_normal_f32", "synth_normal_bf16"):
        getattr(lib, name).restype = None
        getattr(lib, name).argtypes = [u64, u64, u64, dbl, vp]
    lib.synth_rmsnorm_rows.restype = None
    lib.synth_rmsnorm_rows.argtypes = [u64, u64, u64, ctypes.c_int, dbl, ctypes.c_int, vp]
    lib.synth_uniform_int.restype = None
    lib.synth_uniform_int.argtypes = [u64, u64, i32, i32, vp]
    lib.synth_permutation.restype = None
    lib.synth_permutation.argtypes = [u64, i32, vp]
    lib.synth_f64_to_bf16.restype = ctypes.c_uint16
    lib.synth_f64_to_bf16.argtypes = [dbl]
    _ = i64
    _lib = lib
    return lib


def key(seed: int, tag: str) -> int:
    return int(_load().synth_key(seed, tag.encode()))


def normal(seed: int, tag: str, shape, std: float = 1.0, dtype: str = "f64", start: int = 0):
    """N(0, std^2) draws of the stream (seed, tag), elements [start, start + size)."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    k = key(seed, tag)
    if dtype == "f64":
        out = np.empty(n, np.float64)
        lib.synth_normal_f64(k, start, n, std, out.ctypes.data)
    elif dtype == "f32":
        out = np.empty(n, np.float32)
        lib.synth_normal_f32(k, start, n, std, out.ctypes.data)
    elif dtype == "bf16":
        out = np.empty(n, np.uint16)
        lib.synth_normal_bf16(k, start, n, std, out.ctypes.data)
    else:
        raise ValueError(dtype)
    return out.reshape(shape)


def rmsnorm_rows(seed: int, tag: str, rows: int, width: int, dtype: str, eps: float = 1e-6,
                 row0: int = 0):
    """Rows of N(0,1) draws, each divided by its RMS (no gain)."""
    lib = _load()
    if dtype == "bf16":
        out = np.empty((rows, width), np.uint16)
    elif dtype == "f32":
        out = np.empty((rows, width), np.float32)
    else:
        raise ValueError(dtype)
    lib.synth_rmsnorm_rows(key(seed, tag), row0, rows, width, eps, 1 if dtype == "bf16" else 0,
                           out.ctypes.data)
    return out


def uniform_int(seed: int, tag: str, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    _load().synth_uniform_int(key(seed, tag), n, lo, hi, out.ctypes.data)
    return out


def permutation(seed: int, tag: str, n: int) -> np.ndarray:
    out = np.empty(n, np.int32)
    _load().synth_permutation(key(seed, tag), n, out.ctypes.data)
    return out


def f64_to_bf16_bits(x: float) -> int:
    return int(_load().synth_f64_to_bf16(float(x)))


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------------
# Workloads
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    """Shape, layout and seed of one decode step.

    ``kv_lens[b]`` counts every token sequence b attends over, the n_q new ones
    included: query j of sequence b sits at position ``kv_lens[b] - n_q + j``.
    """
    name: str
    cid: int
    dtype: str                 # "f32" or "bf16": cache, weights and query dtype
    h: int
    d_c: int
    d_r: int
    d_n: int
    d_v: int
    batch: int
    n_q: int
    kv_lens: np.ndarray        # int32 [batch]
    paged: bool
    block_size: int = 64
    pool_blocks: int = 0
    block_table: Optional[np.ndarray] = None   # int32 [batch, max_blocks]
    gated: bool = False
    d_model: int = 0
    seed: int = 0
    rope_base: float = 10000.0
    rms_norm_latent: bool = True

    @property
    def row(self) -> int:
        return self.d_c + self.d_r

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.d_n + self.d_r))

    @property
    def kv_max(self) -> int:
        return int(self.kv_lens.max())

    @property
    def max_blocks(self) -> int:
        return (self.kv_max + self.block_size - 1) // self.block_size

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def cache_bytes_visible(self) -> int:
        return int(self.kv_lens.astype(np.int64).sum()) * self.row * self.elem_bytes


def _paged_table(seed: int, kv_lens: np.ndarray, block_size: int, pool_factor: float = 1.25):
    need = [(int(n) + block_size - 1) // block_size for n in kv_lens]
    total = int(sum(need))
    pool = int(np.ceil(total * pool_factor))
    perm = permutation(seed, "block_table", pool)
    max_blocks = max(need)
    table = np.full((len(kv_lens), max_blocks), -1, np.int32)
    k = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[k:k + nb]
        k += nb
    return pool, table


def make_workload(cid: int, batch: Optional[int] = None, ctx: Optional[int] = None,
                  ctx_range: Optional[tuple] = None, seed: Optional[int] = None) -> Workload:
    """One of the five decode workloads, optionally shrunk (batch / context).

    1 tiny fp32 (h=4, d_c=32, d_rope=8, d_qk_nope=d_v=16, B=1, 64 cached + 1 query)
    2 DeepSeek-shaped (h=128, d_c=512, d_rope=64, d_qk_nope=d_v=128, B=32, 4096 + 1), contiguous
    3 paged long context (same dims, B=4, 32768 + 1), 64-token blocks, pool 1.25x
    4 ragged (same dims, B=64, cached lengths uniform in [512, 16384], 2 queries), paged
    5 gated, no position (h=64, d_rope=0, B=16, 65536 + 1, gate from d_model=4096), contiguous
    """
    s = 41000 + cid if seed is None else seed
    if cid == 1:
        B = batch or 1
        N = 64 if ctx is None else ctx
        return Workload("tiny_fp32", 1, "f32", 4, 32, 8, 16, 16, B, 1,
                        np.full(B, N + 1, np.int32), False, seed=s, rms_norm_latent=False)
    if cid == 2:
        B = batch or 32
        N = 4096 if ctx is None else ctx
        return Workload("deepseek_b32_ctx4096", 2, "bf16", 128, 512, 64, 128, 128, B, 1,
                        np.full(B, N + 1, np.int32), False, seed=s)
    if cid == 3:
        B = batch or 4
        N = 32768 if ctx is None else ctx
        kv = np.full(B, N + 1, np.int32)
        pool, table = _paged_table(s, kv, 64)
        return Workload("paged_b4_ctx32768", 3, "bf16", 128, 512, 64, 128, 128, B, 1, kv, True,
                        64, pool, table, seed=s)
    if cid == 4:
        B = batch or 64
        lo, hi = ctx_range or (512, 16384)
        n_q = 2
        kv = uniform_int(s, "ctx_len", B, lo, hi) + n_q
        pool, table = _paged_table(s, kv, 64)
        return Workload("ragged_b64_nq2", 4, "bf16", 128, 512, 64, 128, 128, B, n_q,
                        kv.astype(np.int32), True, 64, pool, table, seed=s)
    if cid == 5:
        B = batch or 16
        N = 65536 if ctx is None else ctx
        return Workload("gated_h64_b16_ctx65536", 5, "bf16", 64, 512, 0, 128, 128, B, 1,
                        np.full(B, N + 1, np.int32), False, gated=True, d_model=4096, seed=s)
    raise ValueError("unknown workload %r" % cid)


def draw(w: Workload) -> dict:
    """All tensors of one decode step, as host arrays.

    c_kv   [B, kv_max, d_c]   latent per token (RMS-normalised rows for the bf16 workloads)
    k_r    [B, kv_max, d_r]   raw (unrotated) decoupled key, or None when d_r == 0
    q_nope [B, n_q, h, d_n]
    q_r    [B, n_q, h, d_r]   raw (unrotated), or None
    w_uk   [d_c, h*d_n]       head i owns columns i*d_n .. i*d_n + d_n - 1
    w_uv   [d_c, h*d_v]
    x      [B, n_q, d_model]  gate input (gated workload only)
    w_g    [d_model, h*d_v]

    Token t of sequence b is stream row b * kv_max + t, so a shorter sequence
    is a prefix of what a longer one would draw.
    """
    s, dt = w.seed, w.dtype
    B, T = w.batch, w.kv_max
    out = {}
    if w.rms_norm_latent:
        out["c_kv"] = rmsnorm_rows(s, "c_kv", B * T, w.d_c, dt).reshape(B, T, w.d_c)
    else:
        out["c_kv"] = normal(s, "c_kv", (B, T, w.d_c), 1.0, dt)
    out["k_r"] = normal(s, "k_r", (B, T, w.d_r), 1.0, dt) if w.d_r else None
    out["q_nope"] = normal(s, "q_nope", (B, w.n_q, w.h, w.d_n), 1.0, dt)
    out["q_r"] = normal(s, "q_r", (B, w.n_q, w.h, w.d_r), 1.0, dt) if w.d_r else None
    wstd = 1.0 / np.sqrt(w.d_c)
    out["w_uk"] = normal(s, "w_uk", (w.d_c, w.h * w.d_n), wstd, dt)
    out["w_uv"] = normal(s, "w_uv", (w.d_c, w.h * w.d_v), wstd, dt)
    if w.gated:
        out["x"] = normal(s, "x", (B, w.n_q, w.d_model), 1.0, dt)
        out["w_g"] = normal(s, "w_g", (w.d_model, w.h * w.d_v), 1.0 / np.sqrt(w.d_model), dt)
    else:
        out["x"] = None
        out["w_g"] = None
    return out


# --------------------------------------------------------------------------------------
# Fused append (hidden state -> latent cache row)
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class ProjWorkload:
    """Shape, layout and seed of one fused latent append: each sequence's n_new new
    tokens go to positions pos0[b] .. pos0[b] + n_new - 1 of its cache."""
    name: str
    dtype: str                 # "f32" or "bf16": hidden state, weights and cache
    d_model: int
    d_c: int
    d_r: int
    batch: int
    n_new: int
    pos0: np.ndarray           # int32 [batch]
    paged: bool
    block_size: int = 64
    pool_blocks: int = 0
    block_table: Optional[np.ndarray] = None
    seed: int = 0
    rope_base: float = 10000.0
    eps: float = 1e-6

    @property
    def row(self) -> int:
        return self.d_c + self.d_r

    @property
    def rows(self) -> int:
        return self.batch * self.n_new

    @property
    def t_max(self) -> int:
        return int(self.pos0.max()) + self.n_new

    @property
    def max_blocks(self) -> int:
        return (self.t_max + self.block_size - 1) // self.block_size

    def positions(self) -> np.ndarray:
        """Position of every new token, [batch * n_new] in (b, j) order."""
        return (self.pos0.astype(np.int64)[:, None] + np.arange(self.n_new)[None, :]).reshape(-1)


def make_projection(kind: str = "deepseek", batch: Optional[int] = None, n_new: int = 1,
                    d_model: Optional[int] = None, pos: Optional[int] = None,
                    pos_range: Optional[tuple] = None, paged: bool = False,
                    seed: Optional[int] = None) -> ProjWorkload:
    """A fused-append workload.

    deepseek  bf16, d_model=4096, d_c=512, d_rope=64, B=32, one new token at slot 4096
              (the decode step of the DeepSeek-shaped workload)
    nope      bf16, d_model=4096, d_c=512, d_rope=0, B=16 (the position-free variant)
    tiny      fp32, d_model=24, d_c=32, d_rope=8, B=2 (the tiny layer)
    Positions are `pos` for every sequence, or uniform in `pos_range` (inclusive).
    """
    s = 41006 if seed is None else seed
    if kind == "deepseek":
        dt, dm, dc, dr, B = "bf16", 4096, 512, 64, 32
    elif kind == "nope":
        dt, dm, dc, dr, B = "bf16", 4096, 512, 0, 16
    elif kind == "tiny":
        dt, dm, dc, dr, B = "f32", 24, 32, 8, 2
    else:
        raise ValueError("unknown projection workload %r" % kind)
    B = batch or B
    dm = d_model or dm
    if pos_range is not None:
        pos0 = uniform_int(s, "pos0", B, pos_range[0], pos_range[1])
    else:
        pos0 = np.full(B, 4096 if pos is None else pos, np.int32)
    w = ProjWorkload("fused_append_%s_b%d_n%d_dmodel%d" % (kind, B, n_new, dm), dt, dm, dc, dr, B, n_new,
                     pos0.astype(np.int32), paged, seed=s)
    if paged:
        w.pool_blocks, w.block_table = _paged_table(s, w.pos0 + n_new, w.block_size)
    return w


def draw_projection(w: ProjWorkload) -> dict:
    """Host tensors of one fused append.

    hidden [B, n_new, d_model]  N(0, 1)
    w_dkv  [d_model, d_c]       N(0, 1/d_model), so c = h . W_DKV is about N(0, 1)
    w_kr   [d_model, d_r]       N(0, 1/d_model), or None when d_r == 0
    gain   [d_c] fp32           1 + N(0, 0.1^2), the RMSNorm gain
    """
    s, dt = w.seed, w.dtype
    std = 1.0 / np.sqrt(w.d_model)
    return {
        "hidden": normal(s, "hidden", (w.batch, w.n_new, w.d_model), 1.0, dt),
        "w_dkv": normal(s, "w_dkv", (w.d_model, w.d_c), std, dt),
        "w_kr": normal(s, "w_kr", (w.d_model, w.d_r), std, dt) if w.d_r else None,
        "gain": (1.0 + normal(s, "gain", (w.d_c,), 0.1, "f64")).astype(np.float32),
    }
