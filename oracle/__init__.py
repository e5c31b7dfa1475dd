"""ORACLE — test infrastructure, not the product.

Python entry to the fp64 CPU definition of MLA decode in ``oracle.c``. Only the
tests, the smoke check and the benchmark's CPU-baseline leg may import this
package; the GPU library never calls it and shares no code with it.

Every function here is pinned by ``tests/test_oracle_pins.py`` against facts the
source pages or mathematics fix (see each test's docstring); no function is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

F64, F32, BF16 = 0, 1, 2


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, portable x86-64-v3 code)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class _Dims(ctypes.Structure):
    _fields_ = [("h", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_r", ctypes.c_int32),
                ("d_n", ctypes.c_int32), ("d_v", ctypes.c_int32), ("scale", ctypes.c_double),
                ("rope_base", ctypes.c_double), ("store_bf16", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=True)
    lib = ctypes.CDLL(_LIB)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.oracle_mla_decode.restype = i32
    lib.oracle_mla_decode.argtypes = [ctypes.POINTER(_Dims), i32, i32, i32, i32, vp, vp, vp, vp,
                                      vp, vp, vp, vp, vp, i32, i32, vp, vp, i32, vp, vp, vp, i64]
    lib.oracle_rope.restype = None
    lib.oracle_rope.argtypes = [vp, i32, i64, ctypes.c_double, vp]
    lib.oracle_round_bf16.restype = ctypes.c_double
    lib.oracle_round_bf16.argtypes = [ctypes.c_double]
    lib.oracle_cache_keys.restype = None
    lib.oracle_cache_keys.argtypes = [ctypes.POINTER(_Dims), i32, i32, i32, vp, vp, vp]
    lib.oracle_project_latent.restype = i32
    lib.oracle_project_latent.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, ctypes.c_double,
                                          vp, ctypes.c_double, vp]
    lib.oracle_round_bf16_array.restype = None
    lib.oracle_round_bf16_array.argtypes = [i64, vp, vp]
    lib.oracle_threads.restype = i32
    lib.oracle_threads.argtypes = []
    _lib = lib
    return lib


def threads() -> int:
    return int(_load().oracle_threads())


def _type_of(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float64, float32 or uint16 (bf16 bits), got %s" % a.dtype)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def rope(x: np.ndarray, pos: int, base: float = 10000.0) -> np.ndarray:
    """RoPE of one vector (pairs (2k, 2k+1) rotated by pos * base^(-2k/d))."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty_like(x)
    _load().oracle_rope(x.ctypes.data, x.shape[0], int(pos), float(base), out.ctypes.data)
    return out


def round_bf16(x: float) -> float:
    return float(_load().oracle_round_bf16(float(x)))


def mla_decode(*, h: int, d_c: int, d_r: int, d_n: int, d_v: int, c_kv, k_r, kv_lens, q_nope,
               q_r, w_uk, w_uv, x=None, w_g=None, scale: Optional[float] = None,
               rope_base: float = 10000.0, store_bf16: bool = False, absorbed: bool = False,
               select: Optional[Sequence] = None, want_lse: bool = False,
               probs_len: int = 0):
    """Decode output ``out [B, n_q, h*d_v]`` in fp64 (and optionally lse, probs).

    All tensors share one dtype: float64, float32 or uint16 bf16 bits.
    ``c_kv [B, T, d_c]``, ``k_r [B, T, d_r]`` raw, ``q_nope [B, n_q, h, d_n]``,
    ``q_r [B, n_q, h, d_r]`` raw, ``w_uk [d_c, h*d_n]``, ``w_uv [d_c, h*d_v]``,
    ``x [B, n_q, d_model]``, ``w_g [d_model, h*d_v]``; ``kv_lens [B]`` counts the
    n_q new tokens. ``select`` is a list of (b, head) pairs; unselected outputs
    stay NaN. ``scale`` defaults to 1/sqrt(d_n + d_r).
    """
    c_kv = np.ascontiguousarray(c_kv)
    t = _type_of(c_kv)
    B, T, _ = c_kv.shape
    q_nope = np.ascontiguousarray(q_nope)
    n_q = q_nope.shape[1]
    arrs = [c_kv, k_r, q_nope, q_r, w_uk, w_uv, x, w_g]
    arrs = [None if a is None else np.ascontiguousarray(a) for a in arrs]
    for a in arrs:
        if a is not None and _type_of(a) != t:
            raise TypeError("all oracle inputs must share one dtype")
    c_kv, k_r, q_nope, q_r, w_uk, w_uv, x, w_g = arrs
    if d_r and (k_r is None or q_r is None):
        raise ValueError("d_r > 0 needs k_r and q_r")
    kv = np.ascontiguousarray(kv_lens, np.int32)
    dims = _Dims(h, d_c, d_r, d_n, d_v, 1.0 / np.sqrt(d_n + d_r) if scale is None else scale,
                 rope_base, 1 if store_bf16 else 0)
    out = np.full((B, n_q, h * d_v), np.nan)
    lse = np.full((B, n_q, h), np.nan) if want_lse else None
    probs = np.zeros((B, n_q, h, probs_len)) if probs_len else None
    if select is None:
        n_sel, sb, sh = -1, None, None
    else:
        sel = np.asarray(select, np.int32).reshape(-1, 2)
        n_sel = sel.shape[0]
        sb = np.ascontiguousarray(sel[:, 0])
        sh = np.ascontiguousarray(sel[:, 1])
    d_model = 0 if x is None else x.shape[-1]
    rc = _load().oracle_mla_decode(
        ctypes.byref(dims), B, n_q, T, t, _ptr(c_kv), _ptr(k_r), kv.ctypes.data, _ptr(q_nope),
        _ptr(q_r), _ptr(w_uk), _ptr(w_uv), _ptr(x), _ptr(w_g), d_model, n_sel, _ptr(sb), _ptr(sh),
        1 if absorbed else 0, out.ctypes.data, _ptr(lse), _ptr(probs), probs_len)
    if rc != 0:
        raise ValueError("oracle rejected the shapes (kv_len < n_q, kv_len > T or odd d_r)")
    res = [out]
    if want_lse:
        res.append(lse)
    if probs_len:
        res.append(probs)
    return res[0] if len(res) == 1 else tuple(res)


def cache_keys(*, d_r: int, k_r, kv_lens, rope_base: float = 10000.0, store_bf16: bool = True):
    """The rotated decoupled keys as the cache stores them, fp64 [B, T, d_r]."""
    k_r = np.ascontiguousarray(k_r)
    B, T, _ = k_r.shape
    kv = np.ascontiguousarray(kv_lens, np.int32)
    dims = _Dims(1, 0, d_r, 0, 0, 1.0, rope_base, 1 if store_bf16 else 0)
    out = np.full((B, T, d_r), np.nan)
    _load().oracle_cache_keys(ctypes.byref(dims), B, T, _type_of(k_r), k_r.ctypes.data,
                              kv.ctypes.data, out.ctypes.data)
    return out


def unabsorbed_flops(h, d_c, d_n, d_v, d_r, kv_lens, n_q, d_model=0) -> float:
    """Floating-point operations the explicit-K/V definition executes."""
    kv = np.asarray(kv_lens, np.float64)
    proj = 2.0 * h * kv.sum() * d_c * (d_n + d_v)
    vis = sum(float(n) - n_q + j + 1 for n in kv for j in range(n_q))
    attn = 2.0 * h * vis * (d_n + d_r + d_v)
    gate = 2.0 * len(kv) * n_q * d_model * h * d_v
    return proj + attn + gate


def explicit_kv(*, c_kv, w_uk, w_uv, kv_lens, h: int, d_n: int, d_v: int):
    """The explicit per-head keys and values of every cached token, the form the
    non-absorbed decode attends over (MLA tutorial page §3.2: k = c_KV · W_UK and
    v = c_KV · W_UV; §2.2 for the head split of W_UK and W_UV): fp64
    ``K [B, T, h, d_n]`` and ``V [B, T, h, d_v]`` from ``c_kv [B, T, d_c]`` and the
    formula-layout ``w_uk [d_c, h*d_n]``, ``w_uv [d_c, h*d_v]`` (one dtype: float64,
    float32 or bf16 bits). Slots past ``kv_lens[b]`` are NaN."""
    def f64(a):
        a = np.asarray(a)
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 \
            else a.astype(np.float64)
    c = f64(c_kv)
    uk, uv = f64(w_uk), f64(w_uv)
    B, T, _ = c.shape
    K = np.full((B, T, h, d_n), np.nan)
    V = np.full((B, T, h, d_v), np.nan)
    for b in range(B):
        n = int(kv_lens[b])
        K[b, :n] = (c[b, :n] @ uk).reshape(n, h, d_n)
        V[b, :n] = (c[b, :n] @ uv).reshape(n, h, d_v)
    return K, V


def latent_decode(*, q_abs, q_r, c_kv, k_r, kv_lens, scale: float, rope_base: float = 10000.0,
                  store_bf16: bool = True):
    """Attention in latent space for a given absorbed query, the step that weight-level
    absorption leaves at run time (MLA tutorial page §2.2: W_UK absorbed into the
    query's up-projection and W_UV into the output projection; §5.1: the scores
    q_abs · c_KV and the weighted sum attn · c_KV stay in latent space; interview
    guide §6.2 for the decoupled RoPE key). Per sequence b, query j (at position
    p_j = kv_len - n_q + j) and head i:

        s_t   = scale * (q_abs · c_t + RoPE(q_R, p_j) · k̃_R,t),  t <= p_j
        o_lat = Σ_t softmax(s)_t c_t

    ``q_abs [B, n_q, h, d_c]``, ``q_r [B, n_q, h, d_r]`` raw (or None), ``c_kv [B, T, d_c]``,
    ``k_r [B, T, d_r]`` raw (or None); bf16 bits, float32 or float64. k̃_R is the rotated
    key as the cache stores it (``cache_keys``). Returns fp64 ``o_lat [B, n_q, h, d_c]``
    and ``lse [B, n_q, h]``."""
    def f64(a):
        if a is None:
            return None
        a = np.asarray(a)
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if a.dtype == np.uint16 \
            else a.astype(np.float64)
    qa, qr, c = f64(q_abs), f64(q_r), f64(c_kv)
    B, n_q, h, d_c = qa.shape
    d_r = 0 if qr is None else qr.shape[-1]
    kr = cache_keys(d_r=d_r, k_r=k_r, kv_lens=kv_lens, rope_base=rope_base, store_bf16=store_bf16) if d_r else None
    o_lat = np.full((B, n_q, h, d_c), np.nan)
    lse = np.full((B, n_q, h), np.nan)
    for b in range(B):
        T = int(kv_lens[b])
        for j in range(n_q):
            pos = T - n_q + j
            s = qa[b, j] @ c[b, :pos + 1].T                                   # [h, t]
            if d_r:
                qrot = np.stack([rope(qr[b, j, i], pos, rope_base) for i in range(h)])
                s = s + qrot @ kr[b, :pos + 1].T
            s = scale * s
            m = s.max(axis=1, keepdims=True)
            e = np.exp(s - m)
            z = e.sum(axis=1, keepdims=True)
            o_lat[b, j] = (e / z) @ c[b, :pos + 1]
            lse[b, j] = (m + np.log(z))[:, 0]
    return o_lat, lse


def round_bf16_array(x) -> np.ndarray:
    """Nearest-even bf16 value of every element (fp64 in, fp64 out)."""
    x = np.ascontiguousarray(x, np.float64)
    out = np.empty_like(x)
    _load().oracle_round_bf16_array(x.size, x.ctypes.data, out.ctypes.data)
    return out


def project_latent(*, hidden, w_dkv, w_kr=None, gain=None, eps: float = 1e-6, pos,
                   rope_base: float = 10000.0) -> np.ndarray:
    """Cache rows ``[M, d_c + d_r]`` in fp64 from hidden states: the RMS-normalised
    down-projection ``gain * c / sqrt(mean(c^2) + eps)`` with ``c = h . W_DKV``,
    followed by ``RoPE(h . W_KR, pos)``.

    ``hidden [..., d_model]`` (leading dims flattened to M), ``w_dkv [d_model, d_c]``,
    ``w_kr [d_model, d_r]`` or None, one dtype (float64, float32 or bf16 bits);
    ``gain [d_c]`` (any float dtype) or None for ones; ``pos`` one position per row.
    """
    hidden = np.ascontiguousarray(hidden)
    t = _type_of(hidden)
    d_model = hidden.shape[-1]
    M = hidden.size // d_model if d_model else 0
    w_dkv = np.ascontiguousarray(w_dkv)
    d_c = w_dkv.shape[1]
    d_r = 0 if w_kr is None else np.asarray(w_kr).shape[1]
    if w_kr is not None:
        w_kr = np.ascontiguousarray(w_kr)
    for a in (w_dkv, w_kr):
        if a is not None and (_type_of(a) != t or a.shape[0] != d_model):
            raise TypeError("weights must share the hidden state's dtype and d_model")
    g = None if gain is None else np.ascontiguousarray(gain, np.float64)
    p = np.ascontiguousarray(np.broadcast_to(np.asarray(pos, np.int64).reshape(-1), (M,)))
    out = np.full((M, d_c + d_r), np.nan)
    rc = _load().oracle_project_latent(M, d_model, d_c, d_r, t, hidden.ctypes.data,
                                       w_dkv.ctypes.data, _ptr(w_kr), _ptr(g), float(eps),
                                       p.ctypes.data, float(rope_base), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the shapes (odd d_r, d_r > 1024 or eps < 0)")
    return out
