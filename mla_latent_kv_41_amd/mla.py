"""Python binding of libmla (ctypes): argument marshalling only.

The functions carry the C entry points' names (include/mla.h) and take torch
tensors (or raw integer device pointers). Every step of the decode runs in the
library's HIP kernels; PyTorch only provides device memory and the stream.
Importing this module fails loudly when libmla.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
# MLA_LIB_PATH selects another build of the same library (the phase-stamp tool's
# instrumented build); by default the in-tree libmla.so
LIB_PATH = os.environ.get("MLA_LIB_PATH") or os.path.join(HERE, "libmla.so")

MLA_OK, MLA_E_NULL, MLA_E_SHAPE, MLA_E_DTYPE, MLA_E_UNSUPPORTED, MLA_E_WORKSPACE, MLA_E_HIP = range(7)
MLA_F32, MLA_BF16 = 0, 1

EXPORTS = ("mla_absorb_weights", "mla_append_latent", "mla_decode", "mla_decode_paged",
           "mla_decode_noalloc", "mla_decode_latent", "mla_expand_kv", "mla_decode_explicit",
           "mla_pack_down_weights",
           "mla_project_append", "mla_status_string")


class MLAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, status_string(status), status))


class mla_dims(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("d_qk_nope", ctypes.c_int32), ("d_v", ctypes.c_int32), ("scale", ctypes.c_float),
                ("rope_base", ctypes.c_float), ("dtype", ctypes.c_int32)]


class mla_cache_layout(ctypes.Structure):
    _fields_ = [("block_table", ctypes.c_void_p), ("t_max", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("n_blocks", ctypes.c_int32)]


class mla_decode_args(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q", ctypes.c_int32), ("kv_lens", ctypes.c_void_p),
                ("kv_lens_host", ctypes.c_void_p), ("max_kv_len", ctypes.c_int32),
                ("q_nope", ctypes.c_void_p), ("q_rope", ctypes.c_void_p),
                ("packed_w", ctypes.c_void_p), ("gate_x", ctypes.c_void_p),
                ("w_gate", ctypes.c_void_p), ("d_model", ctypes.c_int32),
                ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.POINTER(ctypes.c_size_t)),
                ("num_splits", ctypes.c_int32), ("ev_attn_begin", ctypes.c_void_p),
                ("ev_attn_end", ctypes.c_void_p)]


class mla_project_args(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_new", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("hidden", ctypes.c_void_p), ("packed_down", ctypes.c_void_p),
                ("norm_gain", ctypes.c_void_p), ("norm_eps", ctypes.c_float), ("pos0", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.POINTER(ctypes.c_size_t)),
                ("k_splits", ctypes.c_int32)]


_lib = None


def lib():
    """The loaded libmla.so; raises if it was not built (no fallback path exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmla.so is not built (run __graft_entry__.build() or "
                               "python -m mla_latent_kv_41_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        st = ctypes.c_int32
        vp = ctypes.c_void_p
        L.mla_absorb_weights.restype = st
        L.mla_absorb_weights.argtypes = [ctypes.POINTER(mla_dims), vp, vp, vp,
                                         ctypes.POINTER(ctypes.c_size_t), vp]
        L.mla_append_latent.restype = st
        L.mla_append_latent.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.POINTER(mla_cache_layout),
                                        ctypes.c_int32, ctypes.c_int32, vp, vp, vp, vp]
        L.mla_decode.restype = st
        L.mla_decode.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.c_int32,
                                 ctypes.POINTER(mla_decode_args), vp]
        L.mla_decode_paged.restype = st
        L.mla_decode_paged.argtypes = [ctypes.POINTER(mla_dims), vp, vp, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.POINTER(mla_decode_args), vp]
        L.mla_decode_noalloc.restype = st
        L.mla_decode_noalloc.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.POINTER(mla_cache_layout),
                                         ctypes.POINTER(mla_decode_args), vp]
        L.mla_decode_latent.restype = st
        L.mla_decode_latent.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.POINTER(mla_cache_layout),
                                        ctypes.POINTER(mla_decode_args), vp]
        L.mla_expand_kv.restype = st
        L.mla_expand_kv.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.POINTER(mla_cache_layout), ctypes.c_int32,
                                    vp, ctypes.c_int32, vp, vp, vp, vp, vp, ctypes.POINTER(ctypes.c_size_t), vp]
        L.mla_decode_explicit.restype = st
        L.mla_decode_explicit.argtypes = [ctypes.POINTER(mla_dims), vp, vp, vp, ctypes.POINTER(mla_cache_layout),
                                          ctypes.POINTER(mla_decode_args), vp]
        L.mla_pack_down_weights.restype = st
        L.mla_pack_down_weights.argtypes = [ctypes.POINTER(mla_dims), ctypes.c_int32, vp, vp, vp,
                                            ctypes.POINTER(ctypes.c_size_t), vp]
        L.mla_project_append.restype = st
        L.mla_project_append.argtypes = [ctypes.POINTER(mla_dims), vp, ctypes.POINTER(mla_cache_layout),
                                         ctypes.POINTER(mla_project_args), vp]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_status_string.argtypes = [ctypes.c_int32]
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().mla_status_string(s).decode()


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dims(n_heads: int, d_c: int, d_rope: int, d_qk_nope: int, d_v: int, dtype: int,
         scale: float = 0.0, rope_base: float = 0.0) -> mla_dims:
    return mla_dims(n_heads, d_c, d_rope, d_qk_nope, d_v, scale, rope_base, dtype)


def _check(status: int, where: str) -> int:
    if status != MLA_OK:
        raise MLAError(status, where)
    return status


# ------------------------------------------------------------------------------ absorb

def mla_absorb_weights(d: mla_dims, w_uk=None, w_uv=None, packed=None, packed_bytes=None,
                       stream=None) -> int:
    """Pack W_UK / W_UV once. With packed=None returns the needed byte count."""
    n = ctypes.c_size_t(0 if packed_bytes is None else packed_bytes)
    if packed is None:
        _check(lib().mla_absorb_weights(ctypes.byref(d), None, None, None, ctypes.byref(n), None),
               "mla_absorb_weights")
        return n.value
    if packed_bytes is None:
        n.value = packed.numel() * packed.element_size()
    _check(lib().mla_absorb_weights(ctypes.byref(d), _ptr(w_uk), _ptr(w_uv), _ptr(packed),
                                    ctypes.byref(n), _stream(stream)), "mla_absorb_weights")
    return n.value


# ------------------------------------------------------------------------------ append

def mla_append_latent(d: mla_dims, cache, *, c_kv, k_r, pos0, t_max: int = 0, block_table=None,
                      block_size: int = 0, max_blocks: int = 0, n_blocks: int = 0,
                      batch: Optional[int] = None, n_new: Optional[int] = None, stream=None) -> int:
    """Write [c_KV ‖ RoPE(k_R)] rows at positions pos0[b] + j."""
    B = batch if batch is not None else c_kv.shape[0]
    N = n_new if n_new is not None else c_kv.shape[1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    return _check(lib().mla_append_latent(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), B, N,
                                          _ptr(c_kv), _ptr(k_r), _ptr(pos0), _stream(stream)),
                  "mla_append_latent")


# ------------------------------------------------------------------------------ fused append

def mla_pack_down_weights(d: mla_dims, d_model: int, w_dkv=None, w_kr=None, packed=None,
                          packed_bytes=None, stream=None) -> int:
    """Pack [W_DKV ‖ W_KR] once. With packed=None returns the needed byte count."""
    n = ctypes.c_size_t(0 if packed_bytes is None else packed_bytes)
    if packed is None:
        _check(lib().mla_pack_down_weights(ctypes.byref(d), d_model, None, None, None, ctypes.byref(n),
                                           None), "mla_pack_down_weights")
        return n.value
    if packed_bytes is None:
        n.value = packed.numel() * packed.element_size()
    _check(lib().mla_pack_down_weights(ctypes.byref(d), d_model, _ptr(w_dkv), _ptr(w_kr), _ptr(packed),
                                       ctypes.byref(n), _stream(stream)), "mla_pack_down_weights")
    return n.value


def _project_args(*, batch, n_new, d_model, hidden, packed_down, norm_gain, norm_eps, pos0,
                  workspace, workspace_bytes, k_splits):
    nbytes = ctypes.c_size_t(workspace_bytes)
    a = mla_project_args(batch, n_new, d_model, _ptr(hidden), _ptr(packed_down), _ptr(norm_gain),
                         norm_eps, _ptr(pos0), _ptr(workspace), ctypes.pointer(nbytes), k_splits)
    return a, nbytes


def mla_project_append(d: mla_dims, cache, *, hidden, packed_down, pos0, norm_gain=None,
                       norm_eps: float = 1e-6, t_max: int = 0, block_table=None, block_size: int = 0,
                       max_blocks: int = 0, n_blocks: int = 0, workspace=None, k_splits: int = 0,
                       d_model: Optional[int] = None, batch: Optional[int] = None,
                       n_new: Optional[int] = None, stream=None) -> int:
    """Write [gain * RMSNorm(h . W_DKV) ‖ RoPE(h . W_KR)] rows at positions pos0[b] + j."""
    B = batch if batch is not None else hidden.shape[0]
    N = n_new if n_new is not None else hidden.shape[1]
    D = d_model if d_model is not None else hidden.shape[-1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    common = dict(batch=B, n_new=N, d_model=D, hidden=hidden, packed_down=packed_down,
                  norm_gain=norm_gain, norm_eps=norm_eps, pos0=pos0, k_splits=k_splits)

    def query():
        a, n = _project_args(workspace=None, workspace_bytes=0, **common)
        _check(lib().mla_project_append(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), ctypes.byref(a),
                                        None), "mla_project_append")
        return n.value

    ws = _workspace_for(query, workspace, hidden.device)
    a, n = _project_args(workspace=ws, workspace_bytes=ws.numel() * ws.element_size(), **common)
    return _check(lib().mla_project_append(ctypes.byref(d), _ptr(cache), ctypes.byref(layout),
                                           ctypes.byref(a), _stream(stream)), "mla_project_append")


def prepare_project_append(d: mla_dims, cache, *, hidden, packed_down, pos0, workspace, norm_gain=None,
                           norm_eps: float = 1e-6, t_max: int = 0, block_table=None, block_size: int = 0,
                           max_blocks: int = 0, n_blocks: int = 0, k_splits: int = 0, stream=None):
    """mla_project_append with its arguments marshalled once: returns a function of
    no arguments that makes the same call (for loops where Python's per-call
    argument building would outlast the GPU work). The tensors must stay alive."""
    B, N, D = hidden.shape[0], hidden.shape[1], hidden.shape[-1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    a, n = _project_args(batch=B, n_new=N, d_model=D, hidden=hidden, packed_down=packed_down,
                         norm_gain=norm_gain, norm_eps=norm_eps, pos0=pos0, workspace=workspace,
                         workspace_bytes=workspace.numel() * workspace.element_size(), k_splits=k_splits)
    fn, dref, cref, lref, aref = (lib().mla_project_append, ctypes.byref(d), _ptr(cache),
                                  ctypes.byref(layout), ctypes.byref(a))
    st = _stream(stream)
    keep = (d, layout, a, n)

    def call():
        _ = keep
        return _check(fn(dref, cref, lref, aref, st), "mla_project_append")
    return call


def project_workspace_bytes(d: mla_dims, *, batch: int, n_new: int, d_model: int, k_splits: int = 0) -> int:
    """Workspace mla_project_append needs (pure host arithmetic; no device access)."""
    layout = mla_cache_layout(None, 1, 0, 0, 0)
    a, n = _project_args(batch=batch, n_new=n_new, d_model=d_model, hidden=None, packed_down=None,
                         norm_gain=None, norm_eps=1e-6, pos0=None, workspace=None, workspace_bytes=0,
                         k_splits=k_splits)
    _check(lib().mla_project_append(ctypes.byref(d), None, ctypes.byref(layout), ctypes.byref(a), None),
           "project_workspace_bytes")
    return n.value


# ------------------------------------------------------------------------------ decode

def _decode_args(*, batch, n_q, kv_lens, kv_lens_host, max_kv_len, q_nope, q_rope, packed_w,
                 gate_x, w_gate, out, lse, workspace, workspace_bytes, num_splits, events):
    nbytes = ctypes.c_size_t(workspace_bytes)
    host = None
    if kv_lens_host is not None:
        host = (ctypes.c_int32 * len(kv_lens_host))(*[int(v) for v in kv_lens_host])
    d_model = 0 if gate_x is None else int(gate_x.shape[-1])
    ev0, ev1 = (None, None) if events is None else events
    a = mla_decode_args(batch, n_q, _ptr(kv_lens), ctypes.cast(host, ctypes.c_void_p) if host else None,
                        max_kv_len, _ptr(q_nope), _ptr(q_rope), _ptr(packed_w), _ptr(gate_x),
                        _ptr(w_gate), d_model, _ptr(out), _ptr(lse), _ptr(workspace),
                        ctypes.pointer(nbytes), num_splits, ev0, ev1)
    return a, nbytes, host


def _workspace_for(query, workspace, device):
    if workspace is not None:
        return workspace
    import torch
    n = query()
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def mla_decode(d: mla_dims, cache, t_max: int, *, kv_lens, max_kv_len: int, q_nope, q_rope,
               packed_w, out, kv_lens_host: Optional[Sequence[int]] = None, gate_x=None, w_gate=None,
               lse=None, workspace=None, num_splits: int = 0, events=None, stream=None) -> int:
    """Absorbed decode over a contiguous cache [B][t_max][d_c + d_rope]."""
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    common = dict(batch=B, n_q=n_q, kv_lens=kv_lens, kv_lens_host=kv_lens_host,
                  max_kv_len=max_kv_len, q_nope=q_nope, q_rope=q_rope, packed_w=packed_w,
                  gate_x=gate_x, w_gate=w_gate, out=out, lse=lse, num_splits=num_splits,
                  events=events)

    def query():
        a, n, _h = _decode_args(workspace=None, workspace_bytes=0, **common)
        _check(lib().mla_decode(ctypes.byref(d), _ptr(cache), t_max, ctypes.byref(a), None), "mla_decode")
        return n.value

    ws = _workspace_for(query, workspace, q_nope.device)
    a, n, _h = _decode_args(workspace=ws, workspace_bytes=ws.numel() * ws.element_size(), **common)
    return _check(lib().mla_decode(ctypes.byref(d), _ptr(cache), t_max, ctypes.byref(a), _stream(stream)),
                  "mla_decode")


def mla_decode_paged(d: mla_dims, pool, block_table, block_size: int, max_blocks: int,
                     n_blocks: int, *, kv_lens, max_kv_len: int, q_nope, q_rope, packed_w, out,
                     kv_lens_host: Optional[Sequence[int]] = None, gate_x=None, w_gate=None,
                     lse=None, workspace=None, num_splits: int = 0, events=None, stream=None) -> int:
    """Absorbed decode over a paged pool [n_blocks][block_size][d_c + d_rope]."""
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    common = dict(batch=B, n_q=n_q, kv_lens=kv_lens, kv_lens_host=kv_lens_host,
                  max_kv_len=max_kv_len, q_nope=q_nope, q_rope=q_rope, packed_w=packed_w,
                  gate_x=gate_x, w_gate=w_gate, out=out, lse=lse, num_splits=num_splits,
                  events=events)

    def query():
        a, n, _h = _decode_args(workspace=None, workspace_bytes=0, **common)
        _check(lib().mla_decode_paged(ctypes.byref(d), _ptr(pool), _ptr(block_table), block_size,
                                      max_blocks, n_blocks, ctypes.byref(a), None), "mla_decode_paged")
        return n.value

    ws = _workspace_for(query, workspace, q_nope.device)
    a, n, _h = _decode_args(workspace=ws, workspace_bytes=ws.numel() * ws.element_size(), **common)
    return _check(lib().mla_decode_paged(ctypes.byref(d), _ptr(pool), _ptr(block_table), block_size,
                                         max_blocks, n_blocks, ctypes.byref(a), _stream(stream)),
                  "mla_decode_paged")


def mla_decode_noalloc(d: mla_dims, cache, *, kv_lens, max_kv_len: int, q_nope, q_rope, packed_w, out,
                       t_max: int = 0, block_table=None, block_size: int = 0, max_blocks: int = 0,
                       n_blocks: int = 0, kv_lens_host: Optional[Sequence[int]] = None, gate_x=None,
                       w_gate=None, lse=None, num_splits: int = 0, events=None, stream=None) -> int:
    """Decode with the library's own per-GPU scratch array as the workspace (no
    workspace argument; contiguous cache when block_table is None, else paged)."""
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    a, n, _h = _decode_args(batch=B, n_q=n_q, kv_lens=kv_lens, kv_lens_host=kv_lens_host,
                            max_kv_len=max_kv_len, q_nope=q_nope, q_rope=q_rope, packed_w=packed_w,
                            gate_x=gate_x, w_gate=w_gate, out=out, lse=lse, workspace=None,
                            workspace_bytes=0, num_splits=num_splits, events=events)
    return _check(lib().mla_decode_noalloc(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), ctypes.byref(a),
                                           _stream(stream)), "mla_decode_noalloc")


def mla_decode_latent(d: mla_dims, cache, *, kv_lens, max_kv_len: int, q_abs, q_rope, o_lat, t_max: int = 0,
                      block_table=None, block_size: int = 0, max_blocks: int = 0, n_blocks: int = 0,
                      kv_lens_host: Optional[Sequence[int]] = None, lse=None, workspace=None,
                      num_splits: int = 0, events=None, stream=None) -> int:
    """Attention over the latent cache for an absorbed query given by the caller
    (q_abs [B, n_q, h, d_c] fp32); writes the merged latent output o_lat [B, n_q, h, d_c]."""
    B, n_q = q_abs.shape[0], q_abs.shape[1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    common = dict(batch=B, n_q=n_q, kv_lens=kv_lens, kv_lens_host=kv_lens_host, max_kv_len=max_kv_len,
                  q_nope=q_abs, q_rope=q_rope, packed_w=None, gate_x=None, w_gate=None, out=o_lat, lse=lse,
                  num_splits=num_splits, events=events)

    def query():
        a, n, _h = _decode_args(workspace=None, workspace_bytes=0, **common)
        _check(lib().mla_decode_latent(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), ctypes.byref(a), None),
               "mla_decode_latent")
        return n.value

    ws = _workspace_for(query, workspace, q_abs.device)
    a, n, _h = _decode_args(workspace=ws, workspace_bytes=ws.numel() * ws.element_size(), **common)
    return _check(lib().mla_decode_latent(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), ctypes.byref(a),
                                          _stream(stream)), "mla_decode_latent")


def mla_expand_kv(d: mla_dims, cache, *, kv_lens, max_kv_len: int, w_uk, w_uv, k_out, v_out, batch: int,
                  t_max: int = 0, block_table=None, block_size: int = 0, max_blocks: int = 0, n_blocks: int = 0,
                  workspace=None, stream=None) -> int:
    """Explicit per-head K and V (fp32) of every cached token: the non-absorbed form."""
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)

    def query():
        n = ctypes.c_size_t(0)
        _check(lib().mla_expand_kv(ctypes.byref(d), None, ctypes.byref(layout), batch, None, max_kv_len, None,
                                   None, None, None, None, ctypes.byref(n), None), "mla_expand_kv")
        return n.value

    ws = _workspace_for(query, workspace, w_uk.device)
    n = ctypes.c_size_t(ws.numel() * ws.element_size())
    return _check(lib().mla_expand_kv(ctypes.byref(d), _ptr(cache), ctypes.byref(layout), batch, _ptr(kv_lens),
                                      max_kv_len, _ptr(w_uk), _ptr(w_uv), _ptr(k_out), _ptr(v_out), _ptr(ws),
                                      ctypes.byref(n), _stream(stream)), "mla_expand_kv")


def mla_decode_explicit(d: mla_dims, k, v, cache, *, kv_lens, max_kv_len: int, q_nope, q_rope, out,
                        t_max: int = 0, block_table=None, block_size: int = 0, max_blocks: int = 0,
                        n_blocks: int = 0, kv_lens_host: Optional[Sequence[int]] = None, gate_x=None,
                        w_gate=None, lse=None, workspace=None, num_splits: int = 0, events=None,
                        stream=None) -> int:
    """Standard attention over explicit per-head K and V (the non-absorbed decode)."""
    B, n_q = q_nope.shape[0], q_nope.shape[1]
    layout = mla_cache_layout(_ptr(block_table), t_max, block_size, max_blocks, n_blocks)
    common = dict(batch=B, n_q=n_q, kv_lens=kv_lens, kv_lens_host=kv_lens_host, max_kv_len=max_kv_len,
                  q_nope=q_nope, q_rope=q_rope, packed_w=None, gate_x=gate_x, w_gate=w_gate, out=out, lse=lse,
                  num_splits=num_splits, events=events)

    def query():
        a, n, _h = _decode_args(workspace=None, workspace_bytes=0, **common)
        _check(lib().mla_decode_explicit(ctypes.byref(d), None, None, None, ctypes.byref(layout), ctypes.byref(a),
                                         None), "mla_decode_explicit")
        return n.value

    ws = _workspace_for(query, workspace, q_nope.device)
    a, n, _h = _decode_args(workspace=ws, workspace_bytes=ws.numel() * ws.element_size(), **common)
    return _check(lib().mla_decode_explicit(ctypes.byref(d), _ptr(k), _ptr(v), _ptr(cache), ctypes.byref(layout),
                                            ctypes.byref(a), _stream(stream)), "mla_decode_explicit")


def decode_workspace_bytes(d: mla_dims, *, batch: int, n_q: int, max_kv_len: int,
                           kv_lens_host=None, gated: bool = False, num_splits: int = 0,
                           paged: bool = False, block_size: int = 64) -> int:
    """Workspace the decode call needs (pure host arithmetic; no device access)."""
    a, n, _h = _decode_args(batch=batch, n_q=n_q, kv_lens=None, kv_lens_host=kv_lens_host,
                            max_kv_len=max_kv_len, q_nope=None, q_rope=None, packed_w=None,
                            gate_x=None, w_gate=None, out=None, lse=None, workspace=None,
                            workspace_bytes=0, num_splits=num_splits, events=None)
    if gated:
        a.gate_x = 1  # only its presence matters for the size
        a.w_gate = 1
        a.d_model = 4096
    if paged:
        mb = (max_kv_len + block_size - 1) // block_size
        st = lib().mla_decode_paged(ctypes.byref(d), None, None, block_size, mb, mb, ctypes.byref(a), None)
    else:
        st = lib().mla_decode(ctypes.byref(d), None, max_kv_len, ctypes.byref(a), None)
    _check(st, "decode_workspace_bytes")
    return n.value
