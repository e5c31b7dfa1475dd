"""The allocation-free decode, mla_decode_noalloc, through the C ABI: it runs the
same kernels as mla_decode / mla_decode_paged with the library's own per-GPU
scratch array as the workspace, so its outputs must equal theirs bit for bit. Two
calls in a row, the second with a smaller input (the array keeps the first call's
contents), then a call too large for the array, rejected on the host."""
import ctypes

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_latent_kv_41_amd import mla, synth  # noqa: E402
from mla_latent_kv_41_amd.harness import GpuStep  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    mla.lib()


def noalloc(step, out, lse):
    w = step.w
    kw = dict(kv_lens=step.kv_lens, max_kv_len=w.kv_max, q_nope=step.q_nope, q_rope=step.q_rope,
              packed_w=step.packed, out=out, lse=lse, kv_lens_host=step.kv_lens_host,
              gate_x=step.gate_x, w_gate=step.w_gate)
    if w.paged:
        mla.mla_decode_noalloc(step.dims, step.pool, block_table=step.block_table, block_size=w.block_size,
                               max_blocks=w.max_blocks, n_blocks=step.n_blocks, **kw)
    else:
        mla.mla_decode_noalloc(step.dims, step.cache, t_max=step.t_max, **kw)


def compare(w, with_oracle):
    print("case %s B=%d n_q=%d kv=[%d..%d] paged=%s" % (w.name, w.batch, w.n_q, w.kv_lens.min(),
                                                        w.kv_lens.max(), w.paged), flush=True)
    t = synth.draw(w)
    step = GpuStep(w, t)
    ref = step.decode().clone()
    ref_lse = step.lse.clone()
    out = torch.full_like(ref, float("nan"))
    lse = torch.full_like(ref_lse, float("nan"))
    noalloc(step, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "output differs from the workspace call"
    assert torch.equal(lse, ref_lse), "lse differs from the workspace call"
    if with_oracle:
        o = oracle.mla_decode(h=w.h, d_c=w.d_c, d_r=w.d_r, d_n=w.d_n, d_v=w.d_v, c_kv=t["c_kv"],
                              k_r=t["k_r"], kv_lens=w.kv_lens, q_nope=t["q_nope"], q_r=t["q_r"],
                              w_uk=t["w_uk"], w_uv=t["w_uv"], x=t.get("x"), w_g=t.get("w_g"),
                              store_bf16=True)
        g = out.cpu().numpy().astype(np.float64)
        err = np.max(np.abs(g - o)) / np.sqrt(np.mean(o ** 2))
        print("  against the oracle: max-abs / rms %.4f" % err, flush=True)
        assert err <= 2e-2


def test_noalloc_equals_the_workspace_call_twice():
    # 1: the DeepSeek-shaped step (contiguous, fast form, about 38 MB of workspace)
    compare(synth.make_workload(2), with_oracle=False)
    # 2: smaller, paged and ragged, both attention forms (lengths on both sides of
    #    4096), two queries per sequence
    w = synth.make_workload(4, batch=3, ctx_range=(0, 10))
    w.kv_lens = np.array([300, 5000, 4100], np.int32)
    w.pool_blocks, w.block_table = synth._paged_table(w.seed, w.kv_lens, 64)
    compare(w, with_oracle=True)


def test_noalloc_rejects_a_call_past_its_scratch():
    d = mla.dims(128, 512, 64, 128, 128, mla.MLA_BF16)
    lay = mla.mla_cache_layout(None, 65537, 0, 0, 0)
    a, n, _h = mla._decode_args(batch=64, n_q=1, kv_lens=None, kv_lens_host=None, max_kv_len=65537,
                                q_nope=None, q_rope=None, packed_w=None, gate_x=None, w_gate=None,
                                out=None, lse=None, workspace=None, workspace_bytes=0, num_splits=0,
                                events=None)
    st = mla.lib().mla_decode_noalloc(ctypes.byref(d), None, ctypes.byref(lay), ctypes.byref(a), None)
    assert st == mla.MLA_E_WORKSPACE
