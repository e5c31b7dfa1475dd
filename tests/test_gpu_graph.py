"""The decode step under HIP graph capture: a captured step, replayed several times
with eager steps on other inputs between the replays, must give the eager step's
output and lse bit for bit on every replay (the library launches kernels only, no
memsets or allocations, and its merge order is fixed). Through the C ABI."""
import copy
import sys

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from mla_latent_kv_41_amd import mla, synth  # noqa: E402
from mla_latent_kv_41_amd.harness import GpuStep  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    mla.lib()


@pytest.mark.parametrize("cid,kw", [
    (2, dict(batch=4, ctx=1500)),                 # precise form
    (2, dict(batch=2, ctx=5000)),                 # fast form
    (4, dict(batch=6, ctx_range=(200, 6000))),    # paged, ragged, two queries, both forms
    (5, dict(batch=3, ctx=700)),                  # gated, h = 64
])
def test_graph_replays_match_the_eager_step(cid, kw):
    w = synth.make_workload(cid, **kw)
    print("graph case %d B=%d kv=[%d..%d]" % (cid, w.batch, w.kv_lens.min(), w.kv_lens.max()), flush=True)
    sys.stdout.flush()
    step = GpuStep(w, synth.draw(w))
    w2 = copy.copy(w)
    w2.seed = w.seed + 1
    other = GpuStep(w2, synth.draw(w2))           # different inputs, same shapes
    step.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse = step.out.clone(), step.lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.decode()
    torch.cuda.synchronize()
    for r in range(4):
        step.out.fill_(float("nan"))
        step.lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, ref_out), "replay %d: out" % r
        assert torch.equal(step.lse, ref_lse), "replay %d: lse" % r
        other.decode()                            # eager work between replays
        torch.cuda.synchronize()
        assert not torch.equal(other.out, ref_out)
