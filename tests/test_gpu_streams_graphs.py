"""The decode on several streams at once and under HIP graph capture.

The library keeps no state between calls, so decodes of different layers on two
streams at once give the same bits as one at a time. A decode step captured into
a graph (its workspace allocated beforehand; the path launches kernels only, no
memset) replays to the eager result; the replays are interleaved with other
eager decodes and synchronisations, and every replay is checked. Streams keep
the default priority."""
import sys

import numpy as np
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def two_layers():
    wa = synth.make_workload(2, batch=4, ctx=1500)
    wb = synth.make_workload(4, batch=3, ctx_range=(300, 1200), seed=777)   # paged, two queries
    a, b = GpuStep(wa, synth.draw(wa)), GpuStep(wb, synth.draw(wb))
    ra, rb = a.decode().clone(), b.decode().clone()     # also allocates the workspaces
    torch.cuda.synchronize()
    return a, b, ra, rb


def test_two_streams_at_once_match_one_at_a_time():
    say("two streams")
    a, b, ra, rb = two_layers()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        a.out.fill_(float("nan"))
        b.out.fill_(float("nan"))
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            a.decode(stream=s1)
        with torch.cuda.stream(s2):
            b.decode(stream=s2)
        torch.cuda.synchronize()
        assert torch.equal(a.out, ra), rep
        assert torch.equal(b.out, rb), rep


def test_graph_replays_match_the_eager_decode():
    say("graph capture")
    a, b, ra, rb = two_layers()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        a.decode()                                      # warm-up on the capture's side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        a.decode()
    torch.cuda.synchronize()
    for rep in range(4):
        a.out.fill_(float("nan"))
        b.out.fill_(float("nan"))
        b.decode()                                      # other eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(a.out, ra), rep
        assert torch.equal(b.out, rb), rep
        say("  replay %d matches" % rep)


def test_graph_of_a_serving_step_with_the_fused_append():
    """One serving step as a graph: the new token's latent from its hidden state
    (mla_project_append) into the cache, then the decode over the grown cache. Each
    replay follows a fresh hidden state copied into the captured input buffer and
    matches the same two calls run eagerly on an identical copy of the layer."""
    from mla_latent_kv_41_amd.harness import to_device
    say("graph of a serving step")
    w = synth.make_workload(2, batch=4, ctx=800)
    t = synth.draw(w)
    g_step, e_step = GpuStep(w, t), GpuStep(w, t)         # captured copy, eager copy
    wp = synth.make_projection("deepseek", batch=4, pos=800)  # the new token's slot
    tp = synth.draw_projection(wp)
    d = mla.dims(128, 512, 64, 128, 128, mla.MLA_BF16)
    packed = torch.empty(mla.mla_pack_down_weights(d, wp.d_model), dtype=torch.uint8, device="cuda")
    mla.mla_pack_down_weights(d, wp.d_model, to_device(tp["w_dkv"]), to_device(tp["w_kr"]), packed)
    gain = to_device(tp["gain"])
    pos0 = torch.full((4,), 800, dtype=torch.int32, device="cuda")
    hidden = torch.empty((4, 1, wp.d_model), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mla.project_workspace_bytes(d, batch=4, n_new=1, d_model=wp.d_model),
                     dtype=torch.uint8, device="cuda")

    def serve(step):
        mla.mla_project_append(d, step.cache, hidden=hidden, packed_down=packed, pos0=pos0, norm_gain=gain,
                               norm_eps=wp.eps, t_max=step.t_max, workspace=ws)
        step.decode()

    hidden.copy_(to_device(synth.normal(5, "serve_hidden", (4, 1, wp.d_model), 1.0, "bf16")))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        serve(g_step)                                   # warm-up; allocates the decode workspace
    torch.cuda.current_stream().wait_stream(side)
    e_step.decode()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        serve(g_step)
    torch.cuda.synchronize()
    for rep in range(3):
        hidden.copy_(to_device(synth.normal(100 + rep, "serve_hidden", (4, 1, wp.d_model), 1.0, "bf16")))
        torch.cuda.synchronize()
        g_step.out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        serve(e_step)                                   # the same step, eagerly
        torch.cuda.synchronize()
        assert torch.equal(g_step.cache[:, 800], e_step.cache[:, 800]), rep
        assert torch.equal(g_step.out, e_step.out), rep
        say("  replay %d matches" % rep)
