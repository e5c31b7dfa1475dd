"""GPU parity of the fused latent append (mla_pack_down_weights + mla_project_append,
through the C ABI) against the fp64 oracle on the same seeded inputs.

bf16: each stored element is the oracle's exact value v rounded once to bf16 after
an fp32 computation. The products accumulate in fp32 on the matrix cores and the
up to 32 split partials are added in fp32: at most 32 roundings of a sum of order
the row's scale, each at most 2^-24 of it, so about 2e-6 of the row's RMS (the
latent part and the key part each have their own). The bound checked is
|stored - v| <= ulp_bf16/2 + 1e-5 * RMS (five times that margin), and at least
99% of the elements must carry exactly the bits of v rounded to bf16.
fp32: max-abs <= 1e-5, the fp32 criterion of the tiny layer.
Every slot the call must not write is NaN-poisoned and must stay NaN.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from mla_latent_kv_41_amd import mla, synth  # noqa: E402
from mla_latent_kv_41_amd.harness import bf16_bits, to_device  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm device")
    mla.lib()  # fails loudly when the library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_rows(w, t):
    return oracle.project_latent(hidden=t["hidden"], w_dkv=t["w_dkv"], w_kr=t["w_kr"], gain=t["gain"],
                                 eps=w.eps, pos=w.positions(), rope_base=w.rope_base)


def bits_of(rounded):
    """bf16 bit patterns of values that are already bf16 (exact through fp32)."""
    return (np.asarray(rounded, np.float64).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def run_fused(w, t, k_splits=0, fill=float("nan")):
    """Pack the weights, fill a poisoned cache, run the fused append; returns the cache."""
    dev = "cuda"
    dt = mla.MLA_F32 if w.dtype == "f32" else mla.MLA_BF16
    d = mla.dims(128 if dt == mla.MLA_BF16 else 4, w.d_c, w.d_r, 128 if dt == mla.MLA_BF16 else 16,
                 128 if dt == mla.MLA_BF16 else 16, dt, rope_base=w.rope_base)
    tdt = torch.float32 if dt == mla.MLA_F32 else torch.bfloat16
    w_dkv, w_kr = to_device(t["w_dkv"], dev), to_device(t["w_kr"], dev)
    packed = torch.empty(mla.mla_pack_down_weights(d, w.d_model), dtype=torch.uint8, device=dev)
    mla.mla_pack_down_weights(d, w.d_model, w_dkv, w_kr, packed)
    hidden = to_device(t["hidden"], dev)
    gain = to_device(t["gain"], dev)
    pos0 = torch.from_numpy(w.pos0.astype(np.int32)).to(dev)
    if w.paged:
        cache = torch.full((w.pool_blocks, w.block_size, w.row), fill, dtype=tdt, device=dev)
        table = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)
        mla.mla_project_append(d, cache, hidden=hidden, packed_down=packed, pos0=pos0, norm_gain=gain,
                               norm_eps=w.eps, block_table=table, block_size=w.block_size,
                               max_blocks=w.max_blocks, n_blocks=w.pool_blocks, k_splits=k_splits)
    else:
        cache = torch.full((w.batch, w.t_max, w.row), fill, dtype=tdt, device=dev)
        mla.mla_project_append(d, cache, hidden=hidden, packed_down=packed, pos0=pos0, norm_gain=gain,
                               norm_eps=w.eps, t_max=w.t_max, k_splits=k_splits)
    torch.cuda.synchronize()
    return cache


def written_rows(w, cache):
    """The rows of the new tokens, [batch * n_new, row], plus a mask of every slot."""
    slots = []
    for b in range(w.batch):
        for j in range(w.n_new):
            p = int(w.pos0[b]) + j
            if w.paged:
                slots.append(int(w.block_table[b, p // w.block_size]) * w.block_size + p % w.block_size)
            else:
                slots.append(b * w.t_max + p)
    flat = cache.reshape(-1, w.row)
    idx = torch.tensor(slots, dtype=torch.long, device=cache.device)
    keep = torch.ones(flat.shape[0], dtype=torch.bool, device=cache.device)
    keep[idx] = False
    return flat[idx], flat[keep]


def ulp_bf16(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def row_scale(ref, d_c):
    """RMS of each row's latent part and key part, broadcast to the elements."""
    s = np.empty_like(ref)
    s[:, :d_c] = np.sqrt(np.mean(ref[:, :d_c] ** 2, axis=1, keepdims=True))
    if ref.shape[1] > d_c:
        s[:, d_c:] = np.sqrt(np.mean(ref[:, d_c:] ** 2, axis=1, keepdims=True))
    return s


def within_bound(got_bits, ref, d_c, what):
    got = synth.bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref)
    tol = 0.5 * ulp_bf16(np.maximum(np.abs(got), np.abs(ref))) + 1e-5 * row_scale(ref, d_c)
    worst = np.unravel_index(int(np.argmax(err / tol)), err.shape)
    say("  %s: worst err/bound %.3f at %s (value %.6e, err %.3e)"
        % (what, float((err / tol)[worst]), worst, ref[worst], err[worst]))
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= tol), what


def check_bf16_rows(w, cache, ref, what):
    rows, rest = written_rows(w, cache)
    assert bool(torch.isnan(rest.float()).all()), what + ": a slot outside the new rows was written"
    got = bf16_bits(rows)
    want = bits_of(oracle.round_bf16_array(ref))
    same = float(np.mean(got == want))
    say("  %s: %d values, %.4f%% bit-identical" % (what, got.size, 100 * same))
    within_bound(got, ref, w.d_c, what)
    assert same >= 0.99, what
    return got


def test_fused_append_deepseek_shape():
    """B = 32 new tokens, d_model = 4096, d_c + d_rope = 576, written at slot 4096:
    the launch configuration the benchmark times."""
    w = synth.make_projection("deepseek")
    t = synth.draw_projection(w)
    say("fused append deepseek: B=%d d_model=%d" % (w.batch, w.d_model))
    cache = run_fused(w, t)
    check_bf16_rows(w, cache, oracle_rows(w, t), "deepseek")


def test_fused_append_paged_ragged_positions_several_tokens():
    """Paged pool, random positions, 3 new tokens per sequence (60 rows: two row
    blocks of the product with a ragged tail)."""
    w = synth.make_projection("deepseek", batch=20, n_new=3, pos_range=(0, 3000), paged=True)
    t = synth.draw_projection(w)
    say("fused append paged: rows=%d pool=%d" % (w.rows, w.pool_blocks))
    cache = run_fused(w, t)
    check_bf16_rows(w, cache, oracle_rows(w, t), "paged")


def test_fused_append_without_rope():
    w = synth.make_projection("nope")
    t = synth.draw_projection(w)
    say("fused append d_rope=0: B=%d" % w.batch)
    cache = run_fused(w, t)
    check_bf16_rows(w, cache, oracle_rows(w, t), "nope")


@pytest.mark.parametrize("d_model,k_splits", [(2048, 0), (4096 + 16, 0), (1024, 1), (4096, 4), (4096, 16),
                                               (16384, 0)])
def test_fused_append_widths_and_splits(d_model, k_splits):
    """Other widths and forced split counts (one split with a 16-row tail chunk
    at 4112; 4, 16 and the default 32 at 4096; 512-row splits at 16384): all
    within the bound."""
    w = synth.make_projection("deepseek", batch=5, n_new=2, d_model=d_model, pos_range=(0, 500))
    t = synth.draw_projection(w)
    say("fused append d_model=%d k_splits=%d" % (d_model, k_splits))
    cache = run_fused(w, t, k_splits=k_splits)
    check_bf16_rows(w, cache, oracle_rows(w, t), "d_model %d splits %d" % (d_model, k_splits))


def test_fused_append_split_count_changes_little():
    """The same rows with 1 and 32 splits differ only by the summation order: each
    is within the bound of the oracle, and they agree on at least 99% of the bits."""
    w = synth.make_projection("deepseek", batch=8, pos_range=(0, 100))
    t = synth.draw_projection(w)
    ref = oracle_rows(w, t)
    a = bf16_bits(written_rows(w, run_fused(w, t, k_splits=1))[0])
    b = bf16_bits(written_rows(w, run_fused(w, t, k_splits=32))[0])
    within_bound(a, ref, w.d_c, "1 split")
    within_bound(b, ref, w.d_c, "32 splits")
    same = float(np.mean(a == b))
    say("  splits 1 vs 32: %.4f%% identical" % (100 * same))
    assert same >= 0.99


def test_fused_append_tiny_fp32():
    say("fused append tiny fp32")
    for paged in (False, True):
        wp = synth.make_projection("tiny", batch=3, n_new=2, pos_range=(0, 70), paged=paged)
        t = synth.draw_projection(wp)
        cache = run_fused(wp, t)
        rows, rest = written_rows(wp, cache)
        assert bool(torch.isnan(rest).all())
        ref = oracle_rows(wp, t)
        err = float(np.max(np.abs(rows.cpu().numpy().astype(np.float64) - ref)))
        say("  paged=%s: max-abs %.3e (limit 1e-5)" % (paged, err))
        assert err <= 1e-5


def test_fused_append_feeds_the_decode():
    """A token appended from its hidden state is attended to like any other. Each
    sequence's token 0 is replaced by a fused-append row (position 0, where RoPE is
    the identity, so the row's stored k_R is also its unrotated k_R); the decode over
    64 tokens then matches the oracle decode given that row's bits as token 0."""
    from mla_latent_kv_41_amd.harness import GpuStep
    wd = synth.make_workload(2, batch=4, ctx=63)
    td = synth.draw(wd)
    wp = synth.make_projection("deepseek", batch=4, pos=0)
    tp = synth.draw_projection(wp)
    say("fused append then decode: B=4, 64 tokens")
    step = GpuStep(wd, td)
    fused = run_fused(wp, tp)                         # [4, 1, 576], the rows at slot 0
    step.cache[:, 0] = fused[:, 0]
    out = step.decode().cpu().numpy()
    torch.cuda.synchronize()
    bits = bits_of(oracle.round_bf16_array(oracle_rows(wp, tp)))
    c_kv, k_r = td["c_kv"].copy(), td["k_r"].copy()
    c_kv[:, 0] = bits[:, :512]
    k_r[:, 0] = bits[:, 512:]
    ref = oracle.mla_decode(h=wd.h, d_c=wd.d_c, d_r=wd.d_r, d_n=wd.d_n, d_v=wd.d_v, c_kv=c_kv, k_r=k_r,
                            kv_lens=wd.kv_lens, q_nope=td["q_nope"], q_r=td["q_r"],
                            w_uk=td["w_uk"], w_uv=td["w_uv"], store_bf16=True)
    err = float(np.max(np.abs(out - ref)))
    rms = float(np.sqrt(np.mean(ref * ref)))
    say("  decode over fused rows: max-abs %.3e, rms %.3e" % (err, rms))
    assert err <= 2e-2 * rms


def test_fused_append_skips_rows_outside_the_cache():
    """Rows whose position is negative or past the cache, or whose block-table entry
    is -1 or past the pool, are skipped: the kernels' own range checks, no access
    outside the buffers. Every other row is written as usual."""
    say("fused append out-of-range rows")
    # contiguous: t_max = 64; sequence 1 starts at 63 (its second token falls off the
    # end), sequence 2 at -1 (its first token is skipped), sequence 3 far past the end
    w = synth.make_projection("deepseek", batch=4, n_new=2, pos=0)
    w.pos0 = np.array([10, 63, -1, 500], np.int32)
    t = synth.draw_projection(w)
    ref = oracle.round_bf16_array(oracle_rows(w, t))
    d = mla.dims(128, w.d_c, w.d_r, 128, 128, mla.MLA_BF16)
    packed = torch.empty(mla.mla_pack_down_weights(d, w.d_model), dtype=torch.uint8, device="cuda")
    mla.mla_pack_down_weights(d, w.d_model, to_device(t["w_dkv"]), to_device(t["w_kr"]), packed)
    cache = torch.full((4, 64, w.row), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_project_append(d, cache, hidden=to_device(t["hidden"]), packed_down=packed,
                           pos0=torch.from_numpy(w.pos0).cuda(), norm_gain=to_device(t["gain"]),
                           norm_eps=w.eps, t_max=64)
    torch.cuda.synchronize()
    written = {(0, 10): 0, (0, 11): 1, (1, 63): 2, (2, 0): 5}   # (b, slot) -> oracle row
    flat = cache.float().cpu().numpy()
    for b in range(4):
        for s_ in range(64):
            if (b, s_) in written:
                got = synth.bf16_bits_to_f64(bf16_bits(cache[b, s_]))
                np.testing.assert_allclose(got, ref[written[(b, s_)]], rtol=0.0079, atol=1e-4)
            else:
                assert np.isnan(flat[b, s_]).all(), (b, s_)
    # paged: table rows with a -1 entry and an id past the pool
    wp = synth.make_projection("deepseek", batch=3, n_new=1, pos=0, paged=True)
    wp.pos0 = np.array([5, 70, 130], np.int32)
    pool_blocks = 4
    table = np.array([[1, 2, 0], [3, -1, 0], [2, 0, 9]], np.int32)  # seq 1 -> -1, seq 2 -> 9 >= pool
    tp = synth.draw_projection(wp)
    refp = oracle.round_bf16_array(oracle_rows(wp, tp))
    pool = torch.full((pool_blocks, 64, wp.row), float("nan"), dtype=torch.bfloat16, device="cuda")
    mla.mla_project_append(d, pool, hidden=to_device(tp["hidden"]), packed_down=packed,
                           pos0=torch.from_numpy(wp.pos0).cuda(), norm_gain=to_device(tp["gain"]),
                           norm_eps=wp.eps, block_table=torch.from_numpy(table).cuda(), block_size=64,
                           max_blocks=3, n_blocks=pool_blocks)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f64(bf16_bits(pool[1, 5]))
    np.testing.assert_allclose(got, refp[0], rtol=0.0079, atol=1e-4)
    rest = pool.float().reshape(-1, wp.row)
    keep = torch.ones(rest.shape[0], dtype=torch.bool)
    keep[1 * 64 + 5] = False
    assert bool(torch.isnan(rest[keep.cuda()]).all())


def test_decode_loop_with_fused_append():
    """Three decode steps in a row, as a serving loop runs them: each step appends
    every sequence's new token from its hidden state at position kv_len - 1 (paged
    cache, ragged lengths), then decodes over the grown cache. Each step's output
    matches the oracle decode over the same tokens, given in fp64: the drawn ones
    widened exactly, each new token's latent as the oracle's fused append stores it
    (rounded to bf16) and its key unrotated and unrounded, which the oracle decode
    rotates at the token's position and rounds, as the cache does."""
    from mla_latent_kv_41_amd.harness import GpuStep
    B, steps = 4, 3
    wd = synth.make_workload(4, batch=B, ctx_range=(300, 600))  # paged, ragged
    wd.n_q = 1
    base = (wd.kv_lens - 2 + 1).astype(np.int64)                 # lengths before the loop, one query
    bs = wd.block_size
    need = (base + steps + bs - 1) // bs
    pool = int(need.sum()) + 2
    table = np.full((B, int(need.max())), -1, np.int32)
    perm = synth.permutation(7, "loop_table", pool)
    k = 0
    for b in range(B):
        table[b, :need[b]] = perm[k:k + need[b]]
        k += int(need[b])
    wd.block_table, wd.pool_blocks = table, pool
    wd.kv_lens = (base + steps).astype(np.int32)                  # sizes the buffers
    td = synth.draw(wd)
    say("decode loop: B=%d, lengths %s, %d steps" % (B, list(base), steps))
    step = GpuStep(wd, td)            # appends drawn tokens 0 .. base + steps - 1
    d = mla.dims(128, 512, 64, 128, 128, mla.MLA_BF16)
    wp = synth.make_projection("deepseek", batch=B, pos=0)
    tp = synth.draw_projection(wp)
    packed = torch.empty(mla.mla_pack_down_weights(d, wp.d_model), dtype=torch.uint8, device="cuda")
    mla.mla_pack_down_weights(d, wp.d_model, to_device(tp["w_dkv"]), to_device(tp["w_kr"]), packed)
    gain = to_device(tp["gain"])
    f64 = synth.bf16_bits_to_f64
    c_ref, k_ref = f64(td["c_kv"]), f64(td["k_r"])
    q_nope, q_r, w_uk, w_uv = f64(td["q_nope"]), f64(td["q_r"]), f64(td["w_uk"]), f64(td["w_uv"])
    for s in range(steps):
        lens = base + s + 1                                        # the new token at lens - 1
        hid = synth.normal(41100 + s, "loop_hidden", (B, 1, wp.d_model), 1.0, "bf16")
        pos0 = (lens - 1).astype(np.int32)
        mla.mla_project_append(d, step.pool, hidden=to_device(hid), packed_down=packed,
                               pos0=torch.from_numpy(pos0).cuda(), norm_gain=gain, norm_eps=wp.eps,
                               block_table=step.block_table, block_size=bs, max_blocks=table.shape[1],
                               n_blocks=pool)
        # at position 0 RoPE is the identity: the key part is the unrotated projection
        rows = oracle.project_latent(hidden=hid, w_dkv=tp["w_dkv"], w_kr=tp["w_kr"], gain=tp["gain"],
                                     eps=wp.eps, pos=np.zeros(B, np.int64))
        for b in range(B):
            c_ref[b, lens[b] - 1] = oracle.round_bf16_array(rows[b, :512])
            k_ref[b, lens[b] - 1] = rows[b, 512:]
        step.kv_lens = torch.from_numpy(lens.astype(np.int32)).cuda()
        step.kv_lens_host = [int(v) for v in lens]
        out = step.decode().cpu().numpy()
        torch.cuda.synchronize()
        ref = oracle.mla_decode(h=128, d_c=512, d_r=64, d_n=128, d_v=128, c_kv=c_ref, k_r=k_ref,
                                kv_lens=lens.astype(np.int32), q_nope=q_nope, q_r=q_r, w_uk=w_uk,
                                w_uv=w_uv, store_bf16=True)
        err = float(np.max(np.abs(out - ref)))
        rms = float(np.sqrt(np.mean(ref * ref)))
        say("  step %d: max-abs %.3e, rms %.3e, ratio %.4f" % (s, err, rms, err / rms))
        assert err <= 2e-2 * rms, s
