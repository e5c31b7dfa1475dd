"""The seeded input generator: deterministic, sliceable, with the stated moments."""
import numpy as np
import torch

from mla_latent_kv_41_amd import synth


def test_streams_are_deterministic_and_sliceable():
    a = synth.normal(1, "x", (1000,), 1.0, "f64")
    b = synth.normal(1, "x", (1000,), 1.0, "f64")
    np.testing.assert_array_equal(a, b)
    tail = synth.normal(1, "x", (400,), 1.0, "f64", start=600)
    np.testing.assert_array_equal(a[600:], tail)
    assert not np.array_equal(a, synth.normal(1, "y", (1000,), 1.0, "f64"))
    assert not np.array_equal(a, synth.normal(2, "x", (1000,), 1.0, "f64"))


def test_normal_moments():
    z = synth.normal(5, "m", (400000,), 1.0, "f64")
    assert abs(z.mean()) < 0.01
    assert abs(z.var() - 1.0) < 0.01
    assert abs(np.mean(z ** 4) - 3.0) < 0.05       # Gaussian kurtosis
    w = synth.normal(5, "w", (200000,), 1.0 / np.sqrt(512), "f64")
    assert abs(w.var() * 512 - 1.0) < 0.02


def test_bf16_draws_are_rounded_to_nearest_even():
    d = synth.normal(9, "b", (5000,), 1.0, "f64")
    bits = synth.normal(9, "b", (5000,), 1.0, "bf16")
    ref = torch.from_numpy(d).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_rmsnorm_rows_have_unit_rms():
    r = synth.rmsnorm_rows(3, "c", 64, 512, "f32")
    rms = np.sqrt(np.mean(r.astype(np.float64) ** 2, axis=1))
    np.testing.assert_allclose(rms, 1.0, rtol=1e-5)
    rb = synth.bf16_bits_to_f64(synth.rmsnorm_rows(3, "c", 64, 512, "bf16"))
    np.testing.assert_allclose(rb, r.astype(np.float64), rtol=2 ** -8, atol=0)


def test_integers_and_permutations():
    v = synth.uniform_int(4, "len", 20000, 512, 16384)
    assert v.min() >= 512 and v.max() <= 16384
    assert abs(v.mean() - (512 + 16384) / 2) < 100
    p = synth.permutation(4, "perm", 2565)
    np.testing.assert_array_equal(np.sort(p), np.arange(2565))


def test_workload_shapes():
    w = synth.make_workload(2)
    assert (w.h, w.d_c, w.d_r, w.d_n, w.d_v, w.batch, w.n_q) == (128, 512, 64, 128, 128, 32, 1)
    assert w.kv_max == 4097 and w.row == 576
    assert w.cache_bytes_visible() == 32 * 4097 * 576 * 2
    w3 = synth.make_workload(3)
    assert w3.paged and w3.max_blocks == 513 and w3.pool_blocks == int(np.ceil(4 * 513 * 1.25))
    used = w3.block_table[w3.block_table >= 0]
    assert len(np.unique(used)) == used.size == 4 * 513
    w4 = synth.make_workload(4)
    assert w4.n_q == 2 and w4.kv_lens.min() >= 514 and w4.kv_lens.max() <= 16386
    w5 = synth.make_workload(5)
    assert w5.gated and w5.d_r == 0 and w5.d_model == 4096 and w5.kv_max == 65537
    w1 = synth.make_workload(1)
    assert w1.dtype == "f32" and w1.scale == 1.0 / np.sqrt(24)
