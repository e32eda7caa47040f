"""The seeded input generators (shared by both sides, no adapter arithmetic)."""

import numpy as np
import pytest

import synth


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0,
                                  65504.0, 1e-30], np.float32)])
    mine = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(mine, ref.view(np.uint16))
    back = synth.bf16_bits_to_f32(mine)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16)
                          .to(torch.float32).numpy())


@pytest.mark.parametrize("bits,group", [(4, 64), (3, 128), (2, 64)])
def test_rtn_error_within_half_step(bits, group):
    rng = np.random.default_rng(bits)
    w = (0.02 * rng.standard_normal((8, 256))).astype(np.float32)
    wq = synth.rtn_quantize(w, bits, group)
    g = w.reshape(8, -1, group)
    s = (g.max(2) - g.min(2)) / (2 ** bits - 1)
    err = (w - wq).reshape(8, -1, group)
    # min/max RTN never clips: every error is within half a step (plus fp32
    # rounding of the reconstruction)
    assert np.all(np.abs(err) <= s[..., None] * (0.5 + 1e-5))
    # the reconstruction has at most 2^b distinct levels per group
    for i in range(8):
        for q in range(g.shape[1]):
            assert len(np.unique(wq.reshape(8, -1, group)[i, q])) <= 2 ** bits


def test_layer_is_deterministic_and_shaped():
    spec = synth.config_specs("c1")[0]
    a = synth.make_layer(spec, seed=0)
    b = synth.make_layer(spec, seed=0)
    assert np.array_equal(a.dwq, b.dwq)
    assert a.dwq.shape == (256, 256) and a.dwq.dtype == np.float32
    n_out = int(np.sum(np.abs(a.w0) > 0.02 * 6))
    assert n_out > 100          # 0.5% of 65536 = 327 outliers x20
    x, dy = synth.make_activations(spec, seed=0)
    assert x.shape == (64, 256) and x.dtype == np.float32
    assert dy.shape == (64, 256)
    c = synth.make_layer(spec, seed=1)
    assert not np.array_equal(a.dwq, c.dwq)


def test_budgets_of_configs():
    assert synth.config_specs("c2")[0].p == 524288
    assert synth.config_specs("c3")[0].p == 1179648
    assert synth.config_specs("c4")[0].p == 1048576
    ps = [s.p for s in synth.config_specs("c5")]
    assert ps == [524288, 327680, 327680, 524288]


def test_shared_x_stream():
    q, k = synth.config_specs("c5")[:2]
    xq, _ = synth.make_activations(q, 0, T=8, x_stream=0)
    xk, _ = synth.make_activations(k, 0, T=8, x_stream=0)
    assert np.array_equal(xq, xk) and xq.dtype == np.uint16
