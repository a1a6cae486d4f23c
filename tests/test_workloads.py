"""The seeded input generator (CPU only)."""
import math

import numpy as np

import cssd_workloads as wl


def test_deterministic_and_seed_dependent():
    a = wl.random_forward(7, 2, 33, 3, 16, 32, 16)
    b = wl.random_forward(7, 2, 33, 3, 16, 32, 16)
    c = wl.random_forward(8, 2, 33, 3, 16, 32, 16)
    for name in ("x_re", "x_im", "B_re", "B_im", "C_re", "C_im", "dt", "A_re", "A_im", "Dskip"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
        assert not np.array_equal(getattr(a, name), getattr(c, name)), name
        assert getattr(a, name).dtype == np.float32


def test_config0_recipe():
    inp = wl.config0()
    assert inp.shape == dict(B=1, T=64, H=2, D=16, N=16, C=16)
    assert np.all((inp.A_re <= -0.1) & (inp.A_re >= -1.0))
    assert np.all(np.abs(inp.A_im) <= math.pi)
    assert inp.h0_re is None and inp.Dskip.shape == (2,)


def test_plane_variance_is_one_half():
    inp = wl.random_forward(3, 4, 256, 4, 64, 64, 64)
    for name in ("x_re", "x_im", "B_re", "C_im"):
        v = float(np.var(getattr(inp, name)))
        assert abs(v - 0.5) < 0.01, (name, v)


def test_long_decay_targets():
    H = 48
    a_re = -np.linspace(0.1, 1.0, H).astype(np.float32)
    dt = wl.long_decay_dt(2, (1, 4096, H), a_re)
    mag = np.exp(np.logaddexp(0.0, dt.astype(np.float64)) * a_re.astype(np.float64))
    assert mag.min() >= 0.5 - 1e-5 and mag.max() <= 0.9999 + 1e-5
    assert (mag > 0.999).mean() > 0.1 and (mag < 0.6).mean() > 0.01


def test_round_bf16_ties_to_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1.0 + 2 ** -9], dtype=np.float32)
    got = wl.round_bf16(vals)
    assert got.tolist() == [1.0, 1.0, 1.015625, -2.5, 1.0]
    assert wl.bf16_bits(got).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x3F80]


def test_pam_mapping_shapes():
    p = wl.pam_draw(3, 2, 16, 3, 8)
    assert np.allclose(np.abs(p.K), 1 / math.sqrt(8), rtol=1e-6)
    re = wl.pam_to_scan(p, 8, "re")
    cx = wl.pam_to_scan(p, 8, "complex")
    assert re.shape["N"] == 16 and cx.shape["N"] == 8
    assert re.Dskip is None and np.all(re.A_im == 0)


def test_decode_steps_stack():
    s = wl.decode_steps(4, 3, 2, 3, 16, 32)
    assert s.x_re.shape == (3, 2, 3, 16) and s.B_re.shape == (3, 2, 3, 32) and s.dt.shape == (3, 2, 3)
    one = wl.decode_step(4, 1, 2, 3, 16, 32)
    assert np.array_equal(s.C_im[1], one.C_im)
