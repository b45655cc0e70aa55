"""Pins of oracle/quant.py: hand-worked groups and rows, exhaustive
nearest-value checks of every element, idempotence and round-trip bounds."""
import numpy as np

from oracle import formats as F
from oracle import quant as Q
from tests._golden import table


def _bf16(vals):
    return F.f64_to_bf16_rne(np.asarray(vals, dtype=np.float64))


def _check_fixture(name, given):
    t = table(name)
    x = _bf16([[float(v) for v in t["values"]]])
    codes, scales, ts = Q.nvfp4_encode(x, tscale=np.float32(1.0) if given else None)
    assert ts == np.float32(float(t["tscale"][0]))
    assert scales.ravel().tolist() == [int(v, 16) for v in t["scales"]]
    assert codes.ravel().tolist() == [int(v, 16) for v in t["packed"]]


def test_nvfp4_worked_dynamic_scale():
    _check_fixture("nvfp4_group.txt", given=False)


def test_nvfp4_worked_given_scale():
    _check_fixture("nvfp4_given.txt", given=True)


def test_nvfp4_reciprocal_reading():
    _check_fixture("nvfp4_recip.txt", given=True)


def test_int8_worked_row():
    t = table("int8_row.txt")
    q, s = Q.int8_encode(_bf16([[float(v) for v in t["values"]]]))
    assert s[0] == np.float32(float(t["scale"][0]))
    assert q.ravel().tolist() == [int(v) for v in t["q"]]


def _rand_bf16(rng, shape, outliers=0, mult=1.0):
    x = rng.standard_normal(shape)
    if outliers:
        cols = rng.choice(shape[1], outliers, replace=False)
        x[:, cols] *= mult
    return _bf16(x)


def test_nvfp4_each_element_is_nearest_grid_point():
    # independent check of steps 3-5: for every element, the chosen code is
    # the nearest E2M1 value to x*inv (exhaustive distance, ties to even),
    # with inv recomputed from the stored scale; scales are the nearest E4M3
    rng = np.random.default_rng(21)
    x = _rand_bf16(rng, (64, 256), outliers=4, mult=20.0)
    codes, scales, st = Q.nvfp4_encode(x)
    xf = F.bf16_to_f32(x)
    assert st == np.float32(np.max(np.abs(xf)) / np.float32(2688))
    g = np.float32(1) / (np.float32(6) * st)
    amax_g = np.abs(xf).reshape(64, 16, 16).max(axis=2)
    sc = (amax_g * g).astype(np.float32).astype(np.float64)
    dist = np.abs(sc[..., None] - F.E4M3_VAL)
    assert np.all(dist[np.arange(64)[:, None], np.arange(16)[None, :], scales] <= dist.min(-1))
    d = (F.e4m3_decode(scales).astype(np.float32) * st).astype(np.float32)
    inv = np.float32(1) / d
    y = (xf.reshape(64, 16, 16) * inv[..., None]).astype(np.float32).astype(np.float64)
    c = Q.nvfp4_unpack(codes).reshape(64, 16, 16)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    dist = np.abs(np.abs(y)[..., None] - grid)
    chosen = dist[..., :][np.arange(64)[:, None, None], np.arange(16)[None, :, None],
                          np.arange(16)[None, None, :], c & 7]
    assert np.all(chosen <= dist.min(-1))
    assert np.all(((c & 8) != 0) == np.signbit(y))


def test_nvfp4_idempotent_power_of_two_scale():
    rng = np.random.default_rng(3)
    x = F.bf16_to_f32(_rand_bf16(rng, (32, 128), outliers=2, mult=30.0))
    for st in (np.float32(2.0 ** -4), np.float32(2.0 ** -2)):
        c1, s1, _ = Q.nvfp4_encode_f32(x, tscale=st)
        xhat = Q.nvfp4_decode(c1, s1, st)
        assert np.array_equal(xhat.astype(np.float32).astype(np.float64), xhat)
        c2, s2, _ = Q.nvfp4_encode_f32(xhat.astype(np.float32), tscale=st)
        np.testing.assert_array_equal(c1, c2)
        np.testing.assert_array_equal(s1, s2)


def test_nvfp4_idempotent_dynamic_scale():
    rng = np.random.default_rng(4)
    x = F.bf16_to_f32(_rand_bf16(rng, (32, 128)))
    c1, s1, t1 = Q.nvfp4_encode_f32(x)
    xhat = Q.nvfp4_decode(c1, s1, t1).astype(np.float32)
    c2, s2, t2 = Q.nvfp4_encode_f32(xhat)
    assert abs(float(t2) - float(t1)) <= float(np.spacing(t1))
    np.testing.assert_array_equal(s1, s2)
    np.testing.assert_array_equal(c1, c2)


def test_nvfp4_round_trip_bound():
    # |x - xhat| <= half the local E2M1 step times the group scale
    rng = np.random.default_rng(6)
    x = _rand_bf16(rng, (128, 256), outliers=3, mult=30.0)
    c, s, st = Q.nvfp4_encode(x)
    xhat = Q.nvfp4_decode(c, s, st)
    xf = F.bf16_to_f64(x)
    d = (F.e4m3_decode(s).astype(np.float32) * st).astype(np.float64)
    e = np.abs(F.e2m1_decode(Q.nvfp4_unpack(c))).reshape(128, 16, 16)
    half_step = np.where(e < 2, 0.25, np.where(e < 4, 0.5, 1.0))
    err = np.abs(xf - xhat).reshape(128, 16, 16)
    assert np.all(err <= half_step * d[..., None] * (1 + 2.0 ** -20))


def test_nvfp4_zero_tensor_and_negative_zero():
    x = np.zeros((2, 32), np.uint16)
    x[1, 5] = 0x8000
    c, s, st = Q.nvfp4_encode(x)
    assert st == 0 and not s.any()
    u = Q.nvfp4_unpack(c)
    assert u[1, 5] == 8 and u.sum() == 8


def test_int8_idempotent_and_round_trip():
    rng = np.random.default_rng(8)
    x = _rand_bf16(rng, (64, 512), outliers=5, mult=30.0)
    q, s = Q.int8_encode(x)
    xf = F.bf16_to_f64(x)
    xhat = Q.int8_decode(q, s)
    assert np.all(np.abs(xf - xhat) <= (s.astype(np.float64)[:, None] / 2) * (1 + 2.0 ** -20))
    q2, s2 = Q.int8_encode_f32(xhat.astype(np.float32))
    np.testing.assert_array_equal(q, q2)
    assert np.all(np.abs(s2.astype(np.float64) - s) <= np.spacing(s))


def test_int8_every_bf16_value():
    # all 2^16 bf16 patterns (finite ones), one row each with a fixed amax
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f64(bits)
    bits = bits[np.isfinite(v) & (np.abs(v) <= 1000)]
    rows = np.stack([bits, np.full_like(bits, F.f64_to_bf16_rne(1000.0))], axis=1)
    q, s = Q.int8_encode(rows)
    assert np.all(s == np.float32(1000.0) / np.float32(127))
    inv = np.float32(1) / s[0]
    want = np.clip(np.rint((F.bf16_to_f32(bits) * inv).astype(np.float32)), -127, 127)
    np.testing.assert_array_equal(q[:, 0], want.astype(np.int8))
    # nearest integer (ties to even) of the float32 product, checked exactly
    y = (F.bf16_to_f32(bits) * inv).astype(np.float64)
    assert np.all(np.abs(y - q[:, 0]) <= 0.5)
    tie = np.abs(y - np.trunc(y)) == 0.5
    assert np.all(q[tie, 0] % 2 == 0)


def test_int8_zero_row():
    q, s = Q.int8_encode(np.zeros((1, 16), np.uint16))
    assert s[0] == 0 and not q.any()
