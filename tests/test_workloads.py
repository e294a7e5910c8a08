"""The seeded input generators: deterministic, the stated shapes and distributions, bf16-exact."""
import numpy as np

from exact_flow_delta_amd import workloads as W


def test_deterministic_and_salted():
    w = W.workload(3, B=1, H=2, L=64)
    a = W.make_fwd_inputs(w)
    b = W.make_fwd_inputs(w)
    c = W.make_fwd_inputs(w, salt=1)
    for name in ("q", "k", "v", "beta"):
        np.testing.assert_array_equal(a[name], b[name])
        assert not np.array_equal(a[name], c[name])


def test_bf16_rounding_is_rne_and_exact():
    x = np.array([1.0, 1.00390625, 1.005859375, -3.3, 1e-30, 65504.0], dtype=np.float32)
    r = W.round_bf16(x)
    # representable: low 16 bits are zero, and rounding is idempotent
    assert np.all((r.view(np.uint32) & 0xFFFF) == 0)
    np.testing.assert_array_equal(W.round_bf16(r), r)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: ties go to the even mantissa (1.0)
    assert r[1] == np.float32(1.0)
    assert r[2] == np.float32(1.0078125)
    assert np.max(np.abs(r - x) / np.abs(x)) <= 2.0 ** -8
    bits = W.bf16_bits(r)
    back = (bits.view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(back, r)


def test_shapes_and_dtypes():
    for cid, over in [(1, {}), (2, dict(B=1, H=2, L=128)), (3, dict(B=1, H=2, L=128)), (4, dict(H=2, L=256))]:
        w = W.workload(cid, **over)
        x = W.make_fwd_inputs(w)
        assert x["q"].shape == (w.B, w.H, w.L, w.d_k) and x["q"].dtype == np.float32
        assert x["v"].shape == (w.B, w.H, w.L, w.d_v)
        assert x["beta"].shape == (w.B, w.H, w.L) and np.all((x["beta"] > 0) & (x["beta"] < 1))
        if w.dtype == "bf16":
            for n in ("q", "k", "v"):
                np.testing.assert_array_equal(W.round_bf16(x[n]), x[n])
        assert (x["initial_state"] is not None) == (cid == 2)


def test_stiff_workload_spans_lambda_range():
    w = W.workload(2, B=1, H=4, L=2048)
    x = W.make_fwd_inputs(w)
    lam = np.sum(x["k"].astype(np.float64) ** 2, axis=-1)
    assert lam.min() < 1e-5 and lam.max() > 500
    assert 0.05 < np.std(x["initial_state"]) < 0.2


def test_long_context_mask_shared_across_heads():
    w = W.workload(4, H=3, L=4096)
    x = W.make_fwd_inputs(w)
    big = np.sqrt(np.mean(x["k"].astype(np.float64) ** 2, axis=-1)) > 3.5
    assert np.array_equal(big[0, 0], big[0, 1]) and np.array_equal(big[0, 0], big[0, 2])
    assert 0.07 < big.mean() < 0.13


def test_decode_inputs():
    w = W.workload(5, B=4, H=2)
    s = W.make_decode_state(w)
    assert s.shape == (8, 128, 128)
    t0 = W.make_decode_token(w, 0)
    t1 = W.make_decode_token(w, 1)
    assert t0["k"].shape == (8, 128) and not np.array_equal(t0["k"], t1["k"])


def test_rel_max_err():
    assert W.rel_max_err(np.ones(3), np.ones(3)) == 0.0
    assert abs(W.rel_max_err(np.array([1.0, 2.1]), np.array([1.0, 2.0])) - 0.05) < 1e-12
    assert W.rel_max_err(np.zeros(0), np.zeros(0)) == 0.0
