"""The fp64 oracle against its pins (see oracle_pins.py for what pins what)."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(lib, pin):
    pin(lib)


def test_oracle_rejects_bad_arguments(lib):
    import numpy as np
    z = np.zeros((1, 1, 4, 8), np.uint16)
    with pytest.raises(TypeError):
        oracle.attention_fwd(z.astype(np.float32), z, z, scale=1.0, causal=False, dtype="f16", lib=lib)
    with pytest.raises(RuntimeError):
        oracle.attention_rows(z, z, z, np.array([4]), scale=1.0, causal=False, dtype="f16", lib=lib)
    with pytest.raises(RuntimeError):
        oracle.attention_bwd_rows(z, z, z, z, np.array([0]), np.array([4]), scale=1.0,
                                  causal=False, dtype="f16", lib=lib)
    with pytest.raises(ValueError):
        oracle.attention_bwd(z, z, z, z[:, :, :3], scale=1.0, causal=False, dtype="f16", lib=lib)


def test_gradient_rule():
    """The gradient parity rule accepts rounding-sized errors and rejects a
    dropped term, a sign error and a value where the reference is zero."""
    import numpy as np
    from oracle import parity
    rng = np.random.default_rng(0)
    ref = rng.standard_normal((2, 3, 50, 16))
    u = parity.GRAD_U["bf16"]
    assert parity.grad_ok(parity.compare_grad(ref * (1 + u / 2), ref, "bf16"))
    assert parity.grad_ok(parity.compare_grad(ref + u * rng.standard_normal(ref.shape) * 0.5, ref, "bf16"))
    assert not parity.grad_ok(parity.compare_grad(ref * 0.98, ref, "bf16"))
    bad = ref.copy()
    bad[1, 2, 7, 3] = -bad[1, 2, 7, 3]
    assert not parity.grad_ok(parity.compare_grad(bad, ref, "bf16"))
    z = np.zeros((1, 1, 4, 4))
    assert parity.grad_ok(parity.compare_grad(z, z, "f16"))
    assert not parity.grad_ok(parity.compare_grad(z + 1e-30, z, "f16"))
    assert parity.grad_ok(parity.compare_grad(z + 1e-6, z, "f16", zero_tol=2e-6))
    assert not parity.grad_ok(parity.compare_grad(z + 3e-6, z, "f16", zero_tol=2e-6))
    # the cancellation bound: 2 D 2^-24 sum|dO v| (scaled by scale max|K| for dQ);
    # with dropout the storage rounding u of O is added
    D = 4
    qq, kk, vv, gg = (np.ones((1, 1, 2, D)) for _ in range(4))
    tol = parity.cancellation_tolerances(qq, 2 * kk, vv, gg, 0.5, "bf16")
    assert abs(tol["dq"] - 0.5 * (2 * D * 2.0 ** -24) * D * 2.0) < 1e-15 and tol["dv"] == 0.0
    tol_d = parity.cancellation_tolerances(qq, kk, vv, gg, 0.5, "bf16", dropout_p=0.5)
    assert abs(tol_d["dk"] - 0.5 * (2 * D * 2.0 ** -24 + 2.0 ** -8) * 2.0 * D * 1.0) < 1e-12
    nanv = ref.copy()
    nanv[0, 0, 0, 0] = np.nan
    assert not parity.grad_ok(parity.compare_grad(nanv, ref, "f16"))
