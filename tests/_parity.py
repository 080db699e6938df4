"""Shared helpers of the GPU parity tests: tolerance checks and the bridge
that hands the same seeded inputs to the library and to the fp64 oracle."""
import numpy as np

# Tolerances for bf16 inputs with fp32 accumulation, over each whole tensor.
MAX_ABS = 2e-2
REL_L2 = 5e-3
LSE_MAX_ABS = 2e-2


def to64(t):
    return t.detach().to("cpu").double().numpy()


def compare(name, got, ref, max_abs=MAX_ABS, rel_l2=REL_L2):
    """Assert max|got-ref| <= max_abs and ||got-ref||/||ref|| <= rel_l2."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if got.size == 0:
        return 0.0, 0.0
    diff = got - ref
    ma = float(np.max(np.abs(diff)))
    nr = float(np.linalg.norm(ref))
    rl = float(np.linalg.norm(diff) / nr) if nr > 0 else float(np.linalg.norm(diff))
    assert ma <= max_abs, f"{name}: max abs err {ma:.3e} > {max_abs}"
    assert rl <= rel_l2, f"{name}: rel L2 err {rl:.3e} > {rel_l2}"
    return ma, rl


def compare_lse(name, got, ref, max_abs=LSE_MAX_ABS):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    ninf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), ninf), f"{name}: -inf pattern differs"
    if (~ninf).any():
        ma = float(np.max(np.abs(got[~ninf] - ref[~ninf])))
        assert ma <= max_abs, f"{name}: max abs err {ma:.3e} > {max_abs}"
