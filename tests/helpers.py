"""Shared tolerance checks for the parity tests."""

import numpy as np

# Tolerances (one reading of "1e-4 relative for fp32, 2e-2 absolute for bf16
# inputs with fp32 accumulation"): fp32 elementwise |g - r| <= 1e-4 |r| + 1e-5
# and relative L2 error <= 1e-4; bf16 elementwise |g - r| <= 2e-2.
FP32_RTOL = 1e-4
FP32_ATOL = 1e-5
BF16_ATOL = 2e-2


def assert_close(got, ref, dtype="f32", what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), f"{what}: finite pattern differs"
    g, r = got[fin], ref[fin]
    if g.size == 0:
        return
    err = np.abs(g - r)
    if dtype == "bf16":
        worst = float(err.max())
        assert worst <= BF16_ATOL, f"{what}: max abs err {worst:.3e} > {BF16_ATOL}"
    else:
        lim = FP32_RTOL * np.abs(r) + FP32_ATOL
        bad = err > lim
        assert not bad.any(), (f"{what}: {int(bad.sum())} elements over 1e-4 rel "
                               f"(worst abs {float(err.max()):.3e})")
        nr = float(np.linalg.norm(r))
        if nr > 0:
            rel = float(np.linalg.norm(g - r)) / nr
            assert rel <= FP32_RTOL, f"{what}: relative L2 {rel:.3e} > {FP32_RTOL}"


# Gradients (backward through time) are sums over every token of products
# whose terms cancel, so an element can be small next to its neighbours.
# Reading for fp32: |g - r| <= 1e-4 |r| + 1e-5 max|r| elementwise (the
# absolute part scaled to the tensor), and relative L2 error <= 1e-4.
def assert_grad_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} != {ref.shape}"
    assert np.isfinite(got).all(), f"{what}: non-finite values"
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    err = np.abs(got - ref)
    lim = FP32_RTOL * np.abs(ref) + FP32_ATOL * max(scale, 1e-30)
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {ref.size} elements over tolerance "
                           f"(worst abs {float(err.max()):.3e}, scale {scale:.3e})")
    nr = float(np.linalg.norm(ref))
    if nr > 0:
        rel = float(np.linalg.norm(got - ref)) / nr
        assert rel <= FP32_RTOL, f"{what}: relative L2 {rel:.3e} > {FP32_RTOL}"
