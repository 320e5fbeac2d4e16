"""Shared helpers of the GPU parity tests (tolerances and selection-parity rules)."""
import numpy as np

SCORE_RTOL = 2e-3          # relative tolerance on column scores (fp32 from bf16 vs fp64)
MASS_RTOL = 1e-4           # relative tolerance on the total mass W*G per group


def score_floor(R: int, L: int) -> float:
    """Absolute floor: 0.1% of a uniform column's score, scaled by the tolerance.

    It only absorbs exponentials that fp32 flushes or rounds to denormals."""
    return SCORE_RTOL * 1e-3 * R / L


def assert_scores_close(got: np.ndarray, want: np.ndarray, R: int, L: int, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    tol = SCORE_RTOL * np.abs(want) + score_floor(R, L)
    err = np.abs(got - want)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err / tol), err.shape)
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} scores out of tolerance; worst at {i}: "
            f"got {got[i]:.9g} want {want[i]:.9g} (rel {err[i] / max(abs(want[i]), 1e-300):.3g})")


def assert_mass(got: np.ndarray, R: int):
    sums = np.asarray(got, dtype=np.float64).sum(axis=-1)
    assert np.all(np.abs(sums - R) <= MASS_RTOL * R), sums


def assert_topk_parity(got_idx: np.ndarray, oracle_vals: np.ndarray, budget: int,
                       oracle_prio=None, robust_prio=None, rel: float = SCORE_RTOL):
    """Selection parity of a GPU top-k against the oracle's fp64 values.

    Per row: with v* the oracle's budget-th value within the boundary priority
    class, every element whose oracle value differs from v* by more than
    rel*|v*| (and whose priority is robust) must be chosen by the GPU exactly
    when the oracle chooses it.  Output rows must be ascending and of length
    budget."""
    H, n = oracle_vals.shape
    for h in range(H):
        sel = np.asarray(got_idx[h, :budget], dtype=np.int64)
        assert len(sel) == budget
        assert np.all(np.diff(sel) > 0), "GPU top-k output is not strictly ascending"
        assert sel.min(initial=0) >= 0 and sel.max(initial=-1) < n
        v = oracle_vals[h]
        pr = np.zeros(n, dtype=np.int64) if oracle_prio is None else np.asarray(oracle_prio[h], np.int64)
        order = np.lexsort((np.arange(n), -v, -pr))
        if budget == 0:
            continue
        kth = order[budget - 1]
        vstar, pstar = v[kth], pr[kth]
        chosen_o = np.zeros(n, dtype=bool)
        chosen_o[order[:budget]] = True
        chosen_g = np.zeros(n, dtype=bool)
        chosen_g[sel] = True
        robust = np.ones(n, dtype=bool) if robust_prio is None else np.asarray(robust_prio[h], bool)
        same_class = pr == pstar
        decidable = robust & (~same_class | (np.abs(v - vstar) > rel * abs(vstar)))
        mism = decidable & (chosen_o != chosen_g)
        assert not mism.any(), (
            f"row {h}: {mism.sum()} decidable elements differ, e.g. index {np.nonzero(mism)[0][:5]}; "
            f"v*={vstar:.6g}")
