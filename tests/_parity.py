"""Acceptance rules for comparing the GPU path with the oracle.

Logits: on every row, |I_gpu - I_oracle| <= 2e-3 * max_s |I_oracle[t, s]| over the
finite entries, and the -inf pattern must match exactly.

One stated exception, for two kinds of degenerate row: rows with at most
FLOOR_MAX_KEYS valid keys, whose maximum is the largest of a handful of sums whose
terms can cancel (a single key's heads may all but cancel, and a one-key row has
nothing else to set its scale), and rows whose valid logits are all exactly 0 (every
head's score ReLU'd away on every key, common at H = 1), where the relative bound
is 0. For them the bound is stated against the size of the terms instead:
2^-11 * max_s A[t, s], with A[t, s] = sum_h |w| * k_scale * sum_d |q k| (the
oracle's ``magnitude=True``). 2^-11 covers the matrix cores' accumulation error of
a 128-term dot product, which ``tests/test_gpu_accumulation.py`` measures on
adversarial sums and asserts to be below 2^-11.75. Every row with more valid keys is
held to the plain 2e-3 bound whether or not a magnitude array is passed.

Top-k: index sets must match, except that an index in one set and not the other
must carry an oracle logit within that same tolerance of the row's k-th oracle
value (a near-tie the fp32 path may order differently); the number of -1 pads must
match exactly.
"""

from __future__ import annotations

import numpy as np

REL_TOL = 2e-3
MAG_FLOOR = 2.0 ** -11
FLOOR_MAX_KEYS = 4


def uses_floor(oracle_row: np.ndarray, mag_row: np.ndarray | None) -> bool:
    """True when the row is held to the magnitude floor: a magnitude row is given and
    the row has between 1 and FLOOR_MAX_KEYS finite (valid) entries, or has some and
    all of them are exactly 0."""
    if mag_row is None:
        return False
    fin = np.isfinite(oracle_row)
    n = int(fin.sum())
    return 0 < n <= FLOOR_MAX_KEYS or (n > 0 and not np.any(oracle_row[fin]))


def row_tolerance(oracle_row: np.ndarray, mag_row: np.ndarray | None = None) -> float:
    fin = np.isfinite(oracle_row)
    tol = REL_TOL * (float(np.abs(oracle_row[fin]).max()) if fin.any() else 0.0)
    if uses_floor(oracle_row, mag_row):
        tol = max(tol, MAG_FLOOR * float(mag_row[fin].max()))
    return tol


def check_logits(gpu: np.ndarray, oracle: np.ndarray, mag: np.ndarray | None = None, rows=None, what: str = "",
                 allow_floor: bool = True) -> float:
    """Asserts the logits rule; returns the worst error relative to the plain row scale
    (2e-3 * max |I|) over the rows held to the plain bound. ``allow_floor=False``
    holds every row, short ones included, to the plain bound. Prints how many rows
    were held to the floor."""
    gpu = np.asarray(gpu, dtype=np.float64)
    oracle = np.asarray(oracle, dtype=np.float64)
    assert gpu.shape == oracle.shape, (gpu.shape, oracle.shape)
    worst = 0.0
    floored = 0
    rows = range(gpu.shape[0]) if rows is None else rows
    for i, r in enumerate(rows):
        g, o = gpu[i], oracle[i]
        fin_o = np.isfinite(o)
        assert np.array_equal(np.isneginf(g), ~fin_o), f"{what} row {r}: -inf pattern differs"
        assert not np.isnan(g).any(), f"{what} row {r}: NaN"
        if fin_o.any():
            m = None if (mag is None or not allow_floor) else mag[i]
            plain = row_tolerance(o)
            tol = row_tolerance(o, m)
            err = np.abs(g[fin_o] - o[fin_o]).max()
            if uses_floor(o, m):
                floored += 1
            else:
                worst = max(worst, err / max(plain, 1e-300) * REL_TOL)
            assert err <= tol, f"{what} row {r}: max err {err:.3e} > tol {tol:.3e} (plain {plain:.3e})"
    if floored:
        print(f"{what}: {floored} of {len(rows)} rows (<= {FLOOR_MAX_KEYS} valid keys, or all 0) held to the "
              f"magnitude floor")
    return worst


def check_topk(gpu_idx: np.ndarray, oracle_idx: np.ndarray, oracle_logits: np.ndarray, starts, what: str = "",
               mag: np.ndarray | None = None):
    """gpu_idx / oracle_idx are [rows, k] int32 (column - start, -1 padded); oracle_logits
    holds the matching oracle rows (and ``mag`` their magnitudes, for the floor)."""
    gpu_idx = np.asarray(gpu_idx)
    oracle_idx = np.asarray(oracle_idx)
    for r in range(gpu_idx.shape[0]):
        g, o = gpu_idx[r], oracle_idx[r]
        assert (g == -1).sum() == (o == -1).sum(), f"{what} row {r}: pad count differs"
        gs, os_ = set(g[g >= 0].tolist()), set(o[o >= 0].tolist())
        assert len(gs) == (g >= 0).sum(), f"{what} row {r}: duplicate indices"
        diff = gs ^ os_
        if not diff:
            continue
        st = int(starts[r]) if starts is not None else 0
        row = oracle_logits[r]
        kth = min(row[st + c] for c in os_)
        tol = row_tolerance(row, None if mag is None else mag[r])
        for c in diff:
            assert abs(row[st + c] - kth) <= tol, f"{what} row {r}: index {c} differs beyond a near-tie"
