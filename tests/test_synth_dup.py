"""The dup-40 stand-in for the 64-table one-hot batch: expected repeat
fractions of Zipf-Mandelbrot draws, the per-table shift solve, and the
generated tables' measured repeat fractions (CPU only)."""
import numpy as np
import pytest
import torch

import synth


def exact_dup(n, alpha, q, draws):
    """1 - E[distinct] / draws summed over every rank (no binning)."""
    k = np.arange(1, n + 1, dtype=np.float64)
    w = (k + q) ** -alpha
    p = w / w.sum()
    return 1.0 - float(np.sum(-np.expm1(draws * np.log1p(-p)))) / draws


@pytest.mark.parametrize("n,q", [(1000, 0.0), (200_000, 0.0), (200_000, 300.0), (3_000_000, 174.0)])
def test_expected_dup_matches_the_exact_sum(n, q):
    assert synth.expected_dup(n, 1.2, q, 16384) == pytest.approx(exact_dup(n, 1.2, q, 16384), abs=2e-5)


def test_expected_dup_limits():
    # a table of one row: every draw after the first repeats it
    assert synth.expected_dup(1, 1.2, 0.0, 100) == pytest.approx(0.99, abs=1e-12)
    # uniform draws (q huge) over n rows: 1 - n (1 - (1 - 1/n)^B) / B
    n, B = 5000, 16384
    assert synth.expected_dup(n, 1.2, 1e12, B) == pytest.approx(1 - n * (1 - (1 - 1 / n) ** B) / B, abs=1e-6)


def test_shift_reaches_the_target_where_the_table_allows():
    sizes = synth.table_sizes(0, 64)
    for n in sizes:
        q = synth.zm_shift(n, 1.2, 16384, synth.DUP40)
        d = synth.expected_dup(n, 1.2, q, 16384)
        if q < 1e12:
            assert d == pytest.approx(synth.DUP40, abs=1e-4)
        else:  # too small: uniform draws, still above the target
            assert d >= synth.DUP40
            assert synth.expected_dup(n, 1.2, 1e11, 16384) >= synth.DUP40


def test_generated_tables_repeat_as_expected():
    sizes = synth.table_sizes(0, 64)
    big = [t for t, n in enumerate(sizes) if n > 100_000][:3]
    w = synth.workload("c5d40", iteration=0, device="cpu", tables=big)
    z = synth.workload("c5", iteration=0, device="cpu", tables=big)
    for j, t in enumerate(big):
        assert w.dup[j] == pytest.approx(synth.DUP40, abs=0.02)
        q = synth.zm_shift(sizes[t], 1.2, 16384, synth.DUP40)
        assert abs(w.dup[j] - synth.expected_dup(sizes[t], 1.2, q, 16384)) < 0.02
        # plain Zipf(1.2) repeats far more often (0.77-0.95 on these sizes)
        assert z.dup[j] > 0.7
    assert w.x.shape == (len(big), 16384, 256) and w.eb_mode == 1
