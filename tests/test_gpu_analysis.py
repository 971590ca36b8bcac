"""GPU parity of the offline-analysis helpers (section III-C): eq. (1)'s
pattern counts per segment against the oracle, the stream written on the way,
a following compression on the same plan (the counting pass leaves raw rows in
the hash tables), and the Drop_2x schedule through the whole path."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402
import oracle as O  # noqa: E402


def say(*a):
    print(*a, flush=True)


def dup_rows(rng, T, B, D, scale=0.1, frac_unique=0.4):
    base = rng.normal(0, scale, (T, max(1, int(B * frac_unique) + 1), D)).astype(np.float32)
    idx = rng.integers(0, base.shape[1], (T, B))
    return np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)


CASES = [  # T, B, D, P, eb mode, eb, hash bits
    (3, 1000, 128, 1, ec.EB_REL_RANGE, 0.01, 0),
    (2, 700, 64, 2, ec.EB_ABS, 5e-3, 0),
    (2, 300, 24, 1, ec.EB_REL_RANGE, 0.02, 0),
    (2, 900, 256, 1, ec.EB_ABS, 1e-2, 3),
    (4, 130, 128, 3, ec.EB_REL_RANGE, 0.05, 1),
    (1, 0, 64, 1, ec.EB_ABS, 1e-3, 0),
]


@pytest.mark.parametrize("T,B,D,P,mode,eb,bits", CASES)
def test_homo_counts_match_the_oracle(T, B, D, P, mode, eb, bits):
    say(f"[homo] T={T} B={B} D={D} P={P} mode={mode} bits={bits}")
    rng = np.random.default_rng(T * 100 + D + B)
    x = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.3)
    if B > 0:
        # rows differing by less than a bin, an outlier, a NaN, a constant table
        x[:, 1::7] += rng.uniform(-1e-5, 1e-5, x[:, 1::7].shape).astype(np.float32)
        x[0, 2, 0] = 1e6
        x[-1, 3, -1] = np.nan
        if T > 2:
            x[1] = 0.5
    plan = ec.Plan(T, B, D, P, mode, eb, debug_hash_bits=bits)
    xd = torch.from_numpy(x).cuda()
    out = plan.empty_stream()
    no, nq = plan.homo_counts(xd, out, 4)
    cfg = O.Config(T=T, B=B, D=D, P=P, eb_mode=mode, eb=(eb,))
    ono, onq = O.homo_counts(cfg, 4, x)
    assert no == [int(v) for v in ono]
    assert nq == [int(v) for v in onq]
    _, nbytes, _ = plan.ratio()
    ref = O.compress(cfg, 4, x, debug=False)
    assert np.array_equal(out[:nbytes].cpu().numpy(), ref.stream)
    # the next compression on the same plan clears the raw rows out of its tables
    x2 = dup_rows(rng, T, B, D, scale=0.05, frac_unique=0.2)
    plan.compress(torch.from_numpy(x2).cuda(), out, 5)
    _, nbytes, _ = plan.ratio()
    assert np.array_equal(out[:nbytes].cpu().numpy(), O.compress(cfg, 5, x2, debug=False).stream)


@pytest.mark.parametrize("it", [0, 99, 100, 250])
def test_drop_schedule_through_the_path(it):
    """Drop_2x: twice the base bound until iteration 100, the base bound after."""
    T, B, D = 2, 500, 128
    rng = np.random.default_rng(it)
    x = dup_rows(rng, T, B, D, scale=0.05)
    sched = {"kind": ec.SCHED_STEP, "k": 2.0, "phase": 100, "steps": 1}
    plan = ec.Plan(T, B, D, 1, ec.EB_ABS, 1e-3, schedule=sched)
    ebs = torch.full((T,), -1.0, device="cuda")
    plan.debug_attach(eb=ebs)
    out = plan.empty_stream()
    plan.compress(torch.from_numpy(x).cuda(), out, it)
    _, nbytes, _ = plan.ratio()
    cfg = O.Config(T=T, B=B, D=D, eb_mode=ec.EB_ABS, eb=(1e-3,), sched_kind=ec.SCHED_STEP,
                   sched_k=2.0, sched_phase=100, sched_steps=1)
    assert np.array_equal(out[:nbytes].cpu().numpy(), O.compress(cfg, it, x, debug=False).stream)
    want = np.float32(2e-3) if it < 100 else np.float32(1e-3)
    assert np.all(ebs.cpu().numpy() == want)
