"""The compression entry point that allocates nothing (ec_compress_static,
for callers that cannot allocate device memory): its streams must equal
ec_compress's byte for byte (hence the oracle's), on two calls in a row whose
second input is smaller than the first, so the scratch still holds the first
call's hash tables and staging when the second runs."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import error_bounded_lossy_amd as ec  # noqa: E402
import oracle as O  # noqa: E402


def _rows(rng, T, B, D, scale, frac_unique):
    base = rng.normal(0, scale, (T, max(1, int(B * frac_unique)), D)).astype(np.float32)
    idx = rng.integers(0, base.shape[1], (T, B))
    return np.take_along_axis(base, idx[:, :, None], axis=1).astype(np.float32)


CASES = [  # (T, B, D, P, eb mode, eb): the second call's input is smaller
    ((4, 3000, 128, 1, ec.EB_REL_RANGE, 0.01), (2, 700, 128, 2, ec.EB_ABS, 2e-3)),
    ((3, 2000, 256, 1, ec.EB_ABS, 1e-3), (2, 130, 24, 1, ec.EB_REL_RANGE, 0.02)),
]


@pytest.mark.parametrize("first,second", CASES)
def test_static_scratch_matches_workspace_calls(first, second):
    rng = np.random.default_rng(first[2] + second[2])
    for call, (T, B, D, P, mode, eb) in enumerate((first, second)):
        print(f"[no-alloc] call {call}: T={T} B={B} D={D} P={P} mode={mode}", flush=True)
        x = _rows(rng, T, B, D, 0.05, 0.3)
        x[0, 3, 1] = 1e6  # an outlier
        xd = torch.from_numpy(x).cuda()
        ref_plan = ec.Plan(T, B, D, P, mode, eb)
        st_plan = ec.Plan(T, B, D, P, mode, eb, workspace=False)
        a, b = ref_plan.empty_stream(), st_plan.empty_stream()
        b.fill_(0xAB)
        ref_plan.compress(xd, a, 7)
        _, na, _ = ref_plan.ratio()
        st_plan.compress_static(xd, b, 7)
        _, nb, _ = st_plan.ratio()
        assert na == nb
        assert torch.equal(a[:na], b[:nb]), f"call {call}: streams differ"
        cfg = O.Config(T=T, B=B, D=D, P=P, eb_mode=mode, eb=(eb,))
        ref = O.compress(cfg, 7, x, debug=False)
        assert np.array_equal(b[:nb].cpu().numpy(), ref.stream), f"call {call}: oracle differs"
        # decompression with the workspace-less plan
        y = torch.full_like(xd, float("nan"))
        st_plan.decompress(b[:nb], y)
        st_plan.ratio()
        yo = O.decompress(cfg, ref.stream)
        np.testing.assert_array_equal(y.cpu().numpy().view(np.uint32), yo.view(np.uint32))


def test_static_scratch_limits_and_plan_without_workspace():
    # a plan beyond the scratch: rejected on the host, nothing enqueued
    big = ec.Plan(64, 16384, 256, 1, ec.EB_ABS, 1e-3, workspace=False)
    assert big.workspace_bytes > 64 << 20
    x = torch.zeros(64, 16384, 256, device="cuda")
    out = big.empty_stream()
    with pytest.raises(ec.ECError) as e:
        big.compress_static(x, out, 0)
    assert e.value.status == ec.EC_ERR_CAPACITY
    del x, out
    # ec_compress needs a workspace
    small = ec.Plan(1, 64, 64, 1, ec.EB_ABS, 1e-3, workspace=False)
    with pytest.raises(ec.ECError) as e:
        small.compress(torch.zeros(1, 64, 64, device="cuda"), small.empty_stream(), 0)
    assert e.value.status == ec.EC_ERR_INVALID
