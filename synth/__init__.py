"""Seeded synthetic embedding-lookup and gradient tensors.

This module only draws inputs; it holds none of the compressor's arithmetic
and serves both the HIP path and the oracle (they always receive the same
realized tensor, copied between devices, so cross-device bit equality of the
generator itself is never relied on).

The stand-ins keep the structure that arXiv 2407.04272 describes for the
Criteo Kaggle / Terabyte lookups (section IV-A: 26 categorical features;
section III-C Fig. 6: table sizes spanning orders of magnitude; section III-D:
unbalanced, skewed query frequencies; fp32 embedding vectors).  No dataset
record is reproduced: every value comes from a counter-based SplitMix64
stream keyed by (seed, purpose, coordinates), so a 1e7-row table is never
materialized -- only the rows that a batch looks up are generated.

Workloads (name -> shape, error bound):
  c1  1 x 2048 x 16, one table of 100,000 rows, one-hot Zipf(1.05), abs eb 1e-4
  c2  26 x 4096 x 64, log-uniform table sizes 1e3..1e7, one-hot Zipf(a_t),
      a_t ~ U[0.9, 1.2], eb = 0.01 * range per table
  c3  26 x 8192 x 128, multi-hot pooled (1..20 indices, Zipf(1.05), fp32 sum in
      index order), eb = 0.005 * range * (1 + t/1000)^-1/2, t = iteration
  c4  26 x 8192 x 128 gradients: N(0, 1e-3) rows, 5% of rows Laplace(0, 1e-2),
      rows that share an index replaced by their fp32 sum in row order,
      abs eb 1e-5
  c5  64 x 16384 x 256, one-hot Zipf(1.2), eb = 0.01 * range per table
  c5d40  c5 with Zipf-Mandelbrot draws P(k) ~ (k + q_t)^-1.2, the shift q_t
      solved per table so that 16384 draws repeat a row with expected
      fraction 0.40 (tables too small for that are drawn uniformly, the
      closest their size allows)

One-hot workloads carry the measured fraction of rows that repeat an earlier
row of their table (`Workload.dup`).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

_M64 = (1 << 64) - 1


def _s64(v: int) -> int:
    """Reinterpret an unsigned 64-bit constant as a signed int64."""
    v &= _M64
    return v - (1 << 64) if v >= (1 << 63) else v


_GOLDEN = _s64(0x9E3779B97F4A7C15)
_MIX1 = _s64(0xBF58476D1CE4E5B9)
_MIX2 = _s64(0x94D049BB133111EB)


def _shr(z: torch.Tensor, k: int) -> torch.Tensor:
    """Logical right shift of int64 bit patterns."""
    return (z >> k) & ((1 << (64 - k)) - 1)


def splitmix64(z: torch.Tensor) -> torch.Tensor:
    """SplitMix64 output function applied to int64 bit patterns (wrapping)."""
    z = z + _GOLDEN
    z = (z ^ _shr(z, 30)) * _MIX1
    z = (z ^ _shr(z, 27)) * _MIX2
    return z ^ _shr(z, 31)


def keyed(seed: int, purpose: int, *coords, device="cpu") -> torch.Tensor:
    """Hash of (seed, purpose, coords...) -> int64 bit patterns; coords broadcast."""
    h = splitmix64(torch.tensor([_s64(seed * 0x100000001B3 + purpose)], dtype=torch.int64,
                                device=device))
    for c in coords:
        if not torch.is_tensor(c):
            c = torch.tensor(c, dtype=torch.int64, device=device)
        h = splitmix64(h ^ c.to(torch.int64))
    return h


def u01_f64(h: torch.Tensor) -> torch.Tensor:
    """Uniform double in [0, 1) from the top 53 bits."""
    return _shr(h, 11).to(torch.float64) * (2.0 ** -53)


def sym_f32(h: torch.Tensor, half_width: float) -> torch.Tensor:
    """Uniform fp32 in [-half_width, half_width): (m * 2^-23 - 1) * half_width, 24-bit m."""
    m = _shr(h, 40).to(torch.float32) * (2.0 ** -23)
    return (m - 1.0) * torch.tensor(half_width, dtype=torch.float32, device=h.device)


# purposes (distinct hash streams)
P_TABLE_SIZE, P_ALPHA, P_VALUE, P_INDEX, P_COUNT, P_GRAD, P_HEAVY, P_LAPLACE = range(1, 9)


def table_sizes(seed: int, T: int) -> list[int]:
    """Log-uniform table sizes N_t = round(10^(3 + 4u)) in [1e3, 1e7]."""
    u = u01_f64(keyed(seed, P_TABLE_SIZE, torch.arange(T)))
    return [int(round(10.0 ** (3.0 + 4.0 * float(v)))) for v in u]


def zipf_cdf(n: int, alpha: float, device="cpu") -> torch.Tensor:
    """Normalized CDF of P(k) ~ k^-alpha on k = 1..n (double)."""
    k = torch.arange(1, n + 1, dtype=torch.float64, device=device)
    w = k.pow(-alpha)
    c = torch.cumsum(w, 0)
    return c / c[-1]


def zm_cdf(n: int, alpha: float, q: float, device="cpu") -> torch.Tensor:
    """Normalized CDF of the Zipf-Mandelbrot law P(k) ~ (k + q)^-alpha, k = 1..n."""
    k = torch.arange(1, n + 1, dtype=torch.float64, device=device)
    c = torch.cumsum((k + q).pow(-alpha), 0)
    return c / c[-1]


def expected_dup(n: int, alpha: float, q: float, draws: int) -> float:
    """Expected fraction of `draws` independent draws of P(k) ~ (k + q)^-alpha
    on k = 1..n that repeat an earlier draw: 1 - E[distinct] / draws, with
    E[distinct] = sum_k 1 - (1 - p_k)^draws.  Exact over the first 65536 ranks;
    beyond, ranks are grouped in geometric bins (ratio about 1.002) that take
    the weight of their middle rank."""
    head = min(n, 65536)
    k = torch.arange(1, head + 1, dtype=torch.float64)
    w = (k + q).pow(-alpha)
    cnt = torch.ones_like(w)
    if n > head:
        nb = max(1, int(torch.log(torch.tensor(n / head)).item() / 0.002))
        e = torch.unique(torch.round(torch.logspace(torch.log10(torch.tensor(head + 0.5)).item(),
                                                    torch.log10(torch.tensor(n + 0.5)).item(),
                                                    nb + 1, dtype=torch.float64))) + 0.5
        e = torch.unique(torch.clamp(e, head + 0.5, n + 0.5))  # edges between ranks
        e[0], e[-1] = head + 0.5, n + 0.5
        lo, hi = torch.ceil(e[:-1]), torch.floor(e[1:])
        c = hi - lo + 1
        keep = c > 0
        lo, hi, c = lo[keep], hi[keep], c[keep]
        w = torch.cat([w, ((lo + hi) / 2 + q).pow(-alpha)])
        cnt = torch.cat([cnt, c])
    p = w / (w * cnt).sum()
    distinct = (cnt * -torch.expm1(draws * torch.log1p(-p))).sum().item()
    return 1.0 - distinct / draws


_ZM_SHIFT: dict = {}


def zm_shift(n: int, alpha: float, draws: int, target: float) -> float:
    """Shift q >= 0 with expected_dup(n, alpha, q, draws) = target (bisection on
    log q; the expected fraction falls as q grows).  A table too small to get
    down to the target is drawn (nearly) uniformly: q = 1e12."""
    key = (n, alpha, draws, target)
    if key not in _ZM_SHIFT:
        if expected_dup(n, alpha, 1e12, draws) >= target:
            q = 1e12
        elif expected_dup(n, alpha, 0.0, draws) <= target:
            q = 0.0
        else:
            lo, hi = -3.0, 12.0
            for _ in range(48):
                mid = 0.5 * (lo + hi)
                if expected_dup(n, alpha, 10.0 ** mid, draws) > target:
                    lo = mid
                else:
                    hi = mid
            q = 10.0 ** (0.5 * (lo + hi))
        _ZM_SHIFT[key] = q
    return _ZM_SHIFT[key]


def dup_fraction(idx: torch.Tensor) -> float:
    """Fraction of the lookups that repeat an earlier row of the table."""
    return 1.0 - torch.unique(idx).numel() / max(1, idx.numel())


def zipf_rows(cdf: torch.Tensor, h: torch.Tensor) -> torch.Tensor:
    """Inverse-CDF Zipf draw: rank k (1-based) -> table row k-1."""
    u = u01_f64(h)
    r = torch.searchsorted(cdf, u, right=True)
    return torch.clamp(r, max=cdf.numel() - 1)


def table_rows(seed: int, t: int, rows: torch.Tensor, D: int, n_rows: int) -> torch.Tensor:
    """Embedding rows of table t: U(-1/sqrt(N_t), +1/sqrt(N_t)) fp32, [len(rows), D]."""
    dev = rows.device
    cols = torch.arange(D, device=dev, dtype=torch.int64)
    h = keyed(seed, P_VALUE, t, rows.to(torch.int64)[:, None], cols[None, :], device=dev)
    return sym_f32(h, float(1.0 / (n_rows ** 0.5)))


def _lookup_one_hot(seed, it, t, B, D, n_rows, alpha, device, shift=None):
    cdf = zipf_cdf(n_rows, alpha, device) if shift is None else zm_cdf(n_rows, alpha, shift, device)
    idx = zipf_rows(cdf, keyed(seed, P_INDEX, it, t, torch.arange(B, device=device),
                               device=device))
    uniq, inv = torch.unique(idx, return_inverse=True)
    vals = table_rows(seed, t, uniq, D, n_rows)
    return vals[inv], idx


def _lookup_pooled(seed, it, t, B, D, n_rows, alpha, max_hot, device):
    cdf = zipf_cdf(n_rows, alpha, device)
    b = torch.arange(B, device=device, dtype=torch.int64)
    cnt = 1 + (u01_f64(keyed(seed, P_COUNT, it, t, b, device=device)) * max_hot).to(torch.int64)
    cnt = torch.clamp(cnt, 1, max_hot)
    slots = torch.arange(max_hot, device=device, dtype=torch.int64)
    idx = zipf_rows(cdf, keyed(seed, P_INDEX, it, t, b[:, None] * 64 + slots[None, :],
                               device=device))
    uniq, inv = torch.unique(idx, return_inverse=True)
    vals = table_rows(seed, t, uniq, D, n_rows)
    acc = torch.zeros(B, D, dtype=torch.float32, device=device)
    for j in range(max_hot):  # fp32 sum in index order
        v = vals[inv[:, j]]
        acc = torch.where((cnt > j)[:, None], acc + v, acc)
    return acc


def _gradients(seed, it, t, B, D, n_rows, device):
    b = torch.arange(B, device=device, dtype=torch.int64)
    cols = torch.arange(D, device=device, dtype=torch.int64)
    h1 = keyed(seed, P_GRAD, it, t, b[:, None], cols[None, :] * 2, device=device)
    h2 = keyed(seed, P_GRAD, it, t, b[:, None], cols[None, :] * 2 + 1, device=device)
    u1 = torch.clamp(u01_f64(h1), min=2.0 ** -53)
    u2 = u01_f64(h2)
    g = (1e-3 * torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * torch.pi * u2))
    heavy = u01_f64(keyed(seed, P_HEAVY, it, t, b, device=device)) < 0.05
    u3 = u01_f64(keyed(seed, P_LAPLACE, it, t, b[:, None], cols[None, :], device=device)) - 0.5
    lap = -1e-2 * torch.sign(u3) * torch.log(torch.clamp(1.0 - 2.0 * u3.abs(), min=2.0 ** -53))
    g = torch.where(heavy[:, None], lap, g).to(torch.float32)
    # rows sharing an index: every such row becomes the fp32 sum, in row order
    cdf = zipf_cdf(n_rows, 1.05, device)
    idx = zipf_rows(cdf, keyed(seed, P_INDEX, it, t, b, device=device))
    order = torch.sort(idx * B + b).indices          # stable: by (index, row)
    sidx = idx[order]
    start = torch.ones(B, dtype=torch.bool, device=device)
    start[1:] = sidx[1:] != sidx[:-1]
    gid = torch.cumsum(start.to(torch.int64), 0) - 1
    first_pos = torch.nonzero(start).squeeze(1)
    rank = torch.arange(B, device=device) - first_pos[gid]
    ng = int(first_pos.numel())
    acc = torch.zeros(ng, D, dtype=torch.float32, device=device)
    gs = g[order]
    for j in range(int(rank.max().item()) + 1):
        m = rank == j
        acc[gid[m]] = acc[gid[m]] + gs[m]
    out = torch.empty_like(g)
    out[order] = acc[gid]
    return out


@dataclass
class Workload:
    """A synthetic batch plus the error-bound policy it is compressed under."""
    name: str
    x: torch.Tensor                 # [T, B, D] fp32
    eb_mode: int                    # 0 absolute, 1 range-relative
    eb: list = field(default_factory=list)
    sched_kind: int = 0             # 0 none, 1 (1 + i/t0)^-1/2, 2 staircase
    sched_t0: float = 1000.0
    iteration: int = 0
    dup: list | None = None         # one-hot workloads: measured repeat fraction per table

    @property
    def shape(self):
        return tuple(self.x.shape)


SHAPES = {
    "c1": (1, 2048, 16),
    "c2": (26, 4096, 64),
    "c3": (26, 8192, 128),
    "c4": (26, 8192, 128),
    "c5": (64, 16384, 256),
    "c5d40": (64, 16384, 256),
}
DUP40 = 0.40  # the c5d40 target: expected fraction of repeated rows per table


def workload(name: str, iteration: int = 0, device="cpu", seed: int = 0,
             tables: list[int] | None = None) -> Workload:
    """Build workload `name` for `iteration` (the batch seed is (seed, iteration)).

    `tables` restricts generation to a subset of table ids (same values as in
    the full batch); the result then has len(tables) tables.
    """
    T, B, D = SHAPES[name]
    ts = list(range(T)) if tables is None else list(tables)
    out = []
    dup = []
    if name == "c1":
        for t in ts:
            v, idx = _lookup_one_hot(seed, iteration, t, B, D, 100_000, 1.05, device)
            out.append(v)
            dup.append(dup_fraction(idx))
        x = torch.stack(out)
        return Workload(name, x, 0, [1e-4] * len(ts), iteration=iteration, dup=dup)
    sizes = table_sizes(seed, T)
    if name == "c2":
        alphas = (0.9 + 0.3 * u01_f64(keyed(seed, P_ALPHA, torch.arange(T)))).tolist()
        for t in ts:
            v, idx = _lookup_one_hot(seed, iteration, t, B, D, sizes[t], alphas[t], device)
            out.append(v)
            dup.append(dup_fraction(idx))
        return Workload(name, torch.stack(out), 1, [0.01] * len(ts), iteration=iteration, dup=dup)
    if name == "c3":
        for t in ts:
            out.append(_lookup_pooled(seed, iteration, t, B, D, sizes[t], 1.05, 20, device))
        return Workload(name, torch.stack(out), 1, [0.005] * len(ts), sched_kind=1,
                        sched_t0=1000.0, iteration=iteration)
    if name == "c4":
        for t in ts:
            out.append(_gradients(seed, iteration, t, B, D, sizes[t], device))
        return Workload(name, torch.stack(out), 0, [1e-5] * len(ts), iteration=iteration)
    if name in ("c5", "c5d40"):
        for t in ts:
            shift = zm_shift(sizes[t], 1.2, B, DUP40) if name == "c5d40" else None
            v, idx = _lookup_one_hot(seed, iteration, t, B, D, sizes[t], 1.2, device, shift)
            out.append(v)
            dup.append(dup_fraction(idx))
        return Workload(name, torch.stack(out), 1, [0.01] * len(ts), iteration=iteration, dup=dup)
    raise KeyError(name)
