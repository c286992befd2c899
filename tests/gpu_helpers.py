"""Shared helpers for the GPU parity tests (host-side marshalling and checks)."""
import sys

import numpy as np
import torch

# fp16 output tolerance of the decomposition (elementwise, against the oracle)
ATOL = 1e-3
RTOL = 2e-3


def say(*a):
    """Print and flush: names the case before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda", 0)


def h2d(a):
    """numpy array -> device tensor (fp16 stays fp16)."""
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def d2h(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a


def assert_fp16_close(got, ref, what=""):
    """|got - ref| <= ATOL + RTOL*|ref| elementwise; infinities must match exactly."""
    g = bits(got).view(np.float16).astype(np.float64)
    r = bits(ref).view(np.float16).astype(np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert not np.isnan(g).any(), "%s: NaN in GPU output" % what
    fin = np.isfinite(r)
    assert np.array_equal(g[~fin], r[~fin]), "%s: infinities differ" % what
    err = np.zeros(r.shape)
    err[fin] = np.abs(g[fin] - r[fin])
    tol = ATOL + RTOL * np.abs(np.where(fin, r, 0.0))
    bad = fin & (err > tol)
    if bad.any():
        first = np.argwhere(bad)[:5]
        worst = np.unravel_index(np.argmax(np.where(fin, err - tol, -np.inf)), r.shape)
        raise AssertionError("%s: %d of %d outputs out of tolerance; worst at %s: got %.6g ref %.6g; first %s"
                             % (what, int(bad.sum()), bad.size, tuple(int(i) for i in worst),
                                g[worst], r[worst], first.tolist()))


def assert_equal_exact(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, "%s: shape %s vs %s" % (what, got.shape, ref.shape)
    if not np.array_equal(got, ref):
        d = np.argwhere(got != ref)
        raise AssertionError("%s: %d mismatches; first %s: got %s ref %s"
                             % (what, len(d), d[:4].tolist(),
                                [got[tuple(i)] for i in d[:4]], [ref[tuple(i)] for i in d[:4]]))


def sample_rows(T, n_random=62, seed=1234):
    """Rows 0 and T-1 plus seeded random rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    r = rng.choice(T, size=min(T, n_random), replace=False)
    return np.unique(np.concatenate([[0, T - 1], r])).astype(np.int64)


def tile_rows(T, tile=256, per_tile=4, seed=4321):
    """`per_tile` seeded rows from every `tile`-row block of [0, T), plus rows
    0 and T-1 (sorted, unique): a sample that covers every tile row of the GEMM."""
    rng = np.random.default_rng(seed)
    picks = [[0, T - 1]]
    for r0 in range(0, T, tile):
        r1 = min(T, r0 + tile)
        picks.append(r0 + rng.choice(r1 - r0, size=min(per_tile, r1 - r0), replace=False))
    return np.unique(np.concatenate(picks)).astype(np.int64)
