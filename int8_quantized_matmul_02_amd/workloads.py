"""Seeded synthetic inputs for the LLM.int8() decomposition matmul.

This module only draws random fp16 activations and weights; it holds none of
the method's arithmetic (no quantization, no outlier detection, no product),
so both the HIP path and the CPU oracle can be fed from it.

Recipe (numpy ``Generator(PCG64)``; values drawn in fp32 and rounded to fp16):
  * activations X [T,K]: background N(0,1); background draws with |x| >= 6 are
    redrawn so the number of outlier columns is exactly the planted count;
  * outlier feature dims: ``rng.choice(K, n, replace=False)``, sorted; each
    (row, dim) holds sign * U(lo,hi) with probability p (the pages describe a
    handful of fixed hidden dims holding magnitudes well above 6 in 25-75 % of
    the sequence positions -- LLM.int8() paper summary, sections on outlier
    features);
  * weights W_t [N,K] (the stored transpose of W [K,N], row n = output column
    n): N(0, 0.02) with 0.02 read as the standard deviation;
  * X and W come from two independent child streams of one SeedSequence, so a
    weight does not change when the activation shape does.
"""
import numpy as np

BACKGROUND_LIMIT = 6.0


def _streams(seed):
    ss = np.random.SeedSequence(seed)
    sx, sw = ss.spawn(2)
    return np.random.Generator(np.random.PCG64(sx)), np.random.Generator(np.random.PCG64(sw))


def background(rng, T, K):
    """N(0,1) [T,K] fp32 with every |x| >= 6 redrawn."""
    x = rng.standard_normal((T, K), dtype=np.float32)
    while True:
        bad = np.abs(x) >= BACKGROUND_LIMIT
        cnt = int(bad.sum())
        if cnt == 0:
            return x
        x[bad] = rng.standard_normal(cnt, dtype=np.float32)


def plant_outliers(rng, x, n_dims, lo, hi, p):
    """Overwrite n_dims random columns of x with sign*U(lo,hi) in a fraction p of rows.

    Returns the sorted planted dims.  Draw order: dims, row masks, signs,
    magnitudes."""
    T, K = x.shape
    if n_dims == 0:
        return np.zeros((0,), np.int64)
    dims = np.sort(rng.choice(K, n_dims, replace=False))
    mask = rng.random((T, n_dims)) < p
    signs = np.where(rng.random((T, n_dims)) < 0.5, -1.0, 1.0).astype(np.float32)
    mags = rng.uniform(lo, hi, (T, n_dims)).astype(np.float32)
    vals = signs * mags
    for j, d in enumerate(dims):
        x[mask[:, j], d] = vals[mask[:, j], j]
    return dims


def weights(rng, N, K, std=0.02, chunk_rows=4096):
    """W_t [N,K] fp16 ~ N(0, std), drawn in row chunks to bound host memory."""
    W = np.empty((N, K), np.float16)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        W[r0:r1] = (rng.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(std)).astype(np.float16)
    return W


def activations(T, K, n_dims, lo, hi, p, seed=0):
    rx, _ = _streams(seed)
    x = background(rx, T, K)
    dims = plant_outliers(rx, x, n_dims, lo, hi, p)
    return x.astype(np.float16), dims


def case(T, K, N, n_dims=3, lo=8.0, hi=30.0, p=0.25, seed=0, std=0.02):
    """Generic seeded case: X [T,K] fp16, W_t [N,K] fp16, planted dims."""
    rx, rw = _streams(seed)
    x = background(rx, T, K)
    dims = plant_outliers(rx, x, n_dims, lo, hi, p)
    W_t = weights(rw, N, K, std)
    return x.astype(np.float16), W_t, dims


# ---------------------------------------------------------------------------
# The five workloads.  Each returns a dict of fp16 arrays plus the threshold.
# ---------------------------------------------------------------------------

def tiny(seed=0):
    """X [16,256] N(0,1) with columns 7 and 200 set to N(0,1)*20; W [256,256]."""
    rx, rw = _streams(seed)
    x = background(rx, 16, 256)
    for d in (7, 200):
        x[:, d] = rx.standard_normal(16, dtype=np.float32) * np.float32(20.0)
    W_t = weights(rw, 256, 256)
    return dict(X=x.astype(np.float16), W_t=W_t, threshold=6.0, dims=np.array([7, 200]))


def up_proj_1p3b(seed=0):
    """X [2048,2048], 3 dims +-U(8,30) in 25 % of rows; W [2048,8192]."""
    X, W_t, dims = case(2048, 2048, 8192, n_dims=3, lo=8.0, hi=30.0, p=0.25, seed=seed)
    return dict(X=X, W_t=W_t, threshold=6.0, dims=dims)


def ffn_6p7b(seed=0, with_fc2=True):
    """X [4096,4096], 6 dims +-U(20,60) in 75 % of rows; W1 [4096,16384], W2 [16384,4096]."""
    rx, rw = _streams(seed)
    x = background(rx, 4096, 4096)
    dims = plant_outliers(rx, x, 6, 20.0, 60.0, 0.75)
    W1_t = weights(rw, 16384, 4096)
    d = dict(X=x.astype(np.float16), W_t=W1_t, threshold=6.0, dims=dims)
    if with_fc2:
        d["W2_t"] = weights(rw, 4096, 16384)
    return d


def decode_175b(T, seed=0, with_weight=True):
    """X [T,12288], 6 dims +-U(20,60) in every row; W [12288,49152] (604 MB as int8)."""
    rx, rw = _streams(seed)
    x = background(rx, T, 12288)
    dims = plant_outliers(rx, x, 6, 20.0, 60.0, 1.0)
    d = dict(X=x.astype(np.float16), threshold=6.0, dims=dims)
    if with_weight:
        d["W_t"] = weights(rw, 49152, 12288)
    return d


def attn_proj_sweep(n_dims=6, T=4096, seed=0, with_weight=True):
    """X [4096,12288] with n_dims dims +-U(10,100) in 75 % of rows; W [12288,12288].

    T < 4096 takes the first T rows of the same draw (the ragged case)."""
    rx, rw = _streams(seed)
    x = background(rx, 4096, 12288)
    dims = plant_outliers(rx, x, n_dims, 10.0, 100.0, 0.75)
    d = dict(X=x[:T].astype(np.float16), threshold=6.0, dims=dims)
    if with_weight:
        d["W_t"] = weights(rw, 12288, 12288)
    return d
