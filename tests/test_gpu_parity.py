"""GPU parity of every entry point against the CPU oracle, on small and medium
shapes that span several tiles and ragged tails.

Bar: bit-exact CB, SCB, outlier list and count, row scales, Xq and the int32
accumulators; fp16 output within |d| <= 1e-3 + 2e-3*|ref| (infinities equal).
Inputs come only from the seeded generator; expected values only from the
oracle.  Everything goes through the C ABI (via the ctypes binding).
"""
import numpy as np
import pytest
import torch

import oracle
from int8_quantized_matmul_02_amd import llmint8 as L
from int8_quantized_matmul_02_amd import workloads
from tests.gpu_helpers import (assert_equal_exact, assert_fp16_close, bits, d2h, dev, h2d, say)

pytestmark = pytest.mark.gpu

SHAPES = [
    # (T, K, N)
    (1, 64, 64),
    (16, 256, 256),
    (17, 128, 192),
    (100, 320, 320),
    (129, 512, 384),
    (300, 576, 640),
    (513, 1024, 256),
    (1030, 320, 320),   # w_out gathered both ways (threshold 6: up to 32 outliers; 0: all)
]


@pytest.mark.parametrize("N,K", [(64, 64), (256, 256), (192, 1088), (1024, 2048)])
def test_quantize_weight_exact(N, K):
    say("quantize_weight N=%d K=%d" % (N, K))
    _, W_t, _ = workloads.case(1, K, N, n_dims=0, seed=N + K)
    W_t[N // 2] = 0.0                      # an all-zero output column
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    CBr, SCBr = oracle.quantize_weight(W_t)
    assert_equal_exact(d2h(CB), CBr, "CB")
    assert_equal_exact(d2h(SCB), SCBr, "SCB")


# Few rows take the one-launch kernel (T = 1 with K <= 65536, (1, 65536) at
# the limit; T <= 16 with K <= 16384, (4, 16384) and (16, 16384) at it); the
# rest, (1, 65600), (4, 16448), (16, 16448) and (17, 1024) just past, the
# three-kernel chain.  (2048, 1088) and (2304, 576) have the detection split
# into 8 row ranges with an 8-byte tail of flags per range (K % 128 = 64),
# which the row kernels' blocks OR across lanes.
@pytest.mark.parametrize("T,K", [(1, 64), (16, 256), (100, 320), (513, 1024), (2000, 2048),
                                 (1, 133120), (1, 65536), (1, 65600), (2, 12288), (3, 1088),
                                 (4, 16384), (4, 16448), (9, 12288), (16, 16384), (16, 16448),
                                 (17, 1024), (1027, 640), (1024, 16384), (1024, 16448),
                                 (2048, 1088), (2304, 576)])
@pytest.mark.parametrize("thr", [6.0, 0.0, np.inf, 2.5])
def test_quantize_act_exact(T, K, thr):
    say("quantize_act T=%d K=%d thr=%s" % (T, K, thr))
    X, _, dims = workloads.case(T, K, 64, n_dims=min(5, K // 16), lo=8, hi=40, p=0.4, seed=T * 7 + K)
    if T > 3:
        X[3] = 0.0                         # an all-zero row
    X[:, K - 1] = 0.0                      # an all-zero column
    X[T // 2, 5] = 6.0                     # exactly at the threshold: not an outlier at 6.0
    Xq, a, O, n = L.llmint8_quantize_act(h2d(X), thr)
    Or = oracle.outlier_columns(X, thr)
    Xqr, ar = oracle.quantize_rows(X, Or)
    n_g = int(d2h(n)[0])
    assert n_g == Or.size, (n_g, Or.size)
    assert_equal_exact(d2h(O)[:n_g], Or, "O")
    assert_equal_exact(d2h(a), ar, "row absmax")
    assert_equal_exact(d2h(Xq), Xqr, "Xq")


@pytest.mark.parametrize("T,K,N", SHAPES + [(16, 133120, 64), (40, 133120, 64)])
@pytest.mark.parametrize("path", [L.PATH_AUTO, L.PATH_GEMM, L.PATH_DECODE])
def test_igemm_i32_exact(T, K, N, path):
    if path == L.PATH_DECODE and T > 16:
        pytest.skip("the weight-streaming kernel takes T <= 16")
    say("igemm_i32 T=%d K=%d N=%d path=%d" % (T, K, N, path))
    rng = np.random.default_rng(T + K + N)
    if K == 133120:     # the largest supported K with every product at +-127^2: int32 extremes
        A = np.full((T, K), 127, np.int8)
        A[1::2] = -127
        B = np.full((N, K), 127, np.int8)
        B[::3] = -127
    else:
        A = rng.integers(-127, 128, (T, K)).astype(np.int8)
        B = rng.integers(-127, 128, (N, K)).astype(np.int8)
    C = L.llmint8_igemm_i32(h2d(A), h2d(B), path=path)
    Cr = oracle.int_gemm(A, B)
    assert_equal_exact(d2h(C), Cr, "C")


@pytest.mark.parametrize("T,K,N", SHAPES)
@pytest.mark.parametrize("thr", [6.0, 0.0, np.inf])
@pytest.mark.parametrize("use_bias", [False, True])
def test_matmul_parity(T, K, N, thr, use_bias):
    say("matmul T=%d K=%d N=%d thr=%s bias=%s" % (T, K, N, thr, use_bias))
    X, W_t, dims = workloads.case(T, K, N, n_dims=min(6, K // 16), lo=8, hi=60, p=0.5,
                                  seed=T + 3 * K + 5 * N)
    bias = (np.random.default_rng(7).standard_normal(N)).astype(np.float16) if use_bias else None
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, ar = oracle.matmul(X, CBr, SCBr, thr, bias=bias)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    paths = [L.PATH_AUTO, L.PATH_GEMM] + ([L.PATH_DECODE] if T <= 16 else [])
    for p in paths:
        out = L.llmint8_matmul_path(h2d(X), CB, SCB, thr, bias=h2d(bias) if use_bias else None, path=p)
        assert_fp16_close(d2h(out), ref, "out path=%d" % p)


# K values for the weight-streaming kernel (512 bytes of each weight row per
# stage, rotation period 6): one stage shorter than, equal to and just over a
# stage; every remainder length 1..6 after whole periods; a partial last
# stage overlapping the one before it.
DECODE_K = [64, 448, 512, 576, 1024, 1536, 2048, 2560, 3072, 3584, 4160, 6656]


@pytest.mark.parametrize("T", [1, 2, 5, 9, 16])
@pytest.mark.parametrize("K", DECODE_K)
def test_decode_path_shapes(T, K):
    """Weight-streaming path across its stage counts; T = 1/2 crosses from
    row-major to fragment-ordered activations (the one-launch quantization
    serves all of these shapes)."""
    N = 192
    say("decode shapes T=%d K=%d N=%d" % (T, K, N))
    X, W_t, _ = workloads.case(T, K, N, n_dims=min(6, K // 16), lo=8, hi=60, p=0.5, seed=K + T)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, 6.0)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_path(h2d(X), CB, SCB, 6.0, path=L.PATH_DECODE)
    assert_fp16_close(d2h(out), ref, "out")
    rng = np.random.default_rng(K * 17 + T)
    A = rng.integers(-127, 128, (T, K)).astype(np.int8)
    C = L.llmint8_igemm_i32(h2d(A), CB, path=L.PATH_DECODE)
    assert_equal_exact(d2h(C), oracle.int_gemm(A, CBr), "C")


def test_matmul_entry_point_matches_path_auto():
    X, W_t, _ = workloads.case(200, 256, 192, n_dims=3, seed=3)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    Xd = h2d(X)
    a = d2h(L.llmint8_matmul(Xd, CB, SCB, 6.0))
    b = d2h(L.llmint8_matmul_path(Xd, CB, SCB, 6.0, path=L.PATH_AUTO))
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_overflow_to_inf():
    """Integer inputs with absmax 127 give an exact product beyond 65504: +-inf on both sides."""
    T, K, N = 32, 64, 64
    X = np.full((T, K), 127.0, np.float16)
    X[1::2] *= -1
    W_t = np.full((N, K), 127.0, np.float16)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, 1000.0)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    for p in (L.PATH_GEMM,):
        out = d2h(L.llmint8_matmul_path(h2d(X), CB, SCB, 1000.0, path=p))
        assert_fp16_close(out, ref, "overflow")
    assert np.all(np.isinf(bits(ref).view(np.float16)))


def test_error_statuses():
    d = dev()
    X = torch.zeros((4, 64), dtype=torch.float16, device=d)
    CB = torch.zeros((64, 64), dtype=torch.int8, device=d)
    SCB = torch.zeros((64,), dtype=torch.float32, device=d)
    with pytest.raises(L.LLMInt8Error) as e:
        L.llmint8_matmul(X, CB, SCB, float("nan"))
    assert e.value.status == 1
    with pytest.raises(L.LLMInt8Error) as e:
        L.llmint8_matmul(X, CB, SCB, -1.0)
    assert e.value.status == 1
    X2 = torch.zeros((4, 96), dtype=torch.float16, device=d)
    CB2 = torch.zeros((64, 96), dtype=torch.int8, device=d)
    with pytest.raises(L.LLMInt8Error) as e:
        L.llmint8_matmul(X2, CB2, SCB, 6.0)
    assert e.value.status == 2
    ws = torch.empty((16,), dtype=torch.uint8, device=d)
    with pytest.raises(L.LLMInt8Error) as e:
        L.llmint8_matmul(X, CB, SCB, 6.0, ws=ws)
    assert e.value.status == 3
    Xbig = torch.zeros((17, 64), dtype=torch.float16, device=d)
    with pytest.raises(L.LLMInt8Error) as e:
        L.llmint8_matmul_path(Xbig, CB, SCB, 6.0, path=L.PATH_DECODE)
    assert e.value.status == 2
    # nothing was written by the rejected calls
    out = torch.full((4, 64), 7.0, dtype=torch.float16, device=d)
    with pytest.raises(L.LLMInt8Error):
        L.llmint8_matmul(X, CB, SCB, float("nan"), out=out)
    assert bool((out == 7.0).all())


def test_stream_asynchrony_and_ordering():
    """Calls enqueue on the caller's current stream without synchronizing it."""
    X, W_t, _ = workloads.case(256, 512, 512, n_dims=3, seed=9)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, 6.0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Xd = h2d(X)
        CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
        out = L.llmint8_matmul(Xd, CB, SCB, 6.0)
        ev = torch.cuda.Event()
        ev.record(s)
    ev.synchronize()
    assert_fp16_close(out.cpu().numpy(), ref, "side stream")


# One activation row: the one-launch quantization serves K up to 65536 (the
# separate three-kernel chain takes over past it).  Outlier counts around 1024
# and well past it (the weight-streaming epilogue walks the outlier list in
# groups of 8), every column an outlier (threshold 0), none (threshold inf),
# and K at and past 16384 (the limit of the few-rows kernel for T > 1).
@pytest.mark.parametrize("K,n_dims,thr", [(8192, 1023, 6.0), (8192, 1024, 6.0), (8192, 1025, 6.0),
                                           (8192, 3000, 6.0), (16384, 6, 0.0), (16384, 6, np.inf),
                                           (12288, 6, 6.0), (16448, 6, 6.0)])
@pytest.mark.parametrize("relu", [False, True])
def test_one_row_decode(K, n_dims, thr, relu):
    N = 320
    say("one-row decode K=%d n_dims=%d thr=%s relu=%s" % (K, n_dims, thr, relu))
    X, W_t, dims = workloads.case(1, K, N, n_dims=n_dims, lo=8, hi=60, p=1.0, seed=K + n_dims)
    bias = np.random.default_rng(K).standard_normal(N).astype(np.float16)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, _ = oracle.matmul(X, CBr, SCBr, thr, bias=bias, relu=relu)
    if np.isfinite(thr) and thr > 0:
        assert Or.size == n_dims
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_act(h2d(X), CB, SCB, thr, L.ACT_RELU if relu else L.ACT_NONE,
                               bias=h2d(bias))
    assert_fp16_close(d2h(out), ref, "one-row decode")


# The tiled GEMM switches from 8 wavefronts (128 x 64 each) to 4 (128 x 128)
# above K = 6144: both sides of the switch, each output kernel template (bias
# on and off, ReLU on and off), up to 32 outlier columns.
@pytest.mark.parametrize("K", [6144, 6272])
@pytest.mark.parametrize("use_bias", [False, True])
@pytest.mark.parametrize("relu", [False, True])
def test_gemm_wave_shapes_around_switch(K, use_bias, relu):
    T, N = 300, 320
    say("gemm switch K=%d bias=%s relu=%s" % (K, use_bias, relu))
    X, W_t, dims = workloads.case(T, K, N, n_dims=20, lo=8, hi=60, p=0.5, seed=K + 7)
    bias = np.random.default_rng(K).standard_normal(N).astype(np.float16) if use_bias else None
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, _ = oracle.matmul(X, CBr, SCBr, 6.0, bias=bias, relu=relu)
    assert 0 < Or.size <= 32
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_act(h2d(X), CB, SCB, 6.0, L.ACT_RELU if relu else L.ACT_NONE,
                               bias=h2d(bias) if use_bias else None)
    assert_fp16_close(d2h(out), ref, "out")


# Decode shapes past the few-rows kernel's K limit (2 <= T <= 16, K > 16384):
# the three-kernel quantization writes Xq in the fragment order the
# weight-streaming kernel reads.
@pytest.mark.parametrize("T,K", [(4, 16448), (16, 24576)])
@pytest.mark.parametrize("thr", [6.0, 0.0, np.inf])
def test_decode_past_few_rows_limit(T, K, thr):
    N = 256
    say("decode past the few-rows limit T=%d K=%d thr=%s" % (T, K, thr))
    X, W_t, _ = workloads.case(T, K, N, n_dims=6, lo=8, hi=60, p=1.0, seed=T + K)
    bias = np.random.default_rng(T).standard_normal(N).astype(np.float16)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, _, _ = oracle.matmul(X, CBr, SCBr, thr, bias=bias)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_path(h2d(X), CB, SCB, thr, bias=h2d(bias), path=L.PATH_DECODE)
    assert_fp16_close(d2h(out), ref, "out")


def test_concurrent_streams():
    """Two default-priority streams each run their own shape (a GEMM-path and a
    weight-streaming call, with their own outputs and workspaces) at the same
    time, several calls deep; both results against the oracle."""
    cases = [workloads.case(1000, 1024, 768, n_dims=5, seed=21),
             workloads.case(8, 2048, 1024, n_dims=4, seed=22)]
    refs, ops = [], []
    for X, W_t, _ in cases:
        CBr, SCBr = oracle.quantize_weight(W_t)
        refs.append(oracle.matmul(X, CBr, SCBr, 6.0)[0])
        CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
        ops.append((h2d(X), CB, SCB))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for s, (Xd, CB, SCB) in zip(streams, ops):
        with torch.cuda.stream(s):
            ws = torch.empty((L.llmint8_workspace_bytes(Xd.shape[0], Xd.shape[1], CB.shape[0]),),
                             dtype=torch.uint8, device=Xd.device)
            out = torch.empty((Xd.shape[0], CB.shape[0]), dtype=torch.float16, device=Xd.device)
            outs.append((out, ws))
    for rep in range(4):
        for s, (Xd, CB, SCB), (out, ws) in zip(streams, ops, outs):
            with torch.cuda.stream(s):
                L.llmint8_matmul(Xd, CB, SCB, 6.0, out=out, ws=ws)
    torch.cuda.synchronize()
    for (out, _), ref, what in zip(outs, refs, ("GEMM stream", "decode stream")):
        assert_fp16_close(out.cpu().numpy(), ref, what)


# More than 32 outlier columns on the GEMM path: the fp16 pass reads either
# compact gathered operands (scattered outliers, at most 1024 of them after
# padding) or X and CB in place over the 64-column groups that hold outliers,
# with the non-outlier columns of each group masked (clustered outliers, or
# more than 1024).  Cases on both sides of each choice, a K whose stages are
# 64 bytes (K % 128 != 0), ragged T and N, bias and ReLU.
def _planted(T, K, N, cols, seed, lo=8.0, hi=60.0, p=0.6):
    X, W_t, _ = workloads.case(T, K, N, n_dims=0, seed=seed)
    rng = np.random.default_rng(seed + 1)
    X = X.astype(np.float32)
    for c in cols:
        rows = rng.random(T) < p
        rows[rng.integers(T)] = True      # every planted column holds an outlier
        X[rows, c] = rng.uniform(lo, hi, rows.sum()) * np.where(rng.random(rows.sum()) < 0.5, -1, 1)
    return X.astype(np.float16), W_t


MANY_CASES = {
    # name: (T, K, N, columns)
    "compact33": (300, 4096, 320, np.arange(33) * 97 + 5),
    "compact200": (260, 4160, 384, np.arange(200) * 20 + 3),
    "compact1000": (300, 8192, 256, np.arange(1000) * 8 + 1),
    "dense1030_spread": (300, 8256, 320, np.arange(1030) * 8 + 2),
    "dense_clustered": (513, 4096, 320, np.arange(1000, 1200)),
    "dense_partial_groups": (300, 4160, 448, np.concatenate([np.arange(64, 128), [130, 199, 4100],
                                                            np.arange(2048, 2048 + 61)])),
}


@pytest.mark.parametrize("case", sorted(MANY_CASES))
@pytest.mark.parametrize("use_bias,relu", [(False, False), (True, True)])
def test_many_outliers_compact_and_dense(case, use_bias, relu):
    T, K, N, cols = MANY_CASES[case]
    say("many outliers %s T=%d K=%d N=%d n=%d bias=%s relu=%s" % (case, T, K, N, len(cols), use_bias, relu))
    X, W_t = _planted(T, K, N, cols, seed=len(cols) + K)
    bias = np.random.default_rng(N).standard_normal(N).astype(np.float16) if use_bias else None
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, _ = oracle.matmul(X, CBr, SCBr, 6.0, bias=bias, relu=relu)
    assert Or.size == len(cols)
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_act(h2d(X), CB, SCB, 6.0, L.ACT_RELU if relu else L.ACT_NONE,
                               bias=h2d(bias) if use_bias else None)
    assert_fp16_close(d2h(out), ref, case)


# Kept-column mode of the int8 part: with T >= 512 rows and the kept
# (non-outlier) columns rounded up to 128 at most a quarter of K, the int8
# product runs over the compacted kept columns only.  Cases at the quarter
# (kc = K/4) and one column past it, one row short of 512, a ragged T, a K
# whose stages are 64 bytes, a wider K, more weight rows than rows (a row
# block builds several compacted weight rows), and a K past one 16 KB round
# of the weight-row compaction (a second, partial round).
KEPT_CASES = {
    # name: (T, K, N, number of outlier columns, drawn at random)
    "kept_at_cap": (512, 1024, 320, 768),
    "kept_past_cap": (512, 1024, 256, 767),
    "kept_one_row_short": (511, 1024, 320, 800),
    "kept_ragged_T": (600, 2048, 256, 1600),
    "kept_k64_stages": (512, 1088, 256, 900),
    "kept_wide": (1024, 4096, 512, 3500),
    "kept_n_past_t": (512, 1024, 1280, 800),
    "kept_two_rounds": (512, 17408, 128, 14000),
}


@pytest.mark.parametrize("case", sorted(KEPT_CASES))
@pytest.mark.parametrize("use_bias,relu", [(False, False), (True, True)])
def test_kept_column_mode(case, use_bias, relu):
    T, K, N, n = KEPT_CASES[case]
    say("kept columns %s T=%d K=%d N=%d n=%d bias=%s relu=%s" % (case, T, K, N, n, use_bias, relu))
    cols = np.sort(np.random.default_rng(K + n).choice(K, n, replace=False))
    X, W_t = _planted(T, K, N, cols, seed=n + K)
    bias = np.random.default_rng(N).standard_normal(N).astype(np.float16) if use_bias else None
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, _ = oracle.matmul(X, CBr, SCBr, 6.0, bias=bias, relu=relu)
    assert Or.size == n
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    out = L.llmint8_matmul_act(h2d(X), CB, SCB, 6.0, L.ACT_RELU if relu else L.ACT_NONE,
                               bias=h2d(bias) if use_bias else None)
    assert_fp16_close(d2h(out), ref, case)


@pytest.mark.parametrize("T", [300, 512])
@pytest.mark.parametrize("thr", [0.0, 0.4])
def test_nearly_every_column_an_outlier(thr, T):
    """Threshold 0 with an all-zero column (n = K - 1: the int8 part still runs,
    and the group holding that column is masked), and a threshold that leaves a
    few small-valued columns out of the outlier set; with 512 rows the int8
    part takes the kept-column mode (at most 4 kept columns)."""
    K, N = 1088, 320
    say("nearly all outliers T=%d thr=%s" % (T, thr))
    X, W_t, _ = workloads.case(T, K, N, n_dims=0, seed=int(thr * 10) + 7)
    X = X.astype(np.float32)
    X[:, 100] = 0.0
    X[:, [5, 700, 1087]] *= 0.05
    X = X.astype(np.float16)
    CBr, SCBr = oracle.quantize_weight(W_t)
    ref, Or, _ = oracle.matmul(X, CBr, SCBr, thr)
    assert K - 4 <= Or.size < K
    CB, SCB = L.llmint8_quantize_weight(h2d(W_t))
    assert_fp16_close(d2h(L.llmint8_matmul(h2d(X), CB, SCB, thr)), ref, "out")
