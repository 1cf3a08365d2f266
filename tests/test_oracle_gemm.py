"""Pins of the oracle GEMM (CPU only).

The oracle computes R[m][n] = sA[m] sB[n] sum_k a(m,k) b(k,n) on rcr operands.
It is pinned by closed forms (identity B, all-ones operands), by an
independent pure-Python triple loop written from the rcr index definition on
small shapes with padded leading dimensions, and by its per-element form.  A
transposed operand, a wrong leading dimension, a dropped scale or a wrong sign
fails at least one of these.
"""

import numpy as np
import pytest

from oracle import codecs
from oracle.gemm import gemm, gemm_entry


def rand_codes(fmt, shape, rng, lo=-3, hi=3):
    vals = rng.integers(lo, hi + 1, size=shape).astype(np.float64) / 2
    return codecs.encode(fmt, vals)


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e4m3", "e5m2"])
def test_identity_b_gives_scaled_a(fmt):
    rng = np.random.default_rng(1)
    M, K = 7, 12
    a = rand_codes(fmt, (M, K), rng)
    eye = codecs.encode(fmt, np.eye(K))          # column-major identity == identity
    sa = 2.0 ** rng.integers(-2, 3, size=M)
    sb = 2.0 ** rng.integers(-2, 3, size=K)
    r = gemm(fmt, a, eye, M, K, K, scale_a=sa, scale_b=sb)
    expect = codecs.decode(fmt, a) * sa[:, None] * sb[None, :]
    assert np.array_equal(r, expect)


def test_all_ones_gives_k():
    M, N, K = 5, 9, 33
    one = codecs.encode("f16", np.ones(M * K))
    oneb = codecs.encode("f16", np.ones(N * K))
    assert np.array_equal(gemm("f16", one, oneb, M, N, K), np.full((M, N), float(K)))


@pytest.mark.parametrize("fmt", ["f16", "bf16", "e4m3", "e5m2"])
def test_matches_triple_loop_with_leading_dimensions(fmt):
    rng = np.random.default_rng(2)
    M, N, K, lda, ldb = 5, 4, 6, 9, 8
    a = rand_codes(fmt, (M * lda,), rng)
    b = rand_codes(fmt, (N * ldb,), rng)
    sa = rng.uniform(0.5, 2, M).astype(np.float32)
    sb = rng.uniform(0.5, 2, N).astype(np.float32)
    r = gemm(fmt, a, b, M, N, K, lda=lda, ldb=ldb, scale_a=sa, scale_b=sb)
    av = [float(v) for v in codecs.decode(fmt, a)]
    bv = [float(v) for v in codecs.decode(fmt, b)]
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += av[m * lda + k] * bv[n * ldb + k]   # A row-major, B column-major
            expect = acc * float(sa[m]) * float(sb[n])
            assert r[m, n] == pytest.approx(expect, rel=1e-14, abs=1e-14)
            assert gemm_entry(fmt, a, b, m, n, K, lda, ldb, sa, sb) == pytest.approx(expect, rel=1e-14, abs=1e-14)


def test_nonsymmetric_hand_example():
    # A = [[1, 2], [3, 4]] (row-major), B = [[5, 6], [7, 8]] stored column-major
    # as [5, 7, 6, 8]; A @ B = [[19, 22], [43, 50]].
    a = codecs.encode("f16", [1, 2, 3, 4])
    b = codecs.encode("f16", [5, 7, 6, 8])
    assert gemm("f16", a, b, 2, 2, 2).tolist() == [[19.0, 22.0], [43.0, 50.0]]


def test_rejects_short_buffers():
    with pytest.raises(ValueError):
        gemm("f16", np.zeros(5, np.uint16), np.zeros(6, np.uint16), 2, 2, 3)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_per_tensor_scales_by_triple_loop(fmt):
    # One scale for all of A and one for all of B (per-tensor quantisation):
    # an independent loop, and the per-element form.
    rng = np.random.default_rng(3)
    M, N, K = 4, 5, 7
    a = rand_codes(fmt, (M * K,), rng)
    b = rand_codes(fmt, (N * K,), rng)
    sa, sb = np.float32(1.75), np.float32(0.375)
    r = gemm(fmt, a, b, M, N, K, scale_a=[sa], scale_b=[sb], scale_mode="tensor")
    av = [float(v) for v in codecs.decode(fmt, a)]
    bv = [float(v) for v in codecs.decode(fmt, b)]
    for m in range(M):
        for n in range(N):
            acc = sum(av[m * K + k] * bv[n * K + k] for k in range(K))
            assert r[m, n] == pytest.approx(acc * float(sa) * float(sb), rel=1e-14, abs=1e-14)
            e = gemm_entry(fmt, a, b, m, n, K, scale_a=[sa], scale_b=[sb], scale_mode="tensor")
            assert e == pytest.approx(r[m, n], rel=1e-14, abs=1e-14)
    with pytest.raises(ValueError):
        gemm(fmt, a, b, M, N, K, scale_a=[sa, sa], scale_mode="tensor")
    with pytest.raises(ValueError):
        gemm(fmt, a, b, M, N, K, scale_mode="block")


# --- MX (e8m0 block-scaled) GEMM -------------------------------------------
from oracle.gemm import MX_BLOCK, gemm_mx, gemm_mx_entry  # noqa: E402


def mx_operands(rng, M, N, K, fmt="e4m3", lo=120, hi=134):
    a = codecs.encode(fmt, rng.integers(-6, 7, size=M * K).astype(np.float64) / 4)
    b = codecs.encode(fmt, rng.integers(-6, 7, size=N * K).astype(np.float64) / 4)
    sa = rng.integers(lo, hi + 1, size=M * (K // MX_BLOCK)).astype(np.uint8)
    sb = rng.integers(lo, hi + 1, size=N * (K // MX_BLOCK)).astype(np.uint8)
    return a, b, sa, sb


def test_mx_equal_block_scales_is_per_tensor():
    # Every block scale equal: 2^(ea-127) * 2^(eb-127) times the plain GEMM,
    # which is the per-tensor scaled GEMM of the pinned oracle.
    rng = np.random.default_rng(21)
    M, N, K = 9, 7, 128
    a, b, _, _ = mx_operands(rng, M, N, K)
    sa = np.full(M * 4, 130, np.uint8)
    sb = np.full(N * 4, 124, np.uint8)
    got = gemm_mx("e4m3", a, b, sa, sb, M, N, K)
    ref = gemm("e4m3", a, b, M, N, K, scale_a=[2.0 ** 3], scale_b=[2.0 ** -3], scale_mode="tensor")
    assert np.array_equal(got, ref)


def test_mx_row_constant_scales_are_rowcol():
    # Scales that vary by row (column) but not by block: the per-row /
    # per-column scaled GEMM.
    rng = np.random.default_rng(22)
    M, N, K = 6, 5, 96
    a, b, _, _ = mx_operands(rng, M, N, K, "e5m2")
    ea = rng.integers(120, 135, size=M)
    eb = rng.integers(120, 135, size=N)
    sa = np.repeat(ea, K // MX_BLOCK).astype(np.uint8)
    sb = np.repeat(eb, K // MX_BLOCK).astype(np.uint8)
    got = gemm_mx("e5m2", a, b, sa, sb, M, N, K)
    ref = gemm("e5m2", a, b, M, N, K, scale_a=2.0 ** (ea - 127.0), scale_b=2.0 ** (eb - 127.0))
    assert np.array_equal(got, ref)


def test_mx_blocks_split_the_reduction():
    # R = sum over blocks of each block's scales times the plain GEMM of that
    # block's K slice (so a scale applied to the wrong block, or a block of
    # the wrong width, fails).
    rng = np.random.default_rng(23)
    M, N, K = 5, 4, 160
    a, b, sa, sb = mx_operands(rng, M, N, K)
    nb = K // MX_BLOCK
    A2, B2 = a.reshape(M, K), b.reshape(N, K)
    S_a, S_b = sa.reshape(M, nb), sb.reshape(N, nb)
    ref = np.zeros((M, N))
    for blk in range(nb):
        sl = slice(blk * MX_BLOCK, (blk + 1) * MX_BLOCK)
        part = gemm("e4m3", np.ascontiguousarray(A2[:, sl]), np.ascontiguousarray(B2[:, sl]),
                    M, N, MX_BLOCK)
        ref += part * (2.0 ** (S_a[:, blk:blk + 1] - 127.0)) * (2.0 ** (S_b[:, blk][None, :] - 127.0))
    assert np.array_equal(gemm_mx("e4m3", a, b, sa, sb, M, N, K), ref)


def test_mx_triple_loop_and_entry():
    rng = np.random.default_rng(24)
    M, N, K = 3, 4, 64
    a, b, sa, sb = mx_operands(rng, M, N, K)
    ad = codecs.decode("e4m3", a).reshape(M, K)
    bd = codecs.decode("e4m3", b).reshape(N, K)
    R = gemm_mx("e4m3", a, b, sa, sb, M, N, K)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                acc += ad[m, k] * bd[n, k] * 2.0 ** (int(sa[m * 2 + k // 32]) - 127) * \
                    2.0 ** (int(sb[n * 2 + k // 32]) - 127)
            assert R[m, n] == acc
            assert gemm_mx_entry("e4m3", a, b, sa, sb, m, n, K) == R[m, n]


def test_mx_rejects_partial_blocks():
    with pytest.raises(ValueError):
        gemm_mx("e4m3", np.zeros(40, np.uint8), np.zeros(40, np.uint8), np.zeros(1, np.uint8),
                np.zeros(1, np.uint8), 1, 1, 40)
