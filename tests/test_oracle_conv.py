"""Pins of the oracle forward convolution and input gradient (CPU only).

Checked against: torch's float64 ``conv2d`` and ``conv2d_input`` (library
routines, NCHW, so layouts are permuted on the way in and out); the 1x1 /
stride-1 / no-padding case, which is the GEMM X W^T (forward) and dY W
(dgrad); the adjoint identity <fwd(X), dY> = <X, dgrad(dY)>, which ties the
two together and fails for a flipped, transposed or shifted filter; pure
Python loops over the definitions on tiny shapes; grouped convolution as
independent dense problems per group; and the single-element entries
against the whole result.
"""

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle.conv import dgrad, dgrad_entry, forward, forward_entry
from oracle.wgrad import out_size


def rand_codes(fmt, shape, rng):
    return codecs.encode(fmt, rng.integers(-4, 5, size=shape).astype(np.float64) / 4)


CASES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, groups
    (2, 5, 6, 3, 4, 3, 3, 1, 1, 1, 1, 1),
    (1, 7, 7, 4, 6, 3, 3, 2, 2, 1, 1, 2),
    (2, 6, 5, 8, 8, 3, 2, 2, 1, 1, 0, 4),
    (1, 4, 4, 2, 2, 1, 1, 1, 1, 0, 0, 1),
    (3, 5, 5, 6, 3, 2, 3, 1, 2, 0, 1, 3),
    (1, 8, 9, 4, 4, 3, 3, 3, 2, 2, 1, 1),
]


def operands(case, rng, fmt="bf16"):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    ho, wo = out_size(H, W, R, S, sh, sw, ph, pw)
    x = rand_codes(fmt, (N, H, W, C), rng)
    w = rand_codes(fmt, (K, R, S, C // g), rng)
    dy = rand_codes(fmt, (N, ho, wo, K), rng)
    return x, w, dy


def to_t(fmt, codes, perm):
    return torch.from_numpy(codecs.decode(fmt, codes)).permute(*perm)


@pytest.mark.parametrize("case", CASES)
def test_forward_matches_torch_conv2d(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    x, w, _ = operands(case, np.random.default_rng(sum(case)))
    y = forward("bf16", x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    ref = torch.nn.functional.conv2d(to_t("bf16", x, (0, 3, 1, 2)), to_t("bf16", w, (0, 3, 1, 2)),
                                     stride=(sh, sw), padding=(ph, pw), groups=g)
    ref = ref.permute(0, 2, 3, 1).numpy()
    assert y.shape == ref.shape
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_dgrad_matches_torch_conv2d_input(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    _, w, dy = operands(case, np.random.default_rng(sum(case) + 1))
    dx = dgrad("bf16", dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    ref = torch.nn.grad.conv2d_input((N, C, H, W), to_t("bf16", w, (0, 3, 1, 2)),
                                     to_t("bf16", dy, (0, 3, 1, 2)), stride=(sh, sw),
                                     padding=(ph, pw), groups=g)
    ref = ref.permute(0, 2, 3, 1).numpy()
    assert dx.shape == ref.shape
    assert np.allclose(dx, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("case", CASES)
def test_adjoint_identity(case):
    # <fwd(X), dY> = <X, dgrad(dY)> for any X, dY: dgrad is the adjoint of
    # the forward map.  With quarter-integer inputs both sides are exact.
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    x, w, dy = operands(case, np.random.default_rng(sum(case) + 2))
    y = forward("bf16", x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    dx = dgrad("bf16", dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    lhs = float(np.sum(y * codecs.decode("bf16", dy)))
    rhs = float(np.sum(codecs.decode("bf16", x) * dx))
    assert lhs == rhs


def test_pointwise_is_a_gemm():
    rng = np.random.default_rng(5)
    N, H, W, C, K = 2, 3, 4, 5, 6
    x = rand_codes("f16", (N, H, W, C), rng)
    w = rand_codes("f16", (K, 1, 1, C), rng)
    dy = rand_codes("f16", (N, H, W, K), rng)
    xm = codecs.decode("f16", x).reshape(-1, C)
    wm = codecs.decode("f16", w).reshape(K, C)
    dym = codecs.decode("f16", dy).reshape(-1, K)
    y = forward("f16", x, w, N, H, W, C, K, 1, 1)
    assert np.array_equal(y.reshape(-1, K), xm @ wm.T)
    dx = dgrad("f16", dy, w, N, H, W, C, K, 1, 1)
    assert np.array_equal(dx.reshape(-1, C), dym @ wm)


def loops_forward(x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g):
    ho, wo = out_size(H, W, R, S, sh, sw, ph, pw)
    cpg, kpg = C // g, K // g
    y = np.zeros((N, ho, wo, K))
    for n in range(N):
        for i in range(ho):
            for j in range(wo):
                for k in range(K):
                    gg = k // kpg
                    for r in range(R):
                        for s in range(S):
                            h, ww = i * sh - ph + r, j * sw - pw + s
                            if 0 <= h < H and 0 <= ww < W:
                                for c in range(cpg):
                                    y[n, i, j, k] += x[n, h, ww, gg * cpg + c] * w[k, r, s, c]
    return y


def loops_dgrad(dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g):
    ho, wo = out_size(H, W, R, S, sh, sw, ph, pw)
    cpg, kpg = C // g, K // g
    dx = np.zeros((N, H, W, C))
    for n in range(N):
        for i in range(ho):
            for j in range(wo):
                for k in range(K):
                    gg = k // kpg
                    for r in range(R):
                        for s in range(S):
                            h, ww = i * sh - ph + r, j * sw - pw + s
                            if 0 <= h < H and 0 <= ww < W:
                                for c in range(cpg):
                                    dx[n, h, ww, gg * cpg + c] += dy[n, i, j, k] * w[k, r, s, c]
    return dx


@pytest.mark.parametrize("case", CASES[:4])
def test_brute_force_loops(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    x, w, dy = operands(case, np.random.default_rng(sum(case) + 3), "f16")
    xd, wd, dyd = (codecs.decode("f16", a) for a in (x, w, dy))
    assert np.array_equal(forward("f16", x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g),
                          loops_forward(xd, wd, N, H, W, C, K, R, S, sh, sw, ph, pw, g))
    assert np.array_equal(dgrad("f16", dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g),
                          loops_dgrad(dyd, wd, N, H, W, C, K, R, S, sh, sw, ph, pw, g))


def test_grouped_is_per_group_dense():
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = 2, 6, 6, 8, 12, 3, 3, 2, 1, 1, 1, 4
    rng = np.random.default_rng(9)
    x, w, dy = operands((N, H, W, C, K, R, S, sh, sw, ph, pw, g), rng)
    y = forward("bf16", x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    dx = dgrad("bf16", dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    cpg, kpg = C // g, K // g
    for gg in range(g):
        xg = np.ascontiguousarray(x[..., gg * cpg:(gg + 1) * cpg])
        wg = np.ascontiguousarray(w[gg * kpg:(gg + 1) * kpg])
        dyg = np.ascontiguousarray(dy[..., gg * kpg:(gg + 1) * kpg])
        assert np.array_equal(y[..., gg * kpg:(gg + 1) * kpg],
                              forward("bf16", xg, wg, N, H, W, cpg, kpg, R, S, sh, sw, ph, pw, 1))
        assert np.array_equal(dx[..., gg * cpg:(gg + 1) * cpg],
                              dgrad("bf16", dyg, wg, N, H, W, cpg, kpg, R, S, sh, sw, ph, pw, 1))


@pytest.mark.parametrize("case", CASES)
def test_entries_equal_the_whole(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    x, w, dy = operands(case, np.random.default_rng(sum(case) + 4))
    y = forward("bf16", x, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    dx = dgrad("bf16", dy, w, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    rng = np.random.default_rng(1)
    for _ in range(12):
        n, i, j, k = (int(rng.integers(d)) for d in y.shape)
        assert forward_entry("bf16", x, w, N, H, W, C, K, R, S, n, i, j, k, sh, sw, ph, pw, g) == y[n, i, j, k]
        n, i, j, c = (int(rng.integers(d)) for d in dx.shape)
        assert dgrad_entry("bf16", dy, w, N, H, W, C, K, R, S, n, i, j, c, sh, sw, ph, pw, g) == dx[n, i, j, c]
