"""Pins of the oracle conv wgrad (CPU only).

Checked against: torch's float64 ``conv2d_weight`` (a library routine, NCHW,
so the layouts are permuted on the way in and out); the 1x1 / stride-1 /
no-padding special case, which is the GEMM dY^T X; a pure-Python loop over the
definition on tiny shapes; and the grouped case as independent dense problems
per group.  A wrong padding sign, a swapped r/s, a wrong group offset or a
transposed result fails one of these.
"""

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle.wgrad import out_size, wgrad, wgrad_entry


def rand_codes(fmt, shape, rng):
    return codecs.encode(fmt, rng.integers(-4, 5, size=shape).astype(np.float64) / 4)


CASES = [
    # N, H, W, C, K, R, S, sh, sw, ph, pw, groups
    (2, 5, 6, 3, 4, 3, 3, 1, 1, 1, 1, 1),
    (1, 7, 7, 4, 6, 3, 3, 2, 2, 1, 1, 2),
    (2, 6, 5, 8, 8, 3, 2, 2, 1, 1, 0, 4),
    (1, 4, 4, 2, 2, 1, 1, 1, 1, 0, 0, 1),
    (3, 5, 5, 6, 3, 2, 3, 1, 2, 0, 1, 3),
]


@pytest.mark.parametrize("case", CASES)
def test_matches_torch_conv2d_weight(case):
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = case
    rng = np.random.default_rng(sum(case))
    ho, wo = out_size(H, W, R, S, sh, sw, ph, pw)
    x = rand_codes("bf16", (N, H, W, C), rng)
    dy = rand_codes("bf16", (N, ho, wo, K), rng)
    dw = wgrad("bf16", x, dy, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    xt = torch.from_numpy(codecs.decode("bf16", x)).permute(0, 3, 1, 2)
    dyt = torch.from_numpy(codecs.decode("bf16", dy)).permute(0, 3, 1, 2)
    ref = torch.nn.grad.conv2d_weight(xt, (K, C // g, R, S), dyt, stride=(sh, sw),
                                      padding=(ph, pw), groups=g)
    ref = ref.permute(0, 2, 3, 1).numpy()          # KCRS -> KRSC
    assert dw.shape == ref.shape
    assert np.allclose(dw, ref, rtol=1e-12, atol=1e-12)


def test_pointwise_is_dyT_x():
    rng = np.random.default_rng(3)
    N, H, W, C, K = 2, 3, 4, 5, 6
    x = rand_codes("f16", (N, H, W, C), rng)
    dy = rand_codes("f16", (N, H, W, K), rng)
    dw = wgrad("f16", x, dy, N, H, W, C, K, 1, 1)
    xm = codecs.decode("f16", x).reshape(-1, C)
    dym = codecs.decode("f16", dy).reshape(-1, K)
    assert np.array_equal(dw[:, 0, 0, :], dym.T @ xm)


def test_matches_definition_loop():
    rng = np.random.default_rng(4)
    N, H, W, C, K, R, S, sh, sw, ph, pw, g = 2, 5, 4, 4, 4, 3, 2, 2, 1, 1, 1, 2
    ho, wo = out_size(H, W, R, S, sh, sw, ph, pw)
    x = rand_codes("f16", (N, H, W, C), rng)
    dy = rand_codes("f16", (N, ho, wo, K), rng)
    dw = wgrad("f16", x, dy, N, H, W, C, K, R, S, sh, sw, ph, pw, g)
    xv = codecs.decode("f16", x)
    dyv = codecs.decode("f16", dy)
    cpg, kpg = C // g, K // g
    for k in range(K):
        gi = k // kpg
        for r in range(R):
            for s in range(S):
                for c in range(cpg):
                    acc = 0.0
                    for n in range(N):
                        for i in range(ho):
                            for j in range(wo):
                                hi, wi = i * sh - ph + r, j * sw - pw + s
                                if 0 <= hi < H and 0 <= wi < W:
                                    acc += dyv[n, i, j, k] * xv[n, hi, wi, gi * cpg + c]
                    assert dw[k, r, s, c] == acc
                    assert wgrad_entry("f16", x, dy, N, H, W, C, K, R, S, k, r, s, c,
                                       sh, sw, ph, pw, g) == acc


def test_grouped_is_blockwise_dense():
    rng = np.random.default_rng(5)
    N, H, W, C, K, R, S, g = 2, 6, 6, 8, 4, 3, 3, 2
    ho, wo = out_size(H, W, R, S, 2, 2, 1, 1)
    x = rand_codes("bf16", (N, H, W, C), rng)
    dy = rand_codes("bf16", (N, ho, wo, K), rng)
    dw = wgrad("bf16", x, dy, N, H, W, C, K, R, S, 2, 2, 1, 1, g)
    cpg, kpg = C // g, K // g
    for gi in range(g):
        xs = np.ascontiguousarray(x[..., gi * cpg:(gi + 1) * cpg])
        dys = np.ascontiguousarray(dy[..., gi * kpg:(gi + 1) * kpg])
        dense = wgrad("bf16", xs, dys, N, H, W, cpg, kpg, R, S, 2, 2, 1, 1, 1)
        assert np.array_equal(dw[gi * kpg:(gi + 1) * kpg], dense)
