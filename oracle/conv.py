"""Forward convolution and its input gradient (dgrad) by their definitions
(oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The other two convolutions of a layer, run as implicit GEMMs on the same
stream-K engine as the weight gradient (rocm-libraries PR #13151 "feat(rocke):
stream-K for implicit-GEMM conv wgrad": the "docs" commit points the
forward-convolution future-work note at the stream-K port, and review items
2-3 ask for forward convolution on the family-agnostic partitioner).  Layouts
and readings are those of ``oracle/wgrad.py``: NHWC activations, KRSC filter
(K x R x S x Cpg), ``Ho = (H + 2*pad_h - R) // stride_h + 1`` (likewise Wo),
dilation 1, group ``g`` maps input channels ``[g*Cpg, (g+1)*Cpg)`` to output
channels ``[g*Kpg, (g+1)*Kpg)``.

Forward:

    Y[n][ho][wo][k] = sum_{r, s, c'} X[n][ho*sh - ph + r][wo*sw - pw + s][g*Cpg + c']
                                     * W[k][r][s][c']            (g = k // Kpg)

with X taken as zero outside the image.

Input gradient: the adjoint of the forward map in X, i.e. every forward term
X[n][h][w][c] * W[k][r][s][c'] with h = ho*sh - ph + r, w = wo*sw - pw + s
contributes dY[n][ho][wo][k] * W[k][r][s][c'] to dX[n][h][w][c]:

    dX[n][h][w][g*Cpg + c'] = sum over (ho, wo, r, s, k in group g) with
                              ho*sh - ph + r = h and wo*sw - pw + s = w of
                              dY[n][ho][wo][k] * W[k][r][s][c'].

Both are evaluated in float64 on the decoded codes; numpy's float64 matmul
(a library primitive) does the per-tap, per-group channel contraction.
"""

import numpy as np

from .codecs import decode
from .wgrad import out_size, shifted_input


def _check(C, K, groups, ho, wo):
    if C % groups or K % groups:
        raise ValueError("groups must divide C and K")
    if ho <= 0 or wo <= 0:
        raise ValueError("empty output image")


def forward(fmt, x_codes, w_codes, N, H, W, C, K, R, S,
            stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """float64 Y with shape (N, Ho, Wo, K)."""
    ho, wo = out_size(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
    _check(C, K, groups, ho, wo)
    cpg, kpg = C // groups, K // groups
    x = decode(fmt, np.asarray(x_codes).reshape(N, H, W, C))
    w = decode(fmt, np.asarray(w_codes).reshape(K, R, S, cpg))
    y = np.zeros((N, ho, wo, K), dtype=np.float64)
    for r in range(R):
        for s in range(S):
            xs = shifted_input(x, r, s, ho, wo, stride_h, stride_w, pad_h, pad_w)
            for g in range(groups):
                y[..., g * kpg:(g + 1) * kpg] += (
                    xs[..., g * cpg:(g + 1) * cpg] @ w[g * kpg:(g + 1) * kpg, r, s, :].T)
    return y


def dgrad(fmt, dy_codes, w_codes, N, H, W, C, K, R, S,
          stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """float64 dX with shape (N, H, W, C)."""
    ho, wo = out_size(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
    _check(C, K, groups, ho, wo)
    cpg, kpg = C // groups, K // groups
    dy = decode(fmt, np.asarray(dy_codes).reshape(N, ho, wo, K))
    w = decode(fmt, np.asarray(w_codes).reshape(K, R, S, cpg))
    dx = np.zeros((N, H, W, C), dtype=np.float64)
    for r in range(R):
        hi = np.arange(ho) * stride_h - pad_h + r        # input row of each output row
        vh = (hi >= 0) & (hi < H)
        for s in range(S):
            wi = np.arange(wo) * stride_w - pad_w + s
            vw = (wi >= 0) & (wi < W)
            for g in range(groups):
                # contribution of tap (r, s) at every output pixel: (N, Ho, Wo, Cpg)
                t = dy[..., g * kpg:(g + 1) * kpg] @ w[g * kpg:(g + 1) * kpg, r, s, :]
                t = t[:, vh][:, :, vw]
                # distinct output pixels of one tap land on distinct input
                # pixels, so one fancy-indexed add per tap is exact
                dx[:, hi[vh][:, None], wi[vw][None, :], g * cpg:(g + 1) * cpg] += t
    return dx


def forward_entry(fmt, x_codes, w_codes, N, H, W, C, K, R, S, n, ho, wo, k,
                  stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """One output element Y[n][ho][wo][k] computed on its own."""
    cpg, kpg = C // groups, K // groups
    g = k // kpg
    x = np.asarray(x_codes).reshape(N, H, W, C)
    w = np.asarray(w_codes).reshape(K, R, S, cpg)
    acc = 0.0
    for r in range(R):
        h = ho * stride_h - pad_h + r
        if not 0 <= h < H:
            continue
        for s in range(S):
            wi = wo * stride_w - pad_w + s
            if not 0 <= wi < W:
                continue
            acc += float(np.dot(decode(fmt, x[n, h, wi, g * cpg:(g + 1) * cpg]),
                                decode(fmt, w[k, r, s, :])))
    return acc


def dgrad_entry(fmt, dy_codes, w_codes, N, H, W, C, K, R, S, n, h, w_, c,
                stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """One input-gradient element dX[n][h][w_][c] computed on its own."""
    ho_n, wo_n = out_size(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
    cpg, kpg = C // groups, K // groups
    g, cc = c // cpg, c % cpg
    dy = np.asarray(dy_codes).reshape(N, ho_n, wo_n, K)
    w = np.asarray(w_codes).reshape(K, R, S, cpg)
    acc = 0.0
    for r in range(R):
        t = h + pad_h - r
        if t % stride_h or not 0 <= t // stride_h < ho_n:
            continue
        for s in range(S):
            u = w_ + pad_w - s
            if u % stride_w or not 0 <= u // stride_w < wo_n:
                continue
            acc += float(np.dot(decode(fmt, dy[n, t // stride_h, u // stride_w, g * kpg:(g + 1) * kpg]),
                                decode(fmt, w[g * kpg:(g + 1) * kpg, r, s, cc])))
    return acc
