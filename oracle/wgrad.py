"""Backward-weight convolution by its definition (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Follows the wgrad problem of rocm-libraries PR #13151 ("feat(rocke): stream-K
for implicit-GEMM conv wgrad": Motivation, and the commit porting stream-K to
the backward-weight convolution): the filter gradient has the filter's size
while the reduction runs over every output pixel of every image.  Readings we
take where the page is silent:

* activations are NHWC: ``X[n][h][w][c]`` and ``dY[n][ho][wo][k]``;
* output size ``Ho = (H + 2*pad_h - R) // stride_h + 1`` (likewise ``Wo``),
  dilation 1;
* grouped convolution in the usual sense: group ``g`` maps input channels
  ``[g*Cpg, (g+1)*Cpg)`` to output channels ``[g*Kpg, (g+1)*Kpg)``;
* the gradient is laid out K x R x S x Cpg (KRSC), row-major.

Definition:

    dW[k][r][s][c'] = sum_{n, ho, wo} dY[n][ho][wo][k]
                      * X[n][ho*stride_h - pad_h + r][wo*stride_w - pad_w + s][g*Cpg + c']

with ``g = k // Kpg`` and a term of zero wherever the X index falls outside
the image (the padding).  No im2col matrix is formed: for each filter tap
(r, s) the shifted input is gathered and multiplied with dY by numpy's
float64 matmul, one group at a time.
"""

import numpy as np

from .codecs import decode


def out_size(h, w, r, s, stride_h, stride_w, pad_h, pad_w):
    ho = (h + 2 * pad_h - r) // stride_h + 1
    wo = (w + 2 * pad_w - s) // stride_w + 1
    return ho, wo


def shifted_input(x, r, s, ho, wo, stride_h, stride_w, pad_h, pad_w):
    """``xs[n][i][j][c] = X[n][i*stride_h - pad_h + r][j*stride_w - pad_w + s][c]``
    with zero outside the image."""
    n, h, w, c = x.shape
    hi = np.arange(ho) * stride_h - pad_h + r
    wi = np.arange(wo) * stride_w - pad_w + s
    vh = (hi >= 0) & (hi < h)
    vw = (wi >= 0) & (wi < w)
    xs = np.zeros((n, ho, wo, c), dtype=np.float64)
    sub = x[:, np.clip(hi, 0, h - 1)][:, :, np.clip(wi, 0, w - 1)]
    mask = (vh[:, None] & vw[None, :])[None, :, :, None]
    xs[...] = np.where(mask, sub, 0.0)
    return xs


def wgrad(fmt, x_codes, dy_codes, N, H, W, C, K, R, S,
          stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """float64 dW with shape (K, R, S, C // groups)."""
    if C % groups or K % groups:
        raise ValueError("groups must divide C and K")
    ho, wo = out_size(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
    if ho <= 0 or wo <= 0:
        raise ValueError("empty output image")
    cpg, kpg = C // groups, K // groups
    x = decode(fmt, np.asarray(x_codes).reshape(N, H, W, C))
    dy = decode(fmt, np.asarray(dy_codes).reshape(N, ho, wo, K))
    dy2 = dy.reshape(N * ho * wo, K)
    dw = np.zeros((K, R, S, cpg), dtype=np.float64)
    for r in range(R):
        for s in range(S):
            xs = shifted_input(x, r, s, ho, wo, stride_h, stride_w, pad_h, pad_w)
            xs2 = xs.reshape(N * ho * wo, C)
            for g in range(groups):
                dw[g * kpg:(g + 1) * kpg, r, s, :] = (
                    dy2[:, g * kpg:(g + 1) * kpg].T @ xs2[:, g * cpg:(g + 1) * cpg])
    return dw


def wgrad_entry(fmt, x_codes, dy_codes, N, H, W, C, K, R, S, k, r, s, c,
                stride_h=1, stride_w=1, pad_h=0, pad_w=0, groups=1):
    """One gradient element dW[k][r][s][c] computed on its own."""
    ho, wo = out_size(H, W, R, S, stride_h, stride_w, pad_h, pad_w)
    cpg, kpg = C // groups, K // groups
    g = k // kpg
    x = np.asarray(x_codes).reshape(N, H, W, C)
    dy = np.asarray(dy_codes).reshape(N, ho, wo, K)
    hi = np.arange(ho) * stride_h - pad_h + r
    wi = np.arange(wo) * stride_w - pad_w + s
    vh = (hi >= 0) & (hi < H)
    vw = (wi >= 0) & (wi < W)
    xv = decode(fmt, x[:, np.clip(hi, 0, H - 1)][:, :, np.clip(wi, 0, W - 1), g * cpg + c])
    xv = np.where((vh[:, None] & vw[None, :])[None], xv, 0.0)
    dv = decode(fmt, dy[:, :, :, k])
    return float(np.sum(xv * dv))
