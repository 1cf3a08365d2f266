"""Plain GEMM with optional per-row A and per-column B scales (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Definition followed ("gemm_rowcolquant dispatcher bridge" PR, final
description, scope section; and the stream-K GEMM bridge commit
"feat(ck-tile): stream-K GEMM TE to dispatcher bridge", Validation):

    R[m][n] = sA[m] * sB[n] * sum_{k < K} a(m, k) * b(k, n)

in the "rcr" layout: A row-major (element (m, k) at ``A[m*lda + k]``), B
column-major (element (k, n) at ``B[n*ldb + k]``), C row-major.  The scales
are float32 vectors of length M and N (``scale_mode="rowcol"``), or one
float each for the whole of A and of B (``scale_mode="tensor"``, the
per-tensor sibling "tensor_quant" named in that PR's final description:
sA[m] = sA, sB[n] = sB); an absent scale is 1.  Everything is
evaluated in float64 on the decoded input codes, so the result is the exact
product sum up to float64 rounding.  The matrix product itself is numpy's
float64 matmul (a library primitive); there is no blocking or reordering here.
"""

import numpy as np

from .codecs import decode, decode_e8m0


def operand_matrix(fmt, codes, rows, cols, ld):
    """Decode a ``rows x cols`` block stored with leading dimension ``ld``."""
    flat = np.asarray(codes).reshape(-1)
    if ld < cols:
        raise ValueError("leading dimension smaller than the row length")
    need = (rows - 1) * ld + cols if rows > 0 else 0
    if flat.size < need:
        raise ValueError("operand buffer too small")
    if rows == 0 or cols == 0:
        return np.zeros((rows, cols))
    padded = np.zeros(rows * ld, dtype=flat.dtype)
    padded[:need] = flat[:need]
    return decode(fmt, padded.reshape(rows, ld)[:, :cols])


def scale_vectors(scale_a, scale_b, M, N, scale_mode):
    """Per-row and per-column float64 scale vectors (None stays None)."""
    if scale_mode not in ("rowcol", "tensor"):
        raise ValueError("unknown scale mode")
    out = []
    for s, n in ((scale_a, M), (scale_b, N)):
        if s is None:
            out.append(None)
            continue
        s = np.asarray(s, dtype=np.float64).reshape(-1)
        if scale_mode == "tensor":
            if s.size != 1:
                raise ValueError("a per-tensor scale is one value")
            s = np.full(n, s[0])
        elif s.size != n:
            raise ValueError("scale length")
        out.append(s)
    return out


def gemm(fmt, a_codes, b_codes, M, N, K, lda=None, ldb=None,
         scale_a=None, scale_b=None, scale_mode="rowcol"):
    """float64 ``R`` (M x N) for rcr operands holding ``fmt`` codes."""
    scale_a, scale_b = scale_vectors(scale_a, scale_b, M, N, scale_mode)
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    a = operand_matrix(fmt, a_codes, M, K, lda)          # a[m][k]
    bt = operand_matrix(fmt, b_codes, N, K, ldb)         # bt[n][k] = b(k, n)
    r = a @ bt.T
    if scale_a is not None:
        r = r * np.asarray(scale_a, dtype=np.float64).reshape(M, 1)
    if scale_b is not None:
        r = r * np.asarray(scale_b, dtype=np.float64).reshape(1, N)
    return r


def gemm_entry(fmt, a_codes, b_codes, m, n, K, lda=None, ldb=None,
               scale_a=None, scale_b=None, scale_mode="rowcol"):
    """One output element R[m][n], computed on its own (for sampled checks of
    outputs too large to form whole)."""
    if scale_mode == "tensor":
        m_s = n_s = 0
    elif scale_mode == "rowcol":
        m_s, n_s = m, n
    else:
        raise ValueError("unknown scale mode")
    lda = K if lda is None else lda
    ldb = K if ldb is None else ldb
    a_row = decode(fmt, np.asarray(a_codes).reshape(-1)[m * lda: m * lda + K])
    b_col = decode(fmt, np.asarray(b_codes).reshape(-1)[n * ldb: n * ldb + K])
    v = float(np.dot(a_row, b_col))
    if scale_a is not None:
        v *= float(np.asarray(scale_a).reshape(-1)[m_s])
    if scale_b is not None:
        v *= float(np.asarray(scale_b).reshape(-1)[n_s])
    return v


# OCP Microscaling: one shared scale per block of this many consecutive
# elements along the reduction.
MX_BLOCK = 32


def gemm_mx(fmt, a_codes, b_codes, sa_codes, sb_codes, M, N, K):
    """float64 ``R`` (M x N) of a block-scaled (MX) GEMM in the rcr layout:

        R[m][n] = sum over blocks b of K (32 elements each) of
                  2^(sa[m][b] - 127) * 2^(sb[n][b] - 127)
                  * sum_{k in block b} a(m, k) * b(k, n)

    with ``sa`` M x K/32 and ``sb`` N x K/32 E8M0 codes, row-major (the
    scaled-operand definition of the OCP Microscaling formats, applied to
    each operand's 32-element blocks along K; the gfx950 scaled f8f6f4 MFMA
    takes one such scale per 32-element block, the "mfma.scale...f8f6f4"
    instruction named in the wgrad page's arch table, for the MX / microscaling
    bquant variants of the "gemm_rowcolquant dispatcher bridge" PR's combined
    follow-up).  K must be a multiple of 32."""
    if K % MX_BLOCK:
        raise ValueError("K must be a multiple of the MX block")
    nb = K // MX_BLOCK
    a = operand_matrix(fmt, a_codes, M, K, K)
    bt = operand_matrix(fmt, b_codes, N, K, K)
    sa = decode_e8m0(np.asarray(sa_codes).reshape(M, nb))
    sb = decode_e8m0(np.asarray(sb_codes).reshape(N, nb))
    r = np.zeros((M, N))
    for blk in range(nb):
        ks = slice(blk * MX_BLOCK, (blk + 1) * MX_BLOCK)
        r += (sa[:, blk:blk + 1] * sb[:, blk][None, :]) * (a[:, ks] @ bt[:, ks].T)
    return r


def gemm_mx_entry(fmt, a_codes, b_codes, sa_codes, sb_codes, m, n, K):
    """One output element of ``gemm_mx`` computed on its own."""
    nb = K // MX_BLOCK
    a_row = decode(fmt, np.asarray(a_codes).reshape(-1)[m * K:(m + 1) * K])
    b_col = decode(fmt, np.asarray(b_codes).reshape(-1)[n * K:(n + 1) * K])
    sa = decode_e8m0(np.asarray(sa_codes).reshape(-1)[m * nb:(m + 1) * nb])
    sb = decode_e8m0(np.asarray(sb_codes).reshape(-1)[n * nb:(n + 1) * nb])
    return float(sum(sa[b] * sb[b] * np.dot(a_row[b * MX_BLOCK:(b + 1) * MX_BLOCK],
                                            b_col[b * MX_BLOCK:(b + 1) * MX_BLOCK])
                     for b in range(nb)))
