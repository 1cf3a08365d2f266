"""GPU parity of the GEMM with OCP MX (E8M0) block scales, through the C ABI:
one E8M0 scale per 32 consecutive K elements of each row of A and each
column of B, applied by the gfx950 scaled f8f6f4 MFMA per operand lane.

* Integer-exact operands (small integers, scales 2^-4 .. 2^4 varying per
  block) are bit-exact against the oracle for e4m3 and e5m2, every launch
  mode x fix-up, with ragged M and N tiles: a scale applied to the wrong
  block, row or column, or a wrong bias, changes the result.
* Random data (N(0,1) quantised, scales 2^-3 .. 2^3) within 2e-2.
* Padded operand and output rows (lda, ldb > K, ldc > N) with compact scale
  arrays: bit-exact, padding untouched.
* A full-size 8192^3 e4m3 launch on sampled entries.
* Unsupported MX arguments (wrong tile, K not a multiple of 128, 16-bit
  inputs, a missing scale array) are -2.
"""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth
from oracle.gemm import gemm_mx, gemm_mx_entry

from helpers import assert_close, decode_out, out_buffer, to_dev

pytestmark = pytest.mark.gpu

MODES = ["dp", "dp_sk", "persistent"]
REDS = ["linear", "tree", "atomic", "workspace"]
TILE = "128x128x128"
TILES = ["128x128x128", "256x256x128"]


def e8m0(n, seed, lo, hi):
    return (127 + synth.rng(seed).integers(lo, hi + 1, n)).astype(np.uint8)


def run(A, B, SA, SB, M, N, K, fmt, fmt_c, mode, red, ctas, tile=TILE):
    dC = out_buffer(fmt_c, M * N)
    plan = skg.gemm(to_dev(A, fmt), to_dev(B, fmt), dC,
                    torch.from_numpy(SA).to("cuda"), torch.from_numpy(SB).to("cuda"),
                    M=M, N=N, K=K, dtype_ab=fmt, dtype_c=fmt_c, tile=tile, mode=mode,
                    reduction=red, ctas=ctas, scale_mode="mx")
    torch.cuda.synchronize()
    return decode_out(dC, fmt_c).reshape(M, N), plan


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_integer_exact_all_modes_and_fixups(fmt, tile):
    tm = int(tile.split("x")[0])
    M, N, K = 2 * tm + 40, tm + 72, 18 * 128
    A = synth.integer_codes(fmt, M * K, 51, 0.2)
    B = synth.integer_codes(fmt, N * K, 52, 0.2)
    SA, SB = e8m0(M * K // 32, 53, -4, 4), e8m0(N * K // 32, 54, -4, 4)
    R = gemm_mx(fmt, A, B, SA, SB, M, N, K)
    assert np.array_equal(R.astype(np.float32).astype(np.float64), R)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (5, 13):
                Y, plan = run(A, B, SA, SB, M, N, K, fmt, "f32", mode, red, ctas, tile)
                assert np.array_equal(Y, R), "%s %s %s %s ctas=%d: not bit-exact (max diff %g)" % (
                    tile, fmt, mode, red, ctas, np.nanmax(np.abs(Y - R)))


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_random_within_tolerance(fmt, tile):
    M, N, K = 3 * 128 + 8, 2 * 128 + 16, 20 * 128
    A = synth.to_codes(synth.draw("normal", M * K, 61), fmt)
    B = synth.to_codes(synth.draw("normal", N * K, 62), fmt)
    SA, SB = e8m0(M * K // 32, 63, -3, 3), e8m0(N * K // 32, 64, -3, 3)
    R = gemm_mx(fmt, A, B, SA, SB, M, N, K)
    for mode, red, fmt_c in (("dp", "linear", "bf16"), ("dp_sk", "tree", "bf16"),
                             ("persistent", "workspace", "f32"), ("dp_sk", "atomic", "f32")):
        Y, plan = run(A, B, SA, SB, M, N, K, fmt, fmt_c, mode, red, 11, tile)
        assert_close(Y, R, fmt, "mx %s %s %s %s" % (tile, fmt, mode, red))


@pytest.mark.parametrize("tile", TILES)
def test_leading_dimensions(tile):
    # A and B rows wider than K (lda, ldb > K) and C rows wider than N, with
    # the scale arrays still M x K/32 and N x K/32: bit-exact against the
    # oracle on the compact operands, and C's padding columns keep their NaN.
    tm = int(tile.split("x")[0])
    M, N, K = tm + 8, 72, 2 * 128
    lda, ldb, ldc = K + 48, K + 16, N + 4
    A = synth.integer_codes("e4m3", M * lda, 81, 0.2)
    B = synth.integer_codes("e4m3", N * ldb, 82, 0.2)
    SA, SB = e8m0(M * K // 32, 83, -4, 4), e8m0(N * K // 32, 84, -4, 4)
    Ac = np.ascontiguousarray(A.reshape(M, lda)[:, :K]).reshape(-1)
    Bc = np.ascontiguousarray(B.reshape(N, ldb)[:, :K]).reshape(-1)
    R = gemm_mx("e4m3", Ac, Bc, SA, SB, M, N, K)
    dA, dB = to_dev(A, "e4m3"), to_dev(B, "e4m3")
    dSA, dSB = torch.from_numpy(SA).to("cuda"), torch.from_numpy(SB).to("cuda")
    for mode, red, ctas in [("dp", "linear", 1), ("dp_sk", "tree", 5), ("persistent", "linear", 3),
                            ("dp_sk", "atomic", 4), ("persistent", "workspace", 7)]:
        dC = out_buffer("f32", M * ldc)
        skg.gemm(dA, dB, dC, dSA, dSB, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc, dtype_ab="e4m3",
                 dtype_c="f32", tile=tile, mode=mode, reduction=red, ctas=ctas, scale_mode="mx")
        torch.cuda.synchronize()
        Y = decode_out(dC, "f32").reshape(M, ldc)
        what = "%s %s %s ctas=%d" % (tile, mode, red, ctas)
        assert np.array_equal(Y[:, :N], R), what
        assert np.isnan(Y[:, N:]).all(), what + ": padding written"


@pytest.mark.parametrize("tile,ctas", [("128x128x128", 512), ("256x256x128", 256)])
def test_full_size_sampled(tile, ctas):
    M = N = K = 8192
    g = synth.rng(71)
    A = synth.to_codes(synth.draw("normal", M * K, 72), "e4m3")
    B = synth.to_codes(synth.draw("normal", N * K, 73), "e4m3")
    SA, SB = e8m0(M * K // 32, 74, -3, 3), e8m0(N * K // 32, 75, -3, 3)
    Y, plan = run(A, B, SA, SB, M, N, K, "e4m3", "bf16", "persistent", "workspace", ctas, tile)
    assert not np.isnan(Y).any(), "unwritten outputs"
    idx = [(int(g.integers(M)), int(g.integers(N))) for _ in range(400)]
    ref = np.array([gemm_mx_entry("e4m3", A, B, SA, SB, m, n, K) for m, n in idx])
    got = np.array([Y[m, n] for m, n in idx])
    err = np.max(np.abs(got - ref)) / np.max(np.abs(ref))
    assert err <= 2e-2, err


def test_mx_rejections():
    M, N, K = 128, 128, 256
    base = dict(M=M, N=N, K=K, dtype_ab="e4m3", dtype_c="bf16", tile=TILE, mode="dp_sk",
                reduction="linear", ctas=4, scale_mode="mx")
    for bad in (dict(tile="256x256x64"), dict(K=192), dict(dtype_ab="bf16", tile="128x128x64")):
        with pytest.raises(skg.SkgError) as ei:
            skg.plan_gemm(**dict(base, **bad))
        assert ei.value.status == -2
    A = torch.zeros(M * K, dtype=torch.uint8, device="cuda")
    C = out_buffer("bf16", M * N)
    with pytest.raises(skg.SkgError) as ei:
        skg.gemm(A, A, C, None, None, **base)
    assert ei.value.status == -2 and "scale" in ei.value.msg
