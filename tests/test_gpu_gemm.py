"""GPU parity of the GEMM path against the oracle (through the C ABI).

* Every tile instance x launch mode x fix-up on ragged shapes that span
  several tiles and split tiles between up to four stream-K CTAs, on random
  data (tolerance 5e-3 for fp16/bf16 inputs, 2e-2 for fp8) and on
  integer-exact data (bit-exact: every product and fp32 partial sum is exact,
  so any missed or repeated MAC iteration shows).
* The five workloads' GEMMs at full size in the launch configuration the
  benchmark times, checked on sampled entries computed one by one by the
  oracle, plus the whole output scanned for unwritten rows.
* Unsupported arguments come back as -2 with the output untouched.
"""

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth
from oracle import codecs
from oracle.gemm import gemm as oracle_gemm, gemm_entry

from helpers import TOL, assert_close, decode_out, out_buffer, rel_err, to_dev, to_dev_f32

pytestmark = pytest.mark.gpu

MODES = ["dp", "dp_sk", "persistent"]
REDS = ["linear", "tree", "atomic", "workspace"]
TILE_DT = [("128x128x32", "f16"), ("128x128x32", "bf16"), ("256x256x64", "bf16"),
           ("256x256x64", "f16"), ("128x128x64", "bf16"), ("256x128x64", "f16"),
           ("256x256x128", "e4m3"), ("256x256x128", "e5m2"), ("128x128x128", "e4m3"),
           ("128x128x128", "e5m2")]
FP8 = ("e4m3", "e5m2")


def run(A, B, M, N, K, fmt, fmt_c, tile, mode, red, ctas, sa=None, sb=None, ws=None, C=None,
        scale_mode="rowcol"):
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    dC = C if C is not None else out_buffer(fmt_c, M * N)
    dsa = to_dev_f32(sa) if sa is not None else None
    dsb = to_dev_f32(sb) if sb is not None else None
    plan = skg.gemm(dA, dB, dC, dsa, dsb, workspace=ws, M=M, N=N, K=K, dtype_ab=fmt,
                    dtype_c=fmt_c, tile=tile, mode=mode, reduction=red, ctas=ctas,
                    scale_mode=scale_mode)
    torch.cuda.synchronize()
    return decode_out(dC, fmt_c).reshape(M, N), plan


def shape_for(tile, k_tail=False):
    tm, tn, tk = map(int, tile.split("x"))
    # 3 x 2 tiles with ragged last row and column of tiles, 24 MAC iterations
    # (plus a partial 25th with k_tail: 16 more K elements).
    return 2 * tm + tm // 3 + 8, tn + tn // 2 + 8, 24 * tk + (16 if k_tail else 0)


@pytest.mark.parametrize("tile,fmt", TILE_DT)
def test_random_all_modes_and_fixups(tile, fmt):
    M, N, K = shape_for(tile)
    g = synth.rng(11)
    dist = "normal" if fmt in FP8 else "uniform"
    A = synth.to_codes(synth.draw(dist, M * K, 1), fmt)
    B = synth.to_codes(synth.draw(dist, N * K, 2), fmt)
    sa = synth.draw("scale", M, 3).astype(np.float32)
    sb = synth.draw("scale", N, 4).astype(np.float32)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb)
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (4, 7, 13):
                fmt_c = "f32" if red == "atomic" else ("bf16" if int(g.integers(2)) else "f16")
                if fmt_c == "f16" and fmt in FP8:
                    fmt_c = "bf16"
                Y, plan = run(A, B, M, N, K, fmt, fmt_c, tile, mode, red, ctas, sa, sb)
                assert_close(Y, R, fmt, "%s %s %s %s ctas=%d" % (tile, fmt, mode, red, ctas))
                if mode == "dp":
                    break


@pytest.mark.parametrize("tile,fmt", TILE_DT)
def test_data_parallel_plan_same_bits_for_every_reduction(tile, fmt):
    # A plan without stream-K CTAs runs no fix-up, so the reduction it names
    # (and the kernel family that name selects) cannot change a bit of C:
    # all-DP launches (dp mode, persistent with a pool that divides the
    # tiles) give the same output under every reduction.
    M, N, K = shape_for(tile)
    dist = "normal" if fmt in FP8 else "uniform"
    A = synth.to_codes(synth.draw(dist, M * K, 21), fmt)
    B = synth.to_codes(synth.draw(dist, N * K, 22), fmt)
    sa = synth.draw("scale", M, 23).astype(np.float32)
    sb = synth.draw("scale", N, 24).astype(np.float32)
    ref = None
    for mode, ctas in (("dp", 4), ("persistent", 3), ("persistent", 6)):
        for red in REDS:
            Y, plan = run(A, B, M, N, K, fmt, "f32", tile, mode, red, ctas, sa, sb)
            assert plan["sk_ctas"] == 0 and plan["dp_tiles"] == plan["tiles"], (mode, red, ctas)
            if ref is None:
                ref = Y
            assert np.array_equal(Y, ref), "%s %s %s %s ctas=%d" % (tile, fmt, mode, red, ctas)


@pytest.mark.parametrize("tile,fmt", TILE_DT)
def test_leading_dimensions_and_tiny_shapes(tile, fmt):
    # rcr operands in rows wider than the K they hold (lda, ldb > K) and C
    # rows wider than N (ldc > N), down to a single output element and one
    # 16-byte slice of K: the oracle's result bit for bit on integer data,
    # in every launch mode and fix-up, and C's padding columns keep what
    # they held.
    eb = 1 if fmt in FP8 else 2
    kq = 16 // eb  # the K granule: 16 bytes
    tm, tn, tk = map(int, tile.split("x"))
    shapes = [(1, 1, kq), (3, 5, 2 * kq), (tm + 3, 2, tk + kq), (2, tn + 9, 3 * tk - kq)]
    for si, (M, N, K) in enumerate(shapes):
        lda, ldb = K + 3 * kq, K + kq
        ldc = (N + 3) // 4 * 4 + 4  # fp32 C: 16-byte rows, 4 spare columns at least
        A = synth.integer_codes(fmt, M * lda, 171 + si, 0.15)
        B = synth.integer_codes(fmt, N * ldb, 181 + si, 0.15)
        sa, sb = synth.pow2_scales(M, 191 + si), synth.pow2_scales(N, 201 + si)
        R = oracle_gemm(fmt, A, B, M, N, K, lda=lda, ldb=ldb, scale_a=sa, scale_b=sb)
        dA, dB, dsa, dsb = to_dev(A, fmt), to_dev(B, fmt), to_dev_f32(sa), to_dev_f32(sb)
        for mode, red, ctas in [("dp", "linear", 1), ("dp_sk", "tree", 3), ("persistent", "linear", 5),
                                ("dp_sk", "atomic", 4), ("persistent", "workspace", 3)]:
            dC = out_buffer("f32", M * ldc)
            plan = skg.gemm(dA, dB, dC, dsa, dsb, M=M, N=N, K=K, lda=lda, ldb=ldb, ldc=ldc,
                            dtype_ab=fmt, dtype_c="f32", tile=tile, mode=mode, reduction=red,
                            ctas=ctas)
            torch.cuda.synchronize()
            Y = decode_out(dC, "f32").reshape(M, ldc)
            what = "%s %s M=%d N=%d K=%d %s %s ctas=%d" % (tile, fmt, M, N, K, mode, red, ctas)
            assert np.array_equal(Y[:, :N], R), what
            assert np.isnan(Y[:, N:]).all(), what + ": padding of C written"


def exact_in(fmt_c, R):
    if fmt_c == "f32":
        return np.array_equal(R.astype(np.float32).astype(np.float64), R)
    return np.array_equal(codecs.decode(fmt_c, codecs.encode(fmt_c, R)), R)


@pytest.mark.parametrize("k_tail", [False, True])
@pytest.mark.parametrize("tile,fmt", TILE_DT)
def test_integer_exact_all_modes_and_fixups(tile, fmt, k_tail):
    M, N, K = shape_for(tile, k_tail)
    A = synth.integer_codes(fmt, M * K, 21, 0.15)
    B = synth.integer_codes(fmt, N * K, 22, 0.15)
    sa = synth.pow2_scales(M, 23)
    sb = synth.pow2_scales(N, 24)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb)
    outs = [f for f in ("f16", "bf16", "f32") if exact_in(f, R)]
    assert "f32" in outs and len(outs) >= 2, outs
    k = 0
    for mode in MODES:
        for red in REDS:
            if mode == "dp" and red != "linear":
                continue
            for ctas in (5, 13):
                fmt_c = "f32" if red == "atomic" else outs[k % len(outs)]
                k += 1
                Y, plan = run(A, B, M, N, K, fmt, fmt_c, tile, mode, red, ctas, sa, sb)
                label = "%s %s %s %s ctas=%d -> %s" % (tile, fmt, mode, red, ctas, fmt_c)
                assert np.array_equal(Y, R), label + ": not bit-exact (max diff %g)" % np.nanmax(np.abs(Y - R))


def test_plan_reaches_four_contributors():
    # The random/integer matrix above must exercise folds of up to four CTAs.
    M, N, K = shape_for("128x128x32")
    plan = skg.plan_gemm(M=M, N=N, K=K, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                         mode="dp_sk", reduction="tree", ctas=13)
    assert plan["max_contrib"] >= 3 and plan["tree_rounds"] >= 2


@pytest.mark.parametrize("tile,fmt", [("128x128x32", "f16"), ("256x256x64", "bf16"),
                                      ("256x256x128", "e4m3")])
def test_many_contributors_integer_exact(tile, fmt):
    # One ragged tile shared by 20 stream-K CTAs: a linear owner folds 19
    # partners (more than the flags it checks in its first round trip), a
    # tree folds over 5 rounds.  Bit-exact on integer-exact inputs, in both
    # launch modes.
    tm, tn, tk = map(int, tile.split("x"))
    M, N, K = tm - 24, tn - 40, 40 * tk
    A = synth.integer_codes(fmt, M * K, 31, 0.15)
    B = synth.integer_codes(fmt, N * K, 32, 0.15)
    R = oracle_gemm(fmt, A, B, M, N, K)
    assert exact_in("f32", R)
    for mode in ("dp_sk", "persistent"):
        for red in ("linear", "tree"):
            Y, plan = run(A, B, M, N, K, fmt, "f32", tile, mode, red, 20)
            assert plan["sk_ctas"] == 20 and plan["max_contrib"] == 20, plan
            assert np.array_equal(Y, R), "%s %s %s %s: not bit-exact" % (tile, fmt, mode, red)


def test_unsupported_args_leave_output_untouched():
    M, N, K = 64, 64, 64
    A = synth.to_codes(synth.draw("uniform", M * K, 1), "f16")
    dA, dB = to_dev(A, "f16"), to_dev(A, "f16")
    dC = out_buffer("f16", M * N)
    before = dC.clone()
    bad = [dict(reduction="atomic"),                  # atomic needs an fp32 C
           dict(ctas=0), dict(ctas=-3), dict(K=60),   # K not 16-byte multiple
           dict(tile="256x256x128"),                  # fp8-only tile
           dict(mode=7)]
    for b in bad:
        kw = dict(M=M, N=N, K=K, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                  mode="dp_sk", reduction="linear", ctas=4)
        kw.update(b)
        with pytest.raises(skg.SkgError) as ei:
            skg.gemm(dA, dB, dC, workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"),
                     **kw)
        assert ei.value.status == -2, b
    torch.cuda.synchronize()
    assert torch.equal(before, dC)
    # a workspace smaller than the plan needs (one tile of 20 iterations
    # over 3 stream-K CTAs needs flags and partials)
    K2 = 640
    A2 = synth.to_codes(synth.draw("uniform", M * K2, 1), "f16")
    dA2 = to_dev(A2, "f16")
    kw = dict(M=M, N=N, K=K2, dtype_ab="f16", dtype_c="f16", tile="128x128x32", mode="dp_sk",
              reduction="linear", ctas=3)
    assert skg.plan_gemm(**kw)["workspace_bytes"] > 16
    with pytest.raises(skg.SkgError) as ei:
        skg.gemm(dA2, dA2, dC, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"), **kw)
    assert ei.value.status == -2 and "workspace" in ei.value.msg
    torch.cuda.synchronize()
    assert torch.equal(before, dC)


def test_default_pool_and_device():
    cus, per_cu = skg.skg_device_info(0, skg.TILES["256x256x64"], skg.DTYPES["bf16"])
    assert cus >= 1 and per_cu >= 1
    plan = skg.plan_gemm(M=4864, N=4096, K=4096, dtype_ab="bf16", dtype_c="bf16",
                         tile="256x256x64", mode="dp_sk", reduction="tree", ctas=-1)
    assert plan["pool"] == cus
    plan = skg.plan_gemm(M=4864, N=4096, K=4096, dtype_ab="bf16", dtype_c="bf16",
                         tile="256x256x64", mode="dp_sk", reduction="workspace", ctas=-1)
    assert plan["pool"] == cus * min(4, per_cu)


def sampled_check(Y, wl, inp, n=1500):
    g = synth.rng(99)
    ms = g.integers(0, wl.M, n)
    ns = g.integers(0, wl.N, n)
    ref = np.array([gemm_entry(wl.dtype_ab, inp["A"], inp["B"], int(m), int(c), wl.K,
                               scale_a=inp.get("scale_a"), scale_b=inp.get("scale_b"))
                    for m, c in zip(ms, ns)])
    got = Y[ms, ns]
    return rel_err(got, ref)


@pytest.mark.parametrize("index", [1, 2, 5])
def test_workload_full_size(index):
    wl = synth.WORKLOADS[index]
    inp = wl.inputs()
    for mode in wl.modes:
        for red in wl.reductions:
            Y, plan = run(inp["A"], inp["B"], wl.M, wl.N, wl.K, wl.dtype_ab, wl.dtype_c, wl.tile,
                          mode, red, wl.ctas, inp.get("scale_a"), inp.get("scale_b"))
            assert not np.isnan(Y).any(), "unwritten outputs"
            if index == 1:
                R = oracle_gemm(wl.dtype_ab, inp["A"], inp["B"], wl.M, wl.N, wl.K)
                assert_close(Y, R, wl.dtype_ab, wl.name)
            else:
                err = sampled_check(Y, wl, inp)
                assert err <= TOL[wl.dtype_ab], "%s %s %s: %.3e" % (wl.name, mode, red, err)


SEL_TILE_DT = [("128x128x32", "f16"), ("256x256x64", "bf16"), ("256x256x128", "e4m3")]


@pytest.mark.parametrize("tile,fmt", SEL_TILE_DT)
def test_split_k_and_auto_integer_exact(tile, fmt):
    # 3 x 2 tiles of 25 MAC iterations: split-K slices that divide the
    # reduction and ones that straddle, every fix-up; "auto" on explicit and
    # default pools (stream-K here: a ragged wave over a long reduction).
    M, N, K = shape_for(tile, True)
    A = synth.integer_codes(fmt, M * K, 41, 0.15)
    B = synth.integer_codes(fmt, N * K, 42, 0.15)
    sa, sb = synth.pow2_scales(M, 43), synth.pow2_scales(N, 44)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb)
    fmt_c = "f32"
    cases = [("splitk", "workspace", 5, 5), ("splitk", "tree", 3, 3), ("splitk", "linear", 2, 2),
             ("splitk", "atomic", 25, 25), ("splitk", "workspace", 40, 25),
             ("splitk", "tree", 1, 1), ("auto", "auto", 7, 1), ("auto", "tree", 64, 1),
             ("auto", "auto", -1, None)]
    for mode, red, ctas, slices in cases:
        Y, plan = run(A, B, M, N, K, fmt, fmt_c, tile, mode, red, ctas, sa, sb)
        label = "%s %s %s %s ctas=%d" % (tile, fmt, mode, red, ctas)
        assert np.array_equal(Y, R), label + ": not bit-exact (max diff %g)" % np.nanmax(np.abs(Y - R))
        assert plan["requested_mode"] == skg.MODES[mode], label
        if slices is not None:
            assert plan["slices"] == slices, (label, plan["slices"])
        if mode == "auto" and ctas != -1:
            assert plan["mode"] == skg.MODES["dp_sk"] and plan["sk_ctas"] > 0, label


@pytest.mark.parametrize("tile,fmt", SEL_TILE_DT)
def test_auto_splits_one_short_tile(tile, fmt):
    # One tile whose iterations are fewer than the pool: the stream-K
    # partition would have no stream-K CTAs, so "auto" runs split-K with
    # slices of at least eight iterations (40 iterations over a 64-CTA pool:
    # 5 slices).
    tm, tn, tk = map(int, tile.split("x"))
    M, N, K = tm - 3, tn - 8, 40 * tk
    g = synth.rng(51)
    dist = "normal" if fmt in FP8 else "uniform"
    A = synth.to_codes(synth.draw(dist, M * K, 52), fmt)
    B = synth.to_codes(synth.draw(dist, N * K, 53), fmt)
    R = oracle_gemm(fmt, A, B, M, N, K)
    Y, plan = run(A, B, M, N, K, fmt, "bf16", tile, "auto", "auto", 64)
    assert plan["slices"] == 5 and plan["sk_ctas"] == 5 and plan["dp_tiles"] == 0
    assert plan["reduction"] == skg.REDUCTIONS["workspace"]
    assert_close(Y, R, fmt, "%s auto one short tile" % tile)


@pytest.mark.parametrize("tile,fmt", [("256x256x128", "e4m3"), ("256x256x128", "e5m2"),
                                      ("256x256x64", "bf16"), ("128x128x32", "f16")])
def test_per_tensor_scales(tile, fmt):
    # One scale for all of A and one for all of B: bit-exact on integer data
    # with power-of-two scales, every launch mode and fix-up; random data
    # within the tolerance.
    M, N, K = shape_for(tile, True)
    A = synth.integer_codes(fmt, M * K, 71, 0.15)
    B = synth.integer_codes(fmt, N * K, 72, 0.15)
    sa, sb = np.array([0.5], np.float32), np.array([4.0], np.float32)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb, scale_mode="tensor")
    for mode, red, ctas in [("dp", "linear", 1), ("dp_sk", "linear", 5), ("dp_sk", "tree", 13),
                            ("persistent", "workspace", 7), ("persistent", "atomic", 4),
                            ("splitk", "tree", 3)]:
        Y, plan = run(A, B, M, N, K, fmt, "f32", tile, mode, red, ctas, sa, sb,
                      scale_mode="tensor")
        assert np.array_equal(Y, R), "%s %s %s %s per-tensor not bit-exact" % (tile, fmt, mode, red)
    A = synth.to_codes(synth.draw("normal", M * K, 73), fmt)
    B = synth.to_codes(synth.draw("normal", N * K, 74), fmt)
    sa, sb = np.array([1.37], np.float32), np.array([0.61], np.float32)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb, scale_mode="tensor")
    Y, plan = run(A, B, M, N, K, fmt, "bf16", tile, "dp_sk", "tree", 7, sa, sb,
                  scale_mode="tensor")
    assert_close(Y, R, fmt, "%s %s per-tensor random" % (tile, fmt))
    # one scale pointer only: the other operand is unscaled
    R = oracle_gemm(fmt, A, B, M, N, K, scale_b=sb, scale_mode="tensor")
    Y, plan = run(A, B, M, N, K, fmt, "bf16", tile, "dp_sk", "linear", 7, None, sb,
                  scale_mode="tensor")
    assert_close(Y, R, fmt, "%s %s per-tensor B only" % (tile, fmt))


def test_e5m2_workload_shape_sampled():
    # The fp8 workload's shape and launch with E5M2 operands and per-tensor
    # scales, checked on sampled outputs.
    wl = synth.WORKLOADS[5]
    M = N = K = 8192
    A = synth.to_codes(synth.draw("normal", M * K, 81), "e5m2")
    B = synth.to_codes(synth.draw("normal", N * K, 82), "e5m2")
    sa, sb = np.array([1.25], np.float32), np.array([0.75], np.float32)
    Y, plan = run(A, B, M, N, K, "e5m2", "bf16", wl.tile, wl.modes[0], wl.reductions[0], wl.ctas,
                  sa, sb, scale_mode="tensor")
    assert not np.isnan(Y).any(), "unwritten outputs"
    g = synth.rng(98)
    ms, ns = g.integers(0, M, 800), g.integers(0, N, 800)
    ref = np.array([gemm_entry("e5m2", A, B, int(m), int(c), K, scale_a=sa, scale_b=sb,
                               scale_mode="tensor") for m, c in zip(ms, ns)])
    assert rel_err(Y[ms, ns], ref) <= TOL["e5m2"]


@pytest.mark.parametrize("tile,fmt", [("128x128x32", "f16"), ("256x256x64", "bf16"),
                                      ("256x256x128", "e4m3")])
def test_xcd_sk_order_integer_exact(tile, fmt):
    # Stream-K CTAs dealt to the XCDs in contiguous runs (not the GEMM
    # default): same results bit for bit, every mode and fix-up, pools that
    # are and are not multiples of 8.
    M, N, K = shape_for(tile, True)
    A = synth.integer_codes(fmt, M * K, 91, 0.15)
    B = synth.integer_codes(fmt, N * K, 92, 0.15)
    sa, sb = synth.pow2_scales(M, 93), synth.pow2_scales(N, 94)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb)
    for mode in ("dp_sk", "persistent"):
        for red in REDS:
            for ctas in (8, 13, 16):
                dA, dB = to_dev(A, fmt), to_dev(B, fmt)
                dC = out_buffer("f32", M * N)
                plan = skg.gemm(dA, dB, dC, to_dev_f32(sa), to_dev_f32(sb), M=M, N=N, K=K,
                                dtype_ab=fmt, dtype_c="f32", tile=tile, mode=mode, reduction=red,
                                ctas=ctas, sk_order="xcd")
                torch.cuda.synchronize()
                assert plan["sk_order"] == skg.SK_ORDERS["xcd"]
                Y = decode_out(dC, "f32").reshape(M, N)
                assert np.array_equal(Y, R), "%s %s %s %s ctas=%d xcd order" % (tile, fmt, mode,
                                                                                red, ctas)


@pytest.mark.parametrize("tile,fmt", [("128x128x32", "f16"), ("256x256x64", "bf16")])
def test_kmajor_sk_order_integer_exact(tile, fmt):
    # Whole K slices per stream-K CTA, dealt slice by slice: bit-exact in
    # every mode and fix-up.
    M, N, K = shape_for(tile, True)
    A = synth.integer_codes(fmt, M * K, 95, 0.15)
    B = synth.integer_codes(fmt, N * K, 96, 0.15)
    R = oracle_gemm(fmt, A, B, M, N, K)
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    p0 = skg.plan_gemm(M=M, N=N, K=K, dtype_ab=fmt, dtype_c="f32", tile=tile, mode="dp_sk",
                       reduction="tree", ctas=8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    for S in [d for d in (2, 3, 5, ipt) if ipt % d == 0]:
        for mode in ("dp_sk", "persistent"):
            for red in REDS:
                dC = out_buffer("f32", M * N)
                plan = skg.gemm(dA, dB, dC, None, None, M=M, N=N, K=K, dtype_ab=fmt,
                                dtype_c="f32", tile=tile, mode=mode, reduction=red, ctas=T * S,
                                sk_order="kmajor")
                torch.cuda.synchronize()
                assert plan["sk_order"] == skg.SK_ORDERS["kmajor"], (T, S)
                Y = decode_out(dC, "f32").reshape(M, N)
                assert np.array_equal(Y, R), "%s %s %s %s S=%d kmajor" % (tile, fmt, mode, red, S)


@pytest.mark.parametrize("tile,fmt", [("128x128x32", "f16"), ("256x256x64", "bf16"),
                                      ("256x128x64", "f16"), ("256x256x128", "e4m3")])
def test_scatter_fixup_integer_exact(tile, fmt):
    # The reduce-scatter fix-up on whole-slice pools with per-row / per-column
    # power-of-two scales applied by the contributors that write each part,
    # ragged edge tiles included: bit-exact in both launch modes.
    M, N, K = shape_for(tile)
    A = synth.integer_codes(fmt, M * K, 101, 0.15)
    B = synth.integer_codes(fmt, N * K, 102, 0.15)
    sa, sb = synth.pow2_scales(M, 103), synth.pow2_scales(N, 104)
    R = oracle_gemm(fmt, A, B, M, N, K, scale_a=sa, scale_b=sb)
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    p0 = skg.plan_gemm(M=M, N=N, K=K, dtype_ab=fmt, dtype_c="f32", tile=tile, mode="dp_sk",
                       reduction="tree", ctas=8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    for S in [d for d in (2, 3, 4, 8, ipt) if ipt % d == 0]:
        for mode in ("dp_sk", "persistent"):
            dC = out_buffer("f32", M * N)
            plan = skg.gemm(dA, dB, dC, to_dev_f32(sa), to_dev_f32(sb), M=M, N=N, K=K,
                            dtype_ab=fmt, dtype_c="f32", tile=tile, mode=mode, reduction="scatter",
                            ctas=T * S)
            torch.cuda.synchronize()
            assert plan["reduction"] == skg.REDUCTIONS["scatter"]
            Y = decode_out(dC, "f32").reshape(M, N)
            assert np.array_equal(Y, R), "%s %s %s S=%d scatter" % (tile, fmt, mode, S)


@pytest.mark.parametrize("tile,fmt,fmt_c", [("256x256x64", "bf16", "bf16"),
                                            ("128x128x64", "f16", "f32"),
                                            ("256x256x128", "e4m3", "bf16")])
def test_scatter_is_linear_bit_for_bit(tile, fmt, fmt_c):
    # Random data with per-row / per-column scales: the reduce-scatter adds
    # the partials in the linear fix-up's order and applies the same
    # epilogue, so for the same partition both give the same bits.
    M, N, K = shape_for(tile)
    A = synth.to_codes(synth.draw("normal", M * K, 111), fmt)
    B = synth.to_codes(synth.draw("normal", N * K, 112), fmt)
    sa = np.random.default_rng(113).uniform(0.5, 2.0, M).astype(np.float32)
    sb = np.random.default_rng(114).uniform(0.5, 2.0, N).astype(np.float32)
    dA, dB, dsa, dsb = to_dev(A, fmt), to_dev(B, fmt), to_dev_f32(sa), to_dev_f32(sb)
    p0 = skg.plan_gemm(M=M, N=N, K=K, dtype_ab=fmt, dtype_c=fmt_c, tile=tile, mode="dp_sk",
                       reduction="tree", ctas=8)
    T, ipt = p0["tiles"], p0["iters_per_tile"]
    for S in [d for d in (2, 3, 8) if ipt % d == 0]:
        for mode in ("dp_sk", "persistent"):
            out = {}
            for red in ("scatter", "linear"):
                dC = out_buffer(fmt_c, M * N)
                plan = skg.gemm(dA, dB, dC, dsa, dsb, M=M, N=N, K=K, dtype_ab=fmt, dtype_c=fmt_c,
                                tile=tile, mode=mode, reduction=red, ctas=T * S)
                torch.cuda.synchronize()
                assert plan["sk_ctas"] == T * S
                out[red] = dC.cpu().numpy().copy()
            assert np.array_equal(out["scatter"], out["linear"]), "%s %s %s S=%d" % (tile, fmt,
                                                                                    mode, S)


@pytest.mark.parametrize("fmt_c", ["f16", "bf16"])
def test_scatter_fixup_16bit_output(fmt_c):
    # Random data, 16-bit output: the part a contributor writes goes through
    # the same rounding as the copy-out (within the tolerance of the format).
    tile, fmt = "128x128x64", "bf16"
    M, N, K = shape_for(tile)
    A = synth.to_codes(synth.draw("uniform", M * K, 1), fmt)
    B = synth.to_codes(synth.draw("uniform", N * K, 2), fmt)
    R = oracle_gemm(fmt, A, B, M, N, K)
    dA, dB = to_dev(A, fmt), to_dev(B, fmt)
    for S in (2, 3, 8):
        dC = out_buffer(fmt_c, M * N)
        skg.gemm(dA, dB, dC, None, None, M=M, N=N, K=K, dtype_ab=fmt, dtype_c=fmt_c, tile=tile,
                 mode="dp_sk", reduction="scatter", ctas=6 * S)
        torch.cuda.synchronize()
        assert_close(decode_out(dC, fmt_c).reshape(M, N), R, fmt, "scatter S=%d %s" % (S, fmt_c))
