"""Error paths of the run calls, forced from the host so that every kernel
still ends normally (the status codes of the stream-K GEMM bridge,
composable_kernel commit "feat(ck-tile): stream-K GEMM TE to dispatcher
bridge", Changes: -1 for a HIP error; and the bounded hand-off wait of
rocm-libraries PR #13151, whose review notes that forward progress rests on
in-order dispatch, which the hardware does not promise).

* SKG_FAULT=launch: the run call returns -1 with a reason where it would
  launch the stream-K kernel; the output is untouched; the next call without
  the switch works.
* SKG_FAULT=handoff: stream-K CTAs never raise their flags and the waits
  poll only 64 times, so every hand-off wait gives up.  The library counts
  exactly one give-up per (fold, wave) -- 4 waves x (contributors - 1) per
  shared tile, for linear and tree alike -- the kernel ends, data-parallel
  tiles and single-contributor tiles stay exact (the values of the shared
  tiles are unspecified after a give-up), and the next launch without the
  switch is exact again.
"""

import os

import numpy as np
import pytest
import torch

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import synth
from oracle import partition as P
from oracle.gemm import gemm as oracle_gemm

from helpers import decode_out, out_buffer, to_dev

pytestmark = pytest.mark.gpu


class fault:
    def __init__(self, kind):
        self.kind = kind

    def __enter__(self):
        os.environ["SKG_FAULT"] = self.kind

    def __exit__(self, *exc):
        os.environ.pop("SKG_FAULT", None)


M, N, K, TILE = 300, 420, 2560, "128x128x32"


def operands():
    A = synth.integer_codes("f16", M * K, 41, 0.15)
    B = synth.integer_codes("f16", N * K, 42, 0.15)
    return A, B, oracle_gemm("f16", A, B, M, N, K)


def test_forced_launch_failure_returns_minus_one():
    A, B, R = operands()
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    C = out_buffer("f32", M * N)
    kw = dict(M=M, N=N, K=K, dtype_ab="f16", dtype_c="f32", tile=TILE, mode="dp_sk",
              reduction="linear", ctas=5)
    with fault("launch"):
        with pytest.raises(skg.SkgError) as ei:
            skg.gemm(dA, dB, C, **kw)
    assert ei.value.status == -1 and "SKG_FAULT" in ei.value.msg
    torch.cuda.synchronize()
    assert torch.isnan(C.view(torch.float32)).all(), "output touched by a failed call"
    skg.gemm(dA, dB, C, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(decode_out(C, "f32").reshape(M, N), R)


@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
@pytest.mark.parametrize("reduction", ["linear", "tree"])
def test_forced_handoff_give_up_is_counted_and_poisons(mode, reduction):
    A, B, R = operands()
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    C = out_buffer("f32", M * N)
    ctas = 7
    kw = dict(M=M, N=N, K=K, dtype_ab="f16", dtype_c="f32", tile=TILE, mode=mode,
              reduction=reduction, ctas=ctas)
    plan = skg.plan_gemm(**kw)
    tm, tn, tk = 128, 128, 32
    tiles_m, tiles_n, ipt = P.gemm_tiles(M, N, K, tm, tn, tk)
    op = P.plan(tiles_m, tiles_n, ipt, tm, tn, 4, mode, reduction, ctas)
    assert plan["sk_ctas"] == ctas and op.sk_tiles > 0
    # Contributors of every stream-K tile from the oracle partitioner.
    contrib = {}
    for s in range(op.sk_tiles):
        contrib[op.dp_tiles + s] = len(op.contributors(s))
    assert max(contrib.values()) >= 2
    expected = 4 * sum(n - 1 for n in contrib.values())
    skg.skg_fixup_timeouts(reset=True)
    with fault("handoff"):
        skg.gemm(dA, dB, C, **kw)
    torch.cuda.synchronize()
    got = skg.skg_fixup_timeouts(reset=True)
    assert got == expected, (got, expected)
    Y = decode_out(C, "f32").reshape(M, N)
    for tile in range(tiles_m * tiles_n):
        tmi, tni = divmod(tile, tiles_n)
        blk = Y[tmi * tm:(tmi + 1) * tm, tni * tn:(tni + 1) * tn]
        ref = R[tmi * tm:(tmi + 1) * tm, tni * tn:(tni + 1) * tn]
        if contrib.get(tile, 1) == 1:
            assert np.array_equal(blk, ref), "tile %d" % tile
    # The switch off again: the same launch is exact and nothing gives up.
    skg.gemm(dA, dB, C, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(decode_out(C, "f32").reshape(M, N), R)


@pytest.mark.parametrize("mode", ["dp_sk", "persistent"])
def test_forced_handoff_give_up_is_counted_scatter(mode):
    # Scatter: every contributor publishes (no flag raised under the switch)
    # and each of its waves then polls all of the tile's flags, gives up and
    # counts once; tiles held by a single CTA stay exact.
    A, B, R = operands()
    dA, dB = to_dev(A, "f16"), to_dev(B, "f16")
    C = out_buffer("f32", M * N)
    tm, tn, tk = 128, 128, 32
    tiles_m, tiles_n, ipt = P.gemm_tiles(M, N, K, tm, tn, tk)
    T = tiles_m * tiles_n
    S = next(d for d in (2, 3, 4, 5) if ipt % d == 0)
    kw = dict(M=M, N=N, K=K, dtype_ab="f16", dtype_c="f32", tile=TILE, mode=mode,
              reduction="scatter", ctas=T * S)
    plan = skg.plan_gemm(**kw)
    assert plan["sk_ctas"] == T * S and plan["sk_tiles"] == T
    skg.skg_fixup_timeouts(reset=True)
    with fault("handoff"):
        skg.gemm(dA, dB, C, **kw)
    torch.cuda.synchronize()
    got = skg.skg_fixup_timeouts(reset=True)
    assert got == 4 * T * S, (got, 4 * T * S)
    skg.gemm(dA, dB, C, **kw)
    torch.cuda.synchronize()
    assert np.array_equal(decode_out(C, "f32").reshape(M, N), R)
