"""CPU tests of the HIP library's host side (no GPU needed, no compute calls).

* libskgemm.so loads and exports every function include/skgemm.h declares.
* The C++ planner equals the oracle partitioner field by field over a sweep
  of GEMM and wgrad shapes, tiles, modes, reductions and pools.
* Unsupported arguments are rejected with -2 and a reason.
* The built gfx950 code object orders the flag hand-off the way the engine
  implements release/acquire (rocm-libraries PR #13151, test plan: flag
  ordering pinned in the ISA): partials stored and loaded at device scope
  (sc1), every flag store right after a full wait for the wave's earlier
  stores, device-scope polls -- and no L2-wide write-back or invalidation
  anywhere (the test asserts their absence).
"""

import os
import re
import subprocess
import tempfile

import pytest

import implicit_gemm_conv_dp_amd as skg
from implicit_gemm_conv_dp_amd import _lib
from oracle import partition as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "skgemm.h")
TILES = {name: tuple(map(int, name.split("w")[0].split("x"))) for name in skg.TILES}


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(skg_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert {"skg_run_gemm", "skg_run_wgrad", "skg_plan_gemm", "skg_plan_wgrad",
            "skg_last_error", "skg_default_pool", "skg_device_info", "skg_tile_info"} <= set(names)
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTS), "binding and header disagree"


def test_tile_table():
    for name, tid in skg.TILES.items():
        info = skg.skg_tile_info(tid)
        assert (info.tm, info.tn, info.tk) == TILES[name]
        assert info.n_waves == 4
        assert info.group_block == (4 if name in ("64x144x32", "128x64x32") else 0)
    with pytest.raises(skg.SkgError) as ei:
        skg.skg_tile_info(99)
    assert ei.value.status == -2


def test_default_pool_matches_oracle_and_pages():
    # 304 CUs x 4 = 1216 for the atomic / workspace reductions.
    assert skg.skg_default_pool(_lib.RED_WORKSPACE, 304, 8) == 1216
    for red, name in [(0, "linear"), (1, "tree"), (2, "atomic"), (3, "workspace")]:
        for cus in (1, 80, 256, 304):
            for per in (1, 2, 3, 8):
                assert skg.skg_default_pool(red, cus, per) == P.default_pool(name, cus, per)
    for bad in [(7, 256, 1), (0, 0, 1), (0, 256, 0)]:
        with pytest.raises(skg.SkgError) as ei:
            skg.skg_default_pool(*bad)
        assert ei.value.status == -2


FIELDS = ["tiles_m", "tiles_n", "tiles", "iters_per_tile", "pool", "dp_tiles", "sk_tiles",
          "sk_ctas", "sk_iters", "iters_per_sk_cta", "extra_iters", "grid", "max_contrib",
          "linear_partners", "tree_rounds", "flags_bytes", "partials_bytes", "workspace_bytes"]


def same_plan(c, o):
    for f in FIELDS:
        ov = getattr(o, f)
        assert c[f] == ov, (f, c[f], ov)


GEMM_TILE_DT = [("128x128x32", "f16"), ("256x256x64", "bf16"), ("256x256x128", "e4m3"),
                ("256x256x128", "e5m2"), ("128x128x128", "e4m3"),
                ("128x128x64", "bf16"), ("256x128x64", "f16")]


@pytest.mark.parametrize("tile,dt", GEMM_TILE_DT)
def test_gemm_plan_equals_oracle(tile, dt):
    tm, tn, tk = TILES[tile]
    n = 0
    for M in (1, tm - 1, tm, 3 * tm + 5, 4864):
        for N in (16, tn, 2 * tn + 8, 4096):
            for K in (tk, 5 * tk, 4096 + tk):
                for mode in ("dp", "dp_sk", "persistent"):
                    for red in ("linear", "tree", "atomic", "workspace"):
                        for ctas in (1, 6, 77, 256, 1216):
                            dtc = "f32" if red == "atomic" else "bf16"
                            c = skg.plan_gemm(M=M, N=N, K=K, dtype_ab=dt, dtype_c=dtc, tile=tile,
                                              mode=mode, reduction=red, ctas=ctas)
                            tiles = P.gemm_tiles(M, N, K, tm, tn, tk)
                            o = P.plan(*tiles, tm, tn, 4, mode, red, ctas)
                            same_plan(c, o)
                            n += 1
    assert n > 1000


def test_workload_plans():
    # 256x256x4096 fp16 over a 6-CTA pool: ranges that straddle tiles.
    c = skg.plan_gemm(M=256, N=256, K=4096, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                      mode="dp_sk", reduction="linear", ctas=6)
    assert (c["sk_ctas"], c["iters_per_sk_cta"], c["extra_iters"], c["max_contrib"]) == (6, 85, 2, 3)
    c = skg.plan_gemm(M=4864, N=4096, K=4096, dtype_ab="bf16", dtype_c="bf16", tile="256x256x64",
                      mode="dp_sk", reduction="tree", ctas=256)
    assert (c["dp_tiles"], c["sk_tiles"], c["iters_per_sk_cta"], c["tree_rounds"],
            c["flags_bytes"]) == (256, 48, 12, 3, 4096)
    c = skg.plan_gemm(M=8192, N=8192, K=8192, dtype_ab="e4m3", dtype_c="bf16", tile="256x256x128",
                      mode="persistent", reduction="workspace", ctas=256)
    assert c["sk_ctas"] == 0 and c["grid"] == 256 and c["workspace_bytes"] == 0


WGRAD_SHAPES = [
    (32, 56, 56, 256, 256, 3, 3, (1, 1), (1, 1), 1),
    (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32),
    (2, 9, 9, 16, 24, 3, 3, (1, 1), (1, 1), 1),
    (3, 11, 10, 32, 16, 3, 3, (2, 2), (1, 1), 1),
    (2, 12, 12, 64, 32, 3, 3, (2, 2), (1, 1), 4),
    (1, 17, 15, 144, 40, 3, 2, (1, 2), (1, 0), 1),
]


@pytest.mark.parametrize("tile", ["128x128x32", "32x64x64", "128x128x64", "256x128x64"])
def test_wgrad_plan_equals_oracle(tile):
    tm, tn, tk = TILES[tile]
    for (n, h, w, c, k, r, s, st, pd, g) in WGRAD_SHAPES:
        for mode in ("dp", "dp_sk", "persistent"):
            for red in ("linear", "tree", "atomic", "workspace"):
                for ctas in (3, 7, 11, 256, 1024):
                    cp = skg.plan_wgrad(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd,
                                        groups=g, dtype="bf16", tile=tile, mode=mode,
                                        reduction=red, ctas=ctas)
                    tiles = P.wgrad_tiles(n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g,
                                          tm, tn, tk)
                    same_plan(cp, P.plan(*tiles, tm, tn, 4, mode, red, ctas))


# Grouped shapes with 16 input and 16 output channels per group: the
# workload's layer, a ragged last M tile (6 groups: 4 + 2), one group, 1x1
# and 5x5 filters (1 and 3 N tiles of nine taps), stride 1 and 2.
BD_SHAPES = [
    (64, 28, 28, 512, 512, 3, 3, (2, 2), (1, 1), 32),
    (2, 9, 9, 96, 96, 3, 3, (1, 1), (1, 1), 6),
    (3, 7, 5, 16, 16, 3, 3, (1, 1), (0, 1), 1),
    (2, 8, 8, 64, 64, 1, 1, (1, 1), (0, 0), 4),
    (2, 11, 9, 80, 80, 5, 5, (2, 1), (2, 2), 5),
]


def test_block_diagonal_wgrad_plan_equals_oracle():
    tm, tn, tk = TILES["64x144x32"]
    for (n, h, w, c, k, r, s, st, pd, g) in BD_SHAPES:
        for mode in ("dp", "dp_sk", "persistent", "splitk"):
            for red in ("linear", "tree", "atomic", "workspace", "scatter"):
                for ctas in (3, 7, 8, 16, 224, 256):
                    tiles = P.wgrad_tiles(n, h, w, c, k, r, s, st[0], st[1], pd[0], pd[1], g,
                                          tm, tn, tk, group_block=4)
                    T = tiles[0] * tiles[1]
                    rm, rr, rc, S = P.resolve_launch(T, tiles[2], mode, red, ctas)
                    try:
                        o = P.plan(*tiles, tm, tn, 4, rm, rr, rc)
                    except ValueError:
                        rejected(skg.plan_wgrad, n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st,
                                 pad=pd, groups=g, dtype="bf16", tile="64x144x32", mode=mode,
                                 reduction=red, ctas=ctas)
                        continue
                    cp = skg.plan_wgrad(n=n, h=h, w=w, c=c, k=k, r=r, s=s, stride=st, pad=pd,
                                        groups=g, dtype="bf16", tile="64x144x32", mode=mode,
                                        reduction=red, ctas=ctas)
                    same_plan(cp, o)
    # the workload's layer: 8 tiles of 392 iterations
    cp = skg.plan_wgrad(n=64, h=28, w=28, c=512, k=512, r=3, s=3, stride=(2, 2), pad=(1, 1),
                        groups=32, dtype="bf16", tile="64x144x32", mode="dp_sk",
                        reduction="linear", ctas=256)
    assert (cp["tiles_m"], cp["tiles_n"], cp["iters_per_tile"]) == (8, 1, 392)


def test_block_diagonal_wgrad_needs_16_channels_per_group():
    kw = dict(n=2, h=8, w=8, r=3, s=3, stride=(1, 1), pad=(1, 1), dtype="f16",
              tile="64x144x32", mode="dp_sk", reduction="tree", ctas=4)
    for c, k, g in ((64, 64, 2), (64, 128, 4), (128, 64, 4), (256, 256, 8)):
        msg = rejected(skg.plan_wgrad, c=c, k=k, groups=g, **kw)
        assert "16 input and 16 output channels" in msg
    assert skg.plan_wgrad(c=64, k=64, groups=4, **kw)["tiles_m"] == 1


def rejected(fn, **kw):
    with pytest.raises(skg.SkgError) as ei:
        fn(**kw)
    assert ei.value.status == -2
    assert ei.value.msg
    return ei.value.msg


def test_gemm_validation_rejects():
    base = dict(M=256, N=256, K=256, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                mode="dp_sk", reduction="linear", ctas=8)

    def bad(**over):
        kw = dict(base)
        kw.update(over)
        return rejected(skg.plan_gemm, **kw)

    assert "atomic" in bad(reduction="atomic")
    assert "ctas" in bad(ctas=0)
    assert "ctas" in bad(ctas=-5)
    assert "mode" in bad(mode=9)
    assert "reduction" in bad(reduction=9)
    assert "tile" in bad(tile=17)
    assert "instance" in bad(tile="256x256x128")
    assert "instance" in bad(dtype_ab="e4m3")
    assert "instance" in bad(dtype_ab="e5m2")
    assert "scale mode" in bad(scale_mode=3)
    assert "dtype" in bad(dtype_c="e4m3")
    assert "positive" in bad(M=0)
    assert "16 bytes" in bad(K=100)
    assert "leading" in bad(lda=128)
    assert "16 bytes" in bad(ldc=257)


def test_wgrad_validation_rejects():
    base = dict(n=2, h=9, w=9, c=16, k=24, r=3, s=3, stride=(1, 1), pad=(1, 1), groups=1,
                dtype="bf16", tile="128x128x64", mode="dp_sk", reduction="linear", ctas=8)

    def bad(**over):
        kw = dict(base)
        kw.update(over)
        return rejected(skg.plan_wgrad, **kw)

    assert "groups" in bad(groups=3)
    assert "multiples of 8" in bad(c=12)
    assert "dtype" in bad(dtype="e4m3")
    assert "instance" in bad(tile="256x256x128")
    assert "empty" in bad(h=1, pad=(0, 0))
    assert "stride" in bad(stride=(0, 1))
    assert "ctas" in bad(ctas=0)


def test_default_pool_needs_a_device():
    # Without a GPU the default pool cannot be resolved: -1 (HIP error), and
    # the library stays usable.
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present")
    except ImportError:
        pass
    with pytest.raises(skg.SkgError) as ei:
        skg.plan_gemm(M=256, N=256, K=256, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                      mode="dp_sk", reduction="linear", ctas=-1)
    assert ei.value.status == -1
    assert skg.plan_gemm(M=256, N=256, K=256, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
                         mode="dp_sk", reduction="linear", ctas=4)["pool"] == 4


# --- flag ordering in the built code object -------------------------------
LLVM = "/opt/rocm/llvm/bin"


def code_objects(tmp):
    """Disassembly of every gfx950 code object bundled in the library."""
    fat = os.path.join(tmp, "fatbin")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section",
                    ".hip_fatbin=" + fat, _lib.LIB_PATH, os.path.join(tmp, "lib.copy")],
                   check=True, capture_output=True)
    data = open(fat, "rb").read()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    out = []
    for i, s in enumerate(starts):
        e = starts[i + 1] if i + 1 < len(starts) else len(data)
        part = os.path.join(tmp, "b%d" % i)
        open(part, "wb").write(data[s:e])
        co = part + ".co"
        r = subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--type=o", "--unbundle",
                            "--input=" + part, "--output=" + co,
                            "--targets=hipv4-amdgcn-amd-amdhsa--gfx950"], capture_output=True)
        if r.returncode != 0 or not os.path.getsize(co):
            continue
        dis = subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", co], check=True,
                             capture_output=True, text=True).stdout
        out.append(dis)
    return out


def kernels(dis):
    parts = re.split(r"\n[0-9a-f]+ <(\w+)>:\n", dis)
    return {parts[i]: parts[i + 1] for i in range(1, len(parts) - 1, 2)}


def instrs(body):
    res = []
    for line in body.split("\n"):
        t = line.strip()
        if not t or t.startswith(";"):
            continue
        res.append(t.split("//")[0].strip())
    return res


def test_flag_ordering_in_isa():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("library not built")
    with tempfile.TemporaryDirectory() as tmp:
        objs = code_objects(tmp)
    assert objs, "no gfx950 code object in the library"
    n_kernels = n_atomic = 0
    for dis in objs:
        for name, body in kernels(dis).items():
            if "sk_kernel" not in name:
                continue
            n_kernels += 1
            ins = instrs(body)
            # No L2-wide write-back or invalidation anywhere in the kernel.
            assert not any(x.startswith(("buffer_wbl2", "buffer_inv")) for x in ins), name
            # The last template argument is the fix-up family: 1 = atomic /
            # workspace, which hands nothing on and waits for nothing.
            fam = re.search(r"ELi([01])EEEvNT", name)
            assert fam, name
            if fam.group(1) == "1":
                n_atomic += 1
                assert not any(x.endswith("sc1") and x.startswith(("global_store", "global_load"))
                               for x in ins), name + ": flags in an atomic-family kernel"
                assert any(x.startswith("global_atomic_add_f32") for x in ins), name
                continue
            # Partials go out and come back at device scope (sc1).
            assert any(x.startswith("buffer_store_dwordx4") and x.endswith("sc1") for x in ins), name
            assert any(x.startswith("buffer_load_dwordx4") and x.endswith("sc1") for x in ins), name
            # The flag store (the only device-scope global store) comes right
            # after a wait for every earlier store of the wave: a full vmcnt
            # drain with no store between it and the flag (the compiler may
            # add weaker waits of its own in between).
            flags = [i for i, x in enumerate(ins)
                     if x.startswith("global_store_dword ") and x.endswith("sc1")]
            assert flags, name + ": no device-scope flag store"
            for i in flags:
                w = [j for j in range(max(0, i - 6), i)
                     if ins[j].startswith("s_waitcnt") and "vmcnt(0)" in ins[j]]
                assert w, name
                between = ins[w[-1] + 1:i]
                assert not any(x.startswith(("buffer_store", "global_store")) for x in between), name
            polls = [x for x in ins if x.startswith("global_load_dword ") and x.endswith("sc1")]
            assert polls, name + ": no device-scope poll"
    assert n_kernels >= 40 and n_atomic == n_kernels // 2


def test_sk_order_resolution_and_rejection():
    g = dict(M=600, N=400, K=4096, dtype_ab="f16", dtype_c="f16", tile="128x128x32",
             mode="dp_sk", reduction="tree", ctas=13)
    assert skg.plan_gemm(**g)["sk_order"] == _lib.SK_ORDER_BLOCK
    assert skg.plan_gemm(sk_order="xcd", **g)["sk_order"] == _lib.SK_ORDER_XCD
    w = dict(n=2, h=9, w=9, c=16, k=24, r=3, s=3, stride=(1, 1), pad=(1, 1), groups=1,
             dtype="bf16", tile="128x128x64", mode="dp_sk", reduction="linear", ctas=8)
    assert skg.plan_wgrad(**w)["sk_order"] == _lib.SK_ORDER_XCD
    assert skg.plan_wgrad(sk_order="block", **w)["sk_order"] == _lib.SK_ORDER_BLOCK
    # the order changes no field of the partition
    a, b = skg.plan_gemm(**g), skg.plan_gemm(sk_order="xcd", **g)
    assert all(a[f] == b[f] for f in FIELDS)
    assert "order" in rejected(skg.plan_gemm, sk_order=4, **g)
    assert "order" in rejected(skg.plan_wgrad, sk_order=-1, **w)


def test_kmajor_order_needs_whole_slices():
    # K-major runs only where every stream-K CTA holds one whole slice of one
    # tile (split-K, or a pool that divides the iterations so); any other
    # partition reports the XCD order it falls back to.
    g = dict(M=512, N=512, K=8192, dtype_ab="bf16", dtype_c="bf16", tile="256x256x64")
    p = skg.plan_gemm(mode="splitk", reduction="workspace", ctas=16, sk_order="kmajor", **g)  # 16 slices
    S = p["iters_per_tile"] // p["iters_per_sk_cta"]
    assert p["extra_iters"] == 0 and p["sk_ctas"] == p["sk_tiles"] * S and S > 1
    assert p["sk_order"] == _lib.SK_ORDER_KMAJOR
    q = skg.plan_gemm(mode="dp_sk", reduction="tree", ctas=7, sk_order="kmajor", **g)
    assert q["extra_iters"] != 0 and q["sk_order"] == _lib.SK_ORDER_XCD
    w = dict(n=4, h=14, w=14, c=64, k=64, r=3, s=3, stride=(1, 1), pad=(1, 1), groups=1,
             dtype="f16", tile="128x128x64", mode="dp_sk", reduction="linear")
    pw = skg.plan_wgrad(ctas=2 * 5, sk_order="kmajor", **w)  # 5 tiles x 2 slices of 6.5 iterations
    assert pw["sk_order"] == _lib.SK_ORDER_XCD
    pw = skg.plan_wgrad(ctas=5 * 13, sk_order="kmajor", **w)  # 5 tiles x 13 slices of 1 iteration
    assert pw["iters_per_tile"] == 13 and pw["sk_order"] == _lib.SK_ORDER_KMAJOR


def kmajor_map(sk_ctas, sk_tiles):
    """The block -> stream-K CTA map documented for SKG_SK_ORDER_KMAJOR."""
    S = sk_ctas // sk_tiles
    q, r = sk_ctas // 8, sk_ctas % 8
    out = []
    for b in range(sk_ctas):
        c = (b % 8) * q + min(b % 8, r) + b // 8
        s, t = c // sk_tiles, c % sk_tiles
        out.append(t * S + s)
    return out


def test_kmajor_order_is_a_permutation_grouping_slices_by_xcd():
    # Every CTA runs once, and the CTAs an XCD runs are whole slices (the same
    # k range) of consecutive tiles: at most ceil(run / tiles) + 1 distinct
    # slices per XCD.
    for T, S in [(1, 7), (9, 28), (18, 14), (5, 13), (3, 100), (16, 16), (7, 1)]:
        m = kmajor_map(T * S, T)
        assert sorted(m) == list(range(T * S)), (T, S)
        for x in range(8):
            cs = [m[b] for b in range(x, T * S, 8)]
            slices = {c % S for c in cs}
            assert len(slices) <= -(-len(cs) // T) + 1, (T, S, x)


def test_xcd_order_is_a_permutation_into_contiguous_runs():
    # The block -> stream-K CTA map documented for SKG_SK_ORDER_XCD: every
    # CTA runs exactly once, and the CTAs of one XCD (blocks b with the same
    # b mod 8) form one contiguous run, in block order.
    for S in list(range(1, 70)) + [255, 256, 257, 480, 1216]:
        q, r = S // 8, S % 8
        m = [(b % 8) * q + min(b % 8, r) + b // 8 for b in range(S)]
        assert sorted(m) == list(range(S)), S
        for x in range(8):
            run = [m[b] for b in range(x, S, 8)]
            assert run == list(range(run[0], run[0] + len(run))) if run else True, (S, x)


def test_scatter_plan_matches_oracle_and_rejects_partial_slices():
    # The reduce-scatter fix-up: accepted on whole-slice partitions with the
    # oracle's plan (linear / tree workspace), -2 before any launch otherwise.
    g = dict(M=512, N=384, K=64 * 24, dtype_ab="bf16", dtype_c="f32", tile="128x128x64")
    for S in (2, 3, 4, 6, 8, 12, 24):
        c = skg.plan_gemm(mode="dp_sk", reduction="scatter", ctas=12 * S, **g)
        o = P.plan(4, 3, 24, 128, 128, 4, "dp_sk", "scatter", 12 * S)
        assert all(c[f] == getattr(o, f) for f in FIELDS), S
        assert c["reduction"] == _lib.RED_SCATTER
        t = skg.plan_gemm(mode="dp_sk", reduction="tree", ctas=12 * S, **g)
        assert c["workspace_bytes"] == t["workspace_bytes"] > 0
        sp = skg.plan_gemm(mode="splitk", reduction="scatter", ctas=S, **g)
        assert sp["slices"] == S and sp["sk_ctas"] == 12 * S
    for ctas in (5, 13, 12 * 5, 12 * 7):   # ranges straddling tiles / uneven slices
        msg = rejected(skg.plan_gemm, mode="dp_sk", reduction="scatter", ctas=ctas, **g)
        assert "whole slice" in msg, ctas
    assert "whole slice" in rejected(skg.plan_gemm, mode="splitk", reduction="scatter", ctas=5, **g)
    # nothing to reduce: accepted
    assert skg.plan_gemm(mode="dp", reduction="scatter", ctas=12, **g)["sk_ctas"] == 0
    assert skg.skg_default_pool(_lib.RED_SCATTER, 304, 8) == 304
    assert "reduction" in rejected(skg.plan_gemm, mode="dp_sk", reduction=6, ctas=24, **g)
