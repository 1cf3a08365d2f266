"""Shared test helpers: device upload / download of operand codes and the
comparison metric.  The metric (max |Y - R| / max |R|, the infinity-norm
relative error) is our reading of the pages' "max relative error"; it is
test logic, not part of either implementation.  Alongside it, the
element-wise relative error over the entries with |R| >= 2^-4 max |R| is
computed and bounded, Inf and NaN entries fail, and rows holding a NaN are
reported as unwritten."""

import numpy as np
import torch

from oracle import codecs

VIEW = {"f16": torch.int16, "bf16": torch.int16, "e4m3": torch.uint8, "e5m2": torch.uint8,
        "f32": torch.int32}
NPV = {"f16": np.int16, "bf16": np.int16, "e4m3": np.uint8, "e5m2": np.uint8, "f32": np.int32}
TOL = {"f16": 5e-3, "bf16": 5e-3, "e4m3": 2e-2, "e5m2": 2e-2}


def to_dev(codes, fmt):
    a = np.ascontiguousarray(codes).view(NPV[fmt])
    return torch.from_numpy(a).to("cuda")


def to_dev_f32(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda")


def out_buffer(fmt, n, poison=True):
    t = torch.empty(n, dtype=VIEW[fmt], device="cuda")
    if poison:
        t.view(torch.uint8).fill_(0xFF)   # NaN in f16, bf16 and f32
    return t


def decode_out(t, fmt):
    a = t.cpu().numpy()
    if fmt == "f32":
        return a.view(np.float32).astype(np.float64)
    return codecs.decode(fmt, a.view(np.uint16))


def rel_err(y, r):
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    denom = np.max(np.abs(r))
    if denom == 0:
        return float(np.max(np.abs(y)))
    return float(np.max(np.abs(y - r)) / denom)


def unwritten_rows(y2d):
    """Rows (or output channels) holding any NaN: never written."""
    bad = np.isnan(y2d).any(axis=1)
    return np.nonzero(bad)[0].tolist()


# Floor of the element-wise diagnostic, relative to max |R|.
ELEM_FLOOR = 2.0 ** -4


def elem_rel_err(y, r, floor=ELEM_FLOOR):
    """max |Y - R| / |R| over the entries with |R| >= floor * max |R| (0 when
    no entry qualifies).  Entries that small relative to the largest are left
    out: on zero-mean data a relative error without a floor is unbounded."""
    y = np.asarray(y, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    big = np.abs(r) >= floor * np.max(np.abs(r))
    if not big.any():
        return 0.0
    return float(np.max(np.abs(y[big] - r[big]) / np.abs(r[big])))


def assert_close(y2d, r2d, fmt_in, label=""):
    rows = unwritten_rows(y2d)
    assert not rows, "%s: unwritten output rows %s" % (label, rows[:16])
    assert not np.isinf(y2d).any(), "%s: Inf in the output" % label
    err = rel_err(y2d, r2d)
    assert err <= TOL[fmt_in], "%s: max rel err %.3e > %.1e" % (label, err, TOL[fmt_in])
    # Entries at least 2^-4 of the largest: their own relative error cannot
    # exceed 16x the infinity-norm bound; anything beyond that is an entry
    # computed wrongly, not rounding.
    e = elem_rel_err(y2d, r2d)
    assert e <= TOL[fmt_in] / ELEM_FLOOR, "%s: element-wise rel err %.3e (|R| >= 2^-4 max)" % (label, e)
    DIAGS.append((fmt_in, label, err, e))
    return err


# (input format, label, infinity-norm rel err, element-wise rel err) of every
# assert_close in the session; conftest prints a summary at the end.
DIAGS = []
