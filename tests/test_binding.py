"""CPU tests of the Python binding's marshalling (no GPU): a workspace the
binding allocates for a call is tied to the stream the kernel is launched
on, whichever stream the caller passes, and a caller's workspace is passed
through untouched."""

import implicit_gemm_conv_dp_amd as skg


class FakeBuffer:
    def __init__(self, nbytes):
        self.nbytes = nbytes
        self.recorded = []

    def record_stream(self, s):
        self.recorded.append(s)

    def data_ptr(self):
        return 0x10000

    def numel(self):
        return self.nbytes

    def element_size(self):
        return 1


class FakeStream:
    def __init__(self, handle):
        self.cuda_stream = handle


def test_temporary_workspace_is_tied_to_the_launch_stream(monkeypatch):
    made = []

    def fake_workspace_for(plan, device):
        b = FakeBuffer(max(int(plan["workspace_bytes"]), 1))
        made.append(b)
        return b

    calls = []
    monkeypatch.setattr(skg, "workspace_for", fake_workspace_for)
    side = FakeStream(0xABC)   # not the current stream
    plan = {"workspace_bytes": 4096}
    skg._run(lambda *a: calls.append(a), "args", plan, "cuda:0", None, side)
    assert len(made) == 1 and made[0].recorded == [side]
    assert calls == [("args", 0x10000, 4096, 0xABC)]


def test_caller_workspace_is_passed_through(monkeypatch):
    monkeypatch.setattr(skg, "workspace_for", lambda *a: (_ for _ in ()).throw(AssertionError))
    calls = []
    ws = FakeBuffer(8192)
    skg._run(lambda *a: calls.append(a), "args", {"workspace_bytes": 100}, "cuda:0", ws,
             FakeStream(7))
    assert ws.recorded == [] and calls == [("args", 0x10000, 8192, 7)]


def test_workspace_bytes_call_equals_plan():
    g = dict(M=4864, N=4096, K=4096, dtype_ab="bf16", dtype_c="bf16", tile="256x256x64",
             mode="dp_sk", reduction="tree", ctas=256)
    assert skg.skg_gemm_workspace_bytes(skg.gemm_args(**g)) == \
        skg.plan_gemm(**g)["workspace_bytes"] == 4096 + 256 * 256 * 256 * 4
    w = dict(n=32, h=56, w=56, c=256, k=256, r=3, s=3, stride=(1, 1), pad=(1, 1), groups=1,
             dtype="f16", tile="256x128x64", mode="dp_sk", reduction="workspace", ctas=256)
    assert skg.skg_wgrad_workspace_bytes(skg.wgrad_args(**w)) == \
        skg.plan_wgrad(**w)["workspace_bytes"] == 18 * 256 * 128 * 4
