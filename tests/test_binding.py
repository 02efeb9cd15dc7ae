"""Host-side behaviour of the Python binding (no GPU, no compute call).

The binding allocates the backward's and decode's scratch (and the wrappers'
outputs) with torch on the current stream.  When the work is enqueued on
another stream, those blocks must be recorded as in use by that stream, or
torch's caching allocator may hand them to a new allocation on the current
stream while the kernels still read or write them.  These tests replace the
library and torch's allocation with recording stand-ins and check that every
path that allocates records the stream it launches on.
"""

from types import SimpleNamespace

import pytest
import torch

from io_aware_exact_09_amd import fa


class FakeTensor:
    """Just enough of a device tensor for the binding's checks."""
    _next = 1

    def __init__(self, shape, dtype=torch.bfloat16):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = SimpleNamespace(type="cuda")
        self.recorded = []
        self._ptr = FakeTensor._next << 24
        FakeTensor._next += 1

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return self._ptr

    def numel(self):
        n = 1
        for s in self.shape:
            n *= s
        return n

    def element_size(self):
        return 2 if self.dtype == torch.bfloat16 else 4 if self.dtype != torch.uint8 else 1

    def record_stream(self, s):
        self.recorded.append(s)


class FakeLib:
    """Every entry point returns FA_OK; size queries return 4096."""

    def __getattr__(self, name):
        if name.endswith("_bytes"):
            return lambda *a: 4096
        if name == "fa_decode_num_splits":
            return lambda *a: 4
        return lambda *a: 0


@pytest.fixture
def fake(monkeypatch):
    made = []

    def empty(*shape, dtype=None, device=None, **kw):
        if len(shape) == 1 and isinstance(shape[0], (tuple, list, torch.Size)):
            shape = tuple(shape[0])
        t = FakeTensor(shape if shape else (1,), dtype or torch.float32)
        made.append(t)
        return t

    def empty_like(x, **kw):
        t = FakeTensor(x.shape, x.dtype)
        made.append(t)
        return t

    monkeypatch.setattr(fa, "load_library", lambda *a, **k: FakeLib())
    monkeypatch.setattr(fa.torch, "empty", empty)
    monkeypatch.setattr(fa.torch, "empty_like", empty_like)
    monkeypatch.setattr(fa.torch.cuda, "current_stream", lambda *a: SimpleNamespace(cuda_stream=0))
    return made


def side_stream():
    return SimpleNamespace(cuda_stream=0x1234)


def qkv(B=1, H=2, N=128, d=64, Hkv=None):
    q = FakeTensor((B, H, N, d))
    k = FakeTensor((B, Hkv or H, N, d))
    v = FakeTensor((B, Hkv or H, N, d))
    return q, k, v


def test_scratch_records_the_launch_stream(fake):
    q, _, _ = qkv()
    s = side_stream()
    ws = fa._scratch(100, q, s)
    assert ws.recorded == [s]
    ws2 = fa._scratch(100, q, None)          # current stream: nothing to record
    assert ws2.recorded == []


@pytest.mark.parametrize("entry", ["fa_bwd", "fa_bwd_dropout", "fa_bwd_gqa"])
def test_backward_workspace_is_recorded_on_the_launch_stream(fake, entry):
    q, k, v = qkv(Hkv=1 if entry == "fa_bwd_gqa" else None)
    o, do = FakeTensor(q.shape), FakeTensor(q.shape)
    lse = FakeTensor(q.shape[:3], torch.float32)
    dq, dk, dv = FakeTensor(q.shape), FakeTensor(k.shape), FakeTensor(v.shape)
    s = side_stream()
    args = (q, k, v, o, do, lse, dq, dk, dv, 0.125)
    if entry == "fa_bwd_dropout":
        getattr(fa, entry)(*args, 0.1, 7, stream=s)
    else:
        getattr(fa, entry)(*args, stream=s)
    ws = [t for t in fake if t.dtype == torch.uint8]
    assert len(ws) == 1 and ws[0].recorded == [s]
    # a caller-supplied workspace is the caller's to manage: nothing allocated
    fake.clear()
    getattr(fa, entry)(*args, *((0.1, 7) if entry == "fa_bwd_dropout" else ()),
                       workspace=FakeTensor((4096,), torch.uint8), stream=s)
    assert fake == []


def test_decode_workspace_is_recorded_on_the_launch_stream(fake):
    q = FakeTensor((2, 8, 1, 128))
    k, v = FakeTensor((2, 2, 4096, 128)), FakeTensor((2, 2, 4096, 128))
    o, lse = FakeTensor(q.shape), FakeTensor(q.shape[:3], torch.float32)
    s = side_stream()
    fa.fa_decode(q, k, v, o, lse, 0.1, stream=s)
    ws = [t for t in fake if t.dtype == torch.uint8]
    assert len(ws) == 1 and ws[0].recorded == [s]


def test_wrapper_outputs_are_recorded_on_the_launch_stream(fake):
    q, k, v = qkv()
    s = side_stream()
    o, lse = fa.forward(q, k, v, 0.125, stream=s)
    assert o.recorded == [s] and lse.recorded == [s]
    do = FakeTensor(q.shape)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, 0.125, stream=s)
    assert all(t.recorded == [s] for t in (dq, dk, dv))
    fake.clear()
    o2, lse2 = fa.forward(q, k, v, 0.125)
    assert o2.recorded == [] and lse2.recorded == []
