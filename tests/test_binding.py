"""The Python binding refuses bad tensor arguments before any pointer reaches
the library (CPU only).  Stand-in tensors carry the device, dtype, shape and
size that the checks look at; the library is replaced by a proxy that answers
the host-only size queries and fails the test if any device entry point is
called.  Also checks that Lane.begin records its tensors on the lane's stream,
so the caching allocator keeps their memory until the lane's kernels are done.
"""

import ctypes

import numpy as np
import pytest
import torch

from lib_util import ensure_built

import bit_moe_expert_fp9_amd as dm
from bit_moe_expert_fp9_amd import duckmoe as dmm

H, I, E, K = 1040, 336, 24, 8


class FakeTensor:
    """What the binding's checks read from a tensor, without device memory."""

    def __init__(self, shape, dtype, device="cuda:0", contiguous=True):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self._contiguous = contiguous
        self.streams = []

    def dim(self):
        return len(self.shape)

    def numel(self):
        return int(np.prod(self.shape)) if self.shape else 1

    def is_contiguous(self):
        return self._contiguous

    def element_size(self):
        return torch.empty(0, dtype=self.dtype).element_size()

    def data_ptr(self):
        return 1 << 20

    def record_stream(self, s):
        self.streams.append(s)


class FakeStream:
    cuda_stream = 0


class HostOnlyLib:
    """The real library for size queries; any other entry point fails the test."""

    HOST = {"duckmoe_workspace_bytes", "duckmoe_prefill_workspace_bytes",
            "duckmoe_stack_workspace_bytes", "duckmoe_strerror"}

    def __init__(self, real, allow=()):
        self.real = real
        self.allow = dict(allow)
        self.calls = []

    def __getattr__(self, name):
        if name in self.HOST:
            return getattr(self.real, name)
        if name in self.allow:
            def f(*a):
                self.calls.append(name)
                return self.allow[name]
            return f
        raise AssertionError("%s reached the library" % name)


@pytest.fixture
def fake_lib(monkeypatch):
    real = ensure_built()
    proxy = HostOnlyLib(real)
    monkeypatch.setattr(dmm, "lib", lambda: proxy)
    return proxy


def fake_layer(device="cuda:0", I=I):
    lay = dm.Layer.__new__(dm.Layer)
    lay.hidden, lay.inter, lay.n_routed, lay.top_k = H, I, E, K
    mat = H * I
    lay.gu_body = FakeTensor(((E + 1) * 2 * mat,), torch.uint8, device)
    lay.gu_sign = FakeTensor(((E + 1) * 2 * mat // 8,), torch.uint8, device)
    lay.dn_body = FakeTensor(((E + 1) * mat,), torch.uint8, device)
    lay.dn_sign = FakeTensor(((E + 1) * mat // 8,), torch.uint8, device)
    lay.struct = dm.LayerStruct(H, I, E, K, 256, 256, 256, 256)
    return lay


def layer_args(T=2, ns=1, I=I, **over):
    lay = fake_layer(I=I)
    a = dict(x=FakeTensor((T, H), torch.float32), ids=FakeTensor((T, K), torch.int32),
             w=FakeTensor((T, K), torch.float32),
             out=FakeTensor((T, H) if ns == 1 else (ns, T, H), torch.float32),
             ws=FakeTensor((lay.workspace_bytes(T, ns),), torch.uint8))
    a.update(over)
    return lay, a


def test_layer_call_accepts_good_arguments(fake_lib):
    fake_lib.allow["duckmoe_moe_layer"] = 0
    lay, a = layer_args()
    dm.moe_layer(lay, a["x"], a["ids"], a["w"], out=a["out"], ws=a["ws"], stream=FakeStream())
    assert fake_lib.calls == ["duckmoe_moe_layer"]


@pytest.mark.parametrize("case, msg", [
    (dict(x=torch.zeros(2, H)), "device tensor"),                        # a host tensor
    (dict(x=FakeTensor((2, H + 16), torch.float32)), "x must be"),        # wrong hidden size
    (dict(x=FakeTensor((2, H), torch.float64)), "must be torch.float32"),
    (dict(x=FakeTensor((2, H), torch.float32, "cuda:1")), "is on"),     # not the layer's device
    (dict(x=FakeTensor((2, H), torch.float32, contiguous=False)), "contiguous"),
    (dict(ids=FakeTensor((2, K + 1), torch.int32)), "ids must have shape"),
    (dict(ids=FakeTensor((2, K), torch.int64)), "int32"),
    (dict(w=FakeTensor((1, K), torch.float32)), "w must have shape"),
    (dict(out=FakeTensor((1, H), torch.float32)), "out holds"),
    (dict(out=FakeTensor((2, H), torch.int32)), "out must be"),
    (dict(ws=FakeTensor((1024,), torch.uint8)), "ws holds"),
    (dict(ws=FakeTensor((1 << 20,), torch.int32)), "ws must be"),
])
def test_layer_call_rejects(fake_lib, case, msg):
    lay, a = layer_args(**case)
    with pytest.raises(ValueError, match=msg):
        dm.moe_layer(lay, a["x"], a["ids"], a["w"], out=a["out"], ws=a["ws"])


def test_token_count_and_shards(fake_lib):
    lay = fake_layer()
    with pytest.raises(ValueError, match="tokens"):
        dm.moe_layer(lay, FakeTensor((9, H), torch.float32), FakeTensor((9, K), torch.int32),
                     FakeTensor((9, K), torch.float32))
    # 32 shard partials need a [32, T, H] output: a [T, H] one would be written 32x past its end
    lay, a = layer_args(T=2, ns=3, I=1536, out=FakeTensor((2, H), torch.float32))
    with pytest.raises(ValueError, match="out holds"):
        dm.moe_layer(lay, a["x"], a["ids"], a["w"], out=a["out"], n_shards=3, ws=a["ws"])


def test_other_entry_points_reject(fake_lib):
    lay = fake_layer()
    f32, i32, u8 = torch.float32, torch.int32, torch.uint8
    with pytest.raises(ValueError, match="expert"):
        dm.expert_ffn(lay, E + 1, FakeTensor((1, H), f32))
    with pytest.raises(ValueError, match="required"):
        dm.moe_layer_noalloc(lay, FakeTensor((1, H), f32), FakeTensor((1, K), i32),
                             FakeTensor((1, K), f32), None)
    with pytest.raises(ValueError, match="out holds"):
        dm.moe_layer_noalloc(lay, FakeTensor((1, H), f32), FakeTensor((1, K), i32),
                             FakeTensor((1, K), f32), FakeTensor((H - 1,), f32))
    with pytest.raises(ValueError, match="ids must have shape"):
        dm.moe_prefill(lay, FakeTensor((70, H), f32), FakeTensor((70, K - 1), i32),
                       FakeTensor((70, K - 1), f32))
    with pytest.raises(ValueError, match="ws holds"):
        dm.moe_prefill(lay, FakeTensor((70, H), f32), FakeTensor((70, K), i32),
                       FakeTensor((70, K), f32), out=FakeTensor((70, H), f32),
                       ws=FakeTensor((4096,), u8))
    with pytest.raises(ValueError, match="x holds"):
        dm.gemv_fp9(FakeTensor((256, 512), u8), FakeTensor((256, 64), u8), FakeTensor((500,), f32))
    with pytest.raises(ValueError, match="sign holds"):
        dm.gemv_fp9(FakeTensor((256, 512), u8), FakeTensor((255, 64), u8), FakeTensor((512,), f32))
    with pytest.raises(ValueError, match="n = "):
        dm.decode_fp9(FakeTensor((100,), u8), FakeTensor((13,), u8), n=101)
    with pytest.raises(ValueError, match="device tensor"):
        dm.moe_plan(torch.zeros((1, K), dtype=i32), E)
    with pytest.raises(ValueError, match="exceeds"):
        dm.read_probe(FakeTensor((1024,), u8), 2048, FakeTensor((1,), i32))
    with pytest.raises(ValueError, match="out holds"):
        dm.rms_normalize(FakeTensor((2, H), f32), out=FakeTensor((2, H - 1), f32))
    with pytest.raises(ValueError, match="body holds"):
        dm.quantize_fp9_device(FakeTensor((16, 64), f32), body=FakeTensor((16 * 63,), u8),
                               sign=FakeTensor((128,), u8))
    with pytest.raises(ValueError, match="shape"):
        lay.set_expert(0, np.zeros((I, H), np.float32), np.zeros((I, H), np.float32),
                       np.zeros((I, H), np.float32))


def test_stack_rejects(fake_lib):
    lays = [fake_layer() for _ in range(3)]
    st = dm.Stack.__new__(dm.Stack)
    st.layers = lays
    st.structs = (dm.LayerStruct * 3)(*[l.struct for l in lays])
    f32, i32 = torch.float32, torch.int32
    with pytest.raises(ValueError, match="ids must have shape"):
        dm.moe_stack(st, FakeTensor((2, H), f32), FakeTensor((2, 2, K), i32),
                     FakeTensor((3, 2, K), f32))
    with pytest.raises(ValueError, match="ws holds"):
        dm.moe_stack(st, FakeTensor((2, H), f32), FakeTensor((3, 2, K), i32),
                     FakeTensor((3, 2, K), f32), out=FakeTensor((2, H), f32),
                     ws=FakeTensor((100,), torch.uint8))


def test_lane_begin_records_streams(fake_lib):
    fake_lib.allow["duckmoe_lane_begin"] = 0
    lay = fake_layer()
    lane = dm.Lane.__new__(dm.Lane)
    lane.max_tokens = 1
    lane.stream = FakeStream()
    lane.ws = FakeTensor((lay.workspace_bytes(1),), torch.uint8)
    lane.struct = dmm.LaneStruct(0, 0, 0, None, None, 0)
    x, ids, w = (FakeTensor((1, H), torch.float32), FakeTensor((1, K), torch.int32),
                 FakeTensor((1, K), torch.float32))
    out = FakeTensor((1, H), torch.float32)
    lane.begin(lay, x, ids, w, out, producer=FakeStream())
    assert fake_lib.calls == ["duckmoe_lane_begin"]
    for t in (x, ids, w, out):
        assert t.streams == [lane.stream]
    # more tokens than the lane's workspace was sized for
    with pytest.raises(ValueError, match="tokens"):
        lane.begin(lay, FakeTensor((2, H), torch.float32), FakeTensor((2, K), torch.int32),
                   FakeTensor((2, K), torch.float32), FakeTensor((2, H), torch.float32),
                   producer=FakeStream())
    assert fake_lib.calls == ["duckmoe_lane_begin"]
