"""The C ABI loads, exports every declared entry point, and rejects bad
arguments on the host before launching anything (CPU only: no GPU needed,
since every call here returns before touching the HIP runtime)."""

import ctypes
import os
import re

import numpy as np
import pytest

from lib_util import ROOT, ensure_built

import bit_moe_expert_fp9_amd as dm
from bit_moe_expert_fp9_amd.duckmoe import LayerStruct

HEADER = os.path.join(ROOT, "include", "duckmoe.h")


@pytest.fixture(scope="module")
def L():
    return ensure_built()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(duckmoe_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(dm.EXPORTS) == names


def test_strerror(L):
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert L.duckmoe_strerror(code)
    assert dm.strerror(-4) == "workspace too small"


def test_quantize_errors(L):
    w = np.zeros((2, 8), dtype=np.float32)
    b = np.zeros((2, 8), dtype=np.uint8)
    s = np.zeros((2, 1), dtype=np.uint8)
    f = L.duckmoe_quantize_fp9
    assert f(w.ctypes.data, 2, 8, b.ctypes.data, s.ctypes.data) == 0
    assert f(w.ctypes.data, 2, 12, b.ctypes.data, s.ctypes.data) == dm.duckmoe.ESHAPE
    assert f(w.ctypes.data, -1, 8, b.ctypes.data, s.ctypes.data) == dm.duckmoe.EINVAL
    assert f(None, 2, 8, b.ctypes.data, s.ctypes.data) == dm.duckmoe.EINVAL
    assert f(None, 0, 8, None, None) == 0
    w[1, 3] = np.nan
    assert f(w.ctypes.data, 2, 8, b.ctypes.data, s.ctypes.data) == dm.duckmoe.ENONFINITE


FAKE = 0x10000  # an aligned address that is never dereferenced


def fake_layer(H=7168, I=2048, E=256, k=8):
    return LayerStruct(H, I, E, k, FAKE, FAKE, FAKE, FAKE)


def test_workspace_bytes(L):
    lay = fake_layer()
    f = L.duckmoe_workspace_bytes
    # 1 KiB header (status, plan) + h' [T*top_k+1][T][I] f32
    hdr = 1024
    assert f(ctypes.byref(lay), 1, 1) == hdr + 9 * 1 * 2048 * 4
    assert f(ctypes.byref(lay), 2, 32) == hdr + 17 * 2 * 2048 * 4
    assert f(ctypes.byref(lay), 0, 1) == 0
    assert f(ctypes.byref(lay), 9, 1) == 0
    assert f(ctypes.byref(lay), 1, 3) == 0      # 2048 / 3 not integral
    assert f(ctypes.byref(lay), 1, 64) == 0     # slice of 32 < 64
    wide = fake_layer(I=3072)                    # 3 chunks of 1024: no shard partials
    assert f(ctypes.byref(wide), 1, 1) == hdr + 9 * 3072 * 4
    assert f(ctypes.byref(wide), 1, 3) == 0
    dense = fake_layer(I=18432, E=0, k=1)        # a dense MLP: one expert, index 0
    assert f(ctypes.byref(dense), 1, 1) == hdr + 2 * 18432 * 4
    assert f(None, 1, 1) == 0


def call_layer(L, lay, x=FAKE, ids=FAKE, w=FAKE, T=1, out=FAKE, ns=1, ws=FAKE,
               ws_bytes=1 << 30, fn="duckmoe_moe_layer"):
    return getattr(L, fn)(ctypes.byref(lay) if lay is not None else None, x, ids, w, T, out,
                          ns, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["duckmoe_moe_layer", "duckmoe_moe_gate_up", "duckmoe_moe_down"])
def test_layer_argument_errors(L, fn):
    E = dm.duckmoe
    lay = fake_layer()
    c = lambda **kw: call_layer(L, lay, fn=fn, **kw)
    assert call_layer(L, None, fn=fn) == E.EINVAL
    assert c(T=0) == E.EINVAL
    assert c(T=9) == E.EINVAL
    assert c(ids=None) == E.EINVAL
    assert c(w=None) == E.EINVAL
    assert c(x=None) == E.EINVAL
    assert c(out=None) == E.EINVAL
    assert c(ws=None) == E.EINVAL
    assert c(x=FAKE + 4) == E.EINVAL      # x must be 16-byte aligned
    assert c(ws=FAKE + 16) == E.EINVAL    # workspace 256-byte aligned
    assert c(ns=3) == E.ESHAPE
    assert c(ns=64) == E.ESHAPE
    assert c(ws_bytes=1000) == E.EWORKSPACE
    big = fake_layer(k=40)
    assert call_layer(L, big, T=2, fn=fn) == E.ESHAPE   # T * top_k > 64
    for bad in (fake_layer(H=7160), fake_layer(I=2040), fake_layer(I=32784), fake_layer(E=-1),
                fake_layer(E=9000), fake_layer(k=0), fake_layer(H=65536, I=16384)):
        assert call_layer(L, bad, fn=fn) == E.ESHAPE
    mis = LayerStruct(7168, 2048, 256, 8, FAKE + 8, FAKE, FAKE, FAKE)
    assert call_layer(L, mis, fn=fn) == E.EINVAL


def prefill_ws_expected(H, I, E, k, T):
    """Workspace of a prefill call, from the documented parts (256-byte aligned
    each): header, list offsets, tile table, per-entry token/weight, tok_entry,
    x hi/lo + scales, h' hi/lo + per-unit scales, y."""
    a = lambda n: (n + 255) // 256 * 256
    Hp, Ip = -(-H // 128) * 128, -(-I // 128) * 128
    A = T * (k + 1)
    tiles = -(-A // 64) + E + 1
    parts = [256, (E + 2) * 4, tiles * 16, A * 4, A * 4, T * (k + 1) * 4, T * Hp * 2, T * Hp * 2,
             T * 4, A * Ip * 2, A * Ip * 2, A * (Ip // 128) * 4, A * H * 4]
    return sum(a(p) for p in parts)


def test_prefill_workspace_bytes(L):
    lay = fake_layer()
    f = lambda T, routed=1, lay=lay: L.duckmoe_prefill_workspace_bytes(ctypes.byref(lay), T, routed)
    for T in (1, 63, 2048, 32768):
        assert f(T) == prefill_ws_expected(7168, 2048, 256, 8, T)
    assert f(100, 0) == prefill_ws_expected(7168, 2048, 256, 0, 100)
    odd = fake_layer(H=1040, I=336, E=24, k=8)
    assert f(333, lay=odd) == prefill_ws_expected(1040, 336, 24, 8, 333)
    assert f(0) == 0 and f(32769) == 0
    assert f(1, lay=fake_layer(E=1025)) == 0          # more routed experts than the lists take
    assert f(1, lay=fake_layer(k=33)) == 0            # top_k above 32 with ids
    assert f(1, 0, lay=fake_layer(k=33)) > 0          # ... but fine without ids
    assert L.duckmoe_prefill_workspace_bytes(None, 1, 1) == 0


def test_prefill_errors(L):
    E = dm.duckmoe
    lay = fake_layer()

    def c(lay=lay, x=FAKE, ids=FAKE, w=FAKE, T=4, out=FAKE, ws=FAKE, wsb=1 << 40):
        return L.duckmoe_moe_prefill(ctypes.byref(lay) if lay is not None else None, x, ids, w,
                                     T, out, ws, wsb, None)
    assert c(lay=None) == E.EINVAL
    assert c(T=0) == E.EINVAL and c(T=32769) == E.EINVAL
    assert c(w=None) == E.EINVAL
    assert c(x=None) == E.EINVAL and c(out=None) == E.EINVAL and c(ws=None) == E.EINVAL
    assert c(x=FAKE + 4) == E.EINVAL and c(out=FAKE + 8) == E.EINVAL
    assert c(ws=FAKE + 16) == E.EINVAL
    assert c(wsb=1000) == E.EWORKSPACE
    assert c(ids=None, w=None, wsb=1000) == E.EWORKSPACE   # shared-only: w unused
    for bad in (fake_layer(H=7160), fake_layer(I=2040), fake_layer(E=1025), fake_layer(k=33),
                fake_layer(H=65536, I=16384)):
        assert c(lay=bad) == E.ESHAPE
    # x hi/lo above 2 GiB
    assert c(lay=fake_layer(H=32768, I=2048), T=32768) == E.ESHAPE
    mis = LayerStruct(7168, 2048, 256, 8, FAKE, FAKE + 1, FAKE, FAKE)
    assert c(lay=mis) == E.EINVAL
    p = L.duckmoe_prefill_plan
    assert p(FAKE, FAKE, 0, 8, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.EINVAL
    assert p(FAKE, FAKE, 4, 33, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.EINVAL
    assert p(FAKE, FAKE, 4, 8, 1025, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.EINVAL
    assert p(None, FAKE, 4, 8, 256, FAKE, FAKE, FAKE, FAKE, FAKE, None) == E.EINVAL
    assert p(FAKE, FAKE, 4, 8, 256, FAKE, FAKE, FAKE, None, FAKE, None) == E.EINVAL


def test_expert_ffn_errors(L):
    E = dm.duckmoe
    lay = fake_layer()
    f = lambda e, T=1, ns=1, wsb=1 << 30: L.duckmoe_expert_ffn(ctypes.byref(lay), e, FAKE, T, FAKE,
                                                             ns, FAKE, wsb, None)
    assert f(-1) == E.EINVAL
    assert f(257) == E.EINVAL
    assert f(0, T=0) == E.EINVAL
    assert f(0, ns=5) == E.ESHAPE
    assert f(0, wsb=100) == E.EWORKSPACE


def test_building_block_errors(L):
    E = dm.duckmoe
    assert L.duckmoe_decode_fp9(FAKE, FAKE, -1, FAKE, None) == E.EINVAL
    assert L.duckmoe_decode_fp9(None, FAKE, 8, FAKE, None) == E.EINVAL
    assert L.duckmoe_decode_fp9(FAKE, FAKE, 0, FAKE, None) == 0
    assert L.duckmoe_gemv_fp9(FAKE, FAKE, 4, 12, FAKE, FAKE, None) == E.ESHAPE
    assert L.duckmoe_gemv_fp9(FAKE, FAKE, 4, 16, FAKE + 4, FAKE, None) == E.EINVAL
    assert L.duckmoe_gemv_fp9(FAKE, FAKE, 0, 16, FAKE, FAKE, None) == 0
    assert L.duckmoe_moe_plan(FAKE, 9, 8, 256, FAKE, FAKE, None) == E.EINVAL
    assert L.duckmoe_moe_plan(FAKE, 8, 9, 256, FAKE, FAKE, None) == E.ESHAPE
    assert L.duckmoe_moe_plan(None, 1, 8, 256, FAKE, FAKE, None) == E.EINVAL
    assert L.duckmoe_status(None, None, None) == E.EINVAL


def test_device_quantizer_and_glue_errors(L):
    E = dm.duckmoe
    q = L.duckmoe_quantize_fp9_device
    assert q(None, 2, 8, FAKE, FAKE, None, None) == E.EINVAL
    assert q(FAKE, -1, 8, FAKE, FAKE, None, None) == E.EINVAL
    assert q(FAKE, 2, 12, FAKE, FAKE, None, None) == E.ESHAPE
    assert q(FAKE + 4, 2, 8, FAKE, FAKE, None, None) == E.EINVAL   # w 16-byte aligned
    assert q(FAKE, 2, 8, FAKE + 4, FAKE, None, None) == E.EINVAL   # body 8-byte aligned
    assert q(FAKE, 0, 8, FAKE, FAKE, None, None) == 0
    assert q(None, 0, 8, None, None, None, None) == 0
    r = L.duckmoe_rms_normalize
    assert r(None, 1, 16, 0.0, FAKE, None) == E.EINVAL
    assert r(FAKE, -1, 16, 0.0, FAKE, None) == E.EINVAL
    assert r(FAKE, 1, 0, 0.0, FAKE, None) == E.EINVAL
    assert r(FAKE, 1, 16, -1.0, FAKE, None) == E.EINVAL
    assert r(FAKE, 1, 16, float("nan"), FAKE, None) == E.EINVAL
    assert r(FAKE, 0, 16, 0.0, FAKE, None) == 0


def test_fp8_converter_errors(L):
    E = dm.duckmoe
    f = lambda fp8=FAKE, sc=FAKE, r=2, c=8, b=128, body=FAKE, sign=FAKE: \
        L.duckmoe_fp8_to_fp9(fp8, sc, r, c, b, body, sign, None, None)
    assert f(r=-1) == E.EINVAL
    assert f(b=4) == E.EINVAL
    assert f(c=12) == E.ESHAPE
    assert f(b=100) == E.ESHAPE
    assert f(fp8=None) == E.EINVAL
    assert f(sc=None) == E.EINVAL
    assert f(fp8=FAKE + 4) == E.EINVAL
    assert f(body=FAKE + 4) == E.EINVAL
    assert f(sc=FAKE + 2) == E.EINVAL
    assert f(r=0, fp8=None, sc=None, body=None, sign=None) == 0


def test_lane_errors(L):
    from bit_moe_expert_fp9_amd.duckmoe import LaneStruct
    E = dm.duckmoe
    assert L.duckmoe_lane_init(None) == E.EINVAL
    assert L.duckmoe_lane_destroy(None) == E.EINVAL
    assert L.duckmoe_lane_finish(None, None) == E.EINVAL
    lane = LaneStruct(None, FAKE, 1 << 30, None, None)       # events never created
    lay = fake_layer()
    assert L.duckmoe_lane_begin(ctypes.byref(lane), ctypes.byref(lay), FAKE, FAKE, FAKE, 1,
                                FAKE, None) == E.EINVAL
    assert L.duckmoe_lane_finish(ctypes.byref(lane), None) == E.EINVAL
    assert L.duckmoe_lane_destroy(ctypes.byref(lane)) == 0   # nothing to release


def test_read_probe_errors(L):
    E = dm.duckmoe
    assert L.duckmoe_read_probe(None, 1024, FAKE, None) == E.EINVAL
    assert L.duckmoe_read_probe(FAKE, 1000, FAKE, None) == E.EINVAL
    assert L.duckmoe_read_probe(FAKE + 4, 1024, FAKE, None) == E.EINVAL
    assert L.duckmoe_read_probe(FAKE, 1024, None, None) == E.EINVAL
    assert L.duckmoe_read_probe(FAKE, 0, FAKE, None) == 0


def test_stack_errors(L):
    E = dm.duckmoe
    layers = (LayerStruct * 3)(fake_layer(), fake_layer(), fake_layer())
    wsb = L.duckmoe_stack_workspace_bytes
    one = 1024 + 9 * 2048 * 4
    assert wsb(layers, 3, 1) == (one + 255) // 256 * 256 + 2 * 7168 * 4
    assert wsb(layers, 0, 1) == 0
    assert wsb(layers, 3, 9) == 0
    assert wsb(None, 3, 1) == 0
    mixed = (LayerStruct * 2)(fake_layer(), fake_layer(I=1024))
    assert wsb(mixed, 2, 1) == 0
    st = lambda lay, n=3, x=FAKE, ids=FAKE, w=FAKE, T=1, eps=0.0, out=FAKE, ws=FAKE, b=1 << 30: \
        L.duckmoe_moe_stack(lay, n, x, ids, w, T, eps, out, ws, b, None)
    assert st(mixed, 2) == E.ESHAPE
    assert st(layers, 0) == E.EINVAL
    assert st(layers, T=9) == E.EINVAL
    assert st(layers, x=None) == E.EINVAL
    assert st(layers, ids=None) == E.EINVAL
    assert st(layers, eps=-1.0) == E.EINVAL
    assert st(layers, ws=FAKE + 16) == E.EINVAL
    assert st(layers, b=1000) == E.EWORKSPACE


def test_binding_raises_without_library(monkeypatch, tmp_path):
    from bit_moe_expert_fp9_amd import duckmoe
    monkeypatch.setattr(duckmoe, "_lib", None)
    monkeypatch.setattr(duckmoe, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        duckmoe.quantize_fp9(np.zeros((1, 8), dtype=np.float32))


def test_bench_refuses_several_gpus():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says why,
    before it touches torch or the library."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
