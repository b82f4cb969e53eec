"""ctypes binding of libduckmoe (include/duckmoe.h).

Argument marshalling only: every step of the path runs inside the library.
torch provides device memory and the current stream; nothing here computes.
If the library is not built every call raises: there is no fallback.
"""

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import synth

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libduckmoe.so")

OK, EINVAL, ESHAPE, ENONFINITE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
STATUS_BAD_ID, STATUS_DUP_ID = 1, 2
MAX_TOKENS = 8

_lib = None


class DuckMoeError(RuntimeError):
    def __init__(self, code, where):
        super().__init__("%s: %s (%d)" % (where, strerror(code), code))
        self.code = code


class LayerStruct(ctypes.Structure):
    _fields_ = [
        ("hidden", ctypes.c_int32),
        ("inter", ctypes.c_int32),
        ("n_routed", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("gu_body", ctypes.c_void_p),
        ("gu_sign", ctypes.c_void_p),
        ("dn_body", ctypes.c_void_p),
        ("dn_sign", ctypes.c_void_p),
    ]


class LaneStruct(ctypes.Structure):
    _fields_ = [
        ("stream", ctypes.c_void_p),
        ("ws", ctypes.c_void_p),
        ("ws_bytes", ctypes.c_size_t),
        ("ready", ctypes.c_void_p),
        ("done", ctypes.c_void_p),
        ("cus", ctypes.c_int32),
    ]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_LAYER_ARGS = [ctypes.POINTER(LayerStruct), _P, _P, _P, _I32, _P, _I32, _P, _SZ, _P]

_SIGNATURES = {
    "duckmoe_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "duckmoe_quantize_fp9": ([_P, _I64, _I64, _P, _P], ctypes.c_int),
    "duckmoe_workspace_bytes": ([ctypes.POINTER(LayerStruct), _I32, _I32], _SZ),
    "duckmoe_moe_layer": (_LAYER_ARGS, ctypes.c_int),
    "duckmoe_moe_layer_noalloc": ([ctypes.POINTER(LayerStruct), _P, _P, _P, _I32, _P, _I32, _P],
                                  ctypes.c_int),
    "duckmoe_moe_gate_up": (_LAYER_ARGS, ctypes.c_int),
    "duckmoe_moe_down": (_LAYER_ARGS, ctypes.c_int),
    "duckmoe_expert_ffn": ([ctypes.POINTER(LayerStruct), _I32, _P, _I32, _P, _I32, _P, _SZ, _P],
                           ctypes.c_int),
    "duckmoe_status": ([_P, ctypes.POINTER(_I32), _P], ctypes.c_int),
    "duckmoe_decode_fp9": ([_P, _P, _I64, _P, _P], ctypes.c_int),
    "duckmoe_gemv_fp9": ([_P, _P, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "duckmoe_moe_plan": ([_P, _I32, _I32, _I32, _P, _P, _P], ctypes.c_int),
    "duckmoe_fp8_to_fp9": ([_P, _P, _I64, _I64, _I32, _P, _P, _P, _P], ctypes.c_int),
    "duckmoe_lane_init": ([ctypes.POINTER(LaneStruct)], ctypes.c_int),
    "duckmoe_lane_destroy": ([ctypes.POINTER(LaneStruct)], ctypes.c_int),
    "duckmoe_lane_begin": ([ctypes.POINTER(LaneStruct), ctypes.POINTER(LayerStruct), _P, _P, _P,
                            _I32, _P, _P], ctypes.c_int),
    "duckmoe_lane_finish": ([ctypes.POINTER(LaneStruct), _P], ctypes.c_int),
    "duckmoe_read_probe": ([_P, _SZ, _P, _P], ctypes.c_int),
    "duckmoe_quantize_fp9_device": ([_P, _I64, _I64, _P, _P, _P, _P], ctypes.c_int),
    "duckmoe_rms_normalize": ([_P, _I32, _I32, ctypes.c_float, _P, _P], ctypes.c_int),
    "duckmoe_stack_workspace_bytes": ([ctypes.POINTER(LayerStruct), _I32, _I32], _SZ),
    "duckmoe_moe_stack": ([ctypes.POINTER(LayerStruct), _I32, _P, _P, _P, _I32, ctypes.c_float,
                           _P, _P, _SZ, _P], ctypes.c_int),
    "duckmoe_prefill_workspace_bytes": ([ctypes.POINTER(LayerStruct), _I32, _I32], _SZ),
    "duckmoe_moe_prefill": ([ctypes.POINTER(LayerStruct), _P, _P, _P, _I32, _P, _P, _SZ, _P],
                            ctypes.c_int),
    "duckmoe_prefill_plan": ([_P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P], ctypes.c_int),
}

EXPORTS = tuple(_SIGNATURES)


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libduckmoe.so is not built: run "
                               "`python -m bit_moe_expert_fp9_amd.build` (needs hipcc)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def strerror(code):
    try:
        return lib().duckmoe_strerror(code).decode()
    except RuntimeError:
        return "error %d" % code


def _check(rc, where):
    if rc != OK:
        raise DuckMoeError(rc, where)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need_device(t, dtype, name, shape=None, numel=None, device=None):
    """Check a tensor argument before its pointer reaches the library: a
    contiguous device tensor of `dtype`, optionally of exactly `shape`, with at
    least `numel` elements, on `device`.  Raises ValueError (nothing is launched)."""
    if t is None:
        raise ValueError("%s is required" % name)
    dev = getattr(t, "device", None)
    if dev is None or dev.type != "cuda":
        raise ValueError("%s must be a device tensor" % name)
    if device is not None and dev != device:
        raise ValueError("%s is on %s, the layer's weights on %s" % (name, dev, device))
    if t.dtype != dtype:
        raise ValueError("%s must be %s, is %s" % (name, dtype, t.dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, has %s" % (name, tuple(shape), tuple(t.shape)))
    if numel is not None and t.numel() < numel:
        raise ValueError("%s holds %d elements, needs at least %d" % (name, t.numel(), numel))


def _need_tokens(T, limit=None):
    limit = MAX_TOKENS if limit is None else limit
    if not 1 <= T <= limit:
        raise ValueError("T = %d tokens: must be in [1, %d]" % (T, limit))


# ------------------------------------------------------------------ host ----

def quantize_fp9(w, body=None, sign=None):
    """float32 [rows, cols] -> (body uint8 [rows, cols], sign uint8 [rows, cols/8]).

    Host call into the library; `body`/`sign` may be preallocated numpy arrays.
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("quantize_fp9 takes a 2-D array")
    rows, cols = w.shape
    if body is None:
        body = np.empty((rows, cols), dtype=np.uint8)
    if sign is None:
        sign = np.empty((rows, max(cols // 8, 0)), dtype=np.uint8)
    rc = lib().duckmoe_quantize_fp9(w.ctypes.data, rows, cols, body.ctypes.data,
                                    sign.ctypes.data)
    _check(rc, "duckmoe_quantize_fp9")
    return body, sign


def quantize_fp9_device(w, body=None, sign=None, nonfinite=None, stream=None):
    """Device float32 [rows, cols] -> (body uint8, sign uint8) on the GPU.

    `body`/`sign` may be preallocated device tensors (flat or shaped, with at
    least rows*cols and rows*cols/8 elements from their start); `nonfinite`, a
    device int32 tensor, is set to 1 if w holds a NaN.
    """
    import torch
    _need_device(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [rows, cols]")
    rows, cols = w.shape
    if body is None:
        body = torch.empty((rows, cols), dtype=torch.uint8, device=w.device)
    if sign is None:
        sign = torch.empty((rows, max(cols // 8, 0)), dtype=torch.uint8, device=w.device)
    _need_device(body, torch.uint8, "body", numel=rows * cols, device=w.device)
    _need_device(sign, torch.uint8, "sign", numel=rows * (cols // 8), device=w.device)
    if nonfinite is not None:
        _need_device(nonfinite, torch.int32, "nonfinite", numel=1, device=w.device)
    _check(lib().duckmoe_quantize_fp9_device(_ptr(w), rows, cols, _ptr(body), _ptr(sign),
                                             _ptr(nonfinite), _stream(stream)),
           "duckmoe_quantize_fp9_device")
    return body, sign


def fp8_to_fp9_device(codes, scale, block=128, body=None, sign=None, nonfinite=None,
                      stream=None):
    """Device E4M3 codes [rows, cols] (uint8) with float32 block scales
    [ceil(rows/block), ceil(cols/block)] -> (body, sign) fp9 planes on the GPU."""
    import torch
    _need_device(codes, torch.uint8, "codes")
    if codes.dim() != 2 or block < 1:
        raise ValueError("codes must be 2-D [rows, cols] and block >= 1")
    rows, cols = codes.shape
    nb = (-(-rows // block), -(-cols // block))
    _need_device(scale, torch.float32, "scale", shape=nb, device=codes.device)
    if body is None:
        body = torch.empty((rows, cols), dtype=torch.uint8, device=codes.device)
    if sign is None:
        sign = torch.empty((rows, max(cols // 8, 0)), dtype=torch.uint8, device=codes.device)
    _need_device(body, torch.uint8, "body", numel=rows * cols, device=codes.device)
    _need_device(sign, torch.uint8, "sign", numel=rows * (cols // 8), device=codes.device)
    if nonfinite is not None:
        _need_device(nonfinite, torch.int32, "nonfinite", numel=1, device=codes.device)
    _check(lib().duckmoe_fp8_to_fp9(_ptr(codes), _ptr(scale), rows, cols, block, _ptr(body),
                                    _ptr(sign), _ptr(nonfinite), _stream(stream)),
           "duckmoe_fp8_to_fp9")
    return body, sign


# ----------------------------------------------------------------- layer ----

class Layer:
    """One MoE layer's fp9 expert weights resident on the device."""

    def __init__(self, hidden, inter, n_routed, top_k, device="cuda"):
        import torch
        self.hidden, self.inter, self.n_routed, self.top_k = hidden, inter, n_routed, top_k
        E = n_routed + 1
        mat = inter * hidden
        self.gu_body = torch.empty(E * 2 * mat, dtype=torch.uint8, device=device)
        self.gu_sign = torch.empty(E * 2 * mat // 8, dtype=torch.uint8, device=device)
        self.dn_body = torch.empty(E * mat, dtype=torch.uint8, device=device)
        self.dn_sign = torch.empty(E * mat // 8, dtype=torch.uint8, device=device)
        self.struct = LayerStruct(hidden, inter, n_routed, top_k, self.gu_body.data_ptr(),
                                  self.gu_sign.data_ptr(), self.dn_body.data_ptr(),
                                  self.dn_sign.data_ptr())

    @property
    def n_experts(self):
        return self.n_routed + 1

    @property
    def device(self):
        return self.gu_body.device

    def _expert_index(self, e):
        if not 0 <= e <= self.n_routed:
            raise ValueError("expert %d: must be in [0, %d]" % (e, self.n_routed))

    def expert_bytes(self):
        """fp9 bytes one expert streams (3 matrices, body + sign)."""
        return 3 * self.inter * self.hidden * 9 // 8

    def set_expert(self, e, gate, up, down):
        """Quantize float32 matrices (gate/up [I,H], down [H,I]) into expert e."""
        import torch
        H, I = self.hidden, self.inter
        mat = I * H
        self._expert_index(e)
        for a, shp, name in ((gate, (I, H), "gate"), (up, (I, H), "up"), (down, (H, I), "down")):
            if tuple(np.shape(a)) != shp:
                raise ValueError("%s must have shape %s" % (name, shp))
        gb, gs = quantize_fp9(np.concatenate([gate, up], axis=0))
        db, dsn = quantize_fp9(down)
        self.gu_body[e * 2 * mat:(e + 1) * 2 * mat].copy_(torch.from_numpy(gb.reshape(-1)))
        self.gu_sign[e * 2 * mat // 8:(e + 1) * 2 * mat // 8].copy_(torch.from_numpy(gs.reshape(-1)))
        self.dn_body[e * mat:(e + 1) * mat].copy_(torch.from_numpy(db.reshape(-1)))
        self.dn_sign[e * mat // 8:(e + 1) * mat // 8].copy_(torch.from_numpy(dsn.reshape(-1)))

    def set_expert_device(self, e, gate, up, down, nonfinite=None, stream=None):
        """Quantize device float32 matrices (gate/up [I,H], down [H,I]) into
        expert e with the device quantizer (asynchronous on `stream`)."""
        H, I = self.hidden, self.inter
        mat = I * H
        self._expert_index(e)
        for a, shp, name in ((gate, (I, H), "gate"), (up, (I, H), "up"), (down, (H, I), "down")):
            if tuple(a.shape) != shp:
                raise ValueError("%s must have shape %s" % (name, shp))
        for src, rows, body, sign in ((gate, I, self.gu_body[e * 2 * mat:], self.gu_sign[e * 2 * mat // 8:]),
                                      (up, I, self.gu_body[(e * 2 + 1) * mat:],
                                       self.gu_sign[(e * 2 + 1) * mat // 8:]),
                                      (down, H, self.dn_body[e * mat:], self.dn_sign[e * mat // 8:])):
            quantize_fp9_device(src, body=body, sign=sign, nonfinite=nonfinite, stream=stream)

    def set_expert_fp8(self, e, gate, up, down, block=128, nonfinite=None, stream=None):
        """Convert fp8 matrices into expert e on the GPU.  gate, up, down are
        (codes uint8, scale float32) device pairs: gate/up codes [I, H], down
        [H, I], scales on 128 x 128 blocks (see duckmoe_fp8_to_fp9)."""
        H, I = self.hidden, self.inter
        mat = I * H
        self._expert_index(e)
        for (codes, _), shp, name in ((gate, (I, H), "gate"), (up, (I, H), "up"),
                                      (down, (H, I), "down")):
            if tuple(codes.shape) != shp:
                raise ValueError("%s codes must have shape %s" % (name, shp))
        for (codes, sc), body, sign in ((gate, self.gu_body[e * 2 * mat:], self.gu_sign[e * 2 * mat // 8:]),
                                        (up, self.gu_body[(e * 2 + 1) * mat:],
                                         self.gu_sign[(e * 2 + 1) * mat // 8:]),
                                        (down, self.dn_body[e * mat:], self.dn_sign[e * mat // 8:])):
            fp8_to_fp9_device(codes, sc, block, body=body, sign=sign, nonfinite=nonfinite,
                              stream=stream)

    def fill_synthetic_device(self, seed, workload, layer):
        """Draw every expert with synth.weights_device and quantize it on the GPU."""
        import torch
        H, I = self.hidden, self.inter
        flag = torch.zeros(1, dtype=torch.int32, device=self.gu_body.device)
        for e in range(self.n_experts):
            g = synth.weights_device(seed, workload, layer, e, synth.GATE, (I, H), self.gu_body.device)
            u = synth.weights_device(seed, workload, layer, e, synth.UP, (I, H), self.gu_body.device)
            d = synth.weights_device(seed, workload, layer, e, synth.DOWN, (H, I), self.gu_body.device)
            self.set_expert_device(e, g, u, d, nonfinite=flag)
        if int(flag.item()):
            raise DuckMoeError(ENONFINITE, "fill_synthetic_device")
        return self

    def fill_synthetic(self, seed, workload, layer, threads=None):
        """Draw every expert from synth.weights and upload it (threaded)."""
        H, I = self.hidden, self.inter

        def one(e):
            gate = synth.weights(seed, workload, layer, e, synth.GATE, (I, H))
            up = synth.weights(seed, workload, layer, e, synth.UP, (I, H))
            down = synth.weights(seed, workload, layer, e, synth.DOWN, (H, I))
            self.set_expert(e, gate, up, down)

        if threads is None:
            threads = min(16, len(os.sched_getaffinity(0)))
        with ThreadPoolExecutor(max(1, threads)) as ex:
            list(ex.map(one, range(self.n_experts)))
        import torch
        torch.cuda.synchronize()
        return self

    def workspace_bytes(self, T, n_shards=1):
        n = lib().duckmoe_workspace_bytes(ctypes.byref(self.struct), T, n_shards)
        if n == 0:
            raise DuckMoeError(EINVAL, "duckmoe_workspace_bytes")
        return n

    def workspace(self, T, n_shards=1):
        """A device workspace for T tokens (needs no initialisation)."""
        import torch
        return torch.empty(self.workspace_bytes(T, n_shards), dtype=torch.uint8,
                           device=self.gu_body.device)

    def prefill_workspace_bytes(self, T, routed=True):
        n = lib().duckmoe_prefill_workspace_bytes(ctypes.byref(self.struct), T, int(routed))
        if n == 0:
            raise DuckMoeError(EINVAL, "duckmoe_prefill_workspace_bytes")
        return n

    def prefill_workspace(self, T, routed=True):
        """A device workspace for a prefill call of T tokens (no initialisation)."""
        import torch
        return torch.empty(self.prefill_workspace_bytes(T, routed), dtype=torch.uint8,
                           device=self.gu_body.device)


def _layer_args(layer, x, ids, w, out, n_shards):
    """Checks shared by the layer calls; returns (T, out)."""
    import torch
    dev = layer.device
    _need_device(x, torch.float32, "x", device=dev)
    if x.dim() != 2 or x.shape[1] != layer.hidden:
        raise ValueError("x must be [T, %d], is %s" % (layer.hidden, tuple(x.shape)))
    T = x.shape[0]
    _need_tokens(T)
    if ids is not None:
        _need_device(ids, torch.int32, "ids", shape=(T, layer.top_k), device=dev)
        _need_device(w, torch.float32, "w", shape=(T, layer.top_k), device=dev)
    if n_shards < 1:
        raise ValueError("n_shards must be >= 1")
    shape = (T, layer.hidden) if n_shards == 1 else (n_shards, T, layer.hidden)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=dev)
    _need_device(out, torch.float32, "out", numel=n_shards * T * layer.hidden, device=dev)
    return T, out


def _need_ws(ws, nbytes, device):
    import torch
    _need_device(ws, torch.uint8, "ws", numel=nbytes, device=device)


def _layer_call(fname, layer, x, ids, w, out, n_shards, ws, stream):
    if ids is None:
        raise ValueError("ids and w are required")
    T, out = _layer_args(layer, x, ids, w, out, n_shards)
    if ws is None:
        ws = layer.workspace(T, n_shards)
    _need_ws(ws, layer.workspace_bytes(T, n_shards), layer.device)
    rc = getattr(lib(), fname)(ctypes.byref(layer.struct), _ptr(x), _ptr(ids), _ptr(w), T,
                               _ptr(out), n_shards, _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, fname)
    return out


def moe_layer(layer, x, ids, w, out=None, n_shards=1, ws=None, stream=None):
    """out = shared(x) + sum_i w[:, i] * expert_{ids[:, i]}(x); device tensors."""
    return _layer_call("duckmoe_moe_layer", layer, x, ids, w, out, n_shards, ws, stream)


def moe_layer_noalloc(layer, x, ids, w, out, n_shards=1, stream=None):
    """moe_layer on the library's static device workspace (no workspace argument);
    `out` is the caller's ([T, H], or [n_shards, T, H] for shard partials)."""
    if ids is None or out is None:
        raise ValueError("ids, w and out are required")
    T, out = _layer_args(layer, x, ids, w, out, n_shards)
    rc = lib().duckmoe_moe_layer_noalloc(ctypes.byref(layer.struct), _ptr(x), _ptr(ids), _ptr(w),
                                         T, _ptr(out), n_shards, _stream(stream))
    _check(rc, "duckmoe_moe_layer_noalloc")
    return out


def moe_gate_up(layer, x, ids, w, ws, out=None, n_shards=1, stream=None):
    return _layer_call("duckmoe_moe_gate_up", layer, x, ids, w, out, n_shards, ws, stream)


def moe_down(layer, x, ids, w, ws, out=None, n_shards=1, stream=None):
    return _layer_call("duckmoe_moe_down", layer, x, ids, w, out, n_shards, ws, stream)


def expert_ffn(layer, e, x, out=None, n_shards=1, ws=None, stream=None):
    layer._expert_index(e)
    T, out = _layer_args(layer, x, None, None, out, n_shards)
    if ws is None:
        ws = layer.workspace(T, n_shards)
    _need_ws(ws, layer.workspace_bytes(T, n_shards), layer.device)
    rc = lib().duckmoe_expert_ffn(ctypes.byref(layer.struct), e, _ptr(x), T, _ptr(out),
                                  n_shards, _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "duckmoe_expert_ffn")
    return out


def moe_prefill(layer, x, ids, w, out=None, ws=None, stream=None):
    """The routed layer for many tokens (grouped by expert); ids None runs the
    shared (or only) expert alone."""
    import torch
    dev = layer.device
    _need_device(x, torch.float32, "x", device=dev)
    if x.dim() != 2 or x.shape[1] != layer.hidden:
        raise ValueError("x must be [T, %d], is %s" % (layer.hidden, tuple(x.shape)))
    T = x.shape[0]
    _need_tokens(T, 32768)
    if ids is not None:
        _need_device(ids, torch.int32, "ids", shape=(T, layer.top_k), device=dev)
        _need_device(w, torch.float32, "w", shape=(T, layer.top_k), device=dev)
    if out is None:
        out = torch.empty((T, layer.hidden), dtype=torch.float32, device=dev)
    _need_device(out, torch.float32, "out", numel=T * layer.hidden, device=dev)
    if ws is None:
        ws = layer.prefill_workspace(T, ids is not None)
    _need_ws(ws, layer.prefill_workspace_bytes(T, ids is not None), dev)
    rc = lib().duckmoe_moe_prefill(ctypes.byref(layer.struct), _ptr(x), _ptr(ids), _ptr(w), T,
                                   _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
    _check(rc, "duckmoe_moe_prefill")
    return out


def prefill_plan(ids, w, n_routed, stream=None):
    """Device per-expert token lists (test export) -> (offsets, tokens, weights,
    tok_entry, status) as host numpy arrays."""
    import torch
    _need_device(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError("ids must be [T, top_k]")
    T, k = ids.shape
    dev = ids.device
    _need_device(w, torch.float32, "w", shape=(T, k), device=dev)
    offsets = torch.zeros(n_routed + 2, dtype=torch.int32, device=dev)
    tokens = torch.full((T * (k + 1),), -1, dtype=torch.int32, device=dev)
    weights = torch.zeros(T * (k + 1), dtype=torch.float32, device=dev)
    tok_entry = torch.full((T, k + 1), -7, dtype=torch.int32, device=dev)
    st = torch.full((1,), -1, dtype=torch.int32, device=dev)
    _check(lib().duckmoe_prefill_plan(_ptr(ids), _ptr(w), T, k, n_routed, _ptr(offsets),
                                      _ptr(tokens), _ptr(weights), _ptr(tok_entry), _ptr(st),
                                      _stream(stream)), "duckmoe_prefill_plan")
    off = offsets.cpu().numpy()
    n = int(off[-1])
    return (off, tokens[:n].cpu().numpy(), weights[:n].cpu().numpy(),
            tok_entry.cpu().numpy(), int(st.item()))


def rms_normalize(x, eps=0.0, out=None, stream=None):
    """y[t] = x[t] / sqrt(mean(x[t]^2) + eps) on the device (x [T, H] float32)."""
    import torch
    _need_device(x, torch.float32, "x")
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    if out is None:
        out = torch.empty_like(x)
    _need_device(out, torch.float32, "out", numel=T * H, device=x.device)
    _check(lib().duckmoe_rms_normalize(_ptr(x), T, H, float(eps), _ptr(out), _stream(stream)),
           "duckmoe_rms_normalize")
    return out


class Stack:
    """A chain of equally shaped layers run by duckmoe_moe_stack."""

    def __init__(self, layers):
        self.layers = list(layers)
        self.structs = (LayerStruct * len(self.layers))(*[l.struct for l in self.layers])

    def workspace_bytes(self, T):
        n = lib().duckmoe_stack_workspace_bytes(self.structs, len(self.layers), T)
        if n == 0:
            raise DuckMoeError(EINVAL, "duckmoe_stack_workspace_bytes")
        return n

    def workspace(self, T):
        import torch
        return torch.empty(self.workspace_bytes(T), dtype=torch.uint8,
                           device=self.layers[0].gu_body.device)


def moe_stack(stack, x, ids, w, eps=0.0, out=None, ws=None, stream=None):
    """Run every layer of `stack` with the RMS glue in between (see the header).

    x [T, H] float32; ids int32 / w float32 [n_layers, T, top_k]; device tensors.
    """
    import torch
    lay = stack.layers[0]
    dev = lay.device
    _need_device(x, torch.float32, "x", device=dev)
    if x.dim() != 2 or x.shape[1] != lay.hidden:
        raise ValueError("x must be [T, %d], is %s" % (lay.hidden, tuple(x.shape)))
    T = x.shape[0]
    _need_tokens(T)
    n = len(stack.layers)
    _need_device(ids, torch.int32, "ids", shape=(n, T, lay.top_k), device=dev)
    _need_device(w, torch.float32, "w", shape=(n, T, lay.top_k), device=dev)
    if out is None:
        out = torch.empty_like(x)
    _need_device(out, torch.float32, "out", numel=T * lay.hidden, device=dev)
    if ws is None:
        ws = stack.workspace(T)
    _need_ws(ws, stack.workspace_bytes(T), dev)
    _check(lib().duckmoe_moe_stack(stack.structs, len(stack.layers), _ptr(x), _ptr(ids), _ptr(w),
                                   T, float(eps), _ptr(out), _ptr(ws), ws.numel(),
                                   _stream(stream)), "duckmoe_moe_stack")
    return out


def read_probe(buf, nbytes, sink, stream=None):
    """Plain streaming read of the first nbytes of device tensor buf (calibration)."""
    import torch
    _need_device(buf, buf.dtype if buf is not None else None, "buf")
    if nbytes > buf.numel() * buf.element_size():
        raise ValueError("nbytes %d exceeds buf's %d bytes" % (nbytes, buf.numel() * buf.element_size()))
    _need_device(sink, torch.int32, "sink", numel=1, device=buf.device)
    _check(lib().duckmoe_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)),
           "duckmoe_read_probe")


class Lane:
    """An asynchronous lane: its own stream (default priority), workspace and
    events (see duckmoe_lane_* in the header).

    cus (> 0) gives the lane a CU budget: its persistent grids are sized to
    that many CUs, so two lanes with half the device each fill it once
    between them and run side by side (by default each lane's grids fill the
    whole device, and two lanes at once wait for each other's workgroups).

    The tensors handed to begin are recorded on the lane's stream
    (Tensor.record_stream), so torch's caching allocator does not give their
    memory to new tensors before the lane's kernels have read and written
    them, even if the caller drops them right after begin.  close() waits for
    the lane's last layer before it releases the workspace and the events.
    """

    def __init__(self, layer, max_tokens=1, cus=0):
        import torch
        self.max_tokens = max_tokens
        self.stream = torch.cuda.Stream(device=layer.gu_body.device)
        self.ws = layer.workspace(max_tokens)
        self.ws.record_stream(self.stream)
        self.struct = LaneStruct(self.stream.cuda_stream, self.ws.data_ptr(), self.ws.numel(),
                                 None, None, int(cus))
        _check(lib().duckmoe_lane_init(ctypes.byref(self.struct)), "duckmoe_lane_init")

    @property
    def cus(self):
        """CUs the lane's kernels may use (0: the whole device)."""
        return self.struct.cus

    def begin(self, layer, x, ids, w, out, producer=None):
        """Start the layer for this lane once `producer` (default: the current
        stream) has produced x, ids and w; returns at once."""
        if ids is None or out is None:
            raise ValueError("ids, w and out are required")
        T, out = _layer_args(layer, x, ids, w, out, 1)
        _need_tokens(T, self.max_tokens)
        if self.ws is None:
            raise ValueError("the lane is closed")
        _check(lib().duckmoe_lane_begin(ctypes.byref(self.struct), ctypes.byref(layer.struct),
                                        _ptr(x), _ptr(ids), _ptr(w), T, _ptr(out),
                                        _stream(producer)), "duckmoe_lane_begin")
        for t in (x, ids, w, out):
            t.record_stream(self.stream)

    def finish(self, consumer=None, block=False):
        """Make `consumer` (default: the current stream) wait for the lane's
        layer, or block the host if block=True."""
        c = ctypes.c_void_p(0) if block else _stream(consumer)
        _check(lib().duckmoe_lane_finish(ctypes.byref(self.struct), c), "duckmoe_lane_finish")

    def close(self):
        if self.struct.done or self.struct.ready:
            # the lane's kernels may still use the workspace: wait for them first
            self.stream.synchronize()
            _check(lib().duckmoe_lane_destroy(ctypes.byref(self.struct)), "duckmoe_lane_destroy")
        self.ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # pragma: no cover - interpreter shutdown
            pass


def status(ws, stream=None):
    import torch
    _need_device(ws, torch.uint8, "ws", numel=8)
    st = _I32(0)
    _check(lib().duckmoe_status(_ptr(ws), ctypes.byref(st), _stream(stream)), "duckmoe_status")
    return st.value


# --------------------------------------------------------- building blocks ----

def decode_fp9(body, sign, n=None, out=None, stream=None):
    """Device decode of fp9 planes to float32 (test export)."""
    import torch
    _need_device(body, torch.uint8, "body")
    n = body.numel() if n is None else n
    if not 0 <= n <= body.numel():
        raise ValueError("n = %d: body holds %d codes" % (n, body.numel()))
    _need_device(sign, torch.uint8, "sign", numel=(n + 7) // 8, device=body.device)
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=body.device)
    _need_device(out, torch.float32, "out", numel=n, device=body.device)
    _check(lib().duckmoe_decode_fp9(_ptr(body), _ptr(sign), n, _ptr(out), _stream(stream)),
           "duckmoe_decode_fp9")
    return out


def gemv_fp9(body, sign, x, out=None, stream=None):
    """y = W x with W in fp9 planes body [rows, cols], sign [rows, cols/8]."""
    import torch
    _need_device(body, torch.uint8, "body")
    if body.dim() != 2:
        raise ValueError("body must be 2-D [rows, cols]")
    rows, cols = body.shape
    _need_device(sign, torch.uint8, "sign", numel=rows * (cols // 8), device=body.device)
    _need_device(x, torch.float32, "x", numel=cols, device=body.device)
    if out is None:
        out = torch.empty(rows, dtype=torch.float32, device=body.device)
    _need_device(out, torch.float32, "out", numel=rows, device=body.device)
    _check(lib().duckmoe_gemv_fp9(_ptr(body), _ptr(sign), rows, cols, _ptr(x), _ptr(out),
                                  _stream(stream)), "duckmoe_gemv_fp9")
    return out


def moe_plan(ids, n_routed, stream=None):
    """Device expert-selection plan -> expert indices in slot order (shared
    first, then the distinct valid ids by first appearance)."""
    import torch
    _need_device(ids, torch.int32, "ids")
    if ids.dim() != 2:
        raise ValueError("ids must be [T, top_k]")
    T, k = ids.shape
    uniq = torch.full((T * k + 1,), -1, dtype=torch.int32, device=ids.device)
    n = torch.zeros(1, dtype=torch.int32, device=ids.device)
    _check(lib().duckmoe_moe_plan(_ptr(ids), T, k, n_routed, _ptr(uniq), _ptr(n),
                                  _stream(stream)), "duckmoe_moe_plan")
    cnt = int(n.item())
    return uniq[:cnt].cpu().tolist()
