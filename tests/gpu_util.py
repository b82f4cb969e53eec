"""Shared pieces of the GPU parity tests: tolerance check, oracle expert cache."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from bit_moe_expert_fp9_amd import synth

# f32 output bar: relative L2 error <= 1e-5 and max-abs error <= 1e-4 * max|ref|
REL_L2 = 1e-5
MAX_ABS_FRAC = 1e-4


def check_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = got - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(err) / nref if nref > 0 else np.linalg.norm(err)
    mref = np.abs(ref).max()
    mx = np.abs(err).max() / mref if mref > 0 else np.abs(err).max()
    assert rel <= REL_L2 and mx <= MAX_ABS_FRAC, \
        "%s: rel_l2=%.3e max_abs/max|ref|=%.3e" % (what, rel, mx)
    return rel, mx


class OracleExperts:
    """Oracle-side expert codes: the synthetic float32 weights quantized by the
    oracle's own quantizer (never by the library), cached per expert."""

    def __init__(self, seed, workload, layer, hidden, inter, device_drawn=False):
        """device_drawn: the layer's weights come from synth.weights_device (the
        float32 draws are copied to the host; only the drawing is on the GPU)."""
        self.key = (seed, workload, layer)
        self.H, self.I = hidden, inter
        self.device_drawn = device_drawn
        self.cache = {}

    def _draw(self, e, m, shape):
        s, wl, l = self.key
        if self.device_drawn:
            return synth.weights_device(s, wl, l, e, m, shape).cpu().numpy()
        return synth.weights(s, wl, l, e, m, shape)

    def _make(self, e):
        gate = self._draw(e, synth.GATE, (self.I, self.H))
        up = self._draw(e, synth.UP, (self.I, self.H))
        down = self._draw(e, synth.DOWN, (self.H, self.I))
        return (oracle.quantize(gate), oracle.quantize(up), oracle.quantize(down))

    def prefetch(self, experts):
        todo = [int(e) for e in set(int(e) for e in experts) if int(e) not in self.cache]
        if not todo:
            return
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(todo)))
        with ThreadPoolExecutor(workers) as ex:
            for e, codes in zip(todo, ex.map(self._make, todo)):
                self.cache[e] = codes

    def __call__(self, e):
        e = int(e)
        if e not in self.cache:
            self.cache[e] = self._make(e)
        return self.cache[e]


def say(*a):
    """Progress line that names the case before a GPU step (flushed)."""
    print("[gpu-test]", *a, flush=True)
