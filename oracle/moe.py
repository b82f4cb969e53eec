"""Routed-expert MoE FFN, oracle side (float64 numpy).  TEST INFRASTRUCTURE ONLY.

What the path computes, with the readings taken where the pages are silent:

* fp9 GEMV (memoir page, fp9 section "在只有 AVX2 的 N100 上，我先做出了单核
  MLP fp9"): y = W x with the fp9 weights decoded exactly and the products
  summed; the first fp9 workload on the pages is a dense MLP forward.
* expert FFN: the pages put the FFN/MoE expert layers on the boxes (memoir,
  section "真正埋下伏笔的是内存；R1 之后，问题第一次被改写") but never name
  the activation.  Reading: the DeepSeek-V3 SwiGLU expert,
  y = W_down (silu(W_gate x) * (W_up x)), silu(z) = z / (1 + exp(-z)).
* routed layer (chapter 9 page, section 9.2 "两条路线的判断"): each token picks
  top_k = 8 routed experts (the page's "8 tokens (top_k=8)" is read as 8 experts
  per token); one shared expert always runs with weight 1:
  out_t = shared(x_t) + sum_i w[t, i] * expert_{ids[t, i]}(x_t).
  Tokens are independent.
* shard partials (memoir, section "真正难的不是把参数塞下，而是通信": tensor
  parallel split; section "先用 Qwen3 练级，再让 Qwen3.5 充当高压试炼场":
  sub-128 slices; section "16 tok/s 之后：一段没有跑通的路": per-box work then
  a host reduce; ds4 glossary page "张量并行（Tensor Parallelism, TP）", section
  "形态一：Mac-to-Mac 张量并行（RDMA）": partial sums stay f32).  Reading: the
  intermediate dimension is cut into n_shards equal slices; shard r keeps
  gate/up rows and down columns of its slice for every expert (the shared one
  too), so the shard partials add up to the full output.
* expert selection plan: ascending distinct routed ids of the batch, then the
  shared expert (index n_routed) last; per (slot, token) the routing weight,
  summed if a token lists an id twice, 0 if the token does not use the slot.

All arithmetic is float64; weights are decoded with the closed form.
"""

import numpy as np

from .fp9 import decode

_TABLE = None


def _decode_fast(codes):
    """Closed-form decode, applied through a 512-entry table for big arrays."""
    global _TABLE
    if _TABLE is None:
        _TABLE = decode(np.arange(512))
    return _TABLE[np.asarray(codes).astype(np.int64)]


def gemv(codes, x):
    """y[n] = sum_k decode(codes[n, k]) * x[k], in float64."""
    W = _decode_fast(codes)
    xv = np.asarray(x, dtype=np.float64)
    if W.ndim != 2 or xv.shape != (W.shape[1],):
        raise ValueError("gemv: shape mismatch")
    return W @ xv


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


class _Decoded:
    """An expert's three matrices decoded to float64 (gate [I,H], up [I,H], down [H,I])."""

    def __init__(self, expert):
        gate, up, down = expert
        self.gate = _decode_fast(gate)
        self.up = _decode_fast(up)
        self.down = _decode_fast(down)
        I, H = self.gate.shape
        if self.up.shape != (I, H) or self.down.shape != (H, I):
            raise ValueError("expert matrices have inconsistent shapes")


def _ffn_one(dec, xt, lo=0, hi=None):
    """One token through one expert, intermediate indices restricted to [lo, hi)."""
    if hi is None:
        hi = dec.gate.shape[0]
    g = dec.gate[lo:hi] @ xt
    v = dec.up[lo:hi] @ xt
    h = silu(g) * v
    return dec.down[:, lo:hi] @ h


def expert_ffn(expert, x):
    """expert = (gate codes [I,H], up codes [I,H], down codes [H,I]); x [T,H] -> [T,H]."""
    dec = _Decoded(expert)
    X = np.atleast_2d(np.asarray(x, dtype=np.float64))
    return np.stack([_ffn_one(dec, X[t]) for t in range(X.shape[0])])


def moe_plan(ids, n_routed):
    """Expert-selection plan for a batch of routed ids [T, top_k].

    Returns (slots, slot_weights_fn) where slots is the list of expert indices
    (ascending distinct routed ids, then n_routed for the shared expert).
    """
    ids = np.asarray(ids, dtype=np.int64)
    if np.any((ids < 0) | (ids >= n_routed)):
        raise ValueError("routed expert id out of range")
    uniq = sorted(set(int(i) for i in ids.ravel()))
    return uniq + [int(n_routed)]


def moe_slot_weights(ids, w, n_routed):
    """[n_slots, T] routing weight of each plan slot for each token (shared = 1)."""
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(w, dtype=np.float64)
    slots = moe_plan(ids, n_routed)
    T = ids.shape[0]
    out = np.zeros((len(slots), T), dtype=np.float64)
    for s, e in enumerate(slots[:-1]):
        for t in range(T):
            for i in range(ids.shape[1]):
                if ids[t, i] == e:
                    out[s, t] += w[t, i]
    out[-1, :] = 1.0
    return out


def _check_batch(x, ids, w):
    X = np.atleast_2d(np.asarray(x, dtype=np.float64))
    ids = np.atleast_2d(np.asarray(ids, dtype=np.int64))
    w = np.atleast_2d(np.asarray(w, dtype=np.float64))
    if ids.shape != w.shape or ids.shape[0] != X.shape[0]:
        raise ValueError("x, ids and w disagree on the batch size")
    return X, ids, w


def moe_layer(get_expert, x, ids, w, n_routed):
    """out_t = shared(x_t) + sum_i w[t,i] * expert_{ids[t,i]}(x_t), float64.

    get_expert(e) returns the (gate, up, down) code matrices of expert e; the
    shared expert is index n_routed.
    """
    X, ids, w = _check_batch(x, ids, w)
    moe_plan(ids, n_routed)  # range check
    cache = {}

    def dec(e):
        if e not in cache:
            cache[e] = _Decoded(get_expert(e))
        return cache[e]

    out = []
    for t in range(X.shape[0]):
        acc = _ffn_one(dec(n_routed), X[t])
        for i in range(ids.shape[1]):
            acc = acc + w[t, i] * _ffn_one(dec(int(ids[t, i])), X[t])
        out.append(acc)
    return np.stack(out)


def moe_partials(get_expert, x, ids, w, n_routed, n_shards):
    """[n_shards, T, H]: shard r's share of moe_layer (intermediate slice r)."""
    X, ids, w = _check_batch(x, ids, w)
    moe_plan(ids, n_routed)
    cache = {}

    def dec(e):
        if e not in cache:
            cache[e] = _Decoded(get_expert(e))
        return cache[e]

    inter = dec(n_routed).gate.shape[0]
    if n_shards < 1 or inter % n_shards != 0:
        raise ValueError("n_shards must divide the intermediate size")
    width = inter // n_shards
    res = []
    for r in range(n_shards):
        lo, hi = r * width, (r + 1) * width
        per_t = []
        for t in range(X.shape[0]):
            acc = _ffn_one(dec(n_routed), X[t], lo, hi)
            for i in range(ids.shape[1]):
                acc = acc + w[t, i] * _ffn_one(dec(int(ids[t, i])), X[t], lo, hi)
            per_t.append(acc)
        res.append(np.stack(per_t))
    return np.stack(res)


def rms_normalize(v, eps=0.0):
    """Glue between stacked layers: v / sqrt(mean(v^2) + eps) per token, float64.

    Not on the pages' MoE path (their GPU stage normalises between layers:
    chapter page "第 9 章 MTP1 dual-lane overlap", section 9.5); used only to
    chain layers without overflow.  eps = 0 is the plain reading; a positive
    eps is the usual RMSNorm guard against an all-zero row.
    """
    V = np.atleast_2d(np.asarray(v, dtype=np.float64))
    return V / np.sqrt(np.mean(V * V, axis=1, keepdims=True) + float(eps))


def prefill_plan(ids, w, n_routed):
    """Per-expert token lists of a prefill batch (the grouping of a grouped GEMM).

    The pages leave the larger-T expert path open (memoir page, section
    "限制条件": the fp9 prefill kernel is far from the machine's peak, and
    contexts were tested up to 2048 tokens); the lists are the plain grouping
    of the batch's (token, expert) pairs by expert.  Reading taken:

    * list positions p = 0 .. n_routed: p = 0 is the shared expert (index
      n_routed), p >= 1 is routed expert p - 1;
    * list p holds, in ascending token order, every token that uses its expert:
      all tokens for the shared expert, tokens with at least one ids[t, i] == e
      for a routed one; each token at most once per list;
    * the entry's weight is 1 for the shared expert, else the sum of w[t, i]
      over the positions i where the token lists e (summed in list order);
    * entries are numbered list by list: offsets[p] is the first entry of list
      p, offsets[n_routed + 1] the total;
    * tok_entry[t, 0] is token t's shared entry; tok_entry[t, 1 + i] is the
      entry of (ids[t, i], t) when i is the first position of that id in the
      token's list, and -1 for a repeat.

    Returns (offsets [n_routed + 2], tokens [A], weights [A] float64,
    tok_entry [T, top_k + 1]).  Out-of-range ids are rejected.
    """
    ids = np.atleast_2d(np.asarray(ids, dtype=np.int64))
    w = np.atleast_2d(np.asarray(w, dtype=np.float64))
    if ids.shape != w.shape:
        raise ValueError("ids and w disagree")
    if np.any((ids < 0) | (ids >= n_routed)):
        raise ValueError("routed expert id out of range")
    T, K = ids.shape
    lists = [[(t, 1.0) for t in range(T)]]
    for e in range(n_routed):
        lst = []
        for t in range(T):
            hit = [i for i in range(K) if ids[t, i] == e]
            if hit:
                s = 0.0
                for i in hit:
                    s += w[t, i]
                lst.append((t, s))
        lists.append(lst)
    offsets = np.zeros(n_routed + 2, dtype=np.int64)
    for p, lst in enumerate(lists):
        offsets[p + 1] = offsets[p] + len(lst)
    tokens = np.array([t for lst in lists for t, _ in lst], dtype=np.int64)
    weights = np.array([s for lst in lists for _, s in lst], dtype=np.float64)
    tok_entry = np.full((T, K + 1), -1, dtype=np.int64)
    for p, lst in enumerate(lists):
        for r, (t, _) in enumerate(lst):
            if p == 0:
                tok_entry[t, 0] = offsets[0] + r
            else:
                first = min(i for i in range(K) if ids[t, i] == p - 1)
                tok_entry[t, 1 + first] = offsets[p] + r
    return offsets, tokens, weights, tok_entry
