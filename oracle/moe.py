"""Oracle forward pass of one ternary-expert MoE block, float64 (test infrastructure only).

The block, as the release pages describe it:
  1. router logits plus the router delta            l = (W_r + dW_r) x
     (Scion README "The idea": corrections include router deltas; 35B-A3B card
     "Weight Representation": exact router deltas)
  2. top-k selection, with an always-on shared expert when the layer has one
     (FlashNext card "Model Overview": top-10 routed + 1 shared; 35B-A3B card
     "Model Overview": top-8)
  3. grouping of (token, slot) pairs per expert, the mul_mat_id view
     (Scion README "Serving notes")
  4. each selected expert's SwiGLU FFN over ternary weights scale * t
  5. the gate-weighted combine
  6. the rank-r correction on the MoE block output, on the residual stream:
     y += B (A x)  (Scion README "The idea" and "What the experiments
     established": corrections live on the residual stream; 35B-A3B card
     "Weight Representation": rank-512 branches on the MoE block output)

Readings where the pages are silent: gating is the softmax over the k selected
logits; ties order experts by lower index; the activation is SwiGLU,
silu(gate) * up with gate rows [0, f) and up rows [f, 2f) stored as two
matrices; the correction reads the block input x; the shared expert has weight 1.

Everything is float64.  fp16 x bf16 products are exact in float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from . import codec


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 is the upper half of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


f16_to_f64 = codec.f16_to_f64


@dataclass
class Banks:
    """One layer's expert containers, laid out as the library receives them:
    bank e occupies data[offsets[e]:] as [gate f x d | up f x d | down d x f]
    containers of format formats[e]; banks 0..E-1 are routed, E..E+S-1 shared."""
    data: np.ndarray      # uint8
    offsets: np.ndarray   # int64 [E+S]
    formats: np.ndarray   # uint8 [E+S]
    d_model: int
    d_ff: int
    n_experts: int
    n_shared: int

    def matrices(self, e: int):
        """(W_gate [f,d], W_up [f,d], W_down [d,f]) of bank e as float64 scale * t."""
        fmt = int(self.formats[e])
        d, f = self.d_model, self.d_ff
        pos = int(self.offsets[e])
        out = []
        for rows, cols in ((f, d), (f, d), (d, f)):
            nbytes = codec.packed_bytes(fmt, rows * cols)
            out.append(codec.decode(fmt, self.data[pos:pos + nbytes], rows * cols).reshape(rows, cols))
            pos += nbytes
        return tuple(out)


class LazyBanks(Banks):
    """Banks whose containers are packed with the oracle codec on first use.
    source(e) returns ([gate, up, down] trits, [gate, up, down] scale bits)."""

    def __init__(self, source, formats, d_model, d_ff, n_experts, n_shared, cache=16):
        self.source = source
        self.formats = np.asarray(formats, dtype=np.uint8)
        self.d_model, self.d_ff = d_model, d_ff
        self.n_experts, self.n_shared = n_experts, n_shared
        self._cache = {}
        self._cache_size = cache

    def container(self, e: int) -> np.ndarray:
        """Bank e's [gate | up | down] container bytes, packed by the oracle codec."""
        trits, scales = self.source(e)
        return np.concatenate([codec.pack(int(self.formats[e]), t, s) for t, s in zip(trits, scales)])

    def matrices(self, e: int):
        if e not in self._cache:
            if len(self._cache) >= self._cache_size:
                self._cache.pop(next(iter(self._cache)))
            fmt = int(self.formats[e])
            data = self.container(e)
            d, f = self.d_model, self.d_ff
            out, pos = [], 0
            for rows, cols in ((f, d), (f, d), (d, f)):
                nbytes = codec.packed_bytes(fmt, rows * cols)
                out.append(codec.decode(fmt, data[pos:pos + nbytes], rows * cols).reshape(rows, cols))
                pos += nbytes
            self._cache[e] = tuple(out)
        return self._cache[e]


def pack_banks(trits_scales, formats, d_model, d_ff, n_experts, n_shared) -> Banks:
    """Build a Banks from per-bank ([gate, up, down] trits, [gate, up, down] scale bits)."""
    chunks, offsets, pos = [], [], 0
    for e, (trits, scales) in enumerate(trits_scales):
        offsets.append(pos)
        for t, s in zip(trits, scales):
            c = codec.pack(int(formats[e]), t, s)
            chunks.append(c)
            pos += c.size
    return Banks(np.concatenate(chunks), np.array(offsets, dtype=np.int64),
                 np.asarray(formats, dtype=np.uint8), d_model, d_ff, n_experts, n_shared)


# --------------------------------------------------------------------------- routing
def router_logits(x: np.ndarray, w_r: np.ndarray, dw_r: Optional[np.ndarray]) -> np.ndarray:
    """l[t, e] = sum_j (W_r[e, j] + dW_r[e, j]) x[t, j]."""
    w = w_r if dw_r is None else w_r + dw_r
    return x @ w.T


def factored_delta(u_bits, v_bits) -> np.ndarray:
    """The router delta given as two low-rank fp16 factors, dW_r = U V with U
    [E, rd] and V [rd, d] (FlashNext card, "Weight Representation": the router
    deltas ship as rank-512 F16 factors), formed exactly in float64."""
    return f16_to_f64(u_bits) @ f16_to_f64(v_bits)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Per token, the k experts with the largest logits, in rank order; equal
    logits order by lower expert index (so -0.0 and +0.0 tie)."""
    T, E = logits.shape
    if not np.all(np.isfinite(logits)):
        raise ValueError("non-finite router logit")
    idx = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))
        idx[t] = order[:k]
    return idx


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """w_i = exp(l_{s_i} - l_{s_1}) / sum_j exp(l_{s_j} - l_{s_1}): softmax over the k selected."""
    sel = np.take_along_axis(logits, idx, axis=1)
    ex = np.exp(sel - sel[:, :1])
    return ex / ex.sum(axis=1, keepdims=True)


def grouping(idx: np.ndarray, n_experts: int):
    """counts[e], offsets (exclusive scan, offsets[E] = T*k) and perm: the flat
    slot ids t*k + i ordered by (expert, token)."""
    T, k = idx.shape
    counts = np.zeros(n_experts, dtype=np.int64)
    for e in idx.reshape(-1):
        counts[e] += 1
    offsets = np.zeros(n_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    fill = offsets[:-1].copy()
    perm = np.empty(T * k, dtype=np.int64)
    for t in range(T):                  # tokens in increasing order ...
        for i in range(k):
            e = idx[t, i]
            perm[fill[e]] = t * k + i   # ... land in increasing order within each expert
            fill[e] += 1
    return counts, offsets, perm


# --------------------------------------------------------------------------- experts
def silu(g: np.ndarray) -> np.ndarray:
    return g / (1.0 + np.exp(-g))


def expert_ffn(w_gate, w_up, w_down, xs: np.ndarray) -> np.ndarray:
    """SwiGLU FFN rows: o = W_down (silu(W_gate x) * (W_up x)) for each row x of xs."""
    g = xs @ w_gate.T
    u = xs @ w_up.T
    return (silu(g) * u) @ w_down.T


def correction(x: np.ndarray, a: Optional[np.ndarray], b: Optional[np.ndarray]) -> np.ndarray:
    """B (A x) per token: the rank-r branch on the MoE block output."""
    if a is None or b is None:
        return np.zeros_like(x)
    return (x @ a.T) @ b.T


def lowrank_apply(x_bits, y_bits, a_bits, b_bits) -> np.ndarray:
    """y + B (A x) per token, the same rank-r branch applied to another tensor:
    the releases carry rank-512 branches on the attention output as well as on
    the MoE block output (Scion-35B-A3B card, "Weight Representation").  x and
    y are bf16 bits [T, d] (y None for zero), A [r, d] and B [d, r] fp16 bits."""
    x = bf16_to_f64(x_bits)
    y = np.zeros_like(x) if y_bits is None else bf16_to_f64(y_bits)
    return y + correction(x, f16_to_f64(a_bits), f16_to_f64(b_bits))


@dataclass
class Result:
    y: np.ndarray         # [T, d] float64
    logits: np.ndarray    # [T, E]
    idx: np.ndarray       # [T, k] rank order
    w: np.ndarray         # [T, k]
    counts: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray


def forward(x_bits, router_bits, delta_bits, banks: Banks, a_bits, b_bits, top_k: int,
            forced_idx: Optional[np.ndarray] = None, delta_factors=None, banks_subset=None) -> Result:
    """The block's forward pass over tokens x (bf16 bits [T, d]).  forced_idx, if
    given, replaces the oracle's own top-k choice (gate weights are still the
    softmax of the oracle's logits at those indices).  delta_factors, if given,
    is (U, V) in fp16 bits, the router delta U V in place of delta_bits.

    banks_subset, if given, is a collection of bank numbers (routed 0..E-1,
    shared E..E+S-1): y then holds only those banks' terms and no correction.
    y is a sum of per-bank terms plus the correction, so the results over
    disjoint subsets that cover every bank, plus correction(x, A, B), add up to
    the whole block (up to the order of the float64 additions)."""
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    E = banks.n_experts
    w_r = f16_to_f64(router_bits)
    if delta_factors is not None:
        if delta_bits is not None:
            raise ValueError("give the router delta dense or as factors, not both")
        dw_r = factored_delta(*delta_factors)
    else:
        dw_r = None if delta_bits is None else f16_to_f64(delta_bits)
    a = None if a_bits is None else f16_to_f64(a_bits)
    b = None if b_bits is None else f16_to_f64(b_bits)

    logits = router_logits(x, w_r, dw_r)
    idx = select_topk(logits, top_k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    w = gate_weights(logits, idx)
    counts, offsets, perm = grouping(idx, E)

    wanted = (lambda e: True) if banks_subset is None else set(int(e) for e in banks_subset).__contains__
    y = np.zeros_like(x)
    for e in range(E):                        # routed experts, one at a time
        if counts[e] == 0 or not wanted(e):
            continue
        slots = perm[offsets[e]:offsets[e + 1]]
        toks, which = slots // top_k, slots % top_k
        o = expert_ffn(*banks.matrices(e), x[toks])
        y[toks] += w[toks, which][:, None] * o
    for s in range(banks.n_shared):           # always-on shared experts, weight 1
        if wanted(E + s):
            y += expert_ffn(*banks.matrices(E + s), x)
    if banks_subset is None:
        y += correction(x, a, b)
    return Result(y, logits, idx, w, counts, offsets, perm)


def forward_bruteforce(x_bits, router_bits, delta_bits, banks: Banks, a_bits, b_bits,
                       top_k: int) -> np.ndarray:
    """No grouping at all: every expert on every token, then the top-k mask."""
    x = bf16_to_f64(x_bits)
    T = x.shape[0]
    E = banks.n_experts
    w_r = f16_to_f64(router_bits)
    dw_r = None if delta_bits is None else f16_to_f64(delta_bits)
    logits = router_logits(x, w_r, dw_r)
    idx = select_topk(logits, top_k)
    w = gate_weights(logits, idx)
    mask = np.zeros((T, E))
    for t in range(T):
        for i in range(top_k):
            mask[t, idx[t, i]] = w[t, i]
    y = np.zeros_like(x)
    for e in range(E + banks.n_shared):
        o = expert_ffn(*banks.matrices(e), x)
        y += (mask[:, e:e + 1] if e < E else 1.0) * o
    a = None if a_bits is None else f16_to_f64(a_bits)
    b = None if b_bits is None else f16_to_f64(b_bits)
    return y + correction(x, a, b)
