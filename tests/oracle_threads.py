"""The float64 oracle over many tokens, with its banks spread over threads (test infrastructure).

At full layer size the oracle spends its time decoding every expert bank that a
batch touches: about 0.2 s per bank on one core, and a Flash-Next-shaped layer
has 513 banks.  The block output is a sum of one term per bank plus the rank-r
correction.  So each thread runs oracle.moe.forward restricted to its share of
the banks (banks_subset), and the partial outputs are added up with the
correction.  numpy releases the interpreter lock inside its array loops and BLAS
calls, so the threads decode in parallel.  Every term is computed by the oracle
itself; only the order of the float64 additions differs from one serial call
(about 1e-16 relative).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import moe as omoe

try:
    from threadpoolctl import threadpool_limits
except ImportError:  # pragma: no cover - BLAS threads then stay as they are
    threadpool_limits = None


def n_workers() -> int:
    """Threads to use: the CPUs this process may run on, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _assign(costs, n):
    """Longest-processing-time-first split of banks (by cost) into n lists."""
    loads = [0.0] * n
    parts = [[] for _ in range(n)]
    for e in np.argsort(-np.asarray(costs), kind="stable"):
        j = int(np.argmin(loads))
        parts[j].append(int(e))
        loads[j] += costs[e]
    return [p for p in parts if p]


def forward_y(L, x_bits, router_bits, delta_bits, a_bits, b_bits, top_k, forced_idx, delta_factors=None,
              threads=None):
    """y (float64 [T, d]) of oracle.moe.forward(x_bits, router_bits, delta_bits, <L's banks>, a_bits,
    b_bits, top_k, forced_idx=forced_idx, delta_factors=delta_factors), computed bank by bank on
    threads.  L is a tests.layer_fixtures.Layer (its bank source, formats and shape)."""
    c = L.cfg
    E, S = c.n_experts, c.n_shared
    idx = np.asarray(forced_idx, dtype=np.int64)
    T = idx.shape[0]
    tok = np.bincount(idx.reshape(-1), minlength=E).astype(np.float64)
    tok = np.concatenate([tok, np.full(S, float(T))])
    # cost per bank, in seconds on one core: its decode plus its tokens' products
    costs = np.where(tok > 0, 0.2 + tok * 6.0 * c.d_model * c.d_ff / 3e10, 0.0)
    n = threads or n_workers()
    parts = _assign(costs, n) if costs.sum() > 0 else []

    def run(subset):
        banks = omoe.LazyBanks(L.source, L.formats, c.d_model, c.d_ff, E, S, cache=2)
        return omoe.forward(x_bits, router_bits, delta_bits, banks, None, None, top_k, forced_idx=idx,
                            delta_factors=delta_factors, banks_subset=subset).y

    x = omoe.bf16_to_f64(x_bits)
    a = None if a_bits is None else omoe.f16_to_f64(a_bits)
    b = None if b_bits is None else omoe.f16_to_f64(b_bits)
    y = omoe.correction(x, a, b)
    if not parts:
        return y

    def all_parts():
        if len(parts) == 1:
            return [run(parts[0])]
        with ThreadPoolExecutor(len(parts)) as ex:
            return list(ex.map(run, parts))

    if threadpool_limits is not None:
        with threadpool_limits(1):
            ys = all_parts()
    else:
        ys = all_parts()
    for p in ys:
        y += p
    return y
