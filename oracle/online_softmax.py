"""Online-softmax recurrence in fp64: TEST INFRASTRUCTURE ONLY.

This is the method the GPU kernel runs, written out in the order the pages give
it and in their notation, for one query row at a time.  It exists so the tests
can show that the recurrence reaches the plain definition computed by the
oracle (the induction argument of the page "FlashAttention and kernels",
gtadkapally.com, section "Online softmax: keep a running max and a running sum"), and so the
printed worked examples can pin each intermediate state.

State per query row: running maximum ``m`` (starts at -inf), running
denominator ``l`` (starts at 0) and unnormalised output ``o`` (starts at 0).
For each block of scores (same page, "From a sum to an output row"; "4 Triton and
Custom Kernels", section 4.8, the four-step update):

1. ``m_new = max(m, max(block))`` and ``alpha = exp(m - m_new)``; on the first
   block ``exp(-inf) = 0``.
2. ``w_j = exp(s_j - m_new)`` for each key of the block.
3. ``l = alpha * l + sum_j w_j`` and ``o = alpha * o + sum_j w_j * v_j``.
4. ``m = m_new``.

After the last block the output is ``o / l`` and the log-sum-exp is
``m + ln(l)``.  Pure Python/NumPy, sized for small inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


@dataclass
class RowState:
    m: float = -math.inf
    l: float = 0.0
    o: np.ndarray | None = None
    trace: list = field(default_factory=list)


def _exp(x: float) -> float:
    return 0.0 if x == -math.inf else math.exp(x)


def update(state: RowState, scores, values) -> RowState:
    """Fold one block of (scaled) scores and their value rows into ``state``."""
    scores = [float(s) for s in scores]
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    if state.o is None:
        state.o = np.zeros(values.shape[1], dtype=np.float64)
    if not scores:
        return state
    m_new = max(state.m, max(scores))
    alpha = _exp(state.m - m_new)
    w = [_exp(s - m_new) for s in scores]
    state.l = alpha * state.l + math.fsum(w)
    contrib = np.zeros_like(state.o)
    for wj, vj in zip(w, values):
        contrib += wj * vj
    state.o = alpha * state.o + contrib
    state.m = m_new
    state.trace.append(dict(m=state.m, alpha=alpha, l=state.l, o=state.o.copy(), w=list(w)))
    return state


def merge(a: RowState, b: RowState) -> RowState:
    """Combine the states of two disjoint key sets of one row: m = max(m_a, m_b),
    l = l_a e^(m_a - m) + l_b e^(m_b - m), o = o_a e^(m_a - m) + o_b e^(m_b - m).
    The merge of two partial (m, l) states asked for in "FlashAttention and
    kernels" (the online max/sum exercise), and the step Flash-Decoding applies
    to the states of its key splits (same page, "FlashAttention-2, -3, and what
    came after"); an empty state (m = -inf, l = 0) is its identity."""
    m = max(a.m, b.m)
    out = RowState(m=m)
    if m == -math.inf:
        out.l, out.o = 0.0, (a.o if a.o is not None else b.o)
        return out
    ea, eb = _exp(a.m - m), _exp(b.m - m)
    out.l = a.l * ea + b.l * eb
    oa = a.o if a.o is not None else 0.0
    ob = b.o if b.o is not None else 0.0
    out.o = oa * ea + ob * eb
    return out


def online_max_sum(xs) -> tuple[float, float]:
    """One element at a time: ``m_new = max(m, x)``, ``l = l e^(m - m_new) + e^(x - m_new)``."""
    m, l = -math.inf, 0.0
    for x in xs:
        m_new = max(m, float(x))
        l = l * _exp(m - m_new) + _exp(float(x) - m_new)
        m = m_new
    return m, l


def attend_row(scores, values, block_sizes) -> tuple[np.ndarray, float, RowState]:
    """Run the recurrence over ``scores`` split into consecutive blocks.

    ``block_sizes`` is an int (uniform blocks, last one ragged) or a list of
    block lengths summing to ``len(scores)``.  Returns ``(o / l, m + ln l, state)``.
    """
    scores = list(scores)
    values = np.asarray(values, dtype=np.float64).reshape(len(scores), -1)
    n = len(scores)
    if isinstance(block_sizes, int):
        bounds = list(range(0, n, block_sizes)) + [n]
    else:
        assert sum(block_sizes) == n
        bounds = [0]
        for b in block_sizes:
            bounds.append(bounds[-1] + b)
    st = RowState()
    for a, b in zip(bounds[:-1], bounds[1:]):
        update(st, scores[a:b], values[a:b])
    return st.o / st.l, st.m + math.log(st.l), st


def attention_recurrence(q, k, v, scale: float, causal: bool, block: int):
    """Whole-head attention through the recurrence, one query row at a time.

    ``q, k, v`` are fp64 arrays [N, d]; scores are ``scale * q_i . k_j``.
    Returns ``(O [N, d], LSE [N])``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    out = np.zeros((n, v.shape[1]))
    lse = np.zeros(n)
    for i in range(n):
        nk = i + 1 if causal else k.shape[0]
        s = [scale * float(np.dot(q[i], k[j])) for j in range(nk)]
        o, L, _ = attend_row(s, v[:nk], block)
        out[i] = o
        lse[i] = L
    return out, lse
