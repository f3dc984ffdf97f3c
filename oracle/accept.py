"""Oracle for the acceptance step: greedy and rejection sampling.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Row conventions (packed varlen, as the verify pass produces them): sequence
``b`` has ``T_b = k_b + 1`` target rows ``cu[b] .. cu[b+1]-1`` (row ``i`` is
the target's prediction after verify token ``i``) and ``k_b`` draft positions
packed at ``cu[b] - b .. cu[b] - b + k_b - 1``.

Output layout (lmdeploy PR 3945, review of ``reject_sampler.py``: one row per
sequence of width ``max_spec_len + 1``, the accepted drafts followed by one
recovered/bonus token, padded with -1): ``out[b] = [x_1 .. x_a, y, -1 ...]``
and ``accept_len[b] = a``.

Greedy (onnxruntime-genai PR 2457, commit messages on the greedy MTP step and
on the device argmax of the verify rows): ``g_i = argmax`` of target row ``i``
(lowest index on ties), ``a`` = length of the leading run with
``draft_i == g_i``, ``y = g_a``.

Rejection sampling (Leviathan et al. 2023, Algorithm 1; Chen et al. 2023),
temperature 1, with the uniforms supplied by the caller: position ``i`` with
draft ``x`` is accepted iff ``u_accept[i] * q_i(x) < p_i(x)``; at the first
rejection ``y`` is drawn from ``max(0, p_i - q_i)`` (normalised) by inverse
CDF with ``u_final[b]``; if all ``k_b`` drafts pass, ``y`` is drawn from
``p_{k_b}`` the same way.  ``p`` / ``q`` are the float64 softmaxes of the
target / draft logits.
"""

import numpy as np


def softmax64(z):
    """Float64 softmax of one logits row: ``e = exp(z - max z); e / sum(e)``."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(z - z.max())
    return e / e.sum()


def icdf(w, u):
    """Inverse-CDF draw from non-negative weights ``w`` with uniform ``u``.

    ``C = cumsum(w)`` in index order, ``t = u * C[-1]``; returns the first
    index ``y`` with ``C[y] > t``.  If rounding leaves none, returns the last
    index with ``w > 0``.
    """
    w = np.asarray(w, dtype=np.float64)
    C = np.cumsum(w)
    t = float(u) * C[-1]
    hit = np.nonzero(C > t)[0]
    if hit.size:
        return int(hit[0])
    return int(np.nonzero(w > 0)[0][-1])


def _layout(B, max_T):
    return np.zeros(B, dtype=np.int32), np.full((B, max_T), -1, dtype=np.int32)


def greedy_accept(target_logits, draft_tokens, cu_seqlens, max_T, bonus_tokens=None):
    """Greedy acceptance.  Returns ``(accept_len[B], out_tokens[B, max_T])``.

    ``bonus_tokens`` (optional, one per sequence): when every draft is
    accepted the emitted bonus token is the supplied one instead of the last
    row's argmax (lmdeploy PR 3945, ``reject_sampler.py``: pre-sampled
    ``bonus_token_ids``).
    """
    target_logits = np.asarray(target_logits, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    accept_len, out = _layout(B, max_T)
    for b in range(B):
        T = int(cu[b + 1] - cu[b])
        k = T - 1
        d0 = int(cu[b]) - b
        g = [int(np.argmax(target_logits[cu[b] + i])) for i in range(T)]
        a = 0
        while a < k and int(draft_tokens[d0 + a]) == g[a]:
            a += 1
        out[b, :a] = draft_tokens[d0:d0 + a]
        out[b, a] = int(bonus_tokens[b]) if (bonus_tokens is not None and a == k) else g[a]
        accept_len[b] = a
    return accept_len, out


def rejection_accept(target_logits, draft_logits, draft_tokens, u_accept,
                     u_final, cu_seqlens, max_T, return_margins=False,
                     bonus_tokens=None):
    """Speculative (rejection) sampling acceptance.

    ``draft_logits = None``: the draft distribution of each position is the
    point mass on the draft token (lmdeploy PR 3945, ``reject_sampler.py``
    with ``draft_probs = None``); Algorithm 1 then accepts iff ``u < p(x)``
    and the residual is ``p`` with ``x`` removed.  ``bonus_tokens``
    (optional): when every draft is accepted the supplied token is emitted
    instead of a draw from the last target row (pre-sampled
    ``bonus_token_ids`` of the same file).

    Returns ``(accept_len[B], out_tokens[B, max_T])`` and, with
    ``return_margins``, a list per sequence of the distances of each decision
    from its threshold: ``|u q(x) - p(x)|`` per tested draft and
    ``min(|t - C[y-1]|, |t - C[y]|)`` for the final draw (a GPU result that
    differs must sit inside float64 rounding of one of these).
    """
    target_logits = np.asarray(target_logits, dtype=np.float64)
    if draft_logits is not None:
        draft_logits = np.asarray(draft_logits, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    V = target_logits.shape[1]
    accept_len, out = _layout(B, max_T)
    margins = []
    for b in range(B):
        T = int(cu[b + 1] - cu[b])
        k = T - 1
        d0 = int(cu[b]) - b
        m_b = []
        a, w = k, None
        for i in range(k):
            p = softmax64(target_logits[cu[b] + i])
            x = int(draft_tokens[d0 + i])
            if draft_logits is None:
                q = np.zeros(V)
                q[x] = 1.0
            else:
                q = softmax64(draft_logits[d0 + i])
            lhs = float(np.float64(u_accept[d0 + i]) * q[x])
            m_b.append(abs(lhs - p[x]))
            if lhs < p[x]:
                continue
            r = np.maximum(p - q, 0.0)
            if r.sum() == 0.0:
                r = p          # p == q up to rounding: fall back to p
            a, w = i, r
            break
        if w is None and bonus_tokens is not None:
            y = int(bonus_tokens[b])
            m_b.append(float('inf'))      # no draw: nothing to be near
        else:
            if w is None:
                w = softmax64(target_logits[cu[b] + k])
            y = icdf(w, u_final[b])
            C = np.cumsum(w)
            t = float(u_final[b]) * C[-1]
            lo = C[y - 1] if y > 0 else 0.0
            m_b.append(min(abs(t - lo), abs(C[y] - t)))
        margins.append(m_b)
        out[b, :a] = draft_tokens[d0:d0 + a]
        out[b, a] = y
        accept_len[b] = a
    if return_margins:
        return accept_len, out, margins
    return accept_len, out
