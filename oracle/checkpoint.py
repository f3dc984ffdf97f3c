"""Oracle for the checkpoint-series commit of the recurrent and conv states.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The other way the pages roll back a partially accepted draft
("microsoft/onnxruntime-genai pull request 2457", commit messages on emitting
the per-token state series and on ``CommitPrefix``): during the step the
packed varlen operators publish the state after every token into a window of
``W`` slots -- the short convolution's ``prefix_states`` writes slot ``j``
after local token ``j``, GatedDeltaNet's ``checkpoints`` writes slot ``W - 1``
after the last token -- and after acceptance ``CommitPrefix`` stages the slot
of the accepted prefix as the new state instead of the step's final state.

Readings written out here:
* the series is per sequence, ``[B, W, ...]``, with ``W >= T_b``;
* GatedDeltaNet is end-aligned: token ``j`` of a ``T_b``-token sequence goes
  to slot ``W - T_b + j``; the conv is front-aligned: token ``j`` to slot
  ``j``; slots no token maps to keep their contents;
* the state after token ``j`` is the state a run over tokens ``0..j`` leaves
  (``gdn_step`` / ``conv_step`` committing ``j + 1`` tokens);
* the verify pass leaves the state bank untouched;
* ``CommitPrefix`` with ``c_b`` kept tokens copies the slot of token
  ``c_b - 1`` into the sequence's state slot; ``c_b = 0`` keeps the state.
"""

import numpy as np

from .gdn import GDN_COMMIT_ONLY, GDN_VERIFY_ONLY, gdn_step
from .short_conv import CONV_COMMIT_ONLY, CONV_VERIFY_ONLY, conv_step


def _one(cu, b):
    """Batch of sequence b alone: its rows and a one-sequence cu_seqlens."""
    lo, hi = int(cu[b]), int(cu[b + 1])
    return slice(lo, hi), np.array([0, hi - lo])


def gdn_checkpoints(state, state_slot, q, k, v, alpha, beta, cu_seqlens, window,
                    series=None):
    """Verify with a checkpoint series.

    Returns ``(o, series)``: the outputs of every verify token (as
    ``gdn_step`` in VERIFY_ONLY mode) and the float64 series
    ``[B, W, H, dv, dk]`` (a copy of ``series`` with the written slots
    replaced; zeros if None).
    """
    state = np.asarray(state, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    W = int(window)
    o, _ = gdn_step(state, state_slot, q, k, v, alpha, beta, cu, None, GDN_VERIFY_ONLY)
    shp = (B, W) + state.shape[1:]
    out = np.zeros(shp) if series is None else np.array(series, dtype=np.float64, copy=True)
    for b in range(B):
        rows, cu1 = _one(cu, b)
        T = int(cu[b + 1] - cu[b])
        slot = b if state_slot is None else int(state_slot[b])
        for j in range(T):
            _, S = gdn_step(state[slot:slot + 1], None, None, k[rows], v[rows], alpha[rows],
                            beta[rows], cu1, np.array([j + 1]), GDN_COMMIT_ONLY)
            out[b, W - T + j] = S[0]
    return o, out


def gdn_commit_prefix(state, state_slot, series, cu_seqlens, commit_len, window):
    """``CommitPrefix`` for GatedDeltaNet: a float64 copy of the bank with
    ``state[slot_b] = series[b, W - T_b + c_b - 1]`` where ``c_b >= 1``."""
    bank = np.array(state, dtype=np.float64, copy=True)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    W = int(window)
    for b in range(len(cu) - 1):
        c = int(commit_len[b])
        if c == 0:
            continue
        T = int(cu[b + 1] - cu[b])
        slot = b if state_slot is None else int(state_slot[b])
        bank[slot] = series[b, W - T + c - 1]
    return bank


def conv_checkpoints(state, state_slot, x, weight, bias, cu_seqlens, window, silu=False,
                     series=None):
    """Short-conv verify with its prefix-state series ``[B, W, K-1, C]``
    (slot ``j`` = the window after local token ``j``)."""
    state = np.asarray(state, dtype=np.float64)
    x = np.asarray(x, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = len(cu) - 1
    W = int(window)
    y, _ = conv_step(state, state_slot, x, weight, bias, cu, None, CONV_VERIFY_ONLY, silu=silu)
    shp = (B, W) + state.shape[1:]
    out = np.zeros(shp) if series is None else np.array(series, dtype=np.float64, copy=True)
    for b in range(B):
        rows, cu1 = _one(cu, b)
        T = int(cu[b + 1] - cu[b])
        slot = b if state_slot is None else int(state_slot[b])
        for j in range(T):
            _, S = conv_step(state[slot:slot + 1], None, x[rows], weight, bias, cu1,
                             np.array([j + 1]), CONV_COMMIT_ONLY, silu=silu)
            out[b, j] = S[0]
    return y, out


def conv_commit_prefix(state, state_slot, series, cu_seqlens, commit_len):
    """``CommitPrefix`` for the conv: ``state[slot_b] = series[b, c_b - 1]``
    where ``c_b >= 1``."""
    bank = np.array(state, dtype=np.float64, copy=True)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    for b in range(len(cu) - 1):
        c = int(commit_len[b])
        if c == 0:
            continue
        slot = b if state_slot is None else int(state_slot[b])
        bank[slot] = series[b, c - 1]
    return bank
