"""Pins of the checkpoint-series oracle against things other than itself.

* GatedDeltaNet, end-aligned: every slot times its token's query is that
  token's output (o_t = S_t q_t), so the slot of token t holds S_t; slot W - 1
  holds the state after the last token;
* conv, front-aligned: slot j is the last K - 1 rows of [state, x_0 .. x_j]
  (copies of inputs), and each output y_t is the convolution of the window in
  slot t - 1 (the state for t = 0) with x_t;
* CommitPrefix equals committing the same prefix by replay (COMMIT_ONLY), for
  every c_b including 0 and T_b; slots no token maps to, and the state bank,
  are left as they were.
"""

import numpy as np
import pytest

import oracle.checkpoint as ck
from oracle.gdn import GDN_COMMIT_ONLY, gdn_step
from oracle.short_conv import CONV_COMMIT_ONLY, _silu, conv_step

RNG = np.random.default_rng(777)


def _gdn_case(T=(1, 3, 4), H=2, dk=4, dv=3, slots=None):
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    n = cu[-1]
    B = len(T)
    ns = B if slots is None else slots
    state = RNG.normal(size=(ns, H, dv, dk)) * 0.3
    q = RNG.normal(size=(n, H, dk))
    k = RNG.normal(size=(n, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = RNG.normal(size=(n, H, dv))
    alpha = RNG.uniform(0.8, 1.0, size=(n, H))
    beta = RNG.uniform(0.0, 1.0, size=(n, H))
    return state, q, k, v, alpha, beta, cu


@pytest.mark.parametrize("W", [4, 6])
def test_gdn_slots_hold_the_state_after_their_token(W):
    state, q, k, v, alpha, beta, cu = _gdn_case()
    sentinel = np.full((3, W, 2, 3, 4), 7.5)
    o, series = ck.gdn_checkpoints(state, None, q, k, v, alpha, beta, cu, W, series=sentinel)
    for b in range(3):
        T = int(cu[b + 1] - cu[b])
        for t in range(T):
            x = cu[b] + t
            for h in range(2):
                np.testing.assert_allclose(series[b, W - T + t, h] @ q[x, h], o[x, h],
                                           rtol=1e-12, atol=1e-12)
        assert np.all(series[b, :W - T] == 7.5)          # slots with no token
        _, S = gdn_step(state, None, None, k, v, alpha, beta, cu, np.diff(cu), GDN_COMMIT_ONLY)
        np.testing.assert_allclose(series[b, W - 1], S[b], rtol=1e-12, atol=1e-14)


def test_gdn_commit_prefix_equals_replay_commit():
    state, q, k, v, alpha, beta, cu = _gdn_case(T=(2, 4, 1, 3), slots=7)
    slots = np.array([5, 0, 3, 6])
    W = 5
    _, series = ck.gdn_checkpoints(state, slots, q, k, v, alpha, beta, cu, W)
    T = np.diff(cu)
    for trial in range(6):
        c = np.array([RNG.integers(0, t + 1) for t in T])
        if trial == 0:
            c = np.zeros_like(T)
        if trial == 1:
            c = T.copy()
        got = ck.gdn_commit_prefix(state, slots, series, cu, c, W)
        _, ref = gdn_step(state, slots, None, k, v, alpha, beta, cu, c, GDN_COMMIT_ONLY)
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)
        for s in (1, 2, 4):                              # slots of no sequence
            assert np.array_equal(got[s], state[s])


def _conv_case(T=(1, 2, 5), K=4, C=5):
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    state = RNG.normal(size=(len(T), K - 1, C))
    x = RNG.normal(size=(cu[-1], C))
    w = RNG.normal(size=(C, K))
    bias = RNG.normal(size=(C,))
    return state, x, w, bias, cu


@pytest.mark.parametrize("silu", [False, True])
def test_conv_slots_are_input_windows_and_drive_the_outputs(silu):
    state, x, w, bias, cu = _conv_case()
    W = 6
    sentinel = np.full((3, W, 3, 5), -2.0)
    y, series = ck.conv_checkpoints(state, None, x, w, bias, cu, W, silu=silu, series=sentinel)
    K = w.shape[1]
    for b in range(3):
        T = int(cu[b + 1] - cu[b])
        z = np.concatenate([state[b], x[cu[b]:cu[b + 1]]], axis=0)
        for j in range(T):
            assert np.array_equal(series[b, j], z[j + 1:j + K])
        assert np.all(series[b, T:] == -2.0)
        for t in range(T):
            win = state[b] if t == 0 else series[b, t - 1]
            u = np.sum(w * np.concatenate([win, x[cu[b] + t][None]], axis=0).T, axis=1) + bias
            np.testing.assert_allclose(y[cu[b] + t], _silu(u) if silu else u,
                                       rtol=1e-12, atol=1e-12)


def test_conv_commit_prefix_equals_replay_commit():
    state, x, w, bias, cu = _conv_case(T=(3, 1, 4))
    W = 4
    _, series = ck.conv_checkpoints(state, None, x, w, bias, cu, W)
    T = np.diff(cu)
    for c in (np.zeros_like(T), T.copy(), np.array([2, 0, 3])):
        got = ck.conv_commit_prefix(state, None, series, cu, c)
        _, ref = conv_step(state, None, x, w, bias, cu, c, CONV_COMMIT_ONLY)
        assert np.array_equal(got, ref)
