"""Pins of the short-convolution oracle against things other than itself.

* library routine: torch's grouped conv1d (one group per channel) on the
  state-padded sequence, float64 on the CPU;
* closed forms: a tap on the newest input copies x; a tap on the oldest
  reads the input K-1 steps back (from the state for the first tokens);
  SiLU against scipy's logistic function;
* invariants: commit at c equals running over the first c tokens only;
  c = 0 keeps the state bit for bit; VERIFY_ONLY leaves it; COMMIT_ONLY and
  VERIFY_COMMIT store the same state; a multi-token step equals T
  single-token steps (the state series: slot j is the state after token j);
  linearity in (state, x) without bias and activation.
"""

import numpy as np
import pytest
import torch
from scipy.special import expit

import oracle.short_conv as sc

RNG = np.random.default_rng(1234)


def _case(B=3, K=4, C=7, T=(1, 2, 5), slots=None):
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    ns = B if slots is None else slots
    state = RNG.normal(size=(ns, K - 1, C))
    x = RNG.normal(size=(cu[-1], C))
    w = RNG.normal(size=(C, K))
    bias = RNG.normal(size=(C,))
    return state, x, w, bias, cu


@pytest.mark.parametrize("silu", [False, True])
def test_matches_grouped_conv1d(silu):
    state, x, w, bias, cu = _case()
    y, _ = sc.conv_step(state, None, x, w, bias, cu, None, sc.CONV_VERIFY_ONLY, silu=silu)
    C, K = w.shape
    for b in range(len(cu) - 1):
        z = np.concatenate([state[b], x[cu[b]:cu[b + 1]]], axis=0)   # [K-1+T, C]
        inp = torch.from_numpy(z.T[None].copy())                       # [1, C, L]
        ref = torch.nn.functional.conv1d(inp, torch.from_numpy(w[:, None, :].copy()),
                                         torch.from_numpy(bias), groups=C)[0].T.numpy()
        if silu:
            ref = ref * expit(ref)
        np.testing.assert_allclose(y[cu[b]:cu[b + 1]], ref, rtol=1e-12, atol=1e-12)


def test_newest_and_oldest_taps():
    state, x, w, bias, cu = _case(T=(1, 3, 6))
    C, K = w.shape
    newest = np.zeros_like(w)
    newest[:, K - 1] = 1.0
    y, _ = sc.conv_step(state, None, x, newest, None, cu, None, sc.CONV_VERIFY_ONLY)
    assert np.array_equal(y, x)
    oldest = np.zeros_like(w)
    oldest[:, 0] = 1.0
    y, _ = sc.conv_step(state, None, x, oldest, None, cu, None, sc.CONV_VERIFY_ONLY)
    for b in range(len(cu) - 1):
        T = cu[b + 1] - cu[b]
        for t in range(T):
            src = state[b][t] if t < K - 1 else x[cu[b] + t - (K - 1)]
            assert np.array_equal(y[cu[b] + t], src)


def test_silu_closed_form():
    u = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(sc._silu(u), u * expit(u), rtol=1e-14, atol=1e-300)
    assert sc._silu(np.array([0.0]))[0] == 0.0


def test_commit_equals_run_on_prefix_and_modes():
    state, x, w, bias, cu = _case(B=4, T=(1, 2, 4, 6))
    B = len(cu) - 1
    for trial in range(5):
        c = np.array([RNG.integers(0, cu[b + 1] - cu[b] + 1) for b in range(B)])
        y_vc, S_vc = sc.conv_step(state, None, x, w, bias, cu, c, sc.CONV_VERIFY_COMMIT)
        _, S_co = sc.conv_step(state, None, x, w, bias, cu, c, sc.CONV_COMMIT_ONLY)
        y_vo, S_vo = sc.conv_step(state, None, x, w, bias, cu, None, sc.CONV_VERIFY_ONLY)
        assert np.array_equal(S_vc, S_co)
        assert np.array_equal(S_vo, state)
        assert np.array_equal(y_vc, y_vo)
        # run on the first c tokens only
        pre_cu = np.concatenate([[0], np.cumsum(c)]).astype(np.int64)
        pre_x = np.concatenate([x[cu[b]:cu[b] + c[b]] for b in range(B)], axis=0)
        _, S_pre = sc.conv_step(state, None, pre_x, w, bias, pre_cu, c, sc.CONV_COMMIT_ONLY)
        assert np.array_equal(S_vc, S_pre)
        for b in range(B):
            if c[b] == 0:
                assert np.array_equal(S_vc[b], state[b])


def test_state_series_single_token_steps():
    """T single-token steps (each committing its token) give the outputs and
    the final state of one T-token step committing all T."""
    state, x, w, bias, cu = _case(B=2, T=(5, 3))
    B = len(cu) - 1
    T_all = np.diff(cu)
    y_full, S_full = sc.conv_step(state, None, x, w, bias, cu, T_all, sc.CONV_VERIFY_COMMIT,
                                  silu=True)
    S = state.copy()
    for b in range(B):
        for t in range(T_all[b]):
            one_cu = np.array([0, 1])
            y1, S_b = sc.conv_step(S[b:b + 1], None, x[cu[b] + t:cu[b] + t + 1], w, bias,
                                   one_cu, np.array([1]), sc.CONV_VERIFY_COMMIT, silu=True)
            np.testing.assert_allclose(y1[0], y_full[cu[b] + t], rtol=0, atol=1e-13)
            S[b] = S_b[0]
    np.testing.assert_array_equal(S, S_full)


def test_linear_in_state_and_input():
    s1, x1, w, _, cu = _case()
    s2 = RNG.normal(size=s1.shape)
    x2 = RNG.normal(size=x1.shape)
    a, b = 0.75, -1.5
    y1, _ = sc.conv_step(s1, None, x1, w, None, cu, None, sc.CONV_VERIFY_ONLY)
    y2, _ = sc.conv_step(s2, None, x2, w, None, cu, None, sc.CONV_VERIFY_ONLY)
    y3, _ = sc.conv_step(a * s1 + b * s2, None, a * x1 + b * x2, w, None, cu, None,
                         sc.CONV_VERIFY_ONLY)
    np.testing.assert_allclose(y3, a * y1 + b * y2, rtol=1e-12, atol=1e-12)


def test_state_slots_route_rows():
    state, x, w, bias, cu = _case(B=3, slots=6)
    slots = np.array([4, 0, 2])
    c = np.array([1, 2, 3])
    y, S = sc.conv_step(state, slots, x, w, bias, cu, c, sc.CONV_VERIFY_COMMIT)
    # the same as running each sequence on its own slot as slot 0
    for b in range(3):
        rows = slice(cu[b], cu[b + 1])
        yb, Sb = sc.conv_step(state[slots[b]:slots[b] + 1], None, x[rows], w, bias,
                              np.array([0, cu[b + 1] - cu[b]]), c[b:b + 1],
                              sc.CONV_VERIFY_COMMIT)
        assert np.array_equal(y[rows], yb)
        assert np.array_equal(S[slots[b]], Sb[0])
    untouched = [s for s in range(6) if s not in slots]
    assert np.array_equal(S[untouched], state[untouched])
