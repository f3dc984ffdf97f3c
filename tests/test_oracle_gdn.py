"""Pins of the GDN oracle against things other than itself.

* a hand-derived two-token example with exact binary fractions
  (tests/golden/gdn_two_token_2x2.txt);
* special cases: alpha = 1, beta = 0 leaves the state unchanged bit for bit;
  alpha = 0, beta = 1 with a unit key stores v k^T and outputs v (k . q);
  alpha = 0, beta = 0 zeroes the state; beta = 0 scales it by the product of
  the alphas, however small;
  beta = 1 with a unit key makes S_t k_t = v_t for any alpha; with q = k and a
  unit key, o_t = alpha (1 - beta) S_{t-1} k + beta v;
* an independent formulation: the unrolled product
  S_T = S_0 A_1 ... A_T + sum_t beta_t v_t k_t^T A_{t+1} ... A_T with the
  dk x dk matrices A_t = alpha_t (I - beta_t k_t k_t^T) built explicitly;
* invariants: committing at c equals running on only the first c tokens
  ("undo equals never applied"); VERIFY_ONLY leaves the bank untouched; the
  rows of the state evolve independently; state slots are honoured.
"""

import os

import numpy as np
import pytest

import oracle
from oracle import GDN_COMMIT_ONLY, GDN_VERIFY_COMMIT, GDN_VERIFY_ONLY

GOLDEN = os.path.join(os.path.dirname(__file__), 'golden')


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith('#'):
                continue
            key, rest = line.split(':', 1)
            vals[key.strip()] = np.array([float(x) for x in rest.split()])
    return vals


def _rand_case(rng, T, H=3, dk=8, dv=6, unit_k=True, num_slots=None):
    B = len(T)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    n = cu[-1]
    ns = B if num_slots is None else num_slots
    state = 0.1 * rng.standard_normal((ns, H, dv, dk))
    q = rng.standard_normal((n, H, dk))
    k = rng.standard_normal((n, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((n, H, dv))
    alpha = rng.uniform(0.5, 1.0, (n, H))
    beta = rng.uniform(0.0, 1.0, (n, H))
    return dict(cu=cu, state=state, q=q, k=k, v=v, alpha=alpha, beta=beta)


def test_golden_two_token_example():
    g = _read_golden('gdn_two_token_2x2.txt')
    state = g['S0'].reshape(1, 1, 2, 2)
    k = g['k'].reshape(2, 1, 2)
    v = g['v'].reshape(2, 1, 2)
    q = g['q'].reshape(2, 1, 2)
    alpha = g['alpha'].reshape(2, 1)
    beta = g['beta'].reshape(2, 1)
    cu = np.array([0, 2])
    for c in range(3):
        o, S = oracle.gdn_step(state, None, q, k, v, alpha, beta, cu,
                               np.array([c]), GDN_VERIFY_COMMIT)
        np.testing.assert_array_equal(o.reshape(-1), g['o'])
        np.testing.assert_array_equal(S.reshape(-1), g[f'S_commit_{c}'])


def test_identity_gates_leave_state_unchanged():
    rng = np.random.default_rng(1)
    c = _rand_case(rng, [4, 2, 8])
    c['alpha'][:] = 1.0
    c['beta'][:] = 0.0
    o, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], np.array([4, 2, 8]),
                           GDN_VERIFY_COMMIT)
    np.testing.assert_array_equal(S, c['state'])
    for b in range(3):
        for x in range(c['cu'][b], c['cu'][b + 1]):
            for h in range(3):
                np.testing.assert_allclose(o[x, h], c['state'][b, h] @ c['q'][x, h],
                                           rtol=0, atol=1e-15)


def test_beta_one_unit_key_stores_value():
    rng = np.random.default_rng(2)
    c = _rand_case(rng, [1, 1, 1, 1])
    c['beta'][:] = 1.0
    _, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], np.ones(4, int),
                           GDN_VERIFY_COMMIT)
    for b in range(4):
        for h in range(3):
            np.testing.assert_allclose(S[b, h] @ c['k'][b, h], c['v'][b, h],
                                       rtol=0, atol=1e-13)


def test_zero_and_tiny_decay_closed_forms():
    """Gates at the edge of their range.  alpha = 0 and beta = 1 with a unit
    key: every token forgets the state and stores v k^T, so S_t = v_t k_t^T
    and o_t = v_t (k_t . q_t); alpha = 0 and beta = 0 zero the state and the
    output; beta = 0 with a tiny alpha scales the state by the product of the
    alphas (1e-12 * 1e-6 ... far below 2^-20)."""
    rng = np.random.default_rng(12)
    T = [1, 2, 3, 4]
    c = _rand_case(rng, T)
    c['alpha'][:] = 0.0
    c['beta'][:] = 1.0
    o, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'], c['alpha'], c['beta'],
                           c['cu'], np.array(T), GDN_VERIFY_COMMIT)
    for b in range(len(T)):
        last = c['cu'][b + 1] - 1
        for h in range(3):
            np.testing.assert_allclose(S[b, h], np.outer(c['v'][last, h], c['k'][last, h]),
                                       rtol=0, atol=1e-15)
            for x in range(c['cu'][b], c['cu'][b + 1]):
                np.testing.assert_allclose(o[x, h], c['v'][x, h] * (c['k'][x, h] @ c['q'][x, h]),
                                           rtol=0, atol=1e-14)
    c['beta'][:] = 0.0
    o, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'], c['alpha'], c['beta'],
                           c['cu'], np.array(T), GDN_VERIFY_COMMIT)
    assert not S.any() and not o.any()
    c['alpha'] = np.where(np.arange(len(c['alpha']))[:, None] % 2 == 0, 1e-12, 1e-6) \
        * np.ones_like(c['alpha'])
    _, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'], c['alpha'], c['beta'],
                           c['cu'], np.array(T), GDN_VERIFY_COMMIT)
    for b in range(len(T)):
        prod = np.prod(c['alpha'][c['cu'][b]:c['cu'][b + 1]], axis=0)
        for h in range(3):
            np.testing.assert_allclose(S[b, h], prod[h] * c['state'][b, h], rtol=1e-14, atol=0)


def test_output_closed_form_with_q_equal_k():
    rng = np.random.default_rng(3)
    c = _rand_case(rng, [1, 1, 1])
    c['q'] = c['k'].copy()
    o, _ = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], None, GDN_VERIFY_ONLY)
    for b in range(3):
        for h in range(3):
            a, bt = c['alpha'][b, h], c['beta'][b, h]
            expect = a * (1 - bt) * (c['state'][b, h] @ c['k'][b, h]) + bt * c['v'][b, h]
            np.testing.assert_allclose(o[b, h], expect, rtol=0, atol=1e-13)


def test_unrolled_product_formulation():
    rng = np.random.default_rng(4)
    T = [5, 3, 8]
    c = _rand_case(rng, T, H=2, dk=7, dv=5, unit_k=False)
    _, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], np.array(T),
                           GDN_VERIFY_COMMIT)
    dk = 7
    for b in range(3):
        rows = range(c['cu'][b], c['cu'][b + 1])
        for h in range(2):
            A = [c['alpha'][x, h] * (np.eye(dk) - c['beta'][x, h]
                                     * np.outer(c['k'][x, h], c['k'][x, h]))
                 for x in rows]
            tail = [np.eye(dk)]
            for M in reversed(A):
                tail.insert(0, M @ tail[0])        # tail[i] = A_i ... A_T
            expect = c['state'][b, h] @ tail[0]
            for i, x in enumerate(rows):
                expect = expect + c['beta'][x, h] * np.outer(c['v'][x, h], c['k'][x, h]) @ tail[i + 1]
            scale = np.abs(expect).max()
            assert np.abs(S[b, h] - expect).max() <= 1e-12 * scale


@pytest.mark.parametrize("mode", [GDN_VERIFY_COMMIT, GDN_COMMIT_ONLY])
def test_commit_equals_never_applied(mode):
    rng = np.random.default_rng(5)
    T = [4, 4, 8, 1, 3]
    commit = np.array([0, 4, 3, 1, 2])
    c = _rand_case(rng, T)
    _, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], commit, mode)
    for b, cb in enumerate(commit):
        # run a one-sequence batch holding only the first cb tokens
        lo = c['cu'][b]
        sl = slice(lo, lo + cb)
        cu1 = np.array([0, cb])
        _, S1 = oracle.gdn_step(c['state'][b:b + 1], None, c['q'][sl],
                                c['k'][sl], c['v'][sl], c['alpha'][sl],
                                c['beta'][sl], cu1, np.array([cb]),
                                GDN_VERIFY_COMMIT)
        np.testing.assert_array_equal(S[b], S1[0])
    if mode == GDN_VERIFY_COMMIT:
        o_only, S_only = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                                         c['alpha'], c['beta'], c['cu'], None,
                                         GDN_VERIFY_ONLY)
        np.testing.assert_array_equal(S_only, c['state'])
        o_vc, _ = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                                  c['alpha'], c['beta'], c['cu'], commit,
                                  GDN_VERIFY_COMMIT)
        np.testing.assert_array_equal(o_only, o_vc)


def test_rows_evolve_independently():
    rng = np.random.default_rng(6)
    c = _rand_case(rng, [4, 6], dv=9)
    rows = np.array([0, 3, 4, 8])
    o, S = oracle.gdn_step(c['state'], None, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], np.array([3, 6]),
                           GDN_VERIFY_COMMIT)
    o2, S2 = oracle.gdn_step(c['state'][:, :, rows], None, c['q'], c['k'],
                             c['v'][:, :, rows], c['alpha'], c['beta'], c['cu'],
                             np.array([3, 6]), GDN_VERIFY_COMMIT)
    # BLAS may block a matrix-vector product differently for another row
    # count, so equality is up to float64 rounding.
    np.testing.assert_allclose(S[:, :, rows], S2, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[:, :, rows], o2, rtol=0, atol=1e-14)


def test_state_slots_are_honoured():
    rng = np.random.default_rng(7)
    c = _rand_case(rng, [2, 3], num_slots=5)
    slots = np.array([4, 1])
    o, S = oracle.gdn_step(c['state'], slots, c['q'], c['k'], c['v'],
                           c['alpha'], c['beta'], c['cu'], np.array([2, 1]),
                           GDN_VERIFY_COMMIT)
    untouched = [0, 2, 3]
    np.testing.assert_array_equal(S[untouched], c['state'][untouched])
    for b, s in enumerate(slots):
        sl = slice(c['cu'][b], c['cu'][b + 1])
        o1, S1 = oracle.gdn_step(c['state'][s:s + 1], None, c['q'][sl],
                                 c['k'][sl], c['v'][sl], c['alpha'][sl],
                                 c['beta'][sl], np.array([0, sl.stop - sl.start]),
                                 np.array([[2, 1][b]]), GDN_VERIFY_COMMIT)
        np.testing.assert_array_equal(S[s], S1[0])
        np.testing.assert_array_equal(o[sl], o1)
