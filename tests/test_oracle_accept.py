"""Pins of the acceptance oracle against things other than itself.

* inverse CDF: closed-form answers on hand-made weight vectors;
* greedy: a brute-force prefix compare whose argmax is found another way,
  ties resolved to the lowest index, and a toy bigram decoder in which
  speculative decoding with greedy acceptance must reproduce plain greedy
  decoding token for token (the lossless property the onnxruntime-genai
  pull request 2457 reports for its MTP path);
* rejection sampling, against the statement of speculative sampling
  (Leviathan et al. 2023, Theorem 1; Chen et al. 2023):
  - exact enumeration on a tiny vocabulary: the oracle is treated as a black
    box that is piecewise constant in its uniforms; the measure of every
    output set is found by bisection and summed exactly; the token emitted at
    each position must follow the target distribution p_i, and each position
    must be accepted with probability sum_x min(p_i, q_i);
  - Monte-Carlo with fresh uniforms and drafts drawn from q (chi-square);
  - special cases: q = p always accepts; disjoint supports always reject at
    the first position and then draw from p;
* the output layout of the lmdeploy reject sampler
  (tests/golden/reject_sampler_layout.txt).
"""

import itertools
import os
from collections import defaultdict

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), 'golden')
NEG = -1.0e4          # exp(NEG - max) underflows to exactly 0.0 in float64


# ----------------------------------------------------------------- icdf
def test_icdf_closed_forms():
    w = np.array([1.0, 0.0, 3.0])
    assert oracle.icdf(w, 0.0) == 0
    assert oracle.icdf(w, 0.2499) == 0
    assert oracle.icdf(w, 0.25) == 2            # C = [1, 1, 4]; t = 1 -> C > 1
    assert oracle.icdf(w, 0.99) == 2
    assert oracle.icdf(np.array([0.0, 0.0, 2.0, 0.0]), 0.0) == 2
    assert oracle.icdf(np.array([0.5, 0.5]), 0.5) == 1
    # u = 1 is outside [0, 1): no C[y] > t, the fallback returns the last
    # index with positive weight.
    assert oracle.icdf(np.array([0.3, 0.7, 0.0]), 1.0) == 1


def test_softmax64_closed_form():
    z = np.array([0.0, np.log(3.0), NEG])
    np.testing.assert_allclose(oracle.softmax64(z), [0.25, 0.75, 0.0],
                               rtol=1e-15, atol=0)


# ----------------------------------------------------------------- greedy
def _first_max_index(row):
    return int(np.flatnonzero(row == row.max())[0])


@pytest.mark.parametrize("seed", range(5))
def test_greedy_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    B, V = 7, 13
    ks = rng.integers(0, 6, B)
    cu = np.concatenate([[0], np.cumsum(ks + 1)])
    # coarse values make ties frequent
    logits = rng.integers(-3, 4, (cu[-1], V)).astype(np.float64)
    drafts = []
    for b in range(B):
        for i in range(ks[b]):
            g = _first_max_index(logits[cu[b] + i])
            drafts.append(g if rng.random() < 0.7 else int(rng.integers(0, V)))
    drafts = np.array(drafts, dtype=np.int64)
    max_T = int(ks.max() + 1)
    acc, out = oracle.greedy_accept(logits, drafts, cu, max_T)
    for b in range(B):
        d = drafts[cu[b] - b: cu[b] - b + ks[b]]
        g = [_first_max_index(logits[cu[b] + i]) for i in range(ks[b] + 1)]
        match = np.array([d[i] == g[i] for i in range(ks[b])], dtype=bool)
        a = int(np.cumprod(match).sum()) if ks[b] else 0
        assert acc[b] == a
        expect = list(d[:a]) + [g[a]] + [-1] * (max_T - a - 1)
        assert out[b].tolist() == expect


def test_greedy_ties_take_lowest_index():
    V = 8
    row = np.zeros(V)
    row[[2, 5, 7]] = 4.0
    logits = np.stack([row, row])
    acc, out = oracle.greedy_accept(logits, np.array([5]), [0, 2], 2)
    assert acc.tolist() == [0] and out.tolist() == [[2, -1]]
    acc, out = oracle.greedy_accept(logits, np.array([2]), [0, 2], 2)
    assert acc.tolist() == [1] and out.tolist() == [[2, 2]]


def test_toy_bigram_greedy_speculation_is_lossless():
    rng = np.random.default_rng(11)
    V, k, n_out = 40, 3, 200
    target = rng.standard_normal((V, V))
    draft = target + 0.8 * rng.standard_normal((V, V))
    # plain greedy decoding
    seq = [0]
    while len(seq) < n_out:
        seq.append(_first_max_index(target[seq[-1]]))
    # speculative decoding: greedy drafts, verify k+1 rows, keep a+1 tokens
    spec = [0]
    rounds = 0
    while len(spec) < n_out:
        d = []
        last = spec[-1]
        for _ in range(k):
            last = _first_max_index(draft[last])
            d.append(last)
        verify_tokens = [spec[-1]] + d
        rows = np.stack([target[t] for t in verify_tokens])
        acc, out = oracle.greedy_accept(rows, np.array(d), [0, k + 1], k + 1)
        spec.extend(int(t) for t in out[0, :acc[0] + 1])
        rounds += 1
    assert spec[:n_out] == seq
    assert rounds < n_out - 1          # speculation did accept something


# ----------------------------------------------------------------- layout
def _read_layout():
    rows = []
    with open(os.path.join(GOLDEN, 'reject_sampler_layout.txt')) as f:
        for line in f:
            if line.startswith('row'):
                rows.append([int(x) for x in line.split(':')[1].split()])
            elif line.startswith('max_spec_len'):
                msl = int(line.split(':')[1])
    return msl, np.array(rows)


def _one_hot_rows(idx, V):
    z = np.full((len(idx), V), NEG)
    z[np.arange(len(idx)), idx] = 0.0
    return z


@pytest.mark.parametrize("mode", ["greedy", "rejection"])
def test_reject_sampler_layout(mode):
    msl, expect = _read_layout()
    V = 5
    cu = [0, 3, 6, 9]
    target = _one_hot_rows([0, 1, 2, 0, 3, 3, 1, 4, 4], V)
    drafts = np.array([0, 1, 3, 4, 2, 2])
    draft_logits = _one_hot_rows(drafts, V)
    if mode == "greedy":
        acc, out = oracle.greedy_accept(target, drafts, cu, msl + 1)
    else:
        rng = np.random.default_rng(0)
        acc, out = oracle.rejection_accept(target, draft_logits, drafts,
                                           rng.random(6), rng.random(3), cu,
                                           msl + 1)
    np.testing.assert_array_equal(out, expect)
    np.testing.assert_array_equal(acc, [2, 0, 0])


# ----------------------------------------------------------------- rejection
def _run_one(target, draft, x, u_acc, u_fin):
    k = len(x)
    acc, out = oracle.rejection_accept(target, draft, np.array(x), np.array(u_acc),
                                       np.array([u_fin]), [0, k + 1], k + 1)
    return int(acc[0]), tuple(int(t) for t in out[0, :acc[0] + 1])


def _threshold(f, iters=60):
    """f(u) is True on [0, tau) and False on [tau, 1); return tau."""
    if not f(0.0):
        return 0.0
    hi_u = np.nextafter(1.0, 0.0)
    if f(hi_u):
        return 1.0
    lo, hi = 0.0, hi_u
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        if f(mid):
            lo = mid
        else:
            hi = mid
    return hi


def _step_measure(g, iters=60):
    """Measure of each value of the non-decreasing step function g on [0, 1)."""
    out = defaultdict(float)
    start = 0.0
    while True:
        y = g(start)
        end_u = np.nextafter(1.0, 0.0)
        if g(end_u) == y:
            out[y] += 1.0 - start
            return out
        lo, hi = start, end_u
        for _ in range(iters):
            mid = 0.5 * (lo + hi)
            if g(mid) == y:
                lo = mid
            else:
                hi = mid
        out[y] += hi - start
        start = hi


def _enumerate(target, draft, V, k):
    """Exact distribution of (a, emitted tokens) with drafts x ~ q."""
    q = [special.softmax(draft[i]) for i in range(k)]
    dist = defaultdict(float)
    for x in itertools.product(range(V), repeat=k):
        wx = float(np.prod([q[i][x[i]] for i in range(k)]))
        if wx == 0.0:
            continue
        taus = []
        for i in range(k):
            def acc_at(u, i=i):
                ua = [0.0] * k
                ua[i] = u
                a, _ = _run_one(target, draft, x, ua, 0.5)
                return a > i
            taus.append(_threshold(acc_at))
        for a in range(k + 1):
            pa = float(np.prod(taus[:a])) * ((1.0 - taus[a]) if a < k else 1.0)
            if pa <= 0.0:
                continue
            ua = [t * 0.5 for t in taus[:a]] + \
                 ([0.5 * (1.0 + taus[a])] if a < k else []) + [0.0] * (k - a - 1)
            meas = _step_measure(lambda u: _run_one(target, draft, x, ua, u)[1])
            for tokens, m in meas.items():
                dist[tokens] += wx * pa * m
    return dist


def _check_theorem(dist, target, draft, V, k):
    p = [special.softmax(target[i]) for i in range(k + 1)]
    q = [special.softmax(draft[i]) for i in range(k)]
    total = sum(dist.values())
    assert abs(total - 1.0) < 1e-9
    reach = 1.0
    for i in range(k + 1):
        marg = np.zeros(V)
        for tokens, m in dist.items():
            if len(tokens) > i:
                marg[tokens[i]] += m
        mass = marg.sum()
        np.testing.assert_allclose(mass, reach, rtol=0, atol=1e-9)
        np.testing.assert_allclose(marg / mass, p[i], rtol=0, atol=1e-9)
        if i < k:
            reach *= np.minimum(p[i], q[i]).sum()


@pytest.mark.parametrize("seed,V,k", [(0, 3, 1), (1, 4, 2), (2, 3, 2), (3, 4, 1)])
def test_rejection_exact_enumeration(seed, V, k):
    rng = np.random.default_rng(seed)
    target = 1.5 * rng.standard_normal((k + 1, V))
    draft = 1.5 * rng.standard_normal((k, V))
    dist = _enumerate(target, draft, V, k)
    _check_theorem(dist, target, draft, V, k)


def test_rejection_exact_enumeration_with_zero_probabilities():
    V, k = 4, 2
    target = np.array([[0.0, 1.0, NEG, 0.5], [NEG, 0.3, 0.0, -1.0], [0.2, NEG, 0.0, 1.0]])
    draft = np.array([[NEG, 0.0, 2.0, -1.0], [1.0, 0.0, NEG, 0.0]])
    dist = _enumerate(target, draft, V, k)
    _check_theorem(dist, target, draft, V, k)


def test_rejection_q_equal_p_always_accepts():
    rng = np.random.default_rng(3)
    V, k, B = 6, 3, 20
    target = rng.standard_normal((B * (k + 1), V))
    cu = np.arange(B + 1) * (k + 1)
    rows = [cu[b] + i for b in range(B) for i in range(k)]
    draft = target[rows]
    drafts = rng.integers(0, V, B * k)
    acc, out = oracle.rejection_accept(target, draft, drafts, rng.random(B * k),
                                       rng.random(B), cu, k + 1)
    assert (acc == k).all()
    np.testing.assert_array_equal(out[:, :k], drafts.reshape(B, k))


def test_rejection_disjoint_supports_draw_from_p():
    V = 4
    target = np.array([[0.0, np.log(3.0), NEG, NEG], [0.0, 0.0, 0.0, 0.0]])
    draft = np.array([[NEG, NEG, 0.0, 0.0]])
    for x in (2, 3):
        a, _ = _run_one(target, draft, [x], [0.0], 0.5)
        assert a == 0
        meas = _step_measure(lambda u: _run_one(target, draft, [x], [0.0], u)[1])
        assert set(meas) == {(0,), (1,)}
        np.testing.assert_allclose([meas[(0,)], meas[(1,)]], [0.25, 0.75],
                                   rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", [0])
def test_rejection_monte_carlo(seed):
    rng = np.random.default_rng(seed)
    V, k, N = 6, 3, 120000
    target_rows = 1.2 * rng.standard_normal((k + 1, V))
    draft_rows = 1.2 * rng.standard_normal((k, V))
    q = [special.softmax(r) for r in draft_rows]
    p = [special.softmax(r) for r in target_rows]
    target = np.tile(target_rows, (N, 1))
    draft = np.tile(draft_rows, (N, 1))
    drafts = np.stack([rng.choice(V, size=N, p=q[i]) for i in range(k)], 1).reshape(-1)
    cu = np.arange(N + 1) * (k + 1)
    acc, out = oracle.rejection_accept(target, draft, drafts, rng.random(N * k),
                                       rng.random(N), cu, k + 1)
    for i in range(k + 1):
        sel = acc >= i
        counts = np.bincount(out[sel, i], minlength=V)
        expected = p[i] * sel.sum()
        keep = expected > 5
        chi2 = (((counts - expected) ** 2)[keep] / expected[keep]).sum()
        pval = stats.chi2.sf(chi2, keep.sum() - 1)
        assert pval > 1e-3, (i, counts, expected)
        if i < k:
            rate = (acc[sel] > i).mean()
            alpha = np.minimum(p[i], q[i]).sum()
            se = np.sqrt(alpha * (1 - alpha) / sel.sum())
            assert abs(rate - alpha) < 4 * se


# ------------------------------------------------ one-hot drafts, supplied bonus
def _run_one_hot(target, x, u_acc, u_fin):
    k = len(x)
    acc, out = oracle.rejection_accept(target, None, np.array(x), np.array(u_acc),
                                       np.array([u_fin]), [0, k + 1], k + 1)
    return int(acc[0]), tuple(int(t) for t in out[0, :acc[0] + 1])


@pytest.mark.parametrize("seed,V,k", [(5, 3, 1), (6, 4, 2), (7, 3, 2)])
def test_one_hot_drafts_exact_enumeration(seed, V, k):
    """Deterministic drafts (point-mass draft distributions): emitted token i,
    given the chain reached i, is distributed as p_i exactly, and the chain
    reaches i with probability prod_{j<i} p_j(x_j) -- Theorem 1 of Leviathan
    et al. with q_i the point mass, measured exactly over the uniforms."""
    rng = np.random.default_rng(seed)
    target = 1.5 * rng.standard_normal((k + 1, V))
    p = [special.softmax(target[i]) for i in range(k + 1)]
    for x in itertools.product(range(V), repeat=k):
        taus = []
        for i in range(k):
            def acc_at(u, i=i):
                ua = [0.0] * k
                ua[i] = u
                return _run_one_hot(target, list(x), ua, 0.5)[0] > i
            taus.append(_threshold(acc_at))
        np.testing.assert_allclose(taus, [p[i][x[i]] for i in range(k)], rtol=0, atol=1e-12)
        dist = defaultdict(float)
        for a in range(k + 1):
            pa = float(np.prod(taus[:a])) * ((1.0 - taus[a]) if a < k else 1.0)
            if pa <= 0.0:
                continue
            ua = [t * 0.5 for t in taus[:a]] + \
                 ([0.5 * (1.0 + taus[a])] if a < k else []) + [0.0] * (k - a - 1)
            meas = _step_measure(lambda u: _run_one_hot(target, list(x), ua, u)[1])
            for tokens, m in meas.items():
                dist[tokens] += pa * m
        reach = 1.0
        for i in range(k + 1):
            marg = np.zeros(V)
            for tokens, m in dist.items():
                if len(tokens) > i:
                    marg[tokens[i]] += m
            np.testing.assert_allclose(marg.sum(), reach, rtol=0, atol=1e-9)
            np.testing.assert_allclose(marg / marg.sum(), p[i], rtol=0, atol=1e-9)
            if i < k:
                reach *= p[i][x[i]]


def test_one_hot_equals_point_mass_draft_logits():
    """draft_logits = None is the general path with draft rows that are
    -inf everywhere but the draft token."""
    rng = np.random.default_rng(8)
    V, B = 7, 12
    T = rng.integers(1, 5, B)
    cu = np.concatenate([[0], np.cumsum(T)])
    target = 2.0 * rng.standard_normal((cu[-1], V))
    nd = cu[-1] - B
    drafts = rng.integers(0, V, nd)
    point = np.full((nd, V), NEG)
    point[np.arange(nd), drafts] = 0.0
    for trial in range(20):
        ua, uf = rng.random(nd), rng.random(B)
        a1, o1 = oracle.rejection_accept(target, None, drafts, ua, uf, cu, 5)
        a2, o2 = oracle.rejection_accept(target, point, drafts, ua, uf, cu, 5)
        np.testing.assert_array_equal(a1, a2)
        np.testing.assert_array_equal(o1, o2)


@pytest.mark.parametrize("mode", ['greedy', 'rejection'])
def test_supplied_bonus_replaces_only_the_bonus(mode):
    rng = np.random.default_rng(9)
    V, B, k = 9, 30, 2
    cu = np.arange(B + 1) * (k + 1)
    target = 2.0 * rng.standard_normal((cu[-1], V))
    if mode == 'greedy':
        g = target.argmax(axis=1)
        drafts = np.array([g[cu[b] + i] if rng.random() < 0.8 else (g[cu[b] + i] + 1) % V
                           for b in range(B) for i in range(k)])
    else:
        drafts = rng.integers(0, V, B * k)
    draft = 2.0 * rng.standard_normal((B * k, V))
    ua, uf = 0.5 * rng.random(B * k), rng.random(B)
    bonus = rng.integers(0, V, B)
    if mode == 'greedy':
        a0, o0 = oracle.greedy_accept(target, drafts, cu, k + 1)
        a1, o1 = oracle.greedy_accept(target, drafts, cu, k + 1, bonus_tokens=bonus)
    else:
        a0, o0 = oracle.rejection_accept(target, draft, drafts, ua, uf, cu, k + 1)
        a1, o1 = oracle.rejection_accept(target, draft, drafts, ua, uf, cu, k + 1,
                                         bonus_tokens=bonus)
    np.testing.assert_array_equal(a0, a1)
    full = a0 == k
    assert full.any() and (~full).any()
    np.testing.assert_array_equal(o1[full, k], bonus[full])
    np.testing.assert_array_equal(o1[~full], o0[~full])
    np.testing.assert_array_equal(o1[:, :k], o0[:, :k])
