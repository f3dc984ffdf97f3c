"""Pins of the whole-step oracle.

A toy hybrid decoder (one attention layer over a paged KV cache, one GDN
layer with a short causal convolution beside it, a linear read-out) is
decoded twice with the oracle:

* plainly, one token per step (a step with no drafts);
* speculatively, k greedy drafts from a cheap bigram drafter per step,
  verified in one step that commits ``accept_len + 1`` tokens.

Greedy speculative decoding must emit exactly the plain greedy tokens, and
after the same number of tokens both runs must hold the same recurrent and
convolution states and the same cached K/V for every committed position.  This pins the
bookkeeping of the step (commit length, context growth, "undo equals never
applied" for the state, idempotent KV append) against plain decoding, which
shares none of it.
"""

import numpy as np

import oracle
from oracle import GDN_VERIFY_ONLY


class ToyModel:
    def __init__(self, seed=0, V=24, dm=16, Hq=2, Hkv=1, D=8, H=2, dk=8, dv=8, C=6, K=3):
        r = np.random.default_rng(seed)
        self.C, self.K = C, K
        self.V, self.Hq, self.Hkv, self.D, self.H, self.dk, self.dv = V, Hq, Hkv, D, H, dk, dv
        self.E = r.standard_normal((V, dm))
        self.Wq = r.standard_normal((dm, Hq * D)) / 4
        self.Wk = r.standard_normal((dm, Hkv * D)) / 4
        self.Wv = r.standard_normal((dm, Hkv * D))
        self.Gq = r.standard_normal((dm, H * dk))
        self.Gk = r.standard_normal((dm, H * dk))
        self.Gv = r.standard_normal((dm, H * dv))
        self.ga = r.standard_normal((dm, H))
        self.gb = r.standard_normal((dm, H))
        self.Wc = r.standard_normal((dm, C))
        self.conv_w = r.standard_normal((C, K)) / np.sqrt(K)
        self.conv_b = r.standard_normal(C) * 0.1
        self.Wo = r.standard_normal((Hq * D + H * dv + C, V)) * 2
        self.draft_table = r.standard_normal((V, V))

    def layer_inputs(self, tokens):
        x = self.E[np.asarray(tokens)]
        n = len(tokens)
        nrm = lambda a: a / np.linalg.norm(a, axis=-1, keepdims=True)
        return {
            'q': (x @ self.Wq).reshape(n, self.Hq, self.D),
            'k_new': (x @ self.Wk).reshape(n, self.Hkv, self.D),
            'v_new': (x @ self.Wv).reshape(n, self.Hkv, self.D),
            'gq': nrm((x @ self.Gq).reshape(n, self.H, self.dk)),
            'gk': nrm((x @ self.Gk).reshape(n, self.H, self.dk)),
            'gv': (x @ self.Gv).reshape(n, self.H, self.dv),
            'alpha': 0.8 + 0.2 / (1 + np.exp(-(x @ self.ga))),
            'beta': 1 / (1 + np.exp(-(x @ self.gb))),
            'cx': x @ self.Wc,
        }

    def conv(self, state, cx):
        return {'state': state, 'x': cx, 'weight': self.conv_w, 'bias': self.conv_b,
                'silu': True}

    def logits(self, attn_o, gdn_o, conv_o):
        n = attn_o.shape[0]
        return np.concatenate([attn_o.reshape(n, -1), gdn_o.reshape(n, -1), conv_o], 1) @ self.Wo


def _decode(model, n_out, k, P=4, max_pages=32):
    """Decode n_out tokens with k drafts per step (k = 0: plain decoding)."""
    rng = np.random.default_rng(1)
    num_pages = max_pages
    table = rng.permutation(num_pages)[None, :]
    kc = np.zeros((num_pages, model.Hkv, P, model.D))
    vc = np.zeros_like(kc)
    state = np.zeros((1, model.H, model.dv, model.dk))
    cstate = np.zeros((1, model.K - 1, model.C))
    ctx = np.array([0])
    tokens = [3]
    while len(tokens) < n_out:
        drafts = []
        last = tokens[-1]
        for _ in range(k):
            last = int(np.argmax(model.draft_table[last]))
            drafts.append(last)
        verify = [tokens[-1]] + drafts
        cu = np.array([0, len(verify)])
        li = model.layer_inputs(verify)
        attn_o = oracle.verify_attention(li['q'], li['k_new'], li['v_new'], kc, vc,
                                         table, ctx, cu, P)
        gdn_o, _ = oracle.gdn_step(state, None, li['gq'], li['gk'], li['gv'],
                                   li['alpha'], li['beta'], cu, None, GDN_VERIFY_ONLY)
        conv_o, _ = oracle.conv_step(cstate, None, li['cx'], model.conv_w, model.conv_b, cu,
                                     None, oracle.CONV_VERIFY_ONLY, silu=True)
        logits = model.logits(attn_o, gdn_o, conv_o)
        layers = [
            {'kind': 'attn', 'q': li['q'], 'k_new': li['k_new'], 'v_new': li['v_new'],
             'k_cache': kc, 'v_cache': vc},
            {'kind': 'gdn', 'state': state, 'q': li['gq'], 'k': li['gk'], 'v': li['gv'],
             'alpha': li['alpha'], 'beta': li['beta'], 'conv': model.conv(cstate, li['cx'])},
        ]
        res = oracle.verify_step(layers, cu, ctx, table, P, k + 1, 'greedy',
                                 {'target_logits': logits,
                                  'draft_tokens': np.array(drafts, dtype=np.int64)})
        a = int(res['accept_len'][0])
        assert res['commit_len'][0] == a + 1
        assert res['ctx_lens'][0] == ctx[0] + a + 1
        tokens.extend(int(t) for t in res['out_tokens'][0, :a + 1])
        kc, vc = res['k_cache'][0], res['v_cache'][0]
        state = res['state'][1]
        np.testing.assert_array_equal(res['conv_outputs'][1], conv_o)
        cstate = res['conv_state'][1]
        ctx = res['ctx_lens']
    return tokens, kc, vc, (state, cstate), int(ctx[0]), table


def test_toy_hybrid_speculative_decoding_is_lossless():
    model = ToyModel()
    for k in (1, 3, 5):
        spec, kc1, vc1, st1, ctx1, table = _decode(model, 60, k=k)
        # plain decoding adds one token per step, so it stops at exactly the
        # speculative run's length; both have then processed tokens[:-1]
        plain, kc0, vc0, st0, ctx0, _ = _decode(model, len(spec), k=0)
        assert spec == plain
        assert ctx0 == ctx1 == len(spec) - 1
        np.testing.assert_allclose(st1[0], st0[0], rtol=0, atol=1e-12)
        # the convolution state holds copies of the last K-1 committed inputs
        np.testing.assert_allclose(st1[1], st0[1], rtol=0, atol=1e-12)
        # The toy projections are matmuls over 1 or k+1 rows, which BLAS may
        # round differently, so cached rows agree to float64 rounding.
        for pos in range(ctx0):
            page, slot = table[0, pos // 4], pos % 4
            np.testing.assert_allclose(kc1[page, :, slot], kc0[page, :, slot],
                                       rtol=0, atol=1e-13)
            np.testing.assert_allclose(vc1[page, :, slot], vc0[page, :, slot],
                                       rtol=0, atol=1e-13)


def test_step_outputs_and_bookkeeping():
    rng = np.random.default_rng(3)
    model = ToyModel(seed=4)
    P, num_pages = 4, 40
    B = 3
    T = [4, 2, 5]
    cu = np.concatenate([[0], np.cumsum(T)])
    ctx = np.array([5, 0, 9])
    table = rng.permutation(num_pages)[:B * 6].reshape(B, 6)
    kc = rng.standard_normal((num_pages, 1, P, 8))
    vc = rng.standard_normal((num_pages, 1, P, 8))
    state = rng.standard_normal((B, 2, 8, 8)) * 0.1
    tokens = rng.integers(0, model.V, cu[-1])
    li = model.layer_inputs(tokens)
    drafts = rng.integers(0, model.V, cu[-1] - B)
    logits = rng.standard_normal((cu[-1], model.V))
    layers = [
        {'kind': 'attn', 'q': li['q'], 'k_new': li['k_new'], 'v_new': li['v_new'],
         'k_cache': kc, 'v_cache': vc},
        {'kind': 'gdn', 'state': state, 'q': li['gq'], 'k': li['gk'], 'v': li['gv'],
         'alpha': li['alpha'], 'beta': li['beta']},
    ]
    res = oracle.verify_step(layers, cu, ctx, table, P, 5, 'greedy',
                             {'target_logits': logits, 'draft_tokens': drafts})
    acc, out = oracle.greedy_accept(logits, drafts, cu, 5)
    np.testing.assert_array_equal(res['accept_len'], acc)
    np.testing.assert_array_equal(res['out_tokens'], out)
    np.testing.assert_array_equal(res['commit_len'], acc + 1)
    np.testing.assert_array_equal(res['ctx_lens'], ctx + acc + 1)
    _, S = oracle.gdn_step(state, None, li['gq'], li['gk'], li['gv'], li['alpha'],
                           li['beta'], cu, acc + 1, oracle.GDN_VERIFY_COMMIT)
    np.testing.assert_array_equal(res['state'][1], S)
    assert res['state'][0] is None and res['k_cache'][1] is None
