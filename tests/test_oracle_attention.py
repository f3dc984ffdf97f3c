"""Pins of the attention oracle against things other than itself.

* a dense causal reference computed by torch's scaled_dot_product_attention
  (float64, CPU, explicit boolean mask) on per-sequence K/V that the test
  scatters into the paged pool itself;
* closed forms: a single visible key returns its value; equal keys return
  the mean of the visible values; distinct constant value heads expose the
  GQA grouping;
* invariants: a random physical page permutation (with the matching block
  table) changes nothing;
* brute force on the append: every slot of a pool of unique values is
  checked, including in-flight runs that straddle a page boundary.
"""

import numpy as np
import pytest
import torch

import oracle


def _scatter(dense_list, table, page_size, num_pages, Hkv, D):
    """Write dense per-sequence [L, Hkv, D] arrays into a pool, page by page."""
    pool = np.random.default_rng(99).standard_normal((num_pages, Hkv, page_size, D))
    for b, dense in enumerate(dense_list):
        L = dense.shape[0]
        for pi in range(-(-L // page_size)):
            lo, hi = pi * page_size, min(L, (pi + 1) * page_size)
            for s in range(lo, hi):
                pool[table[b][pi], :, s - lo, :] = dense[s]
    return pool


def _case(rng, ctx, T, page_size, Hq, Hkv, D, spare_pages=3):
    B = len(ctx)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    need = [-(-(L + t) // page_size) for L, t in zip(ctx, T)]
    num_pages = sum(need) + spare_pages
    perm = rng.permutation(num_pages)
    table = np.full((B, max(need) + 1), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    dk = [rng.standard_normal((L, Hkv, D)) for L in ctx]
    dvv = [rng.standard_normal((L, Hkv, D)) for L in ctx]
    kc = _scatter(dk, table, page_size, num_pages, Hkv, D)
    vc = _scatter(dvv, table, page_size, num_pages, Hkv, D)
    q = rng.standard_normal((cu[-1], Hq, D))
    kn = rng.standard_normal((cu[-1], Hkv, D))
    vn = rng.standard_normal((cu[-1], Hkv, D))
    return dict(ctx=np.array(ctx), T=T, cu=cu, table=table, kc=kc, vc=vc,
                q=q, kn=kn, vn=vn, dense_k=dk, dense_v=dvv,
                num_pages=num_pages)


def _sdpa_reference(c, Hq, Hkv, D, scale):
    out = np.zeros_like(c['q'])
    G = Hq // Hkv
    for b, (L, T) in enumerate(zip(c['ctx'], c['T'])):
        s0 = c['cu'][b]
        K = np.concatenate([c['dense_k'][b], c['kn'][s0:s0 + T]])   # [L+T, Hkv, D]
        V = np.concatenate([c['dense_v'][b], c['vn'][s0:s0 + T]])
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Qt = torch.from_numpy(c['q'][s0:s0 + T]).permute(1, 0, 2)   # [Hq, T, D]
        # query j sees keys 0 .. L + j
        mask = torch.arange(L + T)[None, :] <= (L + torch.arange(T))[:, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            Qt, Kt, Vt, attn_mask=mask, scale=scale)
        out[s0:s0 + T] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("seed,ctx,T,P,Hq,Hkv,D", [
    (0, [37, 50], [4, 4], 16, 4, 2, 64),
    (1, [0, 1, 15, 16, 17], [1, 2, 3, 4, 8], 16, 8, 2, 32),
    (2, [14, 15, 30, 31, 63], [4, 4, 4, 4, 1], 16, 4, 4, 16),
    (3, [5, 9], [8, 5], 4, 6, 3, 8),
    (4, [100, 3, 64], [1, 1, 1], 32, 4, 1, 16),           # T = 1: decode
])
def test_attention_matches_sdpa(seed, ctx, T, P, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    c = _case(rng, ctx, T, P, Hq, Hkv, D)
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                  c['table'], c['ctx'], c['cu'], P)
    ref = _sdpa_reference(c, Hq, Hkv, D, 1.0 / np.sqrt(D))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_attention_explicit_scale():
    rng = np.random.default_rng(5)
    c = _case(rng, [20, 7], [3, 2], 8, 4, 2, 16)
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                  c['table'], c['ctx'], c['cu'], 8, scale=0.3)
    ref = _sdpa_reference(c, 4, 2, 16, 0.3)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_single_visible_key_returns_its_value():
    # Empty context: in-flight token 0 sees only itself.
    rng = np.random.default_rng(6)
    c = _case(rng, [0, 0], [3, 1], 4, 4, 2, 8)
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                  c['table'], c['ctx'], c['cu'], 4)
    for b in range(2):
        row = c['cu'][b]
        for h in range(4):
            np.testing.assert_array_equal(got[row, h], c['vn'][row, h // 2])


def test_equal_keys_give_mean_of_visible_values():
    rng = np.random.default_rng(7)
    c = _case(rng, [9, 13], [4, 2], 4, 2, 1, 8)
    key = rng.standard_normal(8)
    c['kc'][:] = key
    c['kn'][:] = key
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                  c['table'], c['ctx'], c['cu'], 4)
    for b, (L, T) in enumerate(zip(c['ctx'], c['T'])):
        s0 = c['cu'][b]
        for j in range(T):
            vis = np.concatenate([c['dense_v'][b], c['vn'][s0:s0 + j + 1]])
            for h in range(2):
                np.testing.assert_allclose(got[s0 + j, h], vis[:, 0].mean(0),
                                           rtol=0, atol=1e-13)


def test_gqa_grouping_is_contiguous():
    # Value head g holds the constant g, so o[h] = g(h) = h * Hkv // Hq.
    rng = np.random.default_rng(8)
    Hq, Hkv = 8, 4
    c = _case(rng, [10, 3], [2, 4], 4, Hq, Hkv, 4)
    for g in range(Hkv):
        c['vc'][:, g] = g
        c['vn'][:, g] = g
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                  c['table'], c['ctx'], c['cu'], 4)
    for h in range(Hq):
        np.testing.assert_allclose(got[:, h], h // (Hq // Hkv), atol=1e-13)


def test_physical_page_permutation_invariance():
    rng = np.random.default_rng(9)
    c = _case(rng, [33, 70, 5], [4, 3, 2], 16, 4, 2, 16, spare_pages=5)
    base = oracle.verify_attention(c['q'], c['kn'], c['vn'], c['kc'], c['vc'],
                                   c['table'], c['ctx'], c['cu'], 16)
    perm = rng.permutation(c['num_pages'])          # new id of old page
    kc2 = np.empty_like(c['kc'])
    vc2 = np.empty_like(c['vc'])
    kc2[perm] = c['kc']
    vc2[perm] = c['vc']
    table2 = np.where(c['table'] >= 0, perm[np.maximum(c['table'], 0)], -1)
    got = oracle.verify_attention(c['q'], c['kn'], c['vn'], kc2, vc2, table2,
                                  c['ctx'], c['cu'], 16)
    np.testing.assert_array_equal(got, base)


@pytest.mark.parametrize("P,ctx,T", [
    (16, [14, 15, 16, 0, 31], [4, 4, 4, 4, 1]),      # straddles, exact fit
    (4, [2, 3, 7], [8, 1, 5]),
])
def test_append_slots_brute_force(P, ctx, T):
    rng = np.random.default_rng(10)
    Hkv, D = 2, 3
    c = _case(rng, ctx, T, P, 2, Hkv, D)
    # unique pool values: encode (page, head, slot, d)
    shape = c['kc'].shape
    kc = np.arange(np.prod(shape), dtype=np.float64).reshape(shape)
    vc = -kc
    kn = 1e9 + np.arange(np.prod(c['kn'].shape), dtype=np.float64).reshape(c['kn'].shape)
    vn = -kn
    k2, v2 = oracle.append_kv(kc, vc, kn, vn, c['table'], c['ctx'], c['cu'], P)
    expected_written = {}
    for b, (L, t) in enumerate(zip(ctx, T)):
        for j in range(t):
            pos = L + j
            expected_written[(int(c['table'][b, pos // P]), pos % P)] = c['cu'][b] + j
    for page in range(shape[0]):
        for slot in range(P):
            key = (page, slot)
            if key in expected_written:
                row = expected_written[key]
                np.testing.assert_array_equal(k2[page, :, slot], kn[row])
                np.testing.assert_array_equal(v2[page, :, slot], vn[row])
            else:
                np.testing.assert_array_equal(k2[page, :, slot], kc[page, :, slot])
                np.testing.assert_array_equal(v2[page, :, slot], vc[page, :, slot])
    # inputs are not modified
    np.testing.assert_array_equal(kc, np.arange(np.prod(shape)).reshape(shape))


def test_gather_reads_back_scattered_context():
    rng = np.random.default_rng(11)
    c = _case(rng, [45, 16, 1], [1, 1, 1], 16, 2, 2, 4)
    for b, L in enumerate(c['ctx']):
        np.testing.assert_array_equal(
            oracle.gather_context(c['kc'], c['table'][b], L, 16), c['dense_k'][b])
