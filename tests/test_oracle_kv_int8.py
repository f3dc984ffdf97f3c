"""Pins of the INT8-KV oracle against things other than itself.

* codes on the grid: x = s * n (s a power of two, so x and x / s are exact in
  fp32) gives back n for every n in [-127, 127], with a different scale on
  every (head, channel) so a transposed or misbroadcast scale fails;
* ties: (n + 1/2) s rounds to the even neighbour; saturation at +-127
  (never -128);
* bound: |s code - x| <= s / 2 inside the range, up to the fp32 quotient's
  rounding (random x, random scales);
* dequantization of a pool against an explicit loop over every element;
* attention: with K/V on the grid the INT8 attention equals torch's
  scaled_dot_product_attention (float64, explicit mask) on the float values;
* the in-flight rows enter as their codes: each verify token's output equals
  a one-token call that reads the earlier in-flight positions back from the
  appended INT8 pages.
"""

import numpy as np
import pytest
import torch

import oracle.kv_int8 as kv8

RNG = np.random.default_rng(4321)


def _pow2_scales(Hkv, D):
    return np.ldexp(1.0, RNG.integers(-9, -2, size=(Hkv, D))).astype(np.float32)


def test_grid_round_trip_per_channel():
    Hkv, D = 3, 10
    s = _pow2_scales(Hkv, D)
    n = np.arange(-127, 128)
    x = n[:, None, None] * s[None].astype(np.float64)          # [255, Hkv, D], exact
    codes = kv8.quantize_int8(x, s)
    assert codes.dtype == np.int8
    np.testing.assert_array_equal(codes, np.broadcast_to(n[:, None, None], codes.shape))
    np.testing.assert_array_equal(kv8.dequantize_rows(codes, s), x)


def test_ties_to_even_and_saturation():
    s = np.full((1, 4), 0.25, dtype=np.float32)
    x = np.array([[[0.5 * 0.25, 1.5 * 0.25, 2.5 * 0.25, -0.5 * 0.25]],
                  [[-1.5 * 0.25, -2.5 * 0.25, 126.5 * 0.25, -126.5 * 0.25]],
                  [[1000.0, -1000.0, 127.49 * 0.25, -127.51 * 0.25]]])
    codes = kv8.quantize_int8(x, s)
    np.testing.assert_array_equal(codes[0, 0], [0, 2, 2, 0])
    np.testing.assert_array_equal(codes[1, 0], [-2, -2, 126, -126])
    np.testing.assert_array_equal(codes[2, 0], [127, -127, 127, -127])
    assert codes.min() >= -127


def test_error_bound_inside_range():
    Hkv, D = 4, 16
    s = (RNG.uniform(0.5, 1.5, size=(Hkv, D)) * 4.0 / 127).astype(np.float32)
    x = RNG.uniform(-1, 1, size=(500, Hkv, D)) * (127 * s.astype(np.float64))
    x = x.astype(np.float32).astype(np.float64)
    err = np.abs(kv8.dequantize_rows(kv8.quantize_int8(x, s), s) - x)
    # half a step, plus the fp32 quotient's rounding (|x / s| <= 127, so at
    # most 127 * 2^-24 of a step) that can move a near-tie across
    assert np.all(err <= (0.5 + 2.0 ** -16) * s.astype(np.float64))


def test_dequantize_pool_elementwise():
    npg, Hkv, P, D = 3, 2, 4, 5
    codes = RNG.integers(-127, 128, size=(npg, Hkv, P, D)).astype(np.int8)
    s = RNG.uniform(0.01, 0.1, size=(Hkv, D))
    got = kv8.dequantize_pool(codes, s)
    for a in range(npg):
        for h in range(Hkv):
            for p in range(P):
                for d in range(D):
                    assert got[a, h, p, d] == float(codes[a, h, p, d]) * s[h, d]


def _grid_case(ctx, T, P, Hq, Hkv, D):
    """Pools and in-flight rows whose values lie on the per-channel grid."""
    B = len(ctx)
    cu = np.concatenate([[0], np.cumsum(T)]).astype(np.int64)
    need = [-(-(L + t) // P) for L, t in zip(ctx, T)]
    num_pages = sum(need) + 2
    perm = RNG.permutation(num_pages)
    table = np.full((B, max(need) + 1), -1, dtype=np.int64)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
    ks, vs = _pow2_scales(Hkv, D), _pow2_scales(Hkv, D)
    kc = RNG.integers(-127, 128, size=(num_pages, Hkv, P, D)).astype(np.int8)
    vc = RNG.integers(-127, 128, size=(num_pages, Hkv, P, D)).astype(np.int8)
    kn_codes = RNG.integers(-127, 128, size=(cu[-1], Hkv, D))
    vn_codes = RNG.integers(-127, 128, size=(cu[-1], Hkv, D))
    q = RNG.standard_normal((cu[-1], Hq, D))
    return dict(cu=cu, table=table, ks=ks, vs=vs, kc=kc, vc=vc, q=q,
                kn=kn_codes * ks.astype(np.float64), vn=vn_codes * vs.astype(np.float64),
                ctx=np.array(ctx), T=T)


def test_grid_attention_matches_sdpa():
    Hq, Hkv, D, P = 4, 2, 8, 4
    c = _grid_case([5, 0, 9], [2, 3, 1], P, Hq, Hkv, D)
    o = kv8.verify_attention_int8(c['q'], c['kn'], c['vn'], c['kc'], c['vc'], c['ks'], c['vs'],
                                  c['table'], c['ctx'], c['cu'], P)
    G = Hq // Hkv
    for b, (L, T) in enumerate(zip(c['ctx'], c['T'])):
        pos = np.arange(L)
        pages, slots = c['table'][b][pos // P], pos % P
        Kd = np.concatenate([c['kc'][pages, :, slots, :] * c['ks'].astype(np.float64),
                             c['kn'][c['cu'][b]:c['cu'][b] + T]], axis=0)
        Vd = np.concatenate([c['vc'][pages, :, slots, :] * c['vs'].astype(np.float64),
                             c['vn'][c['cu'][b]:c['cu'][b] + T]], axis=0)
        n = L + T
        mask = np.zeros((T, n), dtype=bool)
        for j in range(T):
            mask[j, :L + j + 1] = True
        for h in range(Hq):
            g = h // G
            qh = torch.from_numpy(c['q'][c['cu'][b]:c['cu'][b] + T, h][None, None].copy())
            ref = torch.nn.functional.scaled_dot_product_attention(
                qh, torch.from_numpy(Kd[:, g][None, None].copy()),
                torch.from_numpy(Vd[:, g][None, None].copy()),
                attn_mask=torch.from_numpy(mask)[None, None])[0, 0].numpy()
            np.testing.assert_allclose(o[c['cu'][b]:c['cu'][b] + T, h], ref,
                                       rtol=1e-12, atol=1e-12)


def test_in_flight_rows_read_back_from_pages():
    Hq, Hkv, D, P = 2, 1, 8, 4
    ctx, T = [3, 6], [4, 3]
    c = _grid_case(ctx, T, P, Hq, Hkv, D)
    # off-grid in-flight rows: their codes differ from the raw values
    kn = RNG.standard_normal(c['kn'].shape) * 0.01
    vn = RNG.standard_normal(c['vn'].shape) * 0.01
    o = kv8.verify_attention_int8(c['q'], kn, vn, c['kc'], c['vc'], c['ks'], c['vs'],
                                  c['table'], c['ctx'], c['cu'], P)
    k2, v2 = kv8.append_kv_int8(c['kc'], c['vc'], kn, vn, c['ks'], c['vs'], c['table'],
                                c['ctx'], c['cu'], P)
    assert k2.dtype == np.int8
    for b in range(len(ctx)):
        for j in range(T[b]):
            r = c['cu'][b] + j
            one = kv8.verify_attention_int8(c['q'][r:r + 1], kn[r:r + 1], vn[r:r + 1], k2, v2,
                                            c['ks'], c['vs'], c['table'][b:b + 1],
                                            np.array([ctx[b] + j]), np.array([0, 1]), P)
            np.testing.assert_allclose(one[0], o[r], rtol=1e-12, atol=1e-14)
    # and the raw in-flight values would give a different answer
    raw = kv8.verify_attention(c['q'], kn, vn, kv8.dequantize_pool(c['kc'], c['ks']),
                               kv8.dequantize_pool(c['vc'], c['vs']), c['table'], c['ctx'],
                               c['cu'], P)
    assert not np.allclose(raw, o, rtol=0, atol=1e-9)


@pytest.mark.parametrize("bad", [0.0, np.inf])
def test_degenerate_scales_stay_in_range(bad):
    s = np.array([[bad, 0.5]], dtype=np.float32)
    codes = kv8.quantize_int8(np.array([[[1.0, -300.0]]]), s)
    assert codes.dtype == np.int8 and np.all(np.abs(codes.astype(int)) <= 127)
