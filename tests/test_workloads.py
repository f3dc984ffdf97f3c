"""Host-side checks of the seeded input generators (no GPU)."""

import numpy as np
import torch

import oracle
import workloads as wl


def test_batch_block_table_is_a_valid_injective_map():
    for i, w in enumerate(wl.WORKLOADS):
        if w.name == 'stress_ragged_long':
            continue            # large pool; covered by the smaller variant below
        b = wl.make_batch(w, seed=i)
        cu = b.cu_seqlens.tolist()
        assert cu[0] == 0 and all(cu[j + 1] - cu[j] == b.T[j] for j in range(b.B))
        assert max(b.T) <= b.max_T
        used = []
        for s in range(b.B):
            need = -(-(b.ctx[s] + b.T[s]) // b.P)
            row = b.block_table[s].tolist()
            assert all(0 <= p < b.num_pages for p in row[:need])
            assert all(p == -1 for p in row[need:])
            used += row[:need]
        assert len(used) == len(set(used))


def test_stress_shape_is_ragged_and_fragmented():
    w = wl.WORKLOADS[4]
    small = wl.Workload(**{**w.__dict__, 'B': 64, 'ctx': (100, 300)})
    b = wl.make_batch(small, seed=4)
    assert min(b.T) >= 2 and max(b.T) <= 8 and len(set(b.T)) > 3
    need = sum(-(-(L + t) // b.P) for L, t in zip(b.ctx, b.T))
    assert b.num_pages >= 1.2 * need


def test_generators_are_deterministic():
    w = wl.WORKLOADS[0]
    b1, b2 = wl.make_batch(w, 0), wl.make_batch(w, 0)
    assert torch.equal(b1.block_table, b2.block_table)
    g1, g2 = wl.make_gdn_layer(w, b1, 5), wl.make_gdn_layer(w, b2, 5)
    for key in g1:
        assert torch.equal(g1[key], g2[key])
    a1 = wl.make_accept(w, b1, 9, 'rejection')
    a2 = wl.make_accept(w, b2, 9, 'rejection')
    for key in a1:
        assert torch.equal(a1[key], a2[key])


def test_gdn_inputs_follow_recipe():
    w = wl.WORKLOADS[2]
    b = wl.make_batch(w, 2)
    g = wl.make_gdn_layer(w, b, 3)
    assert g['state'].dtype == torch.float32 and g['q'].dtype == torch.bfloat16
    n = g['k'].float().norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-2)
    assert 0.8 < g['alpha'].mean() < 0.9 and 0.4 < g['beta'].mean() < 0.6
    assert abs(g['state'].std().item() - 0.1) < 1e-3
    c = wl.make_commit_len(b, 7)
    assert c.min() >= 1 and c.max() <= 4


def test_greedy_drafts_hit_about_seventy_percent():
    w = wl.WORKLOADS[0]
    w = wl.Workload(**{**w.__dict__, 'B': 200, 'ctx_fixed': None, 'ctx': (1, 2)})
    b = wl.make_batch(w, 1)
    a = wl.make_accept(w, b, 2, 'greedy')
    acc, _ = oracle.greedy_accept(a['target_logits'].double().numpy(),
                                  a['draft_tokens'].numpy(), b.cu_seqlens.numpy(), b.max_T)
    # leading-run mean for p = 0.7, k = 3 is 0.7 + 0.49 + 0.343 = 1.533
    assert 1.3 < acc.mean() < 1.75


def test_rejection_drafts_accept_about_seventy_percent():
    w = wl.WORKLOADS[0]
    w = wl.Workload(**{**w.__dict__, 'B': 100, 'ctx_fixed': None, 'ctx': (1, 2)})
    b = wl.make_batch(w, 1)
    a = wl.make_accept(w, b, 3, 'rejection')
    acc, _ = oracle.rejection_accept(a['target_logits'].double().numpy(),
                                     a['draft_logits'].double().numpy(),
                                     a['draft_tokens'].numpy(), a['u_accept'].numpy(),
                                     a['u_final'].numpy(), b.cu_seqlens.numpy(), b.max_T)
    assert 1.1 < acc.mean() < 1.9
