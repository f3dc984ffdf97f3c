"""Edge cases of the whole step on the GPU, against the oracle.

* sequences with no draft (T_b = 1): only the bonus / argmax token is
  emitted, commit 1, in batches that mix them with the longest chains
  (k_b = 7, T_b = 8), and batches with no draft at all;
* a single sequence;
* empty contexts (L_b = 0) next to long ones.
Same tolerances as the per-op tests; integers bit-exact.
"""

import pytest
import torch

import workloads as wl
from block_draft_verification_spec_amd import binding as bd
from gpu_helpers import DEV, say
from test_gpu_step import compare, make_step, oracle_step, run_step

pytestmark = pytest.mark.gpu


def _fresh(layers):
    for l in layers:
        if l['kind'] == 'attn':
            l['k_cache'] = l['k_cache'].clone()
            l['v_cache'] = l['v_cache'].clone()
        else:
            l['state'] = l['state'].clone()


def _run_case(w, batch, seed, mode):
    layers, acc = make_step(w, batch, seed, 'greedy' if mode == 0 else 'rejection')
    ref = oracle_step(w, batch, layers, acc, mode)
    before = [(l.get('k_cache'), l.get('v_cache')) for l in layers]
    _fresh(layers)
    res = run_step(w, batch, layers, acc, mode)
    compare(w, layers, res, ref, before)
    return res


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
@pytest.mark.parametrize("ks", [[0, 3], [0, 0], [0]])
def test_tiny_fp32_without_drafts(mode, ks):
    w = wl.WORKLOADS[0]
    w = wl.Workload(**{**w.__dict__, 'B': len(ks)})
    batch = wl.make_batch(w, 5, DEV, k_override=ks, ctx_override=list(w.ctx_fixed)[:len(ks)])
    say('edge tiny fp32 ks', ks, 'mode', mode)
    res = _run_case(w, batch, 6, mode)
    for b, k in enumerate(ks):
        if k == 0:
            assert res['acc'][b] == 0 and res['out'][b][0] >= 0
            assert int(res['commit'][b]) == 1


@pytest.mark.parametrize("mode", [bd.SV_ACCEPT_GREEDY, bd.SV_ACCEPT_REJECTION])
def test_hybrid_bf16_mixed_chain_lengths(mode):
    """bf16 hybrid group (3 GDN + 1 attention layers, the full head shapes),
    eight sequences with k_b in {0 .. 7} and contexts from empty to long."""
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 8, 'layers': wl._hybrid(1)})
    ks = [0, 7, 1, 0, 5, 7, 2, 3]
    batch = wl.make_batch(w, 9, DEV, k_override=ks,
                          ctx_override=[0, 1, 63, 64, 5000, 0, 129, 8191])
    say('edge hybrid mixed ks', ks, 'mode', mode)
    _run_case(w, batch, 10, mode)


def test_single_sequence():
    w = wl.WORKLOADS[3]
    w = wl.Workload(**{**w.__dict__, 'B': 1, 'layers': wl._hybrid(1)})
    batch = wl.make_batch(w, 11, DEV, k_override=[3], ctx_override=[777])
    _run_case(w, batch, 12, bd.SV_ACCEPT_REJECTION)
