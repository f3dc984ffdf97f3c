"""Benchmark of the block speculative-verification step on one MI355X.

Default workload (--workload 3, hybrid_step_64l): the full hybrid verify
step (64 layers, GDN,GDN,GDN,ATT x 16; B = 64 sequences, k = 3 drafts,
contexts ~U[2048, 8192], 32q/8kv heads, D = 128, bf16 paged KV in 64-token
pages; 48 GDN layers with 32 heads, dk = dv = 128, fp32 state; acceptance
over V = 151936 bf16 logits), synthetic seeded inputs resident in HBM before
timing starts.  --workload 0 / 4 run the tiny fp32 step and the 256-sequence
stress step the same way; --workload 1 / 2 time one paged-attention call /
one GDN verify+commit call per step, rotating over buffer sets of >= 1 GB in
total so the last-level cache cannot serve them.

A step = one call of spec_verify_step: every layer's verify pass, the
acceptance, the GDN commit (deferred schedule: folded into the next step's
verify pass; the timed region ends with a flush so every accepted token of
every timed step is committed) and the ctx_lens update.  The same steps are
also captured into HIP graphs and replayed (reported beside the eager
figures).

Prints one JSON line.  value = verified draft tokens per second (sum_b k_b
per step) over the timed steps; the per-step median, p10 and p90 come from
HIP events between the steps (for the single-call workloads 1 and 2, whose
calls last tens of microseconds, from a second pass: an event between calls
costs a few microseconds, so the timed pass records events only at its two
ends).  Also reported: algorithmic HBM bytes per step and GB/s (% of the
8 TB/s peak and of the copy / read rates measured in the same run), the
roofline of the dominant kernel (back-to-back launches between two HIP
events on the stream it runs on), and the CPU oracle timed on a bounded
sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ATTN_SOURCE = os.path.join(ROOT, 'block_draft_verification_spec_amd', 'csrc', 'attention.hip')
TRAFFIC_FILE = os.path.join(ROOT, 'profiles', 'attention_hybrid_step_64l_traffic.txt')


def parse():
    p = argparse.ArgumentParser()
    p.add_argument('--gpus', type=int, default=1)
    p.add_argument('--steps', type=int, default=20)
    p.add_argument('--warmup', type=int, default=5)
    p.add_argument('--workload', type=int, default=3, help='index into workloads.WORKLOADS')
    p.add_argument('--accept', choices=['rejection', 'greedy'], default='rejection')
    p.add_argument('--schedule', choices=['deferred', 'two_phase'], default='deferred')
    p.add_argument('--kv-format', choices=['bf16', 'int8'], default='bf16',
                   help='page format of the step\'s attention layers (int8: per-channel codes)')
    p.add_argument('--state-dtype', choices=['f32', 'f16'], default='f32',
                   help='storage of the step\'s GDN state bank')
    p.add_argument('--no-cpu-baseline', action='store_true')
    p.add_argument('--no-graph', action='store_true', help='skip the graph-replay timing')
    p.add_argument('--no-next-rows', action='store_true',
                   help='skip the side timings of the NEXT rows (hybrid step only)')
    p.add_argument('--attn-reps', type=int, default=3,
                   help='passes over the attention layers for the per-launch timing')
    p.add_argument('--seed', type=int, default=3)
    p.add_argument('--calibrate-copy', action='store_true',
                   help='only run a plain 1 GiB device copy (counter calibration)')
    p.add_argument('--cpu-budget', type=float, default=15.0,
                   help='seconds of oracle work for the CPU baseline sample')
    return p.parse_args()


def calibrate_copy():
    """A plain device-to-device copy of exactly 1 GiB, three times: the
    reference for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = 1 << 30
    x = torch.ones(n, dtype=torch.uint8, device='cuda')
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({'calibrate_copy_bytes': n, 'copies': 3}), flush=True)


def short_conv_timing(w, batch, sb, commit, stream, dev, reps=20):
    """One short-convolution layer of the linear-attention layers (C = the q,
    k and v features, K = 4, SiLU), deferred schedule: replay the previous
    step's accepted inputs, verify this step's.  Four independent layers are
    cycled so the timing is not an L2 replay."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    layers = [wl.make_conv_layer(w, batch, 3000 + i, dev) for i in range(4)]
    for c in layers:
        c['out'] = torch.empty_like(c['x'])
        c['pend'] = bd.make_conv_pending(sb, c['x'], commit)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)

    def run(c):
        bd.short_conv_verify_commit(sb, bd.SV_GDN_VERIFY_ONLY, c['state'], c['x'], c['weight'],
                                    c['bias'], None, c['out'], activation=bd.SV_ACT_SILU,
                                    pending=c['pend'], stream=stream)
    for c in layers:
        run(c)
    e0.record(stream)
    for _ in range(reps):
        for c in layers:
            run(c)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * len(layers))
    s, C, K, T, B = 2, w.conv_C, w.conv_K, batch.total_T, batch.B
    # state read + write, current inputs and outputs, the replayed (accepted)
    # pending inputs, taps and bias
    pend_rows = int(commit.sum().item())
    nbytes = 2 * B * (K - 1) * C * s + 2 * T * C * s + pend_rows * C * s + C * K * 4 + C * 4
    return {'layer_ms': round(ms, 4), 'bytes': nbytes,
            'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1), 'C': C, 'K': K,
            'schedule': 'deferred (pending replay + verify)'}


def gdn_state_dtype_timing(w, batch, sb, commit, stream, dev, reps=4):
    """One GDN layer, deferred schedule (replay the previous step's accepted
    tokens, verify this step's), with the state bank stored as fp32 and as
    fp16 (fp32 arithmetic either way).  Sixteen independent layers are
    cycled: their 2.1 GB of fp32 state is far beyond the last-level cache,
    as in the step."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    res = {}
    for name, sdt in (('fp32_state', torch.float32), ('fp16_state', torch.float16)):
        layers = [wl.make_gdn_layer(w, batch, 4000 + i, dev, state_dtype=sdt) for i in range(16)]
        for l in layers:
            l['out'] = torch.empty_like(l['v'])
            l['pend'] = bd.make_gdn_pending(sb, l['k'], l['v'], l['alpha'], l['beta'], commit)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)

        def run(l, s=stream):
            bd.gdn_verify_commit(sb, bd.SV_GDN_VERIFY_ONLY, l['state'], l['q'], l['k'], l['v'],
                                 l['alpha'], l['beta'], None, l['out'], pending=l['pend'],
                                 stream=s)
        for l in layers:
            run(l)
        e0.record(stream)
        for _ in range(reps):
            for l in layers:
                run(l)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * len(layers))
        gms = graph_block_ms(stream, [(lambda l=l: run(l, None)) for l in layers]) / len(layers)
        es = torch.finfo(sdt).bits // 8
        T = batch.total_T
        pend_rows = int(commit.sum().item())
        # state read + write, current q/k/v/gates/out, replayed k/v/gates
        nbytes = (2 * batch.B * w.H * w.dv * w.dk * es + T * w.H * (2 * w.dk + 2 * w.dv) * 2
                  + T * w.H * 8 + pend_rows * w.H * ((w.dk + w.dv) * 2 + 8))
        res[name] = {'layer_ms': round(ms, 4), 'bytes': nbytes,
                     'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1),
                     'layer_ms_graph': round(gms, 4),
                     'GBps_graph': round(nbytes / (gms * 1e-3) / 1e9, 1)}
        del layers
    res['schedule'] = 'deferred (pending replay + verify)'
    res['graph'] = 'the same sixteen calls replayed from a HIP graph'
    return res


def checkpoint_timing(w, batch, sb, commit, stream, dev, reps=10):
    """The checkpoint-series commit of the pages against the replay commit:
    per GDN layer (fp32 state) and per short-conv layer, the verify that
    writes the per-token series plus CommitPrefix of the accepted slot.  Four
    independent layers are cycled."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    W = batch.max_T
    T = batch.total_T
    kept = int((commit > 0).sum().item())
    res = {'window': W}

    def timed(layers, run):
        for l in layers:
            run(l)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            for l in layers:
                run(l)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * len(layers))

    gl = [wl.make_gdn_layer(w, batch, 6000 + i, dev) for i in range(4)]
    for l in gl:
        l['out'] = torch.empty_like(l['v'])
        l['ck'] = torch.empty((batch.B, W, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)

    def run_g(l):
        bd.gdn_verify_checkpoint(sb, l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                                 l['out'], l['ck'], stream=stream)
        bd.gdn_commit_prefix(sb, l['state'], l['ck'], commit, stream=stream)
    ms = timed(gl, run_g)
    tile = w.H * w.dv * w.dk * 4
    nbytes = (batch.B * tile + T * tile + 2 * kept * tile + T * w.H * (2 * w.dk + 2 * w.dv) * 2
              + T * w.H * 8)
    res['gdn_layer'] = {'layer_ms': round(ms, 4), 'bytes': nbytes,
                        'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del gl
    cl = [wl.make_conv_layer(w, batch, 7000 + i, dev) for i in range(4)]
    for c in cl:
        c['out'] = torch.empty_like(c['x'])
        c['ps'] = torch.empty((batch.B, W) + tuple(c['state'].shape[1:]), dtype=c['state'].dtype,
                              device=dev)

    def run_c(c):
        bd.short_conv_verify_checkpoint(sb, c['state'], c['x'], c['weight'], c['bias'], c['out'],
                                        c['ps'], activation=bd.SV_ACT_SILU, stream=stream)
        bd.short_conv_commit_prefix(sb, c['state'], c['ps'], commit, stream=stream)
    ms = timed(cl, run_c)
    row = (w.conv_K - 1) * w.conv_C * 2
    nbytes = (batch.B * row + T * row + 2 * kept * row + 2 * T * w.conv_C * 2
              + w.conv_C * (w.conv_K + 1) * 4)
    res['conv_layer'] = {'layer_ms': round(ms, 4), 'bytes': nbytes,
                         'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1)}
    del cl
    return res


def attn_kv8_bytes(w, batch, ctx=None):
    """Algorithmic HBM bytes of one attention layer over INT8 pages: the
    cached codes, the in-flight bf16 rows and their codes, Q, O, the scales
    and the block table (at the given contexts, default the batch's)."""
    ctx = sum(batch.ctx if ctx is None else ctx)
    T = batch.total_T
    per_tok = w.Hq * w.D * 2 + 2 * w.Hkv * w.D * 2 + 2 * w.Hkv * w.D + w.Hq * w.D * 2
    return (ctx * w.Hkv * w.D * 2 + T * per_tok + 2 * w.Hkv * w.D * 4
            + batch.B * batch.block_table.shape[1] * 4)


def attn_kv8_timing(w, batch, sb, ctx, ws, stream, dev, n_layers=16, reps=3):
    """Attention layers over INT8 pages at the step's shape and contexts, back
    to back between two events on the launch stream (the append, stream and
    combine launches of each call)."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    layers = [wl.make_attn_layer_kv8(w, batch, 5000 + i, dev) for i in range(n_layers)]
    for l in layers:
        l['out'] = torch.empty_like(l['q'])

    def run(l, s=stream):
        bd.spec_verify_attention_kv8(sb, l['q'], l['k_new'], l['v_new'], l['k_cache'],
                                     l['v_cache'], l['k_scale'], l['v_scale'],
                                     batch.block_table, ctx, l['out'], workspace=ws,
                                     stream=s)
    for l in layers:
        run(l)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        for l in layers:
            run(l)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (reps * n_layers)
    # the same launches replayed from a HIP graph (captured on the current
    # stream, so the calls take the default stream argument)
    gms = graph_block_ms(stream, [(lambda l=l: run(l, None)) for l in layers]) / n_layers
    nbytes = attn_kv8_bytes(w, batch, ctx.tolist())
    del layers
    return {'layer_ms': round(ms, 4), 'bytes': nbytes,
            'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1),
            'frac_of_peak': round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            'layer_ms_graph': round(gms, 4),
            'GBps_graph': round(nbytes / (gms * 1e-3) / 1e9, 1),
            'frac_of_peak_graph': round(nbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            'launches': reps * n_layers}


def measured_traffic():
    """HBM bytes per attention launch (stream kernel + combine kernel) from the
    committed FETCH_SIZE / WRITE_SIZE counter runs, already scaled by the copy
    calibration; None when the attention source changed since they were taken."""
    import hashlib
    if not os.path.exists(TRAFFIC_FILE):
        return None
    vals = {}
    for ln in open(TRAFFIC_FILE):
        parts = ln.split()
        if len(parts) == 2 and not ln.startswith('#'):
            vals[parts[0]] = parts[1]
    sha = hashlib.sha256(open(ATTN_SOURCE, 'rb').read()).hexdigest()
    if vals.get('source_sha256') != sha:
        return None
    return int(float(vals['fetch_bytes_per_launch']) + float(vals['write_bytes_per_launch']))


def elem_size(dtype):
    import torch
    return torch.finfo(dtype).bits // 8


def attn_bytes(w, batch, ctx=None):
    """Algorithmic HBM bytes of one attention layer (one launch) at the given
    contexts (default: the batch's)."""
    s = elem_size(w.attn_dtype)
    ctx_sum = sum(batch.ctx if ctx is None else ctx)
    T = batch.total_T
    kv_ctx = ctx_sum * w.Hkv * w.D * 2 * s
    per_tok = w.Hq * w.D * s + 2 * w.Hkv * w.D * s + 2 * w.Hkv * w.D * s + w.Hq * w.D * s
    return int(kv_ctx + T * per_tok + batch.B * batch.block_table.shape[1] * 4)


def gdn_bytes(w, batch, state_bytes=4):
    """One GDN layer: the state read and written once (the method's minimum),
    q, k, v, the gates and the outputs."""
    s = elem_size(w.gdn_dtype)
    T = batch.total_T
    return (2 * batch.B * w.H * w.dv * w.dk * state_bytes + T * w.H * (2 * w.dk + w.dv) * s
            + T * w.H * 8 + T * w.H * w.dv * s)


def accept_bytes(w, batch, mode):
    s = elem_size(w.logit_dtype)
    T = batch.total_T
    b = T * w.V * s
    if mode == 'rejection':
        b += (T - batch.B) * w.V * s
    return b


def ceilings(dev):
    """Rates of plain streaming kernels on this GPU, measured in this run:
    a device copy of 2 GiB (read + write bytes), row sums of a 4 GiB fp32
    array in rows of 4096 (read bytes: the output is 1/4096 of the input)
    and a fill of 2 GiB (write bytes)."""
    import torch
    n = 1 << 31
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def rate(fn, nbytes):
        for _ in range(2):
            fn()
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(nbytes * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    copy = rate(lambda: y.copy_(x), 2 * n)
    write = rate(lambda: y.fill_(1.0), n)
    del x, y
    z = torch.ones(2 * n // 4, dtype=torch.float32, device=dev)
    read = rate(lambda: z.view(-1, 4096).sum(dim=1), 2 * n)
    del z
    torch.cuda.empty_cache()
    return {'copy_GBps': copy, 'read_GBps': read, 'write_GBps': write,
            'how': 'torch copy_ of 2 GiB (read + write bytes), row sums over 4 GiB in rows of '
                   '4096 fp32 (read bytes), fill of 2 GiB (write bytes); 5 repetitions each '
                   'between HIP events'}


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {'median': round(float(np.median(a)), 4), 'p10': round(float(np.percentile(a, 10)), 4),
            'p90': round(float(np.percentile(a, 90)), 4), 'n': int(a.size)}


def timed_block(stream, calls):
    """Run the callables back to back on `stream` between two HIP events
    (nothing recorded between them); returns the total time (ms)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for c in calls:
        c()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def graph_block_ms(stream, calls, reps=3):
    """The callables captured into one HIP graph and replayed `reps` times
    back to back between two HIP events on `stream` (no host work between
    the kernels); returns the time per replay (ms)."""
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, capture_error_mode='thread_local'):
        for c in calls:
            c()
    g.replay()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) / reps


def timed_calls(stream, calls):
    """Run the callables back to back on `stream` with a HIP event before
    each one and after the last; returns the per-call times (ms) and the
    total (ms)."""
    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i, c in enumerate(calls):
        c()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(len(calls))]
    return per, ev[0].elapsed_time(ev[-1])


def cpu_baseline(w, batch, layers, acc, mode, draft_tokens_per_step, budget, commit=None):
    """The oracle as it stands, on a bounded sample, scaled to one step.

    Within a time budget: GDN layers on the full batch, one at a time (at
    least one), each the oracle step's two passes (verify, then the commit of
    the accepted tokens; with `commit` given and no acceptance, the single
    verify-and-commit pass); attention of one layer, one sequence at a time (its
    pages only; at least one), scaled to the whole batch by context length;
    acceptance on all rows.  The per-layer costs are then multiplied by the
    layer counts of the step.
    """
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get('num_threads', 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    f64 = lambda t: t.detach().double().cpu().numpy()
    i64 = lambda t: t.detach().cpu().numpy().astype(np.int64)
    cu = i64(batch.cu_seqlens)
    ctx = i64(batch.ctx_lens)
    table = i64(batch.block_table)
    parts = []
    t_acc = 0.0
    if acc is not None:
        ai = [f64(acc['target_logits']), i64(acc['draft_tokens'])]
        t0 = time.perf_counter()
        if mode == 'greedy':
            a_len, _ = oracle.greedy_accept(ai[0], ai[1], cu, batch.max_T)
        else:
            a_len, _ = oracle.rejection_accept(ai[0], f64(acc['draft_logits']), ai[1],
                                               f64(acc['u_accept']), f64(acc['u_final']), cu,
                                               batch.max_T)
        t_acc = time.perf_counter() - t0
        commit = a_len + 1
        parts.append(f'{mode} acceptance on all rows')
    gdn = [l for l in layers if l['kind'] == 'gdn']
    t_gdn, n_gdn_done, t_gdn_sum = 0.0, 0, 0.0
    for g in gdn:
        S, q, k, v = f64(g['state']), f64(g['q']), f64(g['k']), f64(g['v'])
        al, be = f64(g['alpha']), f64(g['beta'])
        t0 = time.perf_counter()
        if acc is not None:
            oracle.gdn_step(S, None, q, k, v, al, be, cu, None, oracle.GDN_VERIFY_ONLY)
            oracle.gdn_step(S, None, None, k, v, al, be, cu, commit, oracle.GDN_COMMIT_ONLY)
        else:
            oracle.gdn_step(S, None, q, k, v, al, be, cu, i64(commit), oracle.GDN_VERIFY_COMMIT)
        t_gdn_sum += time.perf_counter() - t0
        n_gdn_done += 1
        if t_gdn_sum > 0.4 * budget:
            break
    if n_gdn_done:
        t_gdn = t_gdn_sum / n_gdn_done
        parts.append(f'{n_gdn_done} GDN layer(s) on all {batch.B} sequences (verify and commit)')
    att = [l for l in layers if l['kind'] == 'attn']
    t_att, t_att_sample, seqs = 0.0, 0.0, []
    if att:
        a = att[0]
        for b in range(batch.B):
            pages = table[b][table[b] >= 0]
            idx = torch.from_numpy(pages).to(a['k_cache'].device)
            kc, vc = f64(a['k_cache'][idx]), f64(a['v_cache'][idx])
            sub_t = np.arange(len(pages))[None, :]
            rows = slice(cu[b], cu[b + 1])
            q, kn, vn = f64(a['q'][rows]), f64(a['k_new'][rows]), f64(a['v_new'][rows])
            one = np.array([0, cu[b + 1] - cu[b]])
            t0 = time.perf_counter()
            if 'k_scale' in a:   # INT8 pages: the codes and the per-channel scales
                ks, vs = f64(a['k_scale']), f64(a['v_scale'])
                oracle.verify_attention_int8(q, kn, vn, kc, vc, ks, vs, sub_t, ctx[b:b + 1],
                                             one, batch.P)
                oracle.append_kv_int8(kc, vc, kn, vn, ks, vs, sub_t, ctx[b:b + 1], one,
                                      batch.P)
            else:
                oracle.verify_attention(q, kn, vn, kc, vc, sub_t, ctx[b:b + 1], one, batch.P)
                oracle.append_kv(kc, vc, kn, vn, sub_t, ctx[b:b + 1], one, batch.P)
            t_att_sample += time.perf_counter() - t0
            seqs.append(b)
            if t_att_sample > 0.5 * budget:
                break
        t_att = t_att_sample * float(max(ctx.sum(), 1)) / float(max(ctx[seqs].sum(), 1))
        parts.append(f'attention (verify + append) of one layer for {len(seqs)} of {batch.B} '
                     'sequences, scaled by context length')
    n_att = len(att)
    n_gdn = len(gdn)
    t_step = n_att * t_att + n_gdn * t_gdn + t_acc
    return {
        'value': draft_tokens_per_step / t_step, 'unit': 'verified draft tokens/s',
        'cores': int(threads), 'kind': 'oracle',
        'sample': '; '.join(parts) + f'; per-layer times scaled to {n_gdn} GDN + {n_att} '
                  'attention layers per step',
        'seconds_measured': round(t_gdn_sum + t_att_sample + t_acc, 2),
        'seconds_per_step_extrapolated': round(t_step, 3),
        'nproc': os.cpu_count(), 'affinity_cpus': len(os.sched_getaffinity(0)),
    }


def base_line(w, args, steps, warmup, value, ms_step, config):
    import torch
    return {
        'metric': 'verified draft tokens/sec at 1 GPU + achieved HBM GB/s (% of MI355X peak)',
        'value': round(value, 1), 'unit': 'verified draft tokens/s',
        'n_gpus': 1, 'steps': steps, 'warmup': warmup, 'ms_per_step': round(ms_step, 4),
        'higher_is_better': True, 'scaling': 'weak', 'vs_baseline': None,
        'dtype': 'bf16' if w.attn_dtype != torch.float32 else 'f32',
        'data': 'synthetic (seeded; no model weights)', 'config': config,
    }


def graph_replay_ms(make_graphs, replay_plan, finish, stream, steps, two_pass=False):
    """Capture HIP graphs (make_graphs returns them after an eager lead-in),
    replay them `steps` times per replay_plan(i), finish() (the flush), all
    between HIP events; returns the per-replay times and the total / steps.
    two_pass (replays that can be repeated, each well under a millisecond):
    the total from a pass with no event between replays, the per-replay
    times from a second pass."""
    import torch
    graphs = make_graphs()
    calls = [(lambda i=i: graphs[replay_plan(i)].replay()) for i in range(steps)]
    calls.append(finish)
    if two_pass:
        total = timed_block(stream, calls)
        per, _ = timed_calls(stream, calls)
    else:
        per, total = timed_calls(stream, calls)
    return per[:steps], total / steps


def run_step_workload(w, args, dev, ceil):
    """Workloads with attention and GDN layers and acceptance: the step."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    mode = args.accept if args.accept in w.accept_modes else w.accept_modes[-1]
    steps, warmup = args.steps, args.warmup
    kv8 = args.kv_format == 'int8'
    f16 = args.state_dtype == 'f16'
    if kv8 and w.attn_dtype != torch.bfloat16:
        sys.exit(f'--kv-format int8 takes bf16 activations; {w.name} is fp32')
    default_formats = not kv8 and not f16
    # room in every block table for the tokens all eager and graph steps commit
    batch = wl.make_batch(w, args.seed, dev, reserve=w.max_T * (3 * (steps + warmup) + 8))
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = (wl.make_attn_layer_kv8 if kv8 else wl.make_attn_layer)(w, batch, 1000 + i, dev)
            lay['out'] = torch.empty_like(lay['q'])
        else:
            lay = wl.make_gdn_layer(w, batch, 1000 + i, dev,
                                    state_dtype=torch.float16 if f16 else torch.float32)
            lay['out'] = torch.empty_like(lay['v'])
        lay['kind'] = kind
        layers.append(lay)
    acc = wl.make_accept(w, batch, 2000, mode, dev)
    torch.cuda.synchronize()
    print(f'[bench] inputs ready: {w.name}, {len(layers)} layers, '
          f'{torch.cuda.memory_allocated() / 2**30:.1f} GiB', file=sys.stderr, flush=True)

    dt_a = bd.SV_BF16 if w.attn_dtype == torch.bfloat16 else bd.SV_F32
    dt_g = bd.SV_BF16 if w.gdn_dtype == torch.bfloat16 else bd.SV_F32
    amode = bd.SV_ACCEPT_GREEDY if mode == 'greedy' else bd.SV_ACCEPT_REJECTION
    gdn_layers = [bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'], l['beta'],
                               l['out']) for l in layers if l['kind'] == 'gdn']
    step_args = bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table, dt_a,
                       kv_format=bd.SV_KV_INT8 if kv8 else bd.SV_KV_PLAIN),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'],
                       l.get('k_scale'), l.get('v_scale'))
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, dt_g,
                      state_dtype=bd.SV_F16 if f16 else bd.SV_F32), gdn_layers,
        bd.accept_args(amode, acc['target_logits'], acc['draft_tokens'],
                       acc.get('draft_logits'), acc.get('u_accept'), acc.get('u_final')))
    sb = bd.make_batch(batch.cu_seqlens, batch.B, batch.max_T, batch.total_T)
    ws = torch.zeros(bd.spec_verify_step_workspace_bytes(sb, step_args), dtype=torch.uint8,
                     device=dev)
    result = torch.empty(batch.B * (1 + batch.max_T), dtype=torch.int32, device=dev)
    commits = [torch.zeros(batch.B, dtype=torch.int32, device=dev) for _ in range(2)]
    ctx = batch.ctx_lens.clone()
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    deferred = args.schedule == 'deferred'
    sched = bd.SV_SCHEDULE_DEFERRED if deferred else bd.SV_SCHEDULE_TWO_PHASE
    # pending tokens of the previous step: the same input buffers (their
    # values do not change the work), with the previous step's commit lengths
    pend_arr = (bd.SvGdnLayer * max(1, len(gdn_layers)))(*gdn_layers)
    pends = [bd.SvStepPending(sb, pend_arr, commits[j].data_ptr()) for j in range(2)]
    state = {'n': 0}

    def step_call(out_j, pend_j):
        bd.spec_verify_step(sb, step_args, ctx, result, commits[out_j], schedule=sched,
                            pending=pends[pend_j] if pend_j is not None else None,
                            workspace=ws, err=err)

    def one_step():
        i = state['n']
        step_call(i % 2, (i - 1) % 2 if deferred and i > 0 else None)
        state['n'] = i + 1

    def flush():
        if deferred and state['n'] > 0:
            bd.spec_verify_flush(step_args, pends[(state['n'] - 1) % 2], err=err)
            state['n'] = 0

    for _ in range(warmup):
        one_step()
    flush()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f'device error flag {int(err.item())}'
    print('[bench] warmup done', file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    ctx_start = ctx.clone()
    t0 = time.perf_counter()
    per, total = timed_calls(stream, [one_step] * steps + [flush])
    wall = time.perf_counter() - t0
    ms_step = total / steps
    assert int(err.item()) == 0, f'device error flag {int(err.item())}'
    c_last = (ctx - ctx_start).double() / steps          # tokens committed per step
    accepted = result[:batch.B].double().mean().item()
    print(f'[bench] timed {steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / steps:.3f})',
          file=sys.stderr, flush=True)
    # the contexts the timed steps attended at, averaged over the steps
    ctx_mean = (ctx_start.double() + c_last * (steps - 1) / 2.0).tolist()

    graph = None
    if not args.no_graph:
        def make_graphs():
            # eager lead-in so the first graph has a pending commit to replay
            one_step()
            torch.cuda.synchronize()
            gs = []
            pairs = [(1, 0), (0, 1)] if deferred else [(0, None)]
            for out_j, pend_j in pairs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, capture_error_mode='thread_local'):
                    step_call(out_j, pend_j)
                gs.append(g)
            return gs

        def finish():
            state['n'] = steps + 1      # the last replay wrote commits[steps % 2]
            flush()
        gper, gms = graph_replay_ms(make_graphs, lambda i: i % (2 if deferred else 1),
                                    finish, stream, steps)
        assert int(err.item()) == 0, f'device error flag {int(err.item())}'
        graph = {'ms_per_step': round(gms, 4), 'step_ms': percentiles(gper),
                 'value': round((batch.total_T - batch.B) / (gms * 1e-3), 1),
                 'how': 'the same step captured into HIP graphs (one per commit buffer) and '
                        'replayed back to back, flush included'}
        print(f'[bench] graph replay: {gms:.3f} ms/step', file=sys.stderr, flush=True)

    # ---- per-part timing and the dominant kernel's per-launch duration
    att_layers = [l for l in layers if l['kind'] == 'attn']
    gdn_l = [l for l in layers if l['kind'] == 'gdn']
    ctx_fixed = ctx.clone()
    n_launch = 0
    calls = []
    for _ in range(args.attn_reps):
        for l in att_layers:
            if kv8:
                calls.append(lambda l=l: bd.spec_verify_attention_kv8(
                    sb, l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'],
                    l['k_scale'], l['v_scale'], batch.block_table, ctx_fixed, l['out'],
                    workspace=ws, err=err))
            else:
                calls.append(lambda l=l: bd.spec_verify_attention(
                    sb, l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'],
                    batch.block_table, ctx_fixed, l['out'], workspace=ws, err=err))
    att_total = timed_block(stream, calls)
    n_launch = len(calls)
    att_ms_eager = att_total / n_launch
    # the same launches replayed from a HIP graph: the kernels' own time, with
    # no host work (marshalling, launch calls) between them
    att_ms_mean = graph_block_ms(stream, calls) / n_launch
    b_att = (attn_kv8_bytes(w, batch, ctx_fixed.tolist()) if kv8 else
             attn_bytes(w, batch, ctx_fixed.tolist()))
    g_total = timed_block(stream, [
        (lambda l=l: bd.gdn_verify_commit(sb, bd.SV_GDN_VERIFY_COMMIT, l['state'], l['q'],
                                          l['k'], l['v'], l['alpha'], l['beta'], commits[0],
                                          l['out'])) for l in gdn_l])
    gdn_ms = g_total / max(1, len(gdn_l))
    acc_reps = 20
    a_total = timed_block(stream, [
        (lambda: bd.spec_accept(sb, amode, acc['target_logits'], acc['draft_tokens'], result,
                                draft_logits=acc.get('draft_logits'),
                                u_accept=acc.get('u_accept'), u_final=acc.get('u_final'),
                                workspace=ws, err=err))] * acc_reps)
    acc_ms = a_total / acc_reps

    with_conv = None
    if w.name == 'hybrid_step_64l' and not args.no_next_rows and default_formats:
        with_conv = step_with_conv_timing(w, batch, layers, acc, amode, sb, ws, ctx, err, steps,
                                          warmup, stream, dev, sched, deferred)
        print(f'[bench] step with short conv: {with_conv["ms_per_step"]:.3f} ms/step',
              file=sys.stderr, flush=True)

    next_rows = None
    if w.name == 'hybrid_step_64l' and not args.no_next_rows and default_formats:
        next_rows = {'short_conv': short_conv_timing(w, batch, sb, commits[0], stream, dev),
                     'gdn_state_dtype': gdn_state_dtype_timing(w, batch, sb, commits[0], stream,
                                                               dev),
                     'attention_int8_kv': attn_kv8_timing(w, batch, sb, ctx_fixed, ws, stream,
                                                          dev),
                     'checkpoint_commit': checkpoint_timing(w, batch, sb, commits[0], stream,
                                                            dev)}

    T = batch.total_T
    n_att, n_gdn = len(att_layers), len(gdn_l)
    draft_per_step = T - batch.B
    sbytes = 2 if f16 else 4
    b_step = (n_att * (attn_kv8_bytes(w, batch, ctx_mean) if kv8 else
                       attn_bytes(w, batch, ctx_mean))
              + n_gdn * gdn_bytes(w, batch, sbytes) + accept_bytes(w, batch, mode))
    # bytes the schedule actually moves beyond the method's minimum: the
    # replayed tokens' k, v and gates (deferred: read again by the next
    # verify; two-phase: by the batched commit), and under two-phase one more
    # read of every GDN state
    es = elem_size(w.gdn_dtype)
    sum_c = float(c_last.sum().item())
    replay = sum_c * w.H * ((w.dk + w.dv) * es + 8)
    extra = n_gdn * (replay + (0 if deferred else batch.B * w.H * w.dv * w.dk * sbytes))
    pc = percentiles(per[:steps])
    gbs = b_step / (ms_step * 1e-3) / 1e9
    gbs_med = b_step / (pc['median'] * 1e-3) / 1e9
    achieved = b_att / (att_ms_mean * 1e-3) / 1e9
    line = base_line(w, args, steps, warmup, draft_per_step / (ms_step * 1e-3), ms_step, {
        'workload': w.name, 'layers': f'{n_gdn} GDN + {n_att} attention',
        'batch': batch.B, 'drafts_per_seq': f'U{{1..{w.k}}}' if w.ragged_k else w.k,
        'ctx': list(w.ctx), 'Hq_Hkv_D': [w.Hq, w.Hkv, w.D], 'page': batch.P,
        'gdn_H_dk_dv': [w.H, w.dk, w.dv], 'vocab': w.V, 'accept': mode,
        'schedule': args.schedule, 'kv_format': args.kv_format,
        'state_dtype': args.state_dtype})
    if kv8:  # the attention arithmetic: INT8 codes widened to fp16 for the MFMAs
        line['dtype'] = 'f16'
    line.update({
        'step_ms': pc,
        'graph': graph,
        'step_hbm': {'algorithmic_bytes': int(b_step), 'GBps': round(gbs, 1),
                     'frac_of_peak': round(gbs / HBM_PEAK_GBS, 4),
                     'GBps_at_median': round(gbs_med, 1),
                     'frac_of_measured_read': round(gbs / ceil['read_GBps'], 4),
                     'contexts': 'mean over the timed steps',
                     'actual_bytes': int(b_step + extra),
                     'actual_GBps': round((b_step + extra) / (ms_step * 1e-3) / 1e9, 1),
                     'actual_how': f'{args.schedule} schedule: the replayed tokens\' k, v and '
                                   'gates' + ('' if deferred else
                                              ' and one more read of every GDN state')},
        'ceilings': ceil,
        'roofline': {'kernel': ('spec_verify_attention_kv8, one layer (attn_append_kv8 + '
                                'attn_stream_kv8 + attn_combine_bf16 launches)' if kv8 else
                                'spec_verify_attention, one layer (attn_stream_bf16 + '
                                'attn_combine_bf16 launches)' if dt_a == bd.SV_BF16 else
                                'spec_verify_attention, one layer (attn_f32)'),
                     'bound': 'hbm', 'achieved': round(achieved, 1), 'peak': HBM_PEAK_GBS,
                     'unit': 'GB/s', 'frac': round(achieved / HBM_PEAK_GBS, 4),
                     'frac_of_measured_read': round(achieved / ceil['read_GBps'], 4),
                     'traffic': (measured_traffic() if w.name == 'hybrid_step_64l'
                                 and not kv8 else None),
                     'traffic_unit': 'HBM bytes per launch', 'bytes_per_launch': b_att,
                     'launch_ms': round(att_ms_mean, 4), 'launches': n_launch,
                     'launch_ms_eager': round(att_ms_eager, 4),
                     'how': 'the layer\'s launches captured into one HIP graph and replayed '
                            'between two HIP events on the launch stream (launch_ms_eager: the '
                            'same launches issued eagerly)'},
        'parts_ms': {'attention_layer': round(att_ms_mean, 4),
                     'gdn_layer_verify_commit': round(gdn_ms, 4),
                     'acceptance': round(acc_ms, 4)},
        'step_with_short_conv': with_conv,
        'next_rows': next_rows,
        'mean_accept_len': round(accepted, 3),
        # sum_b (a_b + 1) per timed step, from the ctx_lens the steps advanced
        'committed_tokens_per_step': round(c_last.sum().item(), 2),
        'dtype_detail': (('INT8 per-channel KV pages, fp16 MFMA, ' if kv8 else
                          'bf16 I/O and MFMA, ' if dt_a == bd.SV_BF16 else 'fp32 I/O, ')
                         + 'fp32 accumulation, '
                         + ('fp16 GDN state bank (fp32 arithmetic)' if f16 else
                            'fp32 GDN state') + ', fp64 acceptance'),
    })
    if not args.no_cpu_baseline:
        print('[bench] timing the CPU oracle on a bounded sample', file=sys.stderr, flush=True)
        line['cpu_baseline'] = cpu_baseline(w, batch, layers, acc, mode, draft_per_step,
                                           args.cpu_budget)
    return line


def conv_bytes(w, batch, pend_rows):
    """One short-conv layer: state read + write, inputs and outputs, the
    replayed pending inputs, taps and bias."""
    s, C, K, T, B = elem_size(w.gdn_dtype), w.conv_C, w.conv_K, batch.total_T, batch.B
    return 2 * B * (K - 1) * C * s + 2 * T * C * s + pend_rows * C * s + C * K * 4 + C * 4


def step_with_conv_timing(w, batch, layers, acc, amode, sb, ws, ctx, err, steps, warmup,
                          stream, dev, sched, deferred):
    """The same step with every GDN layer's short convolution (C = the q, k
    and v features, K = 4, SiLU) run beside its GDN verify in one launch
    (two-phase: committed in the batched commit launch), timed the same way."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    convs = {}
    g_layers = []
    for i, l in enumerate(layers):
        if l['kind'] == 'gdn':
            c = wl.make_conv_layer(w, batch, 8000 + i, dev)
            c['out'] = torch.empty_like(c['x'])
            convs[i] = c
            g_layers.append(bd.gdn_layer(l['state'], l['q'], l['k'], l['v'], l['alpha'],
                                         l['beta'], l['out'], conv=c))
    dt = bd.SV_BF16 if w.attn_dtype == torch.bfloat16 else bd.SV_F32
    args = bd.StepArgs(
        [1 if l['kind'] == 'attn' else 0 for l in layers],
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table, dt),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'])
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, dt, conv_C=w.conv_C, conv_K=w.conv_K,
                      conv_activation=bd.SV_ACT_SILU), g_layers,
        bd.accept_args(amode, acc['target_logits'], acc['draft_tokens'],
                       acc.get('draft_logits'), acc.get('u_accept'), acc.get('u_final')))
    result = torch.empty(batch.B * (1 + batch.max_T), dtype=torch.int32, device=dev)
    commits = [torch.zeros(batch.B, dtype=torch.int32, device=dev) for _ in range(2)]
    arr = (bd.SvGdnLayer * len(g_layers))(*g_layers)
    pends = [bd.SvStepPending(sb, arr, commits[j].data_ptr()) for j in range(2)]
    st = {'n': 0}

    def one_step():
        i = st['n']
        bd.spec_verify_step(sb, args, ctx, result, commits[i % 2], schedule=sched,
                            pending=pends[(i - 1) % 2] if deferred and i > 0 else None,
                            workspace=ws, err=err)
        st['n'] = i + 1

    def flush():
        if deferred and st['n'] > 0:
            bd.spec_verify_flush(args, pends[(st['n'] - 1) % 2], err=err)
            st['n'] = 0

    for _ in range(warmup):
        one_step()
    flush()
    torch.cuda.synchronize()
    per, total = timed_calls(stream, [one_step] * steps + [flush])
    assert int(err.item()) == 0, f'device error flag {int(err.item())}'
    ms = total / steps
    pend_rows = int(commits[0].sum().item()) if deferred else 0
    b_conv = len(convs) * conv_bytes(w, batch, pend_rows)
    del convs
    return {'ms_per_step': round(ms, 4), 'step_ms': percentiles(per[:steps]),
            'value': round((batch.total_T - batch.B) / (ms * 1e-3), 1),
            'conv_layers': len(g_layers), 'conv_C_K': [w.conv_C, w.conv_K],
            'conv_bytes_per_step': int(b_conv),
            'how': 'every GDN layer\'s short convolution in its GDN verify launch '
                   '(deferred: pending inputs replayed), the flush included'}


def rotation_sets(nbytes_per_set, min_total=1 << 30, min_sets=4):
    return max(min_sets, -(-min_total // nbytes_per_set))


def run_attention_workload(w, args, dev, ceil):
    """Paged verification attention alone: a step is one spec_verify_attention
    call over the batch (KV write-through included), rotating over
    independent buffer sets (pools, q, k_new, v_new) of >= 1 GB in total."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    steps, warmup = args.steps, args.warmup
    batch = wl.make_batch(w, args.seed, dev)
    b_call = attn_bytes(w, batch)
    n_sets = rotation_sets(b_call)
    sets = []
    for i in range(n_sets):
        lay = wl.make_attn_layer(w, batch, 1000 + i, dev)
        lay['out'] = torch.empty_like(lay['q'])
        sets.append(lay)
    sb = bd.make_batch(batch.cu_seqlens, batch.B, batch.max_T, batch.total_T)
    ws = torch.zeros(max(1, bd.spec_verify_attention_workspace_bytes(
        batch.B, batch.total_T, w.Hq, w.Hkv, w.D, batch.block_table.shape[1], batch.P,
        bd.SV_BF16)), dtype=torch.uint8, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print(f'[bench] inputs ready: {w.name}, {n_sets} buffer sets of {b_call / 1e6:.0f} MB',
          file=sys.stderr, flush=True)

    def call(i):
        l = sets[i % n_sets]
        bd.spec_verify_attention(sb, l['q'], l['k_new'], l['v_new'], l['k_cache'],
                                 l['v_cache'], batch.block_table, batch.ctx_lens, l['out'],
                                 workspace=ws, err=err)
    for i in range(warmup):
        call(i)
    stream = torch.cuda.current_stream()
    total = timed_block(stream, [(lambda i=i: call(i)) for i in range(steps)])
    ms = total / steps
    # per-call spread from a second pass with an event between calls (each
    # event adds a few microseconds, so the mean above is taken without them)
    per, _ = timed_calls(stream, [(lambda i=i: call(i)) for i in range(steps)])
    assert int(err.item()) == 0
    graph = None
    if not args.no_graph:
        def make_graphs():
            gs = []
            for i in range(n_sets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, capture_error_mode='thread_local'):
                    call(i)
                gs.append(g)
            return gs
        gper, gms = graph_replay_ms(make_graphs, lambda i: i % n_sets, lambda: None, stream,
                                    steps, two_pass=True)
        graph = {'ms_per_step': round(gms, 4), 'step_ms': percentiles(gper),
                 'how': 'each buffer set\'s call captured into a HIP graph, replayed in turn'}
    draft = batch.total_T - batch.B
    pc = percentiles(per)
    gbs = b_call / (ms * 1e-3) / 1e9
    line = base_line(w, args, steps, warmup, draft / (ms * 1e-3), ms, {
        'workload': w.name, 'layers': '1 attention (the call alone)', 'batch': batch.B,
        'drafts_per_seq': w.k, 'ctx': list(w.ctx), 'Hq_Hkv_D': [w.Hq, w.Hkv, w.D],
        'page': batch.P, 'buffer_sets': n_sets,
        'rotation_bytes': int(n_sets * b_call)})
    line.update({
        'step_ms': pc, 'graph': graph,
        'step_hbm': {'algorithmic_bytes': int(b_call), 'GBps': round(gbs, 1),
                     'frac_of_peak': round(gbs / HBM_PEAK_GBS, 4),
                     'GBps_at_median': round(b_call / (pc['median'] * 1e-3) / 1e9, 1),
                     'frac_of_measured_read': round(gbs / ceil['read_GBps'], 4)},
        'ceilings': ceil,
        'roofline': {'kernel': 'spec_verify_attention (attn_stream_bf16 + attn_combine_bf16)',
                     'bound': 'hbm', 'achieved': round(gbs, 1), 'peak': HBM_PEAK_GBS,
                     'unit': 'GB/s', 'frac': round(gbs / HBM_PEAK_GBS, 4),
                     'frac_of_measured_read': round(gbs / ceil['read_GBps'], 4),
                     'traffic': None, 'bytes_per_launch': int(b_call),
                     'launch_ms': round(ms, 4), 'launches': steps},
    })
    if not args.no_cpu_baseline:
        line['cpu_baseline'] = cpu_baseline(w, batch, [dict(sets[0], kind='attn')], None, None,
                                           draft, args.cpu_budget)
    return line


def run_gdn_workload(w, args, dev, ceil):
    """GDN verify + commit alone: a step is one gdn_verify_commit call
    (VERIFY_COMMIT, commit lengths from the 70 % keep recipe), rotating over
    independent buffer sets (state bank, q, k, v, gates) of >= 1 GB."""
    import torch

    import workloads as wl
    from block_draft_verification_spec_amd import binding as bd
    steps, warmup = args.steps, args.warmup
    batch = wl.make_batch(w, args.seed, dev)
    commit = wl.make_commit_len(batch, args.seed + 1, device=dev)
    b_call = gdn_bytes(w, batch)
    n_sets = rotation_sets(b_call)
    sets = []
    for i in range(n_sets):
        g = wl.make_gdn_layer(w, batch, 1000 + i, dev)
        g['out'] = torch.empty_like(g['v'])
        sets.append(g)
    sb = bd.make_batch(batch.cu_seqlens, batch.B, batch.max_T, batch.total_T)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    print(f'[bench] inputs ready: {w.name}, {n_sets} buffer sets of {b_call / 1e6:.0f} MB',
          file=sys.stderr, flush=True)

    def call(i):
        g = sets[i % n_sets]
        bd.gdn_verify_commit(sb, bd.SV_GDN_VERIFY_COMMIT, g['state'], g['q'], g['k'], g['v'],
                             g['alpha'], g['beta'], commit, g['out'], err=err)
    for i in range(warmup):
        call(i)
    stream = torch.cuda.current_stream()
    total = timed_block(stream, [(lambda i=i: call(i)) for i in range(steps)])
    ms = total / steps
    # per-call spread from a second pass with an event between calls (each
    # event adds a few microseconds, so the mean above is taken without them)
    per, _ = timed_calls(stream, [(lambda i=i: call(i)) for i in range(steps)])
    assert int(err.item()) == 0
    graph = None
    if not args.no_graph:
        def make_graphs():
            gs = []
            for i in range(n_sets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, capture_error_mode='thread_local'):
                    call(i)
                gs.append(g)
            return gs
        gper, gms = graph_replay_ms(make_graphs, lambda i: i % n_sets, lambda: None, stream,
                                    steps, two_pass=True)
        graph = {'ms_per_step': round(gms, 4), 'step_ms': percentiles(gper),
                 'how': 'each buffer set\'s call captured into a HIP graph, replayed in turn'}
    draft = batch.total_T - batch.B
    pc = percentiles(per)
    gbs = b_call / (ms * 1e-3) / 1e9
    line = base_line(w, args, steps, warmup, draft / (ms * 1e-3), ms, {
        'workload': w.name, 'layers': '1 GDN (the call alone, VERIFY_COMMIT)',
        'batch': batch.B, 'drafts_per_seq': w.k, 'gdn_H_dk_dv': [w.H, w.dk, w.dv],
        'state': 'fp32', 'buffer_sets': n_sets, 'rotation_bytes': int(n_sets * b_call)})
    line.update({
        'step_ms': pc, 'graph': graph,
        'step_hbm': {'algorithmic_bytes': int(b_call), 'GBps': round(gbs, 1),
                     'frac_of_peak': round(gbs / HBM_PEAK_GBS, 4),
                     'GBps_at_median': round(b_call / (pc['median'] * 1e-3) / 1e9, 1),
                     'frac_of_measured_copy': round(gbs / ceil['copy_GBps'], 4)},
        'ceilings': ceil,
        'roofline': {'kernel': 'gdn_verify_commit (gdn_kernel)', 'bound': 'hbm',
                     'achieved': round(gbs, 1), 'peak': HBM_PEAK_GBS, 'unit': 'GB/s',
                     'frac': round(gbs / HBM_PEAK_GBS, 4),
                     'frac_of_measured_copy': round(gbs / ceil['copy_GBps'], 4),
                     'traffic': None, 'bytes_per_launch': int(b_call),
                     'launch_ms': round(ms, 4), 'launches': steps},
    })
    if not args.no_cpu_baseline:
        line['cpu_baseline'] = cpu_baseline(w, batch, [dict(sets[0], kind='gdn')], None, None,
                                           draft, args.cpu_budget, commit=commit)
    return line


def main():
    args = parse()
    if args.gpus != 1:
        print(f'bench.py runs on one GPU only (asked for --gpus {args.gpus}): this '
              'library has no multi-GPU path (the step shards by sequence: each GPU would run '
              'this step on its own sequences, KV pool and state slots).',
              file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch

    import workloads as wl

    dev = 'cuda'
    torch.cuda.set_device(0)
    w = wl.WORKLOADS[args.workload]
    ceil = ceilings(dev)
    print(f'[bench] ceilings: {ceil["copy_GBps"]} GB/s copy, {ceil["read_GBps"]} GB/s read',
          file=sys.stderr, flush=True)
    kinds = set(w.layers)
    if kinds == {'attn'}:
        line = run_attention_workload(w, args, dev, ceil)
    elif kinds == {'gdn'}:
        line = run_gdn_workload(w, args, dev, ceil)
    else:
        line = run_step_workload(w, args, dev, ceil)
    print(json.dumps(line), flush=True)


if __name__ == '__main__':
    main()
