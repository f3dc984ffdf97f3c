"""Benchmark of the block speculative-verification step on one MI355X.

Workload: the full hybrid verify step (64 layers, GDN,GDN,GDN,ATT x 16;
B = 64 sequences, k = 3 drafts, contexts ~U[2048, 8192], 32q/8kv heads,
D = 128, bf16 paged KV in 64-token pages; 48 GDN layers with 32 heads,
dk = dv = 128, fp32 state; acceptance over V = 151936 bf16 logits),
synthetic seeded inputs resident in HBM before timing starts.

A step = one call of spec_verify_step: every layer's verify pass, the
acceptance, the GDN commit (deferred schedule: folded into the next step's
verify pass; the timed region ends with a flush so every accepted token of
every timed step is committed) and the ctx_lens update.

Prints one JSON line.  value = verified draft tokens per second (sum_b k_b
per step).  Also reported: algorithmic HBM bytes per step and GB/s (% of the
8 TB/s peak), the roofline of the dominant kernel (the paged attention call,
timed over back-to-back launches with HIP events on the stream it runs on),
and the CPU oracle timed on a bounded sample of the same workload.
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
    p.add_argument('--no-cpu-baseline', action='store_true')
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

        def run(l):
            bd.gdn_verify_commit(sb, bd.SV_GDN_VERIFY_ONLY, l['state'], l['q'], l['k'], l['v'],
                                 l['alpha'], l['beta'], None, l['out'], pending=l['pend'],
                                 stream=stream)
        for l in layers:
            run(l)
        e0.record(stream)
        for _ in range(reps):
            for l in layers:
                run(l)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (reps * len(layers))
        es = torch.finfo(sdt).bits // 8
        T = batch.total_T
        pend_rows = int(commit.sum().item())
        # state read + write, current q/k/v/gates/out, replayed k/v/gates
        nbytes = (2 * batch.B * w.H * w.dv * w.dk * es + T * w.H * (2 * w.dk + 2 * w.dv) * 2
                  + T * w.H * 8 + pend_rows * w.H * ((w.dk + w.dv) * 2 + 8))
        res[name] = {'layer_ms': round(ms, 4), 'bytes': nbytes,
                     'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1)}
        del layers
    res['schedule'] = 'deferred (pending replay + verify)'
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


def attn_kv8_bytes(w, batch):
    """Algorithmic HBM bytes of one attention layer over INT8 pages: the
    cached codes, the in-flight bf16 rows and their codes, Q, O, the scales
    and the block table."""
    ctx = sum(batch.ctx)
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

    def run(l):
        bd.spec_verify_attention_kv8(sb, l['q'], l['k_new'], l['v_new'], l['k_cache'],
                                     l['v_cache'], l['k_scale'], l['v_scale'],
                                     batch.block_table, ctx, l['out'], workspace=ws,
                                     stream=stream)
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
    nbytes = attn_kv8_bytes(w, wl.Batch(**{**batch.__dict__, 'ctx': ctx.tolist()}))
    del layers
    return {'layer_ms': round(ms, 4), 'bytes': nbytes,
            'GBps': round(nbytes / (ms * 1e-3) / 1e9, 1),
            'frac_of_peak': round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
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


def attn_bytes(w, batch):
    """Algorithmic HBM bytes of one attention layer (one launch)."""
    s = 2  # bf16
    ctx = sum(batch.ctx)
    T = batch.total_T
    kv_ctx = ctx * w.Hkv * w.D * 2 * s
    per_tok = w.Hq * w.D * s + 2 * w.Hkv * w.D * s + 2 * w.Hkv * w.D * s + w.Hq * w.D * s
    return kv_ctx + T * per_tok + batch.B * batch.block_table.shape[1] * 4


def gdn_bytes(w, batch):
    s = 2
    T = batch.total_T
    return (2 * batch.B * w.H * w.dv * w.dk * 4 + T * w.H * (2 * w.dk + w.dv) * s
            + T * w.H * 8 + T * w.H * w.dv * s)


def accept_bytes(w, batch, mode):
    s = 2
    T = batch.total_T
    b = T * w.V * s
    if mode == 'rejection':
        b += (T - batch.B) * w.V * s
    return b


def cpu_baseline(w, batch, layers, acc, mode, draft_tokens_per_step, budget):
    """The oracle as it stands, on a bounded sample, scaled to one step.

    Within a time budget: GDN layers on the full batch, one at a time (at
    least one); attention of one layer, one sequence at a time (its pages
    only; at least one), scaled to the whole batch by context length;
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
    # acceptance on the full batch
    ai = [f64(acc['target_logits']), i64(acc['draft_tokens'])]
    t0 = time.perf_counter()
    if mode == 'greedy':
        oracle.greedy_accept(ai[0], ai[1], cu, batch.max_T)
    else:
        oracle.rejection_accept(ai[0], f64(acc['draft_logits']), ai[1], f64(acc['u_accept']),
                                f64(acc['u_final']), cu, batch.max_T)
    t_acc = time.perf_counter() - t0
    # GDN layers on the full batch
    gdn = [l for l in layers if l['kind'] == 'gdn']
    t_gdn_sum, n_gdn_done = 0.0, 0
    for g in gdn:
        args = (f64(g['state']), None, f64(g['q']), f64(g['k']), f64(g['v']),
                f64(g['alpha']), f64(g['beta']), cu, None, oracle.GDN_VERIFY_ONLY)
        t0 = time.perf_counter()
        oracle.gdn_step(*args)
        t_gdn_sum += time.perf_counter() - t0
        n_gdn_done += 1
        if t_gdn_sum > 0.4 * budget:
            break
    t_gdn = t_gdn_sum / n_gdn_done
    # attention, sequence by sequence
    a = next(l for l in layers if l['kind'] == 'attn')
    t_att_sample, seqs = 0.0, []
    for b in range(batch.B):
        pages = table[b][table[b] >= 0]
        idx = torch.from_numpy(pages).to(a['k_cache'].device)
        kc, vc = f64(a['k_cache'][idx]), f64(a['v_cache'][idx])
        sub_t = np.arange(len(pages))[None, :]
        rows = slice(cu[b], cu[b + 1])
        q, kn, vn = f64(a['q'][rows]), f64(a['k_new'][rows]), f64(a['v_new'][rows])
        t0 = time.perf_counter()
        oracle.verify_attention(q, kn, vn, kc, vc, sub_t, ctx[b:b + 1],
                                np.array([0, cu[b + 1] - cu[b]]), batch.P)
        t_att_sample += time.perf_counter() - t0
        seqs.append(b)
        if t_att_sample > 0.5 * budget:
            break
    t_att = t_att_sample * float(ctx.sum()) / float(ctx[seqs].sum())
    n_att = sum(1 for l in layers if l['kind'] == 'attn')
    n_gdn = len(layers) - n_att
    t_step = n_att * t_att + n_gdn * t_gdn + t_acc
    return {
        'value': draft_tokens_per_step / t_step, 'unit': 'verified draft tokens/s',
        'cores': int(threads), 'kind': 'oracle',
        'sample': (f'{n_gdn_done} GDN layer(s) on all {batch.B} sequences, attention of one '
                   f'layer for {len(seqs)} of {batch.B} sequences (scaled by context length), '
                   f'{mode} acceptance on all rows; per-layer times scaled to {n_gdn} GDN + '
                   f'{n_att} attention layers per step'),
        'seconds_measured': round(t_gdn_sum + t_att_sample + t_acc, 2),
        'seconds_per_step_extrapolated': round(t_step, 2),
        'affinity_cpus': len(os.sched_getaffinity(0)),
    }


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
    from block_draft_verification_spec_amd import binding as bd

    dev = 'cuda'
    torch.cuda.set_device(0)
    w = wl.WORKLOADS[args.workload]
    mode = args.accept
    steps, warmup = args.steps, args.warmup
    # room in every block table for the tokens all steps commit
    batch = wl.make_batch(w, args.seed, dev, reserve=w.max_T * (steps + warmup + 2))
    layers = []
    for i, kind in enumerate(w.layers):
        if kind == 'attn':
            lay = wl.make_attn_layer(w, batch, 1000 + i, dev)
            lay['out'] = torch.empty_like(lay['q'])
        else:
            lay = wl.make_gdn_layer(w, batch, 1000 + i, dev)
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
        bd.attn_config(w.Hq, w.Hkv, w.D, batch.P, batch.num_pages, batch.block_table, dt_a),
        [bd.attn_layer(l['q'], l['k_new'], l['v_new'], l['k_cache'], l['v_cache'], l['out'])
         for l in layers if l['kind'] == 'attn'],
        bd.gdn_config(w.H, w.dk, w.dv, batch.B, dt_g), gdn_layers,
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
    pend_arr = (bd.SvGdnLayer * len(gdn_layers))(*gdn_layers)
    state = {'n': 0}

    def one_step():
        i = state['n']
        pend = None
        if deferred and i > 0:
            pend = bd.SvStepPending(sb, pend_arr, commits[(i - 1) % 2].data_ptr())
        bd.spec_verify_step(sb, step_args, ctx, result, commits[i % 2], schedule=sched,
                            pending=pend, workspace=ws, err=err)
        state['n'] = i + 1

    def flush():
        if deferred and state['n'] > 0:
            last = commits[(state['n'] - 1) % 2]
            for l in layers:
                if l['kind'] == 'gdn':
                    bd.gdn_verify_commit(sb, bd.SV_GDN_COMMIT_ONLY, l['state'], l['q'], l['k'],
                                         l['v'], l['alpha'], l['beta'], last, l['out'])
            state['n'] = 0

    for _ in range(warmup):
        one_step()
    flush()
    torch.cuda.synchronize()
    assert int(err.item()) == 0, f'device error flag {int(err.item())}'
    print('[bench] warmup done', file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    t0 = time.perf_counter()
    for _ in range(steps):
        one_step()
    flush()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps
    assert int(err.item()) == 0, f'device error flag {int(err.item())}'
    accepted = result[:batch.B].double().mean().item()
    print(f'[bench] timed {steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / steps:.3f})',
          file=sys.stderr, flush=True)

    # ---- per-part timing and the dominant kernel's per-launch duration
    att_layers = [l for l in layers if l['kind'] == 'attn']
    nbytes_a = bd.spec_verify_attention_workspace_bytes(
        batch.B, batch.total_T, w.Hq, w.Hkv, w.D, batch.block_table.shape[1], batch.P, dt_a)
    ctx_fixed = ctx.clone()
    # back to back over every attention layer, attn_reps times, between two
    # events on the launch stream: the mean per launch (both kernels of a
    # launch and the gap to the next launch)
    n_launch = 0
    s0 = torch.cuda.Event(enable_timing=True)
    s1 = torch.cuda.Event(enable_timing=True)
    s0.record(stream)
    for _ in range(args.attn_reps):
        for l in att_layers:
            bd.spec_verify_attention(sb, l['q'], l['k_new'], l['v_new'], l['k_cache'],
                                     l['v_cache'], batch.block_table, ctx_fixed, l['out'],
                                     workspace=ws, err=err)
            n_launch += 1
    s1.record(stream)
    torch.cuda.synchronize()
    att_ms_mean = s0.elapsed_time(s1) / n_launch
    # attention bytes at the contexts the timed calls used
    cur_ctx = ctx_fixed.tolist()
    b_att = attn_bytes(w, wl.Batch(**{**batch.__dict__, 'ctx': cur_ctx}))
    gdn_l = [l for l in layers if l['kind'] == 'gdn']
    g0 = torch.cuda.Event(enable_timing=True)
    g1 = torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    for l in gdn_l:
        bd.gdn_verify_commit(sb, bd.SV_GDN_VERIFY_COMMIT, l['state'], l['q'], l['k'], l['v'],
                             l['alpha'], l['beta'], commits[0], l['out'])
    g1.record(stream)
    torch.cuda.synchronize()
    gdn_ms = g0.elapsed_time(g1) / max(1, len(gdn_l))

    # acceptance alone (same logits, uniforms and workspace), back to back
    acc_reps = 20
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(acc_reps):
        bd.spec_accept(sb, amode, acc['target_logits'], acc['draft_tokens'], result,
                       draft_logits=acc.get('draft_logits'), u_accept=acc.get('u_accept'),
                       u_final=acc.get('u_final'), workspace=ws, err=err)
    a1.record(stream)
    torch.cuda.synchronize()
    acc_ms = a0.elapsed_time(a1) / acc_reps

    conv = short_conv_timing(w, batch, sb, commits[0], stream, dev)
    gdn_sd = gdn_state_dtype_timing(w, batch, sb, commits[0], stream, dev)
    kv8 = attn_kv8_timing(w, batch, sb, ctx_fixed, ws, stream, dev)
    ckpt = checkpoint_timing(w, batch, sb, commits[0], stream, dev)

    T = batch.total_T
    n_att, n_gdn = len(att_layers), len(gdn_l)
    draft_per_step = T - batch.B
    ctx_mid = [c for c in cur_ctx]
    b_step = (n_att * attn_bytes(w, wl.Batch(**{**batch.__dict__, 'ctx': ctx_mid}))
              + n_gdn * gdn_bytes(w, batch) + accept_bytes(w, batch, mode))
    gbs = b_step / (ms_step * 1e-3) / 1e9
    achieved = b_att / (att_ms_mean * 1e-3) / 1e9

    line = {
        'metric': 'verified draft tokens/sec at 1 GPU + achieved HBM GB/s (% of MI355X peak)',
        'value': round(draft_per_step / (ms_step * 1e-3), 1),
        'unit': 'verified draft tokens/s',
        'n_gpus': 1, 'steps': steps, 'warmup': warmup,
        'ms_per_step': round(ms_step, 4),
        'higher_is_better': True, 'scaling': 'weak', 'vs_baseline': None,
        'dtype': 'bf16',
        'data': 'synthetic (seeded; no model weights)',
        'config': {'workload': w.name, 'layers': f'{n_gdn} GDN + {n_att} attention',
                   'batch': batch.B, 'drafts_per_seq': w.k, 'ctx': list(w.ctx),
                   'Hq_Hkv_D': [w.Hq, w.Hkv, w.D], 'page': batch.P,
                   'gdn_H_dk_dv': [w.H, w.dk, w.dv], 'vocab': w.V, 'accept': mode,
                   'schedule': args.schedule},
        'step_hbm': {'algorithmic_bytes': b_step, 'GBps': round(gbs, 1),
                     'frac_of_peak': round(gbs / HBM_PEAK_GBS, 4)},
        'roofline': {'kernel': 'spec_verify_attention, one layer '
                               '(attn_stream_bf16 + attn_combine_bf16 launches)',
                     'bound': 'hbm', 'achieved': round(achieved, 1), 'peak': HBM_PEAK_GBS,
                     'unit': 'GB/s', 'frac': round(achieved / HBM_PEAK_GBS, 4),
                     'traffic': measured_traffic(), 'traffic_unit': 'HBM bytes per launch',
                     'bytes_per_launch': b_att,
                     'launch_ms': round(att_ms_mean, 4), 'launches': n_launch},
        'parts_ms': {'attention_layer': round(att_ms_mean, 4),
                     'gdn_layer_verify_commit': round(gdn_ms, 4),
                     'acceptance': round(acc_ms, 4)},
        'next_rows': {'short_conv': conv, 'gdn_state_dtype': gdn_sd, 'attention_int8_kv': kv8,
                      'checkpoint_commit': ckpt},
        'mean_accept_len': round(accepted, 3),
        'dtype_detail': 'bf16 I/O and MFMA, fp32 accumulation and GDN state, fp64 acceptance',
    }
    if not args.no_cpu_baseline:
        print('[bench] timing the CPU oracle on a bounded sample', file=sys.stderr, flush=True)
        line['cpu_baseline'] = cpu_baseline(w, batch, layers, acc, mode, draft_per_step,
                                           args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == '__main__':
    main()
