"""Seeded synthetic inputs for the speculative-verification step.

This module only draws inputs: shapes, sizes and value distributions of the
five workloads below, from seeded torch generators, on whichever device the
caller asks for.  It contains none of the verification arithmetic (no
attention, no recurrence, no softmax, no acceptance); both the HIP library
(through the tests and the benchmark) and the CPU oracle (through the tests)
consume the very same tensors it returns.

Where a workload leaves a value unspecified, the choice made here is stated
next to it:

* draft logits for rejection sampling are the target logits plus Gaussian
  noise of standard deviation ``draft_sigma`` (chosen so that the mean of
  ``sum_x min(p, q)`` is about 0.70 at the workload's vocabulary size), and
  the draft tokens are drawn from the draft distribution by the Gumbel-max
  trick (the drafter's own sampling, not the verifier's);
* greedy drafts: each target row that is compared with a draft gets one
  planted logit of 24.0 at a uniformly drawn token (about 8 standard
  deviations above N(0, 3), so it is the row maximum except with probability
  ~1e-10), and the draft equals that token with probability 0.7, otherwise a
  uniformly drawn different token;
* accepted lengths, where a workload supplies them: each draft position is
  kept with probability 0.7 independently and ``a`` is the length of the
  leading kept run, so ``P(a) = 0.3, 0.21, 0.147, 0.343`` at k = 3;
* "N(0, s)" is read as mean 0, standard deviation ``s``.
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

PLANTED_LOGIT = 24.0


@dataclass
class Workload:
    name: str
    B: int
    k: int                     # drafts per sequence (fixed), or max if ragged
    ragged_k: bool             # k_b ~ U{1..k}
    ctx: Tuple[int, int]       # L_b ~ U[lo, hi] (inclusive)
    ctx_fixed: Optional[List[int]] = None
    P: int = 64
    Hq: int = 32
    Hkv: int = 8
    D: int = 128
    attn_dtype: torch.dtype = torch.bfloat16
    H: int = 32
    dk: int = 128
    dv: int = 128
    gdn_dtype: torch.dtype = torch.bfloat16
    gdn_init: str = 'sigmoid'  # alpha/beta recipe: 'sigmoid' or 'uniform'
    qk_norm: str = 'qk'        # which of q, k are L2-normalised
    V: int = 151936
    logit_dtype: torch.dtype = torch.bfloat16
    draft_sigma: float = 0.78
    layers: List[str] = field(default_factory=list)   # 'gdn' / 'attn'
    accept_modes: Tuple[str, ...] = ()
    pool_factor: float = 1.0   # physical pages / pages needed
    min_pool_pages: int = 0
    conv_K: int = 4            # short-convolution width of the linear-attention layers

    @property
    def conv_C(self):
        """Channels through the short convolution: the q, k and v features."""
        return self.H * (2 * self.dk + self.dv)

    @property
    def max_T(self):
        return self.k + 1

    @property
    def max_pages_per_seq(self):
        hi = max(self.ctx_fixed) if self.ctx_fixed else self.ctx[1]
        return -(-(hi + self.max_T) // self.P)


def _hybrid(groups):
    return ['gdn', 'gdn', 'gdn', 'attn'] * groups


WORKLOADS = [
    # 0: tiny fp32 verify step.
    Workload('tiny_fp32_step', B=2, k=3, ragged_k=False, ctx=(37, 50),
             ctx_fixed=[37, 50], P=16, Hq=4, Hkv=2, D=64,
             attn_dtype=torch.float32, H=4, dk=64, dv=64,
             gdn_dtype=torch.float32, gdn_init='uniform', qk_norm='k',
             V=1000, logit_dtype=torch.float32, draft_sigma=0.85,
             layers=['gdn', 'attn'], accept_modes=('greedy', 'rejection'),
             min_pool_pages=12),
    # 1: paged verification attention alone.
    Workload('paged_verify_attention', B=32, k=3, ragged_k=False,
             ctx=(512, 4096), layers=['attn']),
    # 2: GDN verify + commit alone.
    Workload('gdn_verify_commit', B=64, k=3, ragged_k=False, ctx=(0, 0),
             layers=['gdn']),
    # 3: full hybrid step, 48 GDN + 16 attention layers.
    Workload('hybrid_step_64l', B=64, k=3, ragged_k=False, ctx=(2048, 8192),
             layers=_hybrid(16), accept_modes=('greedy', 'rejection')),
    # 4: stress, ragged drafts and long fragmented contexts; one 3:1 group.
    Workload('stress_ragged_long', B=256, k=7, ragged_k=True,
             ctx=(16384, 32768), layers=_hybrid(1),
             accept_modes=('rejection',), pool_factor=1.25),
]


def generator(seed, device='cpu'):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


@dataclass
class Batch:
    B: int
    max_T: int
    T: List[int]               # host copy of T_b
    ctx: List[int]             # host copy of L_b before the step
    cu_seqlens: torch.Tensor   # int32 [B+1]
    ctx_lens: torch.Tensor     # int32 [B]
    block_table: torch.Tensor  # int32 [B, max_pages_per_seq], -1 unused
    num_pages: int
    P: int

    @property
    def total_T(self):
        return int(sum(self.T))


def make_batch(w: Workload, seed: int, device='cpu', ctx_override=None,
               k_override=None, reserve=0) -> Batch:
    """Draft counts, context lengths and a shuffled paged block table.

    The table of sequence b covers ``ctx_b + T_b + reserve`` positions
    (``reserve`` leaves room for later steps)."""
    g = generator(seed)                         # host draws: small
    B = w.B
    if k_override is not None:
        ks = list(k_override)
    elif w.ragged_k:
        ks = torch.randint(1, w.k + 1, (B,), generator=g).tolist()
    else:
        ks = [w.k] * B
    T = [k + 1 for k in ks]
    if ctx_override is not None:
        ctx = list(ctx_override)
    elif w.ctx_fixed is not None:
        ctx = list(w.ctx_fixed)
    else:
        ctx = torch.randint(w.ctx[0], w.ctx[1] + 1, (B,), generator=g).tolist()
    P = w.P
    need = [-(-(L + t + reserve) // P) for L, t in zip(ctx, T)]
    max_pages = max(w.max_pages_per_seq, max(need))
    total_need = sum(need)
    num_pages = max(int(round(total_need * w.pool_factor)), w.min_pool_pages,
                    total_need)
    perm = torch.randperm(num_pages, generator=g)
    table = torch.full((B, max_pages), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        table[b, :need[b]] = perm[off:off + need[b]].to(torch.int32)
        off += need[b]
    cu = torch.zeros(B + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(T, dtype=torch.int32), 0)
    return Batch(B=B, max_T=max(T) if k_override is not None else w.max_T,
                 T=T, ctx=ctx, cu_seqlens=cu.to(device),
                 ctx_lens=torch.tensor(ctx, dtype=torch.int32, device=device),
                 block_table=table.to(device), num_pages=num_pages, P=P)


def _randn(shape, g, device, dtype, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    return x.to(dtype)


def _l2n(x):
    return x / x.norm(dim=-1, keepdim=True)


def make_attn_layer(w: Workload, batch: Batch, seed: int, device='cpu'):
    """q / k_new / v_new rows and a K/V page pool, all ~N(0, 1)."""
    g = generator(seed, device)
    Tt = batch.total_T
    shape_pool = (batch.num_pages, w.Hkv, batch.P, w.D)
    return {
        'q': _randn((Tt, w.Hq, w.D), g, device, w.attn_dtype),
        'k_new': _randn((Tt, w.Hkv, w.D), g, device, w.attn_dtype),
        'v_new': _randn((Tt, w.Hkv, w.D), g, device, w.attn_dtype),
        'k_cache': _randn(shape_pool, g, device, w.attn_dtype),
        'v_cache': _randn(shape_pool, g, device, w.attn_dtype),
    }


def make_attn_layer_kv8(w: Workload, batch: Batch, seed: int, device='cpu'):
    """INT8 pages: bf16 q / k_new / v_new rows ~N(0, 1); page codes drawn as
    round(N(0, 32^2)) clipped to +-127 (a bell-shaped histogram over the code
    range, as calibrated scales give); per-(KV head, channel) fp32 scales
    ~U(0.5, 1.5) * 4 / 127, so rows of the same N(0, 1) data span the range."""
    g = generator(seed, device)
    Tt = batch.total_T
    shape_pool = (batch.num_pages, w.Hkv, batch.P, w.D)

    def codes():
        c = torch.randn(shape_pool, generator=g, device=device).mul_(32.0).round_()
        return c.clamp_(-127, 127).to(torch.int8)

    return {
        'q': _randn((Tt, w.Hq, w.D), g, device, torch.bfloat16),
        'k_new': _randn((Tt, w.Hkv, w.D), g, device, torch.bfloat16),
        'v_new': _randn((Tt, w.Hkv, w.D), g, device, torch.bfloat16),
        'k_cache': codes(),
        'v_cache': codes(),
        'k_scale': (torch.rand((w.Hkv, w.D), generator=g, device=device) + 0.5).mul_(4.0 / 127),
        'v_scale': (torch.rand((w.Hkv, w.D), generator=g, device=device) + 0.5).mul_(4.0 / 127),
    }


def make_gdn_layer(w: Workload, batch: Batch, seed: int, device='cpu',
                   num_slots=None, state_dtype=torch.float32):
    """State bank ~N(0, 0.1) (drawn in fp32, stored as ``state_dtype``),
    q/k/v ~N(0, 1) (L2-normalised as the workload says, before rounding),
    gates alpha / beta in fp32."""
    g = generator(seed, device)
    Tt = batch.total_T
    ns = batch.B if num_slots is None else num_slots
    state = torch.randn((ns, w.H, w.dv, w.dk), generator=g, device=device,
                        dtype=torch.float32).mul_(0.1)
    q = torch.randn((Tt, w.H, w.dk), generator=g, device=device)
    k = torch.randn((Tt, w.H, w.dk), generator=g, device=device)
    v = torch.randn((Tt, w.H, w.dv), generator=g, device=device)
    if 'q' in w.qk_norm:
        q = _l2n(q)
    if 'k' in w.qk_norm:
        k = _l2n(k)
    if w.gdn_init == 'uniform':
        alpha = 0.9 + 0.1 * torch.rand((Tt, w.H), generator=g, device=device)
        beta = torch.rand((Tt, w.H), generator=g, device=device)
    else:
        alpha = torch.sigmoid(2.0 + 0.5 * torch.randn(
            (Tt, w.H), generator=g, device=device))
        beta = torch.sigmoid(torch.randn((Tt, w.H), generator=g,
                                         device=device))
    return {
        'state': state.to(state_dtype),
        'q': q.to(w.gdn_dtype), 'k': k.to(w.gdn_dtype), 'v': v.to(w.gdn_dtype),
        'alpha': alpha.float().contiguous(), 'beta': beta.float().contiguous(),
    }


def make_conv_layer(w: Workload, batch: Batch, seed: int, device='cpu',
                    num_slots=None, bias=True, C=None):
    """Short-convolution inputs: rolling state and inputs ~N(0, 1) in the GDN
    I/O dtype, taps ~N(0, 1/K) and bias ~N(0, 0.1) in fp32.  ``C`` overrides
    the channel count (default: the layer's q, k and v features)."""
    g = generator(seed, device)
    Tt, C, K = batch.total_T, (w.conv_C if C is None else C), w.conv_K
    ns = batch.B if num_slots is None else num_slots
    state = torch.randn((ns, K - 1, C), generator=g, device=device)
    x = torch.randn((Tt, C), generator=g, device=device)
    weight = torch.randn((C, K), generator=g, device=device).mul_(K ** -0.5)
    b = torch.randn((C,), generator=g, device=device).mul_(0.1) if bias else None
    return {
        'state': state.to(w.gdn_dtype), 'x': x.to(w.gdn_dtype),
        'weight': weight.float().contiguous(),
        'bias': None if b is None else b.float().contiguous(),
    }


def make_state_slots(batch: Batch, num_slots: int, seed: int, device='cpu'):
    """A random injective sequence -> state-slot map (fixed-state bank)."""
    g = generator(seed)
    perm = torch.randperm(num_slots, generator=g)[:batch.B]
    return perm.to(torch.int32).to(device)


def make_commit_len(batch: Batch, seed: int, p_keep=0.7, device='cpu'):
    """c_b = a_b + 1 with a_b the leading run of independent keeps."""
    g = generator(seed)
    c = []
    for t in batch.T:
        a = 0
        keep = (torch.rand(t - 1, generator=g) < p_keep).tolist()
        while a < t - 1 and keep[a]:
            a += 1
        c.append(a + 1)
    return torch.tensor(c, dtype=torch.int32, device=device)


def make_accept(w: Workload, batch: Batch, seed: int, mode: str,
                device='cpu', p_match=0.7):
    """Target (and draft) logits, draft tokens and uniforms.

    Target logits ~N(0, 3) in the workload's logit dtype.  Greedy: planted
    row maxima and drafts that hit them with probability ``p_match``.
    Rejection: draft logits = target + N(0, draft_sigma), drafts drawn from
    the draft distribution (Gumbel-max), uniforms in [0, 1) fp32.
    """
    g = generator(seed, device)
    Tt, B, V = batch.total_T, batch.B, w.V
    nd = Tt - B
    target = torch.randn((Tt, V), generator=g, device=device).mul_(3.0)
    cu = batch.cu_seqlens.tolist()
    # Row indices of target rows that are compared with a draft, and the
    # packed index of that draft.
    rows = [cu[b] + i for b in range(B) for i in range(batch.T[b] - 1)]
    out = {}
    if mode == 'greedy':
        gh = generator(seed + 7919)
        plant = torch.randint(0, V, (nd,), generator=gh)
        hit = torch.rand(nd, generator=gh) < p_match
        other = (plant + torch.randint(1, V, (nd,), generator=gh)) % V
        drafts = torch.where(hit, plant, other).to(torch.int32)
        if nd:
            target[torch.tensor(rows, device=device),
                   plant.to(device)] = PLANTED_LOGIT
        out['target_logits'] = target.to(w.logit_dtype)
        out['draft_tokens'] = drafts.to(device)
        out['draft_logits'] = None
        out['u_accept'] = None
        out['u_final'] = None
    elif mode == 'rejection':
        target_c = target.to(w.logit_dtype)
        if nd:
            base = target_c[torch.tensor(rows, device=device)].float()
            draft = base + w.draft_sigma * torch.randn(
                (nd, V), generator=g, device=device)
            draft_c = draft.to(w.logit_dtype)
            u = torch.rand((nd, V), generator=g, device=device)
            u.clamp_(min=1e-12)
            gumbel = -torch.log(-torch.log(u))
            drafts = torch.argmax(draft_c.float() + gumbel, dim=-1)
            del u, gumbel, draft
        else:
            draft_c = torch.empty((0, V), dtype=w.logit_dtype, device=device)
            drafts = torch.empty((0,), dtype=torch.int64, device=device)
        out['target_logits'] = target_c
        out['draft_logits'] = draft_c
        out['draft_tokens'] = drafts.to(torch.int32)
        out['u_accept'] = torch.rand((nd,), generator=g, device=device)
        out['u_final'] = torch.rand((B,), generator=g, device=device)
    else:
        raise ValueError(mode)
    return out
