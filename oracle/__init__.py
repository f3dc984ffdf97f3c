"""CPU oracle for the block speculative-verification step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers, tables or pre/post-processing) and it
imports nothing from ``block_draft_verification_spec_amd``.

Everything here is plain NumPy in float64.  Inputs arrive as NumPy arrays
(bf16 / fp32 values are converted to float64 exactly by the caller); every
reduction is a plain loop or a library primitive (``@``, ``np.sum``,
``np.cumsum``, ``np.argmax``) on float64 data, with no blocking, fusion or
reordering beyond what each definition states.

Sources (the pages are scraped pull-request discussions; none of them prints
a formula, so each function states which published definition it writes out):

* "InternLM/lmdeploy pull request 5019" (TurboMind speculative decoding):
  feature list -- block speculative verification with paged verification
  attention and gated-delta-rule verify / commit kernels; "Two fixes", item 2
  -- the recurrent-state commit runs after the speculative round has accepted
  tokens and computes in float.
* "microsoft/onnxruntime-genai pull request 2457" (Expose speculative draft
  proposals through Engine APIs): commit messages on the direct arena commit
  (no snapshot, no replay forward), on the V-major float32 GatedDeltaNet state
  and the packed varlen operator with ``cu_seqlens`` and pre-cast gates, on
  ``CommitPrefix`` picking the state of the accepted prefix, and on the single
  device argmax readback of the verify rows.
* "InternLM/lmdeploy pull request 3945" ([Feature]: Support speculative
  decoding): review of ``flatten_kv_cache.py`` (paged K/V gathered into dense
  per-sequence states) and of ``reject_sampler.py`` (output ``[batch,
  max_spec_len + 1]`` padded with -1).
* Gated delta rule: S. Yang, J. Kautz, A. Hatamizadeh, "Gated Delta Networks:
  Improving Mamba2 with Delta Rule", ICLR 2025.
* Speculative sampling: Y. Leviathan, M. Kalman, Y. Matias, "Fast Inference
  from Transformers via Speculative Decoding", ICML 2023 (Algorithm 1,
  Theorem 1); C. Chen et al., "Accelerating Large Language Model Decoding with
  Speculative Sampling", 2023.

Parity status: every function in this package is pinned by a ``-m "not gpu"``
test against something other than itself (closed forms, special cases,
library routines, brute force, exact enumeration or Monte-Carlo); see
``tests/test_oracle_*.py``.
"""

from .attention import append_kv, gather_context, verify_attention
from .gdn import GDN_COMMIT_ONLY, GDN_VERIFY_COMMIT, GDN_VERIFY_ONLY, gdn_step
from .accept import greedy_accept, icdf, rejection_accept, softmax64
from .short_conv import CONV_COMMIT_ONLY, CONV_VERIFY_COMMIT, CONV_VERIFY_ONLY, conv_step
from .kv_int8 import (append_kv_int8, dequantize_pool, dequantize_rows, quantize_int8,
                      verify_attention_int8)
from .step import verify_step
from .checkpoint import (conv_checkpoints, conv_commit_prefix, gdn_checkpoints,
                         gdn_commit_prefix)

__all__ = [
    "append_kv", "gather_context", "verify_attention",
    "GDN_VERIFY_COMMIT", "GDN_VERIFY_ONLY", "GDN_COMMIT_ONLY", "gdn_step",
    "greedy_accept", "rejection_accept", "softmax64", "icdf",
    "CONV_VERIFY_COMMIT", "CONV_VERIFY_ONLY", "CONV_COMMIT_ONLY", "conv_step",
    "quantize_int8", "dequantize_rows", "dequantize_pool", "append_kv_int8",
    "verify_attention_int8",
    "verify_step",
    "gdn_checkpoints", "gdn_commit_prefix", "conv_checkpoints", "conv_commit_prefix",
]
