"""Oracle for INT8 per-channel KV pages in the verification attention.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages build the main model with an INT8 KV cache
(``kv_cache_quant_type=int8_per_channel``) whose scales are calibrated per
main-model attention layer and read from a scale file; the MTP head, a single
layer, then keeps an unquantized cache ("microsoft/onnxruntime-genai pull
request 2457", commit message on the MTP head inheriting the KV quantization
options).  They print no formula.  The reading written out here is plain
symmetric per-channel quantization with a static scale for every
(KV head, channel) of a layer, one set for K and one for V:

    code = clip(round_half_even(x / s), -127, 127)      (int8)
    x~   = s * code                                     (dequantized)

The integer decision is taken in fp32: ``x`` is the fp32 value of the stored
activation (bf16 widens exactly), ``s`` the fp32 scale, ``x / s`` the
correctly rounded fp32 quotient.

Attention over an INT8 cache is the plain verification attention of
``attention.py`` over the dequantized cache.  The in-flight keys and values
enter as their dequantized codes too: they are written into the INT8 pages
(the idempotent KV append) and every position is read back from the cache
alike.
"""

import numpy as np

from .attention import append_kv, verify_attention

QMAX = 127


def quantize_int8(x, scale):
    """Codes of rows ``x[..., Hkv, D]`` under per-channel scales ``scale[Hkv, D]``."""
    xf = np.asarray(x, dtype=np.float32)
    sf = np.asarray(scale, dtype=np.float32)
    with np.errstate(divide='ignore', invalid='ignore'):
        ratio = xf / sf                       # fp32 quotient, correctly rounded
    return np.clip(np.rint(ratio), -QMAX, QMAX).astype(np.int8)


def dequantize_rows(codes, scale):
    """``codes[..., Hkv, D]`` -> float64 ``scale * code``."""
    return np.asarray(codes, dtype=np.float64) * np.asarray(scale, dtype=np.float64)


def dequantize_pool(codes, scale):
    """Pool ``codes[num_pages, Hkv, P, D]`` -> float64, channel (h, d) times ``scale[h, d]``."""
    s = np.asarray(scale, dtype=np.float64)
    return np.asarray(codes, dtype=np.float64) * s[None, :, None, :]


def append_kv_int8(k_cache, v_cache, k_new, v_new, k_scale, v_scale, block_table,
                   ctx_lens, cu_seqlens, page_size):
    """INT8 pools with the in-flight rows' codes written at ``L_b + j``."""
    return append_kv(k_cache, v_cache, quantize_int8(k_new, k_scale),
                     quantize_int8(v_new, v_scale), block_table, ctx_lens, cu_seqlens,
                     page_size)


def verify_attention_int8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale,
                          block_table, ctx_lens, cu_seqlens, page_size, scale=None):
    """Verification attention over INT8 pages, float64.  Returns ``o[total_T, Hq, D]``."""
    kq = dequantize_rows(quantize_int8(k_new, k_scale), k_scale)
    vq = dequantize_rows(quantize_int8(v_new, v_scale), v_scale)
    return verify_attention(q, kq, vq, dequantize_pool(k_cache, k_scale),
                            dequantize_pool(v_cache, v_scale), block_table, ctx_lens,
                            cu_seqlens, page_size, scale)
