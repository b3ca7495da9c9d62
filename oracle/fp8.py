"""fp64 CPU oracle for the FP8 forward pass: decoding of 8-bit inputs and
attention on the decoded values.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import or call this module;
the product path never touches it, and it imports nothing from that path.

The pages name FP8 only as a feature of FlashAttention-3 on H100
(explainer page "Flash Attention", section "Versionen: Flash Attention 2 und
Flash Attention 3", hardware-accelerated FP8 quantisation; glossary page
"Flash Attention", section "FlashAttention-2, -3 and -4", close to
1.2 PFLOP/s in FP8).  They fix neither the 8-bit format nor the scaling.
Readings taken:

* the format is E4M3 of the OCP 8-bit floating-point specification (the fp8
  operand format of gfx950's matrix cores): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m * 2^-9; the
  all-ones exponent with all-ones mantissa is NaN; there is no infinity, and
  the largest finite value is 1.75 * 2^8 = 448;
* every (batch, head) of Q, K and V carries one fp32 descale factor: the
  real value of a code c is decode(c) * descale;
* what the forward computes is ordinary attention (the definition in
  ``attention.py``) of the decoded, descaled tensors.  The kernel's own
  rounding of the probabilities to E4M3 before the P V product is an error
  that the parity tolerance covers; the oracle does not model it.
"""

from __future__ import annotations

import numpy as np

from . import attention

__all__ = ["decode_e4m3", "dequantize", "forward_fp8", "forward_rows_fp8"]

E4M3_MAX = 448.0


def decode_e4m3(codes):
    """Real values (fp64) of OCP E4M3 byte codes (any integer array 0..255)."""
    c = np.asarray(codes, dtype=np.int64)
    if c.size and (c.min() < 0 or c.max() > 255):
        raise ValueError("E4M3 codes are bytes")
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp_field = (c >> 3) & 0xF
    mant = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + mant / 8.0) * np.exp2(exp_field.astype(np.float64) - 7.0)
    subnormal = sign * (mant / 8.0) * 2.0 ** -6
    val = np.where(exp_field == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def dequantize(codes, descale):
    """[B, N, H, d] codes and [B, H] descale factors -> fp64 values."""
    descale = np.asarray(descale, dtype=np.float64)
    return decode_e4m3(codes) * descale[:, None, :, None]


def forward_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal, heads=None, window=None):
    """Attention of the decoded inputs: O [B,N,H,d] and LSE [B,H,N] in fp64.

    q8 is [B,N,H,d], k8 and v8 are [B,N,H_kv,d] byte codes; the descale
    arrays are [B,H] for Q and [B,H_kv] for K and V.
    """
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    return attention.forward(q, k, v, scale, causal, heads=heads, window=window)


def forward_rows_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale, causal, picks, window=None):
    """Selected query rows (b, h, i) of ``forward_fp8``, evaluated row by row."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    return attention.forward_rows(q, k, v, scale, causal, picks, window=window)
