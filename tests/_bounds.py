"""Error bars that follow from the arithmetic of the bf16 and e4m3 attention kernels.

Shared by the GPU parity tests.  Each bar is derived from the kernel's
rounding steps, not measured; the tests print the measured error beside it.

* Softmax weights.  The kernel rounds every weight to bf16 (round to nearest
  even, 8 significant bits: relative error at most u = 2^-8) and adds those
  rounded weights to the row sum, the same ones that multiply V.  The row sum
  is a weighted mean of the relative errors, so it is within a factor
  (1 +- 2^-8) of the sum of the exact-rounded-logit weights, and the LSE
  within -ln(1 - 2^-8) = 3.914e-3.
* Row-sum accumulation.  Each lane adds its positive terms in fp32 (about
  n_keys / 2 of them, then the two halves of a lane pair): recursive
  summation of n positive terms is within a relative (n - 1) * 2^-24, so at
  most n_keys * 2^-24 on the LSE.
* Logits.  bf16 products are exact in fp32; the MFMA accumulation over the
  head dim, the fp32 scale*log2(e), the fused scale-and-shift and v_exp_f32
  (about 1 ulp) each add relative errors near 2^-24 of the logit or of the
  weight: for logits of magnitude below 100 that is below 1e-4 on the LSE.
* e4m3 logits.  The e4m3 matrix instruction does not round its 64-product
  sums like fp32: measured on gfx950 it reached 2^-14.6 of the sum of the
  product magnitudes for normally distributed codes and 2^-11.8 for codes
  spread over the whole e4m3 range.  The bars take the worst case, 2^-11.8,
  times scale * max over visible keys of sum_d |q_d k_d| (dequantised), per
  row: a logit moves by at most that, and so does the LSE (a weighted mean of
  the logit errors).
"""

import math

import numpy as np

BF16_U = 2.0 ** -8
FP32_U = 2.0 ** -24
LOGIT_ROUNDING = 1e-4
E4M3_ACC = 2.0 ** -11.8


def lse_bound(n_keys):
    """Largest |LSE_kernel - LSE_exact| of the bf16 path for a row seeing n_keys keys."""
    return -math.log1p(-BF16_U) + n_keys * FP32_U + LOGIT_ROUNDING


def e4m3_logit_error(qd, kd, scale, q_index=None):
    """Per-row bound on the e4m3 matrix instruction's logit error: 2^-11.8 * scale *
    max_j sum_d |q_d k_jd| over every key of kd.  qd [B, H, n, D] (rows of the call,
    dequantised), kd [B, H, L, D] (dequantised).  Returns [B, H, n]."""
    qd = np.abs(np.asarray(qd, dtype=np.float64))
    kd = np.abs(np.asarray(kd, dtype=np.float64))
    if q_index is not None:
        qd = qd[:, :, np.asarray(q_index)]
    B, H = qd.shape[:2]
    out = np.zeros(qd.shape[:3])
    for b in range(B):
        for h in range(H):
            out[b, h] = (qd[b, h] @ kd[b, h].T).max(axis=1)
    return E4M3_ACC * scale * out
