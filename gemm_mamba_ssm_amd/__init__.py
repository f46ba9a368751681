"""w8a16 block-scaled FP8 projections (Mamba-2 in_proj / out_proj) for MI355X.

``out[m, n] = sum_k A[m, k] * E4M3(Wq[n, k]) * scale[n // 128, k // 128]``
with BF16 activations, E4M3 weight bytes, a BF16 128x128 block-scale grid,
fp32 accumulation and BF16 output, computed by the hand-written gfx950 HIP
kernels in ``libw8a16.so`` (C ABI: ``include/w8a16.h``).

* ``w8a16_gemv``    - decode, M = 1..16 rows
* ``w8a16_gemm``    - prefill, any M
* ``w8a16_dequant`` - dequantize only (test path for the decode and scale index)
* ``w8a16_rmsnorm``, ``w8a16_gemv_fused``, ``w8a16_gemm_residual`` - the
  layer's norm prologues and residual epilogue around the projections
* ``w8a16_conv1d_update``, ``w8a16_ssm_decode`` - the Mamba-2 decode step
  between the projections; ``w8a16_gemv_in_proj`` - in_proj with its norm and
  the conv1d update fused
"""
from .binding import (W8A16Error, w8a16_conv1d_update, w8a16_dequant, w8a16_gemm,  # noqa: F401
                      w8a16_gemm_residual, w8a16_gemv, w8a16_gemv_fused, w8a16_gemv_in_proj, w8a16_rmsnorm,
                      w8a16_ssm_decode)
