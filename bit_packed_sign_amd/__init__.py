"""bit_packed_sign_amd -- 1-bit sign-packed GEMV / GEMM and XOR row patching on MI355X (gfx950).

The computation lives in libbin1.so (C ABI: include/bin1.h, HIP kernels in csrc/); the
functions below are its thin torch binding.  ``synth`` holds the seeded input generators.
"""
from .binding import (Bin1Error, ChainPlan, PatchTable, gemm_prefill, gemm_prefill_t2, gemv, gemv_group,  # noqa: F401
                      gemv_group_t2, gemv_noalloc, gemv_pm1, gemv_t2, gemv_workspace_bytes, gemv_ws, kernel_variant, lib,
                      mfma_rate, rank_rows_by_scale, stream_read, xor_bits_apply, xor_patch_apply,
                      xor_patch_apply_multi)
