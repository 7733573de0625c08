"""int3-g64 quantize / pack / dequantize-multiply for MI355X (gfx950).

The compute lives in libqt.so (hand-written HIP kernels behind the C ABI in
include/qt.h); this package only marshals torch device tensors into that ABI.
"""
from .qt import (QtError, QT_BF16, QT_F32, lib, qt_groups, qt_hessian_diag,
                 qt_hessian_diag_noalloc, qt_hessian_scratch_bytes, qt_hessian_workspace_bytes, qt_matmul_i3, qt_matmul_i4, qt_matvec_i3,
                 qt_matvec_i3_grouped, qt_matvec_i4, qt_matvec_i4_grouped, qt_pack_i3, qt_pack_i4, qt_packed_bytes,
                 qt_packed_bytes_i4, qt_quantize_g64, qt_quantize_g64_i4,
                 qt_quantize_g64_signed, qt_status_str, qt_hessian_full, qt_gptq_factor,
                 qt_gptq_i3, qt_gptq_proxy, qt_hessian_full_workspace_bytes,
                 qt_gptq_factor_workspace_bytes, qt_gptq_workspace_bytes,
                 qt_gptq_proxy_workspace_bytes, qt_moe_layer, qt_moe_layer_workspace_bytes)

__all__ = ["QtError", "QT_BF16", "QT_F32", "lib", "qt_groups", "qt_hessian_diag",
           "qt_hessian_diag_noalloc", "qt_hessian_scratch_bytes", "qt_hessian_workspace_bytes", "qt_matmul_i3", "qt_matmul_i4", "qt_matvec_i3",
           "qt_matvec_i3_grouped", "qt_matvec_i4", "qt_matvec_i4_grouped", "qt_pack_i3", "qt_pack_i4",
           "qt_packed_bytes", "qt_packed_bytes_i4", "qt_quantize_g64", "qt_quantize_g64_i4",
           "qt_quantize_g64_signed", "qt_status_str", "qt_hessian_full", "qt_gptq_factor",
           "qt_gptq_i3", "qt_gptq_proxy", "qt_hessian_full_workspace_bytes",
           "qt_gptq_factor_workspace_bytes", "qt_gptq_workspace_bytes",
           "qt_gptq_proxy_workspace_bytes", "qt_moe_layer", "qt_moe_layer_workspace_bytes"]
