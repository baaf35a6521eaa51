"""MI355X (gfx950) library for the RoPE-aligned Q/K rotation and INT4 KV4 path.

The compute lives in the HIP library librrp.so (C-ABI: include/rrp.h); this
package is its torch binding plus the seeded synthetic workloads.
"""
from .api import (ESTIMATORS, RRP_BF16, RRP_F32, RRP_ROPE_HALF_SPLIT, RRP_ROPE_INTERLEAVED, PreparedCall,
                  RrpError, RrpShape, angle_sets, calibrate_angles, calibrate_angles_noalloc,
                  calibrate_workspace_bytes, decode_scores, layer_shape, prepare_decode_scores,
                  prepare_rotate_quantize_qk,
                  new_kv4_cache, new_moments, quant_error_stats, quant_error_stats_workspace_bytes,
                  quant_error_sweep, quant_error_sweep_workspace_bytes, rotate_quantize_qk, rotate_quantize_qkv,
                  sweep_supports)

__all__ = ["ESTIMATORS", "RRP_BF16", "RRP_F32", "RRP_ROPE_HALF_SPLIT", "RRP_ROPE_INTERLEAVED", "PreparedCall",
           "prepare_decode_scores", "prepare_rotate_quantize_qk", "RrpError",
           "RrpShape", "angle_sets", "calibrate_angles", "calibrate_angles_noalloc", "calibrate_workspace_bytes",
           "decode_scores",
           "layer_shape", "new_kv4_cache", "new_moments", "quant_error_stats", "quant_error_stats_workspace_bytes",
           "quant_error_sweep", "quant_error_sweep_workspace_bytes", "rotate_quantize_qk", "rotate_quantize_qkv",
           "sweep_supports"]
