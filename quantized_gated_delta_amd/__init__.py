"""Packed low-bit gated Delta-rule recurrent-state pool for AMD MI355X.

The compute path is the HIP library ``libsq.so`` (kernels for gfx950) behind
the C ABI in ``include/sq.h``; ``sq`` is its thin ctypes binding.
"""
from .sq import (SQ_BF16, SQ_EHIP, SQ_EINVAL, SQ_ENOMEM, SQ_EUNSUPPORTED, SQ_F32, SQ_GATE_GDN,
                 SQ_GATE_KDA, SQ_OK, SQError, StatePool, header_symbols, lib, sq_arith_selfcheck,
                 sq_check_slots,
                 sq_decode_step, sq_decode_update, sq_dequant_state, sq_device_copy,
                 sq_f32_decode_step, sq_issue_probe, SQ_PROBE_OPS_PER_LAUNCH, SQ_PROBE_COUNT,
                 SQ_PROBE_FMA_F32, SQ_PROBE_MUL_F32, SQ_PROBE_MAX3_F32, SQ_PROBE_CVT_BYTE,
                 SQ_PROBE_BFE, SQ_PROBE_ALIGNBIT, SQ_PROBE_FMA_F64, SQ_PROBE_FMA_CVT_PAIR,
                 sq_last_error, sq_pool_bytes, sq_pool_create, sq_pool_destroy, sq_pool_layout,
                 sq_pool_set_row_impact, sq_quant_state, sq_split_step_noalloc,
                 SQ_SPLIT_SCRATCH_BYTES, version)

__all__ = [n for n in dir() if n.startswith(("sq_", "SQ", "StatePool", "lib", "header", "version"))]
