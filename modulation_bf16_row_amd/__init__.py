"""BF16 DiT row epilogues for MI355X (gfx950): a C-ABI HIP library
(``libdit.so``, declared in ``include/dit.h`` and ``include/dit_producers.h``)
and its Python binding.

The binding loads the library on first use and raises if it is missing; it
never falls back to another implementation.  The probes and the timing hook
come from ``libdit_probe.so`` (the same kernel objects, instrumented).
"""
from .binding import (  # noqa: F401
    FAST, LOSSLESS, DitError, DitHipError, DitInvalid, DitUnsupported, LIB_PATH,
    PROBE_LIB_PATH, instrumented, lib, probe_lib,
    dit_ln_modulate, dit_ln_modulate_fp8, dit_gate_add_ln_modulate, dit_gate_add_ln_modulate_fp8,
    dit_modulate_scale_shift, dit_qk_norm_rope, dit_qk_norm_rope_packed, dit_residual_gate_add,
    dit_rmsnorm_scale, dit_rmsnorm_tanh_residual, dit_probe_bf16_round, dit_probe_f32,
    dit_probe_row_sum, dit_probe_unary, dit_probe_copy, dit_probe_fp8, dit_time_next_launch,
    dit_wan_modulation_table,
)
