"""CPU oracle of the MiniMax-H3 DiT forward -- test infrastructure.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never touches it.
"""
from .h3_block import (  # noqa: F401
    MOD_NAMES, adaln_modulate, apply_rope, attention, bf16_to_f64, bias, block_forward,
    WFMT_W8A8, block_steps, build_mod_table, dequant_int8_g32, dit_forward, layer_norm, linear,
    merge_heads, modulation_from_table, modulation_live, qkv_split, rms_norm,
    rope_angles, round_to_bf16, silu, swiglu, weight,
)
from .h3_io import SEGMENTS, embed_inputs, final_heads, segment_rows, velocity_forward  # noqa: F401
from .h3_w8a8 import ACCEPTED_GROUPS, linear_w8a8, linear_w8a8_grouped, quantize_groups, quantize_rows  # noqa: F401
from .h3_sparse import attention_sparse, selected_keys  # noqa: F401
from .h3_sampler import (  # noqa: F401
    base_grid, denoise, euler, extrapolate, fresh_passes, schedule, shift_sigmas,
)
