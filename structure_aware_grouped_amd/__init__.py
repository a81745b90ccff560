"""RaggedShard / DBuffer layout transforms for MI355X (gfx950).

The work runs in librs_hip.so (hand-written HIP kernels behind a C ABI, see
include/rs.h); ``binding`` exposes its calls under the same names.
"""
from .binding import (  # noqa: F401
    Plan,
    PlanSpec,
    plan_from_json,
    plan_to_json,
    rs_adam8_step,
    RsError,
    load,
    rs_block_dequant,
    rs_block_quant,
    rs_block_quant_noalloc,
    rs_pack_scatter,
    rs_plan_build,
    rs_plan_load,
    rs_unpack_dequant,
    rs_unpack_gathered,
)
