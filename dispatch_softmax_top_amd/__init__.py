"""MI355X-native pooled-wave MoE dispatch share: HIP kernels behind a C ABI
(libmoe.so, include/moe.h) with a thin ctypes binding of the same names."""
from ._lib import (EXPORTS, MOE_CALL_BANK, MOE_CALL_COMBINE, MOE_CALL_COMBINE_BWD,  # noqa: F401
                   MOE_CALL_COMBINE_SHARED, MOE_CALL_FFN, MOE_CALL_FFN_BWD, MOE_CALL_PACK,
                   MOE_CALL_PACK_BWD, MOE_CALL_ROUTE, MOE_ROUTE_RENORM, LIB_PATH, MoeDims,
                   MOE_WAVES_CHUNKS, MOE_WAVES_TOKENS, MoeError, lib,
                   moe_abi_version, moe_balance_bias, moe_bank, moe_capacity, moe_combine,
                   moe_combine_backward, moe_combine_shared, moe_expert_counts, moe_expert_ffn,
                   moe_expert_ffn_backward, moe_pack_backward, moe_pack_waves,
                   moe_pack_waves_noalloc, MOE_NOALLOC_SCRATCH_BYTES,
                   moe_profile_collect, moe_profile_enable, moe_profile_read, moe_profile_reset,
                   moe_route, moe_route_backward, moe_route_biased, moe_shared_swiglu,
                   moe_workspace_bytes)
