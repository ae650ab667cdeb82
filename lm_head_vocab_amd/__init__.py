"""MI355X-native fused LM-head loss: one softmax per row, every requested loss
and metric, one combined gradient (C ABI in include/headloss.h, HIP kernels
in csrc/, this thin binding on top)."""

from ._binding import (  # noqa: F401
    ACCUMULATE, CE, ENTROPY, FDCE, FKL, GRPO, GSPO, HINTON, HL_BF16, HL_ERR_HIP, HL_ERR_INVALID_ARG,
    HL_ERR_MISSING_INPUT, HL_ERR_UNSUPPORTED, HL_ERR_WORKSPACE, HL_F16, HL_F32, HL_OK,
    LIB_PATH, NUM_SCALARS, RKL, ROW_COLS, SLOTS, ZLOSS, HeadLossError, Plan,
    Weights, exported_functions_in_header, load_library, scalars_dict, status_str, stream_ceiling,
)
