// Row-wise kernel instances (every teacher mode, softcap on and off): dtype bf16.
#include "hl_device.cuh"

namespace hl {

HL_ROWWISE_GETTER(get_rowwise_bf16, hl::BF16T)

}  // namespace hl
