// Row-wise kernel instances (every teacher mode, softcap on and off): dtype bf16.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_rowwise_bf16, hl::launch_rowwise, hl::BF16T)

}  // namespace hl
