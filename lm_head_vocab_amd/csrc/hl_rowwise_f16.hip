// Row-wise kernel instances (every teacher mode, softcap on and off): dtype f16.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_rowwise_f16, hl::launch_rowwise, hl::F16T)

}  // namespace hl
