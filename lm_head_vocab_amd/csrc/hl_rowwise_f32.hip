// Row-wise kernel instances (every teacher mode, softcap on and off): dtype f32.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_rowwise_f32, hl::launch_rowwise, hl::F32T)

}  // namespace hl
