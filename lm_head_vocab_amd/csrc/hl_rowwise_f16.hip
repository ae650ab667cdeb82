// Row-wise kernel instances (every teacher mode, softcap on and off): dtype f16.
#include "hl_device.cuh"

namespace hl {

HL_ROWWISE_GETTER(get_rowwise_f16, hl::F16T)

}  // namespace hl
