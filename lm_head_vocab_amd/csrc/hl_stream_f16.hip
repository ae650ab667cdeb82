// Forward-only streaming statistics kernel instances (every teacher mode,
// softcap on and off): dtype f16.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_stream_f16, hl::launch_stream_stats, hl::F16T)

}  // namespace hl
