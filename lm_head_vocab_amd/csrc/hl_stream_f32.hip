// Forward-only streaming statistics kernel instances (every teacher mode,
// softcap on and off): dtype f32.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_stream_f32, hl::launch_stream_stats, hl::F32T)

}  // namespace hl
