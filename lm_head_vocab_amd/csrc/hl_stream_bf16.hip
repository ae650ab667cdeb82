// Forward-only streaming statistics kernel instances (every teacher mode,
// softcap on and off): dtype bf16.
#include "hl_device.cuh"

namespace hl {

HL_ROW_KERNEL_GETTER(get_stream_bf16, hl::launch_stream_stats, hl::BF16T)

}  // namespace hl
