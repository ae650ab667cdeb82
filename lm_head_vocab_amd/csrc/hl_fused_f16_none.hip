// Fused-kernel instances: dtype f16, distillation mode none.
#include "hl_device.cuh"

namespace hl {

FusedLauncher get_fused_f16_none(int block, int nvec, bool softcap) {
    HL_FUSED_CASE(hl::F16T, 256, 1, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 256, 2, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 256, 4, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 2, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 4, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 6, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 8, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 10, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 12, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 14, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 16, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 18, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 1024, 20, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 512, 10, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 512, 12, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 512, 16, hl::TM_NONE)
    HL_FUSED_CASE(hl::F16T, 512, 20, hl::TM_NONE)
    return nullptr;
}

}  // namespace hl
