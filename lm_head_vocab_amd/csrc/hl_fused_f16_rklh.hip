// Fused-kernel instances: dtype f16, distillation mode reverse KL, Hinton temperature.
#include "hl_device.cuh"

namespace hl {

FusedLauncher get_fused_f16_rklh(int block, int nvec, bool softcap) {
    HL_FUSED_CASE(hl::F16T, 256, 1, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 256, 2, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 256, 4, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 1024, 2, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 1024, 4, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 1024, 6, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 1024, 8, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 1024, 10, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 6, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 8, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 9, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 10, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 12, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F16T, 512, 13, hl::TM_RKL_H)
    return nullptr;
}

}  // namespace hl
