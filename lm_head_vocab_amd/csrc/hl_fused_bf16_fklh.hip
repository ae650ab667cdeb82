// Fused-kernel instances: dtype bf16, distillation mode forward KL, Hinton temperature.
#include "hl_device.cuh"

namespace hl {

FusedLauncher get_fused_bf16_fklh(int block, int nvec, bool softcap) {
    HL_FUSED_CASE(hl::BF16T, 256, 1, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 256, 2, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 256, 4, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 1024, 2, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 1024, 4, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 1024, 6, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 1024, 8, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 1024, 10, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 6, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 8, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 9, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 10, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 12, hl::TM_FKL_H)
    HL_FUSED_CASE(hl::BF16T, 512, 13, hl::TM_FKL_H)
    return nullptr;
}

}  // namespace hl
