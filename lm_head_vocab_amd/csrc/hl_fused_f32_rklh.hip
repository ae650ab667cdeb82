// Fused-kernel instances: dtype f32, distillation mode reverse KL, Hinton temperature.
#include "hl_device.cuh"

// fp32 teacher slices hold at most 4 vectors per tensor (the fp64 element path
// of the fp32 instances needs the registers; see kF32TeacherNvec).

namespace hl {

FusedLauncher get_fused_f32_rklh(int block, int nvec, bool softcap) {
    HL_FUSED_CASE(hl::F32T, 256, 1, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F32T, 256, 2, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F32T, 256, 4, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F32T, 1024, 2, hl::TM_RKL_H)
    HL_FUSED_CASE(hl::F32T, 1024, 4, hl::TM_RKL_H)
    return nullptr;
}

}  // namespace hl
