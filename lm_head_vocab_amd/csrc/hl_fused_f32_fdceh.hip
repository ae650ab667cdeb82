// Fused-kernel instances: dtype f32, distillation mode from-distribution CE, Hinton temperature.
#include "hl_device.cuh"

// fp32 teacher slices hold at most 4 vectors per tensor (the fp64 element path
// of the fp32 instances needs the registers; see kF32TeacherNvec).

namespace hl {

FusedLauncher get_fused_f32_fdceh(int block, int nvec, bool softcap) {
    HL_FUSED_CASE(hl::F32T, 256, 1, hl::TM_FDCE_H)
    HL_FUSED_CASE(hl::F32T, 256, 2, hl::TM_FDCE_H)
    HL_FUSED_CASE(hl::F32T, 256, 4, hl::TM_FDCE_H)
    HL_FUSED_CASE(hl::F32T, 1024, 2, hl::TM_FDCE_H)
    HL_FUSED_CASE(hl::F32T, 1024, 4, hl::TM_FDCE_H)
    return nullptr;
}

}  // namespace hl
