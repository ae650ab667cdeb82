// Load-mode gradient kernel instances for f16 logits (every teacher mode incl. the Hinton ones, softcap on/off).
#include "hl_device.cuh"

namespace hl {

GradLauncher get_grad_f16(int tmode, bool softcap) {
    switch (tmode) {
        case TM_NONE: return softcap ? &launch_grad<F16T, TM_NONE, true> : &launch_grad<F16T, TM_NONE, false>;
        case TM_FKL: return softcap ? &launch_grad<F16T, TM_FKL, true> : &launch_grad<F16T, TM_FKL, false>;
        case TM_RKL: return softcap ? &launch_grad<F16T, TM_RKL, true> : &launch_grad<F16T, TM_RKL, false>;
        case TM_FDCE: return softcap ? &launch_grad<F16T, TM_FDCE, true> : &launch_grad<F16T, TM_FDCE, false>;
        case TM_FKL_H: return softcap ? &launch_grad<F16T, TM_FKL_H, true> : &launch_grad<F16T, TM_FKL_H, false>;
        case TM_RKL_H: return softcap ? &launch_grad<F16T, TM_RKL_H, true> : &launch_grad<F16T, TM_RKL_H, false>;
        case TM_FDCE_H: return softcap ? &launch_grad<F16T, TM_FDCE_H, true> : &launch_grad<F16T, TM_FDCE_H, false>;
        default: return nullptr;
    }
}

}  // namespace hl
