// The argument checks of iso_fit and iso_vjp_yw, apart from their launches,
// so that an entry point can check a whole call before it queues work of its
// own around the fit (iso_view.hip).
#pragma once

#include "../../include/iso.h"
#include "iso_internal.hpp"

namespace iso {

// 1 when kernels are to be launched (the record filled in, the partition
// handle set up), else the code the call returns (ISO_OK for an empty
// problem, ISO_EINVAL).  Nothing is queued.
int fit_prepare(const void* y, const void* w, int64_t rows, int64_t n, int increasing, double y_min, double y_max,
                int dtype, void* fit, iso_blocks* blocks_out, void* blocks_mem, void* workspace,
                size_t workspace_bytes, void* stream, FitLaunch& a);
int vjp_prepare(const void* grad, const iso_blocks* blocks, const void* y, void* grad_y, void* grad_w,
                void* workspace, size_t workspace_bytes, void* stream, VjpLaunch& v);

}  // namespace iso
