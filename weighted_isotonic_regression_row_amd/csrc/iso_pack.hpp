// Rows of 33 to 512 elements packed several to a wave (iso_pack.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iso_internal.hpp"

namespace iso {

// (kPackedMin, kPackedMax: iso_internal.hpp)

struct PackedLaunch {
    const void* y;
    const void* w;
    void* fit;
    int64_t rows, n;
    int increasing;
    int dtype;
    double lo, hi;
    uint64_t* start_bits;
    uint64_t* clip_bits;
    uint32_t* row_nan;
    int64_t words;
    unsigned long long* status;
    unsigned long long epoch;
    int* cover;   // workspace for the waves left to the second pass: 16 counters
                  // 256 bytes apart (cleared by the launch), then 16 lists of
                  // ceil(waves / 16) entries
    hipStream_t stream;
};

hipError_t launch_rows_packed(const PackedLaunch& l);

}  // namespace iso
