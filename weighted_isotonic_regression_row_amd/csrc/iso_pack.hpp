// Rows of 65 to 512 elements packed several to a wave (iso_pack.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iso {

// Rows of kPackedMin to kPackedMax elements are packed several to a wave
// (shorter rows take the lane kernels).  Longer rows take a wave each
// (k_row_fit with 4 or 8 points per lane), whose output-sensitive finish
// measured as fast as the packed kernels on noise rows of 160 to 256 and
// faster on rows whose every point is a vertex (1e5 rows, float32:
// increasing rows of 160, 0.29 against 0.41 ms packed).
constexpr int kPackedMin = 65;
constexpr int kPackedMax = 128;

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
