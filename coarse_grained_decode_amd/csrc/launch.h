// Internal launchers of the gfx950 SPICY-KV kernels (private to the library).
#pragma once

#include <hip/hip_runtime.h>

#include "spicy.h"
#include "spicy_device.h"

namespace spicy {

spicy_status launch_coarsen(const CoarsenArgs& a, int dtype, int head_dim, hipStream_t stream);
spicy_status launch_decode(const DecodeArgs& a, int dtype, int head_dim, hipStream_t stream);
spicy_status launch_policy(const PolicyArgs& a, hipStream_t stream);
spicy_status launch_merge(const MergeArgs& a, int dtype, int head_dim, hipStream_t stream);
spicy_status launch_compact(const CompactArgs& a, int dtype, hipStream_t stream);

}  // namespace spicy
