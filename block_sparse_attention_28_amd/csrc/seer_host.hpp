// seer_host.hpp -- host-side helpers shared by the C-ABI entry points (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/seer.h"

namespace seer {

// Compute units of the current device, cached once per device id.
int device_cu_count();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// bf16 rows of `d` elements with row stride `stride` keep 16-byte alignment.
inline bool rows_aligned16(const void *base, int64_t stride) {
    return aligned16(base) && stride >= 0 && (stride * 2) % 16 == 0;
}

inline int launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? SEER_OK : SEER_ERR_LAUNCH;
}

// Softmax scales the kernels accept: positive and finite (the running maxima
// are taken on the raw scores and then scaled, which needs a positive scale).
inline bool softmax_scale_ok(float s) { return s > 0.f && s < __builtin_inff(); }

inline bool pow2_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8 || g == 16; }

struct SelectPolicy;
// Checks a caller's selection policy (NULL: the token budget) and converts it.
bool policy_from_host(const seer_select_policy *p, SelectPolicy *out);

}  // namespace seer
