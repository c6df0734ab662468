// Host-side argument checks and the thread-local error text behind
// fp8bs_last_error().
#pragma once
#include <cstdint>
#include "fp8bs.h"

namespace fp8bs {

// Records the message for fp8bs_last_error() and returns `st`.
fp8bs_status fail(fp8bs_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Maps the HIP error state after a launch to a status.
fp8bs_status check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline int elem_size(int32_t dtype) { return dtype == FP8BS_BF16 ? 2 : 4; }
inline bool valid_dtype(int32_t dtype) { return dtype == FP8BS_BF16 || dtype == FP8BS_F32; }

}  // namespace fp8bs
