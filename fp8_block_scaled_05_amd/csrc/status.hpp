// Host-side argument checks and the thread-local error text behind
// fp8bs_last_error().
#pragma once
#include <cstdint>
#include "fp8bs.h"

namespace fp8bs {

// Records the message for fp8bs_last_error() and returns `st`.
fp8bs_status fail(fp8bs_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread's last HIP error before a call's first launch, so that
// check_launch() reports only errors raised by this call's launches (an
// earlier failed HIP call on the thread would otherwise show up here).
void begin_launch();

// Maps the HIP error state after a call's launches to a status.
fp8bs_status check_launch(const char* what);

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

inline int elem_size(int32_t dtype) { return dtype == FP8BS_BF16 ? 2 : 4; }

// A row count or pitch beyond these cannot describe a real allocation (a
// 64-bit argument passed as a 32-bit value can leave garbage in its upper
// half); such calls are rejected instead of launching with wild addresses.
constexpr int64_t kMaxExtent = int64_t(1) << 31;   // elements per dimension
constexpr int64_t kMaxBytes = int64_t(1) << 47;    // bytes spanned by one matrix
inline bool sane_matrix(int64_t rows, int64_t ld, int elt) {
  return rows >= 0 && ld >= 0 && rows <= kMaxExtent && ld <= kMaxExtent &&
         rows * ld <= kMaxBytes / elt;
}
inline bool valid_dtype(int32_t dtype) { return dtype == FP8BS_BF16 || dtype == FP8BS_F32; }

}  // namespace fp8bs
