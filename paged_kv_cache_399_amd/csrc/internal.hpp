// Internal helpers shared by the host translation units of libpkv.so.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <string>

#include "pkv.h"

namespace pkv {

// Record a message for pkv_last_error() on this thread and return `code`.
int fail(int code, const char* fmt, ...);

// Clear nothing; successful calls leave the last message as it was.
inline int ok() { return PKV_OK; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t dtype_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

inline bool dtype_valid(int dt) { return dt == PKV_F32 || dt == PKV_BF16; }

}  // namespace pkv

// Wrap every ABI body: converts stray C++ exceptions into status codes.
#define PKV_TRY_BEGIN try {
#define PKV_TRY_END                                                        \
  }                                                                        \
  catch (const std::bad_alloc&) {                                          \
    return pkv::fail(PKV_ERR_CAPACITY, "host allocation failed");          \
  }                                                                        \
  catch (const std::exception& e) {                                        \
    return pkv::fail(PKV_ERR_INVALID_ARG, "internal error: %s", e.what()); \
  }                                                                        \
  catch (...) {                                                            \
    return pkv::fail(PKV_ERR_INVALID_ARG, "internal error");               \
  }
