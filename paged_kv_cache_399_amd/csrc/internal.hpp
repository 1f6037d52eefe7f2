// Internal helpers shared by the host translation units of libpkv.so.
#pragma once

#include <cstdarg>
#include <cstdint>
#include <string>

#include "pkv.h"

namespace pkv {

// Record a message for pkv_last_error() on this thread and return `code`.
// `fmt` is a printf format (checked by the compiler): a literal percent sign is "%%".
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear nothing; successful calls leave the last message as it was.
inline int ok() { return PKV_OK; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline size_t dtype_size(pkv_dtype dt) { return dt == PKV_F32 ? 4 : 2; }

inline bool dtype_valid(int dt) { return dt == PKV_F32 || dt == PKV_BF16; }

// Attention scale: 0 selects the usual 1 / sqrt(head_dim), rounded to fp32;
// anything else must be finite and positive.  Returns false if refused.
inline bool resolve_scale(float* scale, int32_t head_dim) {
  if (*scale == 0.f && head_dim > 0) *scale = (float)(1.0 / __builtin_sqrt((double)head_dim));
  return __builtin_isfinite(*scale) && *scale > 0.f;
}

inline bool layout_valid(int l) { return l == PKV_LAYOUT_HEAD_MAJOR || l == PKV_LAYOUT_TOKEN_MAJOR; }

// Element strides of the key cache inside a block: between KV heads and
// between tokens (a token's head_dim row is contiguous in both layouts).
struct KStrides {
  int32_t head, tok;
};
inline KStrides k_strides(int layout, int32_t hkv, int32_t p, int32_t d) {
  if (layout == PKV_LAYOUT_TOKEN_MAJOR) return KStrides{d, hkv * d};
  return KStrides{p * d, d};
}

// Block-table patch carried entirely in kernel arguments (no staging copy):
// lens[len0 + i] = w[i] (i < n_len); shared[sh0 + i] = w[n_len + i]
// (i < n_sh); slots[slot0 + i] = w[n_len + n_sh + i] (i < n_slot); then
// n_ent (row, col, value) triples; then n_reset (row, from) pairs whose row
// entries [from, max_blocks) become -1.
constexpr int kPatchWords = 896;
struct TablePatchArgs {
  int32_t* table;
  int32_t* lens;
  int32_t* slots;
  int32_t* shared;
  int32_t max_blocks, n_len, len0, n_slot, slot0, n_ent, n_reset, n_sh, sh0, unused;
  int32_t w[kPatchWords];
};

// Enqueue one patch (defined with the device kernels).  Returns a status.
int launch_table_patch(const TablePatchArgs& args, void* stream);

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
