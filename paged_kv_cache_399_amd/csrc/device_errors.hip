// Per-device error word that kernels set when they meet an index they had to
// clamp or skip (bad block-table entry, slot or copy pair).
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.hpp"
#include "internal.hpp"

namespace {
__device__ int32_t g_pkv_error_word;

constexpr int kMaxDevices = 64;
int32_t* g_word_ptr[kMaxDevices] = {};
std::mutex g_word_mu;
}  // namespace

namespace pkv {

int device_error_word(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(PKV_ERR_UNSUPPORTED, "device id %d", dev);
  std::lock_guard<std::mutex> lk(g_word_mu);
  if (!g_word_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_pkv_error_word));
    if (e != hipSuccess || !p)
      return fail(PKV_ERR_HIP, "hipGetSymbolAddress(error word): %s", hipGetErrorString(e));
    g_word_ptr[dev] = (int32_t*)p;
  }
  *out = g_word_ptr[dev];
  return PKV_OK;
}

}  // namespace pkv

extern "C" int pkv_check_device_errors(void* stream, int32_t* flags_out) {
  PKV_TRY_BEGIN
  int32_t* word = nullptr;
  int rc = pkv::device_error_word(&word);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t flags = 0;
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipMemcpy(&flags, word, sizeof flags, hipMemcpyDeviceToHost);
  const int32_t zero = 0;
  if (e == hipSuccess && flags) e = hipMemcpy(word, &zero, sizeof zero, hipMemcpyHostToDevice);
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "reading device errors: %s", hipGetErrorString(e));
  if (flags_out) *flags_out = flags;
  if (flags) return pkv::fail(PKV_ERR_DEVICE, "kernels flagged bad indices (bits 0x%x)", flags);
  return PKV_OK;
  PKV_TRY_END
}
