// Decode with a library-owned scratch array instead of a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The decode pair keeps one buffer between its two kernels: the per-token
// intermediate, fp16 [M x inter].  Here it lives in `scratch`, a file-scope
// device array of kScratchBytes.  Each GPU holds its own copy of the array at
// its own address; the host resolves that address once per device with
// hipGetSymbolAddress and passes it to the kernels exactly as the workspace
// pointer of zinc_mlp_q4k_decode (the array's name in host code is only a
// host-side stand-in and is never handed to a kernel).  The intermediate is
// fully written by the first kernel before the second reads it, so nothing
// needs clearing between calls.
#include "../../include/zinc_mlp.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = 512u << 10;   // M * inter * 2 bytes, 256-byte aligned, at most this
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The address of this device's copy of `scratch`, resolved on the first call
// made with `dev` current and kept for the life of the process.
hipError_t scratch_for(int dev, void** out) {
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

size_t zinc_mlp_q4k_decode_noalloc_max_bytes(void) { return kScratchBytes; }

int zinc_mlp_q4k_decode_noalloc(const void* w_gate, const void* w_up, const void* w_down, int32_t hidden,
                                int32_t inter, const void* x_f16, void* y_f16, int32_t M, int32_t inter_shift,
                                int32_t out_shift, void* stream) {
  // the argument checks of zinc_mlp_q4k_decode, then the scratch limit, all
  // before any HIP call
  if (!w_gate || !w_up || !w_down || !x_f16 || !y_f16) return ZINC_ERR_NULL;
  if (hidden <= 0 || hidden % 256 != 0 || hidden > 16384 || inter <= 0 || inter % 256 != 0 || inter > 65536)
    return ZINC_ERR_SHAPE;
  if (!aligned16(w_gate) || !aligned16(w_up) || !aligned16(w_down) || !aligned16(x_f16) || !aligned16(y_f16))
    return ZINC_ERR_ALIGN;
  if (M < 0 || M > 8) return ZINC_ERR_ARG;
  if (inter_shift < 0 || inter_shift > 30 || out_shift < 0 || out_shift > 30) return ZINC_ERR_ARG;
  if (M == 0) return ZINC_OK;
  if (zinc::decode_workspace_bytes(M, hidden, inter) > kScratchBytes) return ZINC_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1, cur = -1;
  hipError_t e = hipStreamGetDevice(s, &dev);
  if (e == hipSuccess) e = hipGetDevice(&cur);
  if (e != hipSuccess) return zinc::status_from_hip(e);
  if (dev != cur || dev < 0 || dev >= kMaxDevices) return ZINC_ERR_ARG;   // the stream must be the current device's
  void* ws = nullptr;
  e = scratch_for(dev, &ws);
  if (e != hipSuccess) return zinc::status_from_hip(e);
  (void)hipGetLastError();
  return zinc::status_from_hip(
      zinc::launch_decode(w_gate, w_up, w_down, hidden, inter, x_f16, y_f16, M, inter_shift, out_shift, ws, s));
}

}  // extern "C"
