// la_noalloc.hip -- la_chunk_fwd for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that
// forbid hipMalloc): the start states of the split plan live in a fixed
// device array of this file instead of a caller-given workspace.
//
// The array is a file-scope __device__ object, so each GPU the library runs
// on holds its own copy from module load until the process ends.  Host code
// never uses the array's name as an address (on the host it is only a
// stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// kept per device.  Every call on one GPU shares that GPU's copy and leaves
// its contents behind; the forward writes every start state before it reads
// it, so nothing has to start at zero.  Two calls that overlap in time on one
// GPU (different streams, or different host threads) race on the array.
#include <hip/hip_runtime.h>

#include <mutex>

#include "la_internal.h"
#include "linattn.h"

namespace {

constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch array (null on failure, with the
// HIP error in *err).
void* scratch_ptr(int dev, hipError_t* err) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_ptr[dev] = p;
  }
  *err = hipSuccess;
  return g_ptr[dev];
}

}  // namespace

extern "C" la_status la_chunk_fwd_noalloc(const la_shape* shape, const void* Q, const void* K,
                                          const void* V, const float* lambda, const float* S0,
                                          void* O, float* S_end, void* stream) {
  // every argument is checked on the host before any HIP call
  const la_status r = la::check_fwd_args(shape, Q, K, V, lambda, S0, O, S_end);
  if (r != LA_OK) return r;
  const size_t need = la_fwd_workspace_bytes(shape);
  if (need > kScratchBytes)
    return la::record_error(LA_ERR_WORKSPACE,
                            "this shape's plan needs %zu bytes of start states; "
                            "la_chunk_fwd_noalloc holds at most %zu (use la_chunk_fwd with a "
                            "workspace)",
                            need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return la::record_error(LA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
      return la::record_error(LA_ERR_UNSUPPORTED, "device %d beyond the %d this entry point serves",
                              dev, kMaxDevices);
    ws = scratch_ptr(dev, &e);
    if (!ws)
      return la::record_error(LA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  }
  return la_chunk_fwd(shape, Q, K, V, lambda, S0, O, S_end, ws, need, stream);
}
