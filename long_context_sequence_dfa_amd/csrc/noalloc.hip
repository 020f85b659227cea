// noalloc.hip -- dfa_attn_bwd_noalloc: the backward with the library's own
// device scratch in place of a caller workspace, for callers that cannot
// allocate device memory.
//
// The scratch is one file-scope device array per GPU (the runtime gives
// every device its own copy when the code object loads there, and keeps it
// until the process ends).  Host code never passes the array's name to a
// kernel or a copy: in host code that name is only a stand-in for the
// symbol.  The device address comes from hipGetSymbolAddress, taken once per
// device with that device current and kept per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dfa.h"

namespace {

constexpr size_t kScratchBytes = size_t{80} << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mu;
void *g_ptr[kMaxDevices];  // scratch address per device, null until taken

// Device address of `device`'s scratch array; `device` must be current.
dfa_status scratch_of(int device, void **out) {
  if (device < 0 || device >= kMaxDevices) return DFA_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[device]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFA_E_HIP;
    g_ptr[device] = p;
  }
  *out = g_ptr[device];
  return DFA_OK;
}

}  // namespace

extern "C" dfa_status dfa_attn_bwd_noalloc(const dfa_attn_desc *d, const dfa_block *blocks,
                                           int64_t n_blocks, const void *q, const void *k,
                                           const void *v, const void *o, const void *d_o,
                                           const float *lse, void *dq, void *dk, void *dv,
                                           void *stream) {
  // the whole host-side validation and the size check come first: a problem
  // larger than the scratch is refused before any HIP call
  size_t need = 0;
  dfa_status st = dfa_workspace_size(d, blocks, n_blocks, DFA_OP_BWD, &need);
  if (st != DFA_OK) return st;
  if (need > kScratchBytes) return DFA_E_WORKSPACE;
  // the scratch of the device the stream runs on, which must be current
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return DFA_E_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess) return DFA_E_HIP;
    if (sdev != cur) return DFA_E_UNSUPPORTED;
  }
  void *ws = nullptr;
  st = scratch_of(cur, &ws);
  if (st != DFA_OK) return st;
  return dfa_attn_bwd_ex(d, blocks, n_blocks, q, k, v, o, d_o, lse, dq, dk, dv, ws, kScratchBytes,
                         nullptr, stream);
}
