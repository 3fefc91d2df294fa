// fa_noalloc.hip -- fa_backward_noalloc: the backward with its workspace in a
// library-owned device array, for callers that cannot allocate device memory
// (code under HIP graph capture, serving loops that forbid hipMalloc).
//
// The backward's only scratch is the workspace of two fp32 row statistics
// per (batch, head, row): D_i = do_i . o_i and -lse_i in the exponent domain.
// Here it lives in `scratch`, a file-scope device array of
// FA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until the
// process ends.  Its device address is looked up once per device with
// hipGetSymbolAddress (host code must never pass the array's own name to a
// kernel: on the host that name is a stand-in, not a device address) and
// kept per device; the kernels receive that address exactly as they receive
// a caller's workspace.  Nothing is cleared: the backward's first kernel
// (bf16: dQ, which also does the preprocess pass; fp32: the preprocess
// kernel) writes every statistic the later kernels read, on the same
// stream, before they run.  All calls on one GPU share its array, so calls
// that overlap in time on one GPU (different streams, or host threads) race
// on it.
#include "fa.h"
#include "fa_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = FA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch`, per device

// Address of this process's `scratch` on the current device (looked up on
// the first call with that device current).
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    if ((reinterpret_cast<uintptr_t>(p) & 255u) != 0) return FA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return FA_OK;
}

}  // namespace

extern "C" int fa_backward_noalloc(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                   const float* lse, void* dq, void* dk, void* dv, int B, int H, int N, int d,
                                   int causal, float scale, int dtype, void* stream) {
  // Validation first, before any HIP call: with no workspace, fa_backward
  // checks every other argument and returns FA_ERR_WORKSPACE only when they
  // are all valid (FA_OK for an empty problem); it enqueues nothing then.
  const int chk = fa_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, nullptr, 0,
                              stream);
  if (chk != FA_ERR_WORKSPACE) return chk;
  if (fa_backward_workspace_size(B, H, N, d) > kScratchBytes) return FA_ERR_SCRATCH;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != FA_OK) return st;
  return fa_backward(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, causal, scale, dtype, ws, kScratchBytes,
                     stream);
}
