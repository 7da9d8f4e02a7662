// ra_bwd.hip -- backward rational-softmax attention for gfx950 (in progress).
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

size_t bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq) {
  const size_t rows = (size_t)B * Hq * Nq;
  return rows * (2 * sizeof(float) + sizeof(float) + sizeof(float) + sizeof(int)) + 256;
}

BwdWorkspace bwd_workspace_layout(void* base, int64_t B, int64_t Hq, int64_t Nq) {
  const size_t rows = (size_t)B * Hq * Nq;
  char* p = static_cast<char*>(base);
  BwdWorkspace ws;
  ws.stats = reinterpret_cast<float*>(p);
  p += rows * 2 * sizeof(float);
  ws.c = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.r = reinterpret_cast<float*>(p);
  p += rows * sizeof(float);
  ws.amax = reinterpret_cast<int*>(p);
  return ws;
}

hipError_t launch_attn_bwd(const AttnProblem&, const void*, const void*, const float*, void*, void*,
                           void*, const BwdWorkspace&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace ra
