// Forward of the convolution that allocates nothing: its workspace is a
// file-scope device array of fixed size instead of caller memory.
//
// The array's name is a host-side stand-in in host code, so its device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "../../include/so2conv.h"

namespace so2 {
int set_error(int code, const std::string& msg);
}

namespace {

constexpr size_t kScratchBytes = size_t(256) << 20;    // 256 MiB per device, held until the process ends

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];    // device address of `scratch`, per device index

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return so2::set_error(SO2_EHIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return so2::set_error(SO2_EUNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return so2::set_error(SO2_EHIP, std::string("hipGetSymbolAddress(scratch) failed: ") + hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SO2_OK;
}

}  // namespace

extern "C" int so2conv_fwd_noalloc(const so2conv_cfg* cfg, const so2conv_graph* g, const void* x, const float* pos,
                                   const float* rbf, const float* env, const void* w_rad, const void* const* w1,
                                   const void* const* w2, void* y, void* stream) {
  if (!cfg || !g) return so2::set_error(SO2_EINVAL, "cfg or graph is NULL");
  // workspace of the smallest edge chunk the forward runs (1024 edges, state recomputed)
  const size_t need = so2conv_chunked_workspace_bytes(cfg, g->n_nodes, g->n_edges, 0, 1024);
  if (need > kScratchBytes)
    return so2::set_error(SO2_EWORKSPACE, "so2conv_fwd_noalloc: this configuration needs " + std::to_string(need) +
                                              " bytes of workspace for a 1024-edge chunk; the fixed scratch holds " +
                                              std::to_string(kScratchBytes) + " bytes (use so2conv_fwd)");
  void* ws = nullptr;
  const int r = scratch_address(&ws);
  if (r != SO2_OK) return r;
  // need == 0: the configuration or graph is invalid, and so2conv_fwd reports why
  return so2conv_fwd(cfg, g, x, pos, rbf, env, w_rad, w1, w2, y, nullptr, ws, kScratchBytes, stream);
}
