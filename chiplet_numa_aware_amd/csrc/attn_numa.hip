// C ABI of the library's shared entry points (include/attn_numa.h): the
// remap table on the host, the row-block height, the XCD count, the
// placement probe and the error text.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn_numa.h"
#include "host_util.hpp"
#include "wg_map.hpp"

namespace attn_numa {
namespace {

// Placement probe: one wave per workgroup; lane 0 records the XCC id the
// workgroup runs on and the coordinates the remap gives it.
__global__ void probe_kernel(int32_t* out, int B, int H_Q, int M, int mapping,
                             int X, int G) {
  if (threadIdx.x != 0) return;
  uint32_t xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const WgCoord c = wg_map(mapping, blockIdx.x, B, H_Q, M, X, G);
  int32_t* p = out + 4 * (uint64_t)blockIdx.x;
  p[0] = (int32_t)(xcc & 0xF);
  p[1] = (int32_t)c.b;
  p[2] = (int32_t)c.h;
  p[3] = (int32_t)c.m;
}


}  // namespace
}  // namespace attn_numa

using namespace attn_numa;

extern "C" {

int attn_wg_map(int mapping, int B, int H_Q, int H_KV, int N, int num_xcd,
                int32_t* out_host) {
  if (!out_host) return ATTN_E_NULL;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N, &M, &W);
  if (rc != ATTN_OK) return rc;
  if (num_xcd < 1) return ATTN_E_SHAPE;
  if (mapping < 0 || mapping > kMaxMapping) return ATTN_E_MAPPING;
  for (int w = 0; w < W; ++w) {
    const WgCoord c = wg_map(mapping, (uint32_t)w, (uint32_t)B, (uint32_t)H_Q,
                             (uint32_t)M, (uint32_t)num_xcd, (uint32_t)(H_Q / H_KV));
    out_host[3 * (int64_t)w + 0] = (int32_t)c.b;
    out_host[3 * (int64_t)w + 1] = (int32_t)c.h;
    out_host[3 * (int64_t)w + 2] = (int32_t)c.m;
  }
  return ATTN_OK;
}

int attn_block_m(void) { return kBlockM; }

int attn_num_xcd(void) {
  int X = 0;
  int rc = resolve_xcd(&X);
  return rc == ATTN_OK ? X : rc;
}

int attn_probe_placement(int mapping, int B, int H_Q, int H_KV, int N,
                         int32_t* dev_out, void* stream) {
  if (!dev_out) return ATTN_E_NULL;
  int M = 0, W = 0;
  int rc = check_shape(B, H_Q, H_KV, N, &M, &W);
  if (rc != ATTN_OK) return rc;
  if (mapping < 0 || mapping > kMaxMapping) return ATTN_E_MAPPING;
  if (!aligned16(dev_out)) return ATTN_E_ALIGN;
  int X = 1;
  rc = resolve_xcd(&X);
  if (rc != ATTN_OK) return rc;
  hipLaunchKernelGGL(probe_kernel, dim3(W), dim3(64), 0,
                     static_cast<hipStream_t>(stream), dev_out, B, H_Q, M,
                     mapping, X, H_Q / H_KV);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "attn_probe_placement launch");
  return ATTN_OK;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULL: return "a required pointer is NULL";
    case ATTN_E_SHAPE:
      return "bad shape (B, H_Q, H_KV, N must be > 0, H_Q % H_KV == 0, "
             "B*H_Q*ceil(N/256) < 2^31, N*d*2 <= 2^31 - 2^16, num_xcd >= 1)";
    case ATTN_E_HEAD_DIM: return "unsupported head dim (need 8 <= d <= 128, d % 8 == 0)";
    case ATTN_E_MAPPING: return "mapping out of range (attention 0..15, cac_gemm 0..3)";
    case ATTN_E_ALIGN: return "device pointer not 16-byte aligned";
    case ATTN_E_HIP:
      return g_err_text[0] ? g_err_text : "HIP runtime error";
    case ATTN_E_NO_DEVICE: return "no HIP device visible";
    case ATTN_E_SCRATCH:
      return "the split workspace would exceed the library's fixed device scratch "
             "(ATTN_SCRATCH_BYTES); use attn_fwd_split with a caller workspace";
    default: return "unknown error code";
  }
}

}  // extern "C"
