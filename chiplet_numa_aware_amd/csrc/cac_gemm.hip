// C ABI of the CAC-scheduled GEMM (include/cac_gemm.h): validation, the
// default cluster shape and the launch on the caller's stream.  Allocates
// nothing and does not synchronise.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/cac_gemm.h"
#include "cac_map.hpp"
#include "gemm_kernel.hpp"
#include "host_util.hpp"

namespace attn_numa {
namespace {

// Tiles one XCD keeps in flight (32 CUs x one workgroup) as 4 tile rows x 8
// tile columns: 12 panels for 32 tiles.
constexpr int kDefaultGroupM = 4;
constexpr int kDefaultGroupN = 8;

struct GemmShape {
  int Mt, Nt, gm, gn, W;
};

int check_gemm(int L, int M, int N, int K, int mapping, int group_m, int group_n,
               GemmShape* s) {
  if (L <= 0 || M <= 0 || N <= 0 || K <= 0) return ATTN_E_SHAPE;
  if (N % 8 != 0 || K % 8 != 0) return ATTN_E_SHAPE;
  // Row offsets within a tile (255 rows of K) and every matrix must fit the
  // range-checked 32-bit buffer offsets.
  if (K > (1 << 20)) return ATTN_E_SHAPE;
  if ((int64_t)M * K * 2 > kMaxHeadBytes || (int64_t)N * K * 2 > kMaxHeadBytes ||
      (int64_t)M * N * 2 > kMaxHeadBytes)
    return ATTN_E_SHAPE;
  const int64_t Mt = ((int64_t)M + kGemmTile - 1) / kGemmTile;
  const int64_t Nt = ((int64_t)N + kGemmTile - 1) / kGemmTile;
  const int64_t W = (int64_t)L * Mt * Nt;
  if (W >= (int64_t(1) << 31)) return ATTN_E_SHAPE;
  if (mapping < 0 || mapping > 3) return ATTN_E_MAPPING;
  if (group_m < 0 || group_n < 0) return ATTN_E_SHAPE;
  s->Mt = (int)Mt;
  s->Nt = (int)Nt;
  s->gm = group_m > 0 ? group_m : kDefaultGroupM;
  s->gn = group_n > 0 ? group_n : kDefaultGroupN;
  // A cluster larger than the grid is clipped to it.
  if (s->gm > s->Mt) s->gm = s->Mt;
  if (s->gn > s->Nt) s->gn = s->Nt;
  s->W = (int)W;
  return ATTN_OK;
}

}  // namespace
}  // namespace attn_numa

using namespace attn_numa;

extern "C" {

int cac_gemm(const void* a, const void* b, void* c, int L, int M, int N, int K,
             int mapping, int group_m, int group_n, void* stream) {
  if (!a || !b || !c) return ATTN_E_NULL;
  GemmShape s;
  int rc = check_gemm(L, M, N, K, mapping, group_m, group_n, &s);
  if (rc != ATTN_OK) return rc;
  if (!aligned16(a) || !aligned16(b) || !aligned16(c)) return ATTN_E_ALIGN;
  int X = 1;
  rc = resolve_xcd(&X);
  if (rc != ATTN_OK) return rc;
  hipLaunchKernelGGL(cac_gemm_kernel, dim3(s.W), dim3(kGemmThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(a),
                     static_cast<const uint16_t*>(b), static_cast<uint16_t*>(c), L, M, N, K,
                     s.Mt, s.Nt, mapping, s.gm, s.gn, X);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "cac_gemm launch");
  return ATTN_OK;
}

int cac_gemm_tile(void) { return kGemmTile; }

int cac_gemm_map(int mapping, int L, int M, int N, int group_m, int group_n,
                 int num_xcd, int32_t* out_host) {
  if (!out_host) return ATTN_E_NULL;
  GemmShape s;
  int rc = check_gemm(L, M, N, 8, mapping, group_m, group_n, &s);
  if (rc != ATTN_OK) return rc;
  if (num_xcd < 1) return ATTN_E_SHAPE;
  for (int w = 0; w < s.W; ++w) {
    const TileCoord t = cac_tile_map(mapping, (uint32_t)w, (uint32_t)L, (uint32_t)s.Mt,
                                     (uint32_t)s.Nt, (uint32_t)s.gm, (uint32_t)s.gn,
                                     (uint32_t)num_xcd);
    out_host[3 * (int64_t)w + 0] = (int32_t)t.l;
    out_host[3 * (int64_t)w + 1] = (int32_t)t.tm;
    out_host[3 * (int64_t)w + 2] = (int32_t)t.tn;
  }
  return ATTN_OK;
}

}  // extern "C"
