/*
 * cac_gemm.h: a tiled bf16 GEMM for MI355X (gfx950) whose workgroups are
 * placed on XCDs by a Compute Affinity Cluster map.  Part of libattn_numa;
 * error codes and attn_strerror() come from attn_numa.h.
 *
 * Passage: "Optimizing Attention on GPUs by Exploiting GPU Architectural
 * NUMA Effects", commentary page, the paragraph that generalises the
 * Attention Compute Cluster to a "Compute Affinity Cluster" (the workgroups
 * that share input data) so that kernels such as GEMM get the same XCD
 * placement.  For C = A B^T a cluster is a block of group_m x group_n output
 * tiles, which share group_m row panels of A and group_n column panels of B.
 */
#ifndef CAC_GEMM_H
#define CAC_GEMM_H

#include <stdint.h>

#include "attn_numa.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Tile map modes: bit 0 = order, bit 1 = chiplet swizzle (as ATTN_MAP_*). */
#define CAC_MAP_NAIVE_ROW_MAJOR 0      /* tiles row-major, ids round-robin over XCDs */
#define CAC_MAP_NAIVE_CLUSTER 1        /* cluster-major order, round-robin */
#define CAC_MAP_SWIZZLED_ROW_MAJOR 2   /* row-major order, XCD x takes slice x */
#define CAC_MAP_SWIZZLED_CLUSTER 3     /* cluster-major, XCD x takes slice x:
                                          one XCD walks whole clusters */

/*
 * cac_gemm: C[l] = A[l] B[l]^T for l < L.
 *
 *   a  device, bf16 [L][M][K], row-major, read only
 *   b  device, bf16 [L][N][K], row-major, read only
 *   c  device, bf16 [L][M][N], row-major, written (every element)
 *   L, M, N, K  > 0; N % 8 == 0, K % 8 == 0, K <= 2^20; M*K*2, N*K*2 and
 *               M*N*2 <= 2^31 - 2^16 bytes; L*ceil(M/256)*ceil(N/256) < 2^31
 *   mapping     CAC_MAP_* (0..3)
 *   group_m, group_n  cluster shape in 256 x 256 tiles; 0 picks 4 x 8 (the 32
 *               tiles one XCD runs at once); clipped to the tile grid
 *   stream      hipStream_t or NULL
 * Arithmetic: bf16 products accumulated in fp32, C rounded to bf16
 * (nearest-even).  C does not depend on mapping or the cluster shape
 * (each tile's sum runs over K in the same order).
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE, ATTN_E_MAPPING, ATTN_E_ALIGN (any pointer
 * not 16-byte aligned), ATTN_E_NO_DEVICE, ATTN_E_HIP.
 */
int cac_gemm(const void* a, const void* b, void* c, int L, int M, int N, int K,
             int mapping, int group_m, int group_n, void* stream);

/* Rows and columns of one C tile (256). Needs no GPU. */
int cac_gemm_tile(void);

/*
 * cac_gemm_map: the tile map cac_gemm uses, on the host.
 *   out_host  host, int32 [W][3], W = L*ceil(M/256)*ceil(N/256): row w gets
 *             (l, tile row, tile column) of workgroup id w
 * Other arguments as cac_gemm (K is not needed).  Needs no GPU.
 * Errors: ATTN_E_NULL, ATTN_E_SHAPE (also num_xcd < 1), ATTN_E_MAPPING.
 */
int cac_gemm_map(int mapping, int L, int M, int N, int group_m, int group_n,
                 int num_xcd, int32_t* out_host);

#ifdef __cplusplus
}
#endif

#endif /* CAC_GEMM_H */
