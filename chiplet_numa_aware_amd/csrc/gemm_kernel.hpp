// Tiled bf16 GEMM for gfx950 whose workgroup -> tile placement is the
// Compute Affinity Cluster map (cac_map.hpp).
//
// C[l] = A[l] B[l]^T for l < L, with A [L][M][K], B [L][N][K] and C [L][M][N]
// row-major bf16 (both operands K-contiguous, the layout of the attention's
// S = Q K^T), fp32 accumulation, C rounded to bf16 (nearest-even).
//
// One workgroup computes one 256 x 256 tile of C with 8 waves (two per
// SIMD, so one wave's LDS waits hide behind the other's MFMAs); wave w owns
// rows 64 (w / 2) .. +64 and columns 128 (w % 2) .. +128 as 4 x 8 blocks of
// v_mfma_f32_16x16x32_bf16.  For the same work this shape draws less power
// than 32x32x16 (measured: the same FLOPs on random operands sustain 2.16
// against 1.89-1.95 GHz under the chip's power limit), and the kernel runs
// 2-7% faster with it.  Each block is computed transposed, C^T = B A^T
// (A operand: 16 columns of B; B operand: 16 rows of A), so a lane's 4
// accumulators are 4 consecutive columns of one C row and the epilogue
// writes 8-byte pieces.  K advances 64 at a time; the A and B
// slices of a K step go from global memory straight into LDS (buffer loads
// with the LDS-direct bit), two stages deep, so a step's loads have one step
// of MFMAs (two waves per SIMD) to land.  An LDS slice is 256 rows of K-step / 8 16-byte
// chunks; chunk c of row r sits at slot c ^ gemm_swz(r), which keeps the
// 16-byte operand reads free of bank conflicts.  Rows past M or N read as zero
// (range-checked buffer offsets), K chunks past K use an offset that is
// always out of range, and stores outside C are dropped.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_kernel.hpp"
#include "cac_map.hpp"

namespace attn_numa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemmTile = 256;   // rows and columns of a C tile
// K per step: 64 with two stages measured 3-10% faster than 32 with four
// (half the barriers; the same 128 KiB of LDS).
constexpr int kGemmBK = 64;                     // K per step (32 or 64)
constexpr int kGemmStages = 128 / kGemmBK;      // LDS stages (4 or 2; 128 KiB)
constexpr int kGemmKC = kGemmBK / 16;           // 16-deep MFMA chunks per step
constexpr int kGemmCPR = kGemmBK / 8;           // 16-byte chunks per LDS row
constexpr int kGemmThreads = 512;
constexpr int kGemmWaves = kGemmThreads / 64;
constexpr int kGemmRowB = kGemmBK * 2;              // bytes of one LDS row
constexpr int kGemmSliceB = kGemmTile * kGemmRowB;  // one operand's K slice (16 KiB)
constexpr int kGemmStageB = 2 * kGemmSliceB;        // A slice, then B slice
constexpr int kGemmLoads = kGemmSliceB / 16 / kGemmThreads;  // 16-byte loads per thread per slice
static_assert(kGemmLoads * 16 * kGemmThreads == kGemmSliceB, "a slice splits into the workgroup");

// Slot of chunk c of LDS row r is c ^ gemm_swz(r).  gfx950's LDS has 64
// banks of 4 bytes (a 256-byte line) and serves a 16-byte read 16 lanes per
// cycle, here 16 consecutive rows reading one chunk.  Rows of 128 bytes (8
// chunks) alternate between the two halves of a line, and the 8 rows of one
// parity take 8 distinct slots; rows of 64 bytes (4 chunks) share a line four
// at a time, and the 4 rows at one position take 4 distinct slots.  Either
// way the 16 reads cover the 64 banks once.
__device__ __forceinline__ int gemm_swz(int r) {
  return kGemmCPR == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7);
}

__global__ __launch_bounds__(kGemmThreads, 1) void cac_gemm_kernel(
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b, uint16_t* __restrict__ c,
    int L, int M, int N, int K, int Mt, int Nt, int mapping, int gm, int gn, int num_xcd) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[kGemmStages * kGemmStageB / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const TileCoord tc = cac_tile_map(mapping, blockIdx.x, L, Mt, Nt, gm, gn, num_xcd);
  const int m0 = (int)tc.tm * kGemmTile, n0 = (int)tc.tn * kGemmTile;
  const uint32_t a_bytes = (uint32_t)M * (uint32_t)K * 2u;
  const uint32_t b_bytes = (uint32_t)N * (uint32_t)K * 2u;
  const uint32_t c_bytes = (uint32_t)M * (uint32_t)N * 2u;
  const u32x4 a_desc = make_desc(a + (uint64_t)tc.l * M * K, a_bytes);
  const u32x4 b_desc = make_desc(b + (uint64_t)tc.l * N * K, b_bytes);

  // Tile loads: instruction i of this thread fills LDS slot P = tid + 512 i of
  // a slice (row P / CPR, slot P % CPR holding chunk (P % CPR) ^ gemm_swz(row)).
  // The row offset of the tile goes in soffset (capped at the buffer size, so
  // rows past the matrix read zero); voffset is the row within the tile and
  // the K position.
  const uint32_t a_soff = min((uint32_t)m0 * (uint32_t)K * 2u, a_bytes);
  const uint32_t b_soff = min((uint32_t)n0 * (uint32_t)K * 2u, b_bytes);
  uint32_t ld_row[kGemmLoads];
  int ld_k[kGemmLoads];
#pragma unroll
  for (int i = 0; i < kGemmLoads; ++i) {
    const int P = tid + kGemmThreads * i;
    const int row = P / kGemmCPR;
    const int chunk = (P % kGemmCPR) ^ gemm_swz(row);
    ld_row[i] = (uint32_t)row * (uint32_t)K * 2u;
    ld_k[i] = chunk * 8;
  }
  const int n_steps = (K + kGemmBK - 1) / kGemmBK;
  auto issue = [&](int step) {
    const int st = step & (kGemmStages - 1);
    const int k0 = step * kGemmBK;
#pragma unroll
    for (int i = 0; i < kGemmLoads; ++i) {
      const int kk = k0 + ld_k[i];
      const uint32_t voff = kk < K ? ld_row[i] + (uint32_t)kk * 2u : kOutOfRange;
      const uint32_t m0b = lds_base + st * kGemmStageB + (wave + kGemmWaves * i) * 1024;
      load_lds(a_desc, voff, a_soff, m0b);
      load_lds(b_desc, voff, b_soff, m0b + kGemmSliceB);
    }
  };

  // Operand reads (v_mfma_f32_16x16x32_bf16): lane (row r16 of a 16-row
  // block, quarter q) reads chunk 4 k32 + q of its row; the 16 lanes of a
  // quarter read 16 consecutive rows of one chunk.
  constexpr int kK32 = kGemmBK / 32;  // 32-deep MFMA steps per K step
  const int r16 = lane & 15, q4 = lane >> 4;
  int rd[kK32];
#pragma unroll
  for (int kc = 0; kc < kK32; ++kc) rd[kc] = r16 * kGemmRowB + (((4 * kc + q4) ^ gemm_swz(r16)) * 16);
  const int wm = 64 * (wave >> 1), wn = 128 * (wave & 1);

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{};

  // Prologue: steps 0 .. stages-2 in flight.
#pragma unroll
  for (int s = 0; s < kGemmStages - 1; ++s)
    if (s < n_steps) issue(s);
  for (int step = 0; step < n_steps; ++step) {
    // Step `step` has landed when at most the loads of the (up to two) later
    // steps already issued are outstanding (loads retire in order).
    const int later = min(n_steps - 1 - step, kGemmStages - 2);
    if (later >= 2)
      wait_vmcnt<4 * kGemmLoads>();
    else if (later == 1)
      wait_vmcnt<2 * kGemmLoads>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    // All 12 operand fragments of the step first (two 16-deep K chunks),
    // then the loads of a later step, then the 16 MFMAs: the MFMAs of chunk 0
    // wait only for its own fragments, and chunk 1's arrive meanwhile.
    const char* sa = lb + (step & (kGemmStages - 1)) * kGemmStageB;
    const char* sb = sa + kGemmSliceB;
    bf16x8 fa[kK32][4], fb[kK32][8];
#pragma unroll
    for (int kc = 0; kc < kK32; ++kc) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[kc][i] = *reinterpret_cast<const bf16x8*>(sa + (wm + 16 * i) * kGemmRowB + rd[kc]);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        fb[kc][j] = *reinterpret_cast<const bf16x8*>(sb + (wn + 16 * j) * kGemmRowB + rd[kc]);
    }
    // The stage written next was last read in step - 1, which every wave
    // finished before the barrier above.
    if (step + kGemmStages - 1 < n_steps) issue(step + kGemmStages - 1);
#pragma unroll
    for (int kc = 0; kc < kK32; ++kc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[kc][j], fa[kc][i], acc[i][j], 0, 0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 12 * kK32, 0);  // the LDS reads
    __builtin_amdgcn_sched_group_barrier(0x008, 32 * kK32, 0);  // then the MFMAs
  }

  // acc[i][j] register r (16x16 block, computed transposed as C^T = B A^T):
  // C row m0 + wm + 16 i + r16, column n0 + wn + 16 j + 4 q4 + r.
  const __amdgpu_buffer_rsrc_t c_rs = make_rsrc(c + (uint64_t)tc.l * M * N, c_bytes);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + wm + 16 * i + r16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = n0 + wn + 16 * j + 4 * q4;
      if (row < M && col < N) {
        u32x2 w;
        w.x = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
        w.y = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, c_rs, ((uint32_t)row * (uint32_t)N + col) * 2u, 0, 0);
      }
    }
  }
}

}  // namespace attn_numa
