// FlashAttention-2 style attention forward for gfx950 (MI355X).
//
// One workgroup computes one (batch, query head, 128-row block), streaming
// every K/V tile of its KV head with an online softmax ("Optimizing Attention
// on GPUs by Exploiting GPU Architectural NUMA Effects", digest page, §3
// Figure 4 and the §4 equation).  Which block a workgroup takes comes from
// wg_map.hpp.
//
// Layout of the work inside a workgroup (256 threads = 4 waves of 64):
//   * wave w owns query rows [32w, 32w+32) of the block; lane l owns query
//     row 32w + (l mod 32); lanes l and l^32 share a row and split its keys.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K from LDS,
//     B = 16 dims x 32 queries of Q kept in registers), so a lane's 16
//     accumulators of a 32x32 block are 16 keys of ITS query row: the row max
//     and row sum are in-lane plus one exchange with lane l^32.
//   * O^T = V^T P^T: P stays in the registers the score MFMA wrote (B operand,
//     16 keys x 32 queries); V^T comes from LDS, where each tile of V is stored
//     transposed ([dim][key]) with keys permuted inside every 16-key chunk so
//     that the 8 keys a lane needs are 16 contiguous bytes.
//   * K and V tiles (BLOCK_N keys) are double-buffered in LDS; tile j+1 is
//     fetched from global memory into registers while tile j is computed.
//   * m (row max, log2 units) and l (row sum) and O live in registers for the
//     whole key loop; O is divided by l once at the end.
//
// Global memory is read and written through buffer resources that cover one
// head (at most 2^31 bytes): rows past N read as zero and stores past N are
// dropped, which handles ragged N without branches and keeps all 64-bit
// address arithmetic scalar.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wg_map.hpp"

namespace attn_numa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockN = 64;     // keys per K/V tile
constexpr int kThreads = 256;   // 4 waves
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)bytes, (int)kBufDword3);
}

// Two bf16 lanes of two dwords packed into one dword: lo16 from a, lo16 from
// b (sel = 0) or hi16 from a, hi16 from b (sel = 1).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// max / sum of a value with the same value in lane l^32.
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                            __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
struct TileCfg {
  static_assert(D == 64 || D == 128, "padded head dim is 64 or 128");
  static constexpr int KC = D / 16;                // 16-dim chunks (S MFMA k)
  static constexpr int DB = D / 32;                // 32-dim blocks of O^T
  static constexpr int NB = kBlockN / 32;          // 32-key blocks of S^T
  static constexpr int NC = kBlockN / 16;          // 16-key chunks (PV k)
  // LDS row strides in dwords.  stride = 4 (mod 32) makes the 8 lanes of a
  // 16-byte LDS access with consecutive rows hit 8 disjoint bank quads.
  static constexpr int KS = D / 2 + 4;             // K: [key][dim]
  static constexpr int VS = kBlockN / 2 + 4;       // V^T: [dim][key slot]
  static constexpr int K_DW = kBlockN * KS;
  static constexpr int V_DW = D * VS;
  static constexpr int STAGE_DW = K_DW + V_DW;
  static constexpr int LDS_BYTES = 2 * STAGE_DW * 4;
  // K: 16-byte chunks per thread per tile.
  static constexpr int K_CHUNKS_PER_ROW = D / 8;
  static constexpr int K_LOADS = kBlockN * K_CHUNKS_PER_ROW / kThreads;
  // V: each thread loads VEC consecutive dims of 8 keys (keys
  // 16c + 8h + 4g + j, h in {0,1}, j in 0..3), which land in 8 consecutive
  // key slots 16c + 8g .. 16c + 8g + 7 of V^T.
  static constexpr int VEC = D / 32;               // 4 (D=128) or 2 (D=64)
};

// Key slot of key offset o (0..15) inside its 16-key chunk: swaps bits 2 and
// 3, so that the keys a PV MFMA lane holds (o = 8h + 4g + j) sit at
// 8g + 4h + j.
//
// V^T thread mapping (t = thread id): for each tile, thread t handles
//   g = lane bit 0, and dims/chunks chosen so that the 8 lanes of an LDS
//   quarter-wave write 8 disjoint bank quads (stride VS = 4 mod 32):
//   D=128 (VEC 4): lane bits [g, dv0, c0], D=64 (VEC 2): lane bits [g, dv0, dv1].
template <int D>
struct VMap {
  int g, c, dv;
  __device__ __forceinline__ explicit VMap(int t) {
    const int lane = t & 63, wave = t >> 6;
    g = lane & 1;
    if (D == 128) {
      // 32 dim groups of 4 (dv) x 4 chunks (c): wave w covers dv in [8w, 8w+8)
      const int dv0 = (lane >> 1) & 1, c0 = (lane >> 2) & 1;
      const int c1 = (lane >> 3) & 1, dvh = (lane >> 4) & 3;
      c = c0 | (c1 << 1);
      dv = wave * 8 + (dv0 | (dvh << 1));
    } else {
      // 32 dim groups of 2 (dv) x 4 chunks (c): wave w covers dv in [8w, 8w+8)
      const int dvl = (lane >> 1) & 3, c01 = (lane >> 3) & 3, dvh = (lane >> 5) & 1;
      c = c01;
      dv = wave * 8 + (dvl | (dvh << 2));
    }
  }
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int B, int H_Q, int H_KV, int N, int d, int M,
    int mapping, int num_xcd, float scale_log2) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * C::STAGE_DW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;     // lane half: which 8 of 16 MFMA k values
  const int l32 = lane & 31;   // query row within the wave / MFMA column

  const WgCoord wc = wg_map(mapping, blockIdx.x, B, H_Q, M, num_xcd);
  const int kvh = (int)wc.h / (H_Q / H_KV);
  const int row0 = (int)wc.m * kBlockM;

  const uint32_t head_elems = (uint32_t)N * (uint32_t)d;
  const uint64_t q_head = ((uint64_t)wc.b * H_Q + wc.h) * head_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * head_elems;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + kv_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + kv_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(o + q_head, head_elems * 2);

  // ---- Q fragments: B operand of S^T = K Q^T, lane holds Q[row][16kc+8g..+7].
  const int my_row = row0 + wave * 32 + l32;
  bf16x8 qf[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    const int col = kc * 16 + g * 8;
    u32x4 t = {0u, 0u, 0u, 0u};
    if (col < d)
      t = __builtin_amdgcn_raw_buffer_load_b128(
          q_rs, (my_row * d + col) * 2, 0, 0);
    qf[kc] = __builtin_bit_cast(bf16x8, t);
  }

  // ---- tile count
  const int n_tiles_all = (N + kBlockN - 1) / kBlockN;
  int n_tiles = n_tiles_all;
  if (CAUSAL) {
    const int last = (row0 + kBlockM + kBlockN - 1) / kBlockN;
    n_tiles = last < n_tiles_all ? last : n_tiles_all;
  }

  // ---- global -> register staging for one K/V tile
  u32x4 kreg[C::K_LOADS];
  uint32_t vreg[8][C::VEC / 2];
  const VMap<D> vm(tid);

  auto load_tile = [&](int tile) {
    const int key0 = tile * kBlockN;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int chunk = tid + i * kThreads;
      const int r = chunk / C::K_CHUNKS_PER_ROW;
      const int col = (chunk % C::K_CHUNKS_PER_ROW) * 8;
      u32x4 t = {0u, 0u, 0u, 0u};
      if (col < d)
        t = __builtin_amdgcn_raw_buffer_load_b128(
            k_rs, ((key0 + r) * d + col) * 2, 0, 0);
      kreg[i] = t;
    }
    const int col = vm.dv * C::VEC;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int h = e >> 2, j = e & 3;
      const int key = key0 + vm.c * 16 + h * 8 + vm.g * 4 + j;
      const int off = (key * d + col) * 2;
      if constexpr (C::VEC == 4) {
        u32x2 t = {0u, 0u};
        if (col < d) t = __builtin_amdgcn_raw_buffer_load_b64(v_rs, off, 0, 0);
        vreg[e][0] = t.x;
        vreg[e][1] = t.y;
      } else {
        uint32_t t = 0u;
        if (col < d) t = __builtin_amdgcn_raw_buffer_load_b32(v_rs, off, 0, 0);
        vreg[e][0] = t;
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint32_t* ks = lds + stage * C::STAGE_DW;
    uint32_t* vs = ks + C::K_DW;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
      const int chunk = tid + i * kThreads;
      const int r = chunk / C::K_CHUNKS_PER_ROW;
      const int cc = chunk % C::K_CHUNKS_PER_ROW;
      *reinterpret_cast<u32x4*>(ks + r * C::KS + cc * 4) = kreg[i];
    }
    // V^T: for each of my VEC dims, 8 keys -> 16 bytes at slot 16c + 8g.
#pragma unroll
    for (int jj = 0; jj < C::VEC; ++jj) {
      const int w = jj >> 1;
      u32x4 t;
      if ((jj & 1) == 0) {
        t.x = pack_lo(vreg[0][w], vreg[1][w]);
        t.y = pack_lo(vreg[2][w], vreg[3][w]);
        t.z = pack_lo(vreg[4][w], vreg[5][w]);
        t.w = pack_lo(vreg[6][w], vreg[7][w]);
      } else {
        t.x = pack_hi(vreg[0][w], vreg[1][w]);
        t.y = pack_hi(vreg[2][w], vreg[3][w]);
        t.z = pack_hi(vreg[4][w], vreg[5][w]);
        t.w = pack_hi(vreg[6][w], vreg[7][w]);
      }
      const int dim = vm.dv * C::VEC + jj;
      *reinterpret_cast<u32x4*>(vs + dim * C::VS + vm.c * 8 + vm.g * 4) = t;
    }
  };

  // ---- running state
  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float m_run = -INFINITY;  // running max of scaled scores, log2 units
  float l_run = 0.f;        // this lane's share of the running row sum

  const int wave_row_last = row0 + wave * 32 + 31;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int tile = 0; tile < n_tiles; ++tile) {
    const int stage = tile & 1;
    const bool has_next = tile + 1 < n_tiles;
    if (has_next) load_tile(tile + 1);

    const int key0 = tile * kBlockN;
    // Causal: a wave whose last row precedes this tile has nothing to do.
    const bool active = !CAUSAL || key0 <= wave_row_last;
    if (active) {
      const uint32_t* ks = lds + stage * C::STAGE_DW;
      const uint32_t* vs = ks + C::K_DW;

      // S^T = K Q^T for the tile: sacc[nb] holds keys 32nb..32nb+31.
      f32x16 sacc[C::NB];
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[nb][r] = 0.f;
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              ks + (nb * 32 + l32) * C::KS + kc * 8 + g * 4);
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc],
                                                             sacc[nb], 0, 0, 0);
        }
      }

      // Mask keys past N, and (causal) keys after the query row.
      // Accumulator r of block nb is key 32nb + 8(r/4) + 4g + (r%4).
      const bool need_mask =
          (key0 + kBlockN > N) || (CAUSAL && key0 + kBlockN - 1 > row0 + wave * 32);
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + nb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
            const bool ok = key < N && (!CAUSAL || key <= my_row);
            sacc[nb][r] = ok ? sacc[nb][r] : -INFINITY;
          }
      }

      // Online softmax (log2 domain, scale folded into one FMA).
      float mx = -INFINITY;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[nb][r]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx * scale_log2);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float rsum = 0.f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p =
              __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[nb][r], scale_log2, -m_use));
          sacc[nb][r] = p;
          rsum += p;
        }
      l_run = l_run * alpha + rsum;
      m_run = m_new;
#pragma unroll
      for (int i = 0; i < C::DB; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;

      // O^T += V^T P^T, 16 keys per MFMA.
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
        const int nb = c >> 1, r0 = (c & 1) * 8;
        u32x4 pw;
        pw.x = pack_bf16x2(sacc[nb][r0 + 0], sacc[nb][r0 + 1]);
        pw.y = pack_bf16x2(sacc[nb][r0 + 2], sacc[nb][r0 + 3]);
        pw.z = pack_bf16x2(sacc[nb][r0 + 4], sacc[nb][r0 + 5]);
        pw.w = pack_bf16x2(sacc[nb][r0 + 6], sacc[nb][r0 + 7]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
        for (int db = 0; db < C::DB; ++db) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(
              vs + (db * 32 + l32) * C::VS + c * 8 + g * 4);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[db],
                                                             0, 0, 0);
        }
      }
    }

    if (has_next) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O /= l, lse = ln2 * (m + log2 l)
  const float l_tot = xhalf_sum(l_run);
  const float inv = 1.f / l_tot;
  // O^T accumulator r of block db is dim 32db + 8(r/4) + 4g + (r%4).
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int col = db * 32 + rr * 8 + g * 4;
      if (col < d) {
        u32x2 w;
        w.x = pack_bf16x2(oacc[db][rr * 4 + 0] * inv, oacc[db][rr * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[db][rr * 4 + 2] * inv, oacc[db][rr * 4 + 3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(w, o_rs, (my_row * d + col) * 2, 0, 0);
      }
    }
  if (lse != nullptr && g == 0 && my_row < N) {
    const float ln2 = 0.6931471805599453f;
    lse[((uint64_t)wc.b * H_Q + wc.h) * (uint64_t)N + my_row] =
        (m_run + __builtin_amdgcn_logf(l_tot)) * ln2;
  }
}

}  // namespace attn_numa
