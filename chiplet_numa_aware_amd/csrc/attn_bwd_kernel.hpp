// Attention backward for gfx950: dQ, dK, dV of sum(dO * O), FlashAttention-2
// style (P is recomputed from Q, K and the forward's lse).  "Optimizing
// Attention on GPUs by Exploiting GPU Architectural NUMA Effects", digest
// page, Q3 results table and the §3 "Backward pass" paragraph (Figure 16):
// the same workgroup remaps applied to FA2's backward kernel.  With S = Q K^T / sqrt(d), P = exp(S - lse):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// Three kernels:
//   * attn_bwd_pre: per query row, D and lse in log2 units (one wave per row).
//   * attn_bwd_dkv: one workgroup per (batch, KV head, 128-key block); each
//     wave owns 32 keys, the block's K and V stay in LDS, and the workgroup
//     streams 32-row tiles of Q, dO (and the rows' lse, D) of every query
//     head of the KV group.  dK and dV accumulate in registers: GQA needs no
//     atomics.
//   * attn_bwd_dq: one workgroup per (batch, query head, 128-row block); each
//     wave owns 32 rows (Q and dO in registers) and streams 32-key K/V tiles.
// Both gradient kernels take their workgroup coordinates from wg_map, so the
// four remaps (and longest first) apply as in the forward pass; every output
// element is written by one workgroup in a fixed order, so results do not
// depend on the mapping.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, as in the forward kernel): a score
// tile is computed so that each lane's 16 accumulators lie in one column, and
// P or dS, rounded to bf16, feed the next MFMA from registers as the B operand
// with the k order the transposing LDS reads (ds_read_b64_tr_b16) produce for
// the A operand.  LDS tiles are 32 rows of D/8 16-byte chunks, chunk c of row
// r at slot c ^ swz(r) (BwdCfg).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_fwd_kernel.hpp"
#include "wg_map.hpp"

namespace attn_numa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdBlock = 128;   // keys (dK/dV kernel) or rows (dQ kernel) per workgroup
constexpr int kBwdThreads = 256;
constexpr int kBwdTile = 32;     // rows of a streamed tile

// D = rowsum(dO * O) (fp32) and lse * log2(e), one wave per row; lane l owns
// columns 2l, 2l+1.  ws holds [lse2 | D], each rows floats.
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ ws, uint64_t rows, int d) {
  const int lane = threadIdx.x & 63;
  const uint64_t row = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  float acc = 0.f;
  const int c = 2 * lane;
  if (c < d) {
    const uint32_t ov = *reinterpret_cast<const uint32_t*>(o + row * d + c);
    const uint32_t dv = *reinterpret_cast<const uint32_t*>(dout + row * d + c);
    acc = __uint_as_float(ov << 16) * __uint_as_float(dv << 16) +
          __uint_as_float(ov & 0xFFFF0000u) * __uint_as_float(dv & 0xFFFF0000u);
  }
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) acc += __shfl_xor(acc, s, 64);
  if (lane == 0) {
    ws[row] = lse[row] * 1.4426950408889634f;
    ws[rows + row] = acc;
  }
}

template <int D>
struct BwdCfg {
  static_assert(D == 64 || D == 128, "padded head dim is 64 or 128");
  static constexpr int KC = D / 16, DB = D / 32, CPR = D / 8, ROWB = D * 2;
  static constexpr int TILE_B = kBwdTile * ROWB;
  static constexpr int SLOTS = kBwdTile * CPR / kBwdThreads;  // 16-byte loads per thread
  static_assert(SLOTS * kBwdThreads == kBwdTile * CPR, "a tile splits into the workgroup");
  // Chunk swizzle.  gfx950's LDS has 64 banks of 4 bytes and serves 16 lanes
  // of a 16-byte read (here: 16 consecutive rows, one chunk) and 32 lanes of
  // a transposing 8-byte read (4 consecutive rows from a multiple of 4, one
  // aligned group of 4 chunks) per cycle; both are free of bank conflicts.
  // D = 128 (256-byte rows, all starting at bank 0): a permutation over
  // r mod 16 whose value / 4 differs among 4 consecutive rows.  D = 64
  // (128-byte rows, alternating bank halves): the 8 rows of one parity go to
  // the 8 slots, rows 4i and 4i+2 to different groups of 4.
  static __device__ __forceinline__ constexpr int swz(int r) {
    return D == 64 ? 4 * ((r >> 1) & 1) + ((r >> 2) & 3) : 4 * (r & 3) + ((r >> 2) & 3);
  }
};

// a ^ K where it is used: the volatile asm keeps the compiler from hoisting
// the XORed addresses out of the loops into registers of their own.
// (k is a constant once the loops around the reads are unrolled.)
__device__ __forceinline__ int xor_at_use(int a, int k) {
  if (k == 0) return a;
  int r;
  asm volatile("v_xor_b32 %0, %1, %2" : "=v"(r) : "s"(k), "v"(a));
  return r;
}

// Per-lane LDS addresses of the two operand kinds, for a tile at byte 0.
// D = 128: only the addresses of chunks 0..7 are kept.  Chunk c + 8 sits at
// slot (c ^ swz) ^ 8, i.e. the address XOR 128; row r + 8 (the second half of
// a transposing read) has swz(r) ^ 2, i.e. the address XOR 32, 8 rows
// further.  The XORs take one VALU op per read instead of twice the address
// registers (which made the dK/dV kernel spill).  D = 64: rows r and r + 8
// differ in the group bit of the swizzle, so both halves of a transposing
// read keep an address.
template <int D>
struct TileAddr {
  using C = BwdCfg<D>;
  static constexpr int NR = C::KC < 4 ? C::KC : 4, NT = C::DB < 2 ? C::DB : 2;
  static constexpr int NH = D == 64 ? 2 : 1;
  int row_addr[NR];     // 16-byte read of row l32, chunk 2kc + g
  int tr_addr[NT][NH];  // transposing read (4 rows x 8 bytes per lane group), rows + 8h
  __device__ __forceinline__ TileAddr(int lane) {
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int kc = 0; kc < NR; ++kc)
      row_addr[kc] = l32 * C::ROWB + (((kc * 2 + g) ^ C::swz(l32)) * 16);
    const int j = lane & 15, kk = j >> 2, qq = j & 3, dhalf = (lane >> 4) & 1;
    const int krow = 4 * g + kk, w = 2 * dhalf + (qq >> 1);
#pragma unroll
    for (int db = 0; db < NT; ++db)
#pragma unroll
      for (int h = 0; h < NH; ++h)
        tr_addr[db][h] = (krow + 8 * h) * C::ROWB +
                         (((4 * db + w) ^ C::swz(krow + 8 * h)) * 16) + (qq & 1) * 8;
  }
  __device__ __forceinline__ int row(int kc) const {
    return xor_at_use(row_addr[kc % NR], (kc / NR) * 128);
  }
  // h = 1: the second half (rows + 8) of a transposing read.
  __device__ __forceinline__ int tr(int db, int h) const {
    if constexpr (NH == 2)
      return xor_at_use(tr_addr[db % NT][h], (db / NT) * 128);
    else
      return xor_at_use(tr_addr[db % NT][0], (db / NT) * 128 + h * 32) + h * 8 * C::ROWB;
  }
};

template <int D>
__device__ __forceinline__ bf16x8 lds_row_frag(const char* lds, int tile_byte,
                                               const TileAddr<D>& a, int kc) {
  return *reinterpret_cast<const bf16x8*>(lds + tile_byte + a.row(kc));
}
// Rows 16c .. 16c+15 of the tile, transposed: output lane (col 32db + l32)
// gets the 8 rows 16c + {4g..4g+3, 8+4g..8+4g+3}.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_frag(const char* lds, int tile_byte,
                                              const TileAddr<D>& a, int c, int db) {
  using C = BwdCfg<D>;
  const char* p = lds + tile_byte + c * 16 * C::ROWB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p + a.tr(db, 0)));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p + a.tr(db, 1)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Loads 32 rows (from row `row0` of a head of `head_rows` rows) of a tensor
// into an LDS tile at byte `tile_byte`: thread t fills slots t + 256 i.
template <int D, bool FULL_D>
__device__ __forceinline__ void bwd_load_tile(u32x4 desc, int row0, int head_rows, int dd,
                                              uint32_t lds_base, int tile_byte, int tid) {
  using C = BwdCfg<D>;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t head_bytes = (uint32_t)head_rows * (uint32_t)dd * 2u;
  const uint32_t soff0 = (uint32_t)row0 * (uint32_t)dd * 2u;
  const uint32_t soff = soff0 < head_bytes ? soff0 : head_bytes;
#pragma unroll
  for (int i = 0; i < C::SLOTS; ++i) {
    const int P = tid + kBwdThreads * i;
    const int row = P / C::CPR;
    const int chunk = (P % C::CPR) ^ C::swz(row);
    const uint32_t voff = (FULL_D || chunk * 8 < dd) ? (uint32_t)(row * dd + chunk * 8) * 2u
                                                     : kOutOfRange;
    load_lds(desc, voff, soff, lds_base + tile_byte + (wave + 4 * i) * 1024);
  }
}

// KB key blocks of 32 per wave (KB * 128 keys per workgroup).  With KB = 2
// every Q and dO fragment read from LDS feeds two MFMAs (half the LDS traffic
// per MFMA); the 2 x 128 dK/dV accumulators then need one wave per SIMD.
template <int D, bool CAUSAL, bool FULL_D, int KB>
__global__ __launch_bounds__(kBwdThreads, KB == 1 ? 2 : 1) void attn_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ ws, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int B, int H_Q, int H_KV, int N, int d, int M, int mapping, int num_xcd,
    float scale_log2, float scale) {
  using C = BwdCfg<D>;
  // LDS: 2 x (Q tile, dO tile), then 2 x [lse2 of the tile's 32 rows | D].
  constexpr int kStat = 4 * C::TILE_B;
  constexpr int kLdsB = kStat + 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) uint32_t lds[kLdsB / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  float* const stat = reinterpret_cast<float*>(lb + kStat);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);
  auto q_tile = [&](int buf) { return buf * 2 * C::TILE_B; };
  auto do_tile = [&](int buf) { return buf * 2 * C::TILE_B + C::TILE_B; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H_Q / H_KV;
  // Key block M - 1 - m: the remap's row block m counts from the block with
  // the least work under a causal mask, and for keys that is the last block
  // (it is seen by the fewest query rows).
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_KV, M, num_xcd, 1);
  const int key0 = (M - 1 - (int)wc.m) * kBwdBlock * KB;
  int my_key[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) my_key[kb] = key0 + (wave * KB + kb) * 32 + l32;
  const int dd = FULL_D ? D : d;
  const uint32_t head_elems = (uint32_t)N * (uint32_t)dd;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + wc.h) * head_elems;
  const uint64_t rows = (uint64_t)B * H_Q * N;
  const TileAddr<D> ta(lane);

  // K and V of this lane's keys, B operands (K^T, V^T): dims 16kc + 8g .. +7.
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + kv_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + kv_head, head_elems * 2);
  bf16x8 kf[KB][C::KC], vf[KB][C::KC];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      const int col = kc * 16 + g * 8;
      const uint32_t off =
          (FULL_D || col < dd) ? (uint32_t)(my_key[kb] * dd + col) * 2u : kOutOfRange;
      kf[kb][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rs, off, 0, 0));
      vf[kb][kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(v_rs, off, 0, 0));
    }

  // Padded head-dim columns are never written by the tile loads.
  if (!FULL_D) {
    for (int i = tid; i < kStat / 16; i += kBwdThreads)
      *reinterpret_cast<u32x4*>(lb + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }

  // Query tiles: every head of the group, tiles qt0 .. nq-1 of each (causal:
  // rows before the block see none of its keys).
  const int nq = (N + kBwdTile - 1) / kBwdTile;
  const int qt0 = CAUSAL ? key0 / kBwdTile : 0;
  const int per_head = nq - qt0;
  const int n_iter = G * per_head;
  auto issue = [&](int it, int buf) {
    const int hg = it / per_head, qt = qt0 + (it - hg * per_head);
    const uint64_t q_head = ((uint64_t)wc.b * H_Q + (int)wc.h * G + hg) * head_elems;
    bwd_load_tile<D, FULL_D>(make_desc(q + q_head, head_elems * 2), qt * kBwdTile, N, dd,
                             lds_base, q_tile(buf), tid);
    bwd_load_tile<D, FULL_D>(make_desc(dout + q_head, head_elems * 2), qt * kBwdTile, N, dd,
                             lds_base, do_tile(buf), tid);
  };
  // lse2 and D of a tile's rows reach LDS through the registers of wave 0.
  float st_l = 0.f, st_d = 0.f;
  auto stat_load = [&](int it) {
    const int hg = it / per_head, qt = qt0 + (it - hg * per_head);
    const int r = min(qt * kBwdTile + l32, N - 1);
    const uint64_t idx = ((uint64_t)wc.b * H_Q + (int)wc.h * G + hg) * N + r;
    st_l = ws[idx];
    st_d = ws[rows + idx];
  };
  auto stat_store = [&](int buf) {
    if (tid < 32) {
      stat[buf * 64 + tid] = st_l;
      stat[buf * 64 + 32 + tid] = st_d;
    }
  };

  f32x16 dk_acc[KB][C::DB], dv_acc[KB][C::DB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
      dk_acc[kb][db] = f32x16{};
      dv_acc[kb][db] = f32x16{};
    }
  if (n_iter > 0) {
    issue(0, 0);
    if (wave == 0) stat_load(0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  stat_store(0);
  __syncthreads();

  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    const int qt = qt0 + it % per_head;
    if (it + 1 < n_iter) {
      issue(it + 1, buf ^ 1);
      if (wave == 0) stat_load(it + 1);
    }
    // S = Q K^T and dP = dO V^T for this wave's keys: lane (key l32 of block
    // kb, half g) holds rows 8(r/4) + 4g + (r%4) of the tile.  Each LDS
    // fragment feeds the KB key blocks.
    f32x16 s[KB], dp[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
    }
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      const bf16x8 qa = lds_row_frag<D>(lb, q_tile(buf), ta, kc);
      const bf16x8 da = lds_row_frag<D>(lb, do_tile(buf), ta, kc);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[kb][kc], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vf[kb][kc], dp[kb], 0, 0, 0);
      }
    }
    const float* st = stat + buf * 64;
    uint32_t pk[KB][8], dsk[KB][8];
    // P and dS of the tile, rounded to bf16; MASKED adds the per-element test
    // (a row past N, a key past N, causal: a key after the row).
    auto softmax_grad = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const f32x4 lrow = *reinterpret_cast<const f32x4*>(st + 8 * c4 + 4 * g);
        const f32x4 drow = *reinterpret_cast<const f32x4*>(st + 32 + 8 * c4 + 4 * g);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          float p4[4], ds4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * c4 + e;
            float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], scale_log2, -lrow[e]));
            if constexpr (MASKED) {
              const int qrow = qt * kBwdTile + 8 * c4 + 4 * g + e;
              const bool ok = qrow < N && my_key[kb] < N && (!CAUSAL || my_key[kb] <= qrow);
              p = ok ? p : 0.f;
            }
            p4[e] = p;
            ds4[e] = p * (dp[kb][r] - drow[e]);
          }
          pk[kb][2 * c4] = pack_bf16x2(p4[0], p4[1]);
          pk[kb][2 * c4 + 1] = pack_bf16x2(p4[2], p4[3]);
          dsk[kb][2 * c4] = pack_bf16x2(ds4[0], ds4[1]);
          dsk[kb][2 * c4 + 1] = pack_bf16x2(ds4[2], ds4[3]);
        }
      }
    };
    // The test is needed only where some (row, key) pair of the wave is out:
    // the tile holding row N-1, the key block holding key N-1, and (causal)
    // tiles whose first row is before the wave's last key.
    const int wave_key_end = key0 + (wave + 1) * KB * 32;  // one past the wave's keys
    const bool full = (qt + 1) * kBwdTile <= N && wave_key_end <= N &&
                      (!CAUSAL || qt * kBwdTile >= wave_key_end - 1);
    if (full)
      softmax_grad(std::false_type{});
    else
      softmax_grad(std::true_type{});
    // dV^T += dO^T P and dK^T += Q^T dS, k = the tile's rows (16 per chunk c);
    // each transposed fragment feeds the KB key blocks.
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const bf16x8 dot = lds_tr_frag<D>(lb, do_tile(buf), ta, c, db);
        const bf16x8 qt_ = lds_tr_frag<D>(lb, q_tile(buf), ta, c, db);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
          const bf16x8 pb = __builtin_bit_cast(
              bf16x8, u32x4{pk[kb][4 * c], pk[kb][4 * c + 1], pk[kb][4 * c + 2], pk[kb][4 * c + 3]});
          const bf16x8 sb = __builtin_bit_cast(
              bf16x8, u32x4{dsk[kb][4 * c], dsk[kb][4 * c + 1], dsk[kb][4 * c + 2], dsk[kb][4 * c + 3]});
          dv_acc[kb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dot, pb, dv_acc[kb][db], 0, 0, 0);
          dk_acc[kb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt_, sb, dk_acc[kb][db], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    if (it + 1 < n_iter) stat_store(buf ^ 1);
    __syncthreads();
  }

  // Accumulator r of block db is dim 32db + 8(r/4) + 4g + (r%4) of the key;
  // rows past N fall outside the buffer and are dropped.
  const __amdgpu_buffer_rsrc_t dk_rs = make_rsrc(dk + kv_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t dv_rs = make_rsrc(dv + kv_head, head_elems * 2);
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col = db * 32 + rr * 8 + g * 4;
        if (FULL_D || col < dd) {
          const uint32_t off = (uint32_t)(my_key[kb] * dd + col) * 2u;
          u32x2 w;
          w.x = pack_bf16x2(dk_acc[kb][db][rr * 4 + 0] * scale, dk_acc[kb][db][rr * 4 + 1] * scale);
          w.y = pack_bf16x2(dk_acc[kb][db][rr * 4 + 2] * scale, dk_acc[kb][db][rr * 4 + 3] * scale);
          __builtin_amdgcn_raw_buffer_store_b64(w, dk_rs, off, 0, 0);
          w.x = pack_bf16x2(dv_acc[kb][db][rr * 4 + 0], dv_acc[kb][db][rr * 4 + 1]);
          w.y = pack_bf16x2(dv_acc[kb][db][rr * 4 + 2], dv_acc[kb][db][rr * 4 + 3]);
          __builtin_amdgcn_raw_buffer_store_b64(w, dv_rs, off, 0, 0);
        }
      }
    }
}

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ ws, uint16_t* __restrict__ dq,
    int B, int H_Q, int H_KV, int N, int d, int M, int mapping, int num_xcd,
    float scale_log2, float scale) {
  using C = BwdCfg<D>;
  // LDS: 2 x (K tile, V tile).
  __shared__ __attribute__((aligned(16))) uint32_t lds[4 * C::TILE_B / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);
  auto k_tile = [&](int buf) { return buf * 2 * C::TILE_B; };
  auto v_tile = [&](int buf) { return buf * 2 * C::TILE_B + C::TILE_B; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, l32 = lane & 31;
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_Q, M, num_xcd, H_Q / H_KV);
  const int kvh = (int)wc.h / (H_Q / H_KV);
  const int row0 = (int)wc.m * kBwdBlock;
  const int my_row = row0 + wave * 32 + l32;
  const int dd = FULL_D ? D : d;
  const uint32_t head_elems = (uint32_t)N * (uint32_t)dd;
  const uint64_t q_head = ((uint64_t)wc.b * H_Q + wc.h) * head_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * head_elems;
  const uint64_t rows = (uint64_t)B * H_Q * N;
  const TileAddr<D> ta(lane);

  // Q and dO of this lane's row as B operands (Q^T, dO^T): dims 16kc+8g..+7.
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(dout + q_head, head_elems * 2);
  bf16x8 qf[C::KC], df[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    const int col = kc * 16 + g * 8;
    const uint32_t off = (FULL_D || col < dd) ? (uint32_t)(my_row * dd + col) * 2u : kOutOfRange;
    qf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, off, 0, 0));
    df[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(do_rs, off, 0, 0));
  }
  const uint64_t ridx = ((uint64_t)wc.b * H_Q + wc.h) * N + (my_row < N ? my_row : N - 1);
  const float lse2 = ws[ridx];
  const float drow = ws[rows + ridx];

  // Padded head-dim columns are never written by the tile loads.
  if (!FULL_D) {
    for (int i = tid; i < 4 * C::TILE_B / 16; i += kBwdThreads)
      *reinterpret_cast<u32x4*>(lb + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  const u32x4 k_desc = make_desc(k + kv_head, head_elems * 2);
  const u32x4 v_desc = make_desc(v + kv_head, head_elems * 2);
  int n_tiles = (N + kBwdTile - 1) / kBwdTile;
  if (CAUSAL) n_tiles = min(n_tiles, (row0 + kBwdBlock + kBwdTile - 1) / kBwdTile);
  bwd_load_tile<D, FULL_D>(k_desc, 0, N, dd, lds_base, k_tile(0), tid);
  bwd_load_tile<D, FULL_D>(v_desc, 0, N, dd, lds_base, v_tile(0), tid);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  f32x16 dq_acc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) dq_acc[db] = f32x16{};
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) {
      bwd_load_tile<D, FULL_D>(k_desc, (j + 1) * kBwdTile, N, dd, lds_base, k_tile(buf ^ 1), tid);
      bwd_load_tile<D, FULL_D>(v_desc, (j + 1) * kBwdTile, N, dd, lds_base, v_tile(buf ^ 1), tid);
    }
    // S^T = K Q^T and dP^T = V dO^T: lane (row l32, half g) holds keys
    // 32j + 8(r/4) + 4g + (r%4).
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_frag<D>(lb, k_tile(buf), ta, kc),
                                                  qf[kc], s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row_frag<D>(lb, v_tile(buf), ta, kc),
                                                   df[kc], dp, 0, 0, 0);
    }
    uint32_t dsk[8];
    // dS^T of the tile; MASKED adds the per-element test (a key past N, a
    // row past N, causal: a key after the row).
    auto softmax_grad = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float ds2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * w + e;
          float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], scale_log2, -lse2));
          if constexpr (MASKED) {
            const int key = j * kBwdTile + (r >> 2) * 8 + g * 4 + (r & 3);
            const bool ok = key < N && my_row < N && (!CAUSAL || key <= my_row);
            p = ok ? p : 0.f;
          }
          ds2[e] = p * (dp[r] - drow);
        }
        dsk[w] = pack_bf16x2(ds2[0], ds2[1]);
      }
    };
    // The test is needed only for the tile holding key N-1, the wave holding
    // row N-1, and (causal) tiles whose last key is after the wave's first row.
    const int wave_row0 = row0 + wave * 32;
    const bool full = (j + 1) * kBwdTile <= N && wave_row0 + 32 <= N &&
                      (!CAUSAL || (j + 1) * kBwdTile - 1 <= wave_row0);
    if (full)
      softmax_grad(std::false_type{});
    else
      softmax_grad(std::true_type{});
    // dQ^T += K^T dS^T (k = the tile's keys, 16 per chunk c).
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const bf16x8 b_ = __builtin_bit_cast(bf16x8, u32x4{dsk[4 * c], dsk[4 * c + 1], dsk[4 * c + 2], dsk[4 * c + 3]});
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        dq_acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            lds_tr_frag<D>(lb, k_tile(buf), ta, c, db), b_, dq_acc[db], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const __amdgpu_buffer_rsrc_t dq_rs = make_rsrc(dq + q_head, head_elems * 2);
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int col = db * 32 + rr * 8 + g * 4;
      if (FULL_D || col < dd) {
        u32x2 w;
        w.x = pack_bf16x2(dq_acc[db][rr * 4 + 0] * scale, dq_acc[db][rr * 4 + 1] * scale);
        w.y = pack_bf16x2(dq_acc[db][rr * 4 + 2] * scale, dq_acc[db][rr * 4 + 3] * scale);
        __builtin_amdgcn_raw_buffer_store_b64(w, dq_rs, (uint32_t)(my_row * dd + col) * 2u, 0, 0);
      }
    }
  }
}

}  // namespace attn_numa
