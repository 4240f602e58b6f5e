// Attention backward for gfx950: dQ, dK, dV of sum(dO * O), FlashAttention-2
// style (P is recomputed from Q, K and the forward's lse).  "Optimizing
// Attention on GPUs by Exploiting GPU Architectural NUMA Effects", digest
// page, Q3 results table and the §3 "Backward pass" paragraph (Figure 16):
// the same workgroup remaps applied to FA2's backward kernel.  With S = Q K^T / sqrt(d), P = exp(S - lse):
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D) with D = rowsum(dO * O),
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d).
// Three kernels:
//   * attn_bwd_pre: per query row, D and lse in log2 units (one wave per row).
//   * attn_bwd_dkv: one workgroup per (batch, KV head, 128-key block), one
//     wave per SIMD; each wave owns 32 keys (K and V in registers) and the
//     workgroup streams 32-row tiles of Q, dO (and the rows' lse, D) of
//     every query head of the KV group through a five-stage LDS ring.  dK
//     and dV accumulate in registers: GQA needs no atomics.
//   * attn_bwd_dq: one workgroup per (batch, query head, 128-row block), two
//     per CU; each wave owns 32 rows (Q and dO in registers) and streams
//     32-key K/V tiles through a four-stage LDS ring.  It uses 16 x 16 MFMA
//     blocks (v_mfma_f32_16x16x32_bf16), which draw less power per FLOP than
//     32 x 32 ones under the chip's power limit (measured 8% faster here).
// Both gradient kernels take their workgroup coordinates from wg_map, so the
// four remaps (and longest first) apply as in the forward pass; every output
// element is written by one workgroup in a fixed order, so results do not
// depend on the mapping.
//
// MFMA layout (dK/dV: v_mfma_f32_32x32x16_bf16 as in the forward kernel;
// dQ: the 16 x 16 x 32 form): a score tile is computed so that each lane's
// accumulators lie in one column, and P or dS, rounded to bf16, feed the next
// MFMA from registers as the B operand with the k order the transposing LDS
// reads (ds_read_b64_tr_b16) produce for the A operand.  LDS tiles are 32 rows of D/8 16-byte chunks, chunk c of row
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

// D = rowsum(dO * O) (fp32) and lse2 = lse * log2(e), one wave per row;
// lane l owns columns 2l, 2l+1.  ws holds [-lse2 | -D] of each (batch, query
// head), N floats each.  Both gradient kernels start their MFMA accumulators
// from these: S from -lse2, with the operand held in registers (K in the
// dK/dV kernel, Q in the dQ kernel) scaled once by log2(e) / sqrt(d) and
// rounded to bf16, so the MFMAs return S log2(e) / sqrt(d) - lse2 and
// P = exp2 of it with no FMA; dP = dO V^T from -D, so they return dP - D, the
// factor of dS = P (dP - D), with no subtraction.  The scaled operand's
// rounding adds about 1.7e-3 relative L2 to the gradients (2.4e-3 -> 3.0e-3
// median on the parity cases).
__global__ __launch_bounds__(256) void attn_bwd_pre_kernel(
    const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, float* __restrict__ ws, uint64_t rows, int d, int N) {
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
    const uint64_t head = row / (uint64_t)N, r = row - head * (uint64_t)N;
    ws[head * 2u * N + r] = -lse[row] * 1.4426950408889634f;  // -lse2: S starts from it
    ws[head * 2u * N + N + r] = -acc;  // -D: the dP accumulators start from it
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

// ---------------------------------------------------------------------------
// dK/dV kernel.  One workgroup per (batch, KV head, 128-key block): four waves
// of 32 keys, one wave per SIMD.  K^T and V^T of a wave's keys (the B
// operands of S = Q K^T and dP = dO V^T) and the dK^T, dV^T accumulators sit
// in AGPRs for the whole kernel.  The workgroup streams 32-row tiles of Q and
// dO, of every query head of the KV group, through a ring of kDkvStages LDS
// stages; tile t+3 is loaded LDS-direct during the body of tile t, one
// instruction per bundle, together with its rows' lse2 and D (one 256-byte
// copy per wave), and first read two bodies later.
//
// The body of tile t is one static schedule of MFMA "bundles":
//   first part:  dV^T += dO^T P and dK^T += Q^T dS of tile t-1, while the
//                VALU forms P and dS of tile t from its S and dP;
//   second part: S and dP of tile t+1;
//   tail:        the first operand fragments of the next body and the stats
//                of tile t+1 are read, then one barrier.
// Every LDS operand is read AHEAD bundles before its MFMA, so after the
// barrier the next body starts with its operands in registers.  The ring
// needs five stages: in body t the MFMAs read tiles t-1 and t+1 and the
// stats of tile t, and the loads go to tile t+3.
constexpr int kDkvStages = 5;

template <int D>
struct DkvCfg {
  using C = BwdCfg<D>;
  static constexpr int DO0 = kDkvStages * C::TILE_B;      // dO tiles (Q tiles at 0)
  static constexpr int ST0 = 2 * kDkvStages * C::TILE_B;  // stats of stage s, wave w
  static constexpr int ST_STAGE = 4 * 256;
  static constexpr int BYTES = ST0 + kDkvStages * ST_STAGE;
  static constexpr int LPT = 2 * C::SLOTS + 1;  // LDS-direct loads per thread and tile
  static constexpr int NA = 4 * C::DB;          // dV and dK MFMAs of a tile
  static constexpr int NB = 2 * C::KC;          // S and dP MFMAs of a tile
  static constexpr int NF = NA + NB;            // bundles per tile
  static constexpr int AHEAD = 4;               // operand fragments in flight
  // Bundles over which P and dS of a tile are formed: the whole tile.  (With
  // the accumulator starts that remove the FMA and the subtraction, keeping
  // them in the first part at D = 128 measured 0.6-1.0% slower.)
  static constexpr int NV = NF;
  static_assert(BYTES <= 160 * 1024, "LDS");
  static_assert(kDkvStages * C::TILE_B <= 65536 - C::TILE_B, "stage offsets fit ds_read immediates");
};

// dP - D in one MFMA: the first 16-deep step of dP = dO V^T starts from the
// rows' -D instead of 0.  The s_nop covers a VALU write of the C block (2
// wait states before an XDL read of it).
__device__ __forceinline__ void mfma_scores_from(f32x16& acc, const bf16x8& a, const bf16x8& b,
                                                 const f32x16& c) {
  asm volatile("s_nop 2\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
               : "=&v"(acc) : "v"(a), "a"(b), "v"(c));
}

// x * c for 8 bf16 values, rounded back to bf16 (nearest even).
__device__ __forceinline__ bf16x8 scale_bf16x8(const bf16x8& x, float c) {
  const u32x4 w = __builtin_bit_cast(u32x4, x);
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = pack_bf16x2(__uint_as_float(w[i] << 16) * c, __uint_as_float(w[i] & 0xFFFF0000u) * c);
  return __builtin_bit_cast(bf16x8, r);
}

// LDS-direct load of 4 bytes per lane: lane l writes LDS at M0 + 4 l.
__device__ __forceinline__ void load_lds_dword(u32x4 desc, uint32_t voff, uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(m0)
      : "memory", "m0");
}

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kBwdThreads, 1) void attn_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ ws, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
    int B, int H_Q, int H_KV, int N, int d, int M, int mapping, int num_xcd,
    float scale_log2, float scale) {
  using C = BwdCfg<D>;
  using L = DkvCfg<D>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[L::BYTES / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);

  const int tid = threadIdx.x, lane = tid & 63;
  const int g = lane >> 5, l32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = H_Q / H_KV;
  // Key block M - 1 - m: the remap's row block m counts from the block with
  // the least work under a causal mask, and for keys that is the last block
  // (it is seen by the fewest query rows).
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_KV, M, num_xcd, 1);
  const int key0 = (M - 1 - (int)wc.m) * kBwdBlock;
  const int my_key = key0 + wave * 32 + l32;
  const int dd = FULL_D ? D : d;
  const uint32_t head_elems = (uint32_t)N * (uint32_t)dd;
  const uint32_t head_bytes = head_elems * 2u;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + wc.h) * head_elems;

  // K^T and V^T of this lane's key (B operands): dims 16kc + 8g .. +7.
  const __amdgpu_buffer_rsrc_t k_rs = make_rsrc(k + kv_head, head_bytes);
  const __amdgpu_buffer_rsrc_t v_rs = make_rsrc(v + kv_head, head_bytes);
  bf16x8 kf[C::KC], vf[C::KC];
  static_for<C::KC>([&](auto kci) {
    constexpr int kc = decltype(kci)::value;
    const int col = kc * 16 + g * 8;
    const uint32_t off = (FULL_D || col < dd) ? (uint32_t)(my_key * dd + col) * 2u : kOutOfRange;
    kf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(k_rs, off, 0, 0));
    vf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(v_rs, off, 0, 0));
  });
  static_for<C::KC>([&](auto kci) { kf[decltype(kci)::value] = scale_bf16x8(kf[decltype(kci)::value], scale_log2); });
  static_for<C::KC>([&](auto kci) {
    xdl_guard_a(kf[decltype(kci)::value]);
    xdl_guard_a(vf[decltype(kci)::value]);
  });

  // Zeroed LDS: the stage of "tile -1" that the first body multiplies by
  // P = dS = 0, and the padded head-dim columns.
  for (int i = tid; i < L::BYTES / 16; i += kBwdThreads)
    *reinterpret_cast<u32x4*>(lb + i * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();

  // ---- Tile sequence: every query head hg of the group, row tiles qt0 ..
  // nq-1 of each (causal: rows before the block see none of its keys).
  const int nq = (N + kBwdTile - 1) / kBwdTile;
  const int qt0 = CAUSAL ? key0 / kBwdTile : 0;
  const int n_iter = G * (nq - qt0);
  const uint64_t q_head0 = ((uint64_t)wc.b * H_Q + (uint64_t)wc.h * G) * head_elems;
  const uint64_t st_head0 = ((uint64_t)wc.b * H_Q + (uint64_t)wc.h * G) * 2u * (uint64_t)N;

  // LDS-direct slots of this thread in a tile: slot P = tid + 256 i holds
  // row P / CPR, chunk (P % CPR) ^ swz(row).
  uint32_t slot_off[C::SLOTS];
  static_for<C::SLOTS>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    const int P = tid + kBwdThreads * i;
    const int row = P / C::CPR;
    const int chunk = (P % C::CPR) ^ C::swz(row);
    slot_off[i] = (FULL_D || chunk * 8 < dd) ? (uint32_t)(row * dd + chunk * 8) * 2u : kOutOfRange;
  });
  // The loads of tile (hg, qt) into stage `stage`: descriptors and offsets
  // (a tile past the sequence, hg == G, reads nothing and writes zeros),
  // issued one instruction per bundle by issue_one<i>, i < LPT.
  struct LoadPlan {
    u32x4 q_desc, do_desc, st_desc;
    uint32_t soff, st_voff, stage;
  };
  // Cursor of the next tile to load: its query head c_hg, row tile c_qt and
  // the descriptors of that head, moved only when the head changes (the
  // scalar 64-bit address arithmetic then runs once per head, not per tile).
  u32x4 c_qd = make_desc(q + q_head0, head_bytes);
  u32x4 c_dod = make_desc(dout + q_head0, head_bytes);
  u32x4 c_std = make_desc(ws + st_head0, (uint32_t)N * 8u);
  int c_hg = 0, c_qt = qt0;
  auto desc_add = [](u32x4& dsc, uint64_t bytes) {
    const uint64_t a = ((uint64_t)(dsc.y & 0xFFFFu) << 32 | dsc.x) + bytes;
    dsc.x = (uint32_t)a;
    dsc.y = (uint32_t)(a >> 32) & 0xFFFFu;
  };
  auto advance = [&]() {
    if (++c_qt == nq) {
      c_qt = qt0;
      // Past the last head the descriptors stay on it; validity then comes
      // from c_hg alone.
      if (++c_hg < G) {
        desc_add(c_qd, (uint64_t)head_elems * 2u);
        desc_add(c_dod, (uint64_t)head_elems * 2u);
        desc_add(c_std, (uint64_t)N * 8u);
      }
    }
  };
  auto plan = [&](int stage) {
    LoadPlan lp;
    const bool valid = c_hg < G;
    lp.q_desc = c_qd;
    lp.do_desc = c_dod;
    const uint32_t soff0 = (uint32_t)(c_qt * kBwdTile) * (uint32_t)dd * 2u;
    lp.soff = (valid && soff0 < head_bytes) ? soff0 : head_bytes;
    // Stats: lanes 0-31 lse2 of rows qt*32 + l32, lanes 32-63 their D.
    lp.st_desc = c_std;
    const int r = min(c_qt * kBwdTile + l32, N - 1);
    lp.st_voff = valid ? (uint32_t)(g * N + r) * 4u : kOutOfRange;
    lp.stage = (uint32_t)stage;
    return lp;
  };
  auto issue_one = [&](const LoadPlan& lp, auto ii) {
    constexpr int i = decltype(ii)::value;
    const uint32_t stage = lp.stage;
    if constexpr (i < C::SLOTS)
      load_lds(lp.q_desc, slot_off[i], lp.soff,
               lds_base + stage * C::TILE_B + (wave + 4 * i) * 1024);
    else if constexpr (i < 2 * C::SLOTS)
      load_lds(lp.do_desc, slot_off[i - C::SLOTS], lp.soff,
               lds_base + L::DO0 + stage * C::TILE_B + (wave + 4 * (i - C::SLOTS)) * 1024);
    else
      load_lds_dword(lp.st_desc, lp.st_voff,
                     lds_base + L::ST0 + stage * L::ST_STAGE + wave * 256);
  };
  auto issue = [&](int stage) {
    const LoadPlan lp = plan(stage);
    static_for<L::LPT>([&](auto ii) { issue_one(lp, ii); });
  };

  // ---- Per-lane LDS addresses.  Row fragment kc (A operand of S or dP):
  // row l32, chunk 2kc + g.  Transposed fragment (c, db) (A operand of dV^T
  // or dK^T): rows 16c + 4g + {0..3} and 16c + 8 + 4g + {0..3} of dims
  // 32db + ..., two ds_read_b64_tr_b16 8 rows apart (as in lds_tr_frag).
  int row_q[C::KC], row_do[C::KC], tr_q[C::DB][2], tr_do[C::DB][2];
  static_for<C::KC>([&](auto kci) {
    constexpr int kc = decltype(kci)::value;
    row_q[kc] = l32 * C::ROWB + (((kc * 2 + g) ^ C::swz(l32)) * 16);
    row_do[kc] = row_q[kc] + L::DO0;
    pin(row_do[kc]);
  });
  {
    const int j = lane & 15, kk = j >> 2, qq = j & 3, dhalf = (lane >> 4) & 1;
    const int krow = 4 * g + kk, w = 2 * dhalf + (qq >> 1);
    static_for<C::DB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
      static_for<2>([&](auto hi) {
        constexpr int h = decltype(hi)::value;
        tr_q[db][h] = (krow + 8 * h) * C::ROWB +
                      (((4 * db + w) ^ C::swz(krow + 8 * h)) * 16) + (qq & 1) * 8;
        tr_do[db][h] = tr_q[db][h] + L::DO0;
        pin(tr_do[db][h]);
      });
    });
  }
  // The dO and stats regions start above the 16-bit immediate of ds_read:
  // their base addresses are pinned so that the compiler keeps one register
  // per address and the stage offsets as immediates.
  int st_addr = L::ST0 + wave * 256 + 16 * g;
  pin(st_addr);

  // Operand fragment f of the body whose tile t has stage PH: f < NA the
  // transposed fragments of tile t-1 (dO^T, Q^T alternating over (c, db)),
  // then the row fragments of tile t+1 (Q, dO alternating over kc).
  auto read_frag = [&](auto phi, auto fi) -> bf16x8 {
    constexpr int PH = decltype(phi)::value, f = decltype(fi)::value;
    if constexpr (f < L::NA) {
      constexpr int sp = (PH + kDkvStages - 1) % kDkvStages;
      constexpr int pair = f / 2, c = pair / C::DB, db = pair % C::DB;
      constexpr int off = sp * C::TILE_B + c * 16 * C::ROWB;
      const int a0 = (f % 2 == 0) ? tr_do[db][0] : tr_q[db][0];
      const int a1 = (f % 2 == 0) ? tr_do[db][1] : tr_q[db][1];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lb + off + a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(lb + off + a1));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      constexpr int sn = (PH + 1) % kDkvStages;
      constexpr int kc = (f - L::NA) / 2;
      const int a = ((f - L::NA) % 2 == 0) ? row_q[kc] : row_do[kc];
      return *reinterpret_cast<const bf16x8*>(lb + sn * C::TILE_B + a);
    }
  };
  // A block of the stats of a tile: part 0 the rows' -lse2, part 128 their
  // -D, element e = row 8 (e / 4) + 4 g + e % 4 (the accumulator order of
  // S and dP).
  auto read_block = [&](int stage, int part) {
    f32x16 nd;
    static_for<4>([&](auto ci) {
      constexpr int c4 = decltype(ci)::value;
      const f32x4 x = *reinterpret_cast<const f32x4*>(lb + st_addr + stage * L::ST_STAGE + part + 32 * c4);
      nd[4 * c4 + 0] = x[0];
      nd[4 * c4 + 1] = x[1];
      nd[4 * c4 + 2] = x[2];
      nd[4 * c4 + 3] = x[3];
    });
    return nd;
  };

  f32x16 dk_acc[C::DB], dv_acc[C::DB];
  static_for<C::DB>([&](auto dbi) {
    dk_acc[decltype(dbi)::value] = f32x16{};
    dv_acc[decltype(dbi)::value] = f32x16{};
  });

  // ---- Prologue: tiles 0-2 in flight, tiles 0 and 1 waited for; S and dP
  // of tile 0; P = dS = 0 for "tile -1" (its stage is zero).
  static_for<3>([&](auto si) {
    issue(decltype(si)::value);
    advance();
  });
  wait_vmcnt<L::LPT>();
  barrier();
  f32x16 s_cur, dp_cur;
  {
    const f32x16 nl0 = read_block(0, 0), nd0 = read_block(0, 128);
    static_for<C::KC>([&](auto kci) {
      constexpr int kc = decltype(kci)::value;
      const bf16x8 qa = *reinterpret_cast<const bf16x8*>(lb + row_q[kc]);
      const bf16x8 da = *reinterpret_cast<const bf16x8*>(lb + row_do[kc]);
      if constexpr (kc == 0)
        mfma_scores_from(s_cur, qa, kf[kc], nl0);
      else
        mfma_scores<true>(s_cur, qa, kf[kc]);
      if constexpr (kc == 0)
        mfma_scores_from(dp_cur, da, vf[kc], nd0);
      else
        mfma_scores<true>(dp_cur, da, vf[kc]);
    });
  }
  uint32_t pk[8], dsk[8];
  static_for<8>([&](auto i) {
    pk[decltype(i)::value] = 0u;
    dsk[decltype(i)::value] = 0u;
  });
  bf16x8 fr[L::AHEAD];
  static_for<L::AHEAD>([&](auto fi) {
    fr[decltype(fi)::value] = read_frag(std::integral_constant<int, 0>{}, fi);
  });

  // Causal / ragged mask of a lane's element (row 8 c4 + 4g + e of the tile):
  // visible iff lo <= row < hi, lo = the lane's key (causal) and hi = N (0 for
  // a key past N).
  const int m_lo = CAUSAL ? my_key : 0;
  const int m_span = my_key < N ? max(N - m_lo, 0) : 0;
  const int wave_key_end = key0 + (wave + 1) * 32;
  int qt_c = qt0;  // row tile of the tile being computed

  auto body = [&](auto phi, bool masked, int span) {
    constexpr int PH = decltype(phi)::value;
    constexpr int s_load = (PH + 3) % kDkvStages, s_next = (PH + 1) % kDkvStages;
    const LoadPlan lp = plan(s_load);
    advance();
    xdl_guard_v(s_cur, dp_cur);
    // A masked element gets S = -inf, hence P = 0 and dS = 0.
    if (masked) {
      const int m_a = qt_c * kBwdTile + 4 * g - m_lo;  // row - lo of element 0
      static_for<16>([&](auto ei) {
        constexpr int e = decltype(ei)::value;
        const bool ok = (uint32_t)(m_a + 8 * (e / 4) + e % 4) < (uint32_t)span;
        s_cur[e] = ok ? s_cur[e] : -__builtin_inff();
      });
    }
    bf16x8 frag[L::NF];
    static_for<L::AHEAD>([&](auto fi) { frag[decltype(fi)::value] = fr[decltype(fi)::value]; });
    const f32x16 nl_nx = read_block(s_next, 0);    // -lse2 of tile t+1, the C of its S
    const f32x16 nd_nx = read_block(s_next, 128);  // -D of tile t+1, the C of its dP
    uint32_t pk_n[8], dsk_n[8];
    float p_e[16], ds_e[16];
    f32x16 s_nx, dp_nx;
    static_for<L::NF>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      if constexpr (f < L::NA) {
        constexpr int pair = f / 2, c = pair / C::DB, db = pair % C::DB;
        if constexpr (f % 2 == 0) {
          const bf16x8 pb = __builtin_bit_cast(
              bf16x8, u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
          mfma_out<0>(dv_acc[db], frag[f], pb);
        } else {
          const bf16x8 sb = __builtin_bit_cast(
              bf16x8, u32x4{dsk[4 * c], dsk[4 * c + 1], dsk[4 * c + 2], dsk[4 * c + 3]});
          mfma_out<0>(dk_acc[db], frag[f], sb);
        }
      } else {
        constexpr int kc = (f - L::NA) / 2;
        if constexpr ((f - L::NA) % 2 == 0)
          if constexpr (kc == 0)
            mfma_scores_from(s_nx, frag[f], kf[kc], nl_nx);
          else
            mfma_scores<true>(s_nx, frag[f], kf[kc]);
        else
          if constexpr (kc == 0)
            mfma_scores_from(dp_nx, frag[f], vf[kc], nd_nx);
          else
            mfma_scores<true>(dp_nx, frag[f], vf[kc]);
      }
      // The tile loads go out one per bundle, behind the MFMA.
      if constexpr (f < L::LPT) issue_one(lp, fi);
      if constexpr (f + L::AHEAD < L::NF)
        frag[f + L::AHEAD] = read_frag(phi, std::integral_constant<int, f + L::AHEAD>{});
      // P and dS of the elements scheduled in this bundle.
      static_for<16>([&](auto ei) {
        constexpr int e = decltype(ei)::value;
        if constexpr (e * L::NV / 16 == f) {
          constexpr int c4 = e / 4, ee = e % 4;
          // Inputs and results are pinned to this bundle, so that the
          // arithmetic neither moves ahead of earlier MFMAs nor sinks into
          // the next body.
          float sv = s_cur[e], dpv = dp_cur[e];
          pin(sv);
          pin(dpv);
          const float p = __builtin_amdgcn_exp2f(sv);  // S log2(e) / sqrt(d) - lse2
          p_e[e] = p;
          ds_e[e] = p * dpv;  // dP - D
          if constexpr (e % 2 == 1) {
            pk_n[e / 2] = pack_bf16x2(p_e[e - 1], p_e[e]);
            dsk_n[e / 2] = pack_bf16x2(ds_e[e - 1], ds_e[e]);
            pin(pk_n[e / 2]);
            pin(dsk_n[e / 2]);
          }
        }
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Tail: the next body's first fragments (tile t, stage PH) and the stats
    // of tile t+1.
    static_for<L::AHEAD>([&](auto fi) {
      fr[decltype(fi)::value] = read_frag(std::integral_constant<int, (PH + 1) % kDkvStages>{}, fi);
    });
    static_for<8>([&](auto i) {
      pk[decltype(i)::value] = pk_n[decltype(i)::value];
      dsk[decltype(i)::value] = dsk_n[decltype(i)::value];
    });
    s_cur = s_nx;
    dp_cur = dp_nx;
    wait_vmcnt<L::LPT>();
    barrier();
  };
  // The tile needs the per-element test only where some (row, key) pair of
  // the wave is out: the tile holding row N-1, the key block holding key N-1,
  // and (causal) tiles whose first row is before the wave's last key.  The
  // sequence is padded to a multiple of the stage count with tiles that are
  // masked out entirely (their loads write zeros), so the loop has one exit
  // and the last tile sits in the last stage.
  const int n_pad = (n_iter + kDkvStages - 1) / kDkvStages * kDkvStages;
  auto step = [&](auto phi, int t) {
    const bool pad = t >= n_iter;
    const bool full = !pad && (qt_c + 1) * kBwdTile <= N && wave_key_end <= N &&
                      (!CAUSAL || qt_c * kBwdTile >= wave_key_end - 1);
    body(phi, !full, pad ? 0 : m_span);
    if (++qt_c == nq) qt_c = qt0;
  };
  for (int t = 0; t < n_pad; t += kDkvStages) {
    step(std::integral_constant<int, 0>{}, t);
    step(std::integral_constant<int, 1>{}, t + 1);
    step(std::integral_constant<int, 2>{}, t + 2);
    step(std::integral_constant<int, 3>{}, t + 3);
    step(std::integral_constant<int, 4>{}, t + 4);
  }
  // dV and dK of the last tile (stage kDkvStages - 1): the first part of one
  // more body.
  {
    bf16x8 frag[L::NA];
    static_for<L::AHEAD>([&](auto fi) { frag[decltype(fi)::value] = fr[decltype(fi)::value]; });
    static_for<L::NA>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      constexpr int pair = f / 2, c = pair / C::DB, db = pair % C::DB;
      if constexpr (f % 2 == 0) {
        const bf16x8 pb = __builtin_bit_cast(
            bf16x8, u32x4{pk[4 * c], pk[4 * c + 1], pk[4 * c + 2], pk[4 * c + 3]});
        mfma_out<0>(dv_acc[db], frag[f], pb);
      } else {
        const bf16x8 sb = __builtin_bit_cast(
            bf16x8, u32x4{dsk[4 * c], dsk[4 * c + 1], dsk[4 * c + 2], dsk[4 * c + 3]});
        mfma_out<0>(dk_acc[db], frag[f], sb);
      }
      if constexpr (f + L::AHEAD < L::NA)
        frag[f + L::AHEAD] = read_frag(std::integral_constant<int, 0>{},
                                       std::integral_constant<int, f + L::AHEAD>{});
    });
  }
  static_for<C::DB>([&](auto dbi) {
    xdl_guard_a(dk_acc[decltype(dbi)::value]);
    xdl_guard_a(dv_acc[decltype(dbi)::value]);
  });

  // Accumulator r of block db is dim 32db + 8(r/4) + 4g + (r%4) of the key;
  // keys past N fall outside the buffer and are dropped.
  const __amdgpu_buffer_rsrc_t dk_rs = make_rsrc(dk + kv_head, head_bytes);
  const __amdgpu_buffer_rsrc_t dv_rs = make_rsrc(dv + kv_head, head_bytes);
  static_for<C::DB>([&](auto dbi) {
    constexpr int db = decltype(dbi)::value;
    static_for<4>([&](auto rri) {
      constexpr int rr = decltype(rri)::value;
      const int col = db * 32 + rr * 8 + g * 4;
      if (FULL_D || col < dd) {
        const uint32_t off = (uint32_t)(my_key * dd + col) * 2u;
        u32x2 w;
        w.x = pack_bf16x2(dk_acc[db][rr * 4 + 0] * scale, dk_acc[db][rr * 4 + 1] * scale);
        w.y = pack_bf16x2(dk_acc[db][rr * 4 + 2] * scale, dk_acc[db][rr * 4 + 3] * scale);
        __builtin_amdgcn_raw_buffer_store_b64(w, dk_rs, off, 0, 0);
        w.x = pack_bf16x2(dv_acc[db][rr * 4 + 0], dv_acc[db][rr * 4 + 1]);
        w.y = pack_bf16x2(dv_acc[db][rr * 4 + 2], dv_acc[db][rr * 4 + 3]);
        __builtin_amdgcn_raw_buffer_store_b64(w, dv_rs, off, 0, 0);
      }
    });
  });
}

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kBwdThreads, 2) void attn_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
    const float* __restrict__ ws, uint16_t* __restrict__ dq,
    int B, int H_Q, int H_KV, int N, int d, int M, int mapping, int num_xcd,
    float scale_log2, float scale) {
  using C = BwdCfg<D>;
  // LDS: kDqStages x (K tile, V tile); tile j is loaded three tiles ahead
  // into stage j % kDqStages.
  constexpr int kDqStages = 4;
  constexpr int kLpt = 2 * C::SLOTS;  // LDS-direct loads per thread and tile
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * kDqStages * C::TILE_B / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);
  auto k_tile = [&](int buf) { return buf * 2 * C::TILE_B; };
  auto v_tile = [&](int buf) { return buf * 2 * C::TILE_B + C::TILE_B; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_Q, M, num_xcd, H_Q / H_KV);
  const int kvh = (int)wc.h / (H_Q / H_KV);
  const int row0 = (int)wc.m * kBwdBlock;
  const int dd = FULL_D ? D : d;
  const uint32_t head_elems = (uint32_t)N * (uint32_t)dd;
  const uint64_t q_head = ((uint64_t)wc.b * H_Q + wc.h) * head_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * head_elems;

  // v_mfma_f32_16x16x32_bf16 throughout: lane (r16, quarter q4) of a
  // 16 x 16 block.  Q and dO of the lane's rows 16 rb + r16 as B operands
  // (Q^T, dO^T): dims 32 ds + 8 q4 .. +7.
  constexpr int kDS = D / 32;  // 32-deep MFMA steps over the head dim
  const int r16 = lane & 15, q4 = lane >> 4;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t do_rs = make_rsrc(dout + q_head, head_elems * 2);
  bf16x8 qf[2][kDS], df[2][kDS];
  int rows[2];
  float lse2[2], drow[2];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    rows[rb] = row0 + wave * 32 + rb * 16 + r16;
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds) {
      const int col = ds * 32 + q4 * 8;
      const uint32_t off = (FULL_D || col < dd) ? (uint32_t)(rows[rb] * dd + col) * 2u : kOutOfRange;
      qf[rb][ds] = scale_bf16x8(
          __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, off, 0, 0)), scale_log2);
      df[rb][ds] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(do_rs, off, 0, 0));
    }
    const uint64_t ridx = ((uint64_t)wc.b * H_Q + wc.h) * 2u * N + (rows[rb] < N ? rows[rb] : N - 1);
    lse2[rb] = ws[ridx];
    drow[rb] = ws[ridx + N];
  }
  // LDS addresses: row fragment (keys 16 kb + r16, chunk 4 ds + q4) and the
  // transposing reads of K^T (output lane r16 of quarter q4: dim 16 db + r16
  // of keys 4 q4 .. +3, and 16 later).
  auto row16 = [&](int tile_byte, int kb, int ds) {
    const int r = kb * 16 + r16;
    return *reinterpret_cast<const bf16x8*>(
        lb + tile_byte + r * C::ROWB + (((4 * ds + q4) ^ C::swz(r)) * 16));
  };
  const int tk = r16 >> 2, tq = r16 & 3;  // source lane 4 tk + tq of the group
  auto tr16 = [&](int tile_byte, int db) {
    const int r = 4 * q4 + tk;
    const int chunk = 2 * db + (tq >> 1);
    const char* p0 = lb + tile_byte + r * C::ROWB + ((chunk ^ C::swz(r)) * 16) + (tq & 1) * 8;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p0 + 16 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // Padded head-dim columns are never written by the tile loads.
  if (!FULL_D) {
    for (int i = tid; i < 2 * kDqStages * C::TILE_B / 16; i += kBwdThreads)
      *reinterpret_cast<u32x4*>(lb + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  }
  const u32x4 k_desc = make_desc(k + kv_head, head_elems * 2);
  const u32x4 v_desc = make_desc(v + kv_head, head_elems * 2);
  int n_tiles = (N + kBwdTile - 1) / kBwdTile;
  if (CAUSAL) n_tiles = min(n_tiles, (row0 + kBwdBlock + kBwdTile - 1) / kBwdTile);
  // Tiles past the last write zeros (their rows are out of range), so every
  // tile issues the same loads and the waits count them uniformly.
  auto issue = [&](int j) {
    const int buf = j & (kDqStages - 1);
    bwd_load_tile<D, FULL_D>(k_desc, j * kBwdTile, N, dd, lds_base, k_tile(buf), tid);
    bwd_load_tile<D, FULL_D>(v_desc, j * kBwdTile, N, dd, lds_base, v_tile(buf), tid);
  };
  issue(0);
  issue(1);
  issue(2);
  wait_vmcnt<2 * kLpt>();
  barrier();

  typedef float f32x4 __attribute__((ext_vector_type(4)));
  constexpr int kDB16 = D / 16;  // 16-dim blocks of dQ^T
  f32x4 dq_acc[2][kDB16];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < kDB16; ++db) dq_acc[rb][db] = f32x4{};
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & (kDqStages - 1);
    issue(j + 3);  // into the stage of tile j-1, which every wave has finished
    // S^T = K Q^T and dP^T = V dO^T, 16 x 16 blocks (kb, rb): element e of
    // lane (r16, q4) is key 32 j + 16 kb + 4 q4 + e of row 16 rb + r16.
    f32x4 s[2][2], dp[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        s[kb][rb] = f32x4{lse2[rb], lse2[rb], lse2[rb], lse2[rb]};  // -lse2
        dp[kb][rb] = f32x4{drow[rb], drow[rb], drow[rb], drow[rb]};  // -D: dP - D
      }
#pragma unroll
    for (int ds = 0; ds < kDS; ++ds)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 ka = row16(k_tile(buf), kb, ds);
        const bf16x8 va = row16(v_tile(buf), kb, ds);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
          s[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[rb][ds], s[kb][rb], 0, 0, 0);
          dp[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, df[rb][ds], dp[kb][rb], 0, 0, 0);
        }
      }
    // dS^T packed as the B operand of dQ^T += K^T dS^T: for row block rb,
    // keys {4 q4 .. +3} then {16 + 4 q4 .. +3}.
    uint32_t dsk[2][4];
    auto softmax_grad = [&](auto masked) {
      constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int w = 0; w < 2; ++w) {
            float ds2[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              const int e = 2 * w + e2;
              float p = __builtin_amdgcn_exp2f(s[kb][rb][e]);
              if constexpr (MASKED) {
                const int key = j * kBwdTile + kb * 16 + q4 * 4 + e;
                const bool ok = key < N && rows[rb] < N && (!CAUSAL || key <= rows[rb]);
                p = ok ? p : 0.f;
              }
              ds2[e2] = p * dp[kb][rb][e];
            }
            dsk[rb][kb * 2 + w] = pack_bf16x2(ds2[0], ds2[1]);
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
    // dQ^T += K^T dS^T over the tile's 32 keys.
#pragma unroll
    for (int db = 0; db < kDB16; ++db) {
      const bf16x8 kt = tr16(k_tile(buf), db);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const bf16x8 b_ = __builtin_bit_cast(
            bf16x8, u32x4{dsk[rb][0], dsk[rb][1], dsk[rb][2], dsk[rb][3]});
        dq_acc[rb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kt, b_, dq_acc[rb][db], 0, 0, 0);
      }
    }
    // Tile j+1 complete (tiles j+2 and j+3 may stay in flight), then the
    // barrier that also frees tile j's stage.
    wait_vmcnt<2 * kLpt>();
    barrier();
  }
  // dQ^T accumulator element e of block (rb, db): dim 16 db + 4 q4 + e of
  // row 16 rb + r16.
  const __amdgpu_buffer_rsrc_t dq_rs = make_rsrc(dq + q_head, head_elems * 2);
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < kDB16; ++db) {
      const int col = db * 16 + q4 * 4;
      if (FULL_D || col < dd) {
        u32x2 w;
        w.x = pack_bf16x2(dq_acc[rb][db][0] * scale, dq_acc[rb][db][1] * scale);
        w.y = pack_bf16x2(dq_acc[rb][db][2] * scale, dq_acc[rb][db][3] * scale);
        __builtin_amdgcn_raw_buffer_store_b64(w, dq_rs, (uint32_t)(rows[rb] * dd + col) * 2u, 0, 0);
      }
    }
}

}  // namespace attn_numa
