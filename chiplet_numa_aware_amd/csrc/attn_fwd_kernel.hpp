// FlashAttention-2 style attention forward for gfx950 (MI355X).
//
// One workgroup computes one (batch, query head, 128-row block), streaming
// every K/V tile of its KV head with an online softmax ("Optimizing Attention
// on GPUs by Exploiting GPU Architectural NUMA Effects", digest page, §3
// Figure 4 and the §4 equation).  Which block a workgroup takes comes from
// wg_map.hpp.
//
// Work inside a workgroup (256 threads = 4 waves of 64):
//   * wave w owns query rows [32w, 32w+32) of the block; lane l owns query
//     row 32w + (l mod 32); lanes l and l^32 share a row and split its keys.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K from LDS,
//     B = 16 dims x 32 queries of Q kept in registers), so a lane's 16
//     accumulators of a 32x32 block are 16 keys of ITS query row: the row max
//     and row sum are in-lane plus one exchange with lane l^32.
//   * O^T = V^T P^T: P stays in the registers the score MFMA wrote (B operand,
//     16 keys x 32 queries); the V^T operand is read from V's row-major LDS
//     tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16).
//   * K and V tiles go from global memory straight into LDS (buffer loads
//     with the LDS-direct bit, no staging registers).  A tile is 64 rows of
//     D/8 16-byte chunks; chunk c of row r sits at slot c ^ (r & 7), which
//     keeps both the K operand reads and the transposing V reads free of
//     bank conflicts.
//   * software pipeline, one barrier per key tile j: the score MFMAs of tile
//     j+1 are issued before the softmax of tile j so the matrix cores work
//     while the VALU exponentiates; K runs one tile ahead of V in LDS (two K
//     and two V buffers), and each tile's loads are issued one iteration
//     before it is read.
//   * online softmax in log2 units with the scale folded into one FMA; the
//     running max m is raised (and O, l rescaled) only when a tile's max
//     exceeds it by more than 2^8, so P <= 256: O / l is unchanged and bf16
//     keeps its relative precision at any scale.
//   * m, l and O live in registers for the whole key loop; O is divided by l
//     once at the end.
//
// Global memory is read and written through buffer resources that cover one
// head (at most 2^31 bytes): rows past N read as zero and stores past N are
// dropped, so ragged N needs no branches; padded head-dim columns use an
// offset that is always out of range.  All 64-bit address arithmetic is
// scalar.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "wg_map.hpp"

namespace attn_numa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlockN = 64;     // keys per K/V tile
constexpr int kThreads = 256;   // 4 waves
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data
constexpr uint32_t kOutOfRange = 0x80000000u; // >= any head's byte size
constexpr float kRescaleSlack = 8.0f;         // log2 of the largest P

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                          uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0,
                                           (int)bytes, (int)kBufDword3);
}

// Raw buffer descriptor (four SGPRs) for LDS-direct loads written as inline
// assembly: base address, stride 0, size in bytes, 32-bit data format.
__device__ __forceinline__ u32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, bytes, kBufDword3};
}

// 16 bytes per lane from buffer `desc` at byte offset `voff` into LDS at
// lds_byte + 16 * lane (out-of-range lanes write nothing).  Issued as inline
// assembly so that the compiler does not treat every later LDS read as
// depending on it; the caller waits (s_waitcnt vmcnt) before a barrier.
__device__ __forceinline__ void load_lds_b128(u32x4 desc, uint32_t voff,
                                              uint32_t lds_byte) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_byte), "v"(voff), "s"(desc)
      : "memory", "m0");
}

// f(std::integral_constant<int, i>{}) for i = 0..N-1, expanded at compile
// time (no reliance on loop unrolling), so every index inside is a constant.
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
  (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Pins a value's computation to this point of the instruction stream: the
// empty asm is ordered with the schedule barriers and the loads, so work that
// reads or writes `x` here cannot be hoisted or sunk into another bundle.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// lo16(a) | lo16(b) << 16 and hi16(a) | hi16(b) << 16.
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
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int ROWB = D * 2;               // bytes per LDS row
  static constexpr int TILE_B = kBlockN * ROWB;    // bytes per K or V tile
  static constexpr int LDS_B = 4 * TILE_B;         // 2 K + 2 V buffers
  // 16-byte LDS-direct loads per thread per operand and tile; one wave
  // instruction fills 64 consecutive 16-byte slots (1 KiB).
  static constexpr int LOADS = kBlockN * CPR / kThreads;
};

// Static schedule of one steady key tile for one wave.
//
// The tile issues T = NS + NP MFMAs (NS score MFMAs of the next tile, then NP
// P V MFMAs of this tile).  Each MFMA is a "bundle": it also issues the LDS
// read of the MFMA operand kDist bundles ahead and a slice of the tile's VALU
// work, so the VALU runs in the MFMA shadow and LDS latency is covered.  The
// VALU work is a list of steps, in dependency order:
//   chunk c = 0..NC-1: 8 x (fma + exp2) of P, 4 x pack to bf16, 4 x two adds
//                      of the row sum  (the packs precede chunk c's P V MFMAs)
//   max of the next tile's scores: NB*8 x max3  (after its score MFMAs)
// and is spread over the bundles in proportion to its cost (4-cycle units;
// fma + exp2 counts 3).
template <int D>
struct TileSchedule {
  using C = TileCfg<D>;
  static constexpr int NS = C::NB * C::KC;
  static constexpr int NP = C::NC * C::DB;
  static constexpr int T = NS + NP;
  static constexpr int STEPS_PER_CHUNK = 16;
  static constexpr int EXP_STEPS = C::NC * STEPS_PER_CHUNK;
  static constexpr int MAX_STEPS = C::NB * 8;
  static constexpr int STEPS = EXP_STEPS + MAX_STEPS;
  static constexpr int cost(int s) {
    if (s >= EXP_STEPS) return 1;
    const int k = s % STEPS_PER_CHUNK;
    return k < 8 ? 3 : (k < 12 ? 1 : 2);
  }
  static constexpr int total_cost() {
    int c = 0;
    for (int s = 0; s < STEPS; ++s) c += cost(s);
    return c;
  }
  // Bundle that runs step s: the one whose share of the total cost contains
  // the step's starting cost.
  static constexpr int bundle(int s) {
    int c = 0;
    for (int i = 0; i < s; ++i) c += cost(i);
    return c * T / total_cost();
  }
  // Score MFMAs of the next tile finish within the first NS bundles; the max
  // steps must come after them, and the bf16 packs of chunk c (its steps
  // 8..11) before P V MFMA NS + c*DB, which opens bundle NS + c*DB.
  static constexpr bool valid() {
    for (int ch = 0; ch < C::NC; ++ch)
      if (bundle(ch * STEPS_PER_CHUNK + 11) >= NS + ch * C::DB) return false;
    return bundle(EXP_STEPS) >= NS;
  }
};

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int B, int H_Q, int H_KV, int N, int d, int M,
    int mapping, int num_xcd, float scale_log2) {
  using C = TileCfg<D>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[C::LDS_B / 4];
  char* const lds_b = reinterpret_cast<char*>(lds);
  // K buffers at [0, 2*TILE_B), V buffers at [2*TILE_B, 4*TILE_B).
  constexpr int kVBase = 2 * C::TILE_B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int g = lane >> 5;     // lane half: which 8 of 16 MFMA k values
  const int l32 = lane & 31;   // query row within the wave / MFMA column

  const WgCoord wc = wg_map(mapping, blockIdx.x, B, H_Q, M, num_xcd);
  const int kvh = (int)wc.h / (H_Q / H_KV);
  const int row0 = (int)wc.m * kBlockM;

  // Row length in elements: the compile-time D when d == D, so that every
  // per-lane offset below is a constant multiple and folds into immediates.
  const int dd = FULL_D ? D : d;
  const uint32_t head_elems = (uint32_t)N * (uint32_t)dd;
  const uint64_t q_head = ((uint64_t)wc.b * H_Q + wc.h) * head_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * head_elems;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, head_elems * 2);
  const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(o + q_head, head_elems * 2);
  const u32x4 k_desc = make_desc(k + kv_head, head_elems * 2);
  const u32x4 v_desc = make_desc(v + kv_head, head_elems * 2);

  // ---- Q fragments: B operand of S^T = K Q^T, lane holds Q[row][16kc+8g..+7].
  const int my_row = row0 + wave * 32 + l32;
  bf16x8 qf[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    const int col = kc * 16 + g * 8;
    const uint32_t off = (FULL_D || col < dd)
                             ? (uint32_t)(my_row * dd + col) * 2u
                             : kOutOfRange;
    qf[kc] = __builtin_bit_cast(
        bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, off, 0, 0));
  }

  // ---- LDS-direct tile loads.  Wave instruction i of wave w fills the 1 KiB
  // block i*4 + w of the tile: lane l writes slot P = 64*(i*4+w) + l, i.e.
  // row P / CPR, slot P % CPR, which holds the row's chunk (slot ^ (row & 7)).
  // Chunks past the head dim get an out-of-range offset and are never
  // written (the buffer was zeroed); rows past N read zero.
  uint32_t ld_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int P = (i * 4 + wave) * 64 + lane;
    const int row = P / C::CPR;
    const int chunk = (P % C::CPR) ^ (row & 7);
    ld_off[i] = (FULL_D || chunk * 8 < dd) ? (uint32_t)(row * dd + chunk * 8) * 2u
                                           : kOutOfRange;
  }
  const uint32_t tile_bytes = (uint32_t)kBlockN * (uint32_t)dd * 2u;
  // An out-of-range offset stays out of range after adding a tile base (both
  // are below 2^31).
  const uint32_t lds_base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) char*)lds_b);
  auto load_one = [&](u32x4 desc, int tile, int lds_byte, int i) {
    load_lds_b128(desc, ld_off[i] + (uint32_t)tile * tile_bytes,
                  lds_base + lds_byte + (i * 4 + wave) * 1024);
  };
  auto load_tile = [&](u32x4 desc, int tile, int lds_byte) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) load_one(desc, tile, lds_byte, i);
  };
  auto load_k = [&](int tile, int buf) { load_tile(k_desc, tile, buf * C::TILE_B); };
  auto load_v = [&](int tile, int buf) { load_tile(v_desc, tile, kVBase + buf * C::TILE_B); };
  // All of this wave's LDS-direct loads have landed (then a barrier makes
  // every wave's visible).
  auto wait_loads = [&]() { __builtin_amdgcn_s_waitcnt(0); };

  // ---- LDS operand addresses (bytes).  K: row nb*32 + l32, chunk 2kc + g.
  int k_addr[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
    k_addr[kc] = l32 * C::ROWB + (((kc * 2 + g) ^ (l32 & 7)) * 16);
  // V^T through ds_read_b64_tr_b16: in each 16-lane group, source lane
  // 4k + q addresses key 16c + 8h + 4g + k, dims 32db + 16*dhalf + 4q..+3,
  // and output lane j receives dim 32db + 16*dhalf + j of the 4 keys.
  int v_addr[C::DB];
  {
    const int j = lane & 15, kk = j >> 2, qq = j & 3;
    const int dhalf = (lane >> 4) & 1;
    const int krow = 4 * g + kk;                 // key & 7 of the 4 keys
    const int w = 2 * dhalf + (qq >> 1);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      v_addr[db] = kVBase + krow * C::ROWB + (((4 * db + w) ^ krow) * 16) + (qq & 1) * 8;
  }
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  auto k_operand = [&](int buf, int nb, int kc) {
    return *reinterpret_cast<const bf16x8*>(lds_b + buf * C::TILE_B + k_addr[kc] +
                                            nb * 32 * C::ROWB);
  };
  auto v_operand = [&](int buf, int c, int db) {
    const char* p = lds_b + buf * C::TILE_B + v_addr[db] + c * 16 * C::ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + 8 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T = K Q^T for one tile from K buffer `buf`: s[nb] = keys 32nb..32nb+31.
  auto scores = [&](int buf, f32x16* s) {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
      f32x16 acc = {};
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_operand(buf, nb, kc),
                                                      qf[kc], acc, 0, 0, 0);
      s[nb] = acc;
    }
  };

  // ---- running state
  f32x16 oacc[C::DB];
#pragma unroll
  for (int i = 0; i < C::DB; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;  // running max of scaled scores, log2 units (lazy)
  float l_run = 0.f;        // this lane's share of the running row sum

  // Scaled row max of a tile of scores (log2 units), both lane halves.
  auto tile_max = [&](const f32x16* s) {
    float mx = -INFINITY;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[nb][r]);
    return xhalf_max(mx) * scale_log2;
  };

  // Raise m only when a tile's max exceeds it by more than the slack (always
  // on the first tile, where m = -inf); the decision is per wave.  Returns the
  // offset to subtract before exponentiating.
  auto update_max = [&](float mx) {
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      // A lane with no visible key yet keeps alpha = 1 (no -inf - -inf).
      const float alpha =
          (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int i = 0; i < C::DB; ++i) oacc[i] *= alpha;
      l_run *= alpha;
      m_run = m_new;
    }
    return (m_run == -INFINITY) ? 0.f : m_run;
  };

  // P = exp2(S * scale - m), l += sum of P in fp32 (before rounding, so that
  // lse is the logsumexp of the scores to fp32 accuracy), P rounded to bf16,
  // and O^T += V^T P^T from V buffer `buf`, one 16-key chunk at a time.
  auto exp_pv = [&](const f32x16* s, float m_use, int buf) {
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      const int nb = c >> 1, r0 = (c & 1) * 8;
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[nb][r0 + e], scale_log2, -m_use));
      // The packed words stay scalars until the MFMA operand is formed: a
      // bit-cast of one element of a 4 x u32 vector to bf16x2 has been
      // miscompiled (to element 0) by this compiler.
      uint32_t pk[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pk[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
        l_run += p[2 * w] + p[2 * w + 1];
      }
      const bf16x8 pb = __builtin_bit_cast(bf16x8, u32x4{pk[0], pk[1], pk[2], pk[3]});
#pragma unroll
      for (int db = 0; db < C::DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand(buf, c, db),
                                                           pb, oacc[db], 0, 0, 0);
    }
  };

  // Mask keys past N and (causal) keys after the query row; accumulator r of
  // block nb is key key0 + 32nb + 8(r/4) + 4g + (r%4).
  auto mask = [&](f32x16* s, int key0) {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + nb * 32 + (r >> 2) * 8 + g * 4 + (r & 3);
        const bool ok = key < N && (!CAUSAL || key <= my_row);
        s[nb][r] = ok ? s[nb][r] : -INFINITY;
      }
  };

  // ---- tiles
  const int n_tiles_all = (N + kBlockN - 1) / kBlockN;
  int n_tiles = n_tiles_all;
  if (CAUSAL) {
    const int last = (row0 + kBlockM + kBlockN - 1) / kBlockN;
    n_tiles = last < n_tiles_all ? last : n_tiles_all;
  }
  // Steady tiles need no mask for any row of the workgroup and have a
  // successor: keys of tile j all < N and (causal) <= the block's first row.
  int n_steady = N / kBlockN;
  if (CAUSAL) {
    const int full = (row0 + 1) / kBlockN;
    n_steady = full < n_steady ? full : n_steady;
  }
  if (n_steady > n_tiles - 1) n_steady = n_tiles - 1;
  const int wave_row_first = row0 + wave * 32;
  const int wave_row_last = wave_row_first + 31;

  // ---- prologue: zero LDS (slots no load writes must read as zero), then
  // K0, V0 -> buffers 0, K1 -> K buffer 1; S_0.
#pragma unroll
  for (int i = 0; i < C::LDS_B / 16 / kThreads; ++i)
    *reinterpret_cast<u32x4*>(lds_b + (i * kThreads + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  load_k(0, 0);
  load_v(0, 0);
  if (n_tiles > 1) load_k(1, 1);
  wait_loads();
  __syncthreads();
  f32x16 s_cur[C::NB], s_next[C::NB];
  scores(0, s_cur);
  __syncthreads();

  int j = 0;
  // Steady state: one basic block per tile after the (rare) rescale branch.
  // Tile j+2's K (clamped to the last tile: a re-load that is never read) and
  // tile j+1's V are fetched while S_{j+1} = K Q^T and the softmax and P V of
  // tile j run; the row max of S_{j+1} is taken under the P V MFMAs.  The
  // schedule interleaves each MFMA with the VALU work of the other stage.
  float mx_cur = tile_max(s_cur);  // used only while tiles are steady
  using TS = TileSchedule<D>;
  static_assert(TS::valid(), "tile schedule breaks a data dependency");
  constexpr int kDist = 4;  // LDS operand prefetch distance, in MFMAs
  for (; j < n_steady; ++j) {
    const float m_use = update_max(mx_cur);
    // LDS operand of MFMA t: a K fragment (score MFMAs) or a V^T fragment.
    auto operand = [&](int t) {
      if (t < TS::NS) return k_operand((j + 1) & 1, t / C::KC, t % C::KC);
      const int u = t - TS::NS;
      return v_operand(j & 1, u / C::DB, u % C::DB);
    };
    // K of tile j+2 (clamped to the last tile: a re-load that is never read)
    // and V of tile j+1 go to the buffers this iteration does not read; the
    // 2*LOADS load instructions are spread over the first bundles, one each,
    // so that the texture units drain between them instead of stalling this
    // wave's issue.
    const int tk = (j + 2 < n_tiles) ? j + 2 : n_tiles - 1;
    bf16x8 ring[kDist + 1];
    static_for<kDist>([&](auto ti) {
      constexpr int t = decltype(ti)::value;
      ring[t] = operand(t);
    });
    f32x16 sn[C::NB];
    static_for<C::NB>([&](auto nbi) { sn[decltype(nbi)::value] = f32x16{}; });
    float pf[C::NC][8];
    uint32_t pk[C::NC][4];
    float mx = -INFINITY;
    auto step = [&](auto sti) {
      constexpr int st = decltype(sti)::value;
      if constexpr (st < TS::EXP_STEPS) {
        constexpr int c = st / TS::STEPS_PER_CHUNK, k = st % TS::STEPS_PER_CHUNK;
        constexpr int nb = c >> 1, r0 = (c & 1) * 8;
        if constexpr (k < 8) {
          float x = s_cur[nb][r0 + k];
          pin(x);
          pf[c][k] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, scale_log2, -m_use));
        } else if constexpr (k < 12) {
          constexpr int w = k - 8;
          pk[c][w] = pack_bf16x2(pf[c][2 * w], pf[c][2 * w + 1]);
        } else {
          constexpr int w = k - 12;
          l_run += pf[c][2 * w] + pf[c][2 * w + 1];
        }
      } else {
        constexpr int i = st - TS::EXP_STEPS;
        constexpr int nb = i / 8, r = (i % 8) * 2;
        mx = fmaxf(fmaxf(mx, sn[nb][r]), sn[nb][r + 1]);
      }
    };
    static_for<TS::T>([&](auto ti) {
      constexpr int t = decltype(ti)::value;
      if constexpr (t < C::LOADS)
        load_one(k_desc, tk, (j & 1) * C::TILE_B, t);
      else if constexpr (t < 2 * C::LOADS)
        load_one(v_desc, j + 1, kVBase + ((j + 1) & 1) * C::TILE_B, t - C::LOADS);
      if constexpr (t + kDist < TS::T) ring[(t + kDist) % (kDist + 1)] = operand(t + kDist);
      const bf16x8 a = ring[t % (kDist + 1)];
      if constexpr (t < TS::NS) {
        constexpr int nb = t / C::KC, kc = t % C::KC;
        sn[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], sn[nb], 0, 0, 0);
      } else {
        constexpr int u = t - TS::NS, c = u / C::DB, db = u % C::DB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, __builtin_bit_cast(bf16x8, u32x4{pk[c][0], pk[c][1], pk[c][2], pk[c][3]}),
            oacc[db], 0, 0, 0);
      }
      static_for<TS::STEPS>([&](auto sti) {
        if constexpr (TS::bundle(decltype(sti)::value) == t) step(sti);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    mx_cur = xhalf_max(mx) * scale_log2;
    wait_loads();
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) s_cur[nb] = sn[nb];
  }
  // Tail: masked tiles (ragged N, causal diagonal) and the last tile.
  for (; j < n_tiles; ++j) {
    const bool has1 = j + 1 < n_tiles;
    const bool has2 = j + 2 < n_tiles;
    if (has2) load_k(j + 2, j & 1);
    if (has1) load_v(j + 1, (j + 1) & 1);
    const int key0 = j * kBlockN;
    // A wave whose last row precedes a tile has nothing to do for it.
    const bool act_next = has1 && (!CAUSAL || key0 + kBlockN <= wave_row_last);
    const bool act_cur = !CAUSAL || key0 <= wave_row_last;
    if (act_next) scores((j + 1) & 1, s_next);
    if (act_cur) {
      if ((key0 + kBlockN > N) ||
          (CAUSAL && key0 + kBlockN - 1 > wave_row_first))
        mask(s_cur, key0);
      const float m_use = update_max(tile_max(s_cur));
      exp_pv(s_cur, m_use, j & 1);
    }
    wait_loads();
    __syncthreads();
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) s_cur[nb] = s_next[nb];
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
      if (FULL_D || col < dd) {
        u32x2 w;
        w.x = pack_bf16x2(oacc[db][rr * 4 + 0] * inv, oacc[db][rr * 4 + 1] * inv);
        w.y = pack_bf16x2(oacc[db][rr * 4 + 2] * inv, oacc[db][rr * 4 + 3] * inv);
        __builtin_amdgcn_raw_buffer_store_b64(
            w, o_rs, (uint32_t)(my_row * dd + col) * 2u, 0, 0);
      }
    }
  if (lse != nullptr && g == 0 && my_row < N) {
    const float ln2 = 0.6931471805599453f;
    lse[((uint64_t)wc.b * H_Q + wc.h) * (uint64_t)N + my_row] =
        (m_run + __builtin_amdgcn_logf(l_tot)) * ln2;
  }
}

}  // namespace attn_numa
