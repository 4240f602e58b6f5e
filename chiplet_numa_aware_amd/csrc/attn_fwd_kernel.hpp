// FlashAttention-2 style attention forward for gfx950 (MI355X).
//
// One workgroup computes one (batch, query head, 256-row block), streaming
// every K/V tile of its KV head with an online softmax ("Optimizing Attention
// on GPUs by Exploiting GPU Architectural NUMA Effects", digest page, §3
// Figure 4 and the §4 equation).  Which block a workgroup takes comes from
// wg_map.hpp.  With split-KV the keys are cut into num_splits tile-aligned
// ranges and each workgroup covers one (row block, range), writing a partial
// result (O normalised over the range, its lse) that a merge kernel combines
// ("Fused Grouped-Query Attention" page, the decode reduction of per-shard
// partial results).
//
// Work inside a workgroup (256 threads = 4 waves of 64; one wave per SIMD,
// one workgroup per CU):
//   * wave w owns query rows [64w, 64w+64) of the block as two 32-row query
//     blocks qb; lane l owns rows 64w + 32qb + (l mod 32); lanes l and l^32
//     share those rows and split their keys.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims of K from LDS,
//     B = 16 dims x 32 queries of Q kept in registers), so a lane's 16
//     accumulators are 16 keys of ITS query row: the row max and row sum are
//     in-lane plus one exchange with lane l^32.  Every K fragment read from
//     LDS feeds both query blocks (two MFMAs).
//   * O^T = V^T P^T: P stays in the registers the score MFMA wrote (B operand,
//     16 keys x 32 queries); the V^T operand is read from V's row-major LDS
//     tile with the gfx950 transposing LDS read (ds_read_b64_tr_b16) and also
//     feeds both query blocks.
//   * K and V tiles (32 keys) go from global memory straight into LDS (buffer
//     loads with the LDS-direct bit, no staging registers), four buffers per
//     operand, so a tile's load has two key tiles of compute to land.  A tile
//     is 32 rows of D/8 16-byte chunks; chunk c of row r sits at slot
//     c ^ (r & 7).  In gfx950's 64-bank LDS that leaves the K operand reads
//     2-way and the transposing V reads 4-way bank-conflicted at D = 128; the
//     operand ring reads four fragments ahead, which hides the extra cycles
//     (a conflict-free swizzle measured no faster).
//   * software pipeline, one barrier per key tile j: the score MFMAs of tile
//     j+1 are issued with the softmax and P V of tile j; a steady tile is a
//     static sequence of MFMA "bundles" (see TileSchedule).  The steady loop
//     is unrolled over the four buffer phases, so every LDS offset is an
//     instruction immediate and the two score register sets swap roles
//     without copies: with one wave per SIMD the wave issues at most one
//     instruction per four cycles, and every instruction beyond the MFMAs
//     and the softmax competes with them for issue.
//   * online softmax in log2 units with the scale folded into one FMA; the
//     running max m is raised (and O, l rescaled) only when a tile's max
//     exceeds it by more than 2^8, so P <= 256: O / l is unchanged and bf16
//     keeps its relative precision at any scale.
//   * m, l and O live in registers for the whole key loop; O is divided by l
//     once at the end.
//
// Global memory is read and written through buffer resources that cover one
// head (at most 2^31 - 2^16 bytes): rows past the end read as zero and bf16
// stores past it are dropped, so ragged lengths need no branches; padded
// head-dim columns use an offset that is always out of range.  All 64-bit address arithmetic is
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
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kBlockN = 32;     // keys per K/V tile
constexpr int kQB = 2;          // 32-row query blocks per wave
constexpr int kWaves = kBlockM / (32 * kQB);  // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 4;      // K (and V) tiles resident in LDS (a power of 2)
constexpr uint32_t kBufDword3 = 0x00020000u;  // raw buffer, 32-bit data
constexpr uint32_t kOutOfRange = 0x80000000u; // >= any head's byte size
constexpr float kRescaleSlack = 8.0f;         // log2 of the largest P
static_assert(kWaves * kQB * 32 == kBlockM && kWaves % 2 == 0,
              "a workgroup covers BLOCK_M rows with an even number of waves");

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

// LDS-direct loads, 16 bytes per lane: lane l reads buffer `desc` at byte
// offset soff + voff (+ the instruction offset) and writes LDS at
// M0 + 16 l (+ the same instruction offset).  The whole offset is
// range-checked against the descriptor's byte count; an out-of-range lane
// writes zero.  M0 is written one instruction before its first use (the
// SALU M0 write -> LDS-DMA read distance).  Issued as inline
// assembly so that the compiler does not treat every later LDS read as
// depending on the loads (it cannot see which LDS bytes they write); the
// kernel orders them itself with s_waitcnt vmcnt before barriers.
__device__ __forceinline__ void load_lds(u32x4 desc, uint32_t voff, uint32_t soff,
                                         uint32_t m0) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(desc), "s"(soff), "s"(m0)
      : "memory", "m0");
}
// Two loads 2048 bytes apart in both memory and LDS, M0 = m0_base + LDS_OFF.
template <int LDS_OFF>
__device__ __forceinline__ void load_lds_pair(u32x4 desc, uint32_t voff, uint32_t soff,
                                              uint32_t m0_base) {
  asm volatile(
      "s_add_u32 m0, %3, %4\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen offset:2048 lds"
      :
      : "v"(voff), "s"(desc), "s"(soff), "s"(m0_base), "i"(LDS_OFF)
      : "memory", "m0");
}

// Waits until at most N vector-memory loads of this wave are outstanding
// (gfx9 s_waitcnt: vmcnt in bits [3:0] and [15:14]; expcnt and lgkmcnt left
// at their maxima, i.e. not waited for).  Loads retire in issue order.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// MFMAs are written as inline assembly so that the register file of every
// operand is fixed: scores (read by the VALU) accumulate in VGPRs, O and the
// loop-invariant Q fragments live in AGPRs.  (The builtin picks the AGPR form
// for every accumulator once a wave may use more than 256 registers, and the
// compiler then copies scores and O between the files on every tile.)
//
// The compiler does not see these as MFMAs, so the dependency distances it
// would enforce are kept here (v_mfma_f32_32x32x16_bf16 is an 8-pass XDL op):
//   * XDL write -> VALU read of the result: 11 wait states.  Scores are read
//     many bundles after their last MFMA; O is read only after xdl_guard_a.
//   * VALU write -> XDL read of an operand: 2 wait states.  P V MFMAs whose
//     P was packed in one of the two preceding bundles issue s_nop first;
//     A operands come from LDS reads (s_waitcnt) and Q passes xdl_guard_a
//     after its copy into AGPRs.
//   * XDL write -> XDL read of the same accumulator: no wait (the pipeline
//     forwards an exactly overlapping SrcC of the same opcode).
template <bool ACCUMULATE>
__device__ __forceinline__ void mfma_scores(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (ACCUMULATE)
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
template <int NOPS>
__device__ __forceinline__ void mfma_out(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  static_assert(NOPS >= 0 && NOPS <= 8, "s_nop takes 0..7");
  if constexpr (NOPS > 0)
    asm volatile("s_nop %3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                 : "+a"(acc) : "v"(a), "v"(b), "n"(NOPS - 1));
  else
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// More than 11 wait states; taking the registers as operands keeps every
// reader (and writer) of them on the far side.
template <typename T>
__device__ __forceinline__ void xdl_guard_v(T& x, T& y) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+v"(x), "+v"(y));
}
template <typename T>
__device__ __forceinline__ void xdl_guard_a(T& x) {
  asm volatile("s_nop 7\n\ts_nop 4" : "+a"(x));
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// also wait for every outstanding load).  The "memory" clobber keeps the
// compiler from moving LDS accesses across it; every LDS read a wave issued
// before it has been consumed by then.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

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

// The remap of this workgroup.  Its result is uniform by construction (a
// function of the workgroup id); reading it back from the first lane states
// that, so every address derived from it stays in scalar registers.
__device__ __forceinline__ WgCoord wg_map_uniform(int mapping, uint32_t w, uint32_t B,
                                                  uint32_t H_Q, uint32_t M, uint32_t X,
                                                  uint32_t G) {
  WgCoord c = wg_map(mapping, w, B, H_Q, M, X, G);
  c.b = __builtin_amdgcn_readfirstlane(c.b);
  c.h = __builtin_amdgcn_readfirstlane(c.h);
  c.m = __builtin_amdgcn_readfirstlane(c.m);
  return c;
}

// Pins a value to this point of the instruction stream: the empty asm is
// ordered with the schedule barriers and the loads, so work that reads `x`
// after it cannot be hoisted into an earlier bundle.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// Two floats rounded to bf16 (round to nearest even), lo in bits [15:0].
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
  static constexpr int NC = kBlockN / 16;          // 16-key chunks (PV k)
  static constexpr int CPR = D / 8;                // 16-byte chunks per row
  static constexpr int ROWB = D * 2;               // bytes per LDS row
  static constexpr int TILE_B = kBlockN * ROWB;    // bytes per K or V tile
  static constexpr int LDS_B = 2 * kStages * TILE_B;
  // 16-byte LDS-direct loads per thread per operand and tile; one wave
  // instruction fills 64 consecutive 16-byte slots (1 KiB).
  static constexpr int LOADS = kBlockN * CPR / kThreads;
  static_assert(LOADS * kThreads == kBlockN * CPR, "tile splits into waves");
};

// Static schedule of one steady key tile for one wave.
//
// The tile issues T = NS + NP MFMAs: NS = KC * kQB score MFMAs of the next
// tile (K fragment kc against query block qb, qb inner), then
// NP = NC * DB * kQB P V MFMAs of this tile (V^T fragment (c, db) against
// query block qb, qb inner).  Each LDS fragment feeds the two MFMAs of a pair
// of bundles.  Every bundle also issues the LDS read of a fragment a few
// ahead, possibly one LDS-direct tile load, and a slice of the tile's VALU
// work, a list of steps in dependency order:
//   chunk (c, qb), c-major: 8 x (fma + exp2) of P, 4 x pack to bf16,
//                           4 x two adds of the row sum
//   max of the next tile's scores: kQB * 8 x max3
// The P V MFMA of fragment (c, 0) and query block qb opens bundle
// NS + 2 c DB + qb and needs chunk (c, qb)'s packs, so the chunks are spread
// in proportion to their cost (4-cycle units; fma + exp2 counts 3) over the
// bundles before the last chunk's deadline, and the max steps, which need
// the score MFMAs, over the bundles after it.
template <int D, bool ONES = false>
struct TileSchedule {
  using C = TileCfg<D>;
  static constexpr int NS = C::KC * kQB;
  static constexpr int NP = C::NC * C::DB * kQB;
  static constexpr int T = NS + NP;
  static constexpr int FRAGS = C::KC + C::NC * C::DB;  // LDS reads per tile
  static constexpr int STEPS_PER_CHUNK = 16;
  static constexpr int CHUNKS = C::NC * kQB;
  static constexpr int EXP_STEPS = CHUNKS * STEPS_PER_CHUNK;
  static constexpr int MAX_STEPS = kQB * 8;
  static constexpr int STEPS = EXP_STEPS + MAX_STEPS;
  // Bundle whose P V MFMA first reads chunk ch = c * kQB + qb.
  static constexpr int deadline(int ch) {
    return NS + (ch / kQB) * C::DB * kQB + ch % kQB;
  }
  static constexpr int E = deadline(CHUNKS - 1);  // exp steps in [0, E)
  static constexpr int cost(int s) {
    if (s >= EXP_STEPS) return 1;
    const int k = s % STEPS_PER_CHUNK;
    return k < 8 ? 3 : (k < 12 ? 1 : (ONES ? 0 : 2));
  }
  static constexpr int cost_before(int s) {
    int c = 0;
    for (int i = 0; i < s; ++i) c += cost(i);
    return c;
  }
  static constexpr int bundle(int s) {
    const int exp_cost = cost_before(EXP_STEPS);
    if (s < EXP_STEPS) return cost_before(s) * E / exp_cost;
    const int max_cost = cost_before(STEPS) - exp_cost;
    return E + (cost_before(s) - exp_cost) * (T - E) / max_cost;
  }
  static constexpr bool valid() {
    for (int ch = 0; ch < CHUNKS; ++ch)
      if (bundle(ch * STEPS_PER_CHUNK + 11) >= deadline(ch)) return false;
    return bundle(EXP_STEPS) >= NS && bundle(STEPS - 1) < T;
  }
};

// Waves per SIMD: D = 128 needs ~484 registers per wave (O and Q of two
// query blocks in AGPRs), so one.  D = 64 fits in 256 (a few values spill
// outside the steady loop), and two waves per SIMD (two workgroups per CU)
// let one wave's softmax VALU work issue beside the other's MFMAs: the D = 64
// tile has about nine VALU issue slots per MFMA, more than one wave hides
// under its own MFMAs (measured 13-16% faster than one wave per SIMD).
template <int D>
constexpr int kWavesPerSimd = D == 64 ? 2 : 1;

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kThreads, kWavesPerSimd<D>) void attn_fwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int B, int H_U, int H_KV, int N_rows, int pos_mod,
    int N_kv, int d, int M_q, int kv_chunk, int num_splits, float* __restrict__ o_ws,
    float* __restrict__ lse_ws, int mapping, int num_xcd, float scale_log2) {
  using C = TileCfg<D>;
  // d < D: the last 16-byte chunk of every V row is padding; its first
  // element is set to 1 in LDS, so the P V MFMA accumulates the row sum of
  // the bf16 P in O^T row D - 8 (block DB - 1, element 12 of lanes 0-31).
  constexpr bool kOnes = !FULL_D;
  using TS = TileSchedule<D, kOnes>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[C::LDS_B / 4];
  char* const lds_b = reinterpret_cast<char*>(lds);
  // K buffers at [0, kStages * TILE_B), V buffers after them.
  constexpr int kVBase = kStages * C::TILE_B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int g = lane >> 5;     // lane half: which 8 of 16 MFMA k values
  const int l32 = lane & 31;   // query row within a query block / MFMA column

  // Rows are grouped in units of N_rows consecutive rows of q, o and lse: a
  // query head (H_U = H_Q, N_rows = N_q), or the G query heads of one KV group
  // (H_U = H_KV, N_rows = G N_q: the heads are contiguous in [B][H_Q][N_q][d]),
  // which fills the rows of a workgroup when N_q is small (decode).  Row r of
  // a unit is at causal position r mod pos_mod (pos_mod = N_q).
  // The remap sees M_q * num_splits row blocks per unit: m' = split * M_q +
  // row block, so the workgroups of one key range are adjacent.
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_U, M_q * num_splits, num_xcd,
                                    (uint32_t)(H_U / H_KV));
  const int kvh = (int)wc.h / (H_U / H_KV);
  const int split = (int)wc.m / M_q;
  const int row0 = ((int)wc.m - split * M_q) * kBlockM;
  // Keys of this workgroup: [kv_begin, kv_end), tile-aligned.  Causal: query
  // row r sees keys <= r + off (bottom-right aligned; off = 0 when N_q == N_kv).
  const int kv_begin = split * kv_chunk;
  const int kv_end = min(kv_begin + kv_chunk, N_kv);
  const int off = CAUSAL ? N_kv - pos_mod : 0;

  // Row length in elements: the compile-time D when d == D, so that every
  // per-lane offset below is a constant multiple and folds into immediates.
  const int dd = FULL_D ? D : d;
  const uint32_t q_elems = (uint32_t)N_rows * (uint32_t)dd;
  const uint32_t kv_elems = (uint32_t)N_kv * (uint32_t)dd;
  const uint64_t q_head = ((uint64_t)wc.b * H_U + wc.h) * q_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * kv_elems;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, q_elems * 2);
  const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(o + q_head, q_elems * 2);
  const u32x4 k_desc = make_desc(k + kv_head, kv_elems * 2);
  const u32x4 v_desc = make_desc(v + kv_head, kv_elems * 2);

  // ---- Q fragments: B operand of S^T = K Q^T; for query block qb the lane
  // holds Q[row][16kc+8g..+7] of row 64 wave + 32 qb + l32.
  const int wave_row_first = row0 + wave * 64;
  // Causal positions spanned by the valid rows (< N_rows) of rows [r0, r1]:
  // exact when the rows lie in one unit, else the whole range 0 .. pos_mod-1.
  auto pos_range = [&](int r0, int r1, int& pmin, int& pmax) {
    r1 = min(r1, N_rows - 1);
    if (r0 / pos_mod == r1 / pos_mod) {
      pmin = r0 % pos_mod;
      pmax = r1 % pos_mod;
    } else {
      pmin = 0;
      pmax = pos_mod - 1;
    }
  };
  // A wave with no valid row only loads its share of the K/V tiles.
  const bool wave_idle = wave_row_first >= N_rows;
  int wave_pmin = 0, wave_pmax = 0, wg_pmin = 0, wg_pmax = 0;
  if (!wave_idle) pos_range(wave_row_first, wave_row_first + 63, wave_pmin, wave_pmax);
  pos_range(row0, row0 + kBlockM - 1, wg_pmin, wg_pmax);
  int my_row[kQB];
  int my_last_key[kQB];  // causal: last key the row sees
  bf16x8 qf[kQB][C::KC];
  static_for<kQB>([&](auto qbi) {
    constexpr int qb = decltype(qbi)::value;
    my_row[qb] = wave_row_first + qb * 32 + l32;
    my_last_key[qb] = my_row[qb] % pos_mod + off;
    static_for<C::KC>([&](auto kci) {
      constexpr int kc = decltype(kci)::value;
      const int col = kc * 16 + g * 8;
      const uint32_t off = (FULL_D || col < dd)
                               ? (uint32_t)(my_row[qb] * dd + col) * 2u
                               : kOutOfRange;
      qf[qb][kc] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, off, 0, 0));
    });
  });
  static_for<kQB>([&](auto qbi) {
    static_for<C::KC>([&](auto kci) { xdl_guard_a(qf[decltype(qbi)::value][decltype(kci)::value]); });
  });

  // ---- LDS-direct tile loads.  A tile is 1 KiB blocks of 64 16-byte slots;
  // instruction i of wave w fills block blk(i, w) = 2 LOADS (w / 2) + (w % 2)
  // + 2 i, so a wave's blocks are 2048 bytes apart: lane l writes slot
  // P = 64 blk + l, i.e. row P / CPR, slot P % CPR, which holds the row's
  // chunk (slot ^ (row & 7)).  Chunks past the head dim get an out-of-range
  // offset and are never written (the buffers were zeroed); rows past N read
  // zero.  When d == D, 2048 bytes is also 8 or 16 whole rows in memory (the
  // swizzle depends on row & 7 only), so a wave's loads go out in pairs under
  // one M0, the second with instruction offset 2048.
  const int wave_blk0 = 2 * C::LOADS * (wave / 2) + (wave % 2);
  uint32_t ld_off[C::LOADS];
  static_for<C::LOADS>([&](auto ii) {
    constexpr int i = decltype(ii)::value;
    const int P = (wave_blk0 + 2 * i) * 64 + lane;
    const int row = P / C::CPR;
    const int chunk = (P % C::CPR) ^ (row & 7);
    ld_off[i] = (FULL_D || chunk * 8 < dd) ? (uint32_t)(row * dd + chunk * 8) * 2u
                                           : kOutOfRange;
  });
  constexpr bool kPairs = FULL_D && C::LOADS % 2 == 0;
  const uint32_t tile_bytes = (uint32_t)kBlockN * (uint32_t)dd * 2u;
  const int32_t head_bytes = (int32_t)(kv_elems * 2u);
  const int tile0 = kv_begin / kBlockN;  // first tile of the key range
  const uint32_t lds_base = (uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) char*)lds_b);
  const uint32_t m0_wave = lds_base + (uint32_t)wave_blk0 * 1024u;
  auto k_buf = [&](int tile) { return (tile & (kStages - 1)) * C::TILE_B; };
  auto v_buf = [&](int tile) { return kVBase + (tile & (kStages - 1)) * C::TILE_B; };
  // d < D: element D - 8 (the first of the padding chunk) of every row of V
  // tile `vbuf_byte` set to 1.  A tile load may rewrite the padding chunk
  // with zeros, so each tile sets it again after the barrier that made its
  // loads visible and before any read of the tile; every wave writes the 32
  // rows itself (identical values), so no other barrier is needed.
  auto ones_col = [&](int vbuf_byte) {
    if constexpr (kOnes) {
      if (lane < kBlockN) {
        const int slot = (C::CPR - 1) ^ (lane & 7);
        *reinterpret_cast<uint16_t*>(lds_b + vbuf_byte + lane * C::ROWB + slot * 16) = 0x3F80u;
      }
    }
  };
  // Byte offset of a tile, capped at the head size: a tile past the end then
  // reads nothing, and soff + kOutOfRange stays below 2^32.
  auto tile_soff = [&](int tile) {
    const uint32_t soff = (uint32_t)(tile0 + tile) * tile_bytes;
    return soff < (uint32_t)head_bytes ? soff : (uint32_t)head_bytes;
  };
  // All loads of one tile of one operand, into LDS buffer `lds_byte`.
  auto load_tile = [&](u32x4 desc, int tile, int lds_byte) {
    const uint32_t soff = tile_soff(tile);
    static_for<C::LOADS>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      load_lds(desc, ld_off[i], soff, m0_wave + lds_byte + i * 2048);
    });
  };
  auto load_k = [&](int tile) { load_tile(k_desc, tile, k_buf(tile)); };
  auto load_v = [&](int tile) { load_tile(v_desc, tile, v_buf(tile)); };

  // ---- LDS operand addresses (bytes).  K: row l32, chunk 2kc + g.
  int k_addr[C::KC];
  static_for<C::KC>([&](auto kci) {
    constexpr int kc = decltype(kci)::value;
    k_addr[kc] = l32 * C::ROWB + (((kc * 2 + g) ^ (l32 & 7)) * 16);
  });
  // V^T through ds_read_b64_tr_b16: in each 16-lane group, source lane
  // 4k + q addresses key 16c + 8h + 4g + k, dims 32db + 16 dhalf + 4q..+3,
  // and output lane j receives dim 32db + 16 dhalf + j of the 4 keys; h = 0
  // and h = 1 are two reads 8 rows apart.
  int v_addr[C::DB];
  {
    const int j = lane & 15, kk = j >> 2, qq = j & 3;
    const int dhalf = (lane >> 4) & 1;
    const int krow = 4 * g + kk;                 // key & 7 of the 4 keys
    const int w = 2 * dhalf + (qq >> 1);
    static_for<C::DB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
      v_addr[db] = krow * C::ROWB + (((4 * db + w) ^ krow) * 16) + (qq & 1) * 8;
    });
  }
  auto k_frag = [&](int buf_byte, int kc) {
    return *reinterpret_cast<const bf16x8*>(lds_b + buf_byte + k_addr[kc]);
  };
  auto v_frag = [&](int buf_byte, int c, int db) {
    const char* p = lds_b + buf_byte + v_addr[db] + c * 16 * C::ROWB;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + 8 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T = K Q^T for one tile from K buffer `buf_byte`, both query blocks.
  auto scores = [&](int buf_byte, f32x16* s) {
    static_for<C::KC>([&](auto kci) {
      constexpr int kc = decltype(kci)::value;
      const bf16x8 a = k_frag(buf_byte, kc);
      static_for<kQB>([&](auto qbi) {
        constexpr int qb = decltype(qbi)::value;
        mfma_scores<(kc > 0)>(s[qb], a, qf[qb][kc]);
      });
    });
  };

  // ---- running state, per query block
  f32x16 oacc[kQB][C::DB];
  float m_run[kQB], l_run[kQB];  // running max (log2 units, lazy), row-sum share
  // Raw score above which a tile raises m: (m + slack) / scale, so that a
  // tile's raw in-lane max is compared without scaling it.
  float m_thr[kQB];
  const float inv_scale_log2 = 1.f / scale_log2;
  static_for<kQB>([&](auto qbi) {
    constexpr int qb = decltype(qbi)::value;
    static_for<C::DB>([&](auto dbi) { oacc[qb][decltype(dbi)::value] = f32x16{}; });
    m_run[qb] = -INFINITY;
    m_thr[qb] = -INFINITY;
    l_run[qb] = 0.f;
  });

  // Raw (unscaled) max of a lane's 16 scores of a tile; the two lane halves
  // of a row are combined only when m is raised.
  auto tile_max = [&](const f32x16& s) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return mx;
  };
  // The running max m is raised only when a tile's max exceeds it by more
  // than the slack (always on a row's first tile, where m = -inf); the
  // decision is per wave.  Both loops leave the loop for a raise, call
  // raise_max and resume the same tile: a conditional update of O inside a
  // loop makes the compiler copy O out of the MFMA accumulators and back on
  // every tile.  Every s_barrier stays matched: the raise path has none.
  auto needs_raise = [&](int qb, float mx) {
    return __builtin_amdgcn_ballot_w64(mx > m_thr[qb]) != 0;
  };
  auto raise_max = [&](int qb, float mx) {
    if (!needs_raise(qb, mx)) return;
    // Both lane halves of a row take the same m (they hold the same rows).
    const float m_new = fmaxf(m_run[qb], xhalf_max(mx) * scale_log2);
    // A lane with no visible key yet keeps alpha = 1 (no -inf - -inf).
    const float alpha = (m_new == -INFINITY)
                            ? 1.f
                            : __builtin_amdgcn_exp2f(m_run[qb] - m_new);
    // O was last written by an MFMA and is next read by one: guard both
    // sides of the VALU update.
    static_for<C::DB>([&](auto dbi) { xdl_guard_a(oacc[qb][decltype(dbi)::value]); });
    static_for<C::DB>([&](auto dbi) { oacc[qb][decltype(dbi)::value] *= alpha; });
    static_for<C::DB>([&](auto dbi) { xdl_guard_a(oacc[qb][decltype(dbi)::value]); });
    l_run[qb] *= alpha;
    m_run[qb] = m_new;
    m_thr[qb] = (m_new + kRescaleSlack) * inv_scale_log2;
  };
  // Offset subtracted before exponentiating (0 while a row has seen no key).
  auto m_offset = [&](int qb) { return (m_run[qb] == -INFINITY) ? 0.f : m_run[qb]; };
  // P = exp2(S * scale - m), l += sum of P in fp32 (before rounding, so that
  // lse is the logsumexp of the scores to fp32 accuracy), P rounded to bf16
  // (kept as scalar words: a bit-cast of one element of a 4 x u32 vector to
  // bf16x2 has been miscompiled to element 0), then O^T += V^T P^T.
  auto exp_pv = [&](const f32x16* s, const float* m_use, int vbuf_byte) {
    static_for<C::NC>([&](auto ci) {
      constexpr int c = decltype(ci)::value;
      uint32_t pk[kQB][4];
      static_for<kQB>([&](auto qbi) {
        constexpr int qb = decltype(qbi)::value;
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          p[e] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s[qb][c * 8 + e], scale_log2, -m_use[qb]));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          pk[qb][w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
          if constexpr (!kOnes) l_run[qb] += p[2 * w] + p[2 * w + 1];
        }
      });
      static_for<C::DB>([&](auto dbi) {
        constexpr int db = decltype(dbi)::value;
        const bf16x8 a = v_frag(vbuf_byte, c, db);
        static_for<kQB>([&](auto qbi) {
          constexpr int qb = decltype(qbi)::value;
          mfma_out<3>(oacc[qb][db], a,
                      __builtin_bit_cast(bf16x8, u32x4{pk[qb][0], pk[qb][1], pk[qb][2], pk[qb][3]}));
        });
      });
    });
  };
  // Mask keys past N and (causal) keys after the query row; accumulator r is
  // key key0 + 8(r/4) + 4g + (r%4).
  auto mask = [&](f32x16* s, int key0) {
    static_for<kQB>([&](auto qbi) {
      constexpr int qb = decltype(qbi)::value;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + (r >> 2) * 8 + g * 4 + (r & 3);
        const bool ok = key < kv_end && (!CAUSAL || key <= my_last_key[qb]);
        s[qb][r] = ok ? s[qb][r] : -INFINITY;
      }
    });
  };

  // ---- tiles j = 0, 1, ... of the key range: keys kv_begin + 32 j ..
  // Keys some row of the workgroup sees end at span_end.
  int span_end = kv_end;
  if (CAUSAL) span_end = min(span_end, wg_pmax + 1 + off);
  const int n_tiles = span_end > kv_begin ? (span_end - kv_begin + kBlockN - 1) / kBlockN : 0;
  // Steady tiles need no mask for any row of the workgroup and have a
  // successor: keys of tile j all < kv_end and (causal) seen by the block's
  // first row.
  int n_steady = (kv_end - kv_begin) / kBlockN;
  if (CAUSAL) {
    const int x = wg_pmin + off + 1 - kv_begin;
    n_steady = min(n_steady, x > 0 ? x / kBlockN : 0);
  }
  n_steady = __builtin_amdgcn_readfirstlane(min(n_steady, n_tiles - 1));  // uniform

  // A workgroup none of whose rows sees a key of its range computes nothing:
  // its rows get O = 0 and lse = -inf.
  if (n_tiles > 0) {

  // ---- prologue: zero LDS (slots no load writes must read as zero), then
  // fill the pipeline.  Tile t's K lives in K buffer t % 4 and its V in V
  // buffer t % 4; while tile j is computed, K of tile j+4 and V of tile j+3
  // are loaded, into the buffers that tiles j and j-1 had (tiles past the
  // end read nothing).
#pragma unroll
  for (int i = 0; i < C::LDS_B / 16 / kThreads; ++i)
    *reinterpret_cast<u32x4*>(lds_b + (i * kThreads + tid) * 16) = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
  static_for<kStages>([&](auto ti) {
    constexpr int t = decltype(ti)::value;
    load_k(t);
    if constexpr (t + 1 < kStages) load_v(t);
  });
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // Scores of tile j live in sb[j & 1].
  f32x16 sb[2][kQB];
  scores(k_buf(0), sb[0]);
  xdl_guard_v(sb[0][0], sb[0][1]);
  // Tile 0's first loads (K of tile 4) go to K buffer 0, which every wave
  // has just read for these scores: no wave may issue them before all have
  // finished reading (the reads completed before the MFMAs that used them).
  // Every later buffer is reloaded only after the barrier that ends the tile
  // its last reads belonged to.
  barrier();

  if (wave_idle) {
    // No valid rows: only this wave's share of every tile load, with one
    // barrier per tile like the computing waves, and the same loads in
    // flight at each barrier (tiles past the end read nothing).
    for (int jj = 0; jj < n_tiles; ++jj) {
      load_k(jj + kStages);
      load_v(jj + kStages - 1);
      wait_vmcnt<3 * C::LOADS>();
      barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
  int j = 0;
  // Steady state: per tile, one basic block of TS::T MFMA bundles; the row
  // max of S_{j+1} is taken under the P V MFMAs.  A tile's loads must land
  // before the barrier that ends the tile after next, so each barrier lets
  // this tile's and the previous tile's loads stay in flight.
  static_assert(TS::valid(), "tile schedule breaks a data dependency");
  static_assert(kStages == 4, "the steady loop is unrolled over four phases");
  constexpr int kDist = 4;  // LDS fragment prefetch distance (fragments)
  static_assert(kDist <= C::KC, "a ring head holds K fragments only");
  float mx_cur[kQB];
  static_for<kQB>([&](auto qbi) {
    constexpr int qb = decltype(qbi)::value;
    mx_cur[qb] = tile_max(sb[0][qb]);
  });
  // Whether the max of tile j (mx_cur) requires raising m before the tile;
  // the wave-wide ballot result is pinned in scalar registers where it is
  // computed.
  auto any_raise = [&]() {
    uint64_t mask = 0;
    static_for<kQB>([&](auto qbi) {
      constexpr int qb = decltype(qbi)::value;
      mask |= __builtin_amdgcn_ballot_w64(mx_cur[qb] > m_thr[qb]);
    });
    asm volatile("" : "+s"(mask));
    return mask != 0;
  };
  bool raise_pending = any_raise();
  // Byte offsets of the next K and V tiles to load (tiles j+4 and j+3).
  uint32_t k_soff = tile_soff(kStages), v_soff = tile_soff(kStages - 1);
  // The first kDist K fragments a steady tile j needs (K of tile j+1) are
  // read before the barrier that opens it, at the end of tile j-1, so that
  // its first MFMAs do not wait for LDS reads issued after that barrier.
  // That needs K of tile j+1 to have landed one barrier earlier than the
  // V data: each barrier that ends a tile t waits for the K loads issued in
  // tile t-1 (loads go out K before V, so vmcnt leaves only V of tile t-1 and
  // tile t's loads in flight).
  bf16x8 ring_head[kDist];
  static_for<kDist>([&](auto fi) {
    constexpr int f = decltype(fi)::value;
    ring_head[f] = k_frag(k_buf(1), f);
  });

  // One steady tile in buffer phase P = j % 4.  Returns false, having done
  // nothing, at the end of the steady tiles or when the running max must be
  // raised first.
  auto steady_tile = [&](auto pc) -> bool {
    constexpr int P = decltype(pc)::value;
    if (j >= n_steady || raise_pending) return false;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    ones_col(kVBase + P * C::TILE_B);
    constexpr int kb = ((P + 1) % kStages) * C::TILE_B;    // K of tile j+1
    constexpr int vb = kVBase + P * C::TILE_B;             // V of tile j
    constexpr int kdst = P * C::TILE_B;                    // K of tile j+4
    constexpr int vdst = kVBase + ((P + kStages - 1) % kStages) * C::TILE_B;  // V of j+3
    // LDS fragment f: K fragment f (f < KC) or V^T fragment (c, db).
    auto frag = [&](int f) {
      if (f < C::KC) return k_frag(kb, f);
      const int u = f - C::KC;
      return v_frag(vb, u / C::DB, u % C::DB);
    };
    bf16x8 ring[kDist + 1];
    static_for<kDist>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      ring[f] = ring_head[f];
    });
    f32x16* const s_cur = sb[cur];
    f32x16* const sn = sb[nxt];
    float mx[kQB];
    static_for<kQB>([&](auto qbi) { mx[decltype(qbi)::value] = -INFINITY; });
    float pf[TS::CHUNKS][8];
    uint32_t pk[TS::CHUNKS][4];
    auto step = [&](auto sti) {
      constexpr int st = decltype(sti)::value;
      if constexpr (st < TS::EXP_STEPS) {
        constexpr int ch = st / TS::STEPS_PER_CHUNK, kk = st % TS::STEPS_PER_CHUNK;
        constexpr int c = ch / kQB, qb = ch % kQB;
        if constexpr (kk < 8) {
          // Pinning the whole score vector (in place, no copy) at a chunk's
          // first step keeps the chunk's exps from moving to earlier bundles.
          if constexpr (kk == 0) pin(s_cur[qb]);
          pf[ch][kk] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s_cur[qb][c * 8 + kk], scale_log2, -m_run[qb]));
        } else if constexpr (kk < 12) {
          constexpr int w = kk - 8;
          pk[ch][w] = pack_bf16x2(pf[ch][2 * w], pf[ch][2 * w + 1]);
        } else if constexpr (!kOnes) {
          constexpr int w = kk - 12;
          l_run[qb] += pf[ch][2 * w] + pf[ch][2 * w + 1];
        }
      } else {
        constexpr int i = st - TS::EXP_STEPS;
        constexpr int qb = i / 8, r = (i % 8) * 2;
        mx[qb] = fmaxf(fmaxf(mx[qb], sn[qb][r]), sn[qb][r + 1]);
      }
    };
    static_for<TS::T>([&](auto ti) {
      constexpr int t = decltype(ti)::value;
      constexpr int f = t / kQB;  // fragment of this bundle's MFMA
      if constexpr (t % kQB == 0 && f + kDist < TS::FRAGS)
        ring[(f + kDist) % (kDist + 1)] = frag(f + kDist);
      const bf16x8 a = ring[f % (kDist + 1)];
      if constexpr (t < TS::NS) {
        constexpr int kc = t / kQB, qb = t % kQB;
        mfma_scores<(kc > 0)>(sn[qb], a, qf[qb][kc]);
      } else {
        constexpr int u = (t - TS::NS) / kQB, qb = (t - TS::NS) % kQB;
        constexpr int c = u / C::DB, db = u % C::DB;
        constexpr int ch = c * kQB + qb;
        // s_nop before the MFMA if its P was packed in one of the two bundles
        // before this one.
        constexpr int pack_b = TS::bundle(ch * TS::STEPS_PER_CHUNK + 11);
        mfma_out<(pack_b >= t - 2) ? 3 : 0>(
            oacc[qb][db], a,
            __builtin_bit_cast(bf16x8, u32x4{pk[ch][0], pk[ch][1], pk[ch][2], pk[ch][3]}));
      }
      // LDS-direct loads in the first bundles, after the MFMA (the first
      // MFMA of a tile then issues right after the barrier): pairs when
      // d == D.
      if constexpr (kPairs) {
        constexpr int NPAIR = C::LOADS / 2;
        if constexpr (t < NPAIR)
          load_lds_pair<kdst + t * 4096>(k_desc, ld_off[2 * t], k_soff, m0_wave);
        else if constexpr (t < 2 * NPAIR)
          load_lds_pair<vdst + (t - NPAIR) * 4096>(v_desc, ld_off[2 * (t - NPAIR)], v_soff,
                                                   m0_wave);
      } else {
        if constexpr (t < C::LOADS)
          load_lds(k_desc, ld_off[t], k_soff, m0_wave + kdst + t * 2048);
        else if constexpr (t < 2 * C::LOADS)
          load_lds(v_desc, ld_off[t - C::LOADS], v_soff, m0_wave + vdst + (t - C::LOADS) * 2048);
      }
      // With D = 64 (about 9 VALU issue slots per MFMA) the bundle's VALU
      // slice is kept after its MFMA: left free, the compiler moves some
      // slices ahead of their MFMA, which puts two slices between one pair of
      // MFMAs and none between the next.  Measured 2% faster at D = 64 and
      // 1% slower at D = 128 (about 5 slots per MFMA), where it is left free.
      if constexpr (D == 64) __builtin_amdgcn_sched_barrier(0);
      static_for<TS::STEPS>([&](auto sti) {
        if constexpr (TS::bundle(decltype(sti)::value) == t) step(sti);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Head of the next tile's ring: K of tile j+2, whose loads (issued in
    // tile j-2) the barrier that ended tile j-1 covers.
    constexpr int kb_next = ((P + 2) % kStages) * C::TILE_B;
    static_for<kDist>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      ring_head[f] = k_frag(kb_next, f);
    });
    static_for<kQB>([&](auto qbi) {
      constexpr int qb = decltype(qbi)::value;
      mx_cur[qb] = mx[qb];
    });
    // The next tile's raise decision is taken here, before the barrier, so
    // that after it only a scalar branch precedes the next tile's MFMAs.
    raise_pending = any_raise();
    k_soff = min(k_soff + tile_bytes, (uint32_t)head_bytes);
    v_soff = min(v_soff + tile_bytes, (uint32_t)head_bytes);
    // After this barrier: V of tile j+1 (loaded during tile j-2) and K of
    // tile j+3 (loaded during tile j-1) have landed.
    wait_vmcnt<3 * C::LOADS>();
    barrier();
    ++j;
    return true;
  };
  // The running max is raised outside the steady loop: a tile whose max
  // needs it makes steady_tile return early, the max (and O, l) are updated,
  // and the loop resumes at that tile.  This keeps O in the MFMA accumulators
  // across the loop (a conditional update inside it makes the compiler copy O
  // out and back every tile).  Steady tiles have no masked keys, so once the
  // first has raised m it is finite.
  for (;;) {
    bool ok = true;
    switch (j & 3) {
      case 0:
        ok = steady_tile(std::integral_constant<int, 0>{});
        if (!ok) break;
        [[fallthrough]];
      case 1:
        ok = steady_tile(std::integral_constant<int, 1>{});
        if (!ok) break;
        [[fallthrough]];
      case 2:
        ok = steady_tile(std::integral_constant<int, 2>{});
        if (!ok) break;
        [[fallthrough]];
      default:
        ok = steady_tile(std::integral_constant<int, 3>{});
    }
    if (ok) continue;
    if (j >= n_steady) break;
    static_for<kQB>([&](auto qbi) {
      constexpr int qb = decltype(qbi)::value;
      raise_max(qb, mx_cur[qb]);
    });
    // The raised thresholds exceed these maxima (m >= max * scale, and the
    // threshold adds the slack of 2^8).
    raise_pending = false;
  }
  // Scores of tile j for the tail (a branch on the uniform j: indexing sb
  // with it would put sb in scratch memory).
  f32x16 s_cur[kQB];
  if (j & 1) {
    static_for<kQB>([&](auto qbi) { s_cur[decltype(qbi)::value] = sb[1][decltype(qbi)::value]; });
  } else {
    static_for<kQB>([&](auto qbi) { s_cur[decltype(qbi)::value] = sb[0][decltype(qbi)::value]; });
  }

  // Tail: masked tiles (ragged N, causal diagonal) and the last tile, with
  // the same buffer rotation; every barrier waits for all loads.  Masking is
  // idempotent, so a tile resumed after a raise is masked again harmlessly.
  float mx_t[kQB];
  for (;;) {
  for (; j < n_tiles; ++j) {
    const int key0 = kv_begin + j * kBlockN;
    // A wave none of whose rows sees a key of a tile has nothing to do for it.
    const bool act_cur = !wave_idle && (!CAUSAL || key0 <= wave_pmax + off);
    bool raise = false;
    if (act_cur) {
      if ((key0 + kBlockN > kv_end) ||
          (CAUSAL && key0 + kBlockN - 1 > wave_pmin + off))
        mask(s_cur, key0);
      static_for<kQB>([&](auto qbi) {
        constexpr int qb = decltype(qbi)::value;
        mx_t[qb] = tile_max(s_cur[qb]);
        raise |= needs_raise(qb, mx_t[qb]);
      });
    }
    if (raise) break;
    if (j + kStages < n_tiles) load_k(j + kStages);
    if (j + kStages - 1 < n_tiles) load_v(j + kStages - 1);
    const bool act_next = !wave_idle && j + 1 < n_tiles && (!CAUSAL || key0 + kBlockN <= wave_pmax + off);
    // act_next implies act_cur, so this tile's softmax and P V MFMAs always
    // separate these score MFMAs from the next iteration's reads of them.
    f32x16 s_next[kQB];
    if (act_next) scores(k_buf(j + 1), s_next);
    if (act_cur) {
      float m_use[kQB];
      static_for<kQB>([&](auto qbi) {
        constexpr int qb = decltype(qbi)::value;
        m_use[qb] = m_offset(qb);
      });
      ones_col(v_buf(j));
      exp_pv(s_cur, m_use, v_buf(j));
    }
    __builtin_amdgcn_s_waitcnt(0);
    barrier();
    static_for<kQB>([&](auto qbi) { s_cur[decltype(qbi)::value] = s_next[decltype(qbi)::value]; });
  }
  if (j >= n_tiles) break;
  static_for<kQB>([&](auto qbi) {
    constexpr int qb = decltype(qbi)::value;
    raise_max(qb, mx_t[qb]);
  });
  }
  }  // !wave_idle
  }  // n_tiles > 0

  // ---- epilogue: O /= l, lse = ln2 (m + log2 l); a row that saw no key
  // (l = 0) gets O = 0 and lse = -inf.  With one split O goes to o as bf16
  // and lse to lse; with several, the split's normalised O goes to o_ws as
  // fp32 [split][b][h][row][d] and its lse to lse_ws [split][b][h][row].
  static_for<kQB>([&](auto qbi) {
    static_for<C::DB>([&](auto dbi) { xdl_guard_a(oacc[decltype(qbi)::value][decltype(dbi)::value]); });
  });
  const bool partial = o_ws != nullptr;
  const uint64_t part_rows =
      (((uint64_t)split * B + wc.b) * H_U + wc.h) * (uint64_t)N_rows;  // first row of the unit
  static_for<kQB>([&](auto qbi) {
    constexpr int qb = decltype(qbi)::value;
    float l_tot;
    if constexpr (kOnes)
      l_tot = xhalf_sum(g == 0 ? oacc[qb][C::DB - 1][12] : 0.f);
    else
      l_tot = xhalf_sum(l_run[qb]);
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.f / l_tot : 0.f;
    const bool row_ok = my_row[qb] < N_rows;
    // O^T accumulator r of block db is dim 32db + 8(r/4) + 4g + (r%4).
    static_for<C::DB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int col = db * 32 + rr * 8 + g * 4;
        if (FULL_D || col < dd) {
          const float o0 = oacc[qb][db][rr * 4 + 0] * inv, o1 = oacc[qb][db][rr * 4 + 1] * inv;
          const float o2 = oacc[qb][db][rr * 4 + 2] * inv, o3 = oacc[qb][db][rr * 4 + 3] * inv;
          if (!partial) {
            u32x2 w;
            w.x = pack_bf16x2(o0, o1);
            w.y = pack_bf16x2(o2, o3);
            __builtin_amdgcn_raw_buffer_store_b64(
                w, o_rs, (uint32_t)(my_row[qb] * dd + col) * 2u, 0, 0);
          } else if (row_ok) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            *reinterpret_cast<f32x4*>(o_ws + (part_rows + my_row[qb]) * (uint64_t)d + col) =
                f32x4{o0, o1, o2, o3};
          }
        }
      }
    });
    if (g == 0 && row_ok) {
      const float ln2 = 0.6931471805599453f;
      const float lse_row = seen ? (m_run[qb] + __builtin_amdgcn_logf(l_tot)) * ln2 : -INFINITY;
      if (partial)
        lse_ws[part_rows + my_row[qb]] = lse_row;
      else if (lse != nullptr)
        lse[((uint64_t)wc.b * H_U + wc.h) * (uint64_t)N_rows + my_row[qb]] = lse_row;
    }
  });
}

}  // namespace attn_numa
