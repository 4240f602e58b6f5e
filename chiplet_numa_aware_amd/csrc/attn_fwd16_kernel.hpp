// Attention forward for head dim padded to 128 on 16 x 16 MFMA blocks
// (v_mfma_f32_16x16x32_bf16).  "Optimizing Attention on GPUs by Exploiting
// GPU Architectural NUMA Effects", digest page §3 (Figure 4) and the §4
// equation: S = Q K^T / sqrt(d), online softmax, O = P V per query row block.
//
// Same workgroup, tiling, LDS pipeline and running-max protocol as
// attn_fwd_kernel (attn_fwd_kernel.hpp), with the MFMAs as 16 x 16 blocks:
// the same bf16 FLOPs draw less power in this form than as
// v_mfma_f32_32x32x16_bf16 (measured on random operands: 2.16 against
// 1.89-1.95 GHz under the chip's power limit), which the power-capped tile
// turns into throughput.
//
// Layout.  A wave owns 64 query rows as four 16-row blocks rb; lane l is
// (r16 = l & 15, quarter q4 = l >> 4).  Per 32-key tile:
//   * S^T = K Q^T as 2 x 4 blocks (16 keys kb x 16 rows rb), k over the head
//     dim in 4 steps ds of 32: A = K fragment (keys 16 kb + r16, dims
//     32 ds + 8 q4 .. +7, one 16-byte LDS read), B = Q^T fragment (row
//     16 rb + r16, same dims, in AGPRs).  Accumulator element e is key
//     16 kb + 4 q4 + e of row 16 rb + r16, so a lane holds 8 keys of each of
//     its 4 rows.
//   * O^T += V^T P^T as 8 x 4 blocks (16 dims db x 16 rows rb) over the 32
//     keys: B = P^T of row block rb, the lane's 8 values in the order keys
//     {4 q4 .. +3, 16 + 4 q4 .. +3}; A = V^T fragment (dims 16 db + r16),
//     two transposing reads (ds_read_b64_tr_b16) 16 key rows apart that
//     deliver exactly that key order.  Accumulator element e is dim
//     16 db + 4 q4 + e of row 16 rb + r16.
// A row's maximum and sum combine the four quarters (lanes r16 + 16 q).
//
// The steady tile is one basic block of 64 MFMA "bundles": the 32 score
// MFMAs of tile j+1 (K fragment f = 4 kb + ds outer, row block inner, so
// each K fragment feeds four consecutive MFMAs), then the 32 P V MFMAs of
// tile j with the row block outer, so that the bf16 P of row block rb is
// needed only from bundle 32 + 8 rb and the exponentials spread over the
// whole tile.  The eight V^T fragments of tile j are read once (bundles
// 16-31) and kept in registers for the four row blocks.  K fragments are
// read three ahead (12 bundles before their first MFMA): at N = 128K two
// ahead measured 1-2.5% slower and four ahead 3-6% slower, and moving the
// V^T reads earlier or spacing them four bundles apart no faster.  The LDS
// keeps the row & 7 swizzle: a swizzle that makes these reads free of bank
// conflicts in gfx950's 64-bank LDS (slot c ^ (2 (r & 7) + ((r >> 3) & 1)))
// measured no faster.
#pragma once

#include "attn_fwd_kernel.hpp"

namespace attn_numa {

typedef float f32x4v __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16 with fixed register files, as mfma_scores and
// mfma_out (same hazard rules: the dependency distances are kept by the
// callers; an exactly overlapping SrcC of the same opcode needs no wait).
template <bool ACCUMULATE>
__device__ __forceinline__ void mfma16_scores(f32x4v& acc, const bf16x8& a, const bf16x8& b) {
  if constexpr (ACCUMULATE)
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "a"(b));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "a"(b));
}
template <int NOPS>
__device__ __forceinline__ void mfma16_out(f32x4v& acc, const bf16x8& a, const bf16x8& b) {
  static_assert(NOPS >= 0 && NOPS <= 8, "s_nop takes 0..7");
  if constexpr (NOPS > 0)
    asm volatile("s_nop %3\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                 : "+a"(acc) : "v"(a), "v"(b), "n"(NOPS - 1));
  else
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Max / sum over the four quarters of a row (lanes r16 + 16 q).
__device__ __forceinline__ float xquad_max(float x) {
  x = fmaxf(x, __uint_as_float(__builtin_amdgcn_ds_bpermute(
                   (int)((((threadIdx.x & 63) ^ 16) << 2)), __float_as_uint(x))));
  return xhalf_max(x);
}
__device__ __forceinline__ float xquad_sum(float x) {
  x += __uint_as_float(__builtin_amdgcn_ds_bpermute(
      (int)((((threadIdx.x & 63) ^ 16) << 2)), __float_as_uint(x)));
  return xhalf_sum(x);
}

// Static schedule of one steady tile (64 bundles, one MFMA each).  The VALU
// work is a list of steps in dependency order:
//   chunk rb: 8 x (fma + exp2) of P (element kb*4 + e), 4 x pack to bf16,
//             4 x two adds of the row sum
//   max rb of the next tile's scores: 4 x max3
// in the order chunk 0, 1, 2, max 0, 1, chunk 3, max 2, 3, spread over the
// first SPAN bundles in proportion to their cost (4-cycle units; fma + exp2
// counts 3).  valid() checks that each chunk is packed at least three
// bundles before its first P V MFMA (bundle 32 + 8 rb) and that each max
// step comes at least four bundles after the last score MFMA of its row
// block (bundle 28 + rb).
struct Tile16 {
  static constexpr int KB = 2, DS = 4, RB = 4, DB = 8;
  static constexpr int NS = KB * DS * RB;
  static constexpr int NP = DB * RB;
  static constexpr int T = NS + NP;
  static constexpr int SPAN = 60;
  static constexpr int NSTEPS = 4 * 16 + 4 * 4;
  // Segment starts: c0 0, c1 16, c2 32, m0 48, m1 52, c3 56, m2 72, m3 76.
  static constexpr bool is_max(int s) {
    return (s >= 48 && s < 56) || s >= 72;
  }
  static constexpr int rb(int s) {
    return s < 16 ? 0 : s < 32 ? 1 : s < 48 ? 2 : s < 52 ? 0 : s < 56 ? 1 : s < 72 ? 3
                                                                                  : s < 76 ? 2 : 3;
  }
  static constexpr int kk(int s) {  // step within its chunk (0..15) or max (0..3)
    return s < 48 ? s % 16 : s < 56 ? (s - 48) % 4 : s < 72 ? s - 56 : (s - 72) % 4;
  }
  static constexpr int cost(int s) {
    if (is_max(s)) return 1;
    const int k = kk(s);
    return k < 8 ? 3 : (k < 12 ? 1 : 2);
  }
  static constexpr int cost_before(int s) {
    int c = 0;
    for (int i = 0; i < s; ++i) c += cost(i);
    return c;
  }
  static constexpr int bundle(int s) { return cost_before(s) * SPAN / cost_before(NSTEPS); }
  static constexpr int deadline(int r) { return NS + 8 * r; }
  static constexpr int pack_bundle(int r) {
    for (int s = 0; s < NSTEPS; ++s)
      if (!is_max(s) && rb(s) == r && kk(s) == 11) return bundle(s);
    return -1;
  }
  static constexpr bool valid() {
    for (int s = 0; s < NSTEPS; ++s) {
      if (is_max(s) && bundle(s) < 28 + rb(s) + 4) return false;
      if (!is_max(s) && kk(s) == 11 && bundle(s) > deadline(rb(s)) - 3) return false;
    }
    return bundle(NSTEPS - 1) < T;
  }
};

template <bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(kThreads, 1) void attn_fwd_kernel_m16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o,
    float* __restrict__ lse, int B, int H_U, int H_KV, int N_rows, int pos_mod,
    int N_kv, int d, int M_q, int kv_chunk, int num_splits, float* __restrict__ o_ws,
    float* __restrict__ lse_ws, int mapping, int num_xcd, float scale_log2) {
  constexpr int D = 128;
  using C = TileCfg<D>;
  using TS = Tile16;
  constexpr int kRB = TS::RB, kKB = TS::KB, kDS = TS::DS, kDB = TS::DB;
  __shared__ __attribute__((aligned(16))) uint32_t lds[C::LDS_B / 4];
  char* const lds_b = reinterpret_cast<char*>(lds);
  // K buffers at [0, kStages * TILE_B), V buffers after them.
  constexpr int kVBase = kStages * C::TILE_B;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform
  const int r16 = lane & 15;   // row within a 16-row block / MFMA column
  const int q4 = lane >> 4;    // quarter: which 8 of 32 MFMA k values

  // Rows are grouped in units of N_rows consecutive rows of q, o and lse: a
  // query head (H_U = H_Q, N_rows = N_q), or the G query heads of one KV group
  // (H_U = H_KV, N_rows = G N_q), which fills the rows of a workgroup when
  // N_q is small.  Row r of a unit is at causal position r mod pos_mod.  The
  // remap sees M_q * num_splits row blocks per unit: m' = split * M_q + row
  // block, so the workgroups of one key range are adjacent.
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

  const int dd = FULL_D ? D : d;
  const uint32_t q_elems = (uint32_t)N_rows * (uint32_t)dd;
  const uint32_t kv_elems = (uint32_t)N_kv * (uint32_t)dd;
  const uint64_t q_head = ((uint64_t)wc.b * H_U + wc.h) * q_elems;
  const uint64_t kv_head = ((uint64_t)wc.b * H_KV + kvh) * kv_elems;
  const __amdgpu_buffer_rsrc_t q_rs = make_rsrc(q + q_head, q_elems * 2);
  const __amdgpu_buffer_rsrc_t o_rs = make_rsrc(o + q_head, q_elems * 2);
  const u32x4 k_desc = make_desc(k + kv_head, kv_elems * 2);
  const u32x4 v_desc = make_desc(v + kv_head, kv_elems * 2);

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
  // ---- Q^T fragments (B operands of S^T = K Q^T): row 16 rb + r16 of the
  // wave, dims 32 ds + 8 q4 .. +7.
  int my_row[kRB];
  int my_last_key[kRB];  // causal: last key the row sees
  bf16x8 qf[kRB][kDS];
  static_for<kRB>([&](auto rbi) {
    constexpr int rb = decltype(rbi)::value;
    my_row[rb] = wave_row_first + rb * 16 + r16;
    my_last_key[rb] = my_row[rb] % pos_mod + off;
    static_for<kDS>([&](auto dsi) {
      constexpr int ds = decltype(dsi)::value;
      const int col = ds * 32 + q4 * 8;
      const uint32_t off = (FULL_D || col < dd)
                               ? (uint32_t)(my_row[rb] * dd + col) * 2u
                               : kOutOfRange;
      qf[rb][ds] = __builtin_bit_cast(
          bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, off, 0, 0));
    });
  });
  static_for<kRB>([&](auto rbi) {
    static_for<kDS>([&](auto dsi) { xdl_guard_a(qf[decltype(rbi)::value][decltype(dsi)::value]); });
  });

  // ---- LDS-direct tile loads (as attn_fwd_kernel): chunk c of tile row r
  // sits at slot c ^ (r & 7); pairs under one M0 when d == D.
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
  auto tile_soff = [&](int tile) {
    const uint32_t soff = (uint32_t)(tile0 + tile) * tile_bytes;
    return soff < (uint32_t)head_bytes ? soff : (uint32_t)head_bytes;
  };
  auto load_tile = [&](u32x4 desc, int tile, int lds_byte) {
    const uint32_t soff = tile_soff(tile);
    static_for<C::LOADS>([&](auto ii) {
      constexpr int i = decltype(ii)::value;
      load_lds(desc, ld_off[i], soff, m0_wave + lds_byte + i * 2048);
    });
  };
  auto load_k = [&](int tile) { load_tile(k_desc, tile, k_buf(tile)); };
  auto load_v = [&](int tile) { load_tile(v_desc, tile, v_buf(tile)); };

  // ---- LDS operand addresses (bytes).  K fragment (kb, ds): row
  // 16 kb + r16, chunk 4 ds + q4 (row r + 16 has the same swizzle).
  int k_addr[kDS];
  static_for<kDS>([&](auto dsi) {
    constexpr int ds = decltype(dsi)::value;
    k_addr[ds] = r16 * C::ROWB + (((ds * 4 + q4) ^ (r16 & 7)) * 16);
  });
  // V^T through ds_read_b64_tr_b16: in each 16-lane group (quarter q4),
  // source lane 4 tk + tq addresses key row 4 q4 + tk, dims 16 db + 4 tq .. +3,
  // and output lane r16 receives dim 16 db + r16 of those 4 keys; the second
  // read takes the key rows 16 further.
  int v_addr[kDB];
  {
    const int tk = r16 >> 2, tq = r16 & 3;
    const int krow = 4 * q4 + tk;
    static_for<kDB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
      v_addr[db] = krow * C::ROWB + (((2 * db + (tq >> 1)) ^ (krow & 7)) * 16) + (tq & 1) * 8;
    });
  }
  auto k_frag = [&](int buf_byte, int f) {  // f = 4 kb + ds
    return *reinterpret_cast<const bf16x8*>(lds_b + buf_byte + (f / kDS) * 16 * C::ROWB +
                                            k_addr[f % kDS]);
  };
  auto v_frag = [&](int buf_byte, int db) {
    const char* p = lds_b + buf_byte + v_addr[db];
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(p + 16 * C::ROWB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // S^T = K Q^T for one tile from K buffer `buf_byte`, all row blocks.
  auto scores = [&](int buf_byte, f32x4v (*s)[kRB]) {
    static_for<kKB * kDS>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      constexpr int kb = f / kDS, ds = f % kDS;
      const bf16x8 a = k_frag(buf_byte, f);
      static_for<kRB>([&](auto rbi) {
        constexpr int rb = decltype(rbi)::value;
        mfma16_scores<(ds > 0)>(s[kb][rb], a, qf[rb][ds]);
      });
    });
  };

  // ---- running state, per row block
  f32x4v oacc[kRB][kDB];
  float m_run[kRB], l_run[kRB];  // running max (log2 units, lazy), row-sum share
  float m_thr[kRB];              // raw score above which a tile raises m
  const float inv_scale_log2 = 1.f / scale_log2;
  static_for<kRB>([&](auto rbi) {
    constexpr int rb = decltype(rbi)::value;
    static_for<kDB>([&](auto dbi) { oacc[rb][decltype(dbi)::value] = f32x4v{}; });
    m_run[rb] = -INFINITY;
    m_thr[rb] = -INFINITY;
    l_run[rb] = 0.f;
  });

  // Raw max of a lane's 8 scores of row block rb; the quarters of a row are
  // combined only when m is raised.
  auto tile_max = [&](f32x4v (*s)[kRB], int rb) {
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, s[kb][rb][e]);
    return mx;
  };
  // The running max m is raised only when a tile's max exceeds it by more
  // than the slack; the decision is per wave, outside the loops (see
  // attn_fwd_kernel).
  auto needs_raise = [&](int rb, float mx) {
    return __builtin_amdgcn_ballot_w64(mx > m_thr[rb]) != 0;
  };
  auto raise_max = [&](int rb, float mx) {
    if (!needs_raise(rb, mx)) return;
    const float m_new = fmaxf(m_run[rb], xquad_max(mx) * scale_log2);
    const float alpha = (m_new == -INFINITY)
                            ? 1.f
                            : __builtin_amdgcn_exp2f(m_run[rb] - m_new);
    static_for<kDB>([&](auto dbi) { xdl_guard_a(oacc[rb][decltype(dbi)::value]); });
    static_for<kDB>([&](auto dbi) { oacc[rb][decltype(dbi)::value] *= alpha; });
    static_for<kDB>([&](auto dbi) { xdl_guard_a(oacc[rb][decltype(dbi)::value]); });
    l_run[rb] *= alpha;
    m_run[rb] = m_new;
    m_thr[rb] = (m_new + kRescaleSlack) * inv_scale_log2;
  };
  auto m_offset = [&](int rb) { return (m_run[rb] == -INFINITY) ? 0.f : m_run[rb]; };
  // P of row block rb (8 values: element kb*4 + e), its row-sum share, and
  // the bf16 B operand of O^T += V^T P^T.
  auto exp_pack = [&](f32x4v (*s)[kRB], int rb, float m_use, uint32_t (&pk)[4]) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i / 4][rb][i % 4], scale_log2, -m_use));
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pk[w] = pack_bf16x2(p[2 * w], p[2 * w + 1]);
      l_run[rb] += p[2 * w] + p[2 * w + 1];
    }
  };
  auto exp_pv = [&](f32x4v (*s)[kRB], const float* m_use, int vbuf_byte) {
    uint32_t pk[kRB][4];
    static_for<kRB>([&](auto rbi) {
      constexpr int rb = decltype(rbi)::value;
      exp_pack(s, rb, m_use[rb], pk[rb]);
    });
    static_for<kDB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
      const bf16x8 a = v_frag(vbuf_byte, db);
      static_for<kRB>([&](auto rbi) {
        constexpr int rb = decltype(rbi)::value;
        mfma16_out<3>(oacc[rb][db], a,
                      __builtin_bit_cast(bf16x8, u32x4{pk[rb][0], pk[rb][1], pk[rb][2], pk[rb][3]}));
      });
    });
  };
  // Mask keys past N and (causal) keys after the query row; element e of
  // block (kb, rb) is key key0 + 16 kb + 4 q4 + e.
  auto mask = [&](f32x4v (*s)[kRB], int key0) {
    static_for<kRB>([&](auto rbi) {
      constexpr int rb = decltype(rbi)::value;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = key0 + kb * 16 + q4 * 4 + e;
          const bool ok = key < kv_end && (!CAUSAL || key <= my_last_key[rb]);
          s[kb][rb][e] = ok ? s[kb][rb][e] : -INFINITY;
        }
    });
  };

  // ---- tiles j = 0, 1, ... of the key range: keys kv_begin + 32 j ..
  int span_end = kv_end;
  if (CAUSAL) span_end = min(span_end, wg_pmax + 1 + off);
  const int n_tiles = span_end > kv_begin ? (span_end - kv_begin + kBlockN - 1) / kBlockN : 0;
  int n_steady = (kv_end - kv_begin) / kBlockN;
  if (CAUSAL) {
    const int x = wg_pmin + off + 1 - kv_begin;
    n_steady = min(n_steady, x > 0 ? x / kBlockN : 0);
  }
  n_steady = __builtin_amdgcn_readfirstlane(min(n_steady, n_tiles - 1));  // uniform

  if (n_tiles > 0) {

  // ---- prologue: zero LDS, fill the pipeline (as attn_fwd_kernel).
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
  f32x4v sb[2][kKB][kRB];
  scores(k_buf(0), sb[0]);
  static_for<kKB>([&](auto kbi) {
    xdl_guard_v(sb[0][decltype(kbi)::value][0], sb[0][decltype(kbi)::value][1]);
    xdl_guard_v(sb[0][decltype(kbi)::value][2], sb[0][decltype(kbi)::value][3]);
  });
  // Tile 0's first loads (K of tile 4) go to K buffer 0, which every wave
  // has just read for these scores.
  barrier();

  if (wave_idle) {
    for (int jj = 0; jj < n_tiles; ++jj) {
      load_k(jj + kStages);
      load_v(jj + kStages - 1);
      wait_vmcnt<3 * C::LOADS>();
      barrier();
    }
    __builtin_amdgcn_s_waitcnt(0);
  } else {
  int j = 0;
  static_assert(TS::valid(), "tile schedule breaks a data dependency");
  static_assert(kStages == 4, "the steady loop is unrolled over four phases");
  constexpr int kDist = 3;  // K fragments read ahead (12 bundles)
  float mx_cur[kRB];
  static_for<kRB>([&](auto rbi) {
    constexpr int rb = decltype(rbi)::value;
    mx_cur[rb] = tile_max(sb[0], rb);
  });
  auto any_raise = [&]() {
    uint64_t msk = 0;
    static_for<kRB>([&](auto rbi) {
      constexpr int rb = decltype(rbi)::value;
      msk |= __builtin_amdgcn_ballot_w64(mx_cur[rb] > m_thr[rb]);
    });
    asm volatile("" : "+s"(msk));
    return msk != 0;
  };
  bool raise_pending = any_raise();
  uint32_t k_soff = tile_soff(kStages), v_soff = tile_soff(kStages - 1);
  // The first kDist K fragments of a steady tile (K of tile j+1) are read
  // before the barrier that opens it (see attn_fwd_kernel).
  bf16x8 ring_head[kDist];
  static_for<kDist>([&](auto fi) {
    constexpr int f = decltype(fi)::value;
    ring_head[f] = k_frag(k_buf(1), f);
  });

  auto steady_tile = [&](auto pc) -> bool {
    constexpr int P = decltype(pc)::value;
    if (j >= n_steady || raise_pending) return false;
    constexpr int cur = P & 1, nxt = cur ^ 1;
    constexpr int kb_byte = ((P + 1) % kStages) * C::TILE_B;  // K of tile j+1
    constexpr int vb = kVBase + P * C::TILE_B;                // V of tile j
    constexpr int kdst = P * C::TILE_B;                       // K of tile j+4
    constexpr int vdst = kVBase + ((P + kStages - 1) % kStages) * C::TILE_B;  // V of j+3
    constexpr int NKF = kKB * kDS;  // K fragments per tile
    bf16x8 ring[kDist + 1];
    static_for<kDist>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      ring[f] = ring_head[f];
    });
    bf16x8 vfr[kDB];
    f32x4v (*const s_cur)[kRB] = sb[cur];
    f32x4v (*const sn)[kRB] = sb[nxt];
    float mx[kRB];
    static_for<kRB>([&](auto rbi) { mx[decltype(rbi)::value] = -INFINITY; });
    float pf[kRB][8];
    uint32_t pk[kRB][4];
    auto step = [&](auto sti) {
      constexpr int st = decltype(sti)::value;
      constexpr int rb = TS::rb(st), kk = TS::kk(st);
      if constexpr (!TS::is_max(st)) {
        if constexpr (kk < 8) {
          if constexpr (kk == 0) {
            pin(s_cur[0][rb]);
            pin(s_cur[1][rb]);
          }
          pf[rb][kk] = __builtin_amdgcn_exp2f(
              __builtin_fmaf(s_cur[kk / 4][rb][kk % 4], scale_log2, -m_run[rb]));
        } else if constexpr (kk < 12) {
          constexpr int w = kk - 8;
          pk[rb][w] = pack_bf16x2(pf[rb][2 * w], pf[rb][2 * w + 1]);
        } else {
          constexpr int w = kk - 12;
          l_run[rb] += pf[rb][2 * w] + pf[rb][2 * w + 1];
        }
      } else {
        constexpr int kb = kk / 2, e = (kk % 2) * 2;
        mx[rb] = fmaxf(fmaxf(mx[rb], sn[kb][rb][e]), sn[kb][rb][e + 1]);
      }
    };
    static_for<TS::T>([&](auto ti) {
      constexpr int t = decltype(ti)::value;
      if constexpr (t < TS::NS) {
        constexpr int f = t / kRB, rb = t % kRB;  // K fragment f = 4 kb + ds
        constexpr int kb = f / kDS, ds = f % kDS;
        if constexpr (rb == 0 && f + kDist < NKF)
          ring[(f + kDist) % (kDist + 1)] = k_frag(kb_byte, f + kDist);
        mfma16_scores<(ds > 0)>(sn[kb][rb], ring[f % (kDist + 1)], qf[rb][ds]);
        // The V^T fragments of tile j, two per K fragment from bundle 16.
        if constexpr (t >= 16 && t % 2 == 0) vfr[(t - 16) / 2] = v_frag(vb, (t - 16) / 2);
      } else {
        constexpr int u = t - TS::NS, rb = u / kDB, db = u % kDB;
        // s_nop before the MFMA if its P was packed in one of the two bundles
        // before this one.
        constexpr int pack_b = TS::pack_bundle(rb);
        mfma16_out<(pack_b >= t - 2) ? 3 : 0>(
            oacc[rb][db], vfr[db],
            __builtin_bit_cast(bf16x8, u32x4{pk[rb][0], pk[rb][1], pk[rb][2], pk[rb][3]}));
      }
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
      static_for<TS::NSTEPS>([&](auto sti) {
        if constexpr (TS::bundle(decltype(sti)::value) == t) step(sti);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    // Head of the next tile's ring: K of tile j+2 (covered by the barrier
    // that ended tile j-1).
    constexpr int kb_next = ((P + 2) % kStages) * C::TILE_B;
    static_for<kDist>([&](auto fi) {
      constexpr int f = decltype(fi)::value;
      ring_head[f] = k_frag(kb_next, f);
    });
    static_for<kRB>([&](auto rbi) {
      constexpr int rb = decltype(rbi)::value;
      mx_cur[rb] = mx[rb];
    });
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
    static_for<kRB>([&](auto rbi) {
      constexpr int rb = decltype(rbi)::value;
      raise_max(rb, mx_cur[rb]);
    });
    raise_pending = false;
  }
  // Scores of tile j for the tail (a branch on the uniform j keeps sb out of
  // scratch memory).
  f32x4v s_cur[kKB][kRB];
  if (j & 1) {
    static_for<kKB>([&](auto kbi) {
      static_for<kRB>([&](auto rbi) {
        s_cur[decltype(kbi)::value][decltype(rbi)::value] = sb[1][decltype(kbi)::value][decltype(rbi)::value];
      });
    });
  } else {
    static_for<kKB>([&](auto kbi) {
      static_for<kRB>([&](auto rbi) {
        s_cur[decltype(kbi)::value][decltype(rbi)::value] = sb[0][decltype(kbi)::value][decltype(rbi)::value];
      });
    });
  }

  // Tail: masked tiles (ragged N, causal diagonal) and the last tile, with
  // the same buffer rotation; every barrier waits for all loads.
  float mx_t[kRB];
  for (;;) {
  for (; j < n_tiles; ++j) {
    const int key0 = kv_begin + j * kBlockN;
    const bool act_cur = !wave_idle && (!CAUSAL || key0 <= wave_pmax + off);
    bool raise = false;
    if (act_cur) {
      if ((key0 + kBlockN > kv_end) ||
          (CAUSAL && key0 + kBlockN - 1 > wave_pmin + off))
        mask(s_cur, key0);
      static_for<kRB>([&](auto rbi) {
        constexpr int rb = decltype(rbi)::value;
        mx_t[rb] = tile_max(s_cur, rb);
        raise |= needs_raise(rb, mx_t[rb]);
      });
    }
    if (raise) break;
    if (j + kStages < n_tiles) load_k(j + kStages);
    if (j + kStages - 1 < n_tiles) load_v(j + kStages - 1);
    const bool act_next = !wave_idle && j + 1 < n_tiles && (!CAUSAL || key0 + kBlockN <= wave_pmax + off);
    f32x4v s_next[kKB][kRB];
    if (act_next) scores(k_buf(j + 1), s_next);
    if (act_cur) {
      float m_use[kRB];
      static_for<kRB>([&](auto rbi) {
        constexpr int rb = decltype(rbi)::value;
        m_use[rb] = m_offset(rb);
      });
      exp_pv(s_cur, m_use, v_buf(j));
    }
    __builtin_amdgcn_s_waitcnt(0);
    barrier();
    static_for<kKB>([&](auto kbi) {
      static_for<kRB>([&](auto rbi) {
        s_cur[decltype(kbi)::value][decltype(rbi)::value] = s_next[decltype(kbi)::value][decltype(rbi)::value];
      });
    });
  }
  if (j >= n_tiles) break;
  static_for<kRB>([&](auto rbi) {
    constexpr int rb = decltype(rbi)::value;
    raise_max(rb, mx_t[rb]);
  });
  }
  }  // !wave_idle
  }  // n_tiles > 0

  // ---- epilogue: O /= l, lse = ln2 (m + log2 l); a row that saw no key
  // gets O = 0 and lse = -inf.  With one split O goes to o as bf16 and lse to
  // lse; with several, the split's normalised O goes to o_ws as fp32
  // [split][b][h][row][d] and its lse to lse_ws [split][b][h][row].
  static_for<kRB>([&](auto rbi) {
    static_for<kDB>([&](auto dbi) { xdl_guard_a(oacc[decltype(rbi)::value][decltype(dbi)::value]); });
  });
  const bool partial = o_ws != nullptr;
  const uint64_t part_rows =
      (((uint64_t)split * B + wc.b) * H_U + wc.h) * (uint64_t)N_rows;  // first row of the unit
  static_for<kRB>([&](auto rbi) {
    constexpr int rb = decltype(rbi)::value;
    const float l_tot = xquad_sum(l_run[rb]);
    const bool seen = l_tot > 0.f;
    const float inv = seen ? 1.f / l_tot : 0.f;
    const bool row_ok = my_row[rb] < N_rows;
    // O^T element e of block (rb, db) is dim 16 db + 4 q4 + e.
    static_for<kDB>([&](auto dbi) {
      constexpr int db = decltype(dbi)::value;
      const int col = db * 16 + q4 * 4;
      if (FULL_D || col < dd) {
        const float o0 = oacc[rb][db][0] * inv, o1 = oacc[rb][db][1] * inv;
        const float o2 = oacc[rb][db][2] * inv, o3 = oacc[rb][db][3] * inv;
        if (!partial) {
          u32x2 w;
          w.x = pack_bf16x2(o0, o1);
          w.y = pack_bf16x2(o2, o3);
          __builtin_amdgcn_raw_buffer_store_b64(
              w, o_rs, (uint32_t)(my_row[rb] * dd + col) * 2u, 0, 0);
        } else if (row_ok) {
          *reinterpret_cast<f32x4v*>(o_ws + (part_rows + my_row[rb]) * (uint64_t)d + col) =
              f32x4v{o0, o1, o2, o3};
        }
      }
    });
    if (q4 == 0 && row_ok) {
      const float ln2 = 0.6931471805599453f;
      const float lse_row = seen ? (m_run[rb] + __builtin_amdgcn_logf(l_tot)) * ln2 : -INFINITY;
      if (partial)
        lse_ws[part_rows + my_row[rb]] = lse_row;
      else if (lse != nullptr)
        lse[((uint64_t)wc.b * H_U + wc.h) * (uint64_t)N_rows + my_row[rb]] = lse_row;
    }
  });
}

}  // namespace attn_numa
