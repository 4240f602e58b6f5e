// Attention forward for units of few query rows (decode): one wave per
// workgroup, one 32-row query block of a unit over one key range.
//
// Same result and conventions as attn_fwd_kernel ("Optimizing Attention on
// GPUs by Exploiting GPU Architectural NUMA Effects", digest page §4
// equation; the split-KV partial results of the "Fused Grouped-Query
// Attention" page's decode reduction): units of N_rows rows (a query head, or
// the G heads of a KV group packed), bottom-right causal mask with row r at
// position r mod pos_mod, key range [split * kv_chunk, ...), normalised O and
// lse per split into the fp32 workspace, or bf16 O and lse directly with one
// split.  The remap is the same wg_map over (unit, split * M_q + row block).
//
// Why a separate kernel: attn_fwd_kernel spends a 64-row MFMA tile per wave
// and key tile, and for a unit of 1-8 rows only one wave of its workgroup
// has rows, so decode time is set by work on empty rows.  Here a workgroup
// is a single wave computing 32 rows (half the MFMAs per tile), the K/V
// buffers are small (32 KiB), and several workgroups share a CU, so the key
// stream, not the MFMAs, sets the pace.
//
// Per key tile (32 keys): S^T = K Q^T (v_mfma_f32_32x32x16_bf16, K from LDS,
// Q in registers; lane (row l32, half g) holds 16 keys of its row), masking,
// an online softmax in log2 units (O and l rescaled when the row max rises),
// P rounded to bf16, O^T += V^T P^T with V^T from transposing LDS reads.
// K/V tiles go global -> LDS directly (LDS-direct buffer loads), STAGES
// buffers per operand; chunk c of row r at slot c ^ (r & 7).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_fwd_kernel.hpp"
#include "wg_map.hpp"

namespace attn_numa {

constexpr int kDecRows = 32;  // query rows per decode workgroup (one wave)

template <int D>
struct DecCfg {
  static constexpr int KC = D / 16, DB = D / 32, CPR = D / 8, ROWB = D * 2;
  static constexpr int TILE_B = kBlockN * ROWB;
  static constexpr int STAGES = D == 64 ? 4 : 2;       // 32 KiB of K/V buffers
  static constexpr int LDS_B = 2 * STAGES * TILE_B;
  static constexpr int LOADS = kBlockN * CPR / 64;     // 16-byte loads per lane per tile
};

template <int D, bool CAUSAL, bool FULL_D>
__global__ __launch_bounds__(64, 2) void attn_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ o, float* __restrict__ lse,
    int B, int H_U, int H_KV, int N_rows, int pos_mod, int N_kv, int d, int M_q,
    int kv_chunk, int num_splits, float* __restrict__ o_ws, float* __restrict__ lse_ws,
    int mapping, int num_xcd, float scale_log2) {
  using C = DecCfg<D>;
  __shared__ __attribute__((aligned(16))) uint32_t lds[C::LDS_B / 4];
  char* const lb = reinterpret_cast<char*>(lds);
  constexpr int kVBase = C::STAGES * C::TILE_B;
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lb);

  const int lane = threadIdx.x;
  const int g = lane >> 5, l32 = lane & 31;
  const WgCoord wc = wg_map_uniform(mapping, blockIdx.x, B, H_U, M_q * num_splits, num_xcd,
                            (uint32_t)(H_U / H_KV));
  const int kvh = (int)wc.h / (H_U / H_KV);
  const int split = (int)wc.m / M_q;
  const int row0 = ((int)wc.m - split * M_q) * kDecRows;
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

  // Q of this lane's row, B operand of S^T = K Q^T: dims 16kc + 8g .. +7.
  const int my_row = row0 + l32;
  const int my_last_key = CAUSAL ? (my_row < N_rows ? my_row % pos_mod : 0) + off : kv_end - 1;
  bf16x8 qf[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    const int col = kc * 16 + g * 8;
    const uint32_t qo = (FULL_D || col < dd) ? (uint32_t)(my_row * dd + col) * 2u : kOutOfRange;
    qf[kc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(q_rs, qo, 0, 0));
  }

  // Keys this block sees: [kv_begin, min(kv_end, last key of its last valid
  // row + 1)); under a causal mask later keys are masked for every row.
  int key_end = kv_end;
  if (CAUSAL) {
    const int last = min(row0 + kDecRows, N_rows) - 1;
    int pmax;
    if (row0 / pos_mod == last / pos_mod) pmax = last % pos_mod;
    else pmax = pos_mod - 1;
    key_end = min(kv_end, pmax + off + 1);
  }
  const int n_tiles = key_end > kv_begin ? (key_end - kv_begin + kBlockN - 1) / kBlockN : 0;

  // Tile loads: instruction i of the wave fills slots 64 i .. 64 i + 63 of a
  // tile (row P / CPR, slot P % CPR holding chunk (P % CPR) ^ (row & 7)).
  uint32_t ld_off[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int P = 64 * i + lane;
    const int row = P / C::CPR;
    const int chunk = (P % C::CPR) ^ (row & 7);
    ld_off[i] = (FULL_D || chunk * 8 < dd) ? (uint32_t)(row * dd + chunk * 8) * 2u : kOutOfRange;
  }
  const uint32_t tile_bytes = (uint32_t)kBlockN * (uint32_t)dd * 2u;
  const uint32_t head_bytes = kv_elems * 2u;
  auto load_tile = [&](int t) {
    const int st = t % C::STAGES;
    const uint32_t so = (uint32_t)(kv_begin / kBlockN + t) * tile_bytes;
    const uint32_t soff = so < head_bytes ? so : head_bytes;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      load_lds(k_desc, ld_off[i], soff, lds_base + st * C::TILE_B + i * 1024);
      load_lds(v_desc, ld_off[i], soff, lds_base + kVBase + st * C::TILE_B + i * 1024);
    }
  };

  // Operand addresses (as attn_fwd_kernel): K row l32, chunk 2kc + g; V^T by
  // transposing reads.
  int k_addr[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) k_addr[kc] = l32 * C::ROWB + (((kc * 2 + g) ^ (l32 & 7)) * 16);
  int v_addr[C::DB];
  {
    const int j = lane & 15, kk = j >> 2, qq = j & 3, dhalf = (lane >> 4) & 1;
    const int krow = 4 * g + kk, w = 2 * dhalf + (qq >> 1);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
      v_addr[db] = krow * C::ROWB + (((4 * db + w) ^ krow) * 16) + (qq & 1) * 8;
  }

  // Padded head-dim columns are never written by the loads.
  if (!FULL_D) {
    for (int i = lane; i < C::LDS_B / 16; i += 64)
      *reinterpret_cast<u32x4*>(lb + i * 16) = u32x4{0u, 0u, 0u, 0u};
    __builtin_amdgcn_s_waitcnt(0);
  }

  f32x16 oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < C::STAGES - 1 && t < n_tiles; ++t) load_tile(t);
  for (int t = 0; t < n_tiles; ++t) {
    // Tile t has landed when only the loads of the later tiles already issued
    // are outstanding (loads retire in order; 2 LOADS per tile).
    const int later = min(n_tiles - 1 - t, C::STAGES - 2);
    if (later >= 2) wait_vmcnt<4 * C::LOADS>();
    else if (later == 1) wait_vmcnt<2 * C::LOADS>();
    else wait_vmcnt<0>();
    // The buffer loaded next was last read in tile t-1.
    if (t + C::STAGES - 1 < n_tiles) load_tile(t + C::STAGES - 1);
    const int st = t % C::STAGES;
    const char* kb = lb + st * C::TILE_B;
    const char* vb = lb + kVBase + st * C::TILE_B;
    const int key0 = kv_begin + t * kBlockN;

    f32x16 s = f32x16{};
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(kb + k_addr[kc]), qf[kc], s, 0, 0, 0);
    // Accumulator r is key key0 + 8(r/4) + 4g + (r%4) of this lane's row.
    float mx = -INFINITY;
    const bool need_mask = key0 + kBlockN > kv_end || (CAUSAL && key0 + kBlockN - 1 > my_last_key);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = key0 + 8 * (r >> 2) + 4 * g + (r & 3);
      if (need_mask && (key >= kv_end || (CAUSAL && key > my_last_key))) s[r] = -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    const float m_new = fmaxf(m_run, xhalf_max(mx) * scale_log2);
    // A row with no visible key yet keeps m = -inf; P is then 0, not NaN.
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * c + e], scale_log2, -m_use));
        l_run += p[e];
      }
      const bf16x8 pb = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                        pack_bf16x2(p[6], p[7])});
#pragma unroll
      for (int db = 0; db < C::DB; ++db) {
        const char* pv = vb + v_addr[db] + c * 16 * C::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(pv));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(pv + 8 * C::ROWB));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
      }
    }
  }

  // Epilogue (as attn_fwd_kernel): O /= l, lse = ln2 (m + log2 l); a row that
  // saw no key gets O = 0 and lse = -inf.
  const bool partial = o_ws != nullptr;
  const uint64_t part_rows = (((uint64_t)split * B + wc.b) * H_U + wc.h) * (uint64_t)N_rows;
  const float l_tot = xhalf_sum(l_run);
  const bool seen = l_tot > 0.f;
  const float inv = seen ? 1.f / l_tot : 0.f;
  const bool row_ok = my_row < N_rows;
#pragma unroll
  for (int db = 0; db < C::DB; ++db) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int col = db * 32 + rr * 8 + g * 4;
      if (FULL_D || col < dd) {
        const float o0 = oacc[db][rr * 4 + 0] * inv, o1 = oacc[db][rr * 4 + 1] * inv;
        const float o2 = oacc[db][rr * 4 + 2] * inv, o3 = oacc[db][rr * 4 + 3] * inv;
        if (!partial) {
          u32x2 w;
          w.x = pack_bf16x2(o0, o1);
          w.y = pack_bf16x2(o2, o3);
          __builtin_amdgcn_raw_buffer_store_b64(w, o_rs, (uint32_t)(my_row * dd + col) * 2u, 0, 0);
        } else if (row_ok) {
          typedef float f32x4_t __attribute__((ext_vector_type(4)));
          *reinterpret_cast<f32x4_t*>(o_ws + (part_rows + my_row) * (uint64_t)d + col) =
              f32x4_t{o0, o1, o2, o3};
        }
      }
    }
  }
  if (g == 0 && row_ok) {
    const float ln2 = 0.6931471805599453f;
    const float lse_row = seen ? (m_run + __builtin_amdgcn_logf(l_tot)) * ln2 : -INFINITY;
    if (partial)
      lse_ws[part_rows + my_row] = lse_row;
    else if (lse != nullptr)
      lse[((uint64_t)wc.b * H_U + wc.h) * (uint64_t)N_rows + my_row] = lse_row;
  }
}

}  // namespace attn_numa
