// qgemv_dev.hpp -- device pieces of the streaming q8_0 GEMV (qgemv.hip): the
// pair cells, the fixed lane trees, the weight DMA and the epilogues of the
// fused QKV/RoPE and gate|up/SwiGLU launches.  Every kernel that computes a
// projection row takes its cells, tree and chunk sums from here, so the row
// gets the same bits whichever kernel computes it.
#pragma once

#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

// The cell of one pair for R rows and one token: (0 + s_A) + s_B.
template <int R>
__device__ __forceinline__ void pair_cells(float (&cell)[R], const uint32_t (&wv)[R][kPairDw],
                                           const uint32_t (&a)[kPairDw], float dxA, float dxB) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int iA = 0, iB = 0;
#pragma unroll
    for (int c = 0; c < 9; ++c) iA = __builtin_amdgcn_sdot4(wv[r][c], a[c], iA, false);
#pragma unroll
    for (int c = 9; c < 17; ++c) iB = __builtin_amdgcn_sdot4(wv[r][c], a[c], iB, false);
    const float dwA = f16_bits_to_f32(wv[r][0]);
    const float dwB = f16_bits_to_f32(wv[r][8] >> 16);
    const float sA = fmul(fmul(dwA, dxA), (float)iA);
    const float sB = fmul(fmul(dwB, dxB), (float)iB);
    cell[r] = fadd(fadd(0.0f, sA), sB);
  }
}

__device__ __forceinline__ void store_out(float v, int n, int t, const float* residual, float* y,
                                          int64_t ldy) {
  float o = v;
  if (residual) o = fadd(residual[(int64_t)t * ldy + n], v);
  y[(int64_t)t * ldy + n] = o;
}

constexpr int kRing = 2;
constexpr int kTable = 32;
// outputs (items x tokens) of a workgroup that the one-chunk kernel keeps until
// the end when it deals the items to its waves on demand; 4 KiB of static LDS,
// which with the output table leaves the 144 KiB of dynamic LDS room
constexpr int kDynFloats = 1024;
// rows per streaming item (one row per item measured best: deeper or wider
// items lowered the bytes in flight per CU)
constexpr int dma_rows(int) { return 1; }
// staged activation bytes per chunk and token: 4096 code bytes + 128 fp32 scales
constexpr int kStageX = 4096;
constexpr int kStageD = 512;
// 8 waves with their rings, the staged activations of sp chunks and the
// output table fit the 160 KiB of LDS (all 8 tokens over 1 or 2 chunks)
constexpr bool stage_fits(int sp, int nt) {
  return 8 * kRing * dma_rows(nt) * 64 * kPairBytes + sp * nt * (kStageX + kStageD) <= kGemvLdsMax &&
         8 * kRing * dma_rows(nt) * 64 * kPairBytes + sp * nt * (kStageX + kStageD) +
                 kTable * 8 * dma_rows(nt) * nt * 4 <= 160 * 1024;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most n DMA instructions of this wave are outstanding.
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// The same for a count held per wave (made scalar here, so the choice is a
// scalar branch), up to 31; a larger n waits for at most 31: longer, never
// shorter.
__device__ __forceinline__ void wait_vmcnt_wave(int n) {
  switch (__builtin_amdgcn_readfirstlane(n)) {
#define SD_WAIT(i) \
  case i: wait_vmcnt<i>(); break;
    SD_WAIT(0) SD_WAIT(1) SD_WAIT(2) SD_WAIT(3) SD_WAIT(4) SD_WAIT(5) SD_WAIT(6) SD_WAIT(7)
    SD_WAIT(8) SD_WAIT(9) SD_WAIT(10) SD_WAIT(11) SD_WAIT(12) SD_WAIT(13) SD_WAIT(14) SD_WAIT(15)
    SD_WAIT(16) SD_WAIT(17) SD_WAIT(18) SD_WAIT(19) SD_WAIT(20) SD_WAIT(21) SD_WAIT(22) SD_WAIT(23)
    SD_WAIT(24) SD_WAIT(25) SD_WAIT(26) SD_WAIT(27) SD_WAIT(28) SD_WAIT(29) SD_WAIT(30)
#undef SD_WAIT
    default: wait_vmcnt<31>(); break;
  }
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Cache policy of the weight DMAs: non-temporal (nt).  Each weight byte is
// read once per pass and a model's weights are many times the 256 MB
// Infinity Cache, so keeping them there buys nothing; with nt the 8B-class
// sweep streams 4-5% faster at 1-4 tokens (same bytes, same outputs).
constexpr int kWeightCpol = 2;

// Issues the DMA of one chunk segment (seg_bytes <= 4352) of one row.  A full
// segment is 4 whole 1 KiB instructions plus one for lanes 0..15; a shorter
// (last) segment is cut at the lane granularity.  Returns the instructions issued.
__device__ __forceinline__ int dma_segment(const uint8_t* g, uint8_t* l, int seg_bytes, int lane) {
  if (seg_bytes == 64 * kPairBytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + j * 1024 + lane * 16),
                                       (lds_ptr)(l + j * 1024), 16, 0, kWeightCpol);
    if (lane < 16)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + 4096 + lane * 16),
                                       (lds_ptr)(l + 4096), 16, 0, kWeightCpol);
    return 5;
  }
  const int n = (seg_bytes + 1023) / 1024;
  for (int j = 0; j < n; ++j)
    if (j * 1024 + lane * 16 < seg_bytes)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + j * 1024 + lane * 16),
                                       (lds_ptr)(l + j * 1024), 16, 0, kWeightCpol);
  return n;
}

// The fixed 64-lane tree of wave_sum_fixed for 2..8 token cells at once
// (transposed butterfly).  At the first level (partners lane ^ 1) a lane keeps
// half of the tokens and hands the other half to its partner, at the second
// (lane ^ 2) half of the rest, and with 5..8 tokens at the third (lane 7 - l
// within 8) the last one.  Every addition combines the same two subtree sums
// as wave_sum_fixed applied to each token, so each token's total has the same
// bits, but the tree costs one pass instead of one per token.  Lane l ends
// with the total of token tree_token(l).  The keep/hand-over choices are
// parities of lane bits (b0 ^ b2, then b1 ^ b2, then b0 ^ b3), chosen so that
// each level's partner holds the opposite choice at its own level and the same
// at every other, and the mirrored partners of the later levels (7 - l, 15 - l)
// hold the same token.  Tokens past NT are zeros whose sums are never used.
__device__ __forceinline__ int tree_token(int lane, int nt) {
  const int b0 = lane & 1, b1 = (lane >> 1) & 1, b2 = (lane >> 2) & 1, b3 = (lane >> 3) & 1;
  if (nt == 2) return b0 ^ b2;
  if (nt <= 4) return 2 * (b0 ^ b2) + (b1 ^ b2);
  return 4 * (b0 ^ b2) + 2 * (b1 ^ b2) + (b0 ^ b3);
}

// lanes whose totals are stored, one per token (tree_token of lanes 0 .. n-1)
constexpr int tree_writers(int nt) { return nt == 2 ? 2 : (nt <= 4 ? 4 : 8); }

template <int NT>
__device__ __forceinline__ float wave_sum_fixed_tr(const float (&v)[NT], int lane) {
  static_assert(NT >= 2 && NT <= 8, "2..8 tokens");
  const bool lo1 = ((lane ^ (lane >> 2)) & 1) == 0;  // keeps the first half of the tokens
  float e;
  if constexpr (NT > 4) {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = i < NT ? v[i < NT ? i : 0] : 0.0f;
    float k[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      k[i] = fadd(lo1 ? w[i] : w[4 + i], dpp_mov<0xB1>(lo1 ? w[4 + i] : w[i]));
    const bool lo2 = (((lane >> 1) ^ (lane >> 2)) & 1) == 0;  // keeps the first two of its four
    float m[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      m[i] = fadd(lo2 ? k[i] : k[2 + i], dpp_mov<0x4E>(lo2 ? k[2 + i] : k[i]));
    const bool lo3 = ((lane ^ (lane >> 3)) & 1) == 0;  // keeps the first of its two
    e = fadd(lo3 ? m[0] : m[1], dpp_mov<0x141>(lo3 ? m[1] : m[0]));
    e = fadd(e, dpp_mov<0x140>(e));  // row_mirror
    return cross_row_sum_fixed(e);
  } else if constexpr (NT == 2) {
    const float keep = lo1 ? v[0] : v[1];
    const float send = lo1 ? v[1] : v[0];
    e = fadd(keep, dpp_mov<0xB1>(send));
    e = fadd(e, dpp_mov<0x4E>(e));
  } else {
    const float v3 = NT == 4 ? v[NT == 4 ? 3 : 0] : 0.0f;
    const float k0 = lo1 ? v[0] : v[2], k1 = lo1 ? v[1] : v3;
    const float s0 = lo1 ? v[2] : v[0], s1 = lo1 ? v3 : v[1];
    const float a = fadd(k0, dpp_mov<0xB1>(s0));
    const float b = fadd(k1, dpp_mov<0xB1>(s1));
    const bool lo2 = (((lane >> 1) ^ (lane >> 2)) & 1) == 0;  // keeps the first of its pair
    e = fadd(lo2 ? a : b, dpp_mov<0x4E>(lo2 ? b : a));
  }
  e = fadd(e, dpp_mov<0x141>(e));  // row_half_mirror
  e = fadd(e, dpp_mov<0x140>(e));  // row_mirror
  return cross_row_sum_fixed(e);
}

// The epilogue of the QKV projection with RoPE for output v of QKV row `row`
// and token t, whose RoPE partner (64 rows away in the same 128-row head) has
// output pv: q rows are stored rotated, k and v rows as projected, and the
// rotated k and the v row go to the fp16 cache row of the token's position.
// The arithmetic of k_rope_kv_step: same angles, same rotation, same fp16
// rounding.
__device__ __forceinline__ void rope_epilogue(const RopeArgs& ra, float v, float pv, int row, int t,
                                              float* y, int64_t ldy) {
  const int hd = row >> 7, d = row & 127, ip = d & 63;
  const bool lo = d < 64;
  float r = v;
  if (hd < ra.n_heads + ra.n_kv) {
    float c, s;
    if (ra.tab_mode == 2) {
      c = ra.cs_tab[2 * (t * 64 + ip)];
      s = ra.cs_tab[2 * (t * 64 + ip) + 1];
    } else {
      rope_angle(ra.pos[t], ip, 128, ra.theta, &c, &s);
      if (ra.tab_mode == 1 && hd == 0 && lo) {
        ra.cs_tab[2 * (t * 64 + ip)] = c;
        ra.cs_tab[2 * (t * 64 + ip) + 1] = s;
      }
    }
    float y0, y1;
    rope_rotate(lo ? v : pv, lo ? pv : v, c, s, &y0, &y1);
    r = lo ? y0 : y1;
  }
  y[(int64_t)t * ldy + row] = hd < ra.n_heads ? r : v;
  if (hd >= ra.n_heads) {
    int sq = 0;
#pragma unroll
    for (int i = 1; i < SD_MAX_SEQS; ++i)
      if (i < ra.seqs.n_seq && t >= ra.seqs.s[i].row0) sq = i;
    const SeqArg& a = ra.seqs.s[sq];
    const int64_t crow = seq_row(a, a.ctx_len - a.n_new + (t - a.row0));
    const bool is_k = hd < ra.n_heads + ra.n_kv;
    const int g = hd - ra.n_heads - (is_k ? 0 : ra.n_kv);
    uint16_t* dst = (is_k ? a.k_w : a.v_w) + crow * a.ld_tok + (int64_t)g * a.ld_head + d;
    *dst = f32_to_f16_bits(r);
  }
}

// The SwiGLU epilogue of the gate|up projection for lane i (0..31) of token
// t's block of unit u (FFN dims 32u .. 32u+31): m = silu(g) * up, quantized as
// one q8 block (amax over the 32 lanes, which must all call this).
__device__ __forceinline__ void swiglu_epilogue(float g, float up, int t, int i, int u, int F, int units,
                                                int8_t* oq, float* od) {
  const float silu = fdiv(g, fadd(1.0f, expf(-g)));
  const float m = fmul(silu, up);
  const float amax = group_max<32>(fabsf(m));
  const float d = q8_scale(amax);
  oq[(int64_t)t * F + 32 * u + i] = (int8_t)q8_code(m, d);
  if (i == 0) od[(int64_t)t * units + u] = d;
}

}  // namespace sd
