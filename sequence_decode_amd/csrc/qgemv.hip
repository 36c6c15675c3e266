// qgemv.hip -- narrow-batch q8_0 matrix-vector product for 1..16 token rows.
//
// What it computes: ds4 pull request 604, "Commit walkthrough / CUDA kernels"
// (narrow-batch q8_0 matmul: every 32-weight block is read from memory once
// and dotted against all token rows).  That kernel gives one warp to each
// output row; this one is laid out for CDNA4 instead:
//
// * Pair streaming.  Two consecutive 34-byte blocks form a 68-byte pair that
//   starts 4-byte aligned, and no dword of a pair holds weights of both blocks
//   (dword 0 = scale A + 2 weights of A, dwords 1..7 = A, dword 8 = 2 weights of
//   A + scale B, dwords 9..16 = B).  A lane loads whole pairs as 4 x dwordx4 +
//   1 dword; the 64 lanes of a wave cover 64 consecutive pairs of a row.
// * Activation staging in LDS.  Each workgroup converts the compact q8
//   activations once into the same padded pair layout (zero bytes where the
//   weight pair has its scales, the two block scales appended), so every weight
//   dword meets its activation dword at the same index and v_dot4 needs no
//   byte shuffles.  The scale bytes meet zeros and add nothing.
// * Fixed reduction order.  Lane l owns pairs l, l+64, l+128, ... of every row
//   and adds s_A then s_B of each pair, in increasing pair order, into one fp32
//   accumulator per (row, token); the 64 lane sums are then combined by a fixed
//   xor butterfly.  The order depends on K alone -- not on the number of
//   tokens, the rows per wave, the grid or the LDS slicing -- so a token row
//   gets the same bits in any batch (the exactness demanded by "feat(qwen4exp):
//   exact 4-slot concurrent serving", "How it stays exact").
// * Exact integer part.  A block dot is at most 32*127*127 in magnitude, an
//   exact int32 and an exact fp32; s_b = (d_w * d_x) * isum is two fp32
//   multiplies, never fused.
#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

// Rows processed together by one wave for a batch of NT tokens: enough bytes
// in flight per wave, within the register budget of ~3 waves per SIMD.
template <int NT>
struct RowsPerWave {
  static constexpr int value = NT <= 2 ? 4 : (NT <= 8 ? 2 : 4);
};

__device__ __forceinline__ void stage_pairs(uint32_t* __restrict__ lds, const int8_t* __restrict__ xq,
                                            int64_t K, const float* __restrict__ xd, int nb,
                                            int nt, int p0, int np) {
  for (int i = threadIdx.x; i < nt * np; i += kGemvThreads) {
    const int t = i / np;
    const int pl = i - t * np;
    const int p = p0 + pl;
    const u32x4a* src = reinterpret_cast<const u32x4a*>(xq + (int64_t)t * K + 64 * (int64_t)p);
    uint32_t a[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x4a q = src[v];
      a[4 * v + 0] = q.x;
      a[4 * v + 1] = q.y;
      a[4 * v + 2] = q.z;
      a[4 * v + 3] = q.w;
    }
    uint32_t o[20];
    o[0] = a[0] << 16;
#pragma unroll
    for (int c = 1; c < 8; ++c) o[c] = (a[c - 1] >> 16) | (a[c] << 16);
    o[8] = a[7] >> 16;
#pragma unroll
    for (int c = 0; c < 8; ++c) o[9 + c] = a[8 + c];
    o[17] = __float_as_uint(xd[(int64_t)t * nb + 2 * p]);
    o[18] = __float_as_uint(xd[(int64_t)t * nb + 2 * p + 1]);
    o[19] = 0u;
    u32x4a* dst = reinterpret_cast<u32x4a*>(lds + (size_t)(t * np + pl) * kActDw);
#pragma unroll
    for (int v = 0; v < 5; ++v) {
      u32x4a q;
      q.x = o[4 * v + 0];
      q.y = o[4 * v + 1];
      q.z = o[4 * v + 2];
      q.w = o[4 * v + 3];
      dst[v] = q;
    }
  }
}

template <int NT, int R>
__global__ __launch_bounds__(kGemvThreads) void k_qgemv_q8_0(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd,
    const float* residual, float* y, int64_t ldy,
    int slice_pairs, int n_slices, int n_row_groups) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = 2 * P;

  if (n_slices == 1) {
    stage_pairs(lds, xq, K, xd, nb, NT, 0, P);
    __syncthreads();
  }

  for (int rg = blockIdx.x; rg < n_row_groups; rg += gridDim.x) {
    const int n0 = (rg * 4 + wave) * R;
    float acc[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[r][t] = 0.0f;

    for (int sl = 0; sl < n_slices; ++sl) {
      const int p0 = sl * slice_pairs;
      const int np = min(slice_pairs, P - p0);
      if (n_slices > 1) {
        __syncthreads();
        stage_pairs(lds, xq, K, xd, nb, NT, p0, np);
        __syncthreads();
      }
      for (int pl = lane; pl < np; pl += 64) {
        const int64_t pbyte = (int64_t)kPairBytes * (p0 + pl);
        uint32_t wv[R][kPairDw];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = n0 + r;
          if (n < N) {
            const uint32_t* src = reinterpret_cast<const uint32_t*>(w + (int64_t)n * row_bytes + pbyte);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              u32x4 q = *reinterpret_cast<const u32x4*>(src + 4 * v);
              wv[r][4 * v + 0] = q.x;
              wv[r][4 * v + 1] = q.y;
              wv[r][4 * v + 2] = q.z;
              wv[r][4 * v + 3] = q.w;
            }
            wv[r][16] = src[16];
          } else {
#pragma unroll
            for (int c = 0; c < kPairDw; ++c) wv[r][c] = 0u;
          }
        }
        float dwA[R], dwB[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          dwA[r] = f16_bits_to_f32(wv[r][0]);
          dwB[r] = f16_bits_to_f32(wv[r][8] >> 16);
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const u32x4a* ap = reinterpret_cast<const u32x4a*>(lds + (size_t)(t * np + pl) * kActDw);
          uint32_t a[20];
#pragma unroll
          for (int v = 0; v < 5; ++v) {
            u32x4a q = ap[v];
            a[4 * v + 0] = q.x;
            a[4 * v + 1] = q.y;
            a[4 * v + 2] = q.z;
            a[4 * v + 3] = q.w;
          }
          const float dxA = __uint_as_float(a[17]);
          const float dxB = __uint_as_float(a[18]);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            int iA = 0, iB = 0;
#pragma unroll
            for (int c = 0; c < 9; ++c) iA = __builtin_amdgcn_sdot4(wv[r][c], a[c], iA, false);
#pragma unroll
            for (int c = 9; c < 17; ++c) iB = __builtin_amdgcn_sdot4(wv[r][c], a[c], iB, false);
            const float sA = fmul(fmul(dwA[r], dxA), (float)iA);
            const float sB = fmul(fmul(dwB[r], dxB), (float)iB);
            acc[r][t] = fadd(fadd(acc[r][t], sA), sB);
          }
        }
      }
    }

#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int n = n0 + r;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float v = wave_sum_fixed(acc[r][t]);
        if (lane == 0 && n < N) {
          float o = v;
          if (residual) o = fadd(residual[(int64_t)t * ldy + n], v);
          y[(int64_t)t * ldy + n] = o;
        }
      }
    }
  }
}

template <int NT>
hipError_t launch_nt(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                     const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  constexpr int R = RowsPerWave<NT>::value;
  const int n_rg = (int)((N + 4 * R - 1) / (4 * R));
  static bool lds_raised = false;  // allow more than 64 KiB of dynamic LDS (160 KiB on gfx950)
  if (!lds_raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_qgemv_q8_0<NT, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemvLdsMax);
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL((k_qgemv_q8_0<NT, R>), dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, residual, y, ldy, pl.slice_pairs, pl.n_slices, n_rg);
  return hipGetLastError();
}

int rows_per_wave(int nt) {
  switch (nt) {
    case 1: return RowsPerWave<1>::value;
    case 2: return RowsPerWave<2>::value;
    case 3: return RowsPerWave<3>::value;
    case 4: return RowsPerWave<4>::value;
    case 5: case 6: case 7: case 8: return RowsPerWave<8>::value;
    default: return RowsPerWave<16>::value;
  }
}

}  // namespace

bool plan_qgemv(int64_t N, int64_t K, int n_tok, GemvPlan* plan) {
  if (N < 1 || K < 256 || K % 256 != 0 || n_tok < 1 || n_tok > SD_MAX_TOKENS) return false;
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 24) return false;
  GemvPlan p;
  p.pairs = (int)(K / 64);
  const size_t per_pair = (size_t)n_tok * kActDw * 4;
  if ((size_t)p.pairs * per_pair <= (size_t)kGemvLdsMax) {
    p.slice_pairs = p.pairs;
    p.n_slices = 1;
  } else {
    int s = (int)(kGemvLdsMax / per_pair) / 64 * 64;
    if (s < 64) return false;
    p.slice_pairs = s;
    p.n_slices = (p.pairs + s - 1) / s;
  }
  p.lds_bytes = (size_t)p.slice_pairs * per_pair;
  p.rows_per_wave = rows_per_wave(n_tok);
  const int64_t n_rg = (N + 4 * p.rows_per_wave - 1) / (4 * p.rows_per_wave);
  int per_cu = (int)((160 * 1024) / p.lds_bytes);
  per_cu = per_cu < 1 ? 1 : (per_cu > 3 ? 3 : per_cu);
  const int64_t max_grid = 256 * (int64_t)per_cu;
  if (n_rg <= max_grid) {
    p.grid = (int)n_rg;
  } else {
    const int64_t iters = (n_rg + max_grid - 1) / max_grid;
    p.grid = (int)((n_rg + iters - 1) / iters);
  }
  *plan = p;
  return true;
}

hipError_t launch_qgemv(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                        int n_tok, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  GemvPlan pl;
  if (!plan_qgemv(N, K, n_tok, &pl)) return hipErrorInvalidValue;
  switch (n_tok) {
#define SD_CASE(n) \
  case n: return launch_nt<n>(pl, w, N, K, xq, xd, residual, y, ldy, st);
    SD_CASE(1) SD_CASE(2) SD_CASE(3) SD_CASE(4) SD_CASE(5) SD_CASE(6) SD_CASE(7) SD_CASE(8)
    SD_CASE(9) SD_CASE(10) SD_CASE(11) SD_CASE(12) SD_CASE(13) SD_CASE(14) SD_CASE(15) SD_CASE(16)
#undef SD_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sd
