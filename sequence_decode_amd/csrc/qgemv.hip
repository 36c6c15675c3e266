// qgemv.hip -- narrow-batch q8_0 matrix-vector product for 1..16 token rows.
//
// What it computes: ds4 pull request 604, "Commit walkthrough / CUDA kernels"
// (narrow-batch q8_0 matmul: every 32-weight block is read from memory once
// and dotted against all token rows).  That kernel gives one warp to each
// output row; this one is laid out for CDNA4 instead:
//
// * Pairs.  Two consecutive 34-byte blocks form a 68-byte pair that starts
//   4-byte aligned, and no dword of a pair holds weights of both blocks
//   (dword 0 = scale A + 2 weights of A, dwords 1..7 = A, dword 8 = 2 weights of
//   A + scale B, dwords 9..16 = B).  A lane owns one pair of a 64-pair chunk;
//   the 64 lanes of a wave cover 4352 contiguous bytes of a row.
// * Activation staging in LDS.  Each workgroup converts the compact q8
//   activations once into the same padded pair layout (zero bytes where the
//   weight pair has its scales, the two block scales appended), so every weight
//   dword meets its activation dword at the same index and v_dot4 needs no
//   byte shuffles.  The scale bytes meet zeros and add nothing.
// * Fixed reduction order.  K splits into chunks of 64 pairs; in chunk c,
//   lane l owns pair 64c + l and forms its cell (0 + s_A) + s_B (lanes past the
//   last pair hold +0).  The 64 cells of a chunk are summed by a fixed lane
//   tree, and the chunk sums are added in chunk order.  This order depends on
//   K alone -- not on the number of tokens, the rows per wave, the grid, which
//   wave handles which chunk, or whether activations sit in registers or LDS --
//   so a token row gets the same bits in any batch (the exactness demanded by
//   "feat(qwen4exp): exact 4-slot concurrent serving", "How it stays exact").
// * Two kernels share that order.  For 1..8 tokens and K <= 16384 the
//   weights stream HBM -> LDS by DMA (global_load_lds) into per-wave rings, the
//   chunks of a row run on different waves, and each lane keeps its pair's
//   activations in registers.  Wider batches stage the activations in LDS and
//   walk the chunks of a row in a loop.
// * Exact integer part.  A block dot is at most 32*127*127 in magnitude, an
//   exact int32 and an exact fp32; s_b = (d_w * d_x) * isum is two fp32
//   multiplies, never fused.
#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

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

template <int R>
__device__ __forceinline__ void load_pair_rows(uint32_t (&wv)[R][kPairDw], const uint8_t* __restrict__ w,
                                               int n0, int N, int64_t row_bytes, int64_t pbyte,
                                               bool valid) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (valid && n0 + r < N) {
      const uint32_t* src = reinterpret_cast<const uint32_t*>(w + (int64_t)(n0 + r) * row_bytes + pbyte);
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
}

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

__device__ __forceinline__ void read_act(uint32_t (&a)[kPairDw], float& dxA, float& dxB,
                                         const uint32_t* __restrict__ lds_pair) {
  const u32x4a* ap = reinterpret_cast<const u32x4a*>(lds_pair);
  uint32_t t[20];
#pragma unroll
  for (int v = 0; v < 5; ++v) {
    u32x4a q = ap[v];
    t[4 * v + 0] = q.x;
    t[4 * v + 1] = q.y;
    t[4 * v + 2] = q.z;
    t[4 * v + 3] = q.w;
  }
#pragma unroll
  for (int c = 0; c < kPairDw; ++c) a[c] = t[c];
  dxA = __uint_as_float(t[17]);
  dxB = __uint_as_float(t[18]);
}

__device__ __forceinline__ void store_out(float v, int n, int t, const float* residual, float* y,
                                          int64_t ldy) {
  float o = v;
  if (residual) o = fadd(residual[(int64_t)t * ldy + n], v);
  y[(int64_t)t * ldy + n] = o;
}

// ---------------------------------------------------------------------------
// 1..8 tokens, K <= 16384 (at most 4 chunks): the streaming kernel.
//
// Wave w of the workgroup takes chunk w % SP (SP = chunks rounded up to 1, 2
// or 4) of row slot w / SP.  Weights never pass through registers on their
// way in: every wave streams the 64-pair segments of its rows (<= 4352 bytes,
// contiguous in memory) with global_load_lds_dwordx4 into a private ring of
// DEPTH LDS slots, so the bytes in flight per CU are set by the ring, not by
// the register budget.  A lane then reads its pair (17 dwords) from LDS; its
// pair's activations for all tokens were loaded once into registers.  With
// SP > 1 the chunk sums of a row meet in LDS and one thread adds them in chunk
// order.  Outputs collect in a small LDS table and are written every kTable
// items: on gfx9 stores share the in-order vmcnt counter with the DMAs, so a
// store inside the loop would make each wait for weights also wait for it.
constexpr int kRing = 2;
constexpr int kTable = 32;
// rows per streaming item (one row per item measured best: deeper or wider
// items lowered the bytes in flight per CU)
constexpr int dma_rows(int nt) { return nt > 0 ? 1 : 1; }

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

// Issues the DMA of one chunk segment (seg_bytes <= 4352) of one row.  A full
// segment is 4 whole 1 KiB instructions plus one for lanes 0..15; a shorter
// (last) segment is cut at the lane granularity.  Returns the instructions issued.
__device__ __forceinline__ int dma_segment(const uint8_t* g, uint8_t* l, int seg_bytes, int lane) {
  typedef __attribute__((address_space(3))) void* lds_ptr;
  if (seg_bytes == 64 * kPairBytes) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + j * 1024 + lane * 16),
                                       (lds_ptr)(l + j * 1024), 16, 0, 0);
    if (lane < 16)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + 4096 + lane * 16),
                                       (lds_ptr)(l + 4096), 16, 0, 0);
    return 5;
  }
  const int n = (seg_bytes + 1023) / 1024;
  for (int j = 0; j < n; ++j)
    if (j * 1024 + lane * 16 < seg_bytes)
      __builtin_amdgcn_global_load_lds(static_cast<const void*>(g + j * 1024 + lane * 16),
                                       (lds_ptr)(l + j * 1024), 16, 0, 0);
  return n;
}

template <int NT, int SP, int R>
__global__ __launch_bounds__(kGemvThreads) void k_qgemv_q8_0_dma(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd,
    const float* residual, float* y, int64_t ldy, int S) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  // chunk sums of the last kTable items, [item % kTable][wave][row * NT + token];
  // written without barriers (one row per item), combined and stored every
  // kTable items
  __shared__ float table[kTable][4][R * NT];
  constexpr int SLOTS = 4 / SP;
  constexpr int SEG = 64 * kPairBytes;  // bytes of a full chunk segment
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int slot = wave / SP;
  const int chunk = wave % SP;
  const int p = 64 * chunk + lane;
  const bool pv = chunk < S && p < P;
  const int seg_pairs = chunk < S ? min(64, P - 64 * chunk) : 0;
  const int seg_bytes = seg_pairs * kPairBytes;
  const int n_ins = seg_bytes == SEG ? 5 : (seg_bytes + 1023) / 1024;
  uint8_t* ring = lds_dyn + wave * (kRing * R * SEG);

  // item k of slot sl covers rows (blockIdx.x + k * gridDim.x) * SLOTS * R + sl * R + [0, R)
  const int stride = (int)gridDim.x * SLOTS * R;
  const int row0 = (int)blockIdx.x * SLOTS * R;
  const int iters = (N - row0 + stride - 1) / stride;  // uniform in the workgroup

  // DMA instructions this wave issues for item k
  auto ins_of = [&](int k) {
    if (k >= iters || seg_bytes == 0) return 0;
    const int r0 = row0 + k * stride + slot * R;
    const int nr = min(R, N - r0);
    return nr > 0 ? nr * n_ins : 0;
  };
  auto issue = [&](int k) {
    if (ins_of(k) == 0) return;
    const int r0 = row0 + k * stride + slot * R;
    uint8_t* l = ring + (k % kRing) * (R * SEG);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r0 + r < N)
        dma_segment(w + (int64_t)(r0 + r) * row_bytes + (int64_t)chunk * SEG, l + r * SEG, seg_bytes, lane);
  };

  for (int d = 0; d < kRing - 1; ++d) issue(d);

  uint32_t act[NT][kPairDw];
  float dxA[NT], dxB[NT];
  {
    const int nb = 2 * P;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (pv) {
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
        act[t][0] = a[0] << 16;
#pragma unroll
        for (int c = 1; c < 8; ++c) act[t][c] = (a[c - 1] >> 16) | (a[c] << 16);
        act[t][8] = a[7] >> 16;
#pragma unroll
        for (int c = 0; c < 8; ++c) act[t][9 + c] = a[8 + c];
        dxA[t] = xd[(int64_t)t * nb + 2 * p];
        dxB[t] = xd[(int64_t)t * nb + 2 * p + 1];
      } else {
#pragma unroll
        for (int c = 0; c < kPairDw; ++c) act[t][c] = 0u;
        dxA[t] = dxB[t] = 0.0f;
      }
    }
  }

  // Combines and stores the outputs of items [kb, kb + cnt): each row gets its
  // chunk sums added in chunk order.
  auto flush = [&](int kb, int cnt) {
    __syncthreads();
    for (int i = threadIdx.x; i < cnt * SLOTS * R * NT; i += kGemvThreads) {
      const int ki = i / (SLOTS * R * NT);
      const int rem = i - ki * (SLOTS * R * NT);
      const int sl = rem / (R * NT);
      const int j = rem - sl * (R * NT);
      const int row = row0 + (kb + ki) * stride + sl * R + j / NT;
      const int e = (kb + ki) % kTable;
      float tot = table[e][sl * SP][j];
      for (int c = 1; c < S; ++c) tot = fadd(tot, table[e][sl * SP + c][j]);
      if (row < N) store_out(tot, row, j % NT, residual, y, ldy);
    }
    __syncthreads();
  };

  int kb = 0;
  for (int k = 0; k < iters; ++k) {
    issue(k + kRing - 1);
    // wait for item k: the only VMEM operations younger than its DMAs are the
    // DMAs of the items issued after it (no global store happens in the loop)
    int younger = 0;
#pragma unroll
    for (int d = 1; d < kRing; ++d) younger += ins_of(k + d);
    wait_vmcnt_rt(younger);
    const int r0 = row0 + k * stride + slot * R;
    const uint8_t* st = ring + (k % kRing) * (R * SEG);
    float v[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (pv && r0 + r < N) {
        const uint32_t* src = reinterpret_cast<const uint32_t*>(st + r * SEG) + lane * kPairDw;
        uint32_t wv[1][kPairDw];
#pragma unroll
        for (int c = 0; c < kPairDw; ++c) wv[0][c] = src[c];
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float cell[1];
          pair_cells<1>(cell, wv, act[t], dxA[t], dxB[t]);
          v[r][t] = cell[0];
        }
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) v[r][t] = 0.0f;
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int t = 0; t < NT; ++t) v[r][t] = wave_sum_fixed(v[r][t]);
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) table[k % kTable][wave][r * NT + t] = v[r][t];
    if (k - kb == kTable - 1) {
      flush(kb, kTable);
      kb = k + 1;
    }
  }
  if (kb < iters) flush(kb, iters - kb);
}

// ---------------------------------------------------------------------------
// Any batch width, any K: one wave per row block; the chunks of the row are
// visited in order by the whole wave, with the activations staged in LDS
// (all of K at once when it fits, else in slices of whole chunks).
template <int NT, int R>
__global__ __launch_bounds__(kGemvThreads) void k_qgemv_q8_0_lds(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd,
    const float* residual, float* y, int64_t ldy,
    int slice_pairs, int n_slices, int n_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nb = 2 * P;
  if (n_slices == 1) {
    stage_pairs(lds, xq, K, xd, nb, NT, 0, P);
    __syncthreads();
  }
  for (int b0 = blockIdx.x * 4; b0 < n_blocks; b0 += gridDim.x * 4) {
    const int n0 = (b0 + wave) * R;
    float tot[R][NT];
    for (int sl = 0; sl < n_slices; ++sl) {
      const int p0 = sl * slice_pairs;
      const int np = min(slice_pairs, P - p0);
      if (n_slices > 1) {
        __syncthreads();
        stage_pairs(lds, xq, K, xd, nb, NT, p0, np);
        __syncthreads();
      }
      for (int cl = 0; cl < (np + 63) / 64; ++cl) {
        const int pl = 64 * cl + lane;
        const bool pv = pl < np;
        const int c = p0 / 64 + cl;
        uint32_t wv[R][kPairDw];
        load_pair_rows<R>(wv, w, n0, N, row_bytes, (int64_t)kPairBytes * (p0 + pl), pv);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          uint32_t a[kPairDw];
          float dxA = 0.0f, dxB = 0.0f;
          if (pv) {
            read_act(a, dxA, dxB, lds + (size_t)(t * np + pl) * kActDw);
          } else {
#pragma unroll
            for (int q = 0; q < kPairDw; ++q) a[q] = 0u;
          }
          float cell[R];
          pair_cells<R>(cell, wv, a, dxA, dxB);
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float cs = wave_sum_fixed(pv ? cell[r] : 0.0f);
            tot[r][t] = c == 0 ? cs : fadd(tot[r][t], cs);
          }
        }
      }
    }
    if (lane == 0)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          if (n0 + r < N) store_out(tot[r][t], n0 + r, t, residual, y, ldy);
  }
}

template <int NT, int SP>
hipError_t launch_dma(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                      const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  constexpr int R = dma_rows(NT);
  static bool lds_raised = false;  // rings of R rows take up to 70 KiB
  if (!lds_raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_qgemv_q8_0_dma<NT, SP, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemvLdsMax);
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL((k_qgemv_q8_0_dma<NT, SP, R>), dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, residual, y, ldy, pl.chunks);
  return hipGetLastError();
}

template <int NT, int R>
hipError_t launch_lds(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                      const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  static bool lds_raised = false;  // allow more than 64 KiB of dynamic LDS (160 KiB on gfx950)
  if (!lds_raised) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_qgemv_q8_0_lds<NT, R>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kGemvLdsMax);
    if (e != hipSuccess) return e;
    lds_raised = true;
  }
  hipLaunchKernelGGL((k_qgemv_q8_0_lds<NT, R>), dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, residual, y, ldy, pl.slice_pairs, pl.n_slices, pl.n_blocks);
  return hipGetLastError();
}

constexpr int lds_rows(int nt) { return nt <= 8 ? 2 : 4; }

template <int NT>
hipError_t launch_dma_nt(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                         const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  switch (pl.sp) {
    case 1: return launch_dma<NT, 1>(pl, w, N, K, xq, xd, residual, y, ldy, st);
    case 2: return launch_dma<NT, 2>(pl, w, N, K, xq, xd, residual, y, ldy, st);
    default: return launch_dma<NT, 4>(pl, w, N, K, xq, xd, residual, y, ldy, st);
  }
}

}  // namespace

bool plan_qgemv(int64_t N, int64_t K, int n_tok, GemvPlan* plan) {
  if (N < 1 || K < 256 || K % 256 != 0 || n_tok < 1 || n_tok > SD_MAX_TOKENS) return false;
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 24) return false;
  GemvPlan p;
  p.pairs = (int)(K / 64);
  p.chunks = (p.pairs + 63) / 64;
  const size_t per_pair = (size_t)n_tok * kActDw * 4;
  p.use_reg = n_tok <= 8 && p.chunks <= 4;
  if (p.use_reg) {
    p.sp = p.chunks == 1 ? 1 : (p.chunks == 2 ? 2 : 4);
    p.rows_per_wave = dma_rows(n_tok);
    p.slice_pairs = p.pairs;
    p.n_slices = 1;
    const int slots = 4 / p.sp;
    p.n_blocks = (int)((N + p.rows_per_wave - 1) / p.rows_per_wave);
    const int64_t wg_needed = (p.n_blocks + slots - 1) / slots;
    const int64_t max_grid = 256 * 2;
    const int64_t iters = (wg_needed + max_grid - 1) / max_grid;
    p.grid = (int)((wg_needed + iters - 1) / iters);
    p.lds_bytes = (size_t)4 * kRing * p.rows_per_wave * 64 * kPairBytes;
    *plan = p;
    return true;
  } else {
    p.sp = 0;
    p.rows_per_wave = n_tok <= 8 ? 2 : 4;
    if ((size_t)p.pairs * per_pair <= (size_t)kGemvLdsMax) {
      p.slice_pairs = p.pairs;
      p.n_slices = 1;
    } else {
      int sl = (int)(kGemvLdsMax / per_pair) / 64 * 64;
      if (sl < 64) return false;
      p.slice_pairs = sl;
      p.n_slices = (p.pairs + sl - 1) / sl;
    }
    p.n_blocks = (int)((N + p.rows_per_wave - 1) / p.rows_per_wave);
    const int64_t wg_needed = (p.n_blocks + 3) / 4;
    const int64_t max_grid = 256 * 3;
    const int64_t iters = (wg_needed + max_grid - 1) / max_grid;
    p.grid = (int)((wg_needed + iters - 1) / iters);
  }
  p.lds_bytes = (size_t)p.slice_pairs * per_pair;
  *plan = p;
  return true;
}

hipError_t launch_qgemv(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                        int n_tok, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  GemvPlan pl;
  if (!plan_qgemv(N, K, n_tok, &pl)) return hipErrorInvalidValue;
  if (pl.use_reg) {
    switch (n_tok) {
      case 1: return launch_dma_nt<1>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 2: return launch_dma_nt<2>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 3: return launch_dma_nt<3>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 4: return launch_dma_nt<4>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 5: return launch_dma_nt<5>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 6: return launch_dma_nt<6>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 7: return launch_dma_nt<7>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      default: return launch_dma_nt<8>(pl, w, N, K, xq, xd, residual, y, ldy, st);
    }
  }
  switch (n_tok) {
#define SD_CASE(n) \
  case n: return launch_lds<n, lds_rows(n)>(pl, w, N, K, xq, xd, residual, y, ldy, st);
    SD_CASE(1) SD_CASE(2) SD_CASE(3) SD_CASE(4) SD_CASE(5) SD_CASE(6) SD_CASE(7) SD_CASE(8)
    SD_CASE(9) SD_CASE(10) SD_CASE(11) SD_CASE(12) SD_CASE(13) SD_CASE(14) SD_CASE(15) SD_CASE(16)
#undef SD_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace sd
