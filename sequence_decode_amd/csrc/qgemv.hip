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
#include <mutex>
#include <type_traits>

#include "device_math.hpp"
#include "internal.hpp"
#include "qgemv_dev.hpp"

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


// ---------------------------------------------------------------------------
// 1..8 tokens, K <= 16384 (at most 4 chunks): the streaming kernel.
//
// NW waves per workgroup; wave w takes chunk w % SP (SP = chunks rounded up to
// 1, 2 or 4) of row slot w / SP.  Weights never pass through registers on
// their way in: every wave streams the 64-pair segments of its rows (<= 4352
// bytes, contiguous in memory) with global_load_lds_dwordx4 into a private
// ring of kRing LDS slots, so the bytes in flight per CU are set by the ring,
// not by the register budget.  A lane then reads its pair (17 dwords) from
// LDS; its pair's activations for all tokens sit in registers.  With SP > 1
// the chunk sums of a row meet in LDS and one thread adds them in chunk order.
// Outputs collect in a small LDS table and are written every kTable items: on
// gfx9 stores share the in-order vmcnt counter with the DMAs, so a store
// inside the loop would make each wait for weights also wait for it.
//
// Activations.  Every workgroup needs the same few KiB of activations, and
// at 4 tokens the copies that all waves fetch from L2 at the start rival the
// weights themselves.  So when they fit (STAGE), one workgroup of 8 waves runs
// per CU and its waves DMA the activations of the workgroup's chunks into LDS
// once, contiguously, before the first weights; each lane then takes its
// pair's share from there.  Over 3 or 4 chunks (4 waves, two workgroups per
// CU) each lane loads its pair's activations itself.

// Kernel argument of the RoPE epilogue: the whole RopeArgs (about 620 bytes)
// only for the ROPE instantiation, an empty struct for every other launch.
struct NoRope {};
template <bool ROPE>
using RopeParam = std::conditional_t<ROPE, RopeArgs, NoRope>;

// RMS prologue: the projection's input is the q8 blocks of
// rmsnorm(x, gamma, eps), which every workgroup computes itself (K <= 4096).
struct NoRms {};
template <bool RMS>
using RmsParam = std::conditional_t<RMS, RmsArgs, NoRms>;

// q8 blocks of rmsnorm(x, gamma) for NT rows of D <= 4096 values into the
// staged-activation layout (codes [NT][kStageX], then scales [NT][kStageD]),
// from the rows held in registers (va: elements j * 1024 + tid, vb: elements
// j * 1024 + tid + 512, j < 4; gm: gamma at the same elements, [0] for va,
// [1] for vb).  No memory is read here, so the weight DMAs in flight are not
// waited for.  Bitwise the outputs of k_rmsnorm_q8<4>: that
// kernel runs 1024 threads per row, thread v summing the squares of elements
// j * 1024 + v in j order, then a fixed 64-lane tree per wave, then its 16 wave
// sums in wave order; here thread tid of 512 plays virtual threads tid and
// tid + 512 (virtual waves w and w + 8) with the same sums in the same order.
template <int NT>
__device__ __forceinline__ void rms_to_stage(const RmsArgs& ra, int64_t D, const float (&va)[NT][4],
                                             const float (&vb)[NT][4], const float (&gm)[2][4], uint8_t* stage,
                                             float (*part)[16]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float sa = 0.0f, sb = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sa = fadd(sa, fmul(va[t][j], va[t][j]));
      sb = fadd(sb, fmul(vb[t][j], vb[t][j]));
    }
    sa = wave_sum_fixed(sa);
    sb = wave_sum_fixed(sb);
    if ((tid & 63) == 0) {
      part[t][wave] = sa;
      part[t][wave + 8] = sb;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float total = part[t][0];
#pragma unroll
    for (int w = 1; w < 16; ++w) total = fadd(total, part[t][w]);
    const float r = fdiv(1.0f, sqrtf(fadd(fdiv(total, (float)D), ra.eps)));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if ((int64_t)j * 1024 + 512 * h >= D) break;  // uniform; blocks of 32 stay whole
        const int64_t i = (int64_t)j * 1024 + tid + 512 * h;
        const bool valid = i < D;
        const float v = h ? vb[t][j] : va[t][j];
        const float o = valid ? fmul(fmul(v, r), gm[h][j]) : 0.0f;
        const float amax = group_max<32>(valid ? fabsf(o) : 0.0f);
        const float d = q8_scale(amax);
        if (valid) {
          stage[t * kStageX + i] = (uint8_t)(int8_t)q8_code(o, d);
          if ((tid & 31) == 0) *reinterpret_cast<float*>(stage + NT * kStageX + t * kStageD + (i >> 5) * 4) = d;
        }
      }
    }
  }
}

// SWI (gate|up rows, one chunk, staged): instead of y, the kernel emits the
// SwiGLU of its outputs as q8 blocks (oq, od), each block from one unit of 32
// gate rows and the matching 32 up rows that one workgroup computes.
//
// ROPE (QKV rows, one chunk, staged): item k of a workgroup takes the 8 rows
// of pair group g = blockIdx.x + k * gridDim.x, head g / 16: slots 0..3 hold
// rows 4 (g % 16) + 0..3 of the head and slots 4..7 their rotation partners
// 64 rows on, so both halves of every RoPE pair meet in the workgroup's table.
template <int NT, int SP, int R, int NW, bool STAGE, bool SWI = false, bool ROPE = false, bool RMS = false>
__global__ __launch_bounds__(64 * NW) void k_qgemv_q8_0_dma(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd,
    const float* residual, float* y, int64_t ldy, int S, int8_t* __restrict__ oq,
    float* __restrict__ od, RopeParam<ROPE> ra, RmsParam<RMS> rn) {
  static_assert(!SWI || (SP == 1 && R == 1 && NW == 8 && STAGE), "SwiGLU output: one chunk, staged");
  static_assert(!ROPE || (SP == 1 && R == 1 && NW == 8 && STAGE && !SWI), "RoPE epilogue: one chunk, staged");
  static_assert(!RMS || (SP == 1 && R == 1 && NW == 8 && STAGE && NT <= 4), "RMS prologue: one chunk, staged");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  // chunk sums of the last kTable items, [item % kTable][wave][row * NT + token];
  // written without barriers (one row per item), combined and stored every
  // kTable items
  __shared__ float table[kTable][NW][R * NT];
  // The one-chunk kernel (plain and SwiGLU) deals its workgroup's items to
  // the waves as they ask (an LDS counter) when the outputs of all of them fit
  // dtab; the waves of a workgroup otherwise finish up to 2 us apart
  // (measured, 8 waves of gate|up at 4 tokens), and every item's arithmetic is
  // the same whichever wave takes it.
  constexpr bool kDynOk = STAGE && SP == 1 && R == 1 && NW == 8 && !ROPE;
  constexpr int kDynMax = kDynFloats / NT;  // items dtab holds
  __shared__ float dtab[kDynOk ? kDynMax : 1][NT];
  __shared__ int s_next;
  constexpr int SLOTS = NW / SP;
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
  // staged activations: codes [SP][NT][kStageX], then scales [SP][NT][kStageD]
  uint8_t* stage = lds_dyn + NW * (kRing * R * SEG);
  const int nb = 2 * P;

  // item k of slot sl covers rows (blockIdx.x + k * gridDim.x) * SLOTS * R + sl * R + [0, R);
  // with SWI, unit u = blockIdx.x + (k / 8) * gridDim.x, and local row
  // lr = 8 (k % 8) + sl is gate row 32u + lr (lr < 32) or up row F + 32u + lr - 32
  // weight items issued before the loop: both ring slots where the start
  // waits on something else anyway (the RMS prologue's arithmetic, the
  // per-wave activation loads), one where the staged copies are all it waits
  // for (a second item in flight there measured slower: QKV 7.3 -> 8.1 us,
  // O 5.8 -> 7.1 us at 4 tokens)
  constexpr int kPre = (RMS || !STAGE) ? kRing : kRing - 1;
  // items 0 .. kPre * NW - 1 go out below, kPre per wave, before the first
  // barrier (of the staging or of the RMS prologue)
  if (kDynOk && threadIdx.x == 0) s_next = kPre * NW;
  const int stride = (int)gridDim.x * SLOTS * R;
  const int row0 = (int)blockIdx.x * SLOTS * R;
  const int F = N / 2;
  const int units = F / 32;
  const int iters = SWI ? ((int)blockIdx.x < units ? 8 * ((units - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) : 0)
                        : (N - row0 + stride - 1) / stride;  // uniform in the workgroup
  auto row_at = [&](int k, int sl) {
    if constexpr (SWI) {
      const int u = (int)blockIdx.x + (k >> 3) * (int)gridDim.x;
      const int lr = ((k & 7) << 3) + sl;
      return lr < 32 ? 32 * u + lr : F + 32 * u + lr - 32;
    }
    if constexpr (ROPE) {
      const int g = (int)blockIdx.x + k * (int)gridDim.x;
      return 128 * (g >> 4) + 4 * (g & 15) + (sl < 4 ? sl : 60 + sl);
    }
    return row0 + k * stride + sl * R;
  };
  auto row_of = [&](int k) { return row_at(k, slot); };

  // DMA instructions this wave issues for item k
  auto ins_of = [&](int k) {
    if (k >= iters || seg_bytes == 0) return 0;
    const int r0 = row_of(k);
    const int nr = min(R, N - r0);
    return nr > 0 ? nr * n_ins : 0;
  };
  auto issue = [&](int k) {
    if (ins_of(k) == 0) return;
    const int r0 = row_of(k);
    uint8_t* l = ring + (k % kRing) * (R * SEG);
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r0 + r < N)
        dma_segment(w + (int64_t)(r0 + r) * row_bytes + (int64_t)chunk * SEG, l + r * SEG, seg_bytes, lane);
  };

  if constexpr (RMS) {
    // this workgroup's own q8 blocks of rmsnorm(x): the rows are loaded (and
    // waited for) before any weight goes out, so that the weights' DMAs,
    // issued next, stay in flight while the norm and the quantization run
    __shared__ float part[NT][16];
    float va[NT][4], vb[NT][4], gm[2][4];
    // every load in bounds (indices past the row read its last element) and
    // unconditional, so they all go out back to back; the values past the
    // row are zeroed after the wait
    const int Ki = (int)K;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ia = min(j * 1024 + (int)threadIdx.x, Ki - 1), ib = min(j * 1024 + (int)threadIdx.x + 512, Ki - 1);
      gm[0][j] = rn.gamma[ia];
      gm[1][j] = rn.gamma[ib];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float* xr = rn.x + (int64_t)t * rn.ldx;
        va[t][j] = xr[ia];
        vb[t][j] = xr[ib];
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      asm volatile("" ::"v"(gm[0][j]), "v"(gm[1][j]));
#pragma unroll
      for (int t = 0; t < NT; ++t) asm volatile("" ::"v"(va[t][j]), "v"(vb[t][j]));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool oka = j * 1024 + (int)threadIdx.x < Ki, okb = j * 1024 + (int)threadIdx.x + 512 < Ki;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        va[t][j] = oka ? va[t][j] : 0.0f;
        vb[t][j] = okb ? vb[t][j] : 0.0f;
      }
    }
    for (int d = 0; d < kPre; ++d) issue(d);
    rms_to_stage<NT>(rn, K, va, vb, gm, stage, part);
  } else if constexpr (STAGE) {
    // The workgroup's activation copies, as a list of (chunk, token, part)
    // with parts 0..3 the 1 KiB quarters of the codes and parts 4..5 the two
    // 256-byte halves of the scales (4-byte DMAs: scales are only 4-byte
    // aligned), dealt to the waves round robin; lanes past the chunk's end
    // issue nothing.  Issued ahead of the weights, so waiting for them leaves
    // the weights in flight.
    for (int i = wave; i < min(S, SP) * NT * 6; i += NW) {
      const int c = i / (NT * 6);
      const int t = (i / 6) % NT;
      const int part = i % 6;
      const int cp = min(64, P - 64 * c);  // pairs of chunk c
      if (part < 4) {
        const int off = part * 1024 + lane * 16;
        if (off < cp * 64)
          __builtin_amdgcn_global_load_lds(
              static_cast<const void*>(xq + (int64_t)t * K + 4096 * (int64_t)c + off),
              (lds_ptr)(stage + (c * NT + t) * kStageX + part * 1024), 16, 0, 0);
      } else {
        const int e = (part - 4) * 64 + lane;  // scale index within the chunk
        if (e < 2 * cp)
          __builtin_amdgcn_global_load_lds(
              static_cast<const void*>(xd + (int64_t)t * nb + 128 * (int64_t)c + e),
              (lds_ptr)(stage + SP * NT * kStageX + (c * NT + t) * kStageD + (part - 4) * 256), 4, 0, 0);
      }
    }
  }

  uint32_t act[NT][kPairDw];
  float dxA[NT], dxB[NT];
  if constexpr (!STAGE) {
    // this lane's pair of activations for every token, loaded before any
    // weight goes out (a load behind the weight DMAs would wait for them);
    // unconditional (lanes past the row read pair 0 and zero it), so that the
    // loads of all tokens go out back to back
    const int64_t pp = pv ? (int64_t)p : 0;
    u32x4a raw[NT][4];
    float rA[NT], rB[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4a* src = reinterpret_cast<const u32x4a*>(xq + (int64_t)t * K + 64 * pp);
#pragma unroll
      for (int v = 0; v < 4; ++v) raw[t][v] = src[v];
      rA[t] = xd[(int64_t)t * nb + 2 * pp];
      rB[t] = xd[(int64_t)t * nb + 2 * pp + 1];
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      uint32_t a[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        a[4 * v + 0] = pv ? raw[t][v].x : 0u;
        a[4 * v + 1] = pv ? raw[t][v].y : 0u;
        a[4 * v + 2] = pv ? raw[t][v].z : 0u;
        a[4 * v + 3] = pv ? raw[t][v].w : 0u;
      }
      act[t][0] = a[0] << 16;
#pragma unroll
      for (int c = 1; c < 8; ++c) act[t][c] = (a[c - 1] >> 16) | (a[c] << 16);
      act[t][8] = a[7] >> 16;
#pragma unroll
      for (int c = 0; c < 8; ++c) act[t][9 + c] = a[8 + c];
      dxA[t] = pv ? rA[t] : 0.0f;
      dxB[t] = pv ? rB[t] : 0.0f;
    }
  }
  if constexpr (!RMS) {
    for (int d = 0; d < kPre; ++d) issue(d);
  }

  if constexpr (STAGE) {
    if constexpr (RMS) {
      // every wave's quantized blocks are in the stage
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      // own copies landed (only the weights of the items issued above may be
      // younger), then everyone's
      int younger = 0;
#pragma unroll
      for (int d = 0; d < kPre; ++d) younger += ins_of(d);
      wait_vmcnt_rt(younger);
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int c = pv ? chunk : 0;
      const u32x4a* src = reinterpret_cast<const u32x4a*>(stage + (c * NT + t) * kStageX + 64 * lane);
      const float* sd = reinterpret_cast<const float*>(stage + SP * NT * kStageX + (c * NT + t) * kStageD);
      uint32_t a[16];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const u32x4a q = src[v];
        a[4 * v + 0] = pv ? q.x : 0u;
        a[4 * v + 1] = pv ? q.y : 0u;
        a[4 * v + 2] = pv ? q.z : 0u;
        a[4 * v + 3] = pv ? q.w : 0u;
      }
      dxA[t] = pv ? sd[2 * lane] : 0.0f;
      dxB[t] = pv ? sd[2 * lane + 1] : 0.0f;
      act[t][0] = a[0] << 16;
#pragma unroll
      for (int c2 = 1; c2 < 8; ++c2) act[t][c2] = (a[c2 - 1] >> 16) | (a[c2] << 16);
      act[t][8] = a[7] >> 16;
#pragma unroll
      for (int c2 = 0; c2 < 8; ++c2) act[t][9 + c2] = a[8 + c2];
    }
  }

  // ROPE epilogue for output v of row `row`, token t, whose RoPE partner
  // (64 rows away in the same head) has output pv
  auto rope_out = [&](float v, float pv, int row, int t) {
    if constexpr (ROPE) rope_epilogue(ra, v, pv, row, t, y, ldy);
  };

  // Combines and stores the outputs of items [kb, kb + cnt): each row gets its
  // chunk sums added in chunk order.
  auto flush = [&](int kb, int cnt) {
    __syncthreads();
    for (int i = threadIdx.x; i < cnt * SLOTS * R * NT; i += 64 * NW) {
      const int ki = i / (SLOTS * R * NT);
      const int rem = i - ki * (SLOTS * R * NT);
      const int sl = rem / (R * NT);
      const int j = rem - sl * (R * NT);
      const int row = row_at(kb + ki, sl) + j / NT;
      const int e = (kb + ki) % kTable;
      float tot = table[e][sl * SP][j];
      for (int c = 1; c < S; ++c) tot = fadd(tot, table[e][sl * SP + c][j]);
      if constexpr (ROPE) {
        if (row < N) rope_out(tot, table[e][sl ^ 4][j], row, j);
      } else {
        if (row < N) store_out(tot, row, j % NT, residual, y, ldy);
      }
    }
    __syncthreads();
  };

  // the cells of the R rows at st (rows r0 ..) for every token
  auto item_cells = [&](const uint8_t* st, int r0, float (&v)[R][NT]) {
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
  };
  // the fixed lane tree over the cells; put(r, t, total) runs on one lane per
  // (row, token)
  auto item_sums = [&](float (&v)[R][NT], auto&& put) {
    if constexpr (NT >= 2 && NT <= 8) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float tot = wave_sum_fixed_tr<NT>(v[r], lane);
        const int tt = tree_token(lane, NT);
        if (lane < tree_writers(NT) && tt < NT) put(r, tt, tot);
      }
    } else {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int t = 0; t < NT; ++t) v[r][t] = wave_sum_fixed(v[r][t]);
      if (lane == 0)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int t = 0; t < NT; ++t) put(r, t, v[r][t]);
    }
  };

  if constexpr (kDynOk) {
    // item i of the workgroup = item i / NW of slot i % NW: the row of the
    // static order.  Wave w starts with items w (and w + NW with two issued
    // ahead), which went out above.
    const int total = NW * iters;
    if (total <= kDynMax) {
      auto row_item = [&](int i) { return row_at(i / NW, i % NW); };
      // (the LDS add is written out: as a builtin the compiler makes it wait
      // for every DMA in flight first, since they write LDS too)
      const uint32_t next_addr = (uint32_t)(uintptr_t)(lds_ptr)&s_next;
      auto grab = [&]() {
        int v = 0;
        if (lane == 0)
          asm volatile("ds_add_rtn_u32 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(next_addr), "v"(1) : "memory");
        return __builtin_amdgcn_readfirstlane(v);
      };
      int cur = wave, cs = 0;  // item this wave computes next, and its ring slot
      int nxt = wave + NW;     // the one after it, if already issued
      bool ahead = kPre == 2;
      while (cur < total) {
        if (!ahead) {
          nxt = grab();
          if (nxt < total && row_item(nxt) < N)
            dma_segment(w + (int64_t)row_item(nxt) * row_bytes, ring + (cs ^ 1) * SEG, seg_bytes, lane);
        }
        ahead = false;
        wait_vmcnt_rt(nxt < total && row_item(nxt) < N ? n_ins : 0);
        const int row = row_item(cur);
        if (row < N) {
          float v[R][NT];
          item_cells(ring + cs * SEG, row, v);
          item_sums(v, [&](int, int t, float tot) { dtab[cur][t] = tot; });
        }
        cur = nxt;
        cs ^= 1;
      }
      __syncthreads();
      if constexpr (SWI) {
        // unit ui of the workgroup: items 64 ui .. 64 ui + 63 are its gate
        // rows 0..31 and up rows 0..31; one 32-lane group per (unit, token)
        for (int e = threadIdx.x; e < (iters / 8) * NT * 32; e += 64 * NW) {
          const int ui = e / (NT * 32);
          const int t = (e >> 5) % NT;
          const int i = e & 31;
          swiglu_epilogue(dtab[64 * ui + i][t], dtab[64 * ui + 32 + i][t], t, i,
                          (int)blockIdx.x + ui * (int)gridDim.x, F, units, oq, od);
        }
      } else {
        for (int i = threadIdx.x; i < total * NT; i += 64 * NW) {
          const int row = row_item(i / NT);
          if (row < N) store_out(dtab[i / NT][i % NT], row, i % NT, residual, y, ldy);
        }
      }
      return;
    }
  }

  int kb = 0;
  for (int k = 0; k < iters; ++k) {
    if (k + kRing - 1 >= kPre) issue(k + kRing - 1);
    // wait for item k: the only VMEM operations younger than its DMAs are the
    // DMAs of the items issued after it (and, with SWI, the block stores below;
    // no other global store happens in the loop)
    int younger = 0;
#pragma unroll
    for (int d = 1; d < kRing; ++d) younger += ins_of(k + d);
    if constexpr (SWI) {
      // the previous unit's block stores (a code and a scale store in each
      // wave that holds a (token, dim) of it) came after this item's DMAs
      if (k > 0 && (k & 7) == 0 && wave * 64 < NT * 32) younger += 2;
    }
    wait_vmcnt_rt(younger);
    const int r0 = row_of(k);
    float v[R][NT];
    item_cells(ring + (k % kRing) * (R * SEG), r0, v);
    item_sums(v, [&](int r, int t, float tot) { table[k % kTable][wave][r * NT + t] = tot; });
    if constexpr (SWI) {
      if ((k & 7) == 7) {
        // the unit's 64 rows are in the table: m = silu(g) * u for 32 dims and
        // every token, quantized as one q8 block per token (32 lanes each).
        // LDS-only barrier: the weights of the next items stay in flight.  The
        // table entries read here are rewritten only 4 units later, after
        // this barrier's successors, which every reader here reaches first.
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const int u = (int)blockIdx.x + (k >> 3) * (int)gridDim.x;
        if ((int)threadIdx.x < NT * 32) {
          const int t = threadIdx.x >> 5;
          const int i = threadIdx.x & 31;
          const int kb8 = k - 7;
          const float g = table[(kb8 + (i >> 3)) % kTable][i & 7][t];
          const float up = table[(kb8 + 4 + (i >> 3)) % kTable][i & 7][t];
          swiglu_epilogue(g, up, t, i, u, F, units, oq, od);
        }
      }
    } else if (k - kb == kTable - 1) {
      flush(kb, kTable);
      kb = k + 1;
    }
  }
  if constexpr (!SWI) {
    if (kb < iters) flush(kb, iters - kb);
  }
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

// ---------------------------------------------------------------------------
// Any batch width on the matrix cores (v_mfma_i32_16x16x64_i8), with the
// same cells, tree and chunk order as the two kernels above, hence the same
// bits.
//
// A workgroup (8 waves) owns tiles of 16 rows.  For K chunk c it stages the
// activations of pairs 64c .. 64c+63 for all tokens in LDS in the padded pair
// layout: dwords 1..16 of each (pair, token) as one 64-byte entry; dword 0
// and the two block scales go to a per-pair table of 16-token vectors.  Wave
// w takes pairs 64c + 8w + j, j = 0..7, of the tile.  Lane (col, kq) loads
// pair bytes 4 + 16kq .. 19 + 16kq of row col (global_load_dwordx4) and pair
// dword 0; the 16-byte pieces of lanes kq = 0, 1 lie in block A (weights 2..31
// and the scale of B, which meets activation zeros), those of kq = 2, 3 in
// block B.  Against token col's activation piece at the same bytes, one MFMA
// sums block A (lanes kq >= 2 feed zeros, read from a zero region of LDS) and
// one sums block B (lanes kq <= 1 feed zeros); weights 0, 1 of block A (pair
// dword 0, whose scale bytes meet zeros) join the first sum through v_dot4.
// The accumulator of lane (col, kq) holds tokens 4kq .. 4kq+3 of row col; the
// lane forms those four cells (0 + s_A) + s_B exactly as the narrow kernels
// do and runs the 8-leaf tree of its pairs in registers.  The eight wave
// subtrees meet in LDS as ((w0+w1)+(w2+w3)) + ((w4+w5)+(w6+w7)), the last
// three levels of the 64-leaf tree, and the chunk sums are added in chunk
// order.  A wave loads the next tile's weights while it works on the current
// one (two register sets), and the per-tile sums alternate between two LDS
// tables, so a tile costs one barrier.
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kMfmaThreads = 512;
constexpr int kMfmaWaves = 8;
constexpr int kMfmaPairs = 8;   // pairs per wave per chunk
constexpr int kMfmaGroup = 8;   // tiles whose running totals a thread keeps across chunks
// LDS (bytes): activations [64 pairs][16 tokens][16 dwords]; per-pair vectors
// [64][3][16] (scale A, scale B, dword 0); zeros covering one wave's read span;
// two tables [8 waves][16 rows][16 tokens]
constexpr int kMfmaActBytes = 64 * 16 * 64;
constexpr int kMfmaScBytes = 64 * 3 * 16 * 4;
constexpr int kMfmaZeroBytes = kMfmaPairs * 1024 + 1024;
constexpr int kMfmaTabBytes = 2 * kMfmaWaves * 256 * 4;

struct MfmaW {  // one wave's weights of one tile: 16 bytes at 4 + 16kq and dword 0 of 8 pairs
  u32x4a q[kMfmaPairs];
  uint32_t d0[kMfmaPairs];
};

__global__ __launch_bounds__(kMfmaThreads, 1) void k_qgemv_q8_0_mfma(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd, int n_tok,
    const float* residual, float* y, int64_t ldy, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  uint32_t* s_act = reinterpret_cast<uint32_t*>(lds_dyn);
  float* s_sc = reinterpret_cast<float*>(lds_dyn + kMfmaActBytes);
  uint32_t* s_zero = reinterpret_cast<uint32_t*>(lds_dyn + kMfmaActBytes + kMfmaScBytes);
  float* s_tab = reinterpret_cast<float*>(lds_dyn + kMfmaActBytes + kMfmaScBytes + kMfmaZeroBytes);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar loop bounds
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int chunks = (P + 63) / 64;
  const int nb = 2 * P;
  const int my_tiles = (int)blockIdx.x < n_tiles ? (n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  // combine: 32 lanes of every wave -> output (row, token)
  const bool comb = lane < 32;
  const int cidx = wave * 32 + (lane & 31);
  const int trow = cidx >> 4;
  const int ttok = cidx & 15;
  for (int e = tid; e < kMfmaZeroBytes / 4; e += kMfmaThreads) s_zero[e] = 0u;
  // this lane's activation piece of pair j: act_l + 256 j dwords (tokens >= n_tok
  // and the other block's lanes read zeros at the same offsets)
  const uint32_t* act_l = s_act + (wave * kMfmaPairs * 16 + col) * 16 + 4 * kq;
  const uint32_t* zero_l = s_zero + col * 16 + 4 * kq;
  const uint32_t* srcA = (kq <= 1 && col < n_tok) ? act_l : zero_l;
  const uint32_t* srcB = (kq >= 2 && col < n_tok) ? act_l : zero_l;
  const float* sc_l = s_sc + wave * kMfmaPairs * 48 + 4 * kq;
  const int bperm_b = (col + 16) * 4;  // lane holding pair dword 8 (the scale of B) for this row

  // weights of item (chunk c, tile) for this wave
  auto load_w = [&](MfmaW& B, int c, int tile) {
    const int np = min(64, P - 64 * c);
    // rows past N read row N-1; their sums stay in their own column and are never stored
    const int n = min(tile * 16 + col, N - 1);
    const uint8_t* pb = w + (int64_t)n * row_bytes + (int64_t)kPairBytes * (64 * (int64_t)c + kMfmaPairs * wave);
    if (kMfmaPairs * wave + kMfmaPairs <= np) {
#pragma unroll
      for (int j = 0; j < kMfmaPairs; ++j) {
        B.q[j] = *reinterpret_cast<const u32x4a*>(pb + kPairBytes * j + 4 + 16 * kq);
        B.d0[j] = *reinterpret_cast<const uint32_t*>(pb + kPairBytes * j);
      }
    } else {
      // last chunk of a row: pairs past the end are zero cells
#pragma unroll
      for (int j = 0; j < kMfmaPairs; ++j) {
        B.q[j] = u32x4a{0u, 0u, 0u, 0u};
        B.d0[j] = 0u;
        if (kMfmaPairs * wave + j < np) {
          B.q[j] = *reinterpret_cast<const u32x4a*>(pb + kPairBytes * j + 4 + 16 * kq);
          B.d0[j] = *reinterpret_cast<const uint32_t*>(pb + kPairBytes * j);
        }
      }
    }
  };

  // this wave's 8-leaf subtree for the 4 tokens of its lane
  auto wave_sub = [&](const MfmaW& B, float (&sub)[4]) {
    struct PairOps {
      v4i DA, DB;
      f32x4 xa, xb;
      u32x4a a0;
      uint32_t dwb;
    };
    auto issue = [&](int j, PairOps& o) {
      const v4i opA = __builtin_bit_cast(v4i, *reinterpret_cast<const u32x4a*>(srcA + j * 256));
      const v4i opB = __builtin_bit_cast(v4i, *reinterpret_cast<const u32x4a*>(srcB + j * 256));
      const v4i wop = __builtin_bit_cast(v4i, B.q[j]);
      const v4i zero = {0, 0, 0, 0};
      o.DA = __builtin_amdgcn_mfma_i32_16x16x64_i8(opA, wop, zero, 0, 0, 0);
      o.DB = __builtin_amdgcn_mfma_i32_16x16x64_i8(opB, wop, zero, 0, 0, 0);
      o.xa = *reinterpret_cast<const f32x4*>(sc_l + j * 48);
      o.xb = *reinterpret_cast<const f32x4*>(sc_l + j * 48 + 16);
      o.a0 = *reinterpret_cast<const u32x4a*>(sc_l + j * 48 + 32);
      o.dwb = (uint32_t)__builtin_amdgcn_ds_bpermute(bperm_b, (int)B.q[j].w);
      // keep program order: a pair's math must not wait for every pair's sums
      asm volatile("" : "+v"(o.DA), "+v"(o.DB));
    };
    float st[3][4];
    auto math = [&](int j, const PairOps& o) {
      const float dwA = f16_bits_to_f32(B.d0[j]);
      const float dwB = f16_bits_to_f32(o.dwb >> 16);
      const float xar[4] = {o.xa.x, o.xa.y, o.xa.z, o.xa.w};
      const float xbr[4] = {o.xb.x, o.xb.y, o.xb.z, o.xb.w};
      const uint32_t a0r[4] = {o.a0.x, o.a0.y, o.a0.z, o.a0.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int iA = __builtin_amdgcn_sdot4((int)B.d0[j], (int)a0r[r], o.DA[r], false);
        const int iB = o.DB[r];
        const float sA = fmul(fmul(dwA, xar[r]), (float)iA);
        const float sB = fmul(fmul(dwB, xbr[r]), (float)iB);
        float v = fadd(fadd(0.0f, sA), sB);
        // 8-leaf tree over j, built as leaves arrive
        if ((j & 1) == 0) {
          st[0][r] = v;
        } else {
          v = fadd(st[0][r], v);
          if ((j & 2) == 0) {
            st[1][r] = v;
          } else {
            v = fadd(st[1][r], v);
            if ((j & 4) == 0) st[2][r] = v;
            else sub[r] = fadd(st[2][r], v);
          }
        }
      }
      asm volatile("" : "+v"(st[0][0]), "+v"(st[0][1]), "+v"(st[0][2]), "+v"(st[0][3]));
    };
    PairOps ops[2];
    issue(0, ops[0]);
#pragma unroll
    for (int j = 0; j < kMfmaPairs; ++j) {
      if (j + 1 < kMfmaPairs) issue(j + 1, ops[(j + 1) & 1]);
      math(j, ops[j & 1]);
    }
  };

  int staged = -1;
  MfmaW wA, wB;
  for (int g0 = 0; g0 < my_tiles; g0 += kMfmaGroup) {
    const int ng = min(kMfmaGroup, my_tiles - g0);
    const int n_items = chunks * ng;  // item i = (chunk i / ng, tile g0 + i % ng)
    float tot[kMfmaGroup];
#pragma unroll
    for (int kk = 0; kk < kMfmaGroup; ++kk) tot[kk] = 0.0f;
    auto tile_of = [&](int i) { return (int)blockIdx.x + (g0 + i % ng) * (int)gridDim.x; };
    auto item = [&](int i, MfmaW& cur, MfmaW& nxt) {
      const int c = i / ng;
      const int kk = i - c * ng;
      if (staged != c) {
        __syncthreads();
        const int np = min(64, P - 64 * c);
        for (int e = tid; e < 64 * 16; e += kMfmaThreads) {
          const int pl = e >> 4;
          const int t = e & 15;
          const int64_t pp = 64 * (int64_t)c + pl;
          uint32_t o[17];
          float da = 0.0f, db = 0.0f;
          if (pl < np && t < n_tok) {
            const u32x4a* src = reinterpret_cast<const u32x4a*>(xq + (int64_t)t * K + 64 * pp);
            uint32_t a[16];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const u32x4a q = src[v];
              a[4 * v + 0] = q.x;
              a[4 * v + 1] = q.y;
              a[4 * v + 2] = q.z;
              a[4 * v + 3] = q.w;
            }
            o[0] = a[0] << 16;
#pragma unroll
            for (int q = 1; q < 8; ++q) o[q] = (a[q - 1] >> 16) | (a[q] << 16);
            o[8] = a[7] >> 16;
#pragma unroll
            for (int q = 0; q < 8; ++q) o[9 + q] = a[8 + q];
            da = xd[(int64_t)t * nb + 2 * pp];
            db = xd[(int64_t)t * nb + 2 * pp + 1];
          } else {
#pragma unroll
            for (int q = 0; q < 17; ++q) o[q] = 0u;
          }
          if (t < n_tok) {
            u32x4a* dst = reinterpret_cast<u32x4a*>(s_act + (pl * 16 + t) * 16);
#pragma unroll
            for (int v = 0; v < 4; ++v)
              dst[v] = u32x4a{o[4 * v + 1], o[4 * v + 2], o[4 * v + 3], o[4 * v + 4]};
          }
          s_sc[(pl * 3 + 0) * 16 + t] = da;
          s_sc[(pl * 3 + 1) * 16 + t] = db;
          s_sc[(pl * 3 + 2) * 16 + t] = __uint_as_float(o[0]);
        }
        __syncthreads();
        staged = c;
      }
      // wait for this tile's weights here, once, before the next tile's loads
      // queue up behind them (the memory counter retires loads in order)
#pragma unroll
      for (int j = 0; j < kMfmaPairs; ++j) asm volatile("" ::"v"(cur.q[j]), "v"(cur.d0[j]));
      if (i + 1 < n_items) load_w(nxt, (i + 1) / ng, tile_of(i + 1));
      float sub[4];
      wave_sub(cur, sub);
      float* tab = s_tab + (i & 1) * (kMfmaWaves * 256);
      *reinterpret_cast<f32x4*>(tab + (wave * 16 + col) * 16 + 4 * kq) = f32x4{sub[0], sub[1], sub[2], sub[3]};
      __syncthreads();
      if (comb) {
        const float* tb = tab + trow * 16 + ttok;
        const float cs = fadd(fadd(fadd(tb[0], tb[256]), fadd(tb[512], tb[768])),
                              fadd(fadd(tb[1024], tb[1280]), fadd(tb[1536], tb[1792])));
#pragma unroll
        for (int q = 0; q < kMfmaGroup; ++q)
          if (q == kk) tot[q] = c == 0 ? cs : fadd(tot[q], cs);
        if (c == chunks - 1) {
          const int n = tile_of(i) * 16 + trow;
          if (n < N && ttok < n_tok) {
            float v = 0.0f;
#pragma unroll
            for (int q = 0; q < kMfmaGroup; ++q)
              if (q == kk) v = tot[q];
            store_out(v, n, ttok, residual, y, ldy);
          }
        }
      }
    };
    load_w(wA, 0, tile_of(0));
    for (int i = 0; i < n_items; i += 2) {
      item(i, wA, wB);
      if (i + 1 < n_items) item(i + 1, wB, wA);
    }
  }
}

// Raises a kernel's dynamic LDS limit to kGemvLdsMax, once per kernel and
// process (thread-safe: concurrent first calls wait for the one that sets it).
template <auto Kern>
hipError_t raise_lds_once() {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              kGemvLdsMax);
  });
  return err;
}

hipError_t launch_mfma(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                       const float* xd, int n_tok, const float* residual, float* y, int64_t ldy,
                       hipStream_t st) {
  // up to 80 KiB of dynamic LDS
  if (hipError_t e = raise_lds_once<&k_qgemv_q8_0_mfma>(); e != hipSuccess) return e;
  hipLaunchKernelGGL(k_qgemv_q8_0_mfma, dim3(pl.grid), dim3(kMfmaThreads), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, n_tok, residual, y, ldy, pl.n_blocks);
  return hipGetLastError();
}

template <int NT, int SP, int NW, bool STAGE, bool SWI = false, bool ROPE = false, bool RMS = false>
hipError_t launch_dma(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                      const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st,
                      int8_t* oq = nullptr, float* od = nullptr, const RopeArgs* ra = nullptr,
                      const RmsArgs* rms = nullptr) {
  constexpr int R = dma_rows(NT);
  // rings and staged activations take up to 140 KiB
  if (hipError_t e = raise_lds_once<&k_qgemv_q8_0_dma<NT, SP, R, NW, STAGE, SWI, ROPE, RMS>>(); e != hipSuccess)
    return e;
  RopeParam<ROPE> rp{};
  if constexpr (ROPE) rp = *ra;
  RmsParam<RMS> rn{};
  if constexpr (RMS) rn = *rms;
  hipLaunchKernelGGL((k_qgemv_q8_0_dma<NT, SP, R, NW, STAGE, SWI, ROPE, RMS>), dim3(pl.grid), dim3(64 * NW), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, residual, y, ldy, pl.chunks, oq, od, rp, rn);
  return hipGetLastError();
}

template <int NT, int R>
hipError_t launch_lds(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                      const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  // allow more than 64 KiB of dynamic LDS (160 KiB on gfx950)
  if (hipError_t e = raise_lds_once<&k_qgemv_q8_0_lds<NT, R>>(); e != hipSuccess) return e;
  hipLaunchKernelGGL((k_qgemv_q8_0_lds<NT, R>), dim3(pl.grid), dim3(kGemvThreads), pl.lds_bytes, st,
                     static_cast<const uint8_t*>(w), (int)N, pl.pairs, (int64_t)(K / 32 * kBlockBytes),
                     xq, K, xd, residual, y, ldy, pl.slice_pairs, pl.n_slices, pl.n_blocks);
  return hipGetLastError();
}

constexpr int lds_rows(int nt) { return nt <= 8 ? 2 : 4; }

template <int NT>
hipError_t launch_dma_nt(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                         const float* xd, const float* residual, float* y, int64_t ldy, hipStream_t st) {
  if (pl.stage) {
    switch (pl.sp) {
      case 1: return launch_dma<NT, 1, 8, true>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      case 2: return launch_dma<NT, 2, 8, true>(pl, w, N, K, xq, xd, residual, y, ldy, st);
      default: return hipErrorInvalidValue;
    }
  }
  if (pl.sp == 4) return launch_dma<NT, 4, 4, false>(pl, w, N, K, xq, xd, residual, y, ldy, st);
  return hipErrorInvalidValue;
}

}  // namespace

size_t mfma_lds_bytes() { return (size_t)kMfmaActBytes + kMfmaScBytes + kMfmaZeroBytes + kMfmaTabBytes; }

bool plan_qgemv(int64_t N, int64_t K, int n_tok, int path, GemvPlan* plan) {
  if (N < 1 || K < 256 || K % 256 != 0 || n_tok < 1 || n_tok > SD_MAX_TOKENS) return false;
  if (N > (int64_t)1 << 30 || K > (int64_t)1 << 24) return false;
  GemvPlan p{};
  p.pairs = (int)(K / 64);
  p.chunks = (p.pairs + 63) / 64;
  const size_t per_pair = (size_t)n_tok * kActDw * 4;
  if (path == SD_GEMV_AUTO) path = n_tok <= 8 && p.chunks <= 4 ? SD_GEMV_NARROW : SD_GEMV_MFMA;
  if (path != SD_GEMV_NARROW && path != SD_GEMV_MFMA) return false;
  p.mfma = path == SD_GEMV_MFMA;
  if (p.mfma) {
    p.use_reg = false;
    p.sp = 0;
    p.rows_per_wave = 0;
    p.slice_pairs = 64;
    p.n_slices = p.chunks;
    p.n_blocks = (int)((N + 15) / 16);  // tiles of 16 rows
    const int64_t max_grid = 256;
    const int64_t iters = (p.n_blocks + max_grid - 1) / max_grid;
    p.grid = (int)((p.n_blocks + iters - 1) / iters);
    p.lds_bytes = mfma_lds_bytes();
    *plan = p;
    return true;
  }
  p.use_reg = n_tok <= 8 && p.chunks <= 4;
  if (p.use_reg) {
    p.sp = p.chunks == 1 ? 1 : (p.chunks == 2 ? 2 : 4);
    // staging paid off with 1 or 2 chunks; over 4 chunks the direct loads of
    // two 4-wave workgroups per CU measured faster
    p.stage = p.sp <= 2 && stage_fits(p.sp, n_tok);
    p.nw = p.stage ? 8 : 4;
    p.rows_per_wave = dma_rows(n_tok);
    p.slice_pairs = p.pairs;
    p.n_slices = 1;
    const int slots = p.nw / p.sp;
    p.n_blocks = (int)((N + p.rows_per_wave - 1) / p.rows_per_wave);
    const int64_t wg_needed = (p.n_blocks + slots - 1) / slots;
    const int64_t max_grid = p.stage ? 256 : 256 * 2;  // one or two workgroups per CU
    const int64_t iters = (wg_needed + max_grid - 1) / max_grid;
    p.grid = (int)((wg_needed + iters - 1) / iters);
    p.lds_bytes = (size_t)p.nw * kRing * p.rows_per_wave * 64 * kPairBytes +
                  (p.stage ? (size_t)p.sp * n_tok * (kStageX + kStageD) : 0);
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
                        int n_tok, const float* residual, float* y, int64_t ldy, hipStream_t st,
                        int path) {
  GemvPlan pl;
  if (!plan_qgemv(N, K, n_tok, path, &pl)) return hipErrorInvalidValue;
  if (pl.mfma) return launch_mfma(pl, w, N, K, xq, xd, n_tok, residual, y, ldy, st);
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

// The gate|up projection (N = 2F rows: gate rows, then up rows) with the
// SwiGLU of its outputs quantized in the same launch: oq / od get exactly what
// launch_swiglu_q8 would make of the projection's outputs.  Needs the staged
// one-chunk streaming kernel (n_tok <= 8, K <= 4096) and F % 32 == 0; else
// hipErrorInvalidValue and nothing is launched.
bool swiglu_fusable(int64_t F, int64_t K, int n_tok) {
  GemvPlan pl;
  if (F < 32 || F % 32 != 0 || F > ((int64_t)1 << 29)) return false;
  if (!plan_qgemv(2 * F, K, n_tok, SD_GEMV_NARROW, &pl)) return false;
  return pl.use_reg && pl.stage && pl.sp == 1;
}

// The RMS prologue pays only for one row: every workgroup normalizes and
// quantizes every row itself, and with two or more rows that work outweighs
// the launch it saves (decode at 2 / 3 / 4 sequences: 820 / 973 / 1000 tok/s
// with it against 834 / 1052 / 1099 without; one sequence: 461 against 437).
bool rms_fusable(int64_t K, int n_tok) { return K <= 4096 && n_tok == 1; }

hipError_t launch_qgemv_swiglu(const void* w, int64_t F, int64_t K, const int8_t* xq, const float* xd,
                               int n_tok, int8_t* oq, float* od, hipStream_t st, const RmsArgs* rms) {
  if (!swiglu_fusable(F, K, n_tok)) return hipErrorInvalidValue;
  if (rms && !rms_fusable(K, n_tok)) return hipErrorInvalidValue;
  GemvPlan pl;
  plan_qgemv(2 * F, K, n_tok, SD_GEMV_NARROW, &pl);
  // one unit (32 gate rows and their 32 up rows, 8 items per wave) at a time
  const int64_t units = F / 32;
  const int64_t per = (units + 255) / 256;
  pl.grid = (int)((units + per - 1) / per);
  if (rms)
    return launch_dma<1, 1, 8, true, true, false, true>(pl, w, 2 * F, K, nullptr, nullptr, nullptr, nullptr, 0, st,
                                                         oq, od, nullptr, rms);
  switch (n_tok) {
#define SD_CASE(n) \
  case n: return launch_dma<n, 1, 8, true, true>(pl, w, 2 * F, K, xq, xd, nullptr, nullptr, 0, st, oq, od);
    SD_CASE(1) SD_CASE(2) SD_CASE(3) SD_CASE(4) SD_CASE(5) SD_CASE(6) SD_CASE(7) SD_CASE(8)
#undef SD_CASE
    default: return hipErrorInvalidValue;
  }
}

// QKV projection with RoPE of q and k and the fp16 K/V write (see
// internal.hpp).  Needs the staged one-chunk streaming kernel (n_tok <= 8,
// K <= 4096) and heads of 128 rows; else hipErrorInvalidValue and nothing is
// launched.
bool qkv_rope_fusable(int64_t N, int64_t K, int n_tok) {
  GemvPlan pl;
  if (N < 128 || N % 128 != 0 || N > ((int64_t)1 << 29)) return false;
  if (!plan_qgemv(N, K, n_tok, SD_GEMV_NARROW, &pl)) return false;
  return pl.use_reg && pl.stage && pl.sp == 1 && pl.chunks == 1;
}

hipError_t launch_qgemv_qkv_rope(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                                 int n_tok, float* y, int64_t ldy, const RopeArgs& ra, hipStream_t st,
                                 const RmsArgs* rms) {
  if (!qkv_rope_fusable(N, K, n_tok)) return hipErrorInvalidValue;
  if (rms && !rms_fusable(K, n_tok)) return hipErrorInvalidValue;
  GemvPlan pl;
  plan_qgemv(N, K, n_tok, SD_GEMV_NARROW, &pl);
  // one pair group (8 rows) per item, as many items per workgroup as the plain launch
  const int64_t groups = N / 8;
  const int64_t per = (groups + 255) / 256;
  pl.grid = (int)((groups + per - 1) / per);
  if (rms)
    return launch_dma<1, 1, 8, true, false, true, true>(pl, w, N, K, nullptr, nullptr, nullptr, y, ldy, st, nullptr,
                                                         nullptr, &ra, rms);
  switch (n_tok) {
#define SD_CASE(n) \
  case n: return launch_dma<n, 1, 8, true, false, true>(pl, w, N, K, xq, xd, nullptr, y, ldy, st, nullptr, nullptr, &ra);
    SD_CASE(1) SD_CASE(2) SD_CASE(3) SD_CASE(4) SD_CASE(5) SD_CASE(6) SD_CASE(7) SD_CASE(8)
#undef SD_CASE
    default: return hipErrorInvalidValue;
  }
}

// y = W q8(rmsnorm(x)) with the norm computed by every workgroup of the
// projection (the output head of the step): the staged one-chunk streaming
// kernel, K <= 4096, one row; else hipErrorInvalidValue.
hipError_t launch_qgemv_rms(const void* w, int64_t N, int64_t K, const RmsArgs& rms, int n_tok, float* y,
                            int64_t ldy, hipStream_t st) {
  GemvPlan pl;
  if (!rms_fusable(K, n_tok) || !plan_qgemv(N, K, n_tok, SD_GEMV_NARROW, &pl)) return hipErrorInvalidValue;
  if (!pl.use_reg || !pl.stage || pl.sp != 1) return hipErrorInvalidValue;
  return launch_dma<1, 1, 8, true, false, false, true>(pl, w, N, K, nullptr, nullptr, nullptr, y, ldy, st, nullptr,
                                                        nullptr, nullptr, &rms);
}

}  // namespace sd
