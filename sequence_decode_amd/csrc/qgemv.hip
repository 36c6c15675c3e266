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
// Any batch width up to 16 on the matrix cores, with the same cells, tree and
// chunk order as the two kernels above, hence the same bits.
//
// Work: tiles of 16 rows.  A workgroup of 8 waves takes tiles blockIdx.x +
// k * gridDim.x and, for each, the K chunks in order (unit = (tile, chunk)).
// Wave w owns pairs 8w .. 8w+7 of every chunk, as two items of 4 pairs; an
// item's weights (16 rows x 4 pairs, 272 contiguous bytes per row) stream into
// the wave's two-slot LDS ring by DMA as whole 16-byte pieces of each row;
// item m + 2 goes out as soon as item m has been read.
//
// Integer sums: one v_mfma_i32_16x16x32_i8 per q8_0 block, A = the 16 tokens'
// activation codes, B = the 16 rows' weight codes, so lane (col, kq) ends with
// the exact block sums of row col for tokens 4kq .. 4kq+3.  The 32 codes of a
// block may be dealt to the four k-groups in any way the two operands share:
// k-group kq takes codes 4kq .. 4kq+3 and 16+4kq .. 19+4kq.  Of block B those
// are weight dwords 9+kq and 13+kq of the pair; block A's codes sit 2 bytes
// into the pair (behind its scale), so they are dwords kq, kq+1 and kq+4, kq+5
// shifted by 16 bits (dword 0 brings codes 0, 1 in its high half, dword 8
// codes 30, 31 in its low half).  Rows sit 272 bytes (68 dwords) apart, so
// each of these reads puts the 64 lanes on 64 distinct banks.
//
// Activations: per chunk each wave loads the codes and block scales of its own
// 8 pairs (contiguous runs of each token's row) and stores them to its own part
// of LDS (a token's 16-byte pieces rotated by the token, so that the reads
// below hit distinct banks); each lane then keeps its token's codes and the
// scales of tokens 4kq .. 4kq+3 in registers for the chunk.  No other wave
// touches that part, so no barrier is needed.  (By DMA instead, or with the
// loads overlapping the first weight DMAs, the launches measured slower.)
//
// Each lane forms its four cells (0 + (dA xA) iA) + (dB xB) iB exactly as the
// streaming kernels do and runs the 8-leaf tree of its pairs in registers;
// the eight wave subtrees meet in LDS as ((w0+w1)+(w2+w3)) + ((w4+w5)+(w6+w7)),
// the top three levels of the 64-leaf tree, and the chunk sums are added in
// chunk order.  The residual rows also come by DMA, and the wave tracks how
// many DMAs it has issued, so each wait names exactly the DMAs that may stay
// in flight (loads and stores issued meanwhile only make a wait longer).
typedef int v4i __attribute__((ext_vector_type(4)));
constexpr int kMfmaThreads = 512;
constexpr int kMfmaWaves = 8;
constexpr int kMfmaRowBytes = 4 * kPairBytes;                      // one row of an item
constexpr int kMfmaItemBytes = 16 * kMfmaRowBytes;                 // 4352
constexpr int kMfmaItemPieces = kMfmaItemBytes / 16;               // 272
constexpr int kMfmaItemDmas = (kMfmaItemPieces + 63) / 64;         // 5
constexpr int kMfmaRingBytes = kMfmaWaves * 2 * kMfmaItemBytes;    // 69632
constexpr int kMfmaActBytes = 64 * 16 * 64;                        // [pair][token][64 B]
constexpr int kMfmaXsBytes = 128 * 16 * 4;                         // [block][token] fp32
constexpr int kMfmaTabBytes = 2 * kMfmaWaves * 256 * 4;            // two [wave][row][token] tables
constexpr int kMfmaResBytes = 256 * 4;                             // [row][token] residual
constexpr int kMfmaLdsBytes = kMfmaRingBytes + kMfmaActBytes + kMfmaXsBytes + kMfmaTabBytes + kMfmaResBytes;
static_assert(kMfmaLdsBytes <= 160 * 1024, "fits the LDS of a CU");

__global__ __launch_bounds__(kMfmaThreads, 1) void k_qgemv_q8_0_mfma(
    const uint8_t* __restrict__ w, int N, int P, int64_t row_bytes,
    const int8_t* __restrict__ xq, int64_t K, const float* __restrict__ xd, int n_tok,
    const float* residual, float* y, int64_t ldy, int n_tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds_dyn[];
  uint8_t* ring = lds_dyn;
  uint8_t* s_act = lds_dyn + kMfmaRingBytes;
  float* s_xs = reinterpret_cast<float*>(s_act + kMfmaActBytes);
  float* s_tab = s_xs + kMfmaXsBytes / 4;
  float* s_res = s_tab + kMfmaTabBytes / 4;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar bounds
  const int col = lane & 15;
  const int kq = lane >> 4;
  const int C = (P + 63) / 64;
  const int nb = 2 * P;
  const int my_tiles = (int)blockIdx.x < n_tiles ? (n_tiles - 1 - (int)blockIdx.x) / (int)gridDim.x + 1 : 0;
  const int n_units = my_tiles * C;
  const int n_items = 2 * n_units;
  auto unit_tile = [&](int u) { return (int)blockIdx.x + (u / C) * (int)gridDim.x; };
  // DMA instructions this wave has issued: every wait below names how many of
  // them may still be outstanding, and only instructions that some lane
  // executes are counted
  int nv = 0;

  // byte offset of this lane's piece of DMA k within an item of a whole tile
  // (pieces as in issue_w below)
  uint32_t doff[kMfmaItemDmas];
#pragma unroll
  for (int k = 0; k < kMfmaItemDmas; ++k) {
    const int q = min(64 * k + lane, kMfmaItemPieces - 1);
    doff[k] = (uint32_t)(q / 17) * (uint32_t)row_bytes + 16u * (uint32_t)(q % 17);
  }
  // item m = half m % 2 of unit m / 2: rows 16T .. 16T+15 (past N: row N-1,
  // never stored), pairs 64c + 8 wave + 4 (m % 2) .. +3 (P % 4 == 0, so an
  // item is whole or past the end); DMA k moves pieces 64k + lane: row
  // piece / 17, bytes 16 (piece % 17) of the row's 272.  Returns the DMAs issued.
  auto issue_w = [&](int m) -> int {
    if (m >= n_items) return 0;
    const int u = m >> 1;
    const int c = u % C;
    const int T = unit_tile(u);
    const int p0 = 64 * c + 8 * wave + 4 * (m & 1);
    if (p0 >= P) return 0;
    uint8_t* slot = ring + (wave * 2 + (m & 1)) * kMfmaItemBytes;
    const int r0 = 16 * T;
    const uint8_t* base = w + (int64_t)r0 * row_bytes + (int64_t)p0 * kPairBytes;
    if (r0 + 16 <= N) {
#pragma unroll
      for (int k = 0; k < kMfmaItemDmas; ++k)
        if (64 * k + lane < kMfmaItemPieces)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(base + doff[k]), (lds_ptr)(slot + 1024 * k), 16, 0,
                                           kWeightCpol);
    } else {
      const int rmax = N - 1 - r0;  // last row of the tile in the matrix
#pragma unroll
      for (int k = 0; k < kMfmaItemDmas; ++k) {
        const int q = 64 * k + lane;
        if (q < kMfmaItemPieces)
          __builtin_amdgcn_global_load_lds(
              static_cast<const void*>(base + (int64_t)min(q / 17, rmax) * row_bytes + 16 * (q % 17)),
              (lds_ptr)(slot + 1024 * k), 16, 0, kWeightCpol);
      }
    }
    return kMfmaItemDmas;
  };
  // the activations of chunk c for this wave's 8 pairs (64c + 8 wave + p,
  // p < 8), in its own part of the stage: the codes of token t at 512 t, piece
  // q of pair p at 16 ((4p + q + t) % 32); the block scales of token t at
  // [16 t .. 16 t + 15] of its 256 floats.  Plain 16-byte loads of
  // contiguous runs of each token's row (tokens 2i and 2i + 1 per code load,
  // all 16 tokens' scales in one), stored to LDS; indices past n_tok or P read
  // valid rows whose values are never used.
  uint8_t* st_codes = s_act + 8192 * wave;
  float* st_scales = s_xs + 256 * wave;
  auto stage_act = [&](int c) {
    const int pw = 64 * c + 8 * wave;  // first pair of the wave in the chunk
    if (pw >= P) return;
    const int v = ((lane & 31) - (lane >> 5)) & 31;  // with t = 2i + lane / 32: (pos - t) % 32
    u32x4 cv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = min(2 * i + (lane >> 5), n_tok - 1);
      const int vv = (v - 2 * i) & 31;
      const int pr = vv >> 2, q = vv & 3;
      cv[i] = *reinterpret_cast<const u32x4*>(xq + (int64_t)t * K + 64 * (int64_t)min(pw + pr, P - 1) + 16 * q);
    }
    const int ts = min(lane >> 2, n_tok - 1);
    // (a wave with only 4 pairs left reads its last 16 blocks ending at the row's end)
    const u32x4 sv = *reinterpret_cast<const u32x4*>(xd + (int64_t)ts * nb + min(2 * pw + 4 * (lane & 3), nb - 4));
#pragma unroll
    for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(st_codes + 1024 * i + 16 * lane) = cv[i];
    *reinterpret_cast<u32x4*>(st_scales + 4 * lane) = sv;
  };

  int r_end = 0;
  int w_end[2] = {0, 0};
  // chunk 0's activations first (their loads are waited for at once; a load
  // issued behind the weights would wait for them), then both ring slots fill;
  // afterwards item m + 2 goes out as soon as item m's slot has been read
  if (n_units > 0) stage_act(0);
  nv += issue_w(0);
  w_end[0] = nv;
  nv += issue_w(1);
  w_end[1] = nv;

  long actA[8], actB[8];   // this lane's token: codes of the wave's pairs (k-group kq)
  float xa[8][4], xb[8][4];  // block scales of tokens 4kq .. 4kq+3
  float tot = 0.0f;          // threads < 256: running total of (row tid / 16, token tid % 16)
  for (int u = 0; u < n_units; ++u) {
    const int c = u % C;
    const int T = unit_tile(u);
    if (u == 0 || C > 1) {
      // this chunk's activations to registers: a wave reads back only the part
      // of the stage that it wrote itself, so no barrier is needed
      if (u > 0) stage_act(c);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int p = 8 * wave + j;
        const bool ok = col < n_tok && 64 * c + p < P;
        const uint32_t* e = reinterpret_cast<const uint32_t*>(st_codes + 512 * col) + kq;
        const uint32_t a0 = e[4 * ((4 * j + 0 + col) & 31)], a1 = e[4 * ((4 * j + 1 + col) & 31)];
        const uint32_t b0 = e[4 * ((4 * j + 2 + col) & 31)], b1 = e[4 * ((4 * j + 3 + col) & 31)];
        actA[j] = ok ? (long)(((uint64_t)a1 << 32) | a0) : 0;
        actB[j] = ok ? (long)(((uint64_t)b1 << 32) | b0) : 0;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool okr = 4 * kq + r < n_tok && 64 * c + p < P;
          const float2 ab = *reinterpret_cast<const float2*>(st_scales + 16 * (4 * kq + r) + 2 * j);
          xa[j][r] = okr ? ab.x : 0.0f;
          xb[j][r] = okr ? ab.y : 0.0f;
        }
      }
      // the reads are done before a later chunk's stores refill the stage
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    const bool last = c == C - 1;
    if (last && residual && wave < 4) {
      // the residual of the tile's outputs (row tid / 16, token tid % 16) to s_res[tid]
      const int row = tid >> 4, tok = tid & 15;
      if (16 * T + 4 * wave < N) {
        if (tok < n_tok && 16 * T + row < N)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(residual + (int64_t)tok * ldy + 16 * T + row),
                                           (lds_ptr)(s_res + 64 * wave), 4, 0, 0);
        ++nv;
      }
      r_end = nv;
    }

    float sub[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 2 * u + h;
      wait_vmcnt_wave(nv - w_end[m & 1]);
      float qs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if (64 * c + 8 * wave + 4 * h < P) {
        const uint8_t* slot = ring + (wave * 2 + (m & 1)) * kMfmaItemBytes + col * kMfmaRowBytes;
        // all reads of the item, then its eight MFMAs, then the cells
        uint32_t wd[4][8];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const uint32_t* rp = reinterpret_cast<const uint32_t*>(slot + kPairBytes * jj);
          const uint32_t* rk = rp + kq;
          wd[jj][0] = rk[0];
          wd[jj][1] = rk[1];
          wd[jj][2] = rk[4];
          wd[jj][3] = rk[5];
          wd[jj][4] = rk[9];
          wd[jj][5] = rk[13];
          wd[jj][6] = rp[0];
          wd[jj][7] = rp[8];
        }
        v4i DA[4], DB[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * h + jj;
          const uint32_t w0 = __builtin_amdgcn_alignbit(wd[jj][1], wd[jj][0], 16);
          const uint32_t w1 = __builtin_amdgcn_alignbit(wd[jj][3], wd[jj][2], 16);
          const long wa = (long)(((uint64_t)w1 << 32) | w0);
          const long wb = (long)(((uint64_t)wd[jj][5] << 32) | wd[jj][4]);
          const v4i zero = {0, 0, 0, 0};
          DA[jj] = __builtin_amdgcn_mfma_i32_16x16x32_i8(actA[j], wa, zero, 0, 0, 0);
          DB[jj] = __builtin_amdgcn_mfma_i32_16x16x32_i8(actB[j], wb, zero, 0, 0, 0);
        }
        float lf[4][4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int j = 4 * h + jj;
          const float dwA = f16_bits_to_f32(wd[jj][6]);
          const float dwB = f16_bits_to_f32(wd[jj][7] >> 16);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sA = fmul(fmul(dwA, xa[j][r]), (float)DA[jj][r]);
            const float sB = fmul(fmul(dwB, xb[j][r]), (float)DB[jj][r]);
            lf[jj][r] = fadd(fadd(0.0f, sA), sB);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) qs[r] = fadd(fadd(lf[0][r], lf[1][r]), fadd(lf[2][r], lf[3][r]));
      }
      // the slot's reads are done (their values are in the sums): refill it
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      nv += issue_w(m + 2);
      w_end[m & 1] = nv;
#pragma unroll
      for (int r = 0; r < 4; ++r) sub[r] = h == 0 ? qs[r] : fadd(sub[r], qs[r]);
    }

    // the wave subtrees of (row col, tokens 4kq .. 4kq+3), then the top levels
    float* tab = s_tab + (u & 1) * (kMfmaWaves * 256);
    *reinterpret_cast<f32x4*>(tab + (wave * 16 + col) * 16 + 4 * kq) = f32x4{sub[0], sub[1], sub[2], sub[3]};
    if (last && residual && wave < 4) wait_vmcnt_wave(nv - r_end);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tid < 256) {
      const float* tb = tab + tid;  // (row tid / 16, token tid % 16) of wave 0's table
      const float cs = fadd(fadd(fadd(tb[0], tb[256]), fadd(tb[512], tb[768])),
                            fadd(fadd(tb[1024], tb[1280]), fadd(tb[1536], tb[1792])));
      tot = c == 0 ? cs : fadd(tot, cs);
      if (last) {
        const int n = 16 * T + (tid >> 4);
        const int tok = tid & 15;
        if (n < N && tok < n_tok) y[(int64_t)tok * ldy + n] = residual ? fadd(s_res[tid], tot) : tot;
      }
    }
  }
}

// Raises a kernel's dynamic LDS limit to Bytes, once per kernel and process
// (thread-safe: concurrent first calls wait for the one that sets it).
template <auto Kern, int Bytes = kGemvLdsMax>
hipError_t raise_lds_once() {
  static std::once_flag once;
  static hipError_t err = hipSuccess;
  std::call_once(once, [] {
    err = hipFuncSetAttribute(reinterpret_cast<const void*>(Kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                              Bytes);
  });
  return err;
}

hipError_t launch_mfma(const GemvPlan& pl, const void* w, int64_t N, int64_t K, const int8_t* xq,
                       const float* xd, int n_tok, const float* residual, float* y, int64_t ldy,
                       hipStream_t st) {
  if (hipError_t e = raise_lds_once<&k_qgemv_q8_0_mfma, kMfmaLdsBytes>(); e != hipSuccess) return e;
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

size_t mfma_lds_bytes() { return (size_t)kMfmaLdsBytes; }

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
