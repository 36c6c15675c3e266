// glue.hip -- activation quantizer and the small per-token kernels of the step.
//
// The quantizer convention (fp32 d = amax/127, codes = roundf(x/d) clamped to
// +-127) is shared by every producer here, as "#1209 Speed up concurrent
// generation, fix QFUSE, and improve prefill monitoring" ("What changed and
// why", item 2) requires of a fused quantizer: it must reproduce the consuming
// quantizer's division and rounding exactly.  Blocks of 32 values map to 32
// consecutive lanes, so the block maximum is a 5-step lane reduction.
#include <math.h>

#include "device_math.hpp"
#include "internal.hpp"

namespace sd {

namespace {

// Quantizes one value per lane; lanes 32k..32k+31 hold one block.  Every lane
// of the wave must call this (the maximum uses cross-lane moves).
__device__ __forceinline__ void quantize_lane(float v, bool valid, int8_t* q_out, float* d_out,
                                              int lane32) {
  const float amax = group_max<32>(valid ? fabsf(v) : 0.0f);
  const float d = q8_scale(amax);
  if (valid) {
    *q_out = (int8_t)q8_code(v, d);
    if (lane32 == 0) *d_out = d;
  }
}

__global__ __launch_bounds__(256) void k_quantize_q8(const float* __restrict__ x, int64_t ldx,
                                                     int n_tok, int64_t K, int8_t* __restrict__ xq,
                                                     float* __restrict__ xd) {
  const int64_t nb = K / 32;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t blk = gid >> 5;
  const int lane32 = threadIdx.x & 31;
  const bool valid = blk < (int64_t)n_tok * nb;
  const int64_t t = valid ? blk / nb : 0;
  const int64_t b = valid ? blk - t * nb : 0;
  const float v = valid ? x[t * ldx + b * 32 + lane32] : 0.0f;
  quantize_lane(v, valid, xq + t * K + b * 32 + lane32, xd + t * nb + b, lane32);
}

// Workgroups of 1024 threads, EPT per token row (blockIdx.y = j): each holds
// the whole row in registers (EPT values per thread, element j*1024 + tid) for
// the sum of squares, which runs per thread in j order, then over the 64 lanes
// of a wave (fixed tree), then over the 16 waves in wave order; workgroup j
// then normalizes and quantizes elements j*1024 .. j*1024 + 1023 only.  Every
// workgroup of a row forms the same sum, so splitting the quantization (the
// costly part: a division per element) over EPT compute units changes no bits.
template <int EPT>
__global__ __launch_bounds__(1024) void k_rmsnorm_q8(const float* __restrict__ x, int64_t ldx,
                                                     int64_t D, const float* __restrict__ gamma,
                                                     float eps, int8_t* __restrict__ xq,
                                                     float* __restrict__ xd, float* y) {
  __shared__ float part[16];
  const int t = blockIdx.x;
  const int js = blockIdx.y;  // the slice this workgroup quantizes
  const int tid = threadIdx.x;
  const float* xr = x + (int64_t)t * ldx;
  const int64_t is = (int64_t)js * 1024 + tid;
  const float gs = is < D ? gamma[is] : 0.0f;
  float v[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int64_t i = (int64_t)j * 1024 + tid;
    v[j] = i < D ? xr[i] : 0.0f;
  }
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < EPT; ++j) ss = fadd(ss, fmul(v[j], v[j]));
  ss = wave_sum_fixed(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  float total = part[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) total = fadd(total, part[w]);
  const float r = fdiv(1.0f, sqrtf(fadd(fdiv(total, (float)D), eps)));
  const int64_t nb = D / 32;
  if ((int64_t)js * 1024 >= D) return;  // uniform: D is a multiple of 32, blocks stay whole
  float vs = v[0];
#pragma unroll
  for (int j = 1; j < EPT; ++j)
    if (j == js) vs = v[j];
  const bool valid = is < D;
  const float o = valid ? fmul(fmul(vs, r), gs) : 0.0f;
  if (valid && y) y[(int64_t)t * D + is] = o;
  quantize_lane(o, valid, xq + (int64_t)t * D + is, xd + (int64_t)t * nb + (is >> 5), tid & 31);
}

__global__ __launch_bounds__(256) void k_swiglu_q8(const float* __restrict__ gu, int64_t ldgu,
                                                   int n_tok, int64_t F, int8_t* __restrict__ xq,
                                                   float* __restrict__ xd, float* y) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const bool valid = gid < (int64_t)n_tok * F;
  const int64_t t = valid ? gid / F : 0;
  const int64_t i = valid ? gid - t * F : 0;
  float m = 0.0f;
  if (valid) {
    const float g = gu[t * ldgu + i];
    const float u = gu[t * ldgu + F + i];
    const float silu = fdiv(g, fadd(1.0f, expf(-g)));
    m = fmul(silu, u);
    if (y) y[t * F + i] = m;
  }
  quantize_lane(m, valid, xq + t * F + i, xd + t * (F / 32) + (i >> 5), threadIdx.x & 31);
}

__global__ __launch_bounds__(256) void k_embed(const uint16_t* __restrict__ table, int64_t V,
                                               int64_t H, const int32_t* __restrict__ tokens,
                                               float* __restrict__ x) {
  const int t = blockIdx.y;
  int64_t tok = tokens[t];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < H; i += (int64_t)gridDim.x * 256)
    x[(int64_t)t * H + i] = f16_bits_to_f32(table[tok * H + i]);
}

// (value, index) selection: larger value wins, equal values go to the lower
// index, NaN never wins.  It is a total order on candidates, so any reduction
// tree gives the same winner.
__device__ __forceinline__ void better(float& v, int32_t& i, float ov, int32_t oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

// Pass 1: workgroup (t, slice) takes kArgSlice logits of row t; every thread
// issues all its loads first, then selects; the workgroup's winner goes to ws.
constexpr int kArgSlice = 8192;

__device__ __forceinline__ void block_best(float& bv, int32_t& bi, float* sv, int32_t* si) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int32_t oi = __shfl_xor(bi, m, 64);
    better(bv, bi, ov, oi);
  }
  if ((threadIdx.x & 63) == 0) {
    sv[threadIdx.x >> 6] = bv;
    si[threadIdx.x >> 6] = bi;
  }
  __syncthreads();
  bv = sv[0];
  bi = si[0];
  for (int w = 1; w < 4; ++w) better(bv, bi, sv[w], si[w]);
}

__global__ __launch_bounds__(256) void k_argmax_slices(const float* __restrict__ logits, int64_t ld,
                                                       int64_t V, float* __restrict__ wv,
                                                       int32_t* __restrict__ wi) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  const int t = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kArgSlice;
  const float* row = logits + (int64_t)t * ld;
  constexpr int PER = kArgSlice / 256;  // 32 values per thread
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t i = base + (int64_t)j * 256 + threadIdx.x;
    v[j] = i < V ? row[i] : -INFINITY;
  }
  float bv = -INFINITY;
  int32_t bi = (int32_t)V;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t i = base + (int64_t)j * 256 + threadIdx.x;
    if (i < V) better(bv, bi, v[j], (int32_t)i);
  }
  block_best(bv, bi, sv, si);
  if (threadIdx.x == 0) {
    wv[(int64_t)t * gridDim.x + blockIdx.x] = bv;
    wi[(int64_t)t * gridDim.x + blockIdx.x] = bi;
  }
}

// Pass 2: one workgroup per row reduces the slice winners.
__global__ __launch_bounds__(256) void k_argmax_final(const float* __restrict__ wv,
                                                      const int32_t* __restrict__ wi, int n_slices,
                                                      int64_t V, int32_t* __restrict__ out) {
  __shared__ float sv[4];
  __shared__ int32_t si[4];
  const int t = blockIdx.x;
  float bv = -INFINITY;
  int32_t bi = (int32_t)V;
  for (int j = threadIdx.x; j < n_slices; j += 256)
    better(bv, bi, wv[(int64_t)t * n_slices + j], wi[(int64_t)t * n_slices + j]);
  block_best(bv, bi, sv, si);
  if (threadIdx.x == 0) out[t] = bi >= V ? 0 : bi;
}

}  // namespace

hipError_t launch_quantize_q8(const float* x, int64_t ldx, int n_tok, int64_t K, int8_t* xq,
                              float* xd, hipStream_t st) {
  const int64_t threads = (int64_t)n_tok * K;  // one lane per value
  const int64_t grid = (threads + 255) / 256;
  hipLaunchKernelGGL(k_quantize_q8, dim3((unsigned)grid), dim3(256), 0, st, x, ldx, n_tok, K, xq, xd);
  return hipGetLastError();
}

hipError_t launch_rmsnorm_q8(const float* x, int64_t ldx, int n_tok, int64_t D, const float* gamma,
                             float eps, int8_t* xq, float* xd, float* y, hipStream_t st) {
  if (D <= 4096)
    hipLaunchKernelGGL(k_rmsnorm_q8<4>, dim3(n_tok, 4), dim3(1024), 0, st, x, ldx, D, gamma, eps, xq, xd, y);
  else if (D <= 8192)
    hipLaunchKernelGGL(k_rmsnorm_q8<8>, dim3(n_tok, 8), dim3(1024), 0, st, x, ldx, D, gamma, eps, xq, xd, y);
  else if (D <= 16384)
    hipLaunchKernelGGL(k_rmsnorm_q8<16>, dim3(n_tok, 16), dim3(1024), 0, st, x, ldx, D, gamma, eps, xq, xd, y);
  else
    hipLaunchKernelGGL(k_rmsnorm_q8<32>, dim3(n_tok, 32), dim3(1024), 0, st, x, ldx, D, gamma, eps, xq, xd, y);
  return hipGetLastError();
}

hipError_t launch_swiglu_q8(const float* gu, int64_t ldgu, int n_tok, int64_t F, int8_t* xq,
                            float* xd, float* y, hipStream_t st) {
  const int64_t grid = ((int64_t)n_tok * F + 255) / 256;
  hipLaunchKernelGGL(k_swiglu_q8, dim3((unsigned)grid), dim3(256), 0, st, gu, ldgu, n_tok, F, xq, xd, y);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t* table, int64_t V, int64_t H, const int32_t* tokens, int n_tok,
                        float* x, hipStream_t st) {
  const int64_t gx = (H + 255) / 256 < 64 ? (H + 255) / 256 : 64;
  hipLaunchKernelGGL(k_embed, dim3((unsigned)gx, n_tok), dim3(256), 0, st, table, V, H, tokens, x);
  return hipGetLastError();
}

size_t argmax_ws_bytes(int n_tok, int64_t V) {
  const int64_t slices = (V + kArgSlice - 1) / kArgSlice;
  return (size_t)n_tok * slices * 8;
}

hipError_t launch_argmax(const float* logits, int64_t ld, int n_tok, int64_t V, int32_t* out,
                         void* ws, hipStream_t st) {
  const int64_t slices = (V + kArgSlice - 1) / kArgSlice;
  float* wv = static_cast<float*>(ws);
  int32_t* wi = reinterpret_cast<int32_t*>(wv + (int64_t)n_tok * slices);
  hipLaunchKernelGGL(k_argmax_slices, dim3((unsigned)slices, n_tok), dim3(256), 0, st, logits, ld, V,
                     wv, wi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_argmax_final, dim3(n_tok), dim3(256), 0, st, wv, wi, (int)slices, V, out);
  return hipGetLastError();
}

namespace {

// ---------------------------------------------------------------------------
// Plain streaming read: every 16-byte word of the buffer loaded once
// (non-temporal, as the GEMV streams its weights), folded by XOR into a
// register that is stored only if it equals a value no real buffer gives, so
// the loads cannot be dropped.  Eight words in flight per thread; workgroups
// take contiguous 64 KiB tiles in grid-stride order.  The achievable-bandwidth
// reference for the kernels above; not part of the decode step.
constexpr int kReadTile = 65536;

__global__ __launch_bounds__(256) void k_stream_read(const u32x4a* __restrict__ buf, int64_t words,
                                                     uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t tile_words = kReadTile / 16;
  for (int64_t t0 = (int64_t)blockIdx.x * tile_words; t0 < words; t0 += (int64_t)gridDim.x * tile_words) {
    const int64_t end = t0 + tile_words < words ? t0 + tile_words : words;
    for (int64_t i = t0 + threadIdx.x; i < end; i += 8 * 256) {
      u32x4a v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t k = i + (int64_t)u * 256;
        v[u] = k < end ? __builtin_nontemporal_load(buf + k) : u32x4a{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (acc == 0x9E3779B9u && threadIdx.x == 0) sink[blockIdx.x & 63] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st) {
  const int64_t words = (int64_t)(bytes / 16);
  const int64_t tiles = (int64_t)((bytes + kReadTile - 1) / kReadTile);
  const int64_t grid = tiles < 2048 ? (tiles > 0 ? tiles : 1) : 2048;  // at most 8 workgroups per CU
  hipLaunchKernelGGL(k_stream_read, dim3((unsigned)grid), dim3(256), 0, st, static_cast<const u32x4a*>(buf),
                     words, sink);
  return hipGetLastError();
}

}  // namespace sd
