// internal.hpp -- declarations shared by the HIP kernels and the C-ABI layer.
// Not part of the public interface (include/seqdecode.h is).
#pragma once

#include <math.h>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_math.hpp"
#include "seqdecode.h"

namespace sd {

// ---------------------------------------------------------------- constants
constexpr int kBlock = 32;          // weights / codes per q8 block
constexpr int kBlockBytes = 34;     // fp16 scale + 32 int8
constexpr int kPairBytes = 68;      // two consecutive blocks; a pair starts 4-byte aligned
constexpr int kPairDw = 17;         // dwords per pair
constexpr int kActDw = 20;          // dwords per pair in the LDS activation layout
constexpr int kGemvThreads = 256;   // four wave64 per workgroup
constexpr int kGemvLdsMax = 144 * 1024;
constexpr int kAttnChunk = SD_ATTN_CHUNK;
constexpr int kAttnSmallChunk = SD_ATTN_SMALL_CHUNK;
constexpr int kAttnSmallSpan = SD_ATTN_SMALL_SPAN;
constexpr int kAttnSmallChunks = kAttnSmallSpan / kAttnSmallChunk;
static_assert(kAttnSmallSpan % kAttnChunk == 0 && kAttnChunk % kAttnSmallChunk == 0, "chunk grid");
constexpr int kAttnHeadDim = 128;
constexpr int kAttnGroup = 4;       // query heads per KV head handled by one workgroup
constexpr int kAttnPartialFloats = 132;  // m, l, 2 pad, o[128]
constexpr int kAttnMaxNew = 4;           // query tokens per sequence in one attention call
constexpr size_t kAttnScratchBytes = SD_ATTN_SCRATCH_BYTES;  // allocation-free attention partials

// Attention chunk grid, fixed in absolute positions: chunk c < kAttnSmallChunks
// holds positions 64c .. 64c+63, later chunks hold 256 positions each from
// kAttnSmallSpan on.  A key's chunk depends on its position alone.
__host__ __device__ constexpr int attn_chunk_of(int j) {
  return j < kAttnSmallSpan ? j / kAttnSmallChunk : kAttnSmallChunks + (j - kAttnSmallSpan) / kAttnChunk;
}
__host__ __device__ constexpr int attn_chunk_begin(int c) {
  return c < kAttnSmallChunks ? c * kAttnSmallChunk : kAttnSmallSpan + (c - kAttnSmallChunks) * kAttnChunk;
}
__host__ __device__ constexpr int attn_chunk_size(int c) {
  return c < kAttnSmallChunks ? kAttnSmallChunk : kAttnChunk;
}
// Chunks that keys lo..hi touch.
__host__ __device__ constexpr int attn_chunks(int lo, int hi) { return attn_chunk_of(hi) - attn_chunk_of(lo) + 1; }
// Most chunks any span of at most SD_MAX_CTX keys touches: the span from 0 has
// the most (chunks are densest at low positions), plus one for a span that
// starts inside a chunk.
constexpr int kAttnMaxChunks = attn_chunks(0, SD_MAX_CTX - 1) + 1;
// Up to this many (64-key chunk, KV head) units in a call, one per workgroup.
constexpr int kAttnSpreadUnits = 320;

// Per-sequence view as passed by value to the attention / append kernels.
struct SeqArg {
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* k_w;
  uint16_t* v_w;
  int64_t ld_tok;
  int64_t ld_head;
  int32_t ctx_len;
  int32_t n_chunks;       // chunks c0 .. c0 + n_chunks - 1 (partials per token and head)
  int32_t ns;             // of them on the 64-key grid (the first ns)
  int32_t pk;             // 64-key chunks per workgroup: 1 or 4
  int32_t large_begin;    // first workgroup of its 256-key units
  int32_t small_begin;    // first workgroup of its 64-key units
  int32_t partial_begin;  // first partial slot of this sequence (per token and head: n_chunks slots)
  int32_t n_new;          // query tokens of the sequence (the newest n_new positions), 1..4
  int32_t row0;           // q / out row of its first query token
  int32_t window;         // attention window in positions, 0 = whole context
  int32_t ring_cap;       // ring of ring_cap rows (position j in row j % ring_cap), 0 = plain
  int32_t lo0;            // lowest position any query token of the call attends to
  int32_t c0;             // chunk (absolute, attn_chunk_of(lo0)) of the first work unit
  const int32_t* btab;    // paged cache: block table (device), else null
  int32_t bshift;         // log2 of the block size (paged)
  int32_t n_blocks;       // blocks in the pool (paged)
  int32_t q8;             // 1: quantized caches (codes kq / vq, fp16 scales kd / vd at offsets / 32)
  int32_t k4;             // with q8: 1 when K is q4_0 (nibble pairs at offsets / 2), 0 for q8_0
  int32_t v4;             // the same for V
  int8_t* kq;
  int8_t* vq;
  uint16_t* kd;
  uint16_t* vd;
};

// Cache row of position j (device): plain, ring or paged.
__device__ inline int64_t seq_row(const SeqArg& a, int64_t j) {
  if (a.btab) {
    int b = a.btab[j >> a.bshift];
    b = b < 0 ? 0 : (b >= a.n_blocks ? a.n_blocks - 1 : b);
    return ((int64_t)b << a.bshift) + (j & ((1 << a.bshift) - 1));
  }
  return a.ring_cap ? j % a.ring_cap : j;
}

struct SeqArgs {
  SeqArg s[SD_MAX_SEQS];
  int32_t n_seq;
  int32_t large_total;  // workgroups holding 256-key units (they come first)
  int32_t units_total;  // all workgroups of the chunk kernel
  int32_t hpw;          // query heads per head group (a workgroup's columns): 1..4
  int32_t vg;           // head groups per KV head (H_q / H_kv / hpw)
};

// Angle pos * theta^(-2i/n_rot) of RoPE pair i, its cosine and sine in fp64,
// rounded to fp32 (every RoPE kernel takes its angles from here).
__device__ inline void rope_angle(int pos, int i, int n_rot, double theta, float* c, float* s) {
  const double inv_freq = pow(theta, (double)(-2 * i) / (double)n_rot);
  const double a = (double)pos * inv_freq;
  double sn, cs;
  sincos(a, &sn, &cs);
  *c = (float)cs;
  *s = (float)sn;
}

// The rotation of one pair: four fp32 products and two sums, unfused.
__device__ inline void rope_rotate(float x0, float x1, float c, float s, float* y0, float* y1) {
  *y0 = fsub(fmul(x0, c), fmul(x1, s));
  *y1 = fadd(fmul(x0, s), fmul(x1, c));
}

// QKV projection with RoPE and the fp16 KV write in its epilogue (the step's
// fp16 caches, heads of 128 dims rotated whole).  tab_mode as in
// launch_rope_kv_step: 1 computes the angles and keeps them in cs_tab
// ([row][pair] (cos, sin)), 2 reads them from there.
struct RopeArgs {
  const int32_t* pos;
  double theta;
  float* cs_tab;
  int32_t tab_mode;
  int32_t n_heads;
  int32_t n_kv;
  SeqArgs seqs;
};

// Input of a projection given as the q8 blocks of rmsnorm(x [n][ldx], gamma,
// eps) (the RMSNorm that precedes the QKV, gate|up and output projections of
// the step), computed by the projection's own workgroups with the arithmetic
// of launch_rmsnorm_q8: the same codes and scales.
struct RmsArgs {
  const float* x;
  int64_t ldx;
  const float* gamma;
  float eps;
};

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments are already validated.
hipError_t launch_quantize_q8(const float* x, int64_t ldx, int n_tok, int64_t K,
                              int8_t* xq, float* xd, hipStream_t st);

// GEMV launch geometry for (N, K, n_tok): lds bytes and slice layout.
struct GemvPlan {
  int pairs;         // K / 64
  int chunks;        // pairs / 64 rounded up: the unit of the fixed reduction order
  bool mfma;         // matrix-core kernel (tiles of 16 rows)
  bool use_reg;      // activations held in registers (1..8 tokens, <= 4 chunks)
  int sp;            // waves per row in the register kernel (1, 2 or 4)
  bool stage;        // register kernel: activations staged once per workgroup in LDS
  int nw;            // register kernel: waves per workgroup (8 staged, else 4)
  int slice_pairs;   // pairs staged per LDS slice (multiple of 64, or all)
  int n_slices;
  size_t lds_bytes;
  int rows_per_wave;
  int n_blocks;      // row blocks of rows_per_wave rows (MFMA kernel: 16-row tiles)
  int grid;
};
// path: SD_GEMV_AUTO, SD_GEMV_NARROW or SD_GEMV_MFMA; every path gives the same bits.
bool plan_qgemv(int64_t N, int64_t K, int n_tok, int path, GemvPlan* plan);
hipError_t launch_qgemv(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                        int n_tok, const float* residual, float* y, int64_t ldy, hipStream_t st,
                        int path = SD_GEMV_AUTO);
// gate|up projection fused with SwiGLU + q8 quantization (see qgemv.hip)
bool swiglu_fusable(int64_t F, int64_t K, int n_tok);
hipError_t launch_qgemv_swiglu(const void* w, int64_t F, int64_t K, const int8_t* xq, const float* xd,
                               int n_tok, int8_t* oq, float* od, hipStream_t st,
                               const RmsArgs* rms = nullptr);
// Whether a staged one-chunk projection takes its input as an RMS prologue
// (K <= 4096, one row): rms != nullptr on the fused launchers replaces xq /
// xd by the q8 blocks of rmsnorm(rms->x).
bool rms_fusable(int64_t K, int n_tok);
hipError_t launch_qgemv_rms(const void* w, int64_t N, int64_t K, const RmsArgs& rms, int n_tok, float* y,
                            int64_t ldy, hipStream_t st);
// QKV projection (N = (n_heads + 2 n_kv) * 128 rows) with RoPE of q and k and
// the fp16 K/V cache write in the same launch: the q rows of y and the cache
// rows get exactly what launch_rope_kv_step makes of the plain projection's
// outputs; the k and v rows of y stay unrotated, as there.
bool qkv_rope_fusable(int64_t N, int64_t K, int n_tok);
hipError_t launch_qgemv_qkv_rope(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                                 int n_tok, float* y, int64_t ldy, const RopeArgs& ra, hipStream_t st,
                                 const RmsArgs* rms = nullptr);

hipError_t launch_rope_posvec(float* x, int n_tok, int n_heads, int head_dim, int64_t ld_tok,
                              int64_t ld_head, const int32_t* pos, double theta, int n_rot,
                              hipStream_t st);
hipError_t launch_kv_append(const float* k_new, const float* v_new, int64_t ld_new,
                            const SeqArgs& seqs, int H_kv, int D, hipStream_t st);
// Fused step helper: rotates q (n_heads) and k (n_kv) rows of qkv in place and
// writes rotated k and v into the cache: row t is token t - row0 of its
// sequence, at position ctx_len - n_new + (t - row0) (row0 set); the last
// n_rot dims of each head rotate.
hipError_t launch_rope_kv_step(float* qkv, int64_t ld_qkv, int rows, int n_heads, int n_kv,
                               int head_dim, int n_rot, const int32_t* pos, double theta,
                               const SeqArgs& seqs, float* cs_tab, int tab_mode, hipStream_t st);

// Fills per-sequence chunk bookkeeping (n_new must be set); returns workspace
// floats needed.
size_t attn_layout(SeqArgs* seqs, int H_q, int H_kv);
hipError_t launch_attn(const float* q, int64_t ld_q, const SeqArgs& seqs, int H_q, int H_kv,
                       float scale, float* out, float* partials, int8_t* oq, float* od,
                       hipStream_t st);
// Device address, on the current device, of the attention scratch array
// (kAttnScratchBytes) used by the allocation-free attention entry point.
hipError_t attn_scratch(float** ptr);

hipError_t launch_rmsnorm_q8(const float* x, int64_t ldx, int n_tok, int64_t D,
                             const float* gamma, float eps, int8_t* xq, float* xd, float* y,
                             hipStream_t st);
hipError_t launch_swiglu_q8(const float* gu, int64_t ldgu, int n_tok, int64_t F, int8_t* xq,
                            float* xd, float* y, hipStream_t st);
hipError_t launch_embed(const uint16_t* table, int64_t V, int64_t H, const int32_t* tokens,
                        int n_tok, float* x, hipStream_t st);
// Plain streaming read of bytes (a multiple of 16) from a 16-byte aligned
// buffer: the achievable-bandwidth reference; sink gets 64 words at most.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);
size_t argmax_ws_bytes(int n_tok, int64_t V);
hipError_t launch_argmax(const float* logits, int64_t ld, int n_tok, int64_t V, int32_t* out,
                         void* ws, hipStream_t st);

}  // namespace sd
