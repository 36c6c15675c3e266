// abi.cpp -- the C entry points of include/seqdecode.h.
//
// Each entry point validates its arguments on the host first (no HIP call is
// made on a rejected call, so the checks also run where no GPU is present),
// then enqueues the kernels on the caller's stream.  Rejections that the pages
// insist on: more than four sequences are refused ("feat(qwen4exp): exact
// 4-slot concurrent serving", "What"), and an unsupported shape is an explicit
// error rather than a silent fallback ("#1209 Speed up concurrent generation,
// fix QFUSE, and improve prefill monitoring", "Performance": a missing native
// type surfaced as an error).
#include <math.h>

#include <algorithm>

#include "internal.hpp"

using namespace sd;

namespace {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline int from_hip(hipError_t e) { return e == hipSuccess ? SD_OK : SD_EHIP; }

inline hipStream_t hs(sd_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

int check_gemv(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd, int n_tok,
               float* y, int64_t ldy, int path = SD_GEMV_AUTO) {
  if (!w || !xq || !xd || !y) return SD_EINVAL;
  if (N < 1 || N > ((int64_t)1 << 30) || K < 1 || n_tok < 1 || n_tok > SD_MAX_TOKENS || ldy < N)
    return SD_EINVAL;
  if (K % 256 != 0 || K > ((int64_t)1 << 24)) return SD_EUNSUPPORTED;
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(y, 4)) return SD_EALIGN;
  if (path != SD_GEMV_AUTO && path != SD_GEMV_NARROW && path != SD_GEMV_MFMA) return SD_EINVAL;
  GemvPlan pl;
  if (!plan_qgemv(N, K, n_tok, path, &pl)) return SD_EUNSUPPORTED;
  return SD_OK;
}

// kv_type: the element type every view must have, -1 (attention: any, but
// the same for all views of the call) or kAnyQuant (any quantized type, the
// same for all views).
constexpr int kAnyQuant = -2;
bool is_kv_type(int t) { return t >= SD_KV_F16 && t <= SD_KV_Q8_Q4; }
bool k_is_q4(int t) { return t == SD_KV_Q4_0 || t == SD_KV_Q4_Q8; }
bool v_is_q4(int t) { return t == SD_KV_Q4_0 || t == SD_KV_Q8_Q4; }

int check_views(const sd_seqview* views, int n_seq, int D, bool attn,
                const int32_t* n_new = nullptr, int kv_type = -1) {
  if (!views || n_seq < 1 || n_seq > SD_MAX_SEQS) return SD_EINVAL;
  for (int s = 0; s < n_seq; ++s) {
    const sd_seqview& v = views[s];
    if (!is_kv_type(v.kv_type)) return SD_EINVAL;
    if (kv_type >= 0 && v.kv_type != kv_type) return SD_EINVAL;
    if (kv_type == kAnyQuant && v.kv_type == SD_KV_F16) return SD_EINVAL;
    if (v.kv_type != views[0].kv_type) return SD_EUNSUPPORTED;
    if (v.kv_type == SD_KV_F16) {
      if (!v.k || !v.v) return SD_EINVAL;
    } else {
      // q8_0 / q4_0: codes and scales, whole 32-dim blocks
      if (!v.k_q8 || !v.v_q8 || !v.k_d || !v.v_d) return SD_EINVAL;
      if (D % 32 != 0) return SD_EINVAL;
      const int64_t m = attn ? 128 : 32;
      if (v.ld_tok % m != 0 || v.ld_head % m != 0) return SD_EALIGN;
      if (attn && (!aligned(v.k_q8, 16) || !aligned(v.v_q8, 16) || !aligned(v.k_d, 8) ||
                   !aligned(v.v_d, 8)))
        return SD_EALIGN;
      if (!aligned(v.k_d, 2) || !aligned(v.v_d, 2)) return SD_EALIGN;
    }
    if (v.capacity < 1 || v.ctx_len < 1) return SD_EINVAL;
    if (v.window < 0 || (v.ring != 0 && v.ring != 1)) return SD_EINVAL;
    const int T = n_new ? n_new[s] : 1;
    if (T < 1 || T > SD_ATTN_MAX_NEW || T > v.ctx_len) return SD_EINVAL;
    if (v.block_table) {
      // paged: blocks of 64, 128 or 256 rows, whole blocks in the pool
      if (v.ring) return SD_EINVAL;
      if (v.block_size != 64 && v.block_size != 128 && v.block_size != 256) return SD_EINVAL;
      if (v.capacity % v.block_size != 0) return SD_EINVAL;
      if (!aligned(v.block_table, 4)) return SD_EALIGN;
    } else if (v.ring) {
      // every position still attended to must have its own row
      if (v.window < 1) return SD_EINVAL;
      const int64_t span = v.ctx_len < (int64_t)v.window + T - 1 ? v.ctx_len : (int64_t)v.window + T - 1;
      if (span > v.capacity) return SD_EINVAL;
    } else if (v.ctx_len > v.capacity) {
      return SD_EINVAL;
    }
    if (attn) {
      // every token's keys span at most SD_MAX_CTX positions (the newest
      // token's span is the longest)
      const int span = v.window ? std::min(v.ctx_len, v.window) : v.ctx_len;
      if (span > SD_MAX_CTX) return SD_EUNSUPPORTED;
    }
    if (v.ld_head < D || v.ld_tok < D) return SD_EINVAL;
    if (v.kv_type == SD_KV_F16) {
      const size_t al = attn ? 16 : 4;
      if (!aligned(v.k, al) || !aligned(v.v, al)) return SD_EALIGN;
      if (attn && (v.ld_tok % 8 != 0 || v.ld_head % 8 != 0)) return SD_EALIGN;
      if (!attn && (v.ld_tok % 2 != 0 || v.ld_head % 2 != 0)) return SD_EALIGN;
    }
  }
  return SD_OK;
}

void fill_seqargs(const sd_seqview* views, int n_seq, SeqArgs* a, const int32_t* n_new = nullptr) {
  *a = SeqArgs{};
  a->n_seq = n_seq;
  for (int s = 0; s < n_seq; ++s) {
    SeqArg& x = a->s[s];
    x.k = views[s].k;
    x.v = views[s].v;
    x.k_w = views[s].k;
    x.v_w = views[s].v;
    x.ld_tok = views[s].ld_tok;
    x.ld_head = views[s].ld_head;
    x.ctx_len = views[s].ctx_len;
    x.n_new = n_new ? n_new[s] : 1;
    x.window = views[s].window;
    x.ring_cap = views[s].ring ? views[s].capacity : 0;
    if (views[s].kv_type != SD_KV_F16) {
      x.q8 = 1;
      x.k4 = k_is_q4(views[s].kv_type);
      x.v4 = v_is_q4(views[s].kv_type);
      x.kq = views[s].k_q8;
      x.vq = views[s].v_q8;
      x.kd = views[s].k_d;
      x.vd = views[s].v_d;
    }
    if (views[s].block_table) {
      x.btab = views[s].block_table;
      x.bshift = __builtin_ctz((unsigned)views[s].block_size);
      x.n_blocks = views[s].capacity / views[s].block_size;
    }
  }
}

// n_new [host]: query tokens per sequence, 1..SD_ATTN_MAX_NEW and <= ctx_len


int attn_common(const float* q, int64_t ld_q, const sd_seqview* views, const int32_t* n_new,
                int n_seq, int H_q, int H_kv, int D, float scale, float* out, void* ws,
                size_t ws_bytes, sd_stream_t stream) {
  if (!q || !out || !ws || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return SD_EINVAL;
  if (D != kAttnHeadDim) return SD_EUNSUPPORTED;
  if (ld_q < (int64_t)H_q * D || !isfinite(scale)) return SD_EINVAL;
  int rc = check_views(views, n_seq, D, true, n_new);
  if (rc != SD_OK) return rc;
  if (!aligned(q, 16) || ld_q % 4 != 0 || !aligned(out, 16) || !aligned(ws, 16)) return SD_EALIGN;
  SeqArgs a;
  fill_seqargs(views, n_seq, &a, n_new);
  const size_t need = attn_layout(&a, H_q, H_kv) * sizeof(float);
  if (ws_bytes < need) return SD_EWORKSPACE;
  return from_hip(launch_attn(q, ld_q, a, H_q, H_kv, scale, out, static_cast<float*>(ws), nullptr,
                              nullptr, hs(stream)));
}

}  // namespace

extern "C" {

const char* sd_status_string(int status) {
  switch (status) {
    case SD_OK: return "SD_OK";
    case SD_EINVAL: return "SD_EINVAL: invalid argument";
    case SD_EUNSUPPORTED: return "SD_EUNSUPPORTED: shape not supported";
    case SD_EALIGN: return "SD_EALIGN: misaligned pointer or stride";
    case SD_EWORKSPACE: return "SD_EWORKSPACE: workspace too small";
    case SD_EHIP: return "SD_EHIP: HIP runtime error";
    default: return "unknown sd_status";
  }
}

int sd_abi_version(void) { return SD_ABI_VERSION; }

int sd_quantize_q8_act(const float* x, int64_t ldx, int n_tok, int64_t K, int8_t* xq, float* xd,
                       sd_stream_t stream) {
  if (!x || !xq || !xd || n_tok < 1 || n_tok > SD_MAX_TOKENS || K < 32 || ldx < K) return SD_EINVAL;
  if (K % 32 != 0 || K > ((int64_t)1 << 24)) return SD_EUNSUPPORTED;
  if (!aligned(x, 4) || !aligned(xq, 16) || !aligned(xd, 4)) return SD_EALIGN;
  return from_hip(launch_quantize_q8(x, ldx, n_tok, K, xq, xd, hs(stream)));
}

int sd_qgemv_q8_0_batch(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                        int n_tok, const float* residual, float* y, int64_t ldy,
                        sd_stream_t stream) {
  int rc = check_gemv(w, N, K, xq, xd, n_tok, y, ldy);
  if (rc != SD_OK) return rc;
  if (residual && !aligned(residual, 4)) return SD_EALIGN;
  return from_hip(launch_qgemv(w, N, K, xq, xd, n_tok, residual, y, ldy, hs(stream)));
}

int sd_qgemv_q8_0_batch_path(const void* w, int64_t N, int64_t K, const int8_t* xq, const float* xd,
                             int n_tok, const float* residual, float* y, int64_t ldy, int path,
                             sd_stream_t stream) {
  int rc = check_gemv(w, N, K, xq, xd, n_tok, y, ldy, path);
  if (rc != SD_OK) return rc;
  if (residual && !aligned(residual, 4)) return SD_EALIGN;
  return from_hip(launch_qgemv(w, N, K, xq, xd, n_tok, residual, y, ldy, hs(stream), path));
}

int sd_rope_posvec(float* x, int n_tok, int n_heads, int head_dim, int64_t ld_tok, int64_t ld_head,
                   const int32_t* pos, double theta, int n_rot, sd_stream_t stream) {
  if (!x || !pos || n_tok < 1 || n_tok > 4096 || n_heads < 1 || n_heads > 4096) return SD_EINVAL;
  if (head_dim < 2 || head_dim > 512 || n_rot < 2 || n_rot > head_dim || n_rot % 2 != 0)
    return SD_EINVAL;
  if (!(theta > 0.0) || !isfinite(theta)) return SD_EINVAL;
  if (ld_head < head_dim || ld_tok < head_dim) return SD_EINVAL;
  if (!aligned(x, 4) || !aligned(pos, 4)) return SD_EALIGN;
  return from_hip(launch_rope_posvec(x, n_tok, n_heads, head_dim, ld_tok, ld_head, pos, theta,
                                     n_rot, hs(stream)));
}

int sd_kv_append_q8_0(const float* k_new, const float* v_new, int64_t ld_new,
                      const sd_seqview* views, int n_seq, int H_kv, int D, sd_stream_t stream) {
  if (!k_new || !v_new || H_kv < 1 || D < 32 || D > 4096 || D % 32 != 0) return SD_EINVAL;
  if (ld_new < (int64_t)H_kv * D) return SD_EINVAL;
  int rc = check_views(views, n_seq, D, false, nullptr, kAnyQuant);
  if (rc != SD_OK) return rc;
  if (!aligned(k_new, 4) || !aligned(v_new, 4)) return SD_EALIGN;
  SeqArgs a;
  fill_seqargs(views, n_seq, &a);
  return from_hip(launch_kv_append(k_new, v_new, ld_new, a, H_kv, D, hs(stream)));
}

int sd_kv_append_f16(const float* k_new, const float* v_new, int64_t ld_new,
                     const sd_seqview* views, int n_seq, int H_kv, int D, sd_stream_t stream) {
  if (!k_new || !v_new || H_kv < 1 || D < 2 || D > 4096 || D % 2 != 0) return SD_EINVAL;
  if (ld_new < (int64_t)H_kv * D) return SD_EINVAL;
  int rc = check_views(views, n_seq, D, false, nullptr, SD_KV_F16);
  if (rc != SD_OK) return rc;
  if (!aligned(k_new, 4) || !aligned(v_new, 4)) return SD_EALIGN;
  SeqArgs a;
  fill_seqargs(views, n_seq, &a);
  return from_hip(launch_kv_append(k_new, v_new, ld_new, a, H_kv, D, hs(stream)));
}

size_t sd_decode_attn_workspace_bytes(const sd_seqview* views, int n_seq, int H_q, int D) {
  return sd_decode_attn_verify_workspace_bytes(views, nullptr, n_seq, H_q, D);
}

size_t sd_decode_attn_verify_workspace_bytes(const sd_seqview* views, const int32_t* n_new,
                                             int n_seq, int H_q, int D) {
  if (!views || n_seq < 1 || n_seq > SD_MAX_SEQS || H_q < 1 || D != kAttnHeadDim) return 0;
  SeqArgs a;
  if (check_views(views, n_seq, D, true, n_new) != SD_OK) return 0;
  fill_seqargs(views, n_seq, &a, n_new);
  // (the partials do not depend on how the query heads share KV heads)
  return attn_layout(&a, H_q, H_q) * sizeof(float);
}

int sd_decode_attn_multiseq(const float* q, int64_t ld_q, const sd_seqview* views, int n_seq,
                            int H_q, int H_kv, int D, float scale, float* out, void* ws,
                            size_t ws_bytes, sd_stream_t stream) {
  return attn_common(q, ld_q, views, nullptr, n_seq, H_q, H_kv, D, scale, out, ws, ws_bytes, stream);
}

int sd_decode_attn_multiseq_noalloc(const float* q, int64_t ld_q, const sd_seqview* views, int n_seq,
                                    int H_q, int H_kv, int D, float scale, float* out,
                                    sd_stream_t stream) {
  if (!q || !out || H_q < 1 || H_kv < 1 || H_q % H_kv != 0) return SD_EINVAL;
  if (D != kAttnHeadDim) return SD_EUNSUPPORTED;
  if (ld_q < (int64_t)H_q * D || !isfinite(scale)) return SD_EINVAL;
  int rc = check_views(views, n_seq, D, true);
  if (rc != SD_OK) return rc;
  if (!aligned(q, 16) || ld_q % 4 != 0 || !aligned(out, 16)) return SD_EALIGN;
  SeqArgs a;
  fill_seqargs(views, n_seq, &a);
  if (attn_layout(&a, H_q, H_kv) * sizeof(float) > kAttnScratchBytes) return SD_EWORKSPACE;
  float* part = nullptr;
  if (attn_scratch(&part) != hipSuccess) return SD_EHIP;
  return from_hip(launch_attn(q, ld_q, a, H_q, H_kv, scale, out, part, nullptr, nullptr, hs(stream)));
}

int sd_decode_attn_verify(const float* q, int64_t ld_q, const sd_seqview* views,
                          const int32_t* n_new, int n_seq, int H_q, int H_kv, int D, float scale,
                          float* out, void* ws, size_t ws_bytes, sd_stream_t stream) {
  if (!n_new) return SD_EINVAL;
  return attn_common(q, ld_q, views, n_new, n_seq, H_q, H_kv, D, scale, out, ws, ws_bytes, stream);
}

int sd_rmsnorm_q8(const float* x, int64_t ldx, int n_tok, int64_t D, const float* gamma, float eps,
                  int8_t* xq, float* xd, float* y, sd_stream_t stream) {
  if (!x || !gamma || !xq || !xd || n_tok < 1 || n_tok > SD_MAX_TOKENS || ldx < D) return SD_EINVAL;
  if (D < 32 || D > 32768 || D % 32 != 0) return SD_EUNSUPPORTED;
  if (!(eps >= 0.0f) || !isfinite(eps)) return SD_EINVAL;
  if (!aligned(x, 4) || !aligned(xq, 4) || !aligned(xd, 4) || (y && !aligned(y, 4))) return SD_EALIGN;
  return from_hip(launch_rmsnorm_q8(x, ldx, n_tok, D, gamma, eps, xq, xd, y, hs(stream)));
}

int sd_swiglu_q8(const float* gu, int64_t ldgu, int n_tok, int64_t F, int8_t* xq, float* xd,
                 float* y, sd_stream_t stream) {
  if (!gu || !xq || !xd || n_tok < 1 || n_tok > SD_MAX_TOKENS || F < 32 || ldgu < 2 * F)
    return SD_EINVAL;
  if (F % 32 != 0 || F > ((int64_t)1 << 24)) return SD_EUNSUPPORTED;
  if (!aligned(gu, 4) || !aligned(xd, 4) || (y && !aligned(y, 4))) return SD_EALIGN;
  return from_hip(launch_swiglu_q8(gu, ldgu, n_tok, F, xq, xd, y, hs(stream)));
}

int sd_qgemv_q8_0_swiglu_q8(const void* w, int64_t F, int64_t K, const int8_t* xq, const float* xd,
                            int n_tok, int8_t* xq_out, float* xd_out, sd_stream_t stream) {
  if (!w || !xq || !xd || !xq_out || !xd_out) return SD_EINVAL;
  if (n_tok < 1 || n_tok > SD_MAX_TOKENS || F < 32 || F > ((int64_t)1 << 29) || K < 1) return SD_EINVAL;
  if (K % 256 != 0 || K > ((int64_t)1 << 24) || F % 32 != 0) return SD_EUNSUPPORTED;
  if (!aligned(w, 16) || !aligned(xq, 16) || !aligned(xd, 4) || !aligned(xd_out, 4)) return SD_EALIGN;
  if (!swiglu_fusable(F, K, n_tok)) return SD_EUNSUPPORTED;  // beyond the one-chunk staged kernel
  return from_hip(launch_qgemv_swiglu(w, F, K, xq, xd, n_tok, xq_out, xd_out, hs(stream)));
}

int sd_embed_f16(const uint16_t* table, int64_t V, int64_t H, const int32_t* tokens, int n_tok,
                 float* x, sd_stream_t stream) {
  if (!table || !tokens || !x || V < 1 || H < 1 || n_tok < 1 || n_tok > 65535) return SD_EINVAL;
  if (!aligned(table, 2) || !aligned(tokens, 4) || !aligned(x, 4)) return SD_EALIGN;
  return from_hip(launch_embed(table, V, H, tokens, n_tok, x, hs(stream)));
}

int sd_hbm_stream_read(const void* buf, size_t bytes, uint32_t* sink, sd_stream_t stream) {
  if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return SD_EINVAL;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return SD_EALIGN;
  return from_hip(launch_stream_read(buf, bytes, sink, hs(stream)));
}

size_t sd_argmax_workspace_bytes(int n_tok, int64_t V) {
  if (n_tok < 1 || n_tok > 65535 || V < 1 || V > INT32_MAX - 1) return 0;
  return argmax_ws_bytes(n_tok, V);
}

int sd_argmax_rows(const float* logits, int64_t ld, int n_tok, int64_t V, int32_t* out, void* ws,
                   size_t ws_bytes, sd_stream_t stream) {
  if (!logits || !out || !ws || n_tok < 1 || n_tok > 65535 || V < 1 || V > INT32_MAX - 1 || ld < V)
    return SD_EINVAL;
  if (!aligned(logits, 4) || !aligned(out, 4) || !aligned(ws, 4)) return SD_EALIGN;
  if (ws_bytes < argmax_ws_bytes(n_tok, V)) return SD_EWORKSPACE;
  return from_hip(launch_argmax(logits, ld, n_tok, V, out, ws, hs(stream)));
}

}  // extern "C"
