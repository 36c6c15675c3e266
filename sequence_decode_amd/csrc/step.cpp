// step.cpp -- sd_decode_step: one fused batched decode step, enqueued from C++.
//
// Structure: ds4 pull request 604, "2. Single-GPU decode batches don't scale"
// and "Commit walkthrough / Graph driver": the dense projections run once on a
// shared batch workspace with one row per sequence, so the weights cross HBM
// once per step; RoPE and the KV append run per sequence at each sequence's own
// position; attention is one multi-sequence launch; the feed-forward block and
// the output head run on the batch; the logits land one row per sequence.
// Every kernel here is row-independent with a fixed reduction order, so a
// sequence's logits are bitwise those of a step that holds it alone (the
// exactness of "feat(qwen4exp): exact 4-slot concurrent serving", "How it
// stays exact").  The ~10 launches per layer are issued from here, not from
// Python, so the host keeps ahead of the GPU.
#include <math.h>

#include <algorithm>

#include "internal.hpp"

using namespace sd;

namespace {

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

struct StepLayout {
  size_t x, aq, ad, qkv, attn_o, gu, part, arg, rope, total;
};

bool model_ok(const sd_model* m) {
  if (!m || !m->layers || !m->tok_embd || !m->out_norm || !m->w_lm_head) return false;
  if (m->n_layers < 1 || m->hidden < 256 || m->vocab < 1 || m->ffn < 256) return false;
  if (m->head_dim != kAttnHeadDim || m->n_kv_heads < 1 || m->n_heads < 1 || m->n_heads % m->n_kv_heads != 0)
    return false;
  if (m->hidden % 256 != 0 || m->ffn % 256 != 0 || (m->n_heads * m->head_dim) % 256 != 0) return false;
  if (m->hidden > 32768 || m->ffn > 32768) return false;
  if (!(m->rms_eps >= 0.0f) || !(m->rope_theta > 0.0)) return false;
  if (m->n_rot < 0 || m->n_rot > m->head_dim || m->n_rot % 2 != 0 || m->window < 0) return false;
  for (int l = 0; l < m->n_layers; ++l) {
    const sd_layer_weights& L = m->layers[l];
    if (!L.w_qkv || !L.w_o || !L.w_gate_up || !L.w_down || !L.attn_norm || !L.ffn_norm) return false;
  }
  return true;
}

StepLayout layout(const sd_model* m, int n, int max_ctx) {
  const size_t qkv_rows = (size_t)(m->n_heads + 2 * m->n_kv_heads) * m->head_dim;
  size_t maxk = (size_t)m->hidden;
  if ((size_t)m->ffn > maxk) maxk = m->ffn;
  if ((size_t)m->n_heads * m->head_dim > maxk) maxk = (size_t)m->n_heads * m->head_dim;
  // a sequence's chunks are at most those of keys 0 .. max_ctx - 1 (chunks are
  // densest at low positions)
  const size_t chunks = (size_t)attn_chunks(0, max_ctx - 1);
  StepLayout L;
  size_t off = 0;
  L.x = off;      off = align_up(off + (size_t)n * m->hidden * 4, 256);
  L.aq = off;     off = align_up(off + (size_t)n * maxk, 256);
  L.ad = off;     off = align_up(off + (size_t)n * (maxk / 32) * 4, 256);
  L.qkv = off;    off = align_up(off + (size_t)n * qkv_rows * 4, 256);
  L.attn_o = off; off = align_up(off + (size_t)n * m->n_heads * m->head_dim * 4, 256);
  L.gu = off;     off = align_up(off + (size_t)n * 2 * m->ffn * 4, 256);
  L.part = off;   off = align_up(off + (size_t)n * chunks * m->n_heads * kAttnPartialFloats * 4, 256);
  L.arg = off;    off = align_up(off + argmax_ws_bytes(n, m->vocab), 256);
  L.rope = off;   off = align_up(off + (size_t)n * (m->head_dim / 2) * 8, 256);
  L.total = off;
  return L;
}

}  // namespace

extern "C" {

size_t sd_decode_step_workspace_bytes(const sd_model* m, int rows, int max_ctx) {
  if (!model_ok(m) || rows < 1 || rows > SD_MAX_TOKENS || max_ctx < 1) return 0;
  return layout(m, rows, max_ctx).total;
}

int sd_decode_step(const sd_model* m, const sd_step_io* io, sd_stream_t stream) {
  if (!model_ok(m)) return SD_EUNSUPPORTED;
  if (!io || !io->seqs || !io->tokens || !io->positions || !io->logits || !io->next_tokens || !io->ws)
    return SD_EINVAL;
  const int n_seq = io->n_seq;
  if (n_seq < 1 || n_seq > SD_MAX_SEQS) return SD_EINVAL;
  int max_ctx = 1, n = 0;  // n = token rows
  for (int s = 0; s < n_seq; ++s) {
    const sd_step_seq& q = io->seqs[s];
    const int T = q.n_new == 0 ? 1 : q.n_new;
    if (T < 1 || T > SD_ATTN_MAX_NEW) return SD_EINVAL;
    if (q.capacity < 1 || q.pos < 0 || (q.ring != 0 && q.ring != 1)) return SD_EINVAL;
    if (q.kv_type < SD_KV_F16 || q.kv_type > SD_KV_Q8_Q4) return SD_EINVAL;
    if (q.kv_type != io->seqs[0].kv_type) return SD_EUNSUPPORTED;
    if (q.kv_type == SD_KV_F16) {
      if (!q.k_cache || !q.v_cache) return SD_EINVAL;
      if (((uintptr_t)q.k_cache % 16) || ((uintptr_t)q.v_cache % 16)) return SD_EALIGN;
    } else {
      if (!q.k_q8 || !q.v_q8 || !q.k_d || !q.v_d) return SD_EINVAL;
      if (((uintptr_t)q.k_q8 % 16) || ((uintptr_t)q.v_q8 % 16) || ((uintptr_t)q.k_d % 8) ||
          ((uintptr_t)q.v_d % 8))
        return SD_EALIGN;
    }
    if (q.pos > 0x7fffffff - T) return SD_EINVAL;
    if (q.block_table) {
      // paged pool: whole blocks of 64, 128 or 256 rows
      if (q.ring) return SD_EINVAL;
      if (q.block_size != 64 && q.block_size != 128 && q.block_size != 256) return SD_EINVAL;
      if (q.capacity % q.block_size != 0) return SD_EINVAL;
      if ((uintptr_t)q.block_table % 4) return SD_EALIGN;
    } else if (q.ring) {
      // a ring keeps the positions still attended to: window + T - 1 of them at most
      if (m->window < 1) return SD_EINVAL;
      const int64_t span = q.pos + T < (int64_t)m->window + T - 1 ? q.pos + T : (int64_t)m->window + T - 1;
      if (span > q.capacity) return SD_EINVAL;
    } else if (q.pos > q.capacity - T) {
      return SD_EINVAL;
    }
    {
      // every token's keys span at most SD_MAX_CTX positions; the sequence's
      // chunks (from lo0's to the last token's) are at most those of max_ctx
      // keys from position 0
      const int lo0 = m->window ? (q.pos - m->window + 1 > 0 ? q.pos - m->window + 1 : 0) : 0;
      const int span = m->window ? std::min(q.pos + T, m->window) : q.pos + T;
      if (span > SD_MAX_CTX) return SD_EUNSUPPORTED;
      const int keys = q.pos + T - attn_chunk_begin(attn_chunk_of(lo0));
      if (keys > max_ctx) max_ctx = keys;
    }
    n += T;
  }
  if (n > SD_MAX_TOKENS) return SD_EINVAL;
  if ((uintptr_t)io->ws % 256 || (uintptr_t)io->logits % 4 || (uintptr_t)io->tokens % 4 ||
      (uintptr_t)io->positions % 4 || (uintptr_t)io->next_tokens % 4)
    return SD_EALIGN;
  const StepLayout W = layout(m, n, max_ctx);
  if (io->ws_bytes < W.total) return SD_EWORKSPACE;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(io->ws);
  float* x = reinterpret_cast<float*>(ws + W.x);
  int8_t* aq = reinterpret_cast<int8_t*>(ws + W.aq);
  float* ad = reinterpret_cast<float*>(ws + W.ad);
  float* qkv = reinterpret_cast<float*>(ws + W.qkv);
  float* attn_o = reinterpret_cast<float*>(ws + W.attn_o);
  float* gu = reinterpret_cast<float*>(ws + W.gu);
  float* part = reinterpret_cast<float*>(ws + W.part);
  float* rope_tab = reinterpret_cast<float*>(ws + W.rope);  // (cos, sin) per row and pair

  const int H = m->hidden, Hq = m->n_heads, Hkv = m->n_kv_heads, D = m->head_dim, F = m->ffn;
  const int64_t QKV = (int64_t)(Hq + 2 * Hkv) * D;
  const int64_t HqD = (int64_t)Hq * D;
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t layer_elems_per_tok = (int64_t)Hkv * D;
  // the FFN's gate|up projection and SwiGLU as one launch where the streaming
  // kernel allows it (up to 4 rows: at 8 the fused launch measured slower than
  // the two it replaces); the SwiGLU q8 output then lives in the gate|up region
  const bool fuse_swiglu = n <= 4 && swiglu_fusable(F, H, n);
  int8_t* fq = reinterpret_cast<int8_t*>(ws + W.gu);
  float* fd = reinterpret_cast<float*>(ws + W.gu + align_up((size_t)n * F, 256));

  SeqArgs sa{};
  sa.n_seq = n_seq;
  for (int s = 0; s < n_seq; ++s) {
    const int T = io->seqs[s].n_new == 0 ? 1 : io->seqs[s].n_new;
    sa.s[s].ld_tok = layer_elems_per_tok;
    sa.s[s].ld_head = D;
    sa.s[s].ctx_len = io->seqs[s].pos + T;
    sa.s[s].n_new = T;
    sa.s[s].window = m->window;
    sa.s[s].ring_cap = io->seqs[s].ring ? io->seqs[s].capacity : 0;
    const int kt = io->seqs[s].kv_type;
    sa.s[s].q8 = kt != SD_KV_F16;
    sa.s[s].k4 = kt == SD_KV_Q4_0 || kt == SD_KV_Q4_Q8;
    sa.s[s].v4 = kt == SD_KV_Q4_0 || kt == SD_KV_Q8_Q4;
    if (io->seqs[s].block_table) {
      sa.s[s].btab = io->seqs[s].block_table;
      sa.s[s].bshift = __builtin_ctz((unsigned)io->seqs[s].block_size);
      sa.s[s].n_blocks = io->seqs[s].capacity / io->seqs[s].block_size;
    }
  }
  attn_layout(&sa, Hq, Hkv);

#define SD_TRY(call)                         \
  do {                                       \
    if ((call) != hipSuccess) return SD_EHIP; \
  } while (0)

  // QKV projection, RoPE and K/V write as one launch where the streaming
  // kernel allows it (fp16 caches, whole 128-dim heads rotated, 1..8 rows)
  bool qkv_rope = D == 128 && (m->n_rot == 0 || m->n_rot == D) && qkv_rope_fusable(QKV, H, n);
  for (int s = 0; s < n_seq; ++s) qkv_rope = qkv_rope && !sa.s[s].q8;
  // the RMSNorm before the QKV, gate|up and output projections computed by
  // those projections' own workgroups (one row, hidden <= 4096): one launch
  // instead of two, the same codes and scales
  const bool rms_in = rms_fusable(H, n);
  GemvPlan qkv_plan, head_plan;
  const bool qkv_rms_plain = rms_in && plan_qgemv(QKV, H, n, SD_GEMV_NARROW, &qkv_plan) && qkv_plan.use_reg &&
                             qkv_plan.stage && qkv_plan.sp == 1;
  const bool head_rms = rms_in && plan_qgemv(m->vocab, H, n, SD_GEMV_NARROW, &head_plan) && head_plan.use_reg &&
                        head_plan.stage && head_plan.sp == 1;
  SD_TRY(launch_embed(m->tok_embd, m->vocab, H, io->tokens, n, x, st));
  for (int l = 0; l < m->n_layers; ++l) {
    const sd_layer_weights& L = m->layers[l];
    for (int s = 0; s < n_seq; ++s) {
      const sd_step_seq& q = io->seqs[s];
      const int64_t off = (int64_t)l * q.capacity * layer_elems_per_tok;
      if (sa.s[s].q8) {
        sa.s[s].kq = q.k_q8 + (sa.s[s].k4 ? off / 2 : off);
        sa.s[s].vq = q.v_q8 + (sa.s[s].v4 ? off / 2 : off);
        sa.s[s].kd = q.k_d + off / 32;
        sa.s[s].vd = q.v_d + off / 32;
      } else {
        sa.s[s].k = q.k_cache + off;
        sa.s[s].v = q.v_cache + off;
        sa.s[s].k_w = q.k_cache + off;
        sa.s[s].v_w = q.v_cache + off;
      }
    }
    const RmsArgs attn_rms{x, H, L.attn_norm, m->rms_eps};
    if (!rms_in) SD_TRY(launch_rmsnorm_q8(x, H, n, H, L.attn_norm, m->rms_eps, aq, ad, nullptr, st));
    if (qkv_rope) {
      // RoPE and the fp16 K/V write in the projection's epilogue (one launch)
      RopeArgs ra{io->positions, m->rope_theta, rope_tab, l == 0 ? 1 : 2, Hq, Hkv, sa};
      SD_TRY(launch_qgemv_qkv_rope(L.w_qkv, QKV, H, aq, ad, n, qkv, QKV, ra, st, rms_in ? &attn_rms : nullptr));
    } else {
      if (qkv_rms_plain) {
        SD_TRY(launch_qgemv_rms(L.w_qkv, QKV, H, attn_rms, n, qkv, QKV, st));
      } else {
        if (rms_in) SD_TRY(launch_rmsnorm_q8(x, H, n, H, L.attn_norm, m->rms_eps, aq, ad, nullptr, st));
        SD_TRY(launch_qgemv(L.w_qkv, QKV, H, aq, ad, n, nullptr, qkv, QKV, st));
      }
      SD_TRY(launch_rope_kv_step(qkv, QKV, n, Hq, Hkv, D, m->n_rot ? m->n_rot : D, io->positions,
                                 m->rope_theta, sa, rope_tab, l == 0 ? 1 : 2, st));
    }
    SD_TRY(launch_attn(qkv, QKV, sa, Hq, Hkv, scale, attn_o, part, aq, ad, st));
    SD_TRY(launch_qgemv(L.w_o, H, HqD, aq, ad, n, x, x, H, st));
    const RmsArgs ffn_rms{x, H, L.ffn_norm, m->rms_eps};
    if (fuse_swiglu && rms_in) {
      // RMSNorm, gate|up and SwiGLU in one launch
      SD_TRY(launch_qgemv_swiglu(L.w_gate_up, F, H, nullptr, nullptr, n, fq, fd, st, &ffn_rms));
      SD_TRY(launch_qgemv(L.w_down, H, F, fq, fd, n, x, x, H, st));
    } else if (fuse_swiglu) {
      // gate|up and SwiGLU in one launch; its q8 output goes to the (here
      // unused) gate|up region, since the launch still reads aq / ad
      SD_TRY(launch_rmsnorm_q8(x, H, n, H, L.ffn_norm, m->rms_eps, aq, ad, nullptr, st));
      SD_TRY(launch_qgemv_swiglu(L.w_gate_up, F, H, aq, ad, n, fq, fd, st));
      SD_TRY(launch_qgemv(L.w_down, H, F, fq, fd, n, x, x, H, st));
    } else {
      SD_TRY(launch_rmsnorm_q8(x, H, n, H, L.ffn_norm, m->rms_eps, aq, ad, nullptr, st));
      SD_TRY(launch_qgemv(L.w_gate_up, 2 * (int64_t)F, H, aq, ad, n, nullptr, gu, 2 * (int64_t)F, st));
      SD_TRY(launch_swiglu_q8(gu, 2 * (int64_t)F, n, F, aq, ad, nullptr, st));
      SD_TRY(launch_qgemv(L.w_down, H, F, aq, ad, n, x, x, H, st));
    }
  }
  if (head_rms) {
    SD_TRY(launch_qgemv_rms(m->w_lm_head, m->vocab, H, RmsArgs{x, H, m->out_norm, m->rms_eps}, n, io->logits,
                            m->vocab, st));
  } else {
    SD_TRY(launch_rmsnorm_q8(x, H, n, H, m->out_norm, m->rms_eps, aq, ad, nullptr, st));
    SD_TRY(launch_qgemv(m->w_lm_head, m->vocab, H, aq, ad, n, nullptr, io->logits, m->vocab, st));
  }
  SD_TRY(launch_argmax(io->logits, m->vocab, n, m->vocab, io->next_tokens, ws + W.arg, st));
#undef SD_TRY
  return SD_OK;
}

}  // extern "C"
