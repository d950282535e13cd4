// Host runtime behind the C ABI in include/sdm.h: configuration checks,
// workspace carving, RoPE table, KV page bookkeeping, the per-sequence state
// machine of the three decoding modes, and the forward driver that enqueues
// the gfx950 kernels on the model's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/sdm.h"
#include "internal.hpp"
#include "page_pool.hpp"

using namespace sdm;

namespace {

thread_local std::string g_err;

sdm_status fail(sdm_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// Check a config; returns SDM_OK or the status with g_err set.
sdm_status check_config(const sdm_config* c) {
  if (!c) return fail(SDM_ERR_ARG, "config is null");
  if (c->n_layers < 1 || c->d_model < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->head_dim < 2 ||
      c->ffn_dim < 1 || c->vocab < 2)
    return fail(SDM_ERR_ARG, "non-positive model dimension");
  if (c->mask_id < 0 || c->mask_id >= c->vocab) return fail(SDM_ERR_ARG, "mask_id outside [0, vocab)");
  if (c->n_q_heads % c->n_kv_heads) return fail(SDM_ERR_UNSUPPORTED, "n_q_heads must be a multiple of n_kv_heads");
  if (c->page_tokens != kPageTokens) return fail(SDM_ERR_UNSUPPORTED, "page_tokens must be %d", kPageTokens);
  if (c->max_seqs < 1 || c->max_block < 1 || c->max_context < 2 || c->max_rows < 1)
    return fail(SDM_ERR_ARG, "non-positive capacity");
  if (c->max_block > c->max_rows) return fail(SDM_ERR_ARG, "max_block exceeds max_rows");
  if (c->max_context > 65536) return fail(SDM_ERR_UNSUPPORTED, "max_context above 65536");
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f)) return fail(SDM_ERR_ARG, "bad rms_eps or rope_base");
  if (c->dtype == SDM_BF16) {
    if (c->head_dim != kHd) return fail(SDM_ERR_UNSUPPORTED, "bf16 models need head_dim %d", kHd);
    if (c->d_model % 32 || c->ffn_dim % 16 || c->vocab % 32)
      return fail(SDM_ERR_UNSUPPORTED, "bf16 models need d_model %% 32 == 0, ffn %% 16 == 0, vocab %% 32 == 0");
    if (c->d_model > 8192) return fail(SDM_ERR_UNSUPPORTED, "bf16 models need d_model <= 8192");
  } else if (c->dtype == SDM_F32) {
    if (c->head_dim % 2 || c->head_dim > 128) return fail(SDM_ERR_UNSUPPORTED, "f32 models need an even head_dim <= 128");
    if (c->n_q_heads > 64) return fail(SDM_ERR_UNSUPPORTED, "f32 models support at most 64 query heads");
  } else {
    return fail(SDM_ERR_UNSUPPORTED, "unknown dtype %d", c->dtype);
  }
  if (c->weight_format == SDM_WEIGHTS_INT4) {
    if (c->dtype != SDM_BF16) return fail(SDM_ERR_UNSUPPORTED, "4-bit weights need a bf16 model");
    if (c->d_model % kW4Group || c->ffn_dim % kW4Group)
      return fail(SDM_ERR_UNSUPPORTED, "4-bit weights need d_model and ffn_dim multiples of %d", kW4Group);
  } else if (c->weight_format != SDM_WEIGHTS_BF16) {
    return fail(SDM_ERR_UNSUPPORTED, "unknown weight format %d", c->weight_format);
  }
  return SDM_OK;
}

struct Dims {
  int L, d, Hq, Hkv, hd, F, V, G, qkv, qd;
  int R, R32, max_pages, max_splits, max_slots, nq_cap;
  int x_cap;             // largest block of quadratic self-speculation (B + B^2 rows); 0: none
  int64_t x_page_elems;  // one candidate's scratch page (one layer)
  bool bf16;
  bool w4;  // decoder matrices are 4-bit
  int64_t elt;
  // bf16 path: elements from the hi plane to the lo plane of each activation buffer
  int64_t xn_plane, q_plane, attn_plane, h_plane;
  int planes;  // 2 for bf16 (hi, lo), 1 for f32
};

Dims dims_of(const sdm_config* c) {
  Dims D;
  D.L = c->n_layers; D.d = c->d_model; D.Hq = c->n_q_heads; D.Hkv = c->n_kv_heads; D.hd = c->head_dim;
  D.F = c->ffn_dim; D.V = c->vocab; D.G = D.Hq / D.Hkv; D.qd = D.Hq * D.hd; D.qkv = D.qd + 2 * D.Hkv * D.hd;
  D.R = c->max_rows; D.R32 = (int)align_up(D.R, 32);
  D.max_pages = (int)pages_for(c->max_context, kPageTokens);
  // one more split than the context needs: a candidate block's own keys
  D.max_splits = (c->max_context + kAttnSplitKeys - 1) / kAttnSplitKeys + 1;
  D.x_cap = 0;
  for (int b = 2; b <= std::min({c->max_block, kPageTokens, kMaxSlots - 1}); ++b)
    if ((int64_t)b * (b + 1) <= c->max_rows) D.x_cap = b;
  D.x_page_elems = 2LL * D.Hkv * kPageTokens * D.hd;
  D.max_slots = std::max(std::min(c->max_seqs, kMaxSlots), D.x_cap ? D.x_cap + 1 : 0);
  D.nq_cap = D.G * D.R + 32 * D.max_slots;
  D.bf16 = c->dtype == SDM_BF16;
  D.w4 = D.bf16 && c->weight_format == SDM_WEIGHTS_INT4;
  D.elt = D.bf16 ? 2 : 4;
  D.planes = D.bf16 ? 2 : 1;
  D.xn_plane = (int64_t)D.R32 * D.d;
  // bf16: packed per (slot, KV head), at most nq_cap columns per head in all
  D.q_plane = D.bf16 ? (int64_t)D.Hkv * D.nq_cap * D.hd : (int64_t)D.R * D.qd;
  D.attn_plane = (int64_t)D.R32 * D.qd;
  D.h_plane = (int64_t)D.R32 * D.F;
  return D;
}

struct Layout {
  int64_t x, xn, q, attn, hbuf, ybuf, part, opart, mlpart, records, tok, conf, margin, rope_cos, rope_sin,
      page_table, slog, sparts, slse, sgap, slogp, sprobe, xkv, total;
};

Layout layout_of(const sdm_config* c) {
  const Dims D = dims_of(c);
  Layout Lo{};
  int64_t off = 0;
  auto take = [&](int64_t bytes) {
    const int64_t o = off;
    off = align_up(off + std::max<int64_t>(bytes, 0), 256);
    return o;
  };
  const int64_t rows_act = D.bf16 ? D.R32 : D.R;
  Lo.x = take((int64_t)D.R * D.d * 4);
  Lo.xn = take(D.planes * rows_act * D.d * D.elt);
  Lo.q = take(D.planes * D.q_plane * D.elt);
  Lo.attn = take(D.planes * rows_act * D.qd * D.elt);
  Lo.hbuf = take(D.planes * rows_act * D.F * D.elt);
  int64_t ycols = 0;
  if (!D.bf16) ycols = std::max<int64_t>(std::max<int64_t>(D.qkv, 2LL * D.F), std::max<int64_t>(D.V, D.d));
  Lo.ybuf = take((int64_t)D.R * ycols * 4);
  // split-K partials of the residual-stream projections (O and down)
  int smax = 1;
  if (D.w4)
    smax = std::max(gemm_config_w4(EPI_PARTIAL, D.d, D.qd, D.R).S, gemm_config_w4(EPI_PARTIAL, D.d, D.F, D.R).S);
  else if (D.bf16)
    smax = std::max(gemm_config(EPI_PARTIAL, D.d, D.qd, D.R).S, gemm_config(EPI_PARTIAL, D.d, D.F, D.R).S);
  Lo.part = take(D.bf16 ? (int64_t)smax * D.R * D.d * 4 : 0);
  Lo.opart = take(D.bf16 ? (int64_t)D.Hkv * D.max_splits * D.hd * D.nq_cap * 4 : 0);
  Lo.mlpart = take(D.bf16 ? (int64_t)D.Hkv * D.max_splits * 2 * D.nq_cap * 4 : 0);
  const int n_vtiles = (D.V + 31) / 32;
  Lo.records = take((int64_t)D.R * n_vtiles * 16);
  Lo.tok = take((int64_t)D.R * 4);
  Lo.conf = take((int64_t)D.R * 4);
  Lo.margin = take((int64_t)D.R * 4);
  Lo.rope_cos = take((int64_t)c->max_context * (D.hd / 2) * 4);
  Lo.rope_sin = take((int64_t)c->max_context * (D.hd / 2) * 4);
  Lo.page_table = take((int64_t)c->max_seqs * D.max_pages * 4);
  // sampling at temperature > 0: the rows' logits (bf16 models; f32 ones keep them in ybuf), per-row parts
  Lo.slog = take(D.bf16 ? (int64_t)D.R * D.V * 4 : 0);
  Lo.sparts = take((int64_t)D.R * kSampleParts * (int64_t)sizeof(SamplePart));
  Lo.slse = take((int64_t)D.R * 4);
  Lo.sgap = take((int64_t)D.R * 4);
  Lo.slogp = take((int64_t)D.R * 4);
  Lo.sprobe = take((int64_t)D.R * 4);
  // quadratic self-speculation: each candidate block's K/V of the current layer
  Lo.xkv = take((int64_t)D.x_cap * D.x_page_elems * D.elt);
  Lo.total = off;
  return Lo;
}

}  // namespace

struct sdm_model {
  sdm_config cfg;
  Dims D;
  Layout lo;
  hipStream_t stream;
  char* ws;
  void* pool;
  int64_t page_elems;
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  std::vector<const void*> attn_norm, w_qkv, w_o, ffn_norm, w_gu, w_down;
  PagePool pages;
  std::vector<SeqState> seqs;
  bool dev_error = false;
  int last_rows = 0;
  // kernel timing window
  int timed_class = -1;
  std::vector<hipEvent_t> ev_begin, ev_end;
  size_t ev_used = 0;

  template <typename T>
  T* at(int64_t off) const { return (T*)(ws + off); }
};

namespace {

sdm_status check_hip(sdm_model* m, hipError_t e, const char* what) {
  if (e == hipSuccess) return SDM_OK;
  m->dev_error = true;
  return fail(SDM_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

#define HIP_TRY(expr, what)                              \
  do {                                                   \
    sdm_status _s = check_hip(m, (expr), what);          \
    if (_s != SDM_OK) return _s;                         \
  } while (0)

sdm_status check_model(const sdm_model* m) {
  if (!m) return fail(SDM_ERR_ARG, "model is null");
  if (m->dev_error) return fail(SDM_ERR_DEVICE, "an earlier HIP error left the model unusable");
  return SDM_OK;
}

sdm_status check_seq(const sdm_model* m, int32_t seq) {
  if (seq < 0 || seq >= m->cfg.max_seqs) return fail(SDM_ERR_CAPACITY, "sequence id %d outside [0, %d)", seq, m->cfg.max_seqs);
  return SDM_OK;
}

// Make sure pages cover positions [0, end) of every listed sequence; all or
// nothing.  New page-table entries are written to the device table.
sdm_status ensure_pages(sdm_model* m, const std::vector<int32_t>& seqs, const std::vector<int32_t>& ends) {
  int64_t need = 0;
  for (size_t i = 0; i < seqs.size(); ++i) {
    const int64_t want = pages_for(ends[i], kPageTokens);
    if (want > m->D.max_pages) return fail(SDM_ERR_CAPACITY, "sequence %d would exceed max_context", seqs[i]);
    need += std::max<int64_t>(0, want - (int64_t)m->seqs[seqs[i]].pages.size());
  }
  if (need > m->pages.free_count())
    return fail(SDM_ERR_CAPACITY, "KV pool exhausted: need %lld pages, %lld free", (long long)need,
                (long long)m->pages.free_count());
  for (size_t i = 0; i < seqs.size(); ++i) {
    SeqState& s = m->seqs[seqs[i]];
    const int64_t want = pages_for(ends[i], kPageTokens);
    const int64_t have = (int64_t)s.pages.size();
    if (want <= have) continue;
    m->pages.take(want - have, &s.pages);
    int* dst = m->at<int>(m->lo.page_table) + (int64_t)seqs[i] * m->D.max_pages;
    for (int64_t p = have; p < want; p += 64) {
      const int n = (int)std::min<int64_t>(64, want - p);
      HIP_TRY(launch_set_ints(dst + p, s.pages.data() + p, n, m->stream), "page table update");
    }
  }
  return SDM_OK;
}

// Committed lengths live on the host and reach the kernels in Slots.
sdm_status set_len(sdm_model* m, int32_t seq, int32_t len) {
  m->seqs[seq].len = len;
  return SDM_OK;
}

// Timing of the launches of one kernel class: the events ride on the kernel's
// own dispatch (start / completion).  A whole forward is bracketed by a pair of
// stream events instead.
struct TimedScope {
  sdm_model* m;
  bool on;
  int cls;
  TimedScope(sdm_model* mm, int c) : m(mm), on(mm->timed_class == c && mm->ev_used < mm->ev_begin.size()), cls(c) {
    if (!on) return;
    if (cls == SDM_K_FORWARD) {
      hipEventRecord(m->ev_begin[m->ev_used], m->stream);
    } else {
      g_ktiming.start = m->ev_begin[m->ev_used];
      g_ktiming.stop = m->ev_end[m->ev_used];
    }
  }
  ~TimedScope() {
    if (!on) return;
    if (cls == SDM_K_FORWARD) hipEventRecord(m->ev_end[m->ev_used], m->stream);
    g_ktiming = KernelTiming{};
    ++m->ev_used;
  }
};

KvView kv_view(const sdm_model* m, int layer) {
  KvView kv;
  kv.pool = m->pool;
  kv.page_elems = m->page_elems;
  kv.layer_off = (int64_t)layer * 2 * m->D.Hkv * kPageTokens * m->D.hd;
  kv.page_table = m->at<int>(m->lo.page_table);
  kv.max_pages = m->D.max_pages;
  kv.Hkv = m->D.Hkv;
  kv.hd = m->D.hd;
  kv.xpool = m->ws + m->lo.xkv;
  kv.x_page_elems = m->D.x_page_elems;
  return kv;
}

// The decoder's weight GEMMs (QKV, O, gate/up, down): bf16 or 4-bit weights.
GemmShape decoder_gemm_shape(const Dims& D, int epi, int N, int K, int M) {
  return D.w4 ? gemm_config_w4(epi, N, K, M) : gemm_config(epi, N, K, M);
}

hipError_t decoder_gemm(const Dims& D, int epi, const void* W, const uint16_t* X, int64_t x_plane, int N, int K, int M,
                        const EpiArgs& ea, hipStream_t st) {
  const GemmShape g = decoder_gemm_shape(D, epi, N, K, M);
  if (D.w4) return launch_gemm_w4(epi, (const uint8_t*)W, X, x_plane, g, ea, st);
  return launch_gemm_bf16(epi, (const uint16_t*)W, X, x_plane, g, ea, st);
}

struct TokenInput {
  const int* tokens = nullptr;  // [M] (TOK_PLAIN)
  int src = TOK_PLAIN;
  const int* anchor = nullptr;  // TOK_DRAFT
};

// One forward over n_seq x T rows at positions len[s] + t; writes K/V of
// the rows into the uncommitted slots; ends with the finish kernel.
// logits_last_only: the LM head runs on the last row only (prefill chunks).
sdm_status forward_body(sdm_model* m, const Slots& sl, int mode, const TokenInput& ti, bool logits_last_only,
                        float* d_logits, FinishArgs fin);

sdm_status forward(sdm_model* m, const Slots& sl, int mode, const TokenInput& ti, bool logits_last_only,
                   float* d_logits, FinishArgs fin) {
  TimedScope ts(m, SDM_K_FORWARD);
  return forward_body(m, sl, mode, ti, logits_last_only, d_logits, fin);
}

sdm_status forward_body(sdm_model* m, const Slots& sl, int mode, const TokenInput& ti, bool logits_last_only,
                        float* d_logits, FinishArgs fin) {
  const Dims& D = m->D;
  const int M = sl.n_seq * sl.T;
  hipStream_t st = m->stream;
  float* x = m->at<float>(m->lo.x);
  void* xn = m->ws + m->lo.xn;
  HIP_TRY(launch_embed(m->cfg.dtype, m->embed, D.d, D.V, ti.tokens, ti.src, ti.anchor, M, sl.T, m->cfg.mask_id, x, st),
          "embed");
  EpiArgs ea{};
  ea.M = M;
  ea.slots = sl;
  ea.Hq = D.Hq;
  ea.q_out = m->at<uint16_t>(m->lo.q);
  ea.q_plane = D.q_plane;
  ea.q_nq_pad = (int)align_up((int64_t)D.G * sl.T, 32);
  ea.rope_cos = m->at<float>(m->lo.rope_cos);
  ea.rope_sin = m->at<float>(m->lo.rope_sin);
  ea.d = D.d;
  ea.h_out = m->at<uint16_t>(m->lo.hbuf);
  ea.h_plane = D.h_plane;
  ea.F = D.F;
  ea.records = m->at<float4>(m->lo.records);
  ea.n_vtiles = (D.V + 31) / 32;
  ea.V = D.V;
  ea.mask_id = m->cfg.mask_id;
  ea.part = m->at<float>(m->lo.part);
  ea.part_stride = (int64_t)D.R * D.d;
  const float eps = m->cfg.rms_eps;
  int nparts = 0;  // split-K partials waiting to be added to the residual by the next RMSNorm

  for (int l = 0; l < D.L; ++l) {
    ea.kv = kv_view(m, l);
    { TimedScope ts(m, SDM_K_NORM);
      HIP_TRY(launch_rmsnorm(m->cfg.dtype, x, ea.part, nparts, ea.part_stride, m->attn_norm[l], eps, M, D.d, 0, xn,
                             D.xn_plane, st),
              "rmsnorm"); }
    nparts = 0;
    if (D.bf16) {
      { TimedScope ts(m, SDM_K_QKV);
      HIP_TRY(decoder_gemm(D, EPI_QKV, m->w_qkv[l], (const uint16_t*)xn, D.xn_plane, D.qkv, D.d, M, ea, st),
              "qkv gemm"); }
      AttnArgs aa{};
      aa.q = ea.q_out;
      aa.q_plane = D.q_plane;
      aa.q_packed = 1;
      aa.kv = ea.kv;
      aa.slots = sl;
      aa.Hq = D.Hq;
      aa.mode = mode;
      aa.scale = 1.f / sqrtf((float)D.hd);
      aa.opart = m->at<float>(m->lo.opart);
      aa.mlpart = m->at<float>(m->lo.mlpart);
      aa.max_splits = D.max_splits;
      aa.nq_pad = (int)align_up((int64_t)D.G * sl.T, 32);
      aa.out = m->at<uint16_t>(m->lo.attn);
      aa.out_packed = 1;
      aa.out_plane = D.attn_plane;
      int grid_splits = 0;
      for (int i = 0; i < sl.n_seq; ++i) grid_splits = std::max(grid_splits, attn_splits(sl, i));
      { TimedScope ts(m, SDM_K_ATTN);
        HIP_TRY(launch_attention_bf16(aa, grid_splits, st), "attention"); }
      { TimedScope ts(m, SDM_K_ATTN_COMBINE);
        HIP_TRY(launch_attn_combine_bf16(aa, st), "attention combine"); }
      { TimedScope ts(m, SDM_K_O);
        nparts = decoder_gemm_shape(D, EPI_PARTIAL, D.d, D.qd, M).S;
        HIP_TRY(decoder_gemm(D, EPI_PARTIAL, m->w_o[l], aa.out, D.attn_plane, D.d, D.qd, M, ea, st), "o gemm"); }
      { TimedScope ts(m, SDM_K_NORM);
        HIP_TRY(launch_rmsnorm(m->cfg.dtype, x, ea.part, nparts, ea.part_stride, m->ffn_norm[l], eps, M, D.d, 0, xn,
                               D.xn_plane, st),
                "rmsnorm"); }
      nparts = 0;
      { TimedScope ts(m, SDM_K_GATE_UP);
        HIP_TRY(decoder_gemm(D, EPI_SWIGLU, m->w_gu[l], (const uint16_t*)xn, D.xn_plane, 2 * D.F, D.d, M, ea, st),
                "gate/up gemm"); }
      { TimedScope ts(m, SDM_K_DOWN);
        nparts = decoder_gemm_shape(D, EPI_PARTIAL, D.d, D.F, M).S;
        HIP_TRY(decoder_gemm(D, EPI_PARTIAL, m->w_down[l], ea.h_out, D.h_plane, D.d, D.F, M, ea, st),
                "down gemm"); }
    } else {
      float* y = m->at<float>(m->lo.ybuf);
      float* qf = m->at<float>(m->lo.q);
      float* af = m->at<float>(m->lo.attn);
      float* hf = m->at<float>(m->lo.hbuf);
      ea.q_out = (uint16_t*)qf;
      HIP_TRY(launch_gemm_f32((const float*)xn, (const float*)m->w_qkv[l], M, D.qkv, D.d, y, st), "qkv gemm");
      HIP_TRY(launch_qkv_post_f32(y, ea, D.hd, st), "qkv post");
      HIP_TRY(launch_attention_f32(qf, ea.kv, sl, D.Hq, mode, af, st), "attention");
      HIP_TRY(launch_gemm_f32(af, (const float*)m->w_o[l], M, D.d, D.qd, y, st), "o gemm");
      HIP_TRY(launch_resid_f32(y, x, M, D.d, st), "residual");
      HIP_TRY(launch_rmsnorm(m->cfg.dtype, x, nullptr, 0, 0, m->ffn_norm[l], eps, M, D.d, 0, xn, 0, st), "rmsnorm");
      HIP_TRY(launch_gemm_f32((const float*)xn, (const float*)m->w_gu[l], M, 2 * D.F, D.d, y, st), "gate/up gemm");
      HIP_TRY(launch_swiglu_f32(y, hf, M, D.F, st), "swiglu");
      HIP_TRY(launch_gemm_f32(hf, (const float*)m->w_down[l], M, D.d, D.F, y, st), "down gemm");
      HIP_TRY(launch_resid_f32(y, x, M, D.d, st), "residual");
    }
  }
  // final norm + LM head on the rows whose logits are needed
  const int ML = logits_last_only ? 1 : M;
  const int row0 = logits_last_only ? M - 1 : 0;
  HIP_TRY(launch_rmsnorm(m->cfg.dtype, x, ea.part, nparts, ea.part_stride, m->final_norm, eps, ML, D.d, row0, xn,
                         D.xn_plane, st),
          "final rmsnorm");
  ea.M = ML;
  ea.logits = d_logits;
  const bool sampling = is_sampling(fin.mode);
  if (sampling && D.bf16 && !d_logits) ea.logits = m->at<float>(m->lo.slog);
  if (D.bf16) {
    TimedScope ts(m, SDM_K_LM_HEAD);
    HIP_TRY(launch_gemm_bf16(EPI_LOGITS, (const uint16_t*)m->lm_head, (const uint16_t*)xn, D.xn_plane,
                             gemm_config(EPI_LOGITS, D.V, D.d, ML),
                             ea, st),
            "lm head");
  } else {
    float* y = m->at<float>(m->lo.ybuf);
    HIP_TRY(launch_gemm_f32((const float*)xn, (const float*)m->lm_head, ML, D.V, D.d, y, st), "lm head");
    HIP_TRY(launch_logit_records_f32(y, ea, st), "vocab records");
  }
  fin.records = ea.records;
  fin.n_vtiles = ea.n_vtiles;
  fin.tok = m->at<int>(m->lo.tok);
  fin.conf = m->at<float>(m->lo.conf);
  fin.margin = m->at<float>(m->lo.margin);
  fin.mask_id = m->cfg.mask_id;
  fin.M = ML;
  if (sampling) {
    fin.logits = D.bf16 ? ea.logits : m->at<float>(m->lo.ybuf);
    fin.V = D.V;
    fin.parts = m->at<SamplePart>(m->lo.sparts);
    fin.lse = m->at<float>(m->lo.slse);
    fin.gap = m->at<float>(m->lo.sgap);
    fin.logp = m->at<float>(m->lo.slogp);
    fin.logp_probe = m->at<float>(m->lo.sprobe);
  }
  { TimedScope ts(m, SDM_K_FINISH);
    HIP_TRY(launch_finish(fin, st), "finish"); }
  m->last_rows = ML;
  return SDM_OK;
}

Slots one_slot(const sdm_model* m, int32_t seq, int T) {
  Slots s{};
  s.n_seq = 1;
  s.T = T;
  s.ids[0] = seq;
  s.len[0] = m->seqs[seq].len;
  return s;
}

// Shared checks of a block call over several sequences.
sdm_status check_block_call(sdm_model* m, int32_t n_seq, const int32_t* h_ids, int32_t B, Slots* sl,
                            std::vector<int32_t>* ids, std::vector<int32_t>* ends) {
  if (n_seq < 1 || n_seq > kMaxSlots) return fail(SDM_ERR_ARG, "n_seq %d outside [1, %d]", n_seq, kMaxSlots);
  if (!h_ids) return fail(SDM_ERR_ARG, "h_seq_ids is null");
  if (B < 1 || B > m->cfg.max_block) return fail(SDM_ERR_ARG, "block %d outside [1, max_block=%d]", B, m->cfg.max_block);
  if ((int64_t)n_seq * B > m->cfg.max_rows) return fail(SDM_ERR_CAPACITY, "n_seq * B exceeds max_rows");
  if (m->D.bf16 && (int64_t)n_seq * align_up((int64_t)m->D.G * B, 32) > m->D.nq_cap)
    return fail(SDM_ERR_CAPACITY, "attention workspace too small for this batch");
  *sl = Slots{};
  sl->n_seq = n_seq;
  sl->T = B;
  for (int i = 0; i < n_seq; ++i) {
    const int32_t s = h_ids[i];
    if (check_seq(m, s) != SDM_OK) return SDM_ERR_CAPACITY;
    for (int j = 0; j < i; ++j)
      if (h_ids[j] == s) return fail(SDM_ERR_ARG, "sequence %d listed twice", s);
    if (!m->seqs[s].prefilled) return fail(SDM_ERR_STATE, "sequence %d has no prompt", s);
    if ((int64_t)m->seqs[s].len + B > m->cfg.max_context)
      return fail(SDM_ERR_CAPACITY, "sequence %d would exceed max_context", s);
    sl->ids[i] = s;
    sl->len[i] = m->seqs[s].len;
    ids->push_back(s);
    ends->push_back(m->seqs[s].len + B);
  }
  return SDM_OK;
}

}  // namespace

// ============================================================================
// C ABI
// ============================================================================
extern "C" {

const char* sdm_last_error(void) { return g_err.c_str(); }

size_t sdm_workspace_bytes(const sdm_config* cfg) {
  if (check_config(cfg) != SDM_OK) return 0;
  return (size_t)layout_of(cfg).total;
}

size_t sdm_kv_page_bytes(const sdm_config* cfg) {
  if (check_config(cfg) != SDM_OK) return 0;
  const Dims D = dims_of(cfg);
  return (size_t)D.L * 2 * D.Hkv * kPageTokens * D.hd * D.elt;
}

size_t sdm_packed_bytes(const sdm_config* cfg, int64_t rows, int64_t cols) {
  if (check_config(cfg) != SDM_OK || rows < 1 || cols < 1) return 0;
  if (cfg->dtype == SDM_BF16) return (size_t)(align_up(rows, 32) * align_up(cols, 16) * 2);
  return (size_t)(rows * cols * 4);
}

sdm_status sdm_pack_matrix(const sdm_config* cfg, int32_t kind, const void* d_src, const void* d_src2, void* d_dst,
                           int64_t rows, int64_t cols, void* hip_stream) {
  sdm_status s = check_config(cfg);
  if (s != SDM_OK) return s;
  if (!d_src || !d_dst || (kind == SDM_PACK_GATE_UP && !d_src2)) return fail(SDM_ERR_ARG, "null pointer");
  if (kind < SDM_PACK_PLAIN || kind > SDM_PACK_GATE_UP) return fail(SDM_ERR_ARG, "unknown pack kind %d", kind);
  if (rows < 1 || cols < 1) return fail(SDM_ERR_ARG, "empty matrix");
  if (cfg->dtype == SDM_BF16) {
    if (cols % 16) return fail(SDM_ERR_UNSUPPORTED, "bf16 packing needs cols %% 16 == 0");
    if (kind == SDM_PACK_GATE_UP ? rows % 16 : rows % 32)
      return fail(SDM_ERR_UNSUPPORTED, "bf16 packing needs rows %% 32 == 0 (%% 16 for gate/up)");
    if (kind == SDM_PACK_QKV && rows % cfg->head_dim) return fail(SDM_ERR_ARG, "qkv rows not a multiple of head_dim");
  }
  hipError_t e = launch_pack(cfg->dtype, kind, d_src, d_src2, d_dst, rows, cols, cfg->head_dim, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(SDM_ERR_DEVICE, "pack: %s", hipGetErrorString(e));
  return SDM_OK;
}

size_t sdm_packed_bytes_int4(const sdm_config* cfg, int64_t rows, int64_t cols) {
  if (check_config(cfg) != SDM_OK || cfg->dtype != SDM_BF16 || rows < 1 || cols < 1 || rows % 32 ||
      cols % kW4Group)
    return 0;
  return (size_t)w4_packed_bytes(rows, cols);
}

sdm_status sdm_pack_matrix_int4(const sdm_config* cfg, int32_t kind, const void* d_codes, const void* d_scales,
                                const void* d_codes2, const void* d_scales2, void* d_dst, int64_t rows, int64_t cols,
                                void* hip_stream) {
  sdm_status s = check_config(cfg);
  if (s != SDM_OK) return s;
  if (cfg->dtype != SDM_BF16) return fail(SDM_ERR_UNSUPPORTED, "4-bit weights need a bf16 config");
  if (kind < SDM_PACK_PLAIN || kind > SDM_PACK_GATE_UP) return fail(SDM_ERR_ARG, "unknown pack kind %d", kind);
  if (!d_codes || !d_scales || !d_dst || (kind == SDM_PACK_GATE_UP && (!d_codes2 || !d_scales2)))
    return fail(SDM_ERR_ARG, "null pointer");
  if (rows < 1 || cols < 1) return fail(SDM_ERR_ARG, "empty matrix");
  if (cols % kW4Group) return fail(SDM_ERR_UNSUPPORTED, "4-bit packing needs cols %% %d == 0", kW4Group);
  if (kind == SDM_PACK_GATE_UP ? rows % 16 : rows % 32)
    return fail(SDM_ERR_UNSUPPORTED, "4-bit packing needs rows %% 32 == 0 (%% 16 for gate/up)");
  if (kind == SDM_PACK_QKV && rows % cfg->head_dim) return fail(SDM_ERR_ARG, "qkv rows not a multiple of head_dim");
  auto misaligned = [](const void* p) { return p && ((uintptr_t)p & 3); };
  if (misaligned(d_codes) || misaligned(d_codes2) || misaligned(d_dst) || misaligned(d_scales) ||
      misaligned(d_scales2))
    return fail(SDM_ERR_ARG, "4-bit packing needs 4-byte aligned buffers");
  hipError_t e = launch_pack_w4(kind, d_codes, d_scales, d_codes2, d_scales2, d_dst, rows, cols, cfg->head_dim,
                                (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(SDM_ERR_DEVICE, "pack: %s", hipGetErrorString(e));
  return SDM_OK;
}

sdm_status sdm_init_model(const sdm_config* cfg, const sdm_weights* w, void* kv_pool, int64_t n_pages,
                          void* workspace, size_t ws_bytes, void* hip_stream, sdm_model** out) {
  sdm_status s = check_config(cfg);
  if (s != SDM_OK) return s;
  if (!w || !kv_pool || !workspace || !out) return fail(SDM_ERR_ARG, "null pointer");
  if (n_pages < 1 || n_pages > (int64_t)1 << 30) return fail(SDM_ERR_ARG, "n_pages out of range");
  if (!w->embed || !w->final_norm || !w->lm_head || !w->attn_norm || !w->w_qkv || !w->w_o || !w->ffn_norm ||
      !w->w_gate_up || !w->w_down)
    return fail(SDM_ERR_ARG, "null weight pointer");
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!w->attn_norm[l] || !w->w_qkv[l] || !w->w_o[l] || !w->ffn_norm[l] || !w->w_gate_up[l] || !w->w_down[l])
      return fail(SDM_ERR_ARG, "null weight pointer in layer %d", l);
  const Layout lo = layout_of(cfg);
  if ((int64_t)ws_bytes < lo.total)
    return fail(SDM_ERR_CAPACITY, "workspace holds %zu bytes, needs %lld", ws_bytes, (long long)lo.total);
  if (((uintptr_t)workspace) % 256) return fail(SDM_ERR_ARG, "workspace must be 256-byte aligned");

  sdm_model* m = new sdm_model();
  m->cfg = *cfg;
  m->D = dims_of(cfg);
  m->lo = lo;
  m->stream = (hipStream_t)hip_stream;
  m->ws = (char*)workspace;
  m->pool = kv_pool;
  m->page_elems = (int64_t)m->D.L * 2 * m->D.Hkv * kPageTokens * m->D.hd;
  m->embed = w->embed;
  m->final_norm = w->final_norm;
  m->lm_head = w->lm_head;
  for (int l = 0; l < cfg->n_layers; ++l) {
    m->attn_norm.push_back(w->attn_norm[l]);
    m->w_qkv.push_back(w->w_qkv[l]);
    m->w_o.push_back(w->w_o[l]);
    m->ffn_norm.push_back(w->ffn_norm[l]);
    m->w_gu.push_back(w->w_gate_up[l]);
    m->w_down.push_back(w->w_down[l]);
  }
  m->pages.reset(n_pages);
  m->seqs.resize(cfg->max_seqs);

  // RoPE table: angle p * base^(-2t/hd) in double, cos/sin stored as float.
  const int half = m->D.hd / 2;
  std::vector<float> cs((size_t)cfg->max_context * half), sn(cs.size());
  for (int p = 0; p < cfg->max_context; ++p)
    for (int t = 0; t < half; ++t) {
      const double inv = std::pow((double)cfg->rope_base, -2.0 * t / m->D.hd);
      const double ang = (double)p * inv;
      cs[(size_t)p * half + t] = (float)std::cos(ang);
      sn[(size_t)p * half + t] = (float)std::sin(ang);
    }
  hipError_t e = hipMemcpyAsync(m->ws + lo.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice, m->stream);
  if (e == hipSuccess)
    e = hipMemcpyAsync(m->ws + lo.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice, m->stream);
  // Attention reads whole 32-key tiles; slots past a sequence's end must hold
  // finite values (their probabilities are exactly 0), so the pool starts zeroed.
  if (e == hipSuccess)
    e = hipMemsetAsync(kv_pool, 0, (size_t)n_pages * (size_t)(m->page_elems * m->D.elt), m->stream);
  // likewise the candidate blocks' scratch pages (keys past B are never written)
  if (e == hipSuccess && m->D.x_cap)
    e = hipMemsetAsync(m->ws + lo.xkv, 0, (size_t)(m->D.x_cap * m->D.x_page_elems * m->D.elt), m->stream);
  if (e == hipSuccess) e = hipStreamSynchronize(m->stream);
  if (e != hipSuccess) {
    delete m;
    return fail(SDM_ERR_DEVICE, "init upload: %s", hipGetErrorString(e));
  }
  *out = m;
  return SDM_OK;
}

static void timing_release(sdm_model* m) {
  for (auto e : m->ev_begin) hipEventDestroy(e);
  for (auto e : m->ev_end) hipEventDestroy(e);
  m->ev_begin.clear();
  m->ev_end.clear();
  m->ev_used = 0;
  m->timed_class = -1;
}

sdm_status sdm_free_model(sdm_model* m) {
  if (!m) return fail(SDM_ERR_ARG, "model is null");
  timing_release(m);
  delete m;
  return SDM_OK;
}

sdm_status sdm_timing_start(sdm_model* m, int32_t kernel_class, int32_t capacity) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if (kernel_class < SDM_K_QKV || kernel_class > SDM_K_FORWARD) return fail(SDM_ERR_ARG, "unknown kernel class");
  if (capacity < 1 || capacity > (1 << 20)) return fail(SDM_ERR_ARG, "capacity out of range");
  timing_release(m);
  m->ev_begin.resize(capacity);
  m->ev_end.resize(capacity);
  for (int i = 0; i < capacity; ++i) {
    if (hipEventCreate(&m->ev_begin[i]) != hipSuccess || hipEventCreate(&m->ev_end[i]) != hipSuccess) {
      m->ev_begin.resize(i);
      m->ev_end.resize(i);
      timing_release(m);
      return fail(SDM_ERR_DEVICE, "hipEventCreate failed");
    }
  }
  m->timed_class = kernel_class;
  return SDM_OK;
}

sdm_status sdm_timing_stop(sdm_model* m, int64_t* launches, double* total_ms, double* min_ms, double* max_ms) {
  if (!m) return fail(SDM_ERR_ARG, "model is null");
  if (m->timed_class < 0) return fail(SDM_ERR_STATE, "no timing window is open");
  HIP_TRY(hipStreamSynchronize(m->stream), "timing sync");
  double tot = 0, mn = 1e300, mx = 0;
  for (size_t i = 0; i < m->ev_used; ++i) {
    float ms = 0;
    HIP_TRY(hipEventElapsedTime(&ms, m->ev_begin[i], m->ev_end[i]), "event time");
    tot += ms;
    mn = std::min(mn, (double)ms);
    mx = std::max(mx, (double)ms);
  }
  if (launches) *launches = (int64_t)m->ev_used;
  if (total_ms) *total_ms = tot;
  if (min_ms) *min_ms = m->ev_used ? mn : 0;
  if (max_ms) *max_ms = mx;
  timing_release(m);
  return SDM_OK;
}

namespace {
struct Sampling {
  bool on = false;
  float inv_t = 1.f;
  uint64_t seed = 0;
};

sdm_status check_sampling(float temperature, uint64_t seed, Sampling* smp) {
  if (!(temperature > 0.f) || !(temperature < INFINITY)) return fail(SDM_ERR_ARG, "temperature must be finite and > 0");
  smp->on = true;
  smp->inv_t = 1.f / temperature;
  smp->seed = seed;
  return SDM_OK;
}

void set_sampling(FinishArgs& fin, const Sampling& smp, int seq) {
  fin.inv_t = smp.inv_t;
  fin.seed = smp.seed;
  fin.seq_id = seq;
}

sdm_status prefill_impl(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t* d_next_token,
                        float* d_logits, const Sampling& smp);
}  // namespace

sdm_status sdm_prefill(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t* d_next_token,
                       float* d_logits) {
  return prefill_impl(m, seq, d_tokens, n, d_next_token, d_logits, Sampling{});
}

sdm_status sdm_prefill_sample(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, float temperature,
                              uint64_t seed, int32_t* d_next_token, float* d_logits) {
  Sampling smp;
  sdm_status s = check_sampling(temperature, seed, &smp);
  if (s != SDM_OK) return s;
  return prefill_impl(m, seq, d_tokens, n, d_next_token, d_logits, smp);
}

namespace {
sdm_status prefill_impl(sdm_model* m, int32_t seq, const int32_t* d_tokens, int32_t n, int32_t* d_next_token,
                        float* d_logits, const Sampling& smp) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if ((s = check_seq(m, seq)) != SDM_OK) return s;
  if (!d_tokens || !d_next_token) return fail(SDM_ERR_ARG, "null pointer");
  if (n < 1) return fail(SDM_ERR_ARG, "empty prompt");
  SeqState& q = m->seqs[seq];
  if (q.prefilled || q.len != 0) return fail(SDM_ERR_STATE, "sequence %d is not empty", seq);
  if ((int64_t)n + 1 > m->cfg.max_context) return fail(SDM_ERR_CAPACITY, "prompt exceeds max_context");
  if ((s = ensure_pages(m, {seq}, {n})) != SDM_OK) return s;
  const int C = m->cfg.max_rows;
  for (int32_t off = 0; off < n; off += C) {
    const int T = std::min(C, n - off);
    const bool last = off + T == n;
    FinishArgs fin{};
    fin.mode = last && smp.on ? FIN_SAMPLE_NEXT : FIN_NEXT;
    fin.slots = one_slot(m, seq, 1);
    fin.T = 1;
    fin.next = d_next_token;
    fin.target_pos = off + T;
    set_sampling(fin, smp, seq);
    TokenInput ti;
    ti.tokens = d_tokens + off;
    // intermediate chunks still run the (cheap, one-row) head so that every
    // chunk leaves the same state behind; only the last chunk's result counts
    if ((s = forward(m, one_slot(m, seq, T), CAUSAL, ti, true, last ? d_logits : nullptr, fin)) != SDM_OK) return s;
    if ((s = set_len(m, seq, off + T)) != SDM_OK) return s;
  }
  q.prefilled = true;
  q.verified = 0;
  return SDM_OK;
}
}  // namespace

namespace {
sdm_status decode_ar_impl(sdm_model* m, int32_t seq, const int32_t* d_token, int32_t* d_next_token, float* d_logits,
                          const Sampling& smp);
}

sdm_status sdm_decode_ar(sdm_model* m, int32_t seq, const int32_t* d_token, int32_t* d_next_token, float* d_logits) {
  return decode_ar_impl(m, seq, d_token, d_next_token, d_logits, Sampling{});
}

sdm_status sdm_decode_ar_sample(sdm_model* m, int32_t seq, const int32_t* d_token, float temperature, uint64_t seed,
                                int32_t* d_next_token, float* d_logits) {
  Sampling smp;
  sdm_status s = check_sampling(temperature, seed, &smp);
  if (s != SDM_OK) return s;
  return decode_ar_impl(m, seq, d_token, d_next_token, d_logits, smp);
}

namespace {
sdm_status decode_ar_impl(sdm_model* m, int32_t seq, const int32_t* d_token, int32_t* d_next_token, float* d_logits,
                          const Sampling& smp) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if ((s = check_seq(m, seq)) != SDM_OK) return s;
  if (!d_token || !d_next_token) return fail(SDM_ERR_ARG, "null pointer");
  SeqState& q = m->seqs[seq];
  if (!q.prefilled) return fail(SDM_ERR_STATE, "sequence %d has no prompt", seq);
  if ((int64_t)q.len + 1 > m->cfg.max_context) return fail(SDM_ERR_CAPACITY, "sequence %d is full", seq);
  if ((s = ensure_pages(m, {seq}, {q.len + 1})) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = smp.on ? FIN_SAMPLE_NEXT : FIN_NEXT;
  fin.slots = one_slot(m, seq, 1);
  fin.T = 1;
  fin.next = d_next_token;
  fin.target_pos = q.len + 1;
  set_sampling(fin, smp, seq);
  TokenInput ti;
  ti.tokens = d_token;
  if ((s = forward(m, one_slot(m, seq, 1), CAUSAL, ti, false, d_logits, fin)) != SDM_OK) return s;
  q.verified = 0;
  return set_len(m, seq, q.len + 1);
}
}  // namespace

sdm_status sdm_draft_block(sdm_model* m, int32_t seq, const int32_t* d_anchor, int32_t B, int32_t* d_block_out,
                           float* d_logits) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if (!d_anchor || !d_block_out) return fail(SDM_ERR_ARG, "null pointer");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, 1, &seq, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_DRAFT;
  fin.slots = sl;
  fin.T = B;
  fin.anchor = d_anchor;
  fin.block = d_block_out;
  TokenInput ti;
  ti.src = TOK_DRAFT;
  ti.anchor = d_anchor;
  if ((s = forward(m, sl, BIDIR, ti, false, d_logits, fin)) != SDM_OK) return s;
  m->seqs[seq].verified = 0;
  return SDM_OK;
}

sdm_status sdm_verify_block(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, const int32_t* d_block, int32_t B,
                            int32_t* d_ar_argmax, int32_t* d_accept_len, float* d_logits) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if (!d_block || !d_ar_argmax || !d_accept_len) return fail(SDM_ERR_ARG, "null pointer");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, n_seq, h_seq_ids, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_VERIFY;
  fin.slots = sl;
  fin.T = B;
  fin.block = (int*)d_block;
  fin.ar_out = d_ar_argmax;
  fin.accept = d_accept_len;
  TokenInput ti;
  ti.tokens = d_block;
  if ((s = forward(m, sl, CAUSAL, ti, false, d_logits, fin)) != SDM_OK) return s;
  for (int32_t id : ids) m->seqs[id].verified = B;
  return SDM_OK;
}

sdm_status sdm_verify_block_quadratic(sdm_model* m, int32_t seq, const int32_t* d_block, int32_t B,
                                      int32_t* d_ar_argmax, int32_t* d_accept_len, int32_t* d_next_blocks,
                                      float* d_logits) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if (!d_block || !d_ar_argmax || !d_accept_len || !d_next_blocks) return fail(SDM_ERR_ARG, "null pointer");
  if (d_block + B > d_next_blocks && d_block < d_next_blocks + (int64_t)B * B)
    return fail(SDM_ERR_ARG, "d_block overlaps d_next_blocks");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, 1, &seq, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if (B < 2) return fail(SDM_ERR_ARG, "quadratic self-speculation needs B >= 2");
  if (B > m->D.x_cap)
    return fail(SDM_ERR_CAPACITY, "block %d needs max_rows >= B * (B + 1) = %d and max_block >= B (largest here: %d)",
                B, B * (B + 1), m->D.x_cap);
  const int32_t n = m->seqs[seq].len;
  if ((int64_t)n + 2 * B > m->cfg.max_context)
    return fail(SDM_ERR_CAPACITY, "candidate blocks would reach past max_context");
  // the block (slot 0, causal) and candidate k at slot 1 + k, positions n+k+1..n+k+B
  sl.n_seq = 1 + B;
  sl.xslot0 = 1;
  for (int k = 0; k < B; ++k) {
    sl.ids[1 + k] = seq;
    sl.len[1 + k] = n + k + 1;
  }
  if (m->D.bf16 && (int64_t)(1 + B) * align_up((int64_t)m->D.G * B, 32) > m->D.nq_cap)
    return fail(SDM_ERR_CAPACITY, "attention workspace too small for the candidate blocks");
  if (attn_splits(sl, B) > std::min(kMaxSplits, m->D.max_splits))
    return fail(SDM_ERR_CAPACITY, "context too long for quadratic self-speculation");
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_QUAD;
  fin.slots = sl;
  fin.T = B;
  fin.block = (int*)d_block;
  fin.ar_out = d_ar_argmax;
  fin.accept = d_accept_len;
  fin.next_blocks = d_next_blocks;
  TokenInput ti;
  ti.tokens = d_block;
  ti.src = TOK_QUAD;
  if ((s = forward(m, sl, CAUSAL, ti, false, d_logits, fin)) != SDM_OK) return s;
  m->seqs[seq].verified = B;
  return SDM_OK;
}

sdm_status sdm_draft_block_sample(sdm_model* m, int32_t seq, const int32_t* d_anchor, int32_t B, float temperature,
                                  uint64_t seed, int32_t* d_block_out, float* d_draft_logits, float* d_draft_stats) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  Sampling smp;
  if ((s = check_sampling(temperature, seed, &smp)) != SDM_OK) return s;
  if (!d_anchor || !d_block_out || !d_draft_logits || !d_draft_stats) return fail(SDM_ERR_ARG, "null pointer");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, 1, &seq, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if (B < 2) return fail(SDM_ERR_ARG, "a sampled draft needs B >= 2");
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_SAMPLE_DRAFT;
  fin.slots = sl;
  fin.T = B;
  fin.anchor = d_anchor;
  fin.block = d_block_out;
  fin.draft_stats = d_draft_stats;
  set_sampling(fin, smp, seq);
  TokenInput ti;
  ti.src = TOK_DRAFT;
  ti.anchor = d_anchor;
  if ((s = forward(m, sl, BIDIR, ti, false, d_draft_logits, fin)) != SDM_OK) return s;
  m->seqs[seq].verified = 0;
  return SDM_OK;
}

sdm_status sdm_verify_block_sample(sdm_model* m, int32_t seq, const int32_t* d_block, int32_t B, float temperature,
                                   uint64_t seed, const float* d_draft_logits, const float* d_draft_stats,
                                   int32_t* d_accept_len, int32_t* d_next_token, float* d_logits) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  Sampling smp;
  if ((s = check_sampling(temperature, seed, &smp)) != SDM_OK) return s;
  if (!d_block || !d_draft_logits || !d_draft_stats || !d_accept_len || !d_next_token)
    return fail(SDM_ERR_ARG, "null pointer");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, 1, &seq, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if (B < 2) return fail(SDM_ERR_ARG, "a sampled verify needs B >= 2");
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_SAMPLE_VERIFY;
  fin.slots = sl;
  fin.T = B;
  fin.block = (int*)d_block;
  fin.accept = d_accept_len;
  fin.next = d_next_token;
  fin.draft_stats = (float*)d_draft_stats;
  fin.draft_logits = d_draft_logits;
  set_sampling(fin, smp, seq);
  TokenInput ti;
  ti.tokens = d_block;
  if ((s = forward(m, sl, CAUSAL, ti, false, d_logits, fin)) != SDM_OK) return s;
  m->seqs[seq].verified = B;
  return SDM_OK;
}

sdm_status sdm_commit_kv(sdm_model* m, int32_t seq, int32_t n_accept) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if ((s = check_seq(m, seq)) != SDM_OK) return s;
  SeqState& q = m->seqs[seq];
  if (q.verified < 1) return fail(SDM_ERR_STATE, "sequence %d has no causal block to commit", seq);
  if (n_accept < 1 || n_accept > q.verified)
    return fail(SDM_ERR_ARG, "n_accept %d outside [1, %d]", n_accept, q.verified);
  q.verified = 0;
  return set_len(m, seq, q.len + n_accept);
}

sdm_status sdm_diffuse_step(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, int32_t* d_block, int32_t B,
                            float tau, int32_t force_all, int32_t* d_n_masked, float* d_conf, float* d_logits) {
  return sdm_diffuse_step_revise(m, n_seq, h_seq_ids, d_block, B, tau, 2.f, force_all, d_n_masked, nullptr, d_conf,
                                 d_logits);
}

sdm_status sdm_diffuse_step_revise(sdm_model* m, int32_t n_seq, const int32_t* h_seq_ids, int32_t* d_block,
                                   int32_t B, float tau, float tau_revise, int32_t force_all, int32_t* d_n_masked,
                                   int32_t* d_n_revised, float* d_conf, float* d_logits) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if (!d_block || !d_n_masked) return fail(SDM_ERR_ARG, "null pointer");
  if (!(tau == tau) || !(tau_revise == tau_revise)) return fail(SDM_ERR_ARG, "tau or tau_revise is NaN");
  Slots sl;
  std::vector<int32_t> ids, ends;
  if ((s = check_block_call(m, n_seq, h_seq_ids, B, &sl, &ids, &ends)) != SDM_OK) return s;
  if ((s = ensure_pages(m, ids, ends)) != SDM_OK) return s;
  FinishArgs fin{};
  fin.mode = FIN_DIFFUSE;
  fin.slots = sl;
  fin.T = B;
  fin.block = d_block;
  fin.n_masked = d_n_masked;
  fin.conf_out = d_conf;
  fin.tau = tau;
  fin.force_all = force_all ? 1 : 0;
  fin.tau_revise = tau_revise;
  fin.n_revised = d_n_revised;
  TokenInput ti;
  ti.tokens = d_block;
  if ((s = forward(m, sl, BIDIR, ti, false, d_logits, fin)) != SDM_OK) return s;
  for (int32_t id : ids) m->seqs[id].verified = 0;
  return SDM_OK;
}

sdm_status sdm_row_stats(sdm_model* m, int32_t* d_tok, float* d_conf, float* d_margin) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  const size_t n = (size_t)m->last_rows * 4;
  if (n == 0) return fail(SDM_ERR_STATE, "no forward has run");
  if (d_tok) HIP_TRY(hipMemcpyAsync(d_tok, m->ws + m->lo.tok, n, hipMemcpyDeviceToDevice, m->stream), "row stats");
  if (d_conf) HIP_TRY(hipMemcpyAsync(d_conf, m->ws + m->lo.conf, n, hipMemcpyDeviceToDevice, m->stream), "row stats");
  if (d_margin)
    HIP_TRY(hipMemcpyAsync(d_margin, m->ws + m->lo.margin, n, hipMemcpyDeviceToDevice, m->stream), "row stats");
  return SDM_OK;
}

sdm_status sdm_seq_reset(sdm_model* m, int32_t seq) {
  sdm_status s = check_model(m);
  if (s != SDM_OK) return s;
  if ((s = check_seq(m, seq)) != SDM_OK) return s;
  SeqState& q = m->seqs[seq];
  m->pages.give_back(q.pages);
  q = SeqState{};
  return set_len(m, seq, 0);
}

sdm_status sdm_seq_length(const sdm_model* m, int32_t seq, int32_t* out) {
  if (!m || !out) return fail(SDM_ERR_ARG, "null pointer");
  if (seq < 0 || seq >= m->cfg.max_seqs) return fail(SDM_ERR_CAPACITY, "sequence id out of range");
  *out = m->seqs[seq].len;
  return SDM_OK;
}

int64_t sdm_free_pages(const sdm_model* m) { return m ? m->pages.free_count() : -1; }

sdm_status sdm_shuffle_free_pages(sdm_model* m, uint64_t seed) {
  if (!m) return fail(SDM_ERR_ARG, "model is null");
  m->pages.shuffle(seed);
  return SDM_OK;
}

// ---- standalone attention op -------------------------------------------------
size_t sdm_attn_pool_bytes(int32_t n_kv_heads, int32_t head_dim, int32_t n_pages) {
  if (n_kv_heads < 1 || head_dim != kHd || n_pages < 1) return 0;
  return (size_t)n_pages * 2 * n_kv_heads * kPageTokens * head_dim * 2;
}

static int64_t attn_ws_layout(int32_t Hq, int32_t Hkv, int32_t T, int32_t max_keys, int64_t* o_ml) {
  const int G = Hq / Hkv;
  const int64_t nq_pad = align_up((int64_t)G * T, 32);
  const int64_t splits = (max_keys + kAttnSplitKeys - 1) / kAttnSplitKeys;
  const int64_t op = align_up(Hkv * splits * kHd * nq_pad * 4, 256);
  const int64_t ml = align_up(Hkv * splits * 2 * nq_pad * 4, 256);
  *o_ml = op;
  return op + ml;
}

size_t sdm_attn_workspace_bytes(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t T, int32_t max_keys) {
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads || head_dim != kHd || T < 1 || max_keys < T) return 0;
  int64_t a;
  return (size_t)attn_ws_layout(n_q_heads, n_kv_heads, T, max_keys, &a);
}

sdm_status sdm_attn_pack_kv(int32_t n_kv_heads, int32_t head_dim, const void* d_k, const void* d_v, int32_t n_keys,
                            const int32_t* d_pages, void* d_pool, void* hip_stream) {
  if (n_kv_heads < 1 || head_dim != kHd) return fail(SDM_ERR_UNSUPPORTED, "attention op needs head_dim %d", kHd);
  if (!d_k || !d_v || !d_pages || !d_pool) return fail(SDM_ERR_ARG, "null pointer");
  if (n_keys < 1) return fail(SDM_ERR_ARG, "no keys");
  hipError_t e = launch_attn_pack_kv(n_kv_heads, (const uint16_t*)d_k, (const uint16_t*)d_v, n_keys, d_pages,
                                     (uint16_t*)d_pool, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(SDM_ERR_DEVICE, "attn pack: %s", hipGetErrorString(e));
  return SDM_OK;
}

}  // extern "C"

namespace {
// Checks shared by both attention entry points (before anything is enqueued).
sdm_status attention_check(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const void* d_q,
                           const void* d_pool, const int32_t* d_pages, int32_t n_prefix, int32_t T, int32_t mode,
                           const void* d_out) {
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads) return fail(SDM_ERR_UNSUPPORTED, "bad head counts");
  if (head_dim != kHd) return fail(SDM_ERR_UNSUPPORTED, "attention op needs head_dim %d", kHd);
  if (!d_q || !d_pool || !d_pages || !d_out) return fail(SDM_ERR_ARG, "null pointer");
  if (n_prefix < 0 || T < 1 || T > 4096) return fail(SDM_ERR_ARG, "bad n_prefix / T");
  if ((int64_t)n_prefix + T > 65536) return fail(SDM_ERR_UNSUPPORTED, "more than 65536 keys");
  if (mode != SDM_CAUSAL && mode != SDM_BIDIR) return fail(SDM_ERR_ARG, "bad mode");
  return SDM_OK;
}

// The attention op with its partials in ws (at least attn_ws_layout bytes).
sdm_status attention_run(int32_t n_q_heads, int32_t n_kv_heads, const void* d_q, const void* d_pool,
                         const int32_t* d_pages, int32_t n_prefix, int32_t T, int32_t mode, void* d_out, char* ws,
                         void* hip_stream) {
  int64_t off_ml;
  attn_ws_layout(n_q_heads, n_kv_heads, T, n_prefix + T, &off_ml);
  hipStream_t st = (hipStream_t)hip_stream;
  const int32_t nkeys = n_prefix + T;
  hipError_t e = hipSuccess;
  AttnArgs aa{};
  aa.q = (const uint16_t*)d_q;
  aa.kv.pool = (void*)d_pool;
  aa.kv.page_elems = 2LL * n_kv_heads * kPageTokens * kHd;
  aa.kv.layer_off = 0;
  aa.kv.page_table = d_pages;
  aa.kv.max_pages = (int)pages_for(nkeys, kPageTokens);
  aa.kv.Hkv = n_kv_heads;
  aa.kv.hd = kHd;
  aa.slots.n_seq = 1;
  aa.slots.T = T;
  aa.slots.ids[0] = 0;
  aa.slots.len[0] = n_prefix;
  aa.Hq = n_q_heads;
  aa.mode = mode;
  aa.scale = 1.f / sqrtf((float)kHd);
  aa.opart = (float*)ws;
  aa.mlpart = (float*)(ws + off_ml);
  aa.max_splits = (nkeys + kAttnSplitKeys - 1) / kAttnSplitKeys;
  aa.nq_pad = (int)align_up((int64_t)(n_q_heads / n_kv_heads) * T, 32);
  aa.out = (uint16_t*)d_out;
  aa.out_packed = 0;
  aa.q_plane = 0;    // the op takes plain row-major bf16 queries
  aa.q_packed = 0;
  aa.out_plane = 0;  // and returns plain bf16
  if (e == hipSuccess) e = launch_attention_bf16(aa, aa.max_splits, st);
  if (e == hipSuccess) e = launch_attn_combine_bf16(aa, st);
  if (e != hipSuccess) return fail(SDM_ERR_DEVICE, "attention: %s", hipGetErrorString(e));
  return SDM_OK;
}
}  // namespace

extern "C" {

sdm_status sdm_attention(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const void* d_q, const void* d_pool,
                         const int32_t* d_pages, int32_t n_prefix, int32_t T, int32_t mode, void* d_out,
                         void* d_workspace, size_t ws_bytes, void* hip_stream) {
  sdm_status s = attention_check(n_q_heads, n_kv_heads, head_dim, d_q, d_pool, d_pages, n_prefix, T, mode, d_out);
  if (s != SDM_OK) return s;
  if (!d_workspace) return fail(SDM_ERR_ARG, "null pointer");
  int64_t off_ml;
  const int64_t need = attn_ws_layout(n_q_heads, n_kv_heads, T, n_prefix + T, &off_ml);
  if ((int64_t)ws_bytes < need) return fail(SDM_ERR_CAPACITY, "attention workspace too small");
  return attention_run(n_q_heads, n_kv_heads, d_q, d_pool, d_pages, n_prefix, T, mode, d_out, (char*)d_workspace,
                       hip_stream);
}

size_t sdm_attention_scratch_max_bytes(void) { return kAttnScratchBytes; }

sdm_status sdm_attention_noalloc(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, const void* d_q,
                                 const void* d_pool, const int32_t* d_pages, int32_t n_prefix, int32_t T,
                                 int32_t mode, void* d_out, void* hip_stream) {
  sdm_status s = attention_check(n_q_heads, n_kv_heads, head_dim, d_q, d_pool, d_pages, n_prefix, T, mode, d_out);
  if (s != SDM_OK) return s;
  int64_t off_ml;
  const int64_t need = attn_ws_layout(n_q_heads, n_kv_heads, T, n_prefix + T, &off_ml);
  if (need > (int64_t)kAttnScratchBytes)
    return fail(SDM_ERR_CAPACITY, "attention partials need %lld bytes, the device scratch holds %zu",
                (long long)need, kAttnScratchBytes);
  void* scratch = nullptr;
  const hipError_t e = attn_scratch_address(&scratch);
  if (e != hipSuccess) return fail(SDM_ERR_DEVICE, "scratch address: %s", hipGetErrorString(e));
  return attention_run(n_q_heads, n_kv_heads, d_q, d_pool, d_pages, n_prefix, T, mode, d_out, (char*)scratch,
                       hip_stream);
}

}  // extern "C"
