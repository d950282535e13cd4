// gfx950 kernels of the block-wise decoding forward.
//
// bf16 path (the 3B/8B/14B-shaped decoders): skinny MFMA GEMMs that stream
// packed weights once per forward with fused epilogues (RoPE + paged KV write,
// residual add, SwiGLU, vocab partial reduction), MFMA block attention over the
// paged KV cache with a split-KV combine, RMSNorm and the per-row selection
// that implements the three modes' token rules.
// f32 path (the tiny decoder): plain VALU kernels with the same semantics.
//
// The operations follow the decoder of the Nemotron-Labs-Diffusion pages as
// restated in the public header: the attention pattern (prefix visible to the
// whole block, block rows bidirectional when drafting/denoising and causal
// when verifying; fintech-frontier-insights, training route / Efficient-DLM
// block-wise attention), the threshold unmask of block diffusion
// (fintech-frontier-insights, diffusion bullet) and the accept rule of
// self-speculation (gsyq.cn explainer, section 2.3).
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "internal.hpp"
#include "placement.hpp"

namespace sdm {

thread_local KernelTiming g_ktiming;

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ uint16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);  // round to nearest, ties to even (finite inputs)
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
// Two values at once with the hardware packed conversion (v_cvt_pk_bf16_f32):
// the same round to nearest, ties to even as f2bf; a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// Second term of the two-term bf16 expansion of x whose first term is hi
// (x - hi is exact in fp32).
__device__ __forceinline__ uint16_t f2bf_lo(float x, uint16_t hi) { return f2bf(x - bf2f(hi)); }

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Row of accumulator register r held by a lane of half h in a 32x32 MFMA C tile.
__device__ __forceinline__ int crow(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---------------------------------------------------------------------------
// Packing (one-time, a permutation)
// ---------------------------------------------------------------------------
// Row of the packed matrix that holds source row r.
__device__ __forceinline__ int64_t pack_row(int kind, int64_t r, int64_t rows, int which, int head_dim) {
  if (kind == 1) {  // QKV: per head, tiles of [16 dims of the first half, 16 partner dims]
    const int64_t head = r / head_dim, dl = r % head_dim, half = dl / (head_dim / 2), t = dl % (head_dim / 2);
    return head * head_dim + 32 * (t / 16) + 16 * half + (t % 16);
  }
  if (kind == 2) {  // GATE_UP: tiles of [16 gate features, the same 16 up features]
    return 32 * (r / 16) + 16 * which + (r % 16);
  }
  return r;
}

__global__ void k_pack_bf16(int kind, const uint16_t* __restrict__ src, int which, uint16_t* __restrict__ dst,
                            int64_t rows, int64_t cols, int64_t out_cols, int head_dim) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * cols) return;
  const int64_t r = i / cols, c = i % cols;
  dst[packed_index(pack_row(kind, r, rows, which, head_dim), c, out_cols)] = src[i];
}

__global__ void k_copy_f32(const float* __restrict__ src, float* __restrict__ dst, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_pack(int dtype, int kind, const void* src, const void* src2, void* dst, int64_t rows, int64_t cols,
                       int head_dim, hipStream_t st) {
  const int64_t n = rows * cols;
  const dim3 blk(256), grd((unsigned)((n + 255) / 256));
  if (dtype == 1) {
    SDM_LAUNCH(k_pack_bf16, grd, blk, 0, st, kind, (const uint16_t*)src, 0, (uint16_t*)dst, rows, cols, cols,
                       head_dim);
    if (kind == 2)
      SDM_LAUNCH(k_pack_bf16, grd, blk, 0, st, kind, (const uint16_t*)src2, 1, (uint16_t*)dst, rows, cols,
                         cols, head_dim);
  } else {
    SDM_LAUNCH(k_copy_f32, grd, blk, 0, st, (const float*)src, (float*)dst, n);
    if (kind == 2) SDM_LAUNCH(k_copy_f32, grd, blk, 0, st, (const float*)src2, (float*)dst + n, n);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Block assembly + embedding gather into the fp32 residual stream
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t i);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t i) { return bf2f(p[i]); }

template <typename T>
__global__ void k_embed(const T* __restrict__ E, int d, int V, const int* __restrict__ tokens, int tok_src,
                        const int* __restrict__ anchor, int T_, int mask_id, float* __restrict__ x) {
  const int m = blockIdx.x;
  int tok;
  if (tok_src == TOK_DRAFT) tok = (m % T_ == 0) ? anchor[m / T_] : mask_id;
  else if (tok_src == TOK_QUAD) tok = m < T_ ? tokens[m] : mask_id;
  else tok = tokens[m];
  tok = tok < 0 ? 0 : (tok >= V ? V - 1 : tok);  // out-of-range ids are clamped, never read out of bounds
  for (int k = threadIdx.x; k < d; k += blockDim.x) x[(int64_t)m * d + k] = load_as_f32<T>(E, (int64_t)tok * d + k);
}

hipError_t launch_embed(int dtype, const void* E, int d, int V, const int* tokens, int tok_src, const int* anchor,
                        int M, int T, int mask_id, float* x, hipStream_t st) {
  if (dtype == 1)
    SDM_LAUNCH(k_embed<uint16_t>, dim3(M), dim3(256), 0, st, (const uint16_t*)E, d, V, tokens, tok_src,
                       anchor, T, mask_id, x);
  else
    SDM_LAUNCH(k_embed<float>, dim3(M), dim3(256), 0, st, (const float*)E, d, V, tokens, tok_src, anchor, T,
                       mask_id, x);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// RMSNorm: y = (x / sqrt(mean(x^2) + eps)) * g.  One workgroup per row, fixed
// reduction order.  bf16: written as hi/lo bf16 planes straight into the
// packed B-operand layout, 8 features (one 16-byte store per plane) per thread
// and chunk.  f32: row-major.
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 512;                    // one workgroup per row
constexpr int kNormChunks = 8192 / 8 / kNormThreads;  // chunks of 8 features per thread: d <= 8192

__global__ __launch_bounds__(kNormThreads) void k_rmsnorm_bf16(float* __restrict__ x, const float* __restrict__ part,
                                                      int nparts, int64_t part_stride,
                                                      const uint16_t* __restrict__ gain, float eps, int d, int row0,
                                                      uint16_t* __restrict__ out, int64_t out_plane) {
  const int m = blockIdx.x;
  float* xr = x + (int64_t)(row0 + m) * d;
  const int nch = d >> 3;
  float v[kNormChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kNormChunks; ++j) {
    const int c = threadIdx.x + kNormThreads * j;
    if (c < nch) {
      const float4 a = ((const float4*)xr)[2 * c], b = ((const float4*)xr)[2 * c + 1];
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      v[j][4] = b.x; v[j][5] = b.y; v[j][6] = b.z; v[j][7] = b.w;
      if (nparts > 0) {
        // residual += sum of the split-K partials of the preceding projection
        // (split order); every plane's loads are issued before the first add
        const float* pr = part + (int64_t)(row0 + m) * d + 8 * c;
        float4 pa[kMaxSplitK], pb[kMaxSplitK];
#pragma unroll
        for (int sp = 0; sp < kMaxSplitK; ++sp)
          if (sp < nparts) {
            pa[sp] = ((const float4*)(pr + sp * part_stride))[0];
            pb[sp] = ((const float4*)(pr + sp * part_stride))[1];
          }
        float pv[8] = {pa[0].x, pa[0].y, pa[0].z, pa[0].w, pb[0].x, pb[0].y, pb[0].z, pb[0].w};
#pragma unroll
        for (int sp = 1; sp < kMaxSplitK; ++sp)
          if (sp < nparts) {
            pv[0] += pa[sp].x; pv[1] += pa[sp].y; pv[2] += pa[sp].z; pv[3] += pa[sp].w;
            pv[4] += pb[sp].x; pv[5] += pb[sp].y; pv[6] += pb[sp].z; pv[7] += pb[sp].w;
          }
#pragma unroll
        for (int e = 0; e < 8; ++e) v[j][e] += pv[e];
        ((float4*)xr)[2 * c] = make_float4(v[j][0], v[j][1], v[j][2], v[j][3]);
        ((float4*)xr)[2 * c + 1] = make_float4(v[j][4], v[j][5], v[j][6], v[j][7]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[j][e] * v[j][e];
    }
  }
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ float wsum[kNormThreads / 64];
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = wsum[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) tot += wsum[w];
  const float r = sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int j = 0; j < kNormChunks; ++j) {
    const int c = threadIdx.x + kNormThreads * j;
    if (c < nch) {
      const u32x4 gv = ((const u32x4*)gain)[c];
      u32x4 oh, ol;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float g0 = __uint_as_float(gv[e] << 16), g1 = __uint_as_float(gv[e] & 0xffff0000u);
        const float y0 = (v[j][2 * e] / r) * g0, y1 = (v[j][2 * e + 1] / r) * g1;
        const uint16_t h0 = f2bf(y0), h1 = f2bf(y1);
        oh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
        ol[e] = (uint32_t)f2bf_lo(y0, h0) | ((uint32_t)f2bf_lo(y1, h1) << 16);
      }
      const int64_t pi = packed_index(m, 8 * c, d);
      *(u32x4*)(out + pi) = oh;
      *(u32x4*)(out + out_plane + pi) = ol;
    }
  }
}

__global__ __launch_bounds__(256) void k_rmsnorm_f32(const float* __restrict__ x, const float* __restrict__ gain,
                                                     float eps, int d, int row0, float* __restrict__ out) {
  const int m = blockIdx.x;
  const float* xr = x + (int64_t)(row0 + m) * d;
  float ss = 0.f;
  for (int k = threadIdx.x; k < d; k += 256) ss += xr[k] * xr[k];
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  __shared__ float part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  const float tot = ((part[0] + part[1]) + part[2]) + part[3];
  const float r = sqrtf(tot / (float)d + eps);
  for (int k = threadIdx.x; k < d; k += 256) out[(int64_t)m * d + k] = (xr[k] / r) * gain[k];
}

hipError_t launch_rmsnorm(int dtype, float* x, const float* part, int nparts, int64_t part_stride, const void* gain,
                          float eps, int M, int d, int row0, void* out, int64_t out_plane, hipStream_t st) {
  if (nparts < 0 || nparts > kMaxSplitK) return hipErrorInvalidValue;  // the kernel adds at most kMaxSplitK planes
  if (dtype == 1)
    SDM_LAUNCH(k_rmsnorm_bf16, dim3(M), dim3(kNormThreads), 0, st, x, part, nparts, part_stride,
                       (const uint16_t*)gain, eps, d, row0, (uint16_t*)out, out_plane);
  else
    SDM_LAUNCH(k_rmsnorm_f32, dim3(M), dim3(256), 0, st, x, (const float*)gain, eps, d, row0, (float*)out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Vocab partial record: (max, lowest argmax, second max, sum exp(l - max)).
// ---------------------------------------------------------------------------
struct Rec {
  float mx;
  int idx;
  float mx2;
  float sum;
};
__device__ __forceinline__ Rec rec_empty() { return Rec{-INFINITY, 0x7fffffff, -INFINITY, 0.f}; }
__device__ __forceinline__ Rec rec_merge(const Rec& a, const Rec& b) {
  const bool a_top = a.mx > b.mx || (a.mx == b.mx && a.idx < b.idx);
  const Rec& t = a_top ? a : b;
  const Rec& o = a_top ? b : a;
  Rec r;
  r.mx = t.mx;
  r.idx = t.idx;
  r.mx2 = fmaxf(t.mx2, o.mx);
  r.sum = t.sum + (o.mx == -INFINITY ? 0.f : o.sum * __expf(o.mx - t.mx));
  return r;
}
__device__ __forceinline__ Rec rec_shfl_xor(const Rec& a, int o) {
  Rec r;
  r.mx = __shfl_xor(a.mx, o);
  r.idx = __shfl_xor(a.idx, o);
  r.mx2 = __shfl_xor(a.mx2, o);
  r.sum = __shfl_xor(a.sum, o);
  return r;
}
__device__ __forceinline__ float4 rec_pack(const Rec& a) { return make_float4(a.mx, __int_as_float(a.idx), a.mx2, a.sum); }
__device__ __forceinline__ Rec rec_unpack(const float4& v) { return Rec{v.x, __float_as_int(v.y), v.z, v.w}; }

// ---------------------------------------------------------------------------
// Epilogues of the bf16 GEMM.  c[16] is a 32x32 C tile in the MFMA layout:
// column m = tile row-of-activations (lane % 32), rows crow(r, lane / 32).
// EpiPre holds the epilogue's inputs that do not depend on the product (RoPE
// cos/sin and the KV page); the GEMM loads it before its K
// loop so those loads' latency hides behind the weight stream.
// ---------------------------------------------------------------------------
struct EpiPre {
  float v[16];
  int pos, page;
};

template <int EPI>
__device__ __forceinline__ void epi_preload(EpiPre& p, int nt, int mt, int lane, const EpiArgs& ea) {
  const int h = lane >> 5;
  const int m = mt * 32 + (lane & 31);
  if (m >= ea.M) return;
  if constexpr (EPI == EPI_QKV) {
    const int slot = m / ea.slots.T, t = m % ea.slots.T;
    const int seq = ea.slots.ids[slot];
    p.pos = ea.slots.len[slot] + t;
    p.page = is_candidate(ea.slots, slot) ? -1 - (slot - ea.slots.xslot0)  // scratch page of the candidate
                                          : ea.kv.page_table[(int64_t)seq * ea.kv.max_pages + p.pos / kPageTokens];
    const int head = nt >> 2, s4 = nt & 3;
    if (head < ea.Hq + ea.kv.Hkv) {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int dl = 16 * s4 + crow(r, h);
        p.v[r] = ea.rope_cos[(int64_t)p.pos * (kHd / 2) + dl];
        p.v[8 + r] = ea.rope_sin[(int64_t)p.pos * (kHd / 2) + dl];
      }
    }
  }
}

template <int EPI, bool PRE>
__device__ __forceinline__ void gemm_epilogue(const float (&c)[16], int nt, int mt, int sk, int lane,
                                              const EpiArgs& ea, const EpiPre& pre_in) {
  const int h = lane >> 5;
  const int m = mt * 32 + (lane & 31);
  const bool valid = m < ea.M;
  if constexpr (EPI == EPI_QKV) {
    if (!valid) return;
    EpiPre pre_local;
    if constexpr (!PRE) epi_preload<EPI_QKV>(pre_local, nt, mt, lane, ea);
    const EpiPre& pre = PRE ? pre_in : pre_local;
    const int pos = pre.pos;
    const int head = nt >> 2, s4 = nt & 3;
    const int Hq = ea.Hq, Hkv = ea.kv.Hkv;
    // a candidate slot's K/V go to its scratch page, key t at page position t
    const bool own = pre.page < 0;
    uint16_t* pool = own ? (uint16_t*)ea.kv.xpool : (uint16_t*)ea.kv.pool;
    const int pk = own ? m % ea.slots.T : pos % kPageTokens;
    uint16_t* kblk = nullptr;
    uint16_t* vblk = nullptr;
    if (head >= Hq) {
      const int64_t base = own ? (int64_t)(-1 - pre.page) * ea.kv.x_page_elems
                               : (int64_t)pre.page * ea.kv.page_elems + ea.kv.layer_off;
      if (head < Hq + Hkv) kblk = pool + base + (int64_t)(head - Hq) * kPageTokens * kHd;
      else vblk = pool + base + (int64_t)(Hkv + head - Hq - Hkv) * kPageTokens * kHd;
    }
    // registers r (dims dl) and r + 8 (dims dl + 64) after RoPE, rounded
    uint16_t hb[16], lb[16];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float y1 = c[r], y2 = c[r + 8];
      if (head < Hq + Hkv) {
        const float cs = pre.v[r], sn = pre.v[8 + r];
        const float x1 = y1, x2 = y2;
        y1 = x1 * cs - x2 * sn;
        y2 = x2 * cs + x1 * sn;
      }
      hb[r] = f2bf(y1);
      hb[r + 8] = f2bf(y2);
      lb[r] = f2bf_lo(y1, hb[r]);
      lb[r + 8] = f2bf_lo(y2, hb[r + 8]);
    }
    // registers 4i..4i+3 hold 4 consecutive dims, contiguous in the packed q
    // and K layouts: one 8-byte store per group
    auto pack4 = [](const uint16_t* v) {
      return make_uint2((uint32_t)v[0] | ((uint32_t)v[1] << 16), (uint32_t)v[2] | ((uint32_t)v[3] << 16));
    };
    if (head < Hq) {
      const int G = Hq / Hkv, T = ea.slots.T;
      const int cq = (head % G) * T + m % T;  // query column within the KV head's group
      uint16_t* q = ea.q_out + ((int64_t)(m / T) * Hkv + head / G) * ea.q_nq_pad * kHd;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 16 * s4 + crow(4 * (i & 1), h) + 64 * (i >> 1);
        const int64_t pi = packed_index(cq, d0, kHd);
        *(uint2*)(q + pi) = pack4(hb + 4 * i);
        *(uint2*)(q + ea.q_plane + pi) = pack4(lb + 4 * i);
      }
    } else if (kblk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = 16 * s4 + crow(4 * (i & 1), h) + 64 * (i >> 1);
        *(uint2*)(kblk + kv_k_index(pk, d0)) = pack4(hb + 4 * i);
      }
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int dl = 16 * s4 + crow(r, h);
        vblk[kv_v_index(pk, dl)] = hb[r];
        vblk[kv_v_index(pk, dl + 64)] = hb[r + 8];
      }
    }
  } else if constexpr (EPI == EPI_PARTIAL) {
    if (!valid) return;
    // rows crow(4j + i, h) = 8j + 4h + i: four contiguous floats per j
    float* pr = ea.part + (int64_t)sk * ea.part_stride + (int64_t)m * ea.d + nt * 32 + 4 * h;
#pragma unroll
    for (int j = 0; j < 4; ++j) *(float4*)(pr + 8 * j) = make_float4(c[4 * j], c[4 * j + 1], c[4 * j + 2], c[4 * j + 3]);
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (!valid) return;
    // registers 4i..4i+3 are features 16 nt + 8i + 4h + 0..3, contiguous in
    // the packed layout: one 8-byte store per plane and group
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      uint32_t hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * i + e;
        const float g = c[r], u = c[r + 8];
        const float s = g / (1.f + expf(-g));
        const float y = s * u;
        const uint16_t hb = f2bf(y), lb = f2bf_lo(y, hb);
        if (e & 1) {
          hw[e >> 1] |= (uint32_t)hb << 16;
          lw[e >> 1] |= (uint32_t)lb << 16;
        } else {
          hw[e >> 1] = hb;
          lw[e >> 1] = lb;
        }
      }
      const int64_t pi = packed_index(m, 16 * nt + crow(4 * i, h), ea.F);
      *(uint2*)(ea.h_out + pi) = make_uint2(hw[0], hw[1]);
      *(uint2*)(ea.h_out + ea.h_plane + pi) = make_uint2(lw[0], lw[1]);
    }
  } else {  // EPI_LOGITS
    Rec a = rec_empty();
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int n = nt * 32 + crow(r, h);
      if (valid && ea.logits) ea.logits[(int64_t)m * ea.V + n] = c[r];
      if (n != ea.mask_id) a = rec_merge(a, Rec{c[r], n, -INFINITY, 1.f});
    }
    const Rec b = rec_shfl_xor(a, 32);
    a = rec_merge(a, b);
    if (valid && h == 0) ea.records[(int64_t)m * ea.n_vtiles + nt] = rec_pack(a);
  }
}

// ---------------------------------------------------------------------------
// Skinny bf16 GEMM  Y[m, n] = sum_k X[m, k] W[n, k]  (fp32 accumulate), X
// given as hi/lo planes: per 16-column block the hi product then the lo
// product go into the same accumulator.
// grid (NT / TP, S, ceil(MTILES / MT)); WAVES waves per workgroup.  Workgroup
// x owns the TP consecutive 32-row weight tiles from TP * x over its K range
// (split sk of S); its waves take that range in 4-block chunks, round robin,
// streaming the packed weights once (1 KiB per tile per wave per load,
// non-temporal) and the activation tiles from L2 -- read once for all TP
// weight tiles.  The waves' partial tiles are summed through LDS in wave
// order, so the summation order depends only on (N, K, S, WAVES) -- never on
// the number of rows, on TP or on the load batch U: every row's result is
// independent of the batch it is computed in.  With TP > 1, wave t reduces and
// finishes tile t.
// ---------------------------------------------------------------------------
// Weight loads: streamed past the caches when a launch reads each weight tile
// once (up to 128 activation rows); cached otherwise, so that the activation
// groups after the first read the matrix from the memory-side cache.
template <int MT>
__device__ __forceinline__ u32x4 load_weight(const u32x4* p) {
  if constexpr (MT < 4) return __builtin_nontemporal_load(p);
  else return *p;
}

template <int EPI, int MT, int TP, int U, int WAVES, bool XMASK = false>
__global__ __launch_bounds__(64 * WAVES) void k_gemm_bf16(const uint16_t* __restrict__ W,
                                                          const uint16_t* __restrict__ X, int64_t x_plane,
                                                          GemmShape g, EpiArgs ea) {
  static_assert(TP <= WAVES, "one finishing wave per weight tile");
  // grid (weight tile groups, K splits, activation groups); launches of four
  // activation tiles run a one-dimensional grid placed by many_row_place
  int nt0, sk, mg;
  if constexpr (MT == 4) {
    // the last weight-tile group may hold fewer than TP tiles
    const int ntg = (g.NT + TP - 1) / TP;
    const ManyRowPlace pl = many_row_place(blockIdx.x, ntg * g.S, (g.MTILES + 3) / 4);
    mg = pl.group;
    nt0 = (pl.unit / g.S) * TP;
    sk = pl.unit % g.S;
  } else {
    nt0 = blockIdx.x * TP;
    sk = blockIdx.y;
    mg = blockIdx.z;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int mt0 = mg * MT;
  const int mcount = min(MT, g.MTILES - mt0);
  const int kbs = g.KB / g.S;  // this workgroup's K range: [sk * kbs, (sk + 1) * kbs)
  // The range goes to the waves in chunks of kGemmChunk k-blocks, round robin,
  // so the workgroup's loads at any moment form one sequential stream; a wave
  // sums its blocks in increasing order (blocks past the last whole chunk go
  // round robin one at a time).  U only batches the loads.
  static_assert(U % kGemmChunk == 0, "loads are batched in whole chunks");
  const int kbase = sk * kbs;
  const int nch = kbs / kGemmChunk;
  constexpr int CB = U / kGemmChunk;                // chunks per load batch
  constexpr int kstep = WAVES * kGemmChunk;         // from one of this wave's chunks to its next
  const int kfull = kbase + nch * kGemmChunk;       // end of the whole chunks
  // block u of a batch starting at this wave's chunk c: a compile-time offset
  // from the batch's first block
  auto boff = [](int u) { return (u / kGemmChunk) * WAVES * kGemmChunk + u % kGemmChunk; };

  f32x16 acc[MT][TP];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < TP; ++t) acc[i][t] = f32x16{0};

  EpiPre pre;
  if constexpr (MT == 1) {
    if (wave < TP) epi_preload<EPI>(pre, nt0 + wave, mt0, lane, ea);
  }

  // tiles of this group: TP, or fewer in a ragged last group of a many-row
  // launch, whose missing tiles load tile nt0 again and are not finished
  const int tvalid = MT == 4 ? min(TP, g.NT - nt0) : TP;
  auto tl = [&](int t) { return MT == 4 && t >= tvalid ? 0 : t; };
  // launches of one or two activation tiles hold exactly that many rows'
  // tiles (the launcher picks MT from the tile count); four-tile launches
  // skip the tiles past the rows
  auto use = [&](int i) { return MT <= 2 || i < mcount; };
  const u32x4* wp = (const u32x4*)W + (int64_t)nt0 * g.KB * 64 + lane;  // tile nt0 + t at t * KB * 64
  const u32x4* xp = (const u32x4*)X + (int64_t)mt0 * g.KB * 64 + lane;
  const u32x4* xq = xp + (x_plane >> 3);  // lo plane
  // XMASK (a one-tile launch of fewer than 32 rows, such as a one-row AR
  // step): only the lanes of the launch's rows load activations; the other
  // operand columns stay zero, and an MFMA output column depends on its own
  // operand column alone, so the rows' results are the same bits.
  static_assert(!XMASK || MT == 1, "row masking serves one-tile launches");
  const bool xrow = !XMASK || (lane & 31) < g.ROWS;
  int kb = kbase + wave * kGemmChunk;  // first block of this wave's next chunk
  u32x4 xh[MT][U], xl[MT][U];
  if constexpr (XMASK) {
#pragma unroll
    for (int u = 0; u < U; ++u) xh[0][u] = xl[0][u] = u32x4{0u, 0u, 0u, 0u};
  }
  for (; kb + (CB - 1) * kstep + kGemmChunk <= kfull; kb += CB * kstep) {
    u32x4 wv[TP][U];
#pragma unroll
    for (int t = 0; t < TP; ++t)
#pragma unroll
      for (int u = 0; u < U; ++u) wv[t][u] = load_weight<MT>(wp + ((int64_t)tl(t) * g.KB + kb + boff(u)) * 64);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (use(i) && xrow) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t o = ((int64_t)i * g.KB + kb + boff(u)) * 64;
          xh[i][u] = xp[o];
          xl[i][u] = xq[o];
        }
      }
    // a few-row launch requests its whole batch before the first product
    // (the compiler would otherwise trade loads in flight for registers)
    if constexpr (MT <= 2) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < TP; ++t)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (use(i)) {
            acc[i][t] = mfma32(wv[t][u], xh[i][u], acc[i][t]);
            acc[i][t] = mfma32(wv[t][u], xl[i][u], acc[i][t]);
          }
  }
  auto one_block = [&](int kb) {
    u32x4 wv[TP];
#pragma unroll
    for (int t = 0; t < TP; ++t) wv[t] = load_weight<MT>(wp + ((int64_t)tl(t) * g.KB + kb) * 64);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      if (use(i)) {
        const int64_t o = ((int64_t)i * g.KB + kb) * 64;
        u32x4 xh = u32x4{0u, 0u, 0u, 0u}, xl = u32x4{0u, 0u, 0u, 0u};
        if (xrow) {
          xh = xp[o];
          xl = xq[o];
        }
#pragma unroll
        for (int t = 0; t < TP; ++t) {
          acc[i][t] = mfma32(wv[t], xh, acc[i][t]);
          acc[i][t] = mfma32(wv[t], xl, acc[i][t]);
        }
      }
  };
  for (; kb + kGemmChunk <= kfull; kb += kstep) {
#pragma unroll
    for (int u = 0; u < kGemmChunk; ++u) one_block(kb + u);
  }
  for (int b = nch * kGemmChunk + wave; b < kbs; b += WAVES) one_block(kbase + b);

  if constexpr (MT == 1) {
    // all TP tiles through LDS at once, a lane's 16 values as four 16-byte
    // words, word i at slot i ^ sw (lanes 4j..4j+3 of each 16 then hit
    // different banks); wave t sums tile t over the waves in order
    __shared__ float4 red[TP][WAVES][64][4];
    const int sw = (lane >> 2) & 3;
#pragma unroll
    for (int t = 0; t < TP; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[t][wave][lane][i ^ sw] = make_float4(acc[0][t][4 * i], acc[0][t][4 * i + 1], acc[0][t][4 * i + 2],
                                                 acc[0][t][4 * i + 3]);
    __syncthreads();
    if (wave < TP) {
      float c[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 v = red[wave][0][lane][i ^ sw];
#pragma unroll
        for (int w = 1; w < WAVES; ++w) {
          const float4 u = red[wave][w][lane][i ^ sw];
          v.x += u.x;
          v.y += u.y;
          v.z += u.z;
          v.w += u.w;
        }
        c[4 * i] = v.x;
        c[4 * i + 1] = v.y;
        c[4 * i + 2] = v.z;
        c[4 * i + 3] = v.w;
      }
      gemm_epilogue<EPI, true>(c, nt0 + wave, mt0, sk, lane, ea, pre);
    }
  } else {
    // the MT x TP output tiles (activation tile major) go through LDS
    // WAVES at a time; wave s sums tile q0 + s over the waves in order and
    // finishes it
    __shared__ float red[WAVES][WAVES][16][64];
    const int ntile = mcount * TP;
#pragma unroll
    for (int q0 = 0; q0 < MT * TP; q0 += WAVES) {
      if (q0 >= ntile) break;
      if (q0 > 0) __syncthreads();
#pragma unroll
      for (int qs = 0; qs < WAVES; ++qs)
        if (q0 + qs < MT * TP && q0 + qs < ntile) {
#pragma unroll
          for (int r = 0; r < 16; ++r) red[qs][wave][r][lane] = acc[(q0 + qs) / TP][(q0 + qs) % TP][r];
        }
      __syncthreads();
      const int q = q0 + wave;
      if (q < ntile && q % TP < tvalid) {
        float c[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = red[wave][0][r][lane];
#pragma unroll
          for (int w = 1; w < WAVES; ++w) v += red[wave][w][r][lane];
          c[r] = v;
        }
        gemm_epilogue<EPI, false>(c, nt0 + q % TP, mt0 + q / TP, sk, lane, ea, pre);
      }
    }
  }
}

template <int EPI, int WAVES>
static void launch_gemm_w(const uint16_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g, const EpiArgs& ea,
                          hipStream_t st) {
  const int MT = g.MTILES <= 1 ? 1 : (g.MTILES == 2 ? 2 : 4);
  const int TP = g.TP;
  const int mgroups = (g.MTILES + MT - 1) / MT;
  const dim3 grd = MT == 4 ? dim3(mgroups * ((g.NT + TP - 1) / TP) * g.S) : dim3(g.NT / TP, g.S, mgroups),
             blk(64 * WAVES);
  // weight loads in flight per wave: 16 tiles at TP 1, 4 * TP otherwise
  constexpr int U1 = WAVES == 8 ? 8 : 16;
  if (MT == 1 && g.ROWS < 32) {
    // fewer rows than the tile: only those rows' activation lanes load
    if (TP == 1) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 1, U1, WAVES, true>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 2, 4, WAVES, true>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 3) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 3, 4, WAVES, true>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_bf16<EPI, 1, 4, 4, WAVES, true>), grd, blk, 0, st, W, X, x_plane, g, ea);
  } else if (MT == 1) {
    if (TP == 1) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 1, U1, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 2, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 3) SDM_LAUNCH((k_gemm_bf16<EPI, 1, 3, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_bf16<EPI, 1, 4, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
  } else if (MT == 2) {
    if (TP == 1) SDM_LAUNCH((k_gemm_bf16<EPI, 2, 1, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_bf16<EPI, 2, 2, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 3) SDM_LAUNCH((k_gemm_bf16<EPI, 2, 3, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_bf16<EPI, 2, 4, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
  } else {
    if (TP == 1) SDM_LAUNCH((k_gemm_bf16<EPI, 4, 1, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_bf16<EPI, 4, 2, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_bf16<EPI, 4, 3, 4, WAVES>), grd, blk, 0, st, W, X, x_plane, g, ea);
  }
}

template <int EPI>
static hipError_t launch_gemm_epi(const uint16_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                                  const EpiArgs& ea, hipStream_t st) {
  if (g.WAVES != 4) return hipErrorInvalidValue;  // every configuration runs four waves
  launch_gemm_w<EPI, 4>(W, X, x_plane, g, ea, st);
  return hipGetLastError();
}

hipError_t launch_gemm_bf16(int epi, const uint16_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                            const EpiArgs& ea, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return launch_gemm_epi<EPI_QKV>(W, X, x_plane, g, ea, st);
    case EPI_SWIGLU: return launch_gemm_epi<EPI_SWIGLU>(W, X, x_plane, g, ea, st);
    case EPI_PARTIAL: return launch_gemm_epi<EPI_PARTIAL>(W, X, x_plane, g, ea, st);
    default: return launch_gemm_epi<EPI_LOGITS>(W, X, x_plane, g, ea, st);
  }
}

// ---------------------------------------------------------------------------
// 4-bit weights (w4a16): packing and GEMM.
// The weight is scale * code with a two's-complement 4-bit code and one bf16
// scale per output row and group of 128 inputs.  The GEMM feeds each code to
// the bf16 MFMA as the exact bf16 integer it is, sums a group's products
// (activation hi and lo planes, as for bf16 weights) from zero, and adds
// scale * group sum to the running total in fp32: in exact arithmetic the
// product of the activations with the dequantized matrix.
// ---------------------------------------------------------------------------
__global__ void k_pack_w4_codes(int kind, const uint32_t* __restrict__ src, int which, uint32_t* __restrict__ dst,
                                int64_t rows, int64_t cols, int head_dim) {
  const int64_t words = cols / 8;  // source words of 8 codes per row
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * words) return;
  const int64_t r = i / words, c0 = (i % words) * 8;
  const int64_t pr = pack_row(kind, r, rows, which, head_dim);
  const int64_t G = cols / kW4Group, grp = c0 / kW4Group;
  const int kb = (int)((c0 % kW4Group) / 16), half = (int)((c0 % 16) / 8);
  const int64_t lane = (pr & 31) + 32 * half;
  dst[((((pr >> 5) * G + grp) * 2 + kb / 4) * 64 + lane) * 4 + kb % 4] = src[i];
}

__global__ void k_pack_w4_scales(int kind, const uint16_t* __restrict__ src, int which, uint16_t* __restrict__ dst,
                                 int64_t rows, int64_t G, int head_dim) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * G) return;
  const int64_t r = i / G, grp = i % G;
  const int64_t pr = pack_row(kind, r, rows, which, head_dim);
  const int rr = (int)(pr & 31);
  const int h = (rr >> 2) & 1, reg = 4 * (rr >> 3) + (rr & 3);  // crow(reg, h) == rr
  dst[(((pr >> 5) * G + grp) * 2 + h) * 16 + reg] = src[i];
}

hipError_t launch_pack_w4(int kind, const void* codes, const void* scales, const void* codes2, const void* scales2,
                          void* dst, int64_t rows, int64_t cols, int head_dim, hipStream_t st) {
  const int64_t out_rows = kind == 2 ? 2 * rows : rows;
  uint32_t* dc = (uint32_t*)dst;
  uint16_t* ds = (uint16_t*)((uint8_t*)dst + w4_scale_offset(out_rows, cols));
  const int64_t nc = rows * (cols / 8), ns = rows * (cols / kW4Group);
  const dim3 blk(256), gc((unsigned)((nc + 255) / 256)), gs((unsigned)((ns + 255) / 256));
  for (int which = 0; which < (kind == 2 ? 2 : 1); ++which) {
    const void* c = which ? codes2 : codes;
    const void* sc = which ? scales2 : scales;
    SDM_LAUNCH(k_pack_w4_codes, gc, blk, 0, st, kind, (const uint32_t*)c, which, dc, rows, cols, head_dim);
    SDM_LAUNCH(k_pack_w4_scales, gs, blk, 0, st, kind, (const uint16_t*)sc, which, ds, rows, cols / kW4Group,
               head_dim);
  }
  return hipGetLastError();
}

// The 8 codes of one k-block of a lane (nibble e at bits 4e) as the bf16 MFMA
// operand, times 16: 4 words, each two bf16 integers 16 * q (element 2j low,
// 2j + 1 high).  Moving a nibble to the top of a byte makes the byte the
// signed integer 16 * q, which converts to fp32 exactly (a byte-select
// convert); its bf16 bits are the top half.  The factor 16 is a power of two:
// every group sum, and every running total built from them, is exactly 16
// times the unscaled one (no rounding differs), and the kernel divides the
// totals by 16 once at the end.
__device__ __forceinline__ u32x4 w4_operand(uint32_t w) {
  const uint32_t even = (w << 4) & 0xF0F0F0F0u, odd = w & 0xF0F0F0F0u;  // codes 2j / 2j + 1 in byte j
  u32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float f0 = (float)(int8_t)(even >> (8 * j));
    const float f1 = (float)(int8_t)(odd >> (8 * j));
    r[j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return r;
}

// Scale r (0..15) of this lane's half from the two words of 8 bf16 each.
__device__ __forceinline__ float w4_scale(const u32x4 (&s)[2], int r) {
  const uint32_t u = s[r >> 3][(r >> 1) & 3];
  return __uint_as_float((r & 1) ? (u & 0xffff0000u) : (u << 16));
}

// Grid (NT / TP, S, ceil(MTILES / MT)), kW4Waves waves (two per SIMD, so
// one wave's code conversion overlaps the other's loads and products).  The
// workgroup's K range goes to the waves by scale group, round robin; a wave
// adds its groups in increasing order and the waves' totals meet in LDS in
// wave order, so a row's result does not depend on the batch it is in.
template <int EPI, int MT, int TP, bool XMASK = false>
__global__ __launch_bounds__(64 * kW4Waves) void k_gemm_w4(const uint8_t* __restrict__ Wc,
                                                           const uint16_t* __restrict__ Ws,
                                                           const uint16_t* __restrict__ X, int64_t x_plane,
                                                           GemmShape g, EpiArgs ea) {
  constexpr int WAVES = kW4Waves, GB = kW4GroupBlocks;
  static_assert(MT * TP <= 4, "a wave holds a total and a group sum per tile");
  const int nt0 = blockIdx.x * TP, sk = blockIdx.y, mg = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63, h = lane >> 5;
  const int mt0 = mg * MT;
  const int mcount = min(MT, g.MTILES - mt0);
  const int kbs = g.KB / g.S;      // this workgroup's K range in k-blocks
  const int G = g.KB / GB;         // scale groups of a row
  const int g0 = sk * kbs / GB;    // first group of the range
  const int ngr = kbs / GB;

  f32x16 tot[MT][TP];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < TP; ++t) tot[i][t] = f32x16{0};

  EpiPre pre;
  if constexpr (MT == 1) {
    if (wave < TP) epi_preload<EPI>(pre, nt0 + wave, mt0, lane, ea);
  }

  // uniform bases, indexed with the lane's offset at each load (no per-lane
  // pointer stays live across the loop)
  const u32x4* wc = (const u32x4*)Wc;  // tile nt, group gr, part p at ((nt * G + gr) * 2 + p) * 64 + lane
  const u32x4* ws = (const u32x4*)Ws;  // tile nt, group gr at (nt * G + gr) * 4 + 2 * h
  const u32x4* xp = (const u32x4*)X + (int64_t)mt0 * g.KB * 64;
  const u32x4* xq = xp + (x_plane >> 3);  // lo plane
  // XMASK (a one-tile launch of fewer than 32 rows): only its rows' lanes
  // load activations; the other operand columns stay zero, and the rows'
  // results are the same bits
  static_assert(!XMASK || MT == 1, "row masking serves one-tile launches");
  const bool xrow = !XMASK || (lane & 31) < g.ROWS;
  for (int gi = wave; gi < ngr; gi += WAVES) {
    const int gr = g0 + gi;
    u32x4 cw[TP][2], sw[TP][2];
#pragma unroll
    for (int t = 0; t < TP; ++t) {
      const int64_t tg = (int64_t)(nt0 + t) * G + gr;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        cw[t][p] = load_weight<MT>(wc + (tg * 2 + p) * 64 + lane);
        sw[t][p] = ws[tg * 4 + p + 2 * h];
      }
    }
    f32x16 acc[MT][TP];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < TP; ++t) acc[i][t] = f32x16{0};
#pragma unroll
    for (int b = 0; b < GB; ++b) {
      u32x4 xh[MT], xl[MT];
      if constexpr (XMASK) xh[0] = xl[0] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int i = 0; i < MT; ++i)
        if ((MT <= 2 || i < mcount) && xrow) {
          const int64_t o = ((int64_t)i * g.KB + gr * GB + b) * 64;
          xh[i] = xp[o + lane];
          xl[i] = xq[o + lane];
        }
#pragma unroll
      for (int t = 0; t < TP; ++t) {
        const u32x4 a = w4_operand(cw[t][b >> 2][b & 3]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          if (MT <= 2 || i < mcount) {
            acc[i][t] = mfma32(a, xh[i], acc[i][t]);
            acc[i][t] = mfma32(a, xl[i], acc[i][t]);
          }
      }
    }
#pragma unroll
    for (int t = 0; t < TP; ++t)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float sc = w4_scale(sw[t], r);
#pragma unroll
        for (int i = 0; i < MT; ++i) tot[i][t][r] = __builtin_fmaf(sc, acc[i][t][r], tot[i][t][r]);
      }
  }

  // The MT x TP output tiles (activation tile major, at most 4) go through
  // LDS; wave q sums tile q over the waves in order (after undoing
  // w4_operand's factor 16, exactly) and finishes it.
  // a lane's 16 values as four 16-byte words, word i at slot i ^ sw (lanes
  // 4j..4j+3 of each 16 then hit different banks)
  __shared__ float4 red[4][WAVES][64][4];
  const int ntile = mcount * TP;
  const int sw = (lane >> 2) & 3;
#pragma unroll
  for (int q = 0; q < MT * TP; ++q)
    if (q < ntile) {
      const f32x16& tq = tot[q / TP][q % TP];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        red[q][wave][lane][i ^ sw] = make_float4(tq[4 * i] * 0.0625f, tq[4 * i + 1] * 0.0625f,
                                                 tq[4 * i + 2] * 0.0625f, tq[4 * i + 3] * 0.0625f);
    }
  __syncthreads();
  if (wave < ntile) {
    float c[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float4 v = red[wave][0][lane][i ^ sw];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) {
        const float4 u = red[wave][w][lane][i ^ sw];
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      c[4 * i] = v.x;
      c[4 * i + 1] = v.y;
      c[4 * i + 2] = v.z;
      c[4 * i + 3] = v.w;
    }
    if constexpr (MT == 1) gemm_epilogue<EPI, true>(c, nt0 + wave, mt0, sk, lane, ea, pre);
    else gemm_epilogue<EPI, false>(c, nt0 + wave % TP, mt0 + wave / TP, sk, lane, ea, pre);
  }
}

template <int EPI>
static hipError_t launch_gemm_w4_epi(const uint8_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                                     const EpiArgs& ea, hipStream_t st) {
  const int MT = g.MTILES <= 1 ? 1 : (g.MTILES == 2 ? 2 : 4);
  const int TP = g.TP;
  if (g.WAVES != kW4Waves || MT * TP > 4 || g.NT % TP || g.KB % (g.S * kW4GroupBlocks)) return hipErrorInvalidValue;
  const uint16_t* Ws = (const uint16_t*)(W + w4_scale_offset((int64_t)g.NT * 32, (int64_t)g.KB * 16));
  const dim3 grd(g.NT / TP, g.S, (g.MTILES + MT - 1) / MT), blk(64 * kW4Waves);
  if (MT == 1 && g.ROWS < 32) {
    // fewer rows than the tile: only those rows' activation lanes load
    if (TP == 1) SDM_LAUNCH((k_gemm_w4<EPI, 1, 1, true>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_w4<EPI, 1, 2, true>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else if (TP == 3) SDM_LAUNCH((k_gemm_w4<EPI, 1, 3, true>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_w4<EPI, 1, 4, true>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
  } else if (MT == 1) {
    if (TP == 1) SDM_LAUNCH((k_gemm_w4<EPI, 1, 1>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else if (TP == 2) SDM_LAUNCH((k_gemm_w4<EPI, 1, 2>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else if (TP == 3) SDM_LAUNCH((k_gemm_w4<EPI, 1, 3>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_w4<EPI, 1, 4>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
  } else if (MT == 2) {
    if (TP == 1) SDM_LAUNCH((k_gemm_w4<EPI, 2, 1>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
    else SDM_LAUNCH((k_gemm_w4<EPI, 2, 2>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
  } else {
    SDM_LAUNCH((k_gemm_w4<EPI, 4, 1>), grd, blk, 0, st, W, Ws, X, x_plane, g, ea);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_w4(int epi, const uint8_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                          const EpiArgs& ea, hipStream_t st) {
  switch (epi) {
    case EPI_QKV: return launch_gemm_w4_epi<EPI_QKV>(W, X, x_plane, g, ea, st);
    case EPI_SWIGLU: return launch_gemm_w4_epi<EPI_SWIGLU>(W, X, x_plane, g, ea, st);
    case EPI_PARTIAL: return launch_gemm_w4_epi<EPI_PARTIAL>(W, X, x_plane, g, ea, st);
    default: return hipErrorInvalidValue;  // the LM head keeps bf16 weights
  }
}

// ---------------------------------------------------------------------------
// Block attention, bf16, head_dim 128, over the paged cache.
// The unit of work is a 64-key page (one KV page of head g) against a query
// tile of 32 columns; the query columns of KV head g are (q head of the
// group, block row).  A page's state (max m, sum l, O) is formed by two
// 32-key tiles: S^T = K Q^T on MFMA (keys x query columns; with QLO the
// query's hi and lo planes both enter the product), an online softmax per
// column, then O^T += V^T P^T on MFMA with P split into bf16 hi + lo parts so
// the product keeps ~16 bits of P.  The four page states of a 256-key split
// are merged in page order, pairwise (empty pages included), into the
// split's partial; the combine kernel merges splits in split order.  Masked
// keys contribute exact zeros and every key range is absolute, so a row's
// result does not depend on how many rows the block has -- nor on which of
// the three launch shapes below computed it:
//   k_attn_bf16        one workgroup per (split, KV head, query tile); wave w
//                      takes page w into registers, the page states meet in
//                      LDS (short contexts: many small workgroups);
//   k_attn_staged_bf16 one workgroup per (split, KV head, group of query
//                      tiles: four, the last up to seven); the four pages go
//                      through LDS once and wave t runs the group's query
//                      tiles t, t+4 over all four (long contexts, batches and
//                      many-row prefill chunks);
//   k_attn_stream_bf16 one workgroup per run of splits of a KV head; pages
//                      stream through two LDS buffers, the next one loading
//                      while the current one is computed (long contexts with
//                      at most four query tiles, no candidate slots).
// ---------------------------------------------------------------------------
// A split's partial O, per (slot, KV head, split): [head_dim / 4][column]
// float4s, so that a wave's lanes (consecutive columns) write and read four
// consecutive dims each in one coalesced 16-byte access.
__device__ __forceinline__ float4* attn_opart4(const AttnArgs& a, int64_t base_idx, int d4, int c) {
  return (float4*)a.opart + (base_idx * (kHd / 4) + d4) * a.nq_pad + c;
}

struct AttnState {
  float m, l;
  f32x16 o[4];  // O^T: dims dt * 32 + crow(r, h), this lane's query column
};

// State of one page (keys [jw, jw + 64)) for this lane's query column.
// kop(i) / vop(i) give the page's K / V^T operand tile i for this lane.
template <bool QLO, class KOp, class VOp>
__device__ __forceinline__ void attn_page_state(const AttnArgs& a, KOp kop, VOp vop, const u32x4 (&qop)[8],
                                                const u32x4 (&qlo)[QLO ? 8 : 1], int jw, int nkeys, int n,
                                                int qpos, bool cval, int h, AttnState& st) {
  st.m = -INFINITY;
  st.l = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) st.o[i] = f32x16{0};
  const int jw1 = min(jw + 64, nkeys);
  // key j is visible to this lane's query iff j < nkeys and (j < n, or the
  // block is bidirectional, or j <= qpos): one bound per lane, 0 (none) for a
  // column past the query tiles
  const int lim = !cval ? 0 : a.mode == BIDIR ? nkeys : min(nkeys, max(n, qpos + 1));
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int jt = jw + 32 * kt;
    if (jt >= jw1) break;  // wave-uniform
    f32x16 sacc = f32x16{0};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      const u32x4 kv = kop(kt * 8 + kb);
      sacc = mfma32(kv, qop[kb], sacc);
      if constexpr (QLO) sacc = mfma32(kv, qlo[kb], sacc);
    }
    float sv[16];
    float mx = -INFINITY;
    // key jt + crow(r, h) is visible iff it is below lim: crow(r, h) - 4h is a
    // compile-time row offset
    const int lt = lim - jt - 4 * h;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = (8 * (r >> 2) + (r & 3)) < lt ? sacc[r] * a.scale : -INFINITY;
      mx = fmaxf(mx, sv[r]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m, mx);
    const float alpha = (st.m == -INFINITY) ? 0.f : __expf(st.m - m_new);
    // a masked score (-inf) gives exp(-inf) = 0; m_safe keeps a lane whose
    // keys are all masked so far (m_new = -inf) away from -inf - -inf
    const float m_safe = (m_new == -INFINITY) ? 0.f : m_new;
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sv[r] = __expf(sv[r] - m_safe);
      psum += sv[r];
    }
    psum += __shfl_xor(psum, 32);
    st.l = st.l * alpha + psum;
    st.m = m_new;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[i][r] *= alpha;
#pragma unroll
    for (int ka = 0; ka < 2; ++ka) {
      // P as two bf16 terms: hi = R(p), lo = R(p - hi), two values at a time
      u32x4 phi, plo;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = sv[8 * ka + 2 * e], p1 = sv[8 * ka + 2 * e + 1];
        const uint32_t hp = f2bf2(p0, p1);
        phi[e] = hp;
        plo[e] = f2bf2(p0 - __uint_as_float(hp << 16), p1 - __uint_as_float(hp & 0xffff0000u));
      }
      const int kbv = 2 * kt + ka;  // 16-key group inside the page
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const u32x4 vv = vop(dt * 4 + kbv);
        st.o[dt] = mfma32(vv, phi, st.o[dt]);
        st.o[dt] = mfma32(vv, plo, st.o[dt]);
      }
    }
  }
}

// Pairwise merge coefficients of a running state (m_a) with a page state
// (m_b): the merged state is (max, a * l_a + b * l_b, a * O_a + b * O_b).
__device__ __forceinline__ void attn_merge_coef(float m_a, float m_b, float& M, float& ca, float& cb) {
  M = fmaxf(m_a, m_b);
  ca = (m_a == -INFINITY) ? 0.f : __expf(m_a - M);
  cb = (m_b == -INFINITY) ? 0.f : __expf(m_b - M);
}

// This lane's query tile operands (QPACK: the QKV epilogue's packed layout,
// columns past nq hold stale values whose scores are masked; else row-major).
template <bool QLO, bool QPACK>
__device__ __forceinline__ void attn_load_q(const AttnArgs& a, int slot, int g, int qt, int t, int head, bool cval,
                                            int lane, u32x4 (&qop)[8], u32x4 (&qlo)[QLO ? 8 : 1]) {
  const int h = lane >> 5;
  if constexpr (QPACK) {
    const u32x4* qp = (const u32x4*)(a.q + ((int64_t)slot * a.kv.Hkv + g) * a.nq_pad * kHd) + qt * 8 * 64 + lane;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qop[kb] = qp[kb * 64];
    if constexpr (QLO) {
      const u32x4* ql = qp + (a.q_plane >> 3);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) qlo[kb] = ql[kb * 64];
    }
  } else {
    const int64_t qo = ((int64_t)(slot * a.slots.T + t) * a.Hq + head) * kHd;
    const u32x4* qp = (const u32x4*)(a.q + qo);
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) qop[kb] = cval ? qp[2 * kb + h] : u32x4{0, 0, 0, 0};
    if constexpr (QLO) {
      const u32x4* ql = (const u32x4*)(a.q + a.q_plane + qo);
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) qlo[kb] = cval ? ql[2 * kb + h] : u32x4{0, 0, 0, 0};
    }
  }
}

__device__ __forceinline__ const uint16_t* attn_page_base(const AttnArgs& a, int seq, int jw) {
  const int page = a.kv.page_table[(int64_t)seq * a.kv.max_pages + jw / kPageTokens];
  return (const uint16_t*)a.kv.pool + (int64_t)page * a.kv.page_elems + a.kv.layer_off;
}

// The keys of split sp of a slot.  A plain slot's splits cover keys
// [0, n + T) of its pages, those below n visible to every row and the block's
// by the mode.  A candidate slot's splits cover keys [0, n) of its pages, all
// visible, then one split over its own block in its scratch page (keys
// 0..T-1, all visible).  Wave w's page starts at key jw; keys [jw, jend)
// exist; keys below jall are visible to every row.
struct AttnKeys {
  bool own;
  int jend, jall, split0;  // split0: first key of the split
};
__device__ __forceinline__ AttnKeys attn_keys(const AttnArgs& a, int slot, int n, int T, int sp, int nsp) {
  AttnKeys k;
  const bool cand = is_candidate(a.slots, slot);
  k.own = cand && sp == nsp - 1;
  k.jend = k.own ? T : (cand ? n : n + T);
  k.jall = cand ? k.jend : n;
  k.split0 = k.own ? 0 : sp * kAttnSplitKeys;
  return k;
}
__device__ __forceinline__ const uint16_t* attn_keys_base(const AttnArgs& a, const AttnKeys& k, int slot, int seq,
                                                          int jw) {
  if (k.own) return (const uint16_t*)a.kv.xpool + (int64_t)(slot - a.slots.xslot0) * a.kv.x_page_elems;
  return attn_page_base(a, seq, jw);
}

// The four page states of one query tile (waves 0..3 hold pages 0..3 of a
// split) meet in LDS; attn_merge_store merges them per column in page order,
// pairwise, and writes the split's partial (all 256 threads; thread (col, dg)
// takes dims 16 dg .. 16 dg + 15 of column col).
struct AttnMergeLds {
  float ml[4][2][32];
  // O as [wave][column][dims / 4], padded to 33 float4 a column so that the
  // merge's 16-byte reads of consecutive columns spread over the banks
  float4 o[4][32][kHd / 4 + 1];
};
__device__ __forceinline__ void attn_merge_put(AttnMergeLds& sm, const AttnState& st, int wave, int lane) {
  const int h = lane >> 5;
  if (h == 0) {
    sm.ml[wave][0][lane & 31] = st.m;
    sm.ml[wave][1][lane & 31] = st.l;
  }
  // registers 4i..4i+3 of dims tile dt hold dims dt * 32 + 8i + 4h + 0..3
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sm.o[wave][lane & 31][dt * 8 + 2 * i + h] =
          make_float4(st.o[dt][4 * i], st.o[dt][4 * i + 1], st.o[dt][4 * i + 2], st.o[dt][4 * i + 3]);
}
__device__ __forceinline__ void attn_merge_store(const AttnArgs& a, const AttnMergeLds& sm, int64_t base_idx, int qt,
                                                 int nq) {
  const int col = threadIdx.x & 31, dg = threadIdx.x >> 5;
  const int cc = qt * 32 + col;
  if (cc >= nq) return;
  float ca[4], cb[4];
  float M = sm.ml[0][0][col], Lsum = sm.ml[0][1][col];
#pragma unroll
  for (int w = 1; w < 4; ++w) {
    float Mn;
    attn_merge_coef(M, sm.ml[w][0][col], Mn, ca[w], cb[w]);
    Lsum = ca[w] * Lsum + cb[w] * sm.ml[w][1][col];
    M = Mn;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    float4 v = sm.o[0][col][4 * dg + j];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 u = sm.o[w][col][4 * dg + j];
      v.x = ca[w] * v.x + cb[w] * u.x;
      v.y = ca[w] * v.y + cb[w] * u.y;
      v.z = ca[w] * v.z + cb[w] * u.z;
      v.w = ca[w] * v.w + cb[w] * u.w;
    }
    *attn_opart4(a, base_idx, 4 * dg + j, cc) = v;
  }
  if (threadIdx.x < 32) {
    a.mlpart[(base_idx * 2 + 0) * a.nq_pad + cc] = M;
    a.mlpart[(base_idx * 2 + 1) * a.nq_pad + cc] = Lsum;
  }
}

// Grid: linear id -> (pair = split * Hkv + g, query tile qt0 + j); workgroups
// sharing a pair get linear ids congruent mod 8 so that they are placed on
// the same XCD and share its L2 for the K/V pages.  qt0 > 0 when the staged
// shape runs the first qt0 tiles.
template <bool QLO, bool QPACK>
__global__ __launch_bounds__(256) void k_attn_bf16(AttnArgs a, int qt0) {
  __shared__ AttnMergeLds sm;
  const int slot = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int seq = a.slots.ids[slot];
  const int T = a.slots.T;
  const int n = a.slots.len[slot];
  const int Hkv = a.kv.Hkv;
  const int G = a.Hq / Hkv;
  const int nq = G * T;
  const int nqt = (nq + 31) >> 5;
  const int nsp = attn_splits(a.slots, slot);
  const int L = blockIdx.x;
  const int nsub = nqt - qt0;  // the query tiles of this launch
  const int qt = qt0 + (L % (8 * nsub)) / 8;
  const int pair = (L / (8 * nsub)) * 8 + (L % 8);
  if (pair >= nsp * Hkv) return;
  const int sp = pair / Hkv, g = pair % Hkv;
  const AttnKeys ks = attn_keys(a, slot, n, T, sp, nsp);
  const int jw = ks.split0 + 64 * wave;  // this wave's page of keys

  // K and V page blocks of head g for this wave's keys: 16 + 16 vectors per lane
  u32x4 kv_k[16], kv_v[16];
  if (jw < ks.jend) {
    const uint16_t* pb = attn_keys_base(a, ks, slot, seq, jw);
    const u32x4* kb = (const u32x4*)(pb + (int64_t)g * kPageTokens * kHd);
    const u32x4* vb = (const u32x4*)(pb + (int64_t)(Hkv + g) * kPageTokens * kHd);
#pragma unroll
    for (int i = 0; i < 16; ++i) kv_k[i] = kb[i * 64 + lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) kv_v[i] = vb[i * 64 + lane];
  }
  const int c = qt * 32 + (lane & 31);
  const bool cval = c < nq;
  const int hl = cval ? c / T : 0, t = cval ? c % T : 0;
  u32x4 qop[8], qlo[QLO ? 8 : 1];
  attn_load_q<QLO, QPACK>(a, slot, g, qt, t, g * G + hl, cval, lane, qop, qlo);
  AttnState st;
  attn_page_state<QLO>(a, [&](int i) { return kv_k[i]; }, [&](int i) { return kv_v[i]; }, qop, qlo, jw, ks.jend,
                       ks.jall, n + t, cval, h, st);
  // the page states meet in LDS; per column, merged in page order
  attn_merge_put(sm, st, wave, lane);
  __syncthreads();
  attn_merge_store(a, sm, ((int64_t)slot * Hkv + g) * a.max_splits + sp, qt, nq);
}

constexpr int kStagedLastGroup = 0, kStagedExact = 1, kStagedFold = 2;

template <bool QLO, bool QPACK>
__global__ __launch_bounds__(256) void k_attn_staged_bf16(AttnArgs a, int rem) {
  // the split's four pages (K operand tiles, then V^T operand tiles); with
  // rem == kStagedFold the same memory then holds the remainder tile's four
  // page states for their merge
  __shared__ u32x4 s_pages[2][4][16][64];
  u32x4 (&s_k)[4][16][64] = s_pages[0];
  u32x4 (&s_v)[4][16][64] = s_pages[1];
  static_assert(sizeof(AttnMergeLds) <= sizeof(s_pages), "the merge fits in the page buffers");
  const int slot = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5;
  const int seq = a.slots.ids[slot];
  const int T = a.slots.T;
  const int n = a.slots.len[slot];
  const int Hkv = a.kv.Hkv;
  const int G = a.Hq / Hkv;
  const int nq = G * T;
  const int nqt = (nq + 31) >> 5;
  const int nsp = attn_splits(a.slots, slot);
  // linear id -> (pair = split * Hkv + g, group of query tiles); the groups
  // of a pair get ids congruent mod 8, so they share an XCD's L2.  Groups
  // hold four tiles.  The nqt % 4 tiles past the last whole group:
  //   kStagedLastGroup  the last group runs them too (up to seven tiles);
  //   kStagedExact      a tile-parallel launch runs them;
  //   kStagedFold       one tile: the last group's wave w forms its page w
  //                     state, and the four meet in LDS as in the
  //                     tile-parallel shape
  const int nqg = rem != kStagedLastGroup || nqt >= 8 ? nqt >> 2 : 1;
  const int L = blockIdx.x;
  const int qg = (L % (8 * nqg)) / 8;
  const int pair = (L / (8 * nqg)) * 8 + (L % 8);
  if (pair >= nsp * Hkv) return;
  const int sp = pair / Hkv, g = pair % Hkv;
  const AttnKeys ks = attn_keys(a, slot, n, T, sp, nsp);
  {
    const int jw = ks.split0 + 64 * wave;  // wave w stages page w
    if (jw < ks.jend) {
      const uint16_t* pb = attn_keys_base(a, ks, slot, seq, jw);
      const u32x4* kb = (const u32x4*)(pb + (int64_t)g * kPageTokens * kHd);
      const u32x4* vb = (const u32x4*)(pb + (int64_t)(Hkv + g) * kPageTokens * kHd);
      u32x4 tk[16], tv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) tk[i] = kb[i * 64 + lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) tv[i] = vb[i * 64 + lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) s_k[wave][i][lane] = tk[i];
#pragma unroll
      for (int i = 0; i < 16; ++i) s_v[wave][i][lane] = tv[i];
    }
  }
  __syncthreads();
  const int qt_end = qg == nqg - 1 && rem == kStagedLastGroup ? nqt : 4 * qg + 4;
  for (int qt = 4 * qg + wave; qt < qt_end; qt += 4) {
    const int c = qt * 32 + (lane & 31);
    const bool cval = c < nq;
    const int hl = cval ? c / T : 0, t = cval ? c % T : 0;
    u32x4 qop[8], qlo[QLO ? 8 : 1];
    attn_load_q<QLO, QPACK>(a, slot, g, qt, t, g * G + hl, cval, lane, qop, qlo);
    AttnState run, pg;
    // page 0 starts the running state, pages 1..3 merge into it in order
#pragma unroll 1
    for (int w = 0; w < 4; ++w) {
      const int jw = ks.split0 + 64 * w;
      AttnState& st = w == 0 ? run : pg;
      // the page's 32 operand tiles come out of LDS in one burst
      u32x4 pk[16], pv[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pk[i] = s_k[w][i][lane];
#pragma unroll
      for (int i = 0; i < 16; ++i) pv[i] = s_v[w][i][lane];
      attn_page_state<QLO>(a, [&](int i) { return pk[i]; }, [&](int i) { return pv[i]; }, qop, qlo, jw, ks.jend,
                           ks.jall, n + t, cval, h, st);
      if (w > 0) {
        float M, ca, cb;
        attn_merge_coef(run.m, pg.m, M, ca, cb);
        run.l = ca * run.l + cb * pg.l;
        run.m = M;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) run.o[dt][r] = ca * run.o[dt][r] + cb * pg.o[dt][r];
      }
    }
    const int64_t base_idx = ((int64_t)slot * Hkv + g) * a.max_splits + sp;
    if (cval) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *attn_opart4(a, base_idx, dt * 8 + 2 * i + h, c) =
              make_float4(run.o[dt][4 * i], run.o[dt][4 * i + 1], run.o[dt][4 * i + 2], run.o[dt][4 * i + 3]);
      if (h == 0) {
        a.mlpart[(base_idx * 2 + 0) * a.nq_pad + c] = run.m;
        a.mlpart[(base_idx * 2 + 1) * a.nq_pad + c] = run.l;
      }
    }
  }
  if (rem == kStagedFold && qg == nqg - 1) {
    // the remainder tile, page by page: wave w forms page w's state
    const int qt = nqt - 1;
    const int c = qt * 32 + (lane & 31);
    const bool cval = c < nq;
    const int hl = cval ? c / T : 0, t = cval ? c % T : 0;
    u32x4 qop[8], qlo[QLO ? 8 : 1];
    attn_load_q<QLO, QPACK>(a, slot, g, qt, t, g * G + hl, cval, lane, qop, qlo);
    u32x4 pk[16], pv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pk[i] = s_k[wave][i][lane];
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = s_v[wave][i][lane];
    AttnState st;
    attn_page_state<QLO>(a, [&](int i) { return pk[i]; }, [&](int i) { return pv[i]; }, qop, qlo,
                         ks.split0 + 64 * wave, ks.jend, ks.jall, n + t, cval, h, st);
    __syncthreads();  // every wave is done with the pages
    AttnMergeLds& sm = *reinterpret_cast<AttnMergeLds*>(&s_pages[0][0][0][0]);
    attn_merge_put(sm, st, wave, lane);
    __syncthreads();
    attn_merge_store(a, sm, ((int64_t)slot * Hkv + g) * a.max_splits + sp, qt, nq);
  }
}

// Long contexts: one workgroup per (slot, KV head, run of ns consecutive
// splits).  The run's pages stream through two LDS page buffers: all 256
// threads load page p + 1 into registers while the waves compute page p
// from the other buffer, then store it and meet at a barrier.  Wave w runs
// query tile w (four tiles at most) and reads the MFMA operands straight
// from LDS.  Each split's four page states merge in page order and its
// partial is written exactly as by the other two shapes, so the results are
// the same bits.  Not used for candidate slots.
constexpr int kStreamMaxRun = 64;  // splits per workgroup of the streaming shape

template <bool QLO, bool QPACK>
__global__ __launch_bounds__(256) void k_attn_stream_bf16(AttnArgs a, int ns) {
  __shared__ u32x4 s_k[2][16][64];  // a page's K operand tiles, two buffers
  __shared__ u32x4 s_v[2][16][64];  //            V^T operand tiles
  __shared__ int s_page[4 * kStreamMaxRun];  // the run's page indices, read once
  const int slot = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, h = lane >> 5;
  const int seq = a.slots.ids[slot];
  const int T = a.slots.T;
  const int n = a.slots.len[slot];
  const int nkeys = n + T;
  const int Hkv = a.kv.Hkv;
  const int G = a.Hq / Hkv;
  const int nq = G * T;
  const int nqt = (nq + 31) >> 5;
  const int nsp = attn_splits(a.slots, slot);
  const int g = blockIdx.x % Hkv;
  const int sp0 = (blockIdx.x / Hkv) * ns;
  if (sp0 >= nsp) return;
  const int npages = (min(nsp, sp0 + ns) - sp0) * 4;
  const int key0 = sp0 * kAttnSplitKeys;
  for (int p = tid; p < npages; p += 256) {
    const int jw = key0 + 64 * p;
    s_page[p] = jw < nkeys ? a.kv.page_table[(int64_t)seq * a.kv.max_pages + jw / kPageTokens] : 0;
  }
  __syncthreads();
  // page p of the run: K block then V block of head g, 1024 vectors each;
  // thread tid moves vectors tid + 256 r of both
  u32x4 rk[4], rv[4];
  auto load_page = [&](int p) {
    const int jw = key0 + 64 * p;
    if (jw < nkeys) {
      const uint16_t* pb = (const uint16_t*)a.kv.pool + (int64_t)s_page[p] * a.kv.page_elems + a.kv.layer_off;
      const u32x4* kb = (const u32x4*)(pb + (int64_t)g * kPageTokens * kHd);
      const u32x4* vb = (const u32x4*)(pb + (int64_t)(Hkv + g) * kPageTokens * kHd);
#pragma unroll
      for (int r = 0; r < 4; ++r) rk[r] = kb[tid + 256 * r];
#pragma unroll
      for (int r = 0; r < 4; ++r) rv[r] = vb[tid + 256 * r];
    }
  };
  auto store_page = [&](int p, int buf) {
    if (key0 + 64 * p < nkeys) {
#pragma unroll
      for (int r = 0; r < 4; ++r) (&s_k[buf][0][0])[tid + 256 * r] = rk[r];
#pragma unroll
      for (int r = 0; r < 4; ++r) (&s_v[buf][0][0])[tid + 256 * r] = rv[r];
    }
  };
  const int qt = wave;
  const bool tile = qt < nqt;
  const int c = qt * 32 + (lane & 31);
  const bool cval = tile && c < nq;
  const int hl = cval ? c / T : 0, t = cval ? c % T : 0;
  u32x4 qop[8], qlo[QLO ? 8 : 1];
  if (tile) attn_load_q<QLO, QPACK>(a, slot, g, qt, t, g * G + hl, cval, lane, qop, qlo);
  load_page(0);
  store_page(0, 0);
  __syncthreads();
  AttnState run, pg;
  for (int sp = 0; 4 * sp < npages; ++sp) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {  // page w of the split, in LDS buffer w & 1
      const int p = 4 * sp + w;
      if (p + 1 < npages) load_page(p + 1);
      if (tile) {
        AttnState& st = w == 0 ? run : pg;
        attn_page_state<QLO>(a, [&](int i) { return s_k[w & 1][i][lane]; },
                             [&](int i) { return s_v[w & 1][i][lane]; }, qop, qlo, key0 + 64 * p, nkeys, n, n + t,
                             cval, h, st);
        if (w > 0) {
          float M, ca, cb;
          attn_merge_coef(run.m, pg.m, M, ca, cb);
          run.l = ca * run.l + cb * pg.l;
          run.m = M;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) run.o[dt][r] = ca * run.o[dt][r] + cb * pg.o[dt][r];
        }
        if (w == 3 && cval) {
          const int64_t base_idx = ((int64_t)slot * Hkv + g) * a.max_splits + sp0 + sp;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              *attn_opart4(a, base_idx, dt * 8 + 2 * i + h, c) =
                  make_float4(run.o[dt][4 * i], run.o[dt][4 * i + 1], run.o[dt][4 * i + 2], run.o[dt][4 * i + 3]);
          if (h == 0) {
            a.mlpart[(base_idx * 2 + 0) * a.nq_pad + c] = run.m;
            a.mlpart[(base_idx * 2 + 1) * a.nq_pad + c] = run.l;
          }
        }
      }
      if (p + 1 < npages) store_page(p + 1, (w & 1) ^ 1);
      __syncthreads();
    }
  }
}

// Merge the splits for 32 query columns x 16 dims of one (slot, KV head):
// o = sum_s w_s O_s / sum_s w_s l_s with w_s = exp(m_s - max_s m_s), split
// order fixed; written as bf16 (hi, plus the lo plane when out_plane is set).
// Thread (column, group) sums 4 consecutive dims of its column, reading each
// split's partial with one 16-byte load (coalesced over the columns) and
// writing each output plane with one 8-byte store.  The splits' (m, l) go
// to LDS, loaded in one batch per thread, and the weights are formed there;
// the partials of the first kPre splits are requested before that pass so
// that both round trips overlap.
constexpr int kCombineThreads = 128;  // 32 columns x 4 groups of 4 dims
__global__ __launch_bounds__(kCombineThreads) void k_attn_combine_bf16(AttnArgs a) {
  __shared__ float s_m[kMaxSplits][32];
  __shared__ float s_l[kMaxSplits][32];
  __shared__ float s_inv[32];
  constexpr int NG = kCombineThreads / 32;  // groups of 4 dims
  const int ct = blockIdx.x, dch = blockIdx.y % (kHd / 16), g = blockIdx.y / (kHd / 16), slot = blockIdx.z;
  const int T = a.slots.T;
  const int Hkv = a.kv.Hkv, G = a.Hq / Hkv, nq = G * T;
  const int nsp = attn_splits(a.slots, slot);
  const int64_t b0 = ((int64_t)slot * Hkv + g) * a.max_splits;
  const int col = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int c = ct * 32 + col;
  const bool cval = c < nq;
  const int d0 = dch * 16 + 4 * grp;  // this thread's dims d0 .. d0 + 3
  constexpr int kPre = 16;
  const int64_t sstride = (int64_t)a.nq_pad * kHd / 4;  // float4s from one split's partial to the next
  const float4* op = cval ? attn_opart4(a, b0, d0 / 4, c) : nullptr;
  float4 pre[kPre];
  if (cval) {
#pragma unroll
    for (int i = 0; i < kPre; ++i)
      if (i < nsp) pre[i] = op[i * sstride];
  }
  // (m, l) of splits grp, grp + NG, ...: the first kML of them in one batch
  constexpr int kML = 32 / NG;
  float pm[kML], pl[kML];
#pragma unroll
  for (int i = 0; i < kML; ++i) {
    const int s = grp + NG * i;
    if (s < nsp && cval) {
      pm[i] = a.mlpart[((b0 + s) * 2) * a.nq_pad + c];
      pl[i] = a.mlpart[((b0 + s) * 2 + 1) * a.nq_pad + c];
    }
  }
#pragma unroll
  for (int i = 0; i < kML; ++i) {
    const int s = grp + NG * i;
    if (s < nsp) {
      s_m[s][col] = cval ? pm[i] : -INFINITY;
      s_l[s][col] = cval ? pl[i] : 0.f;
    }
  }
  // further splits (long contexts) in batches of kML, each batch's loads
  // issued together
  for (int s0 = grp + NG * kML; s0 < nsp; s0 += NG * kML) {
#pragma unroll
    for (int i = 0; i < kML; ++i) {
      const int s = s0 + NG * i;
      if (s < nsp && cval) {
        pm[i] = a.mlpart[((b0 + s) * 2) * a.nq_pad + c];
        pl[i] = a.mlpart[((b0 + s) * 2 + 1) * a.nq_pad + c];
      }
    }
#pragma unroll
    for (int i = 0; i < kML; ++i) {
      const int s = s0 + NG * i;
      if (s < nsp) {
        s_m[s][col] = cval ? pm[i] : -INFINITY;
        s_l[s][col] = cval ? pl[i] : 0.f;
      }
    }
  }
  __syncthreads();
  // the largest max (each group scans splits grp, grp + NG, ...; a max is
  // exact in any order), then every split's weight, both by all threads
  __shared__ float s_gmax[NG][32];
  {
    float mx = -INFINITY;
    for (int s = grp; s < nsp; s += NG) mx = fmaxf(mx, s_m[s][col]);
    s_gmax[grp][col] = mx;
  }
  __syncthreads();
  float M = s_gmax[0][col];
#pragma unroll
  for (int i = 1; i < NG; ++i) M = fmaxf(M, s_gmax[i][col]);
  for (int s = grp; s < nsp; s += NG) {
    const float ms = s_m[s][col];
    s_m[s][col] = (ms == -INFINITY) ? 0.f : __expf(ms - M);  // weight replaces the max
  }
  __syncthreads();
  if (threadIdx.x < 32) {
    float L = 0.f;  // in split order
#pragma unroll 8
    for (int s = 0; s < nsp; ++s) L += s_m[s][col] * s_l[s][col];
    s_inv[col] = 1.f / L;
  }
  __syncthreads();
  if (!cval) return;
  const int hl = c / T, t = c % T;
  const int64_t m = (int64_t)slot * T + t;
  const int64_t K = (int64_t)a.Hq * kHd;
  const float inv = s_inv[col];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  auto add = [&](float w, const float4& q) {
    acc.x += w * q.x;
    acc.y += w * q.y;
    acc.z += w * q.z;
    acc.w += w * q.w;
  };
#pragma unroll
  for (int i = 0; i < kPre; ++i)
    if (i < nsp) add(s_m[i][col], pre[i]);
  // further splits in batches of 16 loads in flight
  int s = kPre;
  for (; s + 16 <= nsp; s += 16) {
    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = op[(s + i) * sstride];
#pragma unroll
    for (int i = 0; i < 16; ++i) add(s_m[s + i][col], v[i]);
  }
  for (; s + 4 <= nsp; s += 4) {
    float4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = op[(s + i) * sstride];
#pragma unroll
    for (int i = 0; i < 4; ++i) add(s_m[s + i][col], v[i]);
  }
  for (; s < nsp; ++s) add(s_m[s][col], op[s * sstride]);
  // 4 consecutive features of row m: one run in either output layout
  const int64_t k = (int64_t)(g * G + hl) * kHd + d0;
  const int64_t oi = a.out_packed ? packed_index(m, k, K) : m * K + k;
  const float o[4] = {acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  uint32_t oh[2], ol[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint16_t h0 = f2bf(o[2 * e]), h1 = f2bf(o[2 * e + 1]);
    oh[e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    ol[e] = (uint32_t)f2bf_lo(o[2 * e], h0) | ((uint32_t)f2bf_lo(o[2 * e + 1], h1) << 16);
  }
  *(uint2*)(a.out + oi) = make_uint2(oh[0], oh[1]);
  if (a.out_plane) *(uint2*)(a.out + a.out_plane + oi) = make_uint2(ol[0], ol[1]);
}

// A launch with explicit timing events, either of which may be null.
template <typename... KArgs, typename... Args>
static void launch_with_events(void (*kern)(KArgs...), dim3 grid, dim3 block, hipStream_t st, hipEvent_t e0,
                               hipEvent_t e1, Args... args) {
  if (e0 || e1) hipExtLaunchKernelGGL(kern, grid, block, 0, st, e0, e1, 0, args...);
  else hipLaunchKernelGGL(kern, grid, block, 0, st, args...);
}

hipError_t launch_attention_bf16(const AttnArgs& a, int grid_splits, hipStream_t st) {
  const int nqt = (a.Hq / a.kv.Hkv * a.slots.T + 31) / 32;
  const int pairs = grid_splits * a.kv.Hkv;
  // long contexts: stream runs of splits through LDS, at least two
  // workgroups per compute unit
  if (a.slots.xslot0 == 0 && nqt <= 4 && (int64_t)pairs * a.slots.n_seq >= kAttnStreamPairs) {
    const int ns = std::min(kStreamMaxRun, std::max(1, (int)((int64_t)pairs * a.slots.n_seq / kAttnStreamPairs)));
    const dim3 grd(a.kv.Hkv * ((grid_splits + ns - 1) / ns), a.slots.n_seq), blk(256);
    if (a.q_plane && a.q_packed) SDM_LAUNCH((k_attn_stream_bf16<true, true>), grd, blk, 0, st, a, ns);
    else if (!a.q_plane && !a.q_packed) SDM_LAUNCH((k_attn_stream_bf16<false, false>), grd, blk, 0, st, a, ns);
    else return hipErrorInvalidValue;
    return hipGetLastError();
  }
  // enough (split, head, group of four query tiles) triples to cover the
  // chip: stage each split once per group and run the group's query tiles
  // (same results as the tile-parallel shape, which reads every page once
  // per query tile)
  const int nqg = nqt >= 8 ? nqt / 4 : 1;
  const bool staged = (int64_t)pairs * nqg * a.slots.n_seq >= kAttnStagedPairs;
  // a remainder of nqt % 4 tiles would make one wave of a group run two
  // tiles while the other three wait: the staged launch then takes whole
  // groups of four, and one remainder tile is folded into the last group
  // page by page (each wave one page state), more go to a tile-parallel
  // launch
  const bool fold = staged && nqt >= 4 && nqt % 4 == 1;
  const bool exact = staged && nqt >= 4 && nqt % 4 > 1;
  const int rem = fold ? kStagedFold : exact ? kStagedExact : kStagedLastGroup;
  const int qt0 = exact ? nqt / 4 * 4 : 0;
  const int64_t pairs8 = (pairs + 7) / 8 * 8;
  const dim3 blk(256);
  const dim3 grd_staged(pairs8 * (exact || fold ? nqt / 4 : nqg), a.slots.n_seq),
      grd_tile(pairs8 * (nqt - qt0), a.slots.n_seq);
  if (!(a.q_plane && a.q_packed) && !(!a.q_plane && !a.q_packed))
    return hipErrorInvalidValue;  // hi/lo queries come packed, plain ones row-major
  // a timed call's events go on its first dispatch's start and its last
  // dispatch's completion
  const KernelTiming kt = g_ktiming;
  g_ktiming = KernelTiming{};
  if (staged) {
    const hipEvent_t e1 = exact ? nullptr : kt.stop;
    if (a.q_plane) launch_with_events(k_attn_staged_bf16<true, true>, grd_staged, blk, st, kt.start, e1, a, rem);
    else launch_with_events(k_attn_staged_bf16<false, false>, grd_staged, blk, st, kt.start, e1, a, rem);
  }
  if (!staged || exact) {
    const hipEvent_t e0 = staged ? nullptr : kt.start;
    if (a.q_plane) launch_with_events(k_attn_bf16<true, true>, grd_tile, blk, st, e0, kt.stop, a, qt0);
    else launch_with_events(k_attn_bf16<false, false>, grd_tile, blk, st, e0, kt.stop, a, qt0);
  }
  return hipGetLastError();
}
hipError_t launch_attn_combine_bf16(const AttnArgs& a, hipStream_t st) {
  SDM_LAUNCH(k_attn_combine_bf16, dim3(a.nq_pad / 32, a.kv.Hkv * (kHd / 16), a.slots.n_seq), dim3(kCombineThreads), 0, st,
             a);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Device-resident scratch of the allocation-free attention entry point: the
// attention partials (per split O, max and sum) live in this array instead of
// a caller workspace.  Each device holds its own copy from the moment the code
// object is loaded on it until the process ends.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kAttnScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t attn_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    // the array's device address on the current device (the name itself is a
    // host-side stand-in that no kernel may be given)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return hipSuccess;
}

// Scatter row-major K/V [n_keys][Hkv][128] into single-layer pages.
__global__ void k_attn_pack_kv(int Hkv, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int n_keys,
                               const int* __restrict__ pages, uint16_t* __restrict__ pool) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)n_keys * Hkv * kHd) return;
  const int d = i % kHd, g = (i / kHd) % Hkv, j = (int)(i / ((int64_t)kHd * Hkv));
  const int64_t page_elems = 2LL * Hkv * kPageTokens * kHd;
  const int page = pages[j / kPageTokens], pk = j % kPageTokens;
  uint16_t* pb = pool + (int64_t)page * page_elems;
  pb[(int64_t)g * kPageTokens * kHd + kv_k_index(pk, d)] = k[i];
  pb[(int64_t)(Hkv + g) * kPageTokens * kHd + kv_v_index(pk, d)] = v[i];
}
hipError_t launch_attn_pack_kv(int Hkv, const uint16_t* k, const uint16_t* v, int n_keys, const int* pages,
                               uint16_t* pool, hipStream_t st) {
  const int64_t n = (int64_t)n_keys * Hkv * kHd;
  SDM_LAUNCH(k_attn_pack_kv, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Hkv, k, v, n_keys, pages,
                     pool);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-row selection: merge a row's vocab records (fixed order) into
// tok = lowest argmax over non-MASK ids, conf = 1 / sum exp(l - max) and the
// top-2 margin.  One workgroup per row; records loaded 8 per thread at a time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_select_rows(const float4* __restrict__ records, int n_vtiles,
                                                     int* __restrict__ tok, float* __restrict__ conf,
                                                     float* __restrict__ margin) {
  const int m = blockIdx.x;
  const float4* rr = records + (int64_t)m * n_vtiles;
  Rec a = rec_empty();
  for (int base = 0; base < n_vtiles; base += 256 * 8) {
    float4 buf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int vt = base + threadIdx.x + 256 * j;
      buf[j] = vt < n_vtiles ? rr[vt] : rec_pack(rec_empty());
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) a = rec_merge(a, rec_unpack(buf[j]));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) a = rec_merge(a, rec_shfl_xor(a, o));
  __shared__ float4 part[4];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = rec_pack(a);
  __syncthreads();
  if (threadIdx.x == 0) {
    Rec r = rec_unpack(part[0]);
    for (int w = 1; w < 4; ++w) r = rec_merge(r, rec_unpack(part[w]));
    tok[m] = r.idx;
    conf[m] = 1.f / r.sum;
    margin[m] = r.mx - r.mx2;
  }
}

// Wave sums and the (confidence, lowest index) maximum for k_finish_mode.
__device__ __forceinline__ int wave_sum_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ __forceinline__ void wave_best(float& c, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float c2 = __shfl_xor(c, o);
    const int i2 = __shfl_xor(i, o);
    if (c2 > c || (c2 == c && i2 < i)) {
      c = c2;
      i = i2;
    }
  }
}

// The mode rules on a sequence's rows.  One wave per slot; lane j takes
// positions j, j + 64, ... so that a block's loads are issued together.
__global__ __launch_bounds__(64) void k_finish_mode(FinishArgs f) {
  const int slot = blockIdx.x, lane = threadIdx.x;
  const int T = f.T;
  const int r0 = slot * T;
  if (f.mode == FIN_NEXT) {
    if (slot == 0 && lane == 0) f.next[0] = f.tok[r0 + T - 1];
  } else if (f.mode == FIN_DRAFT) {
    for (int j = lane; j < T; j += 64) f.block[r0 + j] = j == 0 ? f.anchor[slot] : f.tok[r0 + j];
  } else if (f.mode == FIN_VERIFY || (f.mode == FIN_QUAD && slot == 0)) {
    // k: the leading drafts that equal the AR argmax of the row before them;
    // the first mismatch by a ballot (wave-uniform), every load of a chunk
    // in flight together
    int k = T - 1;
    for (int j0 = 0; j0 < T - 1; j0 += 64) {
      const int j = j0 + lane;
      const bool miss = j < T - 1 && f.block[r0 + j + 1] != f.tok[r0 + j];
      const unsigned long long b = __ballot(miss);
      if (b) {
        k = j0 + __ffsll(b) - 1;
        break;
      }
    }
    for (int j = lane; j < T; j += 64) f.ar_out[r0 + j] = f.tok[r0 + j];
    if (lane == 0) f.accept[slot] = k + 1;
  } else if (f.mode == FIN_QUAD) {
    // candidate k = slot - 1: the next block should the accept length be k + 1
    const int k = slot - 1;
    for (int j = lane; j < T; j += 64) f.next_blocks[k * T + j] = j == 0 ? f.tok[k] : f.tok[r0 + j];
  } else {  // FIN_DIFFUSE
    // masked positions: the unmask rule; written positions: the revise rule
    // (tau_revise >= 1 never fires, conf <= 1).  Each decision reads only its
    // own position's token before the step, and `best` (the most confident
    // masked position, the lowest on ties) is fixed first.
    float bc = -INFINITY;
    int bi = 0x7fffffff, n_m = 0;
    for (int i = lane; i < T; i += 64)
      if (f.block[r0 + i] == f.mask_id) {
        ++n_m;
        const float c = f.conf[r0 + i];
        if (bi == 0x7fffffff || c > bc) {  // ascending i in a lane: strict > keeps the lowest
          bc = c;
          bi = i;
        }
      }
    wave_best(bc, bi);
    n_m = wave_sum_int(n_m);
    const int best = bi == 0x7fffffff ? -1 : bi;
    int n_u = 0, n_r = 0;
    for (int i = lane; i < T; i += 64) {
      if (f.conf_out) f.conf_out[r0 + i] = f.conf[r0 + i];
      const int cur = f.block[r0 + i], t = f.tok[r0 + i];
      if (cur != f.mask_id) {
        if (t != cur && f.conf[r0 + i] > f.tau_revise) {
          f.block[r0 + i] = t;
          ++n_r;
        }
      } else if (f.force_all || i == best || f.conf[r0 + i] > f.tau) {
        f.block[r0 + i] = t;
        ++n_u;
      }
    }
    n_u = wave_sum_int(n_u);
    n_r = wave_sum_int(n_r);
    if (lane == 0) {
      f.n_masked[slot] = n_m - n_u;
      if (f.n_revised) f.n_revised[slot] = n_r;
    }
  }
}

// ---------------------------------------------------------------------------
// Sampling at temperature T > 0 (one sequence).  Random numbers are
// Philox4x64-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2,
// 3") under key (seed, 0) and counter (vocab id / 4, position, sequence,
// purpose); a 64-bit word x gives u = ((x >> 40) + 1/2) * 2^-24.  A row is
// sampled by the Gumbel-max trick: tok = argmax over non-MASK v of
// l_v / T - ln(-ln u_v), lowest id on ties.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void philox4x64_10(uint64_t (&c)[4], uint64_t k0, uint64_t k1) {
  constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
    const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
    const uint64_t n0 = hi1 ^ c[1] ^ k0, n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
    k0 += W0;
    k1 += W1;
  }
}
__device__ __forceinline__ float uniform24(uint64_t x) {
  return ((float)(uint32_t)(x >> 40) + 0.5f) * 5.9604644775390625e-8f;  // 2^-24, exact
}

__device__ __forceinline__ void part_push(SamplePart& a, float score, int v) {
  if (score > a.best) {  // ids arrive in increasing order: strict > keeps the lowest on ties
    a.second = a.best;
    a.best = score;
    a.idx = v;
  } else if (score > a.second) {
    a.second = score;
  }
}
__device__ __forceinline__ void part_merge(SamplePart& a, const SamplePart& b) {
  // the higher score wins, the lower id on equal scores: a thread's 4-id
  // chunks interleave with the other threads', so the merge order says
  // nothing about which part holds the lower ids
  if (b.best > a.best || (b.best == a.best && b.idx < a.idx)) {
    a.second = fmaxf(a.best, b.second);
    a.best = b.best;
    a.idx = b.idx;
  } else {
    a.second = fmaxf(a.second, b.best);
  }
  if (b.s > 0.f) {
    if (a.s == 0.f) {
      a.m = b.m;
      a.s = b.s;
    } else {
      const float mm = fmaxf(a.m, b.m);
      a.s = a.s * __expf(a.m - mm) + b.s * __expf(b.m - mm);
      a.m = mm;
    }
  }
}
__device__ __forceinline__ SamplePart part_empty() {
  SamplePart p;
  p.best = p.second = -INFINITY;
  p.m = -INFINITY;
  p.s = 0.f;
  p.idx = 0x7fffffff;
  p.pad0 = p.pad1 = p.pad2 = 0;
  return p;
}

// part_merge is commutative bit for bit (the weighted sum's two products
// add in either order to the same value; the maxima and the lower-id tie
// rule are symmetric), so a wave's parts merge in a fixed butterfly over
// lane distances 32, 16, ..., 1: a deterministic tree of six levels instead
// of a chain of 63 dependent merges.  Lane 0's result is the one used.
__device__ __forceinline__ SamplePart part_shfl_xor(const SamplePart& a, int o) {
  SamplePart b;
  b.best = __shfl_xor(a.best, o);
  b.second = __shfl_xor(a.second, o);
  b.m = __shfl_xor(a.m, o);
  b.s = __shfl_xor(a.s, o);
  b.idx = __shfl_xor(a.idx, o);
  b.pad0 = b.pad1 = b.pad2 = 0;
  return b;
}
__device__ __forceinline__ SamplePart part_wave_merge(SamplePart a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const SamplePart b = part_shfl_xor(a, o);
    part_merge(a, b);
  }
  return a;
}

// The workgroup's partial: each wave's 64 parts by the butterfly, then the
// four wave results by thread 0 in wave order (deterministic).
__device__ void part_reduce_store(SamplePart mine, SamplePart* out) {
  static_assert(sizeof(SamplePart) == 32, "a part is two 16-byte words");
  __shared__ SamplePart sp[4];
  const SamplePart w = part_wave_merge(mine);
  if ((threadIdx.x & 63) == 0) sp[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    SamplePart a = sp[0];
#pragma unroll
    for (int t = 1; t < 4; ++t) part_merge(a, sp[t]);
    *out = a;
  }
}

// Row scan for sampling.  Grid (kSampleParts, rows); row r of the launch is
// logits row r0 + r with target position pos0 + r.  Thread t of part q takes
// the 4-id chunks q * cpp + t, q * cpp + t + 256, ... (cpp chunks per part);
// ids inside a thread's chunks arrive in increasing order.
__global__ __launch_bounds__(256) void k_sample_partial(FinishArgs f, int r0, int pos0, int purpose) {
  const int r = r0 + blockIdx.y;
  const float* row = f.logits + (int64_t)r * f.V;
  const int nch = (f.V + 3) / 4, cpp = (nch + kSampleParts - 1) / kSampleParts;
  const int c_end = min(nch, (blockIdx.x + 1) * cpp);
  SamplePart a = part_empty();
  float m = -INFINITY, sum = 0.f;
  for (int c = blockIdx.x * cpp + threadIdx.x; c < c_end; c += 256) {
    uint64_t w[4] = {(uint64_t)c, (uint64_t)(pos0 + blockIdx.y), (uint64_t)f.seq_id, (uint64_t)purpose};
    philox4x64_10(w, f.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * c + e;
      if (v >= f.V || v == f.mask_id) continue;
      const float z = row[v] * f.inv_t;
      part_push(a, z - logf(-logf(uniform24(w[e]))), v);
      if (z > m) {
        sum = sum * __expf(m - z) + 1.f;
        m = z;
      } else {
        sum += __expf(z - m);
      }
    }
  }
  a.m = m;
  a.s = sum;
  part_reduce_store(a, f.parts + (int64_t)r * kSampleParts + blockIdx.x);
}

// Merge a row's parts: tok, gap, lse, ln p(tok) and, with a probe,
// ln p(probe).  One wave per row of the launch; lane q loads part q and the
// butterfly merges them.
static_assert(kSampleParts == 64, "one part per lane of a merging wave");
__global__ __launch_bounds__(64) void k_sample_merge(FinishArgs f, int r0, int nrows, const int* probe) {
  const int i = blockIdx.x;
  if (i >= nrows) return;
  const int r = r0 + i;
  const SamplePart a = part_wave_merge(f.parts[(int64_t)r * kSampleParts + threadIdx.x]);
  if (threadIdx.x != 0) return;
  const float lse = a.m + logf(a.s);
  const float* row = f.logits + (int64_t)r * f.V;
  f.tok[r] = a.idx;
  f.lse[r] = lse;
  f.gap[r] = a.best - a.second;
  f.logp[r] = row[a.idx] * f.inv_t - lse;
  if (probe) f.logp_probe[r] = row[probe[i]] * f.inv_t - lse;
}

// Acceptance loop of the sampled verify (one thread): draft j is accepted iff
// ln u_j < ln p_j(d_j) - ln q_j(d_j); accept = k + 1 for k accepted drafts.
// With every draft accepted the emitted token is the last row's sample.
__global__ void k_finish_sample_verify(FinishArgs f) {
  if (threadIdx.x != 0) return;
  const int T = f.T, n = f.slots.len[0];
  int k = 0;
  for (int j = 1; j < T; ++j) {
    uint64_t w[4] = {0, (uint64_t)(n + j), (uint64_t)f.seq_id, (uint64_t)PURPOSE_ACCEPT};
    philox4x64_10(w, f.seed, 0);
    if (!(logf(uniform24(w[0])) < f.logp_probe[j - 1] - f.draft_stats[j])) break;
    ++k;
  }
  f.accept[0] = k + 1;
  if (k == T - 1) f.next[0] = f.tok[T - 1];
}

// Residual draw at the first rejection k + 1 (skipped when every draft was
// accepted): Gumbel-max over ln(p_v - q_v) where p_v > q_v, p from verify row
// k, q from draft row k + 1.  Grid kSampleParts.
__global__ __launch_bounds__(256) void k_residual_partial(FinishArgs f) {
  const int k = f.accept[0] - 1;
  if (k >= f.T - 1) return;
  const int n = f.slots.len[0];
  const float* prow = f.logits + (int64_t)k * f.V;
  const float* qrow = f.draft_logits + (int64_t)(k + 1) * f.V;
  const float lp = f.lse[k], lq = f.draft_stats[f.T + k + 1];
  const int nch = (f.V + 3) / 4, cpp = (nch + kSampleParts - 1) / kSampleParts;
  const int c_end = min(nch, (blockIdx.x + 1) * cpp);
  SamplePart a = part_empty();
  for (int c = blockIdx.x * cpp + threadIdx.x; c < c_end; c += 256) {
    uint64_t w[4] = {(uint64_t)c, (uint64_t)(n + k + 1), (uint64_t)f.seq_id, (uint64_t)PURPOSE_RESIDUAL};
    philox4x64_10(w, f.seed, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = 4 * c + e;
      if (v >= f.V || v == f.mask_id) continue;
      const float d = __expf(prow[v] * f.inv_t - lp) - __expf(qrow[v] * f.inv_t - lq);
      if (d > 0.f) part_push(a, logf(d) - logf(-logf(uniform24(w[e]))), v);
    }
  }
  part_reduce_store(a, f.parts + blockIdx.x);
}

// One wave: lane q loads part q, the butterfly merges them.
__global__ __launch_bounds__(64) void k_residual_merge(FinishArgs f) {
  const int k = f.accept[0] - 1;
  if (k >= f.T - 1) return;
  const SamplePart a = part_wave_merge(f.parts[threadIdx.x]);
  if (threadIdx.x != 0) return;
  // no id with p > q left after rounding: the verify row's own sample at that position
  f.next[0] = a.idx == 0x7fffffff ? f.tok[k] : a.idx;
}

__global__ void k_finish_sample_draft(FinishArgs f) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= f.T) return;
  if (j == 0) {
    f.block[0] = f.anchor[0];
    return;
  }
  f.block[j] = f.tok[j];
  f.draft_stats[j] = f.logp[j];
  f.draft_stats[f.T + j] = f.lse[j];
}

__global__ void k_finish_sample_next(FinishArgs f) {
  if (threadIdx.x == 0) f.next[0] = f.tok[f.M - 1];
}

static hipError_t launch_finish_sample(const FinishArgs& f, hipStream_t st) {
  const int n = f.slots.len[0];
  if (f.mode == FIN_SAMPLE_NEXT) {
    // the last row's logits predict target_pos
    SDM_LAUNCH(k_sample_partial, dim3(kSampleParts, 1), dim3(256), 0, st, f, f.M - 1, f.target_pos,
               (int)PURPOSE_SAMPLE);
    SDM_LAUNCH(k_sample_merge, dim3(1), dim3(64), 0, st, f, f.M - 1, 1, (const int*)nullptr);
    SDM_LAUNCH(k_finish_sample_next, dim3(1), dim3(64), 0, st, f);
  } else if (f.mode == FIN_SAMPLE_DRAFT) {
    // bidirectional rows 1..T-1 predict their own positions n + t
    SDM_LAUNCH(k_sample_partial, dim3(kSampleParts, f.T - 1), dim3(256), 0, st, f, 1, n + 1, (int)PURPOSE_DRAFT);
    SDM_LAUNCH(k_sample_merge, dim3(f.T - 1), dim3(64), 0, st, f, 1, f.T - 1, (const int*)nullptr);
    SDM_LAUNCH(k_finish_sample_draft, dim3((f.T + 63) / 64), dim3(64), 0, st, f);
  } else {
    // causal rows 0..T-1 predict n + t + 1; row t probes draft token block[t + 1]
    SDM_LAUNCH(k_sample_partial, dim3(kSampleParts, f.T), dim3(256), 0, st, f, 0, n + 1, (int)PURPOSE_SAMPLE);
    SDM_LAUNCH(k_sample_merge, dim3(f.T - 1), dim3(64), 0, st, f, 0, f.T - 1, (const int*)(f.block + 1));
    SDM_LAUNCH(k_sample_merge, dim3(1), dim3(64), 0, st, f, f.T - 1, 1, (const int*)nullptr);
    SDM_LAUNCH(k_finish_sample_verify, dim3(1), dim3(64), 0, st, f);
    SDM_LAUNCH(k_residual_partial, dim3(kSampleParts), dim3(256), 0, st, f);
    SDM_LAUNCH(k_residual_merge, dim3(1), dim3(64), 0, st, f);
  }
  return hipGetLastError();
}

hipError_t launch_finish(const FinishArgs& f, hipStream_t st) {
  if (is_sampling(f.mode)) return launch_finish_sample(f, st);
  SDM_LAUNCH(k_select_rows, dim3(f.M), dim3(256), 0, st, f.records, f.n_vtiles, f.tok, f.conf, f.margin);
  SDM_LAUNCH(k_finish_mode, dim3(f.slots.n_seq), dim3(64), 0, st, f);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 path (tiny decoder): plain VALU kernels, one output per thread, each
// reduction in a fixed sequential order.
// ---------------------------------------------------------------------------
__global__ void k_gemm_f32(const float* __restrict__ X, const float* __restrict__ W, int M, int N, int K,
                           float* __restrict__ Y) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x, m = blockIdx.y;
  if (n >= N) return;
  const float* x = X + (int64_t)m * K;
  const float* w = W + (int64_t)n * K;
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(x[k], w[k], acc);
  Y[(int64_t)m * N + n] = acc;
}
hipError_t launch_gemm_f32(const float* X, const float* W, int M, int N, int K, float* Y, hipStream_t st) {
  SDM_LAUNCH(k_gemm_f32, dim3((N + 127) / 128, M), dim3(128), 0, st, X, W, M, N, K, Y);
  return hipGetLastError();
}

// Y [M][(Hq + 2 Hkv) hd] -> RoPE'd q [M][Hq][hd], K/V rows into the pages.
__global__ void k_qkv_post_f32(const float* __restrict__ Y, EpiArgs ea, int hd) {
  const int m = blockIdx.x;
  const int Hq = ea.Hq, Hkv = ea.kv.Hkv, half = hd / 2;
  const int ncols = (Hq + 2 * Hkv) * hd;
  const int slot = m / ea.slots.T, t = m % ea.slots.T;
  const int seq = ea.slots.ids[slot];
  const int pos = ea.slots.len[slot] + t;
  // a candidate slot's K/V go to its scratch page, key t at page position t
  const bool own = is_candidate(ea.slots, slot);
  const int pk = own ? t : pos % kPageTokens;
  float* pool = own ? (float*)ea.kv.xpool : (float*)ea.kv.pool;
  const int64_t pbase =
      own ? (int64_t)(slot - ea.slots.xslot0) * ea.kv.x_page_elems
          : (int64_t)ea.kv.page_table[(int64_t)seq * ea.kv.max_pages + pos / kPageTokens] * ea.kv.page_elems +
                ea.kv.layer_off;
  const float* y = Y + (int64_t)m * ncols;
  for (int i = threadIdx.x; i < (Hq + 2 * Hkv) * half; i += blockDim.x) {
    const int head = i / half, dl = i % half;
    float v1 = y[head * hd + dl], v2 = y[head * hd + dl + half];
    if (head < Hq + Hkv) {
      const float cs = ea.rope_cos[(int64_t)pos * half + dl], sn = ea.rope_sin[(int64_t)pos * half + dl];
      const float x1 = v1, x2 = v2;
      v1 = x1 * cs - x2 * sn;
      v2 = x2 * cs + x1 * sn;
    }
    if (head < Hq) {
      float* q = (float*)ea.q_out + ((int64_t)m * Hq + head) * hd;
      q[dl] = v1;
      q[dl + half] = v2;
    } else {
      const int blk = head - Hq;  // K heads 0..Hkv-1, then V heads
      float* dst = pool + pbase + ((int64_t)blk * kPageTokens + pk) * hd;
      dst[dl] = v1;
      dst[dl + half] = v2;
    }
  }
}
hipError_t launch_qkv_post_f32(const float* Y, const EpiArgs& ea, int hd, hipStream_t st) {
  SDM_LAUNCH(k_qkv_post_f32, dim3(ea.M), dim3(128), 0, st, Y, ea, hd);
  return hipGetLastError();
}

// One thread per (row, q head); keys visited in ascending order.  A
// candidate slot's visible keys are [0, n) of its pages, then its own block in
// its scratch page.
__global__ void k_attn_f32(const float* __restrict__ q, KvView kv, Slots sl, int Hq, int mode,
                           float* __restrict__ out) {
  const int m = blockIdx.x;
  const int head = threadIdx.x;
  if (head >= Hq) return;
  const int hd = kv.hd, Hkv = kv.Hkv;
  const int g = head * Hkv / Hq;
  const int slot = m / sl.T, t = m % sl.T;
  const int seq = sl.ids[slot];
  const int n = sl.len[slot];
  const bool cand = is_candidate(sl, slot);
  const int npaged = cand ? n : ((mode == BIDIR) ? n + sl.T : n + t + 1);  // visible keys in the pages
  const int nvis = npaged + (cand ? sl.T : 0);
  const float* pool = (const float*)kv.pool;
  const float* own = cand ? (const float*)kv.xpool + (int64_t)(slot - sl.xslot0) * kv.x_page_elems : nullptr;
  const int* ptab = kv.page_table + (int64_t)seq * kv.max_pages;
  // element offset of key j's row of K head g (V: + Hkv * kPageTokens * hd) in its page
  auto key_row = [&](int j) -> const float* {
    if (j < npaged)
      return pool + (int64_t)ptab[j / kPageTokens] * kv.page_elems + kv.layer_off +
             ((int64_t)g * kPageTokens + j % kPageTokens) * hd;
    return own + ((int64_t)g * kPageTokens + (j - npaged)) * hd;
  };
  const int64_t vofs = (int64_t)Hkv * kPageTokens * hd;
  const float* qv = q + ((int64_t)m * Hq + head) * hd;
  const float scale = 1.f / sqrtf((float)hd);
  float mx = -INFINITY;
  for (int j = 0; j < nvis; ++j) {
    const float* kr = key_row(j);
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s = fmaf(qv[d], kr[d], s);
    mx = fmaxf(mx, s * scale);
  }
  float acc[128];
  for (int d = 0; d < hd; ++d) acc[d] = 0.f;
  float sum = 0.f;
  for (int j = 0; j < nvis; ++j) {
    const float* kr = key_row(j);
    const float* vr = kr + vofs;
    float s = 0.f;
    for (int d = 0; d < hd; ++d) s = fmaf(qv[d], kr[d], s);
    const float p = expf(s * scale - mx);
    sum += p;
    for (int d = 0; d < hd; ++d) acc[d] = fmaf(p, vr[d], acc[d]);
  }
  float* o = out + ((int64_t)m * Hq + head) * hd;
  for (int d = 0; d < hd; ++d) o[d] = acc[d] / sum;
}
hipError_t launch_attention_f32(const float* q, const KvView& kv, const Slots& sl, int Hq, int mode, float* out,
                                hipStream_t st) {
  SDM_LAUNCH(k_attn_f32, dim3(sl.n_seq * sl.T), dim3(64), 0, st, q, kv, sl, Hq, mode, out);
  return hipGetLastError();
}

__global__ void k_resid_f32(const float* __restrict__ Y, float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) x[i] += Y[i];
}
hipError_t launch_resid_f32(const float* Y, float* x, int M, int d, hipStream_t st) {
  const int64_t n = (int64_t)M * d;
  SDM_LAUNCH(k_resid_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Y, x, n);
  return hipGetLastError();
}

__global__ void k_swiglu_f32(const float* __restrict__ Y, float* __restrict__ hout, int M, int F) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * F) return;
  const int64_t m = i / F, f = i % F;
  const float g = Y[m * 2 * F + f], u = Y[m * 2 * F + F + f];
  hout[i] = g / (1.f + expf(-g)) * u;
}
hipError_t launch_swiglu_f32(const float* Y, float* h, int M, int F, hipStream_t st) {
  const int64_t n = (int64_t)M * F;
  SDM_LAUNCH(k_swiglu_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Y, h, M, F);
  return hipGetLastError();
}

__global__ void k_logit_records_f32(const float* __restrict__ Y, EpiArgs ea) {
  const int m = blockIdx.y;
  const int vt = blockIdx.x * blockDim.x + threadIdx.x;
  if (vt >= ea.n_vtiles) return;
  Rec a = rec_empty();
  for (int i = 0; i < 32; ++i) {
    const int n = vt * 32 + i;
    if (n >= ea.V) break;
    const float v = Y[(int64_t)m * ea.V + n];
    if (ea.logits) ea.logits[(int64_t)m * ea.V + n] = v;
    if (n != ea.mask_id) a = rec_merge(a, Rec{v, n, -INFINITY, 1.f});
  }
  ea.records[(int64_t)m * ea.n_vtiles + vt] = rec_pack(a);
}
hipError_t launch_logit_records_f32(const float* Y, const EpiArgs& ea, hipStream_t st) {
  SDM_LAUNCH(k_logit_records_f32, dim3((ea.n_vtiles + 63) / 64, ea.M), dim3(64), 0, st, Y, ea);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Bookkeeping: write up to 64 ints given by value (page-table rows, lengths).
// ---------------------------------------------------------------------------
struct IntVals {
  int v[64];
};
__global__ void k_set_ints(int* dst, IntVals vals, int n) {
  if ((int)threadIdx.x < n) dst[threadIdx.x] = vals.v[threadIdx.x];
}
hipError_t launch_set_ints(int* dst, const int* vals, int n, hipStream_t st) {
  IntVals iv;
  for (int i = 0; i < n && i < 64; ++i) iv.v[i] = vals[i];
  SDM_LAUNCH(k_set_ints, dim3(1), dim3(64), 0, st, dst, iv, n);
  return hipGetLastError();
}

}  // namespace sdm
