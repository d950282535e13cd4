// Internal declarations shared by the host runtime (sdm_runtime.cpp) and the
// gfx950 kernels (sdm_kernels.hip).  Not part of the public C ABI.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

namespace sdm {

constexpr int kPageTokens = 64;        // KV page size (positions per page)
constexpr int kAttnSplitKeys = 256;    // keys per attention split (absolute ranges)
constexpr int kMaxSlots = 64;          // sequences in one forward
constexpr int kHd = 128;               // bf16 path head dim
constexpr int kAttnStagedPairs = 256;  // (split, KV head, query-tile group) units from which splits are staged in LDS
constexpr int kAttnStreamPairs = 512;  // from which it streams runs of splits (no candidate slots, G*T <= 128)

enum Mode { CAUSAL = 0, BIDIR = 1 };
enum Epi { EPI_QKV = 0, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_PARTIAL = 4 };
enum Finish { FIN_NEXT = 0, FIN_DRAFT = 1, FIN_VERIFY = 2, FIN_DIFFUSE = 3,
              FIN_SAMPLE_NEXT = 4, FIN_SAMPLE_DRAFT = 5, FIN_SAMPLE_VERIFY = 6, FIN_QUAD = 7 };
__host__ __device__ inline bool is_sampling(int fin_mode) {
  return fin_mode >= FIN_SAMPLE_NEXT && fin_mode <= FIN_SAMPLE_VERIFY;
}
// Random-number purposes of the sampling modes (counter word 3).
enum Purpose { PURPOSE_DRAFT = 1, PURPOSE_ACCEPT = 2, PURPOSE_RESIDUAL = 3, PURPOSE_SAMPLE = 4 };
constexpr int kSampleParts = 64;  // workgroups sharing one row's vocabulary when sampling

// One workgroup's share of a sampled row: the two best perturbed scores (the
// best's id, lowest on ties) and the row's max and sum of exp(z - max).
struct SamplePart {
  float best, second, m, s;
  int idx, pad0, pad1, pad2;
};
// Token source of the embedding: the given ids; [anchor, MASK...] per slot;
// the given T ids then MASK for every later row (quadratic self-speculation).
enum TokSrc { TOK_PLAIN = 0, TOK_DRAFT = 1, TOK_QUAD = 2 };

// Activations of the bf16 path travel between kernels as two bf16 planes, hi
// and lo, with value hi + lo: hi = RNE_bf16(x), lo = RNE_bf16(x - hi) (a
// two-term bf16 expansion, about 16 significant bits).  Every plane pair is
// one buffer with the lo plane `plane` elements after the hi plane.  Weights
// and the KV cache are single bf16 values.

// Element (r, c) of a [R, C] matrix in the MFMA 32x32x16 operand layout:
// tiles of 32 rows x 16 columns, 1 KiB each, laid out row-tile major; inside
// a tile lane = (r % 32) + 32 * ((c % 16) / 8) holds the 8 columns c%8.
// The same layout serves the A operand (weights, rows = outputs) and the B
// operand (activations, rows = tokens).
__host__ __device__ inline int64_t packed_index(int64_t r, int64_t c, int64_t C) {
  const int64_t rt = r >> 5, cb = c >> 4;
  const int64_t lane = (r & 31) + 32 * ((c & 15) >> 3);
  return (((rt * (C >> 4) + cb) * 64 + lane) << 3) + (c & 7);
}

// KV page (bf16 path), per layer and KV head: a K block then (after all
// heads' K blocks) a V block, each kPageTokens x 128 elements.
//   K block: A-operand tiles of 32 keys x 16 dims: [key/32][dim/16][64][8].
//   V block: A-operand tiles of V^T, 32 dims x 16 keys: [dim/32][key/16][64][8],
//            where inside a 16-key group the key held by (lane half h', e) is
//            8*(e/4) + 4*h' + e%4 -- the order in which the attention kernel's
//            score tile hands probabilities to the P.V product.
__host__ __device__ inline int kv_k_index(int pk, int d) {
  const int lane = (pk & 31) + 32 * ((d & 15) >> 3);
  return ((((pk >> 5) * (kHd / 16) + (d >> 4)) * 64 + lane) << 3) + (d & 7);
}
__host__ __device__ inline int kv_v_index(int pk, int d) {
  const int r = pk & 15;
  const int hh = (r >> 2) & 1;
  const int e = 4 * (r >> 3) + (r & 3);
  const int lane = (d & 31) + 32 * hh;
  return ((((d >> 5) * (kPageTokens / 16) + (pk >> 4)) * 64 + lane) << 3) + e;
}

// Candidate slots (quadratic self-speculation): when xslot0 > 0, every slot
// s >= xslot0 is a candidate block.  Its rows sit at positions len[s] + t and
// see keys [0, len[s]) of its sequence's pages plus, bidirectionally, its own
// T rows, whose K/V live in the scratch page (s - xslot0) of KvView::xpool
// (key t at page position t) instead of the sequence's pages.
struct Slots {
  int n_seq;   // sequences in this forward
  int T;       // rows per sequence
  int ids[kMaxSlots];
  int len[kMaxSlots];  // committed length per slot: the block's first position
  int xslot0;          // first candidate slot; 0: none
};
__host__ __device__ inline bool is_candidate(const Slots& s, int slot) { return s.xslot0 > 0 && slot >= s.xslot0; }

// Attention splits of one slot: its keys in the sequence's pages in ranges of
// kAttnSplitKeys, then, for a candidate, one more split over its own block.
constexpr int kMaxSplits = 256;  // splits the combine kernel merges per (slot, KV head)
__host__ __device__ inline int attn_splits(const Slots& s, int slot) {
  const bool c = is_candidate(s, slot);
  const int paged = c ? s.len[slot] : s.len[slot] + s.T;
  return (paged + kAttnSplitKeys - 1) / kAttnSplitKeys + (c ? 1 : 0);
}

struct KvView {
  void* pool;            // page base
  int64_t page_elems;    // elements per page
  int64_t layer_off;     // element offset of this layer inside a page
  const int* page_table; // [max_seqs][max_pages]
  int max_pages;
  int Hkv, hd;
  void* xpool;           // candidate slots' own K/V: pages of one layer, x_page_elems apart
  int64_t x_page_elems;
};

struct EpiArgs {
  int M;                 // valid rows
  Slots slots;
  KvView kv;
  int Hq;
  uint16_t* q_out;       // QKV, bf16: per (slot, KV head) a packed [q_nq_pad][hd] operand whose
  int64_t q_plane;       //   column c = (q head within the group) * T + block row; hi plane,
  int q_nq_pad;          //   lo plane q_plane elements later.  f32: row-major [M][Hq][hd]
  const float* rope_cos; // [max_context][hd/2]
  const float* rope_sin;
  int d;                 // PARTIAL: row length of the partial planes
  uint16_t* h_out;       // SWIGLU: packed-B [M32][F] hi plane, lo plane h_plane elements later
  int64_t h_plane;
  int F;
  float4* records;       // LOGITS: [M][n_vtiles] (max, idx bits, max2, sum)
  int n_vtiles;
  float* logits;         // LOGITS: optional [M][V]
  int V, mask_id;
  float* part;           // PARTIAL: [S][rows][d] fp32 split-K partials
  int64_t part_stride;   // elements between splits
};

struct GemmShape {
  int NT, KB;            // 32-row tiles of W, 16-column blocks of K
  int MTILES;            // 32-row tiles of the activations
  int S;                 // workgroups splitting K (EPI_PARTIAL only)
  int WAVES;             // waves per workgroup, splitting the workgroup's K range
  int TP;                // weight tiles per workgroup
  int ROWS;              // activation rows (a one-tile launch loads only these)
};

constexpr int kGemmTargetGroups = 256;  // one workgroup per compute unit
constexpr int kMaxSplitK = 8;           // split-K partial planes the RMSNorm adds
constexpr int kGemmChunk = 4;           // k-blocks per round-robin chunk of a GEMM wave

// Launch configuration of a weight matrix.  The summation order of an output
// -- the K split S, the waves' K ranges and their reduction order -- is a
// function of the matrix shape and its epilogue only (never of the number of
// rows), so every row's result is independent of the batch.  Matrices whose
// outputs are summed into the residual stream (EPI_PARTIAL) are split over S
// workgroups along K so that the grid covers the chip; each split writes an
// fp32 partial that the following RMSNorm adds in split order.
// TP only chooses which workgroup computes which tile: a workgroup takes TP
// weight tiles, so the activations it reads from L2 are shared by TP weight
// streams while about one workgroup per compute unit remains.
inline GemmShape gemm_config(int epi, int N, int K, int rows) {
  GemmShape g;
  g.NT = N / 32;
  g.KB = K / 16;
  g.MTILES = (rows + 31) / 32;
  g.ROWS = rows;
  g.S = 1;
  if (epi == EPI_PARTIAL) {
    // enough splits for two workgroups per compute unit (two waves per SIMD,
    // so one-tile groups overlap their accumulator chains); more while every
    // split would still stream at least 192 k-blocks (very long K), up to
    // four tiles per group.  Fewer splits mean fewer partial planes for the
    // following RMSNorm to add (and to write and read at many rows).
    auto ok = [&](int s) { return s <= kMaxSplitK && g.KB % s == 0 && g.KB / s >= 32; };
    while (g.NT * g.S < 2 * kGemmTargetGroups && ok(2 * g.S)) g.S *= 2;
    while (ok(2 * g.S) && g.KB / (2 * g.S) >= 192 && g.NT * 2 * g.S <= 4 * kGemmTargetGroups) g.S *= 2;
  }
  g.WAVES = 4;
  g.TP = 1;
  const int mt = g.MTILES <= 1 ? 1 : (g.MTILES == 2 ? 2 : 4);  // activation tiles per workgroup
  const int mgroups = (g.MTILES + mt - 1) / mt;
  const int tmax = mt == 4 ? 3 : 4;  // register budget: 4 x 4 accumulator tiles do not fit
  if (mt == 4) {
    // Many-row launches run one workgroup per compute unit, in rounds of
    // kGemmTargetGroups, and are bound by operand bytes into the compute
    // units: 4 activation tiles (two planes) + t weight tiles feed 8t
    // products, so a group of t tiles costs about (8 + t) / 8 tile-times
    // per tile.  Take the t that minimises rounds x (8 + t); the last group
    // may hold fewer tiles.
    int best = 0;
    for (int t = tmax; t >= 1; --t) {
      const int64_t groups = (int64_t)(g.NT + t - 1) / t * g.S * mgroups;
      const int64_t cost = (groups + kGemmTargetGroups - 1) / kGemmTargetGroups * (8 + t);
      if (best == 0 || cost < best) {
        best = (int)cost;
        g.TP = t;
      }
    }
    return g;
  }
  for (int t = tmax; t > 1; --t)
    if (g.NT % t == 0 && (g.NT / t) * g.S * mgroups >= kGemmTargetGroups) {
      g.TP = t;
      break;
    }
  return g;
}

// 4-bit weights (w4a16): group-wise int4 codes, one bf16 scale per output
// row and group of kW4Group input columns.  Packed layout of an [N, K] matrix
// (N a multiple of 32, K of kW4Group), codes first, then scales at byte
// offset w4_scale_offset(N, K):
//   codes:  [N/32][K/128][part 2][lane 64][16 B].  Word j (4 B) of a lane's
//           16 bytes in part p is k-block 4p + j of the group; its nibble e
//           (bits 4e..4e+3, two's complement) is the weight at row
//           32 * tile + lane % 32, column 128 * group + 16 * (4p + j) +
//           8 * (lane / 32) + e -- the k order of the bf16 MFMA A operand.
//   scales: [N/32][K/128][half 2][16] bf16: half h, entry r is the scale of
//           row 32 * tile + crow(r, h), the rows that accumulator register r
//           of a lane of half h holds.
constexpr int kW4Group = 128;
constexpr int kW4GroupBlocks = kW4Group / 16;  // k-blocks per scale group
inline int64_t w4_scale_offset(int64_t N, int64_t K) { return ((N * K / 2) + 255) / 256 * 256; }
inline int64_t w4_packed_bytes(int64_t N, int64_t K) { return w4_scale_offset(N, K) + N * (K / kW4Group) * 2; }

// Launch configuration of a 4-bit matrix.  kW4Waves waves per workgroup take
// the scale groups of its K range round robin.  Split-K (EPI_PARTIAL only):
// the smallest S with every split a whole number of groups (at least one per
// wave) that gives 2 * kGemmTargetGroups (split, tile) pairs, so that
// workgroups of two weight tiles still cover the chip; else the largest valid
// S.  TP: the most weight tiles per workgroup (MT * TP <= 4: a wave holds a
// running total and the current group's sum of each tile) that keep
// kGemmTargetGroups workgroups.  S and the waves depend on the matrix shape
// only, never on the number of rows, so every row's result is independent of
// the batch.
constexpr int kW4Waves = 8;
inline GemmShape gemm_config_w4(int epi, int N, int K, int rows) {
  GemmShape g;
  g.NT = N / 32;
  g.KB = K / 16;
  g.MTILES = (rows + 31) / 32;
  g.ROWS = rows;
  g.S = 1;
  if (epi == EPI_PARTIAL) {
    auto ok = [&](int s) {
      return g.KB % (s * kW4GroupBlocks) == 0 && g.KB / (s * kW4GroupBlocks) >= kW4Waves;
    };
    int best = 1;
    for (int s = 2; s <= kMaxSplitK; s *= 2)
      if (ok(s)) best = s;
    for (int s = 1; s <= kMaxSplitK; s *= 2)
      if (ok(s) && g.NT * s >= 2 * kGemmTargetGroups) {
        best = s;
        break;
      }
    g.S = best;
  }
  g.WAVES = kW4Waves;
  g.TP = 1;
  const int mt = g.MTILES <= 1 ? 1 : (g.MTILES == 2 ? 2 : 4);
  const int mgroups = (g.MTILES + mt - 1) / mt;
  for (int t = 4 / mt; t > 1; --t)
    if (g.NT % t == 0 && (g.NT / t) * g.S * mgroups >= kGemmTargetGroups) {
      g.TP = t;
      break;
    }
  return g;
}

struct AttnArgs {
  const uint16_t* q;     // q_packed: the QKV epilogue's packed layout; else row-major [rows][Hq][hd]
  int64_t q_plane;       // elements to the lo plane; 0: q is plain bf16
  int q_packed;
  KvView kv;
  Slots slots;
  int Hq, mode;
  float scale;
  float* opart;          // [slots][Hkv][max_splits][hd / 4][nq_pad] float4s
  float* mlpart;         // [slots][Hkv][max_splits][2][nq_pad]: max, then sum
  int max_splits, nq_pad;
  uint16_t* out;         // [rows][Hq*hd]: packed-B when out_packed else row-major
  int out_packed;
  int64_t out_plane;     // elements to the lo plane; 0: plain bf16 output
};

struct FinishArgs {
  int mode;              // Finish
  Slots slots;
  int M, T;              // rows, rows per slot
  const float4* records; int n_vtiles;
  int* tok; float* conf; float* margin;   // per-row results (workspace)
  int mask_id;
  const int* anchor;     // DRAFT: device anchor
  int* block;            // DRAFT out / DIFFUSE in-out / VERIFY in [slots][T]
  int* ar_out;           // VERIFY: [slots][T]
  int* accept;           // VERIFY: [slots]
  int* n_masked;         // DIFFUSE: [slots]
  float* conf_out;       // DIFFUSE: optional [slots][T]
  float tau; int force_all;
  float tau_revise;      // DIFFUSE: written positions whose argmax differs with conf > tau_revise take it
  int* n_revised;        // DIFFUSE: optional [slots]
  // sampling modes (one sequence): rows' logits [M][V] at temperature 1 / inv_t
  const float* logits; int V; float inv_t; uint64_t seed; int seq_id;
  int target_pos;        // SAMPLE_NEXT: position of the token the last row predicts
  SamplePart* parts;     // [M][kSampleParts]
  float* lse;            // [M] ln sum_v exp(l_v / T) over non-MASK ids
  float* gap;            // [M] best minus second perturbed score
  float* logp;           // [M] ln p(sampled token)
  float* logp_probe;     // VERIFY: [M] ln p(block[t + 1]) of row t
  float* draft_stats;    // DRAFT out / VERIFY in: [2][T] ln q(d_t), lse of draft row t
  const float* draft_logits;  // VERIFY: the draft forward's logits [T][V]
  int* next;             // NEXT: device token (last row of slot 0)
  int* next_blocks;      // QUAD: [T][T], row k = [a_k, candidate k's argmax at rows 1..T-1]
};

// Kernel timing: when set, the next launch carries these events on its own
// dispatch (start / completion), then the slot is cleared.
struct KernelTiming {
  hipEvent_t start = nullptr, stop = nullptr;
};
extern thread_local KernelTiming g_ktiming;

// Launch a kernel, attaching g_ktiming's events to this dispatch when set.
#define SDM_LAUNCH(kern, grid, block, shmem, stream, ...)                                                        \
  do {                                                                                                          \
    if (::sdm::g_ktiming.start) {                                                                               \
      hipExtLaunchKernelGGL(kern, grid, block, shmem, stream, ::sdm::g_ktiming.start, ::sdm::g_ktiming.stop, 0, \
                            __VA_ARGS__);                                                                       \
      ::sdm::g_ktiming = ::sdm::KernelTiming{};                                                                 \
    } else {                                                                                                    \
      hipLaunchKernelGGL(kern, grid, block, shmem, stream, __VA_ARGS__);                                        \
    }                                                                                                           \
  } while (0)

// ---- launchers (sdm_kernels.hip) -------------------------------------------
hipError_t launch_pack(int dtype, int kind, const void* src, const void* src2, void* dst, int64_t rows, int64_t cols,
                       int head_dim, hipStream_t st);
hipError_t launch_embed(int dtype, const void* E, int d, int V, const int* tokens, int tok_src, const int* anchor,
                        int M, int T, int mask_id, float* x, hipStream_t st);
hipError_t launch_rmsnorm(int dtype, float* x, const float* part, int nparts, int64_t part_stride, const void* gain,
                          float eps, int M, int d, int row0, void* out, int64_t out_plane, hipStream_t st);
hipError_t launch_pack_w4(int kind, const void* codes, const void* scales, const void* codes2, const void* scales2,
                          void* dst, int64_t rows, int64_t cols, int head_dim, hipStream_t st);
hipError_t launch_gemm_w4(int epi, const uint8_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                          const EpiArgs& ea, hipStream_t st);
hipError_t launch_gemm_bf16(int epi, const uint16_t* W, const uint16_t* X, int64_t x_plane, const GemmShape& g,
                            const EpiArgs& ea, hipStream_t st);
hipError_t launch_attention_bf16(const AttnArgs& a, int grid_splits, hipStream_t st);
hipError_t launch_attn_combine_bf16(const AttnArgs& a, hipStream_t st);
hipError_t launch_finish(const FinishArgs& f, hipStream_t st);

// fp32 (VALU) path
hipError_t launch_gemm_f32(const float* X, const float* W, int M, int N, int K, float* Y, hipStream_t st);
hipError_t launch_qkv_post_f32(const float* Y, const EpiArgs& ea, int hd, hipStream_t st);
hipError_t launch_attention_f32(const float* q, const KvView& kv, const Slots& sl, int Hq, int mode, float* out,
                                hipStream_t st);
hipError_t launch_resid_f32(const float* Y, float* x, int M, int d, hipStream_t st);
hipError_t launch_swiglu_f32(const float* Y, float* h, int M, int F, hipStream_t st);
hipError_t launch_logit_records_f32(const float* Y, const EpiArgs& ea, hipStream_t st);

// bookkeeping
hipError_t launch_set_ints(int* dst, const int* vals, int n, hipStream_t st);   // n <= 64, values by value
hipError_t launch_attn_pack_kv(int Hkv, const uint16_t* k, const uint16_t* v, int n_keys, const int* pages,
                               uint16_t* pool, hipStream_t st);

// Allocation-free attention: the device scratch array's address on the
// current device (looked up once per device, then cached).
constexpr size_t kAttnScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
hipError_t attn_scratch_address(void** out);

}  // namespace sdm
