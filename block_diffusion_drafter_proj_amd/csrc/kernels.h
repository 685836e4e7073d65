// Kernel launch interface between the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

constexpr int kMaxSeg = DFLASH_MAX_LAYERS;
constexpr int kMaxChunkReq = 64;  // requests per inject scatter launch

enum Epilogue { EPI_PARTIAL = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3, EPI_TOPK = 4, EPI_ROPE = 5 };

constexpr int kMaxRopeReq = 64;  // requests of one EPI_ROPE launch (skinny sizes: under 64 rows)

struct SlotState;

// EPI_ROPE: the QKV product of the block rows written straight into the
// attention layouts.  Units are pairs of 16-column tiles half a head apart
// (columns j and j + dh/2 of one head), so one thread holds both halves of a
// rotate-half pair: q and k heads are rotated at the block positions
// n .. n+B-1 (n = ctx_len + 1 of the row's request), q goes to
// qb [r][head][16][dh], k to the request's block page [head][16][dh] and v to
// it transposed [head][dh][16].  Rows B..15 of each 16-row tile are never
// written (zero from the handle's set-up).
struct RopeOut {
  const SlotState* state;
  const float* cos_t;  // [max_position, dh/2]
  const float* sin_t;
  void* qb;
  void* blk;
  int B, Hq, Hkv, dh;
  int slots[kMaxRopeReq];
};

// Y[M, N] = X[M, K] * W[N, K]^T with a fused epilogue, W packed by launch_pack.
//  X: virtual concatenation along k of a_parts row-major arrays, each
//     [M, a_part_k] with row stride lda (elements).
//  W: packed 16-row tiles; tile t lives in segment t / seg_tiles at w[seg]
//     (seg_tiles = 0: one segment holding every tile).
//  P: split-K factor; EPI_PARTIAL writes out_f32[p][M][N] for each split.
struct GemmParams {
  const void* a[DFLASH_MAX_FEAT];
  int a_parts, a_part_k, lda;
  int M;
  const void* w[kMaxSeg];
  int seg_tiles;
  int tiles;  // output tiles (ceil(N / 16)); SwiGLU: gate tiles
  int N, K, P;
  int up_tile_off;  // EPI_SWIGLU: tile offset of the up rows in the packed matrix
  float* out_f32;   // EPI_PARTIAL
  void* out_t;      // EPI_SWIGLU (storage dtype)
  int ldt;
  // EPI_RESID (one split): resid[m][n] += y; out_t[m][n] (row stride ldt) =
  // the new residual times gain[n] in the storage dtype, and
  // ssq[m][tile] (ssq_tiles per row) = the sum of squares of the tile's 16 new
  // residual values of row m, so the next product can apply the RMSNorm's
  // 1/rms to its own output
  float* resid;
  int ldr;
  const void* resid_row;  // when set, every row's old residual is this storage-dtype row (the block init)
  const void* gain;
  float* ssq;
  // EPI_SWIGLU: when ssq is set, each row's gate and up values are scaled by
  // 1 / sqrt(sum over ssq_tiles tiles of ssq / ssq_d + eps) before the SwiGLU
  int ssq_tiles, ssq_d;
  float eps;
  unsigned long long* keys;  // EPI_ARGMAX: one per row; EPI_TOPK: [M][gridDim.x][16] sorted lists
  float* dbg;                // EPI_ARGMAX / EPI_TOPK, optional fp32 logits
  int ld_dbg;
  RopeOut rope;              // EPI_ROPE (tiles counts column-tile pairs)
  // tiled kernel only: A (one part) and the SwiGLU output stored in fragment
  // order (frag_index) instead of row-major
  int a_packed, out_packed;
  // 4-bit weights (skinny kernel only): w[seg] points at the codes of the
  // segment's first tile, sb[seg] at its (scale, bias) pairs (q4 layout below)
  int w4;
  const void* sb[kMaxSeg];
};

// 4-bit packed matrix [N, K] (N16 = N rounded up to 16, K a multiple of 128):
//   codes  [N16/16 tiles][K/128][64 lanes][4] u32: lane l of k-step 4 kq + j
//          holds row 16 t + l%16, inputs 32 (4 kq + j) + 8 (l/16) .. +7, one
//          nibble each (byte i: element 2i low, 2i+1 high)
//   scales [N16/16][K/128][16 rows][2] u32, after the codes: (s | b << 16) as
//          bf16 bit patterns, for the groups of 64 inputs 2 kq and 2 kq + 1
__host__ __device__ inline size_t q4_codes_bytes(int N, int K) { return (size_t)((N + 15) / 16) * 16 * K / 2; }
__host__ __device__ inline size_t q4_bytes(int N, int K) { return q4_codes_bytes(N, K) + (size_t)((N + 15) / 16) * 16 * (K / 64) * 4; }
// quantise the storage-dtype (bf16) matrix src [N, K] into the q4 layout at dst
void launch_pack_q4(const void* src, void* dst, int N, int K, hipStream_t s);

struct GemmPlan {
  int P, NW, GP;  // split-K factor, waves per workgroup, workgroups per split
  // kernel: 0 = tiled (gemm_big.hip); 1 = skinny, one 16-row block per grid
  // row; 4 = skinny, up to 64 rows in one block (split-K products only)
  int mt;
};

// Row-wise RMSNorm of fp32 rows into the storage dtype.  The input row is
//   x = (init_row ? init_row : x_in ? x_in[row] : 0) + sum_p part[p][row]
// or, with oconv (the DFlash-2 conv at the producing GEMM's output),
//   x = x_in[row] + w0 * y[row] + w1 * y[row-1],  y[r] = sum_p part[p][r],
// with y[row-1] = embed[last_token] at the start of each request's block;
// x is written to x_out[row] when x_out is set (x_out must differ from x_in
// with oconv and the input conv, whose previous row re-reads x_in).
struct NormParams {
  const float* x_in;       // [M, ld] fp32 residual, or NULL
  const void* init_row;    // storage dtype [d]: every row starts from it, or NULL
  const int* init_tokens;  // [M]: row m starts from init_row[init_tokens[m]] (an embedding table), or NULL
  void* feat;              // optional storage-dtype copy of x [M, d] (a target feature layer)
  const float* part;       // [n_part][M][d] fp32 split-K partials, or NULL
  int n_part;
  float* x_out;            // [M, ld] receives x, or NULL
  int ldx;
  const void* gamma;  // storage dtype [d]
  float eps;
  void* out;  // storage dtype [M, d] (row stride ldo), or fragment order (out_packed)
  int ldo;
  int out_packed;
  int d, M;
  float* dbg;  // optional fp32 copy of x [M, d]
  unsigned long long* zero_keys;  // optional: keys[row] = 0
  // two-tap conv of the normalised rows (DFlash 2): out_i = w0*n_i + w1*n_{i-1}
  // inside each request's block of B rows; row 0 reads embed[last_token[r]]
  const void* conv;        // [2][d] taps (w0, w1) or NULL
  const void* oconv;       // [2][d] taps of the producing GEMM's output conv, or NULL
  const void* embed;       // [V, d]
  const int* last_token;   // [n_req]
  int B, vocab;
  unsigned int* err;
  int ldp;                 // row stride of the partials (0: d)
  const float* otaps;      // dynamic output conv: per-row taps [M][2d] (a, then b) in place of oconv, or NULL
};

// Dynamic two-tap conv taps (DFlash 2): per row and channel c,
//   a = w0[c] + U[c] . t,  b = w1[c] + U[d + c] . t,  t = sum_p t_part[p][row]
// (t the rank-r projection of the conv's input row, from split-K partials).
// The apply form convolves the stored input rows x: out[row] = a x[row] +
// b x[row-1] (x[-1] of a request's block: the embedding of its last verified
// token); the taps form writes (a, b) for a norm that applies them.
struct DConvParams {
  const void* x;        // [M, d] storage dtype (apply), or NULL (taps)
  const float* t;       // t partials: element j of row m, split p at t[p * plane + m * ldt + j]
  int n_part, ldt;
  int lo_off;           // > 0: t also adds the partials lo_off columns further (a hi + lo folded form)
  long long plane;
  const void* U;        // [2d, r] storage dtype
  const void* w;        // static taps [2][d] storage dtype
  int d, r, M, B, vocab;
  const void* embed;    // [V, d]
  const int* last_token;
  void* out;            // apply: storage dtype [M, d] (row stride ldo), or fragment order
  int ldo, out_packed;
  float* taps;          // taps: [M][2d]
  unsigned int* err;
};
void launch_dconv(int dtype, const DConvParams& p, hipStream_t s);
// out [2r, K]: D [r, d] x W [d, K] (fp32 sums) as hi (rows 0..r-1, the sums
// rounded to the storage dtype) + lo (rows r..2r-1, the rest), r <= 64
void launch_fold(int dtype, const void* D, const void* W, void* out, int r, int d, int K, hipStream_t s);

// Greedy selection over split-K partial logits (the vocabulary product of
// 17..64 rows): one workgroup of 4 waves per (chunk of kSelChunk columns,
// row) sums the planes in split order and leaves its best packed key
// (atomic max into keys[row]) or one sorted top-16 list per wave
// (lists[row][chunk * 4 + wave]; a second kernel settles the few lists the
// first one marks).
constexpr int kSelChunk = 4096;
struct LogitSelParams {
  const float* part;  // [n_part][M][N] fp32
  int n_part, M, N;
  float* dbg;  // optional fp32 logits [M][ld_dbg]
  int ld_dbg;
  unsigned long long* keys;   // argmax: one per row (zero on entry)
  unsigned long long* lists;  // top-16: [M][n_lists][16]
  int n_lists;                // 4 * chunks
  int exact;                  // top-16: every list through the exact pass
};
inline int logit_sel_lists(int N) { return 4 * ((N + kSelChunk - 1) / kSelChunk); }
void launch_logit_select(bool topk, const LogitSelParams& p, hipStream_t s);

// Merge of the per-workgroup top-16 lists of the LM head.
struct TopkParams {
  const unsigned long long* lists;  // [M][n_lists][16]
  int n_lists, M, vocab;
  int* draft;        // [M] argmax ids
  int* topk_ids;     // [M][16]
  float* topk_logits;  // [M][16]
};

struct SlotArgs {
  int slots[DFLASH_MAX_BATCH];
};

// Device per-slot state: ctx_len, kv_begin, n_pages (ring size), pad.
struct SlotState {
  int ctx_len, kv_begin, n_pages, pad;
};

struct QkvPostParams {
  const float* qkv;  // [n_part][n_req*B, (Hq+2Hkv)*dh] split-K partials
  int n_part;
  int B, Hq, Hkv;
  const SlotState* state;
  const float* cos_t;  // [max_position, dh/2]
  const float* sin_t;
  void* qb;   // [n_req, Hq, 16, dh]
  void* blk;  // [n_req] pages [2][Hkv][16*dh]
};

struct AttnParams {
  const void* qb;
  const void* blk;
  const void* pool;  // this layer's pages
  const int* page_table;
  int pt_stride;
  const SlotState* state;
  int max_pages;
  int window;
  int Hq, Hkv, B;
  int split_target;  // splits aimed at per (request, KV head)
  int pps_cap;       // at most this many pages per split
  int* n_split;      // [n_req] out: splits of each request (read by k_combine)
  int n_splits;      // grid.x: splits of the longest request
  int KQ;        // key subsets per workgroup (waves = Hq/Hkv * KQ)
  float scale;
  float* part_o;   // [n_req, Hq, n_splits, 16, dh]
  float* part_ml;  // [n_req, Hq, n_splits, 16, 2]
  void* out;       // storage dtype [n_req*B, Hq*dh] (written here when n_splits == 1)
  int ldo;
  int out_packed;  // out in fragment order with ldo columns
  unsigned int* err;
  // Causal mode (a target's verify forward, bf16 only): causal_R new rows per
  // request, already appended to the pages (the slot's device ctx_len counts
  // them), attend causally; there is no block unit.  The grid's z runs over
  // (request, 16-row tile) pairs, n_tiles tiles per request, and qb, part_*
  // and n_split are indexed by that pair.  causal_R = 0: the draft's block.
  int causal_R, n_tiles;
};

struct CombineParams {
  const float* part_o;
  const float* part_ml;
  const int* n_split;  // [n_req] splits of each request
  int n_splits, n_rh, Hq, B;  // n_rh = n_req * Hq
  void* out;  // storage dtype [n_req*B, Hq*dh]
  int ldo;
  int out_packed;  // out in fragment order with ldo columns
  int causal_R, n_tiles;  // causal mode as in AttnParams (B = 16, n_rh over (request, tile) pairs)
};

// Output row of query row q of request (or, in causal mode, (request, tile)
// pair) rv; false for a padding row.
__host__ __device__ inline bool attn_out_row(int causal_R, int n_tiles, int B, int rv, int q, int& m) {
  if (causal_R) {
    const int r = rv / n_tiles, row = (rv - r * n_tiles) * 16 + q;
    m = r * causal_R + row;
    return row < causal_R;
  }
  m = rv * B + q;
  return q < B;
}

struct InjectReq {
  int row_start, count, slot, pos0, final_ctx;
};
struct ScatterParams {
  const float* kv;  // [n_part][rows][ld] split-K partials; a row's K/V of layer l at col0 + l*2*Hkv*dh
  int ld, col0;
  int n_part;
  int rows, L, Hkv;
  int n_req;
  InjectReq req[kMaxChunkReq];
  const float* cos_t;
  const float* sin_t;
  void* pool;
  long long layer_stride;  // elements per layer in the pool
  const int* page_table;
  int pt_stride;
  SlotState* state;
  int window;
  int max_pages;
  unsigned int* err;
};

// k per wave and weight tile of the skinny kernel with mt 16-row tiles
int gemm_kblock(int dtype, int mt);
// The skinny kernel holds up to 64 rows at once for split-K (partial) products.
inline bool gemm_use_mt4(int dtype, int M) { return dtype == DFLASH_BF16 && M > 16 && M <= 64; }
// Tiled MFMA kernel for M >= 64 (bf16): one split, lists of top-16 per row
// for `tiles` 16-row weight tiles.
inline bool gemm_use_big(int dtype, int M) { return dtype == DFLASH_BF16 && M >= 64; }
int gemm_big_lists(int tiles);
int gemm_big_split(int M, int tiles, int K);
void launch_gemm_big(int epi, const GemmParams& p, hipStream_t s);
GemmPlan plan_gemm(int tiles, int K, int kblock, bool single_split, int max_nw = 16);
void launch_gemm(int dtype, int epi, const GemmPlan& pl, const GemmParams& p, hipStream_t s);
size_t packed_elems(int N, int K);
void launch_pack(int dtype, const void* src, void* dst, int N, int K, hipStream_t s);
// z[m][f] = silu(g) * u rounded to the storage dtype, g and u summed in split
// order from the gate/up product's split-K partials part[P][M][2F] (gate
// columns 0..F-1, up columns F..2F-1); z row-major with row stride ldo.
void launch_swiglu_parts(int dtype, const float* part, int P, int M, int F, void* z, int ldo, hipStream_t s);
void launch_rmsnorm(int dtype, const NormParams& p, hipStream_t s);
void launch_qkv_post(int dtype, int dh, int n_req, const QkvPostParams& p, const SlotArgs& sl,
                     hipStream_t s);
void launch_attention(int dtype, int dh, int n_req, const AttnParams& p, const SlotArgs& sl,
                      hipStream_t s);
size_t attn_lds_bytes(int Hq, int Hkv, int dh, int KQ);
// Pages per attention split of a request with n_units pages (the block counts
// as one): `target` splits (fewer if there are fewer pages, more if a split
// would exceed `cap` pages), cut into runs of equal length so that the
// workgroups of one request finish together.  Host and device.
__host__ __device__ inline int split_pages(int n_units, int target, int cap) {
  if (n_units <= 1) return 1;
  int n = (n_units + cap - 1) / cap;
  const int want = target < n_units ? target : n_units;
  if (n < want) n = want;
  return (n_units + n - 1) / n;
}
void launch_combine(int dtype, int dh, const CombineParams& p, hipStream_t s);
void launch_scatter(int dtype, int dh, const ScatterParams& p, hipStream_t s);
// Stream-ordered update of one slot's context length on the device.
void launch_set_ctx(SlotState* state, int slot, int ctx_len, hipStream_t s);
void launch_topk_merge(const TopkParams& p, hipStream_t s);
void launch_finalize(const unsigned long long* keys, int rows, int vocab, int* draft,
                     hipStream_t s);
// Target verify forward: q of the new rows with RoPE (row-major), and causal
// attention over the request's pages (new rows' K/V already scattered).
struct TargetQParams {
  const float* qkv;  // [n_part][M][ld] split-K partials of the QKV product
  int n_part, M, ld, R, Hq, dh;
  const float* cos_t;
  const float* sin_t;
  void* q;  // [M][Hq][dh] storage dtype, or with n_tiles > 0 [n_req * n_tiles][Hq][16][dh] (zero padding rows)
  int n_tiles;
  int pos0[DFLASH_MAX_BATCH];  // position of each request's first new row
};
struct CausalAttnParams {
  const void* q;     // [M][Hq][dh]
  const void* pool;  // this layer's pages
  const int* page_table;
  int pt_stride;
  const SlotState* state;
  int max_pages, Hq, Hkv, R;
  float scale;
  void* out;  // [M][ldo] storage dtype, or fragment order
  int ldo, out_packed;
  unsigned int* err;
  int slots[DFLASH_MAX_BATCH];
  int pos0[DFLASH_MAX_BATCH];
};
void launch_target_q(int dtype, const TargetQParams& p, hipStream_t s);
void launch_causal_attn(int dtype, int dh, int n_req, const CausalAttnParams& p, hipStream_t s);

// DFlash-2 path selector: projected embedding tables (once) and the greedy
// path per request over its top-16 lists.
struct PathParams {
  const int* topk_ids;       // [n_req][B][16]
  const float* topk_logits;  // [n_req][B][16]
  const float* tu;           // [V][r] = E W_u^T
  const float* tv;           // [V][r] = E W_v^T
  int B, r, vocab;
  int* path;           // [n_req][B]
  float* step_scores;  // [n_req][B] or NULL
  unsigned int* err;
};
void launch_sel_table(int dtype, const void* embed, const void* wu, const void* wv, float* tu, float* tv, int V,
                      int d, int r, hipStream_t s);
void launch_select_path(const PathParams& p, int n_req, hipStream_t s);
// Sampled drafting and rejection-sampling verification (DFlash 2).
constexpr int kRowChunks = 16;  // chunks per target row in the sampled verification's first pass
struct SampleParams {
  float temperature;
  int top_k;    // 0 (whole vocabulary) or 1..64; the draft side caps it at 16
  float top_p;  // (0, 1]; below 1 only with top_k >= 1
  int B, vocab;
  const int* dids;    // [n][B][16] the draft's top-16 lists
  const float* dlog;  // [n][B][16]
  const float* v;     // [n][B] uniforms of the draft's draws
  int* draft;         // [n][B] drafted tokens (written by the draft draw, read by the verification)
  const float* tlog;  // [n][B+1][V] the target's logits
  const float* u;     // [n][B+1][2] uniforms: accept test, final draw
  float* row_stat;    // [n][B+1][2] (max of L/T, normaliser) without top-k
  int* row_ids;       // [n][B+1][64] kept top-k ids
  float* row_p;       // [n][B+1][64] their warped probabilities
  int* row_n;         // [n][B+1] kept count
  float* chunk_stat;                // [n][B+1][kRowChunks][2] per-chunk (max, sum) without top-k
  unsigned long long* chunk_list;   // [n][B+1][kRowChunks][64] per-chunk sorted top-64 keys
  int* accept;        // [n]
  int* committed;     // [n][B+1]
  int* last;          // [n]
  unsigned int* err;
};
void launch_draft_sample(const SampleParams& p, int n_req, hipStream_t s);
void launch_verify_sample(const SampleParams& p, int n_req, hipStream_t s);
void launch_verify(int n_req, int B, int vocab, const int* draft, const int* greedy,
                   int* accept, int* committed, int* last, unsigned int* err, hipStream_t s);

}  // namespace dflash
