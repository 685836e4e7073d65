// Host runtime behind the C ABI in include/dflash.h: argument validation,
// the host mirror of every request slot, the workspace carve-up and the
// launch sequence of each call.  Contains no kernels; its one device object
// is the static scratch array of dflash_draft_block_static.
//
// Call sequences (all kernels on the caller's stream, no synchronisation):
//   inject : per chunk of rows  fc GEMM (virtual concat of the n_feat hidden
//            arrays) -> RMSNorm -> all-layer K/V GEMM -> RoPE + page scatter
//   draft  : per layer  RMSNorm (+ residual) -> QKV GEMM -> q/k RoPE ->
//            attention (split over pages; a separate k_combine launch merges
//            the splits of requests that have more than one) -> O GEMM -> RMSNorm (+ residual) -> gate/up GEMM +
//            SwiGLU -> down GEMM; then RMSNorm (+ residual) -> LM head GEMM
//            + argmax -> decode ids.  GEMMs split over K leave fp32 partials
//            that the next kernel adds in a fixed order.
//   verify : one kernel
// dflash_draft_block_static runs the same draft sequence with its scratch
// buffers in a static device array instead of the handle's workspace.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace dflash;

namespace {

thread_local std::string g_err;

dflash_status fail(dflash_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

dflash_status hip_fail(hipError_t e, const char* what) {
  return fail(DFLASH_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

size_t elt(const dflash_config& c) { return c.dtype == DFLASH_BF16 ? 2 : 4; }

// Attention splits: a request with u KV pages (the block counts as one) is
// cut into about kSplitTarget(handle) splits of at most 64 pages; the cut
// depends only on the handle and the request's own context, so a request's
// arithmetic does not depend on the other requests of a call.  Small batches
// aim at enough workgroups to cover the CUs, large batches at few partials.
constexpr int kPpsCap = 64;
int max_units(const dflash_config& c) {
  return c.window ? c.window / 16 + 2 : c.max_pages_per_req + 1;
}
int split_target(const dflash_config& c) {
  return std::min(64, std::max(1, 256 / (c.max_batch * c.n_kv_heads)));
}
// ceil(u / ceil(u / T)) <= T; capped splits number at most ceil(u / 64)
int max_splits(const dflash_config& c) {
  return std::max(split_target(c), (max_units(c) + kPpsCap - 1) / kPpsCap);
}
// Upper bound of (requests x attention splits) handled in one draft call.
int part_pairs(const dflash_config& c) { return c.max_batch * max_splits(c); }

// Split-K factors of every GEMM (fixed by the shapes; the workspace holds
// their partial planes).
struct Plans {
  GemmPlan qkv, o, gateup, down, lm, fc, kv;
  GemmPlan dconv;  // rank-r projection of a conv input (dynamic conv taps)
};

// Width of the O and down products: with dynamic conv taps they carry 2r
// extra output rows (the taps' projection folded into them, as hi + lo).
int out_width(const dflash_config& c) { return c.hidden + (c.conv2 && c.conv_rank ? 2 * c.conv_rank : 0); }

int tiles_of(int n) { return (n + 15) / 16; }

// The skinny QKV product writes q and the block K/V itself (RoPE epilogue,
// no split-K); the tiled one writes split-K partials for k_qkv_post.
bool qkv_rope(const dflash_config& c, int M) {
  return !c.target && !gemm_use_big(c.dtype, M) && !gemm_use_mt4(c.dtype, M) &&
         (M + c.block_size - 1) / c.block_size <= kMaxRopeReq;
}

Plans plans16(const dflash_config& c, int M) {
  const int d = c.hidden, qd = c.n_q_heads * c.head_dim, dn = out_width(c);
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  // 17..64 rows: the split-K products stream their weights once for all
  // rows (skinny kernel, 64-row block); so does the gate/up product, whose
  // SwiGLU then runs on its partials.
  // At exactly 64 rows the tiled kernel (split-K 8 and 12) streams the O and
  // down weights faster than the 64-row block (measured 13 vs 15.5 us per O
  // launch at 33.6 MB), and the QKV and injection products slower.
  if (gemm_use_mt4(c.dtype, M)) {
    const int kb4 = gemm_kblock(c.dtype, 4);
    auto mt4 = [&](int tiles, int K) {
      GemmPlan g = plan_gemm(tiles, K, kb4, false, 8);
      g.mt = 4;
      return g;
    };
    auto tiled = [&](int tiles, int K) { return GemmPlan{gemm_big_split(M, tiles, K), 4, 1, 0}; };
    const bool tiled_ok = gemm_use_big(c.dtype, M);  // exactly 64 rows
    const GemmPlan one{1, 4, 1, 0};
    Plans p;
    p.qkv = mt4(tiles_of(qkvw), d);
    p.o = tiled_ok ? tiled(tiles_of(dn), qd) : mt4(tiles_of(dn), qd);
    // gate/up as one split-K product of 2F columns (weights streamed once for
    // all rows), then the SwiGLU from its partials
    p.gateup = tiled_ok ? one : mt4(tiles_of(2 * c.ffn), d);
    p.down = tiled_ok ? tiled(tiles_of(dn), c.ffn) : mt4(tiles_of(dn), c.ffn);
    p.lm = mt4(tiles_of(c.vocab), d);  // partial logits, then k_logit_select
    p.fc = mt4(tiles_of(d), c.n_feat * d);
    p.kv = mt4(c.n_layers * tiles_of(2 * c.n_kv_heads * c.head_dim), d);
    return p;
  }
  if (gemm_use_big(c.dtype, M)) {  // tiled kernel: split-K only for partial outputs
    auto tiled = [&](int tiles, int K) { return GemmPlan{gemm_big_split(M, tiles, K), 4, 1, 0}; };
    const GemmPlan one{1, 4, 1, 0};
    Plans p;
    p.qkv = tiled(tiles_of(qkvw), d);
    p.o = tiled(tiles_of(dn), qd);
    p.gateup = one;
    p.down = tiled(tiles_of(dn), c.ffn);
    p.lm = one;
    p.fc = tiled(tiles_of(d), c.n_feat * d);
    p.kv = tiled(c.n_layers * tiles_of(2 * c.n_kv_heads * c.head_dim), d);
    return p;
  }
  const int kb = gemm_kblock(c.dtype, 1);
  Plans p;
  p.qkv = qkv_rope(c, M) ? plan_gemm(tiles_of(qkvw) / 2, d, kb, true) : plan_gemm(tiles_of(qkvw), d, kb, false);
  p.o = plan_gemm(tiles_of(dn), qd, kb, false);
  p.gateup = plan_gemm(tiles_of(c.ffn), d, kb, true);
  p.down = plan_gemm(tiles_of(dn), c.ffn, kb, false);
  p.lm = plan_gemm(tiles_of(c.vocab), d, kb, true);
  p.fc = plan_gemm(tiles_of(d), c.n_feat * d, kb, false);
  p.kv = plan_gemm(c.n_layers * tiles_of(2 * c.n_kv_heads * c.head_dim), d, kb, false);
  return p;
}

// The products' plans for M rows.  A 4-bit draft runs every product of its
// quantised matrices on the skinny kernel (one 16-row block up to 16 rows,
// 64-row blocks above, each block streaming the codes once; gate/up above
// 16 rows as split-K partials and the SwiGLU pass); the LM head keeps its
// plan.
Plans make_plans(const dflash_config& c, int M) {
  Plans p = plans16(c, M);
  if (c.conv2 && c.conv_rank) {  // the skinny kernel for the small projection (64-row blocks above 16 rows)
    if (M <= 16) {
      p.dconv = plan_gemm(c.conv_rank / 16, c.hidden, gemm_kblock(c.dtype, 1), false);
    } else {
      p.dconv = plan_gemm(c.conv_rank / 16, c.hidden, gemm_kblock(c.dtype, 4), false, 8);
      p.dconv.mt = c.dtype == DFLASH_BF16 ? 4 : 1;
    }
  }
  if (c.weight_bits != 4) return p;
  const int d = c.hidden, qd = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int kb1 = gemm_kblock(c.dtype, 1), kb4 = gemm_kblock(c.dtype, 4);
  auto w4 = [&](int tiles, int K) {
    if (M <= 16) return plan_gemm(tiles, K, kb1, false);
    GemmPlan g = plan_gemm(tiles, K, kb4, false, 8);
    g.mt = 4;
    return g;
  };
  p.qkv = qkv_rope(c, M) ? plan_gemm(tiles_of(qkvw) / 2, d, kb1, true) : w4(tiles_of(qkvw), d);
  p.o = w4(tiles_of(d), qd);
  p.gateup = M <= 16 ? plan_gemm(tiles_of(c.ffn), d, kb1, true) : w4(tiles_of(2 * c.ffn), d);
  p.down = w4(tiles_of(d), c.ffn);
  p.fc = w4(tiles_of(d), c.n_feat * d);
  p.kv = w4(c.n_layers * tiles_of(2 * c.n_kv_heads * c.head_dim), d);
  return p;
}

// Rows of partial planes a product needs at most: max over M <= max_rows of
// P(M) * M (the split factor depends on the row count).
size_t part_rows(const dflash_config& c, GemmPlan Plans::*f, int max_rows) {
  size_t m = 0;
  for (int M = 1; M <= max_rows; ++M) m = std::max(m, (size_t)(make_plans(c, M).*f).P * M);
  return m;
}

// Per target row of the sampled verification: (max, normaliser), 64 kept
// ids, 64 probabilities, the kept count (floats and ints of 4 bytes).
constexpr int kSampleRowFloats = 2 + 64 + 64 + 1;

// Device memory of a handle, in two parts.  State (kept across calls): slot
// state, error word, page table, RoPE tables, and the block's q / K / V tiles
// whose rows B..15 stay zero.  Scratch (rewritten by every call before it is
// read): the residual stream, GEMM inputs, split-K partial planes, attention
// split partials, selection keys and lists, inject staging.
struct Scratch {
  size_t h, h2, xa, xo, qkv, part_o, part_ml, nsplit, z, keys, tlists, lpart, opart, dpart;
  size_t srow;       // sampled verification: per target row statistics and kept lists
  size_t schunk;     // sampled verification: per row chunk lists (u64) and statistics
  size_t tq;         // target: q of the new rows [M][Hq*dh]
  size_t gpart;      // split-K partials of the gate/up product (17..63 rows)
  size_t xn, tpart, otaps;  // dynamic conv taps
  size_t ssq;               // per 16-column tile sums of squares of the residual rows [M][d/16]
  size_t u, f, kvo;  // inject only (0 when not laid out)
  size_t total;
};

struct Layout {
  size_t state, err, page_table, cos_t, sin_t, qb, blk;
  size_t xa0;  // the block's layer-0 input row, RMSNorm(mask embedding) * g, formed once
  size_t scratch;  // offset of the scratch part in the workspace
  Scratch sc;
  size_t total;
};

// Scratch of a draft call of up to n_req requests (and, with inject, of an
// inject chunk of max_inject_rows rows), offsets from a 256-byte aligned base.
Scratch make_scratch(const dflash_config& c, int n_req, bool inject) {
  Scratch S{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t e = elt(c);
  const size_t M = (size_t)n_req * c.block_size;
  const size_t qd = (size_t)c.n_q_heads * c.head_dim;
  const size_t qkvw = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  S.h = take(sizeof(float) * M * c.hidden);
  // the conv variant alternates the residual stream between two buffers (a
  // norm re-reads the previous row of its input while writing its output)
  S.h2 = c.conv2 ? take(sizeof(float) * M * c.hidden) : 0;
  S.ssq = take(sizeof(float) * M * (size_t)tiles_of(c.hidden));
  S.srow = c.topk ? take(sizeof(float) * (size_t)n_req * (c.block_size + 1) * kSampleRowFloats) : 0;
  S.schunk = c.topk ? take((2 * sizeof(float) + 64 * sizeof(unsigned long long)) * (size_t)n_req *
                           (c.block_size + 1) * kRowChunks)
                    : 0;
  // a target's split attention takes q in 16-row tiles per request
  const size_t n_tiles = c.target ? (size_t)(c.block_size + 15) / 16 : 1;
  S.tq = c.target ? take(e * (size_t)n_req * n_tiles * 16 * qd) : 0;
  // GEMM inputs: rows rounded up to whole 16-row fragments (fragment order)
  const size_t M16 = (M + 15) / 16 * 16;
  S.xa = take(e * M16 * c.hidden);
  S.xo = take(e * M16 * qd);
  S.qkv = take(sizeof(float) * part_rows(c, &Plans::qkv, (int)M) * qkvw);
  const size_t pp = (size_t)n_req * n_tiles * max_splits(c) * c.n_q_heads * 16;
  S.part_o = take(sizeof(float) * pp * c.head_dim);
  S.part_ml = take(sizeof(float) * pp * 2);
  S.nsplit = take(sizeof(int) * n_req * n_tiles);
  S.z = take(e * M16 * c.ffn);
  S.keys = take(sizeof(unsigned long long) * M);
  S.tlists = c.topk ? take(sizeof(unsigned long long) * M * 16 *
                           std::max({256, gemm_big_lists(tiles_of(c.vocab)), logit_sel_lists(c.vocab)}))
                    : 0;
  {  // split-K partial logits of the 64-row vocabulary product
    size_t lrows = 0;
    for (int m = 1; m <= (int)M; ++m) {
      const GemmPlan g = make_plans(c, m).lm;
      if (g.mt == 4) lrows = std::max(lrows, (size_t)g.P * m);
    }
    S.lpart = lrows ? take(sizeof(float) * lrows * c.vocab) : 0;
  }
  {  // split-K partials of the gate/up product, where it runs split
    size_t grows = 0;
    for (int m = 1; m <= (int)M; ++m) {
      const GemmPlan g = make_plans(c, m).gateup;
      if (g.mt == 4) grows = std::max(grows, (size_t)g.P * m);
    }
    S.gpart = grows ? take(sizeof(float) * grows * 2 * c.ffn) : 0;
  }
  S.opart = take(sizeof(float) * part_rows(c, &Plans::o, (int)M) * out_width(c));
  S.dpart = take(sizeof(float) * part_rows(c, &Plans::down, (int)M) * out_width(c));
  if (c.conv2 && c.conv_rank) {  // dynamic conv taps: stored normed rows, the projection's partials, taps
    S.xn = take(e * M16 * c.hidden);
    S.tpart = take(sizeof(float) * part_rows(c, &Plans::dconv, (int)M) * c.conv_rank);
    S.otaps = take(sizeof(float) * M * 2 * c.hidden);
  }
  if (inject) {
    const size_t R = c.max_inject_rows;
    S.u = take(sizeof(float) * part_rows(c, &Plans::fc, (int)R) * c.hidden);
    S.f = take(e * R * c.hidden);
    S.kvo = take(sizeof(float) * part_rows(c, &Plans::kv, (int)R) * (size_t)c.n_layers * 2 * c.n_kv_heads *
                 c.head_dim);
  }
  S.total = off;
  return S;
}

Layout make_layout(const dflash_config& c) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  const size_t e = elt(c);
  const size_t page_elems = 2ull * c.n_kv_heads * 16 * c.head_dim;
  L.state = take(sizeof(SlotState) * c.max_batch);
  L.err = take(16);
  L.page_table = take(sizeof(int32_t) * c.max_batch * (size_t)c.max_pages_per_req);
  L.cos_t = take(sizeof(float) * (size_t)c.max_position * (c.head_dim / 2));
  L.sin_t = take(sizeof(float) * (size_t)c.max_position * (c.head_dim / 2));
  L.qb = take(e * (size_t)c.max_batch * c.n_q_heads * 16 * c.head_dim);
  L.blk = take(e * (size_t)c.max_batch * page_elems);
  L.xa0 = take(e * (size_t)c.hidden);
  L.sc = make_scratch(c, c.max_batch, !c.target);
  L.scratch = take(L.sc.total);
  L.total = off;
  return L;
}

const char* wptr(const void* p, size_t elem_off, size_t e) {
  return reinterpret_cast<const char*>(p) + elem_off * e;
}

// Packed (MFMA fragment order) copies of every weight matrix.
// With a path selector, also the projected embedding tables (fp32 [V, r]).
struct PackedLayout {
  size_t lm_head, fc, wqkv[DFLASH_MAX_LAYERS], wo[DFLASH_MAX_LAYERS], wgateup[DFLASH_MAX_LAYERS],
      wdown[DFLASH_MAX_LAYERS];
  size_t dconv[DFLASH_MAX_LAYERS][2];  // dynamic conv: D of the convs before attention and the MLP
  size_t sel_u, sel_v;
  size_t total;
};

PackedLayout make_packed(const dflash_config& c) {
  PackedLayout P{};
  size_t off = 0;
  const size_t e = elt(c);
  auto take = [&](int N, int K) {
    size_t o = off;
    off = align_up(off + packed_elems(N, K) * e);
    return o;
  };
  // the draft's own matrices: 4-bit codes and scales for a 4-bit draft
  auto takeq = [&](int N, int K) {
    if (c.weight_bits != 4) return take(N, K);
    size_t o = off;
    off = align_up(off + q4_bytes(N, K));
    return o;
  };
  const int d = c.hidden, qd = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  P.lm_head = take(c.vocab, d);
  P.fc = c.target ? 0 : takeq(d, c.n_feat * d);
  const int dn = out_width(c);  // W_o and W_down with D W of the output convs appended
  for (int l = 0; l < c.n_layers; ++l) {
    P.wqkv[l] = takeq(qkvw, d);
    P.wo[l] = takeq(dn, qd);
    P.wgateup[l] = takeq(2 * c.ffn, d);
    P.wdown[l] = takeq(dn, c.ffn);
    if (c.conv2 && c.conv_rank) {
      P.dconv[l][0] = take(c.conv_rank, d);
      P.dconv[l][1] = take(c.conv_rank, d);
    }
  }
  if (c.selector_rank) {
    const size_t tb = sizeof(float) * (size_t)c.vocab * c.selector_rank;
    P.sel_u = off;
    off = align_up(off + tb);
    P.sel_v = off;
    off = align_up(off + tb);
  }
  P.total = off;
  return P;
}

dflash_status validate(const dflash_config* c) {
  if (!c) return fail(DFLASH_E_INVALID, "config is NULL");
  auto bad = [&](const char* what) { return fail(DFLASH_E_INVALID, "config: %s", what); };
  if (c->hidden <= 0 || c->hidden % 256 || c->hidden > 8192) return bad("hidden must be a multiple of 256 in (0, 8192]");
  if (c->head_dim != 64 && c->head_dim != 128) return bad("head_dim must be 64 or 128");
  if (c->n_kv_heads <= 0 || c->n_q_heads <= 0 || c->n_q_heads % c->n_kv_heads)
    return bad("n_q_heads must be a positive multiple of n_kv_heads");
  if (c->n_q_heads / c->n_kv_heads > 8) return bad("at most 8 query heads per KV head");
  if ((c->n_q_heads * c->head_dim) % 256) return bad("n_q_heads*head_dim must be a multiple of 256");
  if (c->ffn <= 0 || c->ffn % 256) return bad("ffn must be a positive multiple of 256");
  if (c->vocab <= 0) return bad("vocab must be positive");
  if (c->n_layers < 1 || c->n_layers > DFLASH_MAX_LAYERS) return bad("n_layers out of range");
  if (c->target != 0 && c->target != 1) return bad("target must be 0 or 1");
  if (c->weight_bits != 16 && c->weight_bits != 4) return bad("weight_bits must be 16 or 4");
  if (c->weight_bits == 4 && (c->dtype != DFLASH_BF16 || c->target))
    return bad("4-bit weights need a bf16 draft (not a target)");
  if (c->conv_rank != 0 && c->conv_rank != 32 && c->conv_rank != 64) return bad("conv_rank must be 0, 32 or 64");
  if (c->conv_rank && (!c->conv2 || c->weight_bits != 16))
    return bad("dynamic conv taps need conv2 and storage-dtype weights");
  if (c->target) {
    if (c->block_size < 1 || c->block_size > 64) return bad("a target takes 1 to 64 rows per request");
    if (c->window || c->conv2 || c->topk || c->selector_rank)
      return bad("a target has no window, conv taps, top-16 lists or path selector");
  } else if (c->block_size < 1 || c->block_size > 16) {
    return bad("block_size must be in [1, 16]");
  }
  if (c->n_feat < 1 || c->n_feat > DFLASH_MAX_FEAT) return bad("n_feat out of range");
  if (c->dtype != DFLASH_BF16 && c->dtype != DFLASH_F32) return bad("unknown dtype");
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return bad("mask_token_id out of range");
  if (c->page_size != DFLASH_PAGE_SIZE) return bad("page_size must be 16");
  if (c->window < 0 || c->window % 16) return bad("window must be 0 or a positive multiple of 16");
  if (c->conv2 != 0 && c->conv2 != 1) return bad("conv2 must be 0 or 1");
  if (c->topk != 0 && c->topk != DFLASH_MAX_TOPK) return bad("topk must be 0 or 16");
  if (c->topk && c->vocab < DFLASH_MAX_TOPK) return bad("topk needs vocab >= 16");
  if (c->max_batch < 1 || c->max_batch > DFLASH_MAX_BATCH) return bad("max_batch out of range");
  if (c->max_pages < 1) return bad("max_pages must be positive");
  if (c->max_pages_per_req < 1 || c->max_pages_per_req > 4095)
    return bad("max_pages_per_req must be in [1, 4095] (contexts up to 65520 tokens)");
  if (c->window > 65472) return bad("window must be at most 65472");
  if (c->window && c->max_pages_per_req < c->window / 16 + 1)
    return bad("max_pages_per_req must hold window/16 + 1 pages");
  if (c->max_position < c->block_size + 2) return bad("max_position too small");
  if (c->max_inject_rows < 1) return bad("max_inject_rows must be positive");
  if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) return bad("rms_eps and rope_theta must be positive");
  if (c->selector_rank < 0 || c->selector_rank > 512 || c->selector_rank % 64)
    return bad("selector_rank must be 0 or a multiple of 64 up to 512");
  if (c->selector_rank && c->topk != DFLASH_MAX_TOPK) return bad("the path selector needs topk 16");
  // the LM head and SwiGLU GEMMs run unsplit: K = hidden must fit 16 waves
  const int max_d = 16 * gemm_kblock(c->dtype, 1);
  if (c->hidden > max_d)
    return fail(DFLASH_E_UNSUPPORTED, "config: hidden above %d is not supported", max_d);
  return DFLASH_OK;
}

struct HostSlot {
  bool bound = false;
  int ctx_len = 0, kv_begin = 0, n_pages = 0;
};

// Launch timing: pairs of events per bracketed launch, reused across runs.
struct Profiler {
  uint32_t mask = 0;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<std::pair<int, size_t>> marks;  // (kernel class, first event index)
};

}  // namespace

struct dflash_handle {
  dflash_config cfg;
  dflash_weights w;
  char* kv;
  char* ws;
  char* packed;
  Layout lay;
  PackedLayout pk;
  std::vector<HostSlot> slots;
  bool dev_init = false;
  Profiler prof;
  std::vector<Scratch> static_sc;  // scratch layouts of static-scratch calls, by request count
};

// Points segment `seg` of g at tile `tile0` of the packed [N, K] matrix at
// offset `off` (4-bit: its codes and scales).
static void set_weights(const dflash_handle* h, GemmParams& g, int seg, size_t off, int N, int K, int tile0 = 0) {
  if (h->cfg.weight_bits == 4) {
    g.w4 = 1;
    g.w[seg] = h->packed + off + (size_t)tile0 * K * 8;
    g.sb[seg] = h->packed + off + q4_codes_bytes(N, K) + (size_t)tile0 * K;
  } else {
    g.w[seg] = h->packed + off + (size_t)tile0 * 16 * K * elt(h->cfg);
  }
}


namespace {

template <typename P>
P* at(dflash_handle* h, size_t off) {
  return reinterpret_cast<P*>(h->ws + off);
}

// a buffer of the scratch part at base sb
template <typename P>
P* sat(char* sb, size_t off) {
  return reinterpret_cast<P*>(sb + off);
}

dflash_status ensure_device(dflash_handle* h) {
  if (h->dev_init) return DFLASH_OK;
  const dflash_config& c = h->cfg;
  const int half = c.head_dim / 2;
  std::vector<float> cs((size_t)c.max_position * half), sn((size_t)c.max_position * half);
  for (int p = 0; p < c.max_position; ++p)
    for (int j = 0; j < half; ++j) {
      const double inv = pow((double)c.rope_theta, -(2.0 * j) / (double)c.head_dim);
      const double a = (double)p * inv;
      cs[(size_t)p * half + j] = (float)cos(a);
      sn[(size_t)p * half + j] = (float)sin(a);
    }
  hipError_t e;
  if ((e = hipMemcpy(h->ws + h->lay.cos_t, cs.data(), cs.size() * 4, hipMemcpyHostToDevice)))
    return hip_fail(e, "rope table upload");
  if ((e = hipMemcpy(h->ws + h->lay.sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice)))
    return hip_fail(e, "rope table upload");
  if ((e = hipMemset(h->ws + h->lay.state, 0, sizeof(SlotState) * c.max_batch)))
    return hip_fail(e, "state init");
  if ((e = hipMemset(h->ws + h->lay.err, 0, 16))) return hip_fail(e, "state init");
  // rows B..15 of the block's q / K / V tiles stay zero (the RoPE epilogue
  // writes rows 0..B-1 only)
  if ((e = hipMemset(h->ws + h->lay.qb, 0, h->lay.blk - h->lay.qb))) return hip_fail(e, "state init");
  if ((e = hipMemset(h->ws + h->lay.blk, 0, elt(c) * (size_t)c.max_batch * 2 * c.n_kv_heads * 16 * c.head_dim)))
    return hip_fail(e, "state init");
  if ((e = hipMemset(h->ws + h->lay.page_table, 0xff,
                     sizeof(int32_t) * c.max_batch * (size_t)c.max_pages_per_req)))
    return hip_fail(e, "page table init");
  // weights into MFMA fragment order (read once here)
  const int d = c.hidden, qd = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  launch_pack(c.dtype, h->w.lm_head, h->packed + h->pk.lm_head, c.vocab, d, nullptr);
  // the draft's own matrices: fragment order, or quantised to 4-bit codes
  auto packq = [&](const void* src, size_t off, int N, int K) {
    if (c.weight_bits == 4)
      launch_pack_q4(src, h->packed + off, N, K, nullptr);
    else
      launch_pack(c.dtype, src, h->packed + off, N, K, nullptr);
  };
  if (!c.target) packq(h->w.fc, h->pk.fc, d, c.n_feat * d);
  const int r = c.conv2 ? c.conv_rank : 0;
  const size_t es = elt(c);
  char* fold = h->ws + h->lay.scratch;  // scratch is free at set-up: D W of an output conv before packing
  if (r && (size_t)2 * r * std::max(qd, c.ffn) * es > h->lay.sc.total)
    return fail(DFLASH_E_CAPACITY, "workspace scratch too small to fold the conv taps' forms");
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& lw = h->w.layers[l];
    packq(lw.wqkv, h->pk.wqkv[l], qkvw, d);
    packq(lw.wo, h->pk.wo[l], d, qd);
    packq(lw.wgateup, h->pk.wgateup[l], 2 * c.ffn, d);
    packq(lw.wdown, h->pk.wdown[l], d, c.ffn);
    if (r) {  // dynamic conv taps: D of the input convs; D W joins W_o and W_down as r extra rows
      const size_t dpt = (size_t)r * d * es;  // bytes of one point's D
      launch_pack(c.dtype, wptr(lw.dconv_d, 0, 1), h->packed + h->pk.dconv[l][0], r, d, nullptr);
      launch_pack(c.dtype, wptr(lw.dconv_d, 2 * dpt, 1), h->packed + h->pk.dconv[l][1], r, d, nullptr);
      launch_fold(c.dtype, wptr(lw.dconv_d, dpt, 1), lw.wo, fold, r, d, qd, nullptr);
      launch_pack(c.dtype, fold, h->packed + h->pk.wo[l] + (size_t)d * qd * es, 2 * r, qd, nullptr);
      launch_fold(c.dtype, wptr(lw.dconv_d, 3 * dpt, 1), lw.wdown, fold, r, d, c.ffn, nullptr);
      launch_pack(c.dtype, fold, h->packed + h->pk.wdown[l] + (size_t)d * c.ffn * es, 2 * r, c.ffn, nullptr);
    }
  }
  if (c.selector_rank)
    launch_sel_table(c.dtype, h->w.embed, h->w.sel_u, h->w.sel_v, reinterpret_cast<float*>(h->packed + h->pk.sel_u),
                     reinterpret_cast<float*>(h->packed + h->pk.sel_v), c.vocab, d, c.selector_rank, nullptr);
  if (!c.target && !c.conv2) {  // every block row enters layer 0 as this row
    NormParams np{};
    np.init_row = wptr(h->w.embed, (size_t)c.mask_token_id * d, es);
    np.gamma = h->w.layers[0].attn_norm;
    np.eps = c.rms_eps;
    np.out = h->ws + h->lay.xa0;
    np.ldo = d;
    np.d = d;
    np.M = 1;
    launch_rmsnorm(c.dtype, np, nullptr);
  }
  if ((e = hipGetLastError())) return hip_fail(e, "weight packing");
  if ((e = hipDeviceSynchronize())) return hip_fail(e, "device init");
  h->dev_init = true;
  return DFLASH_OK;
}

// Bracket one launch of class `k` with events when timing is on for it.
struct ProfScope {
  dflash_handle* h;
  hipStream_t s;
  int k;
  size_t idx;
  bool on;
  ProfScope(dflash_handle* h_, int k_, hipStream_t s_) : h(h_), s(s_), k(k_), idx(0), on(false) {
    Profiler& p = h->prof;
    if (!(p.mask & (1u << k))) return;
    while (p.pool.size() < p.used + 2) {
      hipEvent_t e;
      // timing-only events: without the system-scope fence a record costs the
      // stream no cache writeback (with it, each record left the GPU idle for
      // about 5.6 us between the bracketed launch and its neighbours)
      if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
      p.pool.push_back(e);
    }
    idx = p.used;
    p.used += 2;
    on = hipEventRecord(p.pool[idx], s) == hipSuccess;
  }
  ~ProfScope() {
    if (!on) return;
    if (hipEventRecord(h->prof.pool[idx + 1], s) == hipSuccess) h->prof.marks.push_back({k, idx});
  }
};

dflash_status check_slots(dflash_handle* h, int32_t n_req, const int32_t* slots) {
  if (n_req < 1 || n_req > h->cfg.max_batch) return fail(DFLASH_E_INVALID, "n_req %d out of [1, %d]", n_req, h->cfg.max_batch);
  if (!slots) return fail(DFLASH_E_INVALID, "slots is NULL");
  std::vector<char> seen(h->cfg.max_batch, 0);
  for (int i = 0; i < n_req; ++i) {
    const int s = slots[i];
    if (s < 0 || s >= h->cfg.max_batch) return fail(DFLASH_E_INVALID, "slot %d out of range", s);
    if (seen[s]) return fail(DFLASH_E_INVALID, "slot %d listed twice", s);
    seen[s] = 1;
    if (!h->slots[s].bound) return fail(DFLASH_E_INVALID, "slot %d is not bound", s);
  }
  return DFLASH_OK;
}

// Scratch for callers that cannot allocate (dflash_draft_block_static): one
// static device array per GPU, shared by every handle and call on that GPU.
// Host code never uses the array's name as an address: the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current.
constexpr size_t kStaticScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) char scratch[kStaticScratchBytes];
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];

dflash_status static_scratch(dflash_handle* h, int n_req, char** base, const Scratch** sc) {
  if ((int)h->static_sc.size() <= n_req) h->static_sc.resize(n_req + 1, Scratch{});
  Scratch& S = h->static_sc[n_req];
  if (S.total == 0) S = make_scratch(h->cfg, n_req, false);
  if (S.total > kStaticScratchBytes)
    return fail(DFLASH_E_CAPACITY, "static scratch: %d requests need %zu bytes, above the %zu-byte array", n_req,
                S.total, kStaticScratchBytes);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e) return hip_fail(e, "static scratch: current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(DFLASH_E_UNSUPPORTED, "static scratch: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e) return hip_fail(e, "static scratch: symbol address");
    g_scratch_ptr[dev] = reinterpret_cast<char*>(p);
  }
  *base = g_scratch_ptr[dev];
  *sc = &S;
  return DFLASH_OK;
}

dflash_status launched(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, what);
  return DFLASH_OK;
}

}  // namespace

extern "C" {

int32_t dflash_abi_version(void) { return DFLASH_ABI_VERSION; }

const char* dflash_last_error(void) { return g_err.c_str(); }

dflash_status dflash_validate_config(const dflash_config* cfg) { return validate(cfg); }

dflash_status dflash_feature_layers(int32_t n_target_layers, int32_t k, int32_t* out) {
  if (!out) return fail(DFLASH_E_INVALID, "out is NULL");
  if (k < 2 || n_target_layers < 4) return fail(DFLASH_E_INVALID, "need k >= 2 and n_target_layers >= 4");
  const int first = 1, last = n_target_layers - 3;
  for (int i = 0; i < k; ++i) out[i] = first + (i * (last - first)) / (k - 1);
  return DFLASH_OK;
}

size_t dflash_workspace_bytes(const dflash_config* cfg) {
  if (validate(cfg) != DFLASH_OK) return 0;
  return make_layout(*cfg).total;
}

size_t dflash_packed_weights_bytes(const dflash_config* cfg) {
  if (validate(cfg) != DFLASH_OK) return 0;
  return make_packed(*cfg).total;
}

size_t dflash_kv_pool_bytes(const dflash_config* cfg) {
  if (validate(cfg) != DFLASH_OK) return 0;
  return (size_t)cfg->n_layers * cfg->max_pages * 2ull * cfg->n_kv_heads * 16 * cfg->head_dim * elt(*cfg);
}

dflash_status dflash_create(const dflash_config* cfg, const dflash_weights* w, void* kv_pool,
                            void* workspace, void* packed, dflash_handle** out) {
  if (!out) return fail(DFLASH_E_INVALID, "out is NULL");
  *out = nullptr;
  dflash_status st = validate(cfg);
  if (st) return st;
  if (!w) return fail(DFLASH_E_INVALID, "weights is NULL");
  if (!kv_pool || !workspace || !packed)
    return fail(DFLASH_E_INVALID, "kv_pool, workspace and packed must be set");
  if ((reinterpret_cast<uintptr_t>(kv_pool) | reinterpret_cast<uintptr_t>(workspace) |
       reinterpret_cast<uintptr_t>(packed)) & 255)
    return fail(DFLASH_E_INVALID, "kv_pool, workspace and packed must be 256-byte aligned");
  if (!w->embed || !w->lm_head || !w->final_norm || (!cfg->target && (!w->fc || !w->fc_norm)))
    return fail(DFLASH_E_INVALID, "a model weight pointer is NULL");
  for (int l = 0; l < cfg->n_layers; ++l) {
    const dflash_layer_weights& lw = w->layers[l];
    if (!lw.wqkv || !lw.wo || !lw.wgateup || !lw.wdown || !lw.attn_norm || !lw.mlp_norm)
      return fail(DFLASH_E_INVALID, "layer %d: a weight pointer is NULL", l);
    if (cfg->conv2 && !lw.conv) return fail(DFLASH_E_INVALID, "layer %d: conv taps are NULL", l);
    if (cfg->conv_rank && (!lw.dconv_d || !lw.dconv_u))
      return fail(DFLASH_E_INVALID, "layer %d: dynamic conv forms are NULL", l);
  }
  if (cfg->selector_rank && (!w->sel_u || !w->sel_v))
    return fail(DFLASH_E_INVALID, "selector_rank is set but sel_u / sel_v are NULL");
  dflash_handle* h = new dflash_handle();
  h->cfg = *cfg;
  h->w = *w;
  h->kv = reinterpret_cast<char*>(kv_pool);
  h->ws = reinterpret_cast<char*>(workspace);
  h->packed = reinterpret_cast<char*>(packed);
  h->lay = make_layout(*cfg);
  h->pk = make_packed(*cfg);
  h->slots.resize(cfg->max_batch);
  *out = h;
  return DFLASH_OK;
}

void dflash_destroy(dflash_handle* h) {
  if (!h) return;
  for (hipEvent_t e : h->prof.pool) (void)hipEventDestroy(e);
  delete h;
}

int32_t dflash_context_length(const dflash_handle* h, int32_t slot) {
  if (!h || slot < 0 || slot >= h->cfg.max_batch || !h->slots[slot].bound) return -1;
  return h->slots[slot].ctx_len;
}

dflash_status dflash_bind_request(dflash_handle* h, int32_t slot, const int32_t* page_ids,
                                  int32_t n_pages, int32_t start_pos) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  const dflash_config& c = h->cfg;
  if (slot < 0 || slot >= c.max_batch) return fail(DFLASH_E_INVALID, "slot %d out of range", slot);
  if (n_pages < 1 || n_pages > c.max_pages_per_req)
    return fail(DFLASH_E_INVALID, "n_pages %d out of [1, %d]", n_pages, c.max_pages_per_req);
  if (!page_ids) return fail(DFLASH_E_INVALID, "page_ids is NULL");
  for (int i = 0; i < n_pages; ++i)
    if (page_ids[i] < 0 || page_ids[i] >= c.max_pages)
      return fail(DFLASH_E_INVALID, "page id %d out of [0, %d)", page_ids[i], c.max_pages);
  if (c.window && n_pages < c.window / 16 + 1)
    return fail(DFLASH_E_INVALID, "a window of %d needs at least %d pages", c.window, c.window / 16 + 1);
  if (start_pos < 0 || start_pos + c.block_size + 1 > c.max_position)
    return fail(DFLASH_E_INVALID, "start_pos %d out of range", start_pos);
  if (!c.window && start_pos > n_pages * 16)
    return fail(DFLASH_E_INVALID, "start_pos %d beyond the bound pages", start_pos);
  dflash_status st = ensure_device(h);
  if (st) return st;
  hipError_t e;
  if ((e = hipMemcpy(h->ws + h->lay.page_table + sizeof(int32_t) * (size_t)slot * c.max_pages_per_req,
                     page_ids, sizeof(int32_t) * n_pages, hipMemcpyHostToDevice)))
    return hip_fail(e, "page table upload");
  SlotState s{start_pos, start_pos, n_pages, 0};
  if ((e = hipMemcpy(h->ws + h->lay.state + sizeof(SlotState) * slot, &s, sizeof(s),
                     hipMemcpyHostToDevice)))
    return hip_fail(e, "slot state upload");
  HostSlot& hs = h->slots[slot];
  hs.bound = true;
  hs.ctx_len = start_pos;
  hs.kv_begin = start_pos;
  hs.n_pages = n_pages;
  return DFLASH_OK;
}

dflash_status dflash_inject_context(dflash_handle* h, void* stream, int32_t n_req,
                                    const int32_t* slots, const int32_t* n_new,
                                    const void* const* hidden, void* debug_f) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  const dflash_config& c = h->cfg;
  if (c.target) return fail(DFLASH_E_INVALID, "a target handle has no injection (use dflash_target_forward)");
  dflash_status st = check_slots(h, n_req, slots);
  if (st) return st;
  if (!n_new) return fail(DFLASH_E_INVALID, "n_new is NULL");
  if (!hidden) return fail(DFLASH_E_INVALID, "hidden is NULL");
  for (int k = 0; k < c.n_feat; ++k)
    if (!hidden[k]) return fail(DFLASH_E_INVALID, "hidden[%d] is NULL", k);
  long long total = 0;
  for (int i = 0; i < n_req; ++i) {
    const HostSlot& hs = h->slots[slots[i]];
    if (n_new[i] < 0) return fail(DFLASH_E_INVALID, "n_new[%d] is negative", i);
    const long long end = (long long)hs.ctx_len + n_new[i];
    if (!c.window && end > (long long)hs.n_pages * 16)
      return fail(DFLASH_E_CAPACITY, "slot %d: %lld positions exceed %d bound pages", slots[i], end, hs.n_pages);
    if (end + c.block_size + 1 > c.max_position)
      return fail(DFLASH_E_CAPACITY, "slot %d: position %lld beyond max_position", slots[i], end);
    total += n_new[i];
  }
  if (total == 0) return DFLASH_OK;
  st = ensure_device(h);
  if (st) return st;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t e = elt(c);
  const int d = c.hidden;
  const int kvw = c.n_layers * 2 * c.n_kv_heads * c.head_dim;
  const int R = c.max_inject_rows;
  const int kv_seg_tiles = tiles_of(2 * c.n_kv_heads * c.head_dim);
  char* sb = h->ws + h->lay.scratch;
  const Scratch& sc = h->lay.sc;

  // walk requests in call order, cutting chunks of <= R rows and <= kMaxChunkReq requests
  int req = 0, used = 0;  // current request and rows of it already emitted
  long long row0 = 0;     // global row of the chunk start
  while (row0 < total) {
    ScatterParams sp{};
    int rows = 0;
    sp.n_req = 0;
    while (rows < R && req < n_req && sp.n_req < kMaxChunkReq) {
      const int left = n_new[req] - used;
      if (left == 0) {
        ++req;
        used = 0;
        continue;
      }
      const int take = std::min(left, R - rows);
      const HostSlot& hs = h->slots[slots[req]];
      InjectReq& q = sp.req[sp.n_req++];
      q.row_start = rows;
      q.count = take;
      q.slot = slots[req];
      q.pos0 = hs.ctx_len + used;
      q.final_ctx = hs.ctx_len + n_new[req];
      rows += take;
      used += take;
      if (used == n_new[req]) {
        ++req;
        used = 0;
      }
    }
    const Plans pl = make_plans(c, rows);

    GemmParams g{};
    for (int k = 0; k < c.n_feat; ++k) g.a[k] = wptr(hidden[k], (size_t)row0 * d, e);
    g.a_parts = c.n_feat;
    g.a_part_k = d;
    g.lda = d;
    g.M = rows;
    set_weights(h, g, 0, h->pk.fc, d, c.n_feat * d);
    g.tiles = tiles_of(d);
    g.N = d;
    g.K = c.n_feat * d;
    g.P = pl.fc.P;
    g.out_f32 = sat<float>(sb, sc.u);
    { ProfScope ps(h, DFLASH_KERNEL_FC_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.fc, g, s); }

    NormParams np{};
    np.part = sat<float>(sb, sc.u);
    np.n_part = pl.fc.P;
    np.ldx = d;
    np.gamma = h->w.fc_norm;
    np.eps = c.rms_eps;
    np.out = sb + sc.f;
    np.ldo = d;
    np.d = d;
    np.M = rows;
    { ProfScope ps(h, DFLASH_KERNEL_NORM, s); launch_rmsnorm(c.dtype, np, s); }
    if (debug_f) {
      hipError_t err = hipMemcpyAsync(reinterpret_cast<char*>(debug_f) + (size_t)row0 * d * e,
                                      sb + sc.f, (size_t)rows * d * e,
                                      hipMemcpyDeviceToDevice, s);
      if (err) return hip_fail(err, "debug_f copy");
    }

    GemmParams kv{};
    kv.a[0] = sb + sc.f;
    kv.a_parts = 1;
    kv.a_part_k = d;
    kv.lda = d;
    kv.M = rows;
    // the K/V rows of every layer's fused QKV weight, in place
    for (int l = 0; l < c.n_layers; ++l)
      set_weights(h, kv, l, h->pk.wqkv[l], (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, d,
                  tiles_of(c.n_q_heads * c.head_dim));
    kv.seg_tiles = kv_seg_tiles;
    kv.tiles = c.n_layers * kv_seg_tiles;
    kv.N = kvw;
    kv.K = d;
    kv.P = pl.kv.P;
    kv.out_f32 = sat<float>(sb, sc.kvo);
    { ProfScope ps(h, DFLASH_KERNEL_KV_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.kv, kv, s); }

    sp.kv = sat<float>(sb, sc.kvo);
    sp.ld = kvw;
    sp.col0 = 0;
    sp.n_part = pl.kv.P;
    sp.rows = rows;
    sp.L = c.n_layers;
    sp.Hkv = c.n_kv_heads;
    sp.cos_t = at<float>(h, h->lay.cos_t);
    sp.sin_t = at<float>(h, h->lay.sin_t);
    sp.pool = h->kv;
    sp.layer_stride = (long long)c.max_pages * 2 * c.n_kv_heads * 16 * c.head_dim;
    sp.page_table = at<int>(h, h->lay.page_table);
    sp.pt_stride = c.max_pages_per_req;
    sp.state = at<SlotState>(h, h->lay.state);
    sp.window = c.window;
    sp.max_pages = c.max_pages;
    sp.err = at<unsigned int>(h, h->lay.err);
    { ProfScope ps(h, DFLASH_KERNEL_SCATTER, s); launch_scatter(c.dtype, c.head_dim, sp, s); }
    st = launched("inject");
    if (st) return st;
    row0 += rows;
  }
  for (int i = 0; i < n_req; ++i) h->slots[slots[i]].ctx_len += n_new[i];
  return DFLASH_OK;
}

// The MLP's gate/up product of the normed rows in xa (fragment order when
// xa_packed) into z = silu(gate) * up (fragment order when z_packed): the
// skinny or tiled kernel's SwiGLU epilogue, or from 17 to 63 rows one split-K
// product of all 2F columns and the SwiGLU over its partials.
// ssq: the rows in xa are the residual times the MLP gain, not yet scaled by
// 1/rms; the product applies it from these per-tile sums of squares.
static void gateup_swiglu(dflash_handle* h, hipStream_t s, char* sb, const Scratch& sc, const Plans& pl, int M,
                          int l, int xa_packed, int z_packed, const float* ssq = nullptr) {
  const dflash_config& c = h->cfg;
  GemmParams gu{};
  gu.a[0] = sb + sc.xa;
  gu.a_parts = 1;
  gu.a_part_k = c.hidden;
  gu.lda = c.hidden;
  gu.M = M;
  gu.K = c.hidden;
  gu.a_packed = xa_packed;
  set_weights(h, gu, 0, h->pk.wgateup[l], 2 * c.ffn, c.hidden);
  ProfScope ps(h, DFLASH_KERNEL_GATEUP_GEMM, s);
  if (pl.gateup.mt == 4) {
    float* part = sat<float>(sb, sc.gpart);
    gu.tiles = tiles_of(2 * c.ffn);
    gu.N = 2 * c.ffn;
    gu.P = pl.gateup.P;
    gu.out_f32 = part;
    launch_gemm(c.dtype, EPI_PARTIAL, pl.gateup, gu, s);
    launch_swiglu_parts(c.dtype, part, pl.gateup.P, M, c.ffn, sb + sc.z, c.ffn, s);
    return;
  }
  gu.out_packed = z_packed;
  gu.tiles = tiles_of(c.ffn);
  gu.up_tile_off = tiles_of(c.ffn);
  gu.N = c.ffn;
  gu.P = 1;
  gu.out_t = sb + sc.z;
  gu.ldt = c.ffn;
  gu.ssq = const_cast<float*>(ssq);
  gu.ssq_tiles = tiles_of(c.hidden);
  gu.ssq_d = c.hidden;
  gu.eps = c.rms_eps;
  launch_gemm(c.dtype, EPI_SWIGLU, pl.gateup, gu, s);
}

// Final step of a forward whose normed rows are in xa (fragment order when
// xa_packed): the shared LM head and greedy selection (argmax ids with ties
// to the lowest id; with top-16, the sorted lists as well).  Below 17 rows the
// skinny kernel's argmax or top-16 epilogue; from 17 to 64 rows split-K
// partial logits and the selection pass; from 64 rows the tiled kernel's
// epilogue.
static dflash_status lm_head(dflash_handle* h, hipStream_t s, char* sb, const Scratch& sc, const Plans& pl, int M,
                             int xa_packed, int32_t* draft, int32_t* topk_ids, float* topk_logits,
                             float* debug_logits) {
  const dflash_config& c = h->cfg;
  const int d = c.hidden;
  GemmParams gl{};
  gl.a[0] = sb + sc.xa;
  gl.a_parts = 1;
  gl.a_part_k = d;
  gl.lda = d;
  gl.M = M;
  gl.K = d;
  gl.a_packed = xa_packed;
  gl.w[0] = h->packed + h->pk.lm_head;
  gl.tiles = tiles_of(c.vocab);
  gl.N = c.vocab;
  gl.P = 1;
  if (pl.lm.mt == 4) {  // 17..64 rows: split-K partial logits, then the selection pass
    gl.P = pl.lm.P;
    gl.out_f32 = sat<float>(sb, sc.lpart);
    {
      ProfScope ps(h, DFLASH_KERNEL_LM_HEAD, s);
      launch_gemm(c.dtype, EPI_PARTIAL, pl.lm, gl, s);
    }
    LogitSelParams lp{};
    lp.part = gl.out_f32;
    lp.n_part = pl.lm.P;
    lp.M = M;
    lp.N = c.vocab;
    lp.dbg = debug_logits;
    lp.ld_dbg = c.vocab;
    lp.keys = sat<unsigned long long>(sb, sc.keys);
    lp.lists = sat<unsigned long long>(sb, sc.tlists);
    lp.n_lists = logit_sel_lists(c.vocab);
    {
      ProfScope ps(h, DFLASH_KERNEL_SELECT, s);
      launch_logit_select(c.topk != 0, lp, s);
    }
    if (c.topk) {
      TopkParams tp{};
      tp.lists = lp.lists;
      tp.n_lists = lp.n_lists;
      tp.M = M;
      tp.vocab = c.vocab;
      tp.draft = draft;
      tp.topk_ids = topk_ids;
      tp.topk_logits = topk_logits;
      ProfScope ps(h, DFLASH_KERNEL_TOPK, s);
      launch_topk_merge(tp, s);
    } else {
      ProfScope ps(h, DFLASH_KERNEL_FINALIZE, s);
      launch_finalize(lp.keys, M, c.vocab, draft, s);
    }
    return launched("draft head");
  }
  gl.keys = sat<unsigned long long>(sb, c.topk ? sc.tlists : sc.keys);
  gl.dbg = debug_logits;
  gl.ld_dbg = c.vocab;
  {
    ProfScope ps(h, DFLASH_KERNEL_LM_HEAD, s);
    launch_gemm(c.dtype, c.topk ? EPI_TOPK : EPI_ARGMAX, pl.lm, gl, s);
  }
  if (c.topk) {
    TopkParams tp{};
    tp.lists = gl.keys;
    tp.n_lists = pl.lm.mt == 0 ? gemm_big_lists(gl.tiles) : pl.lm.GP;
    tp.M = M;
    tp.vocab = c.vocab;
    tp.draft = draft;
    tp.topk_ids = topk_ids;
    tp.topk_logits = topk_logits;
    ProfScope ps(h, DFLASH_KERNEL_TOPK, s);
    launch_topk_merge(tp, s);
  } else {
    ProfScope ps(h, DFLASH_KERNEL_FINALIZE, s);
    launch_finalize(sat<unsigned long long>(sb, sc.keys), M, c.vocab, draft, s);
  }
  return launched("draft head");
}

// Steps 3 and 4 with the scratch part at the handle's workspace or, with
// from_static, in the library's static device array.
static dflash_status draft_impl(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                                const int32_t* last_token, int32_t* draft, int32_t* topk_ids,
                                float* topk_logits, const dflash_draft_debug* debug, bool from_static) {
  float* debug_logits = debug ? debug->logits : nullptr;
  float* debug_hidden = debug ? debug->hidden : nullptr;
  const float* hidden_in = debug ? debug->hidden_in : nullptr;
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  const dflash_config& c = h->cfg;
  if (c.target) return fail(DFLASH_E_INVALID, "a target handle does not draft (use dflash_target_forward)");
  dflash_status st = check_slots(h, n_req, slots);
  if (st) return st;
  if (!draft) return fail(DFLASH_E_INVALID, "draft is NULL");
  if (c.conv2 && !last_token) return fail(DFLASH_E_INVALID, "conv2 needs last_token");
  if (c.topk && (!topk_ids || !topk_logits)) return fail(DFLASH_E_INVALID, "topk needs topk_ids and topk_logits");
  for (int i = 0; i < n_req; ++i) {
    const HostSlot& hs = h->slots[slots[i]];
    if (hs.ctx_len + c.block_size + 1 > c.max_position)
      return fail(DFLASH_E_CAPACITY, "slot %d: block positions beyond max_position", slots[i]);
  }
  st = ensure_device(h);
  if (st) return st;
  char* sb = h->ws + h->lay.scratch;
  const Scratch* scp = &h->lay.sc;
  if (from_static) {
    st = static_scratch(h, n_req, &sb, &scp);
    if (st) return st;
  }
  const Scratch& sc = *scp;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t e = elt(c);
  const int d = c.hidden, B = c.block_size, M = n_req * B;
  const int qd = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const Plans pl = make_plans(c, M);
  SlotArgs sl{};
  for (int i = 0; i < n_req; ++i) sl.slots[i] = slots[i];

  // attention plan: KQ key subsets per workgroup (up to 8 waves); splits
  // per request from its own context (the grid covers the longest)
  const int G = c.n_q_heads / c.n_kv_heads;
  const int KQ = std::max(1, 8 / G);
  const int target = split_target(c);
  int splits = 1;
  for (int i = 0; i < n_req; ++i) {
    const HostSlot& hs = h->slots[slots[i]];
    int lo = hs.kv_begin;
    if (c.window) lo = std::max(lo, hs.ctx_len - c.window);
    const int u = (hs.ctx_len > lo ? (hs.ctx_len - 1) / 16 - lo / 16 + 1 : 0) + 1;
    const int pps = split_pages(u, target, kPpsCap);
    splits = std::max(splits, (u + pps - 1) / pps);
  }

  const bool rope = qkv_rope(c, M);
  RopeOut rope_out{};
  if (rope) {
    rope_out.state = at<SlotState>(h, h->lay.state);
    rope_out.cos_t = at<float>(h, h->lay.cos_t);
    rope_out.sin_t = at<float>(h, h->lay.sin_t);
    rope_out.qb = h->ws + h->lay.qb;
    rope_out.blk = h->ws + h->lay.blk;
    rope_out.B = B;
    rope_out.Hq = c.n_q_heads;
    rope_out.Hkv = c.n_kv_heads;
    rope_out.dh = c.head_dim;
    for (int i = 0; i < n_req; ++i) rope_out.slots[i] = slots[i];
  }

  float* hbuf = sat<float>(sb, sc.h);
  float* dpart = sat<float>(sb, sc.dpart);
  float* opart = sat<float>(sb, sc.opart);
  const size_t page_layer = (size_t)c.max_pages * 2 * c.n_kv_heads * 16 * c.head_dim;

  auto gemm_in = [&](const void* a, int K) {
    GemmParams g{};
    g.a[0] = a;
    g.a_parts = 1;
    g.a_part_k = K;
    g.lda = K;
    g.M = M;
    g.K = K;
    return g;
  };

  // DFlash 2 two-tap conv: taps of point k of layer l, [2][d]
  auto conv_taps = [&](int l, int k) { return wptr(h->w.layers[l].conv, (size_t)k * 2 * d, e); };
  auto set_conv = [&](NormParams& np, int l, int k) {
    np.conv = conv_taps(l, k);
    np.embed = h->w.embed;
    np.last_token = last_token;
    np.B = B;
    np.vocab = c.vocab;
    np.err = at<unsigned int>(h, h->lay.err);
  };
  // the output conv of the GEMM whose partials a norm adds (point k of layer l)
  auto set_oconv = [&](NormParams& np, int l, int k, const float* part, int n_part) {
    np.oconv = conv_taps(l, k);
    np.part = part;
    np.n_part = n_part;
    np.embed = h->w.embed;
    np.last_token = last_token;
    np.B = B;
    np.vocab = c.vocab;
    np.err = at<unsigned int>(h, h->lay.err);
  };
  auto norm = [&](const NormParams& np) {
    ProfScope ps(h, np.conv || np.oconv || np.otaps ? DFLASH_KERNEL_CONV : DFLASH_KERNEL_NORM, s);
    launch_rmsnorm(c.dtype, np, s);
  };
  // conv variant: the residual stream alternates between hbuf and halt
  float* halt = c.conv2 ? sat<float>(sb, sc.h2) : hbuf;
  // dynamic conv taps (rank r): the O and down products carry 2r extra output
  // columns, t = (D W) o as hi + lo, from which each output conv's taps are formed; the
  // input convs take the stored normed rows through a D product and apply
  // their taps into the next GEMM's input
  const int r = c.conv2 ? c.conv_rank : 0;
  const int dn = out_width(c);
  float* otaps = r ? sat<float>(sb, sc.otaps) : nullptr;
  if (r && (pl.o.P > 16 || pl.down.P > 16 || pl.dconv.P > 16))  // the taps kernel sums at most 16 splits
    return fail(DFLASH_E_UNSUPPORTED, "dynamic conv taps with more than 16 split-K planes");
  auto dconv_base = [&](DConvParams& dp, int l, int k) {
    dp.U = wptr(h->w.layers[l].dconv_u, (size_t)k * 2 * d * r, e);
    dp.w = conv_taps(l, k);
    dp.d = d;
    dp.r = r;
    dp.M = M;
    dp.B = B;
    dp.vocab = c.vocab;
    dp.embed = h->w.embed;
    dp.last_token = last_token;
    dp.err = at<unsigned int>(h, h->lay.err);
  };
  // output conv k of layer l: taps from the extra columns of the product's partials
  auto dyn_taps = [&](int l, int k, const float* part, int n_part) {
    DConvParams dp{};
    dconv_base(dp, l, k);
    dp.t = part + d;
    dp.lo_off = r;
    dp.ldt = dn;
    dp.plane = (long long)M * dn;
    dp.n_part = n_part;
    dp.taps = otaps;
    ProfScope ps(h, DFLASH_KERNEL_CONV, s);
    launch_dconv(c.dtype, dp, s);
  };
  // input conv k (0 or 2) of layer l: D product of the stored normed rows in xn, then the conv into xa
  auto dyn_in = [&](int l, int k, int out_packed) {
    GemmParams gt = gemm_in(sb + sc.xn, d);
    set_weights(h, gt, 0, h->pk.dconv[l][k / 2], r, d);
    gt.tiles = r / 16;
    gt.N = r;
    gt.P = pl.dconv.P;
    gt.out_f32 = sat<float>(sb, sc.tpart);
    DConvParams dp{};
    dconv_base(dp, l, k);
    dp.x = sb + sc.xn;
    dp.t = gt.out_f32;
    dp.ldt = r;
    dp.plane = (long long)M * r;
    dp.n_part = pl.dconv.P;
    dp.out = sb + sc.xa;
    dp.ldo = d;
    dp.out_packed = out_packed;
    ProfScope ps(h, DFLASH_KERNEL_CONV, s);
    launch_gemm(c.dtype, EPI_PARTIAL, pl.dconv, gt, s);
    launch_dconv(c.dtype, dp, s);
  };
  auto set_otaps = [&](NormParams& np, const float* part, int n_part) {
    np.otaps = otaps;
    np.part = part;
    np.n_part = n_part;
    np.ldp = dn;
    np.embed = h->w.embed;
    np.last_token = last_token;
    np.B = B;
    np.vocab = c.vocab;
    np.err = at<unsigned int>(h, h->lay.err);
  };

  // One-block plans with an unsplit O product (batch 1, no conv): the O
  // epilogue adds into the residual and leaves the gained MLP input with its
  // sums of squares; the gate/up product scales its rows by 1/rms (the
  // RMSNorm's operations, with the scale applied after the product), so no
  // norm launch sits between them.
  const bool resid_o = !c.conv2 && pl.o.mt == 1 && pl.o.P == 1 && pl.gateup.mt == 1 && M <= 16 && d <= 8192;
  float* ssq = sat<float>(sb, sc.ssq);
  // Layer 0 of a block without conv: every row is the mask embedding, so the
  // QKV product reads the row formed once at set-up (row stride 0) and the
  // first residual add starts from the embedding row; no norm launch.
  const bool init0 = !c.conv2 && !hidden_in && !debug_hidden && pl.qkv.mt != 0;
  const void* mask_row = wptr(h->w.embed, (size_t)c.mask_token_id * d, e);

  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& lw = h->w.layers[l];
    // residual: block init (layer 0) or h + previous layer's down-projection
    // partials (with the conv variant folded in by its own launch first)
    NormParams n1{};
    n1.x_out = hbuf;
    if (hidden_in) {
      n1.x_in = hidden_in + (size_t)l * M * d;  // teacher forcing
    } else if (l == 0) {
      n1.init_row = wptr(h->w.embed, (size_t)c.mask_token_id * d, e);
    } else if (c.conv2) {  // previous layer's down output through its conv, into the other buffer
      n1.x_in = hbuf;
      if (r)
        set_otaps(n1, dpart, pl.down.P);
      else
        set_oconv(n1, l - 1, 3, dpart, pl.down.P);
      n1.x_out = halt;
      std::swap(hbuf, halt);
    } else {
      n1.x_in = hbuf;
      n1.part = dpart;
      n1.n_part = pl.down.P;
    }
    if (c.conv2 && !r) set_conv(n1, l, 0);
    n1.ldx = d;
    n1.gamma = lw.attn_norm;
    n1.eps = c.rms_eps;
    n1.out = sb + (r ? sc.xn : sc.xa);
    n1.ldo = d;
    n1.out_packed = !r && pl.qkv.mt == 0;  // the tiled QKV product reads fragment order
    n1.d = d;
    n1.M = M;
    n1.dbg = debug_hidden ? debug_hidden + (size_t)l * M * d : nullptr;
    const bool skip_n1 = init0 && l == 0;
    if (!skip_n1) norm(n1);
    if (r) dyn_in(l, 0, pl.qkv.mt == 0);

    GemmParams g = gemm_in(skip_n1 ? h->ws + h->lay.xa0 : sb + sc.xa, d);
    if (skip_n1) g.lda = 0;
    g.a_packed = pl.qkv.mt == 0;  // written so by the norm, or by the dynamic conv
    set_weights(h, g, 0, h->pk.wqkv[l], qkvw, d);
    g.N = qkvw;
    g.P = pl.qkv.P;
    if (rope) {
      g.tiles = tiles_of(qkvw) / 2;
      g.rope = rope_out;
      ProfScope ps(h, DFLASH_KERNEL_QKV_GEMM, s);
      launch_gemm(c.dtype, EPI_ROPE, pl.qkv, g, s);
    } else {
      g.tiles = tiles_of(qkvw);
      g.out_f32 = sat<float>(sb, sc.qkv);
      ProfScope ps(h, DFLASH_KERNEL_QKV_GEMM, s);
      launch_gemm(c.dtype, EPI_PARTIAL, pl.qkv, g, s);
    }

    QkvPostParams qp{};
    qp.qkv = sat<float>(sb, sc.qkv);
    qp.n_part = pl.qkv.P;
    qp.B = B;
    qp.Hq = c.n_q_heads;
    qp.Hkv = c.n_kv_heads;
    qp.state = at<SlotState>(h, h->lay.state);
    qp.cos_t = at<float>(h, h->lay.cos_t);
    qp.sin_t = at<float>(h, h->lay.sin_t);
    qp.qb = h->ws + h->lay.qb;
    qp.blk = h->ws + h->lay.blk;
    if (!rope) {
      ProfScope ps(h, DFLASH_KERNEL_QKV_POST, s);
      launch_qkv_post(c.dtype, c.head_dim, n_req, qp, sl, s);
    }

    AttnParams ap{};
    ap.qb = h->ws + h->lay.qb;
    ap.blk = h->ws + h->lay.blk;
    ap.pool = h->kv + (size_t)l * page_layer * e;
    ap.page_table = at<int>(h, h->lay.page_table);
    ap.pt_stride = c.max_pages_per_req;
    ap.state = at<SlotState>(h, h->lay.state);
    ap.max_pages = c.max_pages;
    ap.window = c.window;
    ap.Hq = c.n_q_heads;
    ap.Hkv = c.n_kv_heads;
    ap.B = B;
    ap.split_target = target;
    ap.pps_cap = kPpsCap;
    ap.n_split = sat<int>(sb, sc.nsplit);
    ap.n_splits = splits;
    ap.KQ = KQ;
    ap.scale = (float)(1.0 / sqrt((double)c.head_dim));
    ap.part_o = sat<float>(sb, sc.part_o);
    ap.part_ml = sat<float>(sb, sc.part_ml);
    ap.out = sb + sc.xo;
    ap.ldo = qd;
    ap.out_packed = pl.o.mt == 0;
    ap.err = at<unsigned int>(h, h->lay.err);
    { ProfScope ps(h, DFLASH_KERNEL_ATTN, s); launch_attention(c.dtype, c.head_dim, n_req, ap, sl, s); }
    if (splits > 1) {
      CombineParams cp{};
      cp.part_o = ap.part_o;
      cp.part_ml = ap.part_ml;
      cp.n_split = ap.n_split;
      cp.n_splits = splits;
      cp.n_rh = n_req * c.n_q_heads;
      cp.Hq = c.n_q_heads;
      cp.B = B;
      cp.out = ap.out;
      cp.ldo = qd;
      cp.out_packed = ap.out_packed;
      ProfScope ps(h, DFLASH_KERNEL_COMBINE, s);
      launch_combine(c.dtype, c.head_dim, cp, s);
    }

    GemmParams go = gemm_in(sb + sc.xo, qd);
    go.a_packed = ap.out_packed;
    set_weights(h, go, 0, h->pk.wo[l], dn, qd);
    go.tiles = tiles_of(dn);
    go.N = dn;
    go.P = pl.o.P;
    go.out_f32 = opart;
    if (resid_o) {  // residual, gained MLP input and its sums of squares from the O epilogue
      go.resid = hbuf;
      go.ldr = d;
      go.resid_row = skip_n1 ? mask_row : nullptr;
      go.gain = lw.mlp_norm;
      go.out_t = sb + sc.xa;
      go.ldt = d;
      go.ssq = ssq;
      go.ssq_tiles = tiles_of(d);
      { ProfScope ps(h, DFLASH_KERNEL_O_GEMM, s); launch_gemm(c.dtype, EPI_RESID, pl.o, go, s); }
      gateup_swiglu(h, s, sb, sc, pl, M, l, 0, 0, ssq);
    } else {
      ProfScope ps(h, DFLASH_KERNEL_O_GEMM, s);
      launch_gemm(c.dtype, EPI_PARTIAL, pl.o, go, s);
    }
    if (r) dyn_taps(l, 1, opart, pl.o.P);

    NormParams n2{};
    n2.x_in = hbuf;
    if (c.conv2) {  // O output through its conv, into the other buffer
      if (r) {
        set_otaps(n2, opart, pl.o.P);
      } else {
        set_oconv(n2, l, 1, opart, pl.o.P);
        set_conv(n2, l, 2);
      }
      n2.x_out = halt;
      std::swap(hbuf, halt);
    } else {
      n2.part = opart;
      n2.n_part = pl.o.P;
      n2.x_out = hbuf;
      if (skip_n1) {  // the residual so far is the block init
        n2.x_in = nullptr;
        n2.init_row = mask_row;
      }
    }
    n2.ldx = d;
    n2.gamma = lw.mlp_norm;
    n2.eps = c.rms_eps;
    n2.out = sb + (r ? sc.xn : sc.xa);
    n2.ldo = d;
    n2.out_packed = !r && pl.gateup.mt == 0;
    n2.d = d;
    n2.M = M;
    const int z_packed = pl.gateup.mt == 0 && pl.down.mt == 0;  // z for a tiled down product
    if (!resid_o) {
      norm(n2);
      if (r) dyn_in(l, 2, pl.gateup.mt == 0);
      gateup_swiglu(h, s, sb, sc, pl, M, l, pl.gateup.mt == 0, z_packed);
    }

    GemmParams gd = gemm_in(sb + sc.z, c.ffn);
    gd.a_packed = z_packed;
    set_weights(h, gd, 0, h->pk.wdown[l], dn, c.ffn);
    gd.tiles = tiles_of(dn);
    gd.N = dn;
    gd.P = pl.down.P;
    gd.out_f32 = dpart;
    { ProfScope ps(h, DFLASH_KERNEL_DOWN_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.down, gd, s); }
    if (r && !hidden_in) dyn_taps(l, 3, dpart, pl.down.P);  // taken by the next norm (forced rows skip it)
    st = launched("draft layer");
    if (st) return st;
  }

  NormParams nf{};
  nf.x_in = hbuf;
  if (hidden_in) {
    nf.x_in = hidden_in + (size_t)c.n_layers * M * d;  // teacher forcing
  } else if (c.conv2) {
    if (r)
      set_otaps(nf, dpart, pl.down.P);
    else
      set_oconv(nf, c.n_layers - 1, 3, dpart, pl.down.P);
  } else {
    nf.part = dpart;
    nf.n_part = pl.down.P;
    nf.x_out = hbuf;
  }
  nf.ldx = d;
  nf.gamma = h->w.final_norm;
  nf.eps = c.rms_eps;
  nf.out = sb + sc.xa;
  nf.ldo = d;
  nf.out_packed = pl.lm.mt == 0;
  nf.d = d;
  nf.M = M;
  nf.dbg = debug_hidden ? debug_hidden + (size_t)c.n_layers * M * d : nullptr;
  nf.zero_keys = sat<unsigned long long>(sb, sc.keys);
  norm(nf);

  return lm_head(h, s, sb, sc, pl, M, nf.out_packed, draft, topk_ids, topk_logits, debug_logits);
}

dflash_status dflash_draft_block(dflash_handle* h, void* stream, int32_t n_req,
                                 const int32_t* slots, const int32_t* last_token, int32_t* draft,
                                 int32_t* topk_ids, float* topk_logits,
                                 const dflash_draft_debug* debug) {
  return draft_impl(h, stream, n_req, slots, last_token, draft, topk_ids, topk_logits, debug, false);
}

dflash_status dflash_draft_block_static(dflash_handle* h, void* stream, int32_t n_req,
                                        const int32_t* slots, const int32_t* last_token, int32_t* draft,
                                        int32_t* topk_ids, float* topk_logits,
                                        const dflash_draft_debug* debug) {
  return draft_impl(h, stream, n_req, slots, last_token, draft, topk_ids, topk_logits, debug, true);
}

size_t dflash_draft_static_bytes(const dflash_config* cfg, int32_t n_req) {
  if (validate(cfg) != DFLASH_OK || n_req < 1 || n_req > cfg->max_batch) return 0;
  return make_scratch(*cfg, n_req, false).total;
}

dflash_status dflash_set_context_length(dflash_handle* h, void* stream, int32_t slot, int32_t ctx_len) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  if (slot < 0 || slot >= h->cfg.max_batch || !h->slots[slot].bound)
    return fail(DFLASH_E_INVALID, "slot %d is not bound", slot);
  HostSlot& hs = h->slots[slot];
  // without a window, any length the bound pages hold; with one, only a rollback
  const int top = h->cfg.window ? hs.ctx_len : std::min(hs.n_pages * 16, h->cfg.max_position - 1);
  if (ctx_len < hs.kv_begin || ctx_len > top)
    return fail(DFLASH_E_INVALID, "ctx_len %d out of [%d, %d]", ctx_len, hs.kv_begin, top);
  dflash_status st = ensure_device(h);
  if (st) return st;
  launch_set_ctx(at<SlotState>(h, h->lay.state), slot, ctx_len, reinterpret_cast<hipStream_t>(stream));
  st = launched("set context length");
  if (st) return st;
  hs.ctx_len = ctx_len;
  return DFLASH_OK;
}

dflash_status dflash_target_forward(dflash_handle* h, void* stream, int32_t n_req, const int32_t* slots,
                                    int32_t n_rows, const int32_t* tokens, int32_t* greedy, float* logits,
                                    int32_t n_feat_out, const int32_t* feat_layers, void* const* feat_out) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  const dflash_config& c = h->cfg;
  if (!c.target) return fail(DFLASH_E_INVALID, "dflash_target_forward needs a target handle (target 1)");
  dflash_status st = check_slots(h, n_req, slots);
  if (st) return st;
  if (n_rows < 1 || n_rows > c.block_size)
    return fail(DFLASH_E_INVALID, "n_rows %d out of [1, %d]", n_rows, c.block_size);
  if (!tokens || !greedy) return fail(DFLASH_E_INVALID, "tokens and greedy must be set");
  if (n_feat_out < 0 || n_feat_out > DFLASH_MAX_FEAT) return fail(DFLASH_E_INVALID, "n_feat_out out of range");
  if (n_feat_out && (!feat_layers || !feat_out)) return fail(DFLASH_E_INVALID, "feature outputs are NULL");
  for (int k = 0; k < n_feat_out; ++k) {
    if (feat_layers[k] < 0 || feat_layers[k] >= c.n_layers || (k && feat_layers[k] <= feat_layers[k - 1]))
      return fail(DFLASH_E_INVALID, "feature layers must be ascending ids below %d", c.n_layers);
    if (!feat_out[k]) return fail(DFLASH_E_INVALID, "feat_out[%d] is NULL", k);
  }
  for (int i = 0; i < n_req; ++i) {
    const HostSlot& hs = h->slots[slots[i]];
    if ((long long)hs.ctx_len + n_rows > (long long)hs.n_pages * 16)
      return fail(DFLASH_E_CAPACITY, "slot %d: %d + %d positions exceed %d bound pages", slots[i], hs.ctx_len,
                  n_rows, hs.n_pages);
    if (hs.ctx_len + n_rows >= c.max_position)
      return fail(DFLASH_E_CAPACITY, "slot %d: positions beyond max_position", slots[i]);
  }
  st = ensure_device(h);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const size_t e = elt(c);
  const int d = c.hidden, M = n_req * n_rows;
  const int qd = c.n_q_heads * c.head_dim;
  const int qkvw = (c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim;
  const Plans pl = make_plans(c, M);
  char* sb = h->ws + h->lay.scratch;
  const Scratch& sc = h->lay.sc;
  float* hbuf = sat<float>(sb, sc.h);
  float* dpart = sat<float>(sb, sc.dpart);
  float* opart = sat<float>(sb, sc.opart);
  const size_t page_layer = (size_t)c.max_pages * 2 * c.n_kv_heads * 16 * c.head_dim;
  auto feat_of = [&](int layer) -> void* {  // output of feature layer `layer`, or NULL
    for (int k = 0; k < n_feat_out; ++k)
      if (feat_layers[k] == layer) return feat_out[k];
    return nullptr;
  };
  auto gemm_in = [&](const void* a, int K) {
    GemmParams g{};
    g.a[0] = a;
    g.a_parts = 1;
    g.a_part_k = K;
    g.lda = K;
    g.M = M;
    g.K = K;
    return g;
  };
  auto norm = [&](const NormParams& np) {
    ProfScope ps(h, DFLASH_KERNEL_NORM, s);
    launch_rmsnorm(c.dtype, np, s);
  };
  TargetQParams tq{};
  CausalAttnParams ca{};
  SlotArgs sl{};
  for (int i = 0; i < n_req; ++i) {
    tq.pos0[i] = ca.pos0[i] = h->slots[slots[i]].ctx_len;
    ca.slots[i] = sl.slots[i] = slots[i];
  }
  // bf16: split-K attention over (request, 16-row tile) pairs; the grid
  // covers the splits of the longest request's last tile
  const bool split_attn = c.dtype == DFLASH_BF16;
  const int n_tiles = (n_rows + 15) / 16;
  int splits = 1;
  for (int i = 0; i < n_req; ++i) {
    const HostSlot& hs = h->slots[slots[i]];
    const int hi = hs.ctx_len + n_rows;
    const int u = hi > hs.kv_begin ? (hi - 1) / 16 - hs.kv_begin / 16 + 1 : 0;
    const int pps = split_pages(u, split_target(c), kPpsCap);
    splits = std::max(splits, (u + pps - 1) / pps);
  }
  tq.n_tiles = split_attn ? n_tiles : 0;
  for (int l = 0; l < c.n_layers; ++l) {
    const dflash_layer_weights& lw = h->w.layers[l];
    NormParams n1{};
    if (l == 0) {  // token embeddings
      n1.init_row = h->w.embed;
      n1.init_tokens = tokens;
      n1.vocab = c.vocab;
      n1.err = at<unsigned int>(h, h->lay.err);
    } else {  // residual + previous layer's down partials; the feature after layer l-1
      n1.x_in = hbuf;
      n1.part = dpart;
      n1.n_part = pl.down.P;
      n1.feat = feat_of(l - 1);
    }
    n1.x_out = hbuf;
    n1.ldx = d;
    n1.gamma = lw.attn_norm;
    n1.eps = c.rms_eps;
    n1.out = sb + sc.xa;
    n1.ldo = d;
    n1.out_packed = pl.qkv.mt == 0;
    n1.d = d;
    n1.M = M;
    norm(n1);

    GemmParams g = gemm_in(sb + sc.xa, d);
    g.a_packed = n1.out_packed;
    set_weights(h, g, 0, h->pk.wqkv[l], qkvw, d);
    g.N = qkvw;
    g.P = pl.qkv.P;
    g.tiles = tiles_of(qkvw);
    g.out_f32 = sat<float>(sb, sc.qkv);
    { ProfScope ps(h, DFLASH_KERNEL_QKV_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.qkv, g, s); }
    {
      ProfScope ps(h, DFLASH_KERNEL_TARGET_ATTN, s);
      // q of the new rows with RoPE at their positions
      tq.qkv = g.out_f32;
      tq.n_part = pl.qkv.P;
      tq.M = M;
      tq.ld = qkvw;
      tq.R = n_rows;
      tq.Hq = c.n_q_heads;
      tq.dh = c.head_dim;
      tq.cos_t = at<float>(h, h->lay.cos_t);
      tq.sin_t = at<float>(h, h->lay.sin_t);
      tq.q = sb + sc.tq;
      launch_target_q(c.dtype, tq, s);
      // K (RoPE) and V of the new rows appended to the slots' pages, in chunks of requests
      for (int r0 = 0; r0 < n_req; r0 += kMaxChunkReq) {
        const int nr = std::min(kMaxChunkReq, n_req - r0);
        ScatterParams sp{};
        sp.kv = g.out_f32 + (size_t)r0 * n_rows * qkvw;
        sp.ld = qkvw;
        sp.col0 = qd;
        sp.n_part = pl.qkv.P;
        sp.rows = nr * n_rows;
        sp.L = 1;
        sp.Hkv = c.n_kv_heads;
        sp.n_req = nr;
        for (int i = 0; i < nr; ++i) {
          InjectReq& q = sp.req[i];
          q.row_start = i * n_rows;
          q.count = n_rows;
          q.slot = slots[r0 + i];
          q.pos0 = tq.pos0[r0 + i];
          q.final_ctx = q.pos0 + n_rows;
        }
        sp.cos_t = tq.cos_t;
        sp.sin_t = tq.sin_t;
        sp.pool = h->kv + (size_t)l * page_layer * e;
        sp.layer_stride = 0;
        sp.page_table = at<int>(h, h->lay.page_table);
        sp.pt_stride = c.max_pages_per_req;
        sp.state = at<SlotState>(h, h->lay.state);
        sp.window = 0;
        sp.max_pages = c.max_pages;
        sp.err = at<unsigned int>(h, h->lay.err);
        launch_scatter(c.dtype, c.head_dim, sp, s);
      }
      if (split_attn) {  // the split ring kernel in causal mode, then the merge
        AttnParams ap{};
        ap.qb = sb + sc.tq;
        ap.blk = h->ws + h->lay.blk;
        ap.pool = h->kv + (size_t)l * page_layer * e;
        ap.page_table = at<int>(h, h->lay.page_table);
        ap.pt_stride = c.max_pages_per_req;
        ap.state = at<SlotState>(h, h->lay.state);
        ap.max_pages = c.max_pages;
        ap.Hq = c.n_q_heads;
        ap.Hkv = c.n_kv_heads;
        ap.B = 16;
        ap.split_target = split_target(c);
        ap.pps_cap = kPpsCap;
        ap.n_split = sat<int>(sb, sc.nsplit);
        ap.n_splits = splits;
        ap.KQ = 1;
        ap.scale = (float)(1.0 / sqrt((double)c.head_dim));
        ap.part_o = sat<float>(sb, sc.part_o);
        ap.part_ml = sat<float>(sb, sc.part_ml);
        ap.out = sb + sc.xo;
        ap.ldo = qd;
        ap.out_packed = pl.o.mt == 0;
        ap.err = at<unsigned int>(h, h->lay.err);
        ap.causal_R = n_rows;
        ap.n_tiles = n_tiles;
        launch_attention(c.dtype, c.head_dim, n_req * n_tiles, ap, sl, s);
        if (splits > 1) {
          CombineParams cp{};
          cp.part_o = ap.part_o;
          cp.part_ml = ap.part_ml;
          cp.n_split = ap.n_split;
          cp.n_splits = splits;
          cp.n_rh = n_req * n_tiles * c.n_q_heads;
          cp.Hq = c.n_q_heads;
          cp.B = 16;
          cp.out = ap.out;
          cp.ldo = qd;
          cp.out_packed = ap.out_packed;
          cp.causal_R = n_rows;
          cp.n_tiles = n_tiles;
          launch_combine(c.dtype, c.head_dim, cp, s);
        }
      } else {  // fp32: one workgroup per (head, request, tile) over all pages
        ca.q = sb + sc.tq;
        ca.pool = h->kv + (size_t)l * page_layer * e;
        ca.page_table = at<int>(h, h->lay.page_table);
        ca.pt_stride = c.max_pages_per_req;
        ca.state = at<SlotState>(h, h->lay.state);
        ca.max_pages = c.max_pages;
        ca.Hq = c.n_q_heads;
        ca.Hkv = c.n_kv_heads;
        ca.R = n_rows;
        ca.scale = (float)(1.0 / sqrt((double)c.head_dim));
        ca.out = sb + sc.xo;
        ca.ldo = qd;
        ca.out_packed = pl.o.mt == 0;
        ca.err = at<unsigned int>(h, h->lay.err);
        launch_causal_attn(c.dtype, c.head_dim, n_req, ca, s);
      }
    }

    GemmParams go = gemm_in(sb + sc.xo, qd);
    go.a_packed = pl.o.mt == 0;
    set_weights(h, go, 0, h->pk.wo[l], d, qd);
    go.tiles = tiles_of(d);
    go.N = d;
    go.P = pl.o.P;
    go.out_f32 = opart;
    { ProfScope ps(h, DFLASH_KERNEL_O_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.o, go, s); }

    NormParams n2{};
    n2.x_in = hbuf;
    n2.part = opart;
    n2.n_part = pl.o.P;
    n2.x_out = hbuf;
    n2.ldx = d;
    n2.gamma = lw.mlp_norm;
    n2.eps = c.rms_eps;
    n2.out = sb + sc.xa;
    n2.ldo = d;
    n2.out_packed = pl.gateup.mt == 0;
    n2.d = d;
    n2.M = M;
    norm(n2);

    const int z_packed = pl.gateup.mt == 0 && pl.down.mt == 0;  // z for a tiled down product
    gateup_swiglu(h, s, sb, sc, pl, M, l, n2.out_packed, z_packed);

    GemmParams gd = gemm_in(sb + sc.z, c.ffn);
    gd.a_packed = z_packed;
    set_weights(h, gd, 0, h->pk.wdown[l], d, c.ffn);
    gd.tiles = tiles_of(d);
    gd.N = d;
    gd.P = pl.down.P;
    gd.out_f32 = dpart;
    { ProfScope ps(h, DFLASH_KERNEL_DOWN_GEMM, s); launch_gemm(c.dtype, EPI_PARTIAL, pl.down, gd, s); }
    st = launched("target layer");
    if (st) return st;
  }
  NormParams nf{};
  nf.x_in = hbuf;
  nf.part = dpart;
  nf.n_part = pl.down.P;
  nf.feat = feat_of(c.n_layers - 1);
  nf.ldx = d;
  nf.gamma = h->w.final_norm;
  nf.eps = c.rms_eps;
  nf.out = sb + sc.xa;
  nf.ldo = d;
  nf.out_packed = pl.lm.mt == 0;
  nf.d = d;
  nf.M = M;
  nf.zero_keys = sat<unsigned long long>(sb, sc.keys);
  norm(nf);
  st = lm_head(h, s, sb, sc, pl, M, nf.out_packed, greedy, nullptr, nullptr, logits);
  if (st) return st;
  for (int i = 0; i < n_req; ++i) h->slots[slots[i]].ctx_len += n_rows;
  return DFLASH_OK;
}

dflash_status dflash_select_path(dflash_handle* h, void* stream, int32_t n_req, const int32_t* topk_ids,
                                 const float* topk_logits, int32_t* path, float* step_scores) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  const dflash_config& c = h->cfg;
  if (!c.selector_rank) return fail(DFLASH_E_UNSUPPORTED, "the handle has no path selector (selector_rank 0)");
  if (n_req < 1 || n_req > c.max_batch) return fail(DFLASH_E_INVALID, "n_req %d out of [1, %d]", n_req, c.max_batch);
  if (!topk_ids || !topk_logits || !path) return fail(DFLASH_E_INVALID, "a path selector pointer is NULL");
  dflash_status st = ensure_device(h);
  if (st) return st;
  PathParams pp{};
  pp.topk_ids = topk_ids;
  pp.topk_logits = topk_logits;
  pp.tu = reinterpret_cast<const float*>(h->packed + h->pk.sel_u);
  pp.tv = reinterpret_cast<const float*>(h->packed + h->pk.sel_v);
  pp.B = c.block_size;
  pp.r = c.selector_rank;
  pp.vocab = c.vocab;
  pp.path = path;
  pp.step_scores = step_scores;
  pp.err = at<unsigned int>(h, h->lay.err);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    ProfScope ps(h, DFLASH_KERNEL_PATH, s);
    launch_select_path(pp, n_req, s);
  }
  return launched("path selector");
}

static dflash_status check_sampling(const dflash_handle* h, const dflash_sampling* sp) {
  if (!sp) return fail(DFLASH_E_INVALID, "sampling settings are NULL");
  if (!(sp->temperature >= 1e-2f && sp->temperature <= 1e3f))
    return fail(DFLASH_E_INVALID, "temperature %g out of [0.01, 1000]", (double)sp->temperature);
  if (sp->top_k < 0 || sp->top_k > 64) return fail(DFLASH_E_INVALID, "top_k %d out of [0, 64]", sp->top_k);
  if (!(sp->top_p > 0.f && sp->top_p <= 1.f)) return fail(DFLASH_E_INVALID, "top_p %g out of (0, 1]", (double)sp->top_p);
  if (sp->top_p < 1.f && sp->top_k == 0)
    return fail(DFLASH_E_UNSUPPORTED, "top_p below 1 needs top_k >= 1 (no nucleus over the whole vocabulary)");
  if (!h->cfg.topk) return fail(DFLASH_E_UNSUPPORTED, "sampled drafting needs the top-16 lists (topk 16)");
  return DFLASH_OK;
}

static SampleParams sample_params(dflash_handle* h, const dflash_sampling* sp) {
  SampleParams p{};
  p.temperature = sp->temperature;
  p.top_k = sp->top_k;
  p.top_p = sp->top_p;
  p.B = h->cfg.block_size;
  p.vocab = h->cfg.vocab;
  p.err = at<unsigned int>(h, h->lay.err);
  return p;
}

dflash_status dflash_draft_sample(dflash_handle* h, void* stream, int32_t n_req, const dflash_sampling* sampling,
                                  const int32_t* topk_ids, const float* topk_logits, const float* uniforms,
                                  int32_t* draft) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  dflash_status st = check_sampling(h, sampling);
  if (st) return st;
  if (n_req < 1 || n_req > h->cfg.max_batch) return fail(DFLASH_E_INVALID, "n_req %d out of [1, %d]", n_req, h->cfg.max_batch);
  if (!topk_ids || !topk_logits || !uniforms || !draft) return fail(DFLASH_E_INVALID, "a draft-sample pointer is NULL");
  st = ensure_device(h);
  if (st) return st;
  SampleParams p = sample_params(h, sampling);
  p.dids = topk_ids;
  p.dlog = topk_logits;
  p.v = uniforms;
  p.draft = draft;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    ProfScope ps(h, DFLASH_KERNEL_SAMPLE, s);
    launch_draft_sample(p, n_req, s);
  }
  return launched("draft sample");
}

dflash_status dflash_verify_sample(dflash_handle* h, void* stream, int32_t n_req, const dflash_sampling* sampling,
                                   const int32_t* draft, const int32_t* topk_ids, const float* topk_logits,
                                   const float* target_logits, const float* uniforms, int32_t* accept_len,
                                   int32_t* committed, int32_t* last_token) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  dflash_status st = check_sampling(h, sampling);
  if (st) return st;
  if (n_req < 1 || n_req > h->cfg.max_batch) return fail(DFLASH_E_INVALID, "n_req %d out of [1, %d]", n_req, h->cfg.max_batch);
  if (!draft || !topk_ids || !topk_logits || !target_logits || !uniforms || !accept_len || !committed || !last_token)
    return fail(DFLASH_E_INVALID, "a verify-sample pointer is NULL");
  st = ensure_device(h);
  if (st) return st;
  SampleParams p = sample_params(h, sampling);
  p.dids = topk_ids;
  p.dlog = topk_logits;
  p.draft = const_cast<int32_t*>(draft);
  p.tlog = target_logits;
  p.u = uniforms;
  const size_t rows = (size_t)n_req * (h->cfg.block_size + 1);
  float* sr = reinterpret_cast<float*>(h->ws + h->lay.scratch + h->lay.sc.srow);
  p.row_stat = sr;
  p.row_ids = reinterpret_cast<int*>(sr + 2 * rows);
  p.row_p = sr + (2 + 64) * rows;
  p.row_n = reinterpret_cast<int*>(sr + (2 + 128) * rows);
  char* sc = h->ws + h->lay.scratch + h->lay.sc.schunk;
  p.chunk_list = reinterpret_cast<unsigned long long*>(sc);
  p.chunk_stat = reinterpret_cast<float*>(sc + sizeof(unsigned long long) * 64 * kRowChunks * rows);
  p.accept = accept_len;
  p.committed = committed;
  p.last = last_token;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    ProfScope ps(h, DFLASH_KERNEL_VERIFY, s);
    launch_verify_sample(p, n_req, s);
  }
  return launched("verify sample");
}

dflash_status dflash_verify_accept(dflash_handle* h, void* stream, int32_t n_req,
                                   const int32_t* draft, const int32_t* target_greedy,
                                   int32_t* accept_len, int32_t* committed, int32_t* last_token) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  if (n_req < 1 || n_req > h->cfg.max_batch) return fail(DFLASH_E_INVALID, "n_req %d out of [1, %d]", n_req, h->cfg.max_batch);
  if (!draft || !target_greedy || !accept_len || !committed || !last_token)
    return fail(DFLASH_E_INVALID, "a verify pointer is NULL");
  dflash_status st = ensure_device(h);
  if (st) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  {
    ProfScope ps(h, DFLASH_KERNEL_VERIFY, s);
    launch_verify(n_req, h->cfg.block_size, h->cfg.vocab, draft, target_greedy, accept_len,
                  committed, last_token, at<unsigned int>(h, h->lay.err), s);
  }
  return launched("verify");
}

dflash_status dflash_profile_begin(dflash_handle* h, uint32_t mask) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  h->prof.mask = mask & ((1u << DFLASH_KERNEL_COUNT) - 1);
  h->prof.used = 0;
  h->prof.marks.clear();
  return DFLASH_OK;
}

dflash_status dflash_profile_mask(dflash_handle* h, uint32_t mask) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  h->prof.mask = mask & ((1u << DFLASH_KERNEL_COUNT) - 1);
  return DFLASH_OK;
}

dflash_status dflash_profile_end(dflash_handle* h, float* total_ms, int32_t* launches) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  if (!total_ms || !launches) return fail(DFLASH_E_INVALID, "output arrays are NULL");
  Profiler& p = h->prof;
  for (int k = 0; k < DFLASH_KERNEL_COUNT; ++k) {
    total_ms[k] = 0.f;
    launches[k] = 0;
  }
  dflash_status st = DFLASH_OK;
  if (!p.marks.empty()) {
    hipError_t e = hipEventSynchronize(p.pool[p.marks.back().second + 1]);
    if (e) st = hip_fail(e, "profile sync");
    for (const auto& m : p.marks) {
      float ms = 0.f;
      if (!st && (e = hipEventElapsedTime(&ms, p.pool[m.second], p.pool[m.second + 1]))) {
        st = hip_fail(e, "profile elapsed");
        break;
      }
      total_ms[m.first] += ms;
      launches[m.first] += 1;
    }
  }
  p.mask = 0;
  p.used = 0;
  p.marks.clear();
  return st;
}

dflash_status dflash_check(dflash_handle* h, void* stream) {
  if (!h) return fail(DFLASH_E_INVALID, "handle is NULL");
  if (!h->dev_init) return DFLASH_OK;
  hipError_t e;
  if ((e = hipStreamSynchronize(reinterpret_cast<hipStream_t>(stream)))) return hip_fail(e, "sync");
  unsigned int word = 0;
  if ((e = hipMemcpy(&word, h->ws + h->lay.err, sizeof(word), hipMemcpyDeviceToHost)))
    return hip_fail(e, "error word read");
  if (word) {
    if ((e = hipMemset(h->ws + h->lay.err, 0, sizeof(word)))) return hip_fail(e, "error word clear");
    return fail(DFLASH_E_DEVICE, "device error word 0x%x (1: token id out of range, 2/4: page id out of range)", word);
  }
  return DFLASH_OK;
}

}  // extern "C"
