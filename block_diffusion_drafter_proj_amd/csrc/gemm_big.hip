// Tiled MFMA GEMM for many activation rows (M >= 64: batched drafts, long
// injections), where the products are bound by the matrix cores rather than
// by the weight stream.
//
// Y[M, N] = X[M, K] * W[N, K]^T, X row-major bf16 (virtual concatenation of
// a_parts arrays as in the skinny kernel), W packed in MFMA fragment order
// (16 output rows x 32 k per 1 KB fragment, lane-major).
//  * A workgroup of 4 waves (2 x 2) computes a BM x BN output tile; each wave
//    holds a BM/2 x BN/2 tile in 16x16x32 bf16 MFMA accumulators (fp32).
//  * K advances 64 per pipeline stage.  A stage holds both operands in
//    fragment order, written by direct global->LDS 16-byte loads (one 1 KB
//    fragment per wave instruction, no register staging).  ST stages form a
//    ring, so ST-1 stages are in flight while one is multiplied.
//  * Waits are explicit: a wave waits until only the loads of later stages
//    are outstanding, then meets the other waves; its LDS reads of the
//    previous stage are complete at that point, so that buffer is refilled.
//  * Split-K (P > 1) for the partial-output products whose tile grid alone
//    would not fill the chip; each split writes its own fp32 plane and the
//    consumer sums the planes in a fixed order.
//  * Tile order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin;
//    the M-tiles sharing a weight tile go to the same XCD at the same time,
//    so the 32 tiles resident on an XCD form a compact 2-D block whose A and
//    W k-slabs are fetched once into that XCD's L2.
// Epilogues: fp32 partial plane, SwiGLU (a wave's columns are gate columns
// and the matching up columns, so silu(g) * u is formed in registers),
// greedy argmax (row maxima of the two column waves combined in LDS, one
// 64-bit atomic max per row and workgroup) and top-16 (one sorted list of 16
// per row and column wave, merged later).
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kFrag = 64 * 8;  // bf16 elements of one fragment

// A tile configuration: BM x BN output tile, WM x WN waves (each holding a
// BM/WM x BN/WN tile), KF 32-wide k steps per pipeline stage, ST stages.
template <int BM_, int BN_, int WM_, int WN_, int KF_, int ST_>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, KF = KF_, ST = ST_;
  static constexpr int NW = WM * WN;
  static constexpr int TM = BM / WM / 16, TN = BN / WN / 16;  // 16x16 tiles per wave
  static constexpr int FA = BM / 16 * KF, FB = BN / 16 * KF, FS = FA + FB;  // fragments per stage
  static constexpr int LA = FA / NW, LB = FB / NW, LPW = LA + LB;          // loads per wave and stage
  static constexpr int BKS = 32 * KF;                                       // k per stage
  static_assert(FA % NW == 0 && FB % NW == 0 && (ST - 2) * LPW < 64 && TN % 2 == 0, "tile shape");
};

// Column tiles of the output grid: SwiGLU tiles cover BN/2 gate columns.
template <int BN, int EPI>
__host__ __device__ inline int col_tiles(int tiles) {
  constexpr int per = (EPI == EPI_SWIGLU) ? BN / 32 : BN / 16;
  return (tiles + per - 1) / per;
}

template <typename C, int EPI>
__global__ __launch_bounds__(C::NW * 64) __attribute__((amdgpu_waves_per_eu(C::NW / 4, C::NW / 4)))
void k_gemm_tile(GemmParams p) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, KF = C::KF, ST = C::ST;
  constexpr int TM = C::TM, TN = C::TN, FA = C::FA, FS = C::FS, LA = C::LA, LB = C::LB, LPW = C::LPW;
  constexpr int NT = C::NW * 64;
  __shared__ __attribute__((aligned(1024))) bf16 lds[ST * FS * kFrag];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);  // wave index, scalar
  const int wm = wv % WM, wn = wv / WM;
  const int r16 = lane & 15, g = lane >> 4;

  const int n_mt = (p.M + BM - 1) / BM;
  const int n_nt = col_tiles<BN, EPI>(p.tiles);
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int m_tile = slot % n_mt;
  const int col = (slot / n_mt) * 8 + xcd;  // (split, column tile)
  if (col >= n_nt * p.P) return;
  const int n_tile = col % n_nt, split = col / n_nt;
  const int m0 = m_tile * BM;
  const int S32 = p.K / 32;
  const int nk_all = p.K / C::BKS;
  const int ks0 = (int)((long long)split * nk_all / p.P);
  const int nk = (int)((long long)(split + 1) * nk_all / p.P) - ks0;

  // weight tile of stage column jb (0 .. BN/16-1), clamped into the matrix;
  // with SwiGLU each wave's TN columns are TN/2 gate tiles and the matching up tiles
  auto wtile = [&](int jb) -> int {
    if (EPI == EPI_SWIGLU) {
      const int w_ = jb / TN, jj = jb % TN;
      int gt = n_tile * (BN / 32) + w_ * (TN / 2) + (jj % (TN / 2));
      gt = min(gt, p.tiles - 1);
      return jj < TN / 2 ? gt : p.up_tile_off + gt;
    }
    return min(n_tile * (BN / 16) + jb, p.tiles - 1);
  };

  // This wave's share of a stage: LA activation and LB weight fragments
  // (fragment (row or column block r, k step s) sits at r * KF + s).  Their
  // addresses are fixed per workgroup except for the k offset, so they are
  // formed once; the wave index is scalar, so the weight pointers stay in
  // scalar registers and no branch below diverges.
  int a_off[LA];  // element offset inside a part, without the stage's k
#pragma unroll
  for (int i = 0; i < LA; ++i) {
    const int fa = wv * LA + i;
    if (p.a_packed) {  // fragment order: the fragment is 1 KB at (row block, k step)
      const int rb = min(m0 / 16 + fa / KF, (p.M - 1) / 16);
      a_off[i] = (rb * S32 + fa % KF) * kFrag + lane * 8;
    } else {
      const int row = min(m0 + (fa / KF) * 16 + r16, p.M - 1);
      a_off[i] = row * p.lda + (fa % KF) * 32 + 8 * g;
    }
  }
  auto wsrc = [&](int jb) -> const bf16* {  // weight column block jb at k-stage 0
    int tt = wtile(jb);
    int seg = 0;
    if (p.seg_tiles) {
      seg = tt / p.seg_tiles;
      tt -= seg * p.seg_tiles;
    }
    return reinterpret_cast<const bf16*>(p.w[seg]) + (long long)tt * S32 * kFrag;
  };
  const bf16* b_src[LB];  // fragment of k-stage 0
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int fb = wv * LB + i;
    b_src[i] = wsrc(fb / KF) + (fb % KF) * kFrag;
  }

  // activation part of the next stage to load (stages are loaded in k order;
  // a_part_k is a multiple of the stage's k, so a stage never straddles parts)
  int part = ks0 * C::BKS / p.a_part_k;
  int part_k0 = part * p.a_part_k;
  const bf16* apart = reinterpret_cast<const bf16*>(p.a[part]);
  auto load_stage = [&](int kt, int buf) {
    bf16* dst = lds + buf * FS * kFrag;
    const int k0 = kt * C::BKS;
    if (k0 >= part_k0 + p.a_part_k) {
      ++part;
      part_k0 += p.a_part_k;
      apart = reinterpret_cast<const bf16*>(p.a[part]);
    }
    // row-major: k advances along the row; fragment order: 32 k per fragment
    const bf16* abase = apart + (long long)(k0 - part_k0) * (p.a_packed ? 16 : 1);
#pragma unroll
    for (int i = 0; i < LA; ++i) dma16(abase + a_off[i], dst + (wv * LA + i) * kFrag);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      dma16_nt(b_src[i] + (long long)kt * KF * kFrag + lane * 8, dst + (FA + wv * LB + i) * kFrag);
  };


  f32x4 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) load_stage(ks0 + s, s);

  // Stage it sits in LDS buffer it % ST; the loops are unrolled by ST, so the
  // buffer of each pass is a constant.
  auto compute = [&](int u) {
    const bf16* sb = lds + u * FS * kFrag;
    // All of the stage's fragments are read before any product, in a fixed
    // order (the scheduling barriers keep the compiler from sinking each read
    // next to its first use), so later reads complete under earlier MFMAs.
    bf16x8 af[KF][TM], bfr[KF][TN];
#pragma unroll
    for (int k32 = 0; k32 < KF; ++k32) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[k32][i] = *reinterpret_cast<const bf16x8*>(sb + ((wm * TM + i) * KF + k32) * kFrag + lane * 8);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[k32][j] = *reinterpret_cast<const bf16x8*>(sb + (FA + (wn * TN + j) * KF + k32) * kFrag + lane * 8);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int k32 = 0; k32 < KF; ++k32) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step(af[k32][i], bfr[k32][j], acc[i][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto issue = [&](int it, int u) { load_stage(ks0 + it + ST - 1, (u + ST - 1) % ST); };
  int it0 = 0;
  // steady state: every pass waits for the full ring depth and starts a stage
  for (; it0 + 2 * ST - 2 < nk; it0 += ST) {
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      wait_ring<LPW, ST - 2>(ST - 2);
      issue(it0 + u, u);
      compute(u);
    }
  }
  // the last stages: fewer ahead
  for (; it0 < nk; it0 += ST) {
#pragma unroll
    for (int u = 0; u < ST; ++u) {
      const int it = it0 + u;
      if (it < nk) {
        wait_ring<LPW, ST - 2>(nk - 1 - it);
        if (it + ST - 1 < nk) issue(it, u);
        compute(u);
      }
    }
  }

  // ---- epilogues: lane holds rows 4g+q, column r16 of each 16x16 tile ----
  if (EPI == EPI_PARTIAL) {
    float* out = p.out_f32 + (long long)split * p.M * p.N;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + (wm * TM + i) * 16 + 4 * g + q;
          const int n = n_tile * BN + (wn * TN + j) * 16 + r16;
          if (m < p.M && n < p.N) out[(long long)m * p.N + n] = acc[i][j][q];
        }
  } else if (EPI == EPI_SWIGLU) {
    // silu(gate) * up per element into the wave's slice of the (now free)
    // stage ring, then 8 consecutive columns of one row per lane and store:
    // 16-byte writes instead of one element per lane
    constexpr int WR = TM * 16, WC = TN / 2 * 16;  // the wave's output rows and columns
    static_assert(C::NW * WR * WC <= ST * FS * kFrag, "SwiGLU staging fits the ring");
    bf16* stage = lds + wv * WR * WC;
    wait_barrier<0>();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int jj = 0; jj < TN / 2; ++jj)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float gt = acc[i][jj][q], u = acc[i][jj + TN / 2][q];
          stage[(i * 16 + 4 * g + q) * WC + jj * 16 + r16] = (bf16)(gt / (1.0f + expf(-gt)) * u);
        }
    __syncthreads();
    for (int c = lane; c < WR * WC / 8; c += 64) {
      const int rl = c / (WC / 8), cl = (c % (WC / 8)) * 8;
      const int m = m0 + wm * WR + rl;
      const int n = n_tile * (BN / 2) + wn * WC + cl;
      if (m < p.M && n < p.N) {  // N is a multiple of 8: a chunk is all in or all out
        const bf16x8 v = *reinterpret_cast<const bf16x8*>(stage + rl * WC + cl);
        *reinterpret_cast<bf16x8*>(reinterpret_cast<bf16*>(p.out_t) +
                                   (p.out_packed ? frag_index(m, n, p.ldt) : (long long)m * p.ldt + n)) = v;
      }
    }
  } else if (EPI == EPI_ARGMAX) {
    // per lane and row: a running 32-bit order key of the logit (strict > keeps
    // the lowest column on ties, the lane's columns increase with j); the 64-bit
    // (key, id) pair is formed once per row for the reduction across lanes
    unsigned long long* red = reinterpret_cast<unsigned long long*>(lds);  // [WN][BM]
    wait_barrier<0>();  // every wave is done with the stages
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ml = (wm * TM + i) * 16 + 4 * g + q;  // row within the tile
        const int m = m0 + ml;
        uint32_t bk = 0;
        int bn = -1;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n_tile * BN + (wn * TN + j) * 16 + r16;
          const bool ok = m < p.M && n < p.N;
          if (ok && p.dbg) p.dbg[(long long)m * p.ld_dbg + n] = acc[i][j][q];
          const uint32_t k = float_key(acc[i][j][q]);
          const bool better = ok && (bn < 0 || k > bk);
          bk = better ? k : bk;
          bn = better ? n : bn;
        }
        unsigned long long best = bn < 0 ? 0ull : (((unsigned long long)bk << 32) | (uint32_t)(p.N - 1 - bn));
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) best = key_max(best, __shfl_xor(best, o, 64));
        if (r16 == 0) red[wn * BM + ml] = best;
      }
    }
    __syncthreads();
    for (int r = t; r < BM; r += NT) {
      unsigned long long v = red[r];
#pragma unroll
      for (int w_ = 1; w_ < WN; ++w_) v = key_max(v, red[w_ * BM + r]);
      if (m0 + r < p.M) atomicMax(p.keys + m0 + r, v);
    }
  } else {  // EPI_TOPK
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int ml = (wm * TM + i) * 16 + 4 * g + q;  // row within the tile
        const int m = m0 + ml;
        unsigned long long best = 0ull;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n_tile * BN + (wn * TN + j) * 16 + r16;
          const bool ok = m < p.M && n < p.N;
          if (ok && p.dbg) p.dbg[(long long)m * p.ld_dbg + n] = acc[i][j][q];
          const unsigned long long key = ok ? argmax_key(acc[i][j][q], n, p.N) : 0ull;
          best = merge16_desc(best, sort16_desc(key, r16), r16);
        }
        if (m < p.M) p.keys[((long long)m * (WN * n_nt) + WN * n_tile + wn) * 16 + r16] = best;
      }
    }
  }
}

template <typename C, int EPI>
void launch_cfg(const GemmParams& p, hipStream_t s) {
  const int n_mt = (p.M + C::BM - 1) / C::BM;
  const int cols = col_tiles<C::BN, EPI>(p.tiles) * p.P;
  const int groups = (cols + 7) / 8;
  hipLaunchKernelGGL((k_gemm_tile<C, EPI>), dim3(groups * 8 * n_mt), dim3(C::NW * 64), 0, s, p);
}

// Above 128 rows: 256x256 tiles, 16 waves of 64x64 (four per SIMD, 128
// VGPRs each), one 32-wide k step per stage and a 5-stage ring (all 160 KB
// of LDS; three stages in flight while one is multiplied).  Per stage a CU
// moves 128 fragment reads and 32 KB of direct loads through LDS against
// 1024 MFMA cycles per SIMD.  More waves per SIMD keep the matrix cores busy
// across each stage's barrier: one wave of 128x128 per SIMD lost 15-30 %
// against two of 128x64, and four of 64x64 run the vocabulary product 5 %
// faster than two.
// Up to 128 rows (and for top-16, whose sort needs the registers): 128x128
// tiles, 4 waves of 64x64, two k steps per stage, 3 stages.
// 256x192 tiles (8 waves of 64x96, 64-deep k stages, double buffered in
// 112 KB of LDS) are taken where their workgroup count fills the CUs better
// than 256x256: the 24576-wide SwiGLU product gets 512 workgroups (two full
// rounds) instead of 384, whose second round would leave half the CUs idle.
// At 64 rows (4 requests of 16), 64x128 tiles: 4 waves of 32x64 and a
// 72 KB ring, so two workgroups share a CU and no MFMA row is empty; the
// product streams its weights once and is bound by that stream.  Two waves
// across N keep the top-16 list count per row equal to CfgSmall's.
typedef TileCfg<64, 128, 2, 2, 2, 3> Cfg64;
typedef TileCfg<128, 128, 2, 2, 2, 3> CfgSmall;
typedef TileCfg<256, 256, 4, 4, 1, 5> CfgBig;
typedef TileCfg<256, 192, 4, 2, 2, 2> CfgWide;
// 256x128 (8 waves of 128x32, 24 KB stages, 6-deep ring): for a split-K
// product whose K is short and whose columns fit 256 tiles, this grid fills
// the CUs with half the split of 256x256, so the consumer sums half as many
// fp32 planes (the O product at 1,024 rows: its norm reads 2 planes, not 4).
typedef TileCfg<256, 128, 2, 4, 1, 6> CfgTall;
static_assert(Cfg64::WN == CfgSmall::WN && Cfg64::BN == CfgSmall::BN, "top-16 lists per row");

enum { CFG_SMALL, CFG_BIG, CFG_WIDE, CFG_64, CFG_TALL };

// Workgroups with real work and the split-K factor of a partial-output
// product: the largest split whose grid still fits one round of the CUs (a
// grid of more than one round only adds a partly idle round and fp32 planes
// for the consumer to sum), keeping 8 or more 64-wide k blocks per split.
template <typename C, int EPI>
int cfg_work(int M, int tiles, int P) {
  return ((M + C::BM - 1) / C::BM) * col_tiles<C::BN, EPI>(tiles) * P;
}
template <typename C>
int cfg_split(int M, int tiles, int K) {
  const int wgs = cfg_work<C, EPI_PARTIAL>(M, tiles, 1);
  int P = wgs >= 256 ? 1 : 256 / wgs;
  while (P > 1 && K / (64 * P) < 8) --P;
  return P;
}
// share of the CU slots of the last round that has work (one workgroup per CU)
double round_fill(int w) { return (double)w / (256.0 * ((w + 255) / 256)); }

template <int EPI>
int tile_cfg_t(int M, int tiles, int K) {
  if (M <= 64) return CFG_64;
  if (EPI == EPI_TOPK || M <= 128) return CFG_SMALL;
  if (EPI == EPI_ARGMAX) return CFG_BIG;  // the vocabulary-wide product fills the CUs either way
  if (EPI == EPI_PARTIAL && M >= 256 && tiles <= 256 && K <= 4096) return CFG_TALL;
  const int pb = EPI == EPI_PARTIAL ? cfg_split<CfgBig>(M, tiles, K) : 1;
  const int pw = EPI == EPI_PARTIAL ? cfg_split<CfgWide>(M, tiles, K) : 1;
  const double fb = round_fill(cfg_work<CfgBig, EPI>(M, tiles, pb));
  const double fw = round_fill(cfg_work<CfgWide, EPI>(M, tiles, pw));
  return fw > fb + 0.05 ? CFG_WIDE : CFG_BIG;
}

int tile_cfg(int epi, int M, int tiles, int K) {
  switch (epi) {
    case EPI_PARTIAL: return tile_cfg_t<EPI_PARTIAL>(M, tiles, K);
    case EPI_SWIGLU: return tile_cfg_t<EPI_SWIGLU>(M, tiles, K);
    case EPI_ARGMAX: return tile_cfg_t<EPI_ARGMAX>(M, tiles, K);
    case EPI_TOPK: return tile_cfg_t<EPI_TOPK>(M, tiles, K);
    default: return CFG_SMALL;
  }
}

template <int EPI>
void launch_epi(const GemmParams& p, hipStream_t s) {
  switch (tile_cfg_t<EPI>(p.M, p.tiles, p.K)) {
    case CFG_64: launch_cfg<Cfg64, EPI>(p, s); break;
    case CFG_TALL:
      if constexpr (EPI == EPI_PARTIAL) launch_cfg<CfgTall, EPI>(p, s);
      break;
    case CFG_WIDE:
      if constexpr (EPI != EPI_ARGMAX && EPI != EPI_TOPK) launch_cfg<CfgWide, EPI>(p, s);
      break;
    case CFG_BIG:
      if constexpr (EPI != EPI_TOPK) launch_cfg<CfgBig, EPI>(p, s);
      break;
    default: launch_cfg<CfgSmall, EPI>(p, s); break;
  }
}

}  // namespace

// Lists per row written by the top-16 epilogue (one per column wave and tile).
int gemm_big_lists(int tiles) { return CfgSmall::WN * col_tiles<CfgSmall::BN, EPI_TOPK>(tiles); }

// Split-K factor of a partial-output product, for the tile shape the launch
// will pick.
int gemm_big_split(int M, int tiles, int K) {
  switch (tile_cfg(EPI_PARTIAL, M, tiles, K)) {
    case CFG_WIDE: return cfg_split<CfgWide>(M, tiles, K);
    case CFG_BIG: return cfg_split<CfgBig>(M, tiles, K);
    case CFG_64: return cfg_split<Cfg64>(M, tiles, K);
    case CFG_TALL: return cfg_split<CfgTall>(M, tiles, K);
    default: return cfg_split<CfgSmall>(M, tiles, K);
  }
}

void launch_gemm_big(int epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.tiles <= 0) return;
  switch (epi) {
    case EPI_PARTIAL: launch_epi<EPI_PARTIAL>(p, s); break;
    case EPI_SWIGLU: launch_epi<EPI_SWIGLU>(p, s); break;
    case EPI_TOPK: launch_epi<EPI_TOPK>(p, s); break;
    case EPI_ARGMAX: launch_epi<EPI_ARGMAX>(p, s); break;
    default: break;  // EPI_RESID has no tiled form; the runtime never asks for it here
  }
}

}  // namespace dflash
