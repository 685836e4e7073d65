// Tiled MFMA GEMM for many activation rows (M >= 64: batched drafts, long
// injections), where the products are bound by the matrix cores rather than
// by the weight stream.
//
// Y[M, N] = X[M, K] * W[N, K]^T, X row-major bf16 (virtual concatenation of
// a_parts arrays as in the skinny kernel), W packed in MFMA fragment order.
//  * A workgroup (4 waves, 2 x 2) computes a BM x 128 output tile; each wave
//    BM/2 x 64 with 16x16x32 bf16 MFMAs (fp32 accumulators in registers).
//  * K advances 64 at a time through two LDS stages holding both operands in
//    fragment order (one 1 KB fragment per 16 rows x 32 k), so every wave
//    reads its fragments with conflict-free 16-byte LDS loads; the next
//    stage's global loads are in flight while the current stage is consumed.
//  * Tile order is XCD-aware: workgroups are dealt to the 8 XCDs round-robin,
//    and the M-tiles that share a weight tile are given to the same XCD at the
//    same time, so the weight tile comes from HBM once and from L2 after.
// Epilogues: fp32 store (one split), SwiGLU (the 128 columns are 64 gate and
// the matching 64 up columns; the up waves hand their tile to the gate waves
// through LDS), greedy argmax (row maxima of the two column waves combined
// in LDS, one 64-bit atomic max per row and workgroup) and top-16 (sorted
// lists of 16 per row and column wave, merged later).
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kFrag = 64 * 8;  // bf16 elements of one fragment
constexpr int BN = 128;
constexpr int BK = 64;

__device__ __forceinline__ unsigned long long kmax2(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long kmin2(unsigned long long a, unsigned long long b) {
  return a < b ? a : b;
}
__device__ __forceinline__ unsigned long long sort16(unsigned long long v, int i) {
#pragma unroll
  for (int k = 2; k <= 16; k <<= 1)
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned long long o = __shfl_xor(v, j, 64);
      v = (((i & j) == 0) == ((i & k) == 0)) ? kmax2(v, o) : kmin2(v, o);
    }
  return v;
}
__device__ __forceinline__ unsigned long long merge16(unsigned long long cur, unsigned long long nw,
                                                      int i) {
  const int lane = threadIdx.x & 63;
  unsigned long long t = kmax2(cur, __shfl(nw, (lane & 48) | (15 - i), 64));
#pragma unroll
  for (int j = 8; j > 0; j >>= 1) {
    const unsigned long long o = __shfl_xor(t, j, 64);
    t = ((i & j) == 0) ? kmax2(t, o) : kmin2(t, o);
  }
  return t;
}

template <int BM, int EPI>
__global__ __launch_bounds__(256) void k_gemm_big(GemmParams p) {
  constexpr int TM = BM / 32;  // 16-row tiles per wave (wave rows = BM / 2)
  constexpr int TN = 4;        // 16-col tiles per wave (64 columns)
  constexpr int FA = BM / 16 * 2;  // A fragments per stage (BM rows x 64 k)
  constexpr int FB = BN / 16 * 2;  // B fragments per stage
  __shared__ __attribute__((aligned(16))) bf16 lds[2][(FA + FB) * kFrag];
  __shared__ unsigned long long red[BM];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int r16 = lane & 15, g = lane >> 4;

  // XCD-aware tile mapping
  const int n_mt = (p.M + BM - 1) / BM;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int m_tile = slot % n_mt;
  const int n_tile = (slot / n_mt) * 8 + xcd;  // 128-column tile
  const int n_tiles = (EPI == EPI_SWIGLU) ? (p.tiles + 3) / 4 : (p.tiles + 7) / 8;
  if (n_tile >= n_tiles) return;
  const int m0 = m_tile * BM;
  const int S = p.K / 32;

  // 16-row weight tile index of B fragment column j (0..7) of this tile
  auto wtile = [&](int j) -> int {
    if (EPI == EPI_SWIGLU) return j < 4 ? n_tile * 4 + j : p.up_tile_off + n_tile * 4 + (j - 4);
    return n_tile * 8 + j;
  };
  auto wfrag = [&](int j, int ks) -> const bf16* {
    int tt = wtile(j);
    int seg = 0;
    if (p.seg_tiles) {
      seg = tt / p.seg_tiles;
      tt -= seg * p.seg_tiles;
    }
    return reinterpret_cast<const bf16*>(p.w[seg]) + ((long long)tt * S + ks) * kFrag;
  };
  const int wtiles_total = (EPI == EPI_SWIGLU) ? p.up_tile_off + p.tiles : p.tiles;

  // global -> registers for one stage: (FA + FB) fragments, 4 lanes' worth per thread per round
  constexpr int RND = (FA + FB) * 64 / 256;
  bf16x8 stage[RND];
  auto gload = [&](int k0) {
#pragma unroll
    for (int q = 0; q < RND; ++q) {
      const int idx = t + 256 * q;
      const int f = idx >> 6, l = idx & 63;
      bf16x8 v;
      if (f < FA) {
        const int m16 = f >> 1, k32 = f & 1;
        const int row = m0 + m16 * 16 + (l & 15);
        const int k = k0 + k32 * 32 + 8 * (l >> 4);
        const int part = k / p.a_part_k;
        if (row < p.M) {
          v = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const bf16*>(p.a[part]) +
                                               (long long)row * p.lda + (k - part * p.a_part_k));
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
        }
      } else {
        const int fb = f - FA;
        const int j = fb >> 1, k32 = fb & 1;
        const int tt = wtile(j);
        if (tt < wtiles_total && (EPI == EPI_SWIGLU ? (j < 4 ? n_tile * 4 + j : n_tile * 4 + j - 4) < p.tiles : true)) {
          v = *reinterpret_cast<const bf16x8*>(wfrag(j, k0 / 32 + k32) + l * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = (bf16)0.0f;
        }
      }
      stage[q] = v;
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int q = 0; q < RND; ++q) {
      const int idx = t + 256 * q;
      *reinterpret_cast<bf16x8*>(&lds[buf][(idx >> 6) * kFrag + (idx & 63) * 8]) = stage[q];
    }
  };

  // chunk accumulators (one 256-wide slice of K) folded into running totals:
  // the fp32 rounding chain stays short however long K is
  f32x4 acc[TM][TN], tot[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      tot[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

  const int nk = p.K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int k32 = 0; k32 < 2; ++k32) {
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(&lds[cur][((wm * TM + i) * 2 + k32) * kFrag + lane * 8]);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8*>(&lds[cur][(FA + (wn * TN + j) * 2 + k32) * kFrag + lane * 8]);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_step(af[i], bfr[j], acc[i][j]);
    }
    if ((kt & 3) == 3 || kt + 1 == nk) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          tot[i][j] += acc[i][j];
          acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (kt + 1 < nk) {
      sstore(cur ^ 1);
      __syncthreads();
    }
  }
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = tot[i][j];

  // ---- epilogues: lane holds rows 4g+q, column r16 of each 16x16 tile ----
  if (EPI == EPI_PARTIAL || EPI == EPI_RESID) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = m0 + (wm * TM + i) * 16 + 4 * g + q;
          const int n = n_tile * BN + (wn * TN + j) * 16 + r16;
          if (m < p.M && n < p.N) {
            if (EPI == EPI_PARTIAL)
              p.out_f32[(long long)m * p.N + n] = acc[i][j][q];
            else
              p.resid[(long long)m * p.ldr + n] += acc[i][j][q];
          }
        }
  } else if (EPI == EPI_SWIGLU) {
    __syncthreads();  // LDS stages are free now
    float* up = reinterpret_cast<float*>(&lds[0][0]);  // [2 wm][TM*16 rows][64 cols]
    if (wn == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            up[(wm * TM * 16 + i * 16 + 4 * g + q) * 64 + j * 16 + r16] = acc[i][j][q];
    }
    __syncthreads();
    if (wn == 0) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int m = m0 + (wm * TM + i) * 16 + 4 * g + q;
            const int n = n_tile * 64 + j * 16 + r16;
            if (m < p.M && n < p.N) {
              const float gt = acc[i][j][q];
              const float u = up[(wm * TM * 16 + i * 16 + 4 * g + q) * 64 + j * 16 + r16];
              reinterpret_cast<bf16*>(p.out_t)[(long long)m * p.ldt + n] = (bf16)(gt / (1.0f + expf(-gt)) * u);
            }
          }
    }
  } else {  // EPI_ARGMAX / EPI_TOPK
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
          if (EPI == EPI_TOPK) {
            best = merge16(best, sort16(key, r16), r16);
          } else {
            best = kmax2(best, key);
          }
        }
        if (EPI == EPI_TOPK) {
          // one sorted list per row and column wave
          if (m < p.M)
            p.keys[((long long)m * (2 * n_tiles) + 2 * n_tile + wn) * 16 + r16] = best;
        } else {
#pragma unroll
          for (int o = 8; o >= 1; o >>= 1) best = kmax2(best, __shfl_xor(best, o, 64));
          if (wn == 1 && r16 == 0) red[ml] = best;
          __syncthreads();
          if (wn == 0 && r16 == 0 && m < p.M) atomicMax(p.keys + m, kmax2(best, red[ml]));
          __syncthreads();
        }
      }
    }
  }
}

template <int BM, int EPI>
void launch_bm(const GemmParams& p, hipStream_t s) {
  const int n_mt = (p.M + BM - 1) / BM;
  const int n_tiles = (EPI == EPI_SWIGLU) ? (p.tiles + 3) / 4 : (p.tiles + 7) / 8;
  const int groups = (n_tiles + 7) / 8;
  hipLaunchKernelGGL((k_gemm_big<BM, EPI>), dim3(groups * 8 * n_mt), dim3(256), 0, s, p);
}

template <int BM>
void launch_epi(int epi, const GemmParams& p, hipStream_t s) {
  switch (epi) {
    case EPI_PARTIAL: launch_bm<BM, EPI_PARTIAL>(p, s); break;
    case EPI_RESID: launch_bm<BM, EPI_RESID>(p, s); break;
    case EPI_SWIGLU: launch_bm<BM, EPI_SWIGLU>(p, s); break;
    case EPI_TOPK: launch_bm<BM, EPI_TOPK>(p, s); break;
    default: launch_bm<BM, EPI_ARGMAX>(p, s); break;
  }
}

}  // namespace

int gemm_big_lists(int tiles) { return 2 * ((tiles + 7) / 8); }

void launch_gemm_big(int epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.tiles <= 0) return;
  if (p.M <= 64)
    launch_epi<64>(epi, p, s);
  else
    launch_epi<128>(epi, p, s);
}

}  // namespace dflash
