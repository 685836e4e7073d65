// Weight-streaming GEMM for the draft's skinny products (M = batch * block rows).
//
// Y[M, N] = X[M, K] * W[N, K]^T.  At batch 1 every projection of the draft
// forward is bound by streaming W from HBM (16 rows of activations against
// each weight: 16 flop per byte), so the kernel is built around the weight
// stream:
//  * one workgroup (4 waves) owns a 16-row tile of W (two tiles for SwiGLU:
//    gate and up rows of the same output columns);
//  * the 4 waves split K in interleaved 256-element chunks; a lane streams 8
//    contiguous 16-byte pieces of its W row per chunk (each wave reads 16
//    rows x 512 contiguous bytes per chunk) while the next chunk is already
//    in flight;
//  * the products run on MFMA 16x16x32 bf16 (16x16x4 f32 for fp32 weights),
//    the activation tile is the A operand read through L2;
//  * the 4 per-wave partial tiles are summed through LDS in a fixed order
//    (deterministic) and the epilogue is applied once per output.
// Epilogues: plain fp32 store; residual add into the fp32 stream; SwiGLU
// (silu(gate) * up, rounded to the storage dtype); greedy selection (packed
// logit/id key, 64-bit atomic max per row, ties to the lowest id).
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kWaves = 4;
constexpr int kChunk = 256;

template <typename T>
struct WRow {
  const T* p;
  bool ok;
};

template <typename T>
__device__ __forceinline__ void load_w(typename Frag8<T>::type (&w)[8], const T* row, bool ok,
                                       int k0, int g) {
#pragma unroll
  for (int j = 0; j < 8; ++j) w[j] = ok ? load8<T>(row + k0 + 32 * j + 8 * g) : zero8<T>();
}

template <typename T>
__device__ __forceinline__ const T* a_ptr(const GemmParams& p, int m, int k0) {
  int part = k0 / p.a_part_k;
  const T* base = reinterpret_cast<const T*>(p.a[part]);
  return base + (long long)m * p.lda + (k0 - part * p.a_part_k);
}

template <typename T, int MT, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmParams p) {
  constexpr int NACC = (EPI == EPI_SWIGLU) ? 2 : 1;
  typedef typename Frag8<T>::type Frag;
  __shared__ float red[kWaves][MT * NACC][16][17];

  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int tile = blockIdx.x;
  const int m_base = blockIdx.y * 16 * MT;
  const int n0 = tile * 16;

  // weight rows of this lane
  const int seg = n0 / p.seg_rows;
  const int seg_row = n0 - seg * p.seg_rows + r16;
  const bool w_ok = (n0 + r16) < p.N;
  const T* wrow = reinterpret_cast<const T*>(p.w[seg]) + (long long)seg_row * p.K;
  const T* urow = (EPI == EPI_SWIGLU)
                      ? reinterpret_cast<const T*>(p.w_up) + (long long)(n0 + r16) * p.K
                      : nullptr;

  bool a_ok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) a_ok[mt] = (m_base + mt * 16 + r16) < p.M;

  f32x4 acc[MT][NACC];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q = 0; q < NACC; ++q) acc[mt][q] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunks = p.K / kChunk;
  Frag wc[8], wn[8];
  Frag uc[8], un[8];
  int c = wave;
  if (c < nchunks) {
    load_w<T>(wc, wrow, w_ok, c * kChunk, g);
    if (EPI == EPI_SWIGLU) load_w<T>(uc, urow, w_ok, c * kChunk, g);
  }
  for (; c < nchunks; c += kWaves) {
    const int k0 = c * kChunk;
    const bool more = (c + kWaves) < nchunks;
    if (more) {
      load_w<T>(wn, wrow, w_ok, k0 + kWaves * kChunk, g);
      if (EPI == EPI_SWIGLU) load_w<T>(un, urow, w_ok, k0 + kWaves * kChunk, g);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const T* ar = a_ptr<T>(p, m_base + mt * 16 + r16, k0);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        Frag a = a_ok[mt] ? load8<T>(ar + 32 * j + 8 * g) : zero8<T>();
        acc[mt][0] = mfma_step(a, wc[j], acc[mt][0]);
        if (EPI == EPI_SWIGLU) acc[mt][NACC - 1] = mfma_step(a, uc[j], acc[mt][NACC - 1]);
      }
    }
    if (more) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        wc[j] = wn[j];
        if (EPI == EPI_SWIGLU) uc[j] = un[j];
      }
    }
  }

  // cross-wave reduction (fixed order)
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int q = 0; q < NACC; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][mt * NACC + q][4 * g + i][r16] = acc[mt][q][i];
  __syncthreads();

  const int t = threadIdx.x;
  const int row = t >> 4;
  const int col = t & 15;
  const int n = n0 + col;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    float v[NACC];
#pragma unroll
    for (int q = 0; q < NACC; ++q) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) s += red[w][mt * NACC + q][row][col];
      v[q] = s;
    }
    const int m = m_base + mt * 16 + row;
    const bool ok = (m < p.M) && (n < p.N);
    if (EPI == EPI_STORE) {
      if (ok) p.out_f32[(long long)m * p.ldo + n] = v[0];
    } else if (EPI == EPI_RESID) {
      if (ok) p.resid[(long long)m * p.ldr + n] += v[0];
    } else if (EPI == EPI_SWIGLU) {
      if (ok) {
        float gt = v[0];
        float s = gt / (1.0f + expf(-gt));
        reinterpret_cast<T*>(p.out_t)[(long long)m * p.ldt + n] = from_f<T>(s * v[NACC - 1]);
      }
    } else {  // EPI_ARGMAX
      if (ok && p.dbg) p.dbg[(long long)m * p.ld_dbg + n] = v[0];
      unsigned long long key = ok ? argmax_key(v[0], n, p.N) : 0ull;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        unsigned long long other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
      }
      if (col == 0 && m < p.M) atomicMax(p.keys + m, key);
    }
  }
}

template <typename T, int EPI>
void launch_t(const GemmParams& p, hipStream_t s) {
  const int tiles = (p.N + 15) / 16;
  const int mt = p.M <= 16 ? 1 : (p.M <= 32 ? 2 : 4);
  dim3 grid(tiles, (p.M + 16 * mt - 1) / (16 * mt));
  if (mt == 1)
    hipLaunchKernelGGL((k_gemm<T, 1, EPI>), grid, dim3(256), 0, s, p);
  else if (mt == 2)
    hipLaunchKernelGGL((k_gemm<T, 2, EPI>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm<T, 4, EPI>), grid, dim3(256), 0, s, p);
}

template <typename T>
void launch_dt(int epi, const GemmParams& p, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: launch_t<T, EPI_STORE>(p, s); break;
    case EPI_RESID: launch_t<T, EPI_RESID>(p, s); break;
    case EPI_SWIGLU: launch_t<T, EPI_SWIGLU>(p, s); break;
    default: launch_t<T, EPI_ARGMAX>(p, s); break;
  }
}

}  // namespace

void launch_gemm(int dtype, int epi, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.N <= 0) return;
  if (dtype == DFLASH_BF16)
    launch_dt<bf16>(epi, p, s);
  else
    launch_dt<float>(epi, p, s);
}

}  // namespace dflash
