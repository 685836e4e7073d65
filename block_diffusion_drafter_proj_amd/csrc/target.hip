// Target-side verify forward on gfx950 ([guide] "DFlash：块扩散加速的 LLM 推测解码技术",
// section 4: the target runs once over the context and the drafted block and
// checks every drafted token in parallel; section 3.2: its feature layers
// feed the draft).  The target is a causal decoder with its own paged KV
// cache; its projections, norms and MLP run on the draft's GEMM and norm
// kernels.  Two kernels are its own:
//
//  * k_target_q: q of the new rows, split-K partial sums in order, RoPE at
//    each row's absolute position, rounded to the storage dtype, row-major
//    [rows][Hq][dh], or tiled for the split attention.  (K and V of the new
//    rows go into the request's pages through the injection's scatter
//    kernel.)
//
// In bf16 the attention runs on the draft's split-K ring kernel in its
// causal mode (the attention source holds it); fp32 handles use:
//  * k_causal_attn: one workgroup per (query head, request, 16-row tile) of
//    8 waves; wave w takes every 8th pair of 16-position pages of the
//    visible range [kv_begin, last row's position] and runs S^T = K Q^T and
//    O^T = V^T P^T on 16x16x32 MFMA tiles with an online softmax per row
//    (P as an exact bf16 hi + lo pair); row i of the tile sees key positions
//    up to its own.  The waves' (max, sum, O) are merged in LDS in wave
//    order.  Keys outside [kv_begin, ctx + rows) never enter: their scores
//    are -inf and their V is zeroed, so stale or poisoned pages never leak in.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

template <typename T> struct Vec4T;
template <> struct Vec4T<bf16> { typedef bf16x4 type; };
template <> struct Vec4T<float> { typedef f32x4 type; };

// One workgroup of dh/2 threads per (output row, query head): thread j
// rotates the pair (j, j + dh/2).  Output rows are the new rows (row-major
// layout) or, in the tiled layout of the split attention, 16 rows per
// (request, tile) pair with the rows past the request's last one zeroed.
template <typename T>
__global__ __launch_bounds__(64) void k_target_q(TargetQParams p) {
  const int orow = blockIdx.x, hh = blockIdx.y;
  const int j = threadIdx.x;
  const int h2 = p.dh / 2;
  int r, i;  // request, new row of the request
  T* dst;
  if (p.n_tiles) {
    const int rv = orow >> 4;
    r = rv / p.n_tiles;
    i = (rv - r * p.n_tiles) * 16 + (orow & 15);
    dst = reinterpret_cast<T*>(p.q) + ((long long)(rv * p.Hq + hh) * 16 + (orow & 15)) * p.dh;
    if (i >= p.R) {
      dst[j] = from_f<T>(0.f);
      dst[j + h2] = from_f<T>(0.f);
      return;
    }
  } else {
    r = orow / p.R;
    i = orow - r * p.R;
    dst = reinterpret_cast<T*>(p.q) + ((long long)orow * p.Hq + hh) * p.dh;
  }
  const int row = r * p.R + i;
  const int pos = p.pos0[r] + i;
  const long long plane = (long long)p.M * p.ld;
  const float* src = p.qkv + (long long)row * p.ld + hh * p.dh;
  float x1 = 0.f, x2 = 0.f;
  for (int q = 0; q < p.n_part; ++q) {
    x1 += src[q * plane + j];
    x2 += src[q * plane + j + h2];
  }
  const float c = p.cos_t[(long long)pos * h2 + j], sn = p.sin_t[(long long)pos * h2 + j];
  dst[j] = from_f<T>(x1 * c - x2 * sn);
  dst[j + h2] = from_f<T>(x2 * c + x1 * sn);
}

constexpr int kCausalWaves = 8;

template <typename T, int DH>
__global__ __launch_bounds__(64 * kCausalWaves) void k_causal_attn(CausalAttnParams p) {
  typedef typename Frag8<T>::type Frag;
  typedef typename Vec4T<T>::type V4;
  constexpr int NJ = DH / 32;
  constexpr int ND = DH / 16;
  const float NEG = -INFINITY;
  __shared__ float sacc[16][DH + 4];
  __shared__ float sml[kCausalWaves][16][2];

  const int h = blockIdx.x;
  const int r = blockIdx.y;
  const int tile = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int gkv = h / G;
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int slot = p.slots[r];
  const SlotState st = p.state[slot];
  const int pos0 = p.pos0[r];
  const int row0 = tile * 16;
  const int rows = min(16, p.R - row0);  // rows of this tile
  const int lo = st.kv_begin;
  const int hi = pos0 + row0 + rows;    // one past the last row's position
  const int wend = pos0 + p.R;          // one past the last written position
  const int myrow = row0 + l16;         // this lane's query row (column of S^T)
  const int mypos = pos0 + myrow;
  const bool rowok = l16 < rows;
  const int lp0 = lo / 16;
  const int n_lp = hi > lo ? (hi - 1) / 16 - lp0 + 1 : 0;
  const long long page_elems = 2LL * p.Hkv * 16 * DH;
  const T* pool = reinterpret_cast<const T*>(p.pool);

  Frag qf[NJ];
  {
    const T* qrow = reinterpret_cast<const T*>(p.q) + ((long long)(r * p.R + (rowok ? myrow : row0)) * p.Hq + h) * DH;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qf[j] = rowok ? load8<T>(qrow + 32 * j + 8 * g4) : zero8<T>();
  }
  float m_run = NEG, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto page_of = [&](int u) -> const T* {  // visible page u (0 .. n_lp-1), or NULL
    if (u >= n_lp) return nullptr;
    const int page = p.page_table[(long long)slot * p.pt_stride + lp0 + u];
    if (page < 0 || page >= p.max_pages) {
      if (lane == 0) atomicOr(p.err, 2u);
      return nullptr;
    }
    return pool + (long long)page * page_elems;
  };
  Frag kf[2][NJ], kn[2][NJ];
  V4 vv[2][ND], vn[2][ND];
  auto load_pair = [&](int u, Frag (&kd)[2][NJ], V4 (&vd)[2][ND]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const T* b = page_of(u + t);
      if (b) {
        const T* kb = b + (long long)gkv * 16 * DH + l16 * DH + 8 * g4;
        const T* vb = b + (long long)(p.Hkv + gkv) * 16 * DH + l16 * 16 + 4 * g4;
#pragma unroll
        for (int j = 0; j < NJ; ++j) kd[t][j] = load8<T>(kb + 32 * j);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vd[t][dt] = *reinterpret_cast<const V4*>(vb + dt * 256);
      }
    }
  };
  int u = 2 * wave;
  if (u < n_lp) load_pair(u, kf, vv);
  for (; u < n_lp; u += 2 * kCausalWaves) {
    const bool more = u + 2 * kCausalWaves < n_lp;
    if (more) load_pair(u + 2 * kCausalWaves, kn, vn);
    bool has[2], kval[2][4], vval[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      has[t] = u + t < n_lp && page_of(u + t) != nullptr;
      const int kpos = (lp0 + u + t) * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kp = kpos + 4 * g4 + i;
        vval[t][i] = has[t] && kp >= lo && kp < wend;
        kval[t][i] = vval[t][i] && rowok && kp <= mypos;  // causal, per query row
      }
    }
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
      if (has[t]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) sa = mfma_step(kf[t][j], qf[j], sa);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * t + i] = kval[t][i] ? sa[i] * p.scale : NEG;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_run == NEG) ? (m_new == NEG ? 1.f : 0.f) : expf(m_run - m_new);
    float pe[8];
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = (sv[e] == NEG) ? 0.f : expf(sv[e] - m_new);
      ls += pe[e];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * corr + ls;
    m_run = m_new;
    Frag pf, pf_lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = from_f<T>(pe[e]);
      pf_lo[e] = from_f<T>(pe[e] - to_f(pf[e]));
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      o[dt] = o[dt] * corr;
      Frag vf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[4 * t + i] = vval[t][i] ? vv[t][dt][i] : (T)0.0f;
      o[dt] = mfma_step(vf, pf, o[dt]);
      if (sizeof(T) == 2) o[dt] = mfma_step(vf, pf_lo, o[dt]);
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) kf[t][j] = kn[t][j];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vv[t][dt] = vn[t][dt];
      }
    }
  }

  // merge the waves' key subsets in wave order: (max, sum) per row, then O
  if (g4 == 0) {
    sml[wave][l16][0] = m_run;
    sml[wave][l16][1] = l_run;
  }
  __syncthreads();
  float M = NEG;
  for (int w = 0; w < kCausalWaves; ++w) M = fmaxf(M, sml[w][l16][0]);
  float L = 0.f;
  for (int w = 0; w < kCausalWaves; ++w) {
    const float mw = sml[w][l16][0];
    if (mw != NEG) L += sml[w][l16][1] * expf(mw - M);
  }
  const float f = (m_run == NEG) ? 0.f : expf(m_run - M);
  for (int w = 0; w < kCausalWaves; ++w) {
    if (wave == w) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float* a = &sacc[l16][dt * 16 + 4 * g4 + i];
          *a = (w == 0 ? 0.f : *a) + o[dt][i] * f;
        }
    }
    __syncthreads();
  }
  // row-major (or fragment-order) output: rows of the tile, DH columns of head h
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (wave == 0 && rowok) {
    const long long orow = (long long)r * p.R + myrow;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      V4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f<T>(sacc[l16][dt * 16 + 4 * g4 + i] * inv);
      const int col = h * DH + dt * 16 + 4 * g4;
      const long long oi = p.out_packed ? frag_index((int)orow, col, p.ldo) : orow * p.ldo + col;
      *reinterpret_cast<V4*>(reinterpret_cast<T*>(p.out) + oi) = v;
    }
  }
}

}  // namespace

void launch_target_q(int dtype, const TargetQParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  const dim3 grid(p.n_tiles ? p.M / p.R * p.n_tiles * 16 : p.M, p.Hq);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_target_q<bf16>, grid, dim3(p.dh / 2), 0, s, p);
  else
    hipLaunchKernelGGL(k_target_q<float>, grid, dim3(p.dh / 2), 0, s, p);
}

void launch_causal_attn(int dtype, int dh, int n_req, const CausalAttnParams& p, hipStream_t s) {
  if (n_req <= 0) return;
  const dim3 grid(p.Hq, n_req, (p.R + 15) / 16);
  const dim3 block(64 * kCausalWaves);
  if (dtype == DFLASH_BF16) {
    if (dh == 128)
      hipLaunchKernelGGL((k_causal_attn<bf16, 128>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((k_causal_attn<bf16, 64>), grid, block, 0, s, p);
  } else {
    if (dh == 128)
      hipLaunchKernelGGL((k_causal_attn<float, 128>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((k_causal_attn<float, 64>), grid, block, 0, s, p);
  }
}

}  // namespace dflash
