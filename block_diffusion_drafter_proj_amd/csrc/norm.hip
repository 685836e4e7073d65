// Row-wise RMSNorm: out = x / sqrt(mean(x^2) + eps) * gamma, rounded to the
// storage dtype, where x is the residual row plus the split-K partials of the
// GEMM that produced it (written back as the new residual).  The sum of
// squares is a wavefront butterfly followed by a fixed-order sum over the
// waves, so the result does not depend on scheduling.
//
// The first norm of a draft forward also initialises the residual stream:
// every block row starts from the embedding of the mask token ([guide]
// section 3.1: the block is recovered from noise in one forward; the noise is
// read as mask tokens).  The final norm clears the per-row argmax keys that
// the LM head accumulates into.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

template <typename T> struct Out4;
template <> struct Out4<bf16> { typedef bf16x4 type; };
template <> struct Out4<float> { typedef f32x4 type; };

// Sum of 4 values of every thread over the workgroup (fixed order).
__device__ __forceinline__ float block_sum(float v, float* red, int slot) {
  v = wave_sum(v);
  const int t = threadIdx.x;
  const int nw = blockDim.x >> 6;
  if ((t & 63) == 0) red[slot * 16 + (t >> 6)] = v;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nw; ++w) tot += red[slot * 16 + w];
  return tot;
}

// Sum of the split-K partials of one row.
__device__ __forceinline__ f32x4 part_sum4(const NormParams& p, int row, int k, long long plane) {
  f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
  const float* pp = p.part + (long long)row * (p.ldp ? p.ldp : p.d) + k;
  for (int q0 = 0; q0 < p.n_part; q0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < p.n_part) v[q] = *reinterpret_cast<const f32x4*>(pp + (q0 + q) * plane);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < p.n_part) y += v[q];
  }
  return y;
}

// 4 elements of the embedding row of the request's last verified token (the
// block start's previous row at every conv point); a token outside the
// vocabulary is clamped and recorded in the error word.
template <typename T>
__device__ __forceinline__ f32x4 last_embed4(const NormParams& p, int row, int k) {
  int tok = p.last_token[row / p.B];
  if (tok < 0 || tok >= p.vocab) {
    if (threadIdx.x == 0) atomicOr(p.err, 1u);
    tok = 0;
  }
  const T* e = reinterpret_cast<const T*>(p.embed) + (long long)tok * p.d + k;
  f32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = to_f(e[i]);
  return v;
}

// Residual row with a conv'd GEMM output (DFlash 2, output points):
// x[row] = x_in[row] + w0 * y[row] + w1 * y[row-1], y the sum of the GEMM's
// split-K partials and y[row-1] the last verified token's embedding at the
// start of each request's block.
template <typename T>
__device__ __forceinline__ f32x4 load_row4_oconv(const NormParams& p, int row, int k, long long plane,
                                                 f32x4 w0, f32x4 w1) {
  const f32x4 h = *reinterpret_cast<const f32x4*>(p.x_in + (long long)row * p.ldx + k);
  const f32x4 y = part_sum4(p, row, k, plane);
  const f32x4 yp = (row % p.B) == 0 ? last_embed4<T>(p, row, k) : part_sum4(p, row - 1, k, plane);
  f32x4 x;
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = h[i] + w0[i] * y[i] + w1[i] * yp[i];
  return x;
}

template <typename T>
__device__ __forceinline__ f32x4 load_row4(const NormParams& p, int row, int k, long long plane) {
  f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p.init_row) {
    const T* init = reinterpret_cast<const T*>(p.init_row) + k;
    if (p.init_tokens) {  // token embeddings (ids were checked by the caller's kernel or the host)
      int tok = p.init_tokens[row];
      if (tok < 0 || tok >= p.vocab) {
        if (threadIdx.x == 0 && p.err) atomicOr(p.err, 1u);
        tok = 0;
      }
      init += (long long)tok * p.d;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f(init[i]);
  } else if (p.x_in) {
    x = *reinterpret_cast<const f32x4*>(p.x_in + (long long)row * p.ldx + k);
  }
  if (p.n_part) {
    const float* pp = p.part + (long long)row * (p.ldp ? p.ldp : p.d) + k;
    for (int q0 = 0; q0 < p.n_part; q0 += 8) {
      f32x4 v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < p.n_part) v[q] = *reinterpret_cast<const f32x4*>(pp + (q0 + q) * plane);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (q0 + q < p.n_part) x += v[q];
    }
  }
  return x;
}

// One workgroup of d/4 threads per row; every thread owns 4 consecutive
// elements, issues all of its loads (residual and every split-K partial)
// before summing them, and keeps the row in registers across the reduction.
// With a conv, the workgroup also normalises the previous row of the block.
template <typename T>
__global__ __launch_bounds__(1024) void k_rmsnorm(NormParams p) {
  __shared__ float red[32];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int k = 4 * t;
  const long long plane = (long long)p.M * (p.ldp ? p.ldp : p.d);
  const bool first = p.conv && (row % p.B) == 0;
  f32x4 x, xp = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p.otaps) {  // the producing GEMM's output conv with this row's dynamic taps
    const float* ta = p.otaps + (long long)row * 2 * p.d + k;
    x = load_row4_oconv<T>(p, row, k, plane, *reinterpret_cast<const f32x4*>(ta),
                           *reinterpret_cast<const f32x4*>(ta + p.d));
  } else if (p.oconv) {  // the producing GEMM's output conv folded in (this row and, for the input conv, the previous)
    f32x4 ow0, ow1;
    const T* o0 = reinterpret_cast<const T*>(p.oconv) + k;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ow0[i] = to_f(o0[i]);
      ow1[i] = to_f(o0[p.d + i]);
    }
    // y[row - 1] serves both rows: the GEMM output sums y[row], y[row - 1]
    // (and y[row - 2] for the previous row) are each formed once
    const f32x4 h0 = *reinterpret_cast<const f32x4*>(p.x_in + (long long)row * p.ldx + k);
    const f32x4 y0 = part_sum4(p, row, k, plane);
    const f32x4 y1 = (row % p.B) == 0 ? last_embed4<T>(p, row, k) : part_sum4(p, row - 1, k, plane);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = h0[i] + ow0[i] * y0[i] + ow1[i] * y1[i];
    if (p.conv && !first) {  // row - 1 is in the block: y1 is its own y
      const f32x4 h1 = *reinterpret_cast<const f32x4*>(p.x_in + (long long)(row - 1) * p.ldx + k);
      const f32x4 y2 = ((row - 1) % p.B) == 0 ? last_embed4<T>(p, row - 1, k) : part_sum4(p, row - 2, k, plane);
#pragma unroll
      for (int i = 0; i < 4; ++i) xp[i] = h1[i] + ow0[i] * y1[i] + ow1[i] * y2[i];
    }
  } else {
    x = load_row4<T>(p, row, k, plane);
    if (p.conv && !first) xp = load_row4<T>(p, row - 1, k, plane);
  }
  // the row-independent operands are requested with the row: the reduction's
  // barrier below would otherwise hold their loads back for a second round trip
  f32x4 gm, cw0 = f32x4{0.f, 0.f, 0.f, 0.f}, cw1 = f32x4{0.f, 0.f, 0.f, 0.f};
  {
    const T* gamma = reinterpret_cast<const T*>(p.gamma) + k;
#pragma unroll
    for (int i = 0; i < 4; ++i) gm[i] = to_f(gamma[i]);
    if (p.conv) {
      const T* w0 = reinterpret_cast<const T*>(p.conv) + k;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        cw0[i] = to_f(w0[i]);
        cw1[i] = to_f(w0[p.d + i]);
      }
    }
  }
  if (p.x_out) *reinterpret_cast<f32x4*>(p.x_out + (long long)row * p.ldx + k) = x;
  if (p.dbg) *reinterpret_cast<f32x4*>(p.dbg + (long long)row * p.d + k) = x;
  if (p.feat) {
    typename Out4<T>::type fo;
#pragma unroll
    for (int i = 0; i < 4; ++i) fo[i] = from_f<T>(x[i]);
    *reinterpret_cast<typename Out4<T>::type*>(reinterpret_cast<T*>(p.feat) + (long long)row * p.d + k) = fo;
  }
  const float tot = block_sum((x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]), red, 0);
  const float r = 1.0f / sqrtf(tot / (float)p.d + p.eps);
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = x[i] * r * gm[i];
  if (p.conv) {
    f32x4 prev;
    if (first) {
      prev = last_embed4<T>(p, row, k);
    } else {
      const float totp = block_sum((xp[0] * xp[0] + xp[1] * xp[1]) + (xp[2] * xp[2] + xp[3] * xp[3]), red, 1);
      const float rp = 1.0f / sqrtf(totp / (float)p.d + p.eps);
#pragma unroll
      for (int i = 0; i < 4; ++i) prev[i] = xp[i] * rp * gm[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = cw0[i] * y[i] + cw1[i] * prev[i];
  }
  typename Out4<T>::type o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = from_f<T>(y[i]);
  const long long oi = p.out_packed ? frag_index(row, k, p.d) : (long long)row * p.ldo + k;
  *reinterpret_cast<typename Out4<T>::type*>(reinterpret_cast<T*>(p.out) + oi) = o;
  if (p.zero_keys && t == 0) p.zero_keys[row] = 0ull;
}

// RMSNorm into fragment order (the tiled GEMM's operand layout), ROWS rows
// per workgroup (ROWS divides 16, so they sit in one 16-row block).  Output
// chunk c (8 consecutive k of one row, 16 bytes in bf16) is row c mod ROWS,
// k group (c / ROWS) mod 4 and k step c / (4 ROWS), and belongs to thread
// c mod blockDim: the ROWS rows' chunks of one fragment lane group are
// adjacent in memory, so a wave writes whole 64-byte runs and reads 512
// contiguous bytes of each of its rows.  blockDim is a multiple of 64, so
// thread t only ever holds row t mod ROWS; its chunks stay in registers, their
// squares are summed in chunk order, then over the row's lanes of the wave
// (butterfly) and over the waves in order.  Gamma waits in LDS.  No conv taps (those need the previous row of the
// request's block).
constexpr int kNormRows = 4;       // rows per workgroup of the fragment-order norm
constexpr int kNormThreads = 1024;  // its workgroup size at most

template <typename T, int ROWS>
__global__ __launch_bounds__(1024) void k_rmsnorm_frag(NormParams p) {
  constexpr int CMAX = 8;  // chunks per thread: ROWS * d / 8 over blockDim
  __shared__ float red[16 * ROWS];
  __shared__ float rs[ROWS];
  __shared__ float gs[4096];  // gamma, staged while the rows load
  const int t = threadIdx.x, nt = blockDim.x;
  const int row = blockIdx.x * ROWS + t % ROWS;
  const bool live = row < p.M;
  const int cpt = ROWS * p.d / 8 / nt;
  const int S = p.d / 32;
  const long long plane = (long long)p.M * p.d;
  // every row and partial load of the thread is issued before any is used,
  // and gamma is staged after them, so the pass waits for one round trip
  f32x4 x[CMAX][2];
#pragma unroll
  for (int j = 0; j < CMAX; ++j) {
    if (j < cpt) {
      const int q = (t + j * nt) / ROWS;
      const int k = 32 * (q >> 2) + 8 * (q & 3);
      x[j][0] = live ? load_row4<T>(p, row, k, plane) : f32x4{0.f, 0.f, 0.f, 0.f};
      x[j][1] = live ? load_row4<T>(p, row, k + 4, plane) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
  for (int k = t; k < p.d; k += nt) gs[k] = to_f(reinterpret_cast<const T*>(p.gamma)[k]);
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < CMAX; ++j) {
    if (j < cpt) {
      const int q = (t + j * nt) / ROWS;
      const int k = 32 * (q >> 2) + 8 * (q & 3);
      if (live && p.x_out) {
        *reinterpret_cast<f32x4*>(p.x_out + (long long)row * p.ldx + k) = x[j][0];
        *reinterpret_cast<f32x4*>(p.x_out + (long long)row * p.ldx + k + 4) = x[j][1];
      }
      if (live && p.dbg) {
        *reinterpret_cast<f32x4*>(p.dbg + (long long)row * p.d + k) = x[j][0];
        *reinterpret_cast<f32x4*>(p.dbg + (long long)row * p.d + k + 4) = x[j][1];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ss += (x[j][h][0] * x[j][h][0] + x[j][h][1] * x[j][h][1]) + (x[j][h][2] * x[j][h][2] + x[j][h][3] * x[j][h][3]);
    }
  }
  // a row's lanes in a wave are ROWS apart: butterfly over them, then the
  // waves in order
#pragma unroll
  for (int o = 32; o >= ROWS; o >>= 1) ss += __shfl_xor(ss, o, 64);
  if ((t & 63) < ROWS) red[(t >> 6) * ROWS + (t & 63)] = ss;
  __syncthreads();
  if (t < ROWS) {
    float tot = 0.f;
    for (int w = 0; w < nt / 64; ++w) tot += red[w * ROWS + t];
    rs[t] = 1.0f / sqrtf(tot / (float)p.d + p.eps);
  }
  __syncthreads();
  const float r = rs[t % ROWS];
  T* out = reinterpret_cast<T*>(p.out);
  const long long rb = row >> 4;
  const int lane0 = row & 15;
#pragma unroll
  for (int j = 0; j < CMAX; ++j) {
    if (j < cpt) {
      const int q = (t + j * nt) / ROWS;
      const int k = 32 * (q >> 2) + 8 * (q & 3);
      typename Out4<T>::type o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[h][i] = from_f<T>(live ? x[j][h][i] * r * gs[k + 4 * h + i] : 0.f);
      T* dst = out + (((rb * S + (q >> 2)) * 64 + lane0 + 16 * (q & 3)) << 3);  // frag_index(row, k, d)
      *reinterpret_cast<typename Out4<T>::type*>(dst) = o[0];
      *reinterpret_cast<typename Out4<T>::type*>(dst + 4) = o[1];
    }
  }
  if (p.zero_keys && t < ROWS && live) p.zero_keys[row] = 0ull;
}

}  // namespace

void launch_rmsnorm(int dtype, const NormParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  if (p.out_packed && !p.conv && !p.oconv && !p.otaps && !p.ldp && !p.feat && !p.init_tokens && p.d % 256 == 0 &&
      p.d <= 4096) {
    constexpr int R = kNormRows;
    const int nt = std::min(kNormThreads, R * p.d / 8);  // R * d / 8 chunks, at most 8 per thread
    if (dtype == DFLASH_BF16)
      hipLaunchKernelGGL((k_rmsnorm_frag<bf16, R>), dim3((p.M + R - 1) / R), dim3(nt), 0, s, p);
    else
      hipLaunchKernelGGL((k_rmsnorm_frag<float, R>), dim3((p.M + R - 1) / R), dim3(nt), 0, s, p);
    return;
  }
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_rmsnorm<bf16>, dim3(p.M), dim3(p.d / 4), 0, s, p);
  else
    hipLaunchKernelGGL(k_rmsnorm<float>, dim3(p.M), dim3(p.d / 4), 0, s, p);
}

}  // namespace dflash
