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
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

template <typename T> struct Out4;
template <> struct Out4<bf16> { typedef bf16x4 type; };
template <> struct Out4<float> { typedef f32x4 type; };

// One workgroup of d/4 threads per row; every thread owns 4 consecutive
// elements, issues all of its loads (residual and every split-K partial)
// before summing them, and keeps the row in registers across the reduction.
template <typename T>
__global__ __launch_bounds__(1024) void k_rmsnorm(NormParams p) {
  __shared__ float part[16];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int k = 4 * t;
  const long long plane = (long long)p.M * p.d;
  f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
  if (p.init_row) {
    const T* init = reinterpret_cast<const T*>(p.init_row) + k;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = to_f(init[i]);
  } else if (p.x_in) {
    x = *reinterpret_cast<const f32x4*>(p.x_in + (long long)row * p.ldx + k);
  }
  const float* pp = p.part + (long long)row * p.d + k;
  for (int q0 = 0; q0 < p.n_part; q0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < p.n_part) v[q] = *reinterpret_cast<const f32x4*>(pp + (q0 + q) * plane);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q0 + q < p.n_part) x += v[q];
  }
  if (p.x_out) *reinterpret_cast<f32x4*>(p.x_out + (long long)row * p.ldx + k) = x;
  if (p.dbg) *reinterpret_cast<f32x4*>(p.dbg + (long long)row * p.d + k) = x;
  float ss = (x[0] * x[0] + x[1] * x[1]) + (x[2] * x[2] + x[3] * x[3]);
  ss = wave_sum(ss);
  const int nw = blockDim.x >> 6;
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
  for (int w = 0; w < nw; ++w) tot += part[w];
  const float r = 1.0f / sqrtf(tot / (float)p.d + p.eps);
  const T* gamma = reinterpret_cast<const T*>(p.gamma) + k;
  typename Out4<T>::type o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = from_f<T>(x[i] * r * to_f(gamma[i]));
  *reinterpret_cast<typename Out4<T>::type*>(reinterpret_cast<T*>(p.out) + (long long)row * p.ldo + k) = o;
  if (p.zero_keys && t == 0) p.zero_keys[row] = 0ull;
}

}  // namespace

void launch_rmsnorm(int dtype, const NormParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_rmsnorm<bf16>, dim3(p.M), dim3(p.d / 4), 0, s, p);
  else
    hipLaunchKernelGGL(k_rmsnorm<float>, dim3(p.M), dim3(p.d / 4), 0, s, p);
}

}  // namespace dflash
