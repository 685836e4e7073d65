// Row-wise RMSNorm: out = x / sqrt(mean(x^2) + eps) * gamma, rounded to the
// storage dtype.  One 256-thread workgroup per row; the sum of squares is a
// wavefront butterfly followed by a fixed-order sum over the 4 waves, so the
// result does not depend on scheduling.
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

template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(NormParams p) {
  __shared__ float part[4];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const int per = p.d / 256;
  const T* init = reinterpret_cast<const T*>(p.init_row);
  const T* gamma = reinterpret_cast<const T*>(p.gamma);
  T* out = reinterpret_cast<T*>(p.out) + (long long)row * p.ldo;
  const long long plane = (long long)p.M * p.d;

  auto input = [&](int k) {
    float x = init ? to_f(init[k]) : (p.x_in ? p.x_in[(long long)row * p.ldx + k] : 0.f);
    for (int q = 0; q < p.n_part; ++q) x += p.part[q * plane + (long long)row * p.d + k];
    return x;
  };

  float ss = 0.f;
  for (int i = 0; i < per; ++i) {
    const int k = t + 256 * i;
    const float x = input(k);
    if (p.x_out) p.x_out[(long long)row * p.ldx + k] = x;
    if (p.dbg) p.dbg[(long long)row * p.d + k] = x;
    ss += x * x;
  }
  ss = wave_sum(ss);
  if ((t & 63) == 0) part[t >> 6] = ss;
  __syncthreads();
  const float tot = (part[0] + part[1]) + (part[2] + part[3]);
  const float r = 1.0f / sqrtf(tot / (float)p.d + p.eps);
  for (int i = 0; i < per; ++i) {
    const int k = t + 256 * i;
    const float x = p.x_out ? p.x_out[(long long)row * p.ldx + k] : input(k);
    out[k] = from_f<T>(x * r * to_f(gamma[k]));
  }
  if (p.zero_keys && t == 0) p.zero_keys[row] = 0ull;
}

}  // namespace

void launch_rmsnorm(int dtype, const NormParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_rmsnorm<bf16>, dim3(p.M), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_rmsnorm<float>, dim3(p.M), dim3(256), 0, s, p);
}

}  // namespace dflash
