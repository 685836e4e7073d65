// Dynamic two-tap conv taps of the DFlash-2 draft ([guide] "DFlash：块扩散加速的
// LLM 推测解码技术", section 7: a two-tap depthwise conv around attention and
// the MLP, looking at the current and the previous position, the block start
// reading the last verified token; the page calls it dynamic and gives no
// form).  The taps of each row are the static taps plus a rank-r linear
// function of that row of the conv's input: t = D x (r values), then
// a = w0 + U_a t and b = w1 + U_b t per channel.
//
//  * k_dconv: one workgroup per (256 channels, row); t is summed from the
//    split-K partials of the product that formed it (the D product of the
//    stored normed rows before attention and the MLP; rows appended to W_o
//    and W_down after them) into LDS, then each thread forms its channel's
//    two taps from its rows of U (16-byte loads) and either applies them to
//    the stored input rows (writing the next GEMM's input) or writes them for
//    the norm that adds the conv'd projection output into the residual.
//  * k_fold: once per handle, D W for the output convs (their input is the
//    projection's output W o, so D (W o) = (D W) o joins the projection as
//    extra output rows); fp32 sums over 64-wide chunks of D staged in LDS,
//    stored as a storage-dtype pair hi + lo (2r rows), so the product keeps
//    the folded form to about 16 bits.
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

template <typename T> struct Pack8;
template <> struct Pack8<bf16> { typedef bf16x8 type; };
template <> struct Pack8<float> { typedef f32x8 type; };

template <typename T>
__global__ __launch_bounds__(256) void k_dconv(DConvParams p) {
  __shared__ float ts[64];
  const int row = blockIdx.y;
  const int t = threadIdx.x;
  const int c = blockIdx.x * 256 + t;
  if (t < p.r) {
    const float* tp = p.t + (long long)row * p.ldt + t;
    float v = 0.f;
    for (int q = 0; q < p.n_part; ++q) v += tp[q * p.plane];
    if (p.lo_off)  // the folded form's low part (a second set of r columns)
      for (int q = 0; q < p.n_part; ++q) v += tp[q * p.plane + p.lo_off];
    ts[t] = v;
  }
  __syncthreads();
  if (c >= p.d) return;
  const T* U = reinterpret_cast<const T*>(p.U);
  const T* ua = U + (long long)c * p.r;
  const T* ub = U + (long long)(p.d + c) * p.r;
  const T* w = reinterpret_cast<const T*>(p.w);
  float a = to_f(w[c]), b = to_f(w[p.d + c]);
  for (int j = 0; j < p.r; j += 8) {
    const typename Pack8<T>::type va = *reinterpret_cast<const typename Pack8<T>::type*>(ua + j);
    const typename Pack8<T>::type vb = *reinterpret_cast<const typename Pack8<T>::type*>(ub + j);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a += to_f(va[e]) * ts[j + e];
      b += to_f(vb[e]) * ts[j + e];
    }
  }
  if (!p.x) {
    p.taps[(long long)row * 2 * p.d + c] = a;
    p.taps[(long long)row * 2 * p.d + p.d + c] = b;
    return;
  }
  const T* X = reinterpret_cast<const T*>(p.x);
  const float x = to_f(X[(long long)row * p.d + c]);
  float xp;
  if (row % p.B == 0) {
    int tok = p.last_token[row / p.B];
    if (tok < 0 || tok >= p.vocab) {
      if (t == 0) atomicOr(p.err, 1u);
      tok = 0;
    }
    xp = to_f(reinterpret_cast<const T*>(p.embed)[(long long)tok * p.d + c]);
  } else {
    xp = to_f(X[(long long)(row - 1) * p.d + c]);
  }
  const long long oi = p.out_packed ? frag_index(row, c, p.d) : (long long)row * p.ldo + c;
  reinterpret_cast<T*>(p.out)[oi] = from_f<T>(a * x + b * xp);
}

template <typename T>
__global__ __launch_bounds__(256) void k_fold(const T* D, const T* W, T* out, int r, int d, int K) {
  __shared__ float dl[64][65];
  const int k = blockIdx.x * 256 + threadIdx.x;
  float acc[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) acc[j] = 0.f;
  for (int c0 = 0; c0 < d; c0 += 64) {
    __syncthreads();
    for (int i = threadIdx.x; i < 64 * 64; i += 256) {
      const int j = i >> 6, cc = i & 63;
      dl[j][cc] = j < r && c0 + cc < d ? to_f(D[(long long)j * d + c0 + cc]) : 0.f;
    }
    __syncthreads();
    if (k < K) {
      for (int cc = 0; cc < 64 && c0 + cc < d; ++cc) {
        const float wv = to_f(W[(long long)(c0 + cc) * K + k]);
#pragma unroll
        for (int j = 0; j < 64; ++j) acc[j] += dl[j][cc] * wv;
      }
    }
  }
  // rows 0..r-1: the sums rounded to the storage dtype; rows r..2r-1: what
  // that rounding left (so hi + lo carries the fp32 sum to about 16 bits)
  if (k < K)
    for (int j = 0; j < r; ++j) {
      const T hi = from_f<T>(acc[j]);
      out[(long long)j * K + k] = hi;
      out[(long long)(r + j) * K + k] = from_f<T>(acc[j] - to_f(hi));
    }
}

}  // namespace

void launch_dconv(int dtype, const DConvParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  const dim3 grid((p.d + 255) / 256, p.M);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_dconv<bf16>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(k_dconv<float>, grid, dim3(256), 0, s, p);
}

void launch_fold(int dtype, const void* D, const void* W, void* out, int r, int d, int K, hipStream_t s) {
  const dim3 grid((K + 255) / 256);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_fold<bf16>, grid, dim3(256), 0, s, reinterpret_cast<const bf16*>(D),
                       reinterpret_cast<const bf16*>(W), reinterpret_cast<bf16*>(out), r, d, K);
  else
    hipLaunchKernelGGL(k_fold<float>, grid, dim3(256), 0, s, reinterpret_cast<const float*>(D),
                       reinterpret_cast<const float*>(W), reinterpret_cast<float*>(out), r, d, K);
}

}  // namespace dflash
