// Dynamic two-tap conv taps of the DFlash-2 draft ([guide] "DFlash：块扩散加速的
// LLM 推测解码技术", section 7: a two-tap depthwise conv around attention and
// the MLP, looking at the current and the previous position, the block start
// reading the last verified token; the page calls it dynamic and gives no
// form).  The taps of each row are the static taps plus a rank-r linear
// function of that row of the conv's input: t = D x (r values), then
// a = w0 + U_a t and b = w1 + U_b t per channel.
//
//  * k_dconv: one workgroup per (64 channels, 16 rows); t is summed from the
//    split-K partials of the product that formed it (the D product of the
//    stored normed rows before attention and the MLP; rows appended to W_o
//    and W_down after them) into LDS, the rank-r parts of the taps are formed
//    on the matrix cores, and each lane either applies its taps to the stored
//    input rows (writing the next GEMM's input) or writes them for the norm
//    that adds the conv'd projection output into the residual.
//  * k_fold: once per handle, D W for the output convs (their input is the
//    projection's output W o, so D (W o) = (D W) o joins the projection as
//    extra output rows); fp32 sums over 64-wide chunks of D staged in LDS,
//    stored as a storage-dtype pair hi + lo (2r rows), so the product keeps
//    the folded form to about 16 bits.
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

// One workgroup of 4 waves per (64 channels, 16 rows); wave w takes 16
// channels.  The taps' rank-r parts U_a t and U_b t of the 16 rows are two
// 16 x 16 products over r (r = 32 or 64: one or two 32-wide k-steps) on the
// matrix cores: U's rows are the A operand (16-byte loads of a channel's r
// values), t the B operand from LDS (fp32; in bf16 as an exact-to-16-bits
// hi + lo pair, two MFMAs).  A lane then holds one row and four consecutive
// channels of each product.
constexpr int kDcRows = 16, kDcChan = 64, kDcMaxPart = 16;
template <typename T>
__global__ __launch_bounds__(256) void k_dconv(DConvParams p) {
  typedef typename Frag8<T>::type Frag;
  __shared__ float ts[kDcRows][64 + 4];
  const int row0 = blockIdx.y * kDcRows;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int nk = p.r / 32;  // k-steps (1 or 2)
  // U rows of this wave's 16 channels (A operand), requested first
  const int cw = blockIdx.x * kDcChan + wave * 16;  // first channel of the wave
  const int ca = min(cw + l16, p.d - 1);
  const T* U = reinterpret_cast<const T*>(p.U);
  Frag fa[2], fb[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int ss = min(s, nk - 1);
    fa[s] = load8<T>(U + (long long)ca * p.r + 32 * ss + 8 * g4);
    fb[s] = load8<T>(U + (long long)(p.d + ca) * p.r + 32 * ss + 8 * g4);
  }
  // this lane's outputs: row row0 + l16, channels c .. c+3; their static taps
  // and input rows are requested now too, so the kernel waits for memory once
  const int orow = row0 + l16;
  const int oc = cw + 4 * g4;
  const int crow = min(orow, p.M - 1);
  const T* w = reinterpret_cast<const T*>(p.w);
  float w0[4], w1[4], xv[4], xpv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    w0[i] = to_f(w[oc + i]);
    w1[i] = to_f(w[p.d + oc + i]);
  }
  if (p.x) {
    const T* X = reinterpret_cast<const T*>(p.x);
    const T* xr = X + (long long)crow * p.d + oc;
    const T* xpr;
    if (crow % p.B == 0) {
      int tok = p.last_token[crow / p.B];
      if (tok < 0 || tok >= p.vocab) {
        if (orow < p.M) atomicOr(p.err, 1u);
        tok = 0;
      }
      xpr = reinterpret_cast<const T*>(p.embed) + (long long)tok * p.d + oc;
    } else {
      xpr = xr - p.d;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[i] = to_f(xr[i]);
      xpv[i] = to_f(xpr[i]);
    }
  }
  // t of the block's rows, summed over the splits (and the low part): thread
  // (row, 4 consecutive j) reads 16 bytes per split; every load uses a clamped,
  // valid index and a select, so all are in flight together
  {
    const int n4 = p.r / 4;
    const int rr = min(t / n4, kDcRows - 1), j = (t - (t / n4) * n4) * 4;
    const int row = min(row0 + rr, p.M - 1);
    const int nlo = p.lo_off ? 2 : 1;
    const float* tp = p.t + (long long)row * p.ldt + j;
    f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < kDcMaxPart; ++q) {
        const f32x4 x =
            *reinterpret_cast<const f32x4*>(tp + (long long)min(q, p.n_part - 1) * p.plane + min(h, nlo - 1) * p.lo_off);
        if (q < p.n_part && h < nlo) v += x;
      }
    if (t < kDcRows * n4) {
      const bool live = row0 + t / n4 < p.M;
#pragma unroll
      for (int e = 0; e < 4; ++e) ts[t / n4][j + e] = live ? v[e] : 0.f;
    }
  }
  __syncthreads();
  // C[channel][row] = sum_j U[channel][j] t[row][j]
  f32x4 acc_a = f32x4{0.f, 0.f, 0.f, 0.f}, acc_b = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nk; ++s) {
    const float* tr = &ts[l16][32 * s + 8 * g4];
    Frag th, tl;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      th[e] = from_f<T>(tr[e]);
      tl[e] = from_f<T>(tr[e] - to_f(th[e]));
    }
    acc_a = mfma_step(fa[s], th, acc_a);
    acc_b = mfma_step(fb[s], th, acc_b);
    if (sizeof(T) == 2) {
      acc_a = mfma_step(fa[s], tl, acc_a);
      acc_b = mfma_step(fb[s], tl, acc_b);
    }
  }
  if (orow >= p.M) return;
  f32x4 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = w0[i] + acc_a[i];
    b[i] = w1[i] + acc_b[i];
  }
  if (!p.x) {
    *reinterpret_cast<f32x4*>(p.taps + (long long)orow * 2 * p.d + oc) = a;
    *reinterpret_cast<f32x4*>(p.taps + (long long)orow * 2 * p.d + p.d + oc) = b;
    return;
  }
  T* out = reinterpret_cast<T*>(p.out) + (p.out_packed ? frag_index(orow, oc, p.d) : (long long)orow * p.ldo + oc);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = from_f<T>(a[i] * xv[i] + b[i] * xpv[i]);
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
  if (p.M <= 0 || p.n_part < 1 || p.n_part > kDcMaxPart) return;  // the host checks the split count
  const dim3 grid((p.d + kDcChan - 1) / kDcChan, (p.M + kDcRows - 1) / kDcRows);
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
