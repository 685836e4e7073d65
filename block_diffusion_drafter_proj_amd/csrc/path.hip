// DFlash-2 path selector on gfx950 ([guide] "DFlash：块扩散加速的 LLM 推测解码技术",
// section 7, path selector bullet): the top-16 candidates of adjacent block
// positions are scored in pairs by a low-rank bilinear form over their
// shared-embedding rows, s(a, b) = (W_u E[a]) . (W_v E[b]), and one greedy
// path is walked through them.
//
//  * k_sel_table (once, at device initialisation): the projected embedding
//    rows u = E W_u^T and v = E W_v^T for the whole vocabulary, fp32 [V, r]
//    each, so a draft only gathers 16 rows per position instead of
//    projecting its candidates through the 2 x r x d selector weights.
//  * k_select_path (per draft): one workgroup of 16 waves per request.  Wave
//    i forms the 16 x 16 score matrix of positions (i, i+1) on the matrix
//    cores (16x16x4 fp32 MFMA over r; A = the u rows of position i's
//    candidates, B = the v rows of position i+1's) and, for each candidate a
//    of position i, the candidate b of position i+1 maximising logit(b) +
//    s(a, b) (packed keys, ties to the lower candidate index), into LDS; one
//    lane then walks the positions through that table: step i+1 takes the
//    successor of the candidate chosen at step i.
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

// out[v][j] = sum_k E[v][k] W[j][k] for j < r (fp32), W = W_u (z = 0) or W_v
// (z = 1): 64 x 64 output tiles, 32-wide k chunks staged in LDS, 4 x 4
// outputs per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_sel_table(const T* E, const T* Wu, const T* Wv, float* tu, float* tv,
                                                   int V, int d, int r) {
  __shared__ float ea[64][33];
  __shared__ float wa[64][33];
  const T* W = blockIdx.z ? Wv : Wu;
  float* out = blockIdx.z ? tv : tu;
  const int v0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
  for (int k0 = 0; k0 < d; k0 += 32) {
    for (int i = threadIdx.x; i < 64 * 32; i += 256) {
      const int rr = i >> 5, kk = i & 31;
      const int v = v0 + rr;
      ea[rr][kk] = v < V ? to_f(E[(long long)v * d + k0 + kk]) : 0.f;
      wa[rr][kk] = to_f(W[(long long)(j0 + rr) * d + k0 + kk]);
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] += ea[ty * 4 + a][kk] * wa[tx * 4 + b][kk];
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int v = v0 + ty * 4 + a;
    if (v < V)
#pragma unroll
      for (int b = 0; b < 4; ++b) out[(long long)v * r + j0 + tx * 4 + b] = acc[a][b];
  }
}

__global__ __launch_bounds__(1024) void k_select_path(PathParams p) {
  __shared__ int nxt[15][16];    // best successor of each candidate
  __shared__ float nsc[15][16];  // and its score
  __shared__ int cid[16][16];
  __shared__ float clg[16][16];
  const int req = blockIdx.x;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int B = p.B;
  const int* ids = p.topk_ids + (long long)req * B * 16;
  const float* lg = p.topk_logits + (long long)req * B * 16;
  if ((int)threadIdx.x < B * 16) {
    int t = ids[threadIdx.x];
    if (t < 0 || t >= p.vocab) {
      atomicOr(p.err, 1u);
      t = 0;
    }
    cid[threadIdx.x >> 4][threadIdx.x & 15] = t;
    clg[threadIdx.x >> 4][threadIdx.x & 15] = lg[threadIdx.x];
  }
  __syncthreads();
  if (wave < B - 1) {
    // lane l supplies row / column l % 16 and 8 consecutive k of each 32-wide
    // step starting at 8 * (l / 16); A and B agree on which k a lane supplies
    const int row = lane & 15, g = lane >> 4;
    const float* ua = p.tu + (long long)cid[wave][row] * p.r + 8 * g;
    const float* vb = p.tv + (long long)cid[wave + 1][row] * p.r + 8 * g;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    // the rows are scattered over the tables: request 4 k-steps of both
    // operands before multiplying, so a pair waits for r / 128 round trips
    const int nstep = p.r / 32;
    for (int s0 = 0; s0 < nstep; s0 += 4) {
      f32x8 a[4], b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool in = s0 + j < nstep;
        a[j] = in ? load8<float>(ua + 32 * (s0 + j)) : zero8<float>();
        b[j] = in ? load8<float>(vb + 32 * (s0 + j)) : zero8<float>();
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma_step(a[j], b[j], acc);
    }
    // C layout: lane l holds column b = l % 16 (candidate of position i+1)
    // and rows a = 4 * (l / 16) + q (candidates of position i); the 16
    // columns of a row sit in 16 adjacent lanes.  Larger logit(b) + s(a, b)
    // wins, ties to the lower b.
    const float lb = clg[wave + 1][row];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      unsigned long long key = ((unsigned long long)float_key(lb + acc[q]) << 32) | (unsigned)(15 - row);
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) {
        const unsigned long long other = __shfl_xor(key, o, 64);
        key = other > key ? other : key;
      }
      if (row == 0) {
        nxt[wave][4 * g + q] = 15 - (int)(key & 0xffffffffu);
        nsc[wave][4 * g + q] = key_float((uint32_t)(key >> 32));
      }
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  int* path = p.path + (long long)req * B;
  float* score = p.step_scores ? p.step_scores + (long long)req * B : nullptr;
  path[0] = cid[0][0];
  if (score) score[0] = clg[0][0];
  int k = 0;
  for (int i = 0; i + 1 < B; ++i) {
    const int kn = nxt[i][k];
    path[i + 1] = cid[i + 1][kn];
    if (score) score[i + 1] = nsc[i][k];
    k = kn;
  }
}

}  // namespace

void launch_sel_table(int dtype, const void* embed, const void* wu, const void* wv, float* tu, float* tv, int V,
                      int d, int r, hipStream_t s) {
  const dim3 grid((V + 63) / 64, r / 64, 2);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_sel_table<bf16>, grid, dim3(256), 0, s, reinterpret_cast<const bf16*>(embed),
                       reinterpret_cast<const bf16*>(wu), reinterpret_cast<const bf16*>(wv), tu, tv, V, d, r);
  else
    hipLaunchKernelGGL(k_sel_table<float>, grid, dim3(256), 0, s, reinterpret_cast<const float*>(embed),
                       reinterpret_cast<const float*>(wu), reinterpret_cast<const float*>(wv), tu, tv, V, d, r);
}

void launch_select_path(const PathParams& p, int n_req, hipStream_t s) {
  if (n_req <= 0) return;
  hipLaunchKernelGGL(k_select_path, dim3(n_req), dim3(1024), 0, s, p);
}

}  // namespace dflash
