// Greedy selection and prefix acceptance.
//
// k_finalize  decodes the per-row packed argmax key (logit key << 32 |
//             vocab-1-id) left by the LM head into the draft token id.
// k_verify    keeps the longest draft prefix that matches the target's greedy
//             tokens ([news] "DFlash 2 的核心：一次写一块": with 8 drafted and
//             the first 6 matching, 6 are accepted and generation continues
//             at the 7th position; [guide] section 3.3).  One wavefront per
//             request: a ballot of mismatches, the first set bit is the
//             accept length a; the cycle commits d[0..a) and the target's
//             own token G[a], which becomes the next pending token.
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

__global__ __launch_bounds__(256) void k_finalize(const unsigned long long* keys, int rows,
                                                  int vocab, int* draft) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows) return;
  const unsigned long long k = keys[i];
  draft[i] = vocab - 1 - (int)(uint32_t)(k & 0xffffffffull);
}

__global__ __launch_bounds__(64) void k_verify(int B, int vocab, const int* draft,
                                               const int* greedy, int* accept, int* committed,
                                               int* last, unsigned int* err) {
  const int r = blockIdx.x;
  const int i = threadIdx.x;
  const int* d = draft + (long long)r * B;
  const int* g = greedy + (long long)r * (B + 1);
  const int gi = i <= B ? g[i] : 0;
  const bool mismatch = i < B && d[i] != gi;
  const unsigned long long mask = __ballot(mismatch);
  const int a = mask ? (int)__builtin_ctzll(mask) : B;
  const int ga = __shfl(gi, a, 64);
  const bool bad = ga < 0 || ga >= vocab;
  if (i <= B) {
    int v = -1;
    if (i < a) v = d[i];
    else if (i == a) v = bad ? 0 : ga;
    committed[(long long)r * (B + 1) + i] = v;
  }
  if (i == 0) {
    accept[r] = a;
    last[r] = bad ? 0 : ga;
    if (bad) atomicOr(err, 1u);
  }
}

// Sums the split-K partial logits of one row over one chunk of the
// vocabulary (planes in split order, so the result does not depend on
// scheduling).  Wave w takes the 64-column blocks w, w+4, ... of the chunk;
// every lane requests all of its partial values before the first sum, then
// argmax keeps a running maximum key per lane and top-16 a running sorted
// list per 16-lane group, merged across the wave's four groups at the end.
template <bool TOPK>
__global__ __launch_bounds__(256) void k_logit_select(LogitSelParams p) {
  constexpr int NB = kSelChunk / 256;  // column blocks per wave
  __shared__ unsigned long long red[4];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, i16 = lane & 15;
  const long long plane = (long long)p.M * p.N;
  const float* src = p.part + (long long)row * p.N;
  const int c0 = chunk * kSelChunk + wave * 64 + lane;
  float v[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) v[b] = 0.f;
  for (int q = 0; q < p.n_part; ++q) {
    float x[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int n = c0 + 256 * b;
      x[b] = n < p.N ? src[q * plane + n] : 0.f;
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) v[b] += x[b];
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int n = c0 + 256 * b;
    const bool ok = n < p.N;
    if (ok && p.dbg) p.dbg[(long long)row * p.ld_dbg + n] = v[b];
    const unsigned long long key = ok ? argmax_key(v[b], n, p.N) : 0ull;
    if (TOPK)
      best = merge16_desc(best, sort16_desc(key, i16), i16);
    else
      best = key_max(best, key);
  }
  if (TOPK) {
    best = merge16_desc(best, __shfl_xor(best, 16, 64), i16);
    best = merge16_desc(best, __shfl_xor(best, 32, 64), i16);
    if (lane < 16) p.lists[((long long)row * p.n_lists + chunk * 4 + wave) * 16 + lane] = best;
  } else {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) best = key_max(best, __shfl_xor(best, o, 64));
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (t == 0) atomicMax(p.keys + row, key_max(key_max(red[0], red[1]), key_max(red[2], red[3])));
  }
}

// The same selection with 16-byte reads, for a vocabulary that is a multiple
// of 4 (every row then starts 16-byte aligned): wave w takes the 256-column
// blocks w, w+4, ... of the chunk, each lane 4 consecutive columns of a
// block, and the loads of up to 4 planes are all issued before any sum.  The
// selected keys do not depend on the order in which columns are visited.
template <bool TOPK>
__global__ __launch_bounds__(256) void k_logit_select4(LogitSelParams p) {
  constexpr int NB = kSelChunk / 1024;  // 256-column blocks per wave
  __shared__ unsigned long long red[4];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, i16 = lane & 15;
  const long long plane = (long long)p.M * p.N;
  const float* src = p.part + (long long)row * p.N;
  const int c0 = chunk * kSelChunk + wave * 256 + lane * 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 v[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) v[b] = zero;
  for (int q0 = 0; q0 < p.n_part; q0 += 4) {
    f32x4 x[4][NB];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int n = c0 + 1024 * b;
        x[q][b] = q0 + q < p.n_part && n < p.N ? *reinterpret_cast<const f32x4*>(src + (q0 + q) * plane + n) : zero;
      }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int b = 0; b < NB; ++b)
        if (q0 + q < p.n_part) v[b] += x[q][b];
  }
  unsigned long long best = 0ull;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int n = c0 + 1024 * b + k;
      const bool ok = n < p.N;
      if (ok && p.dbg) p.dbg[(long long)row * p.ld_dbg + n] = v[b][k];
      const unsigned long long key = ok ? argmax_key(v[b][k], n, p.N) : 0ull;
      if (TOPK)
        best = merge16_desc(best, sort16_desc(key, i16), i16);
      else
        best = key_max(best, key);
    }
  }
  if (TOPK) {
    best = merge16_desc(best, __shfl_xor(best, 16, 64), i16);
    best = merge16_desc(best, __shfl_xor(best, 32, 64), i16);
    if (lane < 16) p.lists[((long long)row * p.n_lists + chunk * 4 + wave) * 16 + lane] = best;
  } else {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) best = key_max(best, __shfl_xor(best, o, 64));
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (t == 0) atomicMax(p.keys + row, key_max(key_max(red[0], red[1]), key_max(red[2], red[3])));
  }
}

// Merge two lists sorted descending into the 16 largest, sorted descending.
__device__ __forceinline__ void merge_lists(const unsigned long long* a, const unsigned long long* b,
                                            unsigned long long* out) {
  int ia = 0, ib = 0;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const unsigned long long va = a[ia], vb = b[ib];  // ia + ib = k <= 15
    if (va >= vb) {
      out[k] = va;
      ++ia;
    } else {
      out[k] = vb;
      ++ib;
    }
  }
}

// One workgroup per row: every thread first folds lists t, t+256, ... into a
// running top-16, then the 256 running lists are merged pairwise in LDS until
// one list remains; rank 0 is the greedy draft token.
__global__ __launch_bounds__(256) void k_topk_merge(TopkParams p) {
  __shared__ unsigned long long lst[256 * 16];
  const int row = blockIdx.x;
  const int t = threadIdx.x;
  const unsigned long long* src = p.lists + (long long)row * p.n_lists * 16;
  unsigned long long run[16], nxt[16], tmp[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) run[k] = 0ull;
  for (int li = t; li < p.n_lists; li += 256) {
#pragma unroll
    for (int k = 0; k < 16; ++k) nxt[k] = src[(long long)li * 16 + k];
    merge_lists(run, nxt, tmp);
#pragma unroll
    for (int k = 0; k < 16; ++k) run[k] = tmp[k];
  }
#pragma unroll
  for (int k = 0; k < 16; ++k) lst[t * 16 + k] = run[k];
  __syncthreads();
  for (int half = 128; half >= 1; half >>= 1) {
    if (t < half) merge_lists(lst + t * 16, lst + (t + half) * 16, tmp);
    __syncthreads();
    if (t < half) {
#pragma unroll
      for (int k = 0; k < 16; ++k) lst[t * 16 + k] = tmp[k];
    }
    __syncthreads();
  }
  if (t < 16) {
    const unsigned long long key = lst[t];
    const int id = p.vocab - 1 - (int)(uint32_t)(key & 0xffffffffull);
    p.topk_ids[(long long)row * 16 + t] = id;
    p.topk_logits[(long long)row * 16 + t] = key_float((uint32_t)(key >> 32));
    if (t == 0) p.draft[row] = id;
  }
}

}  // namespace

void launch_logit_select(bool topk, const LogitSelParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  const dim3 grid((p.N + kSelChunk - 1) / kSelChunk, p.M);
  if (p.N % 4 == 0) {
    if (topk)
      hipLaunchKernelGGL(k_logit_select4<true>, grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL(k_logit_select4<false>, grid, dim3(256), 0, s, p);
  } else if (topk) {
    hipLaunchKernelGGL(k_logit_select<true>, grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL(k_logit_select<false>, grid, dim3(256), 0, s, p);
  }
}

void launch_topk_merge(const TopkParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  hipLaunchKernelGGL(k_topk_merge, dim3(p.M), dim3(256), 0, s, p);
}

void launch_finalize(const unsigned long long* keys, int rows, int vocab, int* draft,
                     hipStream_t s) {
  if (rows <= 0) return;
  hipLaunchKernelGGL(k_finalize, dim3((rows + 255) / 256), dim3(256), 0, s, keys, rows, vocab,
                     draft);
}

void launch_verify(int n_req, int B, int vocab, const int* draft, const int* greedy, int* accept,
                   int* committed, int* last, unsigned int* err, hipStream_t s) {
  if (n_req <= 0) return;
  hipLaunchKernelGGL(k_verify, dim3(n_req), dim3(64), 0, s, B, vocab, draft, greedy, accept,
                     committed, last, err);
}

}  // namespace dflash
