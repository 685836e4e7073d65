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
