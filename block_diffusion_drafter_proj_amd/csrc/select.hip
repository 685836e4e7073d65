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
// k_logit_select  sums the split-K partial logits of 17..64 rows over one
//             vocabulary chunk and keeps the row's argmax key or one sorted
//             top-16 list per wave (a threshold from the lanes' maxima, then
//             one sort of the few keys that pass);
// k_topk_redo recomputes, by an exact bisection pass, the lists that the
//             threshold pass could not settle;
// k_topk_merge merges a row's lists into its top 16 and draft token.
#include <stdlib.h>

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

// A wave's top-16 list that the candidate pass left to the exact pass.  No
// key has all bits set: its low word, vocab - 1 - id, is below 2^31.
constexpr unsigned long long kListRedo = ~0ull;

// Packs the keys >= thr into the wave's 64 LDS slots by ballot rank (key
// index, then lane); returns how many passed (all counted, the first 64
// stored).  The slots are the wave's own: a wave-level fence orders the
// lanes' LDS writes before the reads.
template <int NK>
__device__ __forceinline__ int pack_candidates(const unsigned long long (&key)[NK], unsigned long long thr,
                                               unsigned long long* cand) {
  int cnt = 0;  // wave-uniform
#pragma unroll
  for (int k = 0; k < NK; ++k) {
    const bool f = key[k] >= thr;
    const unsigned long long m = __ballot(f);
    const int slot = cnt + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(m >> 32),
                                                          __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
    if (f && slot < 64) cand[slot] = key[k];
    cnt += (int)__popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  return cnt;
}

// The 16 largest of the wave's 64 * NK keys (key[k] of every lane), sorted
// descending in lanes 0..15, or kListRedo.  Let tau be the 16th largest of
// the 64 per-lane maxima: those 16 maxima are keys >= tau, so the 16th
// largest key is >= tau and only keys >= tau can rank.  With tau = 0 (fewer
// than 16 lanes hold a nonzero key: the end of the vocabulary) the
// candidates are the nonzero keys and the zero padding fills the list.
// About 20 keys pass for logits without ties; at most 64 are sorted in one
// pass, and a wave with more (which takes many large logits packed into
// fewer than 16 lanes) returns kListRedo, as every wave does with `redo`.
template <int NK>
__device__ __forceinline__ unsigned long long wave_top16(const unsigned long long (&key)[NK],
                                                         unsigned long long* cand, int lane, bool redo) {
  unsigned long long lm = key[0];
#pragma unroll
  for (int k = 1; k < NK; ++k) lm = key_max(lm, key[k]);
  const unsigned long long tau = __shfl(sort64_desc(lm, lane), 15, 64);
  const int cnt = pack_candidates(key, tau ? tau : 1ull, cand);
  const unsigned long long s = sort64_desc(lane < cnt ? cand[lane] : 0ull, lane);
  return cnt <= 64 && !redo ? s : kListRedo;
}

// The same list for any keys: the 16th largest key t by bisection over the
// key range (at least 16 keys >= lo, fewer than 16 >= hi), then the keys
// >= max(t, 1) sorted: the valid keys are distinct, so at most 16 pass, and
// with t = 0 (fewer than 16 nonzero keys) the list is padded with zero keys
// as the padding itself would be.
template <int NK>
__device__ __forceinline__ unsigned long long wave_top16_exact(const unsigned long long (&key)[NK],
                                                               unsigned long long* cand, int lane) {
  static_assert(64 * NK >= 16, "at least 16 keys");
  unsigned long long lo = 0ull, hi = ~0ull;
#pragma unroll 1
  while (hi - lo > 1) {
    const unsigned long long mid = lo + ((hi - lo) >> 1);
    int c = 0;
#pragma unroll
    for (int k = 0; k < NK; ++k) c += (int)__popcll(__ballot(key[k] >= mid));
    if (c >= 16)
      lo = mid;
    else
      hi = mid;
  }
  const int cnt = pack_candidates(key, lo ? lo : 1ull, cand);
  return sort64_desc(lane < cnt ? cand[lane] : 0ull, lane);
}

// Sum of the split-K partial planes (in split order, so the result does not
// depend on scheduling) at the 16 columns lane `lane` of wave `wave` covers
// in one chunk of the vocabulary, as packed keys (zero past the vocabulary);
// every load is requested before the first sum.  Two layouts:
//  VEC4 (vocabulary a multiple of 4, every row 16-byte aligned): the wave
//    takes the 256-column blocks wave, wave + 4, ... of the chunk, each lane
//    4 consecutive columns of a block (column c0 + 1024 b + k, key 4 b + k);
//  scalar: the 64-column blocks wave, wave + 4, ... (column c0 + 256 b).
// The selected keys do not depend on the order in which columns are visited.
template <bool VEC4>
__device__ __forceinline__ void wave_keys(const LogitSelParams& p, int row, int chunk, int wave, int lane,
                                          unsigned long long (&key)[16], bool dbg) {
  const long long plane = (long long)p.M * p.N;
  const float* src = p.part + (long long)row * p.N;
  if constexpr (VEC4) {
    constexpr int NB = kSelChunk / 1024;
    static_assert(4 * NB == 16, "16 keys per lane");
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
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int n = c0 + 1024 * b + k;
        const bool ok = n < p.N;
        if (dbg && ok && p.dbg) p.dbg[(long long)row * p.ld_dbg + n] = v[b][k];
        key[4 * b + k] = ok ? argmax_key(v[b][k], n, p.N) : 0ull;
      }
  } else {
    constexpr int NB = kSelChunk / 256;
    static_assert(NB == 16, "16 keys per lane");
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
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int n = c0 + 256 * b;
      const bool ok = n < p.N;
      if (dbg && ok && p.dbg) p.dbg[(long long)row * p.ld_dbg + n] = v[b];
      key[b] = ok ? argmax_key(v[b], n, p.N) : 0ull;
    }
  }
}

// One workgroup of 4 waves per (chunk, row): argmax reduces the keys to the
// row's maximum (atomic max into keys[row]); top-16 writes each wave's 16
// largest keys as one sorted list, or kListRedo for k_topk_redo.
template <bool VEC4, bool TOPK>
__global__ __launch_bounds__(256) void k_logit_select(LogitSelParams p) {
  __shared__ unsigned long long red[4];
  __shared__ unsigned long long cand[TOPK ? 4 : 1][64];
  const int chunk = blockIdx.x, row = blockIdx.y;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  unsigned long long key[16];
  wave_keys<VEC4>(p, row, chunk, wave, lane, key, true);
  if constexpr (TOPK) {
    const unsigned long long best = wave_top16(key, cand[wave], lane, p.exact != 0);
    if (lane < 16) p.lists[((long long)row * p.n_lists + chunk * 4 + wave) * 16 + lane] = best;
  } else {
    unsigned long long best = key[0];
#pragma unroll
    for (int b = 1; b < 16; ++b) best = key_max(best, key[b]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) best = key_max(best, __shfl_xor(best, o, 64));
    if (lane == 0) red[wave] = best;
    __syncthreads();
    if (t == 0) atomicMax(p.keys + row, key_max(key_max(red[0], red[1]), key_max(red[2], red[3])));
  }
}

// One workgroup per row: wave w looks at the row's lists w, w + 4, ... 64 at
// a time (one load per lane) and recomputes each list marked kListRedo from
// the partial planes with the exact pass.
template <bool VEC4>
__global__ __launch_bounds__(256) void k_topk_redo(LogitSelParams p) {
  __shared__ unsigned long long cand[4][64];
  const int row = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  unsigned long long* lists = p.lists + (long long)row * p.n_lists * 16;
  for (int base = 0; base < p.n_lists; base += 256) {
    const int li = base + 4 * lane + wave;
    const bool redo = li < p.n_lists && lists[(long long)li * 16] == kListRedo;
    unsigned long long m = __ballot(redo);
    while (m) {
      const int l = (int)__builtin_ctzll(m);
      m &= m - 1;
      const int lj = base + 4 * l + wave;  // chunk lj / 4, wave lj % 4 == wave
      unsigned long long key[16];
      wave_keys<VEC4>(p, row, lj >> 2, wave, lane, key, false);
      const unsigned long long best = wave_top16_exact(key, cand[wave], lane);
      if (lane < 16) lists[(long long)lj * 16 + lane] = best;
    }
  }
}

// a := the 16 largest of lists a and b (both sorted descending), sorted
// descending: the elementwise maximum of a and reversed b holds the 16
// largest of the 32 as a bitonic sequence, which four half-cleaner stages
// sort.
__device__ __forceinline__ void top16_merge(unsigned long long (&a)[16], const unsigned long long (&b)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) a[i] = key_max(a[i], b[15 - i]);
#pragma unroll
  for (int j = 8; j >= 1; j >>= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & j) == 0) {
        const unsigned long long hi = key_max(a[i], a[i + j]), lo = key_min(a[i], a[i + j]);
        a[i] = hi;
        a[i + j] = lo;
      }
}

// One wave per row: lane l folds the row's lists l, l + 64, ... into a
// running top 16 in registers (up to four lists requested at once), then the
// lanes' lists are merged across lanes in six rounds (lane l takes lane
// l + o's, o = 32 .. 1); lane 0 ends with the row's top 16, whose rank 0 is
// the greedy draft token.
__global__ __launch_bounds__(64) void k_topk_merge(TopkParams p) {
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  const unsigned long long* src = p.lists + (long long)row * p.n_lists * 16;
  unsigned long long run[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) run[k] = 0ull;
  for (int l0 = lane; l0 < p.n_lists; l0 += 256) {
    unsigned long long nxt[4][16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int li = l0 + 64 * q;
#pragma unroll
      for (int k = 0; k < 16; ++k) nxt[q][k] = li < p.n_lists ? src[(long long)li * 16 + k] : 0ull;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) top16_merge(run, nxt[q]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    unsigned long long nxt[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) nxt[k] = __shfl_down(run[k], o, 64);
    top16_merge(run, nxt);
  }
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const unsigned long long key = run[k];
      const int id = p.vocab - 1 - (int)(uint32_t)(key & 0xffffffffull);
      p.topk_ids[(long long)row * 16 + k] = id;
      p.topk_logits[(long long)row * 16 + k] = key_float((uint32_t)(key >> 32));
      if (k == 0) p.draft[row] = id;
    }
  }
}

}  // namespace

void launch_logit_select(bool topk, const LogitSelParams& lp, hipStream_t s) {
  if (lp.M <= 0) return;
  LogitSelParams p = lp;
  // every top-16 list through the exact pass when DFLASH_SELECT_EXACT is set
  // (the same lists, slower: a check of the candidate pass)
  const char* ex = getenv("DFLASH_SELECT_EXACT");
  p.exact = ex && ex[0] && ex[0] != '0';
  const dim3 grid((p.N + kSelChunk - 1) / kSelChunk, p.M);
  if (p.N % 4 == 0) {
    if (topk) {
      hipLaunchKernelGGL((k_logit_select<true, true>), grid, dim3(256), 0, s, p);
      hipLaunchKernelGGL(k_topk_redo<true>, dim3(p.M), dim3(256), 0, s, p);
    } else {
      hipLaunchKernelGGL((k_logit_select<true, false>), grid, dim3(256), 0, s, p);
    }
  } else if (topk) {
    hipLaunchKernelGGL((k_logit_select<false, true>), grid, dim3(256), 0, s, p);
    hipLaunchKernelGGL(k_topk_redo<false>, dim3(p.M), dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((k_logit_select<false, false>), grid, dim3(256), 0, s, p);
  }
}

void launch_topk_merge(const TopkParams& p, hipStream_t s) {
  if (p.M <= 0) return;
  hipLaunchKernelGGL(k_topk_merge, dim3(p.M), dim3(64), 0, s, p);
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
