// Sampled drafting and lossless rejection-sampling verification on gfx950
// ([guide] "DFlash：块扩散加速的 LLM 推测解码技术", section 7: the DFlash-2 path
// is walked greedily or by sampling, with rejection sampling keeping the
// output distribution exactly the target's; section 3.3: rejected positions
// are resampled by the target).
//
// Sampling settings warp a row of logits as: divide by the temperature, keep
// the top-k (0: all), softmax, keep the smallest prefix (probability
// descending, then id) whose cumulative probability reaches top-p,
// renormalise.  The draft's distribution q at a block position is the warp
// of its top-16 list; the target's p the warp of its full logits row.  A
// draw with uniform v walks its support in a fixed order (the list order; or
// token ids ascending for the target without top-k) and takes the first
// entry whose running sum exceeds v times the total.  Running sums are
// sequential in that order, as are the sums that normalise them.
//
//  * k_draft_sample: one wave per (request, position), the 16 candidates in
//    16 lanes; draws the drafted token from q.
//  * k_row_chunks, k_row_finish: the target's rows (request, position
//    0..B) in kRowChunks chunks each, then one workgroup per row: without top-k
//    the row's max and sum of exp(L / T - max) (per chunk, merged in chunk
//    order); with top-k the k largest logits (ties to the lower id: keys
//    pack the order-preserving logit bits above the inverted id), as sorted
//    64-entry lists per chunk merged by bitonic networks, then warped.
//  * k_verify_sample: one workgroup per request; its waves form each
//    position's p(x) / q(x), then one thread runs the accept test
//    u < p(x) / q(x) position by position, then the final draw from
//    max(0, p - q) (or p after a full block): over the kept list, or over
//    the whole vocabulary, each wave summing a contiguous id range (the wave
//    totals prefixed in wave order) and the wave whose range holds the
//    threshold walking its 64-id blocks with a prefix over the lanes.
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kMaxTopK = 64;  // target-side top-k limit

// Warp of one 16-candidate list held by lanes 0..15 of a wave (lane j holds
// candidate j, list order): returns this lane's normalised probability (0
// beyond the kept prefix).  Every lane of the wave calls it.
__device__ __forceinline__ float warp16(float logit, int j, const SampleParams& p) {
  const int kd = (p.top_k > 0 && p.top_k < 16) ? p.top_k : 16;
  const bool kept = j < kd;
  const float z = logit / p.temperature;
  float m = kept ? z : -INFINITY;
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float e = kept ? expf(z - m) : 0.f;
  const int base = threadIdx.x & 48;  // first lane of this 16-lane group
  // sums in list order (sequential, as every lane walks lanes 0..15 itself)
  float s = 0.f;
  for (int i = 0; i < 16; ++i) s += __shfl(e, base + i, 64);
  float pr = e / s;
  if (p.top_p < 1.f) {
    float c = 0.f, cut = 0.f;
    int keep = 16;
    for (int i = 0; i < 16; ++i) {
      c += __shfl(pr, base + i, 64);
      if (keep == 16 && c >= p.top_p) keep = i + 1;
    }
    pr = j < keep ? pr : 0.f;
    for (int i = 0; i < 16; ++i) cut += __shfl(pr, base + i, 64);
    pr = pr / cut;
  }
  return pr;
}

// Index of the first lane (0..15) whose running sum of w exceeds v * total.
__device__ __forceinline__ int draw16(float w, float v) {
  const int base = threadIdx.x & 48;
  float tot = 0.f;
  for (int i = 0; i < 16; ++i) tot += __shfl(w, base + i, 64);
  const float thr = v * tot;
  float c = 0.f;
  int pick = -1, last = 0;
  for (int i = 0; i < 16; ++i) {
    const float wi = __shfl(w, base + i, 64);
    c += wi;
    if (wi > 0.f) last = i;
    if (pick < 0 && c > thr) pick = i;
  }
  return pick >= 0 ? pick : last;
}

__global__ __launch_bounds__(1024) void k_draft_sample(SampleParams p) {
  const int req = blockIdx.x;
  const int pos = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (pos >= p.B) return;
  const int j = lane & 15;
  const long long li = ((long long)req * p.B + pos) * 16 + j;
  const float w = warp16(p.dlog[li], j, p);
  const int k = draw16(w, p.v[(long long)req * p.B + pos]);
  if (lane == 0) {
    int t = p.dids[((long long)req * p.B + pos) * 16 + k];
    if (t < 0 || t >= p.vocab) {
      atomicOr(p.err, 1u);
      t = 0;
    }
    p.draft[(long long)req * p.B + pos] = t;
  }
}

// Selection key of logit x at id i: larger logit first, then the lower id.
__device__ __forceinline__ unsigned long long sel_key(float x, int i) {
  return ((unsigned long long)float_key(x) << 32) | (0xffffffffu - (unsigned)i);
}

// A row's result from its chunks', by one wave: the statistics merged in
// chunk order (max, rescaled sums) ...
__device__ void finish_stats(const SampleParams& p, int row, int lane) {
  const float2 st = lane < kRowChunks
                        ? reinterpret_cast<const float2*>(p.chunk_stat)[(long long)row * kRowChunks + lane]
                        : make_float2(-INFINITY, 0.f);
  float m = st.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  const float w = st.x > -INFINITY ? st.y * expf(st.x - m) : 0.f;
  float z = 0.f;
  for (int i = 0; i < kRowChunks; ++i) z += __shfl(w, i, 64);
  if (lane == 0) {
    p.row_stat[2 * row] = m;
    p.row_stat[2 * row + 1] = z;
  }
}

// ... or, given the row's sorted top 64 in the wave's lanes, its first k
// warped (softmax at temperature T, then the shortest prefix whose running
// sum reaches top-p, renormalised).
__device__ void finish_list(const SampleParams& p, int row, int lane, unsigned long long e) {
  const unsigned k = (unsigned)min(p.top_k, p.vocab);
  const bool in = lane < (int)k;
  const int id = (int)(0xffffffffu - (unsigned)(e & 0xffffffffu));
  const float z = in ? key_float((unsigned)(e >> 32)) / p.temperature : -INFINITY;
  const float m = __shfl(z, 0, 64);
  const float ex = in ? expf(z - m) : 0.f;
  float pr = ex / wave_sum(ex);
  int keep = (int)k;
  if (p.top_p < 1.f) {
    float c = pr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float u = __shfl_up(c, o, 64);
      if (lane >= o) c += u;
    }
    const unsigned long long reach = __ballot(in && c >= p.top_p);
    if (reach) keep = __ffsll((long long)reach);  // first such lane, plus one
    pr = lane < keep ? pr : 0.f;
    pr = pr / wave_sum(pr);
  }
  if (lane < keep) {
    p.row_ids[(long long)row * kMaxTopK + lane] = id;
    p.row_p[(long long)row * kMaxTopK + lane] = pr;
  }
  if (lane == 0) p.row_n[row] = keep;
}

// The target's rows: one workgroup of 4 waves per (row chunk, row).  Without
// top-k, the chunk's max of L / T and its sum of exp(L / T - max).  With
// top-k, the chunk's 64 largest keys, sorted: every thread takes the largest
// key of its strided elements, and the 64th largest of those 256 maxima,
// tau, is at most the chunk's 64th largest key (64 threads hold a distinct
// key >= tau), so the keys >= tau (at most 64 x the elements per thread;
// typically under 1 %) are gathered in LDS and sorted in batches of 64
// merged into a sorted list per wave, the four lists merged in wave order.
// A chunk with more candidates than the LDS holds folds in all of its keys
// the same way instead.
constexpr int kCandCap = 2048;
__global__ __launch_bounds__(256) void k_row_chunks(SampleParams p) {
  __shared__ unsigned long long sh_list[4][64];
  __shared__ unsigned long long cand[kCandCap];
  __shared__ unsigned sh_cnt;
  __shared__ float red[4];
  const int row = blockIdx.y * (p.B + 1) + blockIdx.x;  // (request, position)
  const int c = blockIdx.z;
  const int V = p.vocab;
  const int per = (V + kRowChunks - 1) / kRowChunks;
  const int c0 = min(V, c * per), c1 = min(V, c0 + per);
  const float* L = p.tlog + (long long)row * V;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // each thread's elements c0 + t + 256 j, read 8 at a time (loads in flight together)
  auto load8s = [&](int j0, float (&x)[8]) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = c0 + t + 256 * (j0 + q);
      x[q] = i < c1 ? L[i] : 0.f;
    }
  };
  const int nj = (c1 - c0 + 255) / 256;
  if (p.top_k == 0) {
    float m = -INFINITY;
    for (int j0 = 0; j0 < nj; j0 += 8) {
      float x[8];
      load8s(j0, x);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (c0 + t + 256 * (j0 + q) < c1) m = fmaxf(m, x[q] / p.temperature);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    float z = 0.f;
    if (m > -INFINITY)
      for (int j0 = 0; j0 < nj; j0 += 8) {
        float x[8];
        load8s(j0, x);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (c0 + t + 256 * (j0 + q) < c1) z += expf(x[q] / p.temperature - m);
      }
    z = wave_sum(z);
    if (lane == 0) red[wave] = z;
    __syncthreads();
    if (t == 0) {
      p.chunk_stat[((long long)row * kRowChunks + c) * 2] = m;
      p.chunk_stat[((long long)row * kRowChunks + c) * 2 + 1] = red[0] + red[1] + red[2] + red[3];
    }
  } else {
    // the threshold: 64th largest of the per-thread maxima (0 = empty key)
    unsigned long long mk = 0ull;
    for (int j0 = 0; j0 < nj; j0 += 8) {
      float x[8];
      load8s(j0, x);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = c0 + t + 256 * (j0 + q);
        if (i < c1) mk = key_max(mk, sel_key(x[q], i));
      }
    }
    sh_list[wave][lane] = sort64_desc(mk, lane);
    if (t == 0) sh_cnt = 0u;
    __syncthreads();
    if (wave == 0) {
      unsigned long long b = sh_list[0][lane];
      for (int w = 1; w < 4; ++w) b = merge64_desc(b, sh_list[w][lane], lane);
      if (lane == 63) sh_list[0][0] = b;  // tau (lane 0's entry is no longer needed)
    }
    __syncthreads();
    const unsigned long long tau = sh_list[0][0];
    for (int j0 = 0; j0 < nj; j0 += 8) {
      float x[8];
      load8s(j0, x);
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int i = c0 + t + 256 * (j0 + q);
        const unsigned long long k = i < c1 ? sel_key(x[q], i) : 0ull;
        if (i < c1 && k >= tau) {
          const unsigned slot = atomicAdd(&sh_cnt, 1u);
          if (slot < kCandCap) cand[slot] = k;
        }
      }
    }
    __syncthreads();
    const unsigned n = sh_cnt;
    unsigned long long best = 0ull, last = 0ull;
    if (n <= kCandCap) {
      for (unsigned b = wave * 64; b < n; b += 256) {
        unsigned long long k = b + lane < n ? cand[b + lane] : 0ull;
        k = sort64_desc(k, lane);
        best = merge64_desc(best, k, lane);
      }
    } else {
      for (int base = c0 + wave * 64; base < c1; base += 256) {
        const int i = base + lane;
        unsigned long long k = i < c1 ? sel_key(L[i], i) : 0ull;
        if (__ballot(k > last)) {
          k = sort64_desc(k, lane);
          best = merge64_desc(best, k, lane);
          last = __shfl(best, 63, 64);
        }
      }
    }
    __syncthreads();  // every read of sh_list above is done
    if (wave > 0) sh_list[wave][lane] = best;
    __syncthreads();
    if (wave == 0) {
      for (int w = 1; w < 4; ++w) best = merge64_desc(best, sh_list[w][lane], lane);
      p.chunk_list[((long long)row * kRowChunks + c) * 64 + lane] = best;
    }
  }
}

// Second pass, one workgroup of 4 waves per row: the chunks' statistics
// merged by wave 0, or the chunks' lists merged four per wave, then the four
// waves' lists by wave 0, which warps the row's first k entries.
__global__ __launch_bounds__(256) void k_row_finish(SampleParams p) {
  __shared__ unsigned long long sh_list[4][64];
  const int row = blockIdx.y * (p.B + 1) + blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  if (p.top_k == 0) {
    if (wave == 0) finish_stats(p, row, lane);
    return;
  }
  const unsigned long long* cl = p.chunk_list + (long long)row * kRowChunks * 64;
  constexpr int kPerWave = kRowChunks / 4;
  unsigned long long ls[kPerWave];
#pragma unroll
  for (int q = 0; q < kPerWave; ++q) ls[q] = cl[(wave * kPerWave + q) * 64 + lane];
  unsigned long long e = ls[0];
#pragma unroll
  for (int q = 1; q < kPerWave; ++q) e = merge64_desc(e, ls[q], lane);
  sh_list[wave][lane] = e;
  __syncthreads();
  if (wave == 0) {
    for (int w = 1; w < 4; ++w) e = merge64_desc(e, sh_list[w][lane], lane);
    finish_list(p, row, lane, e);
  }
}

__global__ __launch_bounds__(1024) void k_verify_sample(SampleParams p) {
  __shared__ int sh_a, sh_tok, sh_last;
  __shared__ float sh_qall[16][16];  // the draft's warped q per position and list entry
  __shared__ int sh_idall[16][16];
  __shared__ float sh_ratio[16];     // p(x) / q(x) of each position's draft, or -1 when q(x) = 0
  __shared__ float csum[17];
  const int req = blockIdx.x;
  const int t = threadIdx.x, nt = blockDim.x;
  const int lane = t & 63, wave = t >> 6;
  const int B = p.B, V = p.vocab;
  const int row0 = req * (B + 1);
  const float* U = p.u + (long long)req * (B + 1) * 2;
  // Every wave with all of its lanes: for each block position its draft's
  // q(x) and the target's p(x) (the rows were finished by k_row_chunks).
  for (int i = wave; i < B; i += nt / 64) {
    const int j = lane & 15;
    const long long li = ((long long)req * B + i) * 16 + j;
    const float q = warp16(p.dlog[li], j, p);  // every 16-lane group computes the same list
    const int cid = p.dids[li];
    const int x = p.draft[(long long)req * B + i];
    // q(x): the first list entry holding x (group 0's lanes), broadcast to the wave
    unsigned long long hit = __ballot(lane < 16 && cid == x);
    const int first = hit ? __ffsll((long long)hit) - 1 : -1;
    const float qx = first >= 0 ? __shfl(q, first, 64) : 0.f;
    float px;
    const int row = row0 + i;
    if (p.top_k == 0) {
      px = (x >= 0 && x < V) ? expf(p.tlog[(long long)row * V + x] / p.temperature - p.row_stat[2 * row]) /
                                   p.row_stat[2 * row + 1]
                             : 0.f;
    } else {
      const int n = p.row_n[row];
      const bool mine = lane < n && p.row_ids[(long long)row * kMaxTopK + lane] == x;
      const float v = mine ? p.row_p[(long long)row * kMaxTopK + lane] : 0.f;
      px = wave_sum(v);  // at most one lane holds x
    }
    if (lane < 16) {
      sh_qall[i][j] = q;
      sh_idall[i][j] = cid;
    }
    if (lane == 0) sh_ratio[i] = qx > 0.f ? px / qx : -1.f;
  }
  __syncthreads();
  if (t == 0) {  // accept test, position by position: u < p(x) / q(x)
    int a = B;
    for (int i = 0; i < B; ++i) {
      const float ratio = sh_ratio[i];
      if (!(ratio >= 0.f && U[2 * i] < ratio)) {
        a = i;
        break;
      }
    }
    sh_a = a;
    sh_tok = 0;
  }
  __syncthreads();
  const int a = sh_a;
  const int row = row0 + a;
  const float v = U[2 * a + 1];
  auto qof = [&](int tok) {  // the draft's probability of tok at the final position (none after a full block)
    float q = 0.f;
    if (a < B)
      for (int i = 0; i < 16; ++i)
        if (sh_idall[a][i] == tok) {
          q = sh_qall[a][i];
          break;
        }
    return q;
  };
  if (p.top_k > 0) {  // draw from the kept list
    if (wave == 0) {
      const int n = p.row_n[row];
      const bool in = lane < n;
      const int id = in ? p.row_ids[(long long)row * kMaxTopK + lane] : -1;
      const float pr = in ? p.row_p[(long long)row * kMaxTopK + lane] : 0.f;
      float r = in ? fmaxf(0.f, pr - qof(id)) : 0.f;
      float tot = 0.f;
      for (int i = 0; i < n; ++i) tot += __shfl(r, i, 64);
      if (!(tot > 0.f)) {  // p == q on the support: draw from p
        r = pr;
        tot = 0.f;
        for (int i = 0; i < n; ++i) tot += __shfl(r, i, 64);
      }
      const float thr = v * tot;
      float c = 0.f;
      int pick = -1, last = 0;
      for (int i = 0; i < n; ++i) {
        const float ri = __shfl(r, i, 64);
        c += ri;
        if (ri > 0.f) last = i;
        if (pick < 0 && c > thr) pick = i;
      }
      if (pick < 0) pick = last;
      const int tok = __shfl(id, pick, 64);
      if (lane == 0) sh_tok = tok;
    }
  } else {  // draw over the whole vocabulary, ids ascending: wave w owns a contiguous id range
    const float m = p.row_stat[2 * row], z = p.row_stat[2 * row + 1];
    const float* L = p.tlog + (long long)row * V;
    const int nw = nt / 64;
    const int span = (V + nw - 1) / nw;
    const int w0 = min(V, wave * span), w1 = min(V, w0 + span);
    for (int pass = 0; pass < 2; ++pass) {  // pass 1 only when max(0, p - q) vanishes: draw from p
      const bool resid = pass == 0 && a < B;
      auto rval = [&](int i, float x) {
        const float pi = expf(x / p.temperature - m) / z;
        return resid ? fmaxf(0.f, pi - qof(i)) : pi;
      };
      // the wave's total: lane partial sums over its 64-id blocks (4 blocks per round), then the lanes
      float acc = 0.f;
      for (int b = w0; b < w1; b += 256) {
        float x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = b + 64 * q + lane;
          x[q] = i < w1 ? L[i] : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = b + 64 * q + lane;
          if (i < w1) acc += rval(i, x[q]);
        }
      }
      acc = wave_sum(acc);
      if (lane == 0) csum[wave] = acc;
      __syncthreads();
      if (t == 0) {  // wave totals prefixed in wave order
        float run = 0.f;
        int last_nz = 0;
        for (int w = 0; w < nw; ++w) {
          const float c = csum[w];
          if (c > 0.f) last_nz = w;
          csum[w] = run;
          run += c;
        }
        csum[nw] = run;
        sh_last = last_nz;
      }
      __syncthreads();
      const float tot = csum[nw];
      if (tot > 0.f || pass == 1) {
        const float thr = v * tot;
        // the wave whose range holds the threshold walks its blocks in id
        // order; if rounding leaves the threshold at the total (or past the
        // wave's own walk), the last positive id seen is taken
        const float lo = csum[wave];
        const float hi = wave + 1 < nw ? csum[wave + 1] : tot;
        if ((lo <= thr && thr < hi) || (thr >= tot && wave == sh_last)) {
          float run = lo;
          int pick = -1, last = -1;
          for (int b4 = w0; b4 < w1 && pick < 0; b4 += 256) {
            float x[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = b4 + 64 * q + lane;
              x[q] = i < w1 ? L[i] : 0.f;
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int b = b4 + 64 * q;
              if (pick >= 0 || b >= w1) break;
              const int i = b + lane;
              const float r = i < w1 ? rval(i, x[q]) : 0.f;
              // inclusive prefix of r over the lanes, in lane order
              float pre = r;
#pragma unroll
              for (int o = 1; o < 64; o <<= 1) {
                const float u = __shfl_up(pre, o, 64);
                if (lane >= o) pre += u;
              }
              const unsigned long long hit = __ballot(run + pre > thr && r > 0.f);
              const unsigned long long pos = __ballot(r > 0.f);
              if (pos) last = b + 63 - __clzll((long long)pos);
              if (hit) pick = b + __ffsll((long long)hit) - 1;
              run += __shfl(pre, 63, 64);
            }
          }
          if (lane == 0) sh_tok = pick >= 0 ? pick : (last >= 0 ? last : w1 - 1);
        }
        break;
      }
      __syncthreads();
    }
  }
  __syncthreads();
  if (t <= B) {
    const int tok = sh_tok;
    int val = -1;
    if (t < a) val = p.draft[(long long)req * B + t];
    else if (t == a) val = tok;
    p.committed[(long long)req * (B + 1) + t] = val;
    if (t == 0) {
      p.accept[req] = a;
      p.last[req] = tok;
    }
  }
}

}  // namespace

void launch_draft_sample(const SampleParams& p, int n_req, hipStream_t s) {
  if (n_req <= 0) return;
  hipLaunchKernelGGL(k_draft_sample, dim3(n_req), dim3(64 * p.B), 0, s, p);
}

void launch_verify_sample(const SampleParams& p, int n_req, hipStream_t s) {
  if (n_req <= 0) return;
  hipLaunchKernelGGL(k_row_chunks, dim3(p.B + 1, n_req, kRowChunks), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_row_finish, dim3(p.B + 1, n_req), dim3(256), 0, s, p);
  hipLaunchKernelGGL(k_verify_sample, dim3(n_req), dim3(1024), 0, s, p);
}

}  // namespace dflash
