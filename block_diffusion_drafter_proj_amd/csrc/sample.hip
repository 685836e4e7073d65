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
//  * k_target_rows: one workgroup per target row (request, position 0..B):
//    without top-k the row's max and sum of exp(L / T - max) (strided
//    partial sums, then the waves in order); with top-k the k largest
//    logits by a 4-pass 8-bit radix select over order-preserving keys
//    (ties at the k-th key to the lower ids, taken in id order), sorted by a
//    64-lane bitonic network, then warped.
//  * k_verify_sample: one workgroup per request; wave 0 runs the accept test
//    u < p(x) / q(x) position by position, then the final draw from
//    max(0, p - q) (or p after a full block): over the kept list, or over
//    the whole vocabulary in contiguous per-thread id chunks whose sums are
//    prefixed in thread order.
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

// 64 keys, one per lane, sorted descending (bitonic network over the wave).
__device__ __forceinline__ unsigned long long sort64_desc(unsigned long long v, int lane) {
#pragma unroll
  for (int k = 2; k <= 64; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      const unsigned long long o = __shfl_xor(v, j, 64);
      const bool desc = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      v = (lower == desc) ? key_max(v, o) : key_min(v, o);
    }
  }
  return v;
}

__global__ __launch_bounds__(1024) void k_target_rows(SampleParams p) {
  __shared__ unsigned hist[256];
  __shared__ unsigned sh_prefix, sh_mask, sh_need, sh_cnt;
  __shared__ unsigned tie_pre[1024];
  __shared__ unsigned long long list[kMaxTopK];
  __shared__ float red[16];
  const int row = blockIdx.y * (p.B + 1) + blockIdx.x;  // (request, position)
  const float* L = p.tlog + (long long)row * p.vocab;
  const int t = threadIdx.x, nt = blockDim.x;
  const int lane = t & 63, wave = t >> 6;
  const int V = p.vocab;
  if (p.top_k == 0) {  // max and normaliser of exp(L / T - max)
    float m = -INFINITY;
    for (int i = t; i < V; i += nt) m = fmaxf(m, L[i] / p.temperature);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
    for (int w = 1; w < nt / 64; ++w) m = fmaxf(m, red[w]);
    __syncthreads();
    float s = 0.f;
    for (int i = t; i < V; i += nt) s += expf(L[i] / p.temperature - m);
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (t == 0) {
      float z = 0.f;
      for (int w = 0; w < nt / 64; ++w) z += red[w];
      p.row_stat[2 * row] = m;
      p.row_stat[2 * row + 1] = z;
    }
    return;
  }
  // radix select of the k-th largest order-preserving key
  const unsigned k = (unsigned)min(p.top_k, V);
  if (t == 0) {
    sh_prefix = 0u;
    sh_mask = 0u;
    sh_need = k;
  }
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = t; i < 256; i += nt) hist[i] = 0u;
    __syncthreads();
    const unsigned prefix = sh_prefix, mask = sh_mask;
    for (int i = t; i < V; i += nt) {
      const unsigned key = float_key(L[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (t == 0) {
      unsigned cum = 0u, need = sh_need;
      for (int b = 255; b >= 0; --b) {
        if (cum + hist[b] >= need) {
          sh_need = need - cum;  // keys equal so far still to take from this bin
          sh_prefix = prefix | ((unsigned)b << shift);
          sh_mask = mask | (255u << shift);
          break;
        }
        cum += hist[b];
      }
      if (pass == 0) sh_cnt = 0u;
    }
    __syncthreads();
  }
  const unsigned thr = sh_prefix, need_eq = sh_need;  // thr: the k-th key; need_eq of the keys == thr
  // keys above the threshold, in any order (sorted below)
  for (int i = t; i < V; i += nt) {
    const unsigned key = float_key(L[i]);
    if (key > thr) list[atomicAdd(&sh_cnt, 1u)] = ((unsigned long long)key << 32) | (0xffffffffu - (unsigned)i);
  }
  // keys equal to the threshold: the need_eq lowest ids, in contiguous id chunks
  const int chunk = (V + nt - 1) / nt;
  const int c0 = min(V, t * chunk), c1 = min(V, c0 + chunk);
  unsigned ties = 0u;
  for (int i = c0; i < c1; ++i) ties += float_key(L[i]) == thr;
  tie_pre[t] = ties;
  __syncthreads();
  if (t == 0) {
    unsigned run = 0u;
    for (int i = 0; i < nt; ++i) {
      const unsigned c = tie_pre[i];
      tie_pre[i] = run;
      run += c;
    }
  }
  __syncthreads();
  const unsigned gt = k - need_eq;  // entries already in the list
  unsigned taken = tie_pre[t];
  for (int i = c0; i < c1 && taken < need_eq; ++i)
    if (float_key(L[i]) == thr) list[gt + taken++] = ((unsigned long long)thr << 32) | (0xffffffffu - (unsigned)i);
  __syncthreads();
  if (wave != 0) return;
  unsigned long long e = lane < (int)k ? list[lane] : 0ull;
  e = sort64_desc(e, lane);  // logit descending, then id ascending
  const bool in = lane < (int)k;
  const int id = (int)(0xffffffffu - (unsigned)(e & 0xffffffffu));
  const float z = in ? key_float((unsigned)(e >> 32)) / p.temperature : -INFINITY;
  const float m = __shfl(z, 0, 64);
  const float ex = in ? expf(z - m) : 0.f;
  float s = 0.f;
  for (int i = 0; i < (int)k; ++i) s += __shfl(ex, i, 64);
  float pr = ex / s;
  int keep = (int)k;
  if (p.top_p < 1.f) {
    float c = 0.f;
    keep = -1;
    for (int i = 0; i < (int)k; ++i) {
      c += __shfl(pr, i, 64);
      if (keep < 0 && c >= p.top_p) keep = i + 1;
    }
    if (keep < 0) keep = (int)k;
    pr = lane < keep ? pr : 0.f;
    float cut = 0.f;
    for (int i = 0; i < keep; ++i) cut += __shfl(pr, i, 64);
    pr = pr / cut;
  }
  if (lane < keep) {
    p.row_ids[(long long)row * kMaxTopK + lane] = id;
    p.row_p[(long long)row * kMaxTopK + lane] = pr;
  }
  if (lane == 0) p.row_n[row] = keep;
}

__global__ __launch_bounds__(1024) void k_verify_sample(SampleParams p) {
  __shared__ int sh_a, sh_tok, sh_last;
  __shared__ float sh_q[16];
  __shared__ int sh_qid[16];
  __shared__ float csum[1024];
  const int req = blockIdx.x;
  const int t = threadIdx.x, nt = blockDim.x;
  const int lane = t & 63, wave = t >> 6;
  const int B = p.B, V = p.vocab;
  const int row0 = req * (B + 1);
  const float* U = p.u + (long long)req * (B + 1) * 2;
  if (t == 0) sh_tok = 0;
  if (wave == 0) {
    // accept test, position by position
    const int j = lane & 15;
    int a = B;
    for (int i = 0; i < B; ++i) {
      const long long li = ((long long)req * B + i) * 16 + j;
      const float q = warp16(p.dlog[li], j, p);
      const int cid = p.dids[li];
      const int x = p.draft[(long long)req * B + i];
      // q(x): the first list entry holding x
      unsigned long long hit = (lane < 16 && cid == x) ? (1ull << j) : 0ull;
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) hit |= __shfl_xor(hit, o, 64);
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
      if (!(qx > 0.f && U[2 * i] < px / qx)) {
        a = i;
        break;
      }
    }
    if (lane == 0) sh_a = a;
    // the draft's q at the final position (none after a full block)
    if (a < B) {
      const long long li = ((long long)req * B + a) * 16 + j;
      const float q = warp16(p.dlog[li], j, p);
      if (lane < 16) {
        sh_q[j] = q;
        sh_qid[j] = p.dids[li];
      }
    } else if (lane < 16) {
      sh_q[lane] = 0.f;
      sh_qid[lane] = -1;
    }
  }
  __syncthreads();
  const int a = sh_a;
  const int row = row0 + a;
  const float v = U[2 * a + 1];
  auto qof = [&](int tok) {  // the draft's probability of tok at the final position
    float q = 0.f;
    for (int i = 0; i < 16; ++i)
      if (sh_qid[i] == tok) {
        q = sh_q[i];
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
  } else {  // draw over the whole vocabulary, ids ascending, in contiguous per-thread chunks
    const float m = p.row_stat[2 * row], z = p.row_stat[2 * row + 1];
    const float* L = p.tlog + (long long)row * V;
    const int chunk = (V + nt - 1) / nt;
    const int c0 = min(V, t * chunk), c1 = min(V, c0 + chunk);
    for (int pass = 0; pass < 2; ++pass) {  // pass 1 only when max(0, p - q) vanishes: draw from p
      const bool resid = pass == 0 && a < B;
      float s = 0.f;
      for (int i = c0; i < c1; ++i) {
        const float pi = expf(L[i] / p.temperature - m) / z;
        s += resid ? fmaxf(0.f, pi - qof(i)) : pi;
      }
      csum[t] = s;
      __syncthreads();
      if (t == 0) {  // chunk sums prefixed in thread order
        float run = 0.f;
        int last_nz = 0;
        for (int i = 0; i < nt; ++i) {
          const float c = csum[i];
          if (c > 0.f) last_nz = i;
          csum[i] = run;
          run += c;
        }
        sh_a = __float_as_int(run);  // total (a is kept in a register)
        sh_last = last_nz;
      }
      __syncthreads();
      const float tot = __int_as_float(sh_a);
      if (tot > 0.f || pass == 1) {
        const float thr = v * tot;
        // the chunk whose range holds the threshold walks its ids; if rounding
        // leaves the threshold at the total, the last chunk with mass takes
        // its last positive id
        const float lo = csum[t];
        const float hi = t + 1 < nt ? csum[t + 1] : tot;
        if ((lo <= thr && thr < hi) || (thr >= tot && t == sh_last)) {
          float c = lo;
          int pick = -1, last = -1;
          for (int i = c0; i < c1; ++i) {
            const float pi = expf(L[i] / p.temperature - m) / z;
            const float ri = resid ? fmaxf(0.f, pi - qof(i)) : pi;
            c += ri;
            if (ri > 0.f) last = i;
            if (pick < 0 && c > thr) pick = i;
          }
          sh_tok = pick >= 0 ? pick : (last >= 0 ? last : c1 - 1);
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
  hipLaunchKernelGGL(k_target_rows, dim3(p.B + 1, n_req), dim3(1024), 0, s, p);
  hipLaunchKernelGGL(k_verify_sample, dim3(n_req), dim3(1024), 0, s, p);
}

}  // namespace dflash
