// Draft attention over the injected context KV and the block's own KV.
//
// Each of the B block rows attends to every visible context position of its
// request and to all B block rows, itself included: attention inside the
// block is bidirectional ([guide] section 3.1, the block is drafted in one
// forward) and the context K/V are those written from the target's features
// ([guide] section 3.2).  Query head j reads KV head j / (Hq / Hkv) (GQA);
// scores are scaled by 1/sqrt(dh).
//
// Layout: a KV page holds 16 positions of one layer as [K | V] x Hkv heads;
// K is stored [16 positions][dh] and V transposed, [dh][16 positions], so
// that both MFMA products read their reduction dimension contiguously.
//
// k_qkv_post   RoPE on the block's q and k at positions n .. n+B-1, rounding
//              to the storage dtype; q to [req][Hq][16][dh], block k/v to one
//              extra page per request (rows >= B zero).
// k_attn       split-K over pages (flash-decoding): a workgroup takes one
//              request, one KV head and a run of pages; each wave owns one
//              query head of the group and its 16 query rows.  S^T = K Q^T and
//              O^T = V^T P^T run on 16x16 MFMA tiles, 32 keys per step, with
//              an online softmax per query row (fp32; P enters the bf16 MFMA
//              as an exact hi + lo pair).  Invalid keys (past ctx_len,
//              before the window, block rows >= B) get probability 0 and their
//              V is zeroed, so stale or poisoned page contents never leak in.
//              Each workgroup holds the G query heads of one KV head times KQ
//              key subsets (up to 8 waves); the subsets are merged in LDS
//              in a fixed order and the split's (max, sum, O) goes to global
//              memory (with a single split the output is written directly).
// k_combine    merges the splits of every (request, head, row) in split order.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

template <typename T> constexpr bool kSplitP = sizeof(T) == 2;  // bf16: P as hi + lo

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };

// One workgroup of 256 threads per (request, head).  q and k heads: a thread
// takes one block row and four consecutive rotate-half pairs (columns j..j+3
// and their partners j+dh/2..), so every partial, cos and sin read is 16
// bytes; V heads: a thread takes one row and dh/16 consecutive dims, written
// transposed.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_qkv_post(QkvPostParams p, SlotArgs sl) {
  const int r = blockIdx.x;
  const int hh = blockIdx.y;
  const int t = threadIdx.x;
  const int ld = (p.Hq + 2 * p.Hkv) * DH;
  const int n = p.state[sl.slots[r]].ctx_len + 1;
  const float* src = p.qkv + (long long)r * p.B * ld + hh * DH;
  const long long plane = (long long)gridDim.x * p.B * ld;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  // sums of the split-K partials of 4 columns at two offsets, in part order;
  // every load of a chunk of 4 parts is issued before any is added
  auto rd2 = [&](long long off1, long long off2, f32x4& x1, f32x4& x2) {
    x1 = zero;
    x2 = zero;
    for (int q0 = 0; q0 < p.n_part; q0 += 4) {
      f32x4 a[4], b[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const bool ok = q0 + q < p.n_part;
        a[q] = ok ? *reinterpret_cast<const f32x4*>(src + (q0 + q) * plane + off1) : zero;
        b[q] = ok ? *reinterpret_cast<const f32x4*>(src + (q0 + q) * plane + off2) : zero;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (q0 + q < p.n_part) {
          x1 += a[q];
          x2 += b[q];
        }
      }
    }
  };
  auto st4 = [](T* d, f32x4 v) {
    typename Vec4<T>::type o;
#pragma unroll
    for (int k = 0; k < 4; ++k) o[k] = from_f<T>(v[k]);
    *reinterpret_cast<typename Vec4<T>::type*>(d) = o;
  };
  constexpr int H2 = DH / 2, QUADS = H2 / 4;
  const long long page_elems = 2LL * p.Hkv * 16 * DH;
  if (hh < p.Hq + p.Hkv) {
    T* dst;
    if (hh < p.Hq)
      dst = reinterpret_cast<T*>(p.qb) + (long long)(r * p.Hq + hh) * 16 * DH;
    else
      dst = reinterpret_cast<T*>(p.blk) + r * page_elems + (long long)(hh - p.Hq) * 16 * DH;
    for (int e = t; e < 16 * QUADS; e += blockDim.x) {
      const int i = e / QUADS;
      const int j = (e - i * QUADS) * 4;
      f32x4 y1 = zero, y2 = zero;
      if (i < p.B) {
        f32x4 x1, x2;
        rd2((long long)i * ld + j, (long long)i * ld + j + H2, x1, x2);
        const long long ti = (long long)(n + i) * H2 + j;
        const f32x4 c = *reinterpret_cast<const f32x4*>(p.cos_t + ti);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(p.sin_t + ti);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          y1[k] = x1[k] * c[k] - x2[k] * sn[k];
          y2[k] = x2[k] * c[k] + x1[k] * sn[k];
        }
      }
      st4(dst + i * DH + j, y1);
      st4(dst + i * DH + j + H2, y2);
    }
  } else {
    constexpr int DPT = DH / 16;  // dims per thread
    const int g = hh - p.Hq - p.Hkv;
    T* dst = reinterpret_cast<T*>(p.blk) + r * page_elems + (long long)(p.Hkv + g) * 16 * DH;
    const int i = t & 15;
    const int d0 = (t >> 4) * DPT;
    f32x4 x1 = zero, x2 = zero;
    if (i < p.B) rd2((long long)i * ld + d0, (long long)i * ld + d0 + (DPT > 4 ? 4 : 0), x1, x2);
#pragma unroll
    for (int k = 0; k < DPT; ++k) dst[(d0 + k) * 16 + i] = from_f<T>(k < 4 ? x1[k] : x2[k - 4]);
  }
}

template <typename T, int DH>
__global__ __launch_bounds__(512) void k_attn(AttnParams p, SlotArgs sl) {
  typedef typename Frag8<T>::type Frag;
  typedef typename Vec4<T>::type V4;
  constexpr int NJ = DH / 32;
  constexpr int ND = DH / 16;
  const float NEG = -INFINITY;
  extern __shared__ float smem[];

  const int gkv = blockIdx.x;
  const int s = blockIdx.y;
  const int r = blockIdx.z;
  const int G = p.Hq / p.Hkv;
  const int KQ = p.KQ;
  const int S = p.n_splits;  // partial-buffer stride (splits of the longest request)
  const int wave = threadIdx.x >> 6;
  const int wq = wave % G;  // query head within the group
  const int kq = wave / G;  // key subset
  const int h = gkv * G + wq;
  const int lane = lane_id();
  const int l16 = lane & 15;
  const int g4 = lane >> 4;
  const int slot = sl.slots[r];
  const SlotState st = p.state[slot];
  const int hi = st.ctx_len;
  int lo = st.kv_begin;
  if (p.window > 0) lo = max(lo, hi - p.window);
  const int lp0 = lo / 16;
  const int n_lp = hi > lo ? (hi - 1) / 16 - lp0 + 1 : 0;
  const int n_units = n_lp + 1;
  const int pps = split_pages(n_units, p.split_target, p.pps_cap);
  const int n_split = (n_units + pps - 1) / pps;
  if (s == 0 && gkv == 0 && threadIdx.x == 0) p.n_split[r] = n_split;
  if (s >= n_split) return;
  const int u_begin = s * pps;
  const int u_end = min(u_begin + pps, n_units);
  const long long page_elems = 2LL * p.Hkv * 16 * DH;
  const T* pool = reinterpret_cast<const T*>(p.pool);
  const T* blk = reinterpret_cast<const T*>(p.blk);

  Frag qf[NJ];
  {
    const T* qrow = reinterpret_cast<const T*>(p.qb) + ((long long)(r * p.Hq + h) * 16 + l16) * DH;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qf[j] = load8<T>(qrow + 32 * j + 8 * g4);
  }

  float m_run = NEG, l_run = 0.f;
  f32x4 o[ND];
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // page ids of the split's context units, one per lane (pps <= 64)
  int my_page = -1;
  {
    const int uu = u_begin + lane;
    if (uu < u_end && uu < n_lp) {
      const int lp = lp0 + uu;
      const int idx = p.window > 0 ? lp % st.n_pages : lp;
      my_page = p.page_table[(long long)slot * p.pt_stride + idx];
      if (my_page < 0 || my_page >= p.max_pages) {
        atomicOr(p.err, 2u);
        my_page = -1;
      }
    }
  }
  auto unit_base = [&](int uu, int& pos0, bool& is_blk) -> const T* {
    pos0 = 0;
    is_blk = false;
    if (uu >= u_end) return nullptr;
    if (uu < n_lp) {
      const int page = __shfl(my_page, uu - u_begin, 64);
      pos0 = (lp0 + uu) * 16;
      return page >= 0 ? pool + (long long)page * page_elems : nullptr;
    }
    is_blk = true;
    return blk + (long long)r * page_elems;
  };

  // pairs of units (32 keys); key subset kq takes every KQ-th pair of the
  // split; the K/V fragments of the next pair are loaded while the current
  // one is multiplied
  Frag kf[2][NJ], kn[2][NJ];
  V4 vv[2][ND], vn[2][ND];
  auto load_pair = [&](int u, Frag (&kd)[2][NJ], V4 (&vd)[2][ND]) {
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int pos0;
      bool is_blk;
      const T* b = unit_base(u + t, pos0, is_blk);
      if (b) {
        const T* kb = b + (long long)gkv * 16 * DH + l16 * DH + 8 * g4;
        const T* vb = b + (long long)(p.Hkv + gkv) * 16 * DH + l16 * 16 + 4 * g4;
#pragma unroll
        for (int j = 0; j < NJ; ++j) kd[t][j] = load8<T>(kb + 32 * j);
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vd[t][dt] = *reinterpret_cast<const V4*>(vb + dt * 256);
      }
    }
  };
  int u = u_begin + 2 * kq;
  if (u < u_end) load_pair(u, kf, vv);
  for (; u < u_end; u += 2 * KQ) {
    const bool more = u + 2 * KQ < u_end;
    if (more) load_pair(u + 2 * KQ, kn, vn);
    const T* base[2];
    bool valid[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      int pos0;
      bool is_blk;
      base[t] = unit_base(u + t, pos0, is_blk);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 4 * g4 + i;
        valid[t][i] = base[t] != nullptr &&
                      (is_blk ? key < p.B : (pos0 + key >= lo && pos0 + key < hi));
      }
    }

    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (base[t]) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) sacc = mfma_step(kf[t][j], qf[j], sacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * t + i] = valid[t][i] ? sacc[i] * p.scale : NEG;
    }
    float mx = sv[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float corr = (m_run == NEG) ? 0.f : expf(m_run - m_new);
    float pe[8];
    float ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pe[e] = (sv[e] == NEG) ? 0.f : expf(sv[e] - m_new);
      ls += pe[e];
    }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * corr + ls;
    m_run = m_new;
    // P enters the PV product at fp32 accuracy: for bf16 storage it is split
    // into hi + lo bf16 parts (two MFMAs); rounding P itself to bf16 would add
    // 2^-9 relative noise per key, which the near-cancelling average over many
    // keys amplifies.
    Frag pf, pf_lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pf[e] = from_f<T>(pe[e]);
      pf_lo[e] = from_f<T>(pe[e] - to_f(pf[e]));
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      o[dt] = o[dt] * corr;
      Frag vf;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) vf[4 * t + i] = valid[t][i] ? vv[t][dt][i] : (T)0.0f;
      o[dt] = mfma_step(vf, pf, o[dt]);
      if (kSplitP<T>) o[dt] = mfma_step(vf, pf_lo, o[dt]);
    }
    if (more) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) kf[t][j] = kn[t][j];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) vv[t][dt] = vn[t][dt];
      }
    }
  }

  // ---- merge the KQ key subsets of each query head (LDS, fixed order) ----
  float* acc = smem;                       // [G][16][DH]
  float* sml = smem + G * 16 * DH;         // [KQ][G][16][2]
  float Mq = m_run, Lq = l_run;
  if (KQ > 1) {
    if (g4 == 0) {
      sml[((kq * G + wq) * 16 + l16) * 2 + 0] = m_run;
      sml[((kq * G + wq) * 16 + l16) * 2 + 1] = l_run;
    }
    __syncthreads();
    Mq = NEG;
    for (int kk = 0; kk < KQ; ++kk) Mq = fmaxf(Mq, sml[((kk * G + wq) * 16 + l16) * 2]);
    Lq = 0.f;
    for (int kk = 0; kk < KQ; ++kk) {
      const float mk = sml[((kk * G + wq) * 16 + l16) * 2];
      if (mk != NEG) Lq += sml[((kk * G + wq) * 16 + l16) * 2 + 1] * expf(mk - Mq);
    }
    const float f = (m_run == NEG) ? 0.f : expf(m_run - Mq);
    float* a = acc + (wq * 16 + l16) * DH + 4 * g4;
    for (int kk = 0; kk < KQ; ++kk) {
      if (kq == kk) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) a[16 * dt + i] = (kk ? a[16 * dt + i] : 0.f) + f * o[dt][i];
      }
      __syncthreads();
    }
  } else {
    float* a = acc + (wq * 16 + l16) * DH + 4 * g4;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[16 * dt + i] = o[dt][i];
    __syncthreads();
  }
  // (Mq, Lq) of (wq, l16) live in the lanes of every key-subset wave; acc holds O

  T* out = reinterpret_cast<T*>(p.out);
  const int nel = G * 16 * DH;
  if (n_split == 1) {
    float* wts = sml + KQ * G * 16 * 2;  // [G][16]: 1 / L
    if (kq == 0 && g4 == 0) wts[wq * 16 + l16] = 1.0f / Lq;
    __syncthreads();
    for (int e = threadIdx.x; e < nel; e += blockDim.x) {
      const int w2 = e / (16 * DH), q = (e / DH) & 15, d = e % DH;
      if (q < p.B)
        out[(long long)(r * p.B + q) * p.ldo + (gkv * G + w2) * DH + d] = from_f<T>(acc[e] * wts[w2 * 16 + q]);
    }
    return;
  }

  // ---- split partial to global; k_combine merges the splits ----
  if (kq == 0 && g4 == 0) {
    const long long pb = ((long long)(r * p.Hq + h) * S + s) * 16 + l16;
    p.part_ml[pb * 2 + 0] = Mq;
    p.part_ml[pb * 2 + 1] = Lq;
  }
  for (int e = threadIdx.x; e < nel; e += blockDim.x) {
    const int w2 = e / (16 * DH), rem = e % (16 * DH);
    p.part_o[((long long)(r * p.Hq + gkv * G + w2) * S + s) * 16 * DH + rem] = acc[e];
  }
}

// bf16 attention with the split's K/V streamed through an LDS ring.
//
// A workgroup takes one request, one KV head and a run of context units
// (pages, then the block's own page).  Wave w computes query head gkv*G + w
// over every key of the run, so each K/V byte comes from HBM once per
// workgroup and the G waves read it from LDS.  Units are staged in pairs (32
// keys, one MFMA reduction step) by direct global->LDS copies, kRing pairs
// deep; every wave makes the same number of copies per stage (a wave with
// nothing left repeats another wave's copy), so the per-wave count of
// outstanding copies fixes how far each wait lets the ring run ahead.  A
// missing unit is copied from the request's block page and fully masked.
// A stage holds the pair's K and V already in MFMA fragment order (each 1 KB
// fragment is lane-major, so every LDS read is a sequential 16-byte-per-lane
// read with no bank conflict); the copies gather the 16 bytes each lane needs.
// Inside the pair, keys are ordered so that both products gather whole
// 16-byte pieces: row 4g+i of score tile t is unit g/2, position
// 8(g%2)+4t+i.  Then a lane of group g holds, across its two score tiles,
// exactly the 8 keys that its PV operand spans (unit g/2, positions
// 8(g%2)..+7: one contiguous 16-byte piece of a V^T row), so P never moves
// between lanes.
constexpr int kRing = 4;

template <int DH, int G>
__global__ __launch_bounds__(64 * G) void k_attn_ring(AttnParams p, SlotArgs sl) {
  constexpr int NJ = DH / 32;             // k32 steps of S^T = K Q^T
  constexpr int ND = DH / 16;             // 16-row tiles of O^T
  constexpr int HEAD = 16 * DH;           // elements of one head's K (or V) in a unit
  constexpr int NCOPY = 2 * NJ + ND;      // fragments per stage: K (2 tiles x NJ), V (ND)
  constexpr int NI = (NCOPY + G - 1) / G; // copies per wave and stage
  constexpr int STAGE = NCOPY * 512;      // elements per stage
  static_assert((kRing - 2) * NI < 64 && NCOPY >= G, "ring shape");
  __shared__ __attribute__((aligned(1024))) bf16 ring[kRing * STAGE];
  const float NEG = -INFINITY;

  // r: the request, or in causal mode the (request, tile) pair
  const int gkv = blockIdx.x, s = blockIdx.y, r = blockIdx.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = gkv * G + wave;
  const int lane = lane_id(), l16 = lane & 15, g4 = lane >> 4;
  const bool causal = p.causal_R > 0;
  const int req = causal ? r / p.n_tiles : r;
  const int slot = sl.slots[req];
  const SlotState st = p.state[slot];
  // causal: the tile's rows sit at positions cpos .. cpos + 15 (capped at the
  // last new row); a key is visible to every row of the tile up to cpos
  const int cpos = causal ? st.ctx_len - p.causal_R + (r - req * p.n_tiles) * 16 : 0;
  const int hi = causal ? min(st.ctx_len, cpos + 16) : st.ctx_len;
  const int hi_all = causal ? cpos + 1 : hi;
  int lo = st.kv_begin;
  if (p.window > 0) lo = max(lo, hi - p.window);
  const int lp0 = lo / 16;
  const int n_lp = hi > lo ? (hi - 1) / 16 - lp0 + 1 : 0;
  const int n_units = causal ? n_lp : n_lp + 1;
  const int pps = split_pages(n_units, p.split_target, p.pps_cap);
  const int n_split = (n_units + pps - 1) / pps;
  if (s == 0 && gkv == 0 && threadIdx.x == 0) p.n_split[r] = n_split;
  if (s >= n_split) return;
  const int u_begin = s * pps;
  const int u_end = min(u_begin + pps, n_units);
  const int n_pairs = (u_end - u_begin + 1) / 2;
  const long long page_elems = 2LL * p.Hkv * 16 * DH;
  const bf16* pool = reinterpret_cast<const bf16*>(p.pool);
  const bf16* blk = reinterpret_cast<const bf16*>(p.blk) + (long long)req * page_elems;  // per request

  bf16x8 qf[NJ];
  {
    const bf16* qrow = reinterpret_cast<const bf16*>(p.qb) + ((long long)(r * p.Hq + h) * 16 + l16) * DH;
#pragma unroll
    for (int j = 0; j < NJ; ++j) qf[j] = load8<bf16>(qrow + 32 * j + 8 * g4);
  }
  // Per-unit tables, lane L describing unit u_begin + L of the split (pps <=
  // 64): its base (the block page stands in for a missing unit, whose keys
  // are masked) and its visible positions as a 16-bit mask.
  // In causal mode a missing unit (odd count) also reads the block page,
  // which is allocated and masked.
  const bf16* my_base = blk;
  unsigned my_vis = 0, my_vis_all = 0;
  {
    const int uu = u_begin + lane;
    if (uu < u_end) {
      if (uu < n_lp) {
        const int lp = lp0 + uu;
        const int idx = p.window > 0 ? lp % st.n_pages : lp;
        const int page = p.page_table[(long long)slot * p.pt_stride + idx];
        if (page < 0 || page >= p.max_pages) {
          atomicOr(p.err, 2u);
        } else {
          my_base = pool + (long long)page * page_elems;
          const int pos0 = lp * 16;
          const int a0 = max(lo - pos0, 0), a1 = min(hi - pos0, 16);
          my_vis = a1 > a0 ? ((1u << a1) - 1u) & ~((1u << a0) - 1u) : 0u;
          const int a2 = min(hi_all - pos0, 16);
          my_vis_all = a2 > a0 ? ((1u << a2) - 1u) & ~((1u << a0) - 1u) : 0u;
        }
      } else {
        my_vis = my_vis_all = (1u << p.B) - 1u;
      }
    }
  }
  // units whose 16 positions are visible to every row: those pairs skip masking
  const unsigned long long full_mask = __ballot(my_vis_all == 0xffffu);
  const unsigned long long base_lo = reinterpret_cast<unsigned long long>(my_base);
  const unsigned b_lo32 = (unsigned)base_lo, b_hi32 = (unsigned)(base_lo >> 32);
  auto unit_ptr = [&](int lane_idx) -> const bf16* {
    const unsigned long long lo32 = (unsigned)__builtin_amdgcn_readlane((int)b_lo32, lane_idx);
    const unsigned long long hi32 = (unsigned)__builtin_amdgcn_readlane((int)b_hi32, lane_idx);
    return reinterpret_cast<const bf16*>(lo32 | (hi32 << 32));
  };
  // this wave's copies: fragment q of the stage is K fragment (tile q / NJ,
  // k step q % NJ) for q < 2 NJ, else V fragment q - 2 NJ; per lane, the unit
  // (0 or 1 of the pair) and the element offset inside it of its 16 bytes
  int c_src[NI], c_dst[NI];
  bool c_u1[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    int q = wave + G * i;
    if (q >= NCOPY) q -= NCOPY;  // nothing left: repeat another wave's copy
    const int fr = lane & 15, fc = lane >> 4;  // fragment row and 8-element column group
    if (q < 2 * NJ) {  // K: row fr of tile t = key (unit g/2, position 8(g%2)+4t+i), g = fr/4, i = fr%4
      const int t = q / NJ, j = q % NJ, gg = fr >> 2;
      c_u1[i] = gg >= 2;
      c_src[i] = gkv * HEAD + (8 * (gg & 1) + 4 * t + (fr & 3)) * DH + 32 * j + 8 * fc;
    } else {  // V^T: dh row dt*16 + fr, keys 8(fc%2)..+7 of unit fc/2
      const int dt = q - 2 * NJ;
      c_u1[i] = fc >= 2;
      c_src[i] = (p.Hkv + gkv) * HEAD + (dt * 16 + fr) * 16 + 8 * (fc & 1);
    }
    c_dst[i] = q * 512;
  }
  auto issue = [&](int pair, int buf) {
    const bf16* b0 = unit_ptr(2 * pair);
    const bf16* b1 = unit_ptr(2 * pair + 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16((c_u1[i] ? b1 : b0) + c_src[i], ring + buf * STAGE + c_dst[i]);
  };

  // Softmax in log2 units with a lazily raised reference max: p = 2^(s*c - m)
  // with c = scale*log2(e).  The reference m of a query is only raised when
  // one of its scores exceeds it by more than 8 (so p <= 2^8, exact in fp32
  // and in the hi + lo bf16 pair); each lane checks its own scores and the
  // cross-lane reduction and rescale of O run only when some lane of the wave
  // needs it, which after the first pair of a long context is rare.  Softmax
  // does not depend on the reference.  m starts at a finite -1e30, so a
  // masked score (-inf) gives p = 2^-inf = 0 with no select, and the first
  // visible score always raises it (the rescale factor 2^(-1e30 - m) is 0).
  // The row sums l come from the matrix cores: a tile of ones joins the PV
  // product as a ninth O tile.
  const float sl2 = p.scale * 1.44269504088896341f;
  float m_run = -1e30f;
  f32x4 o[ND], o_l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (bf16)1.0f;

  // The first kRing - 1 passes only start copies.  With the copies started
  // before the loop instead, the compiler waited for all of them at the loop
  // entry (it cannot see that the ring's own waits cover them); the empty asm
  // keeps the start count opaque so those passes are not peeled back out.
  int it0 = 1 - kRing;
  asm volatile("" : "+s"(it0));
  for (int it = it0; it < n_pairs; ++it) {
    if (it >= 0) wait_ring<NI, kRing - 2>(n_pairs - 1 - it);
    if (it + kRing - 1 < n_pairs) issue(it + kRing - 1, (it + kRing - 1 + kRing) % kRing);
    if (it < 0) continue;
    const bf16* sb = ring + (it % kRing) * STAGE;
    const bool fast = ((full_mask >> (2 * it)) & 3ull) == 3ull;

    // score tiles: sv[4t+i] of a lane in group g4 is key (unit g4/2, position 8(g4%2)+4t+i)
    float sv[8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(sb + (t * NJ + j) * 512 + lane * 8);
        sacc = mfma_step(kf, qf[j], sacc);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[4 * t + i] = sacc[i];
    }
    // Partly visible pair: the lane's 8 keys are bits 8(g4%2)..+7 of its
    // unit's visibility mask.  Masking is written as selects: a divergent
    // branch that stored into one element of the score vector lost that store
    // in code generation.
    // In causal mode a key is further hidden from the query rows before it.
    unsigned vbits = 0xffu;
    if (!fast) {
      const unsigned m0 = __builtin_amdgcn_readlane(my_vis, 2 * it);
      const unsigned m1 = __builtin_amdgcn_readlane(my_vis, 2 * it + 1);
      vbits = (((g4 >> 1) ? m1 : m0) >> (8 * (g4 & 1))) & 0xffu;
      unsigned pbits = vbits;
      if (causal) {
        // key e of this lane: position 16 (lp0 + unit) + 8 (g4 % 2) + e
        const int k0 = 16 * (lp0 + u_begin + 2 * it + (g4 >> 1)) + 8 * (g4 & 1);
        const int lim = cpos + l16 - k0;  // keys e <= lim are at or before this row
        pbits &= lim >= 7 ? 0xffu : lim < 0 ? 0u : (2u << lim) - 1u;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = ((pbits >> e) & 1u) ? sv[e] : NEG;
    }
    float lmx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    if (__ballot(lmx * sl2 > m_run + 8.0f)) {  // false for a lane whose keys are all masked
      float mx = fmaxf(lmx, __shfl_xor(lmx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * sl2;  // the query's max in log2 units
      const float m_new = mx > m_run + 8.0f ? mx : m_run;
      const float corr = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) o[dt] = o[dt] * corr;
      o_l = o_l * corr;
      m_run = m_new;
    }
    float pe[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pe[e] = __builtin_amdgcn_exp2f(fmaf(sv[e], sl2, -m_run));
    // P at fp32 accuracy in the bf16 MFMA: an exact hi + lo pair (the hi
    // halves are widened back to fp32 by moving their bits, not converted)
    bf16x8 pf, pf_lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) pf[e] = (bf16)pe[e];
    {
      const u32x4 w = __builtin_bit_cast(u32x4, pf);
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        pf_lo[2 * k] = (bf16)(pe[2 * k] - __uint_as_float(w[k] << 16));
        pf_lo[2 * k + 1] = (bf16)(pe[2 * k + 1] - __uint_as_float(w[k] & 0xffff0000u));
      }
    }
    o_l = mfma_step(ones, pf, o_l);
    o_l = mfma_step(ones, pf_lo, o_l);
    // V of masked keys is zeroed too: a stale or unwritten position may hold
    // a non-finite pattern, and 0 * inf would poison O
    u32x4 vkeep = u32x4{~0u, ~0u, ~0u, ~0u};
    if (!fast) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        vkeep[k] = (((vbits >> (2 * k)) & 1u) ? 0xffffu : 0u) | (((vbits >> (2 * k + 1)) & 1u) ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
      u32x4 vr = *reinterpret_cast<const u32x4*>(sb + (2 * NJ + dt) * 512 + lane * 8);
      if (!fast) vr &= vkeep;
      const bf16x8 vf = __builtin_bit_cast(bf16x8, vr);
      o[dt] = mfma_step(vf, pf, o[dt]);
      o[dt] = mfma_step(vf, pf_lo, o[dt]);
    }
  }
  const float l_run = o_l[0];  // every row of the ones tile holds the query's sum

  // lane holds query row l16, dims dt*16 + 4*g4 + i
  if (n_split == 1) {
    int m;
    if (attn_out_row(p.causal_R, p.n_tiles, p.B, r, l16, m)) {
      const float inv = 1.0f / l_run;
      bf16* out = reinterpret_cast<bf16*>(p.out);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = (bf16)(o[dt][i] * inv);
        const int k = h * DH + 4 * g4 + dt * 16;
        *reinterpret_cast<bf16x4*>(out + (p.out_packed ? frag_index(m, k, p.ldo) : (long long)m * p.ldo + k)) = v;
      }
    }
    return;
  }
  // split partial; the merge works in natural-log units
  const long long pb = ((long long)(r * p.Hq + h) * p.n_splits + s) * 16 + l16;
  if (g4 == 0) {
    p.part_ml[pb * 2 + 0] = l_run > 0.f ? m_run * 0.693147180559945309f : NEG;
    p.part_ml[pb * 2 + 1] = l_run;
  }
  // The wave's 16 rows of O are contiguous in part_o: staged through the
  // (now idle) ring, rows padded by 4 floats against bank conflicts where
  // that fits, so that each store writes 1 KB of whole lines instead of 64
  // bytes of each of 16 rows.
  constexpr int LDO = G * 16 * (DH + 4) * 4 <= kRing * STAGE * 2 ? DH + 4 : DH;
  __syncthreads();  // every wave is done with the ring
  float* stg = reinterpret_cast<float*>(ring) + wave * 16 * LDO;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) *reinterpret_cast<f32x4*>(stg + l16 * LDO + dt * 16 + 4 * g4) = o[dt];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float* po = p.part_o + (pb - l16) * DH;
#pragma unroll
  for (int k = 0; k < 16 * DH / 256; ++k) {
    const int e = k * 256 + lane * 4;  // element of the wave's block, row e / DH
    *reinterpret_cast<f32x4*>(po + e) = *reinterpret_cast<const f32x4*>(stg + (e / DH) * LDO + e % DH);
  }
}

// One wave per (request, query head, block row): the split partials of the
// row are merged in split order (max, rescaled sums), each lane owning DH/64
// output columns, so every partial is read once and all loads of a lane are
// independent.
template <typename T, int DH>
__global__ __launch_bounds__(256) void k_combine(CombineParams p) {
  constexpr int C = DH / 64;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  const int q = wid % 16;
  const int rh = wid / 16;  // r * Hq + h
  if (rh >= p.n_rh || q >= p.B) return;
  const int r = rh / p.Hq, h = rh - r * p.Hq;
  int m;
  if (!attn_out_row(p.causal_R, p.n_tiles, p.B, r, q, m)) return;
  const int S = p.n_splits;
  const int ns = p.n_split[r];
  const long long pb = (long long)rh * S * 16 + q;
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + pb;
  const float* po = p.part_o + pb * DH + lane * C;
  // lane s holds split s's (max, sum); weights are broadcast by shuffles.  The
  // pairs and the first 16 partial rows are requested together with the
  // split count (bounded by the allocated count S, which needs no load), so
  // the merge waits for one memory round trip; entries past the request's
  // own count are masked once it arrives.
  const float2 raw = lane < S ? ml[lane * 16] : make_float2(-INFINITY, 0.f);
  float v[16][C];
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int c = 0; c < C; ++c) v[k][c] = k < S ? po[(long long)k * 16 * DH + c] : 0.f;
  if (ns <= 1) return;  // written by the attention kernel
  const float2 mine = lane < ns ? raw : make_float2(-INFINITY, 0.f);
  float mx = mine.x;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float w_mine = mine.x == -INFINITY ? 0.f : expf(mine.x - mx);
  float L = 0.f;
  for (int s = 0; s < ns; ++s) L += __shfl(mine.y, s, 64) * __shfl(w_mine, s, 64);
  float acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.f;
  for (int s0 = 0; s0 < ns; s0 += 16) {
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
#pragma unroll
        for (int c = 0; c < C; ++c) v[k][c] = s0 + k < ns ? po[(long long)(s0 + k) * 16 * DH + c] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float w = __shfl(w_mine, (s0 + k) & 63, 64);
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (s0 + k < ns) acc[c] += w * v[k][c];
    }
  }
  const float inv = 1.0f / L;
  const int k = h * DH + lane * C;  // C consecutive k stay contiguous
  T* out = reinterpret_cast<T*>(p.out) + (p.out_packed ? frag_index(m, k, p.ldo) : (long long)m * p.ldo + k);
#pragma unroll
  for (int c = 0; c < C; ++c) out[c] = from_f<T>(acc[c] * inv);
}

// The same merge with two rows per wave (lanes 0-31 row q, lanes 32-63 row
// q + 1 of the same request and head) and 4 consecutive output columns per
// lane, so every partial read is 16 bytes; a half-wave holds the (max, sum)
// of up to 32 splits.  Each output element sees the same operations in the
// same order as in k_combine.
template <typename T>
__global__ __launch_bounds__(256) void k_combine2(CombineParams p) {
  constexpr int DH = 128;
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = lane_id();
  const int half = lane >> 5, hl = lane & 31;
  const int q = (wid & 7) * 2 + half;
  const int rh = wid >> 3;  // r * Hq + h
  if (rh >= p.n_rh) return;
  const int r = rh / p.Hq, h = rh - r * p.Hq;
  int m;
  const bool live = attn_out_row(p.causal_R, p.n_tiles, p.B, r, q, m);
  const int S = p.n_splits;
  const int ns = p.n_split[r];
  if (ns <= 1) return;  // written by the attention kernel
  const long long pb = (long long)rh * S * 16 + q;
  const float2* ml = reinterpret_cast<const float2*>(p.part_ml) + pb;
  const float* po = p.part_o + pb * DH + hl * 4;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const float2 mine = live && hl < ns ? ml[hl * 16] : make_float2(-INFINITY, 0.f);
  f32x4 v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) v[k] = live && k < ns ? *reinterpret_cast<const f32x4*>(po + (long long)k * 16 * DH) : zero;
  float mx = mine.x;
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 64));
  const float w_mine = mine.x == -INFINITY ? 0.f : expf(mine.x - mx);
  const int base = half * 32;
  float L = 0.f;
  for (int s = 0; s < ns; ++s) L += __shfl(mine.y, base + s, 64) * __shfl(w_mine, base + s, 64);
  f32x4 acc = zero;
  for (int s0 = 0; s0 < ns; s0 += 16) {
    if (s0 > 0) {
#pragma unroll
      for (int k = 0; k < 16; ++k)
        v[k] = live && s0 + k < ns ? *reinterpret_cast<const f32x4*>(po + (long long)(s0 + k) * 16 * DH) : zero;
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float w = __shfl(w_mine, base + ((s0 + k) & 31), 64);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (s0 + k < ns) acc[c] += w * v[k][c];
    }
  }
  if (!live) return;
  const float inv = 1.0f / L;
  const int k = h * DH + hl * 4;  // 4 consecutive k stay contiguous
  typename Vec4<T>::type o;
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = from_f<T>(acc[c] * inv);
  T* out = reinterpret_cast<T*>(p.out) + (p.out_packed ? frag_index(m, k, p.ldo) : (long long)m * p.ldo + k);
  *reinterpret_cast<typename Vec4<T>::type*>(out) = o;
}

template <typename T, int DH>
__global__ __launch_bounds__(256) void k_scatter(ScatterParams p) {
  const int row = blockIdx.x;
  const int l = blockIdx.y;
  const int t = threadIdx.x;
  constexpr int H2 = DH / 2, KQ = H2 / 4, VQ = DH / 4;  // 4-element groups per K half-head and V head
  if (row == 0 && l == 0 && t < p.n_req) {
    const InjectReq q = p.req[t];
    p.state[q.slot].ctx_len = q.pos0 + q.count;
  }
  const float* src = p.kv + (long long)row * p.ld + p.col0 + (long long)l * 2 * p.Hkv * DH;
  const long long plane = (long long)p.rows * p.ld;
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  const int nk = p.Hkv * KQ, nv = p.Hkv * VQ;
  // Rounds of 2 groups per thread and kind.  The row's K/V sums depend on the
  // row alone, so their 16-byte loads are issued before the request lookup
  // and the page-table read, which then overlap them; split-K parts are
  // summed in order, every load of a chunk of 4 parts before any addition.
  for (int e0 = 0; e0 < nv; e0 += 512) {
    f32x4 k1[2], k2[2], v[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) k1[i] = k2[i] = v[i] = zero;
    for (int q0 = 0; q0 < p.n_part; q0 += 4) {
      f32x4 a[4][2], b[4][2], c[4][2];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const bool ok = q0 + q < p.n_part;
          const float* sp = src + (q0 + q) * plane;
          const int e = e0 + t + 256 * i;
          const int gk = e / KQ, jk = (e - gk * KQ) * 4;
          const int gv = e / VQ, dv = (e - gv * VQ) * 4;
          a[q][i] = ok && e < nk ? *reinterpret_cast<const f32x4*>(sp + gk * DH + jk) : zero;
          b[q][i] = ok && e < nk ? *reinterpret_cast<const f32x4*>(sp + gk * DH + jk + H2) : zero;
          c[q][i] = ok && e < nv ? *reinterpret_cast<const f32x4*>(sp + (p.Hkv + gv) * DH + dv) : zero;
        }
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          if (q0 + q < p.n_part) {
            k1[i] += a[q][i];
            k2[i] += b[q][i];
            v[i] += c[q][i];
          }
    }
    // the request owning this row: binary search over the row starts
    int ri = 0, rhi = p.n_req - 1;
    while (ri < rhi) {
      const int mid = (ri + rhi + 1) >> 1;
      if (row >= p.req[mid].row_start)
        ri = mid;
      else
        rhi = mid - 1;
    }
    const InjectReq rq = p.req[ri];
    const int pos = rq.pos0 + (row - rq.row_start);
    if (p.window > 0 && pos < rq.final_ctx - p.window) return;
    const int n_pages = p.state[rq.slot].n_pages;
    const int lp = pos / 16;
    const int idx = p.window > 0 ? lp % n_pages : lp;
    const int page = p.page_table[(long long)rq.slot * p.pt_stride + idx];
    if (page < 0 || page >= p.max_pages) {
      if (t == 0 && e0 == 0) atomicOr(p.err, 4u);
      return;
    }
    const long long page_elems = 2LL * p.Hkv * 16 * DH;
    T* pg = reinterpret_cast<T*>(p.pool) + l * p.layer_stride + page * page_elems;
    const int slotpos = pos & 15;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = e0 + t + 256 * i;
      if (e < nk) {  // K with RoPE at the row's position, [16 positions][dh] per head
        const int g = e / KQ, j = (e - g * KQ) * 4;
        const long long ti = (long long)pos * H2 + j;
        const f32x4 cs = *reinterpret_cast<const f32x4*>(p.cos_t + ti);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(p.sin_t + ti);
        typename Vec4<T>::type o1, o2;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          o1[k] = from_f<T>(k1[i][k] * cs[k] - k2[i][k] * sn[k]);
          o2[k] = from_f<T>(k2[i][k] * cs[k] + k1[i][k] * sn[k]);
        }
        T* kd = pg + (long long)(g * 16 + slotpos) * DH + j;
        *reinterpret_cast<typename Vec4<T>::type*>(kd) = o1;
        *reinterpret_cast<typename Vec4<T>::type*>(kd + H2) = o2;
      }
      if (e < nv) {  // V transposed, [dh][16 positions] per head
        const int g = e / VQ, d = (e - g * VQ) * 4;
        T* vd = pg + (long long)(p.Hkv + g) * 16 * DH + slotpos;
#pragma unroll
        for (int k = 0; k < 4; ++k) vd[(d + k) * 16] = from_f<T>(v[i][k]);
      }
    }
  }
}

template <typename T>
void qkv_post_t(int dh, int n_req, const QkvPostParams& p, const SlotArgs& sl, hipStream_t s) {
  dim3 grid(n_req, p.Hq + 2 * p.Hkv);
  if (dh == 128)
    hipLaunchKernelGGL((k_qkv_post<T, 128>), grid, dim3(256), 0, s, p, sl);
  else
    hipLaunchKernelGGL((k_qkv_post<T, 64>), grid, dim3(256), 0, s, p, sl);
}

template <typename T>
void attn_t(int dh, int n_req, const AttnParams& p, const SlotArgs& sl, hipStream_t s) {
  dim3 grid(p.Hkv, p.n_splits, n_req);  // KV head fastest: see attn_ring_t
  const int G = p.Hq / p.Hkv;
  dim3 block(64 * G * p.KQ);
  const size_t lds = attn_lds_bytes(p.Hq, p.Hkv, dh, p.KQ);
  if (dh == 128)
    hipLaunchKernelGGL((k_attn<T, 128>), grid, block, lds, s, p, sl);
  else
    hipLaunchKernelGGL((k_attn<T, 64>), grid, block, lds, s, p, sl);
}

template <int DH>
void attn_ring_t(int n_req, const AttnParams& p, const SlotArgs& sl, hipStream_t s) {
  // KV head fastest: workgroups go to the eight XCDs round-robin by linear
  // id, so with eight KV heads each XCD takes one head of every (request,
  // split) and all XCDs get the same work.  (Split fastest sent split s of
  // every request to XCD s, and the first XCDs carried most of the load.)
  dim3 grid(p.Hkv, p.n_splits, n_req);
  switch (p.Hq / p.Hkv) {
    case 1: hipLaunchKernelGGL((k_attn_ring<DH, 1>), grid, dim3(64), 0, s, p, sl); break;
    case 2: hipLaunchKernelGGL((k_attn_ring<DH, 2>), grid, dim3(128), 0, s, p, sl); break;
    case 3: hipLaunchKernelGGL((k_attn_ring<DH, 3>), grid, dim3(192), 0, s, p, sl); break;
    case 4: hipLaunchKernelGGL((k_attn_ring<DH, 4>), grid, dim3(256), 0, s, p, sl); break;
    case 5: hipLaunchKernelGGL((k_attn_ring<DH, 5>), grid, dim3(320), 0, s, p, sl); break;
    case 6: hipLaunchKernelGGL((k_attn_ring<DH, 6>), grid, dim3(384), 0, s, p, sl); break;
    case 7: hipLaunchKernelGGL((k_attn_ring<DH, 7>), grid, dim3(448), 0, s, p, sl); break;
    default: hipLaunchKernelGGL((k_attn_ring<DH, 8>), grid, dim3(512), 0, s, p, sl); break;
  }
}

template <typename T>
void combine_t(int dh, const CombineParams& p, hipStream_t s) {
  dim3 grid((p.n_rh * 16 + 3) / 4);
  // two rows per wave pays where the merge streams many partials; a small
  // merge (one request: 32 rows of heads) is latency-bound and keeps one row
  // per wave, which spreads it over twice the workgroups
  if (dh == 128 && p.n_splits <= 32 && p.n_rh >= 256)
    hipLaunchKernelGGL((k_combine2<T>), dim3(p.n_rh * 2), dim3(256), 0, s, p);
  else if (dh == 128)
    hipLaunchKernelGGL((k_combine<T, 128>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_combine<T, 64>), grid, dim3(256), 0, s, p);
}

template <typename T>
void scatter_t(int dh, const ScatterParams& p, hipStream_t s) {
  dim3 grid(p.rows, p.L);
  if (dh == 128)
    hipLaunchKernelGGL((k_scatter<T, 128>), grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL((k_scatter<T, 64>), grid, dim3(256), 0, s, p);
}

}  // namespace

size_t attn_lds_bytes(int Hq, int Hkv, int dh, int KQ) {
  const int G = Hq / Hkv;
  return sizeof(float) * ((size_t)G * 16 * dh + (size_t)KQ * G * 16 * 2 + (size_t)G * 16);
}

void launch_qkv_post(int dtype, int dh, int n_req, const QkvPostParams& p, const SlotArgs& sl,
                     hipStream_t s) {
  if (dtype == DFLASH_BF16)
    qkv_post_t<bf16>(dh, n_req, p, sl, s);
  else
    qkv_post_t<float>(dh, n_req, p, sl, s);
}

void launch_attention(int dtype, int dh, int n_req, const AttnParams& p, const SlotArgs& sl,
                      hipStream_t s) {
  if (dtype == DFLASH_BF16) {
    if (dh == 128)
      attn_ring_t<128>(n_req, p, sl, s);
    else
      attn_ring_t<64>(n_req, p, sl, s);
  } else {
    attn_t<float>(dh, n_req, p, sl, s);
  }
}

void launch_combine(int dtype, int dh, const CombineParams& p, hipStream_t s) {
  if (p.n_rh <= 0) return;
  if (dtype == DFLASH_BF16)
    combine_t<bf16>(dh, p, s);
  else
    combine_t<float>(dh, p, s);
}

void launch_scatter(int dtype, int dh, const ScatterParams& p, hipStream_t s) {
  if (p.rows <= 0) return;
  if (dtype == DFLASH_BF16)
    scatter_t<bf16>(dh, p, s);
  else
    scatter_t<float>(dh, p, s);
}

__global__ void k_set_ctx(SlotState* state, int slot, int ctx_len) {
  if (threadIdx.x == 0) state[slot].ctx_len = ctx_len;
}

void launch_set_ctx(SlotState* state, int slot, int ctx_len, hipStream_t s) {
  hipLaunchKernelGGL(k_set_ctx, dim3(1), dim3(64), 0, s, state, slot, ctx_len);
}

}  // namespace dflash
