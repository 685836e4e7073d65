// Weight-streaming GEMM for the draft's skinny products (M = batch * block rows).
//
// Y[M, N] = X[M, K] * W[N, K]^T.  At batch 1 every projection of the draft is
// bound by streaming W from HBM (16 activation rows per weight: 16 flop per
// byte), so the kernel is built around the weight stream:
//
//  * W is packed once (k_pack) into MFMA fragment order,
//      Wp[tile][kstep][lane][8],  tile = 16 output rows, kstep = 32 of K,
//    lane l holding row 16*tile + l%16, k = 32*kstep + 8*(l/16) .. +8, so one
//    wave's fragment is 1 KB of contiguous memory (bf16).
//  * A workgroup of NW waves (up to 16, one workgroup per CU) owns one K range
//    (split p of P) and a strided set of output tiles.  Wave w owns KS
//    k-steps of that range; its activation fragments for them are loaded once
//    into registers.  For every tile the wave then streams KS contiguous
//    fragments (KS KB) of W through a register ring of NBUF tiles, so the next
//    tiles' weights are in flight while the current one is multiplied.
//  * MFMA 16x16x32 bf16 (16x16x4 f32 for fp32 weights); the NW per-wave
//    partial tiles are summed through LDS in a fixed order (deterministic),
//    once per tile, and the epilogue runs once per output element.
//
// Epilogues: split-K partials (fp32, summed by the consuming kernel); residual
// add; SwiGLU (gate and up tiles processed back to back, silu(gate) * up
// rounded to the storage dtype); RoPE (the two halves of a head processed back
// to back, rotated and written in the attention layouts); greedy selection (packed logit/id key,
// running max per row across the workgroup's tiles, one 64-bit atomic max per
// row and workgroup, ties to the lowest id); top-16 (the same keys, a sorted
// list of 16 per row kept across the row's 16 lanes by bitonic sort and merge,
// one list per row and workgroup merged by k_topk_merge).
#include "common.h"
#include "kernels.h"

namespace dflash {

namespace {

constexpr int kFragElems = 64 * 8;  // elements of one wave fragment

template <typename T, int MT>
struct Shape {
  static constexpr int KS = (sizeof(T) == 2 && MT == 1) ? 8 : 4;  // k-steps per wave per tile
  static constexpr int NBUF = (sizeof(T) == 2 ? 16 : 8) / KS;     // tiles in the W ring
};
// 4-bit weights: a tile's KS k-steps are KS / 4 16-byte code loads and as
// many 8-byte (scale, bias) loads per lane, so the ring holds more tiles.
// (The RoPE epilogue's state leaves room for two tiles in the 16-row form.)
template <int MT, int EPI>
struct Shape4 {
  static constexpr int NBUF = MT == 1 ? (EPI == EPI_ROPE ? 2 : 3) : 8;
};

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// One tile's weights for the wave's k-steps, in registers.
template <typename T, int KS, bool W4>
struct WRing {
  typename Frag8<T>::type f[KS];
};
template <typename T, int KS>
struct WRing<T, KS, true> {
  u32x4 q[KS / 4];   // codes of k-steps 4i .. 4i+3
  u32x2 sb[KS / 4];  // (scale, bias) of the two groups of 64 inputs they cover
};

// The 8 codes of one lane's k-step (nibble e = element e) as bf16 values
// 1 + q / 16: each code goes to mantissa bits 3..6 of a bf16 whose exponent
// is that of 1 (0x3F80 | q << 3).  Byte i of x holds codes 2i (low nibble)
// and 2i + 1 (high nibble); they are moved to bits 3..6 of separate bytes,
// paired into 16-bit halves and given the exponent.
__device__ __forceinline__ bf16x8 expand_q4(unsigned x) {
  const unsigned lo = (x << 3) & 0x78787878u, hi = (x >> 1) & 0x78787878u;
  u32x4 r;
  r[0] = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x3F803F80u;
  r[1] = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x3F803F80u;
  r[2] = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x3F803F80u;
  r[3] = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x3F803F80u;
  return __builtin_bit_cast(bf16x8, r);
}

// Workgroups of MT > 1 have at most 8 waves (their activation and weight
// registers need two waves per SIMD at most).
//
// 4-bit weights (W4): per group of 64 inputs the product is
// 16 s * sum x (1 + q / 16) + (b - 16 s) * sum x, which equals
// sum x (s q + b) exactly in real arithmetic: the codes enter the MFMA as
// bf16 values 1 + q / 16 (exact), the group's partial tile is scaled by 16 s
// and the activation sums of the group (formed once per wave on the matrix
// cores with a tile of ones) times (b - 16 s) are added, in fp32.  (The
// offset 1 keeps the cancelled part 16 s * sum x small beside the result.)
template <typename T, int MT, int EPI, bool FEW, bool W4>
__global__ __launch_bounds__(FEW ? 256 : (MT > 1 ? 512 : 1024)) void k_gemm(GemmParams p) {
  constexpr int KS = Shape<T, MT>::KS;
  constexpr int NBUF = W4 ? Shape4<MT, EPI>::NBUF : Shape<T, MT>::NBUF;
  static_assert(!W4 || (sizeof(T) == 2 && KS % 4 == 0), "4-bit weights: bf16 activations, whole code loads");
  constexpr int NSUB = (EPI == EPI_SWIGLU || EPI == EPI_ROPE) ? 2 : 1;
  typedef typename Frag8<T>::type Frag;
  __shared__ float red[2][MT > 1 ? 8 : 16][MT][256];
  // EPI_ROPE: tiles per head and the tile distance of a rotate-half pair
  const int rope_tph = EPI == EPI_ROPE ? p.rope.dh / 16 : 0;
  const int rope_half = rope_tph / 2;

  const int NW = blockDim.x >> 6;
  const int lane = lane_id();
  // wave-uniform (scalar) so that the kernel-argument pointer arrays indexed
  // by the wave's k range are read with scalar loads, not a vector load and
  // a full wait at kernel start
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15;
  const int g = lane >> 4;
  const int GP = gridDim.x / p.P;
  const int pidx = blockIdx.x / GP;
  const int bl = blockIdx.x - pidx * GP;
  const int S = p.K / 32;
  const int s0 = pidx * (S / p.P) + wave * KS;
  const int m_base = blockIdx.y * 16 * MT;
  const int n_units = bl < p.tiles ? (p.tiles - 1 - bl) / GP + 1 : 0;
  const int n_sub = n_units * NSUB;

  // activation fragments of this wave's k-steps, loaded once
  Frag af[MT][KS];
  {
    const int k0 = s0 * 32;
    const int part = k0 / p.a_part_k;
    const T* abase = reinterpret_cast<const T*>(p.a[part]) + (k0 - part * p.a_part_k) + 8 * g;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int m = m_base + mt * 16 + r16;
      const bool ok = m < p.M;
      const T* ar = abase + (long long)m * p.lda;
#pragma unroll
      for (int j = 0; j < KS; ++j) af[mt][j] = ok ? load8<T>(ar + 32 * j) : zero8<T>();
    }
  }

  // 4-bit weights: the activation sums of each group of 64 inputs, in the
  // accumulator layout (a product with a tile of ones)
  f32x4 xs[W4 ? MT : 1][W4 ? KS / 2 : 1];
  if constexpr (W4) {
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int g2 = 0; g2 < KS / 2; ++g2)
        xs[mt][g2] = mfma_step(af[mt][2 * g2 + 1], ones, mfma_step(af[mt][2 * g2], ones, f32x4{0.f, 0.f, 0.f, 0.f}));
  }

  // weight tile of sub-unit `sub` of this workgroup
  auto tile_of = [&](int sub) {
    const int u = sub / NSUB;
    int t = bl + u * GP;
    if (EPI == EPI_SWIGLU && (sub & 1)) t += p.up_tile_off;
    if (EPI == EPI_ROPE) t = (t / rope_half) * rope_tph + t % rope_half + (sub & 1) * rope_half;
    return t;
  };
  typedef WRing<T, KS, W4> Ring;
  auto load_tile = [&](int sub, Ring& r) {
    int t = tile_of(sub);
    int seg = 0, lt = t;
    if (p.seg_tiles) {
      seg = t / p.seg_tiles;
      lt = t - seg * p.seg_tiles;
    }
    if constexpr (W4) {
      const long long u = (long long)lt * (S / 4) + s0 / 4;  // first code unit (4 k-steps) of the wave
      const u32x4* q = reinterpret_cast<const u32x4*>(p.w[seg]) + u * 64 + lane;
      const u32x2* sb = reinterpret_cast<const u32x2*>(p.sb[seg]) + u * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < KS / 4; ++i) {
        r.q[i] = __builtin_nontemporal_load(q + i * 64);
        r.sb[i] = __builtin_nontemporal_load(sb + i * 16);
      }
    } else {
      const T* src = reinterpret_cast<const T*>(p.w[seg]) + ((long long)lt * S + s0) * kFragElems + lane * 8;
#pragma unroll
      for (int j = 0; j < KS; ++j)
        r.f[j] = __builtin_nontemporal_load(reinterpret_cast<const Frag*>(src + j * kFragElems));
    }
  };

  // EPI_RESID: the residual values and gains of the first unit's elements,
  // requested before the weights
  constexpr int EIT0 = (FEW ? 4 : 1) * MT;
  // (clamped addresses; the gains stay in the storage dtype until the
  // epilogue, so nothing waits for them here)
  float pre_x[EPI == EPI_RESID ? EIT0 : 1];
  T pre_g[EPI == EPI_RESID ? EIT0 : 1];
  if (EPI == EPI_RESID) {
#pragma unroll
    for (int it = 0; it < EIT0; ++it) {
      const int e = threadIdx.x + it * (int)blockDim.x;
      const int em = min(m_base + (e >> 8) * 16 + ((e >> 4) & 15), p.M - 1);
      const int n = min(bl * 16 + (e & 15), p.N - 1);
      pre_x[it] = p.resid_row ? to_f(reinterpret_cast<const T*>(p.resid_row)[n]) : p.resid[(long long)em * p.ldr + n];
      pre_g[it] = reinterpret_cast<const T*>(p.gain)[n];
    }
  }

  Ring wb[NBUF];
#pragma unroll
  for (int b = 0; b < NBUF; ++b)
    if (b < n_sub) load_tile(b, wb[b]);

  // EPI_SWIGLU after a residual epilogue: wave w sums the per-tile squares of
  // block row w.  The loads follow the weight ring's (issued before it, the
  // sum would hold the ring back until they arrive); each has a clamped, valid
  // address and its value is selected afterwards.
  constexpr int kSsqMax = 8;  // tiles per lane: hidden sizes up to 64 * 8 * 16
  float ssv[EPI == EPI_SWIGLU ? kSsqMax : 1];
  if (EPI == EPI_SWIGLU && p.ssq) {
    const int m = m_base + wave;
    const long long mc = min(m, p.M - 1);
#pragma unroll
    for (int i = 0; i < kSsqMax; ++i) {
      const int t2 = lane + 64 * i;
      const float x = p.ssq[mc * p.ssq_tiles + min(t2, p.ssq_tiles - 1)];  // a row's tiles are contiguous
      ssv[i] = wave < 16 * MT && m < p.M && t2 < p.ssq_tiles ? x : 0.f;
    }
  }

  // epilogue: element e = t + it * blockDim of the 16 x 16 tile (per m-tile);
  // workgroups with fewer than 4 waves (FEW) take several elements per thread,
  // the others one element per thread and m-tile, which keeps the per-thread
  // epilogue state out of the register budget of the weight ring
  const int t = threadIdx.x;
  constexpr int EIT = (FEW ? 4 : 1) * MT;
  float gate_v[EIT];
  unsigned long long best[EIT];
#pragma unroll
  for (int it = 0; it < EIT; ++it) {
    gate_v[it] = 0.f;
    best[it] = 0ull;
  }
  // EPI_ROPE: position of block row 0 of each epilogue element's request,
  // requested while the weights stream so the epilogue does not wait for the
  // slot and state reads after the reduction
  int rope_n[EIT];
#pragma unroll
  for (int it = 0; it < EIT; ++it) {
    rope_n[it] = 0;
    if (EPI == EPI_ROPE) {
      const int e = t + it * (int)blockDim.x;
      const int em = m_base + (e >> 8) * 16 + ((e >> 4) & 15);
      if (e < 256 * MT && em < p.M) rope_n[it] = p.rope.state[p.rope.slots[em / p.rope.B]].ctx_len + 1;
    }
  }

  // EPI_SWIGLU after a residual epilogue: 1/rms of each row of the block from
  // the producer's per-tile sums of squares (tiles in order per lane, then the
  // wave's lanes by a butterfly), formed while the weights stream
  __shared__ float rs_inv[EPI == EPI_SWIGLU ? 16 * MT : 1];
  if (EPI == EPI_SWIGLU && p.ssq) {
    // row `wave` from the loads above; with fewer waves than rows, the other
    // rows' squares are read here (the same order of additions)
    for (int rr = wave; rr < 16 * MT; rr += NW) {
      float acc = 0.f;
      if (rr == wave) {
#pragma unroll
        for (int i = 0; i < kSsqMax; ++i) acc += ssv[i];
      } else if (m_base + rr < p.M) {
        for (int t2 = lane; t2 < p.ssq_tiles; t2 += 64) acc += p.ssq[(long long)(m_base + rr) * p.ssq_tiles + t2];
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
      if (lane == 0) rs_inv[rr] = 1.0f / sqrtf(acc / (float)p.ssq_d + p.eps);
    }
  }

  for (int i = 0; i < n_sub; i += NBUF) {
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
      const int sub = i + b;
      if (sub < n_sub) {
        f32x4 acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (W4) {
#pragma unroll
          for (int i = 0; i < KS / 4; ++i)
#pragma unroll
            for (int gg = 0; gg < 2; ++gg) {
              const unsigned sbw = wb[b].sb[i][gg];
              const float sc = 16.0f * __uint_as_float(sbw << 16), bi = __uint_as_float(sbw & 0xFFFF0000u);
              const float bp = bi - sc;
              f32x4 tmp[MT];
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) tmp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int jj = 0; jj < 2; ++jj) {
                const bf16x8 wf = expand_q4(wb[b].q[i][2 * gg + jj]);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) tmp[mt] = mfma_step(af[mt][4 * i + 2 * gg + jj], wf, tmp[mt]);
              }
#pragma unroll
              for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  acc[mt][e] = fmaf(sc, tmp[mt][e], fmaf(bp, xs[mt][2 * i + gg][e], acc[mt][e]));
            }
        } else {
#pragma unroll
          for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) acc[mt] = mfma_step(af[mt][j], wb[b].f[j], acc[mt]);
        }
        if (sub + NBUF < n_sub) load_tile(sub + NBUF, wb[b]);
        const int rb = sub & 1;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int q = 0; q < 4; ++q) red[rb][wave][mt][(4 * g + q) * 16 + r16] = acc[mt][q];
        __syncthreads();
#pragma unroll
        for (int it = 0; it < EIT; ++it) {
          const int e = t + it * (int)blockDim.x;
          if (e >= 256 * MT) break;
          const int emt = e >> 8;
          const int ecol = e & 15;
          const int em = m_base + emt * 16 + ((e >> 4) & 15);
          float v = 0.f;
          for (int w2 = 0; w2 < NW; ++w2) v += red[rb][w2][emt][e & 255];
          const int u = sub / NSUB;
          const int tile = EPI == EPI_ROPE ? tile_of(sub) : bl + u * GP;
          const int n = tile * 16 + ecol;
          const bool ok = em < p.M && n < p.N;
          if (EPI == EPI_PARTIAL) {
            if (ok) p.out_f32[((long long)pidx * p.M + em) * p.N + n] = v;
          } else if (EPI == EPI_RESID) {
            float x = 0.f;
            if (ok) {
              float* rp = p.resid + (long long)em * p.ldr + n;
              x = (u == 0 ? pre_x[it] : p.resid_row ? to_f(reinterpret_cast<const T*>(p.resid_row)[n]) : *rp) + v;
              *rp = x;
              const float gn = to_f(u == 0 ? pre_g[it] : reinterpret_cast<const T*>(p.gain)[n]);
              reinterpret_cast<T*>(p.out_t)[(long long)em * p.ldt + n] = from_f<T>(x * gn);
            }
            // the 16 columns of row em sit in 16 adjacent lanes (every lane of
            // the first 256 * MT threads takes part)
            float sq = x * x;
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) sq += __shfl_xor(sq, o, 64);
            if (ecol == 0 && em < p.M) p.ssq[(long long)em * p.ssq_tiles + tile] = sq;
          } else if (EPI == EPI_SWIGLU) {
            if (p.ssq) v *= rs_inv[emt * 16 + ((e >> 4) & 15)];
            if (!(sub & 1)) {
              gate_v[it] = v;
            } else if (ok) {
              const float g0 = gate_v[it];
              const float sg = g0 / (1.0f + expf(-g0));
              reinterpret_cast<T*>(p.out_t)[(long long)em * p.ldt + n] = from_f<T>(sg * v);
            }
          } else if (EPI == EPI_ROPE) {
            if (!(sub & 1)) {
              gate_v[it] = v;  // column j of the head; v below is column j + dh/2
            } else if (ok) {
              const RopeOut& ro = p.rope;
              const int dh = ro.dh, h2 = dh >> 1;
              const int head = (n - h2) / dh;
              const int j = n - h2 - head * dh;
              const int r = em / ro.B, i = em - r * ro.B;
              const float x1 = gate_v[it];
              T* o;
              if (head < ro.Hq + ro.Hkv) {
                const long long ti = (long long)(rope_n[it] + i) * h2 + j;
                const float c = ro.cos_t[ti], sn = ro.sin_t[ti];
                if (head < ro.Hq)
                  o = reinterpret_cast<T*>(ro.qb) + ((long long)(r * ro.Hq + head) * 16 + i) * dh;
                else
                  o = reinterpret_cast<T*>(ro.blk) + ((long long)(r * 2 + 0) * ro.Hkv + head - ro.Hq) * 16 * dh + i * dh;
                o[j] = from_f<T>(x1 * c - v * sn);
                o[j + h2] = from_f<T>(v * c + x1 * sn);
              } else {
                o = reinterpret_cast<T*>(ro.blk) + ((long long)(r * 2 + 1) * ro.Hkv + head - ro.Hq - ro.Hkv) * 16 * dh;
                o[j * 16 + i] = from_f<T>(x1);
                o[(j + h2) * 16 + i] = from_f<T>(v);
              }
            }
          } else if (EPI == EPI_ARGMAX) {  // all 16 columns of a row sit in 16 adjacent lanes
            if (ok && p.dbg) p.dbg[(long long)em * p.ld_dbg + n] = v;
            unsigned long long key = ok ? argmax_key(v, n, p.N) : 0ull;
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
              const unsigned long long other = __shfl_xor(key, o, 64);
              key = other > key ? other : key;
            }
            best[it] = key > best[it] ? key : best[it];
          } else {  // EPI_TOPK: running sorted top-16 of the row across its 16 lanes
            if (ok && p.dbg) p.dbg[(long long)em * p.ld_dbg + n] = v;
            const unsigned long long key = ok ? argmax_key(v, n, p.N) : 0ull;
            best[it] = merge16_desc(best[it], sort16_desc(key, ecol), ecol);
          }
        }
      }
    }
  }
  if (EPI == EPI_TOPK) {
#pragma unroll
    for (int it = 0; it < EIT; ++it) {
      const int e = t + it * (int)blockDim.x;
      if (e >= 256 * MT) break;
      const int em = m_base + (e >> 8) * 16 + ((e >> 4) & 15);
      if (em < p.M) p.keys[((long long)em * gridDim.x + blockIdx.x) * 16 + (e & 15)] = best[it];
    }
  }
  if (EPI == EPI_ARGMAX && n_units > 0) {
#pragma unroll
    for (int it = 0; it < EIT; ++it) {
      const int e = t + it * (int)blockDim.x;
      if (e >= 256 * MT) break;
      const int em = m_base + (e >> 8) * 16 + ((e >> 4) & 15);
      if ((e & 15) == 0 && em < p.M) atomicMax(p.keys + em, best[it]);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_pack(const T* src, T* dst, int N, int K, long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int S = K / 32;
  const int l = (int)(idx & 63);
  const long long ts = idx >> 6;
  const int s = (int)(ts % S);
  const long long tile = ts / S;
  const long long row = tile * 16 + (l & 15);
  const int k = s * 32 + 8 * (l >> 4);
  typedef typename Frag8<T>::type Frag;
  const Frag v = row < N ? load8<T>(src + row * K + k) : zero8<T>();
  *reinterpret_cast<Frag*>(dst + idx * 8) = v;
}

// One thread per 4 consecutive columns of one row: 16-byte loads of every
// split's gate and up partials, summed in split order (the SwiGLU epilogue's
// formula on the summed values).
template <typename T>
__global__ __launch_bounds__(256) void k_swiglu_parts(const float* part, int P, int M, int F, T* z, int ldo) {
  const int f = (blockIdx.x * 256 + threadIdx.x) * 4;
  const int m = blockIdx.y;
  if (f >= F) return;
  const long long plane = (long long)M * 2 * F;
  const float* g = part + (long long)m * 2 * F + f;
  f32x4 gs = *reinterpret_cast<const f32x4*>(g);
  f32x4 us = *reinterpret_cast<const f32x4*>(g + F);
  for (int q = 1; q < P; ++q) {
    gs += *reinterpret_cast<const f32x4*>(g + q * plane);
    us += *reinterpret_cast<const f32x4*>(g + q * plane + F);
  }
  T* o = z + (long long)m * ldo + f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float sg = gs[i] / (1.0f + expf(-gs[i]));
    o[i] = from_f<T>(sg * us[i]);
  }
}

// bf16 rounding (nearest even) of a finite float
__device__ __forceinline__ float round_bf16(float x) {
  unsigned u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

// One thread per (tile, group of 64 inputs, tile row): the group's min and
// max, its bf16 scale and bias, the codes (fp32 steps, IEEE division, round
// half to even), written into the code and scale layouts of the q4 format.
__global__ __launch_bounds__(256) void k_pack_q4(const bf16* src, unsigned* dst, int N, int K, long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int G = K / 64, S4 = K / 128;
  const int r16 = (int)(idx & 15);
  const long long tg = idx >> 4;
  const int g = (int)(tg % G);
  const long long t = tg / G;
  const long long row = t * 16 + r16;
  float w[64];
  if (row < N) {
    const bf16* sp = src + row * K + (long long)g * 64;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bf16x8 v = load8<bf16>(sp + 8 * i);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[8 * i + e] = (float)v[e];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 64; ++i) w[i] = 0.f;
  }
  float lo = w[0], hi = w[0];
#pragma unroll
  for (int i = 1; i < 64; ++i) {
    lo = fminf(lo, w[i]);
    hi = fmaxf(hi, w[i]);
  }
  const float sc = round_bf16(__fdiv_rn(hi - lo, 15.0f));
  const float b = round_bf16(lo);
  unsigned* codes = dst + ((t * S4 + g / 2) * 64) * 4;
#pragma unroll
  for (int h = 0; h < 2; ++h) {  // the group's two k-steps
    const int js = 2 * (g & 1) + h;
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // lanes r16 + 16 c hold inputs 8 c .. 8 c + 7 of the k-step
      unsigned word = 0u;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float qf = sc > 0.f ? rintf(__fdiv_rn(w[32 * h + 8 * c + e] - b, sc)) : 0.f;
        const unsigned q = (unsigned)fminf(fmaxf(qf, 0.f), 15.f);
        word |= q << (4 * e);
      }
      codes[(r16 + 16 * c) * 4 + js] = word;
    }
  }
  unsigned* sb = dst + q4_codes_bytes(N, K) / 4 + ((t * S4 + g / 2) * 16 + r16) * 2 + (g & 1);
  *sb = (__float_as_uint(sc) >> 16) | (__float_as_uint(b) & 0xFFFF0000u);
}

template <typename T, int EPI, bool W4>
void launch_w(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && EPI == EPI_PARTIAL) {
    if (pl.mt == 4) {  // blocks of up to 64 rows: W streamed once per block
      const dim3 grid(pl.GP * p.P, (p.M + 63) / 64);
      if (pl.NW < 4)
        hipLaunchKernelGGL((k_gemm<T, 4, EPI, true, W4>), grid, dim3(64 * pl.NW), 0, s, p);
      else
        hipLaunchKernelGGL((k_gemm<T, 4, EPI, false, W4>), grid, dim3(64 * pl.NW), 0, s, p);
      return;
    }
  }
  // 16-row m-blocks; rows beyond 16 re-stream W
  dim3 grid(pl.GP * p.P, (p.M + 15) / 16);
  dim3 block(64 * pl.NW);
  if (pl.NW < 4)
    hipLaunchKernelGGL((k_gemm<T, 1, EPI, true, W4>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((k_gemm<T, 1, EPI, false, W4>), grid, block, 0, s, p);
}

template <typename T, int EPI>
void launch_t(const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  if constexpr (sizeof(T) == 2 && (EPI == EPI_PARTIAL || EPI == EPI_RESID || EPI == EPI_SWIGLU || EPI == EPI_ROPE)) {
    if (p.w4) {
      launch_w<T, EPI, true>(pl, p, s);
      return;
    }
  }
  launch_w<T, EPI, false>(pl, p, s);
}

template <typename T>
void launch_dt(int epi, const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  switch (epi) {
    case EPI_PARTIAL: launch_t<T, EPI_PARTIAL>(pl, p, s); break;
    case EPI_RESID: launch_t<T, EPI_RESID>(pl, p, s); break;
    case EPI_SWIGLU: launch_t<T, EPI_SWIGLU>(pl, p, s); break;
    case EPI_ROPE: launch_t<T, EPI_ROPE>(pl, p, s); break;
    case EPI_TOPK: launch_t<T, EPI_TOPK>(pl, p, s); break;
    default: launch_t<T, EPI_ARGMAX>(pl, p, s); break;
  }
}

}  // namespace

int gemm_kblock(int dtype, int mt) {
  if (mt == 4) return 32 * Shape<bf16, 4>::KS;
  return 32 * (dtype == DFLASH_BF16 ? Shape<bf16, 1>::KS : Shape<float, 1>::KS);
}

// Split-K factor P, waves per workgroup NW and workgroups per split GP for a
// GEMM of `tiles` 16-row output tiles over K.  Minimises the per-workgroup
// stream (units per workgroup x K / P) with at most 256 workgroups (one per
// CU), penalising fewer than 8 waves per workgroup.
GemmPlan plan_gemm(int tiles, int K, int kblock, bool single_split, int max_nw) {
  GemmPlan best{0, 0, 0, 1};
  double best_cost = 1e300;
  const int kb = K / kblock;
  for (int P = 1; P <= kb; ++P) {
    if (kb % P) continue;
    const int NW = kb / P;
    if (NW > max_nw) continue;
    if (single_split && P != 1) break;
    const int gp_max = 256 / P;
    if (gp_max < 1) break;
    const int units = (tiles + gp_max - 1) / gp_max;
    const int GP = (tiles + units - 1) / units;
    const double eff = NW >= 8 ? 1.0 : NW / 8.0;
    const double cost = (double)units * K / P / eff;
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = GemmPlan{P, NW, GP, 1};
    }
  }
  return best;
}

void launch_gemm(int dtype, int epi, const GemmPlan& pl, const GemmParams& p, hipStream_t s) {
  if (p.M <= 0 || p.tiles <= 0) return;
  if (pl.mt == 0) {
    launch_gemm_big(epi, p, s);
    return;
  }
  if (dtype == DFLASH_BF16)
    launch_dt<bf16>(epi, pl, p, s);
  else
    launch_dt<float>(epi, pl, p, s);
}

void launch_swiglu_parts(int dtype, const float* part, int P, int M, int F, void* z, int ldo, hipStream_t s) {
  if (M <= 0 || F <= 0) return;
  const dim3 grid((F / 4 + 255) / 256, M);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_swiglu_parts<bf16>, grid, dim3(256), 0, s, part, P, M, F, reinterpret_cast<bf16*>(z), ldo);
  else
    hipLaunchKernelGGL(k_swiglu_parts<float>, grid, dim3(256), 0, s, part, P, M, F, reinterpret_cast<float*>(z), ldo);
}

void launch_pack_q4(const void* src, void* dst, int N, int K, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * (K / 64) * 16;
  const int blocks = (int)((total + 255) / 256);
  hipLaunchKernelGGL(k_pack_q4, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const bf16*>(src),
                     reinterpret_cast<unsigned*>(dst), N, K, total);
}

size_t packed_elems(int N, int K) { return (size_t)((N + 15) / 16) * 16 * (size_t)K; }

void launch_pack(int dtype, const void* src, void* dst, int N, int K, hipStream_t s) {
  const long long total = (long long)((N + 15) / 16) * (K / 32) * 64;
  const int blocks = (int)((total + 255) / 256);
  if (dtype == DFLASH_BF16)
    hipLaunchKernelGGL(k_pack<bf16>, dim3(blocks), dim3(256), 0, s,
                       reinterpret_cast<const bf16*>(src), reinterpret_cast<bf16*>(dst), N, K, total);
  else
    hipLaunchKernelGGL(k_pack<float>, dim3(blocks), dim3(256), 0, s,
                       reinterpret_cast<const float*>(src), reinterpret_cast<float*>(dst), N, K, total);
}

}  // namespace dflash
