// Kernel launch interface between the host runtime and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dflash.h"

namespace dflash {

constexpr int kMaxSeg = DFLASH_MAX_LAYERS;
constexpr int kMaxChunkReq = 64;  // requests per inject scatter launch

enum Epilogue { EPI_STORE = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_ARGMAX = 3 };

// Y[M, N] = X[M, K] * W[N, K]^T with a fused epilogue.
//  X: virtual concatenation along k of a_parts row-major arrays, each
//     [M, a_part_k] with row stride lda (elements).
//  W: row-major; rows [s*seg_rows, (s+1)*seg_rows) live at w[s].  With one
//     segment seg_rows may be any N (the last 16-row tile is guarded).
struct GemmParams {
  const void* a[DFLASH_MAX_FEAT];
  int a_parts, a_part_k, lda;
  int M;
  const void* w[kMaxSeg];
  const void* w_up;  // EPI_SWIGLU: up-projection rows, same layout as w[0]
  int seg_rows;
  int N, K;
  float* out_f32;  // EPI_STORE
  int ldo;
  void* out_t;  // EPI_SWIGLU (storage dtype)
  int ldt;
  float* resid;  // EPI_RESID
  int ldr;
  unsigned long long* keys;  // EPI_ARGMAX, one per row
  float* dbg;                // EPI_ARGMAX, optional fp32 logits
  int ld_dbg;
};

// Row-wise RMSNorm of fp32 rows into the storage dtype.
struct NormParams {
  const float* x;      // [M, d] fp32 (ignored when init_row is set)
  float* x_init;       // when init_row: receives init_row in every row
  const void* init_row;  // storage dtype [d]: every row starts from it
  int ldx;
  const void* gamma;  // storage dtype [d]
  float eps;
  void* out;  // storage dtype [M, d]
  int ldo;
  int d, M;
  float* dbg;  // optional fp32 copy of the input rows [M, d]
  unsigned long long* zero_keys;  // optional: keys[row] = 0
};

struct SlotArgs {
  int slots[DFLASH_MAX_BATCH];
};

// Device per-slot state: ctx_len, kv_begin, n_pages (ring size), pad.
struct SlotState {
  int ctx_len, kv_begin, n_pages, pad;
};

struct QkvPostParams {
  const float* qkv;  // [n_req*B, (Hq+2Hkv)*dh]
  int B, Hq, Hkv;
  const SlotState* state;
  const float* cos_t;  // [max_position, dh/2]
  const float* sin_t;
  void* qb;   // [n_req, Hq, 16, dh]
  void* blk;  // [n_req] pages [2][Hkv][16*dh]
};

struct AttnParams {
  const void* qb;
  const void* blk;
  const void* pool;  // this layer's pages
  const int* page_table;
  int pt_stride;
  const SlotState* state;
  int max_pages;
  int window;
  int Hq, Hkv, B;
  int pps;       // units (pages) per split
  int n_splits;  // grid.x
  float scale;
  float* part_o;   // [n_req, Hq, n_splits, 16, dh]
  float* part_ml;  // [n_req, Hq, n_splits, 16, 2]
  unsigned int* err;
};

struct CombineParams {
  const float* part_o;
  const float* part_ml;
  int n_splits, Hq, B;
  void* out;  // storage dtype [n_req*B, Hq*dh]
  int ldo;
};

struct InjectReq {
  int row_start, count, slot, pos0, final_ctx;
};
struct ScatterParams {
  const float* kv;  // [rows, L*2*Hkv*dh]
  int rows, L, Hkv;
  int n_req;
  InjectReq req[kMaxChunkReq];
  const float* cos_t;
  const float* sin_t;
  void* pool;
  long long layer_stride;  // elements per layer in the pool
  const int* page_table;
  int pt_stride;
  SlotState* state;
  int window;
  int max_pages;
  unsigned int* err;
};

void launch_gemm(int dtype, int epi, const GemmParams& p, hipStream_t s);
void launch_rmsnorm(int dtype, const NormParams& p, hipStream_t s);
void launch_qkv_post(int dtype, int dh, int n_req, const QkvPostParams& p, const SlotArgs& sl,
                     hipStream_t s);
void launch_attention(int dtype, int dh, int n_req, const AttnParams& p, const SlotArgs& sl,
                      hipStream_t s);
void launch_combine(int dtype, int dh, int n_req, const CombineParams& p, hipStream_t s);
void launch_scatter(int dtype, int dh, const ScatterParams& p, hipStream_t s);
void launch_finalize(const unsigned long long* keys, int rows, int vocab, int* draft,
                     hipStream_t s);
void launch_verify(int n_req, int B, int vocab, const int* draft, const int* greedy,
                   int* accept, int* committed, int* last, unsigned int* err, hipStream_t s);

}  // namespace dflash
