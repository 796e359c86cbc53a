// Internal interface of the skinny (few-token) GEMM used for every projection of the
// verify and draft paths: Y[m][n] = sum_k X[m][k] * W[n][k], W row-major [n][k].
#pragma once

#include "common.h"

namespace eagle {

// One segment of the activation source X.  Row m of the segment is row idx[m]
// (idx == nullptr: row m) of a row-major matrix with row stride ld (elements).
struct XSeg {
  const void* ptr;
  int dtype;  // EAGLE_BF16 / EAGLE_F32
  int64_t ld;
  const int32_t* idx;
};

// X = [segment a (k < ka) ; segment b (k >= ka)].  RMSNorm is applied as a per-row
// scale in the epilogue, W RMSNorm(x) = (W (gain * x)) * rsqrt(mean_k x[m][k]^2 + eps):
//   norm == 0: no norm;
//   norm == 1: the GEMM stages gain[k] * x[m][k] and accumulates sum_k x^2 itself;
//   norm == 2: X already holds gain * x (written by the producing epilogue) and the
//              row sums of squares come as np partials ssq_in[p][m], summed in order.
// The bf16 MFMA kernel takes bf16 segments only; the fp32 kernel takes either type.
struct XSrc {
  XSeg a, b;
  int ka;
  const void* gain;
  int gain_dtype;
  int norm;
  float eps;
  const float* ssq_in;
  int np;
};

enum EpiKind { EPI_STORE_F32 = 0, EPI_QKV = 1, EPI_RESID = 2, EPI_SILU = 3, EPI_ARGMAX = 4, EPI_TOPK = 5, EPI_SAMPLE = 6 };

struct Epi {
  int kind;
  // EPI_STORE_F32 / EPI_RESID: out[m][n] (+= resid[m][n])
  float* out;
  int64_t ld_out;
  const void* resid;
  int resid_dtype;
  int64_t ld_resid;
  const int32_t* resid_idx;  // row m of the residual is row resid_idx[m] (nullptr: m)
  // EPI_RESID extras for the next normed GEMM: xn[m][n] = bf16(xn_gain[n] * out[m][n])
  // (xn_gain nullptr: 1) and ssq_out[tile][m] = sum over the tile's columns of out^2
  void* xn_out;
  const void* xn_gain;
  float* ssq_out;
  // EPI_SILU: act[m][f] = SiLU(gate) * up, element type act_dtype
  void* act;
  int act_dtype;
  int64_t ld_act;
  // EPI_QKV: rotary at pos[m], scatter into q [m][hq][hd], k/v [m][hkv][hd] (element type out_dtype)
  void* q_out;
  void* k_out;
  void* v_out;
  int out_dtype;
  const int32_t* pos;
  const int32_t* kv_idx;  // k/v of row m go to row kv_idx[m] (< 0: dropped); nullptr: row m
  int hq, hkv, hd;
  float theta;
  // EPI_ARGMAX: per-row packed (value, ~index) keys merged with atomicMax; the last
  // workgroup unpacks them into argmax/max and clears keys and the counter.
  unsigned long long* keys;
  float* dbg_logits;
  int64_t ld_logits;
  int32_t* argmax_out;
  float* max_out;
  int* done;
  // EPI_TOPK: per (row, tile) the tile's top-k (value, index) and its (max, sum exp) pair,
  // row-major so that a row's candidates are contiguous for the per-row merge (n_part =
  // the launch's column tiles)
  float* topk_val;   // [m][n_part][topk]
  int32_t* topk_idx; // [m][n_part][topk]
  float* lse_part;   // [m][n_part][2]
  int topk;
  // EPI_SAMPLE: tempered logits v = inv_t * logit.  For every row c with a parent row
  // gparent[c] (-1: none) in the tile, the tile's value at (gparent[c], ctoken[c]), if
  // that column is in the tile, goes to child_logit[c] and is then left out; over the
  // remaining columns each (row, tile) gets (max v, sum exp(v - max)) and the largest
  // key of v + noise, written as one float4 (max, sum, key low word, key high word) to
  // samp_part[row * n_part + tile].  A child row lies at most max_nodes - 1 rows after
  // its parent.  Row m uses the noise row row_group[m] (< 0: row 0): noise of column c
  // is noise[row_group[m] * ld_noise + c].
  const float* noise;
  int64_t ld_noise;
  const int32_t* row_group;
  float inv_t;
  const int32_t* gparent;
  const int32_t* ctoken;
  int max_nodes;
  float* child_logit;
  float4* samp_part;
  int n_part;  // column tiles of the launch (EPI_SAMPLE, EPI_TOPK)
};

struct GemmDesc {
  const void* w0;
  const void* w1;  // second weight block (dual = 1: tile = gate columns + matching up columns)
  int dual;
  int dtype;       // EAGLE_BF16: MFMA path; EAGLE_F32: VALU path
  int w_layout;    // 0: row-major [n][ldw]; 1: fragment-blocked (eagle_pack_fragments; bf16 only)
  int n;           // output columns (rows of each weight block)
  int k;
  int64_t ldw;
  int m;           // tokens
  XSrc x;
  Epi epi;
  // planning (filled from the GemmPlan at launch)
  int cfg;
  int splits;
  int kps;  // K range per split (multiple of the kernel's K chunk)
  // workspace
  float* partials;
  float* sumsq_part;
  int* counters;
};

struct GemmPlan {
  int cfg;       // tile configuration
  int splits;    // K splits
  int kps;       // K per split
  int tile_cols; // output columns per epilogue tile
  int tile_rows; // weight rows per workgroup tile (both blocks when dual)
  int mt;        // tokens per tile
  int n_tiles;   // epilogue tiles along the output columns (what per-tile outputs are sized by)
  int w_tiles;   // workgroup tiles along the output columns (n_tiles / epilogue halves)
  int m_tiles;
};

GemmPlan plan_gemm(int dtype, int n, int k, int m, int dual, int epi_kind, int head_dim);
// Workspace floats for partials / sum-of-squares and ints for counters of one GEMM.
void gemm_workspace(const GemmPlan& p, size_t* partial_floats, size_t* sumsq_floats, size_t* counter_ints);
int launch_gemm(GemmDesc& d, const GemmPlan& p, hipStream_t s);
// Fragment-blocked copy of a row-major bf16 matrix (layout in eagle.h, eagle_pack_fragments).
void launch_pack_fragments(const void* w, int rows, int cols, void* out, hipStream_t s);

}  // namespace eagle
