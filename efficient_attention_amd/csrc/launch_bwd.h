// Kernel parameter blocks and launchers of the training backward (internal to liborthros.so).
#pragma once

#include "launch.h"

namespace orthros {

// Training backward of one stream's rows: the row at position t (of [B, nrows, Hq, d]) attends
// keys lo(t) .. t with lo(t) = max(0, t - window + 1) of k, v [B, T, Hkv, d].
struct BwdQParams {
  const void* q;           // raw queries of the stream
  const float* alpha;      // the stream's scale-offset [Hq d]
  const float* beta;
  const void* k;
  const void* v;
  const void* o;           // forward output of the stream
  const void* dout;        // its gradient
  const float* lse;        // [B, Hq, nrows] natural-log log-sum-exp of the forward rows
  float* D;                // out: [B, Hq, nrows] rowsum(dout * o); the bf16 kernel stores -D
  float* lse2n;            // out (bf16 kernel): [B, Hq, nrows] -lse in log2 units
  float* dq;               // out (fp32 kernel): [B, nrows, Hq, d] gradient of the post-affine query
  // bf16 kernel with part set: instead of dq, the raw query's gradient dq_raw = alpha (.) dq
  // (bf16, [B, nrows, Hq, d]) and, per 32-row tile and head, the tile's sums of dq (.) q_raw and
  // dq into part[(b nrt + tile) 2 + {0, 1}][Hq d] (nrt = row tiles per sequence)
  const void* qraw;
  void* dq_raw;
  float* part;
  int nrt;
  const int32_t* pos;      // optional: row r sits at position pos[r] (clamped into [0, T));
                           // without it, rows are positions (nrows = T)
  int nrows;
  int B, T, Hq, Hkv, G, window;
  float scale;
};

// Key-side backward: dk, dv [B, T, Hkv, d] from both streams' rows (index 0 base, 1 output);
// a stream's rows are its positions (nrows = T) or a row list pos (as in BwdQParams).
struct BwdKVParams {
  const int32_t* pos[2];
  int nrows[2];
  const void* q[2];
  const float* alpha[2];
  const float* beta[2];
  const void* dout[2];
  const float* lse[2];     // fp32 kernel: the forward's lse; bf16 kernel: -lse in log2 units
  const float* D[2];       // fp32 kernel: rowsum(dout * o); bf16 kernel: its negation
  int window[2];
  const void* k;
  const void* v;
  void* dk;
  void* dv;
  int B, T, Hq, Hkv, G;
  float scale;
};

// Query-side scale-offset gradient of one stream: dq_raw = alpha (.) dq, and the sums over
// all rows of dq (.) q_raw (d alpha) and dq (d beta), in a fixed order (two passes).
struct AffineGradParams {
  const float* dq;         // [rows, n] fp32 post-affine gradient
  const void* q;           // [rows, n] raw queries
  const float* alpha;      // [n]
  void* dq_raw;            // out: [rows, n] in the call's dtype
  float* part;             // [nchunk][2][n] partial sums
  float* dalpha;           // out: [n]
  float* dbeta;            // out: [n]
  int rows, n, chunk_rows, nchunk, bf16;
};

hipError_t launch_bwd_q_f32(const BwdQParams& p, int d, hipStream_t s);
hipError_t launch_bwd_kv_f32(const BwdKVParams& p, int d, hipStream_t s);
hipError_t launch_bwd_q_bf16(const BwdQParams& p, int d, hipStream_t s);
// Both streams' query sides (same shape and head grouping) in one launch, p0's work first.
hipError_t launch_bwd_q_bf16_pair(const BwdQParams& p0, const BwdQParams& p1, int d, hipStream_t s);
hipError_t launch_bwd_kv_bf16(const BwdKVParams& p, int d, hipStream_t s);
hipError_t launch_affine_grad(const AffineGradParams& p, hipStream_t s);
// Only the fixed-order sums of the p[i].nchunk partials of `count` (1 or 2) streams in one launch
// (the bf16 query-side kernel writes the partials).
hipError_t launch_affine_grad_final(const AffineGradParams* p, int count, hipStream_t s);
hipError_t launch_qprep(const void* q0, const void* q1, const float* a0, const float* b0,
                        const float* a1, const float* b1, void* o0, void* o1, idx_t n, int hd,
                        float c, hipStream_t s, int nstreams);

}  // namespace orthros
