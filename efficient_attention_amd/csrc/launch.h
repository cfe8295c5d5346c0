// Kernel parameter blocks and launchers (internal to liborthros.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

typedef int64_t idx_t;

// Bulk cache write (prefill / pre-training): k, v [B, T, Hkv, d] -> cache [B, Hkv, cap, d],
// len[b] = T for every sequence.
struct CacheWriteParams {
  const void* k;
  const void* v;
  void* ck;
  void* cv;
  int32_t* len;
  int B, T, Hkv, d, esize;
  int64_t cap;
};

// Decode append: cache row len[b] <- (k_new, v_new)[b]; len[b]++ unless the cache is full.
struct AppendParams {
  const void* knew;
  const void* vnew;  // [B, Hkv, d]
  void* ck;
  void* cv;
  int32_t* len;
  int32_t* status;
  int B, Hkv, d, esize;
  int64_t cap;
};

// Split-key few-row attention (bf16). One work-group per (split, kv head x head chunk, b).
// Row slots 0..nr_out-1 are output-stream rows (keys 0..n-1); with with_base, slots
// nr_out..2*nr_out-1 are base-stream rows over the window ending at the last key.
struct SplitParams {
  const void* q_out;
  const void* q_base;
  idx_t q_sb, q_sh;  // element strides of the [B, ..., Hq, d] query rows
  const float* a_out;
  const float* b_out;
  const float* a_base;
  const float* b_base;
  const void* k;
  const void* v;
  idx_t k_sb, k_sh, k_st;  // element strides: batch, kv head, token
  const void* knew;
  const void* vnew;
  idx_t kn_sb, kn_sh;    // decode: new key/value strides (batch, kv head)
  const int32_t* len;    // decode: device lengths (keys 0..len-1 cached, key len new)
  int64_t cap;           // decode: cache capacity (device lengths are clamped to it)
  int64_t n_fixed;       // prefill: number of keys
  int B, Hq, Hkv, G, HC, nchunks, window, nsplit, with_base;
  float scale_log2;
  float* pm;  // [rows][nsplit]
  float* pl;  // [rows][nsplit]
  float* po;  // [rows][nsplit][d]
};

// Split merge: row r = (b * Hq + h) * nstreams + stream.
struct MergeParams {
  const float* pm;
  const float* pl;
  const float* po;
  void* out0;  // stream 0 (output stream)
  void* out1;  // stream 1 (base stream, decode)
  idx_t o_sb0, o_sh0, o_sb1, o_sh1;
  int rows, nsplit, d, Hq, nstreams, bf16;
};

// Banded flash attention (bf16): rows t of q attend to keys max(0, t-w+1) .. t.
struct BandParams {
  const void* q;
  idx_t q_sb, q_st, q_sh;
  const float* alpha;
  const float* beta;
  const void* k;
  const void* v;
  idx_t k_sb, k_st, k_sh;
  void* o;
  idx_t o_sb, o_st, o_sh;
  int B, T, Hq, Hkv, G, window;
  float scale_log2;
};

// fp32 rows: one wave per (row, q head, b).
struct RowsF32Params {
  const float* q;
  idx_t q_sb, q_st, q_sh;
  const float* alpha;
  const float* beta;
  const float* k;
  const float* v;
  idx_t k_sb, k_st, k_sh;
  const float* knew;
  const float* vnew;
  idx_t kn_sb, kn_sh;
  const int32_t* len;  // decode: row position = len[b]
  int64_t cap;         // decode: cache capacity (device lengths are clamped to it)
  float* o;
  idx_t o_sb, o_st, o_sh;
  int B, Hq, Hkv, G, d, nrows, t0, window;
  float scale;
};

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_split_rows(const SplitParams& p, int d, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_band(const BandParams& p, int d, hipStream_t s);
hipError_t launch_rows_f32(const RowsF32Params& p, hipStream_t s);

}  // namespace orthros
