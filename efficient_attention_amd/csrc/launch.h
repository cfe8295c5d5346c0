// Kernel parameter blocks and launchers (internal to liborthros.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orthros {

typedef int64_t idx_t;

constexpr int32_t kStatusCacheFull = 1;  // ORTHROS_STATUS_CACHE_FULL
constexpr int32_t kStatusBadPage = 2;    // ORTHROS_STATUS_BAD_PAGE

// Paged key/value cache: a pool [num_pages, Hkv, 2^ps_log2, d] shared by the batch. Token t of
// sequence b is slot t mod 2^ps_log2 of page table[b * tbl_sb + (t >> ps_log2)]; k_sp and k_sh
// are the element strides between pages and between the kv heads of a page. table == nullptr
// means the cache is the contiguous [B, Hkv, cap, d] one.
struct PagedKV {
  const int32_t* table;
  idx_t tbl_sb;
  int64_t num_pages;
  idx_t k_sp, k_sh;
  int ps_log2;
  int32_t* status;  // sticky status word (bit kStatusBadPage)
};

// Element offset of token `key` within kv head 0 of the pool, for the sequence whose table row
// is `tbl` (rows are k_st elements apart inside a page). The key is clamped into [0, cap) so
// the table read stays inside the row. A page index outside [0, num_pages) sets kStatusBadPage
// and *bad, and page 0 stands in for it (readers then stay in bounds; writers must skip).
__device__ __forceinline__ idx_t paged_offset(const PagedKV& pk, const int32_t* tbl, int64_t key,
                                              int64_t cap, idx_t k_st, bool* bad = nullptr) {
  if (key > cap - 1) key = cap - 1;
  if (key < 0) key = 0;
  int32_t page = tbl[key >> pk.ps_log2];
  if (page < 0 || (int64_t)page >= pk.num_pages) {
    __hip_atomic_fetch_or(pk.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (bad) *bad = true;
    page = 0;
  }
  return (idx_t)page * pk.k_sp + (key & (((int64_t)1 << pk.ps_log2) - 1)) * k_st;
}

// Bulk cache write (prefill / pre-training): k, v [B, T, Hkv, d] -> cache [B, Hkv, cap, d],
// len[b] = T for every sequence.
// Rows t of k, v go to cache rows t_first + t; len[b] = t_first + T afterwards.
struct CacheWriteParams {
  const void* k;
  const void* v;
  void* ck;
  void* cv;
  int32_t* len;
  int B, T, Hkv, d, esize;
  int64_t cap;
  int64_t t_first;
  int in_place;  // k, v are the cache rows themselves: only len is set
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
  PagedKV pg;  // paged pool (ck / cv point at it) when pg.table is set
};

// Paged bulk write: token t of k, v [B, T, Hkv, d] goes to position len[b] + t of the paged
// cache (a sequence without room for all T tokens is skipped); paged_advance then moves len,
// except for sequences with no room or with a bad table entry among those positions.
struct PagedWriteParams {
  const void* k;
  const void* v;
  void* ck;
  void* cv;
  int32_t* len;
  int B, T, Hkv, d, esize;
  int64_t cap;
  PagedKV pg;
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
  int64_t n_fixed;       // prefill / SFT: number of keys
  // SFT rows: when pos is set, the output rows of one kv head are the R x G pairs
  // (response row r, head of the group), row r at position pos[r] (keys 0 .. pos[r]), its
  // query at q_out + b q_sb + r q_st + h q_sh; chunks of 16 pairs.
  const int32_t* pos;
  int R;
  idx_t q_st;
  int B, Hq, Hkv, G, HC, nchunks, window, nsplit, with_base;
  float scale_log2;
  PagedKV pg;  // decode over a paged pool (k / v point at it; k_sh, k_sb unused) when set
  float* pm;  // [rows][nsplit]
  float* pl;  // [rows][nsplit]
  float* po;  // [rows][nsplit][d]
};

// Split merge: row r = (b * Hq + h) * nstreams + stream. With rows_out0 set, every "stream" is
// a row index written to out0 + b o_sb0 + stream o_st0 + h o_sh0 (SFT response rows).
struct MergeParams {
  const float* pm;
  const float* pl;
  const float* po;
  void* out0;  // stream 0 (output stream)
  void* out1;  // stream 1 (base stream, decode)
  idx_t o_sb0, o_sh0, o_sb1, o_sh1, o_st0;
  float* lse;  // optional: natural-log log-sum-exp of row r at lse[r]
  int rows, nsplit, d, Hq, nstreams, bf16, rows_out0;
};

// Banded flash attention (bf16). Query row r (0 <= r < nrows; q and o are indexed by r) sits at
// position t_r = pos[r] if pos is set, else t_first + r, and attends to keys
// max(0, t_r - w + 1) .. t_r of k / v, which are indexed by position (keys 0 .. nkeys - 1 exist;
// every t_r must be below nkeys).
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
  const int32_t* pos;  // optional device row positions (nrows of them)
  PagedKV pg;          // optional paged pool (k / v point at it, k_st = d): pages of >= 64 rows
  float* lse;          // optional: natural-log log-sum-exp of row r, head h at b lse_sb + h lse_sh + r
  idx_t lse_sb, lse_sh;
  int B, nrows, nkeys, t_first, Hq, Hkv, G, window;
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
  const int32_t* pos;  // optional row positions (row r at pos[r], clamped to [0, nkeys))
  int64_t nkeys;       // with pos: keys available
  PagedKV pg;          // decode over a paged pool (k / v point at it) when pg.table is set
  float* lse;          // optional: natural-log log-sum-exp of each row (b lse_sb + h lse_sh + row)
  idx_t lse_sb, lse_sh;
  float* o;
  idx_t o_sb, o_st, o_sh;
  int B, Hq, Hkv, G, d, nrows, t0, window;
  float scale;
};

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s);
hipError_t launch_append(const AppendParams& p, hipStream_t s);
hipError_t launch_paged_write(const PagedWriteParams& p, hipStream_t s);
hipError_t launch_split_rows(const SplitParams& p, int d, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, hipStream_t s);
hipError_t launch_band(const BandParams& p, int d, hipStream_t s);
// p0's and p1's rows (same shape and head grouping, same keys) in one launch, p0's first.
hipError_t launch_band_pair(const BandParams& p0, const BandParams& p1, int d, hipStream_t s);
hipError_t launch_rows_f32(const RowsF32Params& p, hipStream_t s);

}  // namespace orthros
