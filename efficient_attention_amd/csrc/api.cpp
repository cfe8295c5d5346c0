// C ABI of liborthros.so: argument validation, workspace layout, kernel dispatch and the
// optional per-stage timing. See include/orthros.h for the contract of every entry point.
#include "orthros.h"

#include <hip/hip_runtime_api.h>

#include <climits>
#include <cmath>
#include <mutex>
#include <vector>

#include "launch.h"
#include "launch_bwd.h"

using namespace orthros;

namespace {

constexpr int kMaxSplits = 64;     // split partials reserved per row in the workspace
constexpr float kLog2e = 1.4426950408889634f;
constexpr size_t kStatusBytes = 256;

struct WsLayout {
  size_t pm, pl, po, total;
};

constexpr int64_t kSftSplitRows = 16;  // SFT: up to this many response rows use split-key rows

// rows_per_head: split-partial rows reserved per (sequence, query head); 2 covers prefill's
// output row and decode's pair, SFT reserves one per response row when it uses split rows.
WsLayout ws_layout(const orthros_shape* s, int64_t rows_per_head = 2) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = (size_t)s->batch * s->num_q_heads * (size_t)rows_per_head;
  WsLayout L;
  L.pm = kStatusBytes;
  L.pl = L.pm + up(rows * kMaxSplits * sizeof(float));
  L.po = L.pl + up(rows * kMaxSplits * sizeof(float));
  L.total = L.po + up(rows * kMaxSplits * (size_t)s->head_dim * sizeof(float));
  return L;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_shape(const orthros_shape* s) {
  if (!s) return ORTHROS_E_INVALID;
  if (s->batch < 1 || s->num_q_heads < 1 || s->num_kv_heads < 1 || s->window < 1 ||
      s->capacity < 1 || s->reserved != 0)
    return ORTHROS_E_INVALID;
  if (s->num_q_heads % s->num_kv_heads) return ORTHROS_E_INVALID;
  if (!(s->softmax_scale <= 0.f) && !std::isfinite(s->softmax_scale)) return ORTHROS_E_INVALID;
  if (s->dtype != ORTHROS_F32 && s->dtype != ORTHROS_BF16) return ORTHROS_E_UNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128) return ORTHROS_E_UNSUPPORTED;
  if (s->batch > 65535) return ORTHROS_E_UNSUPPORTED;
  return ORTHROS_OK;
}

int check_affine(const orthros_affine* a) {
  if (!a) return ORTHROS_E_INVALID;
  const void* ps[4] = {a->alpha_base, a->beta_base, a->alpha_out, a->beta_out};
  for (const void* p : ps)
    if (!p || !aligned16(p)) return ORTHROS_E_INVALID;
  return ORTHROS_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (!p || !aligned16(p)) return ORTHROS_E_INVALID;
  return ORTHROS_OK;
}

int check_ws(const orthros_shape* s, const void* ws, size_t bytes, int64_t rows_per_head = 2) {
  if (!ws || !aligned16(ws)) return ORTHROS_E_WORKSPACE;
  if (bytes < ws_layout(s, rows_per_head).total) return ORTHROS_E_WORKSPACE;
  return ORTHROS_OK;
}

int64_t sft_rows_per_head(int64_t R) { return R <= kSftSplitRows ? (R > 2 ? R : 2) : 2; }

float scale_of(const orthros_shape* s) {
  return s->softmax_scale > 0.f ? s->softmax_scale : 1.f / std::sqrt((float)s->head_dim);
}

int esize(const orthros_shape* s) { return s->dtype == ORTHROS_BF16 ? 2 : 4; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// How T tokens of keys/values [B, T, H_kv, d] reach cache rows t_first .. t_first + T - 1 of
// the head-major cache: copied (*copy = true), or already there, when k and v are the cache's
// own rows. The two layouts describe the same bytes only with one kv head and with B == 1 or
// capacity == T; any other overlap with the cache is an error.
int kv_source(const orthros_shape* s, int64_t T, int64_t t_first, const void* k, const void* v,
              const void* ck, const void* cv, bool* copy) {
  const size_t es = (size_t)esize(s), d = (size_t)s->head_dim;
  const size_t kvb = (size_t)s->batch * (size_t)T * s->num_kv_heads * d * es;
  const size_t cb = (size_t)s->batch * s->num_kv_heads * (size_t)s->capacity * d * es;
  const char* kd = static_cast<const char*>(ck) + (size_t)t_first * d * es;
  const char* vd = static_cast<const char*>(cv) + (size_t)t_first * d * es;
  if (k == kd && v == vd && s->num_kv_heads == 1 && (s->batch == 1 || s->capacity == T)) {
    *copy = false;
    return ORTHROS_OK;
  }
  for (const void* src : {k, v})
    for (const void* dst : {ck, cv})
      if (overlap(src, kvb, dst, cb)) return ORTHROS_E_INVALID;
  *copy = true;
  return ORTHROS_OK;
}

// Keys/values [B, T, H_kv, d] must not overlap a paged pool they are written into.
int kv_outside_pool(const orthros_shape* s, int64_t T, const void* k, const void* v,
                    const orthros_paged_kv* c) {
  const size_t es = (size_t)esize(s), d = (size_t)s->head_dim;
  const size_t kvb = (size_t)s->batch * (size_t)T * s->num_kv_heads * d * es;
  const size_t pb = (size_t)c->num_pages * s->num_kv_heads * (size_t)c->page_size * d * es;
  for (const void* src : {k, v})
    for (const void* dst : {(const void*)c->k_pages, (const void*)c->v_pages})
      if (overlap(src, kvb, dst, pb)) return ORTHROS_E_INVALID;
  return ORTHROS_OK;
}

// ---------------------------------------------------------------------------------------------
// Optional timing: event pairs around every launch while enabled.
struct TimingRec {
  int stage;
  hipEvent_t a, b;
};
struct Timing {
  bool on = false;
  std::vector<TimingRec> recs;
} g_timing;

template <class F>
hipError_t run_stage(int stage, hipStream_t st, F&& f, bool timed = true) {
  if (!g_timing.on || !timed) return f();
  TimingRec r{stage, nullptr, nullptr};
  if (hipEventCreate(&r.a) != hipSuccess || hipEventCreate(&r.b) != hipSuccess) return hipErrorUnknown;
  (void)hipEventRecord(r.a, st);
  const hipError_t e = f();
  (void)hipEventRecord(r.b, st);
  g_timing.recs.push_back(r);
  return e;
}

int launch_rc(hipError_t e) { return e == hipSuccess ? ORTHROS_OK : ORTHROS_E_LAUNCH; }

// Split count for the few-row kernel. Its LDS ring leaves room for one work-group per compute
// unit at head_dim 128 and two at 64, so a launch runs in waves of that many groups per unit:
// pick the split count that minimises (waves x keys per split) plus the merge work per split.
int nsplit_for(int64_t n, int64_t groups, int d) {
  const int64_t kResident = (d == 128 ? 1 : 2) * 256;
  const int64_t tiles = (n + 63) / 64;
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= kMaxSplits && s <= tiles; ++s) {
    const int64_t per = ((n + s - 1) / s + 63) / 64 * 64;
    const int64_t waves = (groups * s + kResident - 1) / kResident;
    const double cost = (double)waves * (double)per + 64.0 * s;  // + merge work per split
    if (cost < best_cost * (1 - 1e-9)) {
      best_cost = cost;
      best = s;
    }
  }
  return best;
}

int heads_per_chunk(int G, bool with_base) {
  const int cap = with_base ? 8 : 16;
  return G < cap ? G : cap;
}

// Paged cache arguments -> kernel view. Page indices are int32, the page size a power of two,
// and the per-sequence capacity (max_pages pages) must be the shape's capacity.
int check_paged(const orthros_shape* s, const orthros_paged_kv* c, void* ws, PagedKV* out) {
  if (!c) return ORTHROS_E_INVALID;
  if (check_ptrs({c->k_pages, c->v_pages, c->block_table})) return ORTHROS_E_INVALID;
  if (c->num_pages < 1 || c->num_pages > INT32_MAX || c->max_pages < 1) return ORTHROS_E_INVALID;
  if (c->page_size < 1 || c->page_size > (1 << 24) || (c->page_size & (c->page_size - 1)))
    return ORTHROS_E_INVALID;
  if ((int64_t)c->max_pages * c->page_size != s->capacity) return ORTHROS_E_INVALID;
  int lg = 0;
  while ((1 << lg) < c->page_size) ++lg;
  out->table = c->block_table;
  out->tbl_sb = c->max_pages;
  out->num_pages = c->num_pages;
  out->k_sh = (idx_t)c->page_size * s->head_dim;
  out->k_sp = out->k_sh * s->num_kv_heads;
  out->ps_log2 = lg;
  out->status = reinterpret_cast<int32_t*>(ws);
  return ORTHROS_OK;
}

// Split count of a decode step: the split grid is sized by the host bound on the lengths.
int decode_nsplit(const orthros_shape* s, int64_t max_len_hint) {
  const int64_t hint = max_len_hint < s->capacity ? max_len_hint : s->capacity;
  const int G = s->num_q_heads / s->num_kv_heads;
  const int nchunks = (G + heads_per_chunk(G, true) - 1) / heads_per_chunk(G, true);
  return nsplit_for(hint + 1, (int64_t)s->batch * s->num_kv_heads * nchunks, s->head_dim);
}

// Where a decode step keeps its split partials ([rows][nsplit] maxima and sums, [rows][nsplit][d]
// partial outputs, rows = 2 B H_q) and its sticky status word.
struct DecodeScratch {
  float* pm;
  float* pl;
  float* po;
  int32_t* status;
};

// One decode step over a contiguous cache (pg.table == nullptr) or a paged pool. Arguments
// are validated by the callers; `timed` lets the per-stage timing record events around its
// launches.
int decode_common(const orthros_shape* s, const void* q_base, const void* q_out,
                  const void* k_new, const void* v_new, const orthros_affine* aff,
                  void* cache_k, void* cache_v, const PagedKV& pg, int32_t* cache_len,
                  int64_t max_len_hint, void* o_base, void* o_out, const DecodeScratch& sc,
                  bool timed, hipStream_t st) {
  int rc;
  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);

  if (s->dtype == ORTHROS_F32) {
    RowsF32Params r{};
    r.q = static_cast<const float*>(q_base);
    r.q_sb = (idx_t)Hq * d; r.q_st = 0; r.q_sh = d;
    r.alpha = aff->alpha_base; r.beta = aff->beta_base;
    r.k = static_cast<const float*>(cache_k); r.v = static_cast<const float*>(cache_v);
    r.k_sb = (idx_t)Hkv * s->capacity * d; r.k_st = d; r.k_sh = s->capacity * d;
    r.pg = pg;
    r.knew = static_cast<const float*>(k_new); r.vnew = static_cast<const float*>(v_new);
    r.kn_sb = (idx_t)Hkv * d; r.kn_sh = d;
    r.len = cache_len; r.cap = s->capacity;
    r.o = static_cast<float*>(o_base); r.o_sb = (idx_t)Hq * d; r.o_st = 0; r.o_sh = d;
    r.B = B; r.Hq = Hq; r.Hkv = Hkv; r.G = G; r.d = d; r.nrows = 1; r.t0 = 0;
    r.window = s->window; r.scale = scale;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(r, st); }, timed));
    if (rc) return rc;
    RowsF32Params o = r;
    o.q = static_cast<const float*>(q_out);
    o.alpha = aff->alpha_out; o.beta = aff->beta_out;
    o.o = static_cast<float*>(o_out);
    o.window = INT_MAX;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(o, st); }, timed));
    if (rc) return rc;
  } else {
    SplitParams sp{};
    sp.q_out = q_out; sp.q_base = q_base; sp.q_sb = (idx_t)Hq * d; sp.q_sh = d;
    sp.a_out = aff->alpha_out; sp.b_out = aff->beta_out;
    sp.a_base = aff->alpha_base; sp.b_base = aff->beta_base;
    sp.k = cache_k; sp.v = cache_v;
    sp.k_sb = (idx_t)Hkv * s->capacity * d; sp.k_sh = s->capacity * d; sp.k_st = d;
    sp.pg = pg;
    sp.knew = k_new; sp.vnew = v_new; sp.kn_sb = (idx_t)Hkv * d; sp.kn_sh = d;
    sp.len = cache_len; sp.cap = s->capacity;
    sp.B = B; sp.Hq = Hq; sp.Hkv = Hkv; sp.G = G;
    sp.HC = heads_per_chunk(G, true);
    sp.nchunks = (G + sp.HC - 1) / sp.HC;
    sp.window = s->window; sp.with_base = 1;
    sp.nsplit = decode_nsplit(s, max_len_hint);
    sp.scale_log2 = scale * kLog2e;
    sp.pm = sc.pm;
    sp.pl = sc.pl;
    sp.po = sc.po;
    rc = launch_rc(run_stage(ORTHROS_STAGE_SPLIT_ROWS, st, [&] { return launch_split_rows(sp, d, st); }, timed));
    if (rc) return rc;
    MergeParams mp{};
    mp.pm = sp.pm; mp.pl = sp.pl; mp.po = sp.po;
    mp.out0 = o_out; mp.o_sb0 = (idx_t)Hq * d; mp.o_sh0 = d;
    mp.out1 = o_base; mp.o_sb1 = (idx_t)Hq * d; mp.o_sh1 = d;
    mp.rows = B * Hq * 2; mp.nsplit = sp.nsplit; mp.d = d; mp.Hq = Hq; mp.nstreams = 2; mp.bf16 = 1;
    rc = launch_rc(run_stage(ORTHROS_STAGE_MERGE, st, [&] { return launch_merge(mp, st); }, timed));
    if (rc) return rc;
  }
  AppendParams ap{k_new, v_new, cache_k, cache_v, cache_len, sc.status, B, Hkv, d, esize(s),
                  s->capacity, pg};
  return launch_rc(run_stage(ORTHROS_STAGE_APPEND, st, [&] { return launch_append(ap, st); }, timed));
}

// Checks shared by the decode entry points (the cache pointers are checked by each).
int check_decode_args(const void* q_base, const void* q_out, const void* k_new,
                      const void* v_new, const orthros_affine* aff, int32_t* cache_len,
                      int64_t max_len_hint, void* o_base, void* o_out) {
  int rc;
  if (max_len_hint < 0) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  return check_ptrs({q_base, q_out, k_new, v_new, cache_len, o_base, o_out});
}

DecodeScratch workspace_scratch(const orthros_shape* s, void* ws) {
  const WsLayout L = ws_layout(s);
  char* w = static_cast<char*>(ws);
  return DecodeScratch{reinterpret_cast<float*>(w + L.pm), reinterpret_cast<float*>(w + L.pl),
                       reinterpret_cast<float*>(w + L.po), reinterpret_cast<int32_t*>(w)};
}

// ---------------------------------------------------------------------------------------------
// The split partials of orthros_decode_step_noalloc live in this array, not in a caller's
// workspace. Each device holds its own copy from the moment the library's code is loaded
// onto it until the process ends. In host code the name stands for a host-side shadow, not
// for device memory: every use goes through the device address looked up below.
static __device__ __align__(256) unsigned char scratch[ORTHROS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per device (the first
// call with that device current) and kept.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return ORTHROS_E_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return ORTHROS_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ORTHROS_E_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ORTHROS_OK;
}

// Split partials packed for the step's own split count, each array 256-byte aligned.
struct NoAllocLayout {
  size_t pm, pl, po, total;
};
NoAllocLayout noalloc_layout(const orthros_shape* s, int nsplit) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows = 2 * (size_t)s->batch * s->num_q_heads;
  NoAllocLayout L;
  L.pm = 0;
  L.pl = up(rows * nsplit * sizeof(float));
  L.po = L.pl + up(rows * nsplit * sizeof(float));
  L.total = L.po + up(rows * nsplit * (size_t)s->head_dim * sizeof(float));
  return L;
}

// Backward workspace: status word | q' per stream (bf16) | D per stream | -lse per stream (bf16) |
// fp32 calls: fp32 dq per stream and the 16-row scale-offset partials | bf16 calls: per-stream
// scale-offset partials of 32-row tiles (the query-side kernel writes them).
struct BwdLayout {
  size_t qp[2], D[2], L2[2], dq[2], part, partq[2], total;
  int chunk_rows, nchunk, nrt[2];
};
// R: rows of the output stream (T for pre-training, the response rows for fine-tuning).
BwdLayout bwd_layout(const orthros_shape* s, int64_t T, int64_t R) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t rows[2] = {(size_t)s->batch * (size_t)T, (size_t)s->batch * (size_t)R};
  const size_t n = (size_t)s->num_q_heads * s->head_dim;
  BwdLayout L;
  L.chunk_rows = 16;  // rows per partial-sum chunk: enough work-groups to keep HBM busy
  const size_t rmax = rows[0] > rows[1] ? rows[0] : rows[1];
  L.nchunk = (int)((rmax + L.chunk_rows - 1) / L.chunk_rows);
  size_t off = kStatusBytes;
  for (int i = 0; i < 2; ++i) {
    L.qp[i] = off;
    off += s->dtype == ORTHROS_BF16 ? up(rows[i] * n * 2) : 0;
  }
  for (int i = 0; i < 2; ++i) { L.D[i] = off; off += up(rows[i] * s->num_q_heads * 4); }
  for (int i = 0; i < 2; ++i) {  // -lse in log2 units, the bf16 key side's score seed
    L.L2[i] = off;
    off += s->dtype == ORTHROS_BF16 ? up(rows[i] * s->num_q_heads * 4) : 0;
  }
  const bool bf = s->dtype == ORTHROS_BF16;
  for (int i = 0; i < 2; ++i) { L.dq[i] = off; off += bf ? 0 : up(rows[i] * n * 4); }
  L.part = off;
  off += bf ? 0 : up((size_t)L.nchunk * 2 * n * 4);
  const int64_t per_seq[2] = {T, R};
  for (int i = 0; i < 2; ++i) {
    L.nrt[i] = (int)((per_seq[i] + 31) / 32);
    L.partq[i] = off;
    off += bf ? up((size_t)s->batch * L.nrt[i] * 2 * n * 4) : 0;
  }
  L.total = off;
  return L;
}

int forward_pt_impl(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                    const void* k, const void* v, const orthros_affine* aff, void* cache_k,
                    void* cache_v, int32_t* cache_len, void* o_base, void* o_out, float* lse_b,
                    float* lse_o, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T < 1 || T > INT_MAX / 2) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  if ((rc = check_ptrs({q_base, q_out, k, v, o_base, o_out}))) return rc;
  const bool any_cache = cache_k || cache_v || cache_len;
  if (any_cache && (rc = check_ptrs({cache_k, cache_v, cache_len}))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (any_cache && T > s->capacity) return ORTHROS_E_INVALID;
  bool copy = true;
  if (any_cache && (rc = kv_source(s, T, 0, k, v, cache_k, cache_v, &copy))) return rc;

  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);

  if (any_cache) {
    CacheWriteParams cw{k, v, cache_k, cache_v, cache_len, B, (int)T, Hkv, d, esize(s), s->capacity,
                        0, copy ? 0 : 1};
    rc = launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_cache_write(cw, st); }));
    if (rc) return rc;
  }

  if (s->dtype == ORTHROS_F32) {
    RowsF32Params r{};
    r.q = static_cast<const float*>(q_base);
    r.q_sb = T * Hq * d; r.q_st = (idx_t)Hq * d; r.q_sh = d;
    r.alpha = aff->alpha_base; r.beta = aff->beta_base;
    r.k = static_cast<const float*>(k); r.v = static_cast<const float*>(v);
    r.k_sb = T * Hkv * d; r.k_st = (idx_t)Hkv * d; r.k_sh = d;
    r.o = static_cast<float*>(o_base);
    r.o_sb = T * Hq * d; r.o_st = (idx_t)Hq * d; r.o_sh = d;
    r.B = B; r.Hq = Hq; r.Hkv = Hkv; r.G = G; r.d = d; r.nrows = (int)T; r.t0 = 0;
    r.window = s->window; r.scale = scale;
    r.lse = lse_b; r.lse_sb = (idx_t)Hq * T; r.lse_sh = T;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(r, st); }));
    if (rc) return rc;
    RowsF32Params o = r;
    o.q = static_cast<const float*>(q_out);
    o.alpha = aff->alpha_out; o.beta = aff->beta_out;
    o.o = static_cast<float*>(o_out);
    o.window = INT_MAX;
    o.lse = lse_o;
    return launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(o, st); }));
  }

  BandParams bp{};
  bp.q = q_base; bp.q_sb = T * Hq * d; bp.q_st = (idx_t)Hq * d; bp.q_sh = d;
  bp.alpha = aff->alpha_base; bp.beta = aff->beta_base;
  bp.k = k; bp.v = v; bp.k_sb = T * Hkv * d; bp.k_st = (idx_t)Hkv * d; bp.k_sh = d;
  bp.o = o_base; bp.o_sb = T * Hq * d; bp.o_st = (idx_t)Hq * d; bp.o_sh = d;
  bp.B = B; bp.nrows = (int)T; bp.nkeys = (int)T; bp.t_first = 0; bp.pos = nullptr;
  bp.Hq = Hq; bp.Hkv = Hkv; bp.G = G;
  bp.window = s->window < (int)T ? s->window : (int)T;
  bp.scale_log2 = scale * kLog2e;
  bp.lse = lse_b; bp.lse_sb = (idx_t)Hq * T; bp.lse_sh = T;
  rc = launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band(bp, d, st); }));
  if (rc) return rc;
  BandParams op = bp;
  op.q = q_out; op.alpha = aff->alpha_out; op.beta = aff->beta_out; op.o = o_out;
  op.lse = lse_o;
  op.window = (int)T;  // window >= T: full causal rows (Eq. 5)
  return launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band(op, d, st); }));
}


// Backward of pre-training (out_pos == nullptr, R == T) or fine-tuning (R response rows at
// out_pos).
int backward_impl(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                  const int32_t* out_pos, int64_t R, const void* k, const void* v,
                  const orthros_affine* aff, const void* o_base, const void* o_out,
                  const float* lse_base, const float* lse_out, const void* do_base,
                  const void* do_out, void* dq_base, void* dq_out, void* dk, void* dv,
                  const orthros_affine_grad* dg, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T < 1 || T > INT_MAX / 2 || R < 1 || R > INT_MAX / 2) return ORTHROS_E_INVALID;
  if (out_pos && ((uintptr_t)out_pos & 3u)) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  if ((rc = check_ptrs({q_base, q_out, k, v, o_base, o_out, lse_base, lse_out, do_base, do_out,
                        dq_base, dq_out, dk, dv}))) return rc;
  if (!dg || check_ptrs({dg->dalpha_base, dg->dbeta_base, dg->dalpha_out, dg->dbeta_out}))
    return ORTHROS_E_INVALID;
  if (!ws || !aligned16(ws)) return ORTHROS_E_WORKSPACE;
  const BwdLayout L = bwd_layout(s, T, R);
  if (ws_bytes < L.total) return ORTHROS_E_WORKSPACE;

  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);
  char* w = static_cast<char*>(ws);
  const bool bf = s->dtype == ORTHROS_BF16;
  const int wb = s->window < (int)T ? s->window : (int)T;

  const void* qs[2] = {q_base, q_out};
  const float* al[2] = {aff->alpha_base, aff->alpha_out};
  const float* be[2] = {aff->beta_base, aff->beta_out};
  const void* os[2] = {o_base, o_out};
  const void* dos[2] = {do_base, do_out};
  const float* lses[2] = {lse_base, lse_out};
  float* Ds[2] = {reinterpret_cast<float*>(w + L.D[0]), reinterpret_cast<float*>(w + L.D[1])};
  float* l2s[2] = {reinterpret_cast<float*>(w + L.L2[0]), reinterpret_cast<float*>(w + L.L2[1])};
  float* dqs[2] = {reinterpret_cast<float*>(w + L.dq[0]), reinterpret_cast<float*>(w + L.dq[1])};
  void* qps[2] = {w + L.qp[0], w + L.qp[1]};
  const int wins[2] = {wb, (int)T};
  const int nrows[2] = {(int)T, (int)R};
  const int32_t* poss[2] = {nullptr, out_pos};
  void* dqo[2] = {dq_base, dq_out};
  if (bf && nrows[0] == nrows[1]) {  // one launch prepares both streams' score operands
    rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_Q, st, [&] {
      return launch_qprep(qs[0], qs[1], al[0], be[0], al[1], be[1], qps[0], qps[1],
                          (idx_t)B * nrows[0] * Hq * d, Hq * d, scale * kLog2e, st, 2);
    }));
    if (rc) return rc;
  } else if (bf) {
    for (int i = 0; i < 2; ++i) {
      rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_Q, st, [&] {
        return launch_qprep(qs[i], qs[i], al[i], be[i], al[i], be[i], qps[i], qps[i],
                            (idx_t)B * nrows[i] * Hq * d, Hq * d, scale * kLog2e, st, 1);
      }));
      if (rc) return rc;
    }
  }
  BwdQParams qp2[2] = {};
  for (int i = 0; i < 2; ++i) {
    BwdQParams q{};
    q.q = bf ? qps[i] : qs[i];
    q.alpha = al[i]; q.beta = be[i];
    q.k = k; q.v = v; q.o = os[i]; q.dout = dos[i]; q.lse = lses[i];
    q.D = Ds[i]; q.lse2n = bf ? l2s[i] : nullptr; q.dq = bf ? nullptr : dqs[i];
    if (bf) {  // the scale-offset step runs in the query-side kernel's epilogue
      q.qraw = qs[i]; q.dq_raw = dqo[i];
      q.part = reinterpret_cast<float*>(w + L.partq[i]); q.nrt = L.nrt[i];
    }
    q.pos = poss[i]; q.nrows = nrows[i];
    q.B = B; q.T = (int)T; q.Hq = Hq; q.Hkv = Hkv; q.G = G; q.window = wins[i]; q.scale = scale;
    qp2[i] = q;
    if (bf) continue;  // both bf16 query sides go in one launch below
    rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_Q, st, [&] { return launch_bwd_q_f32(q, d, st); }));
    if (rc) return rc;
  }
  if (bf) {  // the output stream's (longer, causal) rows first, the base rows after them
    rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_Q, st, [&] { return launch_bwd_q_bf16_pair(qp2[1], qp2[0], d, st); }));
    if (rc) return rc;
  }
  BwdKVParams kv{};
  for (int i = 0; i < 2; ++i) {
    kv.q[i] = bf ? qps[i] : qs[i];
    kv.alpha[i] = al[i]; kv.beta[i] = be[i];
    kv.dout[i] = dos[i]; kv.lse[i] = bf ? l2s[i] : lses[i]; kv.D[i] = Ds[i]; kv.window[i] = wins[i];
    kv.pos[i] = poss[i]; kv.nrows[i] = nrows[i];
  }
  kv.k = k; kv.v = v; kv.dk = dk; kv.dv = dv;
  kv.B = B; kv.T = (int)T; kv.Hq = Hq; kv.Hkv = Hkv; kv.G = G; kv.scale = scale;
  rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_KV, st, [&] {
    return bf ? launch_bwd_kv_bf16(kv, d, st) : launch_bwd_kv_f32(kv, d, st);
  }));
  if (rc) return rc;
  float* da[2] = {dg->dalpha_base, dg->dalpha_out};
  float* db[2] = {dg->dbeta_base, dg->dbeta_out};
  AffineGradParams ag[2] = {};
  for (int i = 0; i < 2; ++i) {
    ag[i].dq = dqs[i]; ag[i].q = qs[i]; ag[i].alpha = al[i]; ag[i].dq_raw = dqo[i];
    ag[i].part = reinterpret_cast<float*>(w + (bf ? L.partq[i] : L.part));
    ag[i].dalpha = da[i]; ag[i].dbeta = db[i];
    ag[i].rows = B * nrows[i]; ag[i].n = Hq * d; ag[i].chunk_rows = L.chunk_rows;
    ag[i].nchunk = bf ? B * L.nrt[i] : L.nchunk;
    ag[i].bf16 = bf ? 1 : 0;
  }
  if (bf)  // both streams' partials were written by the query-side kernels: one launch sums them
    return launch_rc(run_stage(ORTHROS_STAGE_BWD_AFFINE, st, [&] {
      return launch_affine_grad_final(ag, 2, st);
    }));
  for (int i = 0; i < 2; ++i) {  // the fp32 path shares one partial buffer between the streams
    rc = launch_rc(run_stage(ORTHROS_STAGE_BWD_AFFINE, st, [&] { return launch_affine_grad(ag[i], st); }));
    if (rc) return rc;
  }
  return ORTHROS_OK;
}

// Fine-tuning forward; with lse_b / lse_o set it also writes the rows' log-sum-exp.
int forward_sft_impl(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                     const int32_t* out_pos, int64_t R, const void* k, const void* v,
                     const orthros_affine* aff, void* cache_k, void* cache_v,
                     int32_t* cache_len, void* o_base, void* o_out, float* lse_b, float* lse_o,
                     void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T < 1 || T > INT_MAX / 2 || R < 1 || R > INT_MAX / 2) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  if ((rc = check_ptrs({q_base, q_out, k, v, o_base, o_out}))) return rc;
  if (!out_pos || ((uintptr_t)out_pos & 3u)) return ORTHROS_E_INVALID;
  const bool any_cache = cache_k || cache_v || cache_len;
  if (any_cache && (rc = check_ptrs({cache_k, cache_v, cache_len}))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes, sft_rows_per_head(R)))) return rc;
  if (any_cache && T > s->capacity) return ORTHROS_E_INVALID;
  bool copy = true;
  if (any_cache && (rc = kv_source(s, T, 0, k, v, cache_k, cache_v, &copy))) return rc;

  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);
  const WsLayout L = ws_layout(s, sft_rows_per_head(R));
  char* wsc = static_cast<char*>(ws);

  if (any_cache) {
    CacheWriteParams cw{k, v, cache_k, cache_v, cache_len, B, (int)T, Hkv, d, esize(s), s->capacity,
                        0, copy ? 0 : 1};
    rc = launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_cache_write(cw, st); }));
    if (rc) return rc;
  }

  if (s->dtype == ORTHROS_F32) {
    RowsF32Params r{};
    r.q = static_cast<const float*>(q_base);
    r.q_sb = T * Hq * d; r.q_st = (idx_t)Hq * d; r.q_sh = d;
    r.alpha = aff->alpha_base; r.beta = aff->beta_base;
    r.k = static_cast<const float*>(k); r.v = static_cast<const float*>(v);
    r.k_sb = T * Hkv * d; r.k_st = (idx_t)Hkv * d; r.k_sh = d;
    r.o = static_cast<float*>(o_base);
    r.o_sb = T * Hq * d; r.o_st = (idx_t)Hq * d; r.o_sh = d;
    r.B = B; r.Hq = Hq; r.Hkv = Hkv; r.G = G; r.d = d; r.nrows = (int)T; r.t0 = 0;
    r.window = s->window; r.scale = scale; r.nkeys = T;
    r.lse = lse_b; r.lse_sb = (idx_t)Hq * T; r.lse_sh = T;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(r, st); }));
    if (rc) return rc;
    RowsF32Params o = r;
    o.q = static_cast<const float*>(q_out);
    o.q_sb = R * Hq * d; o.q_st = (idx_t)Hq * d;
    o.alpha = aff->alpha_out; o.beta = aff->beta_out;
    o.o = static_cast<float*>(o_out);
    o.o_sb = R * Hq * d; o.o_st = (idx_t)Hq * d;
    o.nrows = (int)R; o.pos = out_pos; o.window = INT_MAX;
    o.lse = lse_o; o.lse_sb = (idx_t)Hq * R; o.lse_sh = R;
    return launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(o, st); }));
  }

  // Base rows: Eq. 4 at every position.
  BandParams bp{};
  bp.q = q_base; bp.q_sb = T * Hq * d; bp.q_st = (idx_t)Hq * d; bp.q_sh = d;
  bp.alpha = aff->alpha_base; bp.beta = aff->beta_base;
  bp.k = k; bp.v = v; bp.k_sb = T * Hkv * d; bp.k_st = (idx_t)Hkv * d; bp.k_sh = d;
  bp.o = o_base; bp.o_sb = T * Hq * d; bp.o_st = (idx_t)Hq * d; bp.o_sh = d;
  bp.B = B; bp.nrows = (int)T; bp.nkeys = (int)T; bp.t_first = 0; bp.pos = nullptr;
  bp.Hq = Hq; bp.Hkv = Hkv; bp.G = G;
  bp.window = s->window < (int)T ? s->window : (int)T;
  bp.scale_log2 = scale * kLog2e;
  bp.lse = lse_b; bp.lse_sb = (idx_t)Hq * T; bp.lse_sh = T;

  if (R > kSftSplitRows) {
    // Many response rows: the banded kernel with the row positions, full causal windows, in
    // one launch with the base rows, the response rows' (longer) work-groups first, so the
    // base rows' work-groups fill the CUs the response rows leave free.
    BandParams op = bp;
    op.q = q_out; op.q_sb = R * Hq * d; op.q_st = (idx_t)Hq * d;
    op.alpha = aff->alpha_out; op.beta = aff->beta_out;
    op.o = o_out; op.o_sb = R * Hq * d; op.o_st = (idx_t)Hq * d;
    op.nrows = (int)R; op.pos = out_pos;
    op.window = (int)T;
    op.lse = lse_o; op.lse_sb = (idx_t)Hq * R; op.lse_sh = R;
    return launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band_pair(op, bp, d, st); }));
  }
  rc = launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band(bp, d, st); }));
  if (rc) return rc;

  // Few response rows: split-key rows, each (row, head) pair over keys 0 .. pos[row].
  SplitParams sp{};
  sp.q_out = q_out; sp.q_sb = R * Hq * d; sp.q_st = (idx_t)Hq * d; sp.q_sh = d;
  sp.a_out = aff->alpha_out; sp.b_out = aff->beta_out;
  sp.a_base = aff->alpha_base; sp.b_base = aff->beta_base;
  sp.k = k; sp.v = v;
  sp.k_sb = T * Hkv * d; sp.k_sh = d; sp.k_st = (idx_t)Hkv * d;
  sp.n_fixed = T;
  sp.pos = out_pos; sp.R = (int)R;
  sp.B = B; sp.Hq = Hq; sp.Hkv = Hkv; sp.G = G;
  sp.HC = 16;
  sp.nchunks = (int)((R * G + 15) / 16);
  sp.window = s->window; sp.with_base = 0;
  sp.nsplit = nsplit_for(T, (int64_t)B * Hkv * sp.nchunks, d);
  sp.scale_log2 = scale * kLog2e;
  sp.pm = reinterpret_cast<float*>(wsc + L.pm);
  sp.pl = reinterpret_cast<float*>(wsc + L.pl);
  sp.po = reinterpret_cast<float*>(wsc + L.po);
  rc = launch_rc(run_stage(ORTHROS_STAGE_SPLIT_ROWS, st, [&] { return launch_split_rows(sp, d, st); }));
  if (rc) return rc;
  MergeParams mp{};
  mp.pm = sp.pm; mp.pl = sp.pl; mp.po = sp.po;
  mp.out0 = o_out; mp.o_sb0 = R * Hq * d; mp.o_st0 = (idx_t)Hq * d; mp.o_sh0 = d;
  mp.rows = (int)(B * Hq * R); mp.nsplit = sp.nsplit; mp.d = d; mp.Hq = Hq;
  mp.nstreams = (int)R; mp.rows_out0 = 1; mp.bf16 = 1;
  mp.lse = lse_o;  // row (b Hq + h) R + r: the [B, Hq, R] layout
  return launch_rc(run_stage(ORTHROS_STAGE_MERGE, st, [&] { return launch_merge(mp, st); }));
}

// A prompt chunk over a contiguous cache (pg.table == nullptr) or a paged pool.
int prefill_chunk_impl(const orthros_shape* s, int64_t past_len, int64_t C, const void* q_base,
                       const void* q_out, const void* k, const void* v, const orthros_affine* aff,
                       void* cache_k, void* cache_v, const PagedKV& pg, int32_t* cache_len,
                       void* o_base, void* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc;
  if (past_len < 0 || C < 1 || C > INT_MAX / 2 || past_len > INT_MAX / 2) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  if ((rc = check_ptrs({q_base, k, v, cache_k, cache_v, cache_len, o_base}))) return rc;
  // the output row is optional (a chunk before the prompt's last one needs none): both or neither
  if ((q_out == nullptr) != (o_out == nullptr)) return ORTHROS_E_INVALID;
  const bool out_row = q_out != nullptr;
  if (out_row && (rc = check_ptrs({q_out, o_out}))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (past_len + C > s->capacity) return ORTHROS_E_INVALID;
  const bool paged = pg.table != nullptr;
  bool copy = true;  // (the paged callers have checked k, v against the pool)
  if (!paged && (rc = kv_source(s, C, past_len, k, v, cache_k, cache_v, &copy))) return rc;

  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);
  const WsLayout L = ws_layout(s);
  char* wsc = static_cast<char*>(ws);
  const int64_t n = past_len + C;  // keys after this chunk
  // (sequence, kv head) strides of the cache: contiguous, or kv head within the sequence's pages
  const idx_t c_sb = paged ? 0 : (idx_t)Hkv * s->capacity * d;
  const idx_t c_sh = paged ? pg.k_sh : (idx_t)s->capacity * d;

  if (paged) {
    PagedWriteParams wp{k, v, cache_k, cache_v, cache_len, B, (int)C, Hkv, d, esize(s),
                        s->capacity, pg};
    rc = launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_paged_write(wp, st); }));
  } else {
    CacheWriteParams cw{k, v, cache_k, cache_v, cache_len, B, (int)C, Hkv, d, esize(s),
                        s->capacity, past_len, copy ? 0 : 1};
    rc = launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_cache_write(cw, st); }));
  }
  if (rc) return rc;

  if (s->dtype == ORTHROS_F32) {
    RowsF32Params r{};
    r.q = static_cast<const float*>(q_base);
    r.q_sb = C * Hq * d; r.q_st = (idx_t)Hq * d; r.q_sh = d;
    r.alpha = aff->alpha_base; r.beta = aff->beta_base;
    r.k = static_cast<const float*>(cache_k); r.v = static_cast<const float*>(cache_v);
    r.k_sb = c_sb; r.k_st = d; r.k_sh = c_sh;
    r.pg = pg; r.cap = s->capacity;
    r.o = static_cast<float*>(o_base);
    r.o_sb = C * Hq * d; r.o_st = (idx_t)Hq * d; r.o_sh = d;
    r.B = B; r.Hq = Hq; r.Hkv = Hkv; r.G = G; r.d = d; r.nrows = (int)C; r.t0 = (int)past_len;
    r.window = s->window; r.scale = scale;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(r, st); }));
    if (rc || !out_row) return rc;
    RowsF32Params o = r;
    o.q = static_cast<const float*>(q_out);
    o.q_sb = (idx_t)Hq * d; o.q_st = 0;
    o.alpha = aff->alpha_out; o.beta = aff->beta_out;
    o.o = static_cast<float*>(o_out);
    o.o_sb = (idx_t)Hq * d; o.o_st = 0;
    o.nrows = 1; o.t0 = (int)(n - 1); o.window = INT_MAX;
    return launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(o, st); }));
  }

  // Base rows of the chunk (positions past_len .. n-1) over the cache, which now holds them.
  BandParams bp{};
  bp.q = q_base; bp.q_sb = C * Hq * d; bp.q_st = (idx_t)Hq * d; bp.q_sh = d;
  bp.alpha = aff->alpha_base; bp.beta = aff->beta_base;
  bp.k = cache_k; bp.v = cache_v; bp.k_sb = c_sb; bp.k_st = d; bp.k_sh = c_sh;
  bp.pg = pg;
  bp.o = o_base; bp.o_sb = C * Hq * d; bp.o_st = (idx_t)Hq * d; bp.o_sh = d;
  bp.B = B; bp.nrows = (int)C; bp.nkeys = (int)n; bp.t_first = (int)past_len; bp.pos = nullptr;
  bp.Hq = Hq; bp.Hkv = Hkv; bp.G = G;
  bp.window = s->window < (int)n ? s->window : (int)n;
  bp.scale_log2 = scale * kLog2e;
  rc = launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band(bp, d, st); }));
  if (rc || !out_row) return rc;

  // Output row at the chunk's last token over the whole cache.
  SplitParams sp{};
  sp.q_out = q_out; sp.q_sb = (idx_t)Hq * d; sp.q_sh = d;
  sp.a_out = aff->alpha_out; sp.b_out = aff->beta_out;
  sp.a_base = aff->alpha_base; sp.b_base = aff->beta_base;
  sp.k = cache_k; sp.v = cache_v;
  sp.k_sb = c_sb; sp.k_sh = c_sh; sp.k_st = d;
  sp.pg = pg; sp.cap = s->capacity;
  sp.n_fixed = n;
  sp.R = 1;
  sp.B = B; sp.Hq = Hq; sp.Hkv = Hkv; sp.G = G;
  sp.HC = heads_per_chunk(G, false);
  sp.nchunks = (G + sp.HC - 1) / sp.HC;
  sp.window = s->window; sp.with_base = 0;
  sp.nsplit = nsplit_for(n, (int64_t)B * Hkv * sp.nchunks, d);
  sp.scale_log2 = scale * kLog2e;
  sp.pm = reinterpret_cast<float*>(wsc + L.pm);
  sp.pl = reinterpret_cast<float*>(wsc + L.pl);
  sp.po = reinterpret_cast<float*>(wsc + L.po);
  rc = launch_rc(run_stage(ORTHROS_STAGE_SPLIT_ROWS, st, [&] { return launch_split_rows(sp, d, st); }));
  if (rc) return rc;
  MergeParams mp{};
  mp.pm = sp.pm; mp.pl = sp.pl; mp.po = sp.po;
  mp.out0 = o_out; mp.o_sb0 = (idx_t)Hq * d; mp.o_sh0 = d;
  mp.rows = B * Hq; mp.nsplit = sp.nsplit; mp.d = d; mp.Hq = Hq; mp.nstreams = 1; mp.bf16 = 1;
  return launch_rc(run_stage(ORTHROS_STAGE_MERGE, st, [&] { return launch_merge(mp, st); }));
}

}  // namespace

extern "C" {

size_t orthros_workspace_bytes(const orthros_shape* shape, int64_t max_rows_T) {
  if (check_shape(shape) != ORTHROS_OK || max_rows_T < 1) return 0;
  return ws_layout(shape, sft_rows_per_head(max_rows_T)).total;
}

const char* orthros_status_string(int code) {
  switch (code) {
    case ORTHROS_OK: return "ok";
    case ORTHROS_E_INVALID: return "invalid argument";
    case ORTHROS_E_UNSUPPORTED: return "unsupported dtype or shape";
    case ORTHROS_E_WORKSPACE: return "workspace missing or too small";
    case ORTHROS_E_LAUNCH: return "HIP launch or runtime failure";
    default: return "unknown status";
  }
}

int orthros_prefill(const orthros_shape* s, int64_t P, const void* q_base, const void* q_out,
                    const void* k, const void* v, const orthros_affine* aff, void* cache_k,
                    void* cache_v, int32_t* cache_len, void* o_base, void* o_out, void* ws,
                    size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (P < 1 || P > INT_MAX / 2) return ORTHROS_E_INVALID;
  if ((rc = check_affine(aff))) return rc;
  if ((rc = check_ptrs({q_base, q_out, k, v, cache_k, cache_v, cache_len, o_base, o_out}))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  if (P > s->capacity) return ORTHROS_E_INVALID;
  bool copy = true;
  if ((rc = kv_source(s, P, 0, k, v, cache_k, cache_v, &copy))) return rc;

  const int B = s->batch, Hq = s->num_q_heads, Hkv = s->num_kv_heads, d = s->head_dim;
  const int G = Hq / Hkv;
  const float scale = scale_of(s);
  const WsLayout L = ws_layout(s);
  char* wsc = static_cast<char*>(ws);

  CacheWriteParams cw{k, v, cache_k, cache_v, cache_len, B, (int)P, Hkv, d, esize(s), s->capacity,
                      0, copy ? 0 : 1};
  rc = launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_cache_write(cw, st); }));
  if (rc) return rc;

  if (s->dtype == ORTHROS_F32) {
    RowsF32Params r{};
    r.q = static_cast<const float*>(q_base);
    r.q_sb = P * Hq * d; r.q_st = (idx_t)Hq * d; r.q_sh = d;
    r.alpha = aff->alpha_base; r.beta = aff->beta_base;
    r.k = static_cast<const float*>(k); r.v = static_cast<const float*>(v);
    r.k_sb = P * Hkv * d; r.k_st = (idx_t)Hkv * d; r.k_sh = d;
    r.o = static_cast<float*>(o_base);
    r.o_sb = P * Hq * d; r.o_st = (idx_t)Hq * d; r.o_sh = d;
    r.B = B; r.Hq = Hq; r.Hkv = Hkv; r.G = G; r.d = d; r.nrows = (int)P; r.t0 = 0;
    r.window = s->window; r.scale = scale;
    rc = launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(r, st); }));
    if (rc) return rc;
    RowsF32Params o = r;
    o.q = static_cast<const float*>(q_out);
    o.q_sb = (idx_t)Hq * d; o.q_st = 0;
    o.alpha = aff->alpha_out; o.beta = aff->beta_out;
    o.o = static_cast<float*>(o_out);
    o.o_sb = (idx_t)Hq * d; o.o_st = 0;
    o.nrows = 1; o.t0 = (int)(P - 1); o.window = INT_MAX;
    return launch_rc(run_stage(ORTHROS_STAGE_ROWS_F32, st, [&] { return launch_rows_f32(o, st); }));
  }

  BandParams bp{};
  bp.q = q_base; bp.q_sb = P * Hq * d; bp.q_st = (idx_t)Hq * d; bp.q_sh = d;
  bp.alpha = aff->alpha_base; bp.beta = aff->beta_base;
  bp.k = k; bp.v = v; bp.k_sb = P * Hkv * d; bp.k_st = (idx_t)Hkv * d; bp.k_sh = d;
  bp.o = o_base; bp.o_sb = P * Hq * d; bp.o_st = (idx_t)Hq * d; bp.o_sh = d;
  bp.B = B; bp.nrows = (int)P; bp.nkeys = (int)P; bp.t_first = 0; bp.pos = nullptr;
  bp.Hq = Hq; bp.Hkv = Hkv; bp.G = G;
  bp.window = s->window < (int)P ? s->window : (int)P;
  bp.scale_log2 = scale * kLog2e;
  rc = launch_rc(run_stage(ORTHROS_STAGE_BAND, st, [&] { return launch_band(bp, d, st); }));
  if (rc) return rc;

  // Output row at the last prompt token over the freshly written cache (head-major).
  SplitParams sp{};
  sp.q_out = q_out; sp.q_sb = (idx_t)Hq * d; sp.q_sh = d;
  sp.a_out = aff->alpha_out; sp.b_out = aff->beta_out;
  sp.a_base = aff->alpha_base; sp.b_base = aff->beta_base;
  sp.k = cache_k; sp.v = cache_v;
  sp.k_sb = (idx_t)Hkv * s->capacity * d; sp.k_sh = s->capacity * d; sp.k_st = d;
  sp.n_fixed = P;
  sp.B = B; sp.Hq = Hq; sp.Hkv = Hkv; sp.G = G;
  sp.HC = heads_per_chunk(G, false);
  sp.nchunks = (G + sp.HC - 1) / sp.HC;
  sp.window = s->window; sp.with_base = 0;
  sp.nsplit = nsplit_for(P, (int64_t)B * Hkv * sp.nchunks, d);
  sp.scale_log2 = scale * kLog2e;
  sp.pm = reinterpret_cast<float*>(wsc + L.pm);
  sp.pl = reinterpret_cast<float*>(wsc + L.pl);
  sp.po = reinterpret_cast<float*>(wsc + L.po);
  rc = launch_rc(run_stage(ORTHROS_STAGE_SPLIT_ROWS, st, [&] { return launch_split_rows(sp, d, st); }));
  if (rc) return rc;
  MergeParams mp{};
  mp.pm = sp.pm; mp.pl = sp.pl; mp.po = sp.po;
  mp.out0 = o_out; mp.o_sb0 = (idx_t)Hq * d; mp.o_sh0 = d;
  mp.out1 = nullptr;
  mp.rows = B * Hq; mp.nsplit = sp.nsplit; mp.d = d; mp.Hq = Hq; mp.nstreams = 1; mp.bf16 = 1;
  return launch_rc(run_stage(ORTHROS_STAGE_MERGE, st, [&] { return launch_merge(mp, st); }));
}

int orthros_decode_step(const orthros_shape* s, const void* q_base, const void* q_out,
                        const void* k_new, const void* v_new, const orthros_affine* aff,
                        void* cache_k, void* cache_v, int32_t* cache_len, int64_t max_len_hint,
                        void* o_base, void* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_ptrs({cache_k, cache_v}))) return rc;
  if ((rc = check_decode_args(q_base, q_out, k_new, v_new, aff, cache_len, max_len_hint, o_base,
                              o_out))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  return decode_common(s, q_base, q_out, k_new, v_new, aff, cache_k, cache_v, PagedKV{},
                       cache_len, max_len_hint, o_base, o_out, workspace_scratch(s, ws), true, st);
}

int orthros_decode_step_noalloc(const orthros_shape* s, const void* q_base, const void* q_out,
                                const void* k_new, const void* v_new, const orthros_affine* aff,
                                void* cache_k, void* cache_v, int32_t* cache_len,
                                int64_t max_len_hint, void* o_base, void* o_out,
                                int32_t* device_status, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_ptrs({cache_k, cache_v}))) return rc;
  if ((rc = check_decode_args(q_base, q_out, k_new, v_new, aff, cache_len, max_len_hint, o_base,
                              o_out))) return rc;
  if (!device_status || ((uintptr_t)device_status & 3u)) return ORTHROS_E_INVALID;
  DecodeScratch sc{nullptr, nullptr, nullptr, device_status};
  if (s->dtype == ORTHROS_BF16) {  // (the fp32 rows use no partials)
    const NoAllocLayout L = noalloc_layout(s, decode_nsplit(s, max_len_hint));
    if (L.total > ORTHROS_NOALLOC_SCRATCH_BYTES) return ORTHROS_E_WORKSPACE;
    void* base = nullptr;
    if ((rc = scratch_on_current_device(&base))) return rc;
    char* b = static_cast<char*>(base);
    sc.pm = reinterpret_cast<float*>(b + L.pm);
    sc.pl = reinterpret_cast<float*>(b + L.pl);
    sc.po = reinterpret_cast<float*>(b + L.po);
  }
  return decode_common(s, q_base, q_out, k_new, v_new, aff, cache_k, cache_v, PagedKV{},
                       cache_len, max_len_hint, o_base, o_out, sc, false, st);
}

int orthros_decode_step_paged(const orthros_shape* s, const void* q_base, const void* q_out,
                              const void* k_new, const void* v_new, const orthros_affine* aff,
                              const orthros_paged_kv* cache, int32_t* cache_len,
                              int64_t max_len_hint, void* o_base, void* o_out, void* ws,
                              size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  PagedKV pg{};
  if ((rc = check_paged(s, cache, ws, &pg))) return rc;
  if ((rc = check_decode_args(q_base, q_out, k_new, v_new, aff, cache_len, max_len_hint, o_base,
                              o_out))) return rc;
  return decode_common(s, q_base, q_out, k_new, v_new, aff, cache->k_pages, cache->v_pages, pg,
                       cache_len, max_len_hint, o_base, o_out, workspace_scratch(s, ws), true, st);
}

int orthros_paged_write(const orthros_shape* s, int64_t T, const void* k, const void* v,
                        const orthros_paged_kv* cache, int32_t* cache_len, void* ws,
                        size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if (T < 1 || T > INT_MAX / 2) return ORTHROS_E_INVALID;
  if ((rc = check_ptrs({k, v, cache_len}))) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  PagedKV pg{};
  if ((rc = check_paged(s, cache, ws, &pg))) return rc;
  if ((rc = kv_outside_pool(s, T, k, v, cache))) return rc;
  PagedWriteParams wp{k, v, cache->k_pages, cache->v_pages, cache_len, s->batch, (int)T,
                      s->num_kv_heads, s->head_dim, esize(s), s->capacity, pg};
  return launch_rc(run_stage(ORTHROS_STAGE_CACHE_WRITE, st, [&] { return launch_paged_write(wp, st); }));
}

int orthros_forward_pt(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                       const void* k, const void* v, const orthros_affine* aff, void* cache_k,
                       void* cache_v, int32_t* cache_len, void* o_base, void* o_out, void* ws,
                       size_t ws_bytes, hipStream_t st) {
  return forward_pt_impl(s, T, q_base, q_out, k, v, aff, cache_k, cache_v, cache_len, o_base,
                         o_out, nullptr, nullptr, ws, ws_bytes, st);
}

int orthros_forward_pt_lse(const orthros_shape* s, int64_t T, const void* q_base,
                           const void* q_out, const void* k, const void* v,
                           const orthros_affine* aff, void* o_base, void* o_out, float* lse_base,
                           float* lse_out, void* ws, size_t ws_bytes, hipStream_t st) {
  if (check_ptrs({lse_base, lse_out})) return ORTHROS_E_INVALID;
  return forward_pt_impl(s, T, q_base, q_out, k, v, aff, nullptr, nullptr, nullptr, o_base,
                         o_out, lse_base, lse_out, ws, ws_bytes, st);
}

size_t orthros_backward_workspace_bytes(const orthros_shape* s, int64_t T) {
  if (check_shape(s) != ORTHROS_OK || T < 1 || T > INT_MAX / 2) return 0;
  return bwd_layout(s, T, T).total;
}

size_t orthros_backward_sft_workspace_bytes(const orthros_shape* s, int64_t T, int64_t R) {
  if (check_shape(s) != ORTHROS_OK || T < 1 || T > INT_MAX / 2 || R < 1 || R > INT_MAX / 2)
    return 0;
  return bwd_layout(s, T, R).total;
}

int orthros_backward_pt(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                        const void* k, const void* v, const orthros_affine* aff,
                        const void* o_base, const void* o_out, const float* lse_base,
                        const float* lse_out, const void* do_base, const void* do_out,
                        void* dq_base, void* dq_out, void* dk, void* dv,
                        const orthros_affine_grad* dg, void* ws, size_t ws_bytes,
                        hipStream_t st) {
  return backward_impl(s, T, q_base, q_out, nullptr, T, k, v, aff, o_base, o_out, lse_base,
                       lse_out, do_base, do_out, dq_base, dq_out, dk, dv, dg, ws, ws_bytes, st);
}

int orthros_backward_sft(const orthros_shape* s, int64_t T, const void* q_base,
                         const void* q_out, const int32_t* out_pos, int64_t R, const void* k,
                         const void* v, const orthros_affine* aff, const void* o_base,
                         const void* o_out, const float* lse_base, const float* lse_out,
                         const void* do_base, const void* do_out, void* dq_base, void* dq_out,
                         void* dk, void* dv, const orthros_affine_grad* dg, void* ws,
                         size_t ws_bytes, hipStream_t st) {
  if (!out_pos) return ORTHROS_E_INVALID;
  return backward_impl(s, T, q_base, q_out, out_pos, R, k, v, aff, o_base, o_out, lse_base,
                       lse_out, do_base, do_out, dq_base, dq_out, dk, dv, dg, ws, ws_bytes, st);
}

int orthros_prefill_chunk(const orthros_shape* s, int64_t past_len, int64_t C,
                          const void* q_base, const void* q_out, const void* k, const void* v,
                          const orthros_affine* aff, void* cache_k, void* cache_v,
                          int32_t* cache_len, void* o_base, void* o_out, void* ws,
                          size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  return prefill_chunk_impl(s, past_len, C, q_base, q_out, k, v, aff, cache_k, cache_v,
                            PagedKV{}, cache_len, o_base, o_out, ws, ws_bytes, st);
}

int orthros_prefill_chunk_paged(const orthros_shape* s, int64_t past_len, int64_t C,
                                const void* q_base, const void* q_out, const void* k,
                                const void* v, const orthros_affine* aff,
                                const orthros_paged_kv* cache, int32_t* cache_len, void* o_base,
                                void* o_out, void* ws, size_t ws_bytes, hipStream_t st) {
  int rc = check_shape(s);
  if (rc) return rc;
  if ((rc = check_ws(s, ws, ws_bytes))) return rc;
  PagedKV pg{};
  if ((rc = check_paged(s, cache, ws, &pg))) return rc;
  // the banded kernel reads one table entry per 64-key tile
  if (s->dtype == ORTHROS_BF16 && cache->page_size < 64) return ORTHROS_E_UNSUPPORTED;
  if (C >= 1 && C <= INT_MAX / 2 && k && v && (rc = kv_outside_pool(s, C, k, v, cache))) return rc;
  return prefill_chunk_impl(s, past_len, C, q_base, q_out, k, v, aff, cache->k_pages,
                            cache->v_pages, pg, cache_len, o_base, o_out, ws, ws_bytes, st);
}

int orthros_forward_sft(const orthros_shape* s, int64_t T, const void* q_base, const void* q_out,
                        const int32_t* out_pos, int64_t R, const void* k, const void* v,
                        const orthros_affine* aff, void* cache_k, void* cache_v,
                        int32_t* cache_len, void* o_base, void* o_out, void* ws,
                        size_t ws_bytes, hipStream_t st) {
  return forward_sft_impl(s, T, q_base, q_out, out_pos, R, k, v, aff, cache_k, cache_v,
                          cache_len, o_base, o_out, nullptr, nullptr, ws, ws_bytes, st);
}

int orthros_forward_sft_lse(const orthros_shape* s, int64_t T, const void* q_base,
                            const void* q_out, const int32_t* out_pos, int64_t R, const void* k,
                            const void* v, const orthros_affine* aff, void* o_base, void* o_out,
                            float* lse_base, float* lse_out, void* ws, size_t ws_bytes,
                            hipStream_t st) {
  if (check_ptrs({lse_base, lse_out})) return ORTHROS_E_INVALID;
  return forward_sft_impl(s, T, q_base, q_out, out_pos, R, k, v, aff, nullptr, nullptr, nullptr,
                          o_base, o_out, lse_base, lse_out, ws, ws_bytes, st);
}

int orthros_read_device_status(void* ws, size_t ws_bytes, int32_t* host_status, int clear,
                               hipStream_t st) {
  if (!ws || !host_status || ws_bytes < kStatusBytes) return ORTHROS_E_INVALID;
  if (hipStreamSynchronize(st) != hipSuccess) return ORTHROS_E_LAUNCH;
  if (hipMemcpy(host_status, ws, sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess) return ORTHROS_E_LAUNCH;
  if (clear) {
    const int32_t zero = 0;
    if (hipMemcpy(ws, &zero, sizeof(int32_t), hipMemcpyHostToDevice) != hipSuccess) return ORTHROS_E_LAUNCH;
  }
  return ORTHROS_OK;
}

int orthros_timing_begin(void) {
  for (auto& r : g_timing.recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_timing.recs.clear();
  g_timing.on = true;
  return ORTHROS_OK;
}

int orthros_timing_end(double* stage_ms, int64_t* stage_launches) {
  if (!stage_ms || !stage_launches) return ORTHROS_E_INVALID;
  for (int i = 0; i < ORTHROS_NUM_STAGES; ++i) {
    stage_ms[i] = 0.0;
    stage_launches[i] = 0;
  }
  int rc = ORTHROS_OK;
  for (auto& r : g_timing.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
      rc = ORTHROS_E_LAUNCH;
    stage_ms[r.stage] += ms;
    stage_launches[r.stage] += 1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_timing.recs.clear();
  g_timing.on = false;
  return rc;
}

}  // extern "C"
