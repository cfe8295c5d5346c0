// Split-key attention for a few query rows against a long key range, bf16 in, fp32 partials.
//
// Serves the output stream's full causal cross-attention ("Orthros: Phase-Aware Heterogeneous
// Attention for Efficient Transformers", §3.1 Eq. 5) at the prediction positions, and in the
// decoding regime (§3.2) the decoupled pair at once: for each (sequence, kv head) the output
// copies of the G query heads (keys 0 .. L) and their base copies (Eq. 4, keys L-w+1 .. L) share
// one pass over the key/value stream, so every cached byte is read once per step.
//
// Layout: one work-group (4 wavefronts) per (split, kv head x head chunk, sequence). The group
// copies 64-key tiles of K and V from global memory straight into a kSS-slot LDS ring (row-major,
// 16-byte slots XOR-swizzled by row), kSS - 1 tiles ahead of their use, so a group keeps up to
// four tiles (128 KB at d = 128) of the stream in flight; wavefront w owns keys 16w .. 16w+15
// of each tile and copies those rows itself:
//   S^T[16 keys x 16 rows] = K . Q^T    4 x mfma_f32_16x16x32_bf16 (d = 128)
//   online softmax over the 16 keys     (exp2 domain; the query carries scale * log2 e)
//   O^T[d x 16 rows]     += V^T . P^T   8 x mfma_f32_16x16x16_bf16 (P^T straight from S^T;
//                                       V^T through the LDS transpose read)
// The four wavefronts' (max, sum, O) are merged in LDS and written as one fp32 partial per
// row and split; merge_kernel combines the splits in a fixed order (deterministic).
#include "common.h"
#include "launch.h"
#include "lds_mfma.h"

namespace orthros {

namespace {
constexpr int kTK = 64;      // keys per tile
constexpr int kRows = 16;    // query rows per work-group (MFMA N)
constexpr int kSS = 5;       // LDS ring slots
// Probabilities are exp2(score - m) with a per-row reference m that moves only when it must
// (fp32 and bf16 share their exponent range, so values up to 2^64 lose nothing): when a lane's
// probabilities could exceed 2^64, or at the row's first keys if their maximum lies outside
// +-kSafeScore (otherwise m stays 0).
constexpr float kLazyBound = 18446744073709551616.f;  // 2^64
constexpr float kSafeScore = 64.f;

template <int D>
struct SplitSmem {
  static constexpr int ROWB = D * 2;           // bytes per K/V row
  static constexpr int TILEB = kTK * ROWB;     // one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;     // K + V
  static constexpr int RING_BYTES = kSS * STAGEB;
  static constexpr int RED_BYTES = 4 * kRows * (D + 2) * 4;
  static constexpr int BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
};
// 16-byte slot of channel chunk c in row r: K rows XOR c with r mod (chunks per row), so the
// 16 rows of a score read hit distinct banks; V rows XOR with an even value (chunk pairs stay
// together) that differs for 8 consecutive rows (row pairs for d = 64), so the 16 rows of a
// transposed read cover the banks twice, the least its 512 bytes need.
template <int D>
__device__ __forceinline__ int k_swz(int r) { return r % (D / 8); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return D == 128 ? 2 * (r % 8) : 2 * ((r >> 1) % 4); }
}  // namespace

template <int D, bool PAGED>
__global__ __launch_bounds__(256) void split_rows_kernel(SplitParams p) {
  using SM = SplitSmem<D>;
  constexpr int ROWB = SM::ROWB, TILEB = SM::TILEB, STAGEB = SM::STAGEB;
  constexpr int NST = D / 32;   // QK k-steps (32 channels each)
  constexpr int NMT = D / 16;   // PV output tiles (16 channels each)
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int LROWS = 1024 / ROWB;         // rows per copy instruction (64 lanes x 16 bytes)
  constexpr int NCOPY = kTK / LROWS / 4;     // copy instructions per wavefront per tensor
  static_assert(NCOPY >= 1 && NCOPY * LROWS * 4 == kTK, "copies cover a tile");
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];

  const int s = blockIdx.x;
  const int g = blockIdx.y / p.nchunks;
  const int chunk = blockIdx.y % p.nchunks;
  const int b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nstreams = p.with_base ? 2 : 1;

  int64_t n, Lnew = -1;
  if (p.len) {
    // keys 0..L-1 come from the cache, key L from this step's input; a length outside
    // [0, capacity] is clamped so no read leaves the cache
    const int64_t L = __builtin_amdgcn_readfirstlane(p.len[b]);  // one sequence per group
    Lnew = L < 0 ? 0 : (L > p.cap ? p.cap : L);
    n = Lnew + 1;
  } else {
    n = p.n_fixed;
  }
  int64_t per = (n + p.nsplit - 1) / p.nsplit;
  per = (per + kTK - 1) / kTK * kTK;
  const int64_t kb = uniform64((int64_t)s * per);  // this split's keys kb .. ke-1
  const int64_t ke = uniform64(kb + per < n ? kb + per : n);

  const int h0 = g * p.G + chunk * p.HC;
  int nr;  // occupied row slots of this chunk (output stream)
  if (p.pos) {
    nr = p.R * p.G - chunk * kRows;
    if (nr > kRows) nr = kRows;
  } else {
    nr = p.G - chunk * p.HC;
    if (nr > p.HC) nr = p.HC;
  }

  // Row slot of this lane (MFMA column) and its key range.
  const int j = lane & 15;
  const int kg = lane >> 4;
  int stream = -1, h = 0, rr = 0;
  int64_t lo = 1, hi = 0;  // empty
  if (p.pos) {
    if (j < nr) {
      const int gr = chunk * kRows + j;
      rr = gr / p.G;
      h = g * p.G + gr % p.G;
      stream = 0;
      lo = 0;
      const int64_t t = p.pos[rr];
      hi = t < 0 ? 0 : (t > n - 1 ? n - 1 : t);  // positions outside [0, n) are clamped
    }
  } else if (j < nr) {
    stream = 0;
    h = h0 + j;
    lo = 0;
    hi = n - 1;
  } else if (p.with_base && j < 2 * nr) {
    stream = 1;
    h = h0 + j - nr;
    lo = n - p.window > 0 ? n - p.window : 0;
    hi = n - 1;
  }

  // Query fragment (B operand of mfma 16x16x32): lane (j, kg) holds channels 32*st + 8*kg + e.
  // The fp32 query is carried as a bf16 pair hi + lo (lo = the rounding residue of hi), and so
  // are the probabilities below: two MFMAs per product keep both near fp32 accuracy, which long
  // rows need (a bf16 query and bf16 probabilities alone leave a relative error of order 3e-3
  // on a 128K-key row). The kernel is bound by memory traffic, so the extra MFMAs are free.
  bf16x8 qf[NST], qf_lo[NST];
  {
    const uint16_t* qsrc = nullptr;
    const float *al = nullptr, *be = nullptr;
    if (stream == 0) {
      qsrc = reinterpret_cast<const uint16_t*>(p.q_out) + (idx_t)b * p.q_sb + (idx_t)rr * p.q_st +
             (idx_t)h * p.q_sh;
      al = p.a_out + (idx_t)h * D;
      be = p.b_out + (idx_t)h * D;
    } else if (stream == 1) {
      qsrc = reinterpret_cast<const uint16_t*>(p.q_base) + (idx_t)b * p.q_sb + (idx_t)h * p.q_sh;
      al = p.a_base + (idx_t)h * D;
      be = p.b_base + (idx_t)h * D;
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int c0 = 32 * st + 8 * kg;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (qsrc) raw = *reinterpret_cast<const u32x4*>(qsrc + c0);
      bf16x8 f, flo;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = raw[e >> 1];
        const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
        const float y = qsrc ? (al[c0 + e] * x + be[c0 + e]) * p.scale_log2 : 0.f;
        f[e] = (__bf16)y;
        flo[e] = (__bf16)(y - (float)f[e]);
      }
      qf[st] = f;
      qf_lo[st] = flo;
    }
  }

  // Cached rows: contiguous [B, Hkv, cap, d], or (PAGED) kv head g of the pages the
  // sequence's table row names.
  const idx_t head_off = PAGED ? (idx_t)g * p.pg.k_sh : (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(p.k) + head_off;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(p.v) + head_off;
  const uint16_t* knew = p.knew ? reinterpret_cast<const uint16_t*>(p.knew) + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh : nullptr;
  const uint16_t* vnew = p.vnew ? reinterpret_cast<const uint16_t*>(p.vnew) + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh : nullptr;
  const int32_t* tbl = PAGED ? p.pg.table + (idx_t)b * p.pg.tbl_sb : nullptr;
  // Pages of 64 keys or more hold whole tiles (tiles start at multiples of 64): one table
  // read per tile. Smaller pages: one per row.
  const bool page_per_tile = PAGED && p.pg.ps_log2 >= 6;

  f32x4 O[NMT];
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt) O[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mref = 0.f, l = 0.f;
  bool seen = false;  // the row met a key of its range in this wavefront's share

  if (kb < ke) {
    const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
    // Copy lanes: instruction i of wavefront wv fills rows (wv NCOPY + i) LROWS .. of a tile,
    // lane l writing slot l % CPR of row l / CPR; it fetches the channel chunk that lands there.
    int crow[NCOPY];
    uint32_t kcb[NCOPY], vcb[NCOPY];  // byte offsets of the fetched chunks within a row
#pragma unroll
    for (int i = 0; i < NCOPY; ++i) {
      crow[i] = (wv * NCOPY + i) * LROWS + lane / CPR;
      kcb[i] = 16u * (uint32_t)((lane % CPR) ^ k_swz<D>(crow[i]));
      vcb[i] = 16u * (uint32_t)((lane % CPR) ^ v_swz<D>(crow[i]));
    }
    const int wv_s = __builtin_amdgcn_readfirstlane(wv);
    // Pages of >= 64 rows: one table entry per tile, read through the scalar cache (the table is
    // constant while the kernel runs) one tile request ahead of its use, as tiles are requested
    // in order.
    auto read_page = [&](int64_t key) -> int32_t {
      const int64_t tc = key < 0 ? 0 : (key > p.cap - 1 ? p.cap - 1 : key);
      const __attribute__((address_space(4))) int32_t* ct =
          (const __attribute__((address_space(4))) int32_t*)(uintptr_t)uniform64((int64_t)(uintptr_t)tbl);
      return ct[tc >> p.pg.ps_log2];
    };
    int32_t next_page = 0;
    if constexpr (PAGED) {
      if (page_per_tile) next_page = read_page(kb);
    }
    // Tile starting at key t0 -> ring slot `slot`. Keys past the split's range re-read its last
    // key; key Lnew comes from this step's input. Every lane carries its own 64-bit address.
    // Each cached byte is read once per call, so the copies carry the non-temporal hint.
    auto load_tile = [&](int64_t t0, int slot) {
      idx_t tile_off = 0;
      if constexpr (PAGED) {
        if (page_per_tile) {
          int32_t page = next_page;
          next_page = read_page(t0 + kTK);
          if (page < 0 || (int64_t)page >= p.pg.num_pages) {
            __hip_atomic_fetch_or(p.pg.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            page = 0;
          }
          // as paged_offset for key t0 (clamped into [0, cap)), minus t0's own rows
          const int64_t tc = t0 > p.cap - 1 ? p.cap - 1 : t0;
          tile_off = (idx_t)page * p.pg.k_sp + (tc & (((int64_t)1 << p.pg.ps_log2) - 1)) * p.k_st - t0 * p.k_st;
        }
      }
      const uint32_t sb = lds0 + (uint32_t)(slot * STAGEB);
#pragma unroll
      for (int i = 0; i < NCOPY; ++i) {
        int64_t key = t0 + crow[i];
        if (key >= ke) key = ke - 1;
        idx_t roff;
        if constexpr (PAGED) {
          roff = page_per_tile ? tile_off + key * p.k_st : paged_offset(p.pg, tbl, key, p.cap, p.k_st);
        } else {
          roff = key * p.k_st;
        }
        const unsigned char* ka = key == Lnew ? reinterpret_cast<const unsigned char*>(knew)
                                              : reinterpret_cast<const unsigned char*>(kbase + roff);
        const unsigned char* va = key == Lnew ? reinterpret_cast<const unsigned char*>(vnew)
                                              : reinterpret_cast<const unsigned char*>(vbase + roff);
        const uint32_t dst = sb + (uint32_t)(wv_s * NCOPY + i) * 1024u;
        stream_to_lds_at(ka + kcb[i], dst);
        stream_to_lds_at(va + vcb[i], dst + TILEB);
      }
    };
    // Waits until at most `ahead` tiles' copies of this wavefront are still in flight (2 NCOPY
    // per tile; the loop issues no other vector memory load whose wait is still pending).
    auto wait_tiles = [&](int ahead) {
      if (ahead >= 3) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * NCOPY) : "memory");
      else if (ahead == 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * NCOPY) : "memory");
      else if (ahead == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NCOPY) : "memory");
      else wait_lds_copies();
    };
    static_assert(kSS - 2 <= 3, "wait_tiles covers up to three tiles beyond the next");

    const int ntl = __builtin_amdgcn_readfirstlane((int)((ke - kb + kTK - 1) / kTK));
    for (int t = 0; t < kSS - 1 && t < ntl; ++t) load_tile(kb + (int64_t)kTK * t, t);
    wait_tiles(ntl - 1 < kSS - 2 ? ntl - 1 : kSS - 2);  // tile 0 has landed
    __syncthreads();
    // LDS read offsets within a slot: score operand (row 16 wv + j, channel chunk 4 st + kg),
    // transposed value operand (lane j of group kg: row 16 wv + 4 kg + j / 4, channels
    // 16 mt + 4 (j % 4) .. + 3, i.e. chunk 2 mt + (j % 4) / 2, half j % 2).
    const int qrow = 16 * wv + j;
    const int vr = 16 * wv + 4 * kg + (j >> 2);
    for (int t = 0; t < ntl; ++t) {
      // tile t + kSS - 1 goes into the slot tile t - 1 left (this wavefront has read its rows)
      if (t + kSS - 1 < ntl) load_tile(kb + (int64_t)kTK * (t + kSS - 1), (t + kSS - 1) % kSS);
      const int64_t t0 = kb + (int64_t)kTK * t;
      const int64_t wk0 = t0 + 16 * wv;  // this wavefront's first key
      if (wk0 < ke) {
        const unsigned char* sk = smem + (t % kSS) * STAGEB;
        const unsigned char* sv = sk + TILEB;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(sk + qrow * ROWB + 16 * ((4 * st + kg) ^ k_swz<D>(qrow)));
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[st], acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf_lo[st], acc, 0, 0, 0);
        }
        float sc[4];
        bool anykey = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t key = wk0 + 4 * kg + r;
          const bool ok = key < ke && key >= lo && key <= hi;
          sc[r] = ok ? acc[r] : kNegInf;
          anykey = anykey || ok;
        }
        float ps;
        s16x4 pb, pb_lo;
        auto probs = [&]() {
          ps = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float pr = fast_exp2(sc[r] - mref);
            ps += pr;
            const uint16_t hb = f32_to_bf16(pr);
            pb[r] = (short)hb;
            pb_lo[r] = (short)f32_to_bf16(pr - bf16_to_f32(hb));
          }
        };
        probs();
        const bool need = !(ps <= kLazyBound) || (!seen && anykey);
        if (__builtin_amdgcn_ballot_w64(need)) {  // rare: move the reference of some rows
          int nrow = need ? 1 : 0;  // the 4 lanes of a row decide together
          nrow |= __shfl_xor(nrow, 16, 64);
          nrow |= __shfl_xor(nrow, 32, 64);
          float mx = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
          const bool move = nrow && mx != kNegInf;
          const bool keep0 = !seen && mx > -kSafeScore && mx < kSafeScore;
          const float nref = move ? (keep0 ? 0.f : mx) : mref;
          const float alpha = seen ? fast_exp2(mref - nref) : 0.f;  // unseen rows hold zeros
          seen = seen || move;
          mref = nref;
          l *= alpha;
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) O[mt] *= alpha;
          probs();
        }
        l += ps;
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt) {
          const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(sv + vr * ROWB + 16 * ((2 * mt + ((j & 3) >> 1)) ^ v_swz<D>(vr)) + 8 * (j & 1)));
          O[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb, O[mt], 0, 0, 0);
          O[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, pb_lo, O[mt], 0, 0, 0);
        }
      }
      {  // this wavefront's rows of tile t + 1 have landed
        const int later = ntl - 2 - t;
        wait_tiles(later < kSS - 2 ? later : kSS - 2);
      }
      // A wavefront copies exactly the rows it reads, so the tiles need no barrier and the
      // wavefronts run apart.
    }
  }

  // Sum of this wavefront's per-lane partial denominators over the 4 lanes of each row.
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);

  // Merge the 4 wavefronts in LDS: red[w] = {m[16], l[16], O[16][D]}.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  constexpr int RW = kRows * (D + 2);
  float* rw = red + wv * RW;
  if (kg == 0) {
    rw[j] = seen ? mref : kNegInf;  // reference of this wavefront's share (-inf: no key)
    rw[kRows + j] = l;
  }
#pragma unroll
  for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) rw[2 * kRows + j * D + 16 * mt + 4 * kg + r] = O[mt][r];
  __syncthreads();

  const int nvalid = p.with_base ? 2 * nr : nr;
  for (int e = tid; e < nvalid * D; e += 256) {
    const int jj = e / D, c = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w * RW + jj]);
    float o = 0.f, den = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float f = fast_exp2(red[w * RW + jj] - M);
        o += f * red[w * RW + 2 * kRows + jj * D + c];
        den += f * red[w * RW + kRows + jj];
      }
    }
    idx_t row;
    if (p.pos) {  // (head, response row) pair
      const int gr = chunk * kRows + jj;
      row = ((idx_t)b * p.Hq + g * p.G + gr % p.G) * p.R + gr / p.G;
    } else {
      const int st = jj < nr ? 0 : 1;
      const int hh = h0 + (jj < nr ? jj : jj - nr);
      row = ((idx_t)b * p.Hq + hh) * nstreams + st;
    }
    p.po[(row * p.nsplit + s) * D + c] = o;
    if (c == 0) {
      p.pm[row * p.nsplit + s] = M;
      p.pl[row * p.nsplit + s] = den;
    }
  }
}

// Combine the split partials of one row: O = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.
// One wavefront per row: lane s holds split s's (max, sum); the weights go through LDS and each
// lane then accumulates its channels over the splits in split order (deterministic).
__global__ __launch_bounds__(64) void merge_kernel(MergeParams p) {
  __shared__ float wgt[64];
  const idx_t row = blockIdx.x;
  const int lane = threadIdx.x;
  const int st = (int)(row % p.nstreams);
  const idx_t bh = row / p.nstreams;
  const int h = (int)(bh % p.Hq);
  const idx_t b = bh / p.Hq;
  const float* pm = p.pm + row * p.nsplit;
  const float* pl = p.pl + row * p.nsplit;
  const float ms = lane < p.nsplit ? pm[lane] : kNegInf;
  const float ls = lane < p.nsplit ? pl[lane] : 0.f;
  float M = ms;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  const float f = (ms == kNegInf) ? 0.f : fast_exp2(ms - M);
  float den = f * ls;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off, 64);
  wgt[lane] = f;
  __syncthreads();
  const float inv = 1.f / den;
  // log-sum-exp of the row's scores (scores here are in log2 units), natural log
  if (p.lse && lane == 0) p.lse[row] = (M + __log2f(den)) * 0.69314718055994531f;
  void* out = (st == 0 || p.rows_out0) ? p.out0 : p.out1;
  const idx_t off = p.rows_out0 ? b * p.o_sb0 + (idx_t)st * p.o_st0 + (idx_t)h * p.o_sh0
                    : st == 0  ? b * p.o_sb0 + (idx_t)h * p.o_sh0
                               : b * p.o_sb1 + (idx_t)h * p.o_sh1;
  const float* po = p.po + row * p.nsplit * p.d;
  for (int c = lane; c < p.d; c += 64) {
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    int s = 0;
    for (; s + 4 <= p.nsplit; s += 4) {
      o0 += wgt[s] * po[(idx_t)s * p.d + c];
      o1 += wgt[s + 1] * po[(idx_t)(s + 1) * p.d + c];
      o2 += wgt[s + 2] * po[(idx_t)(s + 2) * p.d + c];
      o3 += wgt[s + 3] * po[(idx_t)(s + 3) * p.d + c];
    }
    for (; s < p.nsplit; ++s) o0 += wgt[s] * po[(idx_t)s * p.d + c];
    const float o = ((o0 + o1) + (o2 + o3)) * inv;
    if (p.bf16)
      reinterpret_cast<uint16_t*>(out)[off + c] = f32_to_bf16(o);
    else
      reinterpret_cast<float*>(out)[off + c] = o;
  }
}

hipError_t launch_split_rows(const SplitParams& p, int d, hipStream_t s) {
  dim3 grid(p.nsplit, p.Hkv * p.nchunks, p.B);
  if (p.pg.table) {
    if (d == 128)
      hipLaunchKernelGGL((split_rows_kernel<128, true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((split_rows_kernel<64, true>), grid, dim3(256), 0, s, p);
  } else {
    if (d == 128)
      hipLaunchKernelGGL((split_rows_kernel<128, false>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((split_rows_kernel<64, false>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(p.rows), dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace orthros
