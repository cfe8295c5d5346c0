// Banded flash attention, bf16 in / bf16 out, fp32 softmax and accumulation.
//
// Computes "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers", §3.1
// Eq. 4 for every base row t (keys max(0, t-w+1) .. t) and, with a window >= T, Eq. 5 for
// every output row (keys 0 .. t, the pre-training regime of §3.2). The query's scale-offset
// (§3.1, q = alpha (.) q_raw + beta) is applied while the query fragment is loaded, together
// with the score scale and log2 e, and rounded once to bf16.
//
// Work-group: 8 wavefronts (two per SIMD), HPW query heads sharing one kv head x (8 / HPW)
// position blocks of 32 rows. One kv head's 64-key K and V tiles are copied straight from
// global memory into a 4-slot LDS ring (row-major, 16-byte slots XOR-swizzled per row so the
// operand reads hit all 64 banks) and read by all eight wavefronts. The copies are waited for
// only at the barrier that publishes them, never by the reads of the other slots. With the transposed score
// layout S^T (keys x queries) each lane owns one query and its softmax stays in registers:
//   S^T[64 x 32]  = K . Q^T        16 x mfma_f32_32x32x16_bf16 (d = 128)
//   online softmax in the exp2 domain, p = exp2(s - m); the reference m moves only when a half-tile's
//   probabilities could exceed 2^8 (their sum does), so the common path computes no maximum
//   O^T[d x 32]  += V^T . P^T      16 x mfma_f32_32x32x16_bf16; P^T straight from the S^T
//                                  registers; V^T through the LDS transpose read
// The tile loop is software-pipelined over key halves so the vector work issues in the shadow
// of the matrix cores (see the pipeline comment below). Tiles are visited from the diagonal
// downwards.
#include "common.h"
#include "launch.h"
#include "lds_mfma.h"

namespace orthros {

namespace {
constexpr int kTK = 64;      // keys per tile
constexpr int kQW = 32;      // query rows per wavefront
constexpr int kNW = 8;       // wavefronts per work-group (two per SIMD)
constexpr int kThreads = 64 * kNW;
constexpr int kStages = 4;   // LDS ring depth
constexpr float kLazyBound = 256.f;  // largest tolerated sum of a half's probabilities
// Reference of a query that has met no key yet: any finite score then gives an infinite
// tentative probability, which sends the query through the rescale path, and the rescale
// factor exp2(kUnstarted - max) is 0 (nothing has been accumulated).
constexpr float kUnstarted = -1e30f;

}  // namespace

template <int D, int HPW>
__global__ __launch_bounds__(kThreads) void band_kernel(BandParams p) {
  constexpr int NCH = D / 8;             // 16-byte slots per row
  constexpr int ROWB = D * 2;            // bytes per K/V row
  constexpr int TILEB = kTK * ROWB;      // bytes per K (or V) tile
  constexpr int STAGEB = 2 * TILEB;      // K + V
  constexpr int PB = kNW / HPW;          // position blocks per work-group
  constexpr int BMP = kQW * PB;          // positions per work-group
  constexpr int NKS = D / 16;            // QK k-steps
  constexpr int NDT = D / 32;            // O^T tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[kStages * STAGEB];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nhc = p.G / HPW;
  const int npb = (p.nrows + BMP - 1) / BMP;
  const uint32_t total = (uint32_t)p.B * p.Hkv * nhc * npb;
  const uint32_t lid = xcd_swizzle(blockIdx.x, total);
  const bool causal = p.window >= p.nkeys;
  int pb, rest;
  if (causal) {  // a few (sequence, head group) pairs at a time, longest rows first
    int from_longest;
    grouped_order(lid, p.B * p.Hkv * nhc, npb, 32, from_longest, rest);
    pb = npb - 1 - from_longest;
  } else {
    pb = (int)(lid % npb);
    rest = (int)(lid / npb);
  }
  // (integer division runs on the vector ALUs: read the results back as scalars)
  pb = __builtin_amdgcn_readfirstlane(pb);
  const int hc = __builtin_amdgcn_readfirstlane(rest % nhc);
  rest /= nhc;
  const int g = __builtin_amdgcn_readfirstlane(rest % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(rest / p.Hkv);
  const int r0 = pb * BMP;                     // first row of the work-group
  const int h = g * p.G + hc * HPW + (wv % HPW);
  const int r0w = r0 + kQW * (wv / HPW);       // first row of this wavefront
  const int j = lane & 31;   // query column of this lane within a column tile
  const int hh = lane >> 5;  // lane half
  const int row = r0w + j;
  const bool rvalid = row < p.nrows;
  const bool wactive = r0w < p.nrows;

  // Row positions: the lowest and highest of this wavefront's rows and of the work-group's.
  int qmin_w, qmax_w, qmin_b, qmax_b, tq;
  if (!p.pos) {
    const int last_w = r0w + kQW - 1 < p.nrows - 1 ? r0w + kQW - 1 : p.nrows - 1;
    const int last_b = r0 + BMP - 1 < p.nrows - 1 ? r0 + BMP - 1 : p.nrows - 1;
    qmin_w = p.t_first + r0w;
    qmax_w = p.t_first + last_w;
    qmin_b = p.t_first + r0;
    qmax_b = p.t_first + last_b;
    tq = rvalid ? p.t_first + row : qmax_w;
  } else {
    __shared__ int wrange[2 * kNW];
    int mine = rvalid ? p.pos[row] : 0;
    mine = mine < 0 ? 0 : (mine > p.nkeys - 1 ? p.nkeys - 1 : mine);  // clamped into [0, nkeys)
    int lo = rvalid ? mine : 0x7fffffff, hi = rvalid ? mine : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      lo = min(lo, __shfl_xor(lo, off, 64));
      hi = max(hi, __shfl_xor(hi, off, 64));
    }
    qmin_w = __builtin_amdgcn_readfirstlane(lo);
    qmax_w = __builtin_amdgcn_readfirstlane(hi);
    if (lane == 0) {
      wrange[2 * wv] = qmin_w;
      wrange[2 * wv + 1] = qmax_w;
    }
    __syncthreads();
    qmin_b = 0x7fffffff;
    qmax_b = -1;
#pragma unroll
    for (int i = 0; i < kNW; ++i) {
      qmin_b = min(qmin_b, wrange[2 * i]);
      qmax_b = max(qmax_b, wrange[2 * i + 1]);
    }
    tq = rvalid ? mine : qmax_w;  // rows past the end compute on a valid position, unstored
  }

  // Query fragments (B operand of 32x32x16): lane (j, hh) holds query row r0w + j, channels
  // 16 s + 8 hh + e.
  bf16x8 qf[NKS];
  {
    const float* al = p.alpha + (idx_t)h * D;
    const float* be = p.beta + (idx_t)h * D;
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + (idx_t)b * p.q_sb +
                         (idx_t)(rvalid ? row : 0) * p.q_st + (idx_t)h * p.q_sh;
    const float sc = rvalid ? p.scale_log2 : 0.f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int c0 = 16 * s + 8 * hh;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(qr + c0);
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(al + c0);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(al + c0 + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(be + c0);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(be + c0 + 4);
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = raw[e >> 1];
        const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
        const float a = e < 4 ? a0[e] : a1[e - 4];
        const float bb = e < 4 ? b0[e] : b1[e - 4];
        f[e] = (__bf16)((a * x + bb) * sc);
      }
      qf[s] = f;
    }
    // Keep the fragments materialised here, outside the tile loop.
#pragma unroll
    for (int s = 0; s < NKS; ++s) asm volatile("" : "+v"(qf[s]));
  }

  // Key range of the work-group (tiles tile_hi, tile_hi - 64, ..., tile_lo) and of this wave.
  const int w = p.window;
  const int nk = p.nkeys;
  const int glo = qmin_b - w + 1 > 0 ? qmin_b - w + 1 : 0;
  const int ghi = qmax_b < nk - 1 ? qmax_b : nk - 1;
  const int tile_lo = glo / kTK * kTK;
  const int tile_hi = ghi / kTK * kTK;
  const int ntiles = (tile_hi - tile_lo) / kTK + 1;
  // Scalar copies for the loop and the tile copies (the per-wavefront conditions below keep
  // their vector form: as scalar branches they cost the register allocator more than they save).
  const int tile_hi_s = __builtin_amdgcn_readfirstlane(tile_hi);
  const int ntiles_s = __builtin_amdgcn_readfirstlane(ntiles);
  const int wlo = qmin_w - w + 1;  // lowest key any row of this wavefront needs (may be < 0)
  auto tile_key = [&](int e) { return tile_hi - kTK * e; };
  // This wavefront's tiles: ea (holds its highest row) .. eb (holds its lowest key), contiguous.
  const int ea = tile_hi > qmax_w ? (tile_hi - qmax_w + kTK - 1) / kTK : 0;
  const int eb_w = (tile_hi + kTK - 1 - wlo) / kTK;
  const int eb = eb_w < ntiles - 1 ? eb_w : ntiles - 1;
  // Unmasked only if every key of the tile lies in every row's window.
  auto full = [&](int e) {
    const int tb = tile_key(e);
    return (tb + kTK - 1 <= qmin_w) && (tb >= qmax_w - w + 1) && (tb + kTK - 1 <= nk - 1);
  };

  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(p.k) + (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(p.v) + (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;

  // Staging straight from global memory into LDS: one wave instruction fills 64 x 16 B, i.e.
  // LROWS consecutive rows, lane i writing slot i % NCH of row i / NCH (the LDS address of a
  // lane is fixed by its index). The swizzle is therefore applied on the global side: the lane
  // that fills K slot c of row r fetches channel chunk c ^ (r % NCH), and for V chunk c ^ f(r),
  // f(r) = 4 (r % 4) at d = 128 (4 ((r >> 1) % 2) at d = 64). A transposed read serves 32 lanes
  // per LDS cycle: 64 bytes from each of 4 consecutive rows, which f places in four different
  // 16-bank groups (with f = 4 ((r >> 1) % 4), rows r and r + 1 shared one: 2-way conflicts, 155
  // against 239 bytes per clock and CU measured). Wave wv fills rows (wv NINST + i) LROWS ..
  // of every tile.
  constexpr int LROWS = 1024 / ROWB;
  constexpr int NINST = kTK / LROWS / kNW;
  static_assert(NINST >= 1 && NINST * LROWS * kNW == kTK, "staging covers a tile exactly");
  // Each lane's byte offsets within a tile are fixed; a tile's base address is a scalar, so a
  // load is one instruction with no address arithmetic. In the tile holding the last key, rows
  // past the sequence end re-read the last row (every read stays inside K and V).
  const uint32_t rowb = (uint32_t)p.k_st * 2u;  // bytes between consecutive keys
  uint32_t skoff[NINST], svoff[NINST];
  int srow[NINST];
#pragma unroll
  for (int i = 0; i < NINST; ++i) {
    const int r = (wv * NINST + i) * LROWS + lane / NCH;
    const int c = lane % NCH;
    srow[i] = r;
    skoff[i] = (uint32_t)r * rowb + 16u * (uint32_t)(c ^ (r % NCH));
    svoff[i] = (uint32_t)r * rowb + 16u * (uint32_t)(c ^ (NCH == 16 ? 4 * (r % 4) : 4 * ((r >> 1) % 2)));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int wv_s = __builtin_amdgcn_readfirstlane(wv);
  // Paged pool: a 64-key tile lies inside one page (pages hold >= 64 rows, tiles start at
  // multiples of 64), so one table entry (a scalar read) gives the tile's base. Tiles are
  // requested in order 0, 1, 2, ...; the entry of the next one is read a request ahead.
  auto page_of = [&](int e) -> int32_t {
    const int tb = tile_hi_s - kTK * (e < ntiles_s ? e : ntiles_s - 1);
    // read through the scalar cache (the table is constant while the kernel runs): a vector
    // load here would make the wave wait for it, and for every copy in flight, on the spot
    const __attribute__((address_space(4))) int32_t* tbl =
        (const __attribute__((address_space(4))) int32_t*)p.pg.table;
    return tbl[(idx_t)b * p.pg.tbl_sb + (tb >> p.pg.ps_log2)];
  };
  int32_t next_page = p.pg.table ? page_of(0) : 0;
  auto load_tile = [&](int e) {
    const int tb = tile_hi_s - kTK * e;
    idx_t toff = (idx_t)tb * rowb;  // bytes from the (sequence, kv head) base to the tile
    if (p.pg.table) {
      int32_t page = next_page;
      next_page = page_of(e + 1);
      if (page < 0 || (int64_t)page >= p.pg.num_pages) {
        __hip_atomic_fetch_or(p.pg.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        page = 0;
      }
      // bytes: the page's start (k_sp elements of 2 bytes per page) plus the tile's rows
      toff = (idx_t)page * p.pg.k_sp * 2 + (idx_t)(tb & ((1 << p.pg.ps_log2) - 1)) * rowb;
    }
    const unsigned char* kt = reinterpret_cast<const unsigned char*>(kbase) + toff;
    const unsigned char* vt = reinterpret_cast<const unsigned char*>(vbase) + toff;
    unsigned char* st = smem + (e % kStages) * STAGEB;
    if (tb + kTK <= nk) {
#pragma unroll
      for (int i = 0; i < NINST; ++i) {
        const uint32_t kd = lds0 + (uint32_t)(st - smem) + (wv_s * NINST + i) * 1024;
        copy_to_lds(kt, skoff[i], kd);
        copy_to_lds(vt, svoff[i], kd + TILEB);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NINST; ++i) {
        const int over = srow[i] - (nk - 1 - tb);
        const uint32_t back = over > 0 ? (uint32_t)over * rowb : 0u;
        const uint32_t kd = lds0 + (uint32_t)(st - smem) + (wv_s * NINST + i) * 1024;
        copy_to_lds(kt, skoff[i] - back, kd);
        copy_to_lds(vt, svoff[i] - back, kd + TILEB);
      }
    }
  };

  // Per-lane LDS read offsets (bytes within a stage).
  // QK A operand: key row 32 m + j, channel slot 2 s + hh.
  int qk_off[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qk_off[s] = j * ROWB + 16 * ((2 * s + hh) ^ (j % NCH));
  // PV A operand (transpose read): lane group G = lane / 16 supplies, from its lane L, key row
  // 16 ks + 8 h2 + 4 (G / 2) + L / 4 at channels 32 dt + 16 (G % 2) + 4 (L % 4) .. + 3.
  int pv_off[NDT];
  {
    const int G = lane >> 4, L = lane & 15;
    const int row = 4 * (G >> 1) + (L >> 2);  // + 16 ks + 8 h2, which leave f unchanged
    const int fv = NCH == 16 ? 4 * (row % 4) : 4 * ((row >> 1) % 2);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int chunk = 4 * dt + 2 * (G & 1) + ((L & 3) >> 1);
      pv_off[dt] = TILEB + row * ROWB + 16 * (chunk ^ fv) + 8 * (L & 1);
    }
  }

  f32x16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  // This lane's query row r0w + j: reference max (probabilities are exp2(score - mref);
  // kUnstarted until the query meets a key of its window) and this lane's part of the row sum
  // (its half of the keys).
  float mref = kUnstarted, l = 0.f;
  f32x16 zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

  // ---- building blocks ----------------------------------------------------------------------
  // Scores of key half m of tile e (NKS MFMAs): S = K rows 32 m .. 32 m + 31 . Q^T.
  auto qk = [&](f32x16& S, int e, int m) {
    const unsigned char* st = smem + (e % kStages) * STAGEB + 32 * m * ROWB;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(st + qk_off[s]);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? zero16 : S, 0, 0, 0);
    }
  };
  // O^T += V^T . P^T over key half m of tile e (2 16-key steps x NDT MFMAs).
  auto pv = [&](const bf16x8* Ph, int e, int m) {
    unsigned char* st = smem + (e % kStages) * STAGEB;
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        unsigned char* base = st + pv_off[dt] + (16 * (2 * m + k2)) * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(lo, hi), Ph[k2], O[dt], 0, 0, 0);
      }
    }
  };
  // Keys outside the query's window (or past the sequence) of half m of tile e -> -inf.
  auto mask = [&](f32x16& S, int e, int m) {
    const int kb = tile_key(e) + 32 * m + 4 * hh;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = kb + 8 * (r >> 2) + (r & 3);
      const bool ok = k <= tq && k > tq - w && k < nk;
      S[r] = ok ? S[r] : kNegInf;
    }
  };
  // Probabilities of one half against the current reference (bf16, as the PV operand) and
  // this lane's sum of them.
  auto expo = [&](const f32x16& S, bf16x8* Ph) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(S[r] - mref);
      const float p1 = fast_exp2(S[r + 1] - mref);
      s0 += p0;
      s1 += p1;
      Ph[r >> 3][r & 7] = (__bf16)p0;
      Ph[r >> 3][(r & 7) + 1] = (__bf16)p1;
    }
    return s0 + s1;
  };
  // After the tentative probabilities of a half: the reference moves only if a probability of
  // the query could exceed 2^8 (their sum over both lane halves does; a query meeting its first
  // key has an infinite sum). Then O and l are rescaled and this half's probabilities
  // recomputed against the new reference (the scores are kept unshifted, so the other half's
  // need no correction). The new reference is the exact maximum, so the probabilities end up
  // <= 1. The common path tests only this lane's own part of the sum against half the bound
  // (one compare and a branch); the sum over both lane halves is formed only past that test.
  auto settle = [&](const f32x16& S, bf16x8* Ph, float ps) {
    if (__builtin_amdgcn_ballot_w64(!(ps <= 0.5f * kLazyBound))) {
      const float tot = lane_pair_sum(ps);
      const bool need = !(tot <= kLazyBound);
      float a0 = fmaxf(S[0], S[1]), a1 = fmaxf(S[2], S[3]);
#pragma unroll
      for (int r = 4; r < 16; r += 4) {
        a0 = fmaxf(a0, fmaxf(S[r], S[r + 1]));
        a1 = fmaxf(a1, fmaxf(S[r + 2], S[r + 3]));
      }
      const float mx = lane_pair_max(fmaxf(a0, a1));
      const bool move = need && mx != kNegInf;
      const float alpha = move ? fast_exp2(mref - mx) : 1.f;  // 0 when the query starts here
      mref = move ? mx : mref;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
      ps = expo(S, Ph);
    }
    l += ps;
  };

  // ---- pipeline -----------------------------------------------------------------------------
  // Per tile e, in two regions that are each one basic block, so the matrix cores and the
  // vector ALUs work side by side:
  //   A: MFMA scores of keys 32..63 of e and PV of keys 32..63 of e-1 | softmax of keys 0..31 of e
  //   B: MFMA scores of keys 0..31 of e+1 and PV of keys 0..31 of e  | softmax of keys 32..63 of e
  // PV of tile e-1 in A is why the LDS ring holds four tiles.
  // Tiles 0 and 1 before the loop; tile e + 2 is requested in iteration e into the slot tile
  // e - 2 left (free since the previous barrier) and has landed by the barrier that ends
  // iteration e (the barrier waits for outstanding loads). A copy instruction holds up its
  // wavefront for ~100 clocks while the address unit works through the queue, so the two
  // wavefronts of a SIMD take turns: the second (wavefronts 4..7) copies at the top of the tile,
  // while the first computes region A, and the first copies after its region A (1-2% on the
  // 128K prefill against both at the top).
  load_tile(0);
  if (ntiles_s > 1) load_tile(1);
  wait_lds_copies();
  __syncthreads();

  f32x16 S0 = zero16, S1 = zero16;
  bf16x8 P0[2], P1[2];
  for (int e = 0; e < ntiles_s; ++e) {
    const bool copy_late = wv_s < kNW / 2;  // the first wavefront of its SIMD
    if (!copy_late && e + 2 < ntiles_s) load_tile(e + 2);
    if (wactive && e >= ea && e <= eb) {
      const bool prev = e > ea, next = e < eb, fl = full(e);
      // Region A runs at raised wavefront priority, region B at the normal one: the wavefront
      // of a SIMD that is still in region A (the one that lags) gets the issue slots first, so
      // the pair reaches the barrier closer together (2-3% on the 128K prefill).
      __builtin_amdgcn_s_setprio(1);
      if (!prev) qk(S0, e, 0);
      float ps;
      if (prev && fl) {
        qk(S1, e, 1);
        pv(P1, e - 1, 1);
        ps = expo(S0, P0);
        interleave<16, 4, 2, 3>();
      } else if (prev) {
        qk(S1, e, 1);
        pv(P1, e - 1, 1);
        mask(S0, e, 0);
        ps = expo(S0, P0);
      } else {
        qk(S1, e, 1);
        mask(S0, e, 0);
        ps = expo(S0, P0);
      }
      __builtin_amdgcn_s_setprio(0);
      settle(S0, P0, ps);
      if (copy_late && e + 2 < ntiles_s) load_tile(e + 2);
      if (next && fl) {
        qk(S0, e + 1, 0);
        pv(P0, e, 0);
        ps = expo(S1, P1);
        interleave<16, 4, 2, 3>();
      } else if (next) {
        qk(S0, e + 1, 0);
        pv(P0, e, 0);
        mask(S1, e, 1);
        ps = expo(S1, P1);
      } else {
        pv(P0, e, 0);
        mask(S1, e, 1);
        ps = expo(S1, P1);
      }
      settle(S1, P1, ps);
      if (!next) pv(P1, e, 1);
    } else if (copy_late && e + 2 < ntiles_s) {
      load_tile(e + 2);
    }
    wait_lds_copies();  // tile e + 2 has landed before the barrier publishes it
    __syncthreads();
  }

  const float lt = lane_pair_sum(l);  // both lane halves of the query column
  if (rvalid) {
    const float inv = 1.f / lt;
    // log-sum-exp of the row's scaled scores (scores here are in log2 units), natural log
    if (p.lse && hh == 0)
      p.lse[(idx_t)b * p.lse_sb + (idx_t)h * p.lse_sh + row] = (mref + __log2f(lt)) * 0.69314718055994531f;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + (idx_t)b * p.o_sb + (idx_t)row * p.o_st + (idx_t)h * p.o_sh;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c = 32 * dt + 8 * rg + 4 * hh;
        u32x2 wd;
        wd[0] = pack_bf16x2(O[dt][4 * rg + 0] * inv, O[dt][4 * rg + 1] * inv);
        wd[1] = pack_bf16x2(O[dt][4 * rg + 2] * inv, O[dt][4 * rg + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + c) = wd;
      }
  }
}

hipError_t launch_band(const BandParams& p, int d, hipStream_t s) {
  int hpw = 1;
  if (p.G % 8 == 0) hpw = 8;
  else if (p.G % 4 == 0) hpw = 4;
  else if (p.G % 2 == 0) hpw = 2;
  const int bmp = kQW * (kNW / hpw);
  const int npb = (p.nrows + bmp - 1) / bmp;
  const uint32_t total = (uint32_t)p.B * p.Hkv * (p.G / hpw) * npb;
  dim3 grid(total), block(kThreads);
#define ORTHROS_BAND(DD, HH) hipLaunchKernelGGL((band_kernel<DD, HH>), grid, block, 0, s, p)
  if (d == 128) {
    if (hpw == 8) ORTHROS_BAND(128, 8);
    else if (hpw == 4) ORTHROS_BAND(128, 4);
    else if (hpw == 2) ORTHROS_BAND(128, 2);
    else ORTHROS_BAND(128, 1);
  } else {
    if (hpw == 8) ORTHROS_BAND(64, 8);
    else if (hpw == 4) ORTHROS_BAND(64, 4);
    else if (hpw == 2) ORTHROS_BAND(64, 2);
    else ORTHROS_BAND(64, 1);
  }
#undef ORTHROS_BAND
  return hipGetLastError();
}

}  // namespace orthros
