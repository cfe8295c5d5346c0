// Banded flash attention, bf16 in / bf16 out, fp32 softmax and accumulation.
//
// Computes "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers", §3.1
// Eq. 4 for every base row t (keys max(0, t-w+1) .. t) and, with a window >= T, Eq. 5 for
// every output row (keys 0 .. t, the pre-training regime of §3.2). The query's scale-offset
// (§3.1, q = alpha (.) q_raw + beta) is applied while the query fragment is loaded, together
// with the score scale and log2 e, and rounded once to bf16.
//
// Work-group: 8 wavefronts (two per SIMD), HPW query heads sharing one kv head x (8 / HPW)
// position blocks of 32 rows. One kv head's keys and values are copied in 64-key units straight
// from global memory into LDS (two K and two V slots of 128 keys; row-major, 16-byte slots
// XOR-swizzled per row so the operand reads hit all 64 banks) and read by all eight wavefronts.
// The copies are waited for only at the barrier that publishes them, one per 128 keys. With the
// transposed score layout S^T (keys x queries) each lane owns one query and its softmax stays in
// registers; per 32-key chunk:
//   S^T[32 x 32]  = K . Q^T        8 x mfma_f32_32x32x16_bf16 (d = 128)
//   online softmax in the exp2 domain, p = exp2(s - m); the reference m moves only when a
//   chunk's probabilities could exceed 2^8 (their sum does), so the common path computes no
//   maximum
//   O^T[d x 32]  += V^T . P^T      8 x mfma_f32_32x32x16_bf16; P^T straight from the S^T
//                                  registers; V^T through the LDS transpose read
// The key loop is software-pipelined over chunks so the vector work of one chunk issues in the
// shadow of the matrix work of its neighbours (see the pipeline comment below). Keys are visited
// from the diagonal downwards.
#include "common.h"
#include "launch.h"
#include "lds_mfma.h"

namespace orthros {

namespace {
constexpr int kTK = 64;      // keys per copy unit
constexpr int kQW = 32;      // query rows per wavefront
constexpr int kNW = 8;       // wavefronts per work-group (two per SIMD)
constexpr int kThreads = 64 * kNW;
constexpr float kLazyBound = 256.f;  // largest tolerated sum of a chunk's probabilities
// Reference of a query that has met no key yet: any finite score then gives an infinite
// tentative probability, which sends the query through the rescale path, and the rescale
// factor exp2(kUnstarted - max) is 0 (nothing has been accumulated).
constexpr float kUnstarted = -1e30f;

}  // namespace

// PAIR: two row sets over the same keys in one launch, work-groups 0 .. n0-1 serving p0, the
// rest p1 (each set in its own work order), so the second set's work-groups fill the CUs the
// first leaves free instead of waiting for its last work-group. Without PAIR only p0 is used
// (the body stays in the kernel itself: as a separate device function it compiled ~2% slower).
template <int D, int HPW, bool PAIR>
__global__ __launch_bounds__(kThreads) void band_kernel(BandParams p0, BandParams p1, uint32_t n0) {
  const bool second = PAIR && blockIdx.x >= n0;
  const BandParams& p = second ? p1 : p0;
  const uint32_t blk = second ? blockIdx.x - n0 : blockIdx.x;
  constexpr int NCH = D / 8;             // 16-byte slots per row
  constexpr int ROWB = D * 2;            // bytes per K/V row
  constexpr int UNITB = kTK * ROWB;      // bytes per 64-key unit of K (or V)
  constexpr int PB = kNW / HPW;          // position blocks per work-group
  constexpr int BMP = kQW * PB;          // positions per work-group
  constexpr int NKS = D / 16;            // QK k-steps
  constexpr int NDT = D / 32;            // O^T tiles
  __shared__ __attribute__((aligned(16))) unsigned char smem[8 * UNITB];  // K slots 0, 1; V slots 2, 3

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nhc = p.G / HPW;
  const int npb = (p.nrows + BMP - 1) / BMP;
  const uint32_t total = (uint32_t)p.B * p.Hkv * nhc * npb;
  const uint32_t lid = xcd_swizzle(blk, total);
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

  // Key range of the work-group, in 64-key units visited from the top down: unit m holds keys
  // unit_hi - 64 m .. + 63, m = 0 .. nunits - 1. Each unit is two 32-key chunks, upper first, so
  // chunk u holds keys chunk_hi - 32 u .. + 31 and the keys descend throughout.
  const int w = p.window;
  const int nk = p.nkeys;
  const int glo = qmin_b - w + 1 > 0 ? qmin_b - w + 1 : 0;
  const int ghi = qmax_b < nk - 1 ? qmax_b : nk - 1;
  const int unit_lo = glo / kTK * kTK;
  const int unit_hi = ghi / kTK * kTK;
  const int nunits = (unit_hi - unit_lo) / kTK + 1;
  // Scalar copies for the loop and the copies (the per-wavefront conditions below keep their
  // vector form: as scalar branches they cost the register allocator more than they save).
  const int unit_hi_s = __builtin_amdgcn_readfirstlane(unit_hi);
  const int nunits_s = __builtin_amdgcn_readfirstlane(nunits);
  const int nspans = (nunits_s + 1) / 2;  // spans of two units (128 keys)
  const int chunk_hi = unit_hi + 32;
  auto chunk_key = [&](int u) { return chunk_hi - 32 * u; };
  // This wavefront's chunks: ua (holds its highest row) .. ub (holds its lowest key).
  const int wlo = qmin_w - w + 1 > 0 ? qmin_w - w + 1 : 0;  // lowest key any row needs
  const int ua = chunk_hi > qmax_w ? (chunk_hi - qmax_w + 31) / 32 : 0;
  const int ub_w = (chunk_hi + 31 - wlo) / 32;
  const int ub = !wactive ? -1 : (ub_w < 2 * nunits - 1 ? ub_w : 2 * nunits - 1);
  auto in_range = [&](int u) { return (u >= ua) & (u <= ub); };
  // Unmasked only if every key of the chunk lies in every row's window.
  auto full = [&](int u) {
    const int kb = chunk_key(u);
    return (kb + 31 <= qmin_w) & (kb >= qmax_w - w + 1) & (kb + 31 <= nk - 1);
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
  // of every unit.
  constexpr int LROWS = 1024 / ROWB;
  constexpr int NINST = kTK / LROWS / kNW;
  static_assert(NINST >= 1 && NINST * LROWS * kNW == kTK, "staging covers a unit exactly");
  // Each lane's byte offsets within a unit are fixed; a unit's base address is a scalar, so a
  // load is one instruction with no address arithmetic. In the unit holding the last key, rows
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
  // Paged pool: a 64-key unit lies inside one page (pages hold >= 64 rows, units start at
  // multiples of 64), so one table entry (a scalar read) gives the unit's base. The entries a
  // span's copies use are read one span ahead.
  auto page_of = [&](int m) -> int32_t {
    const int tb = unit_hi_s - kTK * (m < nunits_s ? m : nunits_s - 1);
    // read through the scalar cache (the table is constant while the kernel runs): a vector
    // load here would make the wave wait for it, and for every copy in flight, on the spot
    const __attribute__((address_space(4))) int32_t* tbl =
        (const __attribute__((address_space(4))) int32_t*)p.pg.table;
    return tbl[(idx_t)b * p.pg.tbl_sb + (tb >> p.pg.ps_log2)];
  };
  // Bytes from the (sequence, kv head) base to unit m, through its table entry `page` in a
  // paged pool (the page's start, k_sp elements of 2 bytes per page, plus the unit's rows). K
  // and V share it, and a unit's V is copied a span after its K, so each unit's offset is
  // formed once.
  const idx_t page_bytes = (idx_t)p.pg.k_sp * 2;
  const int page_mask = (1 << p.pg.ps_log2) - 1;
  auto unit_off = [&](int m, int32_t page) -> idx_t {
    const int tb = unit_hi_s - kTK * m;
    if (!p.pg.table) return (idx_t)tb * rowb;
    if (page < 0 || (int64_t)page >= p.pg.num_pages) {
      __hip_atomic_fetch_or(p.pg.status, kStatusBadPage, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      page = 0;
    }
    return (idx_t)page * page_bytes + (idx_t)(tb & page_mask) * rowb;
  };
  // Unit m of K (or V), `toff` bytes from `base`, -> LDS byte offset `dst`.
  auto copy_unit = [&](int m, idx_t toff, const uint16_t* base, const uint32_t* off, uint32_t dst) {
    const int tb = unit_hi_s - kTK * m;
    const unsigned char* src = reinterpret_cast<const unsigned char*>(base) + toff;
    const uint32_t d0 = lds0 + dst + (uint32_t)(wv_s * NINST) * 1024u;
    if (tb + kTK <= nk) {
#pragma unroll
      for (int i = 0; i < NINST; ++i) copy_to_lds(src, off[i], d0 + (uint32_t)i * 1024u);
    } else {
#pragma unroll
      for (int i = 0; i < NINST; ++i) {
        const int over = srow[i] - (nk - 1 - tb);
        const uint32_t back = over > 0 ? (uint32_t)over * rowb : 0u;
        copy_to_lds(src, off[i] - back, d0 + (uint32_t)i * 1024u);
      }
    }
  };
  // LDS: K spans in slots 0, 1 (span e = units 2e, 2e + 1 at +0 and +UNITB), V spans in slots
  // 2, 3 (V span e = units 2e - 1, 2e at +0 and +UNITB).
  auto k_dst = [&](int m) { return (uint32_t)(((m >> 1) & 1) * 2 * UNITB + (m & 1) * UNITB); };
  auto v_dst = [&](int m) { return (uint32_t)(4 * UNITB + (((m + 1) >> 1) & 1) * 2 * UNITB + (m & 1 ? 0 : UNITB)); };

  // Per-lane LDS read offsets (bytes within a unit).
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
      pv_off[dt] = row * ROWB + 16 * (chunk ^ fv) + 8 * (L & 1);
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
  // A chunk's rows in LDS: ka / va are this lane's read offsets into the span's K / V slot
  // (formed once per span), at the chunk's constant offset `co` in the slot, which folds into
  // the read instructions.
  // Scores of a chunk (NKS MFMAs): S = K rows of the chunk . Q^T.
  auto qk = [&](f32x16& S, const int* ka, int co) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(smem + ka[s] + co);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], s == 0 ? zero16 : S, 0, 0, 0);
    }
  };
  // O^T += V^T . P^T over a chunk (2 16-key steps x NDT MFMAs).
  auto pv = [&](const bf16x8* Ph, const int* va, int co) {
#pragma unroll
    for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        unsigned char* base = smem + va[dt] + co + 16 * k2 * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(lo, hi), Ph[k2], O[dt], 0, 0, 0);
      }
    }
  };
  // Keys of chunk u outside the query's window (or past the sequence) -> -inf.
  auto mask = [&](f32x16& S, int u) {
    const int kb = chunk_key(u) + 4 * hh;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int k = kb + 8 * (r >> 2) + (r & 3);
      const bool ok = (k <= tq) & (k > tq - w) & (k < nk);
      S[r] = ok ? S[r] : kNegInf;
    }
  };
  // Probabilities of one chunk against the current reference (bf16, as the PV operand) and
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
  // After the tentative probabilities of a chunk: the reference moves only if a probability of
  // the query could exceed 2^8 (their sum over both lane halves does; a query meeting its first
  // key has an infinite sum). Then O and l are rescaled and this chunk's probabilities
  // recomputed against the new reference (the scores are kept unshifted, so no other chunk's
  // need a correction). The new reference is the exact maximum, so the probabilities end up
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
  // Region u, one basic block on the common path, so the matrix cores and the vector ALUs work
  // side by side: MFMA scores of chunk u + 1 (into Sn) and PV of chunk u - 1 (from Pp) | the
  // tentative probabilities of chunk u (from Sc into Pc). Returns this lane's part of their
  // sum, 0 if the wavefront has no keys in chunk u (the settle that follows is then a no-op;
  // kept outside the region's branches, where it stays a branch of its own).
  auto region = [&](int u, const int* ka, const int* va, int co, f32x16& Sn, const bf16x8* Pp,
                    f32x16& Sc, bf16x8* Pc) -> float {
    const bool dn = in_range(u + 1), dp = in_range(u - 1), dc = in_range(u);
    float ps = 0.f;
    if (dn & dp & dc & full(u)) {
      qk(Sn, ka, co);
      pv(Pp, va, co);
      ps = expo(Sc, Pc);
      interleave<16, 4, 2, 3>();
    } else {
      if (dn) qk(Sn, ka, co);
      if (dp) pv(Pp, va, co);
      if (dc) {
        mask(Sc, u);
        ps = expo(Sc, Pc);
      }
    }
    return ps;
  };

  // ---- pipeline -----------------------------------------------------------------------------
  // Regions u = -1, 0, 1, ... in order; region u reads K of chunk u + 1 and V of chunk u - 1.
  // A barrier stands before every region u = 4e - 1, after which the span of regions 4e - 1 ..
  // 4e + 2 reads K units 2e, 2e + 1 (chunks 4e .. 4e + 3) and V units 2e - 1, 2e (chunks
  // 4e - 2 .. 4e + 1), and the region at offset q in the span reads each at the constant offset
  // (q / 2) UNITB + (q even ? 32 rows : 0) in its slot. During the span each wavefront copies
  // its rows of K units 2e + 2, 2e + 3 and V units 2e + 1, 2e + 2 into the slots the previous
  // span read, so two K and two V slots (128 KB at d = 128) suffice, and the copies have landed
  // by the next barrier (each wavefront waits for its own before it). A copy instruction holds
  // up its wavefront while the address unit works through the queue, so the two wavefronts of
  // a SIMD take turns: the second (wavefronts 4..7) copies at the top of the span, the first
  // after its first region.
  // Offset of unit 2e + 1 (its K went with span e - 1's copies, its V goes with span e's) and
  // the table entries of units 2e + 2, 2e + 3.
  idx_t off1 = 0;
  int32_t pg2 = 0, pg3 = 0;
  {
    const idx_t off0 = unit_off(0, p.pg.table ? page_of(0) : 0);
    copy_unit(0, off0, kbase, skoff, k_dst(0));
    copy_unit(0, off0, vbase, svoff, v_dst(0));
    if (nunits_s > 1) {
      off1 = unit_off(1, p.pg.table ? page_of(1) : 0);
      copy_unit(1, off1, kbase, skoff, k_dst(1));
    }
    if (p.pg.table) {
      pg2 = page_of(2);
      pg3 = page_of(3);
    }
  }
  wait_lds_copies();
  __syncthreads();

  f32x16 S0 = zero16, S1 = zero16;
  bf16x8 P0[2], P1[2];
  const bool copy_late = wv_s < kNW / 2;  // the first wavefront of its SIMD
  auto copies = [&](int e) {
    const int m = 2 * e;
    const idx_t off2 = unit_off(m + 2, pg2), off3 = unit_off(m + 3, pg3);
    if (m + 1 < nunits_s) copy_unit(m + 1, off1, vbase, svoff, v_dst(m + 1));
    if (m + 2 < nunits_s) {
      copy_unit(m + 2, off2, vbase, svoff, v_dst(m + 2));
      copy_unit(m + 2, off2, kbase, skoff, k_dst(m + 2));
    }
    if (m + 3 < nunits_s) copy_unit(m + 3, off3, kbase, skoff, k_dst(m + 3));
    off1 = off3;
    if (p.pg.table) {  // the next span's entries, read now (after their last use), used then
      pg2 = page_of(m + 4);
      pg3 = page_of(m + 5);
    }
  };
  for (int e = 0; e <= nspans; ++e) {
    if (!copy_late) copies(e);
    // Read offsets into K span e (slot e % 2) and V span e (slot 2 + e % 2).
    int ka[NKS], va[NDT];
    const int ks = (e & 1) * 2 * UNITB, vs = (4 + 2 * (e & 1)) * UNITB;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      ka[s] = qk_off[s] + ks;
      asm volatile("" : "+v"(ka[s]));  // formed here, not inside each region
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      va[dt] = pv_off[dt] + vs;
      asm volatile("" : "+v"(va[dt]));
    }
    const int u0 = 4 * e - 1;
    // The first half of a span runs at raised wavefront priority: the wavefront of a SIMD
    // that lags (the one that copied first) gets the issue slots first.
    __builtin_amdgcn_s_setprio(1);
    float ps = region(u0, ka, va, 32 * ROWB, S0, P0, S1, P1);
    settle(S1, P1, ps);
    if (copy_late) copies(e);
    ps = region(u0 + 1, ka, va, 0, S1, P1, S0, P0);
    __builtin_amdgcn_s_setprio(0);
    settle(S0, P0, ps);
    ps = region(u0 + 2, ka, va, UNITB + 32 * ROWB, S0, P0, S1, P1);
    settle(S1, P1, ps);
    ps = region(u0 + 3, ka, va, UNITB, S1, P1, S0, P0);
    settle(S0, P0, ps);
    if (e < nspans) {
      wait_lds_copies();  // this wave's copies of the next span have landed
      __syncthreads();
    }
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

namespace {
int band_hpw(int G) { return G % 8 == 0 ? 8 : (G % 4 == 0 ? 4 : (G % 2 == 0 ? 2 : 1)); }
uint32_t band_groups(const BandParams& p, int hpw) {
  const int bmp = kQW * (kNW / hpw);
  const int npb = (p.nrows + bmp - 1) / bmp;
  return (uint32_t)p.B * p.Hkv * (p.G / hpw) * npb;
}
}  // namespace

hipError_t launch_band(const BandParams& p, int d, hipStream_t s) {
  const int hpw = band_hpw(p.G);
  dim3 grid(band_groups(p, hpw)), block(kThreads);
#define ORTHROS_BAND(DD, HH) hipLaunchKernelGGL((band_kernel<DD, HH, false>), grid, block, 0, s, p, p, 0u)
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

hipError_t launch_band_pair(const BandParams& p0, const BandParams& p1, int d, hipStream_t s) {
  const int hpw = band_hpw(p0.G);  // both sets share the head grouping
  const uint32_t n0 = band_groups(p0, hpw);
  dim3 grid(n0 + band_groups(p1, hpw)), block(kThreads);
#define ORTHROS_BAND2(DD, HH) hipLaunchKernelGGL((band_kernel<DD, HH, true>), grid, block, 0, s, p0, p1, n0)
  if (d == 128) {
    if (hpw == 8) ORTHROS_BAND2(128, 8);
    else if (hpw == 4) ORTHROS_BAND2(128, 4);
    else if (hpw == 2) ORTHROS_BAND2(128, 2);
    else ORTHROS_BAND2(128, 1);
  } else {
    if (hpw == 8) ORTHROS_BAND2(64, 8);
    else if (hpw == 4) ORTHROS_BAND2(64, 4);
    else if (hpw == 2) ORTHROS_BAND2(64, 2);
    else ORTHROS_BAND2(64, 1);
  }
#undef ORTHROS_BAND2
  return hipGetLastError();
}

}  // namespace orthros
