// Banded flash attention, bf16 in / bf16 out, fp32 softmax and accumulation.
//
// Computes "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers", §3.1
// Eq. 4 for every base row t (keys max(0, t-w+1) .. t) and, with a window >= T, Eq. 5 for
// every output row (keys 0 .. t, the pre-training regime of §3.2). The query's scale-offset
// (§3.1, q = alpha (.) q_raw + beta) is applied while the query fragment is loaded, together
// with the score scale and log2 e, and rounded once to bf16.
//
// Work-group: 8 wavefronts (2 per SIMD) = HPW query heads sharing one kv head x (8 / HPW)
// position blocks of 32 rows. One kv head's 64-key K and V tiles are staged through LDS
// (double buffered, row-major, 16-byte slots XOR-swizzled per row so the reads below hit all
// 64 banks) and read by all 8 wavefronts. Per wavefront and tile, with the transposed score
// layout S^T (keys x queries) so each lane owns one query and its softmax stays in registers:
//   S^T[64 x 32]  = K . Q^T        16 x mfma_f32_32x32x16_bf16 (d = 128)
//   mask (edge tiles only), online softmax in the exp2 domain with a lazily rescaled max
//   O^T[d x 32]  += V^T . P^T      16 x mfma_f32_32x32x16_bf16; P^T comes straight from the
//                                  S^T registers; V^T is read with the LDS transpose read
//                                  (ds_read_b64_tr_b16) in the key order of those registers
// Tiles are visited from the diagonal downwards, so each row's first tile holds its own key.
// Tiles outside a wavefront's band are skipped; tiles inside every row's band run unmasked.
#include "common.h"
#include "launch.h"

namespace orthros {

namespace {
constexpr int kTK = 64;      // keys per tile
constexpr int kQW = 32;      // query rows per wavefront
constexpr int kNW = 8;       // wavefronts per work-group
constexpr float kTau = 8.f;  // rescale only when the running max grows by more than 2^8

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ bf16x8 cat_tr(s16x4 lo, s16x4 hi) {
  s16x4 v8[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v8);
}
}  // namespace

template <int D, int HPW>
__global__ __launch_bounds__(512) void band_kernel(BandParams p) {
  constexpr int NCH = D / 8;             // 16-byte slots per row
  constexpr int ROWB = D * 2;            // bytes per K/V row
  constexpr int TILEB = kTK * ROWB;      // bytes per K (or V) tile
  constexpr int STAGEB = 2 * TILEB;      // K + V
  constexpr int PB = kNW / HPW;          // position blocks per work-group
  constexpr int BMP = kQW * PB;          // positions per work-group
  constexpr int NKS = D / 16;            // QK k-steps
  constexpr int NDT = D / 32;            // O^T tiles
  constexpr int SCH = kTK * NCH / 512;   // staged chunks per thread per tile (K and V each)
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGEB];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int nhc = p.G / HPW;
  const int npb = (p.T + BMP - 1) / BMP;
  const uint32_t total = (uint32_t)p.B * p.Hkv * nhc * npb;
  const uint32_t lid = xcd_swizzle(blockIdx.x, total);
  const bool causal = p.window >= p.T;
  int pb, rest;
  if (causal) {  // longest rows first
    const int inner = p.B * p.Hkv * nhc;
    pb = npb - 1 - (int)(lid / inner);
    rest = (int)(lid % inner);
  } else {
    pb = (int)(lid % npb);
    rest = (int)(lid / npb);
  }
  const int hc = rest % nhc;
  rest /= nhc;
  const int g = rest % p.Hkv;
  const int b = rest / p.Hkv;
  const int t0 = pb * BMP;
  const int h = g * p.G + hc * HPW + (wv % HPW);
  const int t0w = t0 + kQW * (wv / HPW);
  const int j = lane & 31;   // query column of this lane
  const int hh = lane >> 5;  // lane half
  const int tq = t0w + j;    // this lane's query position

  // Query fragment (B operand of 32x32x16): lane (j, hh) holds channels 16*s + 8*hh + e.
  bf16x8 qf[NKS];
  {
    const bool ok = tq < p.T;
    const uint16_t* qr = reinterpret_cast<const uint16_t*>(p.q) + (idx_t)b * p.q_sb +
                         (idx_t)(ok ? tq : 0) * p.q_st + (idx_t)h * p.q_sh;
    const float* al = p.alpha + (idx_t)h * D;
    const float* be = p.beta + (idx_t)h * D;
    const float sc = ok ? p.scale_log2 : 0.f;
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
  }

  // Key range of the work-group and of this wavefront.
  const int w = p.window;
  const int glo = t0 - w + 1 > 0 ? t0 - w + 1 : 0;
  const int ghi = (t0 + BMP - 1 < p.T - 1) ? t0 + BMP - 1 : p.T - 1;
  const int tile_lo = glo / kTK * kTK;
  const int tile_hi = ghi / kTK * kTK;
  const bool wactive = t0w < p.T;
  const int wmax = (t0w + kQW - 1 < p.T - 1) ? t0w + kQW - 1 : p.T - 1;  // last valid row
  const int wlo = t0w - w + 1;  // lowest key any row of this wavefront needs (may be < 0)

  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(p.k) + (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(p.v) + (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;

  // Staging: thread tid moves chunks ci = tid + 512 i (row ci / NCH, slot ci % NCH) of the K
  // and V tiles. K slot c of row r lives at c ^ (r % NCH); V slot c at c ^ 4((r >> 1) % (NCH/4)).
  int srow[SCH], scol[SCH], skoff[SCH], svoff[SCH];
#pragma unroll
  for (int i = 0; i < SCH; ++i) {
    const int ci = tid + 512 * i;
    const int r = ci / NCH, c = ci % NCH;
    srow[i] = r;
    scol[i] = 8 * c;
    skoff[i] = r * ROWB + 16 * (c ^ (r % NCH));
    svoff[i] = TILEB + r * ROWB + 16 * (c ^ (4 * ((r >> 1) % (NCH / 4))));
  }
  u32x4 kreg[SCH], vreg[SCH];
  auto load_tile = [&](int tb) {
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      int key = tb + srow[i];
      if (key > p.T - 1) key = p.T - 1;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (idx_t)key * p.k_st + scol[i]);
      vreg[i] = *reinterpret_cast<const u32x4*>(vbase + (idx_t)key * p.k_st + scol[i]);
    }
  };
  auto store_tile = [&](int stage) {
    unsigned char* st = smem + stage * STAGEB;
#pragma unroll
    for (int i = 0; i < SCH; ++i) {
      *reinterpret_cast<u32x4*>(st + skoff[i]) = kreg[i];
      *reinterpret_cast<u32x4*>(st + svoff[i]) = vreg[i];
    }
  };

  // Per-lane LDS read offsets (bytes within a stage).
  // QK A operand: key row 32 mt + j, channel slot 2 s + hh.
  int qk_off[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) qk_off[s] = j * ROWB + 16 * ((2 * s + hh) ^ (j % NCH));
  // PV A operand (transpose read): lane group G = lane / 16 supplies, from its lane L, key row
  // 16 ks + 8 h2 + 4 (G / 2) + L / 4 at channels 32 dt + 16 (G % 2) + 4 (L % 4) .. + 3.
  int pv_off[NDT];
  {
    const int G = lane >> 4, L = lane & 15;
    const int row = 4 * (G >> 1) + (L >> 2);  // + 16 ks + 8 h2 (row-independent swizzle)
    const int fv = 4 * ((row >> 1) % (NCH / 4));
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
  float m = kNegInf, l = 0.f;

  auto compute = [&](unsigned char* st, int tb) {
    f32x16 S0, S1;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      S0[r] = 0.f;
      S1[r] = 0.f;
    }
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(st + qk_off[s]);
      const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(st + qk_off[s] + 32 * ROWB);
      S0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], S0, 0, 0, 0);
      S1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], S1, 0, 0, 0);
    }
    // Unmasked only if every key of the tile lies in every row's window.
    const bool full = (tb + kTK - 1 <= t0w) && (tb >= wmax - w + 1) && (tb + kTK - 1 <= p.T - 1);
    if (!full) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int k0 = tb + 8 * (r >> 2) + 4 * hh + (r & 3);
        const int k1 = k0 + 32;
        const bool ok0 = k0 <= tq && k0 > tq - w && k0 < p.T;
        const bool ok1 = k1 <= tq && k1 > tq - w && k1 < p.T;
        S0[r] = ok0 ? S0[r] : kNegInf;
        S1[r] = ok1 ? S1[r] : kNegInf;
      }
    }
    float mx = fmaxf(S0[0], S1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    const float mn = fmaxf(m, mx);
    const bool need = mn > m + kTau;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float alpha = need ? fast_exp2(m - mn) : 1.f;
      m = need ? mn : m;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) O[dt] *= alpha;
    }
    const float ms = m == kNegInf ? 0.f : m;
    bf16x8 P[4];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      P[r >> 3][r & 7] = (__bf16)fast_exp2(S0[r] - ms);
      P[2 + (r >> 3)][r & 7] = (__bf16)fast_exp2(S1[r] - ms);
    }
    // Row sum of the rounded probabilities (the same values the value product uses).
    float ps = 0.f;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) ps += (float)P[q][e];
    l += ps;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        unsigned char* base = st + pv_off[dt] + (16 * ks) * ROWB;
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + 8 * ROWB));
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(lo, hi), P[ks], O[dt], 0, 0, 0);
      }
    }
  };

  load_tile(tile_hi);
  store_tile(0);
  __syncthreads();
  if (tile_hi - kTK >= tile_lo) load_tile(tile_hi - kTK);
  int stage = 0;
  for (int tb = tile_hi; tb >= tile_lo; tb -= kTK) {
    const bool skip = !wactive || tb > wmax || tb + kTK - 1 < wlo;
    if (!skip) compute(smem + stage * STAGEB, tb);
    if (tb - kTK >= tile_lo) {
      store_tile(stage ^ 1);
      if (tb - 2 * kTK >= tile_lo) load_tile(tb - 2 * kTK);
    }
    __syncthreads();
    stage ^= 1;
  }

  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);  // both lane halves
  if (wactive && tq < p.T) {
    const float inv = 1.f / lt;
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + (idx_t)b * p.o_sb + (idx_t)tq * p.o_st + (idx_t)h * p.o_sh;
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
  const int npb = (p.T + bmp - 1) / bmp;
  const uint32_t total = (uint32_t)p.B * p.Hkv * (p.G / hpw) * npb;
  dim3 grid(total), block(512);
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
