// Banded flash attention, bf16 in / bf16 out, fp32 softmax and accumulation.
//
// Computes "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers", §3.1
// Eq. 4 for every base row t (keys max(0, t-w+1) .. t) and, with a window >= T, Eq. 5 for
// every output row (keys 0 .. t, the pre-training regime of §3.2). The query's scale-offset
// (§3.1, q = alpha (.) q_raw + beta) is applied while the query fragment is loaded, together
// with the score scale and log2 e, and rounded once to bf16.
//
// Work-group: 8 wavefronts (2 per SIMD) = HPW query heads sharing one kv head x (8 / HPW)
// position blocks of 32 rows; one kv head's 64-key K/V tiles are staged through LDS (double
// buffered, K row-major, V transposed to key-contiguous) and read by all 8 wavefronts. Per
// wavefront and tile, with the transposed score layout S^T (keys x queries) so each lane owns
// one query and its softmax reductions stay in registers:
//   S^T[64 x 32]  = K . Q^T        16 x mfma_f32_32x32x16_bf16 (d = 128)
//   mask (edge tiles only), online softmax with a lazily rescaled running max
//   O^T[d x 32]  += V^T . P^T      16 x mfma_f32_32x32x16_bf16; P^T comes straight from the
//                                  S^T registers, V^T's keys permuted to match their order
// Tiles are visited from the diagonal downwards, so each row's first tile holds its own key.
// Tiles outside a wavefront's band are skipped; tiles inside every row's band run unmasked.
#include "common.h"
#include "launch.h"

namespace orthros {

namespace {
constexpr int kTK = 64;   // keys per tile
constexpr int kQW = 32;   // query rows per wavefront
constexpr int kNW = 8;    // wavefronts per work-group
constexpr float kTau = 8.f;  // rescale only when the running max grows by more than 2^8

template <int D>
struct BandSmem {
  static constexpr int KSTR = D + 8;
  static constexpr int VSTR = kTK + 8;
  static constexpr int KBUF = kTK * KSTR;
  static constexpr int VBUF = D * VSTR;
  static constexpr int BYTES = 2 * (KBUF + VBUF) * 2;
};

// Position of key k (0..63) inside a V^T row: within every 16 keys the groups of 4 are stored
// in the order 0, 2, 1, 3, which is the key order a 32x32 score tile hands the PV product.
__device__ __forceinline__ int vpos(int k) {
  const int grp = (k >> 2) & 3;
  const int pg = (grp == 1) ? 2 : (grp == 2 ? 1 : grp);
  return (k & ~15) | (pg << 2) | (k & 3);
}
}  // namespace

template <int D, int HPW>
__global__ __launch_bounds__(512) void band_kernel(BandParams p) {
  using SM = BandSmem<D>;
  constexpr int KSTR = SM::KSTR, VSTR = SM::VSTR;
  constexpr int PB = kNW / HPW;          // position blocks per work-group
  constexpr int BMP = kQW * PB;          // positions per work-group
  constexpr int NKS = D / 16;            // QK k-steps
  constexpr int NDT = D / 32;            // O^T tiles
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int KCH = kTK * CPR / 512;   // K chunks per thread
  constexpr int VITEMS = (kTK / 2) * CPR;  // (key pair, chunk) items per tile
  __shared__ __attribute__((aligned(16))) unsigned char smem[SM::BYTES];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = Ks + 2 * SM::KBUF;

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
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      const int c0 = 16 * s + 8 * hh;
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (ok) raw = *reinterpret_cast<const u32x4*>(qr + c0);
      bf16x8 f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t w = raw[e >> 1];
        const float x = (e & 1) ? bf16_hi(w) : bf16_lo(w);
        f[e] = (__bf16)(ok ? (al[c0 + e] * x + be[c0 + e]) * p.scale_log2 : 0.f);
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

  u32x4 kreg[KCH];
  u32x4 vreg[2];
  auto load_tile = [&](int tb) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + 512 * i;
      const int r = ci / CPR, c = ci % CPR;
      int key = tb + r;
      if (key > p.T - 1) key = p.T - 1;
      kreg[i] = *reinterpret_cast<const u32x4*>(kbase + (idx_t)key * p.k_st + 8 * c);
    }
    if (tid < VITEMS) {
      const int c = tid % CPR, kp = tid / CPR;
      int k0 = tb + 2 * kp, k1 = k0 + 1;
      if (k0 > p.T - 1) k0 = p.T - 1;
      if (k1 > p.T - 1) k1 = p.T - 1;
      vreg[0] = *reinterpret_cast<const u32x4*>(vbase + (idx_t)k0 * p.k_st + 8 * c);
      vreg[1] = *reinterpret_cast<const u32x4*>(vbase + (idx_t)k1 * p.k_st + 8 * c);
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = Ks + buf * SM::KBUF;
    uint16_t* vt = Vt + buf * SM::VBUF;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ci = tid + 512 * i;
      const int r = ci / CPR, c = ci % CPR;
      *reinterpret_cast<u32x4*>(ks + r * KSTR + 8 * c) = kreg[i];
    }
    if (tid < VITEMS) {
      const int c = tid % CPR, kp = tid / CPR;
      const int pos = vpos(2 * kp);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t a = vreg[0][e >> 1], bb = vreg[1][e >> 1];
        const uint32_t wd = (e & 1) ? ((a >> 16) | (bb & 0xffff0000u)) : ((a & 0xffffu) | (bb << 16));
        *reinterpret_cast<uint32_t*>(vt + (8 * c + e) * VSTR + pos) = wd;
      }
    }
  };

  f32x16 O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m = kNegInf, l = 0.f;

  load_tile(tile_hi);
  int buf = 0;
  for (int tb = tile_hi; tb >= tile_lo; tb -= kTK) {
    store_tile(buf);
    __syncthreads();
    if (tb - kTK >= tile_lo) load_tile(tb - kTK);

    const bool skip = !wactive || tb > wmax || tb + kTK - 1 < wlo;
    if (!skip) {
      const uint16_t* ks = Ks + buf * SM::KBUF;
      const uint16_t* vt = Vt + buf * SM::VBUF;
      f32x16 S0, S1;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S0[r] = 0.f;
        S1[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(ks + j * KSTR + 16 * s + 8 * hh);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(ks + (32 + j) * KSTR + 16 * s + 8 * hh);
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
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fmaxf(S0[r], S1[r]));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
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
      float ps = 0.f;
      bf16x8 P[4];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p0 = fast_exp2(S0[r] - ms);
        const float p1 = fast_exp2(S1[r] - ms);
        ps += p0 + p1;
        P[r >> 3][r & 7] = (__bf16)p0;
        P[2 + (r >> 3)][r & 7] = (__bf16)p1;
      }
      l += ps;
#pragma unroll
      for (int ks4 = 0; ks4 < 4; ++ks4) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * dt + j) * VSTR + 16 * ks4 + 8 * hh);
          O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, P[ks4], O[dt], 0, 0, 0);
        }
      }
    }
    buf ^= 1;
  }

  const float lt = l + __shfl_xor(l, 32, 64);  // both lane halves of each query column
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
