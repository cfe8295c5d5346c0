// Training backward on the matrix cores (bf16 in, fp32 accumulation).
//
// Gradients of "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers",
// §3.2 Pre-Training regime: base rows (Eq. 4, keys t-w+1 .. t) and output rows (Eq. 5, keys
// 0 .. t) at every position, with respect to the queries, the shared keys and values and the
// scale-offset vectors of §3.1. For a row t with weights P_j = exp(z_j - lse_t) (z_j the scaled
// score, lse_t saved by the forward), output gradient dO and D_t = dO . O_t:
//   dP_j = dO . v_j;  dZ_j = P_j (dP_j - D_t);  dq = s sum_j dZ_j k_j;
//   dk_j += s dZ_j q;  dv_j += P_j dO.
// Kernels:
//   qprep_kernel   q' = bf16((alpha (.) q_raw + beta) s log2 e) for both streams: the score
//                  operand, rounded once as in the forward
//   bwd_q_kernel   per 32 query rows of one stream: dq_raw = alpha (.) dq (the raw query's
//                  gradient) and the rows' scale-offset partial sums, and -D_t and -lse_t (log2
//                  units), the key side's accumulator seeds; bwd_q_pair_kernel runs both
//                  streams' rows in one launch (the bf16 path)
//                    S^T = K Q'^T, dP^T = V dO^T   (A operand: key / value rows from LDS)
//                    dQ^T += K^T dZ^T              (A operand: transposed key reads)
//   bwd_kv_kernel  per 32 keys: dk and dv over both streams' rows of every query head of the
//                  kv head's group
//                    S = Q' K^T, dP = dO V^T       (A operand: query / gradient rows from LDS)
//                    dV^T += dO^T P, dK^T += Q'^T dZ   (A operand: transposed reads)
// Tiles are copied from global memory straight into LDS, 16-byte slots XOR-swizzled by row; a
// product's output registers serve directly as the B operand of the next product, as in the
// forward.
#include "common.h"
#include "launch.h"
#include "launch_bwd.h"
#include "lds_mfma.h"

namespace orthros {

namespace {
constexpr int kTK = 64;     // keys per tile, query side
constexpr int kQW = 32;     // rows per wavefront (query side) / rows per tile (key side)
constexpr int kKNW = 4;     // wavefronts per work-group, key side, 32 keys each
constexpr float kLn2 = 0.69314718055994531f;

// Byte offset of 16-byte slot `chunk` of row `row` of a row-major LDS tile with NCH slots per
// row, the slot index XOR-swizzled by the row. Any 16 consecutive rows place a given slot in
// 16 different 4-bank groups, so a 16-byte row read (16 lanes per LDS cycle, one row each) hits
// all 64 banks; and 4 consecutive rows place a 64-byte run of slots in four different 16-bank
// groups, so a transposed 8-byte read (32 lanes per LDS cycle, 64 bytes from each of 4 rows)
// does too. Rows 16 apart share the swizzle; rows 8 apart differ in its bit 1.
template <int NCH>
__device__ __forceinline__ int swz(int row) {
  return NCH == 16 ? 4 * (row % 4) + (row >> 2) % 4 : 4 * ((row >> 1) % 2) + (row >> 2) % 4;
}
template <int NCH>
__device__ __forceinline__ uint32_t slot_off(int row, int chunk) {
  return (uint32_t)(row * NCH * 16 + 16 * (chunk ^ swz<NCH>(row)));
}

// Transposed-read offsets (bytes, within a tile) for the A operand V^T-style product: lane
// group G = lane / 16 supplies, from its lane L, row 16 ks + 8 h2 + 4 (G / 2) + L / 4 at
// channels 32 dt + 16 (G % 2) + 4 (L % 4) .. + 3; off[h2][dt] covers ks = 0 (ks adds
// 16 ks rows, which leaves the swizzle unchanged).
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, uint32_t (&off)[2][D / 32]) {
  constexpr int NCH = D / 8;
  const int G = lane >> 4, L = lane & 15;
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2) {
    const int row = 8 * h2 + 4 * (G >> 1) + (L >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int chunk = 4 * dt + 2 * (G & 1) + ((L & 3) >> 1);
      off[h2][dt] = slot_off<NCH>(row, chunk) + 8 * (L & 1);
    }
  }
}
}  // namespace

// ---- q' for both streams -----------------------------------------------------------------------
struct QPrepParams {
  const void* q[2];
  const float* alpha[2];
  const float* beta[2];
  void* qp[2];
  idx_t n;   // elements per stream (B T Hq d)
  int hd;    // Hq d (the scale-offset period)
  float c;   // s log2 e
};

// A thread owns 16-byte column chunks of the rows (no index division) and walks the rows of
// its work-group's share; the chunk's scale-offset stays in registers.
__global__ __launch_bounds__(256) void qprep_kernel(QPrepParams p) {
  const int st = blockIdx.y;
  const uint16_t* q = static_cast<const uint16_t*>(p.q[st]);
  uint16_t* o = static_cast<uint16_t*>(p.qp[st]);
  const int nch = p.hd / 8;  // 16-byte chunks per row (hd is a multiple of 8)
  const idx_t rows = p.n / p.hd;
  for (int ch = threadIdx.x; ch < nch; ch += 256) {
    const int c0 = 8 * ch;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(p.alpha[st] + c0);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(p.alpha[st] + c0 + 4);
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(p.beta[st] + c0);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(p.beta[st] + c0 + 4);
#pragma unroll 4
    for (idx_t r = blockIdx.x; r < rows; r += gridDim.x) {
      const idx_t e0 = r * p.hd + c0;
      const u32x4 raw = *reinterpret_cast<const u32x4*>(q + e0);
      u32x4 out;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const uint32_t w = raw[e >> 1];
        const float x0 = bf16_lo(w), x1 = bf16_hi(w);
        const float y0 = ((e < 4 ? a0[e] : a1[e - 4]) * x0 + (e < 4 ? b0[e] : b1[e - 4])) * p.c;
        const float y1 = ((e < 4 ? a0[e + 1] : a1[e - 3]) * x1 + (e < 4 ? b0[e + 1] : b1[e - 3])) * p.c;
        out[e >> 1] = pack_bf16x2(y0, y1);
      }
      *reinterpret_cast<u32x4*>(o + e0) = out;
    }
  }
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Sums v[0..N) over the 32 lanes of each lane half (the lanes sharing lane >> 5), N = 32 M:
// afterwards lane j (= lane & 31) holds in v[0..M) the sums of the original v[M j + i]. Each
// of five steps halves the values a lane holds: the lane keeps one half and adds its partner's
// copy of that half, the partner the other half. Partners are lane j ^ 16 (a swizzle), j ^ 15
// and j ^ 7 (row and half-row mirrors), j ^ 2 and j ^ 1 (quad permutes): the masks span all
// five lane bits, and the bit that decides the kept half (4, 3, 2, 1, 0) differs between
// partners, so both hold the same index range at every step.
template <int N>
__device__ __forceinline__ void lane_transpose_sum(float (&v)[N], int j) {
  static_assert(N % 32 == 0, "32 values or a multiple per lane");
  auto step = [&](auto partner, int n, int bit) {
    const bool up = (j >> bit) & 1;
#pragma unroll
    for (int i = 0; i < n / 2; ++i) {
      const float send = up ? v[i] : v[i + n / 2];
      const float keep = up ? v[i + n / 2] : v[i];
      v[i] = keep + partner(send);
    }
  };
  auto swz16 = [](float x) {  // lane ^ 16 within 32: bit-mode swizzle, xor mask 16
    return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
  };
  auto dpp = [](auto ctrl) {
    return [](float x) {
      return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), decltype(ctrl)::value, 0xF, 0xF, true));
    };
  };
  step(swz16, N, 4);
  step(dpp(std::integral_constant<int, 0x140>{}), N / 2, 3);   // row mirror: lane ^ 15
  step(dpp(std::integral_constant<int, 0x141>{}), N / 4, 2);   // half-row mirror: lane ^ 7
  step(dpp(std::integral_constant<int, 0x4E>{}), N / 8, 1);    // quad permute [2, 3, 0, 1]
  step(dpp(std::integral_constant<int, 0xB1>{}), N / 16, 0);   // quad permute [1, 0, 3, 2]
}

// ---- query side ------------------------------------------------------------------------------
// Work-group: NW wavefronts, HPW query heads of one kv head x (NW / HPW) blocks of 32 rows. p.q
// is q' (prepared); K and V tiles of 64 keys go through a two-slot LDS ring. Rows are positions,
// or (with p.pos) row r sits at position pos[r]. With one or two heads per kv head, NW is 4
// (two work-groups per CU): the work-group's rows then span 128 positions instead of 256, and
// its wavefronts idle on fewer of its tiles (a base-stream wavefront uses w / 64 + 1 of them).
template <int D, int HPW, int NW>
__device__ __forceinline__ void bwd_q_body(const BwdQParams& p, uint32_t blk) {
  constexpr int NCH = D / 8, ROWB = D * 2, TILEB = kTK * ROWB, STAGEB = 2 * TILEB;
  constexpr int PB = NW / HPW, BMP = kQW * PB, NKS = D / 16, NDT = D / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGEB];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = p.T, NR = p.nrows;
  const int nhc = p.G / HPW;
  const int npb = (NR + BMP - 1) / BMP;
  const uint32_t total = (uint32_t)p.B * p.Hkv * nhc * npb;
  const uint32_t lid = xcd_swizzle(blk, total);
  int from_longest, rest;  // a few (sequence, head group) pairs at a time, longest rows first
  grouped_order(lid, p.B * p.Hkv * nhc, npb, 32 * (8 / NW), from_longest, rest);
  const int pb = __builtin_amdgcn_readfirstlane(npb - 1 - from_longest);
  if (pb < 0) return;  // the grid covers exactly npb row blocks; nothing past them
  const int hc = __builtin_amdgcn_readfirstlane(rest % nhc);
  rest /= nhc;
  const int g = __builtin_amdgcn_readfirstlane(rest % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(rest / p.Hkv);
  const int h = g * p.G + hc * HPW + (wv % HPW);
  const int r0 = pb * BMP;
  const int r0w = r0 + kQW * (wv / HPW);
  const int j = lane & 31, hh = lane >> 5;
  const int row = r0w + j;
  const bool rvalid = row < NR;
  const bool wactive = r0w < NR;
  const int qrow = rvalid ? row : NR - 1;
  const int w = p.window < T ? p.window : T;

  // Row data: q' and dO fragments (B operands), D_t = dO . O, lse in log2 units.
  const idx_t rbase = ((idx_t)b * NR + qrow) * p.Hq * D + (idx_t)h * D;
  bf16x8 qf[NKS], dof[NKS];
  float dsum = 0.f;
#pragma unroll
  for (int s = 0; s < NKS; ++s) {
    const int c0 = 16 * s + 8 * hh;
    qf[s] = *reinterpret_cast<const bf16x8*>(static_cast<const uint16_t*>(p.q) + rbase + c0);
    const u32x4 dr = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.dout) + rbase + c0);
    const u32x4 orr = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.o) + rbase + c0);
    dof[s] = __builtin_bit_cast(bf16x8, dr);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dsum += bf16_lo(dr[e]) * bf16_lo(orr[e]) + bf16_hi(dr[e]) * bf16_hi(orr[e]);
  }
  // Wait for the fragments here: a wait the compiler would otherwise leave inside the tile loop
  // would also wait for the tile copies in flight (the hardware counts them with these loads).
#pragma unroll
  for (int s = 0; s < NKS; ++s) asm volatile("" : "+v"(qf[s]));
  const float Dt = lane_pair_sum(dsum);
  const idx_t lrow = ((idx_t)b * p.Hq + h) * NR + qrow;
  const float lse2 = p.lse[lrow] * kLog2e;
  // for the key side, the seeds of its score and dP accumulators: -lse (log2 units) and -D
  if (rvalid && hh == 0) {
    p.D[lrow] = -Dt;
    p.lse2n[lrow] = -lse2;
  }

  // Row positions: the lowest and highest of this wavefront's rows and of the work-group's.
  int qmin_w, qmax_w, qmin_b, qmax_b, tq;
  if (!p.pos) {
    const int last_w = r0w + kQW - 1 < NR - 1 ? r0w + kQW - 1 : NR - 1;
    const int last_b = r0 + BMP - 1 < NR - 1 ? r0 + BMP - 1 : NR - 1;
    qmin_w = r0w;
    qmax_w = last_w;
    qmin_b = r0;
    qmax_b = last_b;
    tq = rvalid ? row : last_w;
  } else {
    __shared__ int wrange[2 * NW];
    int mine = p.pos[qrow];
    mine = mine < 0 ? 0 : (mine > T - 1 ? T - 1 : mine);  // clamped into [0, T)
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
    for (int i = 0; i < NW; ++i) {
      qmin_b = min(qmin_b, wrange[2 * i]);
      qmax_b = max(qmax_b, wrange[2 * i + 1]);
    }
    tq = rvalid ? mine : qmax_w;  // rows past the end compute on a valid position, unstored
  }
  // Key range of the work-group and of this wavefront (tiles ascending from tile_lo).
  const int glo = qmin_b - w + 1 > 0 ? qmin_b - w + 1 : 0;
  const int tile_lo = __builtin_amdgcn_readfirstlane(glo / kTK * kTK);
  const int ntiles = __builtin_amdgcn_readfirstlane((qmax_b / kTK * kTK - glo / kTK * kTK) / kTK + 1);
  const int wlo = qmin_w - w + 1 > 0 ? qmin_w - w + 1 : 0;
  const int ea = (wlo / kTK * kTK - tile_lo) / kTK;
  const int eb = (qmax_w / kTK * kTK - tile_lo) / kTK;
  auto full = [&](int tb) { return tb + kTK - 1 <= qmin_w && tb >= qmax_w - w + 1 && tb + kTK - 1 <= T - 1; };

  // Tile copies (global side swizzled; wave wv fills rows (wv NINST + i) LROWS .. of a tile).
  constexpr int LROWS = 1024 / ROWB;
  constexpr int NINST = kTK / LROWS / NW;
  static_assert(NINST >= 1 && NINST * LROWS * NW == kTK, "copies cover a tile");
  const uint32_t rowb = (uint32_t)p.Hkv * D * 2u;
  const unsigned char* kb = reinterpret_cast<const unsigned char*>(p.k) + ((idx_t)b * T * p.Hkv + g) * D * 2;
  const unsigned char* vb = reinterpret_cast<const unsigned char*>(p.v) + ((idx_t)b * T * p.Hkv + g) * D * 2;
  uint32_t coff[NINST];
  int crow[NINST];
#pragma unroll
  for (int i = 0; i < NINST; ++i) {
    const int r = (wv * NINST + i) * LROWS + lane / NCH;
    const int c = lane % NCH;
    crow[i] = r;
    coff[i] = (uint32_t)r * rowb + 16u * (uint32_t)(c ^ swz<NCH>(r));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  const int wv_s = __builtin_amdgcn_readfirstlane(wv);
  auto load_tile = [&](int e) {
    const int tb = tile_lo + kTK * e;
    const unsigned char* kt = kb + (idx_t)tb * rowb;
    const unsigned char* vt = vb + (idx_t)tb * rowb;
    const uint32_t st = lds0 + (uint32_t)((e & 1) * STAGEB);
    if (tb + kTK <= T) {  // a whole tile
#pragma unroll
      for (int i = 0; i < NINST; ++i) {
        const uint32_t kd = st + (uint32_t)(wv_s * NINST + i) * 1024u;
        copy_to_lds(kt, coff[i], kd);
        copy_to_lds(vt, coff[i], kd + TILEB);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NINST; ++i) {
        const int over = crow[i] - (T - 1 - tb);  // rows past the end re-read the last row
        const uint32_t back = over > 0 ? (uint32_t)over * rowb : 0u;
        const uint32_t kd = st + (uint32_t)(wv_s * NINST + i) * 1024u;
        copy_to_lds(kt, coff[i] - back, kd);
        copy_to_lds(vt, coff[i] - back, kd + TILEB);
      }
    }
  };

  uint32_t rd_off[NKS];
#pragma unroll
  for (int s = 0; s < NKS; ++s) rd_off[s] = slot_off<NCH>(j, 2 * s + hh);
  uint32_t tr_off[2][NDT];
  tr_offsets<D>(lane, tr_off);

  f32x16 dQ[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQ[dt][r] = 0.f;
  // Each lane holds one query row, so its -lse and -D are the same for all 16 registers of a
  // score tile: they seed the accumulators of S and dP, which then come out as s - lse and
  // dP - D with no per-element subtraction.
  f32x16 seedS, seedD;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    seedS[r] = -lse2;
    seedD[r] = -Dt;
  }

  load_tile(0);
  wait_lds_copies();
  __syncthreads();
  for (int e = 0; e < ntiles; ++e) {
    if (e + 1 < ntiles) load_tile(e + 1);
    if (wactive && e >= ea && e <= eb) {
      const int tb = tile_lo + kTK * e;
      const bool fl = full(tb);
      const unsigned char* st = smem + (e & 1) * STAGEB;
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        f32x16 S = seedS, dP = seedD;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(st + 32 * m * ROWB + rd_off[s]);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], S, 0, 0, 0);
        }
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(st + TILEB + 32 * m * ROWB + rd_off[s]);
          dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dof[s], dP, 0, 0, 0);
        }
        if (!fl) {
          const int kk = tb + 32 * m + 4 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kk + 8 * (r >> 2) + (r & 3);
            const bool ok = (key <= tq) & (key > tq - w) & (key < T);  // no branches
            S[r] = ok ? S[r] : kNegInf;
          }
        }
        bf16x8 Z[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float pr = fast_exp2(S[r]);
          Z[r >> 3][r & 7] = (__bf16)(pr * dP[r]);
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const unsigned char* base = st + 16 * (2 * m + k2) * ROWB;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + tr_off[0][dt]));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + tr_off[1][dt]));
            dQ[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(lo, hi), Z[k2], dQ[dt], 0, 0, 0);
          }
        }
      }
    }
    wait_lds_copies();
    __syncthreads();
  }

  if (p.part) {
    // The scale-offset step (§3.1: q = alpha (.) q_raw + beta) folded in: dq_raw = alpha (.) dq,
    // and this wavefront's 32 rows summed into dalpha (dq (.) q_raw) and dbeta (dq) partials.
    if (!wactive) return;
    constexpr int NV = 16 * NDT, M = NV / 32;  // values per lane; sums per lane after reducing
    const idx_t roff = ((idx_t)b * NR + qrow) * p.Hq * D + (idx_t)h * D;
    const uint16_t* qr = static_cast<const uint16_t*>(p.qraw) + roff;
    uint16_t* dr = static_cast<uint16_t*>(p.dq_raw) + roff;
    const float* al = p.alpha + (idx_t)h * D;
    // value k of a lane: channel 32 (k / 16) + 8 ((k % 16) / 4) + 4 hh + k % 4 of its row
    auto chan = [&](int k) { return 32 * (k / 16) + 8 * ((k % 16) / 4) + 4 * hh + k % 4; };
    u32x2 qw[NV / 4];
#pragma unroll
    for (int t = 0; t < NV / 4; ++t)  // issued first: they land while the dbeta sums reduce
      qw[t] = *reinterpret_cast<const u32x2*>(qr + chan(4 * t));
    float x[NV], vs[NV];
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      x[k] = rvalid ? dQ[k / 16][k % 16] * p.scale : 0.f;
      vs[k] = x[k];
    }
    const int chunk = b * p.nrt + r0w / kQW;
    float* prt = p.part + (idx_t)chunk * 2 * p.Hq * D + (idx_t)h * D;
    // after the reduction lane j holds the sums of values M j .. M j + M - 1 (adjacent channels)
    auto store_sums = [&](float* dst) {
      if constexpr (M == 2) {
        *reinterpret_cast<f32x2*>(dst + chan(2 * j)) = f32x2{vs[0], vs[1]};
      } else {
        dst[chan(j)] = vs[0];
      }
    };
    lane_transpose_sum(vs, j);
    store_sums(prt + (idx_t)p.Hq * D);  // [1]: dbeta
#pragma unroll
    for (int t = 0; t < NV / 4; ++t) {
      const float qv[4] = {bf16_lo(qw[t][0]), bf16_hi(qw[t][0]), bf16_lo(qw[t][1]), bf16_hi(qw[t][1])};
      if (rvalid) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(al + chan(4 * t));
        u32x2 o;
        o[0] = pack_bf16x2(a[0] * x[4 * t], a[1] * x[4 * t + 1]);
        o[1] = pack_bf16x2(a[2] * x[4 * t + 2], a[3] * x[4 * t + 3]);
        *reinterpret_cast<u32x2*>(dr + chan(4 * t)) = o;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) vs[4 * t + i] = x[4 * t + i] * qv[i];
    }
    lane_transpose_sum(vs, j);
    store_sums(prt);  // [0]: dalpha
    return;
  }
  if (rvalid) {
    float* out = p.dq + ((idx_t)b * NR + row) * p.Hq * D + (idx_t)h * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 v4;
#pragma unroll
        for (int i = 0; i < 4; ++i) v4[i] = dQ[dt][4 * rg + i] * p.scale;
        *reinterpret_cast<f32x4*>(out + 32 * dt + 8 * rg + 4 * hh) = v4;
      }
  }
}

template <int D, int HPW, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_q_kernel(BwdQParams p) {
  bwd_q_body<D, HPW, NW>(p, blockIdx.x);
}
// Both streams' query sides in one launch: work-groups 0 .. n0-1 serve p0, the rest p1 (each
// stream's own work order within its range), so the second stream's work-groups start as the
// first stream's leave CUs free.
template <int D, int HPW, int NW>
__global__ __launch_bounds__(64 * NW, 8 / NW) void bwd_q_pair_kernel(BwdQParams p0, BwdQParams p1,
                                                                    uint32_t n0) {
  if (blockIdx.x < n0)
    bwd_q_body<D, HPW, NW>(p0, blockIdx.x);
  else
    bwd_q_body<D, HPW, NW>(p1, blockIdx.x - n0);
}

// ---- key side --------------------------------------------------------------------------------
// Work-group: 4 wavefronts, 128 keys of one kv head (wavefront wv owns keys k0 + 32 wv ..).
// The keys' fragments stay in registers, their values in LDS; 32-row query tiles (q', dO,
// lse, D and the rows' positions) of both streams and every head of the group go through a
// two-slot LDS ring. A stream's rows are its positions, or a row list (every tile visited).
template <int D>
__global__ __launch_bounds__(64 * kKNW, 2) void bwd_kv_kernel(BwdKVParams p) {
  constexpr int NCH = D / 8, ROWB = D * 2, NKS = D / 16, NDT = D / 32;
  constexpr int KB = kKNW * 32;                  // keys per work-group
  constexpr int VBYTES = KB * ROWB;              // value block
  constexpr int QTB = kQW * ROWB;                // one 32-row tile
  constexpr int STG = 2 * QTB + 3 * kQW * 4;     // q', dO, lse, D, positions
  __shared__ __attribute__((aligned(16))) unsigned char smem[VBYTES + 2 * STG];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int T = p.T;
  const int nkb = (T + KB - 1) / KB;
  const uint32_t total = (uint32_t)p.B * p.Hkv * nkb;
  const uint32_t lid = xcd_swizzle(blockIdx.x, total);
  const int bg = p.B * p.Hkv;
  int kbo, pr;  // a few (sequence, kv head) pairs at a time, key block 0 (most rows) first
  grouped_order(lid, bg, nkb, 64, kbo, pr);
  const int kbi = __builtin_amdgcn_readfirstlane(kbo);
  const int g = __builtin_amdgcn_readfirstlane(pr % p.Hkv);
  const int b = __builtin_amdgcn_readfirstlane(pr / p.Hkv);
  const int k0 = kbi * KB;
  const int k0w = k0 + 32 * wv;
  const int j = lane & 31, hh = lane >> 5;
  const int key = k0w + j;
  const bool kvalid = key < T;
  const int wk_s = __builtin_amdgcn_readfirstlane(wv);

  const idx_t kst = (idx_t)p.Hkv * D;  // elements between consecutive keys
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + (idx_t)b * T * kst + (idx_t)g * D;
  // K^T fragments (B operand of S = Q' K^T): lane (key j, half hh) holds channels 16 s + 8 hh ..
  bf16x8 kf[NKS];
  {
    const uint16_t* kr = kg + (idx_t)(kvalid ? key : T - 1) * kst;
#pragma unroll
    for (int s = 0; s < NKS; ++s) kf[s] = *reinterpret_cast<const bf16x8*>(kr + 16 * s + 8 * hh);
    // waited for here, not inside the item loop, where the wait would include the item copies
#pragma unroll
    for (int s = 0; s < NKS; ++s) asm volatile("" : "+v"(kf[s]));
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) unsigned char*)smem);
  // Value block -> LDS (rows past the end re-read the last row).
  {
    constexpr int LROWS = 1024 / ROWB;
    constexpr int NV = KB / LROWS / kKNW;
    // 64-bit base at the block's first key; per-lane offsets stay within the block
    const unsigned char* vg = reinterpret_cast<const unsigned char*>(
        static_cast<const uint16_t*>(p.v) + ((idx_t)b * T + k0) * kst + (idx_t)g * D);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = (wv * NV + i) * LROWS + lane / NCH;
      const int c = lane % NCH;
      const int kr = k0 + r < T ? r : T - 1 - k0;  // rows past the end re-read the last key
      copy_to_lds(vg, (uint32_t)kr * (uint32_t)(kst * 2) + 16u * (uint32_t)(c ^ swz<NCH>(r)),
                  lds0 + (uint32_t)(wk_s * NV + i) * 1024u);
    }
  }

  // Row tiles: a stream whose rows are positions covers rows k0 .. min(T-1, k0 + KB - 1 +
  // w_st - 1); a row list is visited whole.
  int wst[2], qt0[2], nqt[2];
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    wst[st] = p.window[st] < T ? p.window[st] : T;
    if (p.pos[st]) {
      qt0[st] = 0;
      nqt[st] = (p.nrows[st] + kQW - 1) / kQW;
    } else {
      const int hi = k0 + KB - 1 + wst[st] - 1 < T - 1 ? k0 + KB - 1 + wst[st] - 1 : T - 1;
      qt0[st] = k0 / kQW;
      nqt[st] = hi / kQW - qt0[st] + 1;
    }
  }
  const int n0 = p.G * nqt[0];
  const int nitems = n0 + p.G * nqt[1];
  // Items in order: stream 0's row tiles head by head, then stream 1's, stepped by counters
  // (no division). The streams' arguments are read once here, so picking one per item is a
  // select, not a load.
  struct Item {
    int st, hd, qt;
  };
  const Item first{n0 > 0 ? 0 : 1, g * p.G, n0 > 0 ? qt0[0] : qt0[1]};
  auto next_item = [&](Item it) {
    ++it.qt;
    if (it.qt == (it.st ? qt0[1] + nqt[1] : qt0[0] + nqt[0])) {
      ++it.hd;
      it.qt = it.st ? qt0[1] : qt0[0];
      if (it.hd == (g + 1) * p.G) {
        it.st = 1;
        it.hd = g * p.G;
        it.qt = qt0[1];
      }
    }
    return it;
  };
  const uint16_t* qs[2] = {static_cast<const uint16_t*>(p.q[0]), static_cast<const uint16_t*>(p.q[1])};
  const uint16_t* ds[2] = {static_cast<const uint16_t*>(p.dout[0]), static_cast<const uint16_t*>(p.dout[1])};
  const float* ls[2] = {p.lse[0], p.lse[1]};
  const float* dd[2] = {p.D[0], p.D[1]};
  const int* ps2[2] = {p.pos[0], p.pos[1]};
  const int nr2[2] = {p.nrows[0], p.nrows[1]};

  // Per-item copies: q' and dO tiles of 32 rows (rows past the end re-read the last row).
  constexpr int LROWS = 1024 / ROWB;
  constexpr int NQI = kQW / LROWS / kKNW;
  static_assert(NQI >= 1 && NQI * LROWS * kKNW == kQW, "copies cover a row tile");
  uint32_t coff[NQI];
  int crow[NQI];
#pragma unroll
  for (int i = 0; i < NQI; ++i) {
    const int r = (wv * NQI + i) * LROWS + lane / NCH;
    const int c = lane % NCH;
    crow[i] = r;
    coff[i] = (uint32_t)r * (uint32_t)(p.Hq * D * 2) + 16u * (uint32_t)(c ^ swz<NCH>(r));
  }
  const uint32_t rowq = (uint32_t)p.Hq * D * 2;
  // The rows' lse, D and raw positions go straight to LDS as well (4 bytes per lane, lanes
  // 0..31 of wavefront 0; rows past the end re-read the last row; a stream without a row list
  // copies its lse into the unused position slot), so no register ever waits for them.
  auto load_item = [&](const Item& it, int slot) {
    const int st = it.st, hd = it.hd, t0 = it.qt * kQW;
    const int NR = st ? nr2[1] : nr2[0];
    const idx_t off0 = ((idx_t)b * NR + t0) * p.Hq * D + (idx_t)hd * D;
    const unsigned char* qg = reinterpret_cast<const unsigned char*>((st ? qs[1] : qs[0]) + off0);
    const unsigned char* dg = reinterpret_cast<const unsigned char*>((st ? ds[1] : ds[0]) + off0);
    const uint32_t sb = lds0 + VBYTES + (uint32_t)(slot * STG);
    if (t0 + kQW <= NR) {  // a whole tile (every tile but a stream's last)
#pragma unroll
      for (int k = 0; k < NQI; ++k) {
        const uint32_t dst = sb + (uint32_t)(wk_s * NQI + k) * 1024u;
        copy_to_lds(qg, coff[k], dst);
        copy_to_lds(dg, coff[k], dst + QTB);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NQI; ++k) {
        const int over = crow[k] - (NR - 1 - t0);  // rows past the end re-read the last row
        const uint32_t back = over > 0 ? (uint32_t)over * rowq : 0u;
        const uint32_t dst = sb + (uint32_t)(wk_s * NQI + k) * 1024u;
        copy_to_lds(qg, coff[k] - back, dst);
        copy_to_lds(dg, coff[k] - back, dst + QTB);
      }
    }
    if (tid < kQW) {
      const int r = t0 + tid < NR ? t0 + tid : NR - 1;
      const idx_t lr0 = ((idx_t)b * p.Hq + hd) * NR;
      const float* lb = (st ? ls[1] : ls[0]) + lr0;
      const int* pl = st ? ps2[1] : ps2[0];
      copy_to_lds_b32(lb, (uint32_t)r * 4u, sb + 2 * QTB);
      copy_to_lds_b32((st ? dd[1] : dd[0]) + lr0, (uint32_t)r * 4u, sb + 2 * QTB + kQW * 4);
      if (pl)
        copy_to_lds_b32(pl, (uint32_t)r * 4u, sb + 2 * QTB + 2 * kQW * 4);
      else
        copy_to_lds_b32(lb, (uint32_t)r * 4u, sb + 2 * QTB + 2 * kQW * 4);
    }
  };

  // LDS offsets, derived inside the loop from two registers (the swizzle is an XOR):
  //   row read of channel slot 2 s + hh of row j:  rd0 ^ 32 s
  //   value block, key 32 wv + j:                   32 wv ROWB + (rd0 ^ 32 s)
  //   transposed read, channel tile dt:             tr0 ^ 64 dt, and 8 rows on:
  //                                                 ((tr0 ^ 64 dt) ^ kTrHi) + 8 ROWB
  const uint32_t rd0_init = slot_off<NCH>(j, hh);
  uint32_t tr_init[2][NDT];
  tr_offsets<D>(lane, tr_init);
  const uint32_t tr0_init = tr_init[0][0];
  constexpr uint32_t kTrHi = 32u;  // the swizzle bit that 8 rows flip
  const uint32_t vrow = (uint32_t)(32 * wv * ROWB);

  f32x16 dK[NDT], dV[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dK[dt][r] = 0.f;
      dV[dt][r] = 0.f;
    }
  f32x16 zero16;
#pragma unroll
  for (int r = 0; r < 16; ++r) zero16[r] = 0.f;

  if (nitems > 0) load_item(first, 0);
  wait_lds_copies();
  __syncthreads();
  Item cur = first;
  for (int i = 0; i < nitems; ++i) {
    const int slot = i & 1;
    const Item nxt = next_item(cur);
    if (i + 1 < nitems) load_item(nxt, slot ^ 1);
    const int st = cur.st;
    const int t0 = cur.qt * kQW;
    const int w = st ? wst[1] : wst[0];
    const int NR = st ? nr2[1] : nr2[0];
    const bool listed = (st ? ps2[1] : ps2[0]) != nullptr;
    const unsigned char* sq = smem + VBYTES + slot * STG;
    const float* rowf = reinterpret_cast<const float*>(sq + 2 * QTB);
    const int* rowp = reinterpret_cast<const int*>(rowf + 2 * kQW);
    // Position of tile row r, -1 past the last row: its own index, or its row-list entry
    // clamped into [0, T).
    auto row_pos = [&](int r, int raw) {
      int ps = listed ? raw : t0 + r;
      ps = ps < 0 ? 0 : (ps > T - 1 ? T - 1 : ps);
      return t0 + r < NR ? ps : -1;
    };
    // rows against keys k0w .. k0w+31: any pair with key <= t < key + w?
    bool need, fl;
    if (!listed) {
      need = t0 + kQW - 1 >= k0w && t0 <= k0w + 31 + w - 1 && k0w < T;
      fl = t0 >= k0w + 31 && t0 + kQW - 1 <= k0w + w - 1 && t0 + kQW - 1 < T && k0w + 31 < T;
    } else {
      bool any = false;  // this lane's 16 rows (both lane halves together cover the tile)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int4 p4 = *reinterpret_cast<const int4*>(rowp + 8 * q4 + 4 * hh);
        const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int t = row_pos(8 * q4 + 4 * hh + k, pv[k]);
          any = any || (t >= 0 && t >= k0w && t <= k0w + 31 + w - 1);
        }
      }
      need = __builtin_amdgcn_ballot_w64(any) != 0 && k0w < T;
      fl = false;
    }
    if (need) {
      const unsigned char* sd = sq + QTB;
      uint32_t rd0 = rd0_init, tr0 = tr0_init;
      asm volatile("" : "+v"(rd0), "+v"(tr0));  // derive the offsets here, not before the loop
      // Register r holds row i(r) = 8 (r / 4) + 4 hh + r % 4 of the tile, column key j. The
      // rows' -lse (log2 units) and -D seed the accumulators, so S and dP come out as s - lse
      // and dP - D.
      f32x16 S, dP;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(rowf + 8 * q4 + 4 * hh);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(rowf + kQW + 8 * q4 + 4 * hh);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          S[4 * q4 + k] = l4[k];
          dP[4 * q4 + k] = d4[k];
        }
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(sq + (rd0 ^ (32u * s)));
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[s], S, 0, 0, 0);
      }
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const bf16x8 da = *reinterpret_cast<const bf16x8*>(sd + (rd0 ^ (32u * s)));
        const bf16x8 vbv = *reinterpret_cast<const bf16x8*>(smem + vrow + (rd0 ^ (32u * s)));
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vbv, dP, 0, 0, 0);
      }
      if (!fl) {  // keys outside a row's window (or rows past the end) -> -inf
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          int4 p4 = {0, 0, 0, 0};
          if (listed) p4 = *reinterpret_cast<const int4*>(rowp + 8 * q4 + 4 * hh);
          const int pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int t = row_pos(8 * q4 + 4 * hh + k, pv[k]);  // -1 past the last row: masked
            const bool ok = key <= t && key > t - w && kvalid;
            S[4 * q4 + k] = ok ? S[4 * q4 + k] : kNegInf;
          }
        }
      }
      bf16x8 Pb[2], Zb[2];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = fast_exp2(S[r]);
        Pb[r >> 3][r & 7] = (__bf16)pr;
        Zb[r >> 3][r & 7] = (__bf16)(pr * dP[r]);
      }
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t tlo = tr0 ^ (64u * dt), thi = (tlo ^ kTrHi) + 8 * ROWB;
          const s16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sd + 16 * k2 * ROWB + tlo));
          const s16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sd + 16 * k2 * ROWB + thi));
          dV[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(dlo, dhi), Pb[k2], dV[dt], 0, 0, 0);
          const s16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sq + 16 * k2 * ROWB + tlo));
          const s16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sq + 16 * k2 * ROWB + thi));
          dK[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cat_tr(qlo, qhi), Zb[k2], dK[dt], 0, 0, 0);
        }
      }
    }
    wait_lds_copies();
    __syncthreads();
    cur = nxt;
  }

  if (kvalid) {
    const idx_t o = ((idx_t)b * T + key) * kst + (idx_t)g * D;
    uint16_t* dkr = static_cast<uint16_t*>(p.dk) + o;
    uint16_t* dvr = static_cast<uint16_t*>(p.dv) + o;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int c = 32 * dt + 8 * rg + 4 * hh;
        u32x2 a, v;
        a[0] = pack_bf16x2(dK[dt][4 * rg + 0] * kLn2, dK[dt][4 * rg + 1] * kLn2);
        a[1] = pack_bf16x2(dK[dt][4 * rg + 2] * kLn2, dK[dt][4 * rg + 3] * kLn2);
        v[0] = pack_bf16x2(dV[dt][4 * rg + 0], dV[dt][4 * rg + 1]);
        v[1] = pack_bf16x2(dV[dt][4 * rg + 2], dV[dt][4 * rg + 3]);
        *reinterpret_cast<u32x2*>(dkr + c) = a;
        *reinterpret_cast<u32x2*>(dvr + c) = v;
      }
  }
}

// ---- launchers -------------------------------------------------------------------------------
hipError_t launch_qprep(const void* q0, const void* q1, const float* a0, const float* b0,
                        const float* a1, const float* b1, void* o0, void* o1, idx_t n, int hd,
                        float c, hipStream_t s, int nstreams) {
  QPrepParams p{{q0, q1}, {a0, a1}, {b0, b1}, {o0, o1}, n, hd, c};
  idx_t blocks = n / hd;  // rows; each work-group walks rows blocks apart
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)blocks, (unsigned)nstreams), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_q_bf16(const BwdQParams& p, int d, hipStream_t s) {
  int hpw = 1;
  if (p.G % 8 == 0) hpw = 8;
  else if (p.G % 4 == 0) hpw = 4;
  else if (p.G % 2 == 0) hpw = 2;
  const int nw = hpw >= 4 ? 8 : 4;  // wavefronts per work-group
  const int bmp = kQW * (nw / hpw);
  const int npb = (p.nrows + bmp - 1) / bmp;  // row blocks, as the kernel derives them
  dim3 grid((unsigned)(p.B * p.Hkv * (p.G / hpw) * npb)), block(64 * nw);
#define ORTHROS_BWDQ(DD, HH) hipLaunchKernelGGL((bwd_q_kernel<DD, HH, (HH >= 4 ? 8 : 4)>), grid, block, 0, s, p)
  if (d == 128) {
    if (hpw == 8) ORTHROS_BWDQ(128, 8);
    else if (hpw == 4) ORTHROS_BWDQ(128, 4);
    else if (hpw == 2) ORTHROS_BWDQ(128, 2);
    else ORTHROS_BWDQ(128, 1);
  } else {
    if (hpw == 8) ORTHROS_BWDQ(64, 8);
    else if (hpw == 4) ORTHROS_BWDQ(64, 4);
    else if (hpw == 2) ORTHROS_BWDQ(64, 2);
    else ORTHROS_BWDQ(64, 1);
  }
#undef ORTHROS_BWDQ
  return hipGetLastError();
}

hipError_t launch_bwd_q_bf16_pair(const BwdQParams& p0, const BwdQParams& p1, int d, hipStream_t s) {
  int hpw = 1;
  if (p0.G % 8 == 0) hpw = 8;
  else if (p0.G % 4 == 0) hpw = 4;
  else if (p0.G % 2 == 0) hpw = 2;
  const int nw = hpw >= 4 ? 8 : 4;  // wavefronts per work-group
  const int bmp = kQW * (nw / hpw);
  const uint32_t n0 = (uint32_t)(p0.B * p0.Hkv * (p0.G / hpw) * ((p0.nrows + bmp - 1) / bmp));
  const uint32_t n1 = (uint32_t)(p1.B * p1.Hkv * (p1.G / hpw) * ((p1.nrows + bmp - 1) / bmp));
  dim3 grid(n0 + n1), block(64 * nw);
#define ORTHROS_BWDQ2(DD, HH) hipLaunchKernelGGL((bwd_q_pair_kernel<DD, HH, (HH >= 4 ? 8 : 4)>), grid, block, 0, s, p0, p1, n0)
  if (d == 128) {
    if (hpw == 8) ORTHROS_BWDQ2(128, 8);
    else if (hpw == 4) ORTHROS_BWDQ2(128, 4);
    else if (hpw == 2) ORTHROS_BWDQ2(128, 2);
    else ORTHROS_BWDQ2(128, 1);
  } else {
    if (hpw == 8) ORTHROS_BWDQ2(64, 8);
    else if (hpw == 4) ORTHROS_BWDQ2(64, 4);
    else if (hpw == 2) ORTHROS_BWDQ2(64, 2);
    else ORTHROS_BWDQ2(64, 1);
  }
#undef ORTHROS_BWDQ2
  return hipGetLastError();
}

hipError_t launch_bwd_kv_bf16(const BwdKVParams& p, int d, hipStream_t s) {
  const int nkb = (p.T + kKNW * 32 - 1) / (kKNW * 32);
  dim3 grid((unsigned)(p.B * p.Hkv * nkb)), block(64 * kKNW);
  if (d == 128)
    hipLaunchKernelGGL(bwd_kv_kernel<128>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(bwd_kv_kernel<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace orthros
