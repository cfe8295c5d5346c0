// fp32 attention rows ("Orthros: Phase-Aware Heterogeneous Attention for Efficient
// Transformers", §3.1 Eq. 4 for base rows with a finite window, Eq. 5 for output rows with an
// unbounded one). Used for every fp32 call: bf16 matrix-core operands cannot meet fp32
// accuracy, so fp32 runs on the vector ALUs, one wavefront per (row, query head, sequence).
#include "common.h"
#include "launch.h"

namespace orthros {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

// One wavefront per (row, query head, sequence). Keys are visited in blocks of 64: lane i
// scores key j0 + i against the whole query (every lane holds all D query values), the block's
// maximum and sum come from two wavefront reductions, and the value rows are then accumulated
// key by key with the output's channels spread over the lanes (each key's probability is read
// from the lane that scored it). An online softmax carries (m, l, o) across blocks.
template <int D>
__global__ __launch_bounds__(64) void rows_f32_kernel(RowsF32Params p) {
  constexpr int E = D / 64;  // output channels per lane
  const int row = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / p.G;
  int64_t t;
  int64_t Lnew = -1;  // decode: index of this step's key (taken from knew/vnew)
  if (p.len) {
    const int64_t L = p.len[b];
    Lnew = L < 0 ? 0 : (L > p.cap ? p.cap : L);  // clamped: no read leaves the cache
    t = Lnew;
  } else if (p.pos) {
    const int64_t pr = p.pos[row];
    t = pr < 0 ? 0 : (pr > p.nkeys - 1 ? p.nkeys - 1 : pr);  // no read leaves k / v
  } else {
    t = (int64_t)p.t0 + row;
  }
  const float* qr = p.q + (idx_t)b * p.q_sb + (idx_t)row * p.q_st + (idx_t)h * p.q_sh;
  const float* al = p.alpha + (idx_t)h * D;
  const float* be = p.beta + (idx_t)h * D;
  float qa[D];  // the scale-offset query (§3.1), times the score scale, in every lane
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qr + c);
    const f32x4 a = *reinterpret_cast<const f32x4*>(al + c);
    const f32x4 bb = *reinterpret_cast<const f32x4*>(be + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) qa[c + i] = (a[i] * x[i] + bb[i]) * p.scale;
  }
  const int64_t lo = t - (int64_t)p.window + 1 > 0 ? t - (int64_t)p.window + 1 : 0;
  // Cached rows: contiguous [B, Hkv, cap, d], or kv head g of the sequence's pages.
  const int32_t* tbl = p.pg.table ? p.pg.table + (idx_t)b * p.pg.tbl_sb : nullptr;
  const idx_t head_off = tbl ? (idx_t)g * p.pg.k_sh : (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;
  const float* kb = p.k + head_off;
  const float* vb = p.v + head_off;
  const float* knew = p.knew ? p.knew + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh : nullptr;
  const float* vnew = p.vnew ? p.vnew + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh : nullptr;
  // Element offset of key j's row from kb / vb (the new key has none: -1).
  auto row_off = [&](int64_t j) -> idx_t {
    if (j == Lnew) return -1;
    return tbl ? paged_offset(p.pg, tbl, j, p.cap, p.k_st) : j * p.k_st;
  };
  float o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) o[e] = 0.f;
  float m = kNegInf, l = 0.f;
  for (int64_t j0 = lo; j0 <= t; j0 += 64) {
    const int64_t j = j0 + lane;
    const bool valid = j <= t;
    const idx_t off = row_off(valid ? j : t);
    const float* kr = off < 0 ? knew : kb + off;
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(kr + c);
      s += qa[c] * k4[0] + qa[c + 1] * k4[1] + qa[c + 2] * k4[2] + qa[c + 3] * k4[3];
    }
    s = valid ? s : kNegInf;
    const float mn = fmaxf(m, wave_max(s));
    const float a = expf(m - mn);  // m = -inf before the first block gives 0
    const float pj = valid ? expf(s - mn) : 0.f;
    l = l * a + wave_sum(pj);
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] *= a;
    m = mn;
    const int nb = t - j0 + 1 < 64 ? (int)(t - j0 + 1) : 64;
    const uint32_t offlo = (uint32_t)off, offhi = (uint32_t)((uint64_t)off >> 32);
    // i is the same in every lane: read lane i's probability and row offset; CH keys' value
    // loads are issued before their products (keys past the block's end weigh 0)
    constexpr int CH = D == 64 ? 32 : 16;
    for (int i0 = 0; i0 < nb; i0 += CH) {
      float pu[CH], vu[CH][E];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        const int i = i0 + u < nb ? i0 + u : nb - 1;
        pu[u] = i0 + u < nb ? __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(pj), i)) : 0.f;
        const idx_t oi = (idx_t)(((uint64_t)__builtin_amdgcn_readlane(offhi, i) << 32) |
                                 __builtin_amdgcn_readlane(offlo, i));
        const float* vr = oi < 0 ? vnew : vb + oi;
#pragma unroll
        for (int e = 0; e < E; ++e) vu[u][e] = vr[lane + 64 * e];
      }
#pragma unroll
      for (int u = 0; u < CH; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) o[e] += pu[u] * vu[u][e];
    }
  }
  float* orow = p.o + (idx_t)b * p.o_sb + (idx_t)row * p.o_st + (idx_t)h * p.o_sh;
  const float inv = 1.f / l;
  if (p.lse && lane == 0) p.lse[(idx_t)b * p.lse_sb + (idx_t)h * p.lse_sh + row] = m + logf(l);
#pragma unroll
  for (int e = 0; e < E; ++e) orow[lane + 64 * e] = o[e] * inv;
}

hipError_t launch_rows_f32(const RowsF32Params& p, hipStream_t s) {
  dim3 grid(p.nrows, p.Hq, p.B);
  if (p.d == 128)
    hipLaunchKernelGGL(rows_f32_kernel<128>, grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(rows_f32_kernel<64>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

}  // namespace orthros
