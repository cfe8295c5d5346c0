// fp32 attention rows ("Orthros: Phase-Aware Heterogeneous Attention for Efficient
// Transformers", §3.1 Eq. 4 for base rows with a finite window, Eq. 5 for output rows with an
// unbounded one). Used for every fp32 call: bf16 matrix-core operands cannot meet fp32
// accuracy, so fp32 runs on the vector ALUs, one wavefront per (row, query head, sequence),
// channels spread over the 64 lanes and keys visited in order with an online softmax.
#include "common.h"
#include "launch.h"

namespace orthros {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void rows_f32_kernel(RowsF32Params p) {
  constexpr int E = D / 64;  // channels per lane
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
  float q[E], o[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane + 64 * e;
    q[e] = (p.alpha[h * D + c] * qr[c] + p.beta[h * D + c]) * p.scale;
    o[e] = 0.f;
  }
  const int64_t lo = t - (int64_t)p.window + 1 > 0 ? t - (int64_t)p.window + 1 : 0;
  float m = kNegInf, l = 0.f;
  // Cached rows: contiguous [B, Hkv, cap, d], or kv head g of the sequence's pages.
  const int32_t* tbl = p.pg.table ? p.pg.table + (idx_t)b * p.pg.tbl_sb : nullptr;
  const idx_t head_off = tbl ? (idx_t)g * p.pg.k_sh : (idx_t)b * p.k_sb + (idx_t)g * p.k_sh;
  const float* kb = p.k + head_off;
  const float* vb = p.v + head_off;
  for (int64_t j = lo; j <= t; ++j) {
    const float* kr;
    const float* vr;
    if (j == Lnew) {
      kr = p.knew + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh;
      vr = p.vnew + (idx_t)b * p.kn_sb + (idx_t)g * p.kn_sh;
    } else {
      const idx_t off = tbl ? paged_offset(p.pg, tbl, j, p.cap, p.k_st) : j * p.k_st;
      kr = kb + off;
      vr = vb + off;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) s += q[e] * kr[lane + 64 * e];
    s = wave_sum(s);
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn);  // m = -inf on the first key gives 0
    const float pj = expf(s - mn);
    l = l * a + pj;
#pragma unroll
    for (int e = 0; e < E; ++e) o[e] = o[e] * a + pj * vr[lane + 64 * e];
    m = mn;
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
