// Training backward on the vector ALUs, and the scale-offset gradient reduction.
//
// Gradients of "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers",
// §3.2 Pre-Training regime (every position has a base row, Eq. 4, and an output row, Eq. 5)
// with respect to the raw queries, the shared keys and values, and the learnable scale-offset
// vectors of §3.1. For one row t with post-affine query q (scores z_j = s q . k_j over its keys,
// weights P_j = exp(z_j - lse_t), output O = sum_j P_j v_j and output gradient dO):
//   D_t = dO . O;  dP_j = dO . v_j;  dZ_j = P_j (dP_j - D_t)
//   dq = s sum_j dZ_j k_j;  dk_j += s dZ_j q;  dv_j += P_j dO
// and through q = alpha (.) q_raw + beta: dq_raw = alpha (.) dq, d alpha = sum dq (.) q_raw,
// d beta = sum dq. fp32 calls use these kernels (one wavefront per row, or per key for dk and
// dv); the bf16 path has matrix-core kernels and shares the reduction.
#include "common.h"
#include "launch.h"
#include "launch_bwd.h"

namespace orthros {

namespace {
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}
}  // namespace

// One wavefront per (row, query head h, sequence b) of one stream: D_t and the post-affine
// query gradient (which includes the score scale s). The row sits at position pos[row] with a
// row list, else at position row.
template <int DIM>
__global__ __launch_bounds__(64) void bwd_q_f32_kernel(BwdQParams p) {
  constexpr int E = DIM / 64;
  const int r = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const int g = h / p.G;
  int t = p.pos ? p.pos[r] : r;
  t = t < 0 ? 0 : (t > p.T - 1 ? p.T - 1 : t);
  const idx_t row = ((idx_t)b * p.nrows + r) * p.Hq + h;  // [B, nrows, Hq] row of q / o / dq
  const float* qr = static_cast<const float*>(p.q) + row * DIM;
  const float* orow = static_cast<const float*>(p.o) + row * DIM;
  const float* dor = static_cast<const float*>(p.dout) + row * DIM;
  float q[E], dO[E], dq[E];
  float dsum = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int c = lane + 64 * e;
    q[e] = (p.alpha[h * DIM + c] * qr[c] + p.beta[h * DIM + c]) * p.scale;
    dO[e] = dor[c];
    dsum += dO[e] * orow[c];
    dq[e] = 0.f;
  }
  const float Dt = wave_sum64(dsum);
  const idx_t lrow = ((idx_t)b * p.Hq + h) * p.nrows + r;
  if (lane == 0) p.D[lrow] = Dt;
  const float lse = p.lse[lrow];
  const int w = p.window < p.T ? p.window : p.T;
  const int lo = t - w + 1 > 0 ? t - w + 1 : 0;
  const idx_t kst = (idx_t)p.Hkv * DIM;
  const float* kb = static_cast<const float*>(p.k) + (idx_t)b * p.T * kst + (idx_t)g * DIM;
  const float* vb = static_cast<const float*>(p.v) + (idx_t)b * p.T * kst + (idx_t)g * DIM;
  for (int j = lo; j <= t; ++j) {
    const float* kj = kb + j * kst;
    const float* vj = vb + j * kst;
    float zs = 0.f, ps = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      zs += q[e] * kj[lane + 64 * e];
      ps += dO[e] * vj[lane + 64 * e];
    }
    const float z = wave_sum64(zs);
    const float dp = wave_sum64(ps);
    const float dz = expf(z - lse) * (dp - Dt);
#pragma unroll
    for (int e = 0; e < E; ++e) dq[e] += dz * kj[lane + 64 * e];
  }
  float* out = p.dq + row * DIM;
#pragma unroll
  for (int e = 0; e < E; ++e) out[lane + 64 * e] = dq[e] * p.scale;
}

// One wavefront per (key j, kv head g, sequence b): dk_j and dv_j over both streams' rows that
// see key j (positions j .. j + w - 1 with the stream's window w) of every query head of the
// group. A stream with a row list visits every listed row and keeps those at such positions.
template <int DIM>
__global__ __launch_bounds__(64) void bwd_kv_f32_kernel(BwdKVParams p) {
  constexpr int E = DIM / 64;
  const int j = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const idx_t kst = (idx_t)p.Hkv * DIM;
  const idx_t krow = ((idx_t)b * p.T + j) * kst + (idx_t)g * DIM;
  const float* kj = static_cast<const float*>(p.k) + krow;
  const float* vj = static_cast<const float*>(p.v) + krow;
  float k[E], v[E], dk[E], dv[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = kj[lane + 64 * e];
    v[e] = vj[lane + 64 * e];
    dk[e] = 0.f;
    dv[e] = 0.f;
  }
  for (int st = 0; st < 2; ++st) {
    const int w = p.window[st] < p.T ? p.window[st] : p.T;  // window >= T: causal
    const int hi = j + w - 1 < p.T - 1 ? j + w - 1 : p.T - 1;
    const int NR = p.nrows[st];
    const int32_t* pos = p.pos[st];
    for (int hg = 0; hg < p.G; ++hg) {
      const int h = g * p.G + hg;
      float a[E], bb[E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        a[e] = p.alpha[st][h * DIM + lane + 64 * e] * p.scale;
        bb[e] = p.beta[st][h * DIM + lane + 64 * e] * p.scale;
      }
      const float* lse = p.lse[st] + ((idx_t)b * p.Hq + h) * NR;
      const float* Dr = p.D[st] + ((idx_t)b * p.Hq + h) * NR;
      const int r_lo = pos ? 0 : j, r_hi = pos ? NR - 1 : hi;
      for (int t = r_lo; t <= r_hi; ++t) {  // t: row index (the position without a list)
        if (pos) {
          int ps = pos[t];
          ps = ps < 0 ? 0 : (ps > p.T - 1 ? p.T - 1 : ps);
          if (ps < j || ps > hi) continue;
        }
        const idx_t row = ((idx_t)b * NR + t) * p.Hq + h;
        const float* qr = static_cast<const float*>(p.q[st]) + row * DIM;
        const float* dor = static_cast<const float*>(p.dout[st]) + row * DIM;
        float q[E], dO[E];
        float zs = 0.f, ps = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          q[e] = a[e] * qr[lane + 64 * e] + bb[e];  // s (alpha q_raw + beta)
          dO[e] = dor[lane + 64 * e];
          zs += q[e] * k[e];
          ps += dO[e] * v[e];
        }
        const float z = wave_sum64(zs);
        const float dp = wave_sum64(ps);
        const float pr = expf(z - lse[t]);
        const float dz = pr * (dp - Dr[t]);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          dv[e] += pr * dO[e];
          dk[e] += dz * q[e];
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    static_cast<float*>(p.dk)[krow + lane + 64 * e] = dk[e];
    static_cast<float*>(p.dv)[krow + lane + 64 * e] = dv[e];
  }
}

// dq_raw = alpha (.) dq for every row, and per chunk of rows the partial sums of dq (.) q_raw
// and dq per column; then the partials are added in chunk order. Each thread owns 4 adjacent
// columns (16-byte loads) and keeps several rows' loads in flight.
__global__ __launch_bounds__(256) void affine_grad_partial_kernel(AffineGradParams p) {
  const int c = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (c >= p.n) return;
  const int r0 = blockIdx.x * p.chunk_rows;
  const int r1 = r0 + p.chunk_rows < p.rows ? r0 + p.chunk_rows : p.rows;
  const f32x4 a = *reinterpret_cast<const f32x4*>(p.alpha + c);
  const float* __restrict__ dq = p.dq;  // dq and q are read once: non-temporal loads
  f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int r = r0; r < r1; ++r) {
    const idx_t i = (idx_t)r * p.n + c;
    const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(dq + i));
    f32x4 qr;
    if (p.bf16) {
      const u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(p.q) + i));
      qr = f32x4{bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1])};
      u32x2 o;
      o[0] = pack_bf16x2(a[0] * x[0], a[1] * x[1]);
      o[1] = pack_bf16x2(a[2] * x[2], a[3] * x[3]);
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.dq_raw) + i) = o;
    } else {
      qr = *reinterpret_cast<const f32x4*>(static_cast<const float*>(p.q) + i);
      *reinterpret_cast<f32x4*>(static_cast<float*>(p.dq_raw) + i) = a * x;
    }
    sa += x * qr;
    sb += x;
  }
  *reinterpret_cast<f32x4*>(p.part + ((idx_t)blockIdx.x * 2 + 0) * p.n + c) = sa;
  *reinterpret_cast<f32x4*>(p.part + ((idx_t)blockIdx.x * 2 + 1) * p.n + c) = sb;
}

// Sum of the chunk partials, per column: 16 slices of 16 threads each add every 16th chunk
// (loads unrolled so several are in flight), then the slices combine in a fixed order.
// One launch serves one or two streams (blockIdx.y picks the parameter set).
struct AffineGradPair {
  AffineGradParams s[2];
};

__device__ __forceinline__ void affine_grad_final_body(const AffineGradParams& p) {
  __shared__ float red[2][16][16];
  const int cl = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int c = blockIdx.x * 16 + cl;
  float sa = 0.f, sb = 0.f;
  if (c < p.n) {
#pragma unroll 8
    for (int k = sl; k < p.nchunk; k += 16) {
      sa += p.part[((idx_t)k * 2 + 0) * p.n + c];
      sb += p.part[((idx_t)k * 2 + 1) * p.n + c];
    }
  }
  red[0][sl][cl] = sa;
  red[1][sl][cl] = sb;
  __syncthreads();
  if (sl == 0 && c < p.n) {
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      a += red[0][k][cl];
      b += red[1][k][cl];
    }
    p.dalpha[c] = a;
    p.dbeta[c] = b;
  }
}

__global__ __launch_bounds__(256) void affine_grad_final_kernel(AffineGradPair pp) {
  if (blockIdx.y == 0) affine_grad_final_body(pp.s[0]);
  else affine_grad_final_body(pp.s[1]);
}

hipError_t launch_bwd_q_f32(const BwdQParams& p, int d, hipStream_t s) {
  dim3 grid(p.nrows, p.Hq, p.B);
  if (d == 128)
    hipLaunchKernelGGL(bwd_q_f32_kernel<128>, grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_q_f32_kernel<64>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_bwd_kv_f32(const BwdKVParams& p, int d, hipStream_t s) {
  dim3 grid(p.T, p.Hkv, p.B);
  if (d == 128)
    hipLaunchKernelGGL(bwd_kv_f32_kernel<128>, grid, dim3(64), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_kv_f32_kernel<64>, grid, dim3(64), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_affine_grad_final(const AffineGradParams* p, int count, hipStream_t s) {
  if (count < 1 || count > 2 || (count == 2 && p[1].n != p[0].n)) return hipErrorInvalidValue;
  AffineGradPair pp{{p[0], p[count > 1 ? 1 : 0]}};
  hipLaunchKernelGGL(affine_grad_final_kernel, dim3((unsigned)((p[0].n + 15) / 16), (unsigned)count), dim3(256), 0, s, pp);
  return hipGetLastError();
}

hipError_t launch_affine_grad(const AffineGradParams& p, hipStream_t s) {
  const unsigned cb4 = (unsigned)((p.n / 4 + 255) / 256);
  hipLaunchKernelGGL(affine_grad_partial_kernel, dim3((unsigned)p.nchunk, cb4), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  AffineGradPair pp{{p, p}};
  hipLaunchKernelGGL(affine_grad_final_kernel, dim3((unsigned)((p.n + 15) / 16), 1u), dim3(256), 0, s, pp);
  return hipGetLastError();
}

}  // namespace orthros
