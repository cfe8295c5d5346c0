// Cache maintenance kernels: the base stream's keys/values go into the full, never-evicted
// layer cache ("Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers",
// §3.1: keys and values come from base tokens only; §3.2: prefilling writes the prompt, each
// decode step's base copy appends its token). The output stream never writes here.
#include "common.h"
#include "launch.h"

namespace orthros {

// One 16-byte chunk per thread-iteration; rows are d*esize bytes (a multiple of 16).
__global__ __launch_bounds__(256) void cache_write_kernel(CacheWriteParams p) {
  const int cpr = p.d * p.esize / 16;  // chunks per row
  const idx_t total = (idx_t)p.B * p.T * p.Hkv * cpr;
  const idx_t stride = (idx_t)gridDim.x * blockDim.x;
  const u32x4* ksrc = reinterpret_cast<const u32x4*>(p.k);
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(p.v);
  u32x4* kdst = reinterpret_cast<u32x4*>(p.ck);
  u32x4* vdst = reinterpret_cast<u32x4*>(p.cv);
  for (idx_t i = (idx_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    // source order [b][t][g][c] (contiguous)
    const idx_t c = i % cpr;
    idx_t r = i / cpr;
    const idx_t g = r % p.Hkv;
    r /= p.Hkv;
    const idx_t t = r % p.T;
    const idx_t b = r / p.T;
    const idx_t dst = ((b * p.Hkv + g) * p.cap + p.t_first + t) * cpr + c;
    kdst[dst] = __builtin_nontemporal_load(ksrc + i);
    vdst[dst] = __builtin_nontemporal_load(vsrc + i);
  }
  if (blockIdx.x == 0) {
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) p.len[b] = (int32_t)(p.t_first + p.T);
  }
}

// One block per sequence: append row len[b] (if there is room), then advance len[b].
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  const int b = blockIdx.x;
  const int32_t L = p.len[b];
  const int cpr = p.d * p.esize / 16;
  if (L >= 0 && L < p.cap) {
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.knew);
    const u32x4* vs = reinterpret_cast<const u32x4*>(p.vnew);
    u32x4* kd = reinterpret_cast<u32x4*>(p.ck);
    u32x4* vd = reinterpret_cast<u32x4*>(p.cv);
    for (int i = threadIdx.x; i < p.Hkv * cpr; i += blockDim.x) {
      const int g = i / cpr, c = i % cpr;
      const idx_t src = ((idx_t)b * p.Hkv + g) * cpr + c;
      const idx_t dst = (((idx_t)b * p.Hkv + g) * p.cap + L) * cpr + c;
      kd[dst] = ks[src];
      vd[dst] = vs[src];
    }
  }
  __syncthreads();  // every thread has read len[b] before it changes
  if (threadIdx.x == 0) {
    if (L >= 0 && L < p.cap) {
      p.len[b] = L + 1;
    } else {
      __hip_atomic_fetch_or(p.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  const idx_t total = (idx_t)p.B * p.T * p.Hkv * (p.d * p.esize / 16);
  idx_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace orthros
