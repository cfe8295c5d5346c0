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
  const idx_t total = p.in_place ? 0 : (idx_t)p.B * p.T * p.Hkv * cpr;
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

// One block per sequence: append row len[b] (if there is room), then advance len[b]. With a
// paged pool the row goes to its page's slot; a bad page index leaves it unwritten.
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
  __shared__ int bad_page;
  const int b = blockIdx.x;
  const int32_t L = p.len[b];
  const int cpr = p.d * p.esize / 16;
  const bool room = L >= 0 && L < p.cap;
  idx_t base = 0;  // element offset of row L within kv head 0
  bool bad = false;
  if (room) {
    if (p.pg.table) {
      base = paged_offset(p.pg, p.pg.table + (idx_t)b * p.pg.tbl_sb, L, p.cap, p.d, &bad);
    } else {
      base = (idx_t)b * p.Hkv * p.cap * p.d + (idx_t)L * p.d;
    }
  }
  const idx_t hstride = p.pg.table ? p.pg.k_sh : p.cap * p.d;  // between kv heads
  if (room && !bad) {
    const u32x4* ks = reinterpret_cast<const u32x4*>(p.knew);
    const u32x4* vs = reinterpret_cast<const u32x4*>(p.vnew);
    u32x4* kd = reinterpret_cast<u32x4*>(p.ck);
    u32x4* vd = reinterpret_cast<u32x4*>(p.cv);
    for (int i = threadIdx.x; i < p.Hkv * cpr; i += blockDim.x) {
      const int g = i / cpr, c = i % cpr;
      const idx_t src = ((idx_t)b * p.Hkv + g) * cpr + c;
      const idx_t dst = (base + (idx_t)g * hstride) * p.esize / 16 + c;
      kd[dst] = ks[src];
      vd[dst] = vs[src];
    }
  }
  if (threadIdx.x == 0) bad_page = bad;
  __syncthreads();  // every thread has read len[b] before it changes
  if (threadIdx.x == 0) {
    if (room) {
      if (!bad_page) p.len[b] = L + 1;
    } else {
      __hip_atomic_fetch_or(p.status, kStatusCacheFull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Paged bulk write, one 16-byte chunk per thread-iteration, source order [b][t][g][c]. Reads
// len[b] (unchanged by this kernel); paged_advance_kernel updates it afterwards.
__global__ __launch_bounds__(256) void paged_write_kernel(PagedWriteParams p) {
  const int cpr = p.d * p.esize / 16;
  const idx_t total = (idx_t)p.B * p.T * p.Hkv * cpr;
  const idx_t stride = (idx_t)gridDim.x * blockDim.x;
  const u32x4* ksrc = reinterpret_cast<const u32x4*>(p.k);
  const u32x4* vsrc = reinterpret_cast<const u32x4*>(p.v);
  u32x4* kdst = reinterpret_cast<u32x4*>(p.ck);
  u32x4* vdst = reinterpret_cast<u32x4*>(p.cv);
  for (idx_t i = (idx_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const idx_t c = i % cpr;
    idx_t r = i / cpr;
    const idx_t g = r % p.Hkv;
    r /= p.Hkv;
    const idx_t t = r % p.T;
    const idx_t b = r / p.T;
    const int64_t L = p.len[b];
    if (L < 0 || L + p.T > p.cap) continue;  // no room: the sequence is left unchanged
    bool bad = false;
    const idx_t off = paged_offset(p.pg, p.pg.table + b * p.pg.tbl_sb, L + t, p.cap, p.d, &bad);
    if (bad) continue;
    const idx_t dst = (off + g * p.pg.k_sh) * p.esize / 16 + c;
    kdst[dst] = __builtin_nontemporal_load(ksrc + i);
    vdst[dst] = __builtin_nontemporal_load(vsrc + i);
  }
}

// One block per sequence: len[b] += T if the write had room and every table entry it went
// through was a valid page (the write kernel skipped rows of a bad entry, so a length that
// counted them would make later steps read rows that were never written).
__global__ __launch_bounds__(256) void paged_advance_kernel(PagedWriteParams p) {
  __shared__ int any_bad;
  const int b = blockIdx.x;
  const int64_t L = p.len[b];
  const bool room = L >= 0 && L + p.T <= p.cap;
  if (threadIdx.x == 0) any_bad = 0;
  __syncthreads();
  if (room) {
    const int32_t* tbl = p.pg.table + (idx_t)b * p.pg.tbl_sb;
    const int64_t first = L >> p.pg.ps_log2, last = (L + p.T - 1) >> p.pg.ps_log2;
    bool bad = false;
    for (int64_t i = first + threadIdx.x; i <= last; i += blockDim.x) {
      const int32_t page = tbl[i];
      bad = bad || page < 0 || (int64_t)page >= p.pg.num_pages;
    }
    if (bad) any_bad = 1;  // (the write kernel has set the status bit)
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (!room) {
      __hip_atomic_fetch_or(p.pg.status, kStatusCacheFull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (!any_bad) {
      p.len[b] = (int32_t)(L + p.T);
    }
  }
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t s) {
  const idx_t total = p.in_place ? 0 : (idx_t)p.B * p.T * p.Hkv * (p.d * p.esize / 16);
  idx_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(cache_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_paged_write(const PagedWriteParams& p, hipStream_t s) {
  const idx_t total = (idx_t)p.B * p.T * p.Hkv * (p.d * p.esize / 16);
  idx_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(paged_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(paged_advance_kernel, dim3((unsigned)p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_append(const AppendParams& p, hipStream_t s) {
  hipLaunchKernelGGL(append_kernel, dim3(p.B), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace orthros
