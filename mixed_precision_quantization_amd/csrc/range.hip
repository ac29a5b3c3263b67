// Range-based per-weight-group mixed precision: the weight side's
// classification and the row gather that stores W in level order.
//
// scmp_vit README, the mixed-precision flag table: range MP, its two
// stream-length levels and the normalised range threshold (a higher
// threshold puts more groups at low precision).  K-band pull request,
// "Guards": range MP has no contraction-axis dispatch, so a weight group is
// a set of whole W rows (output columns).  The contraction itself is
// scmp_matmul_range (matmul.hip), once per level.

#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"

namespace scmp {

__device__ int g_range_counts[2];

// Range (max - min) of each group of `gs` consecutive W rows over all D
// columns.  One block per group.
__global__ void __launch_bounds__(256) k_range_group(const float* W, int N, int D, long long rs, int gs,
                                                     float* rng) {
  __shared__ float smx[4], smn[4];
  const int grp = blockIdx.x, tid = threadIdx.x;
  const int r0 = grp * gs, r1 = min(N, r0 + gs);
  const long long n = (long long)(r1 - r0) * D;
  float mx = -__builtin_inff(), mn = __builtin_inff();
  for (long long e = tid; e < n; e += 256) {
    const int r = r0 + (int)(e / D), c = (int)(e % D);
    const float v = W[(long long)r * rs + c];
    mx = fmaxf(mx, v);
    mn = fminf(mn, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    mn = fminf(mn, __shfl_xor(mn, off, 64));
  }
  if ((tid & 63) == 0) {
    smx[tid >> 6] = mx;
    smn[tid >> 6] = mn;
  }
  __syncthreads();
  if (tid == 0) {
    const float a = fmaxf(fmaxf(smx[0], smx[1]), fmaxf(smx[2], smx[3]));
    const float b = fminf(fminf(smn[0], smn[1]), fminf(smn[2], smn[3]));
    rng[grp] = a - b;
  }
}

// Inclusive block scan of v over 1024 threads (LDS, Hillis-Steele).
__device__ int block_scan_1024(int v, int* s) {
  const int tid = threadIdx.x;
  s[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? s[tid - off] : 0;
    __syncthreads();
    s[tid] += add;
    __syncthreads();
  }
  const int r = s[tid];
  __syncthreads();
  return r;
}

// Normalise the ranges by the largest, pick each group's level, and write
// the W rows of level 0 in order, then those of level 1.  One block of 1024.
__global__ void __launch_bounds__(1024) k_range_finish(float* norm, int n_groups, int N, int gs, float thr,
                                                       uint8_t* level, int32_t* cols) {
  __shared__ float red[16];
  __shared__ int s_scan[1024];
  __shared__ int s_tot[2];
  const int tid = threadIdx.x;
  float top = 0.0f;
  for (int g = tid; g < n_groups; g += 1024) top = fmaxf(top, norm[g]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) top = fmaxf(top, __shfl_xor(top, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = top;
  __syncthreads();
  top = red[0];
  for (int w = 1; w < 16; ++w) top = fmaxf(top, red[w]);
  __syncthreads();
  // Level-0 rows in total (the base of level 1), then positions.
  int low_rows = 0;
  for (int g = tid; g < n_groups; g += 1024) {
    const float x = top > 0.0f ? norm[g] / top : 0.0f;
    if (x < thr) low_rows += min(N, (g + 1) * gs) - g * gs;
  }
  const int low_total = block_scan_1024(low_rows, s_scan);
  if (tid == 1023) s_tot[0] = low_total;
  __syncthreads();
  const int base1 = N - s_tot[0];
  int run0 = 0, run1 = base1;
  for (int c0 = 0; c0 < n_groups; c0 += 1024) {
    const int g = c0 + tid;
    int lev = 0, size = 0;
    float x = 0.0f;
    if (g < n_groups) {
      x = top > 0.0f ? norm[g] / top : 0.0f;
      lev = x < thr ? 1 : 0;
      size = min(N, (g + 1) * gs) - g * gs;
    }
    const int inc0 = block_scan_1024(lev == 0 ? size : 0, s_scan);
    const int inc1 = block_scan_1024(lev == 1 ? size : 0, s_scan);
    if (g < n_groups) {
      const int pos = lev == 0 ? run0 + inc0 - size : run1 + inc1 - size;
      for (int i = 0; i < size; ++i) cols[pos + i] = g * gs + i;
      if (level) level[g] = (uint8_t)lev;
    }
    if (tid == 1023) {
      s_tot[0] = inc0;
      s_tot[1] = inc1;
    }
    __syncthreads();
    run0 += s_tot[0];
    run1 += s_tot[1];
    __syncthreads();
  }
  // Every block-wide read of norm is done: overwrite with the normalised values.
  for (int g = tid; g < n_groups; g += 1024) norm[g] = top > 0.0f ? norm[g] / top : 0.0f;
  if (tid == 0) {
    g_range_counts[0] = base1;
    g_range_counts[1] = N - base1;
  }
}

// dst[g][i] = src[g][idx[i]] (rows of `bytes` bytes; zero rows for indices
// outside [0, n_src)).  One block per (i, g).
__global__ void __launch_bounds__(256) k_gather_rows(const uint8_t* src, int n_src, long long bytes,
                                                     const int32_t* idx, int n_idx, uint8_t* dst, int words) {
  const int i = blockIdx.x, g = blockIdx.y;
  const int r = idx[i];
  const bool ok = r >= 0 && r < n_src;
  uint8_t* d = dst + ((long long)g * n_idx + i) * bytes;
  const uint8_t* s = src + ((long long)g * n_src + (ok ? r : 0)) * bytes;
  if (words) {
    for (long long e = threadIdx.x; e < bytes / 4; e += 256)
      ((uint32_t*)d)[e] = ok ? ((const uint32_t*)s)[e] : 0u;
  } else {
    for (long long e = threadIdx.x; e < bytes; e += 256) d[e] = ok ? s[e] : (uint8_t)0;
  }
}

}  // namespace scmp

using scmp::set_error;

extern "C" int scmp_range_classify(scmp_plan_t plan, const float* W, int N, int D, int64_t rs, float* norm,
                                   uint8_t* level, int32_t* cols, int* n_per_level, void* stream) {
  scmp::clear_error();
  if (!plan) return set_error(SCMP_ERR_ARG, "plan is NULL");
  const scmp::Plan& P = plan->plan;
  if (!P.range_mp) return set_error(SCMP_ERR_ARG, "the plan has no range-based MP");
  if (N < 1 || D < 1) return set_error(SCMP_ERR_ARG, "N and D must be >= 1");
  if (D != P.D) return set_error(SCMP_ERR_PLAN_MISMATCH, "D differs from the plan");
  if (rs < D) return set_error(SCMP_ERR_ARG, "w_row_stride must be >= D");
  if (!W || !norm || !cols || !n_per_level) return set_error(SCMP_ERR_ARG, "W, norm, cols and n_per_level are required");
  const int gs = P.range_group;
  const int n_groups = (N + gs - 1) / gs;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(scmp::k_range_group, dim3(n_groups), dim3(256), 0, st, W, N, D, (long long)rs, gs, norm);
  hipLaunchKernelGGL(scmp::k_range_finish, dim3(1), dim3(1024), 0, st, norm, n_groups, N, gs, P.range_threshold,
                     level, cols);
  hipError_t e = hipGetLastError();
  int counts[2] = {0, 0};
  if (e == hipSuccess)
    e = hipMemcpyFromSymbolAsync(counts, HIP_SYMBOL(scmp::g_range_counts), sizeof counts, 0,
                                 hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("range classification: ") + hipGetErrorString(e));
  n_per_level[0] = counts[0];
  n_per_level[1] = counts[1];
  return SCMP_OK;
}

extern "C" int scmp_gather_rows(const void* src, int G, int n_src, size_t row_bytes, const int32_t* idx,
                                int n_idx, void* dst, void* stream) {
  scmp::clear_error();
  if (G < 0 || n_src < 0 || n_idx < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if ((long long)G * n_idx * (long long)row_bytes == 0) return SCMP_OK;
  if (G > 65535) return set_error(SCMP_ERR_ARG, "G must be <= 65535");
  if (!src || !idx || !dst) return set_error(SCMP_ERR_ARG, "src, idx and dst are required");
  const bool words = row_bytes % 4 == 0 && ((uintptr_t)src & 3) == 0 && ((uintptr_t)dst & 3) == 0;
  hipLaunchKernelGGL(scmp::k_gather_rows, dim3(n_idx, G), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)src,
                     n_src, (long long)row_bytes, idx, n_idx, (uint8_t*)dst, words ? 1 : 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("gather launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}
