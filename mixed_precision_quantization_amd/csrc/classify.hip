// K4: row classification for dynamic mixed precision.
//
// "Precision As You Need" paper notes, Key design 2: the row metric
// (||X_i||_inf, or max_j A_ij for attention rows) is normalised to [0, 1]
// and a descending threshold ladder picks each row's stream length.
// Thresholds are taken as the empirical quantiles of the input: rows are
// ranked by normalised metric (descending, ties by row index) and rung k
// takes the sorted positions [cut_k, cut_(k+1)).  The sorted order is also
// the bucket permutation: every rung is one contiguous run of positions, so
// the matmul sees uniform-length row tiles (Key design 3's early
// termination without divergence inside a tile).

#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"

namespace scmp {

__device__ int g_classify_flags;

struct ClassifyArgs {
  const float* metric;
  float* ghat;
  uint8_t* rung;
  int32_t* perm;
  float* thr;
  int M, n_rungs;
  int cuts[SCMP_MAX_RUNGS + 1];
};

// Ranking key: the normalised metric, with NaN below every number.
__device__ __forceinline__ float rank_key(float v) { return v == v ? v : -1.0f; }

// One block per group: max of the metric, g_hat = g / max.
__global__ void __launch_bounds__(256) k_normalise(ClassifyArgs a) {
  const int g = blockIdx.x;
  const float* m = a.metric + (long long)g * a.M;
  __shared__ float red[4];
  float mx = 0.0f;
  bool bad = false;
  for (int i = threadIdx.x; i < a.M; i += 256) {
    const float v = m[i];
    bad |= !__builtin_isfinite(v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float* gh = a.ghat + (long long)g * a.M;
  for (int i = threadIdx.x; i < a.M; i += 256) gh[i] = mx == 0.0f ? 0.0f : m[i] / mx;
  if (a.thr && threadIdx.x < a.n_rungs - 1) a.thr[(long long)g * (a.n_rungs - 1) + threadIdx.x] = 1.0f;
  if (bad) atomicOr(&g_classify_flags, 1);
}

// 64 rows per block, 4 threads per row each scanning a quarter of every
// tile of keys staged in LDS.  rank_i = #{j : key_j > key_i} +
// #{j < i : key_j == key_i}; then perm[rank_i] = i and the rung from the
// cuts.  The keys form a strict total order, so ranks are a permutation.
__global__ void __launch_bounds__(256) k_rank(ClassifyArgs a) {
  constexpr int TILE = 4096;
  __shared__ float keys[TILE];
  __shared__ int part[4][64];
  const int g = blockIdx.y;
  const float* gh = a.ghat + (long long)g * a.M;
  const int r = threadIdx.x & 63;
  const int qt = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + r;
  const float ki = i < a.M ? rank_key(gh[i]) : 0.0f;
  int rank = 0;
  for (int t0 = 0; t0 < a.M; t0 += TILE) {
    const int n = min(TILE, a.M - t0);
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += 256) keys[j] = rank_key(gh[t0 + j]);
    __syncthreads();
    const int per = (n + 3) / 4;
    const int j0 = qt * per;
    const int j1 = min(n, j0 + per);
    for (int j = j0; j < j1; ++j) {
      const float kj = keys[j];
      rank += (kj > ki) || (kj == ki && (t0 + j) < i);
    }
  }
  part[qt][r] = rank;
  __syncthreads();
  if (qt == 0 && i < a.M) {
    rank = part[0][r] + part[1][r] + part[2][r] + part[3][r];
    a.perm[(long long)g * a.M + rank] = i;
    int k = 0;
    while (k + 1 < a.n_rungs && rank >= a.cuts[k + 1]) ++k;
    if (a.rung) a.rung[(long long)g * a.M + i] = (uint8_t)k;
    if (a.thr) {
      for (int kk = 1; kk < a.n_rungs; ++kk)
        if (rank == a.cuts[kk] - 1) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = gh[i];
    }
  }
}

int read_clear_classify_flags(hipStream_t st, int* flags) {
  int v = 0, zero = 0;
  hipError_t e =
      hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_classify_flags), sizeof(int), 0, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess)
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_classify_flags), &zero, sizeof(int), 0, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("flag readback: ") + hipGetErrorString(e));
  *flags |= v;
  return SCMP_OK;
}

}  // namespace scmp

using scmp::set_error;

extern "C" int scmp_classify_rows(scmp_plan_t plan, const float* metric, int G, int M, float* ghat,
                                  uint8_t* rung, int32_t* perm, float* thresholds, void* stream) {
  scmp::clear_error();
  if (!plan) return set_error(SCMP_ERR_ARG, "plan is NULL");
  if (G < 0 || M < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if ((long long)G * M == 0) return SCMP_OK;
  if (!metric || !ghat || !perm) return set_error(SCMP_ERR_ARG, "metric, ghat and perm are required");
  if (G > 65535) return set_error(SCMP_ERR_ARG, "G must be <= 65535");
  const scmp::Plan& P = plan->plan;
  scmp::ClassifyArgs a;
  a.metric = metric;
  a.ghat = ghat;
  a.rung = rung;
  a.perm = perm;
  a.thr = thresholds;
  a.M = M;
  a.n_rungs = P.n_rungs;
  scmp::row_cuts(P, M, a.cuts);
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(scmp::k_normalise, dim3(G), dim3(256), 0, st, a);
  hipLaunchKernelGGL(scmp::k_rank, dim3((M + 63) / 64, G), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("classify launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}
