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

struct ClassifyArgs {
  const float* metric;
  float* ghat;
  uint8_t* rung;
  int32_t* perm;
  float* thr;
  int* flag;  // this stream's error flag word
  int M, n_rungs;
  int cuts[SCMP_MAX_RUNGS + 1];
};

// Ranking key: the normalised metric, with NaN below every number.
__device__ __forceinline__ float rank_key(float v) { return v == v ? v : -1.0f; }

constexpr int CL_ROWS = 64;     // rows ranked per block
constexpr int CL_WAVES = 8;     // waves per block, each scans 1/8 of every key tile
constexpr int CL_TILE = 8192;   // keys staged in LDS at a time

// One block ranks 64 rows of one group.  Every block first reduces the
// group's largest metric itself (so no separate pass is needed), then
// stages tiles of normalised keys g_j / max in LDS; the 8 waves each count,
// for their 64 rows, the keys that sort before the row:
//   rank_i = #{j < i : key_j >= key_i} + #{j > i : key_j > key_i},
// i.e. descending key, ties by row index.  The keys form a strict total
// order, so the ranks are a permutation; perm[rank_i] = i and the rung
// follows from the cuts.
__global__ void __launch_bounds__(512) k_classify(ClassifyArgs a) {
  __shared__ float keys[CL_TILE];
  __shared__ float red[CL_WAVES];
  __shared__ int part[CL_WAVES][CL_ROWS];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* m = a.metric + (long long)g * a.M;

  float mx = 0.0f;
  bool bad = false;
  for (int j = tid; j < a.M; j += 512) {
    const float v = m[j];
    bad |= !__builtin_isfinite(v);
    mx = fmaxf(mx, v);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < CL_WAVES; ++w) mx = fmaxf(mx, red[w]);
  if (bad && blockIdx.x == 0) atomicOr(a.flag, 1);

  const int i = blockIdx.x * CL_ROWS + lane;
  const float gi = i < a.M ? (mx == 0.0f ? 0.0f : m[i] / mx) : 0.0f;
  const float ki = rank_key(gi);
  int rank = 0;
  for (int t0 = 0; t0 < a.M; t0 += CL_TILE) {
    const int n = min(CL_TILE, a.M - t0);
    __syncthreads();
    for (int j = tid; j < n; j += 512) keys[j] = rank_key(mx == 0.0f ? 0.0f : m[t0 + j] / mx);
    __syncthreads();
    const int per = (n + CL_WAVES - 1) / CL_WAVES;
    const int j0 = wave * per, j1 = min(n, j0 + per);
    // Keys before row i count when >=, keys after it when >, the row itself
    // never: [j0, lo_end) with >=, [hi_start, j1) with >.
    const int li = i - t0;
    const int lo_end = min(max(li, j0), j1);
    const int hi_start = min(max(li + 1, j0), j1);
#pragma unroll 8
    for (int j = j0; j < lo_end; ++j) rank += keys[j] >= ki;
#pragma unroll 8
    for (int j = hi_start; j < j1; ++j) rank += keys[j] > ki;
  }
  part[wave][lane] = rank;
  __syncthreads();
  if (wave == 0 && i < a.M) {
    rank = 0;
#pragma unroll
    for (int w = 0; w < CL_WAVES; ++w) rank += part[w][lane];
    a.ghat[(long long)g * a.M + i] = gi;
    a.perm[(long long)g * a.M + rank] = i;
    int k = 0;
    while (k + 1 < a.n_rungs && rank >= a.cuts[k + 1]) ++k;
    if (a.rung) a.rung[(long long)g * a.M + i] = (uint8_t)k;
    if (a.thr) {
      for (int kk = 1; kk < a.n_rungs; ++kk) {
        if (rank == a.cuts[kk] - 1) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = gi;
        if (a.cuts[kk] == 0 && i == 0) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = 1.0f;
      }
    }
  }
}

// Groups of at most CS_MAXM rows (attention heads of 257 queries): each
// block stages the whole group's keys in LDS and ranks CS_ROWS of its rows
// (the same rank as above), eight lanes per row, lane s of a row comparing
// the keys j = s (mod 8); the eight partial counts meet in a butterfly.  A
// wave's eight rows read the same eight consecutive keys at once, so the
// reads broadcast without bank conflicts.  The work per group is M^2
// comparisons, spread over ceil(M / CS_ROWS) blocks, against the bucket
// form's 2048-bucket clear and scan repeated by each of its blocks.
constexpr int CS_MAXM = 512;
constexpr int CS_ROWS = 64;  // rows ranked per block (512 threads, 8 per row)

__global__ void __launch_bounds__(CS_MAXM) k_classify_small(ClassifyArgs a) {
  __shared__ float s_key[CS_MAXM];
  __shared__ float s_g[CS_MAXM];
  __shared__ float s_red[CS_MAXM / 64];
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int M = a.M;
  const float* m = a.metric + (long long)g * M;
  const bool live = tid < M;
  const float v = live ? m[tid] : 0.0f;
  float mx = live ? fmaxf(0.0f, v) : 0.0f;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_red[wave] = mx;
  const bool bad = live && !__builtin_isfinite(v);
  if (blockIdx.x == 0 && __ballot(bad) && lane == 0) atomicOr(a.flag, 1);
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < CS_MAXM / 64; ++w) mx = fmaxf(mx, s_red[w]);
  if (live) {
    const float gj = mx == 0.0f ? 0.0f : v / mx;
    s_g[tid] = gj;
    s_key[tid] = rank_key(gj);
  }
  __syncthreads();
  // rank_i = #{j : key_j > key_i, or key_j == key_i and j < i}.  Every lane
  // takes part in the butterfly; rows past M read a key and drop the count.
  const int i = blockIdx.x * CS_ROWS + (tid >> 3), s = tid & 7;
  const bool row_live = i < M;
  const float ki = row_live ? s_key[i] : 0.0f;
  int rank = 0;
  for (int j = s; j < M; j += 8) {
    const float kj = s_key[j];
    rank += (kj > ki) || (kj == ki && j < i);
  }
  rank += __shfl_xor(rank, 1, 64);
  rank += __shfl_xor(rank, 2, 64);
  rank += __shfl_xor(rank, 4, 64);
  if (!row_live || s != 0) return;
  const float gi = s_g[i];
  a.ghat[(long long)g * M + i] = gi;
  a.perm[(long long)g * M + rank] = i;
  int k = 0;
  while (k + 1 < a.n_rungs && rank >= a.cuts[k + 1]) ++k;
  if (a.rung) a.rung[(long long)g * M + i] = (uint8_t)k;
  if (a.thr) {
    for (int kk = 1; kk < a.n_rungs; ++kk) {
      if (rank == a.cuts[kk] - 1) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = gi;
      if (a.cuts[kk] == 0 && i == 0) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = 1.0f;
    }
  }
}

// Groups of at most CB_MAXM rows take a bucket form with O(M) work per
// block instead of O(M^2): every block buckets all of its group's keys by
// value in LDS (a monotone map, so every key of a higher bucket sorts
// before every key of a lower one), scans the bucket counts from the top
// and lists each bucket's rows; a row's rank is then the count of rows in
// higher buckets plus the rows of its own bucket that sort before it.
// Equal keys share a bucket, so ties (row index order) are decided by the
// same direct comparison as above; with every key equal the members are
// the whole group and the block does M comparisons per row, spread over
// its eight waves.  A block ranks CL_ROWS x sets rows; the metric is read
// once, into registers, with all of a thread's loads in flight together.
constexpr int CB_MAXM = 18432;
constexpr int CB_PER = CB_MAXM / 512;  // metric values per thread
constexpr int CB_NB = 2048;            // buckets: 0 for negative (and NaN) keys, 1..2047 over [0, 1]

__device__ __forceinline__ int key_bucket(float k) {
  return k < 0.0f ? 0 : min(CB_NB - 1, 1 + (int)(k * (float)(CB_NB - 2)));
}

// Dynamic LDS: s_cnt, s_start [CB_NB] ints, s_key [M] floats, s_mem [M]
// u16 (bytes: 8 CB_NB + 6 M, rounded).
size_t classify_bucket_lds(int M) { return (size_t)8 * CB_NB + (size_t)4 * M + (size_t)2 * ((M + 1) & ~1); }

__global__ void __launch_bounds__(512) k_classify_bucket(ClassifyArgs a, int sets) {
  extern __shared__ __align__(16) unsigned char s_dyn[];
  __shared__ int s_part[CL_WAVES][CL_ROWS];
  __shared__ float s_red[CL_WAVES];
  __shared__ int s_wsum[CL_WAVES];
  const int M = a.M;
  int* const s_cnt = (int*)s_dyn;                       // rows per bucket, then fill counters
  int* const s_start = s_cnt + CB_NB;                   // first list position of each bucket
  float* const s_key = (float*)(s_start + CB_NB);       // rank key of each row
  uint16_t* const s_mem = (uint16_t*)(s_key + M);       // rows listed bucket by bucket, top first
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* m = a.metric + (long long)g * M;

  float v[CB_PER];
  float mx = 0.0f;
  bool bad = false;
#pragma unroll
  for (int u = 0; u < CB_PER; ++u) {
    const int j = tid + 512 * u;
    v[u] = j < M ? m[j] : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < CB_PER; ++u)
    if (tid + 512 * u < M) {
      bad |= !__builtin_isfinite(v[u]);
      mx = fmaxf(mx, v[u]);
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) s_red[wave] = mx;
  for (int b = tid; b < CB_NB; b += 512) s_cnt[b] = 0;
  __syncthreads();
  mx = s_red[0];
#pragma unroll
  for (int w = 1; w < CL_WAVES; ++w) mx = fmaxf(mx, s_red[w]);
  if (bad && blockIdx.x == 0) atomicOr(a.flag, 1);

#pragma unroll
  for (int u = 0; u < CB_PER; ++u) {
    const int j = tid + 512 * u;
    if (j < M) {
      const float k = rank_key(mx == 0.0f ? 0.0f : v[u] / mx);
      s_key[j] = k;
      atomicAdd(&s_cnt[key_bucket(k)], 1);
    }
  }
  __syncthreads();
  // Exclusive scan from the top bucket down: thread t takes buckets
  // 2047 - 4 t - [0, 4).
  {
    int c[4], sum = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = s_cnt[CB_NB - 1 - (4 * tid + q)];
      sum += c[q];
    }
    int incl = sum;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int t = __shfl_up(incl, off, 64);
      if (lane >= off) incl += t;
    }
    if (lane == 63) s_wsum[wave] = incl;
    __syncthreads();
    int run = incl - sum;
    for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      s_start[CB_NB - 1 - (4 * tid + q)] = run;
      run += c[q];
    }
  }
  __syncthreads();
  for (int b = tid; b < CB_NB; b += 512) s_cnt[b] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < CB_PER; ++u) {
    const int j = tid + 512 * u;
    if (j < M) {
      const int b = key_bucket(s_key[j]);
      s_mem[s_start[b] + atomicAdd(&s_cnt[b], 1)] = (uint16_t)j;
    }
  }
  __syncthreads();

  // Ranks of the block's rows: every wave scans an eighth of each row's
  // bucket (the bucket's rows w, w + 8, ...).
  for (int set = 0; set < sets; ++set) {
    const int i = (blockIdx.x * sets + set) * CL_ROWS + lane;
    int n = 0;
    float ki = 0.0f;
    int bi = 0;
    if (i < M) {
      ki = s_key[i];
      bi = key_bucket(ki);
      const int e = s_start[bi] + s_cnt[bi];
      for (int q = s_start[bi] + wave; q < e; q += CL_WAVES) {
        const int j = s_mem[q];
        const float kj = s_key[j];
        n += (kj > ki) || (kj == ki && j < i);
      }
    }
    s_part[wave][lane] = n;
    __syncthreads();
    if (wave == 0 && i < M) {
      int rank = s_start[bi];
#pragma unroll
      for (int w = 0; w < CL_WAVES; ++w) rank += s_part[w][lane];
      const float gi = mx == 0.0f ? 0.0f : m[i] / mx;
      a.ghat[(long long)g * M + i] = gi;
      a.perm[(long long)g * M + rank] = i;
      int k = 0;
      while (k + 1 < a.n_rungs && rank >= a.cuts[k + 1]) ++k;
      if (a.rung) a.rung[(long long)g * M + i] = (uint8_t)k;
      if (a.thr) {
        for (int kk = 1; kk < a.n_rungs; ++kk) {
          if (rank == a.cuts[kk] - 1) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = gi;
          if (a.cuts[kk] == 0 && i == 0) a.thr[(long long)g * (a.n_rungs - 1) + kk - 1] = 1.0f;
        }
      }
    }
    __syncthreads();  // s_part is rewritten by the next set
  }
}

// Largest value of each group: the per-head metric |Q_h|.amax as the
// maximum of the head's row metrics ([VIT] mixed-precision flag table,
// per-head fixed MP on QK).  One block per group.
__global__ void __launch_bounds__(256) k_group_max(const float* in, int M, float* out) {
  __shared__ float red[4];
  const int g = blockIdx.x, tid = threadIdx.x;
  const float* x = in + (long long)g * M;
  float m = -__builtin_inff();
  for (int j = tid; j < M; j += 256) m = fmaxf(m, x[j]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) out[g] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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
  const int fs = scmp::stream_flag(st, &a.flag);
  if (fs != SCMP_OK) return fs;
  const int tiles = (M + scmp::CL_ROWS - 1) / scmp::CL_ROWS;
  if (M <= scmp::CS_MAXM) {
    hipLaunchKernelGGL(scmp::k_classify_small, dim3((M + scmp::CS_ROWS - 1) / scmp::CS_ROWS, G), dim3(scmp::CS_MAXM), 0,
                       st, a);
  } else if (M <= scmp::CB_MAXM) {
    // Large groups rank two sets of rows per block: every block repeats the
    // group's O(M) bucketing, so fewer, fuller blocks cost less.
    const int sets = M > 8192 ? 2 : 1;
    const size_t lds = scmp::classify_bucket_lds(M);
    hipError_t e = hipFuncSetAttribute((const void*)scmp::k_classify_bucket,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("classify LDS: ") + hipGetErrorString(e));
    hipLaunchKernelGGL(scmp::k_classify_bucket, dim3((tiles + sets - 1) / sets, G), dim3(512), lds, st, a, sets);
  } else {
    hipLaunchKernelGGL(scmp::k_classify, dim3(tiles, G), dim3(512), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("classify launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}

extern "C" int scmp_group_max(const float* in_dev, int G, int M, float* out_dev, void* stream) {
  scmp::clear_error();
  if (G < 0 || M < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if (G == 0) return SCMP_OK;
  if (M == 0) return set_error(SCMP_ERR_ARG, "a group needs at least one value");
  if (!in_dev || !out_dev) return set_error(SCMP_ERR_ARG, "in and out are required");
  hipLaunchKernelGGL(scmp::k_group_max, dim3(G), dim3(256), 0, (hipStream_t)stream, in_dev, M, out_dev);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("group max launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}
