// K2: fused symmetric quantisation and C-BSG encoding.
//
// scmp_vit README, "Why it works": per-row bipolar quantisation with
// scale = row abs-max / 127.  K-band pull request, "How the banding works":
// with chunk_d set each contraction chunk carries its own scale.
// "Precision As You Need" paper notes, Key design 1: quantisation and the
// Sobol cumulative-table lookup are fused; the weight side's stream is the
// table row of its level, which every row of the other operand then indexes
// through its two C-BSG counters.
//
// Numerics (must match bit for bit on every input): float32 max of |x|,
// s = a / q and x / s as IEEE float32 divisions (no reciprocal), rint
// (round half to even), clamp to [-q, q]; a == 0 gives s = 0 and zeros.
// The level of an integer is u = (P (x + q) + q) / (2 q) (integer division).

#include <hip/hip_runtime.h>

#include <string>

#include "internal.h"
#include "table.h"

namespace scmp {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ int8_t quant_one(float x, float s, float qf) {
  if (s == 0.0f) return 0;
  float v = __builtin_rintf(x / s);
  v = fminf(fmaxf(v, -qf), qf);
  return (int8_t)(int)v;
}

struct QuantArgs {
  const float* X;
  long long bs, rs, cs;
  int rows, cols, chunk_d, n_chunks, q, P, Wl;
  int unipolar;  // packed streams at the magnitude level round(P |x| / q)
  int8_t* qout;
  float* scales;
  float* metric;
  uint32_t* packed;
  const uint32_t* K;
  int* flag;  // this stream's error flag word
};

// One block (256 threads, 4 waves) per (row, g).  Per-row scales: the whole
// block reduces the row.  Per-chunk scales: each wave takes whole chunks.
__global__ void __launch_bounds__(256) k_quantize(QuantArgs a) {
  const int row = blockIdx.x;
  const int g = blockIdx.y;
  const float* x = a.X + (long long)g * a.bs + (long long)row * a.rs;
  const long long orow = (long long)g * a.rows + row;
  int8_t* qrow = a.qout + orow * a.cols;
  const float qf = (float)a.q;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  __shared__ float red[4];
  bool bad = false;
  float rowmax = 0.0f;

  if (a.chunk_d <= 0) {
    float m = 0.0f;
    for (int c = threadIdx.x; c < a.cols; c += 256) {
      const float v = x[(long long)c * a.cs];
      bad |= !__builtin_isfinite(v);
      m = fmaxf(m, fabsf(v));
    }
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float s = amax == 0.0f ? 0.0f : amax / qf;
    for (int c = threadIdx.x; c < a.cols; c += 256) qrow[c] = quant_one(x[(long long)c * a.cs], s, qf);
    if (threadIdx.x == 0) a.scales[orow] = s;
    rowmax = amax;
  } else {
    float wmax = 0.0f;
    for (int ch = wave; ch < a.n_chunks; ch += 4) {
      const int c0 = ch * a.chunk_d;
      const int c1 = min(c0 + a.chunk_d, a.cols);
      float m = 0.0f;
      for (int c = c0 + lane; c < c1; c += 64) {
        const float v = x[(long long)c * a.cs];
        bad |= !__builtin_isfinite(v);
        m = fmaxf(m, fabsf(v));
      }
      m = wave_max(m);
      const float s = m == 0.0f ? 0.0f : m / qf;
      for (int c = c0 + lane; c < c1; c += 64) qrow[c] = quant_one(x[(long long)c * a.cs], s, qf);
      if (lane == 0) a.scales[orow * a.n_chunks + ch] = s;
      wmax = fmaxf(wmax, m);
    }
    if (lane == 0) red[wave] = wmax;
    __syncthreads();
    rowmax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  }
  if (a.metric && threadIdx.x == 0) a.metric[orow] = rowmax;
  if (bad) atomicOr(a.flag, 1);

  if (a.packed) {
    __syncthreads();  // the block's integers are visible to the block
    uint32_t* prow = a.packed + orow * (long long)a.cols * a.Wl;
    const int total = a.cols * a.Wl;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
      const int c = idx / a.Wl;
      const int w = idx - c * a.Wl;
      const int xi = qrow[c];
      const int u = a.unipolar ? (2 * a.P * abs(xi) + a.q) / (2 * a.q)   // round(P |x| / q)
                               : (a.P * (xi + a.q) + a.q) / (2 * a.q);  // round(P (x + q) / (2 q))
      prow[idx] = a.K[(long long)u * a.Wl + w];
    }
  }
}

// Fast path for unit column stride and 16-byte aligned rows: LPR lanes per
// row (a power of two; 64 / LPR rows per wave, four waves per block),
// float4 loads kept in registers between the max and the quantisation, four
// integers packed per 32-bit store.  Per-chunk scales need chunk_d a power of
// two in [4, 256]: the chunk of a float4 at column c is c / chunk_d, and the
// lanes sharing it are min(chunk_d / 4, LPR) consecutive lanes (an
// xor-shuffle group inside the row's lanes).  R: float4 loads per lane
// (cols <= 4 LPR R).
template <int R, int LPR>
__global__ void __launch_bounds__(256) k_quantize_vec(QuantArgs a) {
  constexpr int RPW = 64 / LPR;  // rows per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane & (LPR - 1);
  const int row = (blockIdx.x * 4 + wave) * RPW + lane / LPR;
  const int g = blockIdx.y;
  const bool live = row < a.rows;
  const float* x = a.X + (long long)g * a.bs + (long long)(live ? row : 0) * a.rs;
  const long long orow = (long long)g * a.rows + row;
  int8_t* qrow = a.qout + orow * a.cols;
  const float qf = (float)a.q;
  // Maximum over the LPR lanes of this row.
  auto row_max = [](float m) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    return m;
  };
  float4 v[R];
  bool bad = false;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = 4 * (LPR * r + sub);
    v[r] = (live && c < a.cols) ? *(const float4*)(x + c) : float4{0.0f, 0.0f, 0.0f, 0.0f};
    bad |= !(__builtin_isfinite(v[r].x) && __builtin_isfinite(v[r].y) && __builtin_isfinite(v[r].z) &&
             __builtin_isfinite(v[r].w));
  }
  auto amax4 = [](float4 t) { return fmaxf(fmaxf(fabsf(t.x), fabsf(t.y)), fmaxf(fabsf(t.z), fabsf(t.w))); };
  auto pack = [&](float4 t, float sc) {
    const uint32_t b0 = (uint8_t)quant_one(t.x, sc, qf), b1 = (uint8_t)quant_one(t.y, sc, qf);
    const uint32_t b2 = (uint8_t)quant_one(t.z, sc, qf), b3 = (uint8_t)quant_one(t.w, sc, qf);
    return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
  };
  float rowmax = 0.0f;
  if (a.chunk_d <= 0) {
    float m = 0.0f;
#pragma unroll
    for (int r = 0; r < R; ++r) m = fmaxf(m, amax4(v[r]));
    m = row_max(m);
    const float s = m == 0.0f ? 0.0f : m / qf;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int c = 4 * (LPR * r + sub);
      if (live && c < a.cols) *(uint32_t*)(qrow + c) = pack(v[r], s);
    }
    if (live && sub == 0) a.scales[orow] = s;
    rowmax = m;
  } else {
    const int group = min(a.chunk_d >> 2, LPR);  // lanes per chunk (power of two)
#pragma unroll
    for (int r = 0; r < R; ++r) {
      float m = amax4(v[r]);
      for (int off = 1; off < group; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      const float s = m == 0.0f ? 0.0f : m / qf;
      const int c = 4 * (LPR * r + sub);
      if (live && c < a.cols) {
        *(uint32_t*)(qrow + c) = pack(v[r], s);
        if ((sub & (group - 1)) == 0) a.scales[orow * a.n_chunks + c / a.chunk_d] = s;
      }
      rowmax = fmaxf(rowmax, m);
    }
    rowmax = row_max(rowmax);
  }
  if (a.metric && live && sub == 0) a.metric[orow] = rowmax;
  if (__ballot(bad) != 0 && lane == 0) atomicOr(a.flag, 1);
}

// Rows of any length up to 64 R with unit column stride but no alignment
// (attention rows of 257 values, say) and one scale per row: one wave per
// row, four rows per block, lane l holding columns l, l + 64, ... in
// registers between the max and the quantisation.
template <int R>
__global__ void __launch_bounds__(256) k_quantize_wave(QuantArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  const int g = blockIdx.y;
  if (row >= a.rows) return;
  const float* x = a.X + (long long)g * a.bs + (long long)row * a.rs;
  const long long orow = (long long)g * a.rows + row;
  int8_t* qrow = a.qout + orow * a.cols;
  const float qf = (float)a.q;
  float v[R];
  bool bad = false;
  float m = 0.0f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = 64 * r + lane;
    v[r] = c < a.cols ? x[c] : 0.0f;
    bad |= !__builtin_isfinite(v[r]);
    m = fmaxf(m, fabsf(v[r]));
  }
  m = wave_max(m);
  const float s = m == 0.0f ? 0.0f : m / qf;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int c = 64 * r + lane;
    if (c < a.cols) qrow[c] = quant_one(v[r], s, qf);
  }
  if (lane == 0) a.scales[orow] = s;
  if (a.metric && lane == 0) a.metric[orow] = m;
  if (__ballot(bad) != 0 && lane == 0) atomicOr(a.flag, 1);
}

}  // namespace scmp

using scmp::set_error;

extern "C" int scmp_quantize_encode(scmp_table_t table, scmp_plan_t plan, const float* X, int G, int rows,
                                    int cols, int64_t batch_stride, int64_t row_stride, int64_t col_stride,
                                    int8_t* q_out, float* scales_out, float* metric_out, uint32_t* packed_out,
                                    void* stream) {
  scmp::clear_error();
  if (!table || !plan) return set_error(SCMP_ERR_ARG, "table or plan is NULL");
  const scmp::Plan& P = plan->plan;
  if (table->p != P.p || table->Lmax != P.Lmax)
    return set_error(SCMP_ERR_PLAN_MISMATCH, "table p / Lmax differ from the plan");
  if (G < 0 || rows < 0 || cols < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if (cols != P.D) return set_error(SCMP_ERR_PLAN_MISMATCH, "cols differs from the plan's D");
  if ((long long)G * rows == 0) return SCMP_OK;
  if (!X || !q_out || !scales_out) return set_error(SCMP_ERR_ARG, "X, q_out and scales_out are required");
  if (G > 65535) return set_error(SCMP_ERR_ARG, "G must be <= 65535");
  scmp::QuantArgs a;
  a.X = X;
  a.bs = batch_stride;
  a.rs = row_stride;
  a.cs = col_stride;
  a.rows = rows;
  a.cols = cols;
  a.chunk_d = P.chunk_d;
  a.n_chunks = P.n_chunks;
  a.q = scmp::qmax(P.p);
  a.P = 1 << P.p;
  a.unipolar = P.mode == SCMP_MODE_UNIPOLAR;
  a.Wl = table->Wl;
  a.qout = q_out;
  a.scales = scales_out;
  a.metric = metric_out;
  a.packed = packed_out;
  a.K = table->K;
  hipStream_t st = (hipStream_t)stream;
  const int fs = scmp::stream_flag(st, &a.flag);
  if (fs != SCMP_OK) return fs;
  // Fast path: unit column stride, 16-byte aligned rows, no packed streams,
  // cols a multiple of 4 up to 4096, chunk_d 0 or a power of two in [4, 256].
  const bool cd_ok = P.chunk_d <= 0 || (P.chunk_d >= 4 && P.chunk_d <= 256 && (P.chunk_d & (P.chunk_d - 1)) == 0);
  const bool vec = col_stride == 1 && !packed_out && cols % 4 == 0 && cols <= 4096 && cd_ok &&
                   ((uintptr_t)X % 16) == 0 && row_stride % 4 == 0 && batch_stride % 4 == 0 &&
                   ((uintptr_t)q_out % 4) == 0;
  // Wave path: unit column stride, one scale per row, no packed streams,
  // rows up to 1024 values, any alignment.
  const bool wave = !vec && col_stride == 1 && !packed_out && P.chunk_d <= 0 && cols <= 1024;
  if (wave) {
    const dim3 grid((rows + 3) / 4, G);
    const int R = (cols + 63) / 64;
    if (R <= 4)
      hipLaunchKernelGGL(scmp::k_quantize_wave<4>, grid, dim3(256), 0, st, a);
    else if (R <= 8)
      hipLaunchKernelGGL(scmp::k_quantize_wave<8>, grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(scmp::k_quantize_wave<16>, grid, dim3(256), 0, st, a);
  } else if (vec) {
    // Lanes per row: the float4 count of a row rounded up to a power of two
    // (4 to 64); rows of more than 256 values take 64 lanes and R loads.
    int lpr = 4;
    while (lpr < 64 && 4 * lpr < cols) lpr <<= 1;
    const int rows_per_block = 4 * (64 / lpr);
    const dim3 grid((rows + rows_per_block - 1) / rows_per_block, G);
    const int R = (cols + 4 * lpr - 1) / (4 * lpr);
    if (lpr == 4)
      hipLaunchKernelGGL((scmp::k_quantize_vec<1, 4>), grid, dim3(256), 0, st, a);
    else if (lpr == 8)
      hipLaunchKernelGGL((scmp::k_quantize_vec<1, 8>), grid, dim3(256), 0, st, a);
    else if (lpr == 16)
      hipLaunchKernelGGL((scmp::k_quantize_vec<1, 16>), grid, dim3(256), 0, st, a);
    else if (lpr == 32)
      hipLaunchKernelGGL((scmp::k_quantize_vec<1, 32>), grid, dim3(256), 0, st, a);
    else if (R <= 1)
      hipLaunchKernelGGL((scmp::k_quantize_vec<1, 64>), grid, dim3(256), 0, st, a);
    else if (R <= 4)
      hipLaunchKernelGGL((scmp::k_quantize_vec<4, 64>), grid, dim3(256), 0, st, a);
    else if (R <= 8)
      hipLaunchKernelGGL((scmp::k_quantize_vec<8, 64>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((scmp::k_quantize_vec<16, 64>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(scmp::k_quantize, dim3(rows, G), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("quantize launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}
