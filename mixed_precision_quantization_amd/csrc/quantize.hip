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

__device__ int g_quant_flags;

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
  int8_t* qout;
  float* scales;
  float* metric;
  uint32_t* packed;
  const uint32_t* K;
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
  if (bad) atomicOr(&g_quant_flags, 1);

  if (a.packed) {
    __syncthreads();  // the block's integers are visible to the block
    uint32_t* prow = a.packed + orow * (long long)a.cols * a.Wl;
    const int total = a.cols * a.Wl;
    for (int idx = threadIdx.x; idx < total; idx += 256) {
      const int c = idx / a.Wl;
      const int w = idx - c * a.Wl;
      const int xi = qrow[c];
      const int u = (a.P * (xi + a.q) + a.q) / (2 * a.q);
      prow[idx] = a.K[(long long)u * a.Wl + w];
    }
  }
}

int read_clear_quant_flags(hipStream_t st, int* flags) {
  int v = 0, zero = 0;
  hipError_t e = hipMemcpyFromSymbolAsync(&v, HIP_SYMBOL(g_quant_flags), sizeof(int), 0, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e == hipSuccess)
    e = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_quant_flags), &zero, sizeof(int), 0, hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("flag readback: ") + hipGetErrorString(e));
  *flags |= v;
  return SCMP_OK;
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
  a.Wl = table->Wl;
  a.qout = q_out;
  a.scales = scales_out;
  a.metric = metric_out;
  a.packed = packed_out;
  a.K = table->K;
  hipLaunchKernelGGL(scmp::k_quantize, dim3(rows, G), dim3(256), 0, (hipStream_t)stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("quantize launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}
