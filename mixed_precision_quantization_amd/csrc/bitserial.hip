// Vector-ALU bit-serial XNOR contraction.
//
// "Precision As You Need" paper notes, Key design 1: A's stream for index d
// is the L-prefix of its table row (n1 ones, n0 zeros) and B's stream is
// produced by two counters gated by A's bits (C-BSG).  Position c of the
// counter domain contributes B_c where A emitted its c-th one (c < n1) and
// NOT B_c where A emitted its c-th zero (c < n0), so per 32-position word
//   XNOR count = popcount(bitselect(B_w, T1_w, T0_w))
// with T1 / T0 the prefix masks of n1 / n0 ones: one bit-select and one
// accumulating popcount per word.  B_w are the packed counter-domain
// streams written by scmp_quantize_encode.  K-band pull request, "How the
// banding works": band b uses L[b][k]; the chunk decode is fused.
//
// Unipolar plans (AND gate, "Precision As You Need" Key design 3; levels of
// the magnitudes) count popcount(B_w & T1_w) per word, so per index the
// count is cum[u_B][n1], taken with the product of the operands' signs;
// their decode is s^A s^B q^2 count / L.

#include <hip/hip_runtime.h>

#include <string>

#include "matmul_common.h"

namespace scmp {

constexpr int BS_BM = 64, BS_BN = 64, BS_DC = 8, BS_WMAX = 8;

// Prefix mask word: bits [0, n) of the stream restricted to word w.
__device__ __forceinline__ uint32_t prefix_word(int n, int w) {
  const int m = n - 32 * w;
  return m <= 0 ? 0u : (m >= 32 ? 0xffffffffu : ((1u << m) - 1u));
}

template <bool COUNTS, bool UNI>
__global__ void __launch_bounds__(256) k_matmul_bitserial(MatmulArgs a) {
  __shared__ __align__(16) uint2 s_t[BS_DC][BS_WMAX][BS_BM];      // (T1, T0) words
  __shared__ __align__(16) uint32_t s_b[BS_DC][BS_WMAX][BS_BN];   // B stream words
  __shared__ __align__(16) int s_sga[UNI ? BS_DC : 1][BS_BM];     // unipolar: -1 where x_A < 0, else 0
  __shared__ __align__(16) int s_sgb[UNI ? BS_DC : 1][BS_BN];     // unipolar: -1 where x_B < 0, else 0
  __shared__ uint16_t s_ncum[MAX_LEVELS];
  __shared__ int s_rows[BS_BM];

  const int tid = threadIdx.x;
  const int g = blockIdx.z;
  int k, pos0, nrows;
  locate_tile(a, blockIdx.y, BS_BM, k, pos0, nrows);
  k = tile_rung(a, g, k);
  const int col0 = blockIdx.x * BS_BN;
  if (tid < BS_BM) s_rows[tid] = tid < nrows ? row_of(a, g, pos0 + tid) : -1;
  const int ty = tid >> 4, tx = tid & 15;
  const int qq = a.q * a.q;

  int cnt[4][4];
  float cacc[4][4];
  int bacc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cnt[i][j] = 0;
      cacc[i][j] = 0.0f;
      bacc[i][j] = 0;
    }

  for (int b = 0; b < a.n_bands; ++b) {
    const int L = a.bandL[b][k];
    const int W = (L + 31) >> 5;
    const float scaleL = (float)qq / (float)L;
    const int dbeg = a.band_cols[b], dend = a.band_cols[b + 1];
    __syncthreads();
    for (int u = tid; u <= a.P; u += 256) s_ncum[u] = a.cum[(long long)u * (a.Lmax + 1) + L];
    for (int d0 = dbeg; d0 < dend; d0 += BS_DC) {
      const int cend = chunk_end(a, d0);
      const int dlim = min(d0 + BS_DC, dend);
      __syncthreads();
      {
        // A masks: thread -> (row r, two d's).
        const int r = tid >> 2, dp = (tid & 3) * 2;
        const int row = s_rows[r];
        const int8_t* src = a.qA + ((long long)g * a.M + (row < 0 ? 0 : row)) * a.D;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int dd = dp + i, d = d0 + dd;
          int n1 = 0, n0 = 0;
          if (UNI) {
            const int x = (row >= 0 && d < dlim) ? (int)src[d] : 0;
            n1 = s_ncum[uni_level_of(x, a.P, a.q)];
            s_sga[UNI ? dd : 0][r] = x < 0 ? -1 : 0;
          } else if (row >= 0 && d < dlim) {
            n1 = s_ncum[level_of((int)src[d], a.P, a.q)];
            n0 = L - n1;
          }
          for (int w = 0; w < W; ++w) s_t[dd][w][r] = make_uint2(prefix_word(n1, w), prefix_word(n0, w));
        }
        // B words: thread -> (col c, two d's).
        const int c = tid >> 2, col = col0 + c;
        const uint32_t* bsrc = a.packedB + ((long long)g * a.N + (col < a.N ? col : 0)) * a.D * a.Wl;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int dd = dp + i, d = d0 + dd;
          for (int w = 0; w < W; ++w) s_b[dd][w][c] = (col < a.N && d < dlim) ? bsrc[(long long)d * a.Wl + w] : 0u;
          if (UNI)
            s_sgb[UNI ? dd : 0][c] = (col < a.N && d < dlim && a.qB[((long long)g * a.N + col) * a.D + d] < 0) ? -1 : 0;
        }
      }
      __syncthreads();
      for (int dd = 0; dd < BS_DC && UNI; ++dd) {
        int t[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) t[i][j] = 0;
        for (int w = 0; w < W; ++w) {
          const uint4 t01 = *(const uint4*)&s_t[dd][w][ty * 4];
          const uint4 t23 = *(const uint4*)&s_t[dd][w][ty * 4 + 2];
          const uint4 bw = *(const uint4*)&s_b[dd][w][tx * 4];
          const uint32_t T1[4] = {t01.x, t01.z, t23.x, t23.z};
          const uint32_t B[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) t[i][j] += __popc(B[j] & T1[i]);
        }
        const int4 ma = *(const int4*)&s_sga[UNI ? dd : 0][ty * 4];
        const int4 mb = *(const int4*)&s_sgb[UNI ? dd : 0][tx * 4];
        const int MA[4] = {ma.x, ma.y, ma.z, ma.w};
        const int MB[4] = {mb.x, mb.y, mb.z, mb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int m = MA[i] ^ MB[j];  // -1 where the signs differ
            cnt[i][j] += (t[i][j] ^ m) - m;
          }
      }
      for (int dd = 0; dd < BS_DC && !UNI; ++dd) {
        for (int w = 0; w < W; ++w) {
          const uint4 t01 = *(const uint4*)&s_t[dd][w][ty * 4];
          const uint4 t23 = *(const uint4*)&s_t[dd][w][ty * 4 + 2];
          const uint4 bw = *(const uint4*)&s_b[dd][w][tx * 4];
          const uint32_t T1[4] = {t01.x, t01.z, t23.x, t23.z};
          const uint32_t T0[4] = {t01.y, t01.w, t23.y, t23.w};
          const uint32_t B[4] = {bw.x, bw.y, bw.z, bw.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) cnt[i][j] += __popc((B[j] & T1[i]) | (~B[j] & T0[i]));
        }
      }
      if (dlim >= cend) {
        const int ch = a.chunk_d > 0 ? (d0 / a.chunk_d) : 0;
        const int cw = cend - (a.chunk_d > 0 ? ch * a.chunk_d : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = s_rows[ty * 4 + i];
          const float sa = row >= 0 ? a.sA[((long long)g * a.M + row) * a.n_chunks + ch] : 0.0f;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int col = col0 + tx * 4 + j;
            const float sb = col < a.N ? a.sB[((long long)g * a.N + col) * a.n_chunks + ch] : 0.0f;
            cacc[i][j] += (sa * sb) * (scaleL * (float)(UNI ? cnt[i][j] : 2 * cnt[i][j] - L * cw));
            if (COUNTS) bacc[i][j] += cnt[i][j];
            cnt[i][j] = 0;
          }
        }
      }
    }
    if (COUNTS) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = s_rows[ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = col0 + tx * 4 + j;
          if (row >= 0 && col < a.N)
            a.counts[(((long long)g * a.M + row) * a.N + col) * a.n_bands + b] = bacc[i][j];
          bacc[i][j] = 0;
        }
      }
    }
  }
  if (a.C) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = s_rows[ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = col0 + tx * 4 + j;
        const int ccol = col < a.N ? out_col(a, col) : -1;
        if (row >= 0 && ccol >= 0)
          a.C[(long long)g * a.bsc + (long long)row * a.ldc + ccol] =
              cacc[i][j] + (a.bias ? a.bias[(long long)g * a.N + col] : 0.0f);
      }
    }
  }
}


int launch_bitserial(const MatmulArgs& a, hipStream_t st) {
  const int RT = a.tile_start[a.n_rungs];
  if (RT == 0) return SCMP_OK;
  if (RT > 65535) return set_error(SCMP_ERR_ARG, "too many row tiles");
  const dim3 grid((a.N + BS_BN - 1) / BS_BN, RT, a.G);
  if (a.unipolar) {
    if (a.counts)
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_matmul_bitserial<true, true>), grid, dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL(HIP_KERNEL_NAME(k_matmul_bitserial<false, true>), grid, dim3(256), 0, st, a);
  } else if (a.counts) {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_matmul_bitserial<true, false>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL(HIP_KERNEL_NAME(k_matmul_bitserial<false, false>), grid, dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("bit-serial launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}

}  // namespace scmp
