// Arguments and device helpers shared by the XNOR contraction kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "internal.h"

namespace scmp {

constexpr int MAX_LEVELS = 257;  // 2^p + 1 levels for p <= 8

struct MatmulArgs {
  const int8_t* qA;
  const float* sA;
  const int32_t* perm;
  const int8_t* qB;
  const uint32_t* packedB;
  const float* sB;
  int32_t* counts;
  float* C;
  const float* bias;  // [G][N] added to every row of C (nullable)
  // Per-group lengths: every row of group g runs rung group_rung[g] of the
  // ladder (nullable).  Tiles then take each group's rows in order (one
  // tiling rung, no permutation); n_ladder is the ladder's rung count.
  const uint8_t* group_rung;
  int n_ladder;
  int unipolar;  // AND gate, sign-magnitude levels (bit-serial and staged matrix-core kernels)
  const uint32_t* K;  // packed indicator rows [P + 1][Wl] (the unipolar operand table)
  // Range MP: C column of each compact weight row (null: the identity).
  // Stores to columns outside [0, ldc) are dropped.
  const int32_t* cmap;
  long long ldc, bsc;
  const uint8_t* pair;
  const uint16_t* cum;
  int G, M, N, D, chunk_d, n_chunks, n_rungs, n_bands, q, P, Wl, Lmax;
  int launch;  // matrix-core launch form: 0 by size, 1 persistent, 2 one block per tile, 3 quarter (persistent)
  int auto_quarter;  // launch 0 may take the quarter form (AUTO; not MFMA)
  int cuts[SCMP_MAX_RUNGS + 1];
  int tile_start[SCMP_MAX_RUNGS + 1];  // first row tile of each rung (128 rows; 64 for bit-serial)
  int band_cols[SCMP_MAX_BANDS + 1];
  int bandL[SCMP_MAX_BANDS][SCMP_MAX_RUNGS];
  unsigned long long pair_off[SCMP_MAX_BANDS][SCMP_MAX_RUNGS];
};

// Level of a stored integer, clamped to [0, P] so that a corrupted input can
// never index outside the tables.
__device__ __forceinline__ int level_of(int x, int P, int q) {
  const int u = (P * (x + q) + q) / (2 * q);
  return u < 0 ? 0 : (u > P ? P : u);
}

// Unipolar level of the magnitude, round(P |x| / q) (q is odd: no ties),
// clamped the same way.
__device__ __forceinline__ int uni_level_of(int x, int P, int q) {
  const int u = (2 * P * abs(x) + q) / (2 * q);
  return u > P ? P : u;
}

// Rung and first sorted position of a row tile (tiles are numbered bucket
// after bucket).
__device__ __forceinline__ void locate_tile(const MatmulArgs& a, int y, int BM, int& k, int& pos0, int& nrows) {
  k = 0;
  while (k + 1 < a.n_rungs && y >= a.tile_start[k + 1]) ++k;
  pos0 = a.cuts[k] + (y - a.tile_start[k]) * BM;
  nrows = min(BM, a.cuts[k + 1] - pos0);
}

// The rung a tile runs: its group's rung with per-group lengths, else the
// tiling rung k (clamped so a corrupted input never indexes past the ladder).
__device__ __forceinline__ int tile_rung(const MatmulArgs& a, int g, int k) {
  if (!a.group_rung) return k;
  const int r = a.group_rung[g];
  return r < a.n_ladder ? r : a.n_ladder - 1;
}

// C column of compact column col (-1 when the store is to be dropped).
__device__ __forceinline__ int out_col(const MatmulArgs& a, int col) {
  if (!a.cmap) return col;
  const int c = a.cmap[col];
  return (c >= 0 && c < a.ldc) ? c : -1;
}

// Original row of a sorted position (the identity without a permutation).
__device__ __forceinline__ int row_of(const MatmulArgs& a, int g, int pos) {
  if (!a.perm) return pos;
  int r = a.perm[(long long)g * a.M + pos];
  return r < 0 ? 0 : (r >= a.M ? a.M - 1 : r);
}

// End of the chunk that contains column d.
__device__ __forceinline__ int chunk_end(const MatmulArgs& a, int d) {
  if (a.chunk_d <= 0) return a.D;
  return min((d / a.chunk_d + 1) * a.chunk_d, a.D);
}

// Host side: fill the tile table of the arguments for a row-tile height BM.
void fill_tiles(MatmulArgs& a, const Plan& P, int BM);

// Matrix-core path (mfma.hip).
size_t mfma_workspace_bytes(const MatmulArgs& a);
int launch_mfma(const MatmulArgs& a, void* ws, size_t ws_bytes, hipStream_t st);
int mfma_issued_macs(const MatmulArgs& a, const void* ws, size_t ws_bytes, hipStream_t st,
                     unsigned long long* macs, unsigned long long* fp4_macs);
int mfma_window_macs(const MatmulArgs& a, const void* ws, size_t ws_bytes, hipStream_t st,
                     unsigned long long* macs);

// Vector-ALU bit-serial path (bitserial.hip).
int launch_bitserial(const MatmulArgs& a, hipStream_t st);
size_t gather_workspace_bytes(const MatmulArgs& a);
int launch_gather(const MatmulArgs& a, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace scmp
