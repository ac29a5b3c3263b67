// Matrix-core XNOR contraction (v_mfma_i32_32x32x32_i8).
//
// "Precision As You Need" paper notes, Key design 1 (C-BSG, decode
// equation) and Key design 3 (early termination per row); K-band pull
// request, "How the banding works" (band b of the contraction axis runs rung
// k at L[b][k]; band partial products are summed).
//
// For contraction index d, A's L-prefix stream has n1 ones and n0 = L - n1
// zeros, and the XNOR count against B's conditional stream is
//   n0 + sum_c B_c (T1_c - T0_c)
// with B_c = K[u_B][c] and T1, T0 the prefix masks of n1, n0 ones.
// T1 - T0 is a run of +1 on [n0, n1) or -1 on [n1, n0), centred on L / 2.
// Folded at the centre it becomes a prefix of hh = ceil(|n1 - n0| / 2)
// paired positions k with sign s, and B becomes the pair sums
// B'_k = B_lo(k) + B_hi(k) in {0, 1, 2} (table.hip), so
//   count = n0 + s * sum_{k < hh} B'_k,
// an exact int8 contraction over ceil(L/2) paired positions per d.
//
// Two launches (the encode passes share one launch, k_prep):
//  prep_rows    per row tile: the window code 16 (2 hh + (s < 0)) (uint16,
//               the byte offset of the row's A fragment in the pattern table)
//               in bucket order, laid out [d][position], the tile's largest
//               hh at each d, and the n0 sum of every row over every chunk
//               ("A side at the row's L").
//  prep_cols    per column tile: the byte offset of each B level's row in
//               the paired table (uint16), laid out [d][column].
// Within every 64 positions (columns) the encode kernels store p and p + 32
// side by side, so one 32-bit LDS read gives a lane both of its row
// (column) subtiles.
//  k_mfma       per (row tile, column tile): stages 32 contraction indices
//               at a time through double-buffered LDS (one barrier per
//               stage), visits only the 32-position steps some row of the
//               tile needs (the tile's largest hh), and decodes per chunk.
// A row tile holds 128 consecutive sorted positions of one rung (one L per
// band), so early termination costs no divergence.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "matmul_common.h"

namespace scmp {

constexpr int MF_BM = 128, MF_BN = 128, MF_DC = 32;
constexpr int PT_STRIDE = 144;  // bytes per level row of the paired table in LDS
constexpr int PREP_BLOCKS = 1024;  // encode blocks aimed for (tiles x parts of the contraction axis)


struct MfmaWs {
  uint32_t* hs;     // [G][RT][Dp/32] blocks: window codes 16 (2 hh + neg) of a row pair, by index
  uint8_t* maxh;    // [G][RT][Dp]    largest |h| of each row tile at each d
  int32_t* rowc;    // [G][n_parts][Mp]   n0 summed over each part of the contraction axis
  uint32_t* ub;     // [G][CT][Dp/32] blocks: paired-table row offsets of a column pair, by index
  // Single-segment plans also keep the codes index-major (the persistent
  // contraction's list steps read one index for every pair); else null.
  uint32_t* hsi;    // [G][Dp][Mp/2]  window code words, by index then row pair
  uint32_t* ubi;    // [G][Dp][Np/2]  table offset words, by index then column pair
  int32_t* rowid;   // [G][Mp]       original row of each sorted position (-1: none)
  float* sas;       // [G][Mp]       row scale of each sorted position (single-segment plans)
  unsigned long long* issued;  // [2] MFMA steps issued over the row tiles: int8 steps, fp4 steps
  unsigned int* work;          // work counter of the persistent contraction
  long long Mp, Np, Dp;
  int RT, CT;
  // The encode kernels split the contraction axis into n_parts parts of
  // part_len columns (whole chunks when chunk_d is set, so a part's n0 sums
  // are the chunk sums; otherwise the decode adds the parts' partial sums).
  int n_parts, part_len;
};

static MfmaWs ws_layout(const MatmulArgs& a, void* base, size_t* total) {
  MfmaWs w{};
  w.RT = a.tile_start[a.n_rungs];
  w.CT = (a.N + MF_BN - 1) / MF_BN;
  w.Mp = (long long)w.RT * MF_BM;
  w.Np = (long long)w.CT * MF_BN;
  w.Dp = ((long long)a.D + MF_DC - 1) / MF_DC * MF_DC;
  {
    // Enough encode blocks to cover the CUs several times over, each with
    // a run of groups long enough to hide its fixed costs.
    const long long tiles = (long long)w.RT * a.G;
    const int unit = a.chunk_d > 0 ? a.chunk_d : MF_DC;
    const int units = (a.D + unit - 1) / unit;
    long long want = tiles > 0 ? (PREP_BLOCKS + tiles - 1) / tiles : 1;
    if (want < 1) want = 1;
    if (want > units) want = units;
    const int per = (int)((units + want - 1) / want);
    w.part_len = per * unit;
    w.n_parts = (a.D + w.part_len - 1) / w.part_len;
  }
  auto al = [](size_t v) { return (v + 255) & ~(size_t)255; };
  size_t off = 0;
  const size_t hs_b = al((size_t)a.G * w.Dp * w.Mp * sizeof(uint16_t));
  const size_t mx_b = al((size_t)a.G * w.RT * w.Dp);
  const int rc_parts = a.chunk_d > 0 ? a.n_chunks : w.n_parts;
  const size_t rc_b = al((size_t)a.G * rc_parts * w.Mp * sizeof(int32_t));
  const size_t ub_b = al((size_t)a.G * w.Dp * w.Np * sizeof(uint16_t));
  const bool index_major = a.chunk_d <= 0 && a.n_bands == 1;
  const size_t hsi_b = index_major ? hs_b : 0;
  const size_t ubi_b = index_major ? ub_b : 0;
  const size_t ri_b = al((size_t)a.G * w.Mp * sizeof(int32_t));
  const size_t sa_b = al((size_t)a.G * w.Mp * sizeof(float));
  const size_t ts_b = al(2 * sizeof(unsigned long long) + sizeof(unsigned int));
  char* p = (char*)base;
  // The step counters first, at an offset that does not depend on the sizes.
  w.issued = (unsigned long long*)(p ? p + off : nullptr);
  w.work = (unsigned int*)(p ? p + off + 2 * sizeof(unsigned long long) : nullptr);
  off += ts_b;
  w.hs = (uint32_t*)(p ? p + off : nullptr);
  off += hs_b;
  w.maxh = (uint8_t*)(p ? p + off : nullptr);
  off += mx_b;
  w.rowc = (int32_t*)(p ? p + off : nullptr);
  off += rc_b;
  w.ub = (uint32_t*)(p ? p + off : nullptr);
  off += ub_b;
  w.hsi = (index_major && p) ? (uint32_t*)(p + off) : nullptr;
  off += hsi_b;
  w.ubi = (index_major && p) ? (uint32_t*)(p + off) : nullptr;
  off += ubi_b;
  w.rowid = (int32_t*)(p ? p + off : nullptr);
  off += ri_b;
  w.sas = (float*)(p ? p + off : nullptr);
  off += sa_b;
  *total = off;
  return w;
}

__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
  return v;
}

// Row (column) pairs.  A 128-wide tile has 64 pairs; pair pr holds
// positions lo(pr) and lo(pr) + 32 with lo(pr) = 64 (pr / 32) + pr mod 32,
// the two rows (columns) one lane supplies to the two 32-wide subtiles of a
// 64-wide wave tile.  The encode buffers keep, per pair, one 32-bit word per
// contraction index: the low half for position lo, the high half for lo + 32.
__device__ __forceinline__ int pair_lo(int pr) { return ((pr & 32) << 1) | (pr & 31); }

// The encode buffers hs and ub are blocked by groups of 32 contraction
// indices: the 64 pairs x 32 indices of one (tile, group) are 2048
// consecutive words, ordered [p / 32][(e % 16) / 4][e / 16][p % 32][e % 4]
// for pair p and index e of the group.  A wave lane that supplies pair
// 32 s + l and the index half h of a group then finds indices
// 16 h + 4 i + [0, 4) at word (8 s + h) 128 + 4 l + 256 i of the block, so
// each of the wave's four 16-byte loads per group reads one contiguous
// kilobyte (a lane per pair with the index axis contiguous would touch 64
// cache lines per load).
__device__ __forceinline__ long long enc_word(long long tile, int ngrp, int d, int p) {
  const int e = d & 31;
  return ((tile * ngrp + (d >> 5)) << 11) + (long long)(((((p >> 5) * 4 + ((e & 15) >> 2)) * 2 + (e >> 4)) * 32 + (p & 31)) * 4 + (e & 3));
}

// Load 8 int8 values x[0..8) (bounds-checked, vectorised when aligned).
__device__ __forceinline__ void load8(const int8_t* src, int valid, int8_t* out) {
  if (valid >= 8 && (((uintptr_t)src) & 7) == 0) {
    const int2 v = *(const int2*)src;
    const int8_t* b = (const int8_t*)&v;
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = b[i];
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = i < valid ? src[i] : (int8_t)0;
  }
}

// ------------------------------------------------------------ prep A ----
// grid (RT, n_parts, G), block 256: wave q takes indices [d0 + 8 q,
// d0 + 8 q + 8) of every group of 32, lane pr the row pair pr (both rows).
// A wave then holds all 64 pairs of its indices: the tile maximum per index
// is a wave reduction, and each index-major store covers 64 consecutive
// pairs.  The block covers indices [part * part_len, ...) of one tile.
__device__ __forceinline__ void prep_rows(const MatmulArgs& a, const MfmaWs& w, int bx) {
  __shared__ uint32_t s_lut[256];
  __shared__ int s_rows[MF_BM];
  __shared__ int s_rc[MF_BM];  // n0 sums of the tile's rows over the current chunk or part
  const int tid = threadIdx.x;
  const int y = bx, part = blockIdx.y, g = blockIdx.z;
  int k, pos0, nrows;
  locate_tile(a, y, MF_BM, k, pos0, nrows);
  k = tile_rung(a, g, k);
  const int lane = tid & 63, q = tid >> 6;
  const int pr = lane;
  const int p_lo = pair_lo(pr), p_hi = p_lo + 32;
  if (tid < MF_BM) {
    s_rows[tid] = tid < nrows ? row_of(a, g, pos0 + tid) : -1;
    s_rc[tid] = 0;
  }
  __syncthreads();
  const int row_lo = s_rows[p_lo], row_hi = s_rows[p_hi];
  const int8_t* src_lo = a.qA + ((long long)g * a.M + (row_lo < 0 ? 0 : row_lo)) * a.D;
  const int8_t* src_hi = a.qA + ((long long)g * a.M + (row_hi < 0 ? 0 : row_hi)) * a.D;
  const long long tile = (long long)g * w.RT + y;
  const int ngrp = (int)(w.Dp / MF_DC);
  const int plo = part * w.part_len;
  const int phi = min(plo + w.part_len, a.D);
  int rc_lo = 0, rc_hi = 0;  // n0 sums of this lane's rows over its indices
  // n0 sums of the tile's rows over the four waves' indices, written to
  // slot `slot` (every wave calls this together).
  auto flush_rc = [&](long long slot) {
    atomicAdd(&s_rc[p_lo], rc_lo);
    atomicAdd(&s_rc[p_hi], rc_hi);
    rc_lo = rc_hi = 0;
    __syncthreads();
    if (tid < MF_BM) {
      w.rowc[slot * w.Mp + (long long)y * MF_BM + tid] = s_rc[tid];
      s_rc[tid] = 0;
    }
    __syncthreads();
  };
  for (int b = 0; b < a.n_bands; ++b) {
    const int lo = max(a.band_cols[b], plo);
    const int dend = min(a.band_cols[b + 1], phi);
    if (lo >= dend) continue;  // uniform over the block
    const int L = a.bandL[b][k];
    __syncthreads();
    // Everything an element needs at this L, per stored value x (entry
    // x + 128): window code (14 bits), the tile-maximum key hh (8 bits) and
    // its n0 term (9 bits), so the per-element work is one table read.
    // Bipolar: the half-window hh of |n1 - n0| with the sign of n1 - n0,
    // and n0 = L - n1.  Unipolar: the whole prefix of n1 positions with the
    // sign of x (hh = n1, kept to 8 bits as 255 = "all 16 half-blocks"),
    // and no n0 term.
    {
      const int x = tid - 128;
      uint32_t e;
      if (a.unipolar) {
        const int n1 = a.cum[(long long)uni_level_of(x, a.P, a.q) * (a.Lmax + 1) + L];
        e = (uint32_t)(16 * (2 * n1 + (x < 0 ? 1 : 0))) | ((uint32_t)min(n1, 255) << 14);
      } else {
        const int n1 = a.cum[(long long)level_of(x, a.P, a.q) * (a.Lmax + 1) + L];
        const int diff = 2 * n1 - L;
        const int hh = ((diff < 0 ? -diff : diff) + 1) >> 1;
        const int code = 16 * (2 * hh + (diff < 0 ? 1 : 0));
        e = (uint32_t)code | ((uint32_t)hh << 14) | ((uint32_t)(L - n1) << 22);
      }
      s_lut[tid] = e;
    }
    __syncthreads();
    // The next group's values are read while this group is encoded.
    int8_t nx_lo[8], nx_hi[8];
    {
      const int span = max(0, min(8, dend - (lo + 8 * q)));
      load8(src_lo + lo + 8 * q, row_lo >= 0 ? span : 0, nx_lo);
      load8(src_hi + lo + 8 * q, row_hi >= 0 ? span : 0, nx_hi);
    }
    for (int d0 = lo; d0 < dend; d0 += MF_DC) {
      const int dfirst = d0 + 8 * q;
      const int span = max(0, min(8, dend - dfirst));
      int8_t x_lo[8], x_hi[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        x_lo[i] = nx_lo[i];
        x_hi[i] = nx_hi[i];
      }
      if (d0 + MF_DC < dend) {
        const int nspan = max(0, min(8, dend - (dfirst + MF_DC)));
        load8(src_lo + dfirst + MF_DC, row_lo >= 0 ? nspan : 0, nx_lo);
        load8(src_hi + dfirst + MF_DC, row_hi >= 0 ? nspan : 0, nx_hi);
      }
      uint32_t word[8];
      int mh[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        int code[2] = {0, 0}, hh[2] = {0, 0};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = i < span && (h == 0 ? row_lo : row_hi) >= 0;
          if (ok) {
            const uint32_t e = s_lut[(int)(h == 0 ? x_lo[i] : x_hi[i]) + 128];
            code[h] = (int)(e & 0x3FFFu);
            hh[h] = (int)((e >> 14) & 0xFFu);
            (h == 0 ? rc_lo : rc_hi) += (int)(e >> 22);
          }
        }
        word[i] = (uint32_t)code[0] | ((uint32_t)code[1] << 16);
        mh[i] = max(hh[0], hh[1]);
      }
      // d0 + 32 <= Dp: the whole group is inside the buffer (indices past
      // the band or D get code 0); dfirst is a multiple of 8.
      *(uint4*)(w.hs + enc_word(tile, ngrp, dfirst, pr)) = uint4{word[0], word[1], word[2], word[3]};
      *(uint4*)(w.hs + enc_word(tile, ngrp, dfirst + 4, pr)) = uint4{word[4], word[5], word[6], word[7]};
      if (w.hsi) {
        uint32_t* di = w.hsi + ((long long)g * w.Dp + dfirst) * (w.Mp / 2) + (long long)y * 64 + pr;
#pragma unroll
        for (int i = 0; i < 8; ++i) di[(long long)i * (w.Mp / 2)] = word[i];
      }
      // Tile maximum per index: over the wave's 64 pairs.
      int mine = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int m = wave_max_i(mh[i]);
        if (lane == i) mine = m;
      }
      if (lane < 8) w.maxh[((long long)g * w.RT + y) * w.Dp + dfirst + lane] = (uint8_t)mine;
      if (a.chunk_d > 0 && ((d0 + MF_DC) % a.chunk_d == 0 || d0 + MF_DC >= a.D))
        flush_rc((long long)g * a.n_chunks + d0 / a.chunk_d);
    }
  }
  if (a.chunk_d <= 0) flush_rc((long long)g * w.n_parts + part);
  if (part == 0 && tid < MF_BM) {
    const long long pos = (long long)g * w.Mp + (long long)y * MF_BM + tid;
    const int row = s_rows[tid];
    w.rowid[pos] = row;
    w.sas[pos] = (a.chunk_d <= 0 && row >= 0) ? a.sA[(long long)g * a.M + row] : 0.0f;
  }
}

// ------------------------------------------------------------ prep B ----
// grid (CT, n_parts, G), block 256: thread -> (column pair cp = tid / 4,
// quarter q = tid % 4), indices [d0 + 8 q, d0 + 8 q + 8) of each group of
// 32 in the block's part of the contraction axis.
__device__ __forceinline__ void prep_cols(const MatmulArgs& a, const MfmaWs& w, int bx) {
  // Table row offset of each stored value x (entry x + 128).  Unipolar:
  // the magnitude's level row, with the sign of x in bit 0 (row offsets are
  // multiples of 16).
  __shared__ uint32_t s_off[256];
  const int tid = threadIdx.x;
  {
    const int x = tid - 128;
    s_off[tid] = a.unipolar ? (uint32_t)(uni_level_of(x, a.P, a.q) * PT_STRIDE) | (x < 0 ? 1u : 0u)
                            : (uint32_t)(level_of(x, a.P, a.q) * PT_STRIDE);
  }
  const int c0 = bx * MF_BN, g = blockIdx.z;
  const int plo = blockIdx.y * w.part_len;
  const int phi = (int)min((long long)plo + w.part_len, w.Dp);
  // The contraction (launched after this kernel on the same stream) adds
  // its issued steps to this counter.
  if (bx == 0 && blockIdx.y == 0 && blockIdx.z == 0 && tid == 0) {
    w.issued[0] = 0;
    w.issued[1] = 0;
    *w.work = 0;
  }
  const int cp = tid >> 2, q = tid & 3;
  const int col_lo = c0 + pair_lo(cp), col_hi = col_lo + 32;
  const int8_t* src_lo = a.qB + ((long long)g * a.N + (col_lo < a.N ? col_lo : 0)) * a.D;
  const int8_t* src_hi = a.qB + ((long long)g * a.N + (col_hi < a.N ? col_hi : 0)) * a.D;
  const long long tile = (long long)g * w.CT + bx;
  const int ngrp = (int)(w.Dp / MF_DC);
  const uint32_t pad = a.unipolar ? 0u : (uint32_t)((a.P >> 1) * PT_STRIDE);
  __syncthreads();
  for (int d0 = plo; d0 < phi; d0 += MF_DC) {
    const int dfirst = d0 + 8 * q;
    const int span = max(0, min(8, a.D - dfirst));
    int8_t x_lo[8], x_hi[8];
    load8(src_lo + dfirst, col_lo < a.N ? span : 0, x_lo);
    load8(src_hi + dfirst, col_hi < a.N ? span : 0, x_hi);
    uint32_t word[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t o_lo = (i < span && col_lo < a.N) ? s_off[(int)x_lo[i] + 128] : pad;
      const uint32_t o_hi = (i < span && col_hi < a.N) ? s_off[(int)x_hi[i] + 128] : pad;
      word[i] = o_lo | (o_hi << 16);
    }
    *(uint4*)(w.ub + enc_word(tile, ngrp, dfirst, cp)) = uint4{word[0], word[1], word[2], word[3]};
    *(uint4*)(w.ub + enc_word(tile, ngrp, dfirst + 4, cp)) = uint4{word[4], word[5], word[6], word[7]};
    if (w.ubi) {
      uint32_t* di = w.ubi + ((long long)g * w.Dp + dfirst) * (w.Np / 2) + (long long)bx * 64 + cp;
#pragma unroll
      for (int i = 0; i < 8; ++i) di[(long long)i * (w.Np / 2)] = word[i];
    }
  }
}

// Both encode passes in one launch, so that they run side by side: blocks
// x < RT encode row tile x, the others column tile x - RT (grid
// (RT + CT, n_parts, G)).
__global__ void __launch_bounds__(256) k_prep(MatmulArgs a, MfmaWs w) {
  if ((int)blockIdx.x < w.RT)
    prep_rows(a, w, (int)blockIdx.x);
  else
    prep_cols(a, w, (int)blockIdx.x - w.RT);
}

// ------------------------------------------------------------- main ----
// The contraction runs on the fp4 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with e2m1 A and B operands at unit
// scales): the A bytes {-1, 0, +1} and the pair sums {0, 1, 2} are exact in
// e2m1, and the fp32 accumulators hold the integer counts exactly (every
// count is below 2^24).  Lane l of a 32 x 32 x 64 MFMA supplies row
// (column) l mod 32 and positions [32 (l / 32), 32 (l / 32) + 32) as 32
// nibbles, low nibble first; each lane half takes two 16-position
// half-blocks of the windowed contraction, X in nibbles 0-15 and Y in
// nibbles 16-31 (the MFMA sums both), so one step of four MFMAs per wave
// covers four half-blocks of its 64 x 64 tile.
typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// A patterns: entry e (16-byte stride, first 8 bytes used) holds
// min(e / 2, 16) leading sign nibbles, 0xA (-1) when e is odd and 0x2 (+1)
// otherwise, then zero nibbles.  A row whose window code is
// c = 16 (2 hh + neg) finds its fragment for positions [kk, kk + 16) at byte
// offset max(c - 32 kk, 0): entry 2 (hh - kk) + neg when hh > kk (the first
// clamp(hh - kk, 0, 16) positions), a zero entry (0 or 1) otherwise.  Rows
// with equal fragments read one address (an LDS broadcast).
constexpr int PAT_WORDS = 258 * 4;
__device__ __forceinline__ void init_patterns(uint32_t* pat, int tid, int nthreads) {
  for (int w = tid; w < PAT_WORDS; w += nthreads) {
    const int e = w >> 2, wd = w & 3, n = min(e >> 1, 16);
    const uint32_t one = (e & 1) ? 0xAu : 0x2u;
    uint32_t x = 0;
    if (wd < 2)
      for (int nib = 0; nib < 8; ++nib)
        if (wd * 8 + nib < n) x |= one << (4 * nib);
    pat[w] = x;
  }
}

// The paired table of band b, rung k as e2m1 nibbles (value v -> code 2 v,
// position p in nibble p mod 2 of byte p / 2), one LDS row of PT_STRIDE
// bytes per B level.
__device__ __forceinline__ void stage_pair_table(uint8_t* pt, const MatmulArgs& a, int b, int k, int KLpad, int tid,
                                                 int nthreads) {
  const uint8_t* src = a.pair + a.pair_off[b][k];
  const int vec_per_row = KLpad >> 4;
  for (int idx = tid; idx < (a.P + 1) * vec_per_row; idx += nthreads) {
    const int u = idx / vec_per_row, v = idx - u * vec_per_row;
    const uint4 x = *(const uint4*)(src + (long long)u * KLpad + v * 16);
    auto pack = [](uint32_t wd) {
      const uint32_t t = wd << 1;  // bytes <= 2: doubling never carries
      return (t & 0xFu) | ((t >> 4) & 0xF0u) | ((t >> 8) & 0xF00u) | ((t >> 12) & 0xF000u);
    };
    *(uint2*)(pt + u * PT_STRIDE + v * 8) = uint2{pack(x.x) | (pack(x.y) << 16), pack(x.z) | (pack(x.w) << 16)};
  }
}

// The unipolar operand table as e2m1 nibbles: row u holds K[u][p] (0 or
// 1, code 0 or 2) for positions p < 256 (zero past Lmax), position p in
// nibble p mod 2 of byte p / 2, one LDS row of PT_STRIDE bytes per level.
// The AND count of a prefix of n1 positions is the sum of its first n1
// entries, whatever L is.
__device__ __forceinline__ void stage_uni_table(uint8_t* pt, const MatmulArgs& a, int tid, int nthreads) {
  for (int idx = tid; idx < (a.P + 1) * 16; idx += nthreads) {
    const int u = idx >> 4, c = idx & 15;  // 16 positions [16 c, 16 c + 16)
    const uint32_t word = (c >> 1) < a.Wl ? a.K[(long long)u * a.Wl + (c >> 1)] : 0u;
    const uint32_t bits = (word >> (16 * (c & 1))) & 0xffffu;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      lo |= ((bits >> i) & 1u) << (4 * i + 1);
      hi |= ((bits >> (i + 8)) & 1u) << (4 * i + 1);
    }
    *(uint2*)(pt + u * PT_STRIDE + c * 8) = uint2{lo, hi};
  }
}

// Operands of one step for this lane half: half-blocks X (row codes hx of
// rows l32 and l32 + 32, column table offsets ux of columns l32 and l32 + 32,
// first position kx) and Y.  A from the pattern table, B from the nibble
// table at row offset + k / 2.
struct Frag {
  v8i a[2], b[2];
};
__device__ __forceinline__ Frag frags_at(const uint8_t* pat, const uint8_t* pt, uint32_t hx, uint32_t ux, uint32_t kx,
                                         uint32_t hy, uint32_t uy, uint32_t ky) {
  Frag f;
  const v2i ax0 = *(const v2i*)(pat + __builtin_elementwise_sub_sat(hx & 0xffffu, 32u * kx));
  const v2i ax1 = *(const v2i*)(pat + __builtin_elementwise_sub_sat(hx >> 16, 32u * kx));
  const v2i ay0 = *(const v2i*)(pat + __builtin_elementwise_sub_sat(hy & 0xffffu, 32u * ky));
  const v2i ay1 = *(const v2i*)(pat + __builtin_elementwise_sub_sat(hy >> 16, 32u * ky));
  const v2i bx0 = *(const v2i*)(pt + (ux & 0xffffu) + (kx >> 1));
  const v2i bx1 = *(const v2i*)(pt + (ux >> 16) + (kx >> 1));
  const v2i by0 = *(const v2i*)(pt + (uy & 0xffffu) + (ky >> 1));
  const v2i by1 = *(const v2i*)(pt + (uy >> 16) + (ky >> 1));
  f.a[0] = v8i{ax0.x, ax0.y, ay0.x, ay0.y, 0, 0, 0, 0};
  f.a[1] = v8i{ax1.x, ax1.y, ay1.x, ay1.y, 0, 0, 0, 0};
  f.b[0] = v8i{bx0.x, bx0.y, by0.x, by0.y, 0, 0, 0, 0};
  f.b[1] = v8i{bx1.x, bx1.y, by1.x, by1.y, 0, 0, 0, 0};
  return f;
}

// frags_at for unipolar operands.  Prefixes reach 256 positions, so a
// pattern offset can pass the table's last entry: entries from 32 on all
// hold 16 sign nibbles, so the offset is clamped to entry 32 or 33 with the
// same parity.  B's row offsets carry the sign of B's value in bit 0,
// applied by flipping the sign bit of every nibble (0x2 -> 0xA; 0x0 ->
// 0x8, which is also zero).
__device__ __forceinline__ Frag frags_at_uni(const uint8_t* pat, const uint8_t* pt, uint32_t hx, uint32_t ux,
                                             uint32_t kx, uint32_t hy, uint32_t uy, uint32_t ky) {
  auto aoff = [](uint32_t code, uint32_t k) {
    const uint32_t o = __builtin_elementwise_sub_sat(code, 32u * k);
    return min(o, 512u + (o & 16u));
  };
  Frag f;
  const v2i ax0 = *(const v2i*)(pat + aoff(hx & 0xffffu, kx));
  const v2i ax1 = *(const v2i*)(pat + aoff(hx >> 16, kx));
  const v2i ay0 = *(const v2i*)(pat + aoff(hy & 0xffffu, ky));
  const v2i ay1 = *(const v2i*)(pat + aoff(hy >> 16, ky));
  const v2i bx0 = *(const v2i*)(pt + (ux & 0xfffeu) + (kx >> 1));
  const v2i bx1 = *(const v2i*)(pt + ((ux >> 16) & 0xfffeu) + (kx >> 1));
  const v2i by0 = *(const v2i*)(pt + (uy & 0xfffeu) + (ky >> 1));
  const v2i by1 = *(const v2i*)(pt + ((uy >> 16) & 0xfffeu) + (ky >> 1));
  auto flip = [](uint32_t u, int sh) { return (int)(0u - ((u >> sh) & 1u)) & (int)0x88888888u; };
  const int sx0 = flip(ux, 0), sx1 = flip(ux, 16), sy0 = flip(uy, 0), sy1 = flip(uy, 16);
  f.a[0] = v8i{ax0.x, ax0.y, ay0.x, ay0.y, 0, 0, 0, 0};
  f.a[1] = v8i{ax1.x, ax1.y, ay1.x, ay1.y, 0, 0, 0, 0};
  f.b[0] = v8i{bx0.x ^ sx0, bx0.y ^ sx0, by0.x ^ sy0, by0.y ^ sy0, 0, 0, 0, 0};
  f.b[1] = v8i{bx1.x ^ sx1, bx1.y ^ sx1, by1.x ^ sy1, by1.y ^ sy1, 0, 0, 0, 0};
  return f;
}

// One step: the wave's 2 x 2 subtiles of 32 x 32.
__device__ __forceinline__ void mma_step(v16f (&acc)[2][2], const Frag& f) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
      acc[i][jj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[jj], acc[i][jj], 4, 4, 0, 127, 0, 127);
}

// ------------------------------------------------------------ staged ----
// One block per 128 x 128 output tile (grid: column tiles, row tiles,
// groups); handles chunk scales and K-bands.  The tile's row and column
// codes pass through LDS 32 contraction indices (a stage) at a time, double
// buffered; one wave lists the stage's work while the stage is stored.
// Two blocks per CU (2 waves per SIMD) for the timed variants; the variants
// that also write per-band counts keep a third accumulator set and run one.
// UNI: the unipolar mode, whose prefixes run up to 16 half-blocks of 16
// positions (8 for the bipolar half-windows); schedule entries then carry
// the half-block index j instead of its first position 16 j.
template <bool CHUNKED, bool COUNTS, bool UNI>
__global__ void __launch_bounds__(256, COUNTS ? 1 : 2) k_mfma(MatmulArgs a, MfmaWs w) {
  constexpr int BM = MF_BM, BN = MF_BN, DC = MF_DC;
  constexpr int NLEV = UNI ? 16 : 8;
  // The two gather tables share one object (the largest, laid out first) so
  // that both sit below 64 KB, where a constant base folds into the LDS
  // instruction's offset.
  struct __align__(16) GatherTables {
    uint8_t pt[MAX_LEVELS * PT_STRIDE];
    uint32_t pat[PAT_WORDS];
  };
  __shared__ GatherTables s_tab;
  const uint8_t* const s_pt = s_tab.pt;
  const uint8_t* const s_pat = (const uint8_t*)s_tab.pat;
  // Stage code words, [pair][index]: rows of SW = DC + 2 words, so that the
  // 32 pairs of a half-wave's 8-byte reads start on 32 distinct bank pairs
  // (34 p mod 64 = 2 (17 p mod 32)).
  constexpr int SW = DC + 2;
  __shared__ __align__(16) uint32_t s_h[2][BM / 2][SW];  // [row pair][index]
  __shared__ __align__(16) uint32_t s_u[2][BN / 2][SW];  // [column pair][index]
  // Stage schedule: the half-blocks past the stage's full levels in order,
  // then padding entries (a zero half-block), and the steps they take.
  constexpr int SCHED_N = DC * NLEV + 16;
  __shared__ __align__(4) uint16_t s_sched[2][SCHED_N];
  __shared__ int s_nsteps[2];
  __shared__ int s_full[2];  // leading levels needed by every index of the stage
  __shared__ __align__(16) int s_rows[BM];
  __shared__ __align__(16) int s_rc[BM];      // n0 sum of each row over the chunk (or axis) being decoded
  __shared__ __align__(16) float s_sa[BM];    // row scale of that chunk

  const int tid = threadIdx.x;
  const int g = blockIdx.z, y = blockIdx.y;  // y: encode tile (128 rows of one rung)
  int k, pos0, nrows;
  locate_tile(a, y, BM, k, pos0, nrows);
  k = tile_rung(a, g, k);
  const long long prow0 = (long long)y * BM;
  const int col0 = blockIdx.x * BN;
  for (int r = tid; r < BM; r += 256) s_rows[r] = r < nrows ? row_of(a, g, pos0 + r) : -1;
  init_patterns(s_tab.pat, tid, 256);

  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int l32 = lane & 31, hf = lane >> 5;
  const int qq = a.q * a.q;
  const int wrow0 = wr * 64;  // first row of this wave
  const int wcol0 = wc * 64;  // first column of this wave

  // Stage loader: thread t reads 16-byte pieces t and t + 256 of the
  // stage's blocks of row and column code words (one contiguous 4 KB per
  // wave and buffer; pieces t and t + 256 hold indices
  // 16 ((t / 32) % 2) + 4 ((t / 64) % 4) + [0, 4) of pairs t % 32 and
  // t % 32 + 32, into named registers so they stay in VGPRs) and stores them
  // as the stage's [pair][index] words (8-byte stores: rows are 8-byte
  // aligned).
  int4 rh0, rh1, ru0, ru1;
  int rmx = 0;
  const int ngrp = (int)(w.Dp / MF_DC);
  const uint32_t* hblk = w.hs + enc_word((long long)g * w.RT + y, ngrp, 0, 0) + 4 * tid;
  const uint32_t* ublk = w.ub + enc_word((long long)g * w.CT + blockIdx.x, ngrp, 0, 0) + 4 * tid;
  const int sp = tid & 31, se = 16 * ((tid >> 5) & 1) + 4 * ((tid >> 6) & 3);
  auto fetch = [&](int d0) {
    const long long gb = (long long)(d0 >> 5) << 11;
    rh0 = *(const int4*)(hblk + gb);
    rh1 = *(const int4*)(hblk + gb + 1024);
    ru0 = *(const int4*)(ublk + gb);
    ru1 = *(const int4*)(ublk + gb + 1024);
    if (tid < DC) rmx = w.maxh[((long long)g * w.RT + y) * w.Dp + d0 + tid];
  };
  auto store = [&](int bf) {
    *(uint2*)&s_h[bf][sp][se] = uint2{(uint32_t)rh0.x, (uint32_t)rh0.y};
    *(uint2*)&s_h[bf][sp][se + 2] = uint2{(uint32_t)rh0.z, (uint32_t)rh0.w};
    *(uint2*)&s_h[bf][sp + 32][se] = uint2{(uint32_t)rh1.x, (uint32_t)rh1.y};
    *(uint2*)&s_h[bf][sp + 32][se + 2] = uint2{(uint32_t)rh1.z, (uint32_t)rh1.w};
    *(uint2*)&s_u[bf][sp][se] = uint2{(uint32_t)ru0.x, (uint32_t)ru0.y};
    *(uint2*)&s_u[bf][sp][se + 2] = uint2{(uint32_t)ru0.z, (uint32_t)ru0.w};
    *(uint2*)&s_u[bf][sp + 32][se] = uint2{(uint32_t)ru1.x, (uint32_t)ru1.y};
    *(uint2*)&s_u[bf][sp + 32][se + 2] = uint2{(uint32_t)ru1.z, (uint32_t)ru1.w};
    if (tid < 64) {
      // Wave 0 lists the stage's half-blocks: index d (lane d < DC holds its
      // tile maximum rmx) needs positions [16 j, 16 j + 16) for every
      // j < ceil(rmx / 16); the leading levels every index needs are swept
      // without a list, the rest are listed level by level, indices in
      // order within a level.  Entry: (d << 10) | kk (4 d, the byte offset
      // of index d's word in a stage row, in bits 8-14, and the first paired
      // position kk = 16 j; UNI: j itself).
      const int m = tid < DC ? rmx : 0;
      int full = 0;
      while (full < NLEV && (unsigned)__ballot(m > 16 * full) == 0xffffffffu) ++full;
      int base = 0;
      for (int j = full; j < NLEV; ++j) {
        const unsigned long long bal = __ballot(m > 16 * j);
        if (bal == 0) break;
        if (m > 16 * j) {
          const int pos = base + (int)__builtin_amdgcn_mbcnt_hi((unsigned)(bal >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((unsigned)bal, 0u));
          s_sched[bf][pos] = (uint16_t)((tid << 10) | (UNI ? j : 16 * j));
        }
        base += __builtin_popcountll(bal);
      }
      // Padding: position 16 NLEV is past every window or prefix (A nibbles
      // all zero).
      if (tid < 16) s_sched[bf][base + tid] = (uint16_t)(UNI ? NLEV : 16 * NLEV);
      if (tid == 0) s_full[bf] = full;
      if (tid == 0) s_nsteps[bf] = (base + 3) >> 2;
    }
  };

  v16f acc[2][2];
  float cacc[2][2][16];
  int bacc[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc[i][j][v] = 0.0f;
        if (CHUNKED) cacc[i][j][v] = 0.0f;
        if (COUNTS) bacc[i][j][v] = 0;
      }
  unsigned long long issued = 0;  // fp4 MFMA steps of this row tile (counted by the x == 0 blocks)

  int buf = 0;
  fetch(a.band_cols[0]);
  for (int b = 0; b < a.n_bands; ++b) {
    const int L = a.bandL[b][k];
    const int KLpad = ((((L + 1) >> 1) + 31) & ~31);
    const float scaleL = (float)qq / (float)L;
    const int dbeg = a.band_cols[b], dend = a.band_cols[b + 1];
    __syncthreads();  // every wave is done with the previous band's table
    if (UNI) {
      if (b == 0) stage_uni_table(s_tab.pt, a, tid, 256);  // one table for every L
    } else {
      stage_pair_table(s_tab.pt, a, b, k, KLpad, tid, 256);
    }
    store(buf);
    __syncthreads();
    for (int d0 = dbeg; d0 < dend; d0 += DC) {
      const int dn = d0 + DC;
      if (dn < a.D) fetch(dn);  // next stage (possibly in the next band) into registers
      {
        // Work of a stage: for every staged index d, the 16-position blocks
        // [16 j, 16 j + 16) of paired positions with j < ceil(mx_d / 16),
        // mx_d being the largest half-window of the tile's rows at d (rows'
        // windows nest inside it; past a row's own window its A nibbles are
        // zero).  Any four half-blocks may share a step: lanes 0-31 take
        // the first two (X, Y), lanes 32-63 the other two.
        const char* hbase = (const char*)&s_h[buf][wr * 32 + l32][0];
        const char* ubase = (const char*)&s_u[buf][wc * 32 + l32][0];
        const uint32_t* sched = (const uint32_t*)&s_sched[buf][0] + hf;  // entry pairs
        const int n = s_nsteps[buf];
        const int full = s_full[buf];
        // Two half-blocks as this lane sees them: the row and column words
        // of X and Y and their schedule entries (X low, Y high half of e).
        struct Item {
          uint32_t hx, ux, hy, uy, e;
        };
        auto item = [&](uint32_t e) __attribute__((always_inline)) {
          const uint32_t ox = (e >> 8) & 0x7cu, oy = (e >> 24) & 0x7cu;
          return Item{*(const uint32_t*)(hbase + ox), *(const uint32_t*)(ubase + ox),
                      *(const uint32_t*)(hbase + oy), *(const uint32_t*)(ubase + oy), e};
        };
        // X and Y on adjacent indices (X even): one 8-byte read per buffer.
        auto item2 = [&](uint32_t e) __attribute__((always_inline)) {
          const uint32_t ox = (e >> 8) & 0x7cu;
          const uint2 h2 = *(const uint2*)(hbase + ox), u2 = *(const uint2*)(ubase + ox);
          return Item{h2.x, u2.x, h2.y, u2.y, e};
        };
        auto frags = [&](const Item& c) __attribute__((always_inline)) {
          if (UNI)
            return frags_at_uni(s_pat, s_pt, c.hx, c.ux, 16u * (c.e & 0x1fu), c.hy, c.uy,
                                16u * ((c.e >> 16) & 0x1fu));
          return frags_at(s_pat, s_pt, c.hx, c.ux, c.e & 0xffu, c.hy, c.uy, (c.e >> 16) & 0xffu);
        };
        // Software-pipelined sweep over steps 0 .. cnt - 1, ent(s) giving the
        // lane's entry pair of step s (any entry past the end is a zero
        // half-block) and itm its codes: while step s's MFMAs run, the
        // fragments of step s + 1, the codes of step s + 2 and the entries of
        // step s + 3 are in flight (LDS reads complete in order, so each is
        // read a step ahead of the reads it addresses).  Two fragment sets
        // are used in turn.
        auto sweep = [&](int cnt, auto&& ent, auto&& itm) __attribute__((always_inline)) {
          uint32_t e2 = ent(2);
          const Item c0 = itm(ent(0));
          Item c1 = itm(ent(1));
          Frag fa = frags(c0), fb;
          int st = 0;
          for (; st + 2 < cnt; st += 2) {
            uint32_t e3 = ent(st + 3);
            Item c2 = itm(e2);
            fb = frags(c1);
            e2 = e3;
            c1 = c2;
            __builtin_amdgcn_sched_barrier(0);  // keep these reads ahead of the MFMAs
            mma_step(acc, fa);
            e3 = ent(st + 4);
            c2 = itm(e2);
            fa = frags(c1);
            e2 = e3;
            c1 = c2;
            __builtin_amdgcn_sched_barrier(0);
            mma_step(acc, fb);
          }
          // Last one or two steps.
          if (cnt - st == 2) fb = frags(c1);
          __builtin_amdgcn_sched_barrier(0);
          mma_step(acc, fa);
          if (cnt - st == 2) mma_step(acc, fb);
        };
        // Full levels: step 8 j + m takes level j of indices 16 hf + 2 m (X)
        // and 16 hf + 2 m + 1 (Y).  Past the last level the entries fall on
        // level full <= NLEV (position <= 16 NLEV <= 256, inside the table
        // rows): read, never used.
        if (full > 0)
          sweep(
              8 * full,
              [&](int st) {
                const uint32_t j = (uint32_t)(st >> 3) & 31u, m = (uint32_t)(st & 7);
                const uint32_t dx = 16u * hf + 2u * m, dy = dx + 1u;
                const uint32_t kj = UNI ? j : 16u * j;
                return ((dx << 10) | kj) | (((dy << 10) | kj) << 16);
              },
              item2);
        // The rest from the stage's list.
        if (n > 0) sweep(n, [&](int st) { return sched[2 * st]; }, item);
        if (blockIdx.x == 0 && tid == 0) issued += n + 8 * full;
      }
      const int cend = chunk_end(a, d0);
      if (CHUNKED && min(dn, dend) >= cend) {
        // Chunk complete: add each row's n0 sum, decode with the chunk scales.
        const int ch = d0 / a.chunk_d;
        const int cw = cend - ch * a.chunk_d;
        for (int r = tid; r < BM; r += 256) {
          const int row = s_rows[r];
          s_rc[r] = w.rowc[((long long)g * a.n_chunks + ch) * w.Mp + prow0 + r];
          s_sa[r] = row >= 0 ? a.sA[((long long)g * a.M + row) * a.n_chunks + ch] : 0.0f;
        }
        __syncthreads();
        float sb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wcol0 + j * 32 + l32;
          sb[j] = col < a.N ? a.sB[((long long)g * a.N + col) * a.n_chunks + ch] : 0.0f;
        }
        // Rows four at a time (accumulator entries v = 4 q .. 4 q + 3 are
        // consecutive rows), used by both column subtiles at once.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = wrow0 + i * 32 + q4 * 8 + hf * 4;
            const int4 rc = *(const int4*)&s_rc[r0];
            const float4 sa = *(const float4*)&s_sa[r0];
            const int rcv[4] = {rc.x, rc.y, rc.z, rc.w};
            const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
              for (int j = 0; j < 2; ++j) {
                const int v = q4 * 4 + e;
                const int cnt = (int)acc[i][j][v] + rcv[e];
                cacc[i][j][v] += (sav[e] * sb[j]) * (scaleL * (float)(UNI ? cnt : 2 * cnt - L * cw));
                if (COUNTS) bacc[i][j][v] += cnt;
                acc[i][j][v] = 0.0f;
              }
          }
        __syncthreads();  // s_rc / s_sa are rewritten at the next chunk
      }
      if (dn < dend) {
        store(buf ^ 1);
        __syncthreads();
        buf ^= 1;
      }
    }
    if (CHUNKED && COUNTS) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wcol0 + j * 32 + l32;
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = wrow0 + i * 32 + (v >> 2) * 8 + hf * 4 + (v & 3);
            const int row = s_rows[r];
            if (row >= 0 && col < a.N)
              a.counts[(((long long)g * a.M + row) * a.N + col) * a.n_bands + b] = bacc[i][j][v];
            bacc[i][j][v] = 0;
          }
        }
    }
    if (dend < a.D) buf ^= 1;  // the next band starts on the other buffer
  }
  if (blockIdx.x == 0 && tid == 0) atomicAdd(w.issued + 1, issued);  // fp4 steps

  if (!CHUNKED) {
    // Each row's n0 sum over the whole contraction axis: the parts' partial
    // sums, added once per row into LDS.
    for (int r = tid; r < BM; r += 256) {
      int tot = 0;
      const int32_t* rc0 = w.rowc + (long long)g * w.n_parts * w.Mp + prow0 + r;
      for (int pt = 0; pt < w.n_parts; ++pt) tot += rc0[(long long)pt * w.Mp];
      s_rc[r] = tot;
    }
    __syncthreads();
  }
  const int L0 = a.bandL[0][k];
  const float scale0 = (float)qq / (float)L0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = col0 + wcol0 + j * 32 + l32;
    const float sb = (!CHUNKED && col < a.N) ? a.sB[(long long)g * a.N + col] : 0.0f;
    const float bj = (a.bias && col < a.N) ? a.bias[(long long)g * a.N + col] : 0.0f;
    const int ccol = col < a.N ? out_col(a, col) : -1;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wrow0 + i * 32 + (v >> 2) * 8 + hf * 4 + (v & 3);
        const int row = s_rows[r];
        if (row < 0 || col >= a.N) continue;
        float out;
        if (CHUNKED) {
          out = cacc[i][j][v];
        } else {
          const int cnt = (int)acc[i][j][v] + s_rc[r];
          if (COUNTS) a.counts[((long long)g * a.M + row) * a.N + col] = cnt;
          const float sa = a.sA[(long long)g * a.M + row];
          out = (sa * sb) * (scale0 * (float)(UNI ? cnt : 2 * cnt - L0 * a.D));
        }
        if (a.C && ccol >= 0) a.C[(long long)g * a.bsc + (long long)row * a.ldc + ccol] = out + bj;
      }
  }
}

// ------------------------------------------------------- persistent ----
// The single-segment contraction (no chunk scales, one band) as a
// persistent kernel: each block takes 128 x 128 output tiles from a work
// counter, in rung order (which balances the rungs' different tile costs),
// so the paired table is staged again only when the rung changes, and the
// next tile's row data are read while the current tile is contracted (its
// output stores then drain behind the next tile's contraction).  Within a
// tile every wave reads its own row and column codes straight from the
// encode buffers into registers, one group of 32 contraction indices ahead,
// with no block-wide synchronisation.  Per group, the levels every index
// needs are swept from those registers; the remaining half-blocks go to a
// list in this wave's own part of LDS and are contracted, four per step,
// when the list fills and at the end, with their codes read from the
// index-major copies of the encode buffers a few steps ahead.
constexpr int FL_LIST = 512;  // list capacity per wave (half-blocks)
constexpr int FL_RING = 4;    // list steps whose codes are in flight

// Work item -> (rung k, group g, encode tile y, column tile x); items run
// rung by rung, then group, row tile, column tile.
struct PersItem {
  int k, g, y, x;
};
__device__ __forceinline__ PersItem pers_item(const MatmulArgs& a, int CT, int item) {
  PersItem it;
  int k = 0, base = 0;
  while (k + 1 < a.n_rungs) {
    const int n = (a.tile_start[k + 1] - a.tile_start[k]) * a.G * CT;
    if (item < base + n) break;
    base += n;
    ++k;
  }
  int r = item - base;
  const int tiles = a.tile_start[k + 1] - a.tile_start[k];
  it.k = k;
  it.x = r % CT;
  r /= CT;
  it.y = a.tile_start[k] + r % tiles;
  it.g = r / tiles;
  return it;
}

template <bool COUNTS>
__global__ void __launch_bounds__(256, COUNTS ? 1 : 2) k_mfma_pers(MatmulArgs a, MfmaWs w, int n_items) {
  struct __align__(16) GatherTables {
    uint8_t pt[MAX_LEVELS * PT_STRIDE];
    uint32_t pat[PAT_WORDS];
  };
  __shared__ GatherTables s_tab;
  __shared__ __align__(8) uint32_t s_list[4][FL_LIST];
  __shared__ __align__(16) int s_rows[2][MF_BM];    // original row of each position (-1: none)
  __shared__ __align__(16) int s_rc[2][MF_BM];      // each row's n0 sum over the contraction axis
  __shared__ __align__(16) float s_sa[2][MF_BM];    // each row's scale
  __shared__ int s_item[2];
  uint8_t* const s_pt = s_tab.pt;
  uint32_t* const s_pat = s_tab.pat;
  constexpr int PAD4 = 8 * FL_RING + 4;  // padding entries past a list's end

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wr = wave >> 1, wc = wave & 1;
  const int l32 = lane & 31, hf = lane >> 5;
  const int wrow0 = wr * 64, wcol0 = wc * 64;
  uint32_t* const list = s_list[wave];
  const int qq = a.q * a.q;

  // Row data of tile y in group g for position tid (< 128): original row,
  // n0 summed over the encode parts, row scale.
  auto row_data = [&](int g, int y, int& row, int& rc, float& sa) __attribute__((always_inline)) {
    const long long pos = (long long)g * w.Mp + (long long)y * MF_BM + tid;
    row = w.rowid[pos];
    sa = w.sas[pos];
    rc = 0;
    const int32_t* rc0 = w.rowc + (long long)g * w.n_parts * w.Mp + (long long)y * MF_BM + tid;
    for (int pt = 0; pt < w.n_parts; ++pt) rc += rc0[(long long)pt * w.Mp];
  };

  init_patterns(s_pat, tid, 256);
  if (tid == 0) {
    s_item[0] = (int)atomicAdd(w.work, 1u);
    s_item[1] = (int)atomicAdd(w.work, 1u);
  }
  __syncthreads();
  int item = s_item[0];
  if (item >= n_items) return;
  if (tid < MF_BM) {
    const PersItem it = pers_item(a, w.CT, item);
    int row, rc;
    float sa;
    row_data(it.g, it.y, row, rc, sa);
    s_rows[0][tid] = row;
    s_rc[0][tid] = rc;
    s_sa[0][tid] = sa;
  }

  const uint8_t* const pat = (const uint8_t*)s_pat;
  auto frags_at = [&](uint32_t hx, uint32_t ux, uint32_t kx, uint32_t hy, uint32_t uy, uint32_t ky)
                      __attribute__((always_inline)) { return scmp::frags_at(pat, s_pt, hx, ux, kx, hy, uy, ky); };
  v16f acc[2][2];
  auto mma = [&](const Frag& f) __attribute__((always_inline)) { mma_step(acc, f); };
  unsigned long long issued = 0;  // fp4 MFMA steps of the column-0 tiles
  int staged_k = -1;
  int cur = 0;

  while (true) {
    const PersItem it = pers_item(a, w.CT, item);
    const int k = tile_rung(a, it.g, it.k), g = it.g, y = it.y;
    const int col0 = it.x * MF_BN;
    const bool count_steps = it.x == 0;
    const int next = s_item[cur ^ 1];
    // The next tile's row data, read now and stored after this tile.
    int nrow = -1, nrc = 0;
    float nsa = 0.0f;
    if (next < n_items && tid < MF_BM) {
      const PersItem nt = pers_item(a, w.CT, next);
      row_data(nt.g, nt.y, nrow, nrc, nsa);
    }
    const int L = a.bandL[0][k];
    if (k != staged_k) {
      // Every wave finished the previous tile (the loop ends on a barrier).
      const int KLpad = ((((L + 1) >> 1) + 31) & ~31);
      stage_pair_table(s_pt, a, 0, k, KLpad, tid, 256);
      __syncthreads();
      staged_k = k;
    }

    // This lane's rows of the encode buffers (row pair wr * 32 + l32 of
    // tile y, column pair wc * 32 + l32 of column tile x), and the
    // index-major copies for list steps.
    const int ngrp_all = (int)(w.Dp / MF_DC);
    const uint32_t* hrow = w.hs + enc_word((long long)g * w.RT + y, ngrp_all, 0, 0) + (8 * wr + hf) * 128 + 4 * l32;
    const uint32_t* urow = w.ub + enc_word((long long)g * w.CT + it.x, ngrp_all, 0, 0) + (8 * wc + hf) * 128 + 4 * l32;
    const uint8_t* mq = w.maxh + ((long long)g * w.RT + y) * w.Dp;
    const uint32_t* hcol = w.hsi + (long long)g * w.Dp * (w.Mp / 2) + (long long)y * 64 + wr * 32 + l32;
    const uint32_t* ucol = w.ubi + (long long)g * w.Dp * (w.Np / 2) + (long long)it.x * 64 + wc * 32 + l32;
    const long long hstr = w.Mp / 2, ustr = w.Np / 2;
    auto hword = [&](uint32_t d) __attribute__((always_inline)) { return hcol[(long long)d * hstr]; };
    auto uword = [&](uint32_t d) __attribute__((always_inline)) { return ucol[(long long)d * ustr]; };

#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // Contract the wave's list of cnt half-blocks, four per step (lanes 0-31
    // take entries 4 s and 4 s + 1, lanes 32-63 entries 4 s + 2 and
    // 4 s + 3).  Slot r of the ring holds the entries and codes of a step
    // FL_RING steps ahead; its fragments are read one step ahead of its
    // MFMAs.  A list entry is (index << 4) | level; level 8 (position 128,
    // past every window) is the zero half-block used as padding, with dpad
    // (any index of the band) for its unused codes.
    auto list_sweep = [&](int cnt, int dpad) __attribute__((always_inline)) {
      if (lane < PAD4) list[cnt + lane] = ((uint32_t)dpad << 4) | 8u;
      const int nsteps = (cnt + 3) >> 2;
      uint2 re[FL_RING];
      uint32_t rhx[FL_RING], rux[FL_RING], rhy[FL_RING], ruy[FL_RING];
      auto fill = [&](int r, uint2 e) __attribute__((always_inline)) {
        re[r] = e;
        rhx[r] = hword(e.x >> 4);
        rux[r] = uword(e.x >> 4);
        rhy[r] = hword(e.y >> 4);
        ruy[r] = uword(e.y >> 4);
      };
      auto frags_r = [&](int r) __attribute__((always_inline)) {
        return frags_at(rhx[r], rux[r], 16u * (re[r].x & 15u), rhy[r], ruy[r], 16u * (re[r].y & 15u));
      };
      const uint2* lst = (const uint2*)list;  // entry pairs
#pragma unroll
      for (int r = 0; r < FL_RING; ++r) fill(r, lst[2 * r + hf]);
      uint2 enext = lst[2 * FL_RING + hf];
      Frag fr[2];
      fr[0] = frags_r(0);
      for (int s0 = 0; s0 < nsteps; s0 += FL_RING) {
#pragma unroll
        for (int r = 0; r < FL_RING; ++r) {
          fr[(r + 1) & 1] = frags_r((r + 1) % FL_RING);
          fill(r, enext);  // slot r now serves step s0 + r + FL_RING
          enext = lst[2 * (s0 + r + FL_RING + 1) + hf];
          __builtin_amdgcn_sched_barrier(0);
          if (s0 + r < nsteps) mma(fr[r & 1]);
        }
      }
      if (count_steps) issued += nsteps;
    };

    const int dbeg = a.band_cols[0], dend = a.band_cols[1];
    const int ngrp = (dend - dbeg + 31) / 32;
    // A group's loads: the codes of indices d0 + 16 hf + m, m < 16 (four
    // 16-byte loads per buffer), and this lane's index maximum (raw: the
    // band's bound is applied where it is used).
    auto load_group = [&](int d0, uint32_t* h, uint32_t* u, int& m) __attribute__((always_inline)) {
      const uint4* hp = (const uint4*)(hrow + ((long long)(d0 >> 5) << 11));
      const uint4* up = (const uint4*)(urow + ((long long)(d0 >> 5) << 11));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 th = hp[64 * i], tu = up[64 * i];
        h[4 * i] = th.x;
        h[4 * i + 1] = th.y;
        h[4 * i + 2] = th.z;
        h[4 * i + 3] = th.w;
        u[4 * i] = tu.x;
        u[4 * i + 1] = tu.y;
        u[4 * i + 2] = tu.z;
        u[4 * i + 3] = tu.w;
      }
      m = mq[d0 + l32];  // d0 + l32 < Dp
    };
    int cnt = 0;  // entries in this wave's list
    // fa: the fragments of the group's first step, read at the end of the
    // previous group.
    Frag fa;
    // One group: its codes (ch, cu) and this lane's index maximum (mx) are
    // in registers; nh, nu: the next group's codes.  A full level takes 8
    // steps: step m pairs indices d0 + 16 hf + m (X) and d0 + 16 hf + 8 + m
    // (Y) in lane half hf.
    auto group = [&](int grp, const uint32_t* ch, const uint32_t* cu, int mx, const uint32_t* nh,
                     const uint32_t* nu) __attribute__((always_inline)) {
      const int d0 = dbeg + 32 * grp;
      const int nl = d0 + l32 < dend ? (mx + 15) >> 4 : 0;
      int full = 0;
      for (int j = 0; j < 8; ++j) {
        const unsigned bal = (unsigned)__ballot(nl > j);
        if (bal == 0) break;
        if (bal == 0xffffffffu && j == full) {
          ++full;
          continue;
        }
        if (hf == 0 && nl > j)
          list[cnt + (int)__builtin_amdgcn_mbcnt_lo(bal, 0u)] = ((uint32_t)(d0 + l32) << 4) | (uint32_t)j;
        cnt += __builtin_popcount(bal);
      }
      if (full > 0) {
        Frag fb;
        for (int j = 0; j < full; ++j) {
          const uint32_t kk = 16u * j;
#pragma unroll
          for (int m = 0; m < 8; m += 2) {
            fb = frags_at(ch[m + 1], cu[m + 1], kk, ch[m + 9], cu[m + 9], kk);
            __builtin_amdgcn_sched_barrier(0);  // keep these reads ahead of the MFMAs
            mma(fa);
            // Next: step m + 2 of this level or step 0 of the next level
            // (after the last level: read, unused; position <= 128 stays
            // inside the table rows).
            if (m + 2 < 8)
              fa = frags_at(ch[m + 2], cu[m + 2], kk, ch[m + 10], cu[m + 10], kk);
            else
              fa = frags_at(ch[0], cu[0], kk + 16u, ch[8], cu[8], kk + 16u);
            __builtin_amdgcn_sched_barrier(0);
            mma(fb);
          }
        }
        if (count_steps) issued += 8 * full;
      }
      // The next group adds at most 256 entries.
      if (cnt > FL_LIST - 256 - PAD4 || (grp == ngrp - 1 && cnt > 0)) {
        list_sweep(cnt, d0);
        cnt = 0;
      }
      // The next group's first step.
      fa = frags_at(nh[0], nu[0], 0u, nh[8], nu[8], 0u);
    };
    if (ngrp > 0) {
      uint32_t ha[16], ua[16], hb[16], ub[16];
      int ma, mb = 0;
      load_group(dbeg, ha, ua, ma);
      fa = frags_at(ha[0], ua[0], 0u, ha[8], ua[8], 0u);
      for (int grp = 0; grp < ngrp; grp += 2) {
        load_group(dbeg + 32 * min(grp + 1, ngrp - 1), hb, ub, mb);
        group(grp, ha, ua, ma, hb, ub);
        if (grp + 1 >= ngrp) break;
        load_group(dbeg + 32 * min(grp + 2, ngrp - 1), ha, ua, ma);
        group(grp + 1, hb, ub, mb, ha, ua);
      }
    }

    // The next tile's row data into the other buffer; the tile after it.
    if (tid < MF_BM) {
      s_rows[cur ^ 1][tid] = nrow;
      s_rc[cur ^ 1][tid] = nrc;
      s_sa[cur ^ 1][tid] = nsa;
    }
    if (tid == 0) s_item[cur] = next < n_items ? (int)atomicAdd(w.work, 1u) : n_items;

    // Decode: rows four at a time (accumulator entries v = 4 q .. 4 q + 3
    // are consecutive rows), each used by both column subtiles.
    const float scale0 = (float)qq / (float)L;
    float sb[2], bj[2];
    int ccol[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = col0 + wcol0 + j * 32 + l32;
      sb[j] = col < a.N ? a.sB[(long long)g * a.N + col] : 0.0f;
      bj[j] = (a.bias && col < a.N) ? a.bias[(long long)g * a.N + col] : 0.0f;
      ccol[j] = col < a.N ? out_col(a, col) : -1;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int r0 = wrow0 + i * 32 + q4 * 8 + hf * 4;
        const int4 rw = *(const int4*)&s_rows[cur][r0];
        const int4 rc = *(const int4*)&s_rc[cur][r0];
        const float4 sa = *(const float4*)&s_sa[cur][r0];
        const int rowv[4] = {rw.x, rw.y, rw.z, rw.w};
        const int rcv[4] = {rc.x, rc.y, rc.z, rc.w};
        const float sav[4] = {sa.x, sa.y, sa.z, sa.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int col = col0 + wcol0 + j * 32 + l32;
            if (rowv[e] < 0 || col >= a.N) continue;
            const int cnt2 = (int)acc[i][j][q4 * 4 + e] + rcv[e];
            if (COUNTS) a.counts[((long long)g * a.M + rowv[e]) * a.N + col] = cnt2;
            if (a.C && ccol[j] >= 0)
              a.C[(long long)g * a.bsc + (long long)rowv[e] * a.ldc + ccol[j]] =
                  (sav[e] * sb[j]) * (scale0 * (float)(2 * cnt2 - L * a.D)) + bj[j];
          }
      }
    __syncthreads();  // publishes the next tile's row data and item
    if (next >= n_items) break;
    item = next;
    cur ^= 1;
  }
  if (tid == 0 && issued) atomicAdd(w.issued + 1, issued);
}

int mfma_issued_macs(const MatmulArgs& a, const void* ws, size_t ws_bytes, hipStream_t st,
                     unsigned long long* macs, unsigned long long* fp4_macs) {
  size_t need = 0;
  MfmaWs w = ws_layout(a, (void*)ws, &need);
  if (!ws || ws_bytes < need)
    return set_error(SCMP_ERR_WORKSPACE, "workspace smaller than scmp_matmul_workspace_bytes reports");
  unsigned long long steps[2] = {0, 0};
  hipError_t e = hipMemcpyAsync(steps, w.issued, sizeof steps, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("work readback: ") + hipGetErrorString(e));
  // A step of a 128 x 128 tile is four MFMAs per wave (2 x 2 subtiles of
  // 32 x 32), four waves: 128 * 128 * K MACs with K = 32 (int8) or 64
  // (fp4), issued by each column tile.
  const unsigned long long per8 = (unsigned long long)w.CT * 128ull * 128ull * 32ull;
  *macs = steps[0] * per8 + steps[1] * 2 * per8;
  if (fp4_macs) *fp4_macs = steps[1] * 2 * per8;
  return SCMP_OK;
}

size_t mfma_workspace_bytes(const MatmulArgs& a) {
  size_t total = 0;
  ws_layout(a, nullptr, &total);
  return total;
}

// The persistent kernel handles one band starting on a 32-index boundary
// and an int item count.
static bool pers_ok(const MatmulArgs& a, const MfmaWs& w) {
  if (a.chunk_d > 0 || a.n_bands != 1 || a.band_cols[0] % MF_DC != 0) return false;
  return (double)a.tile_start[a.n_rungs] * a.G * w.CT < 2147483647.0;
}

// Compute units of the current device (cached per device).
static int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

static void launch_main(const MatmulArgs& a, const MfmaWs& w, dim3 grid, hipStream_t st) {
  const bool counts = a.counts != nullptr;
  if (a.unipolar) {
    // Unipolar plans: the staged kernel with prefixes of up to 16 half-blocks.
    if (a.chunk_d > 0) {
      if (counts)
        hipLaunchKernelGGL((k_mfma<true, true, true>), grid, dim3(256), 0, st, a, w);
      else
        hipLaunchKernelGGL((k_mfma<true, false, true>), grid, dim3(256), 0, st, a, w);
    } else if (counts) {
      hipLaunchKernelGGL((k_mfma<false, true, true>), grid, dim3(256), 0, st, a, w);
    } else {
      hipLaunchKernelGGL((k_mfma<false, false, true>), grid, dim3(256), 0, st, a, w);
    }
  } else if (a.chunk_d > 0) {
    if (counts)
      hipLaunchKernelGGL((k_mfma<true, true, false>), grid, dim3(256), 0, st, a, w);
    else
      hipLaunchKernelGGL((k_mfma<true, false, false>), grid, dim3(256), 0, st, a, w);
  } else if (a.launch == 1 ||
             (a.launch == 0 && pers_ok(a, w) &&
              a.tile_start[a.n_rungs] * a.G * w.CT >= 2 * (counts ? 1 : 2) * device_cus())) {
    // Persistent when every block gets at least two tiles (the table is
    // then staged once for several); a one-pass grid otherwise (its blocks
    // need no work counter or table reuse).
    const int n_items = a.tile_start[a.n_rungs] * a.G * w.CT;
    const int blocks = std::max(1, std::min(n_items, (counts ? 1 : 2) * device_cus()));
    if (counts)
      hipLaunchKernelGGL((k_mfma_pers<true>), dim3(blocks), dim3(256), 0, st, a, w, n_items);
    else
      hipLaunchKernelGGL((k_mfma_pers<false>), dim3(blocks), dim3(256), 0, st, a, w, n_items);
  } else {
    if (counts)
      hipLaunchKernelGGL((k_mfma<false, true, false>), grid, dim3(256), 0, st, a, w);
    else
      hipLaunchKernelGGL((k_mfma<false, false, false>), grid, dim3(256), 0, st, a, w);
  }
}

int launch_mfma(const MatmulArgs& a0, void* ws, size_t ws_bytes, hipStream_t st) {
  size_t need = 0;
  MatmulArgs a = a0;
  MfmaWs w = ws_layout(a, ws, &need);
  if (!ws || ws_bytes < need)
    return set_error(SCMP_ERR_WORKSPACE, "workspace smaller than scmp_matmul_workspace_bytes reports");
  if (w.RT == 0) return SCMP_OK;
  if (w.RT > 65535 || w.CT > 65535 || w.n_parts > 65535)
    return set_error(SCMP_ERR_ARG, "too many tiles");
  if (a.launch == 1 && !pers_ok(a, w))
    return set_error(SCMP_ERR_UNSUPPORTED,
                     "the persistent launch needs a plan without chunk scales and one band");
  hipLaunchKernelGGL(k_prep, dim3(w.RT + w.CT, w.n_parts, a.G), dim3(256), 0, st, a, w);
  launch_main(a, w, dim3(w.CT, w.RT, a.G), st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("mfma launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}

}  // namespace scmp
