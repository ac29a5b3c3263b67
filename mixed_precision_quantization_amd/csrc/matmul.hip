// The C-ABI entry points of the contraction (scmp_matmul and its workspace
// query), the standalone decode, and the device error flags.
//
// "Precision As You Need" paper notes, Key design 1 (C-BSG, decode
// equation) and Key design 3 (per-row early termination); K-band pull
// request, "How the banding works".  The two contraction kernels live in
// mfma.hip (matrix cores, default) and bitserial.hip (vector ALU).

#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "matmul_common.h"
#include "table.h"

namespace scmp {

// Scratch memory of scmp_matmul_noalloc: one array per device that runs the
// library, held until the process ends.  Host code never passes the array's
// name to a kernel; it uses the device address taken once per device below.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
__device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, taken on the first
// call on that device (with it current) and kept per device.
static int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[64] = {nullptr};
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= 64) return set_error(SCMP_ERR_ARG, "device ordinal above 63");
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(SCMP_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return SCMP_OK;
}

void fill_tiles(MatmulArgs& a, const Plan& P, int BM) {
  row_cuts(P, a.M, a.cuts);
  a.tile_start[0] = 0;
  for (int k = 0; k < P.n_rungs; ++k)
    a.tile_start[k + 1] = a.tile_start[k] + (a.cuts[k + 1] - a.cuts[k] + BM - 1) / BM;
}

// Validate the arguments and fill MatmulArgs (no device work).
static int prepare(scmp_table_t table, scmp_plan_t plan, int& algo, int G, int M, int N, MatmulArgs& a) {
  if (!table || !plan) return set_error(SCMP_ERR_ARG, "table or plan is NULL");
  const Plan& P = plan->plan;
  if (table->p != P.p || table->Lmax != P.Lmax)
    return set_error(SCMP_ERR_PLAN_MISMATCH, "table p / Lmax differ from the plan");
  if (algo < SCMP_ALGO_AUTO || algo > SCMP_ALGO_MFMA_QUARTER) return set_error(SCMP_ERR_ARG, "unknown algo");
  if (P.mode == SCMP_MODE_UNIPOLAR &&
      (algo == SCMP_ALGO_MFMA_PERSISTENT || algo == SCMP_ALGO_GATHER || algo == SCMP_ALGO_MFMA_QUARTER))
    return set_error(SCMP_ERR_UNSUPPORTED, "unipolar plans have no persistent, quarter or gather form");
  if (G < 0 || M < 0 || N < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if (G > 65535) return set_error(SCMP_ERR_ARG, "G must be <= 65535");
  if (table->P + 1 > MAX_LEVELS) return set_error(SCMP_ERR_ARG, "table has too many levels");
  a = MatmulArgs{};
  a.pair = table->pair;
  a.K = table->K;
  a.cum = table->cum;
  a.G = G;
  a.M = M;
  a.N = N;
  a.D = P.D;
  a.chunk_d = P.chunk_d;
  a.n_chunks = P.n_chunks;
  a.n_rungs = P.n_rungs;
  a.n_ladder = P.n_rungs;
  a.unipolar = P.mode == SCMP_MODE_UNIPOLAR;
  a.n_bands = P.n_bands;
  a.q = qmax(P.p);
  a.P = 1 << P.p;
  a.Wl = table->Wl;
  a.Lmax = table->Lmax;
  // Segments too long for exact float32 accumulation leave AUTO to an
  // integer path and reject the matrix-core forms (mfma_counts_exact).
  if ((algo == SCMP_ALGO_AUTO || algo == SCMP_ALGO_MFMA || algo == SCMP_ALGO_MFMA_PERSISTENT ||
       algo == SCMP_ALGO_MFMA_ONEPASS || algo == SCMP_ALGO_MFMA_QUARTER) && !mfma_counts_exact(P)) {
    if (algo != SCMP_ALGO_AUTO)
      return set_error(SCMP_ERR_UNSUPPORTED,
                       "the matrix-core accumulators hold counts exactly only while the accumulation segment "
                       "(D, or chunk_d) times (longest L + 1) stays below 2^24; use BITSERIAL or GATHER");
    algo = P.mode == SCMP_MODE_UNIPOLAR ? SCMP_ALGO_BITSERIAL : SCMP_ALGO_GATHER;
  }
  a.launch = algo == SCMP_ALGO_MFMA_PERSISTENT ? 1
             : algo == SCMP_ALGO_MFMA_ONEPASS   ? 2
             : algo == SCMP_ALGO_MFMA_QUARTER   ? 3
                                                : 0;
  a.auto_quarter = algo == SCMP_ALGO_AUTO ? 1 : 0;
  const bool bitserial = algo == SCMP_ALGO_BITSERIAL;
  fill_tiles(a, P, bitserial ? 64 : 128);
  for (int b = 0; b <= P.n_bands; ++b) a.band_cols[b] = P.band_cols[b];
  for (int b = 0; b < P.n_bands; ++b)
    for (int k = 0; k < P.n_rungs; ++k) {
      a.bandL[b][k] = P.band_L[b][k];
      a.pair_off[b][k] = table->pair_off[P.band_L[b][k]];
    }
  return SCMP_OK;
}

// One tiling rung over every group's rows in original order, for per-group
// lengths (the rung of each tile comes from group_rung).
static void group_tiling(MatmulArgs& a, int algo) {
  const int BM = algo == SCMP_ALGO_BITSERIAL ? 64 : 128;
  a.n_rungs = 1;
  a.cuts[0] = 0;
  a.cuts[1] = a.M;
  a.tile_start[0] = 0;
  a.tile_start[1] = (a.M + BM - 1) / BM;
}

// ---------------------------------------------------------------- decode ----

struct DecodeArgs {
  const int32_t* counts;
  const float* sA;
  const float* sB;
  const uint8_t* rung;
  float* C;
  long long ldc, bsc;
  int M, N, D, q, n_rungs, unipolar;
  int L[SCMP_MAX_RUNGS];
};

__global__ void __launch_bounds__(256) k_decode(DecodeArgs a) {
  const int g = blockIdx.z, i = blockIdx.y;
  const int j = blockIdx.x * 256 + threadIdx.x;
  if (j >= a.N) return;
  int k = a.rung ? (int)a.rung[(long long)g * a.M + i] : 0;
  k = k < a.n_rungs ? k : a.n_rungs - 1;
  const int L = a.L[k];
  const int cnt = a.counts[((long long)g * a.M + i) * a.N + j];
  const float sa = a.sA[(long long)g * a.M + i];
  const float sb = a.sB[(long long)g * a.N + j];
  const float scaleL = (float)(a.q * a.q) / (float)L;
  a.C[(long long)g * a.bsc + (long long)i * a.ldc + j] =
      (sa * sb) * (scaleL * (float)(a.unipolar ? cnt : 2 * cnt - L * a.D));
}

}  // namespace scmp

using scmp::set_error;

extern "C" {

int scmp_matmul_workspace_bytes(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                                size_t* bytes) {
  scmp::clear_error();
  if (!bytes) return set_error(SCMP_ERR_ARG, "bytes is NULL");
  *bytes = 0;
  scmp::MatmulArgs a;
  int st = scmp::prepare(table, plan, algo, G, M, N, a);
  if (st != SCMP_OK) return st;
  if (algo == SCMP_ALGO_BITSERIAL || (long long)G * M * N == 0) return SCMP_OK;
  if (algo == SCMP_ALGO_GATHER) {
    *bytes = scmp::gather_workspace_bytes(a);
    return SCMP_OK;
  }
  // Enough for both tilings: rows bucketed by rung, or each group's rows in
  // order (scmp_matmul_group_rungs).
  const size_t by_rung = scmp::mfma_workspace_bytes(a);
  scmp::group_tiling(a, algo);
  const size_t by_group = scmp::mfma_workspace_bytes(a);
  *bytes = by_rung > by_group ? by_rung : by_group;
  return SCMP_OK;
}

}  // extern "C"

// The variants of the contraction beyond scmp_matmul's arguments.
struct Variant {
  const float* bias = nullptr;          // added to every row of C
  const uint8_t* group_rung = nullptr;  // one rung per group
  int range_level = -1;                 // range MP: every row at this level
  const int32_t* cmap = nullptr;        // range MP: C column of each compact column
};

static int matmul_impl(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N, const int8_t* qA,
                       const float* sA, const int32_t* permA, const int8_t* qB, const uint32_t* packedB,
                       const float* sB, const Variant& v, int32_t* counts, float* C, int64_t ldc,
                       int64_t batch_stride_c, void* workspace, size_t workspace_bytes, void* stream) {
  scmp::clear_error();
  const float* bias = v.bias;
  const uint8_t* group_rung = v.group_rung;
  scmp::MatmulArgs a;
  int st0 = scmp::prepare(table, plan, algo, G, M, N, a);
  if (st0 != SCMP_OK) return st0;
  const scmp::Plan& P = plan->plan;
  if (P.range_mp != (v.range_level >= 0))
    return set_error(SCMP_ERR_UNSUPPORTED, P.range_mp ? "range-MP plans run through scmp_matmul_range"
                                                      : "scmp_matmul_range needs a range-MP plan");
  if ((long long)G * M * N == 0) return SCMP_OK;
  if (!qA || !sA || !qB || !sB) return set_error(SCMP_ERR_ARG, "qA, sA, qB and sB are required");
  if (!counts && !C) return set_error(SCMP_ERR_ARG, "at least one of counts and C is required");
  if (C && ldc < N) return set_error(SCMP_ERR_ARG, "ldc must be >= N");
  if (v.range_level >= 0) {
    // Range MP: every row at the level's length, C columns through cmap.
    if (v.range_level >= P.n_rungs) return set_error(SCMP_ERR_ARG, "level must be 0 or 1");
    if (!v.cmap) return set_error(SCMP_ERR_ARG, "cols is required");
    scmp::group_tiling(a, algo);
    for (int b = 0; b < P.n_bands; ++b) {
      a.bandL[b][0] = P.band_L[b][v.range_level];
      a.pair_off[b][0] = table->pair_off[P.band_L[b][v.range_level]];
    }
    a.n_ladder = 1;
    a.cmap = v.cmap;
    permA = nullptr;
  } else if (group_rung) {
    a.group_rung = group_rung;
    scmp::group_tiling(a, algo);
    permA = nullptr;
  } else if (P.n_rungs > 1 && !permA) {
    return set_error(SCMP_ERR_ARG, "mixed precision needs the row permutation");
  }
  const bool bitserial = algo == SCMP_ALGO_BITSERIAL;
  if (bitserial && !packedB) return set_error(SCMP_ERR_ARG, "the bit-serial kernel needs packed B streams");
  a.qA = qA;
  a.sA = sA;
  a.perm = permA;
  a.qB = qB;
  a.packedB = packedB;
  a.sB = sB;
  a.counts = counts;
  a.C = C;
  a.bias = bias;
  a.ldc = ldc;
  a.bsc = batch_stride_c;
  hipStream_t st = (hipStream_t)stream;
  if (bitserial) return scmp::launch_bitserial(a, st);
  if (algo == SCMP_ALGO_GATHER) return scmp::launch_gather(a, workspace, workspace_bytes, st);
  return scmp::launch_mfma(a, workspace, workspace_bytes, st);
}

extern "C" {

int scmp_matmul(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N, const int8_t* qA,
                const float* sA, const int32_t* permA, const int8_t* qB, const uint32_t* packedB,
                const float* sB, int32_t* counts, float* C, int64_t ldc, int64_t batch_stride_c,
                void* workspace, size_t workspace_bytes, void* stream) {
  return matmul_impl(table, plan, algo, G, M, N, qA, sA, permA, qB, packedB, sB, Variant{}, counts, C, ldc,
                     batch_stride_c, workspace, workspace_bytes, stream);
}

int scmp_matmul_noalloc(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N, const int8_t* qA,
                        const float* sA, const int32_t* permA, const int8_t* qB, const uint32_t* packedB,
                        const float* sB, int32_t* counts, float* C, int64_t ldc, int64_t batch_stride_c,
                        void* stream) {
  scmp::clear_error();
  size_t need = 0;
  int st = scmp_matmul_workspace_bytes(table, plan, algo, G, M, N, &need);
  if (st != SCMP_OK) return st;
  if (need > scmp::NOALLOC_SCRATCH_BYTES)
    return set_error(SCMP_ERR_WORKSPACE, "scmp_matmul_noalloc: these sizes need " + std::to_string(need) +
                                             " bytes of scratch, above its 64 MiB maximum; use scmp_matmul "
                                             "with a caller workspace");
  void* ws = nullptr;
  if (need > 0) {
    st = scmp::scratch_address(&ws);
    if (st != SCMP_OK) return st;
  }
  return matmul_impl(table, plan, algo, G, M, N, qA, sA, permA, qB, packedB, sB, Variant{}, counts, C, ldc,
                     batch_stride_c, ws, need > 0 ? scmp::NOALLOC_SCRATCH_BYTES : 0, stream);
}

int scmp_matmul_group_rungs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const int8_t* qA, const float* sA, const int8_t* qB, const uint32_t* packedB,
                            const float* sB, const uint8_t* group_rung, int32_t* counts, float* C, int64_t ldc,
                            int64_t batch_stride_c, void* workspace, size_t workspace_bytes, void* stream) {
  if (!group_rung) {
    scmp::clear_error();
    return set_error(SCMP_ERR_ARG, "group_rung is NULL (use scmp_matmul)");
  }
  Variant v;
  v.group_rung = group_rung;
  return matmul_impl(table, plan, algo, G, M, N, qA, sA, nullptr, qB, packedB, sB, v, counts, C, ldc,
                     batch_stride_c, workspace, workspace_bytes, stream);
}

int scmp_matmul_range(scmp_table_t table, scmp_plan_t plan, int algo, int level, int G, int M, int N,
                      const int8_t* qA, const float* sA, const int8_t* qB, const uint32_t* packedB,
                      const float* sB, const int32_t* cols, int32_t* counts, float* C, int64_t ldc,
                      int64_t batch_stride_c, void* workspace, size_t workspace_bytes, void* stream) {
  if (level < 0 || level > 1) {
    scmp::clear_error();
    return set_error(SCMP_ERR_ARG, "level must be 0 or 1");
  }
  Variant v;
  v.range_level = level;
  v.cmap = cols;
  return matmul_impl(table, plan, algo, G, M, N, qA, sA, nullptr, qB, packedB, sB, v, counts, C, ldc,
                     batch_stride_c, workspace, workspace_bytes, stream);
}

int scmp_matmul_bias(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N, const int8_t* qA,
                     const float* sA, const int32_t* permA, const int8_t* qB, const uint32_t* packedB,
                     const float* sB, const float* bias, int32_t* counts, float* C, int64_t ldc,
                     int64_t batch_stride_c, void* workspace, size_t workspace_bytes, void* stream) {
  if (!bias) {
    scmp::clear_error();
    return set_error(SCMP_ERR_ARG, "bias is NULL (use scmp_matmul)");
  }
  Variant v;
  v.bias = bias;
  return matmul_impl(table, plan, algo, G, M, N, qA, sA, permA, qB, packedB, sB, v, counts, C, ldc,
                     batch_stride_c, workspace, workspace_bytes, stream);
}

int scmp_matmul_issued_macs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const void* workspace, size_t workspace_bytes, unsigned long long* macs,
                            unsigned long long* fp4_macs, void* stream) {
  scmp::clear_error();
  if (!macs) return set_error(SCMP_ERR_ARG, "macs is NULL");
  *macs = 0;
  if (fp4_macs) *fp4_macs = 0;
  scmp::MatmulArgs a;
  int st0 = scmp::prepare(table, plan, algo, G, M, N, a);
  if (st0 != SCMP_OK) return st0;
  if (algo == SCMP_ALGO_BITSERIAL || algo == SCMP_ALGO_GATHER)
    return set_error(SCMP_ERR_UNSUPPORTED, "only the MFMA path counts its steps");
  if ((long long)G * M * N == 0) return SCMP_OK;
  return scmp::mfma_issued_macs(a, workspace, workspace_bytes, (hipStream_t)stream, macs, fp4_macs);
}

int scmp_matmul_window_macs(scmp_table_t table, scmp_plan_t plan, int algo, int G, int M, int N,
                            const void* workspace, size_t workspace_bytes, unsigned long long* macs,
                            void* stream) {
  scmp::clear_error();
  if (!macs) return set_error(SCMP_ERR_ARG, "macs is NULL");
  *macs = 0;
  scmp::MatmulArgs a;
  int st0 = scmp::prepare(table, plan, algo, G, M, N, a);
  if (st0 != SCMP_OK) return st0;
  if (algo == SCMP_ALGO_BITSERIAL || algo == SCMP_ALGO_GATHER)
    return set_error(SCMP_ERR_UNSUPPORTED, "only the MFMA path records its windows");
  if ((long long)G * M * N == 0) return SCMP_OK;
  return scmp::mfma_window_macs(a, workspace, workspace_bytes, (hipStream_t)stream, macs);
}

int scmp_decode(scmp_plan_t plan, int G, int M, int N, const int32_t* counts, const float* sA, const float* sB,
                const uint8_t* rung, float* C, int64_t ldc, int64_t batch_stride_c, void* stream) {
  scmp::clear_error();
  if (!plan) return set_error(SCMP_ERR_ARG, "plan is NULL");
  const scmp::Plan& P = plan->plan;
  if (P.chunk_d > 0 || P.n_bands > 1)
    return set_error(SCMP_ERR_UNSUPPORTED, "chunk scales are decoded inside scmp_matmul");
  if (G < 0 || M < 0 || N < 0) return set_error(SCMP_ERR_ARG, "negative size");
  if ((long long)G * M * N == 0) return SCMP_OK;
  if (!counts || !sA || !sB || !C) return set_error(SCMP_ERR_ARG, "counts, sA, sB and C are required");
  if (P.n_rungs > 1 && !rung) return set_error(SCMP_ERR_ARG, "mixed precision needs the rungs");
  if (ldc < N) return set_error(SCMP_ERR_ARG, "ldc must be >= N");
  if (G > 65535 || M > 65535) return set_error(SCMP_ERR_ARG, "G and M must be <= 65535");
  scmp::DecodeArgs a;
  a.counts = counts;
  a.sA = sA;
  a.sB = sB;
  a.rung = rung;
  a.C = C;
  a.ldc = ldc;
  a.bsc = batch_stride_c;
  a.M = M;
  a.N = N;
  a.D = P.D;
  a.q = scmp::qmax(P.p);
  a.n_rungs = P.n_rungs;
  a.unipolar = P.mode == SCMP_MODE_UNIPOLAR;
  for (int k = 0; k < P.n_rungs; ++k) a.L[k] = P.band_L[0][k];
  hipLaunchKernelGGL(scmp::k_decode, dim3((N + 255) / 256, M, G), dim3(256), 0, (hipStream_t)stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("decode launch: ") + hipGetErrorString(e));
  return SCMP_OK;
}

int scmp_error_flags(void* stream, int* flags_out) {
  scmp::clear_error();
  if (!flags_out) return set_error(SCMP_ERR_ARG, "flags_out is NULL");
  *flags_out = 0;
  hipStream_t st = (hipStream_t)stream;
  int s = scmp::read_clear_stream_flags(st, flags_out);
  if (s != SCMP_OK) return s;
  return (*flags_out & 1) ? SCMP_ERR_NONFINITE : SCMP_OK;
}

}  // extern "C"
