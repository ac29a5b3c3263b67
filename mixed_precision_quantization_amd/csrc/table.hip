// K1: device-resident Sobol cumulative indicator table.
//
// "Precision As You Need" paper notes, Key design 1: a Sobol-8 table
// K[b, l] = 1[r_l <= b] is generated once at layer load, stays resident in
// device memory and is sliced by prefix for any stream length.  Here row
// u = b + 1 (u in [0, P]) holds K[u][l] = 1[r_l < u], packed 32 positions
// per word.  Sobol points are the unscrambled 1-D sequence in Gray-code
// order: r_l = bitreverse_p(l XOR (l >> 1)).
//
// Besides K and its prefix sums cum[u][n], the table holds, for every
// length L <= Lmax, the paired-position table the matrix-core contraction
// reads: with lo(k) = ceil(L/2) - 1 - k and hi(k) = floor(L/2) + k,
// pair_L[u][k] = K[u][lo(k)] + K[u][hi(k)] (only K[u][lo(k)] when the two
// coincide, the centre of an odd L), for k < ceil(L/2), zero-padded to a
// multiple of 32.  An A stream's XNOR window is symmetric about L/2, so the
// contraction only needs these sums (see matmul.hip).

#include <hip/hip_runtime.h>

#include <new>
#include <vector>

#include "internal.h"
#include "table.h"

namespace scmp {

__device__ __forceinline__ int sobol_point(int l, int p) {
  unsigned g = (unsigned)(l ^ (l >> 1));
  return (int)(__builtin_bitreverse32(g) >> (32 - p));
}

// One block per level u; one thread per stream position (padded to a whole
// number of waves).
__global__ void k_table_bits(int p, int Lmax, int Wl, uint16_t* __restrict__ r,
                             uint32_t* __restrict__ K) {
  const int u = blockIdx.x;
  for (int base = 0; base < Wl * 32; base += blockDim.x) {
    const int l = base + threadIdx.x;
    bool bit = false;
    if (l < Lmax) {
      const int rl = sobol_point(l, p);
      bit = rl < u;
      if (u == 0) r[l] = (uint16_t)rl;
    }
    const unsigned long long m = __ballot(bit);
    const int lane = threadIdx.x & 63;
    const int w0 = l >> 5;  // word of this lane
    if (lane == 0 && w0 < Wl) K[(size_t)u * Wl + w0] = (uint32_t)(m & 0xffffffffull);
    if (lane == 32 && w0 < Wl) K[(size_t)u * Wl + w0] = (uint32_t)(m >> 32);
  }
}

// cum[u][n] = number of set bits among K[u][0..n).
__global__ void k_table_cum(int Lmax, int Wl, const uint32_t* __restrict__ K,
                            uint16_t* __restrict__ cum) {
  const int u = blockIdx.x;
  const uint32_t* row = K + (size_t)u * Wl;
  for (int n = threadIdx.x; n <= Lmax; n += blockDim.x) {
    int c = 0;
    const int full = n >> 5;
    for (int w = 0; w < full; ++w) c += __popc(row[w]);
    const int rem = n & 31;
    if (rem) c += __popc(row[full] & ((1u << rem) - 1u));
    cum[(size_t)u * (Lmax + 1) + n] = (uint16_t)c;
  }
}

__device__ __forceinline__ int kbit(const uint32_t* row, int l) { return (row[l >> 5] >> (l & 31)) & 1; }

// blockIdx.x = L - 1; the block fills pair_L for every level.
__global__ void k_table_pair(int P, int Wl, const uint32_t* __restrict__ K,
                             const unsigned long long* __restrict__ off,
                             uint8_t* __restrict__ pair) {
  const int L = blockIdx.x + 1;
  const int KL = (L + 1) >> 1;
  const int KLpad = (KL + 31) & ~31;
  uint8_t* base = pair + off[L];
  const int lo0 = KL - 1;
  const int hi0 = L >> 1;
  for (int idx = threadIdx.x; idx < (P + 1) * KLpad; idx += blockDim.x) {
    const int u = idx / KLpad;
    const int k = idx - u * KLpad;
    int v = 0;
    if (k < KL) {
      const uint32_t* row = K + (size_t)u * Wl;
      const int lo = lo0 - k, hi = hi0 + k;
      v = kbit(row, lo) + (lo != hi ? kbit(row, hi) : 0);
    }
    base[idx] = (uint8_t)v;
  }
}

}  // namespace scmp

using scmp::set_error;

extern "C" {

int scmp_build_sobol_table(int p, int Lmax, void* stream, scmp_table_t* out) {
  scmp::clear_error();
  if (!out) return set_error(SCMP_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (p < 2 || p > 8) return set_error(SCMP_ERR_ARG, "p must be in [2, 8]");
  if (Lmax < 1 || Lmax > (1 << p)) return set_error(SCMP_ERR_ARG, "Lmax must be in [1, 2^p]");
  hipStream_t st = (hipStream_t)stream;
  scmp_table_s* t = new (std::nothrow) scmp_table_s;
  if (!t) return set_error(SCMP_ERR_ARG, "out of host memory");
  t->p = p;
  t->Lmax = Lmax;
  t->P = 1 << p;
  t->Wl = (Lmax + 31) / 32;
  t->pair_off.assign(Lmax + 1, 0);
  unsigned long long acc = 0;
  for (int L = 1; L <= Lmax; ++L) {
    t->pair_off[L] = acc;
    const int KL = (L + 1) / 2;
    acc += (unsigned long long)(t->P + 1) * ((KL + 31) & ~31);
  }
  t->pair_bytes = acc;
  const size_t rb = sizeof(uint16_t) * Lmax;
  const size_t kb = sizeof(uint32_t) * (size_t)(t->P + 1) * t->Wl;
  const size_t cb = sizeof(uint16_t) * (size_t)(t->P + 1) * (Lmax + 1);
  const size_t ob = sizeof(unsigned long long) * (Lmax + 1);
  hipError_t e = hipSuccess;
  e = hipGetDevice(&t->device);
  if (e == hipSuccess) e = hipMalloc((void**)&t->r, rb);
  if (e == hipSuccess) e = hipMalloc((void**)&t->K, kb);
  if (e == hipSuccess) e = hipMalloc((void**)&t->cum, cb);
  if (e == hipSuccess) e = hipMalloc((void**)&t->pair, t->pair_bytes);
  if (e == hipSuccess) e = hipMalloc((void**)&t->pair_off_dev, ob);
  if (e == hipSuccess)
    e = hipMemcpyAsync(t->pair_off_dev, t->pair_off.data(), ob, hipMemcpyHostToDevice, st);
  if (e != hipSuccess) {
    scmp_table_destroy(t);
    return set_error(SCMP_ERR_HIP, std::string("table allocation: ") + hipGetErrorString(e));
  }
  const int threads = ((t->Wl * 32 + 63) / 64) * 64;
  hipLaunchKernelGGL(scmp::k_table_bits, dim3(t->P + 1), dim3(threads < 1024 ? threads : 1024), 0, st, p,
                     Lmax, t->Wl, t->r, t->K);
  hipLaunchKernelGGL(scmp::k_table_cum, dim3(t->P + 1), dim3(256), 0, st, Lmax, t->Wl, t->K, t->cum);
  hipLaunchKernelGGL(scmp::k_table_pair, dim3(Lmax), dim3(256), 0, st, t->P, t->Wl, t->K, t->pair_off_dev,
                     t->pair);
  e = hipGetLastError();
  if (e == hipSuccess) e = hipStreamSynchronize(st);  // one-time build; the host offsets must outlive it
  if (e != hipSuccess) {
    scmp_table_destroy(t);
    return set_error(SCMP_ERR_HIP, std::string("table build: ") + hipGetErrorString(e));
  }
  *out = t;
  return SCMP_OK;
}

int scmp_table_destroy(scmp_table_t t) {
  if (!t) return SCMP_OK;
  (void)hipDeviceSynchronize();
  if (t->r) (void)hipFree(t->r);
  if (t->K) (void)hipFree(t->K);
  if (t->cum) (void)hipFree(t->cum);
  if (t->pair) (void)hipFree(t->pair);
  if (t->pair_off_dev) (void)hipFree(t->pair_off_dev);
  delete t;
  return SCMP_OK;
}

int scmp_table_info(scmp_table_t t, int* p, int* Lmax) {
  if (!t) return set_error(SCMP_ERR_ARG, "table is NULL");
  if (p) *p = t->p;
  if (Lmax) *Lmax = t->Lmax;
  return SCMP_OK;
}

int scmp_table_export(scmp_table_t t, uint16_t* r_dev, uint32_t* K_dev, uint16_t* cum_dev, void* stream) {
  scmp::clear_error();
  if (!t) return set_error(SCMP_ERR_ARG, "table is NULL");
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (r_dev) e = hipMemcpyAsync(r_dev, t->r, sizeof(uint16_t) * t->Lmax, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && K_dev)
    e = hipMemcpyAsync(K_dev, t->K, sizeof(uint32_t) * (size_t)(t->P + 1) * t->Wl, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && cum_dev)
    e = hipMemcpyAsync(cum_dev, t->cum, sizeof(uint16_t) * (size_t)(t->P + 1) * (t->Lmax + 1),
                       hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return set_error(SCMP_ERR_HIP, std::string("table export: ") + hipGetErrorString(e));
  return SCMP_OK;
}

}  // extern "C"
