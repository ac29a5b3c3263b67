// Host-side plan logic: validation ("startup" guards), the K-band ladder and
// the row cuts of the mixed-precision rungs.
//
// Sources: "Precision As You Need" paper notes, Key design 2 (length ladder,
// descending thresholds); scmp_vit README, MP flag table (levels descending,
// one fraction per level, empty = equal split); K-band pull request
// "How the banding works", "Guards" and "Tooling" (L[b][k] per band and
// rung, iso-compute identity never overspent, straight-line tilt rounded
// down with units handed back largest-lost-fraction first, rungs at the
// ceiling untilted, the four startup rejections).

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "internal.h"

namespace scmp {

namespace {
thread_local std::string g_last_error;
}

int set_error(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

void clear_error() { g_last_error.clear(); }

void row_cuts(const Plan& plan, int M, int* cuts) {
  cuts[0] = 0;
  double F = 0.0;
  for (int k = 0; k < plan.n_rungs; ++k) {
    F = F + plan.fractions[k];
    long long c = (k == plan.n_rungs - 1) ? M : (long long)std::floor(F * (double)M + 0.5);
    if (c > M) c = M;
    if (c < cuts[k]) c = cuts[k];
    cuts[k + 1] = (int)c;
  }
}

namespace {

// Straight-line tilt for one rung over B equal-width bands.
void tilt_rung(int Lk, int B, double t, int* out) {
  std::vector<double> raw(B);
  std::vector<int> fl(B);
  long long sum = 0;
  for (int b = 0; b < B; ++b) {
    double x_b = (2.0 * b - (B - 1)) / (double)(B - 1);
    raw[b] = Lk * (1.0 + t * x_b);
    fl[b] = (int)std::floor(raw[b]);
    sum += fl[b];
  }
  long long give = (long long)B * Lk - sum;
  std::vector<int> order(B);
  for (int b = 0; b < B; ++b) order[b] = b;
  std::stable_sort(order.begin(), order.end(), [&](int a, int c) {
    double fa = raw[a] - fl[a], fc = raw[c] - fl[c];
    if (fa != fc) return fa > fc;
    return a < c;
  });
  for (long long i = 0; i < give && i < B; ++i) fl[order[i]] += 1;
  for (int b = 0; b < B; ++b) out[b] = fl[b];
}

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

int build_plan(const scmp_plan_desc* d, Plan& P) {
  if (!d) return set_error(SCMP_ERR_ARG, "plan description is NULL");
  if (d->op < SCMP_OP_LINEAR || d->op > SCMP_OP_AV) return set_error(SCMP_ERR_ARG, "unknown op kind");
  if (d->mode != SCMP_MODE_BIPOLAR && d->mode != SCMP_MODE_UNIPOLAR) return set_error(SCMP_ERR_ARG, "unknown mode");
  if (d->p < 2 || d->p > 8) return set_error(SCMP_ERR_ARG, fmt("p=%lld outside [2, 8]", d->p));
  if (d->Lmax < 1 || d->Lmax > (1 << d->p))
    return set_error(SCMP_ERR_ARG, fmt("Lmax=%lld outside [1, 2^p]", d->Lmax));
  if (d->D < 1) return set_error(SCMP_ERR_ARG, "D must be >= 1");
  if (d->chunk_d < 0) return set_error(SCMP_ERR_ARG, "chunk_d must be >= 0");
  if (d->n_rungs < 1 || d->n_rungs > SCMP_MAX_RUNGS)
    return set_error(SCMP_ERR_ARG, fmt("n_rungs=%lld outside [1, %lld]", d->n_rungs, SCMP_MAX_RUNGS));
  if (!d->levels) return set_error(SCMP_ERR_ARG, "levels is NULL");
  if (d->n_bands < 1 || d->n_bands > SCMP_MAX_BANDS)
    return set_error(SCMP_ERR_ARG, fmt("n_bands=%lld outside [1, %lld]", d->n_bands, SCMP_MAX_BANDS));
  int ceiling = d->ceiling == 0 ? d->Lmax : d->ceiling;
  if (ceiling < 1 || ceiling > d->Lmax)
    return set_error(SCMP_ERR_ARG, fmt("ceiling=%lld outside [1, Lmax=%lld]", ceiling, d->Lmax));

  // [KBAND] "Guards": range MP has no contraction-axis dispatch.
  if (d->range_mp && d->n_bands > 1)
    return set_error(SCMP_ERR_UNSUPPORTED, "K-bands cannot be combined with range-based MP");
  if (d->range_mp) {
    // Weight groups exist only where there are weights (linear ops).
    if (d->op != SCMP_OP_LINEAR) return set_error(SCMP_ERR_UNSUPPORTED, "range-based MP needs a linear op");
    if (d->n_rungs != 2) return set_error(SCMP_ERR_ARG, "range-based MP takes two levels");
    if (d->range_group < 0) return set_error(SCMP_ERR_ARG, "range_group must be >= 0");
    if (!std::isfinite(d->range_threshold) || d->range_threshold < 0.0)
      return set_error(SCMP_ERR_ARG, "range_threshold must be finite and >= 0");
  }
  // [KBAND] "Guards": qk / av contract over the head dimension, no band dispatch.
  if (d->n_bands > 1 && d->op != SCMP_OP_LINEAR)
    return set_error(SCMP_ERR_UNSUPPORTED, "K-bands are only defined for linear ops (not qk/av)");

  P.op = d->op;
  P.mode = d->mode;
  P.range_mp = d->range_mp ? 1 : 0;
  P.range_group = d->range_group > 0 ? d->range_group : 128;
  P.range_threshold = (float)d->range_threshold;
  P.p = d->p;
  P.Lmax = d->Lmax;
  P.D = d->D;
  P.chunk_d = d->chunk_d;
  P.n_chunks = d->chunk_d > 0 ? (d->D + d->chunk_d - 1) / d->chunk_d : 1;
  P.n_rungs = d->n_rungs;
  P.n_bands = d->n_bands;
  P.ceiling = ceiling;
  if (d->chunk_d > 0 && d->chunk_d % 32 != 0)
    return set_error(SCMP_ERR_UNSUPPORTED, fmt("chunk_d=%lld must be a multiple of 32", d->chunk_d));

  for (int k = 0; k < d->n_rungs; ++k) {
    int L = d->levels[k];
    if (L < 1) return set_error(SCMP_ERR_ARG, fmt("level %lld is %lld (< 1)", k, L));
    if (k > 0 && L >= d->levels[k - 1])
      return set_error(SCMP_ERR_ARG, "levels must be strictly descending");
    if (L > ceiling)
      return set_error(SCMP_ERR_CEILING, fmt("level %lld = %lld above the ceiling %lld", k, L, ceiling));
    P.levels[k] = L;
  }
  if (d->fractions) {
    double s = 0.0;
    for (int k = 0; k < d->n_rungs; ++k) {
      double f = d->fractions[k];
      if (!(f >= 0.0) || !std::isfinite(f)) return set_error(SCMP_ERR_ARG, "fractions must be finite and >= 0");
      P.fractions[k] = f;
      s += f;
    }
    if (std::fabs(s - 1.0) > 1e-6) return set_error(SCMP_ERR_ARG, "fractions must sum to 1");
  } else {
    for (int k = 0; k < d->n_rungs; ++k) P.fractions[k] = 1.0 / d->n_rungs;
  }

  // Bands of whole chunks.
  if (d->n_bands > 1) {
    if (d->chunk_d <= 0) return set_error(SCMP_ERR_ARG, "K-bands need chunk_d > 0");
    if (d->band_L && ((d->table_chunk_d != 0 && d->table_chunk_d != d->chunk_d) ||
                      (d->table_D != 0 && d->table_D != d->D)))
      return set_error(SCMP_ERR_PLAN_MISMATCH,
                       fmt("band table priced at chunk_d=%lld, D=%lld does not match this op", d->table_chunk_d,
                           d->table_D));
  }
  long long total = 0;
  for (int b = 0; b < d->n_bands; ++b) {
    int w;
    if (d->band_chunks) {
      w = d->band_chunks[b];
    } else {
      if (P.n_chunks % d->n_bands != 0)
        return set_error(SCMP_ERR_ARG, "an equal band split needs n_chunks divisible by n_bands");
      w = P.n_chunks / d->n_bands;
    }
    if (w < 1) return set_error(SCMP_ERR_ARG, "every band needs at least one chunk");
    P.band_chunks[b] = w;
    total += w;
  }
  if (total != P.n_chunks) return set_error(SCMP_ERR_ARG, "band widths must cover every chunk exactly");
  P.band_cols[0] = 0;
  {
    long long c = 0;
    for (int b = 0; b < d->n_bands; ++b) {
      c += P.band_chunks[b];
      long long col = d->n_bands == 1 ? d->D : c * (long long)(d->chunk_d > 0 ? d->chunk_d : d->D);
      P.band_cols[b + 1] = (int)std::min<long long>(col, d->D);
    }
  }

  // Band lengths.
  if (d->band_L) {
    for (int b = 0; b < d->n_bands; ++b)
      for (int k = 0; k < d->n_rungs; ++k) P.band_L[b][k] = d->band_L[b * d->n_rungs + k];
  } else if (d->n_bands == 1) {
    for (int k = 0; k < d->n_rungs; ++k) P.band_L[0][k] = P.levels[k];
  } else {
    for (int b = 1; b < d->n_bands; ++b)
      if (P.band_cols[b + 1] - P.band_cols[b] != P.band_cols[1] - P.band_cols[0])
        return set_error(SCMP_ERR_ARG, "the straight-line tilt needs bands of equal column width");
    for (int k = 0; k < d->n_rungs; ++k) {
      int col[SCMP_MAX_BANDS];
      if (P.levels[k] >= ceiling) {
        for (int b = 0; b < d->n_bands; ++b) col[b] = P.levels[k];
      } else {
        tilt_rung(P.levels[k], d->n_bands, d->tilt, col);
      }
      for (int b = 0; b < d->n_bands; ++b) P.band_L[b][k] = col[b];
    }
  }
  for (int b = 0; b < d->n_bands; ++b)
    for (int k = 0; k < d->n_rungs; ++k) {
      int L = P.band_L[b][k];
      if (L > ceiling)
        return set_error(SCMP_ERR_CEILING,
                         fmt("band %lld rung %lld length %lld above the ceiling", b, k, L));
      if (L < 1) return set_error(SCMP_ERR_ARG, fmt("band %lld rung %lld length %lld below 1", b, k, L));
    }
  // Per-rung iso-compute identity: never overspent.
  for (int k = 0; k < d->n_rungs; ++k) {
    long long spent = 0;
    for (int b = 0; b < d->n_bands; ++b)
      spent += (long long)(P.band_cols[b + 1] - P.band_cols[b]) * P.band_L[b][k];
    long long budget = (long long)d->D * P.levels[k];
    if (spent > budget)
      return set_error(SCMP_ERR_ISO_COMPUTE,
                       fmt("rung %lld spends %lld bit-positions, budget %lld", k, spent, budget));
    P.budget[k] = (double)spent / (double)budget;
  }
  return SCMP_OK;
}

}  // namespace
bool mfma_counts_exact(const Plan& P) {
  int maxL = 0;
  for (int b = 0; b < P.n_bands; ++b)
    for (int k = 0; k < P.n_rungs; ++k) maxL = P.band_L[b][k] > maxL ? P.band_L[b][k] : maxL;
  const long long seg = (P.chunk_d > 0 && P.chunk_d < P.D) ? P.chunk_d : P.D;
  return seg * (long long)(maxL + 1) < (1LL << 24);
}

}  // namespace scmp

using scmp::set_error;

extern "C" {

const char* scmp_status_string(int status) {
  switch (status) {
    case SCMP_OK: return "SCMP_OK";
    case SCMP_ERR_ARG: return "SCMP_ERR_ARG";
    case SCMP_ERR_CEILING: return "SCMP_ERR_CEILING";
    case SCMP_ERR_ISO_COMPUTE: return "SCMP_ERR_ISO_COMPUTE";
    case SCMP_ERR_UNSUPPORTED: return "SCMP_ERR_UNSUPPORTED";
    case SCMP_ERR_PLAN_MISMATCH: return "SCMP_ERR_PLAN_MISMATCH";
    case SCMP_ERR_NONFINITE: return "SCMP_ERR_NONFINITE";
    case SCMP_ERR_WORKSPACE: return "SCMP_ERR_WORKSPACE";
    case SCMP_ERR_HIP: return "SCMP_ERR_HIP";
    default: return "SCMP_ERR_UNKNOWN";
  }
}

const char* scmp_last_error(void) { return scmp::g_last_error.c_str(); }

int scmp_plan_create(const scmp_plan_desc* desc, scmp_plan_t* out) {
  scmp::clear_error();
  if (!out) return set_error(SCMP_ERR_ARG, "out is NULL");
  *out = nullptr;
  scmp::Plan P;
  int st = scmp::build_plan(desc, P);
  if (st != SCMP_OK) return st;
  scmp_plan_s* h = new (std::nothrow) scmp_plan_s;
  if (!h) return set_error(SCMP_ERR_ARG, "out of host memory");
  h->plan = P;
  *out = h;
  return SCMP_OK;
}

int scmp_plan_destroy(scmp_plan_t plan) {
  delete plan;
  return SCMP_OK;
}

int scmp_plan_query(scmp_plan_t plan, scmp_plan_info* out) {
  if (!plan || !out) return set_error(SCMP_ERR_ARG, "NULL argument");
  const scmp::Plan& P = plan->plan;
  out->op = P.op;
  out->p = P.p;
  out->Lmax = P.Lmax;
  out->D = P.D;
  out->chunk_d = P.chunk_d;
  out->n_chunks = P.n_chunks;
  out->n_rungs = P.n_rungs;
  out->n_bands = P.n_bands;
  out->ceiling = P.ceiling;
  out->mode = P.mode;
  out->range_mp = P.range_mp;
  out->range_group = P.range_group;
  out->mfma_exact = scmp::mfma_counts_exact(P) ? 1 : 0;
  return SCMP_OK;
}

int scmp_plan_band_lengths(scmp_plan_t plan, int* L_out) {
  if (!plan || !L_out) return set_error(SCMP_ERR_ARG, "NULL argument");
  const scmp::Plan& P = plan->plan;
  for (int b = 0; b < P.n_bands; ++b)
    for (int k = 0; k < P.n_rungs; ++k) L_out[b * P.n_rungs + k] = P.band_L[b][k];
  return SCMP_OK;
}

int scmp_plan_band_columns(scmp_plan_t plan, int* cols_out) {
  if (!plan || !cols_out) return set_error(SCMP_ERR_ARG, "NULL argument");
  for (int b = 0; b <= plan->plan.n_bands; ++b) cols_out[b] = plan->plan.band_cols[b];
  return SCMP_OK;
}

int scmp_plan_budget_use(scmp_plan_t plan, double* use_out) {
  if (!plan || !use_out) return set_error(SCMP_ERR_ARG, "NULL argument");
  for (int k = 0; k < plan->plan.n_rungs; ++k) use_out[k] = plan->plan.budget[k];
  return SCMP_OK;
}

int scmp_plan_row_cuts(scmp_plan_t plan, int M, int* cuts_out) {
  if (!plan || !cuts_out) return set_error(SCMP_ERR_ARG, "NULL argument");
  if (M < 0) return set_error(SCMP_ERR_ARG, "M must be >= 0");
  scmp::row_cuts(plan->plan, M, cuts_out);
  return SCMP_OK;
}

}  // extern "C"
