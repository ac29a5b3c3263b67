// Internal declarations shared by the libscmp translation units.
#pragma once

#include <cstdint>
#include <string>

#include "scmp.h"

namespace scmp {

// Plan: everything one SC matmul needs, resolved on the host at creation.
struct Plan {
  int op = 0, p = 8, Lmax = 256, D = 0, chunk_d = 0, n_chunks = 1;
  int n_rungs = 1, n_bands = 1, ceiling = 256;
  int mode = SCMP_MODE_BIPOLAR;
  int range_mp = 0, range_group = 128;  // range-based per-weight-group MP
  float range_threshold = 0.0f;
  int levels[SCMP_MAX_RUNGS] = {};
  double fractions[SCMP_MAX_RUNGS] = {};
  int band_chunks[SCMP_MAX_BANDS] = {};
  int band_cols[SCMP_MAX_BANDS + 1] = {};
  int band_L[SCMP_MAX_BANDS][SCMP_MAX_RUNGS] = {};
  double budget[SCMP_MAX_RUNGS] = {};
};

// Sorted-position cuts for M rows: cuts[0] = 0 .. cuts[n_rungs] = M.
void row_cuts(const Plan& plan, int M, int* cuts);

int set_error(int status, const std::string& msg);
void clear_error();

inline int qmax(int p) { return (1 << (p - 1)) - 1; }

}  // namespace scmp

struct scmp_plan_s {
  scmp::Plan plan;
};
