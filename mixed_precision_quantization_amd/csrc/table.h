// The table object behind scmp_table_t (device buffers owned by the library).
#pragma once

#include <cstdint>
#include <vector>

struct scmp_table_s {
  int p = 8, Lmax = 256, P = 256, Wl = 8, device = 0;
  uint16_t* r = nullptr;       // [Lmax] Sobol points
  uint32_t* K = nullptr;       // [P + 1][Wl] packed indicator rows
  uint16_t* cum = nullptr;     // [P + 1][Lmax + 1] prefix sums
  uint8_t* pair = nullptr;     // paired-position tables, one block per L
  unsigned long long* pair_off_dev = nullptr;  // [Lmax + 1] byte offsets of each L's block
  std::vector<unsigned long long> pair_off;    // host copy
  unsigned long long pair_bytes = 0;
};
