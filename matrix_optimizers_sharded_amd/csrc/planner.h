// Owner planner: which rank owns which whole matrix.
//
// "Riassunto Tecnico: MatrixFSDP", Metodologia, the MatrixShard metadata / global
// planner item: a global planner assigns the owners so as to balance resident bytes
// and optimizer work across the ranks.  The page gives no algorithm.  This one is
// the longest-processing-time rule on the owner's Newton-Schulz work: matrices in
// decreasing order of work, each to the rank with the least work so far (ties: the
// fewest resident bytes, then the lowest rank).  The rule's makespan is within
// 4/3 - 1/(3R) of the optimum for R ranks.  Host code only.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <numeric>
#include <vector>

namespace mo {

// Algorithmic Newton-Schulz flops of one matrix: iters * (m^2 n [X X^T, one
// triangle] + m^3 [A^2, symmetric] + 2 m^2 n [B X]), m = min(r, c), n = max(r, c).
inline double ns_work(int64_t rows, int64_t cols, int iters) {
  const double m = static_cast<double>(std::min(rows, cols));
  const double n = static_cast<double>(std::max(rows, cols));
  return static_cast<double>(iters) * (3.0 * m * m * n + m * m * m);
}

// owner[i] in [0, ranks); rank_work / rank_bytes (nullable) get the per-rank totals.
inline void plan_owners(const int64_t* rows, const int64_t* cols, int count, int ranks, int iters,
                        double bytes_per_element, int32_t* owner, double* rank_work, double* rank_bytes) {
  std::vector<double> work(count), bytes(count);
  for (int i = 0; i < count; ++i) {
    work[i] = ns_work(rows[i], cols[i], iters);
    bytes[i] = static_cast<double>(rows[i]) * static_cast<double>(cols[i]) * bytes_per_element;
  }
  std::vector<int> order(count);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int p, int q) {
    if (work[p] != work[q]) return work[p] > work[q];
    return bytes[p] > bytes[q];
  });
  std::vector<double> lw(ranks, 0.0), lb(ranks, 0.0);
  for (int i : order) {
    int best = 0;
    for (int r = 1; r < ranks; ++r)
      if (lw[r] < lw[best] || (lw[r] == lw[best] && lb[r] < lb[best])) best = r;
    owner[i] = best;
    lw[best] += work[i];
    lb[best] += bytes[i];
  }
  for (int r = 0; r < ranks; ++r) {
    if (rank_work) rank_work[r] = lw[r];
    if (rank_bytes) rank_bytes[r] = lb[r];
  }
}

}  // namespace mo
