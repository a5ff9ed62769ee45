// Base Batch Shuffling: the batch former ahead of the jagged attention path
// (piletech.kr/articles/112134, section 핵심 포인트 / Key points, BBS bullet,
// and section 상세 정리 / Detailed notes, Base Batch Shuffling item: base
// sub-batches of 128 samples are sorted by sequence length and the heaviest
// is merged with the lightest in turn, which evens out the load of the
// batches different GPUs or steps get, with no exchange between ranks).
//
// Host code over host arrays: the sample lengths are known to the data
// loader before anything is copied to the device.  See include/jfa.h for
// the contract.
#include <algorithm>
#include <cstdint>
#include <numeric>
#include <vector>

#include "jfa.h"
#include "jfa_internal.h"

extern "C" int64_t jfa_bbs_batch_count(int64_t n_samples, int32_t base_batch) {
  if (n_samples < 0 || base_batch < 1) return 0;
  const int64_t bases = (n_samples + base_batch - 1) / base_batch;
  return (bases + 1) / 2;
}

extern "C" int jfa_bbs_plan(const int32_t* lengths, int64_t n_samples, int32_t base_batch, int32_t cost,
                            int64_t* perm, int64_t* batch_start) {
  if (n_samples < 0) return jfa::report(JFA_ERR_INVALID_ARGUMENT, "n_samples < 0");
  if (base_batch < 1) return jfa::report(JFA_ERR_INVALID_ARGUMENT, "base_batch < 1");
  if (cost != JFA_BBS_COST_TOKENS && cost != JFA_BBS_COST_PAIRS)
    return jfa::report(JFA_ERR_INVALID_ARGUMENT, "bad cost");
  if (n_samples > 0 && (!lengths || !perm)) return jfa::report(JFA_ERR_INVALID_ARGUMENT, "NULL lengths or perm");
  if (!batch_start) return jfa::report(JFA_ERR_INVALID_ARGUMENT, "NULL batch_start");
  const int64_t nb = (n_samples + base_batch - 1) / base_batch;
  // load of every base batch (consecutive runs of base_batch samples)
  std::vector<int64_t> load(nb, 0);
  for (int64_t i = 0; i < n_samples; ++i) {
    const int64_t x = lengths[i];
    if (x < 0) return jfa::report(JFA_ERR_INVALID_ARGUMENT, "negative length");
    load[i / base_batch] += cost == JFA_BBS_COST_PAIRS ? x * x : x;
  }
  // heaviest first, ties by base-batch index
  std::vector<int64_t> order(nb);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return load[a] > load[b]; });
  int64_t pos = 0, g = 0;
  auto put = [&](int64_t k) {
    const int64_t s = k * base_batch, e = std::min<int64_t>(s + base_batch, n_samples);
    for (int64_t i = s; i < e; ++i) perm[pos++] = i;
  };
  batch_start[0] = 0;
  for (int64_t i = 0; i < nb / 2; ++i) {   // k-th heaviest with k-th lightest
    put(order[i]);
    put(order[nb - 1 - i]);
    batch_start[++g] = pos;
  }
  if (nb % 2) {   // the median base batch alone, last
    put(order[nb / 2]);
    batch_start[++g] = pos;
  }
  return JFA_OK;
}
