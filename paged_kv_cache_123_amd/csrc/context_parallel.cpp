// Host helper of context parallelism ([CSDN] section 2.3): how many of a
// sequence's positions one rank stores.
//
// With W ranks, block size B and interleave I, a table entry names a virtual
// block of B * W positions, cut into runs of I positions dealt to the ranks in
// turn (run k goes to rank k mod W).  Every full virtual block gives each rank
// exactly B positions; the last, partial one of r = L mod (B * W) positions
// holds c = r div I whole runs and a run of r mod I positions, run c.
#include <cstdint>

#include "pagedkv.h"
#include "status.h"

extern "C" int32_t pa_cp_local_context_lens(const int32_t* context_lens, int32_t num_seqs,
                                            int32_t block_size, int32_t cp_world,
                                            int32_t cp_rank, int32_t interleave,
                                            int32_t* local_lens) {
  if (!context_lens || !local_lens || num_seqs < 0 || block_size < 1)
    return pa::fail(PA_EINVAL, "pa_cp_local_context_lens: bad argument");
  if (cp_world < 1 || cp_rank < 0 || cp_rank >= cp_world)
    return pa::fail(PA_EINVAL, "pa_cp_local_context_lens: need 0 <= cp_rank < cp_world");
  if (interleave < 1 || block_size % interleave != 0)
    return pa::fail(PA_EINVAL, "pa_cp_local_context_lens: interleave must divide block_size");
  const int64_t vbs = static_cast<int64_t>(block_size) * cp_world;
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens[s];
    if (L < 0) return pa::fail(PA_EINVAL, "pa_cp_local_context_lens: negative length");
    const int64_t r = L % vbs;
    const int64_t runs = r / interleave, part = r % interleave;
    const int64_t turn = runs % cp_world;  // the rank the partial run goes to
    int64_t n = (L / vbs) * block_size + (runs / cp_world) * interleave;
    if (turn > cp_rank) n += interleave;
    else if (turn == cp_rank) n += part;
    local_lens[s] = static_cast<int32_t>(n);
  }
  return PA_OK;
}
