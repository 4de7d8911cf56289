// Padding rows of a padded layout.  Each expert segment of the receive buffer
// is padded to a multiple of the handle's pad_multiple; the rows after the
// expert's pairs hold zeros, with a zero score (the zero-sentinel scores of
// the padded permute on the torchtitan page, "Implementation").  A grouped
// GEMM over the padded segments then reads zeros, and its weight gradient
// gets nothing from them.
//
// The fill is not a launch of its own: the kernel that writes a call's
// receive rows adds pad_fill_waves(E, pad, NV) wavefronts to its grid, and
// each of them runs pad_fill_wave.  The scatter puts them after its token
// waves, where they overlap its drain; the staged expansion puts them first,
// because the end of its grid is send-row waves past N_send that exit at once
// (its grid is sized for the worst case), behind which the fill would run
// alone.  The padding rows and the pair rows are disjoint, so the two
// kinds of wave never touch the same row.  One fill wave per (expert, block of
// kPadRows padding rows, segment of 64 chunks): it stores one zero chunk per
// lane and row of its block, and the wave of segment 0 also clears the
// block's scores, one row per lane.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace moe {

// Wave w of the fill (0 <= w < pad_fill_waves(E, pad, NV); waves past the
// last expert return at once).
__device__ __forceinline__ void pad_fill_wave(const PadArgs& a, int w) {
  const int lane = lane_id();
  const int per_e = a.nblk * a.ngrp;  // waves per expert
  const int e = w / per_e;
  if (e >= a.E) return;  // wave-uniform
  const int rem = w - e * per_e;
  const int rb = rem / a.ngrp;
  const int grp = rem - rb * a.ngrp;
  const int seg_end = min(a.expert_offset[e + 1], a.R);  // never past the buffer
  const int lo = max(a.expert_offset[e] + a.num_tokens_per_expert[e], 0) + rb * kPadRows;
  const int hi = min(lo + kPadRows, seg_end);
  const int j = grp * kWave + lane;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4* dst = static_cast<u32x4*>(a.dst);
  if (j < a.NV) {
#pragma unroll
    for (int i = 0; i < kPadRows; ++i)
      if (lo + i < hi) store_chunk<true>(dst + (size_t)(lo + i) * a.NV + j, zero);
  }
  if (grp == 0 && a.scores_out && lane < kPadRows && lo + lane < hi) a.scores_out[lo + lane] = 0.f;
}

}  // namespace moe
