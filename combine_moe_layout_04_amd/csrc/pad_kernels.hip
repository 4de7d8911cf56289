// Padding rows of a padded layout.  Each expert segment of the receive buffer
// is padded to a multiple of the handle's pad_multiple; the rows after the
// expert's pairs hold zeros, with a zero score (the zero-sentinel scores of
// the padded permute on the torchtitan page, "Implementation").  A grouped
// GEMM over the padded segments then reads zeros, and its weight gradient
// gets nothing from them.
//
// One wavefront per (expert, segment of 64 chunks): it walks the expert's
// padding rows, storing one zero chunk per lane and row.  The wave of segment
// 0 also clears the scores, one row per lane.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(512) void pad_fill_kernel(PadArgs a) {
  const int lane = lane_id();
  const int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int e = gw / a.ngrp;
  if (e >= a.E) return;  // wave-uniform
  const int grp = gw - e * a.ngrp;
  const int lo = a.expert_offset[e] + a.num_tokens_per_expert[e];
  const int hi = min(a.expert_offset[e + 1], a.R);  // never past the buffer
  const int j = grp * kWave + lane;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4* dst = static_cast<u32x4*>(a.dst);
  if (j < a.NV) {
    for (int p = max(lo, 0); p < hi; ++p) store_chunk<true>(dst + (size_t)p * a.NV + j, zero);
  }
  if (grp == 0 && a.scores_out) {
    for (int p = max(lo, 0) + lane; p < hi; p += kWave) a.scores_out[p] = 0.f;
  }
}

}  // namespace

hipError_t launch_pad_fill(const PadArgs& a0, const Tuning& t, hipStream_t s) {
  PadArgs a = a0;
  a.ngrp = (a.NV + kWave - 1) / kWave;
  const int wpb = t.waves_per_block;
  const int64_t waves = (int64_t)a.E * a.ngrp;
  hipLaunchKernelGGL(pad_fill_kernel, dim3((unsigned)((waves + wpb - 1) / wpb)), dim3(wpb * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
