// Padding rows of a padded layout.  Each expert segment of the receive buffer
// is padded to a multiple of the handle's pad_multiple; the rows after the
// expert's pairs hold zeros, with a zero score (the zero-sentinel scores of
// the padded permute on the torchtitan page, "Implementation").  A grouped
// GEMM over the padded segments then reads zeros, and its weight gradient
// gets nothing from them.
//
// One wavefront per (expert, block of kPadRows padding rows, segment of 64
// chunks): it stores one zero chunk per lane and row of its block, so a
// segment's padding is written by many waves at once.  The wave of segment 0
// also clears the block's scores, one row per lane.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kPadRows = 8;  // padding rows per wave

__global__ __launch_bounds__(512) void pad_fill_kernel(PadArgs a) {
  const int lane = lane_id();
  const int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int per_e = a.nblk * a.ngrp;  // waves per expert
  const int e = gw / per_e;
  if (e >= a.E) return;  // wave-uniform
  const int rem = gw - e * per_e;
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

}  // namespace

int64_t pad_fill_waves(int E, int pad, int NV) {
  // an expert has at most pad-1 padding rows
  return (int64_t)E * ((pad - 1 + kPadRows - 1) / kPadRows) * ((NV + kWave - 1) / kWave);
}

hipError_t launch_pad_fill(const PadArgs& a0, const Tuning& t, hipStream_t s) {
  PadArgs a = a0;
  a.ngrp = (a.NV + kWave - 1) / kWave;
  a.nblk = (a.pad - 1 + kPadRows - 1) / kPadRows;
  const int wpb = t.waves_per_block;
  const int64_t waves = pad_fill_waves(a.E, a.pad, a.NV);
  hipLaunchKernelGGL(pad_fill_kernel, dim3((unsigned)((waves + wpb - 1) / wpb)), dim3(wpb * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
