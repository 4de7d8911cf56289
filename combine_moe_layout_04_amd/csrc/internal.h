// Internal interface between the C ABI (abi.hip) and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

constexpr int kLayoutThreads = 512;  // threads per layout workgroup

// Workspace sections (byte offsets from the workspace base, 256-aligned).
struct WsLayout {
  size_t status, num_tokens_per_expert, num_tokens_per_rank, is_token_in_rank,
      expert_offset, rank_offset, send_offset, token_slot, recv_pos, recv_token,
      recv_k, send_token, tok_mask, hist;
  size_t total;
  int nblk;  // layout workgroups (token tiles)
  int tile;  // tokens per tile
};

constexpr int kMaxPadMultiple = 1024;

// Rows of a receive buffer: T*K pairs plus at most pad-1 padding rows per
// expert segment.
inline int64_t recv_capacity(int64_t T, int K, int E, int pad) {
  return T * K + (int64_t)E * (pad - 1);
}

// layout_pairs: (t,k) pairs per layout tile (512 sizes the workspace: more
// pairs per tile means fewer tiles and a smaller histogram).  pad: expert
// segments padded to a multiple of it (sizes the per-row inverse maps).
WsLayout plan_workspace(int64_t T, int K, int E, int P, int layout_pairs = kLayoutThreads, int pad = 1);


struct LayoutArgs {
  const void* idx;
  int itype, T, K, E, P, epr, nblk, tile;
  int pad;                // expert segments padded to a multiple of this
  int R;                  // receive rows (recv_capacity)
  int* hist;              // [nblk+1][E+1+P]: per tile, bucket counts then partition token counts
  int scanned;            // hist rewritten by layout_scan_kernel: row j the counts of the tiles
                          // before j, row nblk the column totals
  unsigned long long* tok_mask;  // [T] partitions each token is sent to
  int* num_tokens_per_expert;
  int* num_tokens_per_rank;
  uint8_t* is_token_in_rank;
  int* expert_offset;
  int* rank_offset;
  int* send_offset;
  int* token_slot;
  int* recv_pos;
  int* recv_token;
  int* recv_k;
  int* send_token;        // [T*min(K,P)] token of each send row
  int* status;
};

// Dynamic LDS of the two layout kernels.
size_t layout_count_lds(int E, int P, int tile);
size_t layout_rank_lds(int E, int P, int tile, int K);

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s);

// Padding rows of a padded layout: rows [expert_offset[e] + n_e,
// expert_offset[e+1]) of every expert get zero chunks (and a zero score).
// Written by extra waves of the kernel that writes the receive rows.
constexpr int kPadRows = 8;  // padding rows per fill wave

struct PadArgs {
  void* dst;                         // [R, NV] chunks
  float* scores_out;                 // [R] or null
  const int* expert_offset;          // [E+1], padded
  const int* num_tokens_per_expert;  // [E]
  int E, NV, R;
  int pad;                           // the handle's multiple (1: no padding, no fill waves)
  int ngrp;                          // segments per row
  int nblk;                          // row blocks per expert
  int nwaves;                        // fill waves: pad_fill_waves(E, pad, NV), 0 when unpadded
};

// Wavefronts of one padding fill: an expert has at most pad-1 padding rows,
// in blocks of kPadRows, and a row has one segment per 64 chunks.
inline int64_t pad_fill_waves(int E, int pad, int NV) {
  if (pad <= 1) return 0;
  return (int64_t)E * ((pad - 1 + kPadRows - 1) / kPadRows) * ((NV + 63) / 64);
}

// Token-row -> receive-row direction (dispatch, rows of the combine backward).
struct ScatterArgs {
  const void* src;        // [T, NV] chunks
  const int* recv_pos;    // [T, K]
  const float* w;         // [T, K] or null
  void* dst;              // [R, NV] chunks
  float* scores_out;      // [R] or null
  int T, K, NV, R;
  int ngrp;               // wave groups per token (set by the launcher)
  int dtype;
  bool scale;             // dst = round(w * src)
  int* status;
  PadArgs pad;            // padding rows of dst, filled by pad.nwaves waves after the token waves
};

// Receive-row -> token-row direction (combine, unscaled dispatch backward).
struct GatherArgs {
  const void* src;        // [R, NV] chunks
  const int* recv_pos;    // [T, K]
  const float* w;         // [T, K] or null (plain sum)
  void* dst;              // [T, NV] chunks
  int T, K, NV, R;
  int ngrp;               // wave groups per token (set by the launcher)
  int dtype;
  int* status;
};

// Router-weight gradient dot[t,k] = <tok[t], rcv[recv_pos[t,k]]>, one
// workgroup per token; with `gather` it also writes dst[t] = sum_k [w *] rcv.
struct DotArgs {
  const void* tok;        // [T, NV] chunks
  const void* rcv;        // [R, NV] chunks
  const int* recv_pos;    // [T, K]
  const float* w;         // [T, K] or null
  void* dst;              // [T, NV] chunks (gather only)
  float* dot_out;         // [T, K]
  int T, K, NV, R;
  int dtype;
  bool gather;
  int* status;
};

// Staged exchange: a deduplicated send buffer [send_cap, NV] per (token,
// partition) pair, rows send_offset[r] + token_slot[t,r].
struct StagedArgs {
  const void* src;        // send: x [T]; expand: S [send_cap]; reduce: y [R]; combine: Q [send_cap]
  void* dst;              // send: S; expand: recv [R]; reduce: Q; combine: out [T]
  const int* recv_pos;    // [T, K]
  const int* token_slot;  // [T, P]
  const int* send_offset; // [P+1]
  const int* rank_offset; // [P+1]
  const int* send_token;  // [send_cap]
  const unsigned long long* tok_mask;  // [T]
  const float* w;         // [T, K] or null
  float* scores_out;      // expand: [R] or null
  int T, K, P, NV, R;
  int send_cap;           // rows of the send buffer (>= send_offset[P])
  int ngrp;               // wave groups per row (set by the launcher)
  int dtype;
  bool scale;             // expand: dst = round(w * src)
  int* status;
  PadArgs pad;            // expand: padding rows of dst, filled by the grid's first pad.nwaves waves
};

struct Tuning {
  int chunks_per_lane;  // 1, 2, 4: consecutive 64-chunk segments per wave
  int nontemporal;      // 0, 1, 2
  int waves_per_block;  // 1, 2, 4, 8
  int layout_pairs;     // 512, 1024, 2048, 4096
  int gather_mode;      // 0: by row width (LDS-staged from 4 KiB); 1: LDS-staged (gather_lds_kernel);
                        // 2: registers (gather_kernel)
  int gather_waves;     // waves per workgroup of the LDS-staged gather: waves_per_block when
                        // that is set, else 0 (by row width, lds_gather_waves)
  // measurement: when ev_stop is set, the launch goes through
  // hipExtLaunchKernel, which binds ev_stop to the kernel's completion and,
  // when ev_start is set too, records ev_start just before the kernel; null
  // for every other launch
  hipEvent_t ev_start = nullptr;
  hipEvent_t ev_stop = nullptr;
};

// Launches a row kernel, with the tuning's measurement events when it has
// them.
template <typename F, typename... Args>
inline void launch_kernel(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, const Tuning& t,
                          Args... args) {
  if (t.ev_stop)
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t.ev_start, t.ev_stop, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

constexpr int kMaxDotWaves = 16;         // waves of one token-dot workgroup
constexpr size_t kMaxDotLds = 64 * 1024;  // LDS for its per-segment values

size_t dot_lds_bytes(int NV, int K);
int64_t row_waves(int64_t T, int NV, int cpl);

hipError_t launch_scatter(const ScatterArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_gather(const GatherArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_token_dot(const DotArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_send(const StagedArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_expand(const StagedArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_reduce_partitions(const StagedArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_combine_partitions(const StagedArgs& a, const Tuning& t, hipStream_t s);
hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s);

}  // namespace moe
