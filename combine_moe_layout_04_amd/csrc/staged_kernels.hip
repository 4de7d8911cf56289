// Staged exchange on one GPU: the payload a cross-GPU transport would move is
// a physical buffer S with one row per (token, destination partition) pair,
// row send_offset[r] + token_slot[t,r] (a token is sent once per partition
// that hosts one of its experts, not once per expert).
//
//   send   (source side): each token row is loaded once and stored to its
//          partitions' send rows.  One wave per (token, segment).
//   expand (receiver side): each send row is loaded once and stored to the
//          receive rows of its token's experts on that partition (optionally
//          scaled by w[t,k] in float32, and with per-row scores).  One wave per
//          (send row, two segments): the row's partition is the number of
//          partitions whose send range ends at or before it (a ballot over
//          send_offset), its token is send_token[row], and its pairs are the
//          k whose receive row lies in the partition's range.
//   reduce_partitions (receiver side): per send row, the partial sum over
//          its pairs in k order, float32 from +0.0, rounded to the row type.
//          One wave per (send row, two segments), found as in the expansion.
//   combine_partitions (source side): per token, the partial rows of its
//          partitions in ascending partition order, float32 from +0.0,
//          rounded once.  One wave per (token, segment).
//
// A segment is 64 chunks of 16 bytes (one wavefront access); every row index
// is bounds-checked and a bad one raises MOE_STATUS_BAD_POSITION.  Rows
// written once and not read back by the kernel take non-temporal stores.
#include "device_common.h"
#include "internal.h"
#include "pad_fill.h"
#include "../../include/moe_layout.h"

namespace moe {
namespace {

constexpr int KG = 8;  // rows in flight together per wave

template <bool NT>
__device__ __forceinline__ u32x4 load_chunk(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

__device__ __forceinline__ void flag_bad(int* status, bool bad) {
  if (__ballot(bad) && lane_id() == 0) atomicOr(status, MOE_STATUS_BAD_POSITION);
}

// Send rows of token t: lane r < P holds send_offset[r] + token_slot[t,r];
// returns the partition mask (uniform).
__device__ __forceinline__ unsigned long long token_rows(const StagedArgs& a, int t, int& row) {
  const int lane = lane_id();
  row = 0;
  if (lane < a.P) row = a.send_offset[lane] + a.token_slot[(size_t)t * a.P + lane];
  return a.tok_mask[t];
}

// Receiver-side preamble of send row s: token, partition, and the mask of
// the token's k whose receive row is on that partition (lane k < K holds the
// receive row and weight of pair (t,k)).  Returns false for rows past the
// last send row (uniform).
__device__ __forceinline__ bool send_row_pairs(const StagedArgs& a, int s, int& t, uint64_t& kmask,
                                               int& pos, float& w) {
  const int lane = lane_id();
  const int n_send = a.send_offset[a.P];
  if (s >= n_send) return false;
  t = a.send_token[s];
  const bool ended = lane < a.P && a.send_offset[lane + 1] <= s;
  const int r = __popcll(__ballot(ended));  // partition of row s
  const int lo = a.rank_offset[r], hi = a.rank_offset[r + 1];
  pos = 0;
  w = 0.f;
  bool in = false;
  if (lane < a.K && (unsigned)t < (unsigned)a.T) {
    pos = a.recv_pos[(size_t)t * a.K + lane];
    if (a.w) w = a.w[(size_t)t * a.K + lane];
    in = pos >= lo && pos < hi && pos < a.R;
  }
  kmask = __ballot(in);
  return true;
}

template <int DT, bool NT>
__global__ __launch_bounds__(512) void send_kernel(StagedArgs a) {
  const int lane = lane_id();
  const int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int t = gw / a.ngrp;
  if (t >= a.T) return;  // wave-uniform
  const int j = (gw - t * a.ngrp) * kWave + lane;
  // the token row's segment first: its load does not wait for the send rows
  const u32x4* src = static_cast<const u32x4*>(a.src) + (size_t)t * a.NV;
  u32x4* dst = static_cast<u32x4*>(a.dst);
  u32x4 v = {0u, 0u, 0u, 0u};  // defined on every lane: see expand_kernel
  if (j < a.NV) v = src[j];
  int row;
  unsigned long long m = token_rows(a, t, row);
  const bool bad = lane < a.P && ((m >> lane) & 1ull) && (unsigned)row >= (unsigned)a.send_cap;
  if (j - lane == 0) flag_bad(a.status, bad);
  while (m) {  // uniform
    const int r = __builtin_ctzll(m);
    m &= m - 1;
    const int s = read_lane_i(row, r);
    if ((unsigned)s < (unsigned)a.send_cap && j < a.NV) store_chunk<NT>(dst + (size_t)s * a.NV + j, v);
  }
}

template <int DT, bool SCALE, bool NT, int CPL>
__global__ __launch_bounds__(512) void expand_kernel(StagedArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  if (gw < a.pad.nwaves) {  // wave-uniform: the padding waves come first
    pad_fill_wave(a.pad, gw);
    return;
  }
  gw -= a.pad.nwaves;
  const int s = gw / a.ngrp;
  if (s >= a.send_cap) return;  // wave-uniform
  const int grp = gw - s * a.ngrp;
  if (s >= a.send_offset[a.P]) return;  // uniform: a send row past N_send holds nothing
  const int jb = grp * kWave * CPL + lane;
  const u32x4* src = static_cast<const u32x4*>(a.src) + (size_t)s * a.NV;
  u32x4* dst = static_cast<u32x4*>(a.dst);
  // The send row's segments first: their loads need only the row, so they
  // overlap the round trips that find the row's token and pairs.
  // v must hold a defined value on the lanes past the row end as well: the
  // scaled path converts it on every lane, and a conversion of an
  // indeterminate value lets the compiler drop the j < NV guards.
  u32x4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    v[c] = u32x4{0u, 0u, 0u, 0u};
    if (jb + c * kWave < a.NV) v[c] = load_chunk<NT>(src + jb + c * kWave);
  }
  int t, pos;
  float w;
  uint64_t km;
  if (!send_row_pairs(a, s, t, km, pos, w)) return;  // uniform
  if (grp == 0 && a.scores_out && ((km >> lane) & 1ull)) a.scores_out[pos] = w;
  float f[CPL][SCALE ? V : 1];
  if constexpr (SCALE) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) unpack<DT>(v[c], f[c]);
  }
  while (km) {  // uniform
    const int k = __builtin_ctzll(km);
    km &= km - 1;
    u32x4* drow = dst + (size_t)read_lane_i(pos, k) * a.NV;
    const float sc = read_lane_f(w, k);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = jb + c * kWave;
      if (j < a.NV) {
        u32x4 o = v[c];
        if constexpr (SCALE) {
          float g[V];
#pragma unroll
          for (int i = 0; i < V; ++i) g[i] = __fmul_rn(sc, f[c][i]);
          o = pack<DT>(g);
        }
        store_chunk<NT>(drow + j, o);
      }
    }
  }
}

template <int DT, bool WEIGHTED, bool NT, int CPL>
__global__ __launch_bounds__(512) void reduce_partitions_kernel(StagedArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  constexpr int G = KG / CPL;  // pairs in flight together: G * CPL chunks per lane
  const int lane = lane_id();
  const int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int s = gw / a.ngrp;
  if (s >= a.send_cap) return;  // wave-uniform
  const int grp = gw - s * a.ngrp;
  int t, pos;
  float w;
  uint64_t km;
  if (!send_row_pairs(a, s, t, km, pos, w)) return;  // uniform
  const int jb = grp * kWave * CPL + lane;  // this lane's first chunk
  const u32x4* src = static_cast<const u32x4*>(a.src);
  float acc[CPL][V];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[c][i] = 0.f;
  while (km) {  // uniform: groups of up to G pairs in k order, loads issued together
    u32x4 yv[G][CPL];
    int ks[G];
    int n = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      ks[g] = -1;
#pragma unroll
      for (int c = 0; c < CPL; ++c) yv[g][c] = u32x4{0u, 0u, 0u, 0u};
      if (km) {
        const int k = __builtin_ctzll(km);
        km &= km - 1;
        ks[g] = k;
        n = g + 1;
        const u32x4* row = src + (size_t)read_lane_i(pos, k) * a.NV;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = jb + c * kWave;
          if (j < a.NV) yv[g][c] = load_chunk<NT>(row + j);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      if (g < n) {
        const float sc = WEIGHTED ? read_lane_f(w, ks[g]) : 1.f;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          if (jb + c * kWave < a.NV) {
            float f[V];
            unpack<DT>(yv[g][c], f);
            if constexpr (WEIGHTED) {
#pragma unroll
              for (int i = 0; i < V; ++i) acc[c][i] = __fadd_rn(acc[c][i], __fmul_rn(sc, f[i]));
            } else {
#pragma unroll
              for (int i = 0; i < V; ++i) acc[c][i] = __fadd_rn(acc[c][i], f[i]);
            }
          }
        }
      }
    }
  }
  u32x4* dst = static_cast<u32x4*>(a.dst) + (size_t)s * a.NV;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = jb + c * kWave;
    if (j < a.NV) store_chunk<NT>(dst + j, pack<DT>(acc[c]));
  }
}

template <int DT, bool NT, bool NTS>
__global__ __launch_bounds__(512) void combine_partitions_kernel(StagedArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int gw = blockIdx.x * (int)(blockDim.x / kWave) + (int)(threadIdx.x / kWave);
  const int t = gw / a.ngrp;
  if (t >= a.T) return;  // wave-uniform
  const int j = (gw - t * a.ngrp) * kWave + lane;
  int row;
  unsigned long long m = token_rows(a, t, row);
  const bool bad = lane < a.P && ((m >> lane) & 1ull) && (unsigned)row >= (unsigned)a.send_cap;
  if (j - lane == 0) flag_bad(a.status, bad);
  const u32x4* src = static_cast<const u32x4*>(a.src);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
  while (m) {  // uniform: partitions ascending, up to KG rows in flight
    u32x4 qv[KG];
    int n = 0;
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      qv[g] = u32x4{0u, 0u, 0u, 0u};
      if (m) {
        const int r = __builtin_ctzll(m);
        m &= m - 1;
        const int s = read_lane_i(row, r);
        n = g + 1;
        if (j < a.NV && (unsigned)s < (unsigned)a.send_cap) qv[g] = load_chunk<NT>(src + (size_t)s * a.NV + j);
      }
    }
#pragma unroll
    for (int g = 0; g < KG; ++g) {
      if (g < n && j < a.NV) {
        float f[V];
        unpack<DT>(qv[g], f);
#pragma unroll
        for (int i = 0; i < V; ++i) acc[i] = __fadd_rn(acc[i], f[i]);
      }
    }
  }
  if (j < a.NV) {
    u32x4* dst = static_cast<u32x4*>(a.dst) + (size_t)t * a.NV;
    store_chunk<NTS>(dst + j, pack<DT>(acc));
  }
}

// ---- launch geometry ----------------------------------------------------------

// Segments per wave.  A send row's wave (expansion, partition reduce)
// spends two dependent round trips finding its token and pairs before its
// rows move, and moves only about K/P rows, so those kernels take two
// segments per wave: half the lookups per byte.  The send and the merge have
// one lookup round trip and keep one segment.
int groups(int NV, int segs) { return (NV + kWave * segs - 1) / (kWave * segs); }

dim3 grid_for(int64_t rows, int ngrp, int wpb, int64_t extra_waves = 0) {
  const int64_t waves = rows * ngrp + extra_waves;
  return dim3((unsigned)((waves + wpb - 1) / wpb));
}

template <int DT>
hipError_t go_send(StagedArgs a, const Tuning& tu, hipStream_t s) {
  a.ngrp = groups(a.NV, 1);
  const dim3 grid = grid_for(a.T, a.ngrp, tu.waves_per_block), block(tu.waves_per_block * kWave);
  if (tu.nontemporal >= 1)
    launch_kernel(send_kernel<DT, true>, grid, block, 0, s, tu, a);
  else
    launch_kernel(send_kernel<DT, false>, grid, block, 0, s, tu, a);
  return hipGetLastError();
}

template <int DT>
hipError_t go_expand(StagedArgs a, const Tuning& tu, hipStream_t s) {
  constexpr int C = 2;  // segments per wave
  a.ngrp = groups(a.NV, C);
  const dim3 grid = grid_for(a.send_cap, a.ngrp, tu.waves_per_block, a.pad.nwaves),
             block(tu.waves_per_block * kWave);
  const bool nt = tu.nontemporal >= 1;
  if (a.scale) {
    if (nt) launch_kernel(expand_kernel<DT, true, true, C>, grid, block, 0, s, tu, a);
    else launch_kernel(expand_kernel<DT, true, false, C>, grid, block, 0, s, tu, a);
  } else {
    if (nt) launch_kernel(expand_kernel<DT, false, true, C>, grid, block, 0, s, tu, a);
    else launch_kernel(expand_kernel<DT, false, false, C>, grid, block, 0, s, tu, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t go_reduce(StagedArgs a, const Tuning& tu, hipStream_t s) {
  constexpr int C = 2;  // segments per wave
  a.ngrp = groups(a.NV, C);
  const dim3 grid = grid_for(a.send_cap, a.ngrp, tu.waves_per_block), block(tu.waves_per_block * kWave);
  const bool nt = tu.nontemporal >= 1;
  if (a.w) {
    if (nt) launch_kernel(reduce_partitions_kernel<DT, true, true, C>, grid, block, 0, s, tu, a);
    else launch_kernel(reduce_partitions_kernel<DT, true, false, C>, grid, block, 0, s, tu, a);
  } else {
    if (nt) launch_kernel(reduce_partitions_kernel<DT, false, true, C>, grid, block, 0, s, tu, a);
    else launch_kernel(reduce_partitions_kernel<DT, false, false, C>, grid, block, 0, s, tu, a);
  }
  return hipGetLastError();
}

template <int DT>
hipError_t go_combine_partitions(StagedArgs a, const Tuning& tu, hipStream_t s) {
  a.ngrp = groups(a.NV, 1);
  const dim3 grid = grid_for(a.T, a.ngrp, tu.waves_per_block), block(tu.waves_per_block * kWave);
  switch (tu.nontemporal) {
    case 0: launch_kernel(combine_partitions_kernel<DT, false, false>, grid, block, 0, s, tu, a); break;
    case 1: launch_kernel(combine_partitions_kernel<DT, true, false>, grid, block, 0, s, tu, a); break;
    default: launch_kernel(combine_partitions_kernel<DT, true, true>, grid, block, 0, s, tu, a); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_send(const StagedArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? go_send<kF32>(a, t, s) : go_send<kBF16>(a, t, s);
}

hipError_t launch_expand(const StagedArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? go_expand<kF32>(a, t, s) : go_expand<kBF16>(a, t, s);
}

hipError_t launch_reduce_partitions(const StagedArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? go_reduce<kF32>(a, t, s) : go_reduce<kBF16>(a, t, s);
}

hipError_t launch_combine_partitions(const StagedArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? go_combine_partitions<kF32>(a, t, s) : go_combine_partitions<kBF16>(a, t, s);
}

}  // namespace moe
