// Row movement between token order [T,H] and the expert-grouped receive
// buffer [R,H], R = T*K (plus the padding rows of a padded handle).
//
// A row is cut into 16-byte chunks and the chunks into segments of 64: one
// wavefront-wide access is one segment, 1 KiB of one row, fully coalesced.
// The unit of work is a (token, segment) pair, so a token's row is spread
// over several wavefronts: many short-lived waves keep far more HBM requests
// in flight than one wave walking a whole row.
//
//   scatter (token -> receive rows): forward dispatch, and the row part of a
//     combine's backward.  One wave loads its segment of the token row once
//     and stores it to the K receive rows, optionally scaled by w[t,k] in
//     float32 and rounded (scores absorbed before W2).  The receive rows are
//     written once and not read back here, so their stores are non-temporal.
//     On a padded handle, waves after the token waves zero the padding rows
//     (pad_fill.h).
//   gather (receive rows -> token): forward combine, and the backward of an
//     unscaled dispatch.  One wave loads its segment of up to 8 receive rows
//     (non-temporal: read once), sums them in float32 in k order from +0.0
//     (product and sum rounded separately) and rounds once.  For rows of
//     4 KiB and wider the rows are staged in LDS by direct loads instead
//     (gather_lds_kernel, the same sums), which measured 0.3-3 us faster per
//     launch there.
//   token dot (one workgroup per token, one wave per segment): the
//     router-weight gradients <tok[t], rcv[recv_pos[t,k]]>, in the fixed
//     order of moe_layout.h: per-chunk partials in element order, a butterfly
//     fold per segment, then the segment values added in segment order
//     through LDS.  Its gather variant also produces the weighted sum (the
//     backward of a scaled dispatch reads each receive row once for both).
//
// Every receive-row index is bounds-checked against R before it is used; a
// bad one raises MOE_STATUS_BAD_POSITION and the row is skipped.
#include "device_common.h"
#include "internal.h"
#include "pad_fill.h"
#include "../../include/moe_layout.h"

namespace moe {
namespace {

constexpr int KG = 8;  // receive rows per group of loads

template <bool NT>
__device__ __forceinline__ u32x4 load_chunk(const u32x4* p) {
  if constexpr (NT) {
    return __builtin_nontemporal_load(p);
  } else {
    return *p;
  }
}

// The K receive rows and weights of token t: lane k < K holds pair (t,k).
struct Pairs {
  int pos = 0;
  float w = 0.f;
  bool bad = false;
};

__device__ __forceinline__ Pairs load_pairs(const int* recv_pos, const float* w, int t, int K, int R) {
  Pairs q;
  const int lane = lane_id();
  if (lane < K) {
    q.pos = recv_pos[(size_t)t * K + lane];
    if (w) q.w = w[(size_t)t * K + lane];
    q.bad = (unsigned)q.pos >= (unsigned)R;
  }
  return q;
}

// ---- scatter ----------------------------------------------------------------

template <int DT, int CPL, bool SCALE, bool NT>
__global__ __launch_bounds__(512) void scatter_kernel(ScatterArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int gw = blockIdx.x * wpb + (int)(threadIdx.x / kWave);
  const int t = gw / a.ngrp;
  if (t >= a.T) {  // wave-uniform: the padding waves follow the token waves
    const int w = gw - a.T * a.ngrp;
    if (w < a.pad.nwaves) pad_fill_wave(a.pad, w);
    return;
  }
  const int grp = gw - t * a.ngrp;
  const int jb = grp * kWave * CPL + lane;  // this lane's first chunk

  // The token row's segment first: its load needs only t, so it shares a
  // round trip with the pair lookups instead of following them.
  // Lanes past the row end hold zeros: the scaled path converts every lane's
  // chunk, and a conversion of an indeterminate value would let the
  // compiler drop the j < NV guards.
  const u32x4* src = static_cast<const u32x4*>(a.src) + (size_t)t * a.NV;
  u32x4* dst = static_cast<u32x4*>(a.dst);
  u32x4 v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = jb + c * kWave;
    v[c] = u32x4{0u, 0u, 0u, 0u};
    if (j < a.NV) v[c] = src[j];
  }

  const Pairs q = load_pairs(a.recv_pos, a.w, t, a.K, a.R);
  if (grp == 0) {
    if (__ballot(q.bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);
    if (a.scores_out && lane < a.K && !q.bad) a.scores_out[q.pos] = q.w;
  }
  float f[CPL][SCALE ? V : 1];
  if constexpr (SCALE) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) unpack<DT>(v[c], f[c]);
  }
  for (int k = 0; k < a.K; ++k) {
    const int p = read_lane_i(q.pos, k);
    if ((unsigned)p >= (unsigned)a.R) continue;  // uniform
    u32x4* drow = dst + (size_t)p * a.NV;
    const float s = read_lane_f(q.w, k);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = jb + c * kWave;
      if (j < a.NV) {
        u32x4 o = v[c];
        if constexpr (SCALE) {
          float g[V];
#pragma unroll
          for (int i = 0; i < V; ++i) g[i] = __fmul_rn(s, f[c][i]);
          o = pack<DT>(g);
        }
        store_chunk<NT>(drow + j, o);
      }
    }
  }
}

// ---- gather -----------------------------------------------------------------

template <int DT, int CPL, bool WEIGHTED, bool NTL, bool NTS>
__global__ __launch_bounds__(512) void gather_kernel(GatherArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int gw = blockIdx.x * wpb + (int)(threadIdx.x / kWave);
  const int t = gw / a.ngrp;
  if (t >= a.T) return;  // wave-uniform
  const int grp = gw - t * a.ngrp;
  const int jb = grp * kWave * CPL + lane;

  const Pairs q = load_pairs(a.recv_pos, WEIGHTED ? a.w : nullptr, t, a.K, a.R);
  if (grp == 0 && __ballot(q.bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);

  const u32x4* src = static_cast<const u32x4*>(a.src);
  float acc[CPL][V];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int i = 0; i < V; ++i) acc[c][i] = 0.f;

  for (int kg = 0; kg < a.K; kg += KG) {
    u32x4 yv[KG][CPL];
    bool ok[KG];
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int k = kg + kk;
      ok[kk] = false;
      if (k < a.K) {
        const int p = read_lane_i(q.pos, k);
        ok[kk] = (unsigned)p < (unsigned)a.R;
        if (ok[kk]) {
#pragma unroll
          for (int c = 0; c < CPL; ++c) {
            const int j = jb + c * kWave;
            if (j < a.NV) yv[kk][c] = load_chunk<NTL>(src + (size_t)p * a.NV + j);
          }
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      if (ok[kk]) {
        const float s = read_lane_f(q.w, kg + kk);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = jb + c * kWave;
          if (j < a.NV) {
            float f[V];
            unpack<DT>(yv[kk][c], f);
            if constexpr (WEIGHTED) {
#pragma unroll
              for (int i = 0; i < V; ++i) acc[c][i] = __fadd_rn(acc[c][i], __fmul_rn(s, f[i]));
            } else {
#pragma unroll
              for (int i = 0; i < V; ++i) acc[c][i] = __fadd_rn(acc[c][i], f[i]);
            }
          }
        }
      }
    }
  }
  u32x4* dst = static_cast<u32x4*>(a.dst) + (size_t)t * a.NV;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int j = jb + c * kWave;
    if (j < a.NV) store_chunk<NTS>(dst + j, pack<DT>(acc[c]));
  }
}

// ---- gather, receive rows staged in LDS ---------------------------------------
//
// The same sums as gather_kernel (one wave per (token, segment), float32 in k
// order from +0.0), with each receive-row segment loaded straight into the
// wave's slice of LDS by global_load_lds_dwordx4: 64 lanes x 16 bytes land
// contiguously at the slice's base, no VGPR holds a row in flight, and a
// group of up to KG rows is in flight together whatever the register budget.
// The wave then reads its chunks back from LDS for the sum.  Rows of a token
// are not shared between waves, so the staging buys memory-level parallelism,
// not reuse.  One segment per wave (chunks_per_lane is ignored).

template <int DT, bool WEIGHTED, bool NTL, bool NTS>
__global__ __launch_bounds__(512) void gather_lds_kernel(GatherArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  constexpr int kAux = NTL ? 2 : 0;  // cache policy of the LDS loads: non-temporal
  extern __shared__ u32x4 stage[];   // [waves per block][KG][64 lanes]
  const int lane = lane_id();
  const int wib = (int)(threadIdx.x / kWave);
  const int wpb = blockDim.x / kWave;
  const int gw = blockIdx.x * wpb + wib;
  const int t = gw / a.ngrp;
  if (t >= a.T) return;  // wave-uniform
  const int grp = gw - t * a.ngrp;
  const int j = grp * kWave + lane;
  const bool valid = j < a.NV;

  const Pairs q = load_pairs(a.recv_pos, WEIGHTED ? a.w : nullptr, t, a.K, a.R);
  if (grp == 0 && __ballot(q.bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);

  u32x4* buf = stage + (size_t)wib * KG * kWave;
  const u32x4* src = static_cast<const u32x4*>(a.src);
  float acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;

  for (int kg = 0; kg < a.K; kg += KG) {
    if (kg > 0) {
      // the previous group's LDS reads have returned before new rows land
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __asm__ __volatile__("" ::: "memory");
    }
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int k = kg + kk;
      if (k < a.K) {  // uniform
        const int p = read_lane_i(q.pos, k);
        if ((unsigned)p < (unsigned)a.R && valid)
          __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + (size_t)p * a.NV + j),
                                           (__attribute__((address_space(3))) void*)(buf + kk * kWave),
                                           16, 0, kAux);
      }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every staged row has landed
    __asm__ __volatile__("" ::: "memory");
#pragma unroll
    for (int kk = 0; kk < KG; ++kk) {
      const int k = kg + kk;
      if (k < a.K) {
        const int p = read_lane_i(q.pos, k);
        if ((unsigned)p < (unsigned)a.R && valid) {
          float f[V];
          unpack<DT>(buf[kk * kWave + lane], f);
          if constexpr (WEIGHTED) {
            const float s = read_lane_f(q.w, k);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = __fadd_rn(acc[i], __fmul_rn(s, f[i]));
          } else {
#pragma unroll
            for (int i = 0; i < V; ++i) acc[i] = __fadd_rn(acc[i], f[i]);
          }
        }
      }
    }
  }
  if (valid) store_chunk<NTS>(static_cast<u32x4*>(a.dst) + (size_t)t * a.NV + j, pack<DT>(acc));
}

// ---- token dot (router-weight gradients), optionally with the gather ---------

template <int DT, bool GATHER, bool WEIGHTED, bool NTL, bool NTS>
__global__ __launch_bounds__(1024) void token_dot_kernel(DotArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  // Rows in flight per group.  The bfloat16 gather variant keeps a sum and
  // the token segment unpacked beside its rows: with 8 rows it needs 79
  // VGPRs (6 waves per SIMD), with 4 it fits 64 (8 waves per SIMD).
  constexpr int KGD = (GATHER && DT == kBF16) ? 4 : KG;
  extern __shared__ float seg_val[];  // [nseg][K]
  const int lane = lane_id();
  const int wave = (int)(threadIdx.x / kWave);
  const int nw = blockDim.x / kWave;
  const int t = blockIdx.x;
  const int nseg = (a.NV + kWave - 1) / kWave;

  const Pairs q = load_pairs(a.recv_pos, a.w, t, a.K, a.R);
  if (wave == 0 && __ballot(q.bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);

  const u32x4* tok = static_cast<const u32x4*>(a.tok) + (size_t)t * a.NV;
  const u32x4* rcv = static_cast<const u32x4*>(a.rcv);

  for (int sg = wave; sg < nseg; sg += nw) {  // wave-uniform
    const int j = sg * kWave + lane;
    const bool valid = j < a.NV;
    u32x4 xr = u32x4{0u, 0u, 0u, 0u};
    if (valid) xr = tok[j];
    float x[V];
#pragma unroll
    for (int i = 0; i < V; ++i) x[i] = 0.f;
    // The gather variant unpacks the token segment only after its first
    // group of receive-row loads has gone out, so both loads share one round
    // trip.  The row-free dot unpacks it first: its rows then go out after
    // the token's, which measured faster at the 14-segment row width.
    constexpr bool kLate = GATHER;
    if constexpr (!kLate) unpack<DT>(xr, x);
    float acc[GATHER ? V : 1];
#pragma unroll
    for (int i = 0; i < (GATHER ? V : 1); ++i) acc[i] = 0.f;

    for (int kg = 0; kg < a.K; kg += KGD) {
      u32x4 yv[KGD];
      bool ok[KGD];
#pragma unroll
      for (int kk = 0; kk < KGD; ++kk) {
        const int k = kg + kk;
        ok[kk] = false;
        yv[kk] = u32x4{0u, 0u, 0u, 0u};
        if (k < a.K) {
          const int p = read_lane_i(q.pos, k);
          ok[kk] = (unsigned)p < (unsigned)a.R;
          if (ok[kk] && valid) yv[kk] = load_chunk<NTL>(rcv + (size_t)p * a.NV + j);
        }
      }
      if constexpr (kLate) {
        if (kg == 0) unpack<DT>(xr, x);
      }
#pragma unroll
      for (int kk = 0; kk < KGD; ++kk) {
        const int k = kg + kk;
        if (k < a.K) {  // uniform: every lane takes part in the fold
          float c = 0.f;
          if (ok[kk] && valid) {
            float f[V];
            unpack<DT>(yv[kk], f);
#pragma unroll
            for (int i = 0; i < V; ++i) c = __fadd_rn(c, __fmul_rn(x[i], f[i]));
            if constexpr (GATHER) {
              if constexpr (WEIGHTED) {
                const float s = read_lane_f(q.w, k);
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] = __fadd_rn(acc[i], __fmul_rn(s, f[i]));
              } else {
#pragma unroll
                for (int i = 0; i < V; ++i) acc[i] = __fadd_rn(acc[i], f[i]);
              }
            }
          }
          c = fold64(c);
          if (lane == 0) seg_val[sg * a.K + k] = c;
        }
      }
    }
    if constexpr (GATHER) {
      if (valid) {
        u32x4* dst = static_cast<u32x4*>(a.dst) + (size_t)t * a.NV;
        store_chunk<NTS>(dst + j, pack<DT>(acc));
      }
    }
  }
  __syncthreads();
  if ((int)threadIdx.x < a.K) {
    float d = 0.f;
    for (int sg = 0; sg < nseg; ++sg) d = __fadd_rn(d, seg_val[sg * a.K + threadIdx.x]);
    a.dot_out[(size_t)t * a.K + threadIdx.x] = d;
  }
}

// ---- launch geometry and template selection -----------------------------------

int groups_per_token(int NV, int cpl) { return (NV + kWave * cpl - 1) / (kWave * cpl); }

template <int DT, int CPL, bool SCALE>
hipError_t go_scatter(const ScatterArgs& a0, const Tuning& tu, hipStream_t s) {
  ScatterArgs a = a0;
  a.ngrp = groups_per_token(a.NV, CPL);
  const int wpb = tu.waves_per_block;
  const int64_t waves = (int64_t)a.T * a.ngrp + a.pad.nwaves;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb)), block(wpb * kWave);
  if (tu.nontemporal >= 1)
    launch_kernel(scatter_kernel<DT, CPL, SCALE, true>, grid, block, 0, s, tu, a);
  else
    launch_kernel(scatter_kernel<DT, CPL, SCALE, false>, grid, block, 0, s, tu, a);
  return hipGetLastError();
}

template <int DT, int CPL>
hipError_t sc_mode(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  return a.scale ? go_scatter<DT, CPL, true>(a, t, s) : go_scatter<DT, CPL, false>(a, t, s);
}

template <int DT>
hipError_t sc_cpl(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  switch (t.chunks_per_lane) {
    case 2: return sc_mode<DT, 2>(a, t, s);
    case 4: return sc_mode<DT, 4>(a, t, s);
    default: return sc_mode<DT, 1>(a, t, s);
  }
}

template <int DT, int CPL, bool W>
hipError_t go_gather(const GatherArgs& a0, const Tuning& tu, hipStream_t s) {
  GatherArgs a = a0;
  a.ngrp = groups_per_token(a.NV, CPL);
  const int wpb = tu.waves_per_block;
  const int64_t waves = (int64_t)a.T * a.ngrp;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb)), block(wpb * kWave);
  switch (tu.nontemporal) {
    case 0: launch_kernel(gather_kernel<DT, CPL, W, false, false>, grid, block, 0, s, tu, a); break;
    case 1: launch_kernel(gather_kernel<DT, CPL, W, true, false>, grid, block, 0, s, tu, a); break;
    default: launch_kernel(gather_kernel<DT, CPL, W, true, true>, grid, block, 0, s, tu, a); break;
  }
  return hipGetLastError();
}

template <int DT, int CPL>
hipError_t ga_mode(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  return a.w ? go_gather<DT, CPL, true>(a, t, s) : go_gather<DT, CPL, false>(a, t, s);
}

// Waves per workgroup of the LDS-staged gather when the handle leaves it
// open.  Workgroups are dealt to the eight XCDs in turn, so with one wave per
// workgroup the segments of a token row spread over several XCDs.  Measured
// per launch (kernel trace, bfloat16, T = 4096 and 8192, rows of 4 to 14 KiB,
// 1, 2 and 4 waves per workgroup): one wave was the fastest, by 0.1-3.3 us,
// at every width whose segments are all full, except rows of 8 segments,
// where the deal gives XCD x segment x of every row and one wave ran 8 us
// (T = 4096) and 3 us (T = 8192) slower than two or four.  At 5.5 KiB rows
// (a half segment last) the plain sum ran 1.3 us slower with one wave at
// T = 8192.  So one wave for rows of whole segments whose count is not a
// multiple of 8, else the handle's waves_per_block.  Renumbering the
// workgroups so that each XCD takes one contiguous run of tokens measured
// 3-11% slower at every width, for both gathers and the scatter.
int lds_gather_waves(int NV, int ngrp, int waves_per_block) {
  return (NV % kWave == 0 && ngrp % 8 != 0) ? 1 : waves_per_block;
}

template <int DT, bool W>
hipError_t go_gather_lds(const GatherArgs& a0, const Tuning& tu, hipStream_t s) {
  GatherArgs a = a0;
  a.ngrp = groups_per_token(a.NV, 1);
  const int wpb = tu.gather_waves ? tu.gather_waves : lds_gather_waves(a.NV, a.ngrp, tu.waves_per_block);
  const int64_t waves = (int64_t)a.T * a.ngrp;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb)), block(wpb * kWave);
  const uint32_t lds = (uint32_t)(wpb * KG * kWave * sizeof(u32x4));
  switch (tu.nontemporal) {
    case 0: launch_kernel(gather_lds_kernel<DT, W, false, false>, grid, block, lds, s, tu, a); break;
    case 1: launch_kernel(gather_lds_kernel<DT, W, true, false>, grid, block, lds, s, tu, a); break;
    default: launch_kernel(gather_lds_kernel<DT, W, true, true>, grid, block, lds, s, tu, a); break;
  }
  return hipGetLastError();
}

// Which gather reads the receive rows.  By default the LDS-staged one for
// rows of 4 KiB (256 chunks) and wider, the register one below.  Measured per
// launch (kernel trace, bfloat16, register gather at 4 waves per workgroup
// against the LDS-staged one at lds_gather_waves): Qwen3-30B-A3B rows of
// 4 KiB, combine 27.52 vs 26.64 us and dispatch backward 26.58 vs 26.28;
// DeepSeek-V3 rows of 14 KiB, 94.63 vs 91.65 and 92.61 vs 90.47;
// DiffusionGemma rows of 5.5 KiB, plain combine 71.27 vs 69.11.  At rows of
// 0.5-3 KiB neither form was consistently faster over T = 4096-16384.
bool gather_in_lds(const GatherArgs& a, const Tuning& t) {
  if (t.gather_mode == 1) return true;
  if (t.gather_mode == 2) return false;
  return a.NV >= 256;
}

template <int DT>
hipError_t ga_cpl(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  if (gather_in_lds(a, t)) return a.w ? go_gather_lds<DT, true>(a, t, s) : go_gather_lds<DT, false>(a, t, s);
  switch (t.chunks_per_lane) {
    case 2: return ga_mode<DT, 2>(a, t, s);
    case 4: return ga_mode<DT, 4>(a, t, s);
    default: return ga_mode<DT, 1>(a, t, s);
  }
}

template <int DT, bool G, bool W>
hipError_t go_dot(const DotArgs& a, const Tuning& tu, hipStream_t s) {
  const int nseg = (a.NV + kWave - 1) / kWave;
  const int nw = nseg < kMaxDotWaves ? nseg : kMaxDotWaves;
  const size_t lds = (size_t)nseg * a.K * sizeof(float);
  const dim3 grid((unsigned)a.T), block(nw * kWave);
  switch (tu.nontemporal) {
    case 0: launch_kernel(token_dot_kernel<DT, G, W, false, false>, grid, block, lds, s, tu, a); break;
    case 1: launch_kernel(token_dot_kernel<DT, G, W, true, false>, grid, block, lds, s, tu, a); break;
    default: launch_kernel(token_dot_kernel<DT, G, W, true, true>, grid, block, lds, s, tu, a); break;
  }
  return hipGetLastError();
}

template <int DT>
hipError_t dot_mode(const DotArgs& a, const Tuning& t, hipStream_t s) {
  if (!a.gather) return go_dot<DT, false, false>(a, t, s);
  return a.w ? go_dot<DT, true, true>(a, t, s) : go_dot<DT, true, false>(a, t, s);
}

}  // namespace

size_t dot_lds_bytes(int NV, int K) {
  return (size_t)((NV + kWave - 1) / kWave) * (size_t)K * sizeof(float);
}

int64_t row_waves(int64_t T, int NV, int cpl) { return T * groups_per_token(NV, cpl); }

hipError_t launch_scatter(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? sc_cpl<kF32>(a, t, s) : sc_cpl<kBF16>(a, t, s);
}

hipError_t launch_gather(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? ga_cpl<kF32>(a, t, s) : ga_cpl<kBF16>(a, t, s);
}

hipError_t launch_token_dot(const DotArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? dot_mode<kF32>(a, t, s) : dot_mode<kBF16>(a, t, s);
}

}  // namespace moe
