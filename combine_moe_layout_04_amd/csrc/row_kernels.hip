// Row movement between token order [T,H] and the expert-grouped receive
// buffer [R,H], R = T*K.  One wave64 owns one token; its 64 lanes stride the
// row in 16-byte chunks (lane l holds chunks l, l+64, l+128, ...), so every
// wave-wide load or store touches 1 KiB of one row, fully coalesced.
//
//   scatter (token -> receive rows): forward dispatch, and the backward of a
//     combine.  The token row is read from HBM once and stored to each of
//     its K receive rows (grouped by partition, since positions are
//     expert-major); optional float32 scaling by w[t,k], optional per-row
//     scores, optional dot <src[t], other[row]> (router-weight gradient).
//   gather (receive rows -> token): forward combine, and the backward of a
//     dispatch.  The K receive rows of a token are loaded together, reduced
//     in float32 in k order from +0.0 (product and sum rounded separately),
//     rounded once to the row type; optional dot <src[row], other[t]>.
//
// Dots keep one float32 partial per lane and fold the 64 partials with an
// xor butterfly (s = 32..1): the fixed order documented in moe_layout.h.
// Every receive-row index is bounds-checked against R before it is used.
#include "device_common.h"
#include "internal.h"
#include "../../include/moe_layout.h"

namespace moe {
namespace {

// Rows of one token are handled KG receive rows at a time (K <= 32 in any
// number of groups); the dots are fused only when K <= KG (one group).
constexpr int KG = 8;

template <int DT, int CPL, bool SCALE, bool DOT, bool NT>
__global__ __launch_bounds__(512) void scatter_kernel(ScatterArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int t = blockIdx.x * wpb + (int)(threadIdx.x / kWave);
  if (t >= a.T) return;  // wave-uniform

  const u32x4* src = static_cast<const u32x4*>(a.src) + (size_t)t * a.NV;
  u32x4* dst = static_cast<u32x4*>(a.dst);
  const u32x4* oth = static_cast<const u32x4*>(a.other);

  // lane k < K holds the receive row and weight of pair (t,k)
  int mypos = 0;
  float myw = 0.f;
  bool bad = false;
  if (lane < a.K) {
    mypos = a.recv_pos[(size_t)t * a.K + lane];
    if (a.w) myw = a.w[(size_t)t * a.K + lane];
    bad = (unsigned)mypos >= (unsigned)a.R;
  }
  if (__ballot(bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);
  if (a.scores_out && lane < a.K && !bad) a.scores_out[mypos] = myw;

  float L[DOT ? KG : 1];
#pragma unroll
  for (int k = 0; k < (DOT ? KG : 1); ++k) L[k] = 0.f;

  for (int base = 0; base < a.NV; base += kWave * CPL) {
    u32x4 v[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = base + c * kWave + lane;
      if (j < a.NV) v[c] = src[j];
    }
    for (int kg = 0; kg < a.K; kg += KG) {
      // dot operands first, so no store sits between them and their use
      u32x4 yv[DOT ? KG : 1][DOT ? CPL : 1];
      if constexpr (DOT) {
#pragma unroll
        for (int kk = 0; kk < KG; ++kk) {
          const int k = kg + kk;
          if (k < a.K) {
            const int p = read_lane_i(mypos, k);
            if ((unsigned)p < (unsigned)a.R) {
#pragma unroll
              for (int c = 0; c < CPL; ++c) {
                const int j = base + c * kWave + lane;
                if (j < a.NV) yv[kk][c] = oth[(size_t)p * a.NV + j];
              }
            }
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int k = kg + kk;
        if (k < a.K) {
          const int p = read_lane_i(mypos, k);
          if ((unsigned)p < (unsigned)a.R) {
            const float s = read_lane_f(myw, k);
            u32x4* drow = dst + (size_t)p * a.NV;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int j = base + c * kWave + lane;
              if (j < a.NV) {
                u32x4 o = v[c];
                if constexpr (SCALE || DOT) {
                  float f[V];
                  unpack<DT>(v[c], f);
                  if constexpr (DOT) {
                    float g[V];
                    unpack<DT>(yv[kk][c], g);
#pragma unroll
                    for (int i = 0; i < V; ++i) L[kk] = __fadd_rn(L[kk], __fmul_rn(f[i], g[i]));
                  }
                  if constexpr (SCALE) {
#pragma unroll
                    for (int i = 0; i < V; ++i) f[i] = __fmul_rn(s, f[i]);
                    o = pack<DT>(f);
                  }
                }
                store_chunk<NT>(drow + j, o);
              }
            }
          }
        }
      }
    }
  }

  if constexpr (DOT) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      if (k < a.K) {
        const float d = fold64(L[k]);
        if (lane == 0) a.dot_out[(size_t)t * a.K + k] = d;
      }
    }
  }
}

template <int DT, int CPL, bool WEIGHTED, bool DOT, bool NT>
__global__ __launch_bounds__(512) void gather_kernel(GatherArgs a) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int wpb = blockDim.x / kWave;
  const int t = blockIdx.x * wpb + (int)(threadIdx.x / kWave);
  if (t >= a.T) return;  // wave-uniform

  const u32x4* src = static_cast<const u32x4*>(a.src);
  u32x4* dst = static_cast<u32x4*>(a.dst) + (size_t)t * a.NV;
  const u32x4* oth = static_cast<const u32x4*>(a.other) + (DOT ? (size_t)t * a.NV : 0);

  int mypos = 0;
  float myw = 0.f;
  bool bad = false;
  if (lane < a.K) {
    mypos = a.recv_pos[(size_t)t * a.K + lane];
    if constexpr (WEIGHTED) myw = a.w[(size_t)t * a.K + lane];
    bad = (unsigned)mypos >= (unsigned)a.R;
  }
  if (__ballot(bad) && lane == 0) atomicOr(a.status, MOE_STATUS_BAD_POSITION);

  float L[DOT ? KG : 1];
#pragma unroll
  for (int k = 0; k < (DOT ? KG : 1); ++k) L[k] = 0.f;

  for (int base = 0; base < a.NV; base += kWave * CPL) {
    float acc[CPL][V];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[c][i] = 0.f;

    for (int kg = 0; kg < a.K; kg += KG) {
      // the group's rows all in flight before the first use
      u32x4 yv[KG][CPL];
      bool ok[KG];
#pragma unroll
      for (int kk = 0; kk < KG; ++kk) {
        const int k = kg + kk;
        ok[kk] = false;
        if (k < a.K) {
          const int p = read_lane_i(mypos, k);
          ok[kk] = (unsigned)p < (unsigned)a.R;
          if (ok[kk]) {
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
              const int j = base + c * kWave + lane;
              if (j < a.NV) yv[kk][c] = src[(size_t)p * a.NV + j];
            }
          }
        }
      }
      u32x4 xv[DOT ? CPL : 1];
      if constexpr (DOT) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
          const int j = base + c * kWave + lane;
          if (j < a.NV) xv[c] = oth[j];
        }
      }
#pragma unroll
      for (int c = 0; c < CPL; ++c) {
        const int j = base + c * kWave + lane;
        if (j < a.NV) {
          float xf[DOT ? V : 1];
          if constexpr (DOT) unpack<DT>(xv[c], xf);
#pragma unroll
          for (int kk = 0; kk < KG; ++kk) {
            if (ok[kk]) {
              float f[V];
              unpack<DT>(yv[kk][c], f);
              if constexpr (DOT) {
#pragma unroll
                for (int i = 0; i < V; ++i) L[kk] = __fadd_rn(L[kk], __fmul_rn(f[i], xf[i]));
              }
              if constexpr (WEIGHTED) {
                const float s = read_lane_f(myw, kg + kk);
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
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int j = base + c * kWave + lane;
      if (j < a.NV) store_chunk<NT>(dst + j, pack<DT>(acc[c]));
    }
  }

  if constexpr (DOT) {
#pragma unroll
    for (int k = 0; k < KG; ++k) {
      if (k < a.K) {
        const float d = fold64(L[k]);
        if (lane == 0) a.dot_out[(size_t)t * a.K + k] = d;
      }
    }
  }
}

// Router-weight gradient on its own, for K > KG: one wave per pair (t,k),
// dot of token row t of `tok` and receive row recv_pos[t,k] of `rcv`, in the
// same lane order and fold as the fused path.
template <int DT>
__global__ __launch_bounds__(256) void pair_dot_kernel(const u32x4* tok, const u32x4* rcv,
                                                       const int* recv_pos, float* out,
                                                       int T, int K, int NV, int R) {
  constexpr int V = Elems<DT>::kPerChunk;
  const int lane = lane_id();
  const int64_t pair = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
  if (pair >= (int64_t)T * K) return;  // wave-uniform
  const int t = (int)(pair / K);
  const int p = recv_pos[pair];
  float L = 0.f;
  if ((unsigned)p < (unsigned)R) {
    const u32x4* ta = tok + (size_t)t * NV;
    const u32x4* rb = rcv + (size_t)p * NV;
    for (int j = lane; j < NV; j += kWave) {
      float f[V], g[V];
      unpack<DT>(ta[j], f);
      unpack<DT>(rb[j], g);
#pragma unroll
      for (int i = 0; i < V; ++i) L = __fadd_rn(L, __fmul_rn(f[i], g[i]));
    }
  }
  const float d = fold64(L);
  if (lane == 0) out[pair] = d;
}

__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst,
                                                   const u32x4* __restrict__ src, size_t n) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

// ---- template selection ---------------------------------------------------

template <int DT, int CPL, bool SCALE, bool DOT, bool NT>
hipError_t go_scatter(const ScatterArgs& a, int wpb, hipStream_t s) {
  hipLaunchKernelGGL((scatter_kernel<DT, CPL, SCALE, DOT, NT>),
                     dim3((a.T + wpb - 1) / wpb), dim3(wpb * kWave), 0, s, a);
  return hipGetLastError();
}

template <int DT, int CPL, bool SCALE, bool DOT>
hipError_t sc_nt(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  return t.nontemporal >= 1 ? go_scatter<DT, CPL, SCALE, DOT, true>(a, t.waves_per_block, s)
                            : go_scatter<DT, CPL, SCALE, DOT, false>(a, t.waves_per_block, s);
}

template <int DT, int CPL>
hipError_t sc_mode(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  if (a.dot_out && a.K <= KG) return sc_nt<DT, CPL, true, true>(a, t, s);  // dot implies weights
  if (a.scale) return sc_nt<DT, CPL, true, false>(a, t, s);
  return sc_nt<DT, CPL, false, false>(a, t, s);
}

template <int DT>
hipError_t pair_dot(const void* tok, const void* rcv, const int* pos, float* out, int T, int K,
                    int NV, int R, hipStream_t s) {
  const int64_t pairs = (int64_t)T * K;
  const int wpb = 4;
  hipLaunchKernelGGL((pair_dot_kernel<DT>), dim3((unsigned)((pairs + wpb - 1) / wpb)),
                     dim3(wpb * kWave), 0, s, static_cast<const u32x4*>(tok),
                     static_cast<const u32x4*>(rcv), pos, out, T, K, NV, R);
  return hipGetLastError();
}

template <int DT>
hipError_t sc_cpl(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  hipError_t e;
  switch (t.chunks_per_lane) {
    case 1: e = sc_mode<DT, 1>(a, t, s); break;
    case 2: e = sc_mode<DT, 2>(a, t, s); break;
    default: e = sc_mode<DT, 4>(a, t, s); break;
  }
  if (e != hipSuccess || !a.dot_out || a.K <= KG) return e;
  return pair_dot<DT>(a.src, a.other, a.recv_pos, a.dot_out, a.T, a.K, a.NV, a.R, s);
}

template <int DT, int CPL, bool W, bool DOT, bool NT>
hipError_t go_gather(const GatherArgs& a, int wpb, hipStream_t s) {
  hipLaunchKernelGGL((gather_kernel<DT, CPL, W, DOT, NT>),
                     dim3((a.T + wpb - 1) / wpb), dim3(wpb * kWave), 0, s, a);
  return hipGetLastError();
}

template <int DT, int CPL, bool W, bool DOT>
hipError_t ga_nt(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  return t.nontemporal >= 2 ? go_gather<DT, CPL, W, DOT, true>(a, t.waves_per_block, s)
                            : go_gather<DT, CPL, W, DOT, false>(a, t.waves_per_block, s);
}

template <int DT, int CPL>
hipError_t ga_mode(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  if (a.dot_out && a.K <= KG) return ga_nt<DT, CPL, true, true>(a, t, s);  // dot implies weights
  if (a.w) return ga_nt<DT, CPL, true, false>(a, t, s);
  return ga_nt<DT, CPL, false, false>(a, t, s);
}

template <int DT>
hipError_t ga_cpl(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  hipError_t e;
  switch (t.chunks_per_lane) {
    case 1: e = ga_mode<DT, 1>(a, t, s); break;
    case 4: e = ga_mode<DT, 4>(a, t, s); break;
    default: e = ga_mode<DT, 2>(a, t, s); break;
  }
  if (e != hipSuccess || !a.dot_out || a.K <= KG) return e;
  return pair_dot<DT>(a.other, a.src, a.recv_pos, a.dot_out, a.T, a.K, a.NV, a.R, s);
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? sc_cpl<kF32>(a, t, s) : sc_cpl<kBF16>(a, t, s);
}

hipError_t launch_gather(const GatherArgs& a, const Tuning& t, hipStream_t s) {
  return a.dtype == kF32 ? ga_cpl<kF32>(a, t, s) : ga_cpl<kBF16>(a, t, s);
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<u32x4*>(dst), static_cast<const u32x4*>(src), n);
  return hipGetLastError();
}

}  // namespace moe
