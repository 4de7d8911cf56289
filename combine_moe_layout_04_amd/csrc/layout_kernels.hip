// Layout of one routing decision: per-expert and per-partition counts,
// is_token_in_rank, prefix offsets, token send slots and stable receive
// positions.  Two launches over the same token tiles (a tile holds up to a
// few thousand (t,k) pairs, so a layer needs only a handful of workgroups and
// the path is a short chain of memory round trips):
//
//   count: one thread per (t,k) pair: per-tile expert histogram (LDS
//          atomics: counts commute, so the result is deterministic),
//          per-token partition bitmask (LDS atomic OR), is_token_in_rank,
//          per-tile partition token counts.  The two histograms go to one
//          [E+1+P][tiles] array, bucket-major.
//   rank : one flat exclusive scan of that array gives every global offset
//          and this tile's starts (each thread scans a run of it held in
//          registers).  The tile's ids are staged in LDS; each wave ranks a
//          contiguous span of pairs: wave64 ballots match equal ids, a
//          popcount over the lanes below gives the rank inside 64 pairs, and
//          per-(wave, expert) running counters in LDS carry it across rounds.
//          Token send slots come from per-partition ballots over the tile's
//          tokens.  No position is ever taken from an atomic, so the result
//          depends on the routing alone (an activation-checkpoint replay of
//          the same routing reproduces it bit for bit).
//
// Ids outside [0,E) go to an extra bucket E, sorted after every expert, so
// that every position stays inside [0, T*K) even for bad input; the rank
// kernel raises MOE_STATUS_BAD_EXPERT for them.
#include "device_common.h"
#include "internal.h"
#include "../../include/moe_layout.h"

namespace moe {
namespace {

constexpr int kLT = kLayoutThreads;  // threads per layout workgroup
constexpr int kLW = kLT / kWave;     // waves per layout workgroup
constexpr int kScanRegs = 24;        // histogram entries a thread holds in registers

__device__ __forceinline__ int load_expert(const void* idx, int itype, int64_t i, int E) {
  if (itype == MOE_I32) {
    const int v = static_cast<const int*>(idx)[i];
    return (v >= 0 && v < E) ? v : E;
  }
  const long long v = static_cast<const long long*>(idx)[i];
  return (v >= 0 && v < (long long)E) ? (int)v : E;
}

__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int o = __shfl_up(v, d, kWave);
    if (lane >= d) v += o;
  }
  return v;
}

// ---- count ------------------------------------------------------------------

__global__ __launch_bounds__(kLT) void layout_count_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  const int E1 = a.E + 1;
  unsigned long long* msk = reinterpret_cast<unsigned long long*>(smem);  // [tile]
  int* eh = reinterpret_cast<int*>(msk + a.tile);                        // [E+1]
  int* rh = eh + E1;                                                     // [P]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int t0 = b * a.tile;
  const int nt = max(0, min(a.T, t0 + a.tile) - t0);
  for (int i = tid; i < E1 + a.P; i += kLT) eh[i] = 0;
  for (int i = tid; i < nt; i += kLT) msk[i] = 0ull;
  if (b == 0 && tid == 0) *a.status = 0;  // later kernels only OR bits in
  __syncthreads();

  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;
#pragma unroll 8
  for (int i = tid; i < np; i += kLT) {
    const int e = load_expert(a.idx, a.itype, p0 + i, a.E);
    atomicAdd(&eh[e], 1);
    if (e < a.E) atomicOr(&msk[i / a.K], 1ull << (e / a.epr));
  }
  __syncthreads();

  for (int tt = tid; tt < nt; tt += kLT) {
    unsigned long long m = msk[tt];
    while (m) {
      const int r = __ffsll(m) - 1;
      m &= m - 1;
      atomicAdd(&rh[r], 1);
    }
  }
  // is_token_in_rank: whole 32-bit words, then the tail bytes (t0*P is a
  // multiple of 64 because the tile is)
  uint32_t* itr_w = reinterpret_cast<uint32_t*>(a.is_token_in_rank + (size_t)t0 * a.P);
  const int nbytes = nt * a.P;
  for (int wd = tid; wd < nbytes / 4; wd += kLT) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = wd * 4 + q;
      const int tt = i / a.P;
      v |= (uint32_t)((msk[tt] >> (i - tt * a.P)) & 1ull) << (8 * q);
    }
    itr_w[wd] = v;
  }
  for (int i = (nbytes & ~3) + tid; i < nbytes; i += kLT) {
    const int tt = i / a.P;
    a.is_token_in_rank[(size_t)t0 * a.P + i] = (uint8_t)((msk[tt] >> (i - tt * a.P)) & 1ull);
  }
  __syncthreads();

  for (int r = tid; r < E1 + a.P; r += kLT) a.hist[(size_t)r * a.nblk + b] = eh[r];
}

// ---- rank -------------------------------------------------------------------

// Exclusive scan, by the whole workgroup, of the [rows][nblk] histogram read
// row-major.  At (row, j) it is the row's global start plus the row's count
// in the tiles before j.  Writes column b to col_b[rows], column 0 to
// col_0[rows] and the total to col_0[rows].
__device__ void scan_histogram(const int* __restrict__ h, int rows, int nblk, int b, int* col_b,
                               int* col_0, int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int n = rows * nblk;
  const int per = (n + kLT - 1) / kLT;
  const int i0 = min(n, tid * per);
  const int i1 = min(n, i0 + per);
  // the first kScanRegs entries of the run stay in registers (all loads in
  // flight together); longer runs are re-read in the second walk
  int hv[kScanRegs];
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) hv[u] = (i0 + u < i1) ? h[i0 + u] : 0;
  int s = 0;
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) s += hv[u];
  for (int i = i0 + kScanRegs; i < i1; ++i) s += h[i];

  const int inc = wave_inclusive_scan(s);
  if (lane == kWave - 1) wsum[wv] = inc;
  __syncthreads();
  int run = inc - s;
  for (int w = 0; w < wv; ++w) run += wsum[w];
  int row = i0 / nblk;
  int j = i0 - row * nblk;
#pragma unroll
  for (int u = 0; u < kScanRegs; ++u) {
    if (i0 + u < i1) {
      if (j == 0) col_0[row] = run;
      if (j == b) col_b[row] = run;
      run += hv[u];
      if (++j == nblk) {
        j = 0;
        ++row;
      }
    }
  }
  for (int i = i0 + kScanRegs; i < i1; ++i) {
    if (j == 0) col_0[row] = run;
    if (j == b) col_b[row] = run;
    run += h[i];
    if (++j == nblk) {
      j = 0;
      ++row;
    }
  }
  if (i0 < i1 && i1 == n) col_0[rows] = run;
  __syncthreads();
}

__global__ __launch_bounds__(kLT) void layout_rank_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  const int E1 = a.E + 1;
  const int NR = E1 + a.P;                   // histogram rows
  int* base = reinterpret_cast<int*>(smem);  // [NR]   this tile's start of each row
  int* off = base + NR;                      // [NR+1] start of each row, tile 0
  int* cnt = off + NR + 1;                   // [kLW][E+1] per-wave bucket cursors
  int* wsum = cnt + kLW * E1;                // [kLW]
  int* wcnt = wsum + kLW;                    // [kLW][P] per-wave partition counts
  int* carry = wcnt + kLW * a.P;             // [P] slots used by earlier token rounds
  uint16_t* ids = reinterpret_cast<uint16_t*>(carry + a.P);  // [tile*K]

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int t0 = b * a.tile;
  const int nt = max(0, min(a.T, t0 + a.tile) - t0);
  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;

  // 0. stage this tile's ids (bad ids become bucket E)
#pragma unroll 8
  for (int i = tid; i < np; i += kLT) ids[i] = (uint16_t)load_expert(a.idx, a.itype, p0 + i, a.E);
  for (int r = tid; r < a.P; r += kLT) carry[r] = 0;

  // 1. global offsets and this tile's starts (the scan ends with a barrier)
  scan_histogram(a.hist, NR, a.nblk, b, base, off, wsum);
  const int total = off[E1];  // T*K: the bucket rows come first

  // 2. global counts and offsets (tile 0 writes them)
  if (b == 0) {
    for (int e = tid; e < a.E; e += kLT) a.num_tokens_per_expert[e] = off[e + 1] - off[e];
    for (int e = tid; e <= a.E; e += kLT) a.expert_offset[e] = off[e];
    for (int r = tid; r <= a.P; r += kLT) a.rank_offset[r] = off[r * a.epr];
    for (int r = tid; r < a.P; r += kLT) a.num_tokens_per_rank[r] = off[E1 + r + 1] - off[E1 + r];
    for (int r = tid; r <= a.P; r += kLT) a.send_offset[r] = off[E1 + r] - total;
    if (tid == 0 && off[a.E + 1] != off[a.E]) atomicOr(a.status, MOE_STATUS_BAD_EXPERT);
  }

  // 3. per-wave bucket counts over contiguous pair spans of the tile
  const int span = (((np + kLW - 1) / kLW) + kWave - 1) & ~(kWave - 1);
  const int w_lo = min(np, wv * span);
  const int w_hi = min(np, w_lo + span);
  int* mycnt = cnt + wv * E1;
  for (int e = lane; e < E1; e += kWave) mycnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int i = w_lo + lane; i < w_hi; i += kWave) atomicAdd(&mycnt[ids[i]], 1);
  __syncthreads();

  // 4. first receive row of each (wave, bucket)
  for (int e = tid; e < E1; e += kLT) {
    int run = base[e];
    for (int w = 0; w < kLW; ++w) {
      const int c = cnt[w * E1 + e];
      cnt[w * E1 + e] = run;
      run += c;
    }
  }
  __syncthreads();

  // 5. stable rank, 64 pairs at a time (all lanes of the wave take part)
  const int R = a.T * a.K;
  const int nbits = 32 - __clz(a.E + 1);  // enough bits for ids 0..E+1
  for (int b0 = w_lo; b0 < w_hi; b0 += kWave) {
    const int i = b0 + lane;
    const bool act = i < w_hi;
    const int e = act ? (int)ids[i] : a.E + 1;
    uint64_t same = ~0ull;
    for (int bit = 0; bit < nbits; ++bit) {
      const int on = (e >> bit) & 1;
      const uint64_t bb = __ballot(on);
      same &= on ? bb : ~bb;
    }
    const int rank = __popcll(same & lanes_below(lane));
    int start = 0;
    if (act) start = mycnt[e];
    if (act) {
      const int pos = start + rank;
      const int64_t pair = p0 + i;
      if ((unsigned)pos < (unsigned)R) {
        const int t = (int)(pair / a.K);
        a.recv_pos[pair] = pos;
        a.recv_token[pos] = t;
        a.recv_k[pos] = (int)(pair - (int64_t)t * a.K);
      } else {
        atomicOr(a.status, MOE_STATUS_BAD_POSITION);
      }
    }
    // the highest lane of each group moves the counter past the group; the
    // wave barrier keeps the next round's reads after this write
    if (act && (same >> lane) == 1ull) mycnt[e] = start + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }

  // 6. token send slots, one token per thread per round: per partition, a
  //    ballot ranks the round's tokens inside each wave, and the per-wave
  //    counts give each wave its start
  for (int c0 = 0; c0 < nt; c0 += kLT) {  // uniform
    const int tt = c0 + tid;
    unsigned long long m = 0;
    if (tt < nt) {
      for (int k = 0; k < a.K; ++k) {
        const int e = ids[tt * a.K + k];
        if (e < a.E) m |= 1ull << (e / a.epr);
      }
    }
    for (int r = 0; r < a.P; ++r) {
      const uint64_t bal = __ballot((int)((m >> r) & 1ull));
      if (lane == 0) wcnt[wv * a.P + r] = __popcll(bal);
    }
    __syncthreads();
    for (int r = 0; r < a.P; ++r) {  // uniform: every lane takes part in the ballot
      const int on = (int)((m >> r) & 1ull);
      const uint64_t bal = __ballot(on);
      if (tt < nt) {
        int slot = -1;
        if (on) {
          slot = base[E1 + r] - off[E1 + r] + carry[r] + __popcll(bal & lanes_below(lane));
          for (int w = 0; w < wv; ++w) slot += wcnt[w * a.P + r];
        }
        a.token_slot[(size_t)(t0 + tt) * a.P + r] = slot;
      }
    }
    __syncthreads();
    for (int r = tid; r < a.P; r += kLT) {
      int s = 0;
      for (int w = 0; w < kLW; ++w) s += wcnt[w * a.P + r];
      carry[r] += s;
    }
    __syncthreads();
  }
}

}  // namespace

size_t layout_count_lds(int E, int P, int tile) {
  return (size_t)tile * 8 + (size_t)(E + 1 + P) * 4;
}

size_t layout_rank_lds(int E, int P, int tile, int K) {
  const size_t E1 = (size_t)E + 1, NR = E1 + P;
  const size_t ints = NR + (NR + 1) + kLW * E1 + kLW + (size_t)kLW * P + P;
  return ints * 4 + (size_t)tile * K * 2;
}

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(layout_count_kernel, dim3(a.nblk), dim3(kLT), layout_count_lds(a.E, a.P, a.tile),
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(layout_rank_kernel, dim3(a.nblk), dim3(kLT),
                     layout_rank_lds(a.E, a.P, a.tile, a.K), s, a);
  return hipGetLastError();
}

}  // namespace moe
