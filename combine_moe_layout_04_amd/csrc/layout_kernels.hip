// Layout of one routing decision: per-expert and per-partition counts,
// is_token_in_rank, prefix offsets, token send slots and stable receive
// positions.  Two launches over the same token tiles:
//
//   count: one thread per (t,k) pair: per-tile expert histogram (LDS
//          atomics: counts commute, so the result is deterministic),
//          per-token partition bitmask (LDS atomic OR), is_token_in_rank
//          bytes, per-tile partition token counts;
//   rank : global offsets and this tile's starts from one flat scan of the
//          tile histograms (bucket-major, tile-minor), then a
//          stable rank of every (t,k) pair among the pairs of its expert:
//          wave64 ballots match equal expert ids, a popcount over the lanes
//          below gives the rank inside 64 pairs, and per-(wave, expert)
//          running counters in LDS carry it across chunks and waves.
//          No position is ever taken from an atomic, so the result depends
//          on the routing alone (an activation-checkpoint replay of the same
//          routing reproduces it bit for bit).
//
// Ids outside [0,E) go to an extra bucket E, sorted after every expert, so
// that every position stays inside [0, T*K) even for bad input; the rank
// kernel raises MOE_STATUS_BAD_EXPERT for them.
#include "device_common.h"
#include "internal.h"
#include "../../include/moe_layout.h"

namespace moe {
namespace {

constexpr int kLT = 256;            // threads per layout workgroup
constexpr int kLW = kLT / kWave;    // waves per layout workgroup

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

size_t count_lds_bytes(int E, int P, int tile) {
  size_t ints = (size_t)(E + 1 + P);
  return ((ints * 4 + 7) & ~size_t(7)) + (size_t)tile * 8;
}

__global__ __launch_bounds__(kLT) void layout_count_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  int* eh = reinterpret_cast<int*>(smem);                 // [E+1]
  int* rh = eh + (a.E + 1);                                // [P]
  unsigned long long* msk = reinterpret_cast<unsigned long long*>(
      smem + ((size_t(a.E + 1 + a.P) * 4 + 7) & ~size_t(7)));  // [tile]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int t0 = b * a.tile;
  const int t1 = min(a.T, t0 + a.tile);
  const int nt = max(0, t1 - t0);
  for (int i = tid; i < a.E + 1 + a.P; i += kLT) eh[i] = 0;
  for (int i = tid; i < nt; i += kLT) msk[i] = 0ull;
  if (b == 0 && tid == 0) *a.status = 0;  // later kernels only OR bits in
  __syncthreads();

  // one thread per (t,k) pair: coalesced id loads, LDS histogram and masks
  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;
#pragma unroll 4
  for (int i = tid; i < np; i += kLT) {
    const int e = load_expert(a.idx, a.itype, p0 + i, a.E);
    atomicAdd(&eh[e], 1);
    if (e < a.E) atomicOr(&msk[i / a.K], 1ull << (e / a.epr));
  }
  __syncthreads();

  for (int tt = tid; tt < nt; tt += kLT) {
    unsigned long long m = msk[tt];
    a.tok_mask[t0 + tt] = m;
    while (m) {
      const int r = __ffsll(m) - 1;
      m &= m - 1;
      atomicAdd(&rh[r], 1);
    }
  }
  __syncthreads();

  for (int e = tid; e <= a.E; e += kLT) a.ehist[(size_t)e * a.nblk + b] = eh[e];
  for (int r = tid; r < a.P; r += kLT) a.rhist[(size_t)r * a.nblk + b] = rh[r];
  const int nbytes = nt * a.P;
  for (int i = tid; i < nbytes; i += kLT) {
    const int tt = i / a.P;
    const int r = i - tt * a.P;
    a.is_token_in_rank[(size_t)t0 * a.P + i] = (uint8_t)((msk[tt] >> r) & 1ull);
  }
}

// Exclusive scan, by the whole workgroup, of a [rows][nblk] histogram read
// row-major (row = bucket, column = tile).  At (row, j) the scan is the
// bucket's global start plus its count in the tiles before j.  Writes the
// scan's column `b` to col_b[rows], its column 0 to col_0[rows] and the total
// to col_0[rows].  Each thread scans a contiguous run (independent loads),
// then the 256 run sums are scanned across the workgroup.
__device__ void scan_histogram(const int* __restrict__ h, int rows, int nblk, int b, int* col_b,
                               int* col_0, int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int n = rows * nblk;
  const int per = (n + kLT - 1) / kLT;
  const int i0 = min(n, tid * per);
  const int i1 = min(n, i0 + per);
  int s = 0;
#pragma unroll 8
  for (int i = i0; i < i1; ++i) s += h[i];
  const int inc = wave_inclusive_scan(s);
  if (lane == kWave - 1) wsum[wv] = inc;
  __syncthreads();
  int run = inc - s;
  for (int w = 0; w < wv; ++w) run += wsum[w];
  int row = i0 / nblk;
  int j = i0 - row * nblk;
  for (int i = i0; i < i1; ++i) {
    if (j == 0) col_0[row] = run;
    if (j == b) col_b[row] = run;
    run += h[i];
    if (++j == nblk) {
      j = 0;
      ++row;
    }
  }
  if (i0 < i1 && i1 == n) col_0[rows] = run;
  __syncthreads();  // wsum is reused by the next scan
}

size_t rank_lds_ints(int E, int P) {
  const size_t E1 = (size_t)E + 1;
  return E1 /*base*/ + (E1 + 1) /*off*/ + kLW * E1 /*cnt*/ + P /*rbase*/ + (P + 1) /*soff*/ +
         kLW /*wsum*/ + (size_t)kWave * (P + 1) /*stage*/;
}

__global__ __launch_bounds__(kLT) void layout_rank_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  const int E1 = a.E + 1;
  int* base = reinterpret_cast<int*>(smem);  // [E+1] first row of each bucket in this tile
  int* off = base + E1;                      // [E+2] bucket offsets; off[E+1] = total
  int* cnt = off + (E1 + 1);                 // [kLW][E+1]
  int* rbase = cnt + kLW * E1;               // [P] this tile's first send row per partition
  int* soff = rbase + a.P;                   // [P+1] send offsets
  int* wsum = soff + (a.P + 1);              // [kLW]
  int* stage = wsum + kLW;                   // [64][P+1]

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;

  // 1-2. global offsets and this tile's starts, from the tile histograms
  scan_histogram(a.ehist, E1, a.nblk, b, base, off, wsum);
  scan_histogram(a.rhist, a.P, a.nblk, b, rbase, soff, wsum);

  // 3. global counts and offsets (tile 0 writes them)
  if (b == 0) {
    for (int e = tid; e < a.E; e += kLT) a.num_tokens_per_expert[e] = off[e + 1] - off[e];
    for (int e = tid; e <= a.E; e += kLT) a.expert_offset[e] = off[e];
    for (int r = tid; r <= a.P; r += kLT) a.rank_offset[r] = off[r * a.epr];
    for (int r = tid; r < a.P; r += kLT) a.num_tokens_per_rank[r] = soff[r + 1] - soff[r];
    for (int r = tid; r <= a.P; r += kLT) a.send_offset[r] = soff[r];
    if (tid == 0 && off[a.E + 1] != off[a.E]) atomicOr(a.status, MOE_STATUS_BAD_EXPERT);
  }

  // 4. per-wave bucket counts over contiguous pair ranges of this tile
  const int t0 = b * a.tile;
  const int t1 = min(a.T, t0 + a.tile);
  const int np = max(0, t1 - t0) * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;
  const int span = (((np + kLW - 1) / kLW) + kWave - 1) & ~(kWave - 1);
  const int w_lo = min(np, wv * span);
  const int w_hi = min(np, w_lo + span);
  int* mycnt = cnt + wv * E1;
  for (int e = lane; e < E1; e += kWave) mycnt[e] = 0;
  for (int i = w_lo + lane; i < w_hi; i += kWave)
    atomicAdd(&mycnt[load_expert(a.idx, a.itype, p0 + i, a.E)], 1);
  __syncthreads();

  // 5. first receive row of each (wave, bucket)
  for (int e = tid; e < E1; e += kLT) {
    int run = base[e];
    for (int w = 0; w < kLW; ++w) {
      const int c = cnt[w * E1 + e];
      cnt[w * E1 + e] = run;
      run += c;
    }
  }
  __syncthreads();

  // 6. stable rank, 64 pairs at a time (all lanes of the wave take part)
  const int R = a.T * a.K;
  const int nbits = 32 - __clz(a.E + 1);  // enough bits for ids 0..E+1
  for (int base = w_lo; base < w_hi; base += kWave) {
    const int i = base + lane;
    const bool act = i < w_hi;
    const int e = act ? load_expert(a.idx, a.itype, p0 + i, a.E) : a.E + 1;
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
        a.recv_pos[pair] = pos;
        a.recv_token[pos] = (int)(pair / a.K);
        a.recv_k[pos] = (int)(pair - (pair / a.K) * a.K);
      } else {
        atomicOr(a.status, MOE_STATUS_BAD_POSITION);
      }
    }
    // the highest lane of each group moves the counter past the group; the
    // wave barrier keeps the next round's reads after this write
    if (act && (same >> lane) == 1ull) mycnt[e] = start + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }

  // 7. token send slots, one wave, 64 tokens at a time
  if (wv == 0) {
    for (int c0 = t0; c0 < t1; c0 += kWave) {
      const int t = c0 + lane;
      const bool act = t < t1;
      const unsigned long long m = act ? a.tok_mask[t] : 0ull;
      for (int r = 0; r < a.P; ++r) {
        const int on = (int)((m >> r) & 1ull);
        const uint64_t bal = __ballot(on);
        const int run = rbase[r];
        stage[lane * (a.P + 1) + r] = on ? run - soff[r] + __popcll(bal & lanes_below(lane)) : -1;
        if (lane == 0) rbase[r] = run + __popcll(bal);
        __builtin_amdgcn_wave_barrier();
      }
      const int nt = min(kWave, t1 - c0);
      for (int j = lane; j < nt * a.P; j += kWave) {
        const int tt = j / a.P;
        const int r = j - tt * a.P;
        a.token_slot[(size_t)c0 * a.P + j] = stage[tt * (a.P + 1) + r];
      }
      __builtin_amdgcn_wave_barrier();  // stage is rewritten by the next round
    }
  }
}

}  // namespace

hipError_t launch_layout(const LayoutArgs& a, hipStream_t s) {
  const size_t lds_a = count_lds_bytes(a.E, a.P, a.tile);
  const size_t lds_b = rank_lds_ints(a.E, a.P) * 4;
  hipLaunchKernelGGL(layout_count_kernel, dim3(a.nblk), dim3(kLT), lds_a, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(layout_rank_kernel, dim3(a.nblk), dim3(kLT), lds_b, s, a);
  return hipGetLastError();
}

size_t layout_lds_bytes_max(int E, int P, int tile) {
  const size_t a = count_lds_bytes(E, P, tile);
  const size_t b = rank_lds_ints(E, P) * 4;
  return a > b ? a : b;
}

}  // namespace moe
