// Layout of one routing decision: per-expert and per-partition counts,
// is_token_in_rank, prefix offsets, token send slots and stable receive
// positions.  Two launches over the same token tiles; a tile holds at most
// 512 (t,k) pairs, one per thread of a 512-thread workgroup, so each wave
// ranks one round of 64 pairs and a layer spreads over many CUs (beyond 128
// tiles, for very large T, a tile holds more pairs and each wave loops):
//
//   count: one thread per (t,k) pair: per-tile expert histogram (LDS
//          atomics: counts commute, so the result is deterministic),
//          per-token partition bitmask (LDS atomic OR), is_token_in_rank,
//          per-tile partition token counts.  Each tile writes one contiguous
//          row of a [tiles][E+1+P] histogram, and its tokens' masks.
//   rank : every histogram column's total and its count in the tiles before
//          this one (one thread per (column, tile range), all its loads in
//          flight), then one workgroup scan over the columns: every global
//          offset and this tile's starts.  Token send slots come from
//          per-partition ballots over the tile's tokens (with send_token,
//          their inverse).  Each wave ranks a contiguous span of pairs:
//          wave64 ballots match equal ids, a popcount over the lanes below
//          gives the rank inside 64 pairs, and per-(wave, expert) first rows
//          place the waves.  No position is ever taken from an atomic, so
//          the result depends on the routing alone (an activation-checkpoint
//          replay of the same routing reproduces it bit for bit).  Global
//          stores come after the last workgroup barrier: a barrier waits for
//          the workgroup's outstanding memory operations.
//          Two forms: layout_rank_wave_kernel for the usual tile (at most 512
//          pairs, one per thread, so each wave holds one span of 64, and at
//          most 512 columns), with three workgroup barriers; and
//          layout_rank_kernel for larger tiles, which stages the ids in LDS
//          and carries per-(wave, expert) cursors across rounds.
//
// A layout of one tile (at most 512 pairs) is one launch: the wave form of
// the rank kernel does the count itself.
//
// Beyond 128 tiles (and 24576 tiles x columns) a third launch sits between
// the two: layout_scan_kernel rewrites the histogram once into per-tile
// column prefixes and a row of totals, which each rank workgroup reads
// instead of summing every tile (that sum would make the layout quadratic in
// the tile count).
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
constexpr int kColRegs = 64;         // histogram tiles a scan thread loads at once
// Above this many tiles, and tiles x columns, the histogram's columns are
// scanned once, by layout_scan_kernel, instead of by every rank workgroup
// (whose column sums over all tiles would make the layout quadratic in the
// tile count).  Measured per layout against the unscanned form: at E = 128,
// P = 8 (137 columns) 84.6 vs 81.9 us at 130 tiles, level at 196, 178 vs 184
// at 293; at E = 256, P = 64 (321 columns) 204.4 vs 207.2 at 130 tiles.
constexpr int kScanTiles = 128;
constexpr int64_t kScanWork = 24576;  // tiles x columns
constexpr int kScanBatch = 16;       // tiles a column-scan lane loads at once
constexpr int kIdRegs = 2;           // tile ids a thread loads before the scan
// token slots of a tile of at most 64 tokens: ballots per wave, and at most
// this many rounds of the block over the tile's [tokens][P] items
constexpr int kSlotBallots = (MOE_MAX_P + kLW - 1) / kLW;
constexpr int kSlotRounds = (kWave * MOE_MAX_P + kLT - 1) / kLT;
static_assert(kSlotRounds == 8, "the rank kernel's round switch covers 1..8 rounds");

__device__ __forceinline__ int clamp_id(long long v, int E) { return (v >= 0 && v < E) ? (int)v : E; }

__device__ __forceinline__ int load_expert(const void* idx, int itype, int64_t i, int E) {
  if (itype == MOE_I32) return clamp_id(static_cast<const int*>(idx)[i], E);
  return clamp_id(static_cast<const long long*>(idx)[i], E);
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
  const int NR = E1 + a.P;
  unsigned long long* msk = reinterpret_cast<unsigned long long*>(smem);  // [tile]
  int* eh = reinterpret_cast<int*>(msk + a.tile);                        // [E+1]
  int* rh = eh + E1;                                                     // [P]
  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  const int t0 = b * a.tile;
  const int nt = max(0, min(a.T, t0 + a.tile) - t0);
  for (int i = tid; i < NR; i += kLT) eh[i] = 0;
  for (int i = tid; i < nt; i += kLT) msk[i] = 0ull;
  __syncthreads();

  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;
#pragma unroll 4
  for (int i = tid; i < np; i += kLT) {
    const int e = load_expert(a.idx, a.itype, p0 + i, a.E);
    atomicAdd(&eh[e], 1);
    if (e < a.E) atomicOr(&msk[i / a.K], 1ull << (e / a.epr));
  }
  __syncthreads();

  if (nt <= kWave) {  // uniform: lane = token; one ballot per partition, spread over the waves
    const int lane = tid & (kWave - 1);
    const unsigned long long m = lane < nt ? msk[lane] : 0ull;
    for (int r = tid / kWave; r < a.P; r += kLW) {
      const int c = __popcll(__ballot((int)((m >> r) & 1ull)));
      if (lane == 0) rh[r] = c;
    }
  } else {
    for (int tt = tid; tt < nt; tt += kLT) {
      unsigned long long m = msk[tt];
      while (m) {
        const int r = __ffsll(m) - 1;
        m &= m - 1;
        atomicAdd(&rh[r], 1);
      }
    }
  }
  __syncthreads();  // before any global store (a barrier would wait for them)

  for (int tt = tid; tt < nt; tt += kLT) a.tok_mask[t0 + tt] = msk[tt];
  const int nbytes = nt * a.P;
  for (int i = tid; i < nbytes; i += kLT) {
    const int tt = i / a.P;
    a.is_token_in_rank[(size_t)t0 * a.P + i] = (uint8_t)((msk[tt] >> (i - tt * a.P)) & 1ull);
  }
  for (int r = tid; r < NR; r += kLT) a.hist[(size_t)b * NR + r] = eh[r];
  if (b == 0 && tid == 0) *a.status = 0;  // later kernels only OR bits in
}

// ---- rank -------------------------------------------------------------------

// Column sums of the histogram over the tile ranges of scan_histogram: item
// (q, r) sums column r over tiles [q*cpp, (q+1)*cpp), in batches of L
// clamped, unconditional loads (no branch waits on a load, so a batch is in
// flight together); the total goes to part[q][r], the tiles before b to
// part[parts + q][r].
template <int L>
__device__ __forceinline__ void column_sums(const int* __restrict__ h, int NR, int nblk, int b, int parts, int cpp,
                                            int* part) {
  for (int item = threadIdx.x; item < NR * parts; item += kLT) {
    const int q = item / NR;
    const int r = item - q * NR;
    const int j0 = q * cpp;
    const int j1 = min(nblk, j0 + cpp);
    int tot = 0, pre = 0;
    for (int c0 = j0; c0 < j1; c0 += L) {
      int v[L];
#pragma unroll
      for (int u = 0; u < L; ++u) v[u] = h[(size_t)min(c0 + u, j1 - 1) * NR + r];
#pragma unroll
      for (int u = 0; u < L; ++u) {
        const int x = (c0 + u < j1) ? v[u] : 0;
        tot += x;
        pre += (c0 + u < b) ? x : 0;
      }
    }
    part[q * NR + r] = tot;
    part[(parts + q) * NR + r] = pre;
  }
}

// column_sums with a batch of loads sized to the tiles each thread sums,
// rounded up a short ladder.
__device__ __forceinline__ void all_column_sums(const int* __restrict__ h, int NR, int nblk, int b, int parts,
                                                int* part) {
  const int cpp = (nblk + parts - 1) / parts;  // tiles per thread
  if (cpp <= 4)
    column_sums<4>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 8)
    column_sums<8>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 12)
    column_sums<12>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 16)
    column_sums<16>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 24)
    column_sums<24>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 32)
    column_sums<32>(h, NR, nblk, b, parts, cpp, part);
  else if (cpp <= 48)
    column_sums<48>(h, NR, nblk, b, parts, cpp, part);
  else
    column_sums<kColRegs>(h, NR, nblk, b, parts, cpp, part);
}

// Start of every histogram column, globally and at tile b.  The histogram is
// tile-major, h[j * NR + r]: count of column r (a bucket, then a partition)
// in tile j.  Writes col_n[r] = column r's total, col_0[r] = sum of all
// columns before r (col_0[NR] = the total) and col_b[r] = col_0[r] + column
// r's count in the tiles before b.  The first npad columns (the experts)
// take pad * ceil(total / pad) rows in the running sum: padded segments.
// Each thread sums a range of tiles of one column with all its loads in
// flight (clamped, unconditional loads); a workgroup scan over the column
// totals follows.  part: LDS [2][parts][NR].  Ends with a barrier.
// A scanned histogram (scanned != 0, parts == 1) already holds each column's
// count in the tiles before b (row b) and its total (row nblk): two loads.
__device__ void scan_histogram(const int* __restrict__ h, int NR, int nblk, int b, int npad, int pad,
                               int parts, int scanned, int* col_b, int* col_0, int* col_n, int* part,
                               int* wsum) {
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  if (scanned) {
    for (int r = tid; r < NR; r += kLT) {
      part[r] = h[(size_t)nblk * NR + r];
      part[NR + r] = h[(size_t)b * NR + r];
    }
  } else {
    all_column_sums(h, NR, nblk, b, parts, part);
  }
  __syncthreads();
  int carry = 0;
  for (int c0 = 0; c0 < NR; c0 += kLT) {  // uniform
    const int r = c0 + tid;
    int tot = 0, pre = 0;
    if (r < NR) {
      for (int q = 0; q < parts; ++q) {
        tot += part[q * NR + r];
        pre += part[(parts + q) * NR + r];
      }
    }
    const int seg = r < npad ? (tot + pad - 1) / pad * pad : tot;  // rows the column takes
    const int inc = wave_inclusive_scan(seg);
    if (lane == kWave - 1) wsum[wv] = inc;
    __syncthreads();
    int st = carry + inc - seg, all = 0;
#pragma unroll
    for (int w = 0; w < kLW; ++w) {
      const int ws = wsum[w];
      if (w < wv) st += ws;
      all += ws;
    }
    if (r < NR) {
      col_0[r] = st;
      col_b[r] = st + pre;
      col_n[r] = tot;
    }
    carry += all;
    __syncthreads();  // wsum is rewritten by the next chunk
  }
  if (tid == 0) col_0[NR] = carry;
  __syncthreads();
}

// Token slots of a tile of at most 64 tokens, from colm[r] (the tile's
// tokens in partition r, one bit per token): item i of the block is (token
// i / P, partition i % P) for token_slot, a contiguous [tokens][P] block, and
// (partition i / nt, token i % nt) for send_token, partition by partition.
// NR rounds of kLT items, unrolled: both indices advance by kLT per round
// without a division, every round's LDS reads are issued unconditionally
// (clamped) and only the stores are guarded.
template <int NR>
__device__ __forceinline__ void write_slots(const LayoutArgs& a, const unsigned long long* colm, const int* base,
                                            const int* off, int t0, int nt) {
  const int tid = threadIdx.x;
  const int E1 = a.E + 1;
  const int nitems = nt * a.P;
  const int ntd = max(nt, 1);
  int tq = tid / a.P, tr = tid - (tid / a.P) * a.P;  // token-major
  int sr = tid / ntd, st = tid - (tid / ntd) * ntd;  // partition-major
  const int dq = kLT / a.P, dr = kLT - (kLT / a.P) * a.P;
  const int ds = kLT / ntd, dt = kLT - (kLT / ntd) * ntd;
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    const int i = tid + j * kLT;
    {  // past the items (i >= nitems) the token index is clamped, not stored
      const int r = tr;
      const int q = min(tq, kWave - 1);
      const uint64_t bal = colm[r];
      const int slot = base[E1 + r] - off[E1 + r] + __popcll(bal & lanes_below(q));
      if (i < nitems) a.token_slot[(size_t)t0 * a.P + i] = ((bal >> q) & 1ull) ? slot : -1;
    }
    {
      const int r = min(sr, a.P - 1);
      const uint64_t bal = colm[r];
      const int row = base[E1 + r] - off[E1] + __popcll(bal & lanes_below(st));
      if (i < nitems && ((bal >> st) & 1ull)) a.send_token[row] = t0 + st;
    }
    tq += dq;
    tr += dr;
    if (tr >= a.P) { tr -= a.P; ++tq; }
    sr += ds;
    st += dt;
    if (st >= ntd) { st -= ntd; ++sr; }
  }
}

// ---- column scan of a histogram of many tiles --------------------------------
//
// One workgroup per 64 histogram columns, lane = column; its eight waves
// split the tiles into eight contiguous ranges.  Each wave sums its range,
// the waves' sums are scanned through LDS, and each wave walks its range
// again writing, in place, every tile's exclusive prefix (the column's count
// in the tiles before it); row nblk gets the column totals.  Each histogram
// entry is read and written by one thread only.  Linear in the tile count;
// the loads of a lane are batched, clamped and unconditional.
__global__ __launch_bounds__(kLT) void layout_scan_kernel(LayoutArgs a) {
  __shared__ int wpart[kLW][kWave];
  const int NR = a.E + 1 + a.P;
  const int lane = lane_id();
  const int w = (int)(threadIdx.x / kWave);
  const int c = blockIdx.x * kWave + lane;
  const int cc = min(c, NR - 1);  // clamped column for the loads
  const int nb = a.nblk;
  const int ch = (nb + kLW - 1) / kLW;
  const int j0 = min(nb, w * ch), j1 = min(nb, j0 + ch);
  int* h = a.hist;
  int sum = 0;
  for (int j = j0; j < j1; j += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) v[u] = h[(size_t)min(j + u, j1 - 1) * NR + cc];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) sum += (j + u < j1) ? v[u] : 0;
  }
  wpart[w][lane] = sum;
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int q = 0; q < kLW; ++q) run += (q < w) ? wpart[q][lane] : 0;
  for (int j = j0; j < j1; j += kScanBatch) {
    int v[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) v[u] = h[(size_t)min(j + u, j1 - 1) * NR + cc];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      if (c < NR && j + u < j1) {
        h[(size_t)(j + u) * NR + c] = run;
        run += v[u];
      }
    }
  }
  if (w == kLW - 1 && c < NR) h[(size_t)nb * NR + c] = run;  // the last range ends at the total
}

__global__ __launch_bounds__(kLT) void layout_rank_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  const int E1 = a.E + 1;
  const int NR = E1 + a.P;                   // histogram columns
  const int parts = a.scanned ? 1 : max(1, min(a.nblk, kLT / NR));  // threads per column of the scan
  unsigned long long* colm = reinterpret_cast<unsigned long long*>(smem);  // [P] tokens of the tile in partition r
  int* base = reinterpret_cast<int*>(colm + a.P);  // [NR]   this tile's start of each column
  int* off = base + NR;                      // [NR+1] start of each column, tile 0
  int* cnt = off + NR + 1;                   // [kLW][E+1] per-wave bucket cursors
  int* wsum = cnt + kLW * E1;                // [kLW]
  int* wcnt = wsum + kLW;                    // [kLW][P] per-wave partition counts
  int* wpre = wcnt + kLW * a.P;              // [kLW][P] slots before each wave
  int* carry = wpre + kLW * a.P;             // [P] slots used by earlier token rounds
  int* coln = carry + a.P;                   // [NR] column totals (unpadded)
  int* part = coln + NR;                     // [2][parts][NR] scan partials
  uint16_t* ids = reinterpret_cast<uint16_t*>(part + 2 * parts * NR);  // [tile*K]

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int t0 = b * a.tile;
  const int nt = max(0, min(a.T, t0 + a.tile) - t0);
  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;

  // 0. loads whose round trips overlap the scan's: the first kIdRegs ids of
  //    each thread and the first round's token masks (clamped, unconditional
  //    loads; the range checks are applied later)
  long long idv[kIdRegs];
  unsigned long long m0 = 0ull;
  if (np > 0) {  // uniform
    if (a.itype == MOE_I32) {
      const int* src = static_cast<const int*>(a.idx) + p0;
#pragma unroll
      for (int u = 0; u < kIdRegs; ++u) idv[u] = src[min(tid + u * kLT, np - 1)];
    } else {
      const long long* src = static_cast<const long long*>(a.idx) + p0;
#pragma unroll
      for (int u = 0; u < kIdRegs; ++u) idv[u] = src[min(tid + u * kLT, np - 1)];
    }
    // a tile of at most 64 tokens: every wave holds token `lane`'s mask
    m0 = a.tok_mask[t0 + min(nt <= kWave ? lane : tid, nt - 1)];
  }
  for (int r = tid; r < a.P; r += kLT) carry[r] = 0;

  // 1. global offsets and this tile's starts (the scan ends with a barrier)
  scan_histogram(a.hist, NR, a.nblk, b, a.E, a.pad, parts, a.scanned, base, off, coln, part, wsum);
#pragma unroll
  for (int u = 0; u < kIdRegs; ++u) {
    const int i = tid + u * kLT;
    if (i < np) ids[i] = (uint16_t)clamp_id(idv[u], a.E);
  }
  for (int i = tid + kIdRegs * kLT; i < np; i += kLT)
    ids[i] = (uint16_t)load_expert(a.idx, a.itype, p0 + i, a.E);
  __syncthreads();

  // 2. per-wave bucket counts over contiguous pair spans of the tile
  const int span = (((np + kLW - 1) / kLW) + kWave - 1) & ~(kWave - 1);
  const int w_lo = min(np, wv * span);
  const int w_hi = min(np, w_lo + span);
  int* mycnt = cnt + wv * E1;
  for (int e = lane; e < E1; e += kWave) mycnt[e] = 0;
  __builtin_amdgcn_wave_barrier();
  for (int i = w_lo + lane; i < w_hi; i += kWave) atomicAdd(&mycnt[ids[i]], 1);
  __syncthreads();

  // 3. first receive row of each (wave, bucket)
  for (int e = tid; e < E1; e += kLT) {
    int c[kLW];
#pragma unroll
    for (int w = 0; w < kLW; ++w) c[w] = cnt[w * E1 + e];
    int run = base[e];
#pragma unroll
    for (int w = 0; w < kLW; ++w) {
      cnt[w * E1 + e] = run;
      run += c[w];
    }
  }
  __syncthreads();

  // 4. token send slots: per partition, a ballot over the tokens ranks them.
  //    A tile of at most 64 tokens (the usual case) takes one ballot per
  //    partition, the partitions spread over the waves; a token's slot is
  //    then the popcount of its partition's ballot below it, so the tile's
  //    [tokens][P] block of token_slot is written contiguously (coalesced)
  //    and send_token partition by partition (neighbouring send rows).  A
  //    larger tile takes one token per thread per round, with a table of
  //    per-wave starts that places the waves
  if (nt <= kWave) {  // uniform
    const unsigned long long m = lane < nt ? m0 : 0ull;
#pragma unroll
    for (int j = 0; j < kSlotBallots; ++j) {
      const int r = wv + j * kLW;
      if (r < a.P) {  // uniform
        const uint64_t bal = __ballot((int)((m >> r) & 1ull));
        if (lane == 0) colm[r] = bal;
      }
    }
    __syncthreads();  // no global store is outstanding here
    switch ((nt * a.P + kLT - 1) / kLT) {  // uniform: rounds of the block over the tile's items
      case 1: write_slots<1>(a, colm, base, off, t0, nt); break;
      case 2: write_slots<2>(a, colm, base, off, t0, nt); break;
      case 3: write_slots<3>(a, colm, base, off, t0, nt); break;
      case 4: write_slots<4>(a, colm, base, off, t0, nt); break;
      case 5: write_slots<5>(a, colm, base, off, t0, nt); break;
      case 6: write_slots<6>(a, colm, base, off, t0, nt); break;
      case 7: write_slots<7>(a, colm, base, off, t0, nt); break;
      default: write_slots<kSlotRounds>(a, colm, base, off, t0, nt); break;
    }
  } else {
  for (int c0 = 0; c0 < nt; c0 += kLT) {  // uniform
    const int tt = c0 + tid;
    const unsigned long long m = tt < nt ? (c0 == 0 ? m0 : a.tok_mask[t0 + tt]) : 0ull;
    for (int r = 0; r < a.P; ++r) {
      const uint64_t bal = __ballot((int)((m >> r) & 1ull));
      if (lane == 0) wcnt[wv * a.P + r] = __popcll(bal);
    }
    __syncthreads();
    for (int item = tid; item < kLW * a.P; item += kLT) {
      const int w = item / a.P;
      const int r = item - w * a.P;
      int s = carry[r] + base[E1 + r] - off[E1 + r];
#pragma unroll
      for (int u = 0; u < kLW; ++u) {
        const int c = wcnt[u * a.P + r];
        if (u < w) s += c;
      }
      wpre[item] = s;
    }
    __syncthreads();
    for (int r = 0; r < a.P; ++r) {  // uniform: every lane takes part in the ballot
      const int on = (int)((m >> r) & 1ull);
      const uint64_t bal = __ballot(on);
      const int slot = wpre[wv * a.P + r] + __popcll(bal & lanes_below(lane));
      if (tt < nt) {
        a.token_slot[(size_t)(t0 + tt) * a.P + r] = on ? slot : -1;
        if (on) a.send_token[off[E1 + r] - off[E1] + slot] = t0 + tt;
      }
    }
    if (c0 + kLT < nt) {  // more rounds (very large tiles only): carry the counts
      for (int r = tid; r < a.P; r += kLT)
        carry[r] = wpre[(kLW - 1) * a.P + r] + wcnt[(kLW - 1) * a.P + r] - (base[E1 + r] - off[E1 + r]);
      __syncthreads();
    }
  }
  }

  // 5. stable rank, 64 pairs at a time (all lanes of the wave take part)
  const int R = a.R;
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
        const int tq = i / a.K;
        a.recv_pos[pair] = pos;
        a.recv_token[pos] = t0 + tq;
        a.recv_k[pos] = i - tq * a.K;
      } else {
        atomicOr(a.status, MOE_STATUS_BAD_POSITION);
      }
    }
    // the highest lane of each group moves the cursor past the group; the
    // wave barrier keeps the next round's reads after this write
    if (act && (same >> lane) == 1ull) mycnt[e] = start + __popcll(same);
    __builtin_amdgcn_wave_barrier();
  }

  // 6. padded layouts: receive rows that hold no pair get -1 in the inverse
  //    maps; the padding after each expert's pairs (experts strided over the
  //    tiles), then the rows after the last bucket (split over the tiles)
  if (a.pad > 1) {  // uniform
    for (int e = b; e < a.E; e += a.nblk) {
      const int hi = min(off[e + 1], R);
      for (int p = off[e] + coln[e] + tid; p < hi; p += kLT) {
        a.recv_token[p] = -1;
        a.recv_k[p] = -1;
      }
    }
    for (int p = off[E1] + b * kLT + tid; p < R; p += a.nblk * kLT) {
      a.recv_token[p] = -1;
      a.recv_k[p] = -1;
    }
  }

  // 7. global counts, offsets and status (tile 0 writes them)
  if (b == 0) {
    const int total = off[E1];  // the bucket columns come first
    for (int e = tid; e < a.E; e += kLT) a.num_tokens_per_expert[e] = coln[e];
    for (int e = tid; e <= a.E; e += kLT) a.expert_offset[e] = off[e];
    for (int r = tid; r <= a.P; r += kLT) a.rank_offset[r] = off[r * a.epr];
    for (int r = tid; r < a.P; r += kLT) a.num_tokens_per_rank[r] = off[E1 + r + 1] - off[E1 + r];
    for (int r = tid; r <= a.P; r += kLT) a.send_offset[r] = off[E1 + r] - total;
    if (tid == 0 && off[a.E + 1] != off[a.E]) atomicOr(a.status, MOE_STATUS_BAD_EXPERT);
  }
}

// ---- rank, one round of 64 pairs per wave --------------------------------------
//
// The usual case: a tile of at most kLT pairs (one per thread, so wave w holds
// pairs [64w, 64w+64) of the tile) and at most kLT histogram columns.  The
// results equal layout_rank_kernel's, with three workgroup barriers instead of
// about seven: what depends on the tile alone (each pair's rank among the equal
// ids of its wave, the wave's bucket counts, the tile's token masks, the token
// ballots) is done before or beside the scan, and the scan's last step also
// turns the wave counts into each (wave, bucket)'s first receive row.

// kOne: the whole layout is this one tile (T*K <= 512 pairs, one launch
// instead of two).  The tile's counts and token masks are then made here
// instead of read from the count kernel's global arrays: each token's thread
// builds its mask from its K ids, each wave counts its tokens per partition
// by ballots, and the bucket totals are the waves' bucket counts.  This
// kernel also writes the count kernel's outputs: tok_mask, is_token_in_rank
// and the cleared status.
template <bool kOne>
__global__ __launch_bounds__(kLT) void layout_rank_wave_kernel(LayoutArgs a) {
  extern __shared__ __align__(8) unsigned char smem[];
  const int E1 = a.E + 1;
  const int NR = E1 + a.P;  // histogram columns, at most kLT here
  const int parts = max(1, min(a.nblk, kLT / NR));
  const int ngmax = (a.tile + kWave - 1) / kWave;  // token groups of 64 in a tile
  unsigned long long* colm = reinterpret_cast<unsigned long long*>(smem);  // [ngmax][P] group g's tokens in r
  unsigned long long* tm = colm + ngmax * a.P;   // [tile] the tile's token masks
  int* base = reinterpret_cast<int*>(tm + a.tile);  // [NR]   this tile's start of each column
  int* off = base + NR;                          // [NR+1] start of each column, tile 0
  int* coln = off + NR + 1;                      // [NR]   column totals (unpadded)
  int* cnt = coln + NR;                          // [kLW][E+1] wave bucket counts, then first rows
  int* wsum = cnt + kLW * E1;                    // [kLW]
  int* part = wsum + kLW;                        // [2][parts][NR] column partial sums

  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wv = tid / kWave;
  const int t0 = b * a.tile;
  const int nt = max(0, min(a.T, t0 + a.tile) - t0);
  const int np = nt * a.K;
  const int64_t p0 = (int64_t)t0 * a.K;

  // 0. this thread's pair and token mask: their round trips overlap the
  //    histogram's.  Threads without a pair take an id no pair has.
  const int e = tid < np ? load_expert(a.idx, a.itype, p0 + tid, a.E) : a.E + 1;
  const unsigned long long mk = (!kOne && tid < nt) ? a.tok_mask[t0 + tid] : 0ull;
  int* mycnt = cnt + wv * E1;
  for (int j = lane; j < E1; j += kWave) mycnt[j] = 0;
  if constexpr (kOne) {
    // The status word is cleared by an exchange whose result thread 0 keeps:
    // it has completed before barrier (1), so before any later OR into it.
    if (tid == 0) wsum[0] = atomicExch(a.status, 0);
    unsigned long long m = 0ull;
    if (tid < nt) {
      for (int k = 0; k < a.K; ++k) {
        const int ek = load_expert(a.idx, a.itype, (int64_t)tid * a.K + k, a.E);
        if (ek < a.E) m |= 1ull << (ek / a.epr);
      }
      tm[tid] = m;
    }
    int* wrc = part;  // [kLW][P] this wave's tokens per partition
    for (int r = 0; r < a.P; ++r) {  // uniform
      const int c = __popcll(__ballot((int)((m >> r) & 1ull)));
      if (lane == 0) wrc[wv * a.P + r] = c;
    }
  } else {
    // 1. column sums of the histogram, all of a thread's loads in flight
    all_column_sums(a.hist, NR, a.nblk, b, parts, part);
  }

  // 2. rank among the equal ids of this wave (wave64 ballots over the id
  //    bits), and the wave's count of each bucket, written by the highest
  //    lane of each group of equal ids
  const int nbits = 32 - __clz(a.E + 1);  // enough bits for ids 0..E+1
  uint64_t same = ~0ull;
  for (int bit = 0; bit < nbits; ++bit) {
    const int on = (e >> bit) & 1;
    const uint64_t bb = __ballot(on);
    same &= on ? bb : ~bb;
  }
  const int rank = __popcll(same & lanes_below(lane));
  __builtin_amdgcn_wave_barrier();  // the wave's row is cleared before its counts land
  if (tid < np && (same >> lane) == 1ull) mycnt[e] = __popcll(same);
  if (!kOne && tid < nt) tm[tid] = mk;
  __syncthreads();  // (1)

  // 3. the scan's first half: each column's total, its count in the tiles
  //    before this one, and the rows it takes (padded for the experts); a
  //    wave scan over the columns.  Beside it, one ballot per (token group,
  //    partition) over the tile's token masks, spread over the waves.
  int tot = 0, pre = 0;
  if (tid < NR) {
    if constexpr (kOne) {  // one tile: its own counts are the totals, nothing comes before it
      if (tid < E1) {
#pragma unroll
        for (int w = 0; w < kLW; ++w) tot += cnt[w * E1 + tid];
      } else {
#pragma unroll
        for (int w = 0; w < kLW; ++w) tot += part[w * a.P + tid - E1];
      }
    } else {
      for (int q = 0; q < parts; ++q) {
        tot += part[q * NR + tid];
        pre += part[(parts + q) * NR + tid];
      }
    }
  }
  const int seg = (tid < a.E) ? (tot + a.pad - 1) / a.pad * a.pad : tot;  // rows the column takes
  const int inc = wave_inclusive_scan(seg);
  if (lane == kWave - 1) wsum[wv] = inc;
  const int ng = (nt + kWave - 1) / kWave;
  for (int j = wv; j < ng * a.P; j += kLW) {  // uniform per wave
    const int g = j / a.P;
    const int r = j - g * a.P;
    const int t = g * kWave + lane;
    const unsigned long long m = t < nt ? tm[t] : 0ull;
    const uint64_t bal = __ballot((int)((m >> r) & 1ull));
    if (lane == 0) colm[j] = bal;
  }
  __syncthreads();  // (2)

  // 4. every column's start, globally (off) and at this tile (base); for the
  //    buckets, each (wave, bucket)'s first receive row: the tile's start
  //    plus the wave counts of the tile's earlier waves
  if (tid < NR) {
    int st = inc - seg;
#pragma unroll
    for (int w = 0; w < kLW; ++w) {
      const int ws = wsum[w];
      if (w < wv) st += ws;
    }
    off[tid] = st;
    base[tid] = st + pre;
    coln[tid] = tot;
    if (tid == NR - 1) off[NR] = st + seg;
    if (tid < E1) {
      int run = st + pre;
#pragma unroll
      for (int w = 0; w < kLW; ++w) {
        const int c = cnt[w * E1 + tid];
        cnt[w * E1 + tid] = run;
        run += c;
      }
    }
  }
  __syncthreads();  // (3): global stores only from here on

  // 5. stable receive positions
  const int R = a.R;
  if (tid < np) {
    const int pos = cnt[wv * E1 + e] + rank;
    if ((unsigned)pos < (unsigned)R) {
      const int tq = tid / a.K;
      a.recv_pos[p0 + tid] = pos;
      a.recv_token[pos] = t0 + tq;
      a.recv_k[pos] = tid - tq * a.K;
    } else {
      atomicOr(a.status, MOE_STATUS_BAD_POSITION);
    }
  }

  // 6. token send slots and their inverse
  if (nt <= kWave) {  // uniform: one token group, the unrolled store rounds
    switch ((nt * a.P + kLT - 1) / kLT) {
      case 0: break;
      case 1: write_slots<1>(a, colm, base, off, t0, nt); break;
      case 2: write_slots<2>(a, colm, base, off, t0, nt); break;
      case 3: write_slots<3>(a, colm, base, off, t0, nt); break;
      case 4: write_slots<4>(a, colm, base, off, t0, nt); break;
      case 5: write_slots<5>(a, colm, base, off, t0, nt); break;
      case 6: write_slots<6>(a, colm, base, off, t0, nt); break;
      case 7: write_slots<7>(a, colm, base, off, t0, nt); break;
      default: write_slots<kSlotRounds>(a, colm, base, off, t0, nt); break;
    }
  } else {  // several groups of 64 tokens: a token's slot adds the earlier groups' counts
    for (int i = tid; i < nt * a.P; i += kLT) {
      const int tt = i / a.P;
      const int r = i - tt * a.P;
      const int g = tt / kWave;
      const int l = tt - g * kWave;
      int before = 0;
      for (int gg = 0; gg < g; ++gg) before += __popcll(colm[gg * a.P + r]);
      const uint64_t bal = colm[g * a.P + r];
      const int slot = base[E1 + r] - off[E1 + r] + before + __popcll(bal & lanes_below(l));
      const bool on = (bal >> l) & 1ull;
      a.token_slot[(size_t)t0 * a.P + i] = on ? slot : -1;
      if (on) a.send_token[off[E1 + r] - off[E1] + slot] = t0 + tt;
    }
  }

  // 7. padded layouts: receive rows that hold no pair get -1 in the inverse maps
  if (a.pad > 1) {  // uniform
    for (int x = b; x < a.E; x += a.nblk) {
      const int hi = min(off[x + 1], R);
      for (int p = off[x] + coln[x] + tid; p < hi; p += kLT) {
        a.recv_token[p] = -1;
        a.recv_k[p] = -1;
      }
    }
    for (int p = off[E1] + b * kLT + tid; p < R; p += a.nblk * kLT) {
      a.recv_token[p] = -1;
      a.recv_k[p] = -1;
    }
  }

  // 8. global counts, offsets and status (tile 0 writes them)
  if (b == 0) {
    const int total = off[E1];  // the bucket columns come first
    for (int x = tid; x < a.E; x += kLT) a.num_tokens_per_expert[x] = coln[x];
    for (int x = tid; x <= a.E; x += kLT) a.expert_offset[x] = off[x];
    for (int r = tid; r <= a.P; r += kLT) a.rank_offset[r] = off[r * a.epr];
    for (int r = tid; r < a.P; r += kLT) a.num_tokens_per_rank[r] = off[E1 + r + 1] - off[E1 + r];
    for (int r = tid; r <= a.P; r += kLT) a.send_offset[r] = off[E1 + r] - total;
    if (tid == 0 && off[a.E + 1] != off[a.E]) atomicOr(a.status, MOE_STATUS_BAD_EXPERT);
  }

  // 9. one tile: the count kernel's per-token outputs
  if constexpr (kOne) {
    for (int tt = tid; tt < nt; tt += kLT) a.tok_mask[tt] = tm[tt];
    for (int i = tid; i < nt * a.P; i += kLT) {
      const int tt = i / a.P;
      a.is_token_in_rank[i] = (uint8_t)((tm[tt] >> (i - tt * a.P)) & 1ull);
    }
  }
}

}  // namespace

size_t layout_count_lds(int E, int P, int tile) {
  return (size_t)tile * 8 + (size_t)(E + 1 + P) * 4;
}

size_t layout_rank_lds(int E, int P, int tile, int K) {
  const size_t E1 = (size_t)E + 1, NR = E1 + P;
  const size_t parts_nr = NR > (size_t)kLT ? NR : (size_t)kLT;  // parts * NR <= max(kLT, NR)
  const size_t ints = NR + (NR + 1) + kLW * E1 + kLW + 2 * (size_t)kLW * P + P + NR + 2 * parts_nr;
  return (size_t)P * 8 + ints * 4 + (size_t)tile * K * 2;
}

size_t layout_rank_wave_lds(int E, int P, int tile) {
  const size_t E1 = (size_t)E + 1, NR = E1 + P;
  const size_t ngmax = ((size_t)tile + kWave - 1) / kWave;
  const size_t parts_nr = (size_t)kLT;  // parts * NR <= kLT when NR <= kLT
  const size_t ints = NR + (NR + 1) + NR + kLW * E1 + kLW + 2 * parts_nr;
  return (ngmax * P + (size_t)tile) * 8 + ints * 4;
}

bool layout_rank_wave_fits(int K, int E, int P, int tile) {
  return (int64_t)tile * K <= kLT && E + 1 + P <= kLT;
}

hipError_t launch_layout(const LayoutArgs& a0, hipStream_t s) {
  LayoutArgs a = a0;
  a.scanned = (a.nblk > kScanTiles && (int64_t)a.nblk * (a.E + 1 + a.P) > kScanWork) ? 1 : 0;
  if (a.nblk == 1 && layout_rank_wave_fits(a.K, a.E, a.P, a.tile)) {  // one tile: one launch
    hipLaunchKernelGGL(layout_rank_wave_kernel<true>, dim3(1), dim3(kLT), layout_rank_wave_lds(a.E, a.P, a.tile),
                       s, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(layout_count_kernel, dim3(a.nblk), dim3(kLT), layout_count_lds(a.E, a.P, a.tile),
                     s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.scanned) {
    const int NR = a.E + 1 + a.P;
    hipLaunchKernelGGL(layout_scan_kernel, dim3((NR + kWave - 1) / kWave), dim3(kLT), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (!a.scanned && layout_rank_wave_fits(a.K, a.E, a.P, a.tile))
    hipLaunchKernelGGL(layout_rank_wave_kernel<false>, dim3(a.nblk), dim3(kLT),
                       layout_rank_wave_lds(a.E, a.P, a.tile), s, a);
  else
    hipLaunchKernelGGL(layout_rank_kernel, dim3(a.nblk), dim3(kLT),
                       layout_rank_lds(a.E, a.P, a.tile, a.K), s, a);
  return hipGetLastError();
}

}  // namespace moe
