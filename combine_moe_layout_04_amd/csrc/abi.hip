// C ABI of libmoe_layout.so: host-side validation, the workspace plan, the
// opaque handle and stream-ordered launches.  Every argument error is caught
// here, before any HIP call, so a rejected call launches nothing.
#include <atomic>
#include <mutex>
#include <new>

#include "internal.h"
#include "../../include/moe_layout.h"
#include "../../include/moe_bench.h"

struct moe_handle_s {
  static constexpr uint32_t kMagic = 0x4D4F454Cu;  // "MOEL"
  uint32_t magic = kMagic;
  bool has_layout = false;
  int64_t T = 0;
  int K = 0, E = 0, P = 0;
  int pad = 1;     // expert segments padded to a multiple of this (fixed at creation)
  int64_t R = 0;   // receive rows of the current layout: T*K + E*(pad-1)
  char* ws = nullptr;
  moe::WsLayout plan{};
  moe::Tuning tune{};
  hipEvent_t ev_start = nullptr;  // moe_time_next_kernel: for the next kernel launch only
  hipEvent_t ev_stop = nullptr;
};

namespace moe {

static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

WsLayout plan_workspace(int64_t T, int K, int E, int P, int layout_pairs, int pad) {
  WsLayout w{};
  // Token tiles of the layout: at most layout_pairs (t,k) pairs per tile
  // (512: one per thread of a layout workgroup), unless that needs more
  // than 128 tiles;
  // then ~128 tiles, each wave of a tile looping over rounds of 64 pairs.
  // Capped by the LDS the rank kernel stages the tile's ids in (2 bytes per
  // pair, within 64 KiB with its other arrays) and the count kernel's per-
  // token masks (8 bytes per token).
  const int64_t fixed = (int64_t)layout_rank_lds(E, P, 0, K);
  int64_t pair_cap = (65536 - fixed) / 2;
  if (pair_cap > 16384) pair_cap = 16384;
  int64_t tile_max = pair_cap / K;
  if (tile_max > 4096) tile_max = 4096;
  if (tile_max < 1) tile_max = 1;
  int64_t tile = layout_pairs / K;
  if (tile < 1) tile = 1;
  if ((T + tile - 1) / tile > 128) tile = (T + 127) / 128;
  if (tile > tile_max) tile = tile_max;
  int64_t nblk = (T + tile - 1) / tile;
  if (nblk < 1) nblk = 1;
  w.tile = (int)tile;
  w.nblk = (int)nblk;
  const int64_t R = T * K;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + (bytes ? bytes : 1), 256);
    return at;
  };
  w.status = take(4);
  w.num_tokens_per_expert = take((size_t)E * 4);
  w.num_tokens_per_rank = take((size_t)P * 4);
  w.expert_offset = take((size_t)(E + 1) * 4);
  w.rank_offset = take((size_t)(P + 1) * 4);
  w.send_offset = take((size_t)(P + 1) * 4);
  w.is_token_in_rank = take((size_t)T * P);
  w.token_slot = take((size_t)T * P * 4);
  const int64_t cap = recv_capacity(T, K, E, pad);  // the inverse maps have a row per receive row
  w.recv_pos = take((size_t)R * 4);
  w.recv_token = take((size_t)cap * 4);
  w.recv_k = take((size_t)cap * 4);
  w.send_token = take((size_t)T * (K < P ? K : P) * 4);
  w.tok_mask = take((size_t)T * 8);
  w.hist = take((size_t)(E + 1 + P) * (nblk + 1) * 4);  // a row per tile, and the totals of a scanned one
  w.total = o;
  return w;
}

}  // namespace moe

namespace {

bool valid_handle(const moe_handle_s* h) { return h && h->magic == moe_handle_s::kMagic; }

// The tuning of a kernel launch: the handle's, plus the events armed by
// moe_time_next_kernel, which this launch takes (so no later one records them).
moe::Tuning take_tuning(moe_handle_s* h) {
  moe::Tuning t = h->tune;
  t.ev_start = h->ev_start;
  t.ev_stop = h->ev_stop;
  h->ev_start = h->ev_stop = nullptr;
  return t;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elem_bytes(int dtype) { return dtype == MOE_F32 ? 4 : dtype == MOE_BF16 ? 2 : 0; }

int check_shape(int64_t T, int K, int E, int P) {
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (K < 1 || E < 1 || P < 1) return MOE_ERR_SHAPE;
  if (K > MOE_MAX_K || E > MOE_MAX_E || P > MOE_MAX_P) return MOE_ERR_UNSUPPORTED;
  if (E % P != 0 || K > E) return MOE_ERR_SHAPE;
  if (T * (int64_t)K >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

int check_pad(int64_t T, int K, int E, int pad) {
  if (pad < 1 || pad > moe::kMaxPadMultiple) return MOE_ERR_INVALID_ARG;
  if (moe::recv_capacity(T, K, E, pad) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Shared checks of the four row calls.  Returns MOE_OK and NV (16-byte chunks
// per row), or an error.
int check_rows(const moe_handle_s* h, int dtype, int64_t H, int* NV) {
  if (!valid_handle(h)) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  const int eb = elem_bytes(dtype);
  if (eb == 0) return MOE_ERR_UNSUPPORTED;
  if (H < 1 || (H * eb) % 16 != 0) return MOE_ERR_SHAPE;
  const int64_t nv = H * eb / 16;
  if (nv >= (int64_t(1) << 31) || nv * h->R >= (int64_t(1) << 62)) return MOE_ERR_UNSUPPORTED;
  // one wave per (token, segment), then the padding waves: the grid must fit
  // in a 32-bit wave index
  if (moe::row_waves(h->T, (int)nv, 1) + moe::pad_fill_waves(h->E, h->pad, (int)nv) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  *NV = (int)nv;
  return MOE_OK;
}

// The router-weight-gradient kernels keep one float per (segment, k) in LDS.
int check_dot(const moe_handle_s* h, int NV) {
  return moe::dot_lds_bytes(NV, h->K) <= moe::kMaxDotLds ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }


template <typename T>
T* ws_ptr(const moe_handle_s* h, size_t off) {
  return reinterpret_cast<T*>(h->ws + off);
}

// Padded layouts: zero rows (and zero scores) in the padding of every expert
// segment of a receive buffer the call just wrote.  Nothing when unpadded.
// The padding rows a call writes into a padded receive buffer (zero rows and
// zero scores): filled by extra waves of the call's row kernel.  pad = 1 (an
// unpadded handle) adds no wave.
moe::PadArgs pad_rows(const moe_handle_s* h, void* rows, float* scores, int NV) {
  moe::PadArgs p{};
  p.pad = 1;
  if (h->pad <= 1) return p;
  p.dst = rows;
  p.scores_out = scores;
  p.expert_offset = ws_ptr<int>(h, h->plan.expert_offset);
  p.num_tokens_per_expert = ws_ptr<int>(h, h->plan.num_tokens_per_expert);
  p.E = h->E;
  p.NV = NV;
  p.R = (int)h->R;
  p.pad = h->pad;
  p.ngrp = (NV + 63) / 64;
  p.nblk = (h->pad - 1 + moe::kPadRows - 1) / moe::kPadRows;
  p.nwaves = (int)moe::pad_fill_waves(h->E, h->pad, NV);  // fits: checked with the row waves
  return p;
}

}  // namespace

extern "C" {

int moe_workspace_size_padded(int64_t T, int K, int E, int P, int pad_multiple, size_t* bytes) {
  if (!bytes) return MOE_ERR_INVALID_ARG;
  int st = check_shape(T, K, E, P);
  if (st != MOE_OK) return st;
  if ((st = check_pad(T, K, E, pad_multiple)) != MOE_OK) return st;
  *bytes = moe::plan_workspace(T, K, E, P, moe::kLayoutThreads, pad_multiple).total;
  return MOE_OK;
}

int moe_workspace_size(int64_t T, int K, int E, int P, size_t* bytes) {
  return moe_workspace_size_padded(T, K, E, P, 1, bytes);
}

int moe_handle_create(moe_handle_t* out, const moe_tuning* tuning) {
  return moe_handle_create_padded(out, tuning, 1);
}

int moe_handle_create_padded(moe_handle_t* out, const moe_tuning* tuning, int pad_multiple) {
  if (!out) return MOE_ERR_INVALID_ARG;
  if (pad_multiple < 1 || pad_multiple > moe::kMaxPadMultiple) return MOE_ERR_INVALID_ARG;
  // defaults: one segment per wave, non-temporal receive rows and token-row
  // stores, 4 waves per workgroup (the LDS-staged gather: 1 at rows of whole
  // segments not a multiple of 8 in number), 512-pair layout tiles.  Measured on the
  // Qwen3-shaped layer (one box, interleaved runs): non-temporal token-row
  // stores take the step from 149.3 to 145.8 us; two segments per wave then
  // gain nothing in the gathers and cost 3 us in each scatter.
  moe::Tuning t{1, 2, 4, moe::kLayoutThreads, 0, 0};
  if (tuning) {
    const int c = tuning->chunks_per_lane, n = tuning->nontemporal, w = tuning->waves_per_block;
    const int lp = tuning->layout_pairs;
    if (!(c == 0 || c == 1 || c == 2 || c == 4)) return MOE_ERR_INVALID_ARG;
    if (n < 0 || n > 2) return MOE_ERR_INVALID_ARG;
    if (!(w == 0 || w == 1 || w == 2 || w == 4 || w == 8)) return MOE_ERR_INVALID_ARG;
    if (!(lp == 0 || lp == 512 || lp == 1024 || lp == 2048 || lp == 4096)) return MOE_ERR_INVALID_ARG;
    if (tuning->gather_mode < 0 || tuning->gather_mode > 2) return MOE_ERR_INVALID_ARG;
    t.gather_mode = tuning->gather_mode;
    if (c) t.chunks_per_lane = c;
    t.nontemporal = n;
    if (w) t.waves_per_block = t.gather_waves = w;
    if (lp) t.layout_pairs = lp;
  }
  moe_handle_s* h = new (std::nothrow) moe_handle_s();
  if (!h) return MOE_ERR_INVALID_ARG;
  h->tune = t;
  h->pad = pad_multiple;
  *out = h;
  return MOE_OK;
}

int moe_handle_destroy(moe_handle_t h) {
  if (!valid_handle(h)) return MOE_ERR_INVALID_ARG;
  h->magic = 0;
  delete h;
  return MOE_OK;
}

}  // extern "C"

namespace {

// ---- the no-allocation layout's scratch ---------------------------------------
//
// moe_layout_noalloc keeps the layout's per-tile histogram (its only scratch:
// written by the count kernel, read by the rank kernel, dead afterwards) in
// this file-scope device array instead of the caller's workspace.  Every GPU
// the library runs on holds its own copy until the process ends.  In host code
// `scratch` is only a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only that
// address is ever handed to a kernel.
constexpr size_t kScratchBytes = size_t(2) << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's address on the device `stream` runs on.
int scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  if (stream) {
    if (hipStreamGetDevice(stream, &dev) != hipSuccess) return MOE_ERR_HIP;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      int cur = 0;
      if (hipGetDevice(&cur) != hipSuccess) return MOE_ERR_HIP;
      if (cur != dev && hipSetDevice(dev) != hipSuccess) return MOE_ERR_HIP;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev && hipSetDevice(cur) != hipSuccess) return MOE_ERR_HIP;
      if (e != hipSuccess || !p) return MOE_ERR_HIP;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MOE_OK;
}

// moe_layout and moe_layout_noalloc.  static_hist: the histogram goes to the
// per-device scratch array, and the workspace only needs the handle's arrays
// (the sections before the histogram).
int layout_call(moe_handle_s* h, const void* topk_idx, int itype, int64_t T, int K, int E, int P,
                void* workspace, size_t workspace_bytes, bool static_hist, hipStream_t stream) {
  if (!valid_handle(h)) return MOE_ERR_INVALID_ARG;
  int st = check_shape(T, K, E, P);
  if (st != MOE_OK) return st;
  if ((st = check_pad(T, K, E, h->pad)) != MOE_OK) return st;
  if (itype != MOE_I32 && itype != MOE_I64) return MOE_ERR_UNSUPPORTED;
  if (!workspace || (T > 0 && !topk_idx)) return MOE_ERR_INVALID_ARG;
  if (!aligned(workspace, 256)) return MOE_ERR_ALIGNMENT;
  if (T > 0 && !aligned(topk_idx, itype == MOE_I32 ? 4 : 8)) return MOE_ERR_ALIGNMENT;
  const moe::WsLayout sized = moe::plan_workspace(T, K, E, P, moe::kLayoutThreads, h->pad);
  // the histogram is the workspace's last section: without it, the handle's arrays
  if (workspace_bytes < (static_hist ? sized.hist : sized.total)) return MOE_ERR_WORKSPACE;
  // the handle's tile size: never more tiles than the default plan sizes for
  moe::WsLayout plan = moe::plan_workspace(T, K, E, P, h->tune.layout_pairs, h->pad);
  plan.hist = sized.hist;
  int* hist = nullptr;
  if (static_hist) {
    if ((size_t)(E + 1 + P) * (size_t)(plan.nblk + 1) * sizeof(int) > kScratchBytes) return MOE_ERR_SCRATCH;
    void* p = nullptr;
    if ((st = scratch_address(stream, &p)) != MOE_OK) return st;
    hist = static_cast<int*>(p);
  }

  h->has_layout = false;
  h->T = T;
  h->K = K;
  h->E = E;
  h->P = P;
  h->R = moe::recv_capacity(T, K, E, h->pad);
  h->ws = static_cast<char*>(workspace);
  h->plan = plan;

  moe::LayoutArgs a{};
  a.idx = topk_idx;
  a.itype = itype;
  a.T = (int)T;
  a.K = K;
  a.E = E;
  a.P = P;
  a.epr = E / P;
  a.pad = h->pad;
  a.R = (int)h->R;
  a.nblk = plan.nblk;
  a.tile = plan.tile;
  a.hist = static_hist ? hist : ws_ptr<int>(h, plan.hist);
  a.tok_mask = ws_ptr<unsigned long long>(h, plan.tok_mask);
  a.num_tokens_per_expert = ws_ptr<int>(h, plan.num_tokens_per_expert);
  a.num_tokens_per_rank = ws_ptr<int>(h, plan.num_tokens_per_rank);
  a.is_token_in_rank = ws_ptr<uint8_t>(h, plan.is_token_in_rank);
  a.expert_offset = ws_ptr<int>(h, plan.expert_offset);
  a.rank_offset = ws_ptr<int>(h, plan.rank_offset);
  a.send_offset = ws_ptr<int>(h, plan.send_offset);
  a.token_slot = ws_ptr<int>(h, plan.token_slot);
  a.recv_pos = ws_ptr<int>(h, plan.recv_pos);
  a.recv_token = ws_ptr<int>(h, plan.recv_token);
  a.recv_k = ws_ptr<int>(h, plan.recv_k);
  a.send_token = ws_ptr<int>(h, plan.send_token);
  a.status = ws_ptr<int>(h, plan.status);
  const int rc = hip_status(moe::launch_layout(a, stream));
  if (rc == MOE_OK) h->has_layout = true;
  return rc;
}

}  // namespace

extern "C" {

int moe_layout(moe_handle_t h, const void* topk_idx, int itype, int64_t T, int K, int E,
               int P, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layout_call(h, topk_idx, itype, T, K, E, P, workspace, workspace_bytes, false, stream);
}

int moe_layout_noalloc(moe_handle_t h, const void* topk_idx, int itype, int64_t T, int K, int E,
                       int P, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return layout_call(h, topk_idx, itype, T, K, E, P, workspace, workspace_bytes, true, stream);
}

int moe_dispatch(moe_handle_t h, const void* x, int dtype, int64_t H, const float* topk_weights,
                 int scale_rows, void* recv, float* recv_scores, hipStream_t stream) {
  int NV = 0;
  const int st = check_rows(h, dtype, H, &NV);
  if (st != MOE_OK) return st;
  if (scale_rows != 0 && scale_rows != 1) return MOE_ERR_INVALID_ARG;
  if (h->T == 0) return MOE_OK;  // nothing to read or write; empty arrays may be NULL
  if ((scale_rows || recv_scores) && !topk_weights) return MOE_ERR_INVALID_ARG;
  if (!x || !recv) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(recv, 16)) return MOE_ERR_ALIGNMENT;
  if ((topk_weights && !aligned(topk_weights, 4)) || (recv_scores && !aligned(recv_scores, 4)))
    return MOE_ERR_ALIGNMENT;
  moe::ScatterArgs a{};
  a.src = x;
  a.recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
  a.w = topk_weights;
  a.dst = recv;
  a.scores_out = recv_scores;
  a.T = (int)h->T;
  a.K = h->K;
  a.NV = NV;
  a.R = (int)h->R;
  a.dtype = dtype;
  a.scale = scale_rows != 0;
  a.status = ws_ptr<int>(h, h->plan.status);
  a.pad = pad_rows(h, recv, recv_scores, NV);
  return hip_status(moe::launch_scatter(a, take_tuning(h), stream));
}

int moe_combine(moe_handle_t h, const void* y, int dtype, int64_t H, const float* topk_weights,
                void* out, hipStream_t stream) {
  int NV = 0;
  const int st = check_rows(h, dtype, H, &NV);
  if (st != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;
  if (!y || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(out, 16)) return MOE_ERR_ALIGNMENT;
  if (topk_weights && !aligned(topk_weights, 4)) return MOE_ERR_ALIGNMENT;
  moe::GatherArgs a{};
  a.src = y;
  a.recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
  a.w = topk_weights;
  a.dst = out;
  a.T = (int)h->T;
  a.K = h->K;
  a.NV = NV;
  a.R = (int)h->R;
  a.dtype = dtype;
  a.status = ws_ptr<int>(h, h->plan.status);
  return hip_status(moe::launch_gather(a, take_tuning(h), stream));
}

int moe_combine_bwd(moe_handle_t h, const void* grad_out, int dtype, int64_t H,
                    const float* topk_weights, const void* y, void* grad_y, float* grad_w,
                    hipStream_t stream) {
  int NV = 0;
  int st = check_rows(h, dtype, H, &NV);
  if (st != MOE_OK) return st;
  if (grad_w && (st = check_dot(h, NV)) != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;  // nothing to read or write; empty arrays may be NULL
  if (grad_w && (!topk_weights || !y)) return MOE_ERR_INVALID_ARG;
  if (!grad_y && !grad_w) return MOE_ERR_INVALID_ARG;
  if (!grad_out) return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_out, 16) || (grad_y && !aligned(grad_y, 16)) || (grad_w && !aligned(y, 16)))
    return MOE_ERR_ALIGNMENT;
  if ((topk_weights && !aligned(topk_weights, 4)) || (grad_w && !aligned(grad_w, 4)))
    return MOE_ERR_ALIGNMENT;
  // rows: a dispatch of the output gradient, scaled by the weights
  moe::ScatterArgs a{};
  a.src = grad_out;
  a.recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
  a.w = topk_weights;
  a.dst = grad_y;
  a.T = (int)h->T;
  a.K = h->K;
  a.NV = NV;
  a.R = (int)h->R;
  a.dtype = dtype;
  a.scale = topk_weights != nullptr;
  a.status = ws_ptr<int>(h, h->plan.status);
  a.pad = pad_rows(h, grad_y, nullptr, NV);  // no gradient in the padding rows
  if (!grad_w) return hip_status(moe::launch_scatter(a, take_tuning(h), stream));
  // Router-weight gradient: a separate pass over grad_out and y (measured
  // faster than fusing it into the row stores: HBM turns around less).  It
  // goes first: the two passes are independent, and the read-only pass ahead
  // of the row scatter measured level at the Qwen3-30B-A3B shape and 3 us
  // faster per layer at the DeepSeek-V3 shape.
  moe::DotArgs d{};
  d.tok = grad_out;
  d.rcv = y;
  d.recv_pos = a.recv_pos;
  d.w = topk_weights;
  d.dot_out = grad_w;
  d.T = a.T;
  d.K = a.K;
  d.NV = NV;
  d.R = a.R;
  d.dtype = dtype;
  d.gather = false;
  d.status = a.status;
  st = hip_status(moe::launch_token_dot(d, take_tuning(h), stream));
  if (st != MOE_OK || !grad_y) return st;
  return hip_status(moe::launch_scatter(a, take_tuning(h), stream));
}

int moe_dispatch_bwd(moe_handle_t h, const void* grad_recv, int dtype, int64_t H,
                     const float* topk_weights, const void* x, void* grad_x, float* grad_s,
                     hipStream_t stream) {
  int NV = 0;
  int st = check_rows(h, dtype, H, &NV);
  if (st != MOE_OK) return st;
  if (grad_s && (st = check_dot(h, NV)) != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;  // nothing to read or write; empty arrays may be NULL
  if (grad_s && (!topk_weights || !x)) return MOE_ERR_INVALID_ARG;
  if (!grad_x && !grad_s) return MOE_ERR_INVALID_ARG;
  if (!grad_recv) return MOE_ERR_INVALID_ARG;
  if (!aligned(grad_recv, 16) || (grad_x && !aligned(grad_x, 16)) || (grad_s && !aligned(x, 16)))
    return MOE_ERR_ALIGNMENT;
  if ((topk_weights && !aligned(topk_weights, 4)) || (grad_s && !aligned(grad_s, 4)))
    return MOE_ERR_ALIGNMENT;
  if (grad_s) {
    // each receive row is read once for both the weighted sum and the dot
    moe::DotArgs d{};
    d.tok = x;
    d.rcv = grad_recv;
    d.recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
    d.w = topk_weights;
    d.dst = grad_x;
    d.dot_out = grad_s;
    d.T = (int)h->T;
    d.K = h->K;
    d.NV = NV;
    d.R = (int)h->R;
    d.dtype = dtype;
    d.gather = grad_x != nullptr;  // without grad_x: the score gradient only
    d.status = ws_ptr<int>(h, h->plan.status);
    return hip_status(moe::launch_token_dot(d, take_tuning(h), stream));
  }
  moe::GatherArgs a{};
  a.src = grad_recv;
  a.recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
  a.w = topk_weights;
  a.dst = grad_x;
  a.T = (int)h->T;
  a.K = h->K;
  a.NV = NV;
  a.R = (int)h->R;
  a.dtype = dtype;
  a.status = ws_ptr<int>(h, h->plan.status);
  return hip_status(moe::launch_gather(a, take_tuning(h), stream));
}

int moe_recv_capacity(moe_handle_t h, int64_t* rows) {
  if (!valid_handle(h) || !rows) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  *rows = h->R;
  return MOE_OK;
}

int moe_send_capacity(moe_handle_t h, int64_t* rows) {
  if (!valid_handle(h) || !rows) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  *rows = h->T * (h->K < h->P ? h->K : h->P);
  return MOE_OK;
}

}  // extern "C"

namespace {

// Checks shared by the four staged calls; fills the arguments they share.
int staged_args(const moe_handle_s* h, int dtype, int64_t H, int64_t send_rows, moe::StagedArgs* a) {
  int NV = 0;
  const int st = check_rows(h, dtype, H, &NV);
  if (st != MOE_OK) return st;
  const int64_t cap = h->T * (h->K < h->P ? h->K : h->P);
  if (send_rows < cap) return MOE_ERR_SHAPE;
  if (cap * (int64_t)((NV + 63) / 64) + moe::pad_fill_waves(h->E, h->pad, NV) > INT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  *a = moe::StagedArgs{};
  a->recv_pos = ws_ptr<int>(h, h->plan.recv_pos);
  a->token_slot = ws_ptr<int>(h, h->plan.token_slot);
  a->send_offset = ws_ptr<int>(h, h->plan.send_offset);
  a->rank_offset = ws_ptr<int>(h, h->plan.rank_offset);
  a->send_token = ws_ptr<int>(h, h->plan.send_token);
  a->tok_mask = ws_ptr<unsigned long long>(h, h->plan.tok_mask);
  a->T = (int)h->T;
  a->K = h->K;
  a->P = h->P;
  a->NV = NV;
  a->R = (int)h->R;
  a->send_cap = (int)cap;
  a->dtype = dtype;
  a->status = ws_ptr<int>(h, h->plan.status);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_send(moe_handle_t h, const void* x, int dtype, int64_t H, void* send, int64_t send_rows,
             hipStream_t stream) {
  moe::StagedArgs a;
  const int st = staged_args(h, dtype, H, send_rows, &a);
  if (st != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;
  if (!x || !send) return MOE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(send, 16)) return MOE_ERR_ALIGNMENT;
  a.src = x;
  a.dst = send;
  return hip_status(moe::launch_send(a, take_tuning(h), stream));
}

int moe_expand(moe_handle_t h, const void* send, int dtype, int64_t H, int64_t send_rows,
               const float* topk_weights, int scale_rows, void* recv, float* recv_scores,
               hipStream_t stream) {
  moe::StagedArgs a;
  const int st = staged_args(h, dtype, H, send_rows, &a);
  if (st != MOE_OK) return st;
  if (scale_rows != 0 && scale_rows != 1) return MOE_ERR_INVALID_ARG;
  if (h->T == 0) return MOE_OK;  // nothing to read or write; empty arrays may be NULL
  if ((scale_rows || recv_scores) && !topk_weights) return MOE_ERR_INVALID_ARG;
  if (!send || !recv) return MOE_ERR_INVALID_ARG;
  if (!aligned(send, 16) || !aligned(recv, 16)) return MOE_ERR_ALIGNMENT;
  if ((topk_weights && !aligned(topk_weights, 4)) || (recv_scores && !aligned(recv_scores, 4)))
    return MOE_ERR_ALIGNMENT;
  a.src = send;
  a.dst = recv;
  a.w = topk_weights;
  a.scores_out = recv_scores;
  a.scale = scale_rows != 0;
  a.pad = pad_rows(h, recv, recv_scores, a.NV);
  return hip_status(moe::launch_expand(a, take_tuning(h), stream));
}

int moe_reduce_partitions(moe_handle_t h, const void* y, int dtype, int64_t H,
                          const float* topk_weights, void* partial, int64_t send_rows,
                          hipStream_t stream) {
  moe::StagedArgs a;
  const int st = staged_args(h, dtype, H, send_rows, &a);
  if (st != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;
  if (!y || !partial) return MOE_ERR_INVALID_ARG;
  if (!aligned(y, 16) || !aligned(partial, 16)) return MOE_ERR_ALIGNMENT;
  if (topk_weights && !aligned(topk_weights, 4)) return MOE_ERR_ALIGNMENT;
  a.src = y;
  a.dst = partial;
  a.w = topk_weights;
  return hip_status(moe::launch_reduce_partitions(a, take_tuning(h), stream));
}

int moe_combine_partitions(moe_handle_t h, const void* partial, int dtype, int64_t H,
                           int64_t send_rows, void* out, hipStream_t stream) {
  moe::StagedArgs a;
  const int st = staged_args(h, dtype, H, send_rows, &a);
  if (st != MOE_OK) return st;
  if (h->T == 0) return MOE_OK;
  if (!partial || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned(partial, 16) || !aligned(out, 16)) return MOE_ERR_ALIGNMENT;
  a.src = partial;
  a.dst = out;
  return hip_status(moe::launch_combine_partitions(a, take_tuning(h), stream));
}

int moe_handle_field(moe_handle_t h, int field, void** dev_ptr, size_t* bytes) {
  if (!valid_handle(h) || !dev_ptr || !bytes) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  const moe::WsLayout& p = h->plan;
  const size_t T = (size_t)h->T, K = (size_t)h->K, E = (size_t)h->E, P = (size_t)h->P;
  size_t off = 0, n = 0;
  switch (field) {
    case MOE_FIELD_NUM_TOKENS_PER_EXPERT: off = p.num_tokens_per_expert; n = E * 4; break;
    case MOE_FIELD_NUM_TOKENS_PER_RANK: off = p.num_tokens_per_rank; n = P * 4; break;
    case MOE_FIELD_IS_TOKEN_IN_RANK: off = p.is_token_in_rank; n = T * P; break;
    case MOE_FIELD_EXPERT_OFFSET: off = p.expert_offset; n = (E + 1) * 4; break;
    case MOE_FIELD_RANK_OFFSET: off = p.rank_offset; n = (P + 1) * 4; break;
    case MOE_FIELD_SEND_OFFSET: off = p.send_offset; n = (P + 1) * 4; break;
    case MOE_FIELD_TOKEN_SLOT: off = p.token_slot; n = T * P * 4; break;
    case MOE_FIELD_RECV_POS: off = p.recv_pos; n = T * K * 4; break;
    case MOE_FIELD_RECV_TOKEN: off = p.recv_token; n = (size_t)h->R * 4; break;
    case MOE_FIELD_RECV_K: off = p.recv_k; n = (size_t)h->R * 4; break;
    case MOE_FIELD_STATUS: off = p.status; n = 4; break;
    case MOE_FIELD_SEND_TOKEN: off = p.send_token; n = T * (K < P ? K : P) * 4; break;
    default: return MOE_ERR_INVALID_ARG;
  }
  *dev_ptr = h->ws + off;
  *bytes = n;
  return MOE_OK;
}

int moe_handle_dims(moe_handle_t h, int64_t* T, int* K, int* E, int* P) {
  if (!valid_handle(h) || !T || !K || !E || !P) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  *T = h->T;
  *K = h->K;
  *E = h->E;
  *P = h->P;
  return MOE_OK;
}

int moe_handle_check(moe_handle_t h, hipStream_t stream, int* device_status) {
  if (!valid_handle(h) || !device_status) return MOE_ERR_INVALID_ARG;
  if (!h->has_layout) return MOE_ERR_HANDLE;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_ERR_HIP;
  int v = 0;
  if (hipMemcpy(&v, h->ws + h->plan.status, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_HIP;
  *device_status = v;
  return MOE_OK;
}

int moe_bench_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  if (!dst || !src) return MOE_ERR_INVALID_ARG;
  if (bytes % 16 != 0) return MOE_ERR_SHAPE;
  if (!aligned(dst, 16) || !aligned(src, 16)) return MOE_ERR_ALIGNMENT;
  return hip_status(moe::launch_copy(dst, src, bytes, stream));
}

int moe_stream_create_cu_budget(int cu_first, int cu_count, hipStream_t* out) {
  if (!out || cu_first < 0 || cu_count < 1) return MOE_ERR_INVALID_ARG;
  int dev = 0, ncu = 0, nxcc = 1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return MOE_ERR_HIP;
  if (hipDeviceGetAttribute(&nxcc, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess) nxcc = 1;
  // every selected CU must exist (an empty mask would leave the stream's work
  // with no CU to run on), and the runtime numbers CUs round-robin over the
  // XCDs and refuses a mask that leaves one without a CU: a budget takes at
  // least one CU per XCD
  if (ncu < 1 || cu_first + (int64_t)cu_count > ncu || cu_count < nxcc) return MOE_ERR_SHAPE;
  uint32_t mask[64] = {};  // up to 2048 CUs
  const int words = (ncu + 31) / 32;
  if (words > 64) return MOE_ERR_UNSUPPORTED;
  for (int c = cu_first; c < cu_first + cu_count; ++c) mask[c / 32] |= 1u << (c % 32);
  return hip_status(hipExtStreamCreateWithCUMask(out, (uint32_t)words, mask));
}

int moe_stream_destroy(hipStream_t stream) {
  if (!stream) return MOE_ERR_INVALID_ARG;
  return hip_status(hipStreamDestroy(stream));
}

int moe_time_next_kernel(moe_handle_t h, hipEvent_t start, hipEvent_t stop) {
  if (!valid_handle(h)) return MOE_ERR_INVALID_ARG;
  if (start && !stop) return MOE_ERR_INVALID_ARG;
  h->ev_start = start;
  h->ev_stop = stop;
  return MOE_OK;
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument (null pointer, negative size or missing companion argument)";
    case MOE_ERR_SHAPE: return "invalid shape (K<1, K>E, E%P!=0, H<1 or a row that is not whole 16-byte chunks)";
    case MOE_ERR_UNSUPPORTED: return "unsupported (dtype/itype, P>64, E>1024, K>32 or T*K>=2^31)";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer (rows need 16 bytes, workspace 256)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_HANDLE: return "bad handle, or a row call before moe_layout";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH:
      return "the layout's histogram exceeds the static scratch of moe_layout_noalloc (2 MiB); use moe_layout";
    default: return "unknown status";
  }
}

const char* moe_version(void) { return "moe_layout 0.2 (gfx950)"; }

}  // extern "C"
