// kda_conv.hip -- the short causal depthwise convolution over the [q|k|v]
// channels with carried taps: a varlen forward over packed prefills and a
// one-token update (page "model(kimi_linear): ONE-SURFACE ROW 7 -- fold
// Kimi-Linear onto the shared paged runner", B2: CausalConv1dFwd (varlen) /
// CausalConv1dUpdate (decode) in the [q|k|v] conv-state layout).
//
// Per channel c: y[t] = act(bias + sum_j w[j] x[t - (W - 1) + j]); positions
// before the sequence start read the carried taps state[slot, i, :] (the input
// at start - (W - 1) + i).
//
// The op is a stream over HBM (2 bytes in, 2 out per channel and token in
// bf16) with W fused multiply-adds per element, so the design is about access
// shape only:
//   - a thread owns one 16-byte vector of channels (8 bf16 / 4 fp32) over a
//     run of L = 32 consecutive tokens, issues all L row loads before using
//     any, and slides a W-1 tap window through them in registers; a wave
//     reads and writes 1 KB contiguous per token row; outputs are written
//     with streaming (non-temporal) stores;
//   - the W-1 rows before a run are read again by the run's thread (halo);
//     workgroup ids are remapped so that the runs of neighbouring tokens are
//     handled on the same XCD, where that re-read hits the XCD's L2;
//   - sequence boundaries depend on the token only, so the walk over
//     cu_seqlens is uniform across a workgroup; a run inside one sequence
//     (all runs but those meeting a boundary) has no per-token control flow.
// The new taps are written by a second launch after every output row is
// done, so an in-place state is never replaced while a run still reads it.
#include <hip/hip_runtime.h>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int kConvThreads = 256;
constexpr int kConvRun = 32;  // tokens per thread in the forward

template <typename T>
struct CVec;  // 16 bytes of T
template <>
struct CVec<bf16> {
  typedef bf16x8 type;
  static constexpr int n = 8;
};
template <>
struct CVec<float> {
  typedef f32x4 type;
  static constexpr int n = 4;
};

template <typename T>
__device__ __forceinline__ typename CVec<T>::type load16(const T* p) {
  return *reinterpret_cast<const typename CVec<T>::type*>(p);
}
template <typename T>
__device__ __forceinline__ void store16(T* p, typename CVec<T>::type v) {
  *reinterpret_cast<typename CVec<T>::type*>(p) = v;
}
// Streaming store: the forward's outputs are far larger than the caches and
// are next read by another kernel, so they are written without keeping them.
template <typename T>
__device__ __forceinline__ void store16_stream(T* p, typename CVec<T>::type v) {
  __builtin_nontemporal_store(v, reinterpret_cast<typename CVec<T>::type*>(p));
}

// Blocks are dealt to the 8 XCDs round-robin by id; give each XCD a
// contiguous range of logical ids instead (ids past the last full round of 8
// keep their own).
__device__ __forceinline__ int xcd_contiguous(int bid, int nblocks) {
  const int full = nblocks & ~7;
  if (bid >= full) return bid;
  return (bid & 7) * (full >> 3) + (bid >> 3);
}

__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.f + fast_exp2(-z * kLog2e));
}

struct ConvParams {
  const void* x;
  const float* weight;
  const float* bias;
  const int32_t* cu;
  const void* state_in;
  void* state_out;
  const int* slots;
  int n_slots, n_seqs, dim, rows;
  int n_out;
  void* y[3];
  int y_off[4];
};

// Where the thread's channel vector c0 lands in the output blocks.
template <typename T>
struct OutCol {
  T* base;  // block start + column
  int ld;   // block width (row stride)
};
template <typename T>
__device__ __forceinline__ OutCol<T> out_col(const ConvParams& p, int c0) {
  int b = 0;
#pragma unroll
  for (int i = 1; i < 3; ++i)
    if (i < p.n_out && c0 >= p.y_off[i]) b = i;
  const int ld = p.y_off[b + 1] - p.y_off[b];
  return OutCol<T>{reinterpret_cast<T*>(p.y[b]) + (c0 - p.y_off[b]), ld};
}

// Slot of sequence n, or -1 when it is skipped.
__device__ __forceinline__ int slot_of(const ConvParams& p, int n) {
  if (!p.slots) return n;
  const int s = p.slots[n];
  return (s >= 0 && s < p.n_slots) ? s : -1;
}

// Sequence n's token range, clamped into [0, rows] and non-decreasing.
__device__ __forceinline__ void seq_range(const ConvParams& p, int n, int& s, int& e) {
  if (!p.cu) {
    s = 0;
    e = p.rows;
    return;
  }
  s = min(max(p.cu[n], 0), p.rows);
  e = min(max(p.cu[n + 1], s), p.rows);
}

template <typename T, int W>
struct Taps {
  typedef typename CVec<T>::type V;
  static constexpr int VN = CVec<T>::n;
  float w[W][VN];
  float b[VN];

  // The VN * W weights of channels c0 .. c0+VN-1 are consecutive and 16-byte
  // aligned (c0 is a multiple of 4): VN * W / 4 vector loads.  The bias is
  // read through a buffer resource that is empty when there is no bias.
  __device__ __forceinline__ void load(const ConvParams& p, int c0) {
    const f32x4* wp = reinterpret_cast<const f32x4*>(p.weight + (int64_t)c0 * W);
#pragma unroll
    for (int q = 0; q < VN * W / 4; ++q) {
      const f32x4 v = wp[q];
#pragma unroll
      for (int m = 0; m < 4; ++m) w[(4 * q + m) % W][(4 * q + m) / W] = v[m];
    }
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(const_cast<float*>(p.bias), p.bias ? p.dim * 4 : 0);
#pragma unroll
    for (int q = 0; q < VN / 4; ++q) {
      const f32x4 v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rb, (c0 + 4 * q) * 4, 0, 0));
#pragma unroll
      for (int m = 0; m < 4; ++m) b[4 * q + m] = v[m];
    }
  }
  // y for the current token from the W-1 window entries and the input xt
  template <bool SILU>
  __device__ __forceinline__ V apply(const float (&win)[W - 1][VN], V xt) const {
    V out;
#pragma unroll
    for (int e = 0; e < VN; ++e) {
      float acc = b[e];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) acc = fmaf(w[j][e], win[j][e], acc);
      acc = fmaf(w[W - 1][e], to_f32(xt[e]), acc);
      out[e] = from_f32<T>(SILU ? silu(acc) : acc);
    }
    return out;
  }
};

template <typename T>
__device__ __forceinline__ typename CVec<T>::type buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  return __builtin_bit_cast(typename CVec<T>::type, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// The carried taps of `slot` as a buffer resource: W-1 rows of dim values,
// or an empty buffer (every read gives 0) when there is no state or the
// sequence is skipped.  Reads through it need no branch.
template <typename T, int W>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t taps_rsrc(const ConvParams& p, int slot) {
  const bool ok = p.state_in && slot >= 0;
  const T* base = reinterpret_cast<const T*>(p.state_in) + (ok ? (int64_t)slot * (W - 1) * p.dim : 0);
  return make_rsrc(const_cast<T*>(base), ok ? (W - 1) * p.dim * (int)sizeof(T) : 0);
}

// Rows lo .. hi-1 of x as a buffer resource (empty when hi <= lo, and then
// never dereferenced, so x may be NULL).  At most W-1 rows are ever covered.
template <typename T>
struct XRows {
  __amdgpu_buffer_rsrc_t r;
  int lo;
};
template <typename T>
__device__ __forceinline__ XRows<T> x_rows(const ConvParams& p, int lo, int hi) {
  const T* base = reinterpret_cast<const T*>(p.x) + (int64_t)lo * p.dim;
  return XRows<T>{make_rsrc(const_cast<T*>(base), hi > lo ? (hi - lo) * p.dim * (int)sizeof(T) : 0), lo};
}

// Input at position pos of a sequence starting at s: x[pos] when pos >= s
// (read through xr, which covers the rows that can be asked for), else
// carried tap pos - s + W - 1 (0 before the first tap).  Both candidates are
// read through buffer resources, out-of-range reads give 0, and one is
// selected: no load sits behind a branch.
template <typename T, int W>
__device__ __forceinline__ void fetch(const ConvParams& p, __amdgpu_buffer_rsrc_t taps,
                                      const XRows<T>& xr, int c0, int pos, int s,
                                      float (&out)[CVec<T>::n]) {
  constexpr int VN = CVec<T>::n;
  constexpr int ES = (int)sizeof(T);
  const int tap = pos - s + (W - 1);
  const bool in_x = pos >= s;
  const int toff = (!in_x && tap >= 0) ? (tap * p.dim + c0) * ES : kBufferOff;
  const int xoff = (in_x && pos >= xr.lo && pos - xr.lo < W - 1) ? ((pos - xr.lo) * p.dim + c0) * ES
                                                                   : kBufferOff;
  const typename CVec<T>::type vs = buffer_load16<T>(taps, toff);
  const typename CVec<T>::type vx = buffer_load16<T>(xr.r, xoff);
#pragma unroll
  for (int e = 0; e < VN; ++e) out[e] = to_f32(in_x ? vx[e] : vs[e]);
}

template <typename T, int W, bool SILU>
__global__ __launch_bounds__(kConvThreads) void conv_fwd_kernel(ConvParams p, int n_cblocks) {
  typedef typename CVec<T>::type V;
  constexpr int VN = CVec<T>::n, L = kConvRun;
  const int lid = xcd_contiguous(blockIdx.x, gridDim.x);
  const int tb = lid / n_cblocks, cb = lid - tb * n_cblocks;
  const int cv = cb * kConvThreads + threadIdx.x;
  if (cv * VN >= p.dim) return;
  const int c0 = cv * VN;
  const int t0 = tb * L, t1 = min(t0 + L, p.rows);
  const T* x = reinterpret_cast<const T*>(p.x);

  // every row of the run is requested before anything else
  V xr[L];
#pragma unroll
  for (int i = 0; i < L; ++i) xr[i] = load16(x + (int64_t)min(t0 + i, p.rows - 1) * p.dim + c0);
  Taps<T, W> taps;
  taps.load(p, c0);
  const OutCol<T> oc = out_col<T>(p, c0);

  // the sequence holding t0: the last n with start <= t0
  int n = 0;
  if (p.cu) {
    int lo = 0, hi = p.n_seqs - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (min(max(p.cu[mid], 0), p.rows) <= t0) lo = mid;
      else hi = mid - 1;
    }
    n = lo;
  }
  int s, e;
  seq_range(p, n, s, e);
  int slot = slot_of(p, n);
  float win[W - 1][VN];

  if (t0 >= s && t1 <= e) {
    // The whole run lies in sequence n (every run but those that meet a
    // sequence boundary): no per-token control flow.
    if (slot < 0) return;
    {
      const XRows<T> xw = x_rows<T>(p, max(t0 - (W - 1), 0), t0);
      const __amdgpu_buffer_rsrc_t tr = taps_rsrc<T, W>(p, slot);
#pragma unroll
      for (int j = 0; j < W - 1; ++j) fetch<T, W>(p, tr, xw, c0, t0 - (W - 1) + j, s, win[j]);
    }
    const int len = t1 - t0;
#pragma unroll
    for (int i = 0; i < L; ++i) {
      if (i < len)
        store16_stream(oc.base + (int64_t)(t0 + i) * oc.ld, taps.template apply<SILU>(win, xr[i]));
#pragma unroll
      for (int j = 0; j < W - 2; ++j)
#pragma unroll
        for (int v = 0; v < VN; ++v) win[j][v] = win[j + 1][v];
#pragma unroll
      for (int v = 0; v < VN; ++v) win[W - 2][v] = to_f32(xr[i][v]);
    }
    return;
  }

  // A run that meets a sequence boundary: token by token, re-reading each
  // row (it was just fetched above, so from cache).
  {
    const XRows<T> xw = x_rows<T>(p, max(t0 - (W - 1), 0), t0);
    const __amdgpu_buffer_rsrc_t tr = taps_rsrc<T, W>(p, slot);
#pragma unroll
    for (int j = 0; j < W - 1; ++j) fetch<T, W>(p, tr, xw, c0, t0 - (W - 1) + j, s, win[j]);
  }
#pragma unroll 1
  for (int t = t0; t < t1; ++t) {
    if (t >= e && n < p.n_seqs - 1) {
      do {
        ++n;
        seq_range(p, n, s, e);
      } while (t >= e && n < p.n_seqs - 1);
      slot = slot_of(p, n);
      if (t == s) {  // first token of a sequence: the window is its carried taps
        const __amdgpu_buffer_rsrc_t tr = taps_rsrc<T, W>(p, slot);
        const XRows<T> none = x_rows<T>(p, 0, 0);
#pragma unroll
        for (int j = 0; j < W - 1; ++j) fetch<T, W>(p, tr, none, c0, t - (W - 1) + j, s, win[j]);
      }
    }
    const V xt = load16(x + (int64_t)t * p.dim + c0);
    if (t >= s && t < e && slot >= 0)
      store16_stream(oc.base + (int64_t)t * oc.ld, taps.template apply<SILU>(win, xt));
#pragma unroll
    for (int j = 0; j < W - 2; ++j)
#pragma unroll
      for (int v = 0; v < VN; ++v) win[j][v] = win[j + 1][v];
#pragma unroll
    for (int v = 0; v < VN; ++v) win[W - 2][v] = to_f32(xt[v]);
  }
}

// New taps of every sequence: its last W-1 inputs, carried ones included
// when it is shorter than W-1.  One thread per (sequence, channel vector)
// reads all of them before writing, so state_out may be state_in.
template <typename T, int W>
__global__ __launch_bounds__(kConvThreads) void conv_state_kernel(ConvParams p, int n_cblocks) {
  typedef typename CVec<T>::type V;
  constexpr int VN = CVec<T>::n;
  const int n = blockIdx.x / n_cblocks, cb = blockIdx.x - n * n_cblocks;
  const int cv = cb * kConvThreads + threadIdx.x;
  if (cv * VN >= p.dim) return;
  const int slot = slot_of(p, n);
  if (slot < 0) return;
  const int c0 = cv * VN;
  int s, e;
  seq_range(p, n, s, e);
  const __amdgpu_buffer_rsrc_t tr = taps_rsrc<T, W>(p, slot);
  const XRows<T> xw = x_rows<T>(p, max(e - (W - 1), s), e);
  float tap[W - 1][VN];
#pragma unroll
  for (int i = 0; i < W - 1; ++i) fetch<T, W>(p, tr, xw, c0, e - (W - 1) + i, s, tap[i]);
  T* out = reinterpret_cast<T*>(p.state_out) + (int64_t)slot * (W - 1) * p.dim + c0;
#pragma unroll
  for (int i = 0; i < W - 1; ++i) {
    V v;
#pragma unroll
    for (int k = 0; k < VN; ++k) v[k] = from_f32<T>(tap[i][k]);
    store16(out + (int64_t)i * p.dim, v);
  }
}

// One token per sequence: output row n and the taps shifted by one.
template <typename T, int W, bool SILU>
__global__ __launch_bounds__(kConvThreads) void conv_update_kernel(ConvParams p, int n_cblocks) {
  typedef typename CVec<T>::type V;
  constexpr int VN = CVec<T>::n;
  const int n = blockIdx.x / n_cblocks, cb = blockIdx.x - n * n_cblocks;
  const int cv = cb * kConvThreads + threadIdx.x;
  if (cv * VN >= p.dim) return;
  const int slot = slot_of(p, n);
  if (slot < 0) return;
  const int c0 = cv * VN;
  const V xt = load16(reinterpret_cast<const T*>(p.x) + (int64_t)n * p.dim + c0);
  const __amdgpu_buffer_rsrc_t tr = taps_rsrc<T, W>(p, slot);
  float win[W - 1][VN];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) fetch<T, W>(p, tr, x_rows<T>(p, 0, 0), c0, j - (W - 1), 0, win[j]);
  Taps<T, W> taps;
  taps.load(p, c0);
  const OutCol<T> oc = out_col<T>(p, c0);
  store16(oc.base + (int64_t)n * oc.ld, taps.template apply<SILU>(win, xt));
  if (!p.state_out) return;
  T* out = reinterpret_cast<T*>(p.state_out) + (int64_t)slot * (W - 1) * p.dim + c0;
#pragma unroll
  for (int i = 0; i < W - 2; ++i) {
    V v;
#pragma unroll
    for (int k = 0; k < VN; ++k) v[k] = from_f32<T>(win[i + 1][k]);
    store16(out + (int64_t)i * p.dim, v);
  }
  store16(out + (int64_t)(W - 2) * p.dim, xt);
}

ConvParams params_of(const ConvArgs& a) {
  ConvParams p;
  p.x = a.x;
  p.weight = a.weight;
  p.bias = a.bias;
  p.cu = a.cu_seqlens;
  p.state_in = a.state_in;
  p.state_out = a.state_out;
  p.slots = a.slots;
  p.n_slots = a.n_slots;
  p.n_seqs = a.n_seqs;
  p.dim = a.dim;
  p.rows = (int)a.rows;
  p.n_out = a.n_out;
  for (int i = 0; i < 3; ++i) p.y[i] = a.y[i];
  for (int i = 0; i < 4; ++i) p.y_off[i] = a.y_off[i];
  return p;
}

template <typename T, int W>
hipError_t fwd_w(const ConvArgs& a, hipStream_t st) {
  const ConvParams p = params_of(a);
  constexpr int VN = CVec<T>::n;
  const int ncb = (a.dim / VN + kConvThreads - 1) / kConvThreads;
  if (a.rows > 0) {
    const int64_t nb = (a.rows + kConvRun - 1) / kConvRun * ncb;
    if (a.act == CONV_SILU_)
      conv_fwd_kernel<T, W, true><<<dim3((unsigned)nb), dim3(kConvThreads), 0, st>>>(p, ncb);
    else
      conv_fwd_kernel<T, W, false><<<dim3((unsigned)nb), dim3(kConvThreads), 0, st>>>(p, ncb);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.state_out) {
    conv_state_kernel<T, W><<<dim3((unsigned)((int64_t)a.n_seqs * ncb)), dim3(kConvThreads), 0, st>>>(p, ncb);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T, int W>
hipError_t update_w(const ConvArgs& a, hipStream_t st) {
  const ConvParams p = params_of(a);
  constexpr int VN = CVec<T>::n;
  const int ncb = (a.dim / VN + kConvThreads - 1) / kConvThreads;
  const dim3 grid((unsigned)((int64_t)a.n_seqs * ncb));
  if (a.act == CONV_SILU_)
    conv_update_kernel<T, W, true><<<grid, dim3(kConvThreads), 0, st>>>(p, ncb);
  else
    conv_update_kernel<T, W, false><<<grid, dim3(kConvThreads), 0, st>>>(p, ncb);
  return hipGetLastError();
}

template <typename T>
hipError_t fwd_t(const ConvArgs& a, hipStream_t st) {
  switch (a.width) {
    case 2: return fwd_w<T, 2>(a, st);
    case 3: return fwd_w<T, 3>(a, st);
    default: return fwd_w<T, 4>(a, st);
  }
}
template <typename T>
hipError_t update_t(const ConvArgs& a, hipStream_t st) {
  switch (a.width) {
    case 2: return update_w<T, 2>(a, st);
    case 3: return update_w<T, 3>(a, st);
    default: return update_w<T, 4>(a, st);
  }
}

}  // namespace

int64_t conv_fwd_blocks(const ConvArgs& a) {
  const int vn = a.bf16 ? 8 : 4;
  const int64_t ncb = (a.dim / vn + kConvThreads - 1) / kConvThreads;
  return (a.rows + kConvRun - 1) / kConvRun * ncb + (int64_t)a.n_seqs * ncb;
}

hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t st) {
  return a.bf16 ? fwd_t<bf16>(a, st) : fwd_t<float>(a, st);
}

hipError_t launch_conv_update(const ConvArgs& a, hipStream_t st) {
  if (a.n_seqs == 0) return hipSuccess;
  return a.bf16 ? update_t<bf16>(a, st) : update_t<float>(a, st);
}

}  // namespace kda
