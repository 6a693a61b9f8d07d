/*
 * kda_conv.h -- C ABI of libkda, part 2: the short causal convolution that
 * runs over the [q|k|v] channels just before the KDA step.
 *
 * The pages carry the taps of this convolution between calls in the same two
 * forms as the KDA state: a varlen forward over a packed prefill and a
 * one-token update in decode, with the conv state laid out as the
 * concatenated [q|k|v] channels (page "model(kimi_linear): ONE-SURFACE ROW 7
 * -- fold Kimi-Linear onto the shared paged runner", B2: CausalConv1dFwd
 * (varlen) / CausalConv1dUpdate (decode) in the conv_state.chunk(3) [q|k|v]
 * layout; page "Kimi-Linear: paged-incremental decode", squash commit: the
 * conv taps are carried from prefill into decode).  The pages name the ops
 * but not their formula; this library computes, per channel c with width W
 * and weight w[c, 0..W-1],
 *
 *     y[t, c] = act(bias[c] + sum_j w[c, j] * x[t - (W - 1) + j, c])
 *
 * where positions before the start of t's sequence read the carried taps:
 * state[slot, i, c] is the input at position start - (W - 1) + i (oldest
 * first).  After the call the state holds the sequence's last W - 1 inputs
 * (carried taps still among them when the sequence is shorter than W - 1).
 * act is the identity or SiLU, z / (1 + e^-z).
 *
 * Conventions are those of kda.h (struct_size, device pointers owned by the
 * caller, host-side checks before anything is enqueued, kda_status returns,
 * no allocation, no synchronisation).  Every tensor pointer here is read or
 * written as 16-byte vectors and must be 16-byte aligned.
 */
#ifndef KDA_CONV_H
#define KDA_CONV_H

#include "kda.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KDA_CONV_ACT_NONE = 0, KDA_CONV_ACT_SILU = 1 } kda_conv_act;

/* One descriptor for both entry points.
 *
 * Layouts: x [rows, dim] with rows = t_total (forward) or n_seqs (update);
 * weight [dim, W] fp32 (the depthwise kernel, tap j of channel c at
 * weight[c * W + j]); bias [dim] fp32; state_in / state_out
 * [n_state, W - 1, dim] in the dtype of x, n_state = n_slots when
 * state_indices is set, else n_seqs.
 *
 * Output: y is written as n_out column blocks: block i is a dense
 * [rows, y_width[i]] tensor at y[i] holding channels
 * y_width[0] + .. + y_width[i-1] onward.  With n_out = 3 and widths
 * H*dk, H*dk, H*dv the forward writes q, k and v as the separate contiguous
 * tensors kda_chunk_prefill reads, while the state stays in the
 * concatenated [q|k|v] layout.  n_out = 1 (or 0) with y_width[0] = dim (or 0)
 * writes one [rows, dim] tensor.
 *
 * State: state_in NULL reads zero taps; state_out NULL writes none.
 * state_out may be exactly state_in (in-place carry) but may not partly
 * overlap it.  With state_indices (device int32 [n_seqs]) sequence n uses
 * slot state_indices[n] of both; a negative index (or one >= n_slots) skips
 * the sequence: no y rows and no state are written for it.  Indices must be
 * distinct.
 *
 * Aliasing: no y block may overlap another y block, x, weight, bias, a state
 * buffer, cu_seqlens or state_indices; state_out may not overlap any input
 * but state_in (as above). */
typedef struct {
  uint32_t struct_size;         /* sizeof(kda_conv_desc)                        */
  int32_t dtype;                /* kda_dtype of x, y and the state              */
  int32_t n_seqs;               /* N: >= 1 for the forward, >= 0 for update    */
  int32_t dim;                  /* channels, a multiple of 8, 8 .. 2^24         */
  int32_t width;                /* W in {2, 3, 4}; 0 = 4                        */
  int32_t activation;           /* kda_conv_act                                 */
  int64_t t_total;              /* forward: packed tokens (>= 0); update: unused */
  const void* x;
  const float* weight;
  const float* bias;            /* NULL = no bias                               */
  const int32_t* cu_seqlens;    /* forward: device [N + 1], as in kda.h; NULL   */
                                /* allowed when N == 1.  update: unused         */
  const void* state_in;
  void* state_out;
  const int32_t* state_indices; /* NULL, or device [N] slots                    */
  int32_t n_slots;              /* pool size when state_indices is set          */
  int32_t n_out;                /* 1..3 output blocks; 0 = 1                    */
  void* y[3];
  int32_t y_width[3];           /* multiples of 8 summing to dim                */
} kda_conv_desc;

/* Varlen forward over a packed batch (page "model(kimi_linear): ONE-SURFACE
 * ROW 7", B2: CausalConv1dFwd (varlen)).  Sequence n covers rows
 * cu_seqlens[n] .. cu_seqlens[n+1]-1 of x and y.  cu_seqlens is read on the
 * device, clamped to [0, t_total]: contents that break the kda.h rules give
 * unspecified y and state but no access out of bounds; rows outside every
 * sequence are not written.  Enqueues two launches (outputs, then the new
 * taps), so an in-place state is read before it is replaced. */
int kda_causal_conv1d_fwd(const kda_conv_desc* d, void* stream);

/* One-token update for N sequences (page "model(kimi_linear): ONE-SURFACE
 * ROW 7", B2: CausalConv1dUpdate (decode)): row n of x is the next input of
 * sequence n; y row n is its output, and the sequence's taps shift by one.
 * Equal to kda_causal_conv1d_fwd with every length 1.  One launch. */
int kda_causal_conv1d_update(const kda_conv_desc* d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KDA_CONV_H */
