// kda_launch.h -- internal interface between the C ABI (kda_abi.cpp) and the
// kernel launchers.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Decay input: g given (GATE_GIVEN_), or computed in the kernels from the raw
// gate x, a_log [H] and dt_bias [H, d] (GATE_KIMI_); values as kda_gate.
constexpr int GATE_GIVEN_ = 0;
constexpr int GATE_KIMI_ = 1;

struct GateArgs {
  int mode = GATE_GIVEN_;
  const void* x = nullptr;  // dtype of q
  const float* a_log = nullptr;
  const float* dt_bias = nullptr;
};

// Key/query heads and their normalisation: q and k rows hold kheads heads;
// value head h reads key head h / (n_heads / kheads); norm = 1 divides each
// q and k row by sqrt(sum of squares + 1e-6) before use.
struct QkArgs {
  int kheads = 0;  // Hg (== n_heads when not grouped)
  int norm = 0;
};

struct DecodeArgs {
  bool bf16;
  bool state_bf16 = false;  // the state is stored as bf16 (else fp32)
  int n_seqs, n_heads, d;
  QkArgs qk;
  float scale;
  void* state;
  const void *q, *k, *v;
  const float* g;
  const void* beta;
  void* o;
  GateArgs gate;
  const int* slots = nullptr;  // state pool slot per sequence, or NULL (slot n)
  int n_slots = 0;
};

struct PrefillArgs {
  bool bf16;
  bool state_bf16 = false;  // h0 / ht are stored as bf16 (else fp32)
  int n_seqs, n_heads, d, chunk;
  QkArgs qk;
  int64_t t_total;
  float scale;
  const void *q, *k, *v;
  const float* g;
  const void* beta;
  const void* h0;
  const int32_t* cu_seqlens;  // may be NULL when n_seqs == 1
  void* o;
  void* ht;
  GateArgs gate;
  const int* slots = nullptr;  // h0 / ht pool slot per sequence, or NULL (slot n)
  int n_slots = 0;
};

// Recurrent (token-by-token) prefill: the prefill arguments; it uses no chunk
// size and no workspace.
using RecurrentArgs = PrefillArgs;
hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream);

// Upper bound on the number of chunks: sum_n ceil(L_n / C) <= T / C + N.
inline int64_t max_chunks(int64_t t_total, int n_seqs, int chunk) {
  return t_total / chunk + n_seqs;
}

// Whether the (dtype, head dim, chunk) instance is built.
bool prefill_supported(bool bf16, int d, int chunk);
size_t prefill_workspace_bytes(const PrefillArgs& a);
// events: NULL, or four events recorded before the first launch and after
// each of the three launches.
hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream,
                          const hipEvent_t* events);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// The per-head state scan of the two-pass plan for batches (bf16, d = 128,
// chunk 64): one workgroup per (sequence, head) over the blocks the
// chunk-local stage wrote in the per-head layout (ntu chunks per head).
struct ChunkEnt;
hipError_t launch_head_scan(const PrefillArgs& a, const int* status, const int* chunk_off,
                            const ChunkEnt* tab, const unsigned char* blocks, int ntu,
                            hipStream_t stream);

// Short causal conv (values of kda_conv_act in include/kda_conv.h).
constexpr int CONV_NONE_ = 0;
constexpr int CONV_SILU_ = 1;

struct ConvArgs {
  bool bf16;
  int n_seqs, dim, width, act;
  int64_t rows;                 // t_total (forward) or n_seqs (update)
  const void* x;
  const float* weight;
  const float* bias;            // may be NULL
  const int32_t* cu_seqlens;    // forward; may be NULL when n_seqs == 1
  const void* state_in;         // may be NULL (zero taps)
  void* state_out;              // may be NULL, or equal to state_in
  const int* slots = nullptr;   // state slot per sequence, or NULL (slot n)
  int n_slots = 0;
  int n_out;                    // output column blocks, 1..3
  void* y[3];
  int y_off[4];                 // first channel of each block; y_off[n_out] = dim
};
// Workgroups the forward launches (both kernels).
int64_t conv_fwd_blocks(const ConvArgs& a);
hipError_t launch_conv_fwd(const ConvArgs& a, hipStream_t stream);
hipError_t launch_conv_update(const ConvArgs& a, hipStream_t stream);

// Offset of the device status word inside a prefill workspace.
constexpr size_t kWsStatusOffset = 0;

// The no-allocation prefill's workspace: a static device array of this many
// bytes (KDA_NOALLOC_WORKSPACE_BYTES), one per device, held until the process
// ends.  *ptr receives its address on the current device (looked up once per
// device with hipGetSymbolAddress).
constexpr size_t kNoAllocWorkspaceBytes = (size_t)64 << 20;
hipError_t noalloc_workspace(void** ptr);

}  // namespace kda
