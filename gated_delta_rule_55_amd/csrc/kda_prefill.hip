// kda_prefill.hip -- chunked KDA prefill on gfx950.
//
// The pages describe the chunked prefill as a fixed kernel set: chunk-local
// cumulative sum of the per-channel log-decay, beta-scaled decayed K K^T
// (inter and intra sub-blocks), a unit-lower-triangular solve, a recompute of
// W/U with per-key-channel exp2 decay, the inter-chunk state recurrence
// delta_h, and a GLA-style output (page "spike(kimi-linear): chunk_kda prefill
// AOT port -- kernel set + pinned-config recipe", commit message and section
// Delivered).  Here the same arithmetic (kda_chunk_ops.h) runs in three
// launches: the chunk map (varlen chunk table from the device cu_seqlens), the
// chunk-local stage over every (chunk, head) into a workspace, and the state
// scan with the output fused in, which reads the workspace back.
#include <mutex>

#include "kda_chunk_ops.h"
#include "kda_launch.h"

namespace kda {

// Workspace of the no-allocation entry point (kda_chunk_prefill_noalloc):
// every device the library runs on holds its own copy until the process ends.
// Host code never uses this name as an address: it takes the device address
// from hipGetSymbolAddress (noalloc_workspace below).
static __device__ __align__(256) unsigned char scratch[kNoAllocWorkspaceBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch`, per device
}  // namespace

hipError_t noalloc_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {  // first use on this device, which is current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr int kErrSeqlens = -10;  // KDA_ERR_SEQLENS

// Workspace: [header 256 B: status][chunk_off (N+1) int][chunk table NTU]
// [blocks: H x NTU chunk-local result blocks, head-major, so the chunks of
// one head that the scan walks in order are contiguous].
struct WsLayout {
  size_t off_chunk_off, off_tab, off_blocks, total;
};

template <typename TIO, int D, int C>
WsLayout ws_layout(int n_seqs, int n_heads, int64_t ntu) {
  using Gm = Geo<TIO, D, C>;
  WsLayout L;
  L.off_chunk_off = 256;
  L.off_tab = align_up(L.off_chunk_off + sizeof(int) * (size_t)(n_seqs + 1), 256);
  L.off_blocks = align_up(L.off_tab + sizeof(ChunkEnt) * (size_t)ntu, 256);
  L.total = align_up(L.off_blocks + (size_t)ntu * n_heads * Gm::OUT_BYTES, 256);
  return L;
}

// ---------------------------------------------------------------------------
// a0: varlen chunk map.  One workgroup.  Validates cu_seqlens (cu[0] = 0,
// non-decreasing, cu[N] = T, chunk count within the bound) and writes, for
// every chunk, its sequence, first token, length and index within the
// sequence.  On invalid offsets no chunk is emitted and the status word says
// so.
__global__ __launch_bounds__(256) void chunk_map_kernel(const int32_t* __restrict__ cu,
                                                        int n_seqs, int64_t t_total, int chunk,
                                                        int64_t ntu, int* __restrict__ status,
                                                        int* __restrict__ chunk_off,
                                                        ChunkEnt* __restrict__ tab) {
  __shared__ int s_bad;
  __shared__ int s_scan[256];
  __shared__ int s_carry;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad = 0;
    s_carry = 0;
  }
  __syncthreads();
  auto cu_at = [&](int n) -> int64_t {
    if (cu) return cu[n];
    return n == 0 ? 0 : t_total;
  };
  for (int n = tid; n <= n_seqs; n += 256) {
    const int64_t c = cu_at(n);
    bool bad = (n == 0 && c != 0) || (n == n_seqs && c != t_total) || c < 0 || c > t_total;
    if (n < n_seqs && cu_at(n + 1) < c) bad = true;
    if (bad) atomicOr(&s_bad, 1);
  }
  __syncthreads();
  // Exclusive scan of per-sequence chunk counts, 256 sequences at a time.
  for (int base = 0; base < n_seqs && !s_bad; base += 256) {
    const int n = base + tid;
    int cnt = 0;
    if (n < n_seqs) cnt = (int)((cu_at(n + 1) - cu_at(n) + chunk - 1) / chunk);
    s_scan[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int add = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += add;
      __syncthreads();
    }
    const int incl = s_scan[tid];
    if (n < n_seqs) chunk_off[n] = s_carry + incl - cnt;
    __syncthreads();
    if (tid == 255) s_carry += incl;
    __syncthreads();
  }
  if (tid == 0) {
    if (!s_bad && s_carry > ntu) s_bad = 1;
    chunk_off[n_seqs] = s_bad ? 0 : s_carry;
    status[0] = s_bad ? kErrSeqlens : 0;
  }
  __syncthreads();
  if (s_bad) {
    for (int n = tid; n < n_seqs; n += 256) chunk_off[n] = 0;
    return;
  }
  // One table entry per thread: chunk i belongs to the last sequence whose
  // first chunk is <= i (empty sequences own no chunk, so the search never
  // stops on one).  A single long sequence fills its table in parallel.
  const int total = s_carry;
  for (int i = tid; i < total; i += 256) {
    int lo = 0, hi = n_seqs;  // chunk_off[lo] <= i < chunk_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (chunk_off[mid] <= i) lo = mid;
      else hi = mid;
    }
    const int j = i - chunk_off[lo];
    const int64_t p = cu_at(lo) + (int64_t)j * chunk, e = cu_at(lo + 1);
    ChunkEnt ent;
    ent.seq = lo;
    ent.start = (int)p;
    ent.len = (int)((e - p) < chunk ? (e - p) : chunk);
    ent.idx = j;
    tab[i] = ent;
  }
}

// ---------------------------------------------------------------------------
// Two-pass plan, stage 1: chunk-local stage for every (chunk, head).  A
// persistent grid (one workgroup per CU) walks the (chunk, head) items; the
// next item's inputs are loaded while the current one computes.
template <typename TIO, int D, int C, bool GATE, bool HEADL>
__global__ __launch_bounds__(kLocalThreads) void chunk_local_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    DecayIn<TIO> dec, const TIO* __restrict__ beta, int n_heads, QkIn qk, float scale,
    const int* __restrict__ chunk_total, const ChunkEnt* __restrict__ tab,
    unsigned char* __restrict__ blocks, int ntu) {
  using CL = ChunkLocal<TIO, D, C, GATE, HEADL>;
  using Gm = Geo<TIO, D, C>;
  extern __shared__ __align__(16) unsigned char lds[];
  const int n_items = *chunk_total * n_heads;
  // Items run from the last chunk to the first: the blocks written last are
  // still in the Infinity Cache when the scan starts, and it reads the first
  // chunks first.
  auto item = [&](int w) { return n_items - 1 - w; };
  auto fetch = [&](typename CL::Inputs& in, int w) {
    const int it = item(w);
    const ChunkEnt ent = tab[it / n_heads];
    CL::prefetch(in, q, k, v, dec, beta, n_heads, it % n_heads, ent.start, ent.len, qk);
  };
  typename CL::Inputs cur, nxt;
  auto compute = [&](const typename CL::Inputs& in, int w) {
    const int it = item(w);
    const ChunkOut<TIO> out = chunk_out_at<TIO, D, C>(
        blocks + ((size_t)(it % n_heads) * ntu + it / n_heads) * Gm::OUT_BYTES);
    CL::run(lds, in, scale, out, qk, [&] { CL::settle(nxt); });
    __syncthreads();  // the next item overwrites the LDS
  };
  int w = blockIdx.x;
  if (w < n_items) {
    fetch(cur, w);
    CL::settle(cur);
  }
  while (w < n_items) {
    const int w2 = w + gridDim.x;
    // in flight during this item (past the end: the last item again, unused),
    // issued unconditionally so the compiler's load counts stay exact, and
    // settled midway through it, before its output stores
    fetch(nxt, w2 < n_items ? w2 : n_items - 1);
    compute(cur, w);
    cur = nxt;
    w = w2;
  }
}

// Two-pass plan, stage 2: state scan with the output, one workgroup of D/32
// waves per (sequence, head, block of 16 NJ value columns), the next chunks'
// operators loaded while the current one computes.  The column blocks of a
// head all read the chunk's W, Q' and Kg, so wider blocks (NJ tiles of 16
// columns) cut that shared traffic through L2 at the price of fewer, busier
// workgroups.
//
// Which width is faster depends on the batch.  A step's latency grows with
// the width (more MFMA and LDS work per workgroup between barriers), while the
// L2 traffic for the shared operators shrinks with it; measured on MI355X at
// H = 32, d = 128, C = 64 (ms of the scan stage, before the 16-column blocks
// had their L2-warming wave, which took one sequence to 0.53):
//     one 32k sequence:   NJ 1: 0.59   NJ 2: 0.69   NJ 4: 1.04
//     four 32k sequences: NJ 1: 2.24   NJ 2: 1.48   NJ 4: 1.30
// A single sequence is bound by its chain of steps, a batch by the shared
// traffic.  The launch takes the widest block that still leaves every CU at
// least one workgroup (bf16 only: the fp32 fragments are twice the registers).
template <typename TIO, int D, int NJ>
constexpr int kScanTilesMax = (sizeof(TIO) == 2 && (D / 16) % NJ == 0) ? NJ : 1;

template <typename TIO, int D>
int scan_tiles(int n_seqs, int n_heads, int cus) {
  const int64_t heads = (int64_t)n_seqs * n_heads;
  for (int nj : {4, 2}) {
    if (sizeof(TIO) != 2 || (D / 16) % nj != 0) continue;
    if (heads * (D / 16 / nj) >= cus) return nj;
  }
  return 1;
}
// L2 warming: with WARM > 0 the workgroup has one more wave, which computes
// nothing; it writes each step's o from the staging buffer (between the
// step's two barriers, off the chain of steps), and WARM chunks ahead of the
// step the other waves compute, it touches one word of every 128-byte line of
// that chunk's block whose index is jb
// (mod NB), so the NB workgroups of a head bring the whole block into their
// XCD's L2 before their own loads ask for it.  It meets the other waves at
// their barriers (the same count), which keeps it WARM chunks ahead and no
// further, and consumes each load's value three steps after issuing it, so it
// never waits for memory before a barrier.
template <typename TIO, int D, int C, int NJ>
struct ScanWarm {
  static constexpr int NB = (D / 16) / NJ;
  static constexpr int LINES = (int)(Geo<TIO, D, C>::OUT_BYTES / 128);
  static constexpr int NL = (LINES + NB * 64 - 1) / (NB * 64);  // loads per lane per chunk
};

template <typename TIO, int D, int C, int NJ, int WARM>
__global__ __launch_bounds__(64 * (D / 32) + (WARM ? 64 : 0)) void state_scan_kernel(
    const void* __restrict__ h0, void* __restrict__ ht, TIO* __restrict__ o, int n_seqs,
    int n_heads, const int* __restrict__ status, const int* __restrict__ chunk_off,
    const ChunkEnt* __restrict__ tab, unsigned char* __restrict__ blocks, int ntu,
    const int* __restrict__ slots, int n_slots, int state_bf16) {
  using Gm = Geo<TIO, D, C>;
  using SS = ScanStep<TIO, D, C, NJ>;
  constexpr int NB = SS::NB;  // column blocks of 16 NJ columns per head
  extern __shared__ __align__(16) unsigned char lds[];
  if (*status != 0) return;

  // XCD-aware order: the NB column blocks of one (seq, head) share the chunk's
  // operators, so they go to workgroups with the same id mod 8 (same XCD L2).
  const int total = n_seqs * n_heads * NB;
  int y = blockIdx.x;
  if (total % 8 == 0) y = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int jb = y % NB;
  const int h = (y / NB) % n_heads;
  const int n = y / (NB * n_heads);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;

  // h0 / ht of sequence n live in pool slot slots[n] (slot n without a slot
  // table); a negative slot skips the sequence (no o, no state)
  int slot = n;
  if (slots) {
    slot = slots[n];
    if (slot < 0 || slot >= n_slots) return;
  }
  SS::clear_vt(lds);
  constexpr int NTH = 64 * (D / 32);  // threads of the computing waves
  if (WARM && (int)threadIdx.x >= NTH) {
    using SW = ScanWarm<TIO, D, C, NJ>;
    const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
    auto warm = [&](int ci, int (&r)[SW::NL]) {
      ci = ci < c_end ? ci : c_end - 1;
      const __amdgpu_buffer_rsrc_t rr =
          make_rsrc(blocks + ((size_t)h * ntu + ci) * Gm::OUT_BYTES, (int)Gm::OUT_BYTES);
#pragma unroll
      for (int i = 0; i < SW::NL; ++i)
        r[i] = __builtin_amdgcn_raw_buffer_load_b32(rr, (jb + NB * (lane + 64 * i)) * 128, 0, 0);
    };
    int ring[3][SW::NL];
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int i = 0; i < SW::NL; ++i) ring[u][i] = 0;
    int acc = 0;
    const int64_t ostride = (int64_t)n_heads * D;
    __syncthreads();
    for (int ci = c_begin; ci < c_end; ci += 3) {
#pragma unroll
      for (int u = 0; u < 3; ++u) {
#pragma unroll
        for (int i = 0; i < SW::NL; ++i) acc ^= ring[u][i];
        // the table entry is loaded before the warming loads, so using it
        // waits for nothing issued after it
        const bool live = ci + u < c_end;
        const ChunkEnt ent = tab[live ? ci + u : c_end - 1];
        warm(ci + u + WARM, ring[u]);
        __syncthreads();  // the two barriers of a step; o of the step between them
        SS::template store_o<64>(lds, o, ostride, h, jb, __builtin_amdgcn_readfirstlane(ent.start),
                                 live ? __builtin_amdgcn_readfirstlane(ent.len) : 0, lane);
        __syncthreads();
      }
    }
#pragma unroll
    for (int u = 0; u < 3; ++u)
#pragma unroll
      for (int i = 0; i < SW::NL; ++i) acc ^= ring[u][i];
    asm volatile("" ::"v"(acc));  // keeps the warming loads
    return;
  }
  f32x4 S[NJ][2];
  const size_t sbase = ((size_t)slot * n_heads + h) * D * D;
  // no h0: an empty buffer, whose loads read 0 (branch-free, so the compiler
  // keeps exact counts of the loads in flight); a bf16 state is widened
  const int ess = state_bf16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t hr = make_rsrc(
      const_cast<unsigned char*>(static_cast<const unsigned char*>(h0) + (h0 ? sbase * ess : 0)),
      h0 ? D * D * ess : 0);
#pragma unroll
  for (int c = 0; c < NJ; ++c)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = (32 * w + 16 * m + 4 * lg + j) * D + 16 * (NJ * jb + c) + l16;
        const float f32v = buffer_load_f32(hr, state_bf16 ? kBufferOff : e * 4);
        const float b16v = (float)__builtin_bit_cast(
            bf16, __builtin_amdgcn_raw_buffer_load_b16(hr, state_bf16 ? e * 2 : kBufferOff, 0, 0));
        S[c][m][j] = state_bf16 ? b16v : f32v;
      }
  // Take delivery of h0 here, before the operator loads are issued: S then
  // enters the loop with nothing in flight, and the loop's own waits are
  // counted exactly (an empty asm that reads and writes S; emits nothing).
#pragma unroll
  for (int c = 0; c < NJ; ++c)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(S[c][m][j]));
  SS::publish(lds, S);  // read by the first step after the barrier below

  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
  const int64_t ostride = (int64_t)n_heads * D;
  auto out_of = [&](int ci) {
    return chunk_out_at<TIO, D, C>(blocks + ((size_t)h * ntu + ci) * Gm::OUT_BYTES);
  };
  // Three chunks of operators in flight: each buffer keeps its role across the
  // unrolled loop, so no load waits on a later one.
  // Loads past the sequence's last chunk are clamped to it (read, then
  // unused), so every path issues the same loads and the compiler's wait
  // counts stay exact.  Three chunks of operators are in flight: each buffer
  // keeps its role across the unrolled loop, and a step refills its buffer
  // with the chunk three ahead piece by piece as it consumes it.
  typename SS::Ops b0, b1, b2;
  auto clamp = [&](int ci) { return ci < c_end ? ci : c_end - 1; };
  auto fetch = [&](typename SS::Ops& buf, int ci) {
    ci = clamp(ci);
    SS::load(buf, out_of(ci), jb);
    buf.start = tab[ci].start;
    buf.len = tab[ci].len;
  };
  // The three fetches stay in this order (scheduling barriers): the wait
  // counts at the loop head are merged over this prologue and the loop's
  // back edge, so a load of the first buffer that the scheduler sank below
  // the others would make every step wait on recent loads.
  if (c_begin < c_end) {
    fetch(b0, c_begin + 0);
    __builtin_amdgcn_sched_barrier(0);
    fetch(b1, c_begin + 1);
    __builtin_amdgcn_sched_barrier(0);
    fetch(b2, c_begin + 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();
  // The loop body runs its three steps unconditionally (a step past the last
  // chunk has no effect), so the body is one basic block and the compiler
  // cannot sink a refill toward the next iteration.
  auto run_step = [&](typename SS::Ops& buf, int ci) {
    const int cn = clamp(ci + 3);
    const ChunkOut<TIO> nx = out_of(cn);
    SS::template step<NTH, !WARM>(lds, S, buf, o, ostride, h, jb, &nx, tab + cn, ci < c_end);
  };
  for (int ci = c_begin; ci < c_end; ci += 3) {
    run_step(b0, ci);
    run_step(b1, ci + 1);
    run_step(b2, ci + 2);
  }
  if (ht) {
#pragma unroll
    for (int c = 0; c < NJ; ++c)
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const size_t e =
              sbase + (size_t)(32 * w + 16 * m + 4 * lg + j) * D + 16 * (NJ * jb + c) + l16;
          if (state_bf16) static_cast<bf16*>(ht)[e] = (bf16)S[c][m][j];
          else static_cast<float*>(ht)[e] = S[c][m][j];
        }
  }
}

// Chunks of lookahead of the L2-warming wave (0: no warming wave).
constexpr int kScanWarm = 4;

template <typename TIO, int D, int C, int NJ>
hipError_t launch_scan(const PrefillArgs& a, const int* status, const int* chunk_off,
                       const ChunkEnt* tab, unsigned char* blocks, int ntu, hipStream_t stream) {
  using SS = ScanStep<TIO, D, C, NJ>;
  // The warming wave halves the registers each wave may hold (five waves on
  // four SIMDs): only the one-tile bf16 scan leaves room for it.
  constexpr int WARM = (sizeof(TIO) == 2 && NJ == 1) ? kScanWarm : 0;
  static_assert(SS::LDS_BYTES <= 160 * 1024, "scan LDS");
  hipError_t err = hipFuncSetAttribute((const void*)state_scan_kernel<TIO, D, C, NJ, WARM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)SS::LDS_BYTES);
  if (err != hipSuccess) return err;
  const unsigned nblk = (unsigned)((int64_t)a.n_seqs * a.n_heads * SS::NB);
  hipLaunchKernelGGL((state_scan_kernel<TIO, D, C, NJ, WARM>), dim3(nblk),
                     dim3(64 * (D / 32) + (WARM ? 64 : 0)), SS::LDS_BYTES, stream, a.h0, a.ht,
                     (TIO*)a.o, a.n_seqs, a.n_heads, status, chunk_off, tab, blocks, ntu, a.slots,
                     a.n_slots, (int)a.state_bf16);
  return hipGetLastError();
}

// Stage 1 over every chunk of the table, blocks in the layout of the scan
// that follows (HEADL: the per-head scan's).
template <typename TIO, int D, int C, bool HEADL>
hipError_t launch_local(const PrefillArgs& a, const int* chunk_total, const ChunkEnt* tab,
                        unsigned char* blocks, int ntu, unsigned grid, hipStream_t stream) {
  using Gm = Geo<TIO, D, C>;
  const bool gate = a.gate.mode == GATE_KIMI_;
  const void* fn = gate ? (const void*)chunk_local_kernel<TIO, D, C, true, HEADL>
                        : (const void*)chunk_local_kernel<TIO, D, C, false, HEADL>;
  hipError_t err =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)Gm::LOCAL_LDS);
  if (err != hipSuccess) return err;
  const DecayIn<TIO> dec{a.g, static_cast<const TIO*>(a.gate.x), a.gate.a_log,
                         a.gate.dt_bias};
  if (gate)
    hipLaunchKernelGGL((chunk_local_kernel<TIO, D, C, true, HEADL>), dim3(grid),
                       dim3(kLocalThreads), Gm::LOCAL_LDS, stream, (const TIO*)a.q,
                       (const TIO*)a.k, (const TIO*)a.v, dec, (const TIO*)a.beta, a.n_heads,
                       QkIn{a.qk.kheads, a.qk.norm}, a.scale, chunk_total, tab, blocks, ntu);
  else
    hipLaunchKernelGGL((chunk_local_kernel<TIO, D, C, false, HEADL>), dim3(grid),
                       dim3(kLocalThreads), Gm::LOCAL_LDS, stream, (const TIO*)a.q,
                       (const TIO*)a.k, (const TIO*)a.v, dec, (const TIO*)a.beta, a.n_heads,
                       QkIn{a.qk.kheads, a.qk.norm}, a.scale, chunk_total, tab, blocks, ntu);
  return hipGetLastError();
}

template <typename TIO, int D, int C>
hipError_t launch_prefill_t(const PrefillArgs& a, void* workspace, hipStream_t stream,
                            const hipEvent_t* ev) {
  using Gm = Geo<TIO, D, C>;
  if constexpr (!Gm::FITS) {
    return hipErrorInvalidValue;
  } else {
    const int64_t ntu = max_chunks(a.t_total, a.n_seqs, C);
    const WsLayout L = ws_layout<TIO, D, C>(a.n_seqs, a.n_heads, ntu);
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    int* status = reinterpret_cast<int*>(ws + kWsStatusOffset);
    int* chunk_off = reinterpret_cast<int*>(ws + L.off_chunk_off);
    ChunkEnt* tab = reinterpret_cast<ChunkEnt*>(ws + L.off_tab);

    hipError_t err = hipSuccess;
    if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seqs,
                       a.t_total, C, ntu, status, chunk_off, tab);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;

    unsigned char* blocks = ws + L.off_blocks;
    int dev = 0, cus = 0;
    if ((err = hipGetDevice(&dev)) != hipSuccess) return err;
    if ((err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
      return err;
    // Batches of more (sequence, head) pairs than half the CUs take the
    // per-head scan, which reads each block once and runs one workgroup per
    // pair; fewer pairs the column-block scan, whose chain of chunks is
    // shorter per step and which then still fits one round of workgroups
    // (measured on MI355X, H = 32, 4096 tokens per sequence: 128 pairs
    // 0.187 ms column-block against 0.241 per-head, 192 pairs 0.333 against
    // 0.278).
    constexpr bool kHeadBuilt = sizeof(TIO) == 2 && D == 128 && C == 64;
    const bool head = kHeadBuilt && (int64_t)a.n_seqs * a.n_heads * 2 > cus;
    const int64_t items = ntu * a.n_heads;
    const unsigned grid = (unsigned)(items < cus ? items : cus);
    if (head) err = launch_local<TIO, D, C, kHeadBuilt>(a, chunk_off + a.n_seqs, tab, blocks, (int)ntu, grid, stream);
    else err = launch_local<TIO, D, C, false>(a, chunk_off + a.n_seqs, tab, blocks, (int)ntu, grid, stream);
    if (err != hipSuccess) return err;
    if (ev && (err = hipEventRecord(ev[2], stream)) != hipSuccess) return err;
    if (head) {
      err = launch_head_scan(a, status, chunk_off, tab, blocks, (int)ntu, stream);
    } else {
      switch (scan_tiles<TIO, D>(a.n_seqs, a.n_heads, cus)) {
        case 4: err = launch_scan<TIO, D, C, kScanTilesMax<TIO, D, 4>>(a, status, chunk_off, tab, blocks, (int)ntu, stream); break;
        case 2: err = launch_scan<TIO, D, C, kScanTilesMax<TIO, D, 2>>(a, status, chunk_off, tab, blocks, (int)ntu, stream); break;
        default: err = launch_scan<TIO, D, C, 1>(a, status, chunk_off, tab, blocks, (int)ntu, stream); break;
      }
    }
    if (err != hipSuccess) return err;
    if (ev && (err = hipEventRecord(ev[3], stream)) != hipSuccess) return err;
    return hipSuccess;
  }
}

template <typename TIO, int D>
size_t ws_bytes_c(const PrefillArgs& a) {
  const int64_t ntu = max_chunks(a.t_total, a.n_seqs, a.chunk);
  switch (a.chunk) {
    case 16: return ws_layout<TIO, D, 16>(a.n_seqs, a.n_heads, ntu).total;
    case 32: return ws_layout<TIO, D, 32>(a.n_seqs, a.n_heads, ntu).total;
    case 64: return ws_layout<TIO, D, 64>(a.n_seqs, a.n_heads, ntu).total;
  }
  return 0;
}

template <typename TIO, int D>
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t s, const hipEvent_t* ev) {
  switch (a.chunk) {
    case 16: return launch_prefill_t<TIO, D, 16>(a, ws, s, ev);
    case 32: return launch_prefill_t<TIO, D, 32>(a, ws, s, ev);
    case 64: return launch_prefill_t<TIO, D, 64>(a, ws, s, ev);
  }
  return hipErrorInvalidValue;
}

template <typename TIO>
size_t ws_bytes_d(const PrefillArgs& a) {
  switch (a.d) {
    case 32: return ws_bytes_c<TIO, 32>(a);
    case 64: return ws_bytes_c<TIO, 64>(a);
    case 128: return ws_bytes_c<TIO, 128>(a);
  }
  return 0;
}

template <typename TIO>
hipError_t launch_d(const PrefillArgs& a, void* ws, hipStream_t s, const hipEvent_t* ev) {
  switch (a.d) {
    case 32: return launch_c<TIO, 32>(a, ws, s, ev);
    case 64: return launch_c<TIO, 64>(a, ws, s, ev);
    case 128: return launch_c<TIO, 128>(a, ws, s, ev);
  }
  return hipErrorInvalidValue;
}

template <typename TIO>
bool fits_d_c(int d, int c) {
  switch (d * 1000 + c) {
    case 32016: return Geo<TIO, 32, 16>::FITS;
    case 32032: return Geo<TIO, 32, 32>::FITS;
    case 32064: return Geo<TIO, 32, 64>::FITS;
    case 64016: return Geo<TIO, 64, 16>::FITS;
    case 64032: return Geo<TIO, 64, 32>::FITS;
    case 64064: return Geo<TIO, 64, 64>::FITS;
    case 128016: return Geo<TIO, 128, 16>::FITS;
    case 128032: return Geo<TIO, 128, 32>::FITS;
    case 128064: return Geo<TIO, 128, 64>::FITS;
  }
  return false;
}

}  // namespace

bool prefill_supported(bool bf16, int d, int chunk) {
  return bf16 ? fits_d_c<kda::bf16>(d, chunk) : fits_d_c<float>(d, chunk);
}

size_t prefill_workspace_bytes(const PrefillArgs& a) {
  return a.bf16 ? ws_bytes_d<bf16>(a) : ws_bytes_d<float>(a);
}

hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream,
                          const hipEvent_t* ev) {
  return a.bf16 ? launch_d<bf16>(a, workspace, stream, ev)
                : launch_d<float>(a, workspace, stream, ev);
}

}  // namespace kda
