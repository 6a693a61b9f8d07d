// kda_headscan.hip -- the per-head state scan: the inter-chunk state
// recurrence with the GLA-style output fused in (page "spike(kimi-linear):
// chunk_kda prefill AOT port -- kernel set + pinned-config recipe", commit
// message and section Delivered), one workgroup per (sequence, head) reading
// each chunk-local block once.  The two-pass plan takes it for batches of more
// (sequence, head) pairs than half the device's CUs, where the scan is bound
// by workspace bytes rather than by the chain of chunks.  Built with
// the default instruction scheduler: the iterative ILP scheduler used for the
// chunk-local stage raises this kernel past the register file.
#include "kda_chunk_ops.h"
#include "kda_launch.h"

namespace kda {
namespace {

// Waves of a per-head scan workgroup (4: 32 columns each; 8: 16 each, two
// per SIMD within 256 registers, measured no faster: every wave reads all of
// W, Q' and Kg from LDS).
constexpr int kHeadScanWaves = 4;

// ---------------------------------------------------------------------------
// Per-head scan, bf16 operators.
//
// NW waves; wave w owns CPW = 8 / NW 16-column tiles of the whole state, all
// dk rows, in fp32 accumulator tiles S[mt][c] (rows 16mt + 4lg + j, column
// 16 (CPW w + c) + l16).  Every product of a step then stays inside the wave:
//   V  = U - W S          A = W (token rows), B = the wave's own state as
//                         kperm fragments (frag_from_d of two row tiles)
//   O  = Ol + (Q' S)      computed transposed, O^T = S^T Q'^T, with the same
//                         state fragments as A and the Q' fragments as B, so
//                         each lane holds four adjacent columns of one token
//                         and writes them with one 8-byte store
//   S' = diag(Gam) S + Kg^T V   B = V as kperm fragments of its own tiles
// Only the chunk's W, Q', Kg and Gam are needed by every wave: they are
// staged in LDS once per chunk, double buffered, so a step has one barrier.
// They are loaded into registers two chunks ahead and written to LDS at the
// end of the step before the chunk that reads them; U and Ol, of which a
// wave needs only its own columns, go to registers one chunk ahead.  Memory
// counters retire in order, so every load a step waits for was issued at
// least one step earlier than anything issued after it.  Within a step the
// LDS fragments of the next group of products are read before the current
// group's MFMAs issue (scheduling barriers keep that order).  Sums run in the
// same order as in the column-block scan, and Ol, the transposed product
// (ChunkLocal HEADL), rounds like the other: o and the states equal that
// scan's bit for bit.
template <int D, int C, int NW_ = 4>
struct HeadScan {
  using Gm = Geo<bf16, D, C>;
  static constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KBC = Gm::KBC;
  static constexpr int NW = NW_, NT = 64 * NW;
  static constexpr int CPW = DT / NW;  // column tiles per wave
  static constexpr int OPS_BYTES = (int)((Gm::W_ELEMS + Gm::Q_ELEMS + Gm::K_ELEMS) * 2);
  static constexpr int U_OFF = OPS_BYTES;
  static constexpr int OL_OFF = U_OFF + (int)Gm::U_ELEMS * 2;
  static constexpr int GAM_SRC = OL_OFF + (int)Gm::O_ELEMS * 2;  // Gam in the block
  static constexpr int BUF_BYTES = OPS_BYTES + D * 4;               // W, Q', Kg, Gam
  static constexpr int NPIECE = OPS_BYTES / 16 / NT;                // 16-byte pieces / thread
  static constexpr int LDS_BYTES = 2 * BUF_BYTES;
  static constexpr int KG_GROUP = 2;  // dk tiles per group of Kg products
  static_assert(C == 64 && D == 128 && DT % NW == 0, "per-head scan tiling");
  static_assert(OPS_BYTES % (16 * NT) == 0 && D / 4 <= NT, "staging split");
  static_assert(DT % KG_GROUP == 0, "Kg groups");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS size");

  // One chunk's W, Q', Kg and Gam as this thread loads them for staging.
  struct Ops {
    uint4 ops[NPIECE];
    uint4 gam;  // threads < D / 4
  };
  // One chunk's U and Ol for this wave's column tiles, two token tiles per
  // 16-byte load (the per-head layout), and its token range.
  static_assert(TT % 2 == 0, "paired token tiles");
  struct UO {
    uint4 u[CPW][TT / 2], ol[CPW][TT / 2];
    int start, len;
  };

  static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_of(const unsigned char* blk) {
    return make_rsrc(const_cast<unsigned char*>(blk), (int)Gm::OUT_BYTES);
  }
  static __device__ __forceinline__ void fetch_ops(Ops& p, const unsigned char* blk) {
    const int tid = threadIdx.x;
    const __amdgpu_buffer_rsrc_t r = rsrc_of(blk);
#pragma unroll
    for (int i = 0; i < NPIECE; ++i)
      p.ops[i] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (tid + NT * i) * 16, 0, 0));
    p.gam = __builtin_bit_cast(
        uint4, __builtin_amdgcn_raw_buffer_load_b128(
                   r, tid < D / 4 ? GAM_SRC + 16 * tid : kBufferOff, 0, 0));
  }
  static __device__ __forceinline__ void fetch_uo(UO& p, const unsigned char* blk,
                                                  const ChunkEnt* ent) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const __amdgpu_buffer_rsrc_t r = rsrc_of(blk);
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int tp = 0; tp < TT / 2; ++tp) {
        const int f = (((CPW * w + c) * (TT / 2) + tp) * 64 + lane) * 16;
        p.u[c][tp] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, U_OFF + f, 0, 0));
        p.ol[c][tp] =
            __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, OL_OFF + f, 0, 0));
      }
    p.start = ent->start;
    p.len = ent->len;
  }

  // The staged operators of `p` into LDS buffer `buf`.
  static __device__ __forceinline__ void stage(unsigned char* lds, int buf, const Ops& p) {
    const int tid = threadIdx.x;
    unsigned char* b = lds + buf * BUF_BYTES;
#pragma unroll
    for (int i = 0; i < NPIECE; ++i) *reinterpret_cast<uint4*>(b + (tid + NT * i) * 16) = p.ops[i];
    if (tid < D / 4) *reinterpret_cast<uint4*>(b + OPS_BYTES + 16 * tid) = p.gam;
  }

  // LDS fragments of one group of products.
  struct WQ {  // W and Q' of one token tile
    bf16x8 w[KBD], q[KBD];
  };
  struct KG {  // Kg and Gam of KG_GROUP dk tiles
    bf16x8 k[KG_GROUP][KBC];
    f32x4 gam[KG_GROUP];
  };
  static __device__ __forceinline__ void read_wq(WQ& f, const unsigned char* b, int t) {
    const int lane = threadIdx.x & 63;
    const bf16x8* Wl = reinterpret_cast<const bf16x8*>(b);
    const bf16x8* Ql = Wl + TT * KBD * 64;
#pragma unroll
    for (int s = 0; s < KBD; ++s) {
      f.w[s] = Wl[(t * KBD + s) * 64 + lane];
      f.q[s] = Ql[(t * KBD + s) * 64 + lane];
    }
  }
  static __device__ __forceinline__ void read_kg(KG& f, const unsigned char* b, int grp) {
    const int lane = threadIdx.x & 63, lg = lane >> 4;
    const bf16x8* Kl = reinterpret_cast<const bf16x8*>(b) + 2 * TT * KBD * 64;
    const float* Gl = reinterpret_cast<const float*>(b + OPS_BYTES);
#pragma unroll
    for (int i = 0; i < KG_GROUP; ++i) {
      const int mt = KG_GROUP * grp + i;
#pragma unroll
      for (int kc = 0; kc < KBC; ++kc) f.k[i][kc] = Kl[(mt * KBC + kc) * 64 + lane];
      f.gam[i] = *reinterpret_cast<const f32x4*>(Gl + 16 * mt + 4 * lg);
    }
  }

  // One chunk from LDS buffer `buf` and the registers of `p`; live = false
  // (uniform) leaves S and o untouched.
  static __device__ __forceinline__ void step(const unsigned char* lds, int buf, const UO& p,
                                              f32x4 (&S)[DT][CPW], bf16* __restrict__ o,
                                              int64_t ostride, int h, bool live) {
    __builtin_amdgcn_sched_barrier(0);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const unsigned char* b = lds + buf * BUF_BYTES;
    const int start = __builtin_amdgcn_readfirstlane(p.start);
    const int len = live ? __builtin_amdgcn_readfirstlane(p.len) : 0;
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(o + (int64_t)start * ostride, len * (int)ostride * 2);

    WQ fw[2];
    read_wq(fw[0], b, 0);
    bf16x8 sf[KBD][CPW];
#pragma unroll
    for (int s = 0; s < KBD; ++s)
#pragma unroll
      for (int c = 0; c < CPW; ++c) sf[s][c] = frag_from_d<bf16>(S[2 * s][c], S[2 * s + 1][c]);

    // V = U - W S and O = Ol + Q' S, one token tile per group
    f32x4 V[TT][CPW];
    KG fk[2];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t + 1 < TT) read_wq(fw[(t + 1) & 1], b, t + 1);
      else read_kg(fk[0], b, 0);
      __builtin_amdgcn_sched_barrier(0);
      const WQ& f = fw[t & 1];
      f32x4 pv[CPW], po[CPW];
#pragma unroll
      for (int c = 0; c < CPW; ++c) pv[c] = po[c] = zero4();
#pragma unroll
      for (int s = 0; s < KBD; ++s)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          pv[c] = mma32(f.w[s], sf[s][c], pv[c]);  // (W S)[16t + 4lg + j][col l16]
          po[c] = mma32(sf[s][c], f.q[s], po[c]);  // (Q' S)^T[col 4lg + j][16t + l16]
        }
      const int r = 16 * t + l16;  // token of this lane's O values
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const bf16x8 u8 = __builtin_bit_cast(bf16x8, p.u[c][t >> 1]);
        const bf16x8 ol8 = __builtin_bit_cast(bf16x8, p.ol[c][t >> 1]);
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          V[t][c][j] = (float)u8[4 * (t & 1) + j] - pv[c][j];
          ov[j] = (bf16)((float)ol8[4 * (t & 1) + j] + po[c][j]);
        }
        const int off = r < len ? (r * (int)ostride + h * D + 16 * (CPW * w + c) + 4 * lg) * 2
                                : kBufferOff;
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ov), orsrc, off, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // S' = diag(Gam) S + Kg^T V, KG_GROUP dk tiles per group
    bf16x8 vf[KBC][CPW];
#pragma unroll
    for (int kc = 0; kc < KBC; ++kc)
#pragma unroll
      for (int c = 0; c < CPW; ++c) vf[kc][c] = frag_from_d<bf16>(V[2 * kc][c], V[2 * kc + 1][c]);
    constexpr int NG = DT / KG_GROUP;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) read_kg(fk[(g + 1) & 1], b, g + 1);
      __builtin_amdgcn_sched_barrier(0);
      const KG& f = fk[g & 1];
#pragma unroll
      for (int i = 0; i < KG_GROUP; ++i) {
        const int mt = KG_GROUP * g + i;
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
          f32x4 sn = S[mt][c] * f.gam[i];
#pragma unroll
          for (int kc = 0; kc < KBC; ++kc) sn = mma32(f.k[i][kc], vf[kc][c], sn);
#pragma unroll
          for (int j = 0; j < 4; ++j) S[mt][c][j] = live ? sn[j] : S[mt][c][j];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

template <int D, int C, int NW>
__global__ __launch_bounds__(64 * NW) void head_scan_kernel(
    const void* __restrict__ h0, void* __restrict__ ht, bf16* __restrict__ o, int n_heads,
    const int* __restrict__ status, const int* __restrict__ chunk_off,
    const ChunkEnt* __restrict__ tab, const unsigned char* __restrict__ blocks, int ntu,
    const int* __restrict__ slots, int n_slots, int state_bf16) {
  using HS = HeadScan<D, C, NW>;
  using Gm = Geo<bf16, D, C>;
  constexpr int DT = HS::DT, CPW = HS::CPW;
  extern __shared__ __align__(16) unsigned char lds[];
  if (*status != 0) return;
  const int h = blockIdx.x % n_heads, n = blockIdx.x / n_heads;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  // h0 / ht of sequence n live in pool slot slots[n] (slot n without a slot
  // table); a negative slot skips the sequence (no o, no state)
  int slot = n;
  if (slots) {
    slot = slots[n];
    if (slot < 0 || slot >= n_slots) return;
  }
  const int lo = chunk_off[n], hi = chunk_off[n + 1];

  const size_t sbase = ((size_t)slot * n_heads + h) * D * D;
  auto el = [&](int mt, int c, int j) {
    return (16 * mt + 4 * lg + j) * D + 16 * (CPW * w + c) + l16;
  };
  // The entering state: h0 in fp32 or bf16, or zeros (no h0: an empty
  // buffer, whose loads read 0).  Two buffer resources, at most one of them
  // non-empty, so the loads take no branch.
  const bool from16 = h0 && state_bf16;
  const void* src32 = h0 && !state_bf16 ? (const void*)(static_cast<const float*>(h0) + sbase) : nullptr;
  const void* src16 = from16 ? (const void*)(static_cast<const bf16*>(h0) + sbase) : nullptr;
  const __amdgpu_buffer_rsrc_t r32 = make_rsrc(const_cast<void*>(src32), src32 ? D * D * 4 : 0);
  const __amdgpu_buffer_rsrc_t r16 = make_rsrc(const_cast<void*>(src16), src16 ? D * D * 2 : 0);
  f32x4 S[DT][CPW];
#pragma unroll
  for (int mt = 0; mt < DT; ++mt)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = el(mt, c, j);
        const float f32v = buffer_load_f32(r32, from16 ? kBufferOff : e * 4);
        const float b16v = (float)__builtin_bit_cast(
            bf16, __builtin_amdgcn_raw_buffer_load_b16(r16, from16 ? e * 2 : kBufferOff, 0, 0));
        S[mt][c][j] = from16 ? b16v : f32v;
      }
  // S enters the loop with nothing in flight (an empty asm that reads and
  // writes it; emits nothing)
#pragma unroll
  for (int mt = 0; mt < DT; ++mt)
#pragma unroll
    for (int c = 0; c < CPW; ++c) asm volatile("" : "+v"(S[mt][c]));

  if (lo < hi) {
    const int64_t ostride = (int64_t)n_heads * D;
    // past the sequence: its last chunk again (loaded, then unused)
    auto blk = [&](int ci) {
      ci = ci < hi ? ci : hi - 1;
      return blocks + ((size_t)h * ntu + ci) * Gm::OUT_BYTES;
    };
    auto ent = [&](int ci) { return tab + (ci < hi ? ci : hi - 1); };
    // Register sets alternate with the chunk's parity: ops of chunk ci + 2 go
    // to R[ci & 1] while the step of chunk ci runs, U / Ol of chunk ci + 1 to
    // Q[(ci + 1) & 1]; the step's end stages R of chunk ci + 1.
    typename HS::Ops r0, r1;
    typename HS::UO q0, q1;
    HS::fetch_ops(r0, blk(lo));
    HS::fetch_uo(q0, blk(lo), ent(lo));
    HS::fetch_ops(r1, blk(lo + 1));
    HS::stage(lds, 0, r0);
    __syncthreads();
    for (int ci = lo; ci < hi; ci += 2) {
      HS::fetch_ops(r0, blk(ci + 2));
      HS::fetch_uo(q1, blk(ci + 1), ent(ci + 1));
      HS::step(lds, 0, q0, S, o, ostride, h, true);
      HS::stage(lds, 1, r1);
      __syncthreads();
      HS::fetch_ops(r1, blk(ci + 3));
      HS::fetch_uo(q0, blk(ci + 2), ent(ci + 2));
      HS::step(lds, 1, q1, S, o, ostride, h, ci + 1 < hi);
      HS::stage(lds, 0, r0);
      __syncthreads();
    }
  }

  if (!ht) return;
#pragma unroll
  for (int mt = 0; mt < DT; ++mt)
#pragma unroll
    for (int c = 0; c < CPW; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const size_t e = sbase + el(mt, c, j);
        if (state_bf16) static_cast<bf16*>(ht)[e] = (bf16)S[mt][c][j];
        else static_cast<float*>(ht)[e] = S[mt][c][j];
      }
}

}  // namespace

hipError_t launch_head_scan(const PrefillArgs& a, const int* status, const int* chunk_off,
                            const ChunkEnt* tab, const unsigned char* blocks, int ntu,
                            hipStream_t stream) {
  constexpr int D = 128, C = 64, NW = kHeadScanWaves;
  using HS = HeadScan<D, C, NW>;
  hipError_t err = hipFuncSetAttribute((const void*)head_scan_kernel<D, C, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, HS::LDS_BYTES);
  if (err != hipSuccess) return err;
  const unsigned units = (unsigned)((int64_t)a.n_seqs * a.n_heads);
  hipLaunchKernelGGL((head_scan_kernel<D, C, NW>), dim3(units), dim3(HS::NT), HS::LDS_BYTES, stream,
                     a.h0, a.ht, (bf16*)a.o, a.n_heads, status, chunk_off, tab, blocks, ntu,
                     a.slots, a.n_slots, (int)a.state_bf16);
  return hipGetLastError();
}

}  // namespace kda
