// kda_chunk_ops.h -- device building blocks of the chunked KDA prefill:
//   ChunkLocal  the chunk-local stage for one (chunk, head) by one 512-thread
//               workgroup: cumulative decay, decayed Gram matrices, triangular
//               solve, W/U and the chunk's output operators
//   ScanStep    one step of the inter-chunk state recurrence with the output
//               fused in, split over the workgroup's four waves by dk slice
//
// Per chunk of L <= C tokens (rows r, i), with G the inclusive cumulative sum
// of g over the chunk in base 2 (G = log2(e) cumsum(g)), so every decay factor
// is one exp2:
//   A   [r,i] = beta_r sum_c k[r,c] k[i,c] 2^(G[r,c]-G[i,c])     i <  r
//   Aqk [r,i] =        sum_c q[r,c] k[i,c] 2^(G[r,c]-G[i,c])     i <= r
//   T   = (I + A)^-1
//   W   = T diag(beta) (K * 2^G)          U = T diag(beta) V
//   Q'  = scale (Q * 2^G - Aqk W)         Ol = scale Aqk U
//   Kg  = K * 2^(G_last - G)              Gam = 2^G_last
// and the scan over chunks, for the fp32 state S:
//   V = U - W S;   O = Q' S + Ol;   S = diag(Gam) S + Kg^T V.
//
// Decay factors without overflow.  The chunk is cut into 16-token blocks with
// reference points rho_a = G[16a] (block starts) and rho_TT = G[C-1].  Every
// row gets two factors, each <= 1 when g <= 0:
//   Lk[r] = k[r] 2^(G[r] - rho_blk(r))        Lq[r] = q[r] 2^(G[r] - rho_blk(r))
//   Rn[i] = k[i] 2^(rho_blk(i)+1 - G[i])
// and a Gram tile (a, b) is Lk_a . Rn_b^T times the per-channel factor
// 2^(rho_a - rho_{b+1}): 1 for adjacent blocks, <= 1 for farther ones, and the
// block's own decay span (>= 1) on the diagonal.  The diagonal factor is the
// only one above 1; when it exceeds 2^64 for some channel the block's tile is
// summed entry by entry, each term with its own exact factor 2^(G[r]-G[i]) <= 1,
// from the staged k, q and G before the scaled operands replace them.  W, Kg
// and Q * 2^G reuse Lk, Rn and Lq with one more per-channel factor, so each
// element costs two exp2.
#pragma once

#include "kda_device.h"

namespace kda {

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t cmaxz(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kLocalThreads = 512;  // threads of a chunk-local workgroup (8 waves)
constexpr float kSpanMax = 64.0f;  // largest log2 diagonal factor taken on the factored path

// Chunk table entry.
struct ChunkEnt {
  int seq, start, len, idx;
};

// Where one (chunk, head) block of chunk-local outputs lives.
template <typename TIO>
struct ChunkOut {
  TIO *w, *q, *k, *u, *o;
  float* gam;
};

// ---------------------------------------------------------------------------
// Compile-time geometry of one (dtype, head dim, chunk) instance.
template <typename TIO, int D, int C>
struct Geo {
  static constexpr int TT = C / 16;            // token tiles
  static constexpr int DT = D / 16;            // channel tiles
  static constexpr int KBD = D / 32;           // 32-slices over channels (= scan waves)
  static constexpr int KCP = cmax(C, 32);      // token extent padded to a slice
  static constexpr int KBC = KCP / 32;         // 32-slices over tokens
  static constexpr int TP = 16 / sizeof(TIO);  // row pad (elements) = 16 bytes
  // Chunk-local outputs per (chunk, head), in elements of TIO (Gam in floats).
  static constexpr size_t W_ELEMS = (size_t)C * D;    // W^T fragments
  static constexpr size_t Q_ELEMS = (size_t)C * D;    // Q'^T fragments
  static constexpr size_t K_ELEMS = (size_t)KCP * D;  // Kg^T fragments
  static constexpr size_t U_ELEMS = (size_t)C * D;    // U, accumulator order
  static constexpr size_t O_ELEMS = (size_t)C * D;    // Ol, accumulator order
  static constexpr size_t OUT_BYTES = align_up(
      (W_ELEMS + Q_ELEMS + K_ELEMS + U_ELEMS + O_ELEMS) * sizeof(TIO) + (size_t)D * 4, 256);

  // Chunk-local LDS layout (bytes).  Region A holds G until the Gram stage,
  // then A and T, then W^T.
  static constexpr int GS_LD = D + 8;     // fp32 rows of D
  static constexpr int KS_LD = D + TP;    // TIO rows of D
  static constexpr int TK_LD = KCP + TP;  // TIO rows of tokens
  static constexpr int AF_LD = C + 4;     // fp32 rows of C
  // The cumulative-sum phase has the LPC lanes of a channel scan LPC segments
  // of SEG tokens each, rows SEG apart; rows of G are skewed by CPW floats per
  // segment so the LPC segments of a wave's CPW channels fall in distinct
  // banks (without the skew, GS_LD * SEG is a multiple of the 64 banks).
  static constexpr int NWL = kLocalThreads / 64;
  static constexpr int GS_CPW = D / NWL, GS_LPC = 64 / GS_CPW, GS_SEG = C / GS_LPC;
  static_assert(GS_SEG >= 1 && GS_CPW % 4 == 0, "cumulative-sum tiling");
  static __host__ __device__ constexpr int gs_row(int r) { return r * GS_LD + (r / GS_SEG) * GS_CPW; }
  static constexpr size_t SZ_G = ((size_t)C * GS_LD + (size_t)(GS_LPC - 1) * GS_CPW) * 4;
  static constexpr size_t SZ_A = cmaxz(cmaxz(SZ_G, (size_t)2 * C * AF_LD * 4),
                                       (size_t)D * TK_LD * sizeof(TIO));
  static constexpr size_t OFF_GS = 0;
  static constexpr size_t OFF_AS = 0;
  static constexpr size_t OFF_TS = (size_t)C * AF_LD * 4;
  static constexpr size_t OFF_WT = 0;
  static constexpr size_t OFF_LK = align_up(SZ_A, 16);
  static constexpr size_t OFF_LQ = OFF_LK + (size_t)C * KS_LD * sizeof(TIO);
  static constexpr size_t OFF_RN = OFF_LQ + (size_t)C * KS_LD * sizeof(TIO);
  static constexpr size_t OFF_KBT = OFF_RN + (size_t)C * KS_LD * sizeof(TIO);
  static constexpr size_t OFF_VBT = OFF_KBT + (size_t)D * TK_LD * sizeof(TIO);
  static constexpr size_t OFF_TB = OFF_VBT + (size_t)D * TK_LD * sizeof(TIO);
  static constexpr size_t OFF_AQ = OFF_TB + (size_t)C * TK_LD * sizeof(TIO);
  static constexpr size_t OFF_VS = OFF_RN;  // raw v, row-major, until the scaled operands
  static constexpr size_t OFF_RHO = align_up(OFF_AQ + (size_t)C * TK_LD * sizeof(TIO), 16);
  // Per-channel factor vectors: 2^rho_a (TT), diagonal 2^(rho_a - rho_a+1) (TT),
  // Kg 2^(rho_TT - rho_b+1) (TT), far pairs 2^(rho_a - rho_b+1), b <= a - 2.
  static constexpr int NFAR = TT >= 3 ? (TT - 1) * (TT - 2) / 2 : 0;
  static constexpr int NFAC = 3 * TT + NFAR;
  static constexpr size_t OFF_FAC = OFF_RHO + (size_t)(TT + 1) * D * 4;
  static constexpr size_t OFF_BETA = OFF_FAC + (size_t)NFAC * D * 4;
  static constexpr size_t OFF_FLAG = OFF_BETA + (size_t)C * 4;
  // Exact diagonal Gram tiles [TT][2][16][16] fp32 (A_kk, A_qk) for blocks
  // whose decay span is too large to factor: in the T region (not in use
  // until the triangular solve) when they fit there, else after the flags.
  static constexpr size_t EXACT_BYTES = (size_t)TT * 2 * 256 * 4;
  static constexpr bool EXACT_IN_T = EXACT_BYTES <= (size_t)C * TK_LD * sizeof(TIO);
  static constexpr size_t OFF_EXACT = EXACT_IN_T ? OFF_TB : OFF_FLAG + 16;
  static constexpr size_t LOCAL_LDS =
      align_up(EXACT_IN_T ? OFF_FLAG + 16 : OFF_EXACT + EXACT_BYTES, 16);

  // Scan-step V^T rows (tokens padded to a 32-slice, plus a 16-byte pad).
  static constexpr int VT_LD = KCP + TP;

  static constexpr bool FITS = LOCAL_LDS <= 160 * 1024;
};

template <typename TIO, int D, int C>
__device__ __forceinline__ ChunkOut<TIO> chunk_out_at(unsigned char* base) {
  using Gm = Geo<TIO, D, C>;
  ChunkOut<TIO> p;
  p.w = reinterpret_cast<TIO*>(base);
  p.q = p.w + Gm::W_ELEMS;
  p.k = p.q + Gm::Q_ELEMS;
  p.u = p.k + Gm::K_ELEMS;
  p.o = p.u + Gm::U_ELEMS;
  p.gam = reinterpret_cast<float*>(p.o + Gm::O_ELEMS);
  return p;
}

// Within-wave ordering of LDS traffic between lanes.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Lane moves within a row of 16 lanes (DPP).  Lanes without a source read 0.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
// Value of lane i of this lane's 16-lane row (row_newbcast:i); i a constant
// after unrolling.
__device__ __forceinline__ float row_bcast(float x, int i) {
  switch (i) {
    case 0: return dpp<0x150>(x);
    case 1: return dpp<0x151>(x);
    case 2: return dpp<0x152>(x);
    case 3: return dpp<0x153>(x);
    case 4: return dpp<0x154>(x);
    case 5: return dpp<0x155>(x);
    case 6: return dpp<0x156>(x);
    case 7: return dpp<0x157>(x);
    case 8: return dpp<0x158>(x);
    case 9: return dpp<0x159>(x);
    case 10: return dpp<0x15A>(x);
    case 11: return dpp<0x15B>(x);
    case 12: return dpp<0x15C>(x);
    case 13: return dpp<0x15D>(x);
    case 14: return dpp<0x15E>(x);
    default: return dpp<0x15F>(x);
  }
}

// ---------------------------------------------------------------------------
// Chunk-local stage.
// The decay input of the chunk-local stage: g (fp32, natural log) when GATE
// is false, else the raw gate x (TIO), a_log [H] and dt_bias [H, D].
template <typename TIO>
struct DecayIn {
  const float* g;
  const TIO* x;
  const float* a_log;
  const float* dt_bias;
};

// Key heads and q/k normalisation: q and k rows hold kheads heads, value
// head h reads key head h / (n_heads / kheads); norm = 1 divides each q and k
// row by sqrt(sum of squares + kQkNormEps) when it is staged.
struct QkIn {
  int kheads;
  int norm;
};

// HEADL: the layout the per-head scan reads.  Ol is written transposed
// within each 16 x 16 tile (lane l16 holds token 16t + l16, lane group lg its
// value columns 16ct + 4lg + 0..3), the layout of that scan's output tiles,
// and the token tiles 2p, 2p + 1 of one column tile of U and of Ol sit side
// by side for each lane, written with one 16-byte store (elements
// ((ct TT/2 + p) 64 + lane) 8 + 4 (t & 1) + j).  Else U and Ol are in
// accumulator order, ((t DT + ct) 64 + lane) 4 + j.
template <typename TIO, int D, int C, bool GATE = false, bool HEADL = false>
struct ChunkLocal {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  using V4 = typename Vec4<TIO>::type;
  static constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KCP = Gm::KCP, KBC = Gm::KBC;
  static constexpr int GS_LD = Gm::GS_LD, KS_LD = Gm::KS_LD, TK_LD = Gm::TK_LD,
                       AF_LD = Gm::AF_LD;
  static constexpr int NT = kLocalThreads;          // threads of the workgroup
  static constexpr int NW = NT / 64;                // waves
  static constexpr int EPV = 16 / sizeof(TIO);      // elements per 16-byte vector
  static constexpr int VPR = D / EPV;               // vectors per row of q, k, v
  static constexpr int NV = (C * VPR + NT - 1) / NT;  // vectors per thread per tensor
  static constexpr int GPR = D / 4;                 // float4 per row of g
  static constexpr int NG = (C * GPR + NT - 1) / NT;  // float4 per thread of g

  // The chunk's inputs as this thread loads them.  Every load is issued
  // unconditionally (rows at or past L fall outside the buffer resource and
  // read 0) and the masking happens when the registers are staged, so the
  // compiler can count the loads in flight and never has to wait for the
  // whole prefetch early.
  struct Inputs {
    uint4 k[NV], q[NV], v[NV];
    f32x4 g[GATE ? 1 : NG];     // g, four channels per vector
    V4 x[GATE ? NG : 1];        // or the raw gate
    f32x4 bias[GATE ? NG : 1];  // and dt_bias for the same channels
    float ea;                   // exp(a_log[h])
    TIO beta;
    int64_t tok0;
    int len;
  };

  static __device__ __forceinline__ uint4 mask4(uint4 a, unsigned mk) {
    return uint4{a.x & mk, a.y & mk, a.z & mk, a.w & mk};
  }

  // Divide the row that VPR consecutive lanes hold (one 16-byte vector each)
  // by sqrt(sum of squares + eps); returns the factor.  Every lane of the
  // wave must call it.
  static __device__ __forceinline__ float normalise_row(uint4& u) {
    float f[EPV];
    if constexpr (EPV == 8) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, u);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (float)b[e];
    } else {
      const f32x4 b = __builtin_bit_cast(f32x4, u);
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = b[e];
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPV; ++e) ss += f[e] * f[e];
#pragma unroll
    for (int o = 1; o < VPR; o <<= 1) ss += __shfl_xor(ss, o, 64);
    const float r = __builtin_amdgcn_rsqf(ss + kQkNormEps);
    if constexpr (EPV == 8) {
      bf16x8 b;
#pragma unroll
      for (int e = 0; e < 8; ++e) b[e] = (bf16)(f[e] * r);
      u = __builtin_bit_cast(uint4, b);
    } else {
      f32x4 b;
#pragma unroll
      for (int e = 0; e < 4; ++e) b[e] = f[e] * r;
      u = __builtin_bit_cast(uint4, b);
    }
    return r;
  }

  // Issue every global load of one (chunk, head); nothing waits on them here.
  static __device__ __forceinline__ void prefetch(Inputs& in, const TIO* __restrict__ q,
                                                  const TIO* __restrict__ k,
                                                  const TIO* __restrict__ v,
                                                  const DecayIn<TIO>& dec,
                                                  const TIO* __restrict__ beta, int n_heads,
                                                  int h, int64_t tok0, int L, QkIn qk) {
    const int tid = threadIdx.x;
    const int64_t rs = (int64_t)n_heads * D;
    const int64_t ks = (int64_t)qk.kheads * D;                      // q / k row stride
    const int64_t kh = (int64_t)(h / (n_heads / qk.kheads)) * D;    // key head offset
    in.tok0 = tok0;
    in.len = L;
    // Buffer resources over the chunk's L rows of this head: the per-thread
    // offsets depend only on the thread (no address arithmetic per item), and
    // rows at or past L read as 0 (they are masked when staged anyway).  Byte
    // offsets stay below 2^31 for every shape the C ABI accepts (at most
    // 65535 heads: 64 rows x 65535 x 128 x 4 bytes < 2^31).
    const int kst = (int)(ks * sizeof(TIO)), rst = (int)(rs * sizeof(TIO));
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(const_cast<TIO*>(k) + tok0 * ks + kh, L * kst);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(const_cast<TIO*>(q) + tok0 * ks + kh, L * kst);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(const_cast<TIO*>(v) + tok0 * rs + (int64_t)h * D, L * rst);
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int x0 = tid + NT * m;
      const int x = x0 < C * VPR ? x0 : C * VPR - 1;
      const int r = x / VPR, cv = x % VPR;
      in.k[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rk, r * kst + cv * 16, 0, 0));
      in.q[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rq, r * kst + cv * 16, 0, 0));
      in.v[m] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, r * rst + cv * 16, 0, 0));
    }
    const int gst = (int)(rs * (GATE ? sizeof(TIO) : 4));
    const __amdgpu_buffer_rsrc_t rg =
        GATE ? make_rsrc(const_cast<TIO*>(dec.x) + tok0 * rs + (int64_t)h * D, L * gst)
             : make_rsrc(const_cast<float*>(dec.g) + tok0 * rs + (int64_t)h * D, L * gst);
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const int x0 = tid + NT * m;
      const int x = x0 < C * GPR ? x0 : C * GPR - 1;
      const int r = x / GPR, cv = x % GPR;
      if constexpr (GATE) {
        if constexpr (sizeof(TIO) == 2)
          in.x[m] = __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b64(rg, r * gst + cv * 8, 0, 0));
        else
          in.x[m] = __builtin_bit_cast(V4, __builtin_amdgcn_raw_buffer_load_b128(rg, r * gst + cv * 16, 0, 0));
        in.bias[m] = reinterpret_cast<const f32x4*>(dec.dt_bias + (int64_t)h * D)[cv];
      } else {
        in.g[m] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, r * gst + cv * 16, 0, 0));
      }
    }
    in.ea = GATE ? __expf(dec.a_log[h]) : 1.f;
    const __amdgpu_buffer_rsrc_t rb =
        make_rsrc(const_cast<TIO*>(beta) + tok0 * n_heads + h, L * n_heads * (int)sizeof(TIO));
    if constexpr (sizeof(TIO) == 2)
      in.beta = __builtin_bit_cast(TIO, (unsigned short)__builtin_amdgcn_raw_buffer_load_b16(
                                             rb, tid * n_heads * 2, 0, 0));
    else
      in.beta = __builtin_bit_cast(TIO, __builtin_amdgcn_raw_buffer_load_b32(rb, tid * n_heads * 4, 0, 0));
  }

  static __device__ __forceinline__ int fac_sa(int a) { return a; }
  static __device__ __forceinline__ int fac_diag(int a) { return TT + a; }
  static __device__ __forceinline__ int fac_kg(int b) { return 2 * TT + b; }
  static __device__ __forceinline__ int fac_far(int a, int b) {
    return 3 * TT + (a - 2) * (a - 1) / 2 + b;
  }
  // Element offset of a lane's four values of U / Ol tile (t, ct).
  static __device__ __forceinline__ size_t tile_off(int t, int ct, int lane) {
    if constexpr (HEADL) {
      static_assert(TT % 2 == 0, "paired token tiles");
      return ((size_t)(ct * (TT / 2) + (t >> 1)) * 64 + lane) * 8 + 4 * (t & 1);
    } else {
      return ((size_t)(t * DT + ct) * 64 + lane) * 4;
    }
  }
  // Store a lane's four values of U / Ol tile (t, ct); in the per-head layout
  // the odd token tile stores both of its pair (prev: the even tile's).
  static __device__ __forceinline__ void store_tile(TIO* base, int t, int ct, int lane, f32x4 v,
                                                    f32x4 prev, float sc) {
    if constexpr (HEADL && sizeof(TIO) == 2) {
      if (t & 1) {
        bf16x8 f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f[j] = (bf16)(sc * prev[j]);
          f[4 + j] = (bf16)(sc * v[j]);
        }
        *reinterpret_cast<bf16x8*>(base + tile_off(t - 1, ct, lane)) = f;
      }
    } else {
      TIO* p = base + tile_off(t, ct, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = from_f32<TIO>(sc * v[j]);
    }
  }

  // Scale the 8 values of a bf16 / fp32 fragment by 8 per-channel factors.
  static __device__ __forceinline__ FragT scale8(FragT f, const float* fac) {
    const f32x4 f0 = *reinterpret_cast<const f32x4*>(fac);
    const f32x4 f1 = *reinterpret_cast<const f32x4*>(fac + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = from_f32<TIO>(to_f32(f[e]) * f0[e]);
      f[4 + e] = from_f32<TIO>(to_f32(f[4 + e]) * f1[e]);
    }
    return f;
  }

  // Take delivery of every load prefetch() issued into `in` (emits only the
  // wait).  Memory counters retire in order and count stores too, so a
  // prefetch waited for after the previous item's stores would also wait for
  // those stores; settling it before they are issued avoids that.
  template <typename T>
  static __device__ __forceinline__ void touch(T& x) {
    using R = unsigned __attribute__((ext_vector_type(sizeof(T) / 4)));
    static_assert(sizeof(T) % 4 == 0 && sizeof(T) >= 8, "register group");
    R r = __builtin_bit_cast(R, x);
    asm volatile("" : "+v"(r));
    x = __builtin_bit_cast(T, r);
  }
  static __device__ __forceinline__ void settle(Inputs& in) {
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      touch(in.k[m]);
      touch(in.q[m]);
      touch(in.v[m]);
    }
    if constexpr (GATE) {
#pragma unroll
      for (int m = 0; m < NG; ++m) {
        touch(in.x[m]);
        touch(in.bias[m]);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NG; ++m) touch(in.g[m]);
    }
    using B = std::conditional_t<sizeof(TIO) == 2, unsigned short, unsigned>;
    B b = __builtin_bit_cast(B, in.beta);
    asm volatile("" : "+v"(b));
    in.beta = __builtin_bit_cast(TIO, b);
  }

  // The whole stage (every thread of the workgroup must call it).  `in` must
  // have been filled by prefetch() for this (chunk, head) and settled; run()
  // never waits on global memory otherwise.  mid() runs after the Gram
  // tile pairs, before the first output store (the caller settles the next
  // item's prefetch there).
  template <typename Mid>
  static __device__ void run(unsigned char* lds, const Inputs& in, float scale,
                             ChunkOut<TIO> out, QkIn qk, Mid&& mid) {
    float* Gs = reinterpret_cast<float*>(lds + Gm::OFF_GS);
    float* As = reinterpret_cast<float*>(lds + Gm::OFF_AS);
    float* Ts = reinterpret_cast<float*>(lds + Gm::OFF_TS);
    TIO* WT = reinterpret_cast<TIO*>(lds + Gm::OFF_WT);
    TIO* Lk = reinterpret_cast<TIO*>(lds + Gm::OFF_LK);
    TIO* Lq = reinterpret_cast<TIO*>(lds + Gm::OFF_LQ);
    TIO* Rn = reinterpret_cast<TIO*>(lds + Gm::OFF_RN);
    TIO* Vs = reinterpret_cast<TIO*>(lds + Gm::OFF_VS);
    TIO* KBt = reinterpret_cast<TIO*>(lds + Gm::OFF_KBT);
    TIO* VBt = reinterpret_cast<TIO*>(lds + Gm::OFF_VBT);
    TIO* Tb = reinterpret_cast<TIO*>(lds + Gm::OFF_TB);
    TIO* Aq = reinterpret_cast<TIO*>(lds + Gm::OFF_AQ);
    float* rho = reinterpret_cast<float*>(lds + Gm::OFF_RHO);  // [TT + 1][D]
    float* fac = reinterpret_cast<float*>(lds + Gm::OFF_FAC);  // [NFAC][D]
    float* s_beta = reinterpret_cast<float*>(lds + Gm::OFF_BETA);
    int* s_flag = reinterpret_cast<int*>(lds + Gm::OFF_FLAG);
    float* ex = reinterpret_cast<float*>(lds + Gm::OFF_EXACT);  // [TT][2][16][16]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const TIO zero_t = from_f32<TIO>(0.f);
    // (8 rows x 2 channels) groups of the elementwise passes: lanes run along
    // channel pairs, so every LDS access of a row is one conflict-free 2-value
    // word, and each channel's eight tokens leave as one 16-byte transposed
    // store.
    using V2 = typename Vec2<TIO>::type;
    constexpr int NGRP = (C / 8) * (D / 2) / NT > 0 ? (C / 8) * (D / 2) / NT : 1;

    // ---- phase 0: stage k, q, v, g (base 2) and beta; clear padding --------
    // rows at or past the chunk's length are staged as zeros (bit masks, so
    // the registers are never selected by address)
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int x = tid + NT * m;
      uint4 kv = in.k[m], qv = in.q[m];
      if (qk.norm) {  // the VPR lanes holding a row reduce its sum of squares
        normalise_row(kv);
        normalise_row(qv);
      }
      if (x < C * VPR) {
        const int r = x / VPR, cv = x % VPR;
        const unsigned mk = r < in.len ? ~0u : 0u;
        reinterpret_cast<uint4*>(Lk + r * KS_LD)[cv] = mask4(kv, mk);
        reinterpret_cast<uint4*>(Lq + r * KS_LD)[cv] = mask4(qv, mk);
        reinterpret_cast<uint4*>(Vs + r * KS_LD)[cv] = mask4(in.v[m], mk);
      }
    }
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const int x = tid + NT * m;
      if (x < C * GPR) {
        const int r = x / GPR, cv = x % GPR;
        const bool live = r < in.len;
        f32x4 gv;
        if constexpr (GATE) {
#pragma unroll
          for (int e = 0; e < 4; ++e) gv[e] = kimi_gate_log2(to_f32(in.x[m][e]) + in.bias[m][e], in.ea);
        } else {
          gv = in.g[m] * kLog2e;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) gv[e] = live ? gv[e] : 0.f;
        *reinterpret_cast<f32x4*>(Gs + Gm::gs_row(r) + 4 * cv) = gv;
      }
    }
    if (tid < C) s_beta[tid] = tid < in.len ? to_f32(in.beta) : 0.f;
    if (tid == 0) *s_flag = 0;
    {
      constexpr int NZ = C * TK_LD * (int)sizeof(TIO) / 16;  // uint4 per array
      for (int x = tid; x < NZ; x += NT) {
        reinterpret_cast<uint4*>(Tb)[x] = uint4{0, 0, 0, 0};
        reinterpret_cast<uint4*>(Aq)[x] = uint4{0, 0, 0, 0};
      }
      if constexpr (KCP != C) {
        constexpr int NZB = D * TK_LD * (int)sizeof(TIO) / 16;
        for (int x = tid; x < NZB; x += NT) {
          reinterpret_cast<uint4*>(KBt)[x] = uint4{0, 0, 0, 0};
          reinterpret_cast<uint4*>(VBt)[x] = uint4{0, 0, 0, 0};
        }
      }
    }
    __syncthreads();

    // ---- phase 1: cumulative sum over tokens; reference points; beta v ----
    {
      // LPC lanes of one wave share a channel, each scanning SEG tokens held
      // in registers; segment totals are combined with lane shuffles.
      constexpr int CPW = D / NW;    // channels per wave
      constexpr int LPC = 64 / CPW;  // lanes per channel
      constexpr int SEG = C / LPC;   // tokens per lane
      static_assert(CPW == Gm::GS_CPW && SEG == Gm::GS_SEG, "G row skew matches the scan");
      const int c = wave * CPW + lane % CPW;
      const int seg = lane / CPW;
      float gv[SEG];
#pragma unroll
      for (int j = 0; j < SEG; ++j) gv[j] = Gs[Gm::gs_row(seg * SEG + j) + c];
#pragma unroll
      for (int j = 1; j < SEG; ++j) gv[j] += gv[j - 1];
      float before = 0.f;  // sum of the earlier segments' totals
#pragma unroll
      for (int s2 = 0; s2 < LPC - 1; ++s2) {
        const float tot = __shfl(gv[SEG - 1], (lane % CPW) + s2 * CPW, 64);
        if (s2 < seg) before += tot;
      }
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int r = seg * SEG + j;
        const float G = gv[j] + before;
        Gs[Gm::gs_row(r) + c] = G;
        if ((r & 15) == 0) rho[(r >> 4) * D + c] = G;
        if (r == C - 1) rho[TT * D + c] = G;
      }
    }
#pragma unroll
    for (int m = 0; m < NGRP; ++m) {
      const int grp = tid + NT * m;
      const int c = 2 * (grp % (D / 2)), r0 = 8 * (grp / (D / 2));
      if (r0 < C) {
        FragT vb0, vb1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const V2 vv = *reinterpret_cast<const V2*>(Vs + (r0 + e) * KS_LD + c);
          vb0[e] = from_f32<TIO>(s_beta[r0 + e] * to_f32(vv[0]));
          vb1[e] = from_f32<TIO>(s_beta[r0 + e] * to_f32(vv[1]));
        }
        store_frag8(VBt + c * TK_LD + r0, vb0);
        store_frag8(VBt + (c + 1) * TK_LD + r0, vb1);
      }
    }
    __syncthreads();

    // ---- phase 2: per-channel factor vectors, exact diagonal tiles where a
    //      block's decay span is too large to factor, then the scaled
    //      operands Lk, Lq, Rn, beta k 2^G (transposed) -----------------------
    for (int c = tid; c < D; c += NT) {
      float rh[TT + 1];
#pragma unroll
      for (int a = 0; a <= TT; ++a) rh[a] = rho[a * D + c];
      int big = 0;
#pragma unroll
      for (int a = 0; a < TT; ++a) {
        fac[fac_sa(a) * D + c] = fast_exp2(rh[a]);
        fac[fac_diag(a) * D + c] = fast_exp2(rh[a] - rh[a + 1]);
        fac[fac_kg(a) * D + c] = fast_exp2(rh[TT] - rh[a + 1]);
        if (rh[a] - rh[a + 1] > kSpanMax) big |= 1 << a;
#pragma unroll
        for (int b = 0; b + 2 <= a; ++b) fac[fac_far(a, b) * D + c] = fast_exp2(rh[a] - rh[b + 1]);
      }
      if (big) atomicOr(s_flag, big);
    }
    __syncthreads();
    const int flag = *s_flag;  // blocks whose diagonal tile is summed exactly
    if (flag) {
      // entry (a, r, i), i <= r < 16 of block a: sum over channels of
      // k[r] k[i] 2^(G[r] - G[i]) and q[r] k[i] 2^(G[r] - G[i]) from the staged
      // rows (rows past the chunk are zeros); two lanes per entry, half the
      // channels each
      for (int e = tid; e < TT * 512; e += NT) {
        const int half = e & 1, ent = e >> 1;
        const int a = ent >> 8, r = (ent >> 4) & 15, i = ent & 15;
        float sk = 0.f, sq = 0.f;
        if (((flag >> a) & 1) && i <= r) {
          const int rr = 16 * a + r, ii = 16 * a + i;
          for (int c = half * (D / 2); c < (half + 1) * (D / 2); ++c) {
            const float f = fast_exp2(Gs[Gm::gs_row(rr) + c] - Gs[Gm::gs_row(ii) + c]);
            const float ki = to_f32(Lk[ii * KS_LD + c]) * f;
            sk += to_f32(Lk[rr * KS_LD + c]) * ki;
            sq += to_f32(Lq[rr * KS_LD + c]) * ki;
          }
        }
        sk += __shfl_xor(sk, 1, 64);
        sq += __shfl_xor(sq, 1, 64);
        if (half == 0) {
          ex[((a * 2 + 0) * 16 + r) * 16 + i] = sk;
          ex[((a * 2 + 1) * 16 + r) * 16 + i] = sq;
        }
      }
      __syncthreads();  // the staged k and q are replaced next
    }
#pragma unroll
    for (int m = 0; m < NGRP; ++m) {
      const int grp = tid + NT * m;
      const int c = 2 * (grp % (D / 2)), r0 = 8 * (grp / (D / 2));
      if (r0 < C) {
        const int a = r0 >> 4;
        const f32x2 ra = *reinterpret_cast<const f32x2*>(rho + a * D + c);
        const f32x2 rb = *reinterpret_cast<const f32x2*>(rho + (a + 1) * D + c);
        const float sa[2] = {fast_exp2(ra[0]), fast_exp2(ra[1])};
        FragT kb[2];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int r = r0 + e;
          const f32x2 G = *reinterpret_cast<const f32x2*>(Gs + Gm::gs_row(r) + c);
          const V2 kv = *reinterpret_cast<const V2*>(Lk + r * KS_LD + c);
          const V2 qv = *reinterpret_cast<const V2*>(Lq + r * KS_LD + c);
          V2 lk2, lq2, rn2;
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const float el = fast_exp2(G[i] - ra[i]);
            const float er = fast_exp2(rb[i] - G[i]);
            const float lk = to_f32(kv[i]) * el;
            lk2[i] = from_f32<TIO>(lk);
            lq2[i] = from_f32<TIO>(to_f32(qv[i]) * el);
            rn2[i] = from_f32<TIO>(to_f32(kv[i]) * er);
            kb[i][e] = from_f32<TIO>(s_beta[r] * lk * sa[i]);
          }
          *reinterpret_cast<V2*>(Lk + r * KS_LD + c) = lk2;
          *reinterpret_cast<V2*>(Lq + r * KS_LD + c) = lq2;
          *reinterpret_cast<V2*>(Rn + r * KS_LD + c) = rn2;
        }
        store_frag8(KBt + c * TK_LD + r0, kb[0]);
        store_frag8(KBt + (c + 1) * TK_LD + r0, kb[1]);
      }
    }
    __syncthreads();

    // ---- phase 3: decayed Gram tiles; Kg fragments; Gam -------------------
    // The waves with one Gram tile pair fewer than the rest write Kg and Gam
    // to the outputs meanwhile (they read only Rn and the factors).
    {
      constexpr int NPAIR = TT * (TT + 1) / 2;
      constexpr int KGW = (NPAIR % NW == 0) ? 0 : NPAIR % NW;  // first Kg wave
      for (int p = wave; p < NPAIR; p += NW) {
        int a = 0, b = p;
        while (b > a) {
          b -= a + 1;
          ++a;
        }
        f32x4 akk = zero4(), aqk = zero4();
        if (a == b && (flag >> a) & 1) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            akk[j] = ex[((a * 2 + 0) * 16 + 4 * lg + j) * 16 + l16];
            aqk[j] = ex[((a * 2 + 1) * 16 + 4 * lg + j) * 16 + l16];
          }
        } else {
          const TIO* lkr = Lk + (16 * a + l16) * KS_LD;
          const TIO* lqr = Lq + (16 * a + l16) * KS_LD;
          const TIO* rnr = Rn + (16 * b + l16) * KS_LD;
          // adjacent blocks need no factor; the rest one per channel
          const float* fv = nullptr;
          if (a == b) fv = fac + fac_diag(a) * D;
          else if (b + 2 <= a) fv = fac + fac_far(a, b) * D;
#pragma unroll
          for (int s = 0; s < KBD; ++s) {
            const int c0 = 32 * s + 8 * lg;
            const FragT fk = load_frag8<TIO>(lkr + c0);
            const FragT fq = load_frag8<TIO>(lqr + c0);
            FragT fr = load_frag8<TIO>(rnr + c0);
            if (fv) fr = scale8(fr, fv + c0);
            akk = mma32(fk, fr, akk);
            aqk = mma32(fq, fr, aqk);
          }
        }
        // rows 16a + 4lg + j, column 16b + l16
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * a + 4 * lg + j;
          const int ii = 16 * b + l16;
          As[rr * AF_LD + ii] = (ii < rr) ? s_beta[rr] * akk[j] : 0.f;
          Aq[rr * TK_LD + ii] = from_f32<TIO>((ii <= rr) ? aqk[j] : 0.f);
        }
      }
      mid();  // before this item's first store
      if (wave >= KGW) {
        constexpr int NTK = NT - 64 * KGW;  // threads writing Kg
        const int tk = tid - 64 * KGW;
        // Kg^T fragments in kperm token order: element (kt, ts, lane, e) =
        // Kg[32ts + kperm(lg, e)][16kt + l16], Kg = Rn * 2^(rho_TT - rho_{blk+1}).
        for (int slot = tk; slot < DT * KBC * 64; slot += NTK) {
          const int ln = slot & 63;
          const int kt = (slot >> 6) / KBC, ts = (slot >> 6) % KBC;
          const int c = 16 * kt + (ln & 15);
          const int g4 = ln >> 4;
          FragT f;
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int blk = 2 * ts + hh;  // 16-token block of these four tokens
            const float fk = (blk < TT) ? fac[fac_kg(blk < TT ? blk : 0) * D + c] : 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int tok = 16 * blk + 4 * g4 + e;
              f[4 * hh + e] = from_f32<TIO>((blk < TT) ? to_f32(Rn[tok * KS_LD + c]) * fk : 0.f);
            }
          }
          store_frag8(out.k + (size_t)slot * 8, f);
        }
        for (int c = tk; c < D; c += NTK) out.gam[c] = fast_exp2(rho[TT * D + c]);
      }
    }
    __syncthreads();
    if (Gm::EXACT_IN_T && flag) {  // T held the exact tiles: its upper blocks must read 0
      constexpr int NZ = C * TK_LD * (int)sizeof(TIO) / 16;
      for (int x = tid; x < NZ; x += NT) reinterpret_cast<uint4*>(Tb)[x] = uint4{0, 0, 0, 0};
      __syncthreads();
    }

    // ---- phase 4: T = (I + A)^-1 ------------------------------------------
    // Diagonal 16x16 blocks by forward substitution, lane 16a + r holding row
    // r of block a: the multiple A[r][i] of row i of the inverse, reaching the
    // lanes below it by a row broadcast, is subtracted for i = 0 .. 14 in
    // turn.  Columns of the inverse do not interact, so waves 0..3 each take
    // the columns j = wave (mod 4); a row i < j still holds 0 in column j, so
    // the steps before j are skipped.  Then the off-diagonal blocks one band
    // at a time, one wave per block:  T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb
    // (fp32 MFMA).
    auto diag_cols = [&](auto kc) {
      constexpr int K = decltype(kc)::value;
      const int a = lg < TT ? lg : TT - 1;  // rows past the blocks: a copy, unused
      const int r = l16;
      float Ar[16], X[4];
      const float* arow = As + (16 * a + r) * AF_LD + 16 * a;
#pragma unroll
      for (int j4 = 0; j4 < 4; ++j4) {
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(arow + 4 * j4);
#pragma unroll
        for (int e = 0; e < 4; ++e) Ar[4 * j4 + e] = x4[e];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) X[q] = (K + 4 * q == r) ? 1.f : 0.f;
      // A is strictly lower triangular: rows r <= i see a zero multiplier
#pragma unroll
      for (int i = 0; i < 15; ++i) {
        const float m = -Ar[i];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (K + 4 * q <= i) X[q] = fmaf(m, row_bcast(X[q], i), X[q]);
      }
      if (lg < TT) {
        float* trow = Ts + (16 * a + r) * AF_LD + 16 * a;
        TIO* brow = Tb + (16 * a + r) * TK_LD + 16 * a;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          trow[K + 4 * q] = X[q];
          brow[K + 4 * q] = from_f32<TIO>(X[q]);
        }
      }
    };
    switch (wave) {
      case 0: diag_cols(std::integral_constant<int, 0>{}); break;
      case 1: diag_cols(std::integral_constant<int, 1>{}); break;
      case 2: diag_cols(std::integral_constant<int, 2>{}); break;
      case 3: diag_cols(std::integral_constant<int, 3>{}); break;
      default: break;
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d < TT; ++d) {
      const int a = d + wave;
      if (a < TT) {
        const int b = a - d;
        f32x4 pacc = zero4();
        for (int cc = b; cc < a; ++cc) {
          float fa[4], fb[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            fa[m] = As[(16 * a + l16) * AF_LD + 16 * cc + 4 * m + lg];
            fb[m] = Ts[(16 * cc + 4 * m + lg) * AF_LD + 16 * b + l16];
          }
          pacc = mma16_f32(fa, fb, pacc);
        }
        float ta[4], pb[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          ta[m] = Ts[(16 * a + l16) * AF_LD + 16 * a + 4 * lg + m];
          pb[m] = pacc[m];
        }
        const f32x4 tab = mma16_f32(ta, pb, zero4());
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int rr = 16 * a + 4 * lg + m;
          Ts[rr * AF_LD + 16 * b + l16] = -tab[m];
          Tb[rr * TK_LD + 16 * b + l16] = from_f32<TIO>(-tab[m]);
        }
      }
      __syncthreads();
    }

    // ---- phase 5: W^T, U, Q'^T, Ol -> outputs -------------------------------
    // Wave w owns channel tiles ct = w, w + NW, ... of W^T and Q'^T and the
    // same value-column tiles of U and Ol.
#pragma unroll
    for (int ct = wave; ct < DT; ct += NW) {
      const int kb = ct >> 1, hh = ct & 1;
      f32x4 ureg[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        f32x4 wacc = zero4(), uacc = zero4();
#pragma unroll
        for (int s = 0; s <= t / 2; ++s) {
          const FragT fk = load_frag8<TIO>(KBt + (16 * ct + l16) * TK_LD + 32 * s + 8 * lg);
          const FragT ft = load_frag8<TIO>(Tb + (16 * t + l16) * TK_LD + 32 * s + 8 * lg);
          const FragT fv = load_frag8<TIO>(VBt + (16 * ct + l16) * TK_LD + 32 * s + 8 * lg);
          wacc = mma32(fk, ft, wacc);  // W^T[16ct + 4lg + j][16t + l16]
          uacc = mma32(ft, fv, uacc);  // U[16t + 4lg + j][16ct + l16]
        }
        ureg[t] = uacc;
        TIO* wout = out.w + ((size_t)(t * KBD + kb) * 64 + lane) * 8 + 4 * hh;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const TIO wv = from_f32<TIO>(wacc[j]);
          wout[j] = wv;
          WT[(16 * ct + 4 * lg + j) * TK_LD + 16 * t + l16] = wv;
        }
        store_tile(out.u, t, ct, lane, uacc, ureg[t > 0 ? t - 1 : 0], 1.f);
      }
      if constexpr (KCP != C) {
        for (int x = lane; x < 16 * (KCP - C); x += 64)
          WT[(16 * ct + x / (KCP - C)) * TK_LD + C + x % (KCP - C)] = zero_t;
      }
      wave_sync();  // this wave's W^T rows are complete
      f32x4 oprev = zero4();  // Ol of the even token tile of a pair
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s <= t / 2; ++s) {
          const FragT fw = load_frag8<TIO>(WT + (16 * ct + l16) * TK_LD + 32 * s + 8 * lg);
          const FragT fa = load_frag8<TIO>(Aq + (16 * t + l16) * TK_LD + 32 * s + 8 * lg);
          acc = mma32(fw, fa, acc);  // (Aqk W)^T[16ct + 4lg + j][16t + l16]
        }
        const int r = 16 * t + l16;
        const int a = r >> 4;
        TIO* qout = out.q + ((size_t)(t * KBD + kb) * 64 + lane) * 8 + 4 * hh;
        const f32x4 qr = *reinterpret_cast<const f32x4*>(fac + fac_sa(a) * D + 16 * ct + 4 * lg);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = 16 * ct + 4 * lg + j;
          const float qg = to_f32(Lq[r * KS_LD + c]) * qr[j];
          qout[j] = from_f32<TIO>(scale * (qg - acc[j]));
        }
        f32x4 oacc = zero4();
#pragma unroll
        for (int s = 0; s <= t / 2; ++s) {
          const FragT fa = load_frag_perm<TIO>(Aq + (16 * t + l16) * TK_LD + 32 * s, lg);
          f32x4 u1 = zero4();
          if (2 * s + 1 < TT) u1 = ureg[2 * s + 1 < TT ? 2 * s + 1 : TT - 1];
          if constexpr (HEADL) oacc = mma32(frag_from_d<TIO>(ureg[2 * s], u1), fa, oacc);
          else oacc = mma32(fa, frag_from_d<TIO>(ureg[2 * s], u1), oacc);
        }
        store_tile(out.o, t, ct, lane, oacc, oprev, scale);
        oprev = oacc;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// One step of the state scan for NJ tiles of 16 value columns (block jb =
// columns 16 NJ jb .. 16 NJ jb + 16 NJ - 1) by the workgroup's KBD waves.
// Wave w owns
//   - dk slice w of the state: rows 32w .. 32w + 31 of every column tile
//     (accumulator tiles S[c][m], rows 32w + 16m + 4lg + j, column
//     16 (NJ jb + c) + l16), which it updates with Kg^T V;
//   - token tiles t = w + KBD i of the chunk, for which it computes the whole
//     products W S and Q' S over all of dk, so no partial sums cross waves.
// The waves exchange only the state slices (as bf16 B fragments, 1 KB per
// slice and column tile) and V (16 tokens x 16 columns per tile).  The NJ
// column tiles share one load of the chunk's W, Q' and Kg, so a wider block
// reads those operators fewer times in total.
template <typename TIO, int D, int C, int NJ = 1>
struct ScanStep {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  static constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KBC = Gm::KBC;
  static constexpr int VT_LD = Gm::VT_LD;
  static constexpr int NOWN = (TT + KBD - 1) / KBD;  // token tiles a wave owns
  static_assert(DT % NJ == 0, "column tiles per block must divide the head dim");
  static constexpr int NB = DT / NJ;                  // column blocks per head
  // LDS: state slices [NJ][KBD][64] fragments, V^T [NJ][16][VT_LD],
  // o staging [C][OS_LD]
  static constexpr size_t SX_BYTES = (size_t)NJ * KBD * 64 * sizeof(FragT);
  static constexpr size_t OFF_VT = SX_BYTES;
  static constexpr int OS_LD = 16 * NJ + Gm::TP;
  static constexpr size_t OFF_OS = align_up(OFF_VT + (size_t)NJ * 16 * VT_LD * sizeof(TIO), 16);
  static constexpr size_t LDS_BYTES = OFF_OS + (size_t)C * OS_LD * sizeof(TIO);

  // Everything one step reads from a chunk's outputs, for this lane.
  struct Ops {
    FragT w[NOWN][KBD], q[NOWN][KBD], k[2][KBC];
    TIO u[NJ][NOWN][4], ol[NJ][NOWN][4];
    // Gam of row 32w + lane % 32 of the wave's dk slice: one 4-byte load per
    // lane; the step gathers each lane's eight rows with lane shuffles.  (Two
    // 16-byte loads per lane would carry the same 128 bytes through the CU's
    // address unit as 2 KB, and that unit is what the scan waits on.)
    float gl;
    int start, len;  // the chunk's token range (set by the caller)
  };

  static __device__ __forceinline__ int own_tile(int w, int i) {
    const int t = w + KBD * i;
    return t < TT ? t : TT - 1;  // tiles past the chunk are loaded, then unused
  }

  // Loads of one chunk's operators, in three groups that a step consumes in
  // turn (W and Q', then U and Ol, then Kg and Gam), so a step can refill each
  // group as soon as it is done with it.
  static __device__ __forceinline__ void load_wq(Ops& op, const ChunkOut<TIO>& in) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NOWN; ++i)
#pragma unroll
      for (int s = 0; s < KBD; ++s) {
        const size_t f = ((size_t)(own_tile(w, i) * KBD + s) * 64 + lane) * 8;
        op.w[i][s] = load_frag8<TIO>(in.w + f);
        op.q[i][s] = load_frag8<TIO>(in.q + f);
      }
  }
  static __device__ __forceinline__ void load_uo(Ops& op, const ChunkOut<TIO>& in, int jb) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int c = 0; c < NJ; ++c)
#pragma unroll
      for (int i = 0; i < NOWN; ++i) {
        const int t = own_tile(w, i);
        const int ct = NJ * jb + c;
        const TIO* Uc = in.u + ((size_t)(t * DT + ct) * 64 + lane) * 4;
        const TIO* Oc = in.o + ((size_t)(t * DT + ct) * 64 + lane) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          op.u[c][i][j] = Uc[j];
          op.ol[c][i][j] = Oc[j];
        }
      }
  }
  static __device__ __forceinline__ void load_kg(Ops& op, const ChunkOut<TIO>& in) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kc = 0; kc < KBC; ++kc)
        op.k[m][kc] = load_frag8<TIO>(in.k + ((size_t)((2 * w + m) * KBC + kc) * 64 + lane) * 8);
    op.gl = in.gam[32 * w + (lane & 31)];
  }
  static __device__ __forceinline__ void load(Ops& op, const ChunkOut<TIO>& in, int jb) {
    load_wq(op, in);
    load_uo(op, in, jb);
    load_kg(op, in);
  }

  // Publish this wave's state slices as B fragments for the next step (every
  // wave of the workgroup calls it; a barrier must follow before they are read).
  static __device__ __forceinline__ void publish(unsigned char* lds, const f32x4 (&S)[NJ][2]) {
    FragT* Sx = reinterpret_cast<FragT*>(lds);
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int c = 0; c < NJ; ++c) Sx[(c * KBD + w) * 64 + lane] = frag_from_d<TIO>(S[c][0], S[c][1]);
  }

  // The chunk's rows of o from the staging buffer to HBM, by NTS threads
  // (index tid): rows >= len fall outside the buffer resource; 16-byte
  // pieces, EPV values of one row each.  Runs between the two barriers of the
  // step that staged them.
  template <int NTS>
  static __device__ __forceinline__ void store_o(unsigned char* lds, TIO* __restrict__ o,
                                                 int64_t ostride, int h, int jb, int start,
                                                 int len, int tid) {
    const TIO* Os = reinterpret_cast<const TIO*>(lds + OFF_OS);
    constexpr int EPV = 16 / (int)sizeof(TIO), VPRO = 16 * NJ / EPV, NVEC = C * VPRO;
    const __amdgpu_buffer_rsrc_t orsrc =
        make_rsrc(o + (int64_t)start * ostride, len * (int)ostride * (int)sizeof(TIO));
#pragma unroll
    for (int p = 0; p < (NVEC + NTS - 1) / NTS; ++p) {
      const int x0 = tid + NTS * p;
      const int x = x0 < NVEC ? x0 : NVEC - 1;
      const int r = x / VPRO, cv = x % VPRO;
      const uint4 val = *reinterpret_cast<const uint4*>(Os + r * OS_LD + cv * EPV);
      const int off = (x0 < NVEC && r < len)
                          ? (r * (int)ostride + h * D + 16 * NJ * jb + cv * EPV) * (int)sizeof(TIO)
                          : kBufferOff;
      buffer_store16(val, orsrc, off);
    }
  }

  // One chunk: V = U - W S, O = Ol + Q' S (rows < len written to o), then
  // S = diag(Gam) S + Kg^T V, for each of the NJ column tiles.  Expects the
  // state slices published (publish(), then a barrier) and leaves them
  // published for the next step.  Two workgroup barriers.  The workgroup has
  // one wave per dk slice, so the step has no divergent branch and the
  // compiler can count outstanding loads exactly.  NTH: threads of the
  // workgroup.  With `nxt` set, each group of
  // `op` is reloaded from *nxt as soon as the step has consumed it (the loads
  // then overlap the rest of the step); nxt_ent supplies the new token range.
  // live = false (uniform) runs the step without effect: no o rows are
  // written and S keeps its value; the refills still happen.  STORE_O: the
  // step's own waves write o (else another wave of the workgroup calls
  // store_o between the step's barriers).
  template <int NTH, bool STORE_O = true>
  static __device__ __forceinline__ void step(unsigned char* lds, f32x4 (&S)[NJ][2], Ops& op,
                                              TIO* __restrict__ o, int64_t ostride, int h,
                                              int jb, const ChunkOut<TIO>* nxt = nullptr,
                                              const ChunkEnt* nxt_ent = nullptr,
                                              bool live = true) {
    // No instruction crosses a step boundary: the scheduler would otherwise
    // hoist the next steps' conversions of their U and Ol values (loaded one
    // and two steps ago) into this step, whose waits for them then hold up
    // this step's chain.
    __builtin_amdgcn_sched_barrier(0);
    const int start = __builtin_amdgcn_readfirstlane(op.start);
    const int len = live ? __builtin_amdgcn_readfirstlane(op.len) : 0;
    const FragT* Sx = reinterpret_cast<const FragT*>(lds);  // [NJ][KBD][64]
    TIO* Vt = reinterpret_cast<TIO*>(lds + OFF_VT);        // [NJ][16][VT_LD]
    TIO* Os = reinterpret_cast<TIO*>(lds + OFF_OS);        // [C][OS_LD]
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    // Gam of the rows this lane's accumulators hold (32w + 16m + 4lg + j),
    // gathered here, well before the update uses them
    f32x4 gm[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) gm[m][j] = __shfl(op.gl, 16 * m + 4 * lg + j, 64);

    {
#pragma unroll
      for (int c = 0; c < NJ; ++c) {
        FragT sb[KBD];
#pragma unroll
        for (int s2 = 0; s2 < KBD; ++s2) sb[s2] = Sx[(c * KBD + s2) * 64 + lane];
#pragma unroll
        for (int i = 0; i < NOWN; ++i) {
          const int t = w + KBD * i;
          if (TT % KBD == 0 || t < TT) {
            f32x4 pv = zero4(), po = zero4();
#pragma unroll
            for (int s2 = 0; s2 < KBD; ++s2) {
              pv = mma32(op.w[i][s2], sb[s2], pv);
              po = mma32(op.q[i][s2], sb[s2], po);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int r = 16 * t + 4 * lg + j;
              Vt[(c * 16 + l16) * VT_LD + r] = from_f32<TIO>(to_f32(op.u[c][i][j]) - pv[j]);
              Os[r * OS_LD + 16 * c + l16] = from_f32<TIO>(to_f32(op.ol[c][i][j]) + po[j]);
            }
          }
        }
      }
    }
    if (nxt) {
      load_wq(op, *nxt);
      load_uo(op, *nxt, jb);
    }
    __syncthreads();
    if constexpr (STORE_O) store_o<NTH>(lds, o, ostride, h, jb, start, len, (int)threadIdx.x);
    {
#pragma unroll
      for (int c = 0; c < NJ; ++c)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          f32x4 sn = S[c][m] * gm[m];
#pragma unroll
          for (int kc = 0; kc < KBC; ++kc) {
            // Kg fragments are in kperm token order; read V the same way
            const FragT fv = load_frag_perm<TIO>(Vt + (c * 16 + l16) * VT_LD + 32 * kc, lg);
            sn = mma32(op.k[m][kc], fv, sn);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) S[c][m][j] = live ? sn[j] : S[c][m][j];
        }
    }
    publish(lds, S);
    if (nxt) {
      load_kg(op, *nxt);
      op.start = nxt_ent->start;
      op.len = nxt_ent->len;
    }
    __syncthreads();
  }

  // Token slots past the chunk's tiles (C < 32) must read as zero.
  static __device__ __forceinline__ void clear_vt(unsigned char* lds) {
    TIO* Vt = reinterpret_cast<TIO*>(lds + OFF_VT);
    for (int x = threadIdx.x; x < NJ * 16 * VT_LD; x += blockDim.x) Vt[x] = from_f32<TIO>(0.f);
  }
};

}  // namespace kda
