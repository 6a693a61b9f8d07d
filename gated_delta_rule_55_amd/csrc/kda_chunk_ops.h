// kda_chunk_ops.h -- device building blocks of the chunked KDA prefill:
//   ChunkLocal  the chunk-local stage for one (chunk, head) by one 256-thread
//               workgroup: cumulative decay, decayed Gram matrices, triangular
//               solve, W/U and the chunk's output operators
//   ScanStep    one step of the inter-chunk state recurrence with the output
//               fused in, split over the workgroup's four waves by dk slice
// Both are used by the standalone kernels and by the fused kernel.
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
// only one above 1; when it exceeds 2^64 for some channel the tile is summed
// entry by entry from the inputs instead.  W, Kg and Q * 2^G reuse Lk, Rn and
// Lq with one more per-channel factor, so each element costs two exp2.
#pragma once

#include "kda_device.h"

namespace kda {

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t cmaxz(size_t a, size_t b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr float kLog2e = 1.4426950408889634f;
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
  static constexpr size_t SZ_A = cmaxz(cmaxz((size_t)C * GS_LD * 4, (size_t)2 * C * AF_LD * 4),
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
  static constexpr size_t OFF_RHO = align_up(OFF_AQ + (size_t)C * TK_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_BETA = OFF_RHO + (size_t)(TT + 1) * D * 4;
  static constexpr size_t OFF_FLAG = OFF_BETA + (size_t)C * 4;
  static constexpr size_t LOCAL_LDS = align_up(OFF_FLAG + 16, 16);

  // Scan-step LDS (aliases the chunk-local region; the two never overlap).
  static constexpr int VT_LD = KCP + TP;
  static constexpr size_t SCAN_RED = (size_t)KBD * TT * 64 * 16;  // one of v / o partials
  static constexpr size_t SCAN_LDS = 2 * SCAN_RED + (size_t)16 * VT_LD * sizeof(TIO);
  static constexpr size_t FUSED_LDS = cmaxz(LOCAL_LDS, SCAN_LDS);

  static constexpr bool FITS = FUSED_LDS <= 160 * 1024;
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

// ---------------------------------------------------------------------------
// Chunk-local stage.
template <typename TIO, int D, int C>
struct ChunkLocal {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  static constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KCP = Gm::KCP, KBC = Gm::KBC;
  static constexpr int GS_LD = Gm::GS_LD, KS_LD = Gm::KS_LD, TK_LD = Gm::TK_LD,
                       AF_LD = Gm::AF_LD;
  static constexpr int EPV = 16 / sizeof(TIO);      // elements per 16-byte vector
  static constexpr int VPR = D / EPV;               // vectors per row of q, k, v
  static constexpr int NV = (C * VPR + 255) / 256;  // vectors per thread per tensor
  static constexpr int GPR = D / 4;                 // float4 per row of g
  static constexpr int NG = (C * GPR + 255) / 256;  // float4 per thread of g

  // The chunk's inputs as this thread loads them (rows beyond L are zero).
  struct Inputs {
    uint4 k[NV], q[NV], v[NV];
    f32x4 g[NG];
    float beta;
    int64_t tok0;
    int len;
  };

  // Issue every global load of one (chunk, head); nothing waits on them here.
  static __device__ __forceinline__ void prefetch(Inputs& in, const TIO* __restrict__ q,
                                                  const TIO* __restrict__ k,
                                                  const TIO* __restrict__ v,
                                                  const float* __restrict__ g,
                                                  const TIO* __restrict__ beta, int n_heads,
                                                  int h, int64_t tok0, int L) {
    const int tid = threadIdx.x;
    const int64_t rs = (int64_t)n_heads * D;
    in.tok0 = tok0;
    in.len = L;
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int x = tid + 256 * m;
      const int r = x / VPR, cv = x % VPR;
      in.k[m] = in.q[m] = in.v[m] = uint4{0, 0, 0, 0};
      if (x < C * VPR && r < L) {
        const int64_t off = (tok0 + r) * rs + (int64_t)h * D;
        in.k[m] = reinterpret_cast<const uint4*>(k + off)[cv];
        in.q[m] = reinterpret_cast<const uint4*>(q + off)[cv];
        in.v[m] = reinterpret_cast<const uint4*>(v + off)[cv];
      }
    }
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const int x = tid + 256 * m;
      const int r = x / GPR, cv = x % GPR;
      in.g[m] = zero4();
      if (x < C * GPR && r < L)
        in.g[m] = reinterpret_cast<const f32x4*>(g + (tok0 + r) * rs + (int64_t)h * D)[cv];
    }
    in.beta = 0.f;
    if (tid < C && tid < L) in.beta = to_f32(beta[(tok0 + tid) * n_heads + h]);
  }

  // Entry-by-entry Gram tile from the inputs in global memory, for a diagonal
  // tile whose decay span is too large to factor.  Lane holds rows
  // 16a + 4lg + j, column 16a + l16 (accumulator layout).
  static __device__ void exact_diag_tile(int a, f32x4& akk, f32x4& aqk,
                                         const TIO* __restrict__ q, const TIO* __restrict__ k,
                                         const float* __restrict__ g, int n_heads, int h,
                                         int64_t tok0, int L) {
    const int lane = threadIdx.x & 63;
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t rs = (int64_t)n_heads * D;
    const int ii = 16 * a + l16;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 16 * a + 4 * lg + j;
      float sk = 0.f, sq = 0.f;
      if (ii <= rr && rr < L) {
        for (int c = 0; c < D; ++c) {
          float e = 0.f;  // G[rr] - G[ii] = sum of g over (ii, rr]
          for (int t = ii + 1; t <= rr; ++t) e += g[(tok0 + t) * rs + (int64_t)h * D + c];
          const float f = fast_exp2(e * kLog2e);
          const float ki = to_f32(k[(tok0 + ii) * rs + (int64_t)h * D + c]) * f;
          sk += to_f32(k[(tok0 + rr) * rs + (int64_t)h * D + c]) * ki;
          sq += to_f32(q[(tok0 + rr) * rs + (int64_t)h * D + c]) * ki;
        }
      }
      akk[j] = sk;
      aqk[j] = sq;
    }
  }

  // The whole stage.  Six workgroup barriers; all 256 threads must call it.
  // `in` must have been filled by prefetch() for this (chunk, head).
  static __device__ void run(unsigned char* lds, const Inputs& in, float scale,
                             ChunkOut<TIO> out, const TIO* __restrict__ q,
                             const TIO* __restrict__ k, const float* __restrict__ g, int n_heads,
                             int h) {
    float* Gs = reinterpret_cast<float*>(lds + Gm::OFF_GS);
    float* As = reinterpret_cast<float*>(lds + Gm::OFF_AS);
    float* Ts = reinterpret_cast<float*>(lds + Gm::OFF_TS);
    TIO* WT = reinterpret_cast<TIO*>(lds + Gm::OFF_WT);
    TIO* Lk = reinterpret_cast<TIO*>(lds + Gm::OFF_LK);
    TIO* Lq = reinterpret_cast<TIO*>(lds + Gm::OFF_LQ);
    TIO* Rn = reinterpret_cast<TIO*>(lds + Gm::OFF_RN);
    TIO* KBt = reinterpret_cast<TIO*>(lds + Gm::OFF_KBT);
    TIO* VBt = reinterpret_cast<TIO*>(lds + Gm::OFF_VBT);
    TIO* Tb = reinterpret_cast<TIO*>(lds + Gm::OFF_TB);
    TIO* Aq = reinterpret_cast<TIO*>(lds + Gm::OFF_AQ);
    float* rho = reinterpret_cast<float*>(lds + Gm::OFF_RHO);  // [TT + 1][D]
    float* s_beta = reinterpret_cast<float*>(lds + Gm::OFF_BETA);
    int* s_flag = reinterpret_cast<int*>(lds + Gm::OFF_FLAG);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l16 = lane & 15;
    const int lg = lane >> 4;
    const TIO zero_t = from_f32<TIO>(0.f);

    // ---- phase 0: stage k, q, g (base 2) and beta; clear padded operands ----
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int x = tid + 256 * m;
      if (x < C * VPR) {
        const int r = x / VPR, cv = x % VPR;
        reinterpret_cast<uint4*>(Lk + r * KS_LD)[cv] = in.k[m];
        reinterpret_cast<uint4*>(Lq + r * KS_LD)[cv] = in.q[m];
      }
    }
#pragma unroll
    for (int m = 0; m < NG; ++m) {
      const int x = tid + 256 * m;
      if (x < C * GPR) {
        const int r = x / GPR, cv = x % GPR;
        *reinterpret_cast<f32x4*>(Gs + r * GS_LD + 4 * cv) = in.g[m] * kLog2e;
      }
    }
    if (tid < C) s_beta[tid] = in.beta;
    if (tid == 0) *s_flag = 0;
    for (int x = tid; x < C * TK_LD; x += 256) {
      Tb[x] = zero_t;
      Aq[x] = zero_t;
    }
    if constexpr (KCP != C)
      for (int x = tid; x < D * TK_LD; x += 256) {
        KBt[x] = zero_t;
        VBt[x] = zero_t;
      }
    __syncthreads();

    // ---- phase 1: cumulative sum over tokens; beta v transposed ----------
    {
      // LPC lanes of one wave share a channel, each scanning C / LPC tokens;
      // the segment totals are combined with lane shuffles.
      constexpr int CPW = D / 4;         // channels per wave
      constexpr int LPC = 64 / CPW;      // lanes per channel
      constexpr int SEG = C / LPC;       // tokens per lane
      const int c = wave * CPW + lane % CPW;
      const int seg = lane / CPW;
      float run = 0.f;
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        float* p = Gs + (seg * SEG + j) * GS_LD + c;
        run += *p;
        *p = run;
      }
      float before = 0.f;  // sum of the earlier segments' totals
#pragma unroll
      for (int s2 = 0; s2 < LPC - 1; ++s2) {
        const float tot = __shfl(run, (lane % CPW) + s2 * CPW, 64);
        if (s2 < seg) before += tot;
      }
      if (seg > 0) {
#pragma unroll
        for (int j = 0; j < SEG; ++j) Gs[(seg * SEG + j) * GS_LD + c] += before;
      }
    }
#pragma unroll
    for (int m = 0; m < NV; ++m) {
      const int x = tid + 256 * m;
      if (x < C * VPR) {
        const int r = x / VPR, cv = x % VPR;
        const float b = s_beta[r];
        const TIO* ve = reinterpret_cast<const TIO*>(&in.v[m]);
#pragma unroll
        for (int e = 0; e < EPV; ++e)
          VBt[(cv * EPV + e) * TK_LD + r] = from_f32<TIO>(b * to_f32(ve[e]));
      }
    }
    __syncthreads();

    // ---- phase 2: reference points, scaled operands ----------------------
    {
      constexpr int RPS = 256 / D;  // row stride of one thread
      const int c = tid % D;
      const int r0 = tid / D;
      float rh[TT + 1], sa[TT];
#pragma unroll
      for (int a = 0; a < TT; ++a) rh[a] = Gs[(16 * a) * GS_LD + c];
      rh[TT] = Gs[(C - 1) * GS_LD + c];
#pragma unroll
      for (int a = 0; a < TT; ++a) sa[a] = fast_exp2(rh[a]);
      if (r0 == 0) {
#pragma unroll
        for (int a = 0; a <= TT; ++a) rho[a * D + c] = rh[a];
        int big = 0;
#pragma unroll
        for (int a = 0; a < TT; ++a)
          if (rh[a] - rh[a + 1] > kSpanMax) big |= 1 << a;
        if (big) atomicOr(s_flag, big);
      }
#pragma unroll 4
      for (int r = r0; r < C; r += RPS) {
        const int a = r >> 4;
        const float gr = Gs[r * GS_LD + c];
        const float el = fast_exp2(gr - rh[a]);
        const float er = fast_exp2(rh[a + 1] - gr);
        const float kv = to_f32(Lk[r * KS_LD + c]);
        const float qv = to_f32(Lq[r * KS_LD + c]);
        const float lk = kv * el;
        Lk[r * KS_LD + c] = from_f32<TIO>(lk);
        Lq[r * KS_LD + c] = from_f32<TIO>(qv * el);
        Rn[r * KS_LD + c] = from_f32<TIO>(kv * er);
        KBt[c * TK_LD + r] = from_f32<TIO>(s_beta[r] * lk * sa[a]);
      }
    }
    __syncthreads();

    // ---- phase 3: decayed Gram tiles; Kg fragments; Gam ------------------
    {
      constexpr int NPAIR = TT * (TT + 1) / 2;
      const int flag = *s_flag;
      for (int p = wave; p < NPAIR; p += 4) {
        int a = 0, b = p;
        while (b > a) {
          b -= a + 1;
          ++a;
        }
        f32x4 akk = zero4(), aqk = zero4();
        if (a == b && (flag >> a) & 1) {
          exact_diag_tile(a, akk, aqk, q, k, g, n_heads, h, in.tok0, in.len);
        } else {
          const TIO* lkr = Lk + (16 * a + l16) * KS_LD;
          const TIO* lqr = Lq + (16 * a + l16) * KS_LD;
          const TIO* rnr = Rn + (16 * b + l16) * KS_LD;
          const bool scaled = (b != a - 1);  // adjacent blocks need no factor
#pragma unroll
          for (int s = 0; s < KBD; ++s) {
            const int c0 = 32 * s + 8 * lg;
            const FragT fk = load_frag8<TIO>(lkr + c0);
            const FragT fq = load_frag8<TIO>(lqr + c0);
            FragT fr = load_frag8<TIO>(rnr + c0);
            if (scaled) {
              const float* ra = rho + a * D + c0;
              const float* rb = rho + (b + 1) * D + c0;
#pragma unroll
              for (int e = 0; e < 8; ++e)
                fr[e] = from_f32<TIO>(to_f32(fr[e]) * fast_exp2(ra[e] - rb[e]));
            }
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
      // Kg^T fragments in kperm token order: element (kt, ts, lane, e) =
      // Kg[32ts + kperm(lg, e)][16kt + l16], Kg = Rn * 2^(rho_TT - rho_{blk+1}).
      for (int slot = tid; slot < DT * KBC * 64; slot += 256) {
        const int ln = slot & 63;
        const int kt = (slot >> 6) / KBC, ts = (slot >> 6) % KBC;
        const int c = 16 * kt + (ln & 15);
        const int g4 = ln >> 4;
        FragT f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int blk = 2 * ts + hh;  // 16-token block of these four tokens
          float fac = 0.f;
          if (blk < TT) fac = fast_exp2(rho[TT * D + c] - rho[(blk + 1) * D + c]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int tok = 16 * blk + 4 * g4 + e;
            const float val = (blk < TT) ? to_f32(Rn[tok * KS_LD + c]) * fac : 0.f;
            f[4 * hh + e] = from_f32<TIO>(val);
          }
        }
        *reinterpret_cast<FragT*>(out.k + (size_t)slot * 8) = f;
      }
      for (int c = tid; c < D; c += 256) out.gam[c] = fast_exp2(rho[TT * D + c]);
    }
    __syncthreads();

    // ---- phase 4: T = (I + A)^-1 by one wave -------------------------------
    if (wave == 0) {
      // diagonal 16x16 blocks by forward substitution: lane (block lg, column l16)
      if (lg < TT) {
        const int a = lg, j = l16;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float acc = (r == j) ? 1.f : 0.f;
          const float* Ar = As + (16 * a + r) * AF_LD + 16 * a;
#pragma unroll
          for (int i = 0; i < r; ++i) acc -= Ar[i] * x[i];
          x[r] = acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          Ts[(16 * a + r) * AF_LD + 16 * a + j] = x[r];
          Tb[(16 * a + r) * TK_LD + 16 * a + j] = from_f32<TIO>(x[r]);
        }
      }
      // off-diagonal blocks band by band: T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb
#pragma unroll
      for (int d = 1; d < TT; ++d) {
        wave_sync();
        for (int a = d; a < TT; ++a) {
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
      }
    }
    __syncthreads();

    // ---- phase 5: W^T, U, Q'^T, Ol -> outputs -------------------------------
    // Wave w owns channel slices kb = w, w + 4, ... (tiles 2kb, 2kb + 1) of
    // W^T and Q'^T and the same value-column tiles of U and Ol.
    constexpr int MW = (KBD + 3) / 4;
#pragma unroll
    for (int m = 0; m < MW; ++m) {
      const int kb = wave + 4 * m;
      if (kb < KBD) {
        f32x4 ureg[2][TT];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ct = 2 * kb + hh;
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
            ureg[hh][t] = uacc;
            TIO* wout = out.w + ((size_t)(t * KBD + kb) * 64 + lane) * 8 + 4 * hh;
            TIO* uout = out.u + ((size_t)(t * DT + ct) * 64 + lane) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const TIO wv = from_f32<TIO>(wacc[j]);
              wout[j] = wv;
              WT[(16 * ct + 4 * lg + j) * TK_LD + 16 * t + l16] = wv;
              uout[j] = from_f32<TIO>(uacc[j]);
            }
          }
        }
        if constexpr (KCP != C) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh)
            for (int x = lane; x < 16 * (KCP - C); x += 64)
              WT[(32 * kb + 16 * hh + x / (KCP - C)) * TK_LD + C + x % (KCP - C)] = zero_t;
        }
        wave_sync();  // this wave's W^T rows are complete
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int ct = 2 * kb + hh;
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
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int c = 16 * ct + 4 * lg + j;
              const float qg = to_f32(Lq[r * KS_LD + c]) * fast_exp2(rho[a * D + c]);
              qout[j] = from_f32<TIO>(scale * (qg - acc[j]));
            }
            f32x4 oacc = zero4();
#pragma unroll
            for (int s = 0; s <= t / 2; ++s) {
              const FragT fa = load_frag_perm<TIO>(Aq + (16 * t + l16) * TK_LD + 32 * s, lg);
              f32x4 u1 = zero4();
              if (2 * s + 1 < TT) u1 = ureg[hh][2 * s + 1 < TT ? 2 * s + 1 : TT - 1];
              oacc = mma32(fa, frag_from_d<TIO>(ureg[hh][2 * s], u1), oacc);
            }
            TIO* oout = out.o + ((size_t)(t * DT + ct) * 64 + lane) * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j) oout[j] = from_f32<TIO>(scale * oacc[j]);
          }
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// One step of the state scan for 16 value columns (block jb), split over the
// workgroup's KBD waves by dk slice: wave w owns state rows 32w .. 32w + 31
// (accumulator tiles, rows 32w + 16m + 4lg + j, column 16jb + l16).
template <typename TIO, int D, int C>
struct ScanStep {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  static constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KBC = Gm::KBC;
  static constexpr int VT_LD = Gm::VT_LD;
  static constexpr int NOWN = (TT + KBD - 1) / KBD;  // token tiles a wave reduces

  // Everything one step reads from a chunk's outputs, for this lane.
  struct Ops {
    FragT w[TT], q[TT], k[2][KBC];
    TIO u[NOWN][4], ol[NOWN][4];
    f32x4 gam[2];
  };

  static __device__ __forceinline__ void load(Ops& op, const ChunkOut<TIO>& in, int jb) {
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int lg = lane >> 4;
    if (w >= KBD) return;  // waves past the dk slices hold no state
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      op.w[t] = load_frag8<TIO>(in.w + ((size_t)(t * KBD + w) * 64 + lane) * 8);
      op.q[t] = load_frag8<TIO>(in.q + ((size_t)(t * KBD + w) * 64 + lane) * 8);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int kc = 0; kc < KBC; ++kc)
        op.k[m][kc] = load_frag8<TIO>(in.k + ((size_t)((2 * w + m) * KBC + kc) * 64 + lane) * 8);
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
      const int t = w + KBD * i;
      if (t < TT) {
        const TIO* Uc = in.u + ((size_t)(t * DT + jb) * 64 + lane) * 4;
        const TIO* Oc = in.o + ((size_t)(t * DT + jb) * 64 + lane) * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          op.u[i][j] = Uc[j];
          op.ol[i][j] = Oc[j];
        }
      }
    }
    const float* Gc = in.gam + 32 * w + 4 * lg;
    op.gam[0] = *reinterpret_cast<const f32x4*>(Gc);
    op.gam[1] = *reinterpret_cast<const f32x4*>(Gc + 16);
  }

  // One chunk: V = U - W S, O = Ol + Q' S (rows < len written to o), then
  // S = diag(Gam) S + Kg^T V.  Two workgroup barriers.
  static __device__ __forceinline__ void step(unsigned char* lds, f32x4 (&S)[2], const Ops& op,
                                              TIO* __restrict__ o, int64_t ostride, int h,
                                              int jb, int start, int len) {
    f32x4* red_v = reinterpret_cast<f32x4*>(lds);                    // [KBD][TT][64]
    f32x4* red_o = reinterpret_cast<f32x4*>(lds + Gm::SCAN_RED);      // [KBD][TT][64]
    TIO* Vt = reinterpret_cast<TIO*>(lds + 2 * Gm::SCAN_RED);         // [16][VT_LD]
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int l16 = lane & 15, lg = lane >> 4;

    const bool active = w < KBD;  // waves past the dk slices only keep the barriers
    if (active) {
      const FragT sb = frag_from_d<TIO>(S[0], S[1]);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        red_v[(w * TT + t) * 64 + lane] = mma32(op.w[t], sb, zero4());
        red_o[(w * TT + t) * 64 + lane] = mma32(op.q[t], sb, zero4());
      }
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NOWN; ++i) {
      const int t = w + KBD * i;
      if (active && t < TT) {
        f32x4 vv, oo;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          vv[j] = to_f32(op.u[i][j]);
          oo[j] = to_f32(op.ol[i][j]);
        }
#pragma unroll
        for (int ww = 0; ww < KBD; ++ww) {
          vv -= red_v[(ww * TT + t) * 64 + lane];
          oo += red_o[(ww * TT + t) * 64 + lane];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 16 * t + 4 * lg + j;
          Vt[l16 * VT_LD + r] = from_f32<TIO>(vv[j]);
          if (r < len)
            o[(int64_t)(start + r) * ostride + (int64_t)h * D + 16 * jb + l16] = from_f32<TIO>(oo[j]);
        }
      }
    }
    __syncthreads();
    if (!active) return;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      S[m] *= op.gam[m];
#pragma unroll
      for (int kc = 0; kc < KBC; ++kc) {
        // Kg fragments are in kperm token order; read V the same way
        const FragT fv = load_frag_perm<TIO>(Vt + l16 * VT_LD + 32 * kc, lg);
        S[m] = mma32(op.k[m][kc], fv, S[m]);
      }
    }
  }

  // Token slots past the chunk's tiles (C < 32) must read as zero.
  static __device__ __forceinline__ void clear_vt(unsigned char* lds) {
    TIO* Vt = reinterpret_cast<TIO*>(lds + 2 * Gm::SCAN_RED);
    for (int x = threadIdx.x; x < 16 * VT_LD; x += blockDim.x) Vt[x] = from_f32<TIO>(0.f);
  }
};

}  // namespace kda
