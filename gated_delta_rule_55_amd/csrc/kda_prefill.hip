// kda_prefill.hip -- chunked KDA prefill on gfx950.
//
// The pages describe the chunked prefill as a fixed kernel set: chunk-local
// cumulative sum of the per-channel log-decay, beta-scaled decayed K K^T
// (inter and intra sub-blocks), a unit-lower-triangular solve, a recompute of
// W/U with per-key-channel exp2 decay, the inter-chunk state recurrence
// delta_h, and a GLA-style output (page "spike(kimi-linear): chunk_kda prefill
// AOT port -- kernel set + pinned-config recipe", commit message and section
// Delivered).  That set was written as seven launches for another GPU.  Here
// the same arithmetic runs as three launches:
//
//   chunk_map  (one workgroup)    varlen chunk table from device cu_seqlens
//   chunk_local (chunk x head)    cumsum, both decayed Gram matrices, solve,
//                                 W, U, and the chunk's output operators
//   state_scan (seq x head x 16 value columns)
//                                 the sequential recurrence over chunks with
//                                 the output fused in (the per-chunk state is
//                                 never written to memory)
//
// Per chunk of L <= C tokens (rows r, i), with G the inclusive cumulative sum
// of g over the chunk, in base 2 (G2 = log2(e) G) so every decay is one exp2:
//   A   [r,i] = beta_r sum_c k[r,c] k[i,c] 2^(G2[r,c]-G2[i,c])     i <  r
//   Aqk [r,i] =        sum_c q[r,c] k[i,c] 2^(G2[r,c]-G2[i,c])     i <= r
//   T   = (I + A)^-1
//   W   = T diag(beta) (K * 2^G2)          U = T diag(beta) V
//   Q'  = scale (Q * 2^G2 - Aqk W)         Ol = scale Aqk U
//   Kg  = K * 2^(G2_last - G2)             Gam = 2^G2_last
// and the scan over chunks, for the state S (fp32, dk x 16 columns per
// workgroup):
//   V   = U - W S                          (the chunk's delta-rule errors)
//   O   = Q' S + Ol                        (= scale (Q*2^G2 S + Aqk V))
//   S   = diag(Gam) S + Kg^T V
// Folding Aqk into Q' and Ol (Q' S + Ol = scale(Q 2^G2 S + Aqk (U - W S)))
// takes the Aqk product off the scan's serial path.
//
// Overflow: every factor formed is <= 1 for g <= 0, except the right-hand
// factor of a diagonal 16x16 Gram tile, which is referenced to the tile's first
// row and so is at most 2^(decay span of 16 tokens).  A tile whose span exceeds
// 2^64 is computed entry by entry with the exponent difference formed first.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSpanMax = 64.0f;  // max log2 factor of a factored diagonal tile

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Chunk table entry.
struct ChunkEnt {
  int seq, start, len, idx;
};

// ---------------------------------------------------------------------------
// Compile-time geometry of one (dtype, head dim, chunk) instance.
template <typename TIO, int D, int C>
struct Geo {
  static constexpr int TT = C / 16;            // token tiles
  static constexpr int DT = D / 16;            // channel tiles
  static constexpr int KBD = D / 32;           // 32-slices over channels
  static constexpr int KCP = cmax(C, 32);      // token extent padded to a slice
  static constexpr int KBC = KCP / 32;         // 32-slices over tokens
  static constexpr int TP = 16 / sizeof(TIO);  // row pad (elements) = 16 bytes
  // Per-(chunk, head) workspace blocks, in elements of TIO (Gam in floats).
  static constexpr size_t W_ELEMS = (size_t)C * D;    // W^T fragments
  static constexpr size_t Q_ELEMS = (size_t)C * D;    // Q'^T fragments
  static constexpr size_t K_ELEMS = (size_t)KCP * D;  // Kg^T fragments
  static constexpr size_t U_ELEMS = (size_t)C * D;    // U in accumulator layout
  static constexpr size_t O_ELEMS = (size_t)C * D;    // Ol in accumulator layout
  static constexpr size_t CH_BYTES = (W_ELEMS + Q_ELEMS + K_ELEMS + U_ELEMS + O_ELEMS) *
                                         sizeof(TIO) + (size_t)D * sizeof(float);

  // chunk_local LDS layout (bytes).
  static constexpr int GS_LD = D + 4;      // fp32 rows
  static constexpr int KS_LD = D + TP;     // TIO rows of D
  static constexpr int TK_LD = KCP + TP;   // TIO rows of tokens
  static constexpr int AF_LD = C + 4;      // fp32 C x C
  static constexpr size_t OFF_GS = 0;
  static constexpr size_t OFF_KS = align_up(OFF_GS + (size_t)C * GS_LD * 4, 16);
  static constexpr size_t OFF_QS = align_up(OFF_KS + (size_t)C * KS_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_KBT = align_up(OFF_QS + (size_t)C * KS_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_VBT = align_up(OFF_KBT + (size_t)D * TK_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_AS = align_up(OFF_VBT + (size_t)D * TK_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_TS = align_up(OFF_AS + (size_t)C * AF_LD * 4, 16);
  static constexpr size_t OFF_WT = OFF_AS;  // W^T reuses A and T after the solve
  static constexpr size_t OFF_TB = align_up(
      cmax((int)(OFF_TS + (size_t)C * AF_LD * 4), (int)(OFF_WT + (size_t)D * TK_LD * sizeof(TIO))),
      16);
  static constexpr size_t OFF_AQ = align_up(OFF_TB + (size_t)C * TK_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_BETA = align_up(OFF_AQ + (size_t)C * TK_LD * sizeof(TIO), 16);
  static constexpr size_t OFF_SPAN = OFF_BETA + (size_t)C * 4;
  static constexpr size_t LOCAL_LDS = align_up(OFF_SPAN + 4 * 4 + 64 * 4, 16);
  // Instances whose chunk-local stage does not fit in one CU's 160 KB of LDS
  // (fp32 operands at d = 128 with 64-token chunks) are not built.
  static constexpr bool FITS = LOCAL_LDS <= 160 * 1024;
};

// Workspace layout: [header 256 B][chunk_off (N+1) int][chunk_tab NTU ChunkEnt]
// then five TIO arrays and one float array, each [NTU * H][block].
struct WsLayout {
  size_t off_chunk_off, off_tab, off_w, off_q, off_k, off_u, off_o, off_gam, total;
};

template <typename TIO, int D, int C>
WsLayout ws_layout(int n_seqs, int n_heads, int64_t ntu) {
  using G = Geo<TIO, D, C>;
  WsLayout L;
  const size_t nch = (size_t)ntu * n_heads;
  L.off_chunk_off = 256;
  L.off_tab = align_up(L.off_chunk_off + sizeof(int) * (size_t)(n_seqs + 1), 256);
  L.off_w = align_up(L.off_tab + sizeof(ChunkEnt) * (size_t)ntu, 256);
  L.off_q = align_up(L.off_w + nch * G::W_ELEMS * sizeof(TIO), 256);
  L.off_k = align_up(L.off_q + nch * G::Q_ELEMS * sizeof(TIO), 256);
  L.off_u = align_up(L.off_k + nch * G::K_ELEMS * sizeof(TIO), 256);
  L.off_o = align_up(L.off_u + nch * G::U_ELEMS * sizeof(TIO), 256);
  L.off_gam = align_up(L.off_o + nch * G::O_ELEMS * sizeof(TIO), 256);
  L.total = align_up(L.off_gam + nch * (size_t)D * sizeof(float), 256);
  return L;
}

// ---------------------------------------------------------------------------
// a0: varlen chunk map.  One workgroup.  Validates cu_seqlens (cu[0] = 0,
// non-decreasing, cu[N] = T, chunk count within the bound) and writes, for
// every chunk, its sequence, first token, length and index within the
// sequence.  On invalid offsets no chunk is emitted and the status word says so.
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
    const int excl = s_carry + incl - cnt;
    if (n < n_seqs) chunk_off[n] = excl;
    __syncthreads();
    if (tid == 255) s_carry += incl;
    __syncthreads();
  }
  if (tid == 0) {
    if (!s_bad && s_carry > ntu) s_bad = 1;
    chunk_off[n_seqs] = s_bad ? 0 : s_carry;
    *status = s_bad ? -10 /* KDA_ERR_SEQLENS */ : 0;
  }
  __syncthreads();
  if (s_bad) {
    for (int n = tid; n < n_seqs; n += 256) chunk_off[n] = 0;
    return;
  }
  for (int n = tid; n < n_seqs; n += 256) {
    const int64_t s = cu_at(n), e = cu_at(n + 1);
    const int first = chunk_off[n];
    int j = 0;
    for (int64_t p = s; p < e; p += chunk, ++j) {
      ChunkEnt ent;
      ent.seq = n;
      ent.start = (int)p;
      ent.len = (int)((e - p) < chunk ? (e - p) : chunk);
      ent.idx = j;
      tab[first + j] = ent;
    }
  }
}

// ---------------------------------------------------------------------------
// a1-a4: chunk-local stage, one 256-thread workgroup per (chunk, head).
template <typename TIO, int D, int C>
__global__ __launch_bounds__(256) void chunk_local_kernel(
    const TIO* __restrict__ q, const TIO* __restrict__ k, const TIO* __restrict__ v,
    const float* __restrict__ g, const TIO* __restrict__ beta, int n_heads, float scale,
    const int* __restrict__ chunk_off_total, const ChunkEnt* __restrict__ tab,
    TIO* __restrict__ ws_w, TIO* __restrict__ ws_q, TIO* __restrict__ ws_k,
    TIO* __restrict__ ws_u, TIO* __restrict__ ws_o, float* __restrict__ ws_gam) {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KCP = Gm::KCP, KBC = Gm::KBC;
  constexpr int GS_LD = Gm::GS_LD, KS_LD = Gm::KS_LD, TK_LD = Gm::TK_LD, AF_LD = Gm::AF_LD;

  const int ci = blockIdx.x;
  const int h = blockIdx.y;
  if (ci >= *chunk_off_total) return;
  const ChunkEnt ent = tab[ci];
  const int L = ent.len;
  const int64_t tok0 = ent.start;
  const size_t ch = (size_t)ci * n_heads + h;

  extern __shared__ __align__(16) unsigned char lds[];
  float* Gs = reinterpret_cast<float*>(lds + Gm::OFF_GS);     // [C][GS_LD] G2
  TIO* Ks = reinterpret_cast<TIO*>(lds + Gm::OFF_KS);         // [C][KS_LD] k
  TIO* Qs = reinterpret_cast<TIO*>(lds + Gm::OFF_QS);         // [C][KS_LD] q
  TIO* KBt = reinterpret_cast<TIO*>(lds + Gm::OFF_KBT);       // [D][TK_LD] beta k 2^G2, transposed
  TIO* VBt = reinterpret_cast<TIO*>(lds + Gm::OFF_VBT);       // [D][TK_LD] beta v, transposed
  float* As = reinterpret_cast<float*>(lds + Gm::OFF_AS);     // [C][AF_LD] A (kk, beta-scaled)
  float* Ts = reinterpret_cast<float*>(lds + Gm::OFF_TS);     // [C][AF_LD] (I + A)^-1
  TIO* WT = reinterpret_cast<TIO*>(lds + Gm::OFF_WT);         // [D][TK_LD] W^T (after solve)
  TIO* Tb = reinterpret_cast<TIO*>(lds + Gm::OFF_TB);         // [C][TK_LD] T in operand dtype
  TIO* Aq = reinterpret_cast<TIO*>(lds + Gm::OFF_AQ);         // [C][TK_LD] Aqk
  float* s_beta = reinterpret_cast<float*>(lds + Gm::OFF_BETA);
  float* s_span = reinterpret_cast<float*>(lds + Gm::OFF_SPAN);  // [TT] diag tile spans

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int64_t rs = (int64_t)n_heads * D;  // token stride of q, k, v, g

  // ---- zero the operand arrays whose padding / upper tiles are read -------
  {
    const TIO z = from_f32<TIO>(0.f);
    for (int x = tid; x < C * TK_LD; x += 256) {
      Tb[x] = z;
      Aq[x] = z;
    }
    if constexpr (KCP != C)
      for (int x = tid; x < D * TK_LD; x += 256) {
        KBt[x] = z;
        VBt[x] = z;
      }
  }

  // ---- a1: load g, cumulative sum per channel (base 2) -------------------
  {
    constexpr int NSEG = 256 / D;      // token segments per channel
    constexpr int SEG = C / NSEG > 0 ? C / NSEG : 1;
    const int c = tid % D;
    const int seg = tid / D;
    float run = 0.f;
    if (seg * SEG < C) {
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int r = seg * SEG + j;
        const float gv = (r < L) ? g[(tok0 + r) * rs + (int64_t)h * D + c] : 0.f;
        run += gv * kLog2e;
        Gs[r * GS_LD + c] = run;
      }
    }
    // segment totals -> Ts (free until the solve) as scratch
    Ts[seg * D + c] = run;
    __syncthreads();
    if (seg > 0 && seg * SEG < C) {
      float add = 0.f;
      for (int s2 = 0; s2 < seg; ++s2) add += Ts[s2 * D + c];
#pragma unroll
      for (int j = 0; j < SEG; ++j) Gs[(seg * SEG + j) * GS_LD + c] += add;
    }
  }
  // ---- load k, q (rows of D), beta; zero beyond L -------------------------
  {
    constexpr int VPR = D * sizeof(TIO) / 16;  // 16-byte vectors per row
    for (int x = tid; x < C * VPR; x += 256) {
      const int r = x / VPR, cv = x % VPR;
      uint4 kv = {0, 0, 0, 0}, qv = {0, 0, 0, 0};
      if (r < L) {
        const int64_t off = (tok0 + r) * rs + (int64_t)h * D;
        kv = reinterpret_cast<const uint4*>(k + off)[cv];
        qv = reinterpret_cast<const uint4*>(q + off)[cv];
      }
      reinterpret_cast<uint4*>(Ks + r * KS_LD)[cv] = kv;
      reinterpret_cast<uint4*>(Qs + r * KS_LD)[cv] = qv;
    }
    for (int r = tid; r < C; r += 256)
      s_beta[r] = (r < L) ? to_f32(beta[(tok0 + r) * n_heads + h]) : 0.f;
  }
  __syncthreads();

  // spans of the diagonal Gram tiles (max over channels of G2[first]-G2[last])
  if (tid < 64) {
    for (int a = 0; a < TT; ++a) {
      float m = 0.f;
      for (int c = lane; c < D; c += 64) {
        const float s = fabsf(Gs[(16 * a) * GS_LD + c] - Gs[(16 * a + 15) * GS_LD + c]);
        m = fmaxf(m, s);
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
      if (lane == 0) s_span[a] = m;
    }
  }
  __syncthreads();

  // ---- a2: decayed Gram tiles A (kk) and Aqk, pair (a, b) with b <= a ------
  {
    constexpr int NPAIR = TT * (TT + 1) / 2;
    for (int p = wave; p < NPAIR; p += 4) {
      int a = 0, b = p;
      while (b > a) {
        b -= a + 1;
        ++a;
      }
      const int r = 16 * a + l16;  // row this lane feeds (left operand)
      const int i = 16 * b + l16;  // row this lane feeds (right operand)
      const float* Gr = Gs + r * GS_LD;
      const float* Gi = Gs + i * GS_LD;
      const float* Gp = Gs + (16 * a) * GS_LD;  // reference row
      f32x4 akk = zero4(), aqk = zero4();
      const bool exact = (a == b) && (s_span[a] > kSpanMax);
      if (!exact) {
#pragma unroll
        for (int s = 0; s < KBD; ++s) {
          FragT lk, lq, rk;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int c = 32 * s + kstd(lg, e);
            const float ref = Gp[c];
            const float fl = fast_exp2(Gr[c] - ref);
            const float fr = fast_exp2(ref - Gi[c]);
            lk[e] = from_f32<TIO>(to_f32(Ks[r * KS_LD + c]) * fl);
            lq[e] = from_f32<TIO>(to_f32(Qs[r * KS_LD + c]) * fl);
            rk[e] = from_f32<TIO>(to_f32(Ks[i * KS_LD + c]) * fr);
          }
          akk = mma32(lk, rk, akk);
          aqk = mma32(lq, rk, aqk);
        }
      } else {
        // entry by entry: this lane's four entries (rows 4lg+j, column l16)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rr = 16 * a + 4 * lg + j;
          const int ii = 16 * b + l16;
          float sk = 0.f, sq = 0.f;
          for (int c = 0; c < D; ++c) {
            const float f = fast_exp2(fminf(Gs[rr * GS_LD + c] - Gs[ii * GS_LD + c], 0.f));
            const float kk = to_f32(Ks[ii * KS_LD + c]) * f;
            sk += to_f32(Ks[rr * KS_LD + c]) * kk;
            sq += to_f32(Qs[rr * KS_LD + c]) * kk;
          }
          akk[j] = sk;
          aqk[j] = sq;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * a + 4 * lg + j;
        const int ii = 16 * b + l16;
        const float vkk = (ii < rr) ? s_beta[rr] * akk[j] : 0.f;
        const float vqk = (ii <= rr) ? aqk[j] : 0.f;
        As[rr * AF_LD + ii] = vkk;
        Aq[rr * TK_LD + ii] = from_f32<TIO>(vqk);
      }
    }
  }

  // ---- a4 operands: beta k 2^G2 and beta v, transposed; Kg^T fragments; Gam
  {
    for (int x = tid; x < C * D; x += 256) {
      const int i = x / D, c = x % D;  // coalesced over c
      const float b = s_beta[i];
      KBt[c * TK_LD + i] = from_f32<TIO>(b * to_f32(Ks[i * KS_LD + c]) * fast_exp2(Gs[i * GS_LD + c]));
      const float vv = (i < L) ? to_f32(v[(tok0 + i) * rs + (int64_t)h * D + c]) : 0.f;
      VBt[c * TK_LD + i] = from_f32<TIO>(b * vv);
    }
    // Kg^T fragments: element (dt, kc, lane, e) = Kg[32kc + kstd(lg,e)][16dt + l16]
    TIO* kout = ws_k + ch * Gm::K_ELEMS;
    const float* Glast = Gs + (C - 1) * GS_LD;
    for (int slot = tid; slot < DT * KBC * 64; slot += 256) {
      const int ln = slot & 63;
      const int dk = slot >> 6;
      const int dt = dk / KBC, kc = dk % KBC;
      const int c = 16 * dt + (ln & 15);
      FragT f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tok = 32 * kc + kstd(ln >> 4, e);
        float val = 0.f;
        if (tok < C) val = to_f32(Ks[tok * KS_LD + c]) * fast_exp2(Glast[c] - Gs[tok * GS_LD + c]);
        f[e] = from_f32<TIO>(val);
      }
      *reinterpret_cast<FragT*>(kout + (size_t)slot * 8) = f;
    }
    for (int c = tid; c < D; c += 256) ws_gam[ch * D + c] = fast_exp2(Glast[c]);
  }
  __syncthreads();

  // ---- a3: T = (I + A)^-1 --------------------------------------------------
  // Diagonal 16x16 blocks by forward substitution: lane (a = lg, column l16).
  if (wave == 0 && lg < TT) {
    const int a = lg;
    const int j = l16;
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
  __syncthreads();
  // Off-diagonal blocks, one band at a time:
  //   T_ab = -T_aa sum_{c=b}^{a-1} A_ac T_cb      (fp32 matrix cores)
  for (int d = 1; d < TT; ++d) {
    const int a = d + wave;
    if (a < TT) {
      const int b = a - d;
      f32x4 pacc = zero4();
      for (int c = b; c < a; ++c) {
        float fa[4], fb[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          fa[m] = As[(16 * a + l16) * AF_LD + 16 * c + 4 * m + lg];
          fb[m] = Ts[(16 * c + 4 * m + lg) * AF_LD + 16 * b + l16];
        }
        pacc = mma16_f32(fa, fb, pacc);
      }
      // T_aa (row l16, index 4lg + m) times P (rows 4lg + m held in pacc[m])
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

  // ---- a4: W^T = (beta K 2^G2)^T T^T and U = T (beta V) --------------------
  // Wave w owns channel slices kb = w, w+4, ... (channel tiles 2kb, 2kb+1) for
  // W^T, and the same value-column tiles for U.  Both stay in registers for
  // the output operators; W^T also goes to the workspace in the fragment order
  // the scan reads (t, kb, lane, 4hh + j) and U in accumulator order.
  constexpr int MW = (KBD + 3) / 4;
  f32x4 wreg[MW][2][TT];
  f32x4 ureg[MW][2][TT];
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int kb = wave + 4 * m;
    if (kb < KBD) {
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
          wreg[m][hh][t] = wacc;
          ureg[m][hh][t] = uacc;
          TIO* wout = ws_w + ch * Gm::W_ELEMS + ((size_t)(t * KBD + kb) * 64 + lane) * 8 + 4 * hh;
          TIO* uout = ws_u + ch * Gm::U_ELEMS + ((size_t)(t * DT + ct) * 64 + lane) * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wout[j] = from_f32<TIO>(wacc[j]);
            uout[j] = from_f32<TIO>(uacc[j]);
          }
        }
      }
    }
  }
  __syncthreads();  // A and T are dead: W^T may now overwrite them in LDS
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int kb = wave + 4 * m;
    if (kb < KBD) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            WT[(32 * kb + 16 * hh + 4 * lg + j) * TK_LD + 16 * t + l16] =
                from_f32<TIO>(wreg[m][hh][t][j]);
    }
  }
  // zero the padding tokens of W^T (C < 32 only)
  if constexpr (KCP != C)
    for (int x = tid; x < D * (KCP - C); x += 256) {
      const int c = x / (KCP - C), tt = C + x % (KCP - C);
      WT[c * TK_LD + tt] = from_f32<TIO>(0.f);
    }
  __syncthreads();

  // ---- output operators: Q'^T = scale (qg^T - W^T Aqk^T), Ol = scale Aqk U --
#pragma unroll
  for (int m = 0; m < MW; ++m) {
    const int kb = wave + 4 * m;
    if (kb < KBD) {
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
            acc = mma32(fw, fa, acc);  // (W^T Aqk^T)[16ct + 4lg + j][16t + l16]
          }
          const int r = 16 * t + l16;
          TIO* qout = ws_q + ch * Gm::Q_ELEMS + ((size_t)(t * KBD + kb) * 64 + lane) * 8 + 4 * hh;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int c = 16 * ct + 4 * lg + j;
            const float qg = to_f32(Qs[r * KS_LD + c]) * fast_exp2(Gs[r * GS_LD + c]);
            qout[j] = from_f32<TIO>(scale * (qg - acc[j]));
          }
          // Ol = scale Aqk U: A operand rows of Aqk in kperm order, B = U tiles
          f32x4 oacc = zero4();
#pragma unroll
          for (int s = 0; s <= t / 2; ++s) {
            const FragT fa = load_frag_perm<TIO>(Aq + (16 * t + l16) * TK_LD + 32 * s, lg);
            const f32x4 u0 = ureg[m][hh][2 * s];
            f32x4 u1 = zero4();
            if (2 * s + 1 < TT) u1 = ureg[m][hh][2 * s + 1 < TT ? 2 * s + 1 : 0];
            oacc = mma32(fa, frag_from_d<TIO>(u0, u1), oacc);
          }
          TIO* oout = ws_o + ch * Gm::O_ELEMS + ((size_t)(t * DT + ct) * 64 + lane) * 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) oout[j] = from_f32<TIO>(scale * oacc[j]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// a5 + a6: state recurrence over chunks with the output fused in.  One
// workgroup per (sequence, head, 16 value columns); wave w owns state rows
// 32w .. 32w+31 (two 16-row accumulator tiles) and contracts its slice of dk;
// the partial sums meet in LDS.
template <typename TIO, int D, int C>
__global__ __launch_bounds__(64 * (D / 32)) void state_scan_kernel(
    const float* __restrict__ h0, float* __restrict__ ht, TIO* __restrict__ o, int n_seqs,
    int n_heads, const int* __restrict__ status, const int* __restrict__ chunk_off,
    const ChunkEnt* __restrict__ tab, const TIO* __restrict__ ws_w,
    const TIO* __restrict__ ws_q, const TIO* __restrict__ ws_k,
    const TIO* __restrict__ ws_u, const TIO* __restrict__ ws_o,
    const float* __restrict__ ws_gam) {
  using Gm = Geo<TIO, D, C>;
  using FragT = typename Frag<TIO>::type;
  constexpr int TT = Gm::TT, DT = Gm::DT, KBD = Gm::KBD, KCP = Gm::KCP, KBC = Gm::KBC;
  constexpr int NB = D / 16;
  constexpr int VT_LD = KCP + Gm::TP;

  __shared__ __align__(16) f32x4 red_v[KBD][TT][64];
  __shared__ __align__(16) f32x4 red_o[KBD][TT][64];
  __shared__ __align__(16) TIO Vt[16 * VT_LD];

  if (*status != 0) return;

  // XCD-aware order: the NB column blocks of one (seq, head) share the chunk's
  // operators, so they go to workgroups with the same id mod 8 (same XCD L2).
  const int total = n_seqs * n_heads * NB;
  int y = blockIdx.x;
  if (total % 8 == 0) y = (blockIdx.x % 8) * (total / 8) + blockIdx.x / 8;
  const int jb = y % NB;
  const int h = (y / NB) % n_heads;
  const int n = y / (NB * n_heads);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;  // dk slice
  const int l16 = lane & 15;
  const int lg = lane >> 4;

  for (int x = tid; x < 16 * VT_LD; x += 64 * KBD) Vt[x] = from_f32<TIO>(0.f);

  // state tiles: rows 32w + 16m + 4lg + j, column 16jb + l16
  f32x4 S[2];
  const size_t sbase = ((size_t)n * n_heads + h) * D * D;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[m][j] = h0 ? h0[sbase + (size_t)(32 * w + 16 * m + 4 * lg + j) * D + 16 * jb + l16] : 0.f;

  const int c_begin = chunk_off[n], c_end = chunk_off[n + 1];
  const int64_t ostride = (int64_t)n_heads * D;
  __syncthreads();

  for (int ci = c_begin; ci < c_end; ++ci) {
    const ChunkEnt ent = tab[ci];
    const size_t ch = (size_t)ci * n_heads + h;
    const TIO* Wc = ws_w + ch * Gm::W_ELEMS;
    const TIO* Qc = ws_q + ch * Gm::Q_ELEMS;

    const FragT sb = frag_from_d<TIO>(S[0], S[1]);
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const FragT fw = load_frag8<TIO>(Wc + ((size_t)(t * KBD + w) * 64 + lane) * 8);
      const FragT fq = load_frag8<TIO>(Qc + ((size_t)(t * KBD + w) * 64 + lane) * 8);
      red_v[w][t][lane] = mma32(fw, sb, zero4());
      red_o[w][t][lane] = mma32(fq, sb, zero4());
    }
    __syncthreads();
    for (int t = w; t < TT; t += KBD) {
      const TIO* Uc = ws_u + ch * Gm::U_ELEMS + ((size_t)(t * DT + jb) * 64 + lane) * 4;
      const TIO* Oc = ws_o + ch * Gm::O_ELEMS + ((size_t)(t * DT + jb) * 64 + lane) * 4;
      f32x4 vv, oo;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        vv[j] = to_f32(Uc[j]);
        oo[j] = to_f32(Oc[j]);
      }
#pragma unroll
      for (int ww = 0; ww < KBD; ++ww) {
        vv -= red_v[ww][t][lane];
        oo += red_o[ww][t][lane];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = 16 * t + 4 * lg + j;
        Vt[l16 * VT_LD + r] = from_f32<TIO>(vv[j]);
        if (r < ent.len)
          o[(ent.start + r) * ostride + (int64_t)h * D + 16 * jb + l16] = from_f32<TIO>(oo[j]);
      }
    }
    __syncthreads();
    const float* Gc = ws_gam + ch * D;
    const TIO* Kc = ws_k + ch * Gm::K_ELEMS;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int dt = 2 * w + m;
#pragma unroll
      for (int j = 0; j < 4; ++j) S[m][j] *= Gc[32 * w + 16 * m + 4 * lg + j];
#pragma unroll
      for (int kc = 0; kc < KBC; ++kc) {
        const FragT fk = load_frag8<TIO>(Kc + ((size_t)(dt * KBC + kc) * 64 + lane) * 8);
        const FragT fv = load_frag8<TIO>(Vt + l16 * VT_LD + 32 * kc + 8 * lg);
        S[m] = mma32(fk, fv, S[m]);
      }
    }
  }
  if (ht) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        ht[sbase + (size_t)(32 * w + 16 * m + 4 * lg + j) * D + 16 * jb + l16] = S[m][j];
  }
}

template <typename TIO, int D, int C>
hipError_t launch_prefill_t(const PrefillArgs& a, void* workspace, hipStream_t stream) {
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
  TIO* ws_w = reinterpret_cast<TIO*>(ws + L.off_w);
  TIO* ws_q = reinterpret_cast<TIO*>(ws + L.off_q);
  TIO* ws_k = reinterpret_cast<TIO*>(ws + L.off_k);
  TIO* ws_u = reinterpret_cast<TIO*>(ws + L.off_u);
  TIO* ws_o = reinterpret_cast<TIO*>(ws + L.off_o);
  float* ws_gam = reinterpret_cast<float*>(ws + L.off_gam);

  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(256), 0, stream, a.cu_seqlens, a.n_seqs,
                     a.t_total, C, ntu, status, chunk_off, tab);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  if (ntu > 0) {
    static bool attr_set = false;  // per instantiation
    if (!attr_set) {
      err = hipFuncSetAttribute((const void*)chunk_local_kernel<TIO, D, C>,
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)Gm::LOCAL_LDS);
      if (err != hipSuccess) return err;
      attr_set = true;
    }
    hipLaunchKernelGGL((chunk_local_kernel<TIO, D, C>), dim3((unsigned)ntu, (unsigned)a.n_heads),
                       dim3(256), Gm::LOCAL_LDS, stream, (const TIO*)a.q, (const TIO*)a.k,
                       (const TIO*)a.v, a.g, (const TIO*)a.beta, a.n_heads, a.scale,
                       chunk_off + a.n_seqs, tab, ws_w, ws_q, ws_k, ws_u, ws_o, ws_gam);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const unsigned nblk = (unsigned)((int64_t)a.n_seqs * a.n_heads * (D / 16));
  hipLaunchKernelGGL((state_scan_kernel<TIO, D, C>), dim3(nblk), dim3(64 * (D / 32)), 0, stream,
                     a.h0, a.ht, (TIO*)a.o, a.n_seqs, a.n_heads, status, chunk_off, tab, ws_w,
                     ws_q, ws_k, ws_u, ws_o, ws_gam);
  return hipGetLastError();
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
hipError_t launch_c(const PrefillArgs& a, void* ws, hipStream_t s) {
  switch (a.chunk) {
    case 16: return launch_prefill_t<TIO, D, 16>(a, ws, s);
    case 32: return launch_prefill_t<TIO, D, 32>(a, ws, s);
    case 64: return launch_prefill_t<TIO, D, 64>(a, ws, s);
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
hipError_t launch_d(const PrefillArgs& a, void* ws, hipStream_t s) {
  switch (a.d) {
    case 32: return launch_c<TIO, 32>(a, ws, s);
    case 64: return launch_c<TIO, 64>(a, ws, s);
    case 128: return launch_c<TIO, 128>(a, ws, s);
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

hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  return a.bf16 ? launch_d<bf16>(a, workspace, stream) : launch_d<float>(a, workspace, stream);
}

}  // namespace kda
