// kda_decode.hip -- recurrent KDA decode: one token per (sequence, head) on a
// carried fp32 state, updated in place.
//
// The decode form is the token recurrence itself, run once per call on the
// state the caller carries over from the prefill or the previous step (page
// "Kimi-Linear: paged-incremental decode (prefill-once + carried-state
// decode)", squash commit).  Per (n, h):
//     S' = Diag(exp(g)) S                 decay of each key-channel row
//     p  = S'^T k,  r = S'^T q            two column reductions over dk
//     u  = beta (v - p)                   delta-rule error
//     S  = S' + k u^T                     write
//     o  = scale (r + (k . q) u)          = scale S^T q after the write
//
// The step reads the state once and writes it once; it is bound by HBM
// bandwidth (a few flops per state byte), so the kernel is arranged for that:
// one 256-thread workgroup per (n, h); thread (rg, cq) owns four consecutive
// value columns (one 16-byte vector) of D / RG rows; 32 threads cover one
// 512-byte row so every load and store is a full coalesced row segment.  All
// of a thread's state loads are issued before any arithmetic, the two column
// reductions go through LDS, and the updated rows are stored from registers.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// One token's k and q rows held as 4 consecutive elements by each of NQ =
// D / 4 consecutive lanes (NQ divides 64): scale both rows in place to unit
// norm when normalising (x / sqrt(sum x^2 + eps)) and return k . q of the rows
// as used.  Sums are reduced across the NQ lanes with xor shuffles, so every
// lane of the row gets them; every lane of the wave must call it.
template <int NQ>
__device__ __forceinline__ float row_prepare(f32x4& k4, f32x4& q4, int norm) {
  float kk = 0.f, qq = 0.f, kq = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kk += k4[e] * k4[e];
    qq += q4[e] * q4[e];
    kq += k4[e] * q4[e];
  }
#pragma unroll
  for (int off = 1; off < NQ; off <<= 1) {
    kk += __shfl_xor(kk, off, 64);
    qq += __shfl_xor(qq, off, 64);
    kq += __shfl_xor(kq, off, 64);
  }
  const float fk = norm ? __builtin_amdgcn_rsqf(kk + kQkNormEps) : 1.f;
  const float fq = norm ? __builtin_amdgcn_rsqf(qq + kQkNormEps) : 1.f;
  k4 *= fk;
  q4 *= fq;
  return kq * fk * fq;
}

// GATE: the decay comes from the raw gate x with a_log and dt_bias (the Kimi
// gate, see kimi_gate_log2) instead of a given g.
// TS: storage type of the state (fp32, or bf16 rounded once per step).
template <typename TIO, int D, bool GATE, typename TS>
__global__ __launch_bounds__(256) void decode_kernel(TS* __restrict__ state,
                                                     const TIO* __restrict__ q,
                                                     const TIO* __restrict__ k,
                                                     const TIO* __restrict__ v,
                                                     const float* __restrict__ g,
                                                     const TIO* __restrict__ gx,
                                                     const float* __restrict__ a_log,
                                                     const float* __restrict__ dt_bias,
                                                     int n_heads, const TIO* __restrict__ beta,
                                                     TIO* __restrict__ o, float scale,
                                                     const int* __restrict__ slots, int n_slots,
                                                     int kheads, int qk_norm) {
  constexpr int NQ = D / 4;       // column quads per row
  constexpr int RG = 256 / NQ;    // row groups
  constexpr int RPT = D / RG;     // rows per thread
  static_assert(NQ * RG == 256 && RG * RPT == D, "decode tiling");

  __shared__ float s_q[D], s_k[D], s_d[D], s_u[D];
  __shared__ float s_red[2][RG][D];
  __shared__ float s_kq;
  using V4 = typename Vec4<TIO>::type;

  const int tid = threadIdx.x;
  const int cq = tid % NQ;
  const int rg = tid / NQ;
  const int64_t nh = blockIdx.x;
  // the state of sequence n lives in pool slot slots[n] (n without a slot
  // table); a negative slot skips the sequence: nothing is read or written
  int64_t sh = nh;
  if (slots) {
    const int slot = slots[nh / n_heads];
    if (slot < 0 || slot >= n_slots) return;
    sh = (int64_t)slot * n_heads + nh % n_heads;
  }
  TS* S = state + sh * (int64_t)(D * D);

  // Issue every state load first: rows rg + RG * i, columns 4cq .. 4cq + 3.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) s[i] = load_state4(S + (rg + RG * i) * D + 4 * cq);

  // key head of value head h: h / (n_heads / kheads), rows of kheads heads
  const int64_t qk_row = (nh / n_heads) * kheads + (nh % n_heads) / (n_heads / kheads);
  const int h = (int)(nh % n_heads);
  // wave 0 stages the token's rows, four elements per lane (lanes past NQ
  // repeat the row and store nothing); q and k leave normalised when asked
  if (tid < 64) {
    const V4 qv = *reinterpret_cast<const V4*>(q + qk_row * D + 4 * cq);
    const V4 kv = *reinterpret_cast<const V4*>(k + qk_row * D + 4 * cq);
    f32x4 q4, k4, d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q4[e] = to_f32(qv[e]);
      k4[e] = to_f32(kv[e]);
    }
    if constexpr (GATE) {
      const V4 xv = *reinterpret_cast<const V4*>(gx + nh * D + 4 * cq);
      const f32x4 b4 = *reinterpret_cast<const f32x4*>(dt_bias + h * D + 4 * cq);
      const float ea = __expf(a_log[h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = fast_exp2(kimi_gate_log2(to_f32(xv[e]) + b4[e], ea));
    } else {
      const f32x4 g4 = *reinterpret_cast<const f32x4*>(g + nh * D + 4 * cq);
#pragma unroll
      for (int e = 0; e < 4; ++e) d4[e] = __expf(g4[e]);
    }
    const float kq = row_prepare<NQ>(k4, q4, qk_norm);
    if (tid < NQ) {
      *reinterpret_cast<f32x4*>(&s_q[4 * cq]) = q4;
      *reinterpret_cast<f32x4*>(&s_k[4 * cq]) = k4;
      *reinterpret_cast<f32x4*>(&s_d[4 * cq]) = d4;
    }
    if (tid == 0) s_kq = kq;
  }
  __syncthreads();

  f32x4 pk = zero4(), pq = zero4();
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    s[i] *= s_d[r];
    pk += s[i] * s_k[r];
    pq += s[i] * s_q[r];
  }
  *reinterpret_cast<f32x4*>(&s_red[0][rg][4 * cq]) = pk;
  *reinterpret_cast<f32x4*>(&s_red[1][rg][4 * cq]) = pq;
  __syncthreads();

  if (tid < D) {
    float p = 0.f, r = 0.f;
#pragma unroll
    for (int j = 0; j < RG; ++j) {
      p += s_red[0][j][tid];
      r += s_red[1][j][tid];
    }
    const float b = to_f32(beta[nh]);
    const float u = b * (to_f32(v[nh * D + tid]) - p);
    s_u[tid] = u;
    o[nh * D + tid] = from_f32<TIO>(scale * (r + s_kq * u));
  }
  __syncthreads();

  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cq]);
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    store_state4(S + r * D + 4 * cq, s[i] + s_k[r] * u4);
  }
}

// Recurrent prefill: the decode step run over each sequence's tokens in
// order, the state held in registers from the first token to the last (one
// read and one write of the state per sequence).  The pages run decode and
// continuing prefills (T >= 1 new tokens on a carried state) through this
// recurrent op (page "model(kimi_linear): ONE-SURFACE ROW 7 -- fold
// Kimi-Linear onto the shared paged runner", B2: KdaGatedDeltaRule for decode
// and continuing prefills over the state pool keyed by state indices).
// One 256-thread workgroup per (sequence, head), tiled like decode_kernel.
// Tokens go in blocks of B = 1024 / D: each thread loads one 4-element piece
// of q, k, v and the decay input of one token of a block (a block is exactly
// one such load per thread), and the next block's loads are issued when a
// block starts, so they have the whole block's work to arrive in.  A block is
// staged in LDS as fp32 (decay already exp'd) and its tokens run from there
// with two barriers each; a block at the sequence's end runs only its real
// tokens.  cu_seqlens is read clamped to [0, t_total], so any contents stay
// in bounds.
template <typename TIO, int D, bool GATE, typename TS>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const TS* __restrict__ h0, TS* __restrict__ ht, const TIO* __restrict__ q,
    const TIO* __restrict__ k, const TIO* __restrict__ v, const float* __restrict__ g,
    const TIO* __restrict__ gx, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const TIO* __restrict__ beta, TIO* __restrict__ o,
    float scale, int n_heads, int64_t t_total, const int* __restrict__ cu,
    const int* __restrict__ slots, int n_slots, int kheads, int qk_norm) {
  constexpr int NQ = D / 4;
  constexpr int RG = 256 / NQ;
  constexpr int RPT = D / RG;
  constexpr int B = 256 / NQ;  // tokens per block: one 4-element piece per thread
  static_assert(NQ * RG == 256 && RG * RPT == D, "recurrent tiling");
  using V4 = typename Vec4<TIO>::type;

  __shared__ float s_q[B][D], s_k[B][D], s_d[B][D], s_v[B][D], s_b[B], s_kq[B];
  __shared__ float s_u[D];
  __shared__ float s_red[2][RG][D];
  // running-decay form of a block (see fold): k L_j, q L_j, k / L_j per token
  // and channel, L of the block's last token, and whether the block must take
  // the direct form instead
  __shared__ float s_kt[B][D], s_qt[B][D], s_kh[B][D], s_L[D];
  __shared__ int s_direct;

  const int tid = threadIdx.x;
  const int cq = tid % NQ;
  const int rg = tid / NQ;
  const int n = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
  int slot = n;
  if (slots) {
    slot = slots[n];
    if (slot < 0 || slot >= n_slots) return;
  }
  int64_t t0 = cu ? cu[n] : 0, t1 = cu ? cu[n + 1] : t_total;
  t0 = t0 < 0 ? 0 : (t0 > t_total ? t_total : t0);
  t1 = t1 < t0 ? t0 : (t1 > t_total ? t_total : t1);
  const int64_t sb = ((int64_t)slot * n_heads + h) * (int64_t)(D * D);

  // no h0: an empty buffer whose loads read 0 (no branch around the loads)
  constexpr int ESS = (int)sizeof(TS);
  const __amdgpu_buffer_rsrc_t hr =
      make_rsrc(const_cast<TS*>(h0 ? h0 + sb : h0), h0 ? D * D * ESS : 0);
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int off = ((rg + RG * i) * D + 4 * cq) * ESS;
    if constexpr (ESS == 4) {
      s[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(hr, off, 0, 0));
    } else {
      const bf16x4 v = __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(hr, off, 0, 0));
      s[i] = f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    }
  }

  // this thread's piece of a block: token rg of the block, elements 4cq..4cq+3
  const float ea = GATE ? __expf(a_log[h]) : 1.f;
  f32x4 bias4 = zero4();
  if constexpr (GATE) bias4 = *reinterpret_cast<const f32x4*>(dt_bias + h * D + 4 * cq);
  const int kh = h / (n_heads / kheads);  // key head of value head h
  V4 lq, lk, lv, lx;
  f32x4 lg = zero4();
  TIO lb;
  auto fetch = [&](int64_t tb) {  // the block starting at tb (t0 <= tb < t1)
    const int64_t t = tb + rg < t1 ? tb + rg : t1 - 1;
    const int64_t at = (t * n_heads + h) * D + 4 * cq;
    const int64_t akt = (t * kheads + kh) * D + 4 * cq;
    lq = *reinterpret_cast<const V4*>(q + akt);
    lk = *reinterpret_cast<const V4*>(k + akt);
    lv = *reinterpret_cast<const V4*>(v + at);
    if constexpr (GATE) lx = *reinterpret_cast<const V4*>(gx + at);
    else lg = *reinterpret_cast<const f32x4*>(g + at);
    lb = beta[t * n_heads + h];
  };
  // stage the fetched block: q and k rows normalised when asked (the NQ lanes
  // of a row reduce its sums together), k . q per token, decay exp'd (rows
  // past the sequence's end repeat its last token and are never used)
  auto stage = [&](int64_t /*tb*/) {
    f32x4 q4, k4, v4, d4;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      q4[e] = to_f32(lq[e]);
      k4[e] = to_f32(lk[e]);
      v4[e] = to_f32(lv[e]);
      float d;
      if constexpr (GATE) d = fast_exp2(kimi_gate_log2(to_f32(lx[e]) + bias4[e], ea));
      else d = __expf(lg[e]);
      d4[e] = d;
    }
    const float kq = row_prepare<NQ>(k4, q4, qk_norm);
    *reinterpret_cast<f32x4*>(&s_q[rg][4 * cq]) = q4;
    *reinterpret_cast<f32x4*>(&s_k[rg][4 * cq]) = k4;
    *reinterpret_cast<f32x4*>(&s_v[rg][4 * cq]) = v4;
    *reinterpret_cast<f32x4*>(&s_d[rg][4 * cq]) = d4;
    if (cq == 0) {
      s_b[rg] = to_f32(lb);
      s_kq[rg] = kq;
    }
    if (tid == 0) s_direct = 0;
  };
  // Running-decay form of a staged block of nb tokens (one thread per
  // channel, after a barrier; a barrier must follow).  With L_j the product
  // of the block's decays up to token j, the state is carried through the
  // block as S_hat = S / L (per key channel), so a token needs no decay of
  // the state: p = S_hat^T (L_j k), r = S_hat^T (L_j q), S_hat += (k / L_j) u^T,
  // and S = L_last S_hat once at the block's end -- three operations per
  // state value and token instead of four.  A block where some L_j leaves
  // [2^-60, 2^60] (strong decay) keeps the direct form.
  auto fold = [&](int nb) {
    if (tid < D) {
      float L = 1.f;
      bool ok = true;
      for (int j = 0; j < nb; ++j) {
        L *= s_d[j][tid];
        ok = ok && L >= 0x1p-60f && L <= 0x1p60f;
        const float kv = s_k[j][tid];
        s_kt[j][tid] = kv * L;
        s_qt[j][tid] = s_q[j][tid] * L;
        s_kh[j][tid] = kv * __builtin_amdgcn_rcpf(L);
      }
      s_L[tid] = L;
      if (!ok) s_direct = 1;
    }
  };
  auto block_len = [&](int64_t tb) { return t1 - tb < B ? (int)(t1 - tb) : B; };
  if (t0 < t1) {
    fetch(t0);
    stage(t0);
  }
  __syncthreads();
  if (t0 < t1) {
    fold(block_len(t0));
    __syncthreads();
  }
  for (int64_t tb = t0; tb < t1; tb += B) {
    fetch(tb + B < t1 ? tb + B : tb);  // the next block (the current one again at the end)
    const int nb = block_len(tb);      // tokens of this block (uniform)
    const bool direct = s_direct != 0;
    // the running form reads k L_j, q L_j and writes with k / L_j; the
    // direct form decays the state first and uses k and q as they are
    const float(*ka)[D] = direct ? s_k : s_kt;
    const float(*qa)[D] = direct ? s_q : s_qt;
    const float(*wa)[D] = direct ? s_k : s_kh;
#pragma unroll 1
    for (int j = 0; j < nb; ++j) {
      if (direct) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) s[i] *= s_d[j][rg + RG * i];
      }
      f32x4 pk = zero4(), pq = zero4();
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const int r = rg + RG * i;
        pk += s[i] * ka[j][r];
        pq += s[i] * qa[j][r];
      }
      *reinterpret_cast<f32x4*>(&s_red[0][rg][4 * cq]) = pk;
      *reinterpret_cast<f32x4*>(&s_red[1][rg][4 * cq]) = pq;
      __syncthreads();
      if (tid < D) {
        float p = 0.f, r = 0.f;
#pragma unroll
        for (int jj = 0; jj < RG; ++jj) {
          p += s_red[0][jj][tid];
          r += s_red[1][jj][tid];
        }
        const float u = s_b[j] * (s_v[j][tid] - p);
        s_u[tid] = u;
        o[((tb + j) * n_heads + h) * D + tid] = from_f32<TIO>(scale * (r + s_kq[j] * u));
      }
      __syncthreads();
      const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cq]);
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] += wa[j][rg + RG * i] * u4;
    }
    if (!direct) {
#pragma unroll
      for (int i = 0; i < RPT; ++i) s[i] *= s_L[rg + RG * i];
    }
    __syncthreads();  // every token of the block has read it
    if (tb + B < t1) stage(tb + B);
    __syncthreads();
    if (tb + B < t1) {
      fold(block_len(tb + B));
      __syncthreads();
    }
  }
  if (ht) {
#pragma unroll
    for (int i = 0; i < RPT; ++i) store_state4(ht + sb + (rg + RG * i) * D + 4 * cq, s[i]);
  }
}

template <typename TIO, int D, typename TS>
static hipError_t launch_recurrent_s(const RecurrentArgs& a, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.n_seqs * a.n_heads;
  const TS* h0 = static_cast<const TS*>(a.h0);
  TS* ht = static_cast<TS*>(a.ht);
  if (a.gate.mode == GATE_KIMI_)
    hipLaunchKernelGGL((recurrent_kernel<TIO, D, true, TS>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, h0, ht, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v,
                       a.g, (const TIO*)a.gate.x, a.gate.a_log, a.gate.dt_bias,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.n_heads, a.t_total,
                       a.cu_seqlens, a.slots, a.n_slots, a.qk.kheads, a.qk.norm);
  else
    hipLaunchKernelGGL((recurrent_kernel<TIO, D, false, TS>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, h0, ht, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v,
                       a.g, (const TIO*)nullptr, (const float*)nullptr, (const float*)nullptr,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.n_heads, a.t_total,
                       a.cu_seqlens, a.slots, a.n_slots, a.qk.kheads, a.qk.norm);
  return hipGetLastError();
}

// A bf16 state comes with bf16 inputs only (checked by the C ABI).
template <typename TIO, int D>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
  if constexpr (sizeof(TIO) == 2)
    if (a.state_bf16) return launch_recurrent_s<TIO, D, bf16>(a, stream);
  return launch_recurrent_s<TIO, D, float>(a, stream);
}

hipError_t launch_recurrent(const RecurrentArgs& a, hipStream_t stream) {
  if ((int64_t)a.n_seqs * a.n_heads == 0) return hipSuccess;
  const bool bf = a.bf16;
  switch (a.d) {
    case 32:
      return bf ? launch_recurrent_t<bf16, 32>(a, stream) : launch_recurrent_t<float, 32>(a, stream);
    case 64:
      return bf ? launch_recurrent_t<bf16, 64>(a, stream) : launch_recurrent_t<float, 64>(a, stream);
    case 128:
      return bf ? launch_recurrent_t<bf16, 128>(a, stream)
                : launch_recurrent_t<float, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename TIO, int D, typename TS>
static hipError_t launch_decode_s(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.n_seqs * a.n_heads;
  TS* state = static_cast<TS*>(a.state);
  if (a.gate.mode == GATE_KIMI_)
    hipLaunchKernelGGL((decode_kernel<TIO, D, true, TS>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, state, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v, a.g,
                       (const TIO*)a.gate.x, a.gate.a_log, a.gate.dt_bias, a.n_heads,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.slots, a.n_slots, a.qk.kheads,
                       a.qk.norm);
  else
    hipLaunchKernelGGL((decode_kernel<TIO, D, false, TS>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, state, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v, a.g,
                       (const TIO*)nullptr, (const float*)nullptr, (const float*)nullptr,
                       a.n_heads, (const TIO*)a.beta, (TIO*)a.o, a.scale, a.slots, a.n_slots,
                       a.qk.kheads, a.qk.norm);
  return hipGetLastError();
}

template <typename TIO, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  if constexpr (sizeof(TIO) == 2)
    if (a.state_bf16) return launch_decode_s<TIO, D, bf16>(a, stream);
  return launch_decode_s<TIO, D, float>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if ((int64_t)a.n_seqs * a.n_heads == 0) return hipSuccess;
  const bool bf = a.bf16;
  switch (a.d) {
    case 32: return bf ? launch_decode_t<bf16, 32>(a, stream) : launch_decode_t<float, 32>(a, stream);
    case 64: return bf ? launch_decode_t<bf16, 64>(a, stream) : launch_decode_t<float, 64>(a, stream);
    case 128:
      return bf ? launch_decode_t<bf16, 128>(a, stream) : launch_decode_t<float, 128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
