// kda_decode.hip -- recurrent KDA decode: one token per (sequence, head) on a
// carried fp32 state, updated in place.
//
// The decode form is the token recurrence itself, run once per call from the
// state the caller passes ("prefill once, then advance one token per step from
// the carried state"; page "Kimi-Linear: paged-incremental decode
// (prefill-once + carried-state decode)", squash commit).  Per (n, h):
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

// One wave: k . q and, when the rows are to be L2-normalised, the factors
// 1/sqrt(|k|^2 + eps) and 1/sqrt(|q|^2 + eps) (else 1).  The kernels use the
// raw rows and apply the factors to the reductions they feed: k . q, S^T k,
// S^T q and the rank-one write k u^T.
template <int D>
__device__ __forceinline__ void qk_dots(const float* sk, const float* sq, int norm, float* kq,
                                        float* rk, float* rq) {
  const int lane = threadIdx.x & 63;
  float a = 0.f, kk = 0.f, qq = 0.f;
  for (int i = lane; i < D; i += 64) {
    a += sk[i] * sq[i];
    kk += sk[i] * sk[i];
    qq += sq[i] * sq[i];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    a += __shfl_xor(a, off, 64);
    kk += __shfl_xor(kk, off, 64);
    qq += __shfl_xor(qq, off, 64);
  }
  if (lane == 0) {
    const float fk = norm ? __builtin_amdgcn_rsqf(kk + kQkNormEps) : 1.f;
    const float fq = norm ? __builtin_amdgcn_rsqf(qq + kQkNormEps) : 1.f;
    *kq = a * fk * fq;
    *rk = fk;
    *rq = fq;
  }
}

// GATE: the decay comes from the raw gate x with a_log and dt_bias (the Kimi
// gate, see kimi_gate_log2) instead of a given g.
template <typename TIO, int D, bool GATE>
__global__ __launch_bounds__(256) void decode_kernel(float* __restrict__ state,
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
  __shared__ float s_kq, s_rk, s_rq;  // k.q (normalised), 1/|k|, 1/|q| (1 without norm)

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
  float* S = state + sh * (int64_t)(D * D);

  // Issue every state load first: rows rg + RG * i, columns 4cq .. 4cq + 3.
  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = *reinterpret_cast<const f32x4*>(S + (rg + RG * i) * D + 4 * cq);

  // key head of value head h: h / (n_heads / kheads), rows of kheads heads
  const int64_t qk_row = (nh / n_heads) * kheads + (nh % n_heads) / (n_heads / kheads);
  if (tid < D) {
    s_q[tid] = to_f32(q[qk_row * D + tid]);
    s_k[tid] = to_f32(k[qk_row * D + tid]);
    if constexpr (GATE) {
      const int h = (int)(nh % n_heads);
      s_d[tid] = fast_exp2(kimi_gate_log2(to_f32(gx[nh * D + tid]) + dt_bias[h * D + tid],
                                          __expf(a_log[h])));
    } else {
      s_d[tid] = __expf(g[nh * D + tid]);
    }
  }
  __syncthreads();
  if (tid < 64) qk_dots<D>(s_k, s_q, qk_norm, &s_kq, &s_rk, &s_rq);

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
    p *= s_rk;
    r *= s_rq;
    const float b = to_f32(beta[nh]);
    const float u = b * (to_f32(v[nh * D + tid]) - p);
    s_u[tid] = u;
    o[nh * D + tid] = from_f32<TIO>(scale * (r + s_kq * u));
  }
  __syncthreads();

  const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cq]) * s_rk;
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int r = rg + RG * i;
    *reinterpret_cast<f32x4*>(S + r * D + 4 * cq) = s[i] + s_k[r] * u4;
  }
}

// Recurrent prefill: the decode step run over each sequence's tokens in
// order, the state held in registers from the first token to the last (one
// read and one write of the state per sequence).  The pages run decode and
// continuing prefills (T >= 1 new tokens on a carried state) through this
// recurrent op (page "model(kimi_linear): ONE-SURFACE ROW 7 -- fold
// Kimi-Linear onto the shared paged runner", B2: KdaGatedDeltaRule for decode
// and continuing prefills over the state pool keyed by state indices).
// One 256-thread workgroup per (sequence, head), tiled like decode_kernel;
// token t + 1's inputs are loaded while token t computes.  cu_seqlens is read
// clamped to [0, t_total], so any contents stay in bounds.
template <typename TIO, int D, bool GATE>
__global__ __launch_bounds__(256) void recurrent_kernel(
    const float* __restrict__ h0, float* __restrict__ ht, const TIO* __restrict__ q,
    const TIO* __restrict__ k, const TIO* __restrict__ v, const float* __restrict__ g,
    const TIO* __restrict__ gx, const float* __restrict__ a_log,
    const float* __restrict__ dt_bias, const TIO* __restrict__ beta, TIO* __restrict__ o,
    float scale, int n_heads, int64_t t_total, const int* __restrict__ cu,
    const int* __restrict__ slots, int n_slots, int kheads, int qk_norm) {
  constexpr int NQ = D / 4;
  constexpr int RG = 256 / NQ;
  constexpr int RPT = D / RG;
  static_assert(NQ * RG == 256 && RG * RPT == D, "recurrent tiling");

  __shared__ float s_q[2][D], s_k[2][D], s_d[2][D], s_v[2][D], s_u[D];
  __shared__ float s_red[2][RG][D];
  __shared__ float s_kq, s_rk, s_rq, s_b[2];

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

  f32x4 s[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i)
    s[i] = h0 ? *reinterpret_cast<const f32x4*>(h0 + sb + (rg + RG * i) * D + 4 * cq) : zero4();

  const float ea = GATE ? __expf(a_log[h]) : 1.f;
  const float bias_c = (GATE && tid < D) ? dt_bias[h * D + tid] : 0.f;
  // this thread's element of one token (tid < D), loaded ahead
  TIO rq{}, rk{}, rv{}, rx{}, rb{};
  float rg_{};
  const int kh = h / (n_heads / kheads);  // key head of value head h
  auto fetch = [&](int64_t t) {
    if (tid < D) {
      const int64_t at = (t * n_heads + h) * D + tid;
      const int64_t akt = (t * kheads + kh) * D + tid;
      rq = q[akt];
      rk = k[akt];
      rv = v[at];
      if constexpr (GATE) rx = gx[at];
      else rg_ = g[at];
    }
    if (tid == 0) rb = beta[t * n_heads + h];
  };
  if (t0 < t1) fetch(t0);
  for (int64_t t = t0; t < t1; ++t) {
    const int pb = (int)(t & 1);
    if (tid < D) {
      s_q[pb][tid] = to_f32(rq);
      s_k[pb][tid] = to_f32(rk);
      s_v[pb][tid] = to_f32(rv);
      if constexpr (GATE) s_d[pb][tid] = fast_exp2(kimi_gate_log2(to_f32(rx) + bias_c, ea));
      else s_d[pb][tid] = __expf(rg_);
    }
    if (tid == 0) s_b[pb] = to_f32(rb);
    __syncthreads();
    if (t + 1 < t1) fetch(t + 1);
    if (tid < 64) qk_dots<D>(s_k[pb], s_q[pb], qk_norm, &s_kq, &s_rk, &s_rq);
    f32x4 pk = zero4(), pq = zero4();
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      s[i] *= s_d[pb][r];
      pk += s[i] * s_k[pb][r];
      pq += s[i] * s_q[pb][r];
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
      p *= s_rk;
      r *= s_rq;
      const float u = s_b[pb] * (s_v[pb][tid] - p);
      s_u[tid] = u;
      o[(t * n_heads + h) * D + tid] = from_f32<TIO>(scale * (r + s_kq * u));
    }
    __syncthreads();
    const f32x4 u4 = *reinterpret_cast<const f32x4*>(&s_u[4 * cq]) * s_rk;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int r = rg + RG * i;
      s[i] += s_k[pb][r] * u4;
    }
  }
  if (ht) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)
      *reinterpret_cast<f32x4*>(ht + sb + (rg + RG * i) * D + 4 * cq) = s[i];
  }
}

template <typename TIO, int D>
static hipError_t launch_recurrent_t(const RecurrentArgs& a, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.n_seqs * a.n_heads;
  if (a.gate.mode == GATE_KIMI_)
    hipLaunchKernelGGL((recurrent_kernel<TIO, D, true>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, a.h0, a.ht, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v,
                       a.g, (const TIO*)a.gate.x, a.gate.a_log, a.gate.dt_bias,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.n_heads, a.t_total,
                       a.cu_seqlens, a.slots, a.n_slots, a.qk.kheads, a.qk.norm);
  else
    hipLaunchKernelGGL((recurrent_kernel<TIO, D, false>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, a.h0, a.ht, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v,
                       a.g, (const TIO*)nullptr, (const float*)nullptr, (const float*)nullptr,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.n_heads, a.t_total,
                       a.cu_seqlens, a.slots, a.n_slots, a.qk.kheads, a.qk.norm);
  return hipGetLastError();
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

template <typename TIO, int D>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
  const int64_t nblk = (int64_t)a.n_seqs * a.n_heads;
  if (a.gate.mode == GATE_KIMI_)
    hipLaunchKernelGGL((decode_kernel<TIO, D, true>), dim3((unsigned)nblk), dim3(256), 0, stream,
                       a.state, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v, a.g,
                       (const TIO*)a.gate.x, a.gate.a_log, a.gate.dt_bias, a.n_heads,
                       (const TIO*)a.beta, (TIO*)a.o, a.scale, a.slots, a.n_slots, a.qk.kheads,
                       a.qk.norm);
  else
    hipLaunchKernelGGL((decode_kernel<TIO, D, false>), dim3((unsigned)nblk), dim3(256), 0, stream,
                       a.state, (const TIO*)a.q, (const TIO*)a.k, (const TIO*)a.v, a.g,
                       (const TIO*)nullptr, (const float*)nullptr, (const float*)nullptr,
                       a.n_heads, (const TIO*)a.beta, (TIO*)a.o, a.scale, a.slots, a.n_slots,
                       a.qk.kheads, a.qk.norm);
  return hipGetLastError();
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
