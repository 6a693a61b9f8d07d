// kda_abi.cpp -- the C ABI declared in include/kda.h: descriptor validation on
// the host, workspace sizing, and launches on the caller's stream.
//
// Every check runs before anything is enqueued (page "model(kimi_linear):
// ONE-SURFACE ROW 7 -- fold Kimi-Linear onto the shared paged runner",
// section Landed: an explicit choice that cannot be honoured fails loudly
// instead of being replaced).  The library reads no environment variables.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "kda.h"
#include "kda_conv.h"
#include "kda_launch.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  g_last_hip_error = (int)e;
  return KDA_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void* p, int64_t bytes) {
  const uintptr_t lo = (uintptr_t)p;
  return Range{lo, lo + (uintptr_t)(bytes > 0 ? bytes : 0)};
}

bool overlap(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.hi > a.lo && b.hi > b.lo; }

bool supported_d(int d) { return d == 32 || d == 64 || d == 128; }

// State dtype: 0 or fp32, or bf16 with bf16 inputs.  Sets *bf16_state.
int check_state_dtype(int32_t state_dtype, int32_t dtype, bool* bf16_state) {
  if (state_dtype == 0 || state_dtype == KDA_DTYPE_F32) {
    *bf16_state = false;
    return KDA_OK;
  }
  if (state_dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE;
  if (dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
  *bf16_state = true;
  return KDA_OK;
}

// Key heads (0 = H, else a divisor of H) and the q/k normalisation flag.
int check_qk(int32_t n_k_heads, int32_t qk_l2norm, int H, kda::QkArgs* out) {
  const int hg = n_k_heads == 0 ? H : n_k_heads;
  if (hg < 1 || hg > H || H % hg != 0) return KDA_ERR_SHAPE;
  if (qk_l2norm != 0 && qk_l2norm != 1) return KDA_ERR_UNSUPPORTED;
  out->kheads = hg;
  out->norm = qk_l2norm;
  return KDA_OK;
}

// The decay input of a descriptor: g (fp32), or the raw gate x (element size
// es) with a_log [H] and dt_bias [H, D].  `rows` = tokens (prefill) or
// sequences (decode).  Fills the ranges the call reads.
int check_gate(const kda_gate_desc& gt, const float* g, bool work, int64_t rows, int64_t H,
               int64_t D, int64_t es, kda::GateArgs* out, Range (&r)[3]) {
  r[0] = r[1] = r[2] = Range{0, 0};
  if (gt.mode == KDA_GATE_GIVEN) {
    if (work && !g) return KDA_ERR_NULL;
    if (g && !aligned(g, 16)) return KDA_ERR_ALIGN;  // read as 16-byte vectors
    r[0] = range_of(g, rows * H * D * 4);
    *out = kda::GateArgs{};
    return KDA_OK;
  }
  if (gt.mode != KDA_GATE_KIMI) return KDA_ERR_UNSUPPORTED;
  if (work && (!gt.x || !gt.a_log || !gt.dt_bias)) return KDA_ERR_NULL;
  // x and dt_bias are read as vectors, a_log element-wise
  (void)es;
  if ((gt.x && !aligned(gt.x, 16)) || (gt.a_log && !aligned(gt.a_log, 4)) ||
      (gt.dt_bias && !aligned(gt.dt_bias, 16)))
    return KDA_ERR_ALIGN;
  r[0] = range_of(gt.x, rows * H * D * es);
  r[1] = range_of(gt.a_log, H * 4);
  r[2] = range_of(gt.dt_bias, H * D * 4);
  out->mode = kda::GATE_KIMI_;
  out->x = gt.x;
  out->a_log = gt.a_log;
  out->dt_bias = gt.dt_bias;
  return KDA_OK;
}

// Shared checks of the prefill descriptor; fills `a` on success.
// chunked: the chunked prefill (chunk and plan are checked); else the
// recurrent prefill, which ignores them.
int check_prefill(const kda_prefill_desc* d, kda::PrefillArgs* a, bool chunked = true) {
  if (!d) return KDA_ERR_NULL;
  if (d->struct_size != sizeof(kda_prefill_desc)) return KDA_ERR_VERSION;
  if (d->dtype != KDA_DTYPE_F32 && d->dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE;
  if (d->n_seqs < 1 || d->n_heads < 1 || d->n_heads > 65535 || d->t_total < 0 ||
      d->t_total > INT32_MAX - 64)
    return KDA_ERR_SHAPE;
  if (d->dk != d->dv || !supported_d(d->dk)) return KDA_ERR_UNSUPPORTED;
  if (d->state_indices && d->n_slots < 1) return KDA_ERR_SHAPE;
  const int chunk = d->chunk == 0 ? 64 : d->chunk;
  if (chunked) {
    if (chunk != 16 && chunk != 32 && chunk != 64) return KDA_ERR_UNSUPPORTED;
    if (!kda::prefill_supported(d->dtype == KDA_DTYPE_BF16, d->dk, chunk))
      return KDA_ERR_UNSUPPORTED;
  }
  // Workgroup and item counts stay in 32-bit range: the scan runs up to
  // n_seqs x n_heads x (dk / 16) workgroups, the recurrent prefill
  // n_seqs x n_heads, and the chunk-local stage walks up to
  // (t_total / chunk + n_seqs) x n_heads (chunk, head) items.
  if ((int64_t)d->n_seqs * d->n_heads * (d->dk / 16) > INT32_MAX) return KDA_ERR_SHAPE;
  if (chunked && ((int64_t)d->t_total / chunk + d->n_seqs) * d->n_heads > INT32_MAX)
    return KDA_ERR_SHAPE;
  if (!(std::isfinite(d->scale))) return KDA_ERR_SHAPE;
  if (chunked &&
      d->plan != KDA_PLAN_AUTO && d->plan != KDA_PLAN_FUSED && d->plan != KDA_PLAN_TWO_PASS)
    return KDA_ERR_UNSUPPORTED;
  if (d->gate.mode != KDA_GATE_GIVEN && d->gate.mode != KDA_GATE_KIMI) return KDA_ERR_UNSUPPORTED;
  // The fused plan (value reserved) is not built: the chunked prefill runs as
  // the three launches of the two-pass plan only.
  if (chunked && d->plan == KDA_PLAN_FUSED) return KDA_ERR_UNSUPPORTED;
  const int sq = check_qk(d->n_k_heads, d->qk_l2norm, d->n_heads, &a->qk);
  if (sq != KDA_OK) return sq;
  const int sd = check_state_dtype(d->state_dtype, d->dtype, &a->state_bf16);
  if (sd != KDA_OK) return sd;
  a->bf16 = d->dtype == KDA_DTYPE_BF16;
  a->n_seqs = d->n_seqs;
  a->n_heads = d->n_heads;
  a->d = d->dk;
  a->chunk = chunk;
  a->t_total = d->t_total;
  a->scale = d->scale != 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  a->q = d->q;
  a->k = d->k;
  a->v = d->v;
  a->g = d->g;
  a->beta = d->beta;
  a->h0 = d->h0;
  a->cu_seqlens = d->cu_seqlens;
  a->o = d->o;
  a->ht = d->ht;
  a->slots = d->state_indices;
  a->n_slots = d->state_indices ? d->n_slots : 0;
  return KDA_OK;
}

// Checks the pointers; on success `rin` holds every input range the call
// reads (q, k, v, the decay input (3), beta, h0, cu_seqlens, state_indices).
int check_prefill_pointers(const kda_prefill_desc* d, kda::PrefillArgs* a, Range (&rin)[10]) {
  if (!d->cu_seqlens && d->n_seqs != 1) return KDA_ERR_NULL;
  if (d->t_total > 0 && (!d->q || !d->k || !d->v || !d->beta || !d->o)) return KDA_ERR_NULL;
  // q, k, v rows and the states are read as 16-byte vectors; beta, o and
  // the index tables element-wise.
  const uintptr_t es_al = d->dtype == KDA_DTYPE_BF16 ? 2 : 4;
  const void* p16[] = {d->q, d->k, d->v, d->h0, d->ht};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return KDA_ERR_ALIGN;
  const void* pe[] = {d->beta, d->o};
  for (const void* p : pe)
    if (p && !aligned(p, es_al)) return KDA_ERR_ALIGN;
  const void* p4[] = {d->cu_seqlens, d->state_indices};
  for (const void* p : p4)
    if (p && !aligned(p, 4)) return KDA_ERR_ALIGN;

  const int64_t es = a->bf16 ? 2 : 4;
  const int64_t T = d->t_total, H = d->n_heads, D = d->dk;
  // h0 / ht hold N states, or n_slots with a slot table
  const int64_t N = d->state_indices ? d->n_slots : d->n_seqs;
  Range rgate[3];
  const int st = check_gate(d->gate, d->g, T > 0, T, H, D, es, &a->gate, rgate);
  if (st != KDA_OK) return st;
  const int64_t HG = a->qk.kheads;
  const int64_t ess = a->state_bf16 ? 2 : 4;  // bytes per state element
  const Range rq = range_of(d->q, T * HG * D * es), rk = range_of(d->k, T * HG * D * es),
              rv = range_of(d->v, T * H * D * es), rb = range_of(d->beta, T * H * es),
              ro = range_of(d->o, T * H * D * es),
              rh0 = range_of(d->h0, d->h0 ? N * H * D * D * ess : 0),
              rht = range_of(d->ht, d->ht ? N * H * D * D * ess : 0),
              rcu = range_of(d->cu_seqlens, d->cu_seqlens ? ((int64_t)d->n_seqs + 1) * 4 : 0),
              rsi = range_of(d->state_indices, d->state_indices ? (int64_t)d->n_seqs * 4 : 0);
  const Range inputs[10] = {rq, rk, rv, rgate[0], rgate[1], rgate[2], rb, rh0, rcu, rsi};
  for (int i = 0; i < 10; ++i) rin[i] = inputs[i];
  for (const Range& r : inputs)
    if (overlap(ro, r)) return KDA_ERR_ALIAS;
  if (overlap(ro, rht)) return KDA_ERR_ALIAS;
  // ht may be exactly h0 (in-place carry) but may not partly overlap it, nor
  // overlap any other input.
  if (d->ht && d->h0 && d->ht != d->h0 && overlap(rht, rh0)) return KDA_ERR_ALIAS;
  for (const Range& r : inputs)
    if (&r != &inputs[7] && overlap(rht, r)) return KDA_ERR_ALIAS;
  return KDA_OK;
}

// The conv descriptor, for the forward (fwd = true) or the one-token update.
int check_conv(const kda_conv_desc* d, bool fwd, kda::ConvArgs* a) {
  if (!d) return KDA_ERR_NULL;
  if (d->struct_size != sizeof(kda_conv_desc)) return KDA_ERR_VERSION;
  if (d->dtype != KDA_DTYPE_F32 && d->dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE;
  const int W = d->width ? d->width : 4;
  if (W < 2 || W > 4) return KDA_ERR_UNSUPPORTED;
  if (d->activation != KDA_CONV_ACT_NONE && d->activation != KDA_CONV_ACT_SILU)
    return KDA_ERR_UNSUPPORTED;
  // dim <= 2^24 keeps a sequence's taps (W-1 rows) addressable with 32-bit offsets
  if (d->n_seqs < (fwd ? 1 : 0) || d->dim < 8 || d->dim % 8 || d->dim > (1 << 24))
    return KDA_ERR_SHAPE;
  const int64_t rows = fwd ? d->t_total : d->n_seqs;
  if (rows < 0 || rows > INT32_MAX) return KDA_ERR_SHAPE;
  if (d->state_indices && d->n_slots < 1) return KDA_ERR_SHAPE;
  const int n_out = d->n_out ? d->n_out : 1;
  if (n_out < 1 || n_out > 3) return KDA_ERR_SHAPE;
  a->y_off[0] = 0;
  for (int i = 0; i < n_out; ++i) {
    int w = d->y_width[i];
    if (n_out == 1 && w == 0) w = d->dim;
    if (w < 8 || w % 8 || (int64_t)a->y_off[i] + w > d->dim) return KDA_ERR_SHAPE;
    a->y_off[i + 1] = a->y_off[i] + w;
  }
  if (a->y_off[n_out] != d->dim) return KDA_ERR_SHAPE;
  for (int i = n_out + 1; i < 4; ++i) a->y_off[i] = d->dim;
  // workgroups the launches need (one per 16-byte channel vector group)
  const int64_t vn = d->dtype == KDA_DTYPE_BF16 ? 8 : 4;
  const int64_t ncb = (d->dim / vn + 255) / 256;
  if ((rows + 15) / 16 * ncb + (int64_t)d->n_seqs * ncb > INT32_MAX) return KDA_ERR_SHAPE;  // >= the real count

  const bool work = rows > 0;
  if (!d->weight || (work && !d->x)) return KDA_ERR_NULL;
  if (fwd && !d->cu_seqlens && d->n_seqs != 1) return KDA_ERR_NULL;
  for (int i = 0; i < n_out; ++i)
    if (work && !d->y[i]) return KDA_ERR_NULL;
  const void* p16[] = {d->x, d->weight, d->bias, d->state_in, d->state_out, d->y[0],
                       n_out > 1 ? d->y[1] : nullptr, n_out > 2 ? d->y[2] : nullptr};
  for (const void* p : p16)
    if (p && !aligned(p, 16)) return KDA_ERR_ALIGN;
  if ((d->state_indices && !aligned(d->state_indices, 4)) ||
      (fwd && d->cu_seqlens && !aligned(d->cu_seqlens, 4)))
    return KDA_ERR_ALIGN;

  const int64_t es = vn == 8 ? 2 : 4, dim = d->dim, N = d->n_seqs;
  const int64_t n_state = d->state_indices ? d->n_slots : N;
  const Range rst_in = range_of(d->state_in, d->state_in ? n_state * (W - 1) * dim * es : 0),
              rst_out = range_of(d->state_out, d->state_out ? n_state * (W - 1) * dim * es : 0);
  const Range ins[] = {range_of(d->x, rows * dim * es), range_of(d->weight, dim * W * 4),
                       range_of(d->bias, d->bias ? dim * 4 : 0), rst_in,
                       range_of(fwd ? d->cu_seqlens : nullptr, fwd && d->cu_seqlens ? (N + 1) * 4 : 0),
                       range_of(d->state_indices, d->state_indices ? N * 4 : 0)};
  Range ry[3];
  for (int i = 0; i < n_out; ++i) {
    ry[i] = range_of(d->y[i], rows * (a->y_off[i + 1] - a->y_off[i]) * es);
    for (const Range& r : ins)
      if (overlap(ry[i], r)) return KDA_ERR_ALIAS;
    if (overlap(ry[i], rst_out)) return KDA_ERR_ALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(ry[i], ry[j])) return KDA_ERR_ALIAS;
  }
  // state_out may be exactly state_in, never partly over it or another input
  if (d->state_out && d->state_in && d->state_out != d->state_in && overlap(rst_out, rst_in))
    return KDA_ERR_ALIAS;
  for (const Range& r : ins)
    if (&r != &ins[3] && overlap(rst_out, r)) return KDA_ERR_ALIAS;

  a->bf16 = d->dtype == KDA_DTYPE_BF16;
  a->n_seqs = d->n_seqs;
  a->dim = d->dim;
  a->width = W;
  a->act = d->activation;
  a->rows = rows;
  a->x = d->x;
  a->weight = d->weight;
  a->bias = d->bias;
  a->cu_seqlens = fwd ? d->cu_seqlens : nullptr;
  a->state_in = d->state_in;
  a->state_out = d->state_out;
  a->slots = d->state_indices;
  a->n_slots = d->state_indices ? d->n_slots : 0;
  a->n_out = n_out;
  for (int i = 0; i < 3; ++i) a->y[i] = i < n_out ? d->y[i] : nullptr;
  return KDA_OK;
}

}  // namespace

extern "C" {

int kda_abi_version(void) { return KDA_ABI_VERSION; }

const char* kda_status_string(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "required pointer is NULL";
    case KDA_ERR_SHAPE: return "size out of range";
    case KDA_ERR_DTYPE: return "unknown dtype";
    case KDA_ERR_UNSUPPORTED: return "head dim or chunk size not supported";
    case KDA_ERR_ALIGN: return "pointer misaligned";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_HIP: return "HIP launch failed";
    case KDA_ERR_VERSION: return "descriptor struct_size mismatch";
    case KDA_ERR_ALIAS: return "output overlaps an input";
    case KDA_ERR_SEQLENS: return "cu_seqlens content invalid";
    case KDA_ERR_SYNC: return "reserved (no current kernel reports it)";
    default: return "unknown status";
  }
}

int kda_last_hip_error(void) { return g_last_hip_error; }

size_t kda_chunk_prefill_workspace_bytes(const kda_prefill_desc* d, int* status) {
  kda::PrefillArgs a;
  const int st = check_prefill(d, &a);
  if (status) *status = st;
  if (st != KDA_OK) return 0;
  return kda::prefill_workspace_bytes(a);
}

int kda_chunk_prefill_timed(const kda_prefill_desc* d, void* workspace, size_t workspace_bytes,
                            void* stream, void* const* events) {
  kda::PrefillArgs a;
  int st = check_prefill(d, &a);
  if (st != KDA_OK) return st;
  Range rin[10];
  st = check_prefill_pointers(d, &a, rin);
  if (st != KDA_OK) return st;
  const size_t need = kda::prefill_workspace_bytes(a);
  if (!workspace || workspace_bytes < need) return KDA_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return KDA_ERR_ALIGN;
  const Range rw = range_of(workspace, (int64_t)need);
  const int64_t es = a.bf16 ? 2 : 4;
  const int64_t T = d->t_total, H = d->n_heads, D = d->dk;
  const int64_t N = d->state_indices ? d->n_slots : d->n_seqs;
  for (const Range& r : rin)
    if (overlap(rw, r)) return KDA_ERR_ALIAS;
  if (overlap(rw, range_of(d->o, T * H * D * es)) ||
      overlap(rw, range_of(d->ht, d->ht ? N * H * D * D * (a.state_bf16 ? 2 : 4) : 0)))
    return KDA_ERR_ALIAS;
  return hip_status(kda::launch_prefill(a, workspace, (hipStream_t)stream,
                                        reinterpret_cast<const hipEvent_t*>(events)));
}

int kda_chunk_prefill(const kda_prefill_desc* d, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return kda_chunk_prefill_timed(d, workspace, workspace_bytes, stream, nullptr);
}

int kda_chunk_prefill_noalloc(const kda_prefill_desc* d, void* stream) {
  kda::PrefillArgs a;
  int st = check_prefill(d, &a);
  if (st != KDA_OK) return st;
  Range rin[10];
  st = check_prefill_pointers(d, &a, rin);
  if (st != KDA_OK) return st;
  static_assert(kda::kNoAllocWorkspaceBytes == KDA_NOALLOC_WORKSPACE_BYTES, "header limit");
  if (kda::prefill_workspace_bytes(a) > kda::kNoAllocWorkspaceBytes) return KDA_ERR_WORKSPACE;
  void* ws = nullptr;
  const hipError_t e = kda::noalloc_workspace(&ws);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(kda::launch_prefill(a, ws, (hipStream_t)stream, nullptr));
}

int kda_recurrent_prefill(const kda_prefill_desc* d, void* stream) {
  kda::PrefillArgs a;
  int st = check_prefill(d, &a, false);
  if (st != KDA_OK) return st;
  Range rin[10];
  st = check_prefill_pointers(d, &a, rin);
  if (st != KDA_OK) return st;
  return hip_status(kda::launch_recurrent(a, (hipStream_t)stream));
}

int kda_workspace_status(const void* workspace, void* stream) {
  if (!workspace) return KDA_ERR_NULL;
  int host = 0;
  const unsigned char* p = static_cast<const unsigned char*>(workspace) + kda::kWsStatusOffset;
  hipError_t e = hipMemcpyAsync(&host, p, sizeof(int), hipMemcpyDeviceToHost, (hipStream_t)stream);
  if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e);
  return host;
}

int kda_recurrent_decode(const kda_decode_desc* d, void* stream) {
  if (!d) return KDA_ERR_NULL;
  if (d->struct_size != sizeof(kda_decode_desc)) return KDA_ERR_VERSION;
  if (d->dtype != KDA_DTYPE_F32 && d->dtype != KDA_DTYPE_BF16) return KDA_ERR_DTYPE;
  if (d->n_seqs < 0 || d->n_heads < 1 || (int64_t)d->n_seqs * d->n_heads > INT32_MAX)
    return KDA_ERR_SHAPE;
  if (d->dk != d->dv || !supported_d(d->dk)) return KDA_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return KDA_ERR_SHAPE;
  if (d->gate.mode != KDA_GATE_GIVEN && d->gate.mode != KDA_GATE_KIMI) return KDA_ERR_UNSUPPORTED;
  if (d->state_indices && d->n_slots < 1) return KDA_ERR_SHAPE;
  kda::DecodeArgs a;
  const int sq = check_qk(d->n_k_heads, d->qk_l2norm, d->n_heads, &a.qk);
  if (sq != KDA_OK) return sq;
  const int sd = check_state_dtype(d->state_dtype, d->dtype, &a.state_bf16);
  if (sd != KDA_OK) return sd;
  if (d->n_seqs == 0) return KDA_OK;
  if (!d->state || !d->q || !d->k || !d->v || !d->beta || !d->o) return KDA_ERR_NULL;
  const bool bf = d->dtype == KDA_DTYPE_BF16;
  // the state, q and k are read as 16-byte vectors (q, k as pieces of four
  // elements); v, beta, o element-wise
  if (!aligned(d->state, 16) || !aligned(d->q, 16) || !aligned(d->k, 16)) return KDA_ERR_ALIGN;
  if (d->state_indices && !aligned(d->state_indices, 4)) return KDA_ERR_ALIGN;
  const void* pe[] = {d->v, d->beta, d->o};
  for (const void* p : pe)
    if (!aligned(p, bf ? 2 : 4)) return KDA_ERR_ALIGN;
  const int64_t es = bf ? 2 : 4, NH = (int64_t)d->n_seqs * d->n_heads, D = d->dk;
  const int64_t NHG = (int64_t)d->n_seqs * a.qk.kheads;
  Range rgate[3];
  const int st = check_gate(d->gate, d->g, true, d->n_seqs, d->n_heads, D, es, &a.gate, rgate);
  if (st != KDA_OK) return st;
  const Range ro = range_of(d->o, NH * D * es);
  const int64_t NS = (d->state_indices ? (int64_t)d->n_slots : (int64_t)d->n_seqs) * d->n_heads;
  const Range ins[] = {range_of(d->state, NS * D * D * (a.state_bf16 ? 2 : 4)),
                       range_of(d->q, NHG * D * es),
                       range_of(d->k, NHG * D * es),       range_of(d->v, NH * D * es),
                       rgate[0], rgate[1], rgate[2],       range_of(d->beta, NH * es),
                       range_of(d->state_indices, d->state_indices ? (int64_t)d->n_seqs * 4 : 0)};
  for (const Range& r : ins)
    if (overlap(ro, r)) return KDA_ERR_ALIAS;
  for (int i = 1; i < 9; ++i)
    if (overlap(ins[0], ins[i])) return KDA_ERR_ALIAS;
  a.bf16 = bf;
  a.n_seqs = d->n_seqs;
  a.n_heads = d->n_heads;
  a.d = d->dk;
  a.scale = d->scale != 0.f ? d->scale : 1.0f / std::sqrt((float)d->dk);
  a.state = d->state;
  a.q = d->q;
  a.k = d->k;
  a.v = d->v;
  a.g = d->g;
  a.beta = d->beta;
  a.o = d->o;
  a.slots = d->state_indices;
  a.n_slots = d->state_indices ? d->n_slots : 0;
  return hip_status(kda::launch_decode(a, (hipStream_t)stream));
}

int kda_causal_conv1d_fwd(const kda_conv_desc* d, void* stream) {
  kda::ConvArgs a;
  const int st = check_conv(d, true, &a);
  if (st != KDA_OK) return st;
  return hip_status(kda::launch_conv_fwd(a, (hipStream_t)stream));
}

int kda_causal_conv1d_update(const kda_conv_desc* d, void* stream) {
  kda::ConvArgs a;
  const int st = check_conv(d, false, &a);
  if (st != KDA_OK) return st;
  return hip_status(kda::launch_conv_update(a, (hipStream_t)stream));
}

}  // extern "C"
