// C-ABI entry points: synchronous validation, then dispatch to a kernel
// family.  Nothing here allocates, frees or synchronises.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "gdr_internal.h"

// The workspace of gdr_chunked_fwd_noalloc: one copy in each GPU's memory,
// zero at load, held until the process ends.  Host code never uses this name
// as an address (on the host it is only a handle): the device address comes
// from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace gdr {
namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

bool head_dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

size_t elem_size(gdr_dtype t) { return t == GDR_F32 ? 4 : 2; }

// Resolve and check the shape; fills `pr`.
gdr_status resolve(const gdr_shape *s, Problem &pr) {
  if (s == nullptr) return GDR_ERR_NULL;
  if (s->num_seqs < 0 || s->H_k <= 0 || s->H_v <= 0 || s->d_k <= 0 || s->d_v <= 0 ||
      s->total_tokens < 0)
    return GDR_ERR_SHAPE;
  if (s->H_v % s->H_k != 0) return GDR_ERR_SHAPE;
  if (s->cu_seqlens == nullptr) {
    if (s->seq_len < 0) return GDR_ERR_SHAPE;
    if ((int64_t)s->num_seqs * s->seq_len != s->total_tokens) return GDR_ERR_SHAPE;
  }
  if (s->dtype != GDR_F32 && s->dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
  if (!head_dim_ok(s->d_k) || !head_dim_ok(s->d_v)) return GDR_ERR_UNSUPPORTED;
  if (!(s->l2_eps >= 0.0f) || !std::isfinite(s->l2_eps)) return GDR_ERR_SHAPE;
  if (!std::isfinite(s->scale)) return GDR_ERR_SHAPE;
  // element offsets are computed in 64-bit; grid sizes must fit a launch
  if ((int64_t)s->num_seqs * s->H_v * (s->d_v / 16) > 0x7fffffffLL) return GDR_ERR_UNSUPPORTED;
  pr.num_seqs = s->num_seqs;
  pr.seq_len = s->cu_seqlens ? 0 : s->seq_len;
  pr.total = s->total_tokens;
  pr.cu = s->cu_seqlens;
  pr.H_k = s->H_k;
  pr.H_v = s->H_v;
  pr.d_k = s->d_k;
  pr.d_v = s->d_v;
  pr.dtype = static_cast<gdr_dtype>(s->dtype);
  pr.chunk = s->chunk;
  pr.scale = s->scale > 0.0f ? s->scale : 1.0f / std::sqrt((float)s->d_k);
  pr.eps = s->l2_eps;
  return GDR_OK;
}

struct Range {
  uintptr_t lo, hi;
};
Range span(const void *p, size_t bytes) {
  uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return Range{a, a + bytes};
}
bool overlap(Range x, Range y) { return x.lo < y.hi && y.lo < x.hi; }

gdr_status check_fwd(const Problem &pr, const FwdArgs &x) {
  if (!x.A_log || !x.dt_bias) return GDR_ERR_NULL;
  if (pr.total > 0 && (!x.q || !x.k || !x.v || !x.a || !x.b || !x.o)) return GDR_ERR_NULL;
  // row tensors are read and written in 16-byte vectors; per-token scalars
  // (a, b) and the per-head parameters need only their element alignment
  const void *rows[] = {x.q, x.k, x.v, x.s0, x.o, x.sT};
  for (const void *p : rows)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = elem_size(pr.dtype);
  const void *scalars[] = {x.a, x.b};
  for (const void *p : scalars)
    if (p && !aligned_to(p, es)) return GDR_ERR_ALIGN;
  const void *words[] = {x.A_log, x.dt_bias, pr.cu};
  for (const void *p : words)
    if (p && !aligned_to(p, 4)) return GDR_ERR_ALIGN;
  const size_t T = (size_t)pr.total;
  const size_t state_bytes = (size_t)pr.num_seqs * pr.H_v * pr.d_k * pr.d_v * 4;
  // KDA: a and dt_bias carry one value per key channel
  const size_t ga = pr.mode == kModeKDA ? (size_t)pr.d_k : 1;
  const Range ins[] = {
      span(x.q, T * pr.H_k * pr.d_k * es), span(x.k, T * pr.H_k * pr.d_k * es),
      span(x.v, T * pr.H_v * pr.d_v * es), span(x.a, T * pr.H_v * ga * es),
      span(x.b, T * pr.H_v * es),          span(x.A_log, (size_t)pr.H_v * 4),
      span(x.dt_bias, (size_t)pr.H_v * ga * 4),
      span(pr.cu, pr.cu ? (size_t)(pr.num_seqs + 1) * 4 : 0)};
  const Range o = span(x.o, T * pr.H_v * pr.d_v * es);
  const Range sT = span(x.sT, x.sT ? state_bytes : 0);
  const Range s0 = span(x.s0, x.s0 ? state_bytes : 0);
  for (const Range &r : ins) {
    if (r.lo == 0 || r.hi == r.lo) continue;
    if (x.o && o.hi > o.lo && overlap(r, o)) return GDR_ERR_ALIAS;
    if (x.sT && sT.hi > sT.lo && overlap(r, sT)) return GDR_ERR_ALIAS;
  }
  if (x.o && x.sT && o.hi > o.lo && sT.hi > sT.lo && overlap(o, sT)) return GDR_ERR_ALIAS;
  if (x.o && x.s0 && o.hi > o.lo && s0.hi > s0.lo && overlap(o, s0)) return GDR_ERR_ALIAS;
  // final_state may be exactly initial_state, but not a shifted overlap of it
  if (x.s0 && x.sT && x.s0 != x.sT && overlap(s0, sT)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

gdr_status launched(hipError_t e) { return e == hipSuccess ? GDR_OK : GDR_ERR_LAUNCH; }

// A caller's workspace of `need` bytes: present, large enough, 256-byte
// aligned, and overlapping nothing the call reads or writes.
gdr_status check_workspace(const Problem &pr, const FwdArgs &x, const void *workspace,
                           size_t workspace_bytes, size_t need) {
  if (!workspace) return GDR_ERR_NULL;
  if (workspace_bytes < need) return GDR_ERR_WORKSPACE;
  if (!aligned_to(workspace, 256)) return GDR_ERR_ALIGN;
  const size_t es = elem_size(pr.dtype);
  const size_t T = (size_t)pr.total;
  const size_t state_bytes = (size_t)pr.num_seqs * pr.H_v * pr.d_k * pr.d_v * 4;
  const size_t ga = pr.mode == kModeKDA ? (size_t)pr.d_k : 1;  // KDA: per-channel gates
  const Range ws = span(workspace, need);
  const Range others[] = {
      span(x.q, T * pr.H_k * pr.d_k * es), span(x.k, T * pr.H_k * pr.d_k * es),
      span(x.v, T * pr.H_v * pr.d_v * es), span(x.a, T * pr.H_v * ga * es),
      span(x.b, T * pr.H_v * es), span(x.A_log, (size_t)pr.H_v * 4),
      span(x.dt_bias, (size_t)pr.H_v * ga * 4), span(x.s0, x.s0 ? state_bytes : 0),
      span(x.o, T * pr.H_v * pr.d_v * es), span(x.sT, x.sT ? state_bytes : 0),
      span(pr.cu, pr.cu ? (size_t)(pr.num_seqs + 1) * 4 : 0)};
  for (const Range &r : others)
    if (r.lo != 0 && r.hi > r.lo && overlap(r, ws)) return GDR_ERR_ALIAS;
  return GDR_OK;
}

// Whether the cooperative form runs a batch: in one launch when all its
// groups fit the device at once; else in consecutive launches of `per`
// sequences, only when the sequences average at least kCoopMinTokens tokens
// (each launch fills and drains a pipeline of a few chunks, which the
// one-launch form, running every chain at once, does not).
constexpr int64_t kCoopMinTokens = 1024;
}  // namespace
bool coop_runs(const Problem &pr, int per) {
  if (per <= 0 || pr.total <= 0) return false;
  return per >= pr.num_seqs || pr.total >= kCoopMinTokens * pr.num_seqs;
}
namespace {

}  // namespace

// The cooperative form over consecutive batches of `per` sequences on one
// workspace (each launch leaves it zero-filled for the next).  A batch whose
// launch fails runs the one-launch form instead.
hipError_t run_coop_batches(const Problem &pr, const FwdArgs &x, int per, void *ws,
                            hipStream_t stream) {
  const size_t es = elem_size(pr.dtype);
  const size_t state = (size_t)pr.H_v * pr.d_k * pr.d_v;  // fp32 per sequence
  for (int s0 = 0; s0 < pr.num_seqs; s0 += per) {
    Problem sub = pr;
    sub.num_seqs = std::min(per, pr.num_seqs - s0);
    FwdArgs y = x;
    if (pr.cu) {
      sub.cu = pr.cu + s0;  // token offsets stay absolute
    } else {
      const size_t row0 = (size_t)s0 * pr.seq_len;
      sub.total = (int64_t)sub.num_seqs * pr.seq_len;
      auto at = [&](const void *t, size_t per_row) {
        return t ? static_cast<const void *>(static_cast<const char *>(t) + row0 * per_row * es)
                 : nullptr;
      };
      y.q = at(x.q, (size_t)pr.H_k * pr.d_k);
      y.k = at(x.k, (size_t)pr.H_k * pr.d_k);
      y.v = at(x.v, (size_t)pr.H_v * pr.d_v);
      y.a = at(x.a, (size_t)pr.H_v);
      y.b = at(x.b, (size_t)pr.H_v);
      y.o = const_cast<void *>(at(x.o, (size_t)pr.H_v * pr.d_v));
    }
    if (x.s0) y.s0 = x.s0 + (size_t)s0 * state;
    if (x.sT) y.sT = x.sT + (size_t)s0 * state;
    if (launch_chunked_coop(sub, y, ws, stream) != hipSuccess) {
      (void)hipGetLastError();  // a failed launch: the one-launch form
      const hipError_t e = launch_chunked_mfma(sub, y, stream);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

namespace {

// Device address of `scratch` on the current device, looked up on the first
// call per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void *> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

gdr_status scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return GDR_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return GDR_ERR_UNSUPPORTED;
  void *p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
        (void)hipGetLastError();
        return GDR_ERR_LAUNCH;
      }
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return GDR_OK;
}

}  // namespace
}  // namespace gdr

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char *gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_NULL: return "a required pointer is NULL";
    case GDR_ERR_SHAPE: return "inconsistent shape";
    case GDR_ERR_UNSUPPORTED: return "shape or dtype not supported by this build";
    case GDR_ERR_ALIGN: return "tensor pointer breaks its alignment rule";
    case GDR_ERR_WORKSPACE: return "workspace smaller than the call needs";
    case GDR_ERR_LAUNCH: return "kernel launch failed";
    case GDR_ERR_ALIAS: return "an output overlaps an input it may not alias";
  }
  return "unknown status";
}

gdr_status gdr_gates(const gdr_shape *shape, const void *q, const void *k, const void *a,
                     const void *b, const float *A_log, const float *dt_bias, void *q_hat,
                     void *k_hat, float *g, float *beta, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (pr.total > 0) {
    if (q_hat && !q) return GDR_ERR_NULL;
    if (k_hat && !k) return GDR_ERR_NULL;
    if ((g || beta) && (!a || !b || !A_log || !dt_bias)) return GDR_ERR_NULL;
  }
  const size_t es = elem_size(pr.dtype);
  const void *rows[] = {q, k, q_hat, k_hat};
  for (const void *p : rows)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  const void *scalars[] = {a, b};
  for (const void *p : scalars)
    if (p && !aligned_to(p, es)) return GDR_ERR_ALIGN;
  const void *words[] = {A_log, dt_bias, g, beta};
  for (const void *p : words)
    if (p && !aligned_to(p, 4)) return GDR_ERR_ALIGN;
  const size_t T = (size_t)pr.total;
  const Range ins[] = {span(q, T * pr.H_k * pr.d_k * es), span(k, T * pr.H_k * pr.d_k * es),
                       span(a, T * pr.H_v * es), span(b, T * pr.H_v * es)};
  const Range outs[] = {span(q_hat, T * pr.H_k * pr.d_k * es),
                        span(k_hat, T * pr.H_k * pr.d_k * es), span(g, T * pr.H_v * 4),
                        span(beta, T * pr.H_v * 4)};
  for (const Range &o : outs) {
    if (o.lo == 0 || o.hi == o.lo) continue;
    for (const Range &i : ins)
      if (i.lo != 0 && overlap(i, o)) return GDR_ERR_ALIAS;
  }
  for (int i = 0; i < 4; ++i)
    for (int j = i + 1; j < 4; ++j)
      if (outs[i].lo && outs[j].lo && outs[i].hi > outs[i].lo && outs[j].hi > outs[j].lo &&
          overlap(outs[i], outs[j]))
        return GDR_ERR_ALIAS;
  GatesArgs x{q, k, a, b, A_log, dt_bias, q_hat, k_hat, g, beta};
  return launched(launch_gates(pr, x, stream));
}

gdr_status gdr_recurrent_fwd(const gdr_shape *shape, const void *q, const void *k, const void *v,
                             const void *a, const void *b, const float *A_log,
                             const float *dt_bias, const float *initial_state, void *o,
                             float *final_state, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (!recurrent_supports(pr)) return GDR_ERR_UNSUPPORTED;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  return launched(launch_recurrent(pr, x, stream));
}

gdr_status gdr_chunked_fwd(const gdr_shape *shape, const void *q, const void *k, const void *v,
                           const void *a, const void *b, const float *A_log, const float *dt_bias,
                           const float *initial_state, void *o, float *final_state,
                           void *workspace, size_t workspace_bytes, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return GDR_ERR_UNSUPPORTED;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  if (chunked_mfma_supports(pr)) {
    const int per = workspace ? chunked_coop_seqs_per_launch(pr) : 0;
    if (coop_runs(pr, per)) {
      st = check_workspace(pr, x, workspace, workspace_bytes, chunked_coop_workspace_bytes(pr));
      if (st != GDR_OK) return st;
      return launched(run_coop_batches(pr, x, per, workspace, stream));
    }
    return launched(launch_chunked_mfma(pr, x, stream));
  }
  if (!chunked_vec_supports(pr)) return GDR_ERR_UNSUPPORTED;
  return launched(launch_chunked_vec(pr, x, stream));
}

gdr_status gdr_chunked_fwd_noalloc(const gdr_shape *shape, const void *q, const void *k,
                                   const void *v, const void *a, const void *b,
                                   const float *A_log, const float *dt_bias,
                                   const float *initial_state, void *o, float *final_state,
                                   hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return GDR_ERR_UNSUPPORTED;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  if (chunked_mfma_supports(pr)) {
    const size_t need = chunked_coop_workspace_bytes(pr);
    if (need > GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERR_WORKSPACE;
    const int per = chunked_coop_seqs_per_launch(pr);
    if (coop_runs(pr, per)) {
      void *ws = nullptr;
      st = scratch_of_current_device(&ws);
      if (st != GDR_OK) return st;
      Problem first = pr;
      first.num_seqs = per;
      if (clear_chunked_coop(first, ws, stream) != hipSuccess) return GDR_ERR_LAUNCH;
      return launched(run_coop_batches(pr, x, per, ws, stream));
    }
    return launched(launch_chunked_mfma(pr, x, stream));
  }
  if (!chunked_vec_supports(pr)) return GDR_ERR_UNSUPPORTED;
  return launched(launch_chunked_vec(pr, x, stream));
}

size_t gdr_chunked_workspace_bytes(const gdr_shape *shape) {
  using namespace gdr;
  Problem pr;
  if (resolve(shape, pr) != GDR_OK) return 0;
  if (!chunked_mfma_supports(pr)) return 0;
  return chunked_coop_workspace_bytes(pr);
}

gdr_status gdr_conv_silu(const gdr_shape *shape, int32_t width, const void *x, const float *weight,
                         const float *bias, const void *conv_state_in, void *q, void *k, void *v,
                         void *conv_state_out, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (width < 2 || width > 4) return GDR_ERR_UNSUPPORTED;
  if (!weight) return GDR_ERR_NULL;
  if (pr.total > 0 && (!x || !q || !k || !v)) return GDR_ERR_NULL;
  // rows, weights and biases move in 16-byte vectors
  const void *rows[] = {x, q, k, v, weight, bias};
  for (const void *p : rows)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = elem_size(pr.dtype);
  const void *elems[] = {conv_state_in, conv_state_out};
  for (const void *p : elems)
    if (p && !aligned_to(p, es)) return GDR_ERR_ALIGN;
  const void *words[] = {pr.cu};
  for (const void *p : words)
    if (p && !aligned_to(p, 4)) return GDR_ERR_ALIGN;
  const size_t T = (size_t)pr.total;
  const size_t Cq = (size_t)pr.H_k * pr.d_k, Cv = (size_t)pr.H_v * pr.d_v, C = 2 * Cq + Cv;
  const size_t hist = (size_t)pr.num_seqs * C * (width - 1) * es;
  const Range ins[] = {span(x, T * C * es), span(weight, C * width * 4),
                       span(bias, bias ? C * 4 : 0), span(conv_state_in, conv_state_in ? hist : 0),
                       span(pr.cu, pr.cu ? (size_t)(pr.num_seqs + 1) * 4 : 0)};
  const Range outs[] = {span(q, T * Cq * es), span(k, T * Cq * es), span(v, T * Cv * es),
                        span(conv_state_out, conv_state_out ? hist : 0)};
  for (int i = 0; i < 4; ++i) {
    const Range &o = outs[i];
    if (o.lo == 0 || o.hi == o.lo) continue;
    for (int j = 0; j < 5; ++j) {
      const Range &r = ins[j];
      if (r.lo == 0 || r.hi == r.lo) continue;
      // the new history may replace the old one exactly
      if (i == 3 && j == 3 && conv_state_out == conv_state_in) continue;
      if (overlap(r, o)) return GDR_ERR_ALIAS;
    }
    for (int j = i + 1; j < 4; ++j)
      if (outs[j].lo && outs[j].hi > outs[j].lo && overlap(o, outs[j])) return GDR_ERR_ALIAS;
  }
  ConvArgs a{width, x, weight, bias, conv_state_in, conv_state_out, q, k, v};
  return launched(launch_conv_silu(pr, a, stream));
}

gdr_status gdr_gated_rmsnorm(const gdr_shape *shape, const void *o, const void *z,
                             const float *weight, float eps, void *out, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return GDR_ERR_SHAPE;
  if (!weight) return GDR_ERR_NULL;
  if (pr.total > 0 && (!o || !z || !out)) return GDR_ERR_NULL;
  const void *rows[] = {o, z, out};
  for (const void *p : rows)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  if (!aligned_to(weight, 4)) return GDR_ERR_ALIGN;
  const size_t es = elem_size(pr.dtype);
  const size_t bytes = (size_t)pr.total * pr.H_v * pr.d_v * es;
  const Range ro = span(o, bytes), rz = span(z, bytes), rout = span(out, bytes),
              rw = span(weight, (size_t)pr.d_v * 4);
  if (bytes > 0) {
    // out may be o or z exactly (each element is read before the same
    // thread writes it), not a shifted overlap of either
    if (out != o && overlap(rout, ro)) return GDR_ERR_ALIAS;
    if (out != z && overlap(rout, rz)) return GDR_ERR_ALIAS;
    if (overlap(rout, rw)) return GDR_ERR_ALIAS;
  }
  NormArgs a{o, z, weight, eps, out};
  return launched(launch_gated_rmsnorm(pr, a, stream));
}

gdr_status gdr_chunked_fwd_gated_rmsnorm(const gdr_shape *shape, const void *q, const void *k,
                                         const void *v, const void *a, const void *b,
                                         const float *A_log, const float *dt_bias,
                                         const float *initial_state, const void *z,
                                         const float *norm_weight, float norm_eps, void *out,
                                         float *final_state, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  if (pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return GDR_ERR_UNSUPPORTED;
  if (!(norm_eps >= 0.0f) || !std::isfinite(norm_eps)) return GDR_ERR_SHAPE;
  if (!norm_weight) return GDR_ERR_NULL;
  if (pr.total > 0 && !z) return GDR_ERR_NULL;
  if (z && !aligned16(z)) return GDR_ERR_ALIGN;
  if (!aligned_to(norm_weight, 4)) return GDR_ERR_ALIGN;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, out, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  // z and the weight are read to the end: out and final_state must not
  // overlap them
  const size_t es = elem_size(pr.dtype);
  const size_t obytes = (size_t)pr.total * pr.H_v * pr.d_v * es;
  const Range rz = span(z, obytes), rw = span(norm_weight, (size_t)pr.d_v * 4);
  const Range rout = span(out, obytes);
  const Range rsT = span(final_state, final_state ? (size_t)pr.num_seqs * pr.H_v * pr.d_k * pr.d_v * 4 : 0);
  for (const Range &r : {rz, rw}) {
    if (r.hi == r.lo) continue;
    if (rout.hi > rout.lo && overlap(r, rout)) return GDR_ERR_ALIAS;
    if (rsT.hi > rsT.lo && overlap(r, rsT)) return GDR_ERR_ALIAS;
  }
  // the rule into out, then the norm in place: two launches (folding the
  // norm into the rule's cooperative launch was measured slower)
  const NormArgs nm{out, z, norm_weight, norm_eps, out};
  st = gdr_chunked_fwd(shape, q, k, v, a, b, A_log, dt_bias, initial_state, out, final_state,
                       workspace, workspace_bytes, stream);
  if (st != GDR_OK) return st;
  return launched(launch_gated_rmsnorm(pr, nm, stream));
}

namespace gdr {
namespace {
// Segmented chunked form: shape rules, then the workspace layout.
bool chunked_any_supports(const Problem &pr) {
  if (pr.mode == kModeKDA) return chunked_kda_supports(pr) || chunked_vec_supports(pr);
  return chunked_mfma_supports(pr) || chunked_vec_supports(pr);
}
// Whether some sequence has more than one segment (a packed batch: unless
// the whole batch fits one segment, since its lengths stay on the device);
// otherwise the segmented form is the direct one.
bool split_runs(const Problem &pr, int32_t segment_len) {
  return pr.cu ? pr.total > segment_len : pr.seq_len / segment_len > 1;
}
gdr_status split_problem(const gdr_shape *shape, int32_t segment_len, Problem &pr,
                         int mode = kModeRule) {
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  pr.mode = mode;
  if (pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return GDR_ERR_UNSUPPORTED;
  if (segment_len <= 0 || segment_len % pr.chunk != 0) return GDR_ERR_SHAPE;
  if (pr.cu == nullptr && pr.seq_len % segment_len != 0) return GDR_ERR_SHAPE;
  // the segments run on the kernels of the problem itself and, for the
  // transition maps, of the same problem with d_k-wide values
  Problem m = pr;
  m.d_v = pr.d_k;
  if (!chunked_any_supports(pr) || !chunked_any_supports(m)) return GDR_ERR_UNSUPPORTED;
  const int64_t slots = split_slots(pr, segment_len);
  if (slots > 0x7fffffffLL / pr.H_v / (pr.d_k > pr.d_v ? pr.d_k : pr.d_v)) return GDR_ERR_UNSUPPORTED;
  return GDR_OK;
}
}  // namespace
}  // namespace gdr

gdr_status gdr_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                       size_t *bytes) {
  using namespace gdr;
  if (!bytes) return GDR_ERR_NULL;
  Problem pr;
  const gdr_status st = split_problem(shape, segment_len, pr);
  if (st != GDR_OK) return st;
  *bytes = split_runs(pr, segment_len) ? split_layout(pr, segment_len).bytes : 0;
  return GDR_OK;
}

gdr_status gdr_kda_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                           size_t *bytes) {
  using namespace gdr;
  if (!bytes) return GDR_ERR_NULL;
  Problem pr;
  const gdr_status st = split_problem(shape, segment_len, pr, kModeKDA);
  if (st != GDR_OK) return st;
  *bytes = split_runs(pr, segment_len) ? split_layout(pr, segment_len).bytes : 0;
  return GDR_OK;
}

namespace gdr {
namespace {
gdr_status split_call(int mode, const gdr_shape *shape, int32_t segment_len, const void *q,
                      const void *k, const void *v, const void *a, const void *b,
                      const float *A_log, const float *dt_bias, const float *initial_state,
                      void *o, float *final_state, void *workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  Problem pr;
  gdr_status st = split_problem(shape, segment_len, pr, mode);
  if (st != GDR_OK) return st;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  if (!split_runs(pr, segment_len)) {  // one segment a sequence: the direct form
    if (mode == kModeKDA)
      return launched(chunked_kda_supports(pr) ? launch_chunked_kda(pr, x, stream)
                                               : launch_chunked_vec(pr, x, stream));
    if (chunked_mfma_supports(pr)) return launched(launch_chunked_mfma(pr, x, stream));
    return launched(launch_chunked_vec(pr, x, stream));
  }
  const SplitLayout L = split_layout(pr, segment_len);
  st = check_workspace(pr, x, workspace, workspace_bytes, L.bytes);
  if (st != GDR_OK) return st;
  // final_state == initial_state is fine: the initial state is read by the
  // combine pass, before the last launch writes the final state
  return launched(launch_chunked_split(pr, x, segment_len, workspace, stream));
}
}  // namespace
}  // namespace gdr

gdr_status gdr_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len, const void *q,
                                 const void *k, const void *v, const void *a, const void *b,
                                 const float *A_log, const float *dt_bias,
                                 const float *initial_state, void *o, float *final_state,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return gdr::split_call(gdr::kModeRule, shape, segment_len, q, k, v, a, b, A_log, dt_bias,
                         initial_state, o, final_state, workspace, workspace_bytes, stream);
}

gdr_status gdr_kda_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len, const void *q,
                                     const void *k, const void *v, const void *a, const void *b,
                                     const float *A_log, const float *dt_bias,
                                     const float *initial_state, void *o, float *final_state,
                                     void *workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  return gdr::split_call(gdr::kModeKDA, shape, segment_len, q, k, v, a, b, A_log, dt_bias,
                         initial_state, o, final_state, workspace, workspace_bytes, stream);
}

namespace gdr {
namespace {
// SSD: the rule's kernels in mode 1 (q = C, k = B, v = x, a = delta, A_log
// holds A, no b and no dt_bias); z gates the output afterwards.
// Pointer, alignment and aliasing checks of the SSD calls.
gdr_status ssd_check(const Problem &pr, const void *x, const void *delta, const float *A,
                     const void *B, const void *C, const float *initial_state, const void *z,
                     void *y, float *final_state) {
  if (!A) return GDR_ERR_NULL;
  if (pr.total > 0 && (!x || !delta || !B || !C || !y)) return GDR_ERR_NULL;
  const void *rows[] = {x, B, C, z, y, initial_state, final_state};
  for (const void *p : rows)
    if (p && !aligned16(p)) return GDR_ERR_ALIGN;
  const size_t es = elem_size(pr.dtype);
  if (delta && !aligned_to(delta, es)) return GDR_ERR_ALIGN;
  if (!aligned_to(A, 4) || (pr.cu && !aligned_to(pr.cu, 4))) return GDR_ERR_ALIGN;
  const size_t T = (size_t)pr.total;
  const size_t state_bytes = (size_t)pr.num_seqs * pr.H_v * pr.d_k * pr.d_v * 4;
  const Range ins[] = {span(x, T * pr.H_v * pr.d_v * es), span(delta, T * pr.H_v * es),
                       span(A, (size_t)pr.H_v * 4), span(B, T * pr.H_k * pr.d_k * es),
                       span(C, T * pr.H_k * pr.d_k * es), span(z, z ? T * pr.H_v * pr.d_v * es : 0),
                       span(pr.cu, pr.cu ? (size_t)(pr.num_seqs + 1) * 4 : 0)};
  const Range ry = span(y, T * pr.H_v * pr.d_v * es);
  const Range rT = span(final_state, final_state ? state_bytes : 0);
  const Range r0 = span(initial_state, initial_state ? state_bytes : 0);
  for (const Range &r : ins) {
    if (r.lo == 0 || r.hi == r.lo) continue;
    if (ry.hi > ry.lo && overlap(r, ry)) return GDR_ERR_ALIAS;
    if (rT.hi > rT.lo && overlap(r, rT)) return GDR_ERR_ALIAS;
  }
  if (ry.hi > ry.lo && rT.hi > rT.lo && overlap(ry, rT)) return GDR_ERR_ALIAS;
  if (ry.hi > ry.lo && r0.hi > r0.lo && overlap(ry, r0)) return GDR_ERR_ALIAS;
  if (initial_state && final_state && initial_state != final_state && overlap(r0, rT))
    return GDR_ERR_ALIAS;
  return GDR_OK;
}

gdr_status ssd_call(const gdr_shape *shape, bool chunked, const void *x, const void *delta,
                    const float *A, const void *B, const void *C, const float *initial_state,
                    const void *z, void *y, float *final_state, hipStream_t stream) {
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  pr.mode = kModeSSD;
  pr.scale = 1.0f;
  if (chunked && pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return GDR_ERR_UNSUPPORTED;
  st = ssd_check(pr, x, delta, A, B, C, initial_state, z, y, final_state);
  if (st != GDR_OK) return st;
  FwdArgs a{C, B, x, delta, nullptr, A, nullptr, initial_state, y, final_state};
  hipError_t e;
  if (chunked) {
    if (chunked_mfma_supports(pr)) e = launch_chunked_mfma(pr, a, stream);
    else if (chunked_vec_supports(pr)) e = launch_chunked_vec(pr, a, stream);
    else return GDR_ERR_UNSUPPORTED;
  } else {
    if (!recurrent_supports(pr)) return GDR_ERR_UNSUPPORTED;
    e = launch_recurrent(pr, a, stream);
  }
  if (e == hipSuccess && z) e = launch_silu_gate(pr, y, z, stream);
  return launched(e);
}
}  // namespace
}  // namespace gdr

gdr_status gdr_ssd_recurrent_fwd(const gdr_shape *shape, const void *x, const void *delta,
                                 const float *A, const void *B, const void *C,
                                 const float *initial_state, const void *z, void *y,
                                 float *final_state, hipStream_t stream) {
  return gdr::ssd_call(shape, false, x, delta, A, B, C, initial_state, z, y, final_state, stream);
}

gdr_status gdr_ssd_chunked_fwd(const gdr_shape *shape, const void *x, const void *delta,
                               const float *A, const void *B, const void *C,
                               const float *initial_state, const void *z, void *y,
                               float *final_state, hipStream_t stream) {
  return gdr::ssd_call(shape, true, x, delta, A, B, C, initial_state, z, y, final_state, stream);
}

gdr_status gdr_ssd_chunked_split_workspace(const gdr_shape *shape, int32_t segment_len,
                                           size_t *bytes) {
  using namespace gdr;
  if (!bytes) return GDR_ERR_NULL;
  Problem pr;
  const gdr_status st = split_problem(shape, segment_len, pr, kModeSSD);
  if (st != GDR_OK) return st;
  *bytes = split_runs(pr, segment_len) ? split_layout(pr, segment_len).bytes : 0;
  return GDR_OK;
}

gdr_status gdr_ssd_chunked_fwd_split(const gdr_shape *shape, int32_t segment_len, const void *x,
                                     const void *delta, const float *A, const void *B,
                                     const void *C, const float *initial_state, const void *z,
                                     void *y, float *final_state, void *workspace,
                                     size_t workspace_bytes, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = split_problem(shape, segment_len, pr, kModeSSD);
  if (st != GDR_OK) return st;
  pr.scale = 1.0f;
  st = ssd_check(pr, x, delta, A, B, C, initial_state, z, y, final_state);
  if (st != GDR_OK) return st;
  // the rule's argument slots: C for q, B for k, x for v, delta for a, A for A_log
  FwdArgs a{C, B, x, delta, nullptr, A, nullptr, initial_state, y, final_state};
  hipError_t e;
  if (!split_runs(pr, segment_len)) {  // one segment a sequence: the direct form
    e = chunked_mfma_supports(pr) ? launch_chunked_mfma(pr, a, stream)
                                  : launch_chunked_vec(pr, a, stream);
  } else {
    st = check_workspace(pr, a, workspace, workspace_bytes, split_layout(pr, segment_len).bytes);
    if (st != GDR_OK) return st;
    e = launch_chunked_split(pr, a, segment_len, workspace, stream);
  }
  if (e == hipSuccess && z) e = launch_silu_gate(pr, y, z, stream);
  return launched(e);
}

gdr_status gdr_kda_recurrent_fwd(const gdr_shape *shape, const void *q, const void *k,
                                 const void *v, const void *a, const void *b, const float *A_log,
                                 const float *dt_bias, const float *initial_state, void *o,
                                 float *final_state, hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  pr.mode = kModeKDA;
  if (!recurrent_supports(pr)) return GDR_ERR_UNSUPPORTED;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  return launched(launch_recurrent(pr, x, stream));
}

gdr_status gdr_kda_chunked_workspace(const gdr_shape *shape, size_t *bytes) {
  using namespace gdr;
  if (!bytes) return GDR_ERR_NULL;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  pr.mode = kModeKDA;
  if (!kda_two_pass_supports(pr) && !chunked_kda_supports(pr) && !chunked_vec_supports(pr))
    return GDR_ERR_UNSUPPORTED;
  *bytes = kda_two_pass_bytes(pr);
  return GDR_OK;
}

gdr_status gdr_kda_chunked_fwd(const gdr_shape *shape, const void *q, const void *k,
                               const void *v, const void *a, const void *b, const float *A_log,
                               const float *dt_bias, const float *initial_state, void *o,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return st;
  pr.mode = kModeKDA;
  const bool two = kda_two_pass_supports(pr);
  if (!two && !chunked_kda_supports(pr) && !chunked_vec_supports(pr)) return GDR_ERR_UNSUPPORTED;
  FwdArgs x{q, k, v, a, b, A_log, dt_bias, initial_state, o, final_state};
  st = check_fwd(pr, x);
  if (st != GDR_OK) return st;
  if (workspace && two) {
    st = check_workspace(pr, x, workspace, workspace_bytes, kda_two_pass_bytes(pr));
    if (st != GDR_OK) return st;
    return launched(launch_kda_two_pass(pr, x, workspace, stream));
  }
  if (chunked_kda_supports(pr)) return launched(launch_chunked_kda(pr, x, stream));
  if (chunked_vec_supports(pr)) return launched(launch_chunked_vec(pr, x, stream));
  return GDR_ERR_UNSUPPORTED;
}

int gdr_chunked_path(const gdr_shape *shape) {
  using namespace gdr;
  Problem pr;
  gdr_status st = resolve(shape, pr);
  if (st != GDR_OK) return -(int)st;
  if (pr.chunk != 16 && pr.chunk != 32 && pr.chunk != 64) return -(int)GDR_ERR_UNSUPPORTED;
  if (chunked_mfma_supports(pr)) return GDR_PATH_MATRIX_BF16;
  if (chunked_f32mma_supports(pr)) return GDR_PATH_MATRIX_F32;
  if (chunked_vec_supports(pr)) return GDR_PATH_VECTOR_F32;
  return -(int)GDR_ERR_UNSUPPORTED;
}

}  // extern "C"
