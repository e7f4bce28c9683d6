// Sequential (decode) form of the gated delta rule.
//
// GatedDeltaRule.ixx File Reference, "Detailed Description": per value head an
// fp32 state S [d_k, d_v]; per token S <- S*exp(g); delta <- (v - k^T S)*beta;
// S <- S + k (outer) delta; o <- q^T S, with q, k L2-normalised and q scaled.
// Decode runs this sequential form, so its cost is one read and one write of S
// per (sequence, head) per call -- a pure stream of the state through HBM.
//
// A workgroup holds the whole [d_k, d_v] state of one (sequence, value head)
// in registers while it runs that unit's tokens.  Thread (rg, cg) owns columns
// 4cg..4cg+3 of rows rg, rg + RG, rg + 2RG, ...; consecutive threads own
// consecutive 16-byte column groups, so each wave loads and stores whole rows
// (fully coalesced).  The grid is persistent (two workgroups per compute unit)
// and each workgroup walks the units blockIdx.x, + gridDim.x, ...: while it
// works on one unit the state of its next unit is already streaming into a
// second register set, and states are loaded and stored non-temporally (each
// is touched exactly once per call).  On one MI355X this keeps the state
// stream near the rate of a plain in-place copy.
//
// Per token, with the state taken BEFORE the decay (all reassociations of the
// stated order):
//   u_j = k^T S[:, j],  w_j = q^T S[:, j]       (raw q, k; two column reductions)
//   k_hat = k / |k|,  q_hat = scale * q / |q|
//   delta_j = beta * (v_j - alpha * u_j / |k|)
//   o_j     = alpha * scale * w_j / |q| + (q_hat . k_hat) * delta_j
//   S[i, j] = alpha * S[i, j] + k_hat_i * delta_j
// so the state is read once and written once, and the norms and q.k ride along
// in the same reduction as u and w.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

template <int DK, int DV>
struct RecGeom {
  static constexpr int CG = DV / 4;                               // column groups
  static constexpr int RG = (DK < 512 / CG) ? DK : 512 / CG;      // row groups
  static constexpr int NT = CG * RG;                              // threads
  static constexpr int RPT = DK / RG;                             // rows per thread
  static constexpr int NW = (NT + 63) / 64;                       // waves
  static constexpr int RG_PER_WAVE = (64 / CG < RG) ? 64 / CG : RG;
  static constexpr int NRED = 11;  // u[4], w[4], |k|^2, |q|^2, q.k
  static_assert(DV % 4 == 0 && DK % RG == 0, "bad geometry");
};

typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 nt_load4(const float *p) {
  const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store4(float *p, float4 v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4 *>(p));
}

template <typename T>
struct RecParams {
  const T *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  const float *s0;
  T *o;
  float *sT;
  const int32_t *cu;
  int seq_len;
  int units;  // num_seqs * H_v
  int H_k, H_v;
  float scale, eps;
};

// MODE kModeSSD: the Mamba-2 SSD recurrence on the same scan: no norms, no
// erase, g = A delta with delta in `a` and A in `A_log`, beta = delta.
// MODE kModeKDA: one decay per key channel, so row i of S decays by its own
// alpha_i = exp(g[i]); the rows are decayed in place before the reductions and
// the rest is the rule's step with alpha = 1.
template <int DK, int DV, typename T, int MODE>
// (at most 128 registers per lane: two 8-wave workgroups per compute unit)
__global__ __launch_bounds__((RecGeom<DK, DV>::NT)) __attribute__((amdgpu_waves_per_eu(4)))
void recurrent_kernel(RecParams<T> p) {
  using G = RecGeom<DK, DV>;
  constexpr bool SSD = MODE == kModeSSD, KDA = MODE == kModeKDA;
  constexpr int CG = G::CG, RG = G::RG, RPT = G::RPT, NW = G::NW, NRED = G::NRED;
  __shared__ float red[2][NW > 1 ? NW : 1][CG][NRED];

  const int tid = threadIdx.x;
  const int cg = tid % CG;
  const int rg = tid / CG;
  const int wave = tid / 64;

  auto state_at = [&](int u) { return (size_t)u * DK * DV + 4 * cg; };
  auto load_state = [&](int u, float4 *dst) {
    if (p.s0) {
      const float *src = p.s0 + state_at(u);
#pragma unroll
      for (int i = 0; i < RPT; ++i) dst[i] = nt_load4(src + (size_t)(rg + RG * i) * DV);
    } else {
#pragma unroll
      for (int i = 0; i < RPT; ++i) dst[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  float4 S[RPT], Sn[RPT];
  int u = blockIdx.x;
  if (u < p.units) load_state(u, S);
  int step = 0;  // tokens processed by this workgroup (selects the reduction buffer)
  for (; u < p.units; u += gridDim.x) {
    const int un = u + gridDim.x;
    if (un < p.units) load_state(un, Sn);
    const int n = u / p.H_v;
    const int h = u % p.H_v;
    const int hk = h / (p.H_v / p.H_k);
    int64_t t0, t1;
    seq_bounds(p.cu, p.seq_len, n, t0, t1);
    const float neg_exp_A = SSD ? p.A_log[h] : -expf(p.A_log[h]);  // SSD: A itself
    const float dtb = (SSD || KDA) ? 0.0f : p.dt_bias[h];

    for (int64_t t = t0; t < t1; ++t, ++step) {
      const T *kr = p.k + (t * p.H_k + hk) * DK;
      const T *qr = p.q + (t * p.H_k + hk) * DK;
      float kv[RPT], qv[RPT];
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        kv[i] = to_f32(kr[rg + RG * i]);
        qv[i] = to_f32(qr[rg + RG * i]);
      }
      const float4 vv = load4(p.v + (t * p.H_v + h) * DV + 4 * cg);
      const float a_t = KDA ? 0.0f : to_f32(p.a[t * p.H_v + h]);
      const float b_t = SSD ? 0.0f : to_f32(p.b[t * p.H_v + h]);
      // KDA: decay this thread's rows in place first (each by its own
      // alpha), then run the rule's step with alpha = 1
      if constexpr (KDA) {
        // per-row gates through the hardware base-2 units (eight per token
        // per thread: the library expf / log1pf would dominate the step)
        const T *ar = p.a + (t * p.H_v + h) * DK;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
          const float x = to_f32(ar[rg + RG * i]) + p.dt_bias[h * DK + rg + RG * i];
          const float sp = fmaxf(x, 0.f) + 0.6931471805599453f *
                                               __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * 1.4426950408889634f));
          const float al = __builtin_amdgcn_exp2f(neg_exp_A * 1.4426950408889634f * sp);
          S[i].x *= al;
          S[i].y *= al;
          S[i].z *= al;
          S[i].w *= al;
        }
      }

      float r[NRED];
#pragma unroll
      for (int j = 0; j < NRED; ++j) r[j] = 0.f;
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        r[0] += kv[i] * S[i].x;
        r[1] += kv[i] * S[i].y;
        r[2] += kv[i] * S[i].z;
        r[3] += kv[i] * S[i].w;
        r[4] += qv[i] * S[i].x;
        r[5] += qv[i] * S[i].y;
        r[6] += qv[i] * S[i].z;
        r[7] += qv[i] * S[i].w;
        r[8] += kv[i] * kv[i];
        r[9] += qv[i] * qv[i];
        r[10] += qv[i] * kv[i];
      }
      // reduce over the row groups of this wave (lanes that differ by multiples of CG)
#pragma unroll
      for (int off = CG; off < CG * G::RG_PER_WAVE; off <<= 1) {
#pragma unroll
        for (int j = 0; j < NRED; ++j) r[j] += __shfl_xor(r[j], off, 64);
      }
      if constexpr (NW > 1) {
        const int buf = step & 1;
        if (tid % 64 < CG) {
#pragma unroll
          for (int j = 0; j < NRED; ++j) red[buf][wave][cg][j] = r[j];
        }
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NRED; ++j) {
          float sum = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) sum += red[buf][w][cg][j];
          r[j] = sum;
        }
      }
      const float ik = SSD ? 1.0f : rsqrtf(r[8] + p.eps);
      const float iq = SSD ? 1.0f : rsqrtf(r[9] + p.eps) * p.scale;
      const float qk = r[10] * ik * iq;
      const float g = SSD ? neg_exp_A * a_t : (KDA ? 0.0f : log_decay(neg_exp_A, a_t, dtb));
      const float alpha = KDA ? 1.0f : expf(g);  // KDA: rows already decayed
      const float beta = SSD ? a_t : sigmoid_f32(b_t);
      const float au = SSD ? 0.0f : alpha * ik;  // SSD: no erase
      float4 d;
      d.x = beta * (vv.x - au * r[0]);
      d.y = beta * (vv.y - au * r[1]);
      d.z = beta * (vv.z - au * r[2]);
      d.w = beta * (vv.w - au * r[3]);
      if (rg == 0) {
        const float aw = alpha * iq;
        float4 o;
        o.x = aw * r[4] + qk * d.x;
        o.y = aw * r[5] + qk * d.y;
        o.z = aw * r[6] + qk * d.z;
        o.w = aw * r[7] + qk * d.w;
        store4(p.o + (t * p.H_v + h) * DV + 4 * cg, o);
      }
#pragma unroll
      for (int i = 0; i < RPT; ++i) {
        const float kh = kv[i] * ik;
        S[i].x = alpha * S[i].x + kh * d.x;
        S[i].y = alpha * S[i].y + kh * d.y;
        S[i].z = alpha * S[i].z + kh * d.z;
        S[i].w = alpha * S[i].w + kh * d.w;
      }
    }
    if (p.sT) {
      float *dst = p.sT + state_at(u);
#pragma unroll
      for (int i = 0; i < RPT; ++i) nt_store4(dst + (size_t)(rg + RG * i) * DV, S[i]);
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) S[i] = Sn[i];
  }
}

// Compute units of the current device (queried once per device).
int cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

template <int DK, int DV, typename T, int MODE>
hipError_t launch_typed(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  RecParams<T> p;
  p.q = static_cast<const T *>(x.q);
  p.k = static_cast<const T *>(x.k);
  p.v = static_cast<const T *>(x.v);
  p.a = static_cast<const T *>(x.a);
  p.b = static_cast<const T *>(x.b);
  p.A_log = x.A_log;
  p.dt_bias = x.dt_bias;
  p.s0 = x.s0;
  p.o = static_cast<T *>(x.o);
  p.sT = x.sT;
  p.cu = pr.cu;
  p.seq_len = pr.seq_len;
  p.H_k = pr.H_k;
  p.H_v = pr.H_v;
  p.scale = pr.scale;
  p.eps = pr.eps;
  const int64_t units = (int64_t)pr.num_seqs * pr.H_v;
  if (units == 0) return hipSuccess;
  if (units > INT32_MAX) return hipErrorInvalidValue;
  p.units = (int)units;
  // persistent grid: about 16 waves per compute unit
  const int per_cu = RecGeom<DK, DV>::NW >= 8 ? 2 : 16 / RecGeom<DK, DV>::NW;
  const int64_t grid = units < (int64_t)cu_count() * per_cu ? units : (int64_t)cu_count() * per_cu;
  hipLaunchKernelGGL((recurrent_kernel<DK, DV, T, MODE>), dim3((unsigned)grid),
                     dim3(RecGeom<DK, DV>::NT), 0, s, p);
  return hipGetLastError();
}

template <int DK, typename T, int MODE>
hipError_t launch_dv(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  switch (pr.d_v) {
    case 16: return launch_typed<DK, 16, T, MODE>(pr, x, s);
    case 32: return launch_typed<DK, 32, T, MODE>(pr, x, s);
    case 64: return launch_typed<DK, 64, T, MODE>(pr, x, s);
    case 128: return launch_typed<DK, 128, T, MODE>(pr, x, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MODE>
hipError_t launch_dk(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  switch (pr.d_k) {
    case 16: return launch_dv<16, T, MODE>(pr, x, s);
    case 32: return launch_dv<32, T, MODE>(pr, x, s);
    case 64: return launch_dv<64, T, MODE>(pr, x, s);
    case 128: return launch_dv<128, T, MODE>(pr, x, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool recurrent_supports(const Problem &p) {
  auto ok = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; };
  return ok(p.d_k) && ok(p.d_v);
}

hipError_t launch_recurrent(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  const bool f = pr.dtype == GDR_F32;
  if (pr.mode == kModeSSD) return f ? launch_dk<float, kModeSSD>(pr, x, s) : launch_dk<bf16, kModeSSD>(pr, x, s);
  if (pr.mode == kModeKDA) return f ? launch_dk<float, kModeKDA>(pr, x, s) : launch_dk<bf16, kModeKDA>(pr, x, s);
  return f ? launch_dk<float, kModeRule>(pr, x, s) : launch_dk<bf16, kModeRule>(pr, x, s);
}

}  // namespace gdr
