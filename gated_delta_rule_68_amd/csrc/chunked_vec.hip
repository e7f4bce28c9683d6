// Chunked (UT-transform) form of the gated delta rule on the vector ALUs, in
// fp32 throughout.  Serves every supported shape; the matrix-core kernels
// take over bf16 inputs at d_k = d_v = 128, chunk 32 (chunked_mfma.hip) and
// fp32 inputs of the rule at d_k = 64 or 128, chunk 32 (chunked_f32mma.hip).
//
// The regrouping (GatedDeltaRule.ixx File Reference, "Detailed Description":
// one triangular solve per chunk, same arithmetic as the recurrence; Track L
// pull request, L2: the only non-GEMM step is the (I + A)^-1 forward
// substitution).  For one chunk of c tokens with state S at entry, gamma_r the
// in-chunk cumulative log decay (r = 0..c-1) and Gamma_r = exp(gamma_r):
//   A[r][i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)   i < r
//   T       = (I + A)^-1                                    (forward substitution)
//   R       = diag(beta) (V - diag(Gamma) K S)
//   Delta   = T R                                           (the rows are the deltas)
//   P[r][i] = exp(gamma_r - gamma_i) (q_r . k_i)            i <= r
//   O       = diag(Gamma) Q S + P Delta
//   S'      = Gamma_{c-1} S + (diag(exp(gamma_{c-1} - gamma)) K)^T Delta
// Only differences gamma_r - gamma_i with i <= r are exponentiated, so every
// factor is at most 1 (exp(-gamma_i) alone overflows under strong decay).
// A partial last chunk is padded with rows that have k = q = v = 0, g = 0 and
// beta = 0: they add nothing to any sum and leave gamma unchanged.
//
// Launch: one 256-thread workgroup per (sequence, value head, 16-column block
// of d_v); the columns of S evolve independently, so each workgroup carries
// its [d_k, 16] slice of the state in LDS across the sequential chunk loop.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int kVecThreads = 256;
constexpr int kBV = 16;

template <typename T>
struct VecParams {
  const T *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  const float *s0;
  T *o;
  float *sT;
  const int32_t *cu;
  int seq_len;
  int H_k, H_v, d_v;
  float scale, eps;
};

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

template <int DK, int C, bool KDA>
struct VecSmem {
  float K[C][DK + 1];
  float Q[C][DK + 1];
  float S[DK][kBV];
  float V[C][kBV];
  float A[C][C + 1];
  float P[C][C + 1];
  float Tm[C][C + 1];
  float KS[C][kBV];
  float QS[C][kBV];
  float R[C][kBV];
  float D[C][kBV];
  float gam[C];
  float beta[C];
  float eg[C];    // exp(gamma_r)
  float tail[C];  // exp(gamma_{c-1} - gamma_r)
  // KDA: per-channel cumulative log decays, and exp of them (after the Gram
  // stage, the rows of K weighted by exp(gamma_{c-1} - gamma_r) per channel)
  float G[KDA ? C : 1][DK + 1];
  float EG[KDA ? C : 1][DK + 1];
};

// MODE kModeSSD: the Mamba-2 SSD recurrence on the same chunk scan: no
// norms, no erase (A = 0, so T = I and Delta = diag(beta) V without K S),
// g = A delta with delta in `a` and A in `A_log`, beta = delta.
// MODE kModeKDA: one decay per key channel.  gamma becomes gamma[r][c] and
// every exp(gamma_r - gamma_i) moves inside the channel sums:
//   A[r][i] = beta_r sum_c k_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])   (i < r)
//   P[r][i] = sum_c q_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])          (i <= r)
//   K S and Q S take the rows weighted by exp(gamma_r[c]);
//   S'[c] = exp(gamma_{c-1}[c]) S[c] + sum_r k_r[c] exp(gamma_{c-1}[c] - gamma_r[c]) Delta_r
// and again only differences with i <= r are exponentiated.
template <int DK, int C, typename T, int MODE>
__global__ __launch_bounds__(kVecThreads) void chunked_vec_kernel(VecParams<T> p) {
  constexpr bool SSD = MODE == kModeSSD, KDA = MODE == kModeKDA;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  VecSmem<DK, C, KDA> &sm = *reinterpret_cast<VecSmem<DK, C, KDA> *>(smem_raw);
  constexpr int E = (DK + 63) / 64;
  const int nvb = p.d_v / kBV;
  const int vb = blockIdx.x % nvb;
  const int h = (blockIdx.x / nvb) % p.H_v;
  const int n = blockIdx.x / (nvb * p.H_v);
  const int hk = h / (p.H_v / p.H_k);
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const int DV = p.d_v;

  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const size_t state_off = ((size_t)n * p.H_v + h) * DK * DV + (size_t)vb * kBV;
  for (int e = tid; e < DK * kBV; e += kVecThreads) {
    const int d = e / kBV, j = e % kBV;
    sm.S[d][j] = p.s0 ? p.s0[state_off + (size_t)d * DV + j] : 0.0f;
  }
  const float neg_exp_A = SSD ? p.A_log[h] : -expf(p.A_log[h]);  // SSD: A itself
  const float dtb = (SSD || KDA) ? 0.0f : p.dt_bias[h];

  for (int64_t c0 = t0; c0 < t1; c0 += C) {
    const int cl = (int)((t1 - c0) < C ? (t1 - c0) : C);
    // -- stage 1: normalised K and Q rows, the V block, gates
    for (int r2 = wave; r2 < 2 * C; r2 += kVecThreads / 64) {
      const bool is_q = r2 >= C;
      const int r = is_q ? r2 - C : r2;
      float x[E];
      float ss = 0.f;
      const T *src = (is_q ? p.q : p.k) + ((c0 + r) * p.H_k + hk) * DK;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = lane + 64 * e;
        x[e] = (r < cl && i < DK) ? to_f32(src[i]) : 0.f;
        ss += x[e] * x[e];
      }
      ss = wave_sum(ss);
      const float inv = (r < cl) ? (SSD ? 1.0f : rsqrtf(ss + p.eps) * (is_q ? p.scale : 1.0f)) : 0.f;
      float *dst = is_q ? sm.Q[r] : sm.K[r];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int i = lane + 64 * e;
        if (i < DK) dst[i] = x[e] * inv;
      }
    }
    for (int e = tid; e < C * kBV; e += kVecThreads) {
      const int r = e / kBV, j = e % kBV;
      sm.V[r][j] = (r < cl) ? to_f32(p.v[((c0 + r) * p.H_v + h) * DV + vb * kBV + j]) : 0.f;
    }
    if (tid < C) {
      const int r = tid;
      float g = 0.f, bt = 0.f;
      if (r < cl) {
        const float a_r = KDA ? 0.0f : to_f32(p.a[(c0 + r) * p.H_v + h]);
        if constexpr (KDA) {  // the decays are per channel, below
          bt = sigmoid_f32(to_f32(p.b[(c0 + r) * p.H_v + h]));
        } else if constexpr (SSD) {
          g = neg_exp_A * a_r;
          bt = a_r;
        } else {
          g = log_decay(neg_exp_A, a_r, dtb);
          bt = sigmoid_f32(to_f32(p.b[(c0 + r) * p.H_v + h]));
        }
      }
      sm.gam[r] = g;
      sm.beta[r] = bt;
    }
    if constexpr (KDA) {
      for (int e = tid; e < C * DK; e += kVecThreads) {
        const int r = e / DK, c = e % DK;
        sm.G[r][c] = (r < cl) ? log_decay(neg_exp_A,
                                          to_f32(p.a[((c0 + r) * p.H_v + h) * DK + c]),
                                          p.dt_bias[h * DK + c])
                              : 0.f;
      }
    }
    __syncthreads();
    if constexpr (KDA) {  // cumulative over the chunk, one channel per thread
      for (int c = tid; c < DK; c += kVecThreads) {
        float acc = 0.f;
        for (int r = 0; r < C; ++r) {
          acc += sm.G[r][c];
          sm.G[r][c] = acc;
          sm.EG[r][c] = expf(acc);
        }
      }
    }
    if (tid == 0) {
      float acc = 0.f;
      for (int r = 0; r < C; ++r) {
        acc += sm.gam[r];
        sm.gam[r] = acc;
      }
    }
    __syncthreads();
    if (tid < C) {
      sm.eg[tid] = expf(sm.gam[tid]);
      sm.tail[tid] = expf(sm.gam[C - 1] - sm.gam[tid]);
    }
    // -- stage 2: A, P and the state products K S, Q S
    for (int e = tid; e < C * C; e += kVecThreads) {
      const int r = e / C, i = e % C;
      float a_ri = 0.f, p_ri = 0.f;
      if (i <= r) {
        float kk = 0.f, qk = 0.f;
#pragma unroll 8
        for (int d = 0; d < DK; ++d) {
          // KDA: the decay of each channel inside the sum
          const float w = KDA ? expf(sm.G[r][d] - sm.G[i][d]) : 1.0f;
          if constexpr (!SSD) kk += sm.K[r][d] * sm.K[i][d] * w;
          qk += sm.Q[r][d] * sm.K[i][d] * w;
        }
        const float dec = expf(sm.gam[r] - sm.gam[i]);
        p_ri = dec * qk;
        if (!SSD && i < r) a_ri = sm.beta[r] * dec * kk;
      }
      sm.A[r][i] = a_ri;
      sm.P[r][i] = p_ri;
    }
    for (int e = tid; e < C * kBV; e += kVecThreads) {
      const int r = e / kBV, j = e % kBV;
      float ks = 0.f, qs = 0.f;
#pragma unroll 8
      for (int d = 0; d < DK; ++d) {
        const float w = KDA ? sm.EG[r][d] : 1.0f;
        if constexpr (!SSD) ks += sm.K[r][d] * w * sm.S[d][j];
        qs += sm.Q[r][d] * w * sm.S[d][j];
      }
      sm.KS[r][j] = ks;
      sm.QS[r][j] = qs;
    }
    __syncthreads();
    // -- stage 3: T = (I + A)^-1, one column per thread; R = beta (V - Gamma K S)
    //    (SSD: no erase, Delta = beta V straight away)
    if constexpr (SSD) {
      for (int e = tid; e < C * kBV; e += kVecThreads) {
        const int r = e / kBV, j = e % kBV;
        sm.D[r][j] = sm.beta[r] * sm.V[r][j];
      }
      __syncthreads();
    }
    if (!SSD && tid < C) {
      const int j = tid;
      float x[C];
#pragma unroll
      for (int r = 0; r < C; ++r) {
        float s = (r == j) ? 1.0f : 0.0f;
#pragma unroll
        for (int i = 0; i < r; ++i) s -= sm.A[r][i] * x[i];
        x[r] = s;
      }
#pragma unroll
      for (int r = 0; r < C; ++r) sm.Tm[r][j] = x[r];
    }
    if constexpr (KDA) {  // EG is free now: K weighted for the state update
      for (int e = tid; e < C * DK; e += kVecThreads) {
        const int r = e / DK, c = e % DK;
        sm.EG[r][c] = sm.K[r][c] * expf(sm.G[C - 1][c] - sm.G[r][c]);
      }
    }
    if constexpr (!SSD) {
      for (int e = tid; e < C * kBV; e += kVecThreads) {
        const int r = e / kBV, j = e % kBV;
        sm.R[r][j] = sm.beta[r] * (sm.V[r][j] - sm.eg[r] * sm.KS[r][j]);
      }
      __syncthreads();
      // -- stage 4: Delta = T R
      for (int e = tid; e < C * kBV; e += kVecThreads) {
        const int r = e / kBV, j = e % kBV;
        float s = 0.f;
        for (int i = 0; i <= r; ++i) s += sm.Tm[r][i] * sm.R[i][j];
        sm.D[r][j] = s;
      }
      __syncthreads();
    }
    // -- stage 5: O = Gamma Q S + P Delta; S' = Gamma_c S + (tail K)^T Delta
    for (int e = tid; e < C * kBV; e += kVecThreads) {
      const int r = e / kBV, j = e % kBV;
      if (r < cl) {
        float s = sm.eg[r] * sm.QS[r][j];
        for (int i = 0; i <= r; ++i) s += sm.P[r][i] * sm.D[i][j];
        p.o[((c0 + r) * p.H_v + h) * DV + vb * kBV + j] = from_f32<T>(s);
      }
    }
    const float gc = sm.eg[C - 1];
    for (int e = tid; e < DK * kBV; e += kVecThreads) {
      const int d = e / kBV, j = e % kBV;
      if constexpr (KDA) {
        float s = expf(sm.G[C - 1][d]) * sm.S[d][j];
#pragma unroll 8
        for (int r = 0; r < C; ++r) s += sm.EG[r][d] * sm.D[r][j];
        sm.S[d][j] = s;
      } else {
        float s = gc * sm.S[d][j];
#pragma unroll 8
        for (int r = 0; r < C; ++r) s += sm.tail[r] * sm.K[r][d] * sm.D[r][j];
        sm.S[d][j] = s;
      }
    }
    __syncthreads();
  }
  if (p.sT) {
    for (int e = tid; e < DK * kBV; e += kVecThreads) {
      const int d = e / kBV, j = e % kBV;
      p.sT[state_off + (size_t)d * DV + j] = sm.S[d][j];
    }
  }
}

template <int DK, int C, typename T, int MODE>
hipError_t launch_typed(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  VecParams<T> p;
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
  p.d_v = pr.d_v;
  p.scale = pr.scale;
  p.eps = pr.eps;
  const int64_t grid = (int64_t)pr.num_seqs * pr.H_v * (pr.d_v / kBV);
  if (grid == 0) return hipSuccess;
  const size_t smem = sizeof(VecSmem<DK, C, MODE == kModeKDA>);
  auto kern = chunked_vec_kernel<DK, C, T, MODE>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kVecThreads), smem, s, p);
  return hipGetLastError();
}

template <int DK, typename T, int MODE>
hipError_t launch_c(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  switch (pr.chunk) {
    case 16: return launch_typed<DK, 16, T, MODE>(pr, x, s);
    case 32: return launch_typed<DK, 32, T, MODE>(pr, x, s);
    case 64:
      if constexpr (MODE == kModeKDA) return hipErrorInvalidValue;  // LDS: see chunked_vec_supports
      else return launch_typed<DK, 64, T, MODE>(pr, x, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MODE>
hipError_t launch_dk(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  switch (pr.d_k) {
    case 16: return launch_c<16, T, MODE>(pr, x, s);
    case 32: return launch_c<32, T, MODE>(pr, x, s);
    case 64: return launch_c<64, T, MODE>(pr, x, s);
    case 128: return launch_c<128, T, MODE>(pr, x, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool chunked_vec_supports(const Problem &p) {
  auto ok = [](int d) { return d == 16 || d == 32 || d == 64 || d == 128; };
  // KDA keeps two more [chunk, d_k] tiles in LDS: chunk 64 would not fit
  return ok(p.d_k) && ok(p.d_v) &&
         (p.chunk == 16 || p.chunk == 32 || (p.chunk == 64 && p.mode != kModeKDA));
}

hipError_t launch_chunked_vec(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  const bool f = pr.dtype == GDR_F32;
  if (chunked_f32mma_supports(pr)) return launch_chunked_f32mma(pr, x, s);
  if (pr.mode == kModeSSD) return f ? launch_dk<float, kModeSSD>(pr, x, s) : launch_dk<bf16, kModeSSD>(pr, x, s);
  if (pr.mode == kModeKDA) return f ? launch_dk<float, kModeKDA>(pr, x, s) : launch_dk<bf16, kModeKDA>(pr, x, s);
  return f ? launch_dk<float, kModeRule>(pr, x, s) : launch_dk<bf16, kModeRule>(pr, x, s);
}

}  // namespace gdr
