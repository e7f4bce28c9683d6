// The steps either side of the rule (flashprove issue "P1: Qwen3.8-27B port,
// tracking": in_proj outputs -> 4-tap conv1d -> SiLU -> q/k L2 norm and gates
// -> rule -> gated RMSNorm; PLENA_Simulator pull request 113: the short
// convolution has per-channel weights, an optional bias and a history carried
// between calls).  Both are bound by HBM: every thread moves 16-byte vectors,
// consecutive threads consecutive channels, so each row is one coalesced
// sweep.
#include <cstdint>

#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

template <typename T>
struct Vec16 {
  static constexpr int N = 16 / sizeof(T);  // elements per 16-byte vector
};

template <typename T>
__device__ __forceinline__ void load_vec(const T *p, float (&v)[Vec16<T>::N]) {
  typedef T tv __attribute__((ext_vector_type(Vec16<T>::N)));
  const tv x = *reinterpret_cast<const tv *>(p);
#pragma unroll
  for (int i = 0; i < Vec16<T>::N; ++i) v[i] = to_f32(x[i]);
}
template <typename T>
__device__ __forceinline__ void store_vec(T *p, const float (&v)[Vec16<T>::N]) {
  typedef T tv __attribute__((ext_vector_type(Vec16<T>::N)));
  tv x;
#pragma unroll
  for (int i = 0; i < Vec16<T>::N; ++i) x[i] = from_f32<T>(v[i]);
  *reinterpret_cast<tv *>(p) = x;
}

// SiLU(x) = x / (1 + e^-x) from the hardware exp2 and reciprocal (each about
// 1 ulp): e^-x = 2^(-x log2 e).  Large negative x gives x * rcp(inf) = -0,
// large positive x gives x.
__device__ __forceinline__ float silu(float x) {
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// Sequence holding token t: the last n with cu[n] <= t (cu nondecreasing,
// t < cu[N]); empty sequences before it are skipped.
__device__ __forceinline__ int seq_of_token(const int32_t *cu, int seq_len, int num_seqs,
                                            int64_t t) {
  if (!cu) return (int)(t / seq_len);
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {  // smallest n with cu[n + 1] > t
    const int mid = (lo + hi) >> 1;
    if ((int64_t)cu[mid + 1] > t) hi = mid;
    else lo = mid + 1;
  }
  return lo;
}

struct ConvParams {
  const void *x;
  const float *w, *bias;
  const void *s_in;
  void *s_out;
  void *q, *k, *v;
  const int32_t *cu;
  int64_t total;
  int num_seqs, seq_len;
  int C, Cq, Ck, Cv;  // channels: all, q, k, v (q then k then v)
};

constexpr int CONV_THREADS = 256;
constexpr int CONV_TILE = 32;  // tokens per thread

// Convolution + SiLU of one 32-token tile for one 16-byte group of channels.
template <typename T, int W>
__global__ __launch_bounds__(CONV_THREADS) void conv_silu_kernel(ConvParams p) {
  constexpr int V = Vec16<T>::N;
  const int grp = blockIdx.x * CONV_THREADS + threadIdx.x;
  if (grp * V >= p.C) return;
  const int c0 = grp * V;
  const int64_t tb = (int64_t)blockIdx.y * CONV_TILE;
  const int64_t te = tb + CONV_TILE < p.total ? tb + CONV_TILE : p.total;
  const T *x = static_cast<const T *>(p.x);
  const T *s_in = static_cast<const T *>(p.s_in);

  // the V x W weights and V biases of these channels are contiguous: read
  // them as 16-byte vectors (c0 is a multiple of 4, so are V * W and V)
  float w[W][V], b[V];
  {
    const float4 *wp = reinterpret_cast<const float4 *>(p.w + (int64_t)c0 * W);
#pragma unroll
    for (int q = 0; q < V * W / 4; ++q) {
      const float4 f = wp[q];
      const float e[4] = {f.x, f.y, f.z, f.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) w[(4 * q + r) % W][(4 * q + r) / W] = e[r];
    }
#pragma unroll
    for (int q = 0; q < V / 4; ++q) {
      const float4 f = p.bias ? reinterpret_cast<const float4 *>(p.bias + c0)[q]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
      b[4 * q] = f.x; b[4 * q + 1] = f.y; b[4 * q + 2] = f.z; b[4 * q + 3] = f.w;
    }
  }
  // destination: the q, k or v part holding these channels
  T *dst;
  int ld, col;
  if (c0 < p.Cq) {
    dst = static_cast<T *>(p.q); ld = p.Cq; col = c0;
  } else if (c0 < p.Cq + p.Ck) {
    dst = static_cast<T *>(p.k); ld = p.Ck; col = c0 - p.Cq;
  } else {
    dst = static_cast<T *>(p.v); ld = p.Cv; col = c0 - p.Cq - p.Ck;
  }

  // win[j]: the input j + 1 steps before the current token
  float win[W - 1][V];
  int n = seq_of_token(p.cu, p.seq_len, p.num_seqs, tb);
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  // the window before token tb: inputs of the sequence, else its history
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int64_t src = tb - 1 - j;
    if (src >= t0) {
      load_vec(x + src * p.C + c0, win[j]);
    } else {
      const int64_t h = (W - 1) - (t0 - src);  // history entry, oldest first
#pragma unroll
      for (int i = 0; i < V; ++i)
        win[j][i] = s_in ? to_f32(s_in[((int64_t)n * p.C + c0 + i) * (W - 1) + h]) : 0.0f;
    }
  }
  // one output row from the input row xt; the window moves on by one
  auto row = [&](int64_t t, const float (&xt)[V]) {
    float y[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float acc = b[i] + w[W - 1][i] * xt[i];
#pragma unroll
      for (int j = 0; j < W - 1; ++j) acc += w[W - 2 - j][i] * win[j][i];
      y[i] = silu(acc);
    }
    store_vec(dst + t * ld + col, y);
#pragma unroll
    for (int j = W - 2; j > 0; --j)
#pragma unroll
      for (int i = 0; i < V; ++i) win[j][i] = win[j - 1][i];
#pragma unroll
    for (int i = 0; i < V; ++i) win[0][i] = xt[i];
  };
  // the tile in pieces that stay inside one sequence; within a piece the
  // rows go in groups of U whose loads are all issued before any is used
  // (16 rows of 16 bytes in flight per thread: with 4, at 64 tokens per
  // tile, the stream ran at 47% of HBM, now at about 60%)
  constexpr int U = 16;
  int64_t t = tb;
  while (t < te) {
    if (t >= t1) {  // a new sequence starts here (skipping empty ones)
      do {
        ++n;
        seq_bounds(p.cu, p.seq_len, n, t0, t1);
      } while (t >= t1);
#pragma unroll
      for (int j = 0; j < W - 1; ++j)
#pragma unroll
        for (int i = 0; i < V; ++i)
          win[j][i] = s_in ? to_f32(s_in[((int64_t)n * p.C + c0 + i) * (W - 1) + (W - 2 - j)]) : 0.0f;
    }
    const int64_t pe = te < t1 ? te : t1;  // end of this piece
    for (; t + U <= pe; t += U) {
      float xs[U][V];
#pragma unroll
      for (int u = 0; u < U; ++u) load_vec(x + (t + u) * p.C + c0, xs[u]);
#pragma unroll
      for (int u = 0; u < U; ++u) row(t + u, xs[u]);
    }
    for (; t < pe; ++t) {
      float xt[V];
      load_vec(x + t * p.C + c0, xt);
      row(t, xt);
    }
  }
}

// New history: the last W-1 inputs of each sequence, older history moving up
// when the sequence is shorter.  One thread per (sequence, channel); it reads
// all of its entries before writing any, so s_out may be s_in.
template <typename T, int W>
__global__ __launch_bounds__(CONV_THREADS) void conv_state_kernel(ConvParams p) {
  const int64_t id = (int64_t)blockIdx.x * CONV_THREADS + threadIdx.x;
  if (id >= (int64_t)p.num_seqs * p.C) return;
  const int n = (int)(id / p.C), c = (int)(id % p.C);
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const T *x = static_cast<const T *>(p.x);
  const T *s_in = static_cast<const T *>(p.s_in);
  T v[W - 1];
#pragma unroll
  for (int j = 0; j < W - 1; ++j) {
    const int64_t src = t1 - (W - 1) + j;
    if (src >= t0) v[j] = x[src * p.C + c];
    else v[j] = s_in ? s_in[id * (W - 1) + (W - 1) - (t0 - src)] : from_f32<T>(0.0f);
  }
  T *s_out = static_cast<T *>(p.s_out);
#pragma unroll
  for (int j = 0; j < W - 1; ++j) s_out[id * (W - 1) + j] = v[j];
}

template <typename T, int W>
hipError_t launch_conv_typed(const ConvParams &p, hipStream_t s) {
  constexpr int V = Vec16<T>::N;
  if (p.total > 0) {
    const int groups = p.C / V;
    const dim3 grid((groups + CONV_THREADS - 1) / CONV_THREADS,
                    (unsigned)((p.total + CONV_TILE - 1) / CONV_TILE));
    hipLaunchKernelGGL((conv_silu_kernel<T, W>), grid, dim3(CONV_THREADS), 0, s, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.s_out && p.num_seqs > 0) {
    const int64_t n = (int64_t)p.num_seqs * p.C;
    hipLaunchKernelGGL((conv_state_kernel<T, W>), dim3((unsigned)((n + CONV_THREADS - 1) / CONV_THREADS)),
                       dim3(CONV_THREADS), 0, s, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename T>
hipError_t launch_conv_width(const ConvParams &p, int width, hipStream_t s) {
  switch (width) {
    case 2: return launch_conv_typed<T, 2>(p, s);
    case 3: return launch_conv_typed<T, 3>(p, s);
    default: return launch_conv_typed<T, 4>(p, s);
  }
}

// ------------------------------------------------------------ gated RMSNorm
struct NormParams {
  const void *o, *z;
  const float *w;
  void *out;
  int64_t rows;  // tokens x value heads
  int d;
  float eps;
};

constexpr int NORM_THREADS = 256;

template <int CTRL>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// Sum over the tpr consecutive lanes holding one row (tpr a power of two, 2..32):
// swaps inside quads, then the mirror of each half row and of each row of 16
// lanes (every lane of the group already holds its group's sum), then the
// other row of 16 for 32.
__device__ __forceinline__ float row_sum(float s, int tpr) {
  if (tpr >= 2) s = dpp_add<0xB1>(s);   // quad_perm [1, 0, 3, 2]
  if (tpr >= 4) s = dpp_add<0x4E>(s);   // quad_perm [2, 3, 0, 1]
  if (tpr >= 8) s = dpp_add<0x141>(s);  // row_half_mirror
  if (tpr >= 16) s = dpp_add<0x140>(s); // row_mirror
  if (tpr >= 32) s += __shfl_xor(s, 16);
  return s;
}

// Each row of d elements is held by tpr = d / V consecutive lanes; a thread
// holds its part of two rows, NORM_ROWS apart in the grid, so that four
// 16-byte loads are in flight before the first use.
constexpr int NORM_ROWS = 2;
template <typename T>
__global__ __launch_bounds__(NORM_THREADS) void gated_rmsnorm_kernel(NormParams p) {
  constexpr int V = Vec16<T>::N;
  const int tpr = p.d / V;
  const int64_t gid = (int64_t)blockIdx.x * NORM_THREADS + threadIdx.x;
  const int64_t half = (int64_t)gridDim.x * NORM_THREADS / tpr;  // rows per pass
  const int part = (int)(gid % tpr);
  float wv[V];
#pragma unroll
  for (int i = 0; i < V; ++i) wv[i] = p.w[part * V + i];
  float o[NORM_ROWS][V], z[NORM_ROWS][V], ss[NORM_ROWS];
  int64_t off[NORM_ROWS];
  bool live[NORM_ROWS];
#pragma unroll
  for (int k = 0; k < NORM_ROWS; ++k) {
    const int64_t row = gid / tpr + k * half;
    live[k] = row < p.rows;
    off[k] = row * p.d + (int64_t)part * V;
    ss[k] = 0.0f;
    if (live[k]) {
      load_vec(static_cast<const T *>(p.o) + off[k], o[k]);
      load_vec(static_cast<const T *>(p.z) + off[k], z[k]);
    }
  }
#pragma unroll
  for (int k = 0; k < NORM_ROWS; ++k) {
    if (live[k]) {
#pragma unroll
      for (int i = 0; i < V; ++i) ss[k] += o[k][i] * o[k][i];
    }
    ss[k] = row_sum(ss[k], tpr);
  }
#pragma unroll
  for (int k = 0; k < NORM_ROWS; ++k) {
    if (!live[k]) continue;
    const float r = rsqrtf(ss[k] / (float)p.d + p.eps);
    float y[V];
#pragma unroll
    for (int i = 0; i < V; ++i) y[i] = o[k][i] * r * wv[i] * silu(z[k][i]);
    store_vec(static_cast<T *>(p.out) + off[k], y);
  }
}

// y <- y * SiLU(z), elementwise over n 16-byte vectors.
template <typename T>
__global__ __launch_bounds__(NORM_THREADS) void silu_gate_kernel(T *y, const T *z, int64_t nvec) {
  constexpr int V = Vec16<T>::N;
  for (int64_t i = (int64_t)blockIdx.x * NORM_THREADS + threadIdx.x; i < nvec;
       i += (int64_t)gridDim.x * NORM_THREADS) {
    float a[V], g[V];
    load_vec(y + i * V, a);
    load_vec(z + i * V, g);
#pragma unroll
    for (int k = 0; k < V; ++k) a[k] *= silu(g[k]);
    store_vec(y + i * V, a);
  }
}

}  // namespace

hipError_t launch_silu_gate(const Problem &pr, void *y, const void *z, hipStream_t s) {
  const int V = pr.dtype == GDR_F32 ? 4 : 8;
  const int64_t nvec = pr.total * pr.H_v * pr.d_v / V;
  if (nvec == 0) return hipSuccess;
  int64_t blocks = (nvec + NORM_THREADS - 1) / NORM_THREADS;
  if (blocks > 8192) blocks = 8192;
  if (pr.dtype == GDR_F32)
    hipLaunchKernelGGL(silu_gate_kernel<float>, dim3((unsigned)blocks), dim3(NORM_THREADS), 0, s,
                       static_cast<float *>(y), static_cast<const float *>(z), nvec);
  else
    hipLaunchKernelGGL(silu_gate_kernel<bf16>, dim3((unsigned)blocks), dim3(NORM_THREADS), 0, s,
                       static_cast<bf16 *>(y), static_cast<const bf16 *>(z), nvec);
  return hipGetLastError();
}

hipError_t launch_conv_silu(const Problem &pr, const ConvArgs &a, hipStream_t s) {
  ConvParams p;
  p.x = a.x;
  p.w = a.weight;
  p.bias = a.bias;
  p.s_in = a.s_in;
  p.s_out = a.s_out;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.cu = pr.cu;
  p.total = pr.total;
  p.num_seqs = pr.num_seqs;
  p.seq_len = pr.seq_len;
  p.Cq = pr.H_k * pr.d_k;
  p.Ck = pr.H_k * pr.d_k;
  p.Cv = pr.H_v * pr.d_v;
  p.C = p.Cq + p.Ck + p.Cv;
  return pr.dtype == GDR_F32 ? launch_conv_width<float>(p, a.width, s)
                             : launch_conv_width<bf16>(p, a.width, s);
}

hipError_t launch_gated_rmsnorm(const Problem &pr, const NormArgs &a, hipStream_t s) {
  NormParams p;
  p.o = a.o;
  p.z = a.z;
  p.w = a.weight;
  p.out = a.out;
  p.rows = pr.total * pr.H_v;
  p.d = pr.d_v;
  p.eps = a.eps;
  if (p.rows == 0) return hipSuccess;
  const int V = pr.dtype == GDR_F32 ? 4 : 8;
  // NORM_ROWS passes over the rows: each thread takes one row part per pass
  const int64_t threads = (p.rows + NORM_ROWS - 1) / NORM_ROWS * (p.d / V);
  const dim3 grid((unsigned)((threads + NORM_THREADS - 1) / NORM_THREADS));
  if (pr.dtype == GDR_F32)
    hipLaunchKernelGGL(gated_rmsnorm_kernel<float>, grid, dim3(NORM_THREADS), 0, s, p);
  else
    hipLaunchKernelGGL(gated_rmsnorm_kernel<bf16>, grid, dim3(NORM_THREADS), 0, s, p);
  return hipGetLastError();
}

}  // namespace gdr
