// Chunked form with each sequence cut into segments that run in parallel: a
// two-level scan (Track L pull request, L2 and its unbuilt cooperative-parallel
// chunk kernel).  The state update of every token is affine in the state,
// S <- alpha (I - beta k k^T) S + beta k v^T, so over a segment
//     S_out = M S_in + S_loc,
// with M the segment run from S_in = I on v = 0 (d_k = d_v) and S_loc the run
// from S_in = 0 on the real v.  The segments' M and S_loc come from two
// chunked launches over all segments at once; a short sequential pass gives
// every segment its entry state, S_in(p+1) = M_p S_in(p) + S_loc,p; a third
// chunked launch from those entry states writes the outputs.
#include <cstdint>

#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

constexpr int FILL_THREADS = 256;

// dst[i] = 0 for i < n 32-bit words.
__global__ __launch_bounds__(FILL_THREADS) void zero_words_kernel(uint32_t *dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * FILL_THREADS)
    dst[i] = 0u;
}

// count identity matrices of size d x d (fp32).
__global__ __launch_bounds__(FILL_THREADS) void identity_kernel(float *dst, int64_t count, int d) {
  const int64_t n = count * d * d;
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * FILL_THREADS) {
    const int64_t e = i % ((int64_t)d * d);
    dst[i] = (e / d == e % d) ? 1.0f : 0.0f;
  }
}

// Entry states of the segments of one (sequence, value head), 4 columns per
// workgroup:  S_in(0) = S0 (or 0),  S_in(p+1) = M_p S_in(p) + S_loc,p.
// The workgroup keeps its 4 columns of S_in in LDS.  Thread (r, half) holds
// half of row r of M_p in registers, columns 64 half .. (D/2 of them), and the
// same half of M_{p+1} is loaded while segment p is contracted; each thread
// sums its half over the 4 columns, and the two halves of a row (adjacent
// lanes) add up by a lane exchange.  M never passes through LDS, so a step is
// one register-resident contraction of D/2 x 4 and a barrier, and D/4 * (N H)
// workgroups share the work.
constexpr int COMB_COLS = 4;

struct CombParams {
  const float *s0;    // [N, H, D, D] or nullptr
  const float *M;     // [N * P, H, D, D]
  const float *Sloc;  // [N * P, H, D, D]
  float *Sin;         // [N * P, H, D, D]
  int N, P, H;
};

template <int D>
__global__ __launch_bounds__(2 * D) void combine_kernel(CombParams p) {
  constexpr int HALF = D / 2;        // contraction columns per thread
  constexpr int NF4 = HALF / 4;      // float4 of M per thread
  __shared__ __align__(16) float Sb[2][D][COMB_COLS];  // S_in columns, double-buffered
  const int nh = blockIdx.x;                          // n * H + h
  const int n = nh / p.H, h = nh % p.H;
  const int c0 = blockIdx.y * COMB_COLS;
  const int tid = threadIdx.x;
  const int r = tid >> 1, half = tid & 1;
  const int j0 = HALF * half;
  constexpr size_t MAT = (size_t)D * D;
  auto at = [&](int seg) { return ((size_t)(n * p.P + seg) * p.H + h) * MAT; };

  float4 mc[NF4], mn[NF4];
  float lc[2] = {0.f, 0.f}, ln[2] = {0.f, 0.f};  // S_loc[r][c0 + 2 half + 0..1]
  auto fetch = [&](int seg, float4 (&m)[NF4], float (&l)[2]) {
    const float4 *M4 = reinterpret_cast<const float4 *>(p.M + at(seg) + (size_t)r * D + j0);
#pragma unroll
    for (int f = 0; f < NF4; ++f) m[f] = M4[f];
    const float *L = p.Sloc + at(seg) + (size_t)r * D + c0 + 2 * half;
    l[0] = L[0];
    l[1] = L[1];
  };

  // S_in(0): thread (r, half) owns columns c0 + 2 half, +1 of row r
#pragma unroll
  for (int c = 0; c < 2; ++c)
    Sb[0][r][2 * half + c] =
        p.s0 ? p.s0[((size_t)n * p.H + h) * MAT + (size_t)r * D + c0 + 2 * half + c] : 0.0f;
  if (p.P > 1) fetch(0, mc, lc);
  __syncthreads();
  for (int seg = 0;; ++seg) {
    const int cur = seg & 1;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      p.Sin[at(seg) + (size_t)r * D + c0 + 2 * half + c] = Sb[cur][r][2 * half + c];
    if (seg + 1 == p.P) break;
    if (seg + 2 < p.P) fetch(seg + 1, mn, ln);  // in flight during this contraction
    float acc[COMB_COLS] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < NF4; ++f) {
      const float mv[4] = {mc[f].x, mc[f].y, mc[f].z, mc[f].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 sv = *reinterpret_cast<const float4 *>(&Sb[cur][j0 + 4 * f + e][0]);
        acc[0] += mv[e] * sv.x;
        acc[1] += mv[e] * sv.y;
        acc[2] += mv[e] * sv.z;
        acc[3] += mv[e] * sv.w;
      }
    }
#pragma unroll
    for (int c = 0; c < COMB_COLS; ++c) acc[c] += __shfl_xor(acc[c], 1, 64);
    // the other buffer was last read a step ago, behind the previous barrier
    Sb[cur ^ 1][r][2 * half] = acc[2 * half] + lc[0];
    Sb[cur ^ 1][r][2 * half + 1] = acc[2 * half + 1] + lc[1];
#pragma unroll
    for (int f = 0; f < NF4; ++f) mc[f] = mn[f];
    lc[0] = ln[0];
    lc[1] = ln[1];
    __syncthreads();
  }
}

// final_state[n] = Sout[n * P + P - 1] for every sequence (float4 copies).
__global__ __launch_bounds__(FILL_THREADS) void last_state_kernel(const float *Sout, float *out,
                                                                  int N, int P, int64_t per_seq) {
  const int64_t q4 = per_seq / 4;
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < (int64_t)N * q4;
       i += (int64_t)gridDim.x * FILL_THREADS) {
    const int64_t n = i / q4, e = i % q4;
    reinterpret_cast<float4 *>(out)[i] =
        reinterpret_cast<const float4 *>(Sout + ((int64_t)n * P + P - 1) * per_seq)[e];
  }
}

hipError_t chunked_any(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  if (pr.mode == kModeKDA)
    return chunked_kda_supports(pr) ? launch_chunked_kda(pr, x, s) : launch_chunked_vec(pr, x, s);
  if (chunked_mfma_supports(pr)) return launch_chunked_mfma(pr, x, s);
  return launch_chunked_vec(pr, x, s);
}

size_t round256(size_t b) { return (b + 255) & ~(size_t)255; }

template <int D>
hipError_t launch_combine(const CombParams &cp, hipStream_t s) {
  hipLaunchKernelGGL(combine_kernel<D>, dim3(cp.N * cp.H, D / COMB_COLS), dim3(2 * D), 0, s, cp);
  return hipGetLastError();
}

unsigned fill_blocks(int64_t n) {
  const int64_t b = (n + FILL_THREADS - 1) / FILL_THREADS;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

// The segments of a dense batch as a dense batch of num_seqs * P sequences.
Problem segments(const Problem &pr, int segment_len) {
  Problem seg = pr;
  seg.num_seqs = pr.num_seqs * (pr.seq_len / segment_len);
  seg.seq_len = segment_len;
  seg.cu = nullptr;
  return seg;
}

SplitLayout split_layout(const Problem &pr, int segment_len) {
  SplitLayout L;
  const size_t es = pr.dtype == GDR_F32 ? 4 : 2;
  L.P = pr.seq_len / segment_len;
  const size_t NP = (size_t)pr.num_seqs * L.P;
  const size_t st = NP * pr.H_v * pr.d_k * pr.d_v * 4;
  L.zero_v = 0;
  L.ident = L.zero_v + round256((size_t)pr.total * pr.H_v * pr.d_k * es);
  L.M = L.ident + round256(st);
  L.Sloc = L.M + round256(st);
  L.Sin = L.Sloc + round256(st);
  L.prep = L.Sin + round256(st);
  L.bytes = L.prep + round256(kda_two_pass_bytes(segments(pr, segment_len)));
  return L;
}

hipError_t launch_chunked_split(const Problem &pr, const FwdArgs &x, int segment_len,
                                void *workspace, hipStream_t s) {
  const SplitLayout L = split_layout(pr, segment_len);
  char *ws = static_cast<char *>(workspace);
  void *zero_v = ws + L.zero_v;
  float *ident = reinterpret_cast<float *>(ws + L.ident);  // later the segments' final states
  float *M = reinterpret_cast<float *>(ws + L.M);
  float *Sloc = reinterpret_cast<float *>(ws + L.Sloc);
  float *Sin = reinterpret_cast<float *>(ws + L.Sin);
  const int NP = pr.num_seqs * L.P;
  const size_t es = pr.dtype == GDR_F32 ? 4 : 2;
  const int64_t vwords = (int64_t)((size_t)pr.total * pr.H_v * pr.d_k * es / 4);
  hipLaunchKernelGGL(zero_words_kernel, dim3(fill_blocks(vwords)), dim3(FILL_THREADS), 0, s,
                     static_cast<uint32_t *>(zero_v), vwords);
  const int64_t idn = (int64_t)NP * pr.H_v * pr.d_k * pr.d_k;
  hipLaunchKernelGGL(identity_kernel, dim3(fill_blocks(idn)), dim3(FILL_THREADS), 0, s, ident,
                     (int64_t)NP * pr.H_v, pr.d_k);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // the segments as a dense batch of NP sequences
  const Problem seg = segments(pr, segment_len);
  // KDA on the two-launch form: the per-chunk prep depends on q, k, a, b only,
  // so one prep serves the three chain launches below
  void *prep = ws + L.prep;
  const bool two = L.bytes > L.prep;
  if (two && (e = launch_kda_prep(seg, x, prep, s)) != hipSuccess) return e;
  auto chunked = [&](const FwdArgs &y) {
    return two ? launch_kda_chain(seg, y, prep, s) : chunked_any(seg, y, s);
  };
  // S_loc: from zero on the real v;  M: from I on v = 0  (outputs land in o and
  // are overwritten by the last launch)
  FwdArgs a = x;
  a.s0 = nullptr;
  a.sT = Sloc;
  if ((e = chunked(a)) != hipSuccess) return e;
  FwdArgs b = x;
  b.v = zero_v;
  b.s0 = ident;
  b.sT = M;
  if ((e = chunked(b)) != hipSuccess) return e;

  CombParams cp{x.s0, M, Sloc, Sin, pr.num_seqs, L.P, pr.H_v};
  switch (pr.d_k) {
    case 16: e = launch_combine<16>(cp, s); break;
    case 32: e = launch_combine<32>(cp, s); break;
    case 64: e = launch_combine<64>(cp, s); break;
    default: e = launch_combine<128>(cp, s); break;
  }
  if (e != hipSuccess) return e;

  // outputs from the right entry states; the segments' final states reuse
  // the identity buffer, and the last of each sequence is the final state
  FwdArgs c = x;
  c.s0 = Sin;
  c.sT = x.sT ? ident : nullptr;
  if ((e = chunked(c)) != hipSuccess) return e;
  if (x.sT) {
    const int64_t per_seq = (int64_t)pr.H_v * pr.d_k * pr.d_v;
    hipLaunchKernelGGL(last_state_kernel, dim3(fill_blocks((int64_t)pr.num_seqs * per_seq / 4)),
                       dim3(FILL_THREADS), 0, s, ident, x.sT, pr.num_seqs, L.P, per_seq);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdr
