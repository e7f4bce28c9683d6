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

// Segment map of a packed batch, on the device (the lengths never reach the
// host): sequence n of length L_n = cu[n+1] - cu[n] gets P_n = max(1,
// ceil(L_n / seg)) segments, numbered from off[n] = P_0 + .. + P_{n-1}; the
// segments' prefix sums are segcu[off[n] + p] = cu[n] + p seg, and the slots
// past off[N] (at most NP in all: P_n <= L_n / seg + 1) are empty segments at
// the end of the batch.  One workgroup: thread t sums the P_n of a contiguous
// range of sequences, a scan over the threads' sums gives every range its
// first segment, and each thread then writes its range.  A sequence of no
// tokens keeps one empty segment, so its final state is its initial one.
constexpr int MAP_THREADS = 256;

__global__ __launch_bounds__(MAP_THREADS) void segment_map_kernel(const int32_t *cu, int N,
                                                                  int seg, int NP,
                                                                  int32_t *segcu, int32_t *off) {
  __shared__ int32_t part[MAP_THREADS + 1];
  const int t = threadIdx.x;
  const int per = (N + MAP_THREADS - 1) / MAP_THREADS;
  const int n0 = min(t * per, N), n1 = min(n0 + per, N);
  auto count = [&](int n) {
    const int32_t len = max(cu[n + 1] - cu[n], 0);
    return max(1, (len + seg - 1) / seg);
  };
  int32_t sum = 0;
  for (int n = n0; n < n1; ++n) sum += count(n);
  part[t + 1] = sum;
  if (t == 0) part[0] = 0;
  __syncthreads();
  if (t == 0)
    for (int i = 1; i <= MAP_THREADS; ++i) part[i] += part[i - 1];
  __syncthreads();
  int32_t o = part[t];
  for (int n = n0; n < n1; ++n) {
    const int P = count(n);
    off[n] = o;
    for (int q = 0; q < P; ++q)
      if (o + q <= NP) segcu[o + q] = cu[n] + q * seg;
    o += P;
  }
  if (t == 0) off[N] = part[MAP_THREADS];
  // empty segments after the last sequence, and the closing prefix sum
  const int32_t tail = cu[N];
  for (int j = part[MAP_THREADS] + t; j <= NP; j += MAP_THREADS) segcu[j] = tail;
}

// Entry states of the segments of one (sequence, value head), 4 columns per
// workgroup:  S_in(0) = S0 (or 0),  S_in(p+1) = M_p S_in(p) + S_loc,p, with
// M_p [D x D] (D = d_k) and the states [D x dv].  The workgroup keeps its 4
// columns of S_in in LDS.  Thread (r, half) holds half of row r of M_p in
// registers, columns 64 half .. (D/2 of them), and the same half of M_{p+1}
// is loaded while segment p is contracted; each thread sums its half over the
// 4 columns, and the two halves of a row (adjacent lanes) add up by a lane
// exchange.  M never passes through LDS, so a step is one register-resident
// contraction of D/2 x 4 and a barrier, and dv/4 * (N H) workgroups share the
// work.  Sequence n's segments are slots n P .. n P + P - 1 (dense batches,
// off == nullptr) or off[n] .. off[n+1] - 1 (packed).
constexpr int COMB_COLS = 4;

struct CombParams {
  const float *s0;      // [N, H, D, dv] or nullptr
  const float *M;       // [NP, H, D, D]
  const float *Sloc;    // [NP, H, D, dv]
  float *Sin;           // [NP, H, D, dv]
  const int32_t *off;   // [N + 1] segment offsets (packed) or nullptr
  int N, P, H, dv, NP;
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
  const int dv = p.dv;
  // (packed: offsets clamped into the NP slots, which they never leave for a
  // well-formed cu_seqlens)
  const int first = p.off ? min(p.off[n], p.NP) : n * p.P;
  const int nseg = p.off ? min(p.off[n + 1], p.NP) - first : p.P;
  constexpr size_t MAT = (size_t)D * D;
  const size_t ST = (size_t)D * dv;
  auto slot = [&](int seg) { return (size_t)(first + seg) * p.H + h; };

  float4 mc[NF4], mn[NF4];
  float lc[2] = {0.f, 0.f}, ln[2] = {0.f, 0.f};  // S_loc[r][c0 + 2 half + 0..1]
  auto fetch = [&](int seg, float4 (&m)[NF4], float (&l)[2]) {
    const float4 *M4 = reinterpret_cast<const float4 *>(p.M + slot(seg) * MAT + (size_t)r * D + j0);
#pragma unroll
    for (int f = 0; f < NF4; ++f) m[f] = M4[f];
    const float *L = p.Sloc + slot(seg) * ST + (size_t)r * dv + c0 + 2 * half;
    l[0] = L[0];
    l[1] = L[1];
  };

  // S_in(0): thread (r, half) owns columns c0 + 2 half, +1 of row r
#pragma unroll
  for (int c = 0; c < 2; ++c)
    Sb[0][r][2 * half + c] =
        p.s0 ? p.s0[((size_t)n * p.H + h) * ST + (size_t)r * dv + c0 + 2 * half + c] : 0.0f;
  if (nseg > 1) fetch(0, mc, lc);
  __syncthreads();
  for (int seg = 0; seg < nseg; ++seg) {
    const int cur = seg & 1;
#pragma unroll
    for (int c = 0; c < 2; ++c)
      p.Sin[slot(seg) * ST + (size_t)r * dv + c0 + 2 * half + c] = Sb[cur][r][2 * half + c];
    if (seg + 1 == nseg) break;
    if (seg + 2 < nseg) fetch(seg + 1, mn, ln);  // in flight during this contraction
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

// final_state[n] = Sout of sequence n's last segment, slot n P + P - 1 (dense)
// or off[n+1] - 1 (packed) (float4 copies).
__global__ __launch_bounds__(FILL_THREADS) void last_state_kernel(const float *Sout, float *out,
                                                                  const int32_t *off, int N,
                                                                  int P, int NP, int64_t per_seq) {
  const int64_t q4 = per_seq / 4;
  for (int64_t i = (int64_t)blockIdx.x * FILL_THREADS + threadIdx.x; i < (int64_t)N * q4;
       i += (int64_t)gridDim.x * FILL_THREADS) {
    const int64_t n = i / q4, e = i % q4;
    const int64_t last = off ? (int64_t)min(max(off[n + 1] - 1, 0), NP - 1) : n * P + P - 1;
    reinterpret_cast<float4 *>(out)[i] = reinterpret_cast<const float4 *>(Sout + last * per_seq)[e];
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
  hipLaunchKernelGGL(combine_kernel<D>, dim3(cp.N * cp.H, cp.dv / COMB_COLS), dim3(2 * D), 0, s, cp);
  return hipGetLastError();
}

unsigned fill_blocks(int64_t n) {
  const int64_t b = (n + FILL_THREADS - 1) / FILL_THREADS;
  return (unsigned)(b < 4096 ? (b > 0 ? b : 1) : 4096);
}

}  // namespace

Problem segments(const Problem &pr, int segment_len);

// The passes of the rule in bf16 on the matrix cores run in the cooperative
// form when its launches take the segments as gdr_chunked_fwd would take
// them (every segment's (segment, key head) group in one launch, or
// consecutive launches of long enough segments): its workspace, sized for
// the wider of the two pass shapes, or 0.
size_t split_coop_bytes(const Problem &pr, int segment_len) {
  if (pr.mode != kModeRule) return 0;
  Problem seg = segments(pr, segment_len);
  Problem segm = seg;
  segm.d_v = pr.d_k;
  size_t bytes = 0;
  for (const Problem *q : {&seg, &segm}) {
    if (!chunked_mfma_supports(*q) || !coop_runs(*q, chunked_coop_seqs_per_launch(*q))) return 0;
    const size_t b = chunked_coop_workspace_bytes(*q);
    bytes = b > bytes ? b : bytes;
  }
  return bytes;
}

// The segments of a batch as one batch: a dense batch of num_seqs * P
// sequences of segment_len tokens, or for a packed batch a packed batch of
// NP segment slots whose prefix sums (segcu, written on the device by
// segment_map_kernel) are filled in at launch.
Problem segments(const Problem &pr, int segment_len) {
  Problem seg = pr;
  if (pr.cu) {
    seg.num_seqs = (int)split_slots(pr, segment_len);
    seg.seq_len = 0;
  } else {
    seg.num_seqs = pr.num_seqs * (pr.seq_len / segment_len);
    seg.seq_len = segment_len;
    seg.cu = nullptr;
  }
  return seg;
}

int64_t split_slots(const Problem &pr, int segment_len) {
  if (pr.cu) return pr.total / segment_len + pr.num_seqs;
  return (int64_t)pr.num_seqs * (pr.seq_len / segment_len);
}

SplitLayout split_layout(const Problem &pr, int segment_len) {
  SplitLayout L;
  const size_t es = pr.dtype == GDR_F32 ? 4 : 2;
  L.P = pr.cu ? 0 : pr.seq_len / segment_len;
  L.NP = (int)split_slots(pr, segment_len);
  const size_t NP = (size_t)L.NP;
  const size_t st = NP * pr.H_v * pr.d_k * pr.d_v * 4;   // S_loc, S_in, final states
  const size_t stm = NP * pr.H_v * pr.d_k * pr.d_k * 4;  // M and the identities
  L.zero_v = 0;
  L.ident = L.zero_v + round256((size_t)pr.total * pr.H_v * pr.d_k * es);
  L.M = L.ident + round256(stm > st ? stm : st);
  L.Sloc = L.M + round256(stm);
  L.Sin = L.Sloc + round256(st);
  // the M pass writes d_k-wide outputs: into o when d_v == d_k, else here
  L.o_m = L.Sin + round256(st);
  L.coop = L.o_m + (pr.d_k != pr.d_v ? round256((size_t)pr.total * pr.H_v * pr.d_k * es) : 0);
  L.seg_cu = L.coop + round256(split_coop_bytes(pr, segment_len));
  L.seg_off = L.seg_cu + (pr.cu ? round256((NP + 1) * 4) : 0);
  L.prep = L.seg_off + (pr.cu ? round256(((size_t)pr.num_seqs + 1) * 4) : 0);
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
  int32_t *seg_cu = pr.cu ? reinterpret_cast<int32_t *>(ws + L.seg_cu) : nullptr;
  int32_t *seg_off = pr.cu ? reinterpret_cast<int32_t *>(ws + L.seg_off) : nullptr;
  const size_t es = pr.dtype == GDR_F32 ? 4 : 2;
  const int64_t vwords = (int64_t)((size_t)pr.total * pr.H_v * pr.d_k * es / 4);
  hipLaunchKernelGGL(zero_words_kernel, dim3(fill_blocks(vwords)), dim3(FILL_THREADS), 0, s,
                     static_cast<uint32_t *>(zero_v), vwords);
  const int64_t idn = (int64_t)L.NP * pr.H_v * pr.d_k * pr.d_k;
  hipLaunchKernelGGL(identity_kernel, dim3(fill_blocks(idn)), dim3(FILL_THREADS), 0, s, ident,
                     (int64_t)L.NP * pr.H_v, pr.d_k);
  if (pr.cu)
    hipLaunchKernelGGL(segment_map_kernel, dim3(1), dim3(MAP_THREADS), 0, s, pr.cu, pr.num_seqs,
                       segment_len, L.NP, seg_cu, seg_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // the segments as one batch; the M pass with d_k-wide values
  Problem seg = segments(pr, segment_len);
  if (pr.cu) seg.cu = seg_cu;
  Problem segm = seg;
  segm.d_v = pr.d_k;
  // KDA on the two-launch form: the per-chunk prep depends on q, k, a, b only,
  // so one prep serves the three chain launches below
  void *prep = ws + L.prep;
  const bool two = L.bytes > L.prep;
  if (two && (e = launch_kda_prep(seg, x, prep, s)) != hipSuccess) return e;
  // the rule in bf16: the cooperative form, its workspace cleared once here
  // (each of its launches leaves it cleared for the next)
  void *coop = ws + L.coop;
  const bool co = L.seg_cu > L.coop;
  if (co) {
    Problem first = seg;
    first.num_seqs = chunked_coop_seqs_per_launch(seg);
    Problem firstm = segm;
    firstm.num_seqs = chunked_coop_seqs_per_launch(segm);
    const Problem &wide = chunked_coop_workspace_bytes(firstm) > chunked_coop_workspace_bytes(first)
                              ? firstm : first;
    if ((e = clear_chunked_coop(wide, coop, s)) != hipSuccess) return e;
  }
  auto chunked = [&](const Problem &q, const FwdArgs &y) {
    if (two) return launch_kda_chain(q, y, prep, s);
    if (co) return run_coop_batches(q, y, chunked_coop_seqs_per_launch(q), coop, s);
    return chunked_any(q, y, s);
  };
  // S_loc: from zero on the real v;  M: from I on v = 0  (outputs land in o, or
  // in o_m when they are d_k wide, and o is overwritten by the last launch)
  FwdArgs a = x;
  a.s0 = nullptr;
  a.sT = Sloc;
  if ((e = chunked(seg, a)) != hipSuccess) return e;
  FwdArgs b = x;
  b.v = zero_v;
  b.s0 = ident;
  b.sT = M;
  if (pr.d_k != pr.d_v) b.o = ws + L.o_m;
  if ((e = chunked(segm, b)) != hipSuccess) return e;

  CombParams cp{x.s0, M, Sloc, Sin, seg_off, pr.num_seqs, L.P, pr.H_v, pr.d_v, L.NP};
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
  if ((e = chunked(seg, c)) != hipSuccess) return e;
  if (x.sT) {
    const int64_t per_seq = (int64_t)pr.H_v * pr.d_k * pr.d_v;
    hipLaunchKernelGGL(last_state_kernel, dim3(fill_blocks((int64_t)pr.num_seqs * per_seq / 4)),
                       dim3(FILL_THREADS), 0, s, ident, x.sT, seg_off, pr.num_seqs, L.P, L.NP,
                       per_seq);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace gdr
