// Chunked form of the per-channel-decay variant (KDA) in two launches:
//
//  1. kda_prep_kernel, one workgroup per (chunk, value head) over the whole
//     batch at once.  Everything a chunk needs that does not depend on the
//     state: the gates, the in-chunk cumulative decays, the channel-weighted
//     Gram matrices A and P, (I + A)^-1, and the decay-scaled k and q rows.
//     It writes them to a workspace record, each matrix already in the lane
//     order of the matrix-core operand that reads it.
//  2. kda_chain_kernel, one workgroup per (sequence, value head, 32 value
//     columns), which walks the chunks of its sequence in order and does only
//     the state-dependent products; loader waves stage the records through
//     LDS three chunks ahead.
//
// The map is the one the single-kernel form computes (the rule of
// GatedDeltaRule.ixx File Reference, "Detailed Description", with one decay
// per key channel; the KDA core of the Mamba + KDA pull requests of the PLENA
// compiler and simulator).  For a chunk of 32 tokens with state S at entry and
// gamma[r][c] the in-chunk cumulative log decay of channel c (k, q normalised,
// q scaled):
//   A[r][i] = beta_r sum_c k_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])    i < r
//   P[r][i] = sum_c q_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])           i <= r
//   T'      = (I + A)^-1 diag(beta)
//   Delta   = T' (V - (K * exp(gamma)) S)
//   O       = (Q * exp(gamma)) S + P Delta
//   S'      = diag(exp(gamma_31)) S + (K * exp(gamma_31 - gamma))^T Delta
// The prep side splits every pair (r, i) at the highest bit in which r and i
// differ, so that each exponential it takes is of a non-positive number (see
// the level products below); (I + A)^-1 is formed by blocks in fp32.
//
// Why two launches: the state-free work is most of the arithmetic and all of
// the exponentials (7 per key element), and in one kernel it sits on the
// serial chain of chunks.  Here it runs at full occupancy over every (chunk,
// head) of the batch, and the chain keeps only 28 16x16x32 products per
// chunk and 16 columns.  One prep also serves several chain launches on the
// same q, k, a, b (the segmented form's three passes).
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DK = 128;
constexpr int CH = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Workspace record of one (chunk, value head), in bytes.  A "piece" is the 16
// bytes (8 bf16) that one lane passes as the A operand of one
// v_mfma_f32_16x16x32_bf16 (lane l = 16 g + m: row m, k slots 8g..8g+7); a
// block of 64 pieces is one operand.
//  KE  8 operands (rt, tt) = rt * 4 + tt:  (k * exp(gamma))[16 rt + m][32 tt + 8 g + i]
//  QE  the same for q (normalised and scaled)
//  KD  8 operands t = 2 tt + u:  (k * exp(gamma_31 - gamma))^T, row m = state row
//      32 tt + 8 (m / 4) + 4 u + m % 4, slot 8 g + i = chunk position pos(g, i)
//  TB  2 operands a:  T'[16 a + m][pos(g, i)]
//  PB  2 operands a:  P[16 a + m][pos(g, i)]
//  DEC exp(gamma_31) per channel, fp32 [128] (then 512 unused bytes)
// pos(g, i) = 4 g + i for i < 4 and 16 + 4 g + i - 4 otherwise: the order in
// which two 16-row accumulator tiles (positions 4g..4g+3 and 16+4g..16+4g+3
// of each lane) form one operand of k = 32.
constexpr int REC_KE = 0;
constexpr int REC_QE = 8192;
constexpr int REC_KD = 16384;
constexpr int REC_TB = 24576;
constexpr int REC_PB = 26624;
constexpr int REC_DEC = 28672;
constexpr int REC_BYTES = 29696;  // DEC plus 512 unused bytes: 29 copies of 1 KB

__device__ __forceinline__ int pos_of(int g, int i) { return i < 4 ? 4 * g + i : 12 + 4 * g + i; }

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  const bf16x4 a = __builtin_convertvector(lo, bf16x4);
  const bf16x4 b = __builtin_convertvector(hi, bf16x4);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ float xexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-channel decay in log2 units, g log2(e) = -exp(A_log) softplus(x) log2(e),
// softplus through the hardware base-2 units: max(x, 0) + ln2 log2(1 + 2^(-|x| log2 e)).
__device__ __forceinline__ float gate_log2(float neg_exp_A_log2e, float x) {
  const float sp = fmaxf(x, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + xexp2(-fabsf(x) * LOG2E));
  return neg_exp_A_log2e * sp;
}

// First workspace slot of sequence n.  Chunk c of sequence n has slot
// base(n) + c with base(n) = floor(t0_n / 32) + n; since a sequence of L tokens
// starting at t0 has at most floor((t0 % 32 + L) / 32) + 1 chunks, the slots of
// different sequences never meet and floor(total / 32) + num_seqs of them
// cover any batch.
__device__ __forceinline__ int64_t slot_base(const int32_t *cu, int seq_len, int n) {
  const int64_t t0 = cu ? (int64_t)cu[n] : (int64_t)n * seq_len;
  return (t0 >> 5) + n;
}

// ---------------------------------------------------------------- prep

constexpr int PREP_NT = 256;   // 4 waves
constexpr int KP = DK + 8;     // bf16 row pitch (272 B)
constexpr int FP = DK + 4;     // fp32 row pitch (528 B)
constexpr int MP = 36;         // pitch of the 32 x 32 matrices

struct PrepSmem {
  alignas(16) bf16 Kr[CH][KP];   // raw k rows, zero past the chunk
  union {
    alignas(16) bf16 Qr[CH][KP];   // raw q rows (until the level products are done)
    alignas(16) float Tm[CH][MP];  // then T = (I + A)^-1
  };
  alignas(16) float Gm[CH][FP];  // cumulative decay, log2 units
  alignas(16) float Am[CH][MP];  // A, strictly lower part
  alignas(16) float Pm[CH][MP];  // P, strictly lower part
  // level 4's partial products, one per wave (A, P), in accumulator lane
  // order; later the 16 x 16 product A21 T11
  union {
    alignas(16) f32x4 L4[4][2][64];
    alignas(16) float W[16][20];
  };
  alignas(16) float wt[4][DK];   // per-wave column sums of the gates
  alignas(16) float ik[CH];      // 1 / |k_r|
  alignas(16) float iq[CH];      // scale / |q_r|
  alignas(16) float pd[CH];      // P[r][r] = q_r . k_r
  alignas(16) float beta[CH];
};

struct PrepParams {
  const bf16 *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  const int32_t *cu;
  unsigned char *ws;
  int num_seqs, seq_len, H_k, H_v;
  float scale, eps;
};

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

// Workgroup barrier that waits only for this wave's LDS accesses
// (lgkmcnt(0)), not for its global accesses in flight; the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Orders LDS accesses of one wave around a point (its LDS operations run in
// order; this keeps the compiler from moving them).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// The barriers wait for LDS traffic only: no wave of the workgroup reads the
// record stores, which the kernel's end makes visible to the chains.
__global__ __launch_bounds__(PREP_NT) void kda_prep_kernel(PrepParams p) {
  __shared__ PrepSmem sm;
  const int h = (int)(blockIdx.x % (unsigned)p.H_v);
  const int64_t slot = blockIdx.x / (unsigned)p.H_v;
  // the sequence of this slot: the last n with base(n) <= slot
  int lo = 0, hi = p.num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (slot_base(p.cu, p.seq_len, mid) <= slot) lo = mid;
    else hi = mid - 1;
  }
  const int n = lo;
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const int64_t c = slot - slot_base(p.cu, p.seq_len, n);
  if (c < 0 || c * CH >= t1 - t0) return;  // a slot no chunk uses (uniform per workgroup)
  const int64_t c0 = t0 + c * CH;
  const int cl = (int)min((int64_t)CH, t1 - c0);
  unsigned char *rec = p.ws + ((size_t)slot * p.H_v + h) * REC_BYTES;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hk = h / (p.H_v / p.H_k);
  // ---- row phase: thread (r, cg) holds row r, channels 16 cg .. 16 cg + 15.
  // Every load is issued up front (rows past the chunk read its last row and
  // are masked arithmetically), so the loads are in flight together.
  const int r = tid >> 3, cg = tid & 7, cc = 16 * cg;
  const bool valid = r < cl;
  const float vmask = valid ? 1.f : 0.f;
  const int64_t row = c0 + min(r, cl - 1);
  bf16x8 kv[2], qv[2], av[2];
  float4 db[4];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    kv[s] = *reinterpret_cast<const bf16x8 *>(p.k + (row * p.H_k + hk) * DK + cc + 8 * s);
    qv[s] = *reinterpret_cast<const bf16x8 *>(p.q + (row * p.H_k + hk) * DK + cc + 8 * s);
    av[s] = *reinterpret_cast<const bf16x8 *>(p.a + (row * p.H_v + h) * DK + cc + 8 * s);
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    db[e4] = *reinterpret_cast<const float4 *>(p.dt_bias + h * DK + cc + 4 * e4);
  const float braw = static_cast<float>(p.b[(c0 + min(tid & 31, cl - 1)) * p.H_v + h]);
  const float neg_exp_A = -expf(p.A_log[h]) * LOG2E;
  float ssk = 0.f, ssq = 0.f, sqk = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float kf = static_cast<float>(kv[e >> 3][e & 7]), qf = static_cast<float>(qv[e >> 3][e & 7]);
    ssk += kf * kf;
    ssq += qf * qf;
    sqk += qf * kf;
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    ssk += __shfl_xor(ssk, off, 64);
    ssq += __shfl_xor(ssq, off, 64);
    sqk += __shfl_xor(sqk, off, 64);
  }
  const float ik = rsqrtf(ssk + p.eps) * vmask;
  const float iq = rsqrtf(ssq + p.eps) * p.scale * vmask;
  if (cg == 0) {
    sm.ik[r] = ik;
    sm.iq[r] = iq;
    sm.pd[r] = sqk * ik * iq;
  }
  {
    const bf16x8 z8 = {};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      *reinterpret_cast<bf16x8 *>(&sm.Kr[r][cc + 8 * s]) = valid ? kv[s] : z8;
      *reinterpret_cast<bf16x8 *>(&sm.Qr[r][cc + 8 * s]) = valid ? qv[s] : z8;
    }
  }
  // gates, then their cumulative sum down the rows: rows 8w..8w+7 of wave w
  // sit 8 lanes apart, so three shifted adds scan the wave's rows
  float gl[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float4 d = db[e >> 2];
    const float dv = (e & 3) == 0 ? d.x : (e & 3) == 1 ? d.y : (e & 3) == 2 ? d.z : d.w;
    gl[e] = gate_log2(neg_exp_A, static_cast<float>(av[e >> 3][e & 7]) + dv) * vmask;
  }
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float x = gl[e], y;
    y = __shfl_up(x, 8, 64);
    x += lane >= 8 ? y : 0.f;
    y = __shfl_up(x, 16, 64);
    x += lane >= 16 ? y : 0.f;
    y = __shfl_up(x, 32, 64);
    x += lane >= 32 ? y : 0.f;
    gl[e] = x;
  }
  if (lane >= 56) {
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4)
      *reinterpret_cast<float4 *>(&sm.wt[wave][cc + 4 * e4]) =
          make_float4(gl[4 * e4], gl[4 * e4 + 1], gl[4 * e4 + 2], gl[4 * e4 + 3]);
  }
  if (tid < CH) sm.beta[tid] = tid < cl ? sigmoid_f32(braw) : 0.f;
  lds_barrier();
  // carry of the earlier waves (a loop uniform per wave)
  {
    float carry[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) carry[e] = 0.f;
    for (int w = 0; w < wave; ++w) {
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const float4 x = *reinterpret_cast<const float4 *>(&sm.wt[w][cc + 4 * e4]);
        carry[4 * e4] += x.x;
        carry[4 * e4 + 1] += x.y;
        carry[4 * e4 + 2] += x.z;
        carry[4 * e4 + 3] += x.w;
      }
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) gl[e] += carry[e];
  }
#pragma unroll
  for (int e4 = 0; e4 < 4; ++e4)
    *reinterpret_cast<float4 *>(&sm.Gm[r][cc + 4 * e4]) =
        make_float4(gl[4 * e4], gl[4 * e4 + 1], gl[4 * e4 + 2], gl[4 * e4 + 3]);
  // KE, QE pieces of this row: operand (r / 16, cg / 2), lanes m = r % 16 and
  // g = 2 (cg % 2) + {0, 1}
  {
    const int rt = r >> 4, m = r & 15, tt = cg >> 1;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int g = 2 * (cg & 1) + s;
      f32x4 ke0, ke1, qe0, qe1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e0 = xexp2(gl[8 * s + j]), e1 = xexp2(gl[8 * s + 4 + j]);
        ke0[j] = static_cast<float>(kv[s][j]) * ik * e0;
        ke1[j] = static_cast<float>(kv[s][4 + j]) * ik * e1;
        qe0[j] = static_cast<float>(qv[s][j]) * iq * e0;
        qe1[j] = static_cast<float>(qv[s][4 + j]) * iq * e1;
      }
      const size_t piece = ((size_t)(rt * 4 + tt) * 64 + 16 * g + m) * 16;
      *reinterpret_cast<bf16x8 *>(rec + REC_KE + piece) = pack8(ke0, ke1);
      *reinterpret_cast<bf16x8 *>(rec + REC_QE + piece) = pack8(qe0, qe1);
    }
    if (r == 0) {  // exp(gamma_31) per channel: the sum of the four waves' totals
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        float tot = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) tot += sm.wt[w][cc + e];
        reinterpret_cast<float *>(rec + REC_DEC)[cc + e] = xexp2(tot);
      }
    }
  }
  lds_barrier();
  // ---- level products.  Level b (h = 2^b) holds the pairs (r, i), i < r,
  // whose highest differing bit is b: r in the upper half and i in the lower
  // half of a common block of 2h rows.  With ref the last row of the lower
  // half, exp(gamma_r - gamma_i) = exp(gamma_r - gamma_ref) exp(gamma_ref - gamma_i)
  // and both factors are at most 1.  Packing the 16 upper and the 16 lower
  // rows of all blocks, each level is one 16 x 16 x 128 product for A and one
  // for P, of which the entries inside a block are kept.  Wave w takes level
  // w over all channels and level 4 over channels 32w..32w+31 (a partial
  // product; the four are added in a fixed order below); each lane scales its
  // own operand elements.
  {
    const int m = lane & 15, g = lane >> 4;
    auto level = [&](int b, int kb0, int nkb, f32x4 &accA, f32x4 &accP) {
      const int hb = 1 << b, blk = m >> b;
      const int ru = (blk << (b + 1)) | hb | (m & (hb - 1));
      const int rl = (blk << (b + 1)) | (m & (hb - 1));
      const int ref = (blk << (b + 1)) + hb - 1;
      const float iku = sm.ik[ru], iqu = sm.iq[ru], ikl = sm.ik[rl];
      for (int kb = kb0; kb < kb0 + nkb; ++kb) {
        const int ch = 32 * kb + 8 * g;
        const bf16x8 ku = *reinterpret_cast<const bf16x8 *>(&sm.Kr[ru][ch]);
        const bf16x8 qu = *reinterpret_cast<const bf16x8 *>(&sm.Qr[ru][ch]);
        const bf16x8 kl = *reinterpret_cast<const bf16x8 *>(&sm.Kr[rl][ch]);
        f32x4 xk[2], xq[2], yl[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const float4 gu = *reinterpret_cast<const float4 *>(&sm.Gm[ru][ch + 4 * hf]);
          const float4 gr = *reinterpret_cast<const float4 *>(&sm.Gm[ref][ch + 4 * hf]);
          const float4 gw = *reinterpret_cast<const float4 *>(&sm.Gm[rl][ch + 4 * hf]);
          const float guv[4] = {gu.x, gu.y, gu.z, gu.w}, grv[4] = {gr.x, gr.y, gr.z, gr.w},
                      gwv[4] = {gw.x, gw.y, gw.z, gw.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float fu = xexp2(guv[j] - grv[j]), fl = xexp2(grv[j] - gwv[j]);
            xk[hf][j] = static_cast<float>(ku[4 * hf + j]) * iku * fu;
            xq[hf][j] = static_cast<float>(qu[4 * hf + j]) * iqu * fu;
            yl[hf][j] = static_cast<float>(kl[4 * hf + j]) * ikl * fl;
          }
        }
        const bf16x8 y = pack8(yl[0], yl[1]);
        accA = mma32(pack8(xk[0], xk[1]), y, accA);
        accP = mma32(pack8(xq[0], xq[1]), y, accP);
      }
    };
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4 accA = z, accP = z, a4 = z, p4 = z;
    level(wave, 0, 4, accA, accP);
    level(4, wave, 1, a4, p4);
    sm.L4[wave][0][lane] = a4;
    sm.L4[wave][1][lane] = p4;
    // accumulator element j: packed upper row 4g + j against packed lower row m
    const int b = wave, hb = 1 << b, blk = m >> b;
    const int rl = (blk << (b + 1)) | (m & (hb - 1));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int mu = 4 * g + j;
      if ((mu >> b) == blk) {
        const int rr = ((mu >> b) << (b + 1)) | hb | (mu & (hb - 1));
        sm.Am[rr][rl] = sm.beta[rr] * accA[j];
        sm.Pm[rr][rl] = accP[j];
      }
    }
  }
  lds_barrier();
  // ---- T11 = (I + A11)^-1 and T22 = (I + A22)^-1 by forward substitution
  // (wave 0, lanes 0..15 and 16..31: one column each); the other waves add
  // up level 4 (A21 and P's lower-left block) and write the KD operands
  if (wave == 0) {
    if (lane < 32) {
      const int off = 16 * (lane >> 4), j = lane & 15;
      float x[16];
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float acc[4] = {(rr == j) ? 1.0f : 0.0f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < rr; ++i) acc[i & 3] -= sm.Am[off + rr][off + i] * x[i];
        x[rr] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sm.Tm[off + rr][off + j] = x[rr];
    } else {
      // T12 = 0
      const int j = lane & 15, rr0 = 8 * ((lane >> 4) & 1);
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) sm.Tm[rr0 + rr][16 + j] = 0.f;
    }
  } else {
    for (int e = tid - 64; e < 2 * 256; e += PREP_NT - 64) {
      const int which = e >> 8, ln = (e >> 2) & 63, j = e & 3;
      const float s4 = ((sm.L4[0][which][ln][j] + sm.L4[1][which][ln][j]) + sm.L4[2][which][ln][j]) +
                       sm.L4[3][which][ln][j];
      const int rr = 16 + 4 * (ln >> 4) + j, i = ln & 15;
      if (which == 0) sm.Am[rr][i] = sm.beta[rr] * s4;
      else sm.Pm[rr][i] = s4;
    }
    for (int q = tid - 64; q < 8 * 64; q += PREP_NT - 64) {
      const int ln = q & 63, m = ln & 15, g = ln >> 4;
      const int t = q >> 6, tt = t >> 1, u = t & 1;
      const int ch = 32 * tt + 8 * (m >> 2) + 4 * u + (m & 3);
      const float gla = sm.Gm[CH - 1][ch];
      f32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ps = pos_of(g, i);
        const float v = static_cast<float>(sm.Kr[ps][ch]) * sm.ik[ps] * xexp2(gla - sm.Gm[ps][ch]);
        if (i < 4) lo[i] = v;
        else hi[i - 4] = v;
      }
      *reinterpret_cast<bf16x8 *>(rec + REC_KD + (size_t)q * 16) = pack8(lo, hi);
    }
  }
  lds_barrier();
  // ---- T21 = -T22 (A21 T11) (wave 0: lane l computes 4 entries of row
  // l / 4); P's operands (the other waves)
  if (wave == 0) {
    const int rr = lane >> 2, c4 = 4 * (lane & 3);
    float w4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float a = sm.Am[16 + rr][k];
      const float4 t = *reinterpret_cast<const float4 *>(&sm.Tm[k][c4]);
      w4[0] += a * t.x;
      w4[1] += a * t.y;
      w4[2] += a * t.z;
      w4[3] += a * t.w;
    }
    *reinterpret_cast<float4 *>(&sm.W[rr][c4]) = make_float4(w4[0], w4[1], w4[2], w4[3]);
    wave_lds_sync();
    float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float a = sm.Tm[16 + rr][16 + k];
      const float4 wv = *reinterpret_cast<const float4 *>(&sm.W[k][c4]);
      t4[0] -= a * wv.x;
      t4[1] -= a * wv.y;
      t4[2] -= a * wv.z;
      t4[3] -= a * wv.w;
    }
    *reinterpret_cast<float4 *>(&sm.Tm[16 + rr][c4]) = make_float4(t4[0], t4[1], t4[2], t4[3]);
  } else {
    for (int q = tid - 64; q < 2 * 64; q += PREP_NT - 64) {
      const int ln = q & 63, m = ln & 15, g = ln >> 4;
      const int a = q >> 6, rw = 16 * a + m;
      f32x4 lo, hi;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ps = pos_of(g, i);
        const float v = ps > rw ? 0.f : (ps == rw ? sm.pd[rw] : sm.Pm[rw][ps]);
        if (i < 4) lo[i] = v;
        else hi[i - 4] = v;
      }
      *reinterpret_cast<bf16x8 *>(rec + REC_PB + (size_t)q * 16) = pack8(lo, hi);
    }
  }
  lds_barrier();
  // ---- T' = T diag(beta), as the TB operands
  if (tid < 2 * 64) {
    const int a = tid >> 6, m = lane & 15, g = lane >> 4, rw = 16 * a + m;
    f32x4 lo, hi;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ps = pos_of(g, i);
      const float v = sm.Tm[rw][ps] * sm.beta[ps];
      if (i < 4) lo[i] = v;
      else hi[i - 4] = v;
    }
    *reinterpret_cast<bf16x8 *>(rec + REC_TB + (size_t)tid * 16) = pack8(lo, hi);
  }
}

// ---------------------------------------------------------------- chain

constexpr int NST = 4;                    // LDS stages: chunks c .. c+3 in flight
constexpr int V_BYTES = CH * 32 * 2;      // v tile of 32 rows x 32 columns
constexpr int STAGE = REC_BYTES + V_BYTES;
constexpr int REC_COPIES = REC_BYTES / 1024;
constexpr int L0_COPIES = 15;             // loader wave 2: record KB 0..14
constexpr int L1_COPIES = REC_COPIES - L0_COPIES + 2;  // wave 3: the rest and v
static_assert(REC_BYTES % 1024 == 0, "whole 1 KB copies");

struct ChainParams {
  const bf16 *v;
  const unsigned char *ws;
  const float *s0;
  bf16 *o;
  float *sT;
  const int32_t *cu;
  int seq_len, H_v, d_v, nb, units;
  int64_t nslots;
};

// 16 bytes per lane from global memory straight into LDS: lane l's bytes
// land at lds + 16 l (`lds` the same for the whole wave).
__device__ __forceinline__ void dma16(const void *src, unsigned char *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(lds), 16, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const unsigned char *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

// One workgroup of six waves per (sequence, value head, 32 value columns);
// each 16-column block has a state wave and an output wave.
//  - State wave b (wave b): keeps a [128 x 16] slice of the state in 8
//    accumulator tiles for the whole sequence.  Tile t = 2 tt + u holds, in
//    lane (m, g) and element j, state row 32 tt + 8 g + 4 u + j of column m,
//    so the tiles 2tt and 2tt+1 of a lane are state rows 32 tt + 8 g .. + 7:
//    the B operand of k = 32 that K S takes without leaving registers.  Step
//    c: K S, Delta = T' (V - K S), S <- diag(e^gamma_31) S + K_D Delta, then
//    the bf16 operands of the new state and Delta go to LDS for the output
//    wave.
//  - Output wave b (wave 2 + b) trails by half a step: in step c it forms
//    O(c - 1) = Q S(c - 1) + P Delta(c - 1) and then Q S(c), from the
//    operands the state wave left in LDS.
//  - Waves 4 and 5 copy each chunk's record and v tile into a ring of 4 LDS
//    stages three chunks ahead (global_load_lds, never through registers).
// One barrier B(c) ends step c.  It publishes Delta(c), the state operands of
// chunk c + 1 and the data of chunk c + 1, and it frees the stage of chunk
// c - 1 (the output wave keeps that chunk's P in registers).  It waits for
// LDS traffic and the loaders' copies only.  The workgroups of one
// (sequence, head) are dealt to one XCD, where they share the records
// through its L2.
__global__ __launch_bounds__(384) void kda_chain_kernel(ChainParams p) {
  extern __shared__ __align__(16) unsigned char ring[];
  const int bid = blockIdx.x;
  const int vb = (bid >> 3) % p.nb;
  const int unit = 8 * ((bid >> 3) / p.nb) + (bid & 7);
  if (unit >= p.units) return;
  const int h = unit % p.H_v, n = unit / p.H_v;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const int64_t L = t1 - t0;
  const int64_t base = slot_base(p.cu, p.seq_len, n);
  // never read past the workspace, whatever the offsets
  const int nch = (int)max((int64_t)0, min((L + CH - 1) / CH, p.nslots - base));
  const int64_t vstride = (int64_t)p.H_v * p.d_v;
  const int c32 = 32 * vb;  // first column of the workgroup
  const size_t pl = (size_t)lane * 16;

  if (wave >= 4) {
    // ---- loaders
    const int ld = wave - 4;
    auto issue = [&](int c) {
      c = min(c, nch - 1);
      unsigned char *st = ring + (c % NST) * STAGE;
      const unsigned char *rec = p.ws + ((size_t)(base + c) * p.H_v + h) * REC_BYTES;
      if (ld == 0) {
#pragma unroll
        for (int i = 0; i < L0_COPIES; ++i) dma16(rec + i * 1024 + lane * 16, st + i * 1024);
      } else {
#pragma unroll
        for (int i = L0_COPIES; i < REC_COPIES; ++i) dma16(rec + i * 1024 + lane * 16, st + i * 1024);
        const int64_t c0 = t0 + (int64_t)c * CH;
        const int last = (int)min((int64_t)CH, t1 - c0) - 1;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rr = min(16 * i + (lane >> 2), last);
          const int col = min(c32 + 8 * (lane & 3), p.d_v - 8);  // past d_v: any valid column
          dma16(p.v + (c0 + rr) * vstride + (int64_t)h * p.d_v + col, st + REC_BYTES + i * 1024);
        }
      }
    };
    if (nch > 0) {
      issue(0);
      issue(1);
      issue(2);
      if (ld == 0) vm_wait<2 * L0_COPIES>();
      else vm_wait<2 * L1_COPIES>();
      lds_barrier();  // chunk 0 has landed
      for (int c = 0; c < nch; ++c) {
        issue(c + NST - 1);  // into the stage of chunk c - 1, free since B(c - 1)
        if (ld == 0) vm_wait<2 * L0_COPIES>();
        else vm_wait<2 * L1_COPIES>();
        lds_barrier();  // B(c): chunk c + 1 has landed
      }
    }
    return;
  }
  const int blk = wave & 1;
  const int col = c32 + 16 * blk + m;
  const bool live = c32 + 16 * blk < p.d_v;  // d_v = 16: block 1 has no columns
  // hand-off of block b, two parities: the state's 4 B operands (4 KB), then Delta (1 KB)
  unsigned char *xb = ring + NST * STAGE + blk * 2 * 5 * 1024;
  auto sop = [&](int c, int tt) { return xb + (c & 1) * 5 * 1024 + tt * 1024 + pl; };
  auto dop = [&](int c) { return xb + (c & 1) * 5 * 1024 + 4 * 1024 + pl; };
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  if (wave < 2) {
    // ---- state wave
    const size_t st_off = ((size_t)n * p.H_v + h) * DK * p.d_v + col;
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        S[t][j] = (live && p.s0)
                      ? p.s0[st_off + (size_t)(32 * (t >> 1) + 8 * g + 4 * (t & 1) + j) * p.d_v]
                      : 0.f;
    if (nch > 0) {
      bf16x8 sb[4];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        sb[tt] = pack8(S[2 * tt], S[2 * tt + 1]);
        *reinterpret_cast<bf16x8 *>(sop(0, tt)) = sb[tt];
      }
      lds_barrier();  // chunk 0 and the state operands of chunk 0
      for (int c = 0; c < nch; ++c) {
        const unsigned char *st = ring + (c % NST) * STAGE;
        bf16x8 ke[8], tb[2], kd[8];
        f32x4 dc[8];
        float vv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ke[i] = lds8(st + REC_KE + i * 1024 + pl);
        tb[0] = lds8(st + REC_TB + pl);
        tb[1] = lds8(st + REC_TB + 1024 + pl);
        {
          const bf16 *vt = reinterpret_cast<const bf16 *>(st + REC_BYTES);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            vv[j] = static_cast<float>(vt[(4 * g + j) * 32 + 16 * blk + m]);
            vv[4 + j] = static_cast<float>(vt[(16 + 4 * g + j) * 32 + 16 * blk + m]);
          }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          kd[t] = lds8(st + REC_KD + t * 1024 + pl);
          dc[t] = *reinterpret_cast<const f32x4 *>(st + REC_DEC + 4 * (32 * (t >> 1) + 8 * g + 4 * (t & 1)));
        }
        f32x4 ks0 = z, ks1 = z;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          ks0 = mma32(ke[tt], sb[tt], ks0);
          ks1 = mma32(ke[4 + tt], sb[tt], ks1);
        }
        f32x4 u0, u1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          u0[j] = vv[j] - ks0[j];
          u1[j] = vv[4 + j] - ks1[j];
        }
        const bf16x8 ub = pack8(u0, u1);
        const f32x4 d0 = mma32(tb[0], ub, z);
        const f32x4 d1 = mma32(tb[1], ub, z);
        const bf16x8 db = pack8(d0, d1);
        *reinterpret_cast<bf16x8 *>(dop(c)) = db;
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mma32(kd[t], db, S[t] * dc[t]);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          sb[tt] = pack8(S[2 * tt], S[2 * tt + 1]);
          *reinterpret_cast<bf16x8 *>(sop(c + 1, tt)) = sb[tt];
        }
        lds_barrier();  // B(c)
      }
    }
    if (live && p.sT) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          p.sT[st_off + (size_t)(32 * (t >> 1) + 8 * g + 4 * (t & 1) + j) * p.d_v] = S[t][j];
    }
    return;
  }
  // ---- output wave
  if (nch == 0) return;
  bf16 *oh = p.o + (int64_t)h * p.d_v + col;
  f32x4 qs0 = z, qs1 = z;
  bf16x8 pb0 = {}, pb1 = {};
  // O(c) = Q S(c) + P Delta(c), stored as bf16 rows of chunk c
  auto out = [&](int c) {
    const bf16x8 db = lds8(dop(c));
    const f32x4 o0 = mma32(pb0, db, qs0);
    const f32x4 o1 = mma32(pb1, db, qs1);
    if (!live) return;
    const int64_t c0 = t0 + (int64_t)c * CH;
    const int cl = (int)min((int64_t)CH, t1 - c0);
    if (cl == CH) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        oh[(c0 + 4 * g + j) * vstride] = static_cast<bf16>(o0[j]);
        oh[(c0 + 16 + 4 * g + j) * vstride] = static_cast<bf16>(o1[j]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 4 * g + j, r1 = 16 + 4 * g + j;
        if (r0 < cl) oh[(c0 + r0) * vstride] = static_cast<bf16>(o0[j]);
        if (r1 < cl) oh[(c0 + r1) * vstride] = static_cast<bf16>(o1[j]);
      }
    }
  };
  lds_barrier();  // chunk 0 and the state operands of chunk 0
  for (int c = 0; c < nch; ++c) {
    if (c > 0) out(c - 1);  // Delta(c - 1) since B(c - 1)
    const unsigned char *st = ring + (c % NST) * STAGE;
    pb0 = lds8(st + REC_PB + pl);
    pb1 = lds8(st + REC_PB + 1024 + pl);
    qs0 = z;
    qs1 = z;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const bf16x8 sbv = lds8(sop(c, tt));
      qs0 = mma32(lds8(st + REC_QE + tt * 1024 + pl), sbv, qs0);
      qs1 = mma32(lds8(st + REC_QE + (4 + tt) * 1024 + pl), sbv, qs1);
    }
    lds_barrier();  // B(c)
  }
  out(nch - 1);
}

int64_t kda_slots(const Problem &p) { return p.total / CH + p.num_seqs; }

}  // namespace

bool kda_two_pass_supports(const Problem &p) {
  return p.mode == kModeKDA && p.dtype == GDR_BF16 && p.d_k == DK && p.d_v % 16 == 0 &&
         p.d_v >= 16 && p.chunk == CH;
}

size_t kda_two_pass_bytes(const Problem &p) {
  if (!kda_two_pass_supports(p)) return 0;
  return (size_t)kda_slots(p) * p.H_v * REC_BYTES;
}

hipError_t launch_kda_prep(const Problem &pr, const FwdArgs &x, void *workspace, hipStream_t s) {
  const int64_t nslots = kda_slots(pr);
  const int64_t prep_grid = nslots * pr.H_v;
  if ((int64_t)pr.num_seqs * pr.H_v == 0) return hipSuccess;
  if (prep_grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  PrepParams pp;
  pp.q = static_cast<const bf16 *>(x.q);
  pp.k = static_cast<const bf16 *>(x.k);
  pp.a = static_cast<const bf16 *>(x.a);
  pp.b = static_cast<const bf16 *>(x.b);
  pp.A_log = x.A_log;
  pp.dt_bias = x.dt_bias;
  pp.cu = pr.cu;
  pp.ws = static_cast<unsigned char *>(workspace);
  pp.num_seqs = pr.num_seqs;
  pp.seq_len = pr.seq_len;
  pp.H_k = pr.H_k;
  pp.H_v = pr.H_v;
  pp.scale = pr.scale;
  pp.eps = pr.eps;
  // no tokens: every prep workgroup finds an unused slot
  hipLaunchKernelGGL(kda_prep_kernel, dim3((unsigned)prep_grid), dim3(PREP_NT), 0, s, pp);
  return hipGetLastError();
}

hipError_t launch_kda_chain(const Problem &pr, const FwdArgs &x, const void *workspace,
                            hipStream_t s) {
  const int nb = (pr.d_v + 31) / 32;
  const int64_t units = (int64_t)pr.num_seqs * pr.H_v;
  const int64_t chain_grid = (units + 7) / 8 * 8 * nb;
  if (units == 0) return hipSuccess;
  if (chain_grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  ChainParams cp;
  cp.v = static_cast<const bf16 *>(x.v);
  cp.ws = static_cast<const unsigned char *>(workspace);
  cp.s0 = x.s0;
  cp.o = static_cast<bf16 *>(x.o);
  cp.sT = x.sT;
  cp.cu = pr.cu;
  cp.seq_len = pr.seq_len;
  cp.H_v = pr.H_v;
  cp.d_v = pr.d_v;
  cp.nb = nb;
  cp.units = (int)units;
  cp.nslots = kda_slots(pr);
  const size_t smem = (size_t)NST * STAGE + 2 * 2 * 5 * 1024;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_chain_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  // with no tokens the chains copy the initial state (or zeros) to the final one
  hipLaunchKernelGGL(kda_chain_kernel, dim3((unsigned)chain_grid), dim3(384), smem, s, cp);
  return hipGetLastError();
}

hipError_t launch_kda_two_pass(const Problem &pr, const FwdArgs &x, void *workspace,
                               hipStream_t s) {
  const hipError_t e = launch_kda_prep(pr, x, workspace, s);
  if (e != hipSuccess) return e;
  return launch_kda_chain(pr, x, workspace, s);
}

}  // namespace gdr
