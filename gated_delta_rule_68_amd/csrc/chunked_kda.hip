// Chunked form of the per-channel-decay variant (KDA) on the matrix cores:
// bf16 operands, fp32 accumulation, fp32 state.  d_k = 128, d_v = 64 or 128,
// chunk 32, bf16 inputs; other shapes and fp32 inputs run the vector kernel.
//
// The rule of GatedDeltaRule.ixx File Reference ("Detailed Description") with
// its scalar decay replaced by one decay per key channel (the KDA core of the
// Mamba + KDA pull requests of the PLENA compiler and simulator).  For one
// chunk of 32 tokens with state S at entry and gamma[r][c] the in-chunk
// cumulative log decay of channel c (k, q normalised, q scaled):
//   A[r][i] = beta_r sum_c k_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])    i < r
//   P[r][i] = sum_c q_r[c] k_i[c] exp(gamma_r[c] - gamma_i[c])           i <= r
//   R       = diag(beta) (V - (K * exp(gamma)) S)
//   Delta   = (I + A)^-1 R
//   O       = (Q * exp(gamma)) S + P Delta
//   S'      = diag(exp(gamma_31)) S + (K * exp(gamma_31 - gamma))^T Delta
// (* is the elementwise product with the [32, 128] matrix of factors).
//
// Numerics.  Only exponents gamma_r - gamma_i with i <= r are taken, so every
// factor is at most 1:
//  - a pair (r, i), i < r, is split at the highest bit b in which r and i
//    differ: inside their common block of 2h = 2^(b+1) rows, r lies in the
//    upper half and i in the lower one, and with ref the last row of the
//    lower half
//        exp(gamma_r - gamma_i) = exp(gamma_r - gamma_ref) exp(gamma_ref - gamma_i),
//    both factors <= 1 (a factor through a row inside a block would overflow
//    under strong decay).  For each b = 4..0 all such pairs are one 16 x 16
//    product of scaled bf16 tiles on the matrix cores (upper rows against
//    lower rows, packed; the entries of different blocks are dropped), so A
//    and P take ten products and no exponential per pair;
//  - the diagonal of P is q_r . k_r, taken with the norms;
//  - (I + A)^-1 is applied by blocks: Delta_1 = T11 R1 and
//    Delta_2 = T22 (R2 - A21 Delta_1), with T11 = (I + A11)^-1 and
//    T22 = (I + A22)^-1 from forward substitution in fp32.
// The decays are kept in base 2 (log2 e folded into gamma) for exp2.
//
// Launch: 512 threads (8 waves) per (sequence, value head, 32 value
// columns).  Waves 0 and 1 own 16 of the columns each and their [128 x 16]
// slice of S as 8 accumulator tiles for the whole sequence; all waves share
// the per-chunk work that does not touch the state.  Chunks run one after
// the other; the rows of the next chunk are loaded into registers while the
// current one is computed.
//
// Operand lane orders (v_mfma_f32_16x16x16_bf16 and ..._16x16x32_bf16, lane
// l = 16 g + m): A operand row m at k = 4g..4g+3 (8g..8g+7 for x32), B operand
// column m at the same k, accumulator rows 4g..4g+3 of column m.  An
// accumulator is therefore a B operand of a 16x16x16 product as it stands:
// the state tiles feed K S and Q S, and the deltas feed T, P and K^T
// products, without leaving registers.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int DK = 128;
constexpr int CH = 32;
constexpr int NT = 512;          // threads (8 waves)
constexpr int FP = DK + 4;       // fp32 row pitch: rows 16 bytes apart modulo 256
constexpr int MP = 36;           // pitch of the 32 x 32 matrices
// value columns per workgroup: 32 (4 workgroups per head at d_v = 128) beat
// 64 and 128 on the prefill layer (1.80 / 1.86 / 2.12 ms): the chunk work that
// does not touch the state is repeated per workgroup, but the state phases
// shrink and more compute units take part
constexpr int KDA_BW = 32;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

struct KdaParams {
  const bf16 *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias, *s0;
  bf16 *o;
  float *sT;
  const int32_t *cu;
  int seq_len, H_k, H_v;
  float scale, eps;
};

// Padded bf16 tiles.  [rows][128] tiles have a 272-byte row pitch: 16 rows
// read at one column start 16 bytes apart modulo 256, so the operand reads
// (16 rows x 8 bytes x 2 column groups, or 16 rows x 16 bytes) touch distinct
// bank slots.  [rows][32] tiles have an 80-byte pitch, which spreads 16 rows
// over distinct 16-byte slots the same way.  Element offsets are then a
// per-lane base plus constants, which keeps the addresses out of registers.
constexpr int KP = DK + 8;
constexpr int TP = CH + 8;
__device__ __forceinline__ int sw8(int r, int c) { return r * KP + c; }
__device__ __forceinline__ int swT(int r, int c) { return r * TP + c; }

template <int BW>
struct KdaSmem {
  alignas(16) float Gm[CH][FP];   // cumulative decay, log2 units
  alignas(16) bf16 Ke[CH * KP];   // k * exp(gamma)                              (sw8)
  alignas(16) bf16 Qe[CH * KP];   // q * exp(gamma)                              (sw8)
  // level b = 0..4 (h = 2^b): rows with bit b set ("upper", packed in row
  // order) scaled by exp(gamma_r - gamma_ref), rows with bit b clear ("lower")
  // by exp(gamma_ref - gamma_i), ref = the last lower row of the 2h-block
  alignas(16) bf16 KU[5][16 * KP];  // k, upper rows                          (sw8)
  alignas(16) bf16 QU[5][16 * KP];  // q, upper rows
  alignas(16) bf16 KL[5][16 * KP];  // k, lower rows
  alignas(16) bf16 KtT[DK * TP];  // (k * exp(gamma_31 - gamma))^T: [channel][row] (swT)
  alignas(16) bf16 VT[BW * TP];   // v^T of the block's columns: [column][row]    (swT)
  alignas(16) float Am[CH][MP];   // A (strictly lower; upper blocks stay 0)
  alignas(16) float Pm[CH][MP];   // P (lower)
  alignas(16) float Tm[CH][MP];   // T11 in [0,16)^2, T22 in [16,32)^2
  alignas(16) float beta[CH];
  alignas(16) float decay[DK];    // exp(gamma_31) per channel
  alignas(16) float dtb[DK];      // dt_bias of this head
};


__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 pk4(f32x4 x) {
  const bf16x2 lo = __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2);
  const bf16x2 hi = __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2);
  return __builtin_bit_cast(s16x4, u32x2{__builtin_bit_cast(uint32_t, lo),
                                         __builtin_bit_cast(uint32_t, hi)});
}
__device__ __forceinline__ f32x4 ld4(const float *p) {
  const float4 v = *reinterpret_cast<const float4 *>(p);
  return f32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ s16x4 ld_op4(const bf16 *p) {
  return __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ void st4(bf16 *p, float a, float b, float c, float d) {
  *reinterpret_cast<bf16x4 *>(p) = __builtin_convertvector(f32x4{a, b, c, d}, bf16x4);
}
__device__ __forceinline__ float xexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-channel decay in log2 units, g log2(e) = -exp(A_log) softplus(x) log2(e),
// softplus through the hardware base-2 units: max(x, 0) + ln2 log2(1 + 2^(-|x| log2 e)).
__device__ __forceinline__ float gate_log2(float neg_exp_A_log2e, float x) {
  const float sp = fmaxf(x, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + xexp2(-fabsf(x) * LOG2E));
  return neg_exp_A_log2e * sp;
}

// Accumulator tile of a 16x16x32 product of two [16][128] sw8 tiles.
__device__ __forceinline__ f32x4 gram16(const bf16 *X, const bf16 *Y, int m, int g) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
    acc = mma32(*reinterpret_cast<const bf16x8 *>(&X[sw8(m, 32 * kb + 8 * g)]),
                *reinterpret_cast<const bf16x8 *>(&Y[sw8(m, 32 * kb + 8 * g)]), acc);
  return acc;
}

template <int DV, int BW>
__global__ __launch_bounds__(NT) void chunked_kda_kernel(KdaParams p) {
  constexpr int NSW = BW / 16;  // state waves: wave w < NSW owns block columns 16w..16w+15
  constexpr int NVB = DV / BW;  // workgroups per (sequence, head)
  extern __shared__ __align__(16) unsigned char smem_raw[];
  KdaSmem<BW> &sm = *reinterpret_cast<KdaSmem<BW> *>(smem_raw);
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int m = lane & 15, g = lane >> 4;
  const int vb = blockIdx.x % NVB;
  const int h = (blockIdx.x / NVB) % p.H_v;
  const int n = blockIdx.x / (NVB * p.H_v);
  const int hk = h / (p.H_v / p.H_k);
  const int col0 = vb * BW + 16 * wave;  // this wave's first value column (state waves)
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);

  // row-phase mapping: thread t holds row t / 16, channels 8 (t % 16) .. +7
  const int pr = tid >> 4, pc = 8 * (tid & 15);
  constexpr int VC = BW / 16;  // value columns per thread in the row phase
  const float neg_exp_A = -expf(p.A_log[h]) * LOG2E;
  if (tid < DK) sm.dtb[tid] = p.dt_bias[h * DK + tid];

  for (int e = tid; e < CH * MP; e += NT) {
    (&sm.Am[0][0])[e] = 0.f;
    (&sm.Pm[0][0])[e] = 0.f;
    (&sm.Tm[0][0])[e] = 0.f;
  }
  // the state slice: tile t holds rows 16t + 4g + j of column col0 + m
  const size_t state_off = ((size_t)n * p.H_v + h) * DK * DV;
  f32x4 S[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      S[t][j] = (wave < NSW && p.s0) ? p.s0[state_off + (size_t)(16 * t + 4 * g + j) * DV + col0 + m]
                                     : 0.f;

  const int64_t L = t1 - t0;
  const int nch = (int)((L + CH - 1) / CH);
  // prefetch of one chunk's rows (addresses clamped into the sequence)
  typedef __bf16 bf16xv __attribute__((ext_vector_type(VC)));
  bf16x8 pk{}, pq{}, pa{};
  float kh[8], qh[8];  // this thread's normalised k and q (row pr, channels pc..pc+7)
  bf16xv pv{};
  bf16 pb = static_cast<bf16>(0.f);
  auto prefetch = [&](int c) {
    const int last = (int)(L - (int64_t)c * CH) - 1;
    const int64_t row = t0 + (int64_t)c * CH + min(pr, last);
    pk = *reinterpret_cast<const bf16x8 *>(p.k + (row * p.H_k + hk) * DK + pc);
    pq = *reinterpret_cast<const bf16x8 *>(p.q + (row * p.H_k + hk) * DK + pc);
    pa = *reinterpret_cast<const bf16x8 *>(p.a + (row * p.H_v + h) * DK + pc);
    pv = *reinterpret_cast<const bf16xv *>(p.v + (row * p.H_v + h) * DV + vb * BW + VC * (tid & 15));
    if (tid < CH) pb = p.b[(t0 + (int64_t)c * CH + min(tid, last)) * p.H_v + h];
  };
  if (nch > 0) prefetch(0);
  __syncthreads();
  // outputs of the previous chunk, stored one chunk late: after the next
  // chunk's rows have been waited for and before its prefetch is issued, so
  // that no wait for a prefetch also waits for these stores
  f32x4 o_prev0 = {0.f, 0.f, 0.f, 0.f}, o_prev1 = {0.f, 0.f, 0.f, 0.f};
  int64_t c0_prev = 0;
  int cl_prev = 0;
  auto store_outputs = [&]() {
    if (wave < NSW) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 4 * g + j, r1 = 16 + 4 * g + j;
        if (r0 < cl_prev) p.o[((c0_prev + r0) * p.H_v + h) * DV + col0 + m] = static_cast<bf16>(o_prev0[j]);
        if (r1 < cl_prev) p.o[((c0_prev + r1) * p.H_v + h) * DV + col0 + m] = static_cast<bf16>(o_prev1[j]);
      }
    }
  };

  for (int c = 0; c < nch; ++c) {
    const int64_t c0 = t0 + (int64_t)c * CH;
    const int cl = (int)min((int64_t)CH, t1 - c0);
    // ---- 1: normalised rows, gates (log2 units), v^T, beta
    {
      const bool valid = pr < cl;
      float ssk = 0.f, ssq = 0.f, sqk = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kh[e] = static_cast<float>(pk[e]);
        qh[e] = static_cast<float>(pq[e]);
        ssk += kh[e] * kh[e];
        ssq += qh[e] * qh[e];
        sqk += qh[e] * kh[e];
      }
#pragma unroll
      for (int off = 1; off < 16; off <<= 1) {
        ssk += __shfl_xor(ssk, off, 64);
        ssq += __shfl_xor(ssq, off, 64);
        sqk += __shfl_xor(sqk, off, 64);
      }
      const float ik = valid ? rsqrtf(ssk + p.eps) : 0.f;
      const float iq = valid ? rsqrtf(ssq + p.eps) * p.scale : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        kh[e] *= ik;
        qh[e] *= iq;
      }
      if ((tid & 15) == 0) sm.Pm[pr][pr] = sqk * ik * iq;  // exp(0) = 1 on the diagonal
#pragma unroll
      for (int e = 0; e < 8; e += 4) {
        const f32x4 db = ld4(&sm.dtb[pc + e]);
        float gg[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          gg[j] = valid ? gate_log2(neg_exp_A, static_cast<float>(pa[e + j]) + db[j]) : 0.f;
        *reinterpret_cast<float4 *>(&sm.Gm[pr][pc + e]) = make_float4(gg[0], gg[1], gg[2], gg[3]);
      }
#pragma unroll
      for (int j = 0; j < VC; ++j)
        sm.VT[swT(VC * (tid & 15) + j, pr)] = valid ? pv[j] : static_cast<bf16>(0.f);
      if (tid < CH) sm.beta[tid] = tid < cl ? sigmoid_f32(static_cast<float>(pb)) : 0.f;
    }
    __syncthreads();
    if (c > 0) store_outputs();
    if (c + 1 < nch) prefetch(c + 1);
    // ---- 2: cumulative decay per channel (two threads per channel, 16 rows
    //         each, in adjacent lanes); exp(gamma_31)
    if (tid < 2 * DK) {
      const int d = tid >> 1, r0 = 16 * (tid & 1);
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) x[r] = sm.Gm[r0 + r][d];
#pragma unroll
      for (int r = 1; r < 16; ++r) x[r] += x[r - 1];
      const float lo_total = __shfl_xor(x[15], 1, 64);
      if (tid & 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] += lo_total;
        sm.decay[d] = xexp2(x[15]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Gm[r0 + r][d] = x[r];
    }
    __syncthreads();
    // ---- 3a: scaled bf16 operand tiles, from this thread's row and channels
    {
      f32x4 gv[2];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) gv[e4] = ld4(&sm.Gm[pr][pc + 4 * e4]);
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const int col = pc + 4 * e4;
        f32x4 ex, kv, qv;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          ex[j] = xexp2(gv[e4][j]);
          kv[j] = kh[4 * e4 + j];
          qv[j] = qh[4 * e4 + j];
        }
        const f32x4 ke = kv * ex, qe = qv * ex;
        st4(&sm.Ke[sw8(pr, col)], ke[0], ke[1], ke[2], ke[3]);
        st4(&sm.Qe[sw8(pr, col)], qe[0], qe[1], qe[2], qe[3]);
#pragma unroll
        for (int b = 0; b < 5; ++b) {
          const int hb = 1 << b;
          const int ref = ((pr >> (b + 1)) << (b + 1)) + hb - 1;
          const int pk16 = ((pr >> (b + 1)) << b) | (pr & (hb - 1));  // packed row
          const bool upper = (pr & hb) != 0;
          const f32x4 gr = ld4(&sm.Gm[ref][col]);
          f32x4 f;
#pragma unroll
          for (int j = 0; j < 4; ++j) f[j] = xexp2(upper ? gv[e4][j] - gr[j] : gr[j] - gv[e4][j]);
          const f32x4 kf = kv * f;
          if (upper) {
            const f32x4 qf = qv * f;
            st4(&sm.KU[b][sw8(pk16, col)], kf[0], kf[1], kf[2], kf[3]);
            st4(&sm.QU[b][sw8(pk16, col)], qf[0], qf[1], qf[2], qf[3]);
          } else {
            st4(&sm.KL[b][sw8(pk16, col)], kf[0], kf[1], kf[2], kf[3]);
          }
        }
      }
      // K^T weighted by exp(gamma_31 - gamma_r), written transposed
      {
        const f32x4 gl0 = ld4(&sm.Gm[CH - 1][pc]), gl1 = ld4(&sm.Gm[CH - 1][pc + 4]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float gl = e < 4 ? gl0[e & 3] : gl1[e & 3];
          sm.KtT[swT(pc + e, pr)] = static_cast<bf16>(kh[e] * xexp2(gl - gv[e >> 2][e & 3]));
        }
      }
    }
    __syncthreads();
    // ---- 3b: A and P below the diagonal, ten 16 x 16 x 128 products (level
    //          b, A or P) over the waves; the state waves' K S and Q S.
    for (int job = wave; job < 10; job += 8) {
      const int b = job >> 1;
      const bool isA = (job & 1) == 0;
      const f32x4 acc = gram16(isA ? sm.KU[b] : sm.QU[b], sm.KL[b], m, g);
      const int hb = 1 << b;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int mu = 4 * g + j;  // packed upper row; the column m is a packed lower row
        if ((mu >> b) == (m >> b)) {
          const int r = ((mu >> b) << (b + 1)) | hb | (mu & (hb - 1));
          const int i = ((m >> b) << (b + 1)) | (m & (hb - 1));
          if (isA)
            sm.Am[r][i] = sm.beta[r] * acc[j];
          else
            sm.Pm[r][i] = acc[j];
        }
      }
    }
    f32x4 ks[2], qs[2];
    if (wave < NSW) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        ks[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
        qs[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const s16x4 sb = pk4(S[t]);
          ks[rt] = mma16(ld_op4(&sm.Ke[sw8(16 * rt + m, 16 * t + 4 * g)]), sb, ks[rt]);
          qs[rt] = mma16(ld_op4(&sm.Qe[sw8(16 * rt + m, 16 * t + 4 * g)]), sb, qs[rt]);
        }
      }
    }
    __syncthreads();
    // ---- 4: T11 = (I + A11)^-1, T22 = (I + A22)^-1 by forward substitution,
    //         one column per lane (lanes 0..15 and 16..31 of the last wave)
    if (wave == 7 && lane < 32) {
      const int off = 16 * (lane >> 4), j = lane & 15;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc[4] = {(r == j) ? 1.0f : 0.0f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < r; ++i) acc[i & 3] -= sm.Am[off + r][off + i] * x[i];
        x[r] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sm.Tm[off + r][off + j] = x[r];
    }
    __syncthreads();
    // ---- 5: deltas, outputs, state update (each state wave its 16 columns)
    if (wave < NSW) {
      f32x4 R[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const bf16x4 vb4 = __builtin_bit_cast(bf16x4, ld_op4(&sm.VT[swT(16 * wave + m, 16 * rt + 4 * g)]));
        const f32x4 bt = ld4(&sm.beta[16 * rt + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) R[rt][j] = bt[j] * (static_cast<float>(vb4[j]) - ks[rt][j]);
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      const s16x4 t11 = pk4(ld4(&sm.Tm[m][4 * g]));
      const s16x4 t22 = pk4(ld4(&sm.Tm[16 + m][16 + 4 * g]));
      const f32x4 a21 = ld4(&sm.Am[16 + m][4 * g]);
      const s16x4 na21 = pk4(f32x4{-a21[0], -a21[1], -a21[2], -a21[3]});
      const f32x4 d1 = mma16(t11, pk4(R[0]), z);
      const s16x4 d1b = pk4(d1);
      const f32x4 d2 = mma16(t22, pk4(mma16(na21, d1b, R[1])), z);
      const s16x4 d2b = pk4(d2);
      const f32x4 o0 = mma16(pk4(ld4(&sm.Pm[m][4 * g])), d1b, qs[0]);
      const f32x4 o1 = mma16(pk4(ld4(&sm.Pm[16 + m][16 + 4 * g])), d2b,
                             mma16(pk4(ld4(&sm.Pm[16 + m][4 * g])), d1b, qs[1]));
      o_prev0 = o0;
      o_prev1 = o1;
      c0_prev = c0;
      cl_prev = cl;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const f32x4 dc = ld4(&sm.decay[16 * t + 4 * g]);
        f32x4 s = S[t] * dc;
        s = mma16(ld_op4(&sm.KtT[swT(16 * t + m, 4 * g)]), d1b, s);
        s = mma16(ld_op4(&sm.KtT[swT(16 * t + m, 16 + 4 * g)]), d2b, s);
        S[t] = s;
      }
    }
    __syncthreads();
  }
  if (nch > 0) store_outputs();
  if (wave < NSW && p.sT) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        p.sT[state_off + (size_t)(16 * t + 4 * g + j) * DV + col0 + m] = S[t][j];
  }
}

template <int DV, int BW>
hipError_t launch_dv(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  KdaParams p;
  p.q = static_cast<const bf16 *>(x.q);
  p.k = static_cast<const bf16 *>(x.k);
  p.v = static_cast<const bf16 *>(x.v);
  p.a = static_cast<const bf16 *>(x.a);
  p.b = static_cast<const bf16 *>(x.b);
  p.A_log = x.A_log;
  p.dt_bias = x.dt_bias;
  p.s0 = x.s0;
  p.o = static_cast<bf16 *>(x.o);
  p.sT = x.sT;
  p.cu = pr.cu;
  p.seq_len = pr.seq_len;
  p.H_k = pr.H_k;
  p.H_v = pr.H_v;
  p.scale = pr.scale;
  p.eps = pr.eps;
  const int64_t grid = (int64_t)pr.num_seqs * pr.H_v * (DV / BW);
  if (grid == 0) return hipSuccess;
  const size_t smem = sizeof(KdaSmem<BW>);
  auto kern = chunked_kda_kernel<DV, BW>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NT), smem, s, p);
  return hipGetLastError();
}

}  // namespace

bool chunked_kda_supports(const Problem &p) {
  return p.mode == kModeKDA && p.dtype == GDR_BF16 && p.d_k == DK && (p.d_v == 64 || p.d_v == 128) &&
         p.chunk == CH;
}

hipError_t launch_chunked_kda(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  return pr.d_v == 64 ? launch_dv<64, KDA_BW>(pr, x, s) : launch_dv<128, KDA_BW>(pr, x, s);
}

}  // namespace gdr
