// Chunked (UT-transform) form on the gfx950 matrix cores: bf16 operands, fp32
// accumulation, fp32 state.  Instantiated for d_k = d_v = 128 and 32-token
// chunks (the shape the GatedDeltaRule.ixx File Reference, "Detailed
// Description", gives: one triangular solve per 32 steps).
//
// Algebra (per chunk of c <= 32 tokens, S the state at chunk entry, gamma the
// in-chunk cumulative log decay, Gamma = exp(gamma); rows r, i in-chunk):
//   A[r][i] = beta_r exp(gamma_r - gamma_i) (k_r . k_i)    i < r       (K K^T)
//   R       = diag(beta) (V - diag(Gamma) K S)                          (K S)
//   Delta   = (I + A)^-1 R
//   O       = diag(Gamma) Q S + P Delta,  P[r][i] = exp(gamma_r - gamma_i) (q_r . k_i), i <= r
//   S'      = Gamma_last S + K^T diag(exp(gamma_last - gamma)) Delta
// with k, q L2-normalised (q also scaled).  The raw bf16 rows of k and q are
// the matrix operands; 1/|k|, scale/|q| and the decay factors are applied in
// fp32 to the products.  Only differences gamma_r - gamma_i with i <= r are
// exponentiated.
//
// (I + A)^-1 is applied in 16-row blocks: with A_11, A_22 the diagonal blocks,
//   Delta_1 = T_11 R_1,  Delta_2 = T_22 (R_2 - A_21 Delta_1),  T_bb = (I + A_bb)^-1.
// Each T_bb is formed on the matrix cores from the identity, exact for the
// strictly lower (nilpotent, N^16 = 0) N = A_bb,
//   (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8),
// with the leading products carried in split (hi + lo) bf16 so that the
// result keeps fp32-level accuracy before its final rounding to bf16.
//
// Work split.  A workgroup owns (sequence, value head, 32 columns of d_v); the
// columns of S evolve independently.  Six waves, one workgroup barrier per
// chunk, three chunks in flight:
//   * 2 consumer waves each keep a [128 x 16] slice of S in MFMA accumulators
//     for the whole sequence and run chunk c: K S, Q S, the block solve,
//     outputs, K^T Delta;
//   * 2 "prepare" waves form chunk c+1's matrices: P0 the Gram blocks of K,
//     the row norms of k and the inverses T_11, T_22 and -A_21; P1 the norms of
//     q and P;
//   * 2 staging waves lay out chunk c+2 from registers (rows of k, q and v,
//     gates and their running sum) and prefetch the raw rows of chunk c+4.
// Operands that need a transposed tile (k^T for the state update, v for R)
// are read with the transposing LDS read from the row-major tiles.
// Every stage buffer is written in one step and read in later ones only.
//
// Operand lane orders (v_mfma_f32_16x16x32_bf16: lane l = 16 g + m holds A row
// m / B column m at k = 8g..8g+7, and accumulator rows 4g..4g+3 of column m;
// v_mfma_f32_16x16x16_bf16 the same with k = 4g..4g+3).  An accumulator pair
// covering rows 0..15 and 16..31 gives lane l the rows 4g..4g+3 and
// 16+4g..16+4g+3 of its column, which is a valid B operand if the contraction
// index is visited in "slot" order: slot 8g+j is position 4g+j (j < 4) or
// 16+4g+j-4 (j >= 4) of a 32-block.  Every A operand tile is stored in LDS
// with its contraction index in slot order, so the state and the deltas never
// leave registers between products.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int CH = 32;   // tokens per chunk
constexpr int NC = 2;    // consumer waves (16 columns each)
constexpr int BV = 16 * NC;
constexpr int NWAVES = 6;
constexpr int NSTAGE = 3;

// wave roles (wave w runs on SIMD w % 4: each consumer gets a SIMD of its own)
constexpr int W_P0 = 0, W_P1 = 1, W_C0 = 2, W_ST0 = 4;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                    __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}

// Slot of position c (0..31) of a 32-block.
__device__ __forceinline__ int slot_of(int c) {
  return c < 16 ? 8 * (c >> 2) + (c & 3) : 8 * ((c - 16) >> 2) + 4 + (c & 3);
}

__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
  r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
  return r;
}
__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
  bf16x4 r;
  r[0] = (bf16)x[0]; r[1] = (bf16)x[1]; r[2] = (bf16)x[2]; r[3] = (bf16)x[3];
  return r;
}
__device__ __forceinline__ f32x4 unpack4(bf16x4 x) {
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}
__device__ __forceinline__ f32x4 ld4(const float *p) {
  const float4 v = *reinterpret_cast<const float4 *>(p);
  return f32x4{v.x, v.y, v.z, v.w};
}

// exp(x) and log(x) through the hardware base-2 units.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ float fast_log(float x) {
  return __builtin_amdgcn_logf(x) * 0.6931471805599453f;
}

// Cross-lane moves inside rows of 16 lanes (DPP): no LDS traffic.
template <int CTRL, int ROW_MASK = 0xf, bool BOUND_ZERO = true>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}
// Inclusive prefix sum over lanes 0..31 (and, separately, 32..63).
__device__ __forceinline__ float scan32(float x) {
  x += dpp<0x111>(x);  // row_shr:1
  x += dpp<0x112>(x);  // row_shr:2
  x += dpp<0x114>(x);  // row_shr:4
  x += dpp<0x118>(x);  // row_shr:8
  x += dpp<0x142, 0xa, false>(x);  // row_bcast:15 into rows 1 and 3
  return x;
}

// Order this wave's LDS writes before its later LDS reads of other lanes' data.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
}

// Row pitches (elements) of the LDS tiles, padded by 16 bytes so that the 16
// rows one operand read touches fall in different banks.
constexpr int KP = DK + 8;   // bf16 [32][KP]: k, q rows, d_k in slot order
constexpr int TP = CH + 8;   // bf16 [32][TP]: P rows x chunk slots
constexpr int VP = BV + 8;   // bf16 [32][VP]: v rows

struct Stage {
  alignas(16) bf16 K[CH][KP];    // raw k rows                        (staging)
  alignas(16) bf16 Q[CH][KP];    // raw q rows                        (staging)
  alignas(16) bf16 V[CH][VP];    // raw v rows (this workgroup's columns) (staging)
  alignas(16) bf16 P[CH][TP];    // P, columns in slot order          (P1)
  alignas(16) bf16 T[2][16][16]; // (I + A_bb)^-1, natural rows       (P0)
  alignas(16) bf16 nA21[16][16]; // -A_21                             (P0)
  alignas(16) float gam[CH];     // cumulative log decay              (staging)
  alignas(16) float beta[CH];    //                                   (staging)
  alignas(16) float Gam[CH];     // exp(gam)                          (staging)
  alignas(16) float tail[CH];    // exp(gam_last - gam)               (staging)
  alignas(16) float ik[CH];      // 1/|k_r| (0 past the end)          (P0)
  alignas(16) float cR[CH];      // beta Gam ik                       (P0)
  alignas(16) float cD[CH];      // tail ik                           (P0)
  alignas(16) float cO[CH];      // Gam iq                            (P1)
  alignas(16) float Gc;          // exp(gam_last)                     (staging)
  int cl;                        // valid rows of the chunk           (staging)
};

struct Smem {
  Stage st[NSTAGE];
  alignas(16) float p1_ik[CH];   // P1's private copy of 1/|k|
  alignas(16) float p1_iq[CH];   // P1's private copy of scale/|q|
};

struct MfmaParams {
  const bf16 *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  const float *s0;
  bf16 *o;
  float *sT;
  const int32_t *cu;
  int seq_len;
  int num_seqs;
  int H_k, H_v;
  float scale, eps;
};

// Raw rows of one chunk, prefetched by one staging lane sl = 0..127: a block
// of 4 consecutive rows (row quad rq = sl / 16) by 8 columns of k and q
// (d = 8 (sl % 16) ..), the same 4 rows by 2 columns of v, and a_r, b_r of
// row sl % 32.
struct Raw {
  uint4 k[4], q[4];
  uint32_t v[4];
  uint16_t a, b;
};

// Map the launch index so that the workgroups of one (sequence, key head)
// land on the same XCD (blocks are dealt round-robin to the 8 XCDs), sharing
// that XCD's L2 for their common k and q rows.
__device__ __forceinline__ int unit_of_block(int b, int nb) {
  if ((nb & 7) != 0) return b;
  return (b & 7) * (nb >> 3) + (b >> 3);
}

// Issue the loads of one chunk's raw rows (cl >= 1 valid rows).  The loads
// are unconditional -- rows past the end re-read the last valid row; their
// norms, gates and decays are zeroed when the chunk is prepared -- so that
// nothing consumes them here and they stay in flight across the barriers
// until the chunk is staged two steps later.
__device__ __forceinline__ void load_chunk(const MfmaParams &p, Raw &R, int sl, int64_t row0,
                                           int cl, int hk, int h, int col0) {
  const int rq = sl >> 4, db = sl & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(4 * rq + i, cl - 1);
    R.k[i] = *reinterpret_cast<const uint4 *>(p.k + ((row0 + r) * p.H_k + hk) * DK + 8 * db);
    R.q[i] = *reinterpret_cast<const uint4 *>(p.q + ((row0 + r) * p.H_k + hk) * DK + 8 * db);
    R.v[i] = *reinterpret_cast<const uint32_t *>(p.v + ((row0 + r) * p.H_v + h) * DV + col0 + 2 * db);
  }
  const int r = min(sl & 31, cl - 1);
  R.a = __builtin_bit_cast(uint16_t, p.a[(row0 + r) * p.H_v + h]);
  R.b = __builtin_bit_cast(uint16_t, p.b[(row0 + r) * p.H_v + h]);
}

// Staging waves: lay out one chunk from registers (sl = 0..127).
__device__ __forceinline__ void stage_chunk(const Raw &R, Stage &S, int sl, int cl,
                                            float neg_exp_A, float dtb) {
  const int rq = sl >> 4, db = sl & 15;
  const int kb = db >> 2, c0 = 8 * (db & 3);
  const int s0 = 32 * kb + slot_of(c0), s1 = 32 * kb + slot_of(c0 + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint2 *>(&S.K[4 * rq + i][s0]) = make_uint2(R.k[i].x, R.k[i].y);
    *reinterpret_cast<uint2 *>(&S.K[4 * rq + i][s1]) = make_uint2(R.k[i].z, R.k[i].w);
    *reinterpret_cast<uint2 *>(&S.Q[4 * rq + i][s0]) = make_uint2(R.q[i].x, R.q[i].y);
    *reinterpret_cast<uint2 *>(&S.Q[4 * rq + i][s1]) = make_uint2(R.q[i].z, R.q[i].w);
  }
  // v rows: columns 2db, 2db + 1 of rows 4rq..4rq+3
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<uint32_t *>(&S.V[4 * rq + i][2 * db]) = R.v[i];
  // gates of row r = sl % 32, running sum over the 32 rows (every lane of both
  // staging waves derives the same values and stores them identically)
  {
    const int r = sl & 31;
    const bool valid = r < cl;
    const float a_r = __uint_as_float((uint32_t)R.a << 16) + dtb;
    const float b_r = __uint_as_float((uint32_t)R.b << 16);
    const float sp = fmaxf(a_r, 0.f) + fast_log(1.f + fast_exp(-fabsf(a_r)));
    const float g = valid ? neg_exp_A * sp : 0.f;
    const float bt = valid ? __builtin_amdgcn_rcpf(1.f + fast_exp(-b_r)) : 0.f;
    const float cum = scan32(g);
    const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 31));
    S.gam[r] = cum;
    S.beta[r] = bt;
    S.Gam[r] = fast_exp(cum);
    S.tail[r] = fast_exp(last - cum);
    S.Gc = fast_exp(last);
    S.cl = cl;
  }
}

// Transposed operand from a row-major tile with the transposing LDS read
// (ds_read_b64_tr_b16): within each group of 16 lanes, lane i receives
// element i%4 of the 8-byte pieces addressed by lanes 4j + i/4, j = 0..3.
// Lane (m, g) asks for the 4 columns c0 + 4(m%4).. of row r0 + 4g + m/4 and
// receives column c0 + m of rows r0 + 4g + j: a 4-row slice of the
// transpose.  `row_ptr(r, c)` gives the address of element (r, c).
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x4 tr_read(const bf16 *addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(addr));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// A operand of row r, 32-block kb of d_k, from a [32][KP] tile.
__device__ __forceinline__ bf16x8 row_op(const bf16 (*X)[KP], int r, int kb, int g) {
  return *reinterpret_cast<const bf16x8 *>(&X[r][32 * kb + 8 * g]);
}

// (I + N)^-1 for one strictly lower 16x16 block N, given in both lane layouts:
//   na[j] = N[m][4g+j] (A operand layout), nb[j] = N[4g+j][m] (B/accumulator layout).
// Returns T[m][4g+j] (A operand layout).  Transposes ride along: the
// accumulator of X Y is the B layout of X Y, that of Y^T X^T its A layout.
__device__ __forceinline__ f32x4 unit_lower_inverse(f32x4 na, f32x4 nb, int m, int g) {
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x4 na_h = pack4(na), nb_h = pack4(nb);
  const bf16x4 na_l = pack4(na - unpack4(na_h)), nb_l = pack4(nb - unpack4(nb_h));
  // N^2 (split) and (N^2)^T
  f32x4 n2 = mma16(na_h, nb_h, z);
  n2 = mma16(na_l, nb_h, n2);
  n2 = mma16(na_h, nb_l, n2);
  const f32x4 n2t = mma16(nb_h, na_h, z);
  const bf16x4 n2b_h = pack4(n2), n2a = pack4(n2t);
  const bf16x4 n2b_l = pack4(n2 - unpack4(n2b_h));
  // N^4, (N^4)^T, N^8
  const f32x4 n4 = mma16(n2a, n2b_h, z);
  const f32x4 n4t = mma16(n2b_h, n2a, z);
  const bf16x4 n4b = pack4(n4), n4a = pack4(n4t);
  const bf16x4 n8b = pack4(mma16(n4a, n4b, z));
  // pt[j] = P_k[m][4g+j]:  P_1 = I - N,  P_{k+1} = P_k (I + N^(2^k)),
  // i.e. P_{k+1}^T = P_k^T + (N^(2^k))^T P_k^T.
  f32x4 pt;
#pragma unroll
  for (int j = 0; j < 4; ++j) pt[j] = (m == 4 * g + j ? 1.f : 0.f) - na[j];
  const bf16x4 ptb = pack4(pt);
  const f32x4 acc = mma16(n2b_h, ptb, pt);
  pt = mma16(n2b_l, ptb, acc);
  pt = mma16(n4b, pack4(pt), pt);
  pt = mma16(n8b, pack4(pt), pt);
  return pt;
}

// P0: Gram blocks of k, 1/|k|, T_11, T_22, -A_21 of one chunk.
__device__ __forceinline__ void prepare_p0(const MfmaParams &p, Stage &S, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int cl = S.cl;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 t00 = z, t11 = z, t01 = z;  // (K K^T) blocks: rows 4g+j, column m (+16)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 k0 = row_op(S.K, m, kb, g), k1 = row_op(S.K, 16 + m, kb, g);
    t00 = mma32(k0, k0, t00);
    t11 = mma32(k1, k1, t11);
    t01 = mma32(k0, k1, t01);
  }
  // 1/|k_r| from the diagonal: lane (m, g = m/4) holds |k_m|^2 in register m%4
  if (g == (m >> 2)) {
    const int j = m & 3;
    S.ik[m] = (m < cl) ? rsqrtf(t00[j] + p.eps) : 0.f;
    S.ik[16 + m] = (16 + m < cl) ? rsqrtf(t11[j] + p.eps) : 0.f;
  }
  wave_lds_sync();
  const f32x4 ik_lo = ld4(&S.ik[4 * g]), ik_hi = ld4(&S.ik[16 + 4 * g]);
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const f32x4 bt_lo = ld4(&S.beta[4 * g]), bt_hi = ld4(&S.beta[16 + 4 * g]);
  const float ik_m0 = S.ik[m], ik_m1 = S.ik[16 + m];
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  const float bt_m0 = S.beta[m], bt_m1 = S.beta[16 + m];
  // A in both layouts for the two diagonal blocks, and -A_21 in A layout.
  // (K K^T)[4g+j][m] = (K K^T)[m][4g+j]: one accumulator serves both layouts.
  f32x4 na0, nb0, na1, nb1;
  bf16x4 na21;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 4 * g + j;
    nb0[j] = (m < r) ? bt_lo[j] * fast_exp(fminf(gm_lo[j] - gm_m0, 0.f)) * ik_lo[j] * ik_m0 * t00[j] : 0.f;
    na0[j] = (r < m) ? bt_m0 * fast_exp(fminf(gm_m0 - gm_lo[j], 0.f)) * ik_m0 * ik_lo[j] * t00[j] : 0.f;
    nb1[j] = (m < r) ? bt_hi[j] * fast_exp(fminf(gm_hi[j] - gm_m1, 0.f)) * ik_hi[j] * ik_m1 * t11[j] : 0.f;
    na1[j] = (r < m) ? bt_m1 * fast_exp(fminf(gm_m1 - gm_hi[j], 0.f)) * ik_m1 * ik_hi[j] * t11[j] : 0.f;
    // A_21[m][r] = beta_{16+m} exp(gam_{16+m} - gam_r) ik_{16+m} ik_r (K K^T)[r][16+m]
    na21[j] = (bf16)(-(bt_m1 * fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * ik_m1 * ik_lo[j] * t01[j]));
  }
  *reinterpret_cast<bf16x4 *>(&S.nA21[m][4 * g]) = na21;
  const f32x4 T0 = unit_lower_inverse(na0, nb0, m, g);
  const f32x4 T1 = unit_lower_inverse(na1, nb1, m, g);
  *reinterpret_cast<bf16x4 *>(&S.T[0][m][4 * g]) = pack4(T0);
  *reinterpret_cast<bf16x4 *>(&S.T[1][m][4 * g]) = pack4(T1);
  // per-row factors for the consumers
  if (lane < CH) {
    const int r = lane;
    const float ikr = S.ik[r];
    S.cR[r] = S.beta[r] * S.Gam[r] * ikr;
    S.cD[r] = S.tail[r] * ikr;
  }
}

// P1: norms of q (and its own copy of those of k), P and Gam iq.
__device__ __forceinline__ void prepare_p1(const MfmaParams &p, Stage &S, Smem &sm, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const int cl = S.cl;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 kk0 = z, kk1 = z, qq0 = z, qq1 = z;  // Gram diagonal blocks of k and q
  f32x4 p00 = z, p10 = z, p11 = z;  // (K Q^T) blocks: (q_r . k_i), r = 16 rb + m, i = 16 ib + 4g + j
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 k0 = row_op(S.K, m, kb, g), k1 = row_op(S.K, 16 + m, kb, g);
    const bf16x8 q0 = row_op(S.Q, m, kb, g), q1 = row_op(S.Q, 16 + m, kb, g);
    kk0 = mma32(k0, k0, kk0);
    kk1 = mma32(k1, k1, kk1);
    qq0 = mma32(q0, q0, qq0);
    qq1 = mma32(q1, q1, qq1);
    p00 = mma32(k0, q0, p00);
    p10 = mma32(k0, q1, p10);
    p11 = mma32(k1, q1, p11);
  }
  if (g == (m >> 2)) {
    const int j = m & 3;
    sm.p1_ik[m] = (m < cl) ? rsqrtf(kk0[j] + p.eps) : 0.f;
    sm.p1_ik[16 + m] = (16 + m < cl) ? rsqrtf(kk1[j] + p.eps) : 0.f;
    const float iq0 = (m < cl) ? rsqrtf(qq0[j] + p.eps) * p.scale : 0.f;
    const float iq1 = (16 + m < cl) ? rsqrtf(qq1[j] + p.eps) * p.scale : 0.f;
    sm.p1_iq[m] = iq0;
    sm.p1_iq[16 + m] = iq1;
    S.cO[m] = S.Gam[m] * iq0;
    S.cO[16 + m] = S.Gam[16 + m] * iq1;
  }
  wave_lds_sync();
  const f32x4 ik_lo = ld4(&sm.p1_ik[4 * g]), ik_hi = ld4(&sm.p1_ik[16 + 4 * g]);
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const float iq_m0 = sm.p1_iq[m], iq_m1 = sm.p1_iq[16 + m];
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  f32x4 v00, v10, v11;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * g + j;  // column inside its 16-block
    v00[j] = (i <= m) ? fast_exp(fminf(gm_m0 - gm_lo[j], 0.f)) * iq_m0 * ik_lo[j] * p00[j] : 0.f;
    v10[j] = fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * iq_m1 * ik_lo[j] * p10[j];
    v11[j] = (i <= m) ? fast_exp(fminf(gm_m1 - gm_hi[j], 0.f)) * iq_m1 * ik_hi[j] * p11[j] : 0.f;
  }
  const int s_lo = slot_of(4 * g), s_hi = slot_of(16 + 4 * g);
  *reinterpret_cast<bf16x4 *>(&S.P[m][s_lo]) = pack4(v00);
  *reinterpret_cast<bf16x4 *>(&S.P[m][s_hi]) = pack4(z);
  *reinterpret_cast<bf16x4 *>(&S.P[16 + m][s_lo]) = pack4(v10);
  *reinterpret_cast<bf16x4 *>(&S.P[16 + m][s_hi]) = pack4(v11);
}

__global__ __launch_bounds__(64 * NWAVES) void chunked_mfma_kernel(MfmaParams p) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  constexpr int NVB = DV / BV;

  const int unit = unit_of_block(blockIdx.x, gridDim.x);
  const int vb = unit % NVB;
  const int h = (unit / NVB) % p.H_v;
  const int n = unit / (NVB * p.H_v);
  const int hk = h / (p.H_v / p.H_k);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;

  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const int64_t L = t1 - t0;
  const int nch = (int)((L + CH - 1) / CH);
  const size_t state_off = ((size_t)n * p.H_v + h) * DK * DV;
  const float neg_exp_A = -expf(p.A_log[h]);
  const float dtb = p.dt_bias[h];
  const int col0 = vb * BV;
  // step `it` consumes chunk it-2, prepares chunk it-1 and stages chunk it;
  // the step count is even so that the staging loop below, unrolled by two,
  // has a straight-line body (an idle step at the end when nch is odd)
  const int nsteps = (nch + 3) & ~1;

  if (wave >= W_C0 && wave < W_C0 + NC) {
    // ---------------------------------------------------------------- consumers
    const int cw = wave - W_C0;
    const int col = col0 + 16 * cw + m;
    f32x4 S[8];  // S[16t + 4g + j][col]
    if (p.s0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[t][j] = p.s0[state_off + (size_t)(16 * t + 4 * g + j) * DV + col];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
    for (int it = 0; it < nsteps; ++it) {
      const int c = it - 2;
      if (c >= 0 && c < nch) {
        const Stage &st = sm.st[c % NSTAGE];
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        // ks[mt]: (K S)[16mt + 4g + j][m];  qsT[mt]: (Q S)[16mt + m][4g + j]
        f32x4 ks[2] = {z, z}, qsT[2] = {z, z};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            ks[mt] = mma32(row_op(st.K, 16 * mt + m, kb, g), Sb[kb], ks[mt]);
            qsT[mt] = mma32(Sb[kb], row_op(st.Q, 16 * mt + m, kb, g), qsT[mt]);
          }
        }
        // R = beta V - (beta Gam ik) K S, rows 4g..4g+3 and 16+4g..16+4g+3
        // v[4g + j][col] and v[16 + 4g + j][col] (transposing reads of v rows)
        const int vc = 16 * cw + 4 * (m & 3);
        const bf16x8 vv = cat8(tr_read(&st.V[4 * g + (m >> 2)][vc]),
                               tr_read(&st.V[16 + 4 * g + (m >> 2)][vc]));
        const f32x4 bt0 = ld4(&st.beta[4 * g]), bt1 = ld4(&st.beta[16 + 4 * g]);
        const f32x4 cr0 = ld4(&st.cR[4 * g]), cr1 = ld4(&st.cR[16 + 4 * g]);
        f32x4 R0, R1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          R0[j] = bt0[j] * (float)vv[j] - cr0[j] * ks[0][j];
          R1[j] = bt1[j] * (float)vv[4 + j] - cr1[j] * ks[1][j];
        }
        // Delta_1 = T11 R1; Delta_2 = T22 (R2 - A21 Delta_1)
        const bf16x4 t11 = *reinterpret_cast<const bf16x4 *>(&st.T[0][m][4 * g]);
        const bf16x4 t22 = *reinterpret_cast<const bf16x4 *>(&st.T[1][m][4 * g]);
        const bf16x4 na21 = *reinterpret_cast<const bf16x4 *>(&st.nA21[m][4 * g]);
        const f32x4 d1 = mma16(t11, pack4(R0), z);
        const f32x4 r2 = mma16(na21, pack4(d1), R1);
        const f32x4 d2 = mma16(t22, pack4(r2), z);
        const bf16x8 Db = pack8(d1, d2);
        // O^T = Delta^T P^T + (Gam iq Q S)^T: lane (m, g) gets O[16mt + m][4g..4g+3]
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int r = 16 * mt + m;
          const bf16x8 bp = *reinterpret_cast<const bf16x8 *>(&st.P[r][8 * g]);
          const f32x4 oc = mma32(Db, bp, qsT[mt] * st.cO[r]);
          const int64_t row = t0 + (int64_t)c * CH + r;
          if (row < t1)
            *reinterpret_cast<bf16x4 *>(p.o + (row * p.H_v + h) * DV + col0 + 16 * cw + 4 * g) =
                pack4(oc);
        }
        // S <- Gam_last S + K^T diag(tail ik) Delta
        const f32x4 cd0 = ld4(&st.cD[4 * g]), cd1 = ld4(&st.cD[16 + 4 * g]);
        const bf16x8 Dp = pack8(cd0 * d1, cd1 * d2);
        const float gc = st.Gc;
        // A operand k^T[16t + m][slots 8g..8g+7] = k[4g + j][16t + m], k[16 + 4g + j][16t + m]
        // read transposed from the row-major k tile (d_k in slot order per 32-block:
        // four consecutive d stay contiguous)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kc = 32 * (t >> 1) + slot_of(16 * (t & 1) + 4 * (m & 3));
          const bf16x8 akt = cat8(tr_read(&st.K[4 * g + (m >> 2)][kc]),
                                  tr_read(&st.K[16 + 4 * g + (m >> 2)][kc]));
          S[t] = mma32(akt, Dp, S[t] * gc);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
      }
      __syncthreads();
    }
    if (p.sT) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.sT[state_off + (size_t)(16 * t + 4 * g + j) * DV + col] = S[t][j];
    }
  } else if (wave == W_P0 || wave == W_P1) {
    // ---------------------------------------------------------------- prepare
    for (int it = 0; it < nsteps; ++it) {
      const int c = it - 1;
      if (c >= 0 && c < nch) {
        if (wave == W_P0)
          prepare_p0(p, sm.st[c % NSTAGE], lane);
        else
          prepare_p1(p, sm.st[c % NSTAGE], sm, lane);
      }
      __syncthreads();
    }
  } else {
    // ---------------------------------------------------------------- staging
    const int sl = threadIdx.x - 64 * W_ST0;  // 0..127
    Raw ra, rb;  // raw rows of even / odd chunks
    auto rows_of = [&](int c, int64_t &row0, int &cl) {
      row0 = t0 + (int64_t)c * CH;
      const int64_t rem = t1 - row0;
      cl = rem < CH ? (int)rem : CH;
    };
    auto load = [&](Raw &R, int c) {  // clamped to the last chunk: always valid
      int64_t row0;
      int cl;
      rows_of(min(c, nch - 1), row0, cl);
      load_chunk(p, R, sl, row0, cl, hk, h, col0);
    };
    auto stage = [&](Raw &R, int c) {
      int64_t row0;
      int cl;
      rows_of(c, row0, cl);
      stage_chunk(R, sm.st[c % NSTAGE], sl, cl, neg_exp_A, dtb);
    };
    if (nch == 0) {  // nothing to load; keep the barrier count
      for (int it = 0; it < nsteps; ++it) __syncthreads();
      return;
    }
    load(ra, 0);
    // keep the issue order ra-then-rb, as in the loop, so that the loads of
    // ra are always the older ones where the loop consumes them
    __builtin_amdgcn_sched_barrier(0);
    load(rb, 1);
    // Unrolled by two so that each register set is named statically.  The
    // body is straight-line: staging a chunk past the end writes a buffer no
    // one reads again, and loads are clamped to the last chunk.
    // The scheduling barriers keep every read of a register set ahead of the
    // loads that refill it, so that its own loads are always the oldest in
    // flight and the other set's stay in flight while it is staged.
    for (int it = 0; it < nsteps; it += 2) {
      stage(ra, it);
      __builtin_amdgcn_sched_barrier(0);
      load(ra, it + 2);
      __syncthreads();
      stage(rb, it + 1);
      __builtin_amdgcn_sched_barrier(0);
      load(rb, it + 3);
      __syncthreads();
    }
  }
}

hipError_t launch_kernel(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  MfmaParams p;
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
  p.num_seqs = pr.num_seqs;
  p.H_k = pr.H_k;
  p.H_v = pr.H_v;
  p.scale = pr.scale;
  p.eps = pr.eps;
  const int64_t grid = (int64_t)pr.num_seqs * pr.H_v * (DV / BV);
  if (grid == 0) return hipSuccess;
  const size_t smem = sizeof(Smem);
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(chunked_mfma_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(chunked_mfma_kernel, dim3((unsigned)grid), dim3(64 * NWAVES), smem, s, p);
  return hipGetLastError();
}

}  // namespace

bool chunked_mfma_supports(const Problem &p) {
  return p.dtype == GDR_BF16 && p.d_k == DK && p.d_v == DV && p.chunk == CH;
}

hipError_t launch_chunked_mfma(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  return launch_kernel(pr, x, s);
}

}  // namespace gdr
