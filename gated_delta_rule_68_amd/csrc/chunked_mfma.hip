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
// (I + A)^-1 is formed in 16-row blocks and then applied as one 32x32 product:
//   T = [T_11 0; T_21 T_22],  T_bb = (I + A_bb)^-1,  T_21 = -T_22 A_21 T_11.
// Each T_bb is formed on the matrix cores from the identity, exact for the
// strictly lower (nilpotent, N^16 = 0) N = A_bb,
//   (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8).
//
// Work split.  A workgroup owns (sequence, value head, 32 columns of d_v); the
// columns of S evolve independently.  Six waves, one workgroup barrier per
// chunk, three chunks in flight:
//   * 2 consumer waves each keep a [128 x 16] slice of S in MFMA accumulators
//     for the whole sequence and run chunk c: K S, Q S, Delta = T R, the
//     outputs and K^T Delta;
//   * 2 "prepare" waves form chunk c+1's matrices: P0 the Gram blocks of K
//     and T; P1 the output mask P;
//   * 2 staging waves lay out chunk c+2 from registers (rows of k, q and v,
//     their norms, gates and their running sum) and prefetch the raw rows of
//     chunks up to c+2+NPF.
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
constexpr int NSTAGE = 4;       // chunk buffers in LDS (three in use, one being filled ahead)
constexpr int NPF = NSTAGE;     // chunks whose raw rows a staging lane holds in registers

// wave roles (wave w runs on SIMD w % 4): the matrix-heavy consumers share a
// SIMD with the vector-heavy staging waves, P0 and P1 have one each
constexpr int W_C0 = 0, W_P0 = 2, W_P1 = 3, W_ST0 = 4;

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

// Sum over each row of 16 lanes, result in every lane of the row.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

// Sum of squares of the 8 bf16 values packed in a uint4 (bf16 pair dot products).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float sumsq8(const uint4 &x) {
  const bf16x2 w0 = __builtin_bit_cast(bf16x2, x.x), w1 = __builtin_bit_cast(bf16x2, x.y);
  const bf16x2 w2 = __builtin_bit_cast(bf16x2, x.z), w3 = __builtin_bit_cast(bf16x2, x.w);
  float s = __builtin_amdgcn_fdot2_f32_bf16(w0, w0, 0.f, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(w1, w1, s, false);
  s = __builtin_amdgcn_fdot2_f32_bf16(w2, w2, s, false);
  return __builtin_amdgcn_fdot2_f32_bf16(w3, w3, s, false);
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
  alignas(16) bf16 TT[CH][TP];   // (I + A)^-1, columns in slot order (P0)
  alignas(16) float gam[CH];     // cumulative log decay              (staging)
  alignas(16) float beta[CH];    //                                   (staging)
  alignas(16) float Gam[CH];     // exp(gam)                          (staging)
  alignas(16) float tail[CH];    // exp(gam_last - gam)               (staging)
  alignas(16) float ik[CH];      // 1/|k_r| (0 past the end)          (staging)
  float iq[CH];                  // scale/|q_r| (0 past the end); directly after ik (staging)
  alignas(16) float cR[CH];      // beta Gam ik                       (P0)
  alignas(16) float cD[CH];      // tail ik                           (P0)
  alignas(16) float cO[CH];      // Gam iq                            (P1)
  alignas(16) float Gc;          // exp(gam_last)                     (staging)
  int cl;                        // valid rows of the chunk           (staging)
};

struct Smem {
  Stage st[NSTAGE];
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
                                            float neg_exp_A, float dtb, float eps, float scale) {
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
  // row norms of k and q: the 16 lanes of row quad rq hold its 128 columns;
  // afterwards lane db < 4 stores 1/|k| of row 4rq+db, lane 4 <= db < 8
  // scale/|q| of row 4rq+db-4 (ik and iq are adjacent arrays)
  {
    float kk[4], qq[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kk[i] = sumsq8(R.k[i]);
      qq[i] = sumsq8(R.q[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kk[i] = row_sum16(kk[i]);
      qq[i] = row_sum16(qq[i]);
    }
    const int i = db & 3;
    const bool isq = (db & 4) != 0;
    const float k01 = (i & 1) ? kk[1] : kk[0], k23 = (i & 1) ? kk[3] : kk[2];
    const float q01 = (i & 1) ? qq[1] : qq[0], q23 = (i & 1) ? qq[3] : qq[2];
    const float ks = (i & 2) ? k23 : k01, qs = (i & 2) ? q23 : q01;
    const int r = 4 * rq + i;
    const float inv = r < cl ? rsqrtf((isq ? qs : ks) + eps) * (isq ? scale : 1.f) : 0.f;
    if (db < 8) S.ik[r + (isq ? CH : 0)] = inv;
  }
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
    if (sl == 0) {
      S.Gc = fast_exp(last);
      S.cl = cl;
    }
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
// The identity (I + N)^-1 = (I - N)(I + N^2)(I + N^4)(I + N^8) is exact since
// N^16 = 0, and its factors commute.  ta gets T[m][4g+j] (A layout) and, if
// requested, tb gets T[4g+j][m] (B layout).  Transposes ride along: the
// accumulator of X Y is the B layout of X Y, that of Y^T X^T its A layout.
template <bool WANT_B>
__device__ __forceinline__ void unit_lower_inverse(f32x4 na, f32x4 nb, int m, int g, f32x4 &ta,
                                                   f32x4 &tb) {
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const bf16x4 na_h = pack4(na), nb_h = pack4(nb);
  const bf16x4 n2b = pack4(mma16(na_h, nb_h, z));  // N^2
  const bf16x4 n2a = pack4(mma16(nb_h, na_h, z));  // (N^2)^T in B layout = N^2 in A layout
  const bf16x4 n4b = pack4(mma16(n2a, n2b, z));
  const bf16x4 n4a = pack4(mma16(n2b, n2a, z));
  const bf16x4 n8b = pack4(mma16(n4a, n4b, z));
  f32x4 id;
#pragma unroll
  for (int j = 0; j < 4; ++j) id[j] = (m == 4 * g + j) ? 1.f : 0.f;
  // A layout: P_{k+1}^T = P_k^T + (N^(2^k))^T P_k^T, P_1 = I - N
  f32x4 pt = id - na;
  pt = mma16(n2b, pack4(pt), pt);
  pt = mma16(n4b, pack4(pt), pt);
  ta = mma16(n8b, pack4(pt), pt);
  if (WANT_B) {
    // B layout: Q_{k+1} = Q_k + N^(2^k) Q_k, Q_1 = I - N
    const bf16x4 n8a = pack4(mma16(n4b, n4a, z));
    f32x4 q = id - nb;
    q = mma16(n2a, pack4(q), q);
    q = mma16(n4a, pack4(q), q);
    tb = mma16(n8a, pack4(q), q);
  }
}

// P0: Gram blocks of k and T = (I + A)^-1 of one chunk.
// Lane (m, g) holds the Gram entries (k_i . k_m), i = 4g + j, of each block;
// exactly one of i < m, i > m holds off the diagonal, so one decay factor
// exp(-|gam_m - gam_i|) serves both the A-operand (row m) and the B-operand
// (column m) layout of N.
__device__ __forceinline__ void prepare_p0(const MfmaParams &p, Stage &S, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 ik_lo = ld4(&S.ik[4 * g]), ik_hi = ld4(&S.ik[16 + 4 * g]);
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const f32x4 bt_lo = ld4(&S.beta[4 * g]), bt_hi = ld4(&S.beta[16 + 4 * g]);
  const float ik_m0 = S.ik[m], ik_m1 = S.ik[16 + m];
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  const float bt_m0 = S.beta[m], bt_m1 = S.beta[16 + m];
  f32x4 t00 = z, t11 = z, t01 = z;  // (K K^T) blocks: rows 4g+j, column m (+16)
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 k0 = row_op(S.K, m, kb, g), k1 = row_op(S.K, 16 + m, kb, g);
    t00 = mma32(k0, k0, t00);
    t11 = mma32(k1, k1, t11);
    t01 = mma32(k0, k1, t01);
  }
  // A in both layouts for the two diagonal blocks, and -A_21 in A layout.
  f32x4 na0, nb0, na1, nb1;
  bf16x4 na21;
  const float bik_m1 = bt_m1 * ik_m1;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * g + j;
    const float x0 = t00[j] * ik_m0 * ik_lo[j] * fast_exp(-fabsf(gm_m0 - gm_lo[j]));
    na0[j] = (i < m) ? bt_m0 * x0 : 0.f;
    nb0[j] = (i > m) ? bt_lo[j] * x0 : 0.f;
    const float x1 = t11[j] * ik_m1 * ik_hi[j] * fast_exp(-fabsf(gm_m1 - gm_hi[j]));
    na1[j] = (i < m) ? bt_m1 * x1 : 0.f;
    nb1[j] = (i > m) ? bt_hi[j] * x1 : 0.f;
    // A_21[m][i] = beta_{16+m} exp(gam_{16+m} - gam_i) ik_{16+m} ik_i (k_i . k_{16+m})
    na21[j] = (bf16)(-bik_m1 * ik_lo[j] * fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * t01[j]);
  }
  // T = (I + A)^-1 = [T11 0; T21 T22], T_bb = (I + A_bb)^-1, T21 = -T22 A21 T11
  f32x4 t11a, t11b, t22a, unused;
  unit_lower_inverse<true>(na0, nb0, m, g, t11a, t11b);
  unit_lower_inverse<false>(na1, nb1, m, g, t22a, unused);
  const f32x4 z4 = f32x4{0.f, 0.f, 0.f, 0.f};
  // Y = -A21 T11 (B layout); its accumulator is the A layout of Y^T, and
  // Y^T T22^T is the B layout of T21^T, i.e. the A layout of T21.
  const f32x4 y = mma16(na21, pack4(t11b), z4);
  const f32x4 t21a = mma16(pack4(y), pack4(t22a), z4);
  // rows of T with the column index in slot order: row m holds (T11[m][4g..], 0),
  // row 16 + m holds (T21[m][4g..], T22[m][4g..])
  const bf16x4 zb = pack4(z4);
  *reinterpret_cast<bf16x8 *>(&S.TT[m][8 * g]) = cat8(pack4(t11a), zb);
  *reinterpret_cast<bf16x8 *>(&S.TT[16 + m][8 * g]) = cat8(pack4(t21a), pack4(t22a));
  // per-row factors for the consumers
  if (lane < CH) {
    const int r = lane;
    const float ikr = S.ik[r];
    S.cR[r] = S.beta[r] * S.Gam[r] * ikr;
    S.cD[r] = S.tail[r] * ikr;
  }
}

// P1: P and Gam iq of one chunk.
__device__ __forceinline__ void prepare_p1(const MfmaParams &p, Stage &S, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 ik_lo = ld4(&S.ik[4 * g]), ik_hi = ld4(&S.ik[16 + 4 * g]);
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const float iq_m0 = S.iq[m], iq_m1 = S.iq[16 + m];
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  f32x4 p00 = z, p10 = z, p11 = z;  // (K Q^T) blocks: (q_r . k_i), r = 16 rb + m, i = 16 ib + 4g + j
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const bf16x8 k0 = row_op(S.K, m, kb, g), k1 = row_op(S.K, 16 + m, kb, g);
    const bf16x8 q0 = row_op(S.Q, m, kb, g), q1 = row_op(S.Q, 16 + m, kb, g);
    p00 = mma32(k0, q0, p00);
    p10 = mma32(k0, q1, p10);
    p11 = mma32(k1, q1, p11);
  }
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
  if (lane < CH) S.cO[lane] = S.Gam[lane] * S.iq[lane];
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
  // the step count is a multiple of NPF so that the staging loop below,
  // unrolled by NPF, has a straight-line body (idle steps at the end)
  const int nsteps = (nch + 2 + NPF - 1) / NPF * NPF;

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
    // Operands of the next chunk, read from LDS while this wave would
    // otherwise wait at the barrier: rows of k and q (A operands of K S and
    // the B operands of (Q S)^T), k^T (A operand of the state update) and v.
    // The rows of chunk it-1 are complete once step it-1 has ended.
    bf16x8 Kr[2][4], Qr[2][4], Kt[8], vv;
    auto read_operands = [&](const Stage &sn) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          Kr[mt][kb] = row_op(sn.K, 16 * mt + m, kb, g);
          Qr[mt][kb] = row_op(sn.Q, 16 * mt + m, kb, g);
        }
      // k^T[16t + m][slots 8g..8g+7] = k[4g + j][16t + m], k[16 + 4g + j][16t + m]
      // read transposed from the row-major k tile (d_k in slot order per
      // 32-block: four consecutive d stay contiguous)
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int kc = 32 * (t >> 1) + slot_of(16 * (t & 1) + 4 * (m & 3));
        Kt[t] = cat8(tr_read(&sn.K[4 * g + (m >> 2)][kc]), tr_read(&sn.K[16 + 4 * g + (m >> 2)][kc]));
      }
      // v[4g + j][col] and v[16 + 4g + j][col]
      const int vc = 16 * cw + 4 * (m & 3);
      vv = cat8(tr_read(&sn.V[4 * g + (m >> 2)][vc]), tr_read(&sn.V[16 + 4 * g + (m >> 2)][vc]));
    };
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
            ks[mt] = mma32(Kr[mt][kb], Sb[kb], ks[mt]);
            qsT[mt] = mma32(Sb[kb], Qr[mt][kb], qsT[mt]);
          }
        }
        // R = beta V - (beta Gam ik) K S, rows 4g..4g+3 and 16+4g..16+4g+3
        const f32x4 bt0 = ld4(&st.beta[4 * g]), bt1 = ld4(&st.beta[16 + 4 * g]);
        const f32x4 cr0 = ld4(&st.cR[4 * g]), cr1 = ld4(&st.cR[16 + 4 * g]);
        f32x4 R0, R1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          R0[j] = bt0[j] * (float)vv[j] - cr0[j] * ks[0][j];
          R1[j] = bt1[j] * (float)vv[4 + j] - cr1[j] * ks[1][j];
        }
        // Delta = T R: rows 0..15 and 16..31 of T against R in slot order
        const bf16x8 Rb = pack8(R0, R1);
        const bf16x8 ta0 = *reinterpret_cast<const bf16x8 *>(&st.TT[m][8 * g]);
        const bf16x8 ta1 = *reinterpret_cast<const bf16x8 *>(&st.TT[16 + m][8 * g]);
        const f32x4 d1 = mma32(ta0, Rb, z);
        const f32x4 d2 = mma32(ta1, Rb, z);
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
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mma32(Kt[t], Dp, S[t] * gc);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = pack8(S[2 * kb], S[2 * kb + 1]);
      }
      if (it - 1 >= 0 && it - 1 < nch) read_operands(sm.st[(it - 1) % NSTAGE]);
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
          prepare_p1(p, sm.st[c % NSTAGE], lane);
      }
      __syncthreads();
    }
  } else {
    // ---------------------------------------------------------------- staging
    const int sl = threadIdx.x - 64 * W_ST0;  // 0..127
    Raw raw[NPF];  // raw rows of chunks it, it+1, ..., it+NPF-1
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
    auto stage = [&](Raw &R, int c, Stage &buf) {
      int64_t row0;
      int cl;
      rows_of(c, row0, cl);
      stage_chunk(R, buf, sl, cl, neg_exp_A, dtb, p.eps, p.scale);
    };
    if (nch == 0) {  // nothing to load; keep the barrier count
      for (int it = 0; it < nsteps; ++it) __syncthreads();
      return;
    }
    // Keep the issue order of the register sets as in the loop, so that the
    // loads of the set staged next are always the oldest in flight.
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      load(raw[u], u);
      __builtin_amdgcn_sched_barrier(0);
    }
    // Unrolled by NPF so that each register set is named statically.  The
    // body is straight-line: staging a chunk past the end writes a buffer no
    // one reads again, and loads are clamped to the last chunk.
    // The scheduling barriers keep every read of a register set ahead of the
    // loads that refill it, so that its own loads are always the oldest in
    // flight and the other sets' stay in flight while it is staged.
    for (int it = 0; it < nsteps; it += NPF) {
#pragma unroll
      for (int u = 0; u < NPF; ++u) {
        stage(raw[u], it + u, sm.st[u]);  // (it + u) % NSTAGE == u
        __builtin_amdgcn_sched_barrier(0);
        load(raw[u], it + u + NPF);
        __syncthreads();
      }
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
