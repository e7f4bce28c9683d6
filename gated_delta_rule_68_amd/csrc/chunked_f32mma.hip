// Chunked (UT-transform) form of the gated delta rule for fp32 inputs on the
// matrix cores in fp32 (v_mfma_f32_16x16x4_f32: fp32 operands, fp32
// products and sums), for d_k = 64 or 128, d_v = 16, 32, 64 or 128 and
// chunk 32.  Same regrouping and the same arithmetic as chunked_vec.hip
// (GatedDeltaRule.ixx File Reference, "Detailed Description": one triangular
// solve per chunk; Track L pull request, L2: the only non-GEMM step is the
// (I + A)^-1 forward substitution), with its dense products on the matrix
// cores instead of the vector ALUs.  For a chunk of 32 tokens with state S
// at entry, gamma_r the in-chunk cumulative log decay, ik_r = 1/|k_r|,
// iq_r = scale/|q_r| (raw rows k, q):
//   A[r][i] = beta_r exp(gamma_r - gamma_i) ik_r ik_i (k_r . k_i)   i < r
//   P[r][i] = exp(gamma_r - gamma_i) iq_r ik_i (q_r . k_i)          i <= r
//   KS = diag(ik) K S,  QS = diag(iq) Q S
//   T = (I + A)^-1 (forward substitution),  R = diag(beta) (V - diag(Gamma) KS)
//   Delta = T R,  O = diag(Gamma) QS + P Delta
//   S' = Gamma_last S + (diag(exp(gamma_last - gamma) ik) K)^T Delta
// Only differences gamma_r - gamma_i with i <= r are exponentiated.  A partial
// last chunk is padded with zero rows (k = q = v = 0, g = 0, beta = 0).
//
// Launch: one workgroup of four waves per (sequence, value head, 16 columns
// of d_v), the state slice [d_k, 16] in LDS across the chunk loop; the
// column blocks of a (sequence, head) share an XCD.  The raw
// rows of chunk c + 1 are loaded into registers while chunk c is computed,
// and chunk c + 1's gates are formed during chunk c (two gate buffers).
// Per chunk, after the rows are stored and their norms taken:
//   wave 0: the diagonal blocks A11, A22 and their inverses T11 = (I +
//           A11)^-1, T22 = (I + A22)^-1 by forward substitution (one column
//           of one block per pair of lanes);
//   wave 1: the blocks of P;
//   wave 2: K S and from it R (v read straight into the product layout),
//           and the block A21;
//   wave 3: Q S, kept in registers as the start of O, and the next gates;
// then Delta by block substitution on wave 0 (Delta0 = T11 R0, Delta1 =
// T22 (R1 - A21 Delta0): T itself is never formed), O (wave 3) and the
// state update (waves 0-2).
//
// Operand layout: in a product's group of 4 steps, lane group g takes the
// contraction indices 16q + 4g .. 16q + 4g + 3 (any order of the indices
// gives the same sum), so that a lane's 4 operands of a group are one
// 16-byte LDS read.  Tiles read that way keep the contraction index
// contiguous (the state slice, R, Delta and the diagonal blocks of A are
// stored transposed) with a row pitch of 8 mod 64 floats, which spreads
// every pass of such a read over all 16-byte bank slots.
#include "device_common.h"
#include "gdr_internal.h"

namespace gdr {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int CHF = 32;       // tokens per chunk
constexpr int BVF = 16;       // state columns per workgroup
constexpr int NTHREADS = 256;
constexpr int TP = CHF + 8;   // row pitch of the [.][32] tiles (floats)

// x of another lane by a DPP control (0 where the source lane is outside
// the row or the row is not in ROWS).
template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWS, 0xF, false));
}

// Sum of x over each row of 16 lanes, in every lane of the row: within
// quads, then half rows, then rows.
__device__ __forceinline__ float row_sum16(float x) {
  x += dpp<0xB1>(x);   // quad_perm 1,0,3,2
  x += dpp<0x4E>(x);   // quad_perm 2,3,0,1
  x += dpp<0x141>(x);  // row_half_mirror
  return x + dpp<0x140>(x);  // row_mirror
}

// Inclusive prefix sum of x over lanes 0..31, added in lane order (one
// running sum, as a sequential loop would form it): neighbouring sums then
// differ by one rounded addition, and the zero rows past a chunk's end keep
// the last real row's sum exactly, so exp(gamma_last - gamma_r) is exactly 1
// for the last token.  A tree scan rounds neighbours differently, which
// under strong decay (|gamma| in the hundreds) costs one ulp of gamma,
// about 3e-5, in that factor.
__device__ __forceinline__ float scan32(float x, int lane) {
  float acc = 0.f, out = 0.f;
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    acc += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), r));
    out = lane == r ? acc : out;
  }
  return out;
}

// D (16 x 16) += A (16 x 4) B (4 x 16): lane l = 16 g + m holds A[m][g] and
// B[g][m], and gets D rows 4g..4g+3 of column m.
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// A group of 4 steps: a and b hold the lane's operands of its 4 indices.
__device__ __forceinline__ f32x4 mma16(const f32x4 &a, const f32x4 &b, f32x4 c) {
  c = mma4(a[0], b[0], c);
  c = mma4(a[1], b[1], c);
  c = mma4(a[2], b[2], c);
  return mma4(a[3], b[3], c);
}
__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, const f32x4 &v) { *reinterpret_cast<f32x4 *>(p) = v; }

// Gates of one chunk: cumulative log decay, beta, exp of both ends.
struct Gates {
  float gam[CHF], beta[CHF], eg[CHF], tail[CHF];
};

template <int DK>
struct F32Smem {
  static constexpr int RP = DK + 8;  // row pitch of the [.][d_k] tiles
  float K[CHF][RP];    // raw k rows of the chunk (zero past its end)
  float Q[CHF][RP];    // raw q rows
  float ST[BVF][RP];   // the state slice, transposed: ST[j][d] = S[d][j]
  float AT[CHF][TP];   // diagonal blocks of A, transposed: AT[i][r] = A[r][i]
  float A21[16][TP];   // A[16 + r][i], r, i < 16
  float P[CHF][TP];    // lower part used (zero above the diagonal)
  float Tm[CHF][TP];   // diagonal blocks T11, T22 (lower parts used)
  float WT[BVF][TP];   // (R1 - A21 Delta0)^T
  float RT[BVF][TP];   // R^T
  float DT[BVF][TP];   // Delta^T
  Gates gt[2];         // this chunk's and the next one's
  float ik[CHF], iq[CHF], tk[CHF];
};

// Raw inputs of one chunk, held in registers from their load to their use.
// Lane (rg = lane / 16, c = lane % 16) of wave w holds rows
// 16 (w % 2) + rg + 4k (k < 4) of k (w < 2) or q, columns 64 f + 4c .. + 3.
template <int DK>
struct Rows {
  f32x4 kq[4][DK / 64];
  float v[8];   // wave 2: v rows 4g + j and 16 + 4g + j, column m
  float a, b;   // wave 3, lanes 0..31: the gate inputs of row lane
};

// Buffer resource over `bytes` bytes from `base` (raw, no stride): loads at
// byte offsets at or past `bytes` return 0, which pads the last chunk.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const float *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ float bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

// Loads chunk [c0, c0 + cl) (cl >= 1); rows past cl read as zero.
template <int DK>
__device__ __forceinline__ void load_rows(Rows<DK> &x, const Problem &pr, const FwdArgs &f,
                                          int64_t c0, int cl, int h, int hk, int vb, int wave,
                                          int lane) {
  x.a = x.b = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) x.v[u] = 0.f;
  if (wave == 3) {  // first: the gates of this chunk are needed before its rows
    const uint32_t grow = (uint32_t)pr.H_v * 4, gbytes = (uint32_t)(cl - 1) * grow + 4;
    const auto ra = rsrc(static_cast<const float *>(f.a) + c0 * pr.H_v + h, gbytes);
    const auto rb = rsrc(static_cast<const float *>(f.b) + c0 * pr.H_v + h, gbytes);
    const uint32_t off = lane < CHF ? (uint32_t)lane * grow : gbytes;  // lanes 32..63 read 0
    x.a = bload(ra, off);
    x.b = bload(rb, off);
  }
  const uint32_t krow = (uint32_t)pr.H_k * DK * 4;
  const float *kq = static_cast<const float *>(wave < 2 ? f.k : f.q) + (c0 * pr.H_k + hk) * DK;
  const auto rk = rsrc(kq, (uint32_t)(cl - 1) * krow + DK * 4);
  const uint32_t base = (uint32_t)(16 * (wave & 1) + (lane >> 4)) * krow + 16 * (lane & 15);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int e = 0; e < DK / 64; ++e) x.kq[k][e] = bload4(rk, base + 4 * k * krow + 256 * e);
  }
  if (wave == 2) {
    const int m = lane & 15, g = lane >> 4;
    const uint32_t vrow = (uint32_t)pr.H_v * pr.d_v * 4;
    const float *v = static_cast<const float *>(f.v) + (c0 * pr.H_v + h) * pr.d_v + vb * BVF;
    const auto rv = rsrc(v, (uint32_t)(cl - 1) * vrow + BVF * 4);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int r = 16 * (u >> 2) + 4 * g + (u & 3);
      x.v[u] = bload(rv, (uint32_t)r * vrow + 4 * m);
    }
  }
}

// Gates of a chunk of cl rows from the raw a, b of lane r (lanes 0..31).
__device__ __forceinline__ void make_gates(Gates &G, float a, float b, int cl, float neg_exp_A,
                                           float dtb, int lane) {
  const int r = lane;
  const float gr = scan32(r < cl ? log_decay(neg_exp_A, a, dtb) : 0.f, lane);
  G.gam[r] = gr;
  G.beta[r] = r < cl ? sigmoid_f32(b) : 0.f;
  G.eg[r] = expf(gr);
  const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gr), CHF - 1));
  G.tail[r] = expf(last - gr);
}

template <int DK>
__global__ __launch_bounds__(NTHREADS, 2) void chunked_f32mma_kernel(const Problem pr, const FwdArgs x) {
  static_assert(DK % 64 == 0, "tile shape");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  F32Smem<DK> &sm = *reinterpret_cast<F32Smem<DK> *>(smem_raw);
  float *o = static_cast<float *>(x.o);
  const int DV = pr.d_v;
  const int nvb = DV / BVF;
  // Workgroup b runs on XCD b % 8 (workgroups are dealt to the XCDs in
  // turn).  The (sequence, value head) units go to the XCDs in contiguous
  // blocks of uc, and all column blocks of a unit to its unit's XCD: they
  // read the same k and q rows, which then come from one L2.
  const int units = pr.num_seqs * pr.H_v, uc = (units + 7) / 8;
  const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
  const int unit = xcd * uc + slot / nvb;
  if (unit >= units) return;  // the padding of the last XCD's block
  const int vb = slot % nvb;
  const int h = unit % pr.H_v;
  const int n = unit / pr.H_v;
  const int hk = h / (pr.H_v / pr.H_k);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar branches
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z4 = {0.f, 0.f, 0.f, 0.f};

  int64_t t0, t1;
  seq_bounds(pr.cu, pr.seq_len, n, t0, t1);
  const size_t state_off = ((size_t)n * pr.H_v + h) * DK * DV + (size_t)vb * BVF;
  for (int e = tid; e < DK * BVF; e += NTHREADS) {
    const int d = e / BVF, j = e % BVF;
    sm.ST[j][d] = x.s0 ? x.s0[state_off + (size_t)d * DV + j] : 0.0f;
  }
  const float neg_exp_A = -expf(x.A_log[h]);
  const float dtb = x.dt_bias[h];
  auto chunk_len = [&](int64_t c) { return (int)((t1 - c) < CHF ? (t1 - c) : CHF); };

  Rows<DK> rows;
  if (t1 > t0) {
    load_rows(rows, pr, x, t0, chunk_len(t0), h, hk, vb, wave, lane);
    if (wave == 3 && lane < CHF) make_gates(sm.gt[0], rows.a, rows.b, chunk_len(t0), neg_exp_A, dtb, lane);
  }
  int pb = 0;  // gate buffer of this chunk
  for (int64_t c0 = t0; c0 < t1; c0 += CHF, pb ^= 1) {
    const int cl = chunk_len(c0);
    const Gates &G = sm.gt[pb];
    // -- the chunk's rows into LDS and their inverse norms
    {
      float(*X)[F32Smem<DK>::RP] = wave < 2 ? sm.K : sm.Q;
      const int r0 = 16 * (wave & 1) + (lane >> 4);
      float ss[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ss[k] = 0.f;
#pragma unroll
        for (int e = 0; e < DK / 64; ++e) {
          const f32x4 v = rows.kq[k][e];
          st4(&X[r0 + 4 * k][64 * e + 4 * (lane & 15)], v);
          ss[k] += v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
        }
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) ss[k] = row_sum16(ss[k]);
      // lane c < 4 of each row of 16 lanes writes row r0 + 4c
      const int c = lane & 15;
      const float mine = c == 0 ? ss[0] : c == 1 ? ss[1] : c == 2 ? ss[2] : ss[3];
      if (c < 4) {
        const int r = r0 + 4 * c;
        const float inv = r < cl ? rsqrtf(mine + pr.eps) : 0.f;
        (wave < 2 ? sm.ik : sm.iq)[r] = wave < 2 ? inv : inv * pr.scale;
      }
    }
    float vcur[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) vcur[u] = rows.v[u];
    // the next chunk's rows (and its gate inputs, rows.a and rows.b): in
    // flight during this chunk's products
    const bool more = c0 + CHF < t1;
    if (more) load_rows(rows, pr, x, c0 + CHF, chunk_len(c0 + CHF), h, hk, vb, wave, lane);
    __syncthreads();

    f32x4 o0 = z4, o1 = z4;  // wave 3: O rows 0..15 and 16..31
    if (wave < 2) {
      // raw Gram blocks (0,0), (1,1) and, for P, (1,0): K K^T (wave 0),
      // Q K^T (wave 1)
      const float(*Xr)[F32Smem<DK>::RP] = wave == 0 ? sm.K : sm.Q;
      // scale of each of this lane's 12 outputs (block b: (0,0), (1,1),
      // (1,0); element j: row 16 rb + 4g + j, column 16 cb + m), formed
      // while the products run: for A, beta_r ik_r ik_i exp(gamma_r -
      // gamma_i) with i < r; for P, iq_r ik_i exp(gamma_r - gamma_i), i <= r
      f32x4 fac[3];
      {
        const f32x4 gR0 = ld4(&G.gam[4 * g]), gR1 = ld4(&G.gam[16 + 4 * g]);
        const f32x4 bR0 = ld4(&G.beta[4 * g]), bR1 = ld4(&G.beta[16 + 4 * g]);
        const f32x4 kR0 = ld4(&sm.ik[4 * g]), kR1 = ld4(&sm.ik[16 + 4 * g]);
        const f32x4 qR0 = ld4(&sm.iq[4 * g]), qR1 = ld4(&sm.iq[16 + 4 * g]);
        const float gC0 = G.gam[m], gC1 = G.gam[16 + m], kC0 = sm.ik[m], kC1 = sm.ik[16 + m];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = 4 * g + j;  // row within its 16-row block
          const bool keep = wave == 0 ? m < r : m <= r;
          const float s0 = wave == 0 ? bR0[j] * kR0[j] : qR0[j];
          const float s1 = wave == 0 ? bR1[j] * kR1[j] : qR1[j];
          const float e0 = expf(fminf(gR0[j] - gC0, 0.f)), e1 = expf(fminf(gR1[j] - gC1, 0.f));
          const float e2 = expf(fminf(gR1[j] - gC0, 0.f));
          fac[0][j] = keep ? e0 * s0 * kC0 : 0.f;
          fac[1][j] = keep ? e1 * s1 * kC1 : 0.f;
          fac[2][j] = e2 * s1 * kC0;
        }
      }
      f32x4 d00 = z4, d11 = z4, d10 = z4;
#pragma unroll
      for (int q = 0; q < DK / 16; ++q) {
        const int d = 16 * q + 4 * g;
        const f32x4 x0 = ld4(&Xr[m][d]), x1 = ld4(&Xr[16 + m][d]);
        const f32x4 k0 = ld4(&sm.K[m][d]), k1 = ld4(&sm.K[16 + m][d]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          d00 = mma4(x0[u], k0[u], d00);
          d11 = mma4(x1[u], k1[u], d11);
          if (wave == 1) d10 = mma4(x1[u], k0[u], d10);
        }
      }
      if (wave == 1) {  // P, row-major
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          sm.P[4 * g + j][m] = fac[0][j] * d00[j];
          sm.P[16 + 4 * g + j][16 + m] = fac[1][j] * d11[j];
          sm.P[16 + 4 * g + j][m] = fac[2][j] * d10[j];
        }
      } else {
        // A11, A22 transposed: element j of lane (m, g) is A[4g + j][m] (+16)
        st4(&sm.AT[m][4 * g], fac[0] * d00);
        st4(&sm.AT[16 + m][16 + 4 * g], fac[1] * d11);
        // T11 and T22 by forward substitution in column order (once x_i is
        // final it is taken out of every later row), one column of one block
        // per pair of lanes: lane 32p + 16rb + col holds rows 8p .. 8p + 7 of
        // column col of T_rb, and x_i comes from the lane half that holds
        // row i by a permlane swap.  A[r][i] is zero for r <= i, so the
        // updates need no mask.  AT was written by this wave; its LDS
        // accesses complete in order.
        {
          const int part = lane >> 5, rb = (lane >> 4) & 1, col = lane & 15;
          float acc[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] = 8 * part + e == col ? 1.0f : 0.0f;
#pragma unroll
          for (int i = 0; i < 15; ++i) {
            const float xv = acc[i % 8];
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(xv), __float_as_uint(xv), false, false);
            const float xi = __uint_as_float(i < 8 ? sw[0] : sw[1]);  // lanes 0-31 hold rows 0..7
            const float *arow = &sm.AT[16 * rb + i][16 * rb + 8 * part];  // arow[e] = A[8p + e][i]
            const f32x4 a0 = ld4(arow), a1 = ld4(arow + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[e] -= a0[e] * xi;
              acc[4 + e] -= a1[e] * xi;
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.Tm[16 * rb + 8 * part + e][16 * rb + col] = acc[e];
        }
      }
    } else {
      // K S (wave 2) or Q S (wave 3), rows 0..15 and 16..31 of the chunk;
      // wave 2 also the raw Gram block K[16..31] K[0..15]^T of A21
      const float(*Xr)[F32Smem<DK>::RP] = wave == 2 ? sm.K : sm.Q;
      f32x4 d0 = z4, d1 = z4, d10 = z4;
#pragma unroll
      for (int q = 0; q < DK / 16; ++q) {
        const int d = 16 * q + 4 * g;
        const f32x4 sv = ld4(&sm.ST[m][d]);
        const f32x4 x0 = ld4(&Xr[m][d]), x1 = ld4(&Xr[16 + m][d]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          d0 = mma4(x0[u], sv[u], d0);
          d1 = mma4(x1[u], sv[u], d1);
          if (wave == 2) d10 = mma4(x1[u], x0[u], d10);
        }
      }
      const f32x4 eg0 = ld4(&G.eg[4 * g]), eg1 = ld4(&G.eg[16 + 4 * g]);
      if (wave == 2) {  // R = diag(beta) (V - diag(Gamma) diag(ik) K S), stored transposed
        const f32x4 b0 = ld4(&G.beta[4 * g]), b1 = ld4(&G.beta[16 + 4 * g]);
        const f32x4 k0 = ld4(&sm.ik[4 * g]), k1 = ld4(&sm.ik[16 + 4 * g]);
        f32x4 r0, r1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          r0[j] = b0[j] * (vcur[j] - eg0[j] * k0[j] * d0[j]);
          r1[j] = b1[j] * (vcur[4 + j] - eg1[j] * k1[j] * d1[j]);
        }
        st4(&sm.RT[m][4 * g], r0);
        st4(&sm.RT[m][16 + 4 * g], r1);
        // A21[4g + j][m] = beta_r ik_r ik_m exp(gamma_r - gamma_m) (K K^T)[r][m],
        // r = 16 + 4g + j
        const float gC = G.gam[m], kC = sm.ik[m];
        const f32x4 gR = ld4(&G.gam[16 + 4 * g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) sm.A21[4 * g + j][m] = expf(gR[j] - gC) * b1[j] * k1[j] * kC * d10[j];
      } else {
        // O starts at diag(Gamma) diag(iq) Q S
        const f32x4 q0 = ld4(&sm.iq[4 * g]), q1 = ld4(&sm.iq[16 + 4 * g]);
        o0 = eg0 * q0 * d0;
        o1 = eg1 * q1 * d1;
        if (lane < CHF) {
          sm.tk[lane] = G.tail[lane] * sm.ik[lane];
          // the next chunk's gates, into the other buffer
          if (more) make_gates(sm.gt[pb ^ 1], rows.a, rows.b, chunk_len(c0 + CHF), neg_exp_A, dtb, lane);
        }
      }
    }
    __syncthreads();
    // -- Delta, the solution of (I + A) Delta = R, by blocks (wave 0; its
    //    LDS accesses complete in order): Delta0 = T11 R0, then
    //    Delta1 = T22 (R1 - A21 Delta0)
    if (wave == 0) {
      const f32x4 d0 = mma16(ld4(&sm.Tm[m][4 * g]), ld4(&sm.RT[m][4 * g]), z4);
      st4(&sm.DT[m][4 * g], d0);
      const f32x4 w = mma16(-ld4(&sm.A21[m][4 * g]), ld4(&sm.DT[m][4 * g]), ld4(&sm.RT[m][16 + 4 * g]));
      st4(&sm.WT[m][4 * g], w);
      st4(&sm.DT[m][16 + 4 * g], mma16(ld4(&sm.Tm[16 + m][16 + 4 * g]), ld4(&sm.WT[m][4 * g]), z4));
    }
    __syncthreads();
    if (wave == 3) {
      // -- O += P Delta (P12 = 0)
      const f32x4 dl0 = ld4(&sm.DT[m][4 * g]), dl1 = ld4(&sm.DT[m][16 + 4 * g]);
      const f32x4 p00 = ld4(&sm.P[m][4 * g]), p10 = ld4(&sm.P[16 + m][4 * g]);
      const f32x4 p11 = ld4(&sm.P[16 + m][16 + 4 * g]);
      o0 = mma16(p00, dl0, o0);
      o1 = mma16(p10, dl0, o1);
      o1 = mma16(p11, dl1, o1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r0 = 4 * g + j, r1 = 16 + 4 * g + j;
        if (r0 < cl) o[((c0 + r0) * pr.H_v + h) * DV + vb * BVF + m] = o0[j];
        if (r1 < cl) o[((c0 + r1) * pr.H_v + h) * DV + vb * BVF + m] = o1[j];
      }
    } else {
      // -- S' = Gamma_last S + (diag(tail ik) K)^T Delta; wave w < 3 owns
      //    state rows 16t..16t+15 for t = w, w + 3, ... (read and written by
      //    it alone)
      const float gc = G.eg[CHF - 1];
      const f32x4 tk0 = ld4(&sm.tk[4 * g]), tk1 = ld4(&sm.tk[16 + 4 * g]);
      const f32x4 dl0 = ld4(&sm.DT[m][4 * g]), dl1 = ld4(&sm.DT[m][16 + 4 * g]);
#pragma unroll
      for (int u = 0; u < (DK / 16 + 2) / 3; ++u) {
        const int t = wave + 3 * u;
        if (t < DK / 16) {
          f32x4 a0, a1;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            a0[s] = sm.K[4 * g + s][16 * t + m];
            a1[s] = sm.K[16 + 4 * g + s][16 * t + m];
          }
          const f32x4 s4 = ld4(&sm.ST[m][16 * t + 4 * g]);
          f32x4 d = gc * s4;
          d = mma16(tk0 * a0, dl0, d);
          d = mma16(tk1 * a1, dl1, d);
          st4(&sm.ST[m][16 * t + 4 * g], d);
        }
      }
    }
    __syncthreads();  // before the next chunk overwrites K, Q, ik, iq and DT
  }
  if (x.sT) {
    for (int e = tid; e < DK * BVF; e += NTHREADS) {
      const int d = e / BVF, j = e % BVF;
      x.sT[state_off + (size_t)d * DV + j] = sm.ST[j][d];
    }
  }
}

template <int DK>
hipError_t launch_dk(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  const int64_t units = (int64_t)pr.num_seqs * pr.H_v;
  if (units == 0) return hipSuccess;
  const int64_t grid = 8 * ((units + 7) / 8) * (pr.d_v / BVF);  // see the kernel's mapping
  const size_t smem = sizeof(F32Smem<DK>);
  auto kern = chunked_f32mma_kernel<DK>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHREADS), smem, s, pr, x);
  return hipGetLastError();
}

}  // namespace

bool chunked_f32mma_supports(const Problem &p) {
  return p.mode == kModeRule && p.dtype == GDR_F32 && (p.d_k == 64 || p.d_k == 128) &&
         (p.d_v == 16 || p.d_v == 32 || p.d_v == 64 || p.d_v == 128) && p.chunk == CHF;
}

hipError_t launch_chunked_f32mma(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  return pr.d_k == 64 ? launch_dk<64>(pr, x, s) : launch_dk<128>(pr, x, s);
}

}  // namespace gdr
