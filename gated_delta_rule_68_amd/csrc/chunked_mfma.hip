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
// fp32 to the products (the 1/|k_i| of P is applied to the rows of Delta).
// Only differences gamma_r - gamma_i with i <= r are exponentiated.
//
// (I + A)^-1 is formed whole for every chunk, in fp32, and rounded to bf16
// only as the operand of Delta = T R.  With T = [[T11, 0], [T21, T22]] in
// 16-row blocks:
//   T11 = (I + A11)^-1   by a backward sweep on its transpose, (I + A11^T) T11^T = I
//   T22 = (I + A22)^-1   by a forward sweep,                   (I + A22) T22 = I
//   T21 = -T22 (A21 T11) by two fp32 matrix-core products.
// Each sweep is 15 dependent steps; in step i the finished row i is broadcast
// to the other rows of its 16-lane DPP row (row_newbcast) and subtracted with
// the coefficient each row holds, one fused multiply-add per register.  A
// product series such as (I - N)(I + N^2)(I + N^4)(I + N^8) is exact in real
// arithmetic but not usable here: when keys repeat a direction under long
// memory its powers grow like binomial coefficients, and bf16 roundings
// before the cancellation leave O(1) errors in T.
//
// Work split.  A workgroup owns (sequence, value head, 32 columns of d_v); the
// columns of S evolve independently.  Eight waves, one workgroup barrier per
// chunk; chunk c lives in LDS buffer c % NSTAGE from the step its rows are
// requested until the step its outputs are written:
//   * 2 state waves each keep a [128 x 16] slice of S in MFMA accumulators for
//     the whole sequence and run chunk c: K S, R, Delta = T R and
//     S <- Gam_last S + K^T D Delta; they hand the state at chunk entry
//     and diag(1/|k|) Delta (bf16) to
//   * 2 output waves, which form Q S of chunk c in the same step and the
//     outputs O = P Delta + Gam Q S of chunk c one step later;
//   * 2 "prepare" waves form chunk c+1's matrices: P0 the Gram blocks of K
//     and the whole T = (I + A)^-1; P1 the norms of q and the output mask P;
//   * 2 staging waves request the rows of chunk c+2+AHEAD: the k, q, v rows
//     and the raw gates go straight from global memory into LDS
//     (global_load_lds), never through registers; as soon as chunk c+3 has
//     landed, staging wave 0 derives the norms of its k rows and staging
//     wave 1 its gates.
// The k and q tiles are stored unpadded with their 16-byte pieces XOR-swizzled
// per row, so that the operand reads (16 rows at one column) and the
// transposing reads (8 rows at 2 columns) each touch every bank once.
//
// Operand lane orders (v_mfma_f32_16x16x32_bf16: lane l = 16 g + m holds A row
// m / B column m at k = 8g..8g+7, and accumulator rows 4g..4g+3 of column m;
// v_mfma_f32_16x16x16_bf16 the same with k = 4g..4g+3).  An accumulator pair
// covering rows 0..15 and 16..31 gives lane l the rows 4g..4g+3 and
// 16+4g..16+4g+3 of its column, which is a valid B operand if the contraction
// index is visited in "slot" order: slot 8g+j is position 4g+j (j < 4) or
// 16+4g+j-4 (j >= 4) of a 32-block.  The chunk-position operands (T, P and
// k^T) are laid out in slot order; the state tiles hold rows chosen so that
// the d_k operands (rows of k and q) are plain 16-byte reads (state_row), so
// the state and the deltas never leave registers between products.
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

constexpr int DK = 128;
// d_v is a template parameter of the kernel (64 or 128)
constexpr int CH = 32;      // tokens per chunk
constexpr int NC = 2;       // consumer waves (16 columns each)
constexpr int BV = 16 * NC;
constexpr int NWAVES = 8;
constexpr int NSTAGE = 5;   // chunk buffers in LDS
constexpr int AHEAD = 2;    // chunks whose rows are in flight beyond the one being published
static_assert(AHEAD <= NSTAGE - 3, "a buffer is refilled only after its chunk was consumed");

// wave roles (wave w runs on SIMD w % 4): the state waves share a SIMD with
// the light staging waves, the output waves one with P0 and P1
constexpr int W_C0 = 0, W_P0 = 2, W_P1 = 3, W_ST0 = 4, W_O0 = 6;

// vector-memory operations one staging wave issues per chunk
constexpr int ST0_OPS = 8 + 1;       // k rows, half of v
constexpr int ST1_OPS = 8 + 1 + 1;   // q rows, half of v, a and b

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x4 pack4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  return __builtin_shufflevector(pack4(lo), pack4(hi), 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
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

// Wait until at most N vector-memory operations of this wave are in flight
// (s_waitcnt vmcnt(N); the other counters are left alone).  Loads into LDS
// are tracked by this counter only, so they are waited for explicitly
// before the barrier that hands their buffer to the other waves.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | (0xF << 8) | (0x7 << 4) | (N & 15));
}

// Workgroup barrier of the pipeline.  Every LDS access of this wave is
// complete before it (lgkmcnt(0)) and, for a staging wave, every load into
// LDS except the VM newest ones (vmcnt(VM)); global stores and loads into
// registers are not waited for (no other wave reads them).  The empty asm
// statements keep the compiler from moving memory accesses across it.
template <int VM = 63, bool LDS = true>
__device__ __forceinline__ void block_sync() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(((VM >> 4) << 14) | ((LDS ? 0x0 : 0xF) << 8) | (0x7 << 4) | (VM & 15));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------- LDS tiles
// k and q tiles: [32 rows][128 columns] bf16, row pitch 256 bytes; the 16-byte
// piece p of row r is stored at piece position p ^ swz(r), swz a permutation of
// the bits of r % 16 (bit 0 stays, bit 1 <- r bit 3, bit 2 <- r bit 1,
// bit 3 <- r bit 2).  LDS serves 256 bytes a cycle: a 16-byte read in four
// passes of 16 lanes (lane half l / 32 and the parity of lane bits 2..4), an
// 8-byte read in two passes of 32 lanes, and a pass is free of bank conflicts
// when its lanes hit distinct 16- (8-) byte slots modulo 256 bytes.  With
// this swizzle both the row reads (16 rows, one piece each) and the
// transposing reads (8 rows x 4 pieces, alternating 8-byte halves, see
// state_row) fill every slot once.
__device__ __forceinline__ int swz(int r) {
  return (r & 1) | ((r >> 2) & 2) | ((r << 1) & 12);
}
// Element offset of (row r, column d), d a multiple of 4.
__device__ __forceinline__ int kq_off(int r, int d) {
  return r * DK + ((((d >> 3) ^ swz(r & 15)) << 3) | (d & 7));
}

struct Stage {
  alignas(16) bf16 K[CH * DK];   // k rows, swizzled                     (loaded by staging wave 0)
  alignas(16) bf16 Q[CH * DK];   // q rows, swizzled                     (staging wave 1)
  alignas(16) bf16 V[CH * BV];   // v rows, this workgroup's columns     (both)
  // per lane (m, g), written and read by lanes of the same index:
  alignas(16) bf16x8 P[2][64];   // P without 1/|k_i|: rows m, 16 + m at chunk slots 8g.. (P1)
  // T = (I + A)^-1 as A operands of Delta = T R in slot order (P0):
  alignas(16) bf16x4 T0[64];     // rows 0..15: T11[m][4g..4g+3] (slots 8g+4.. are T12 = 0)
  alignas(16) bf16x8 T1[64];     // rows 16..31: T21[m][4g..4g+3], T22[m][4g..4g+3]
  alignas(16) uint32_t ab[2 * CH]; // raw a_r (low half of word r), b_r (word 32 + r) (staging wave 1)
  alignas(16) float gam[CH];     // cumulative log decay                 (staging wave 1, a step early)
  alignas(16) float beta[CH];    //                                      (staging wave 1, a step early)
  alignas(16) float Gam[CH];     // exp(gam)                             (staging wave 1, a step early)
  alignas(16) float tail[CH];    // exp(gam_last - gam)                  (staging wave 1, a step early)
  alignas(16) float ik[CH];      // 1/|k_r| (0 past the end)             (staging wave 0, a step early)
  alignas(16) float iq[CH];      // scale/|q_r| (0 past the end)         (P1)
  alignas(16) float Gc;          // exp(gam_last)                        (staging wave 1, a step early)
  int cl;                        // valid rows of the chunk              (staging wave 1, a step early)
};

struct Smem {
  Stage st[NSTAGE];
  // handed from the state waves to the output waves, per state wave and lane:
  alignas(16) bf16x8 sb[2][NC][4][64];  // state at chunk entry, bf16 B operands (ring by chunk)
  alignas(16) bf16x8 db[2][NC][64];     // diag(1/|k|) Delta of the chunk, bf16 (ring by chunk)
  // P0's own exchange inside one chunk: column m of -A11, row m of -A22 and
  // row m of A21 (columns in the order 4j + g), 80-byte rows so that 16 rows
  // read at one column fill distinct 16-byte bank slots
  alignas(16) float p0x[3][16][20];
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

// State rows held in registers.  Accumulator tile t (t = 0..7) of a
// consumer holds, in lane (m, g) register j, the state row
//   d(t, g, j) = 32 (t / 2) + 8 g + 4 ((t ^ g) % 2) + j
// of column m, so that the tile pair (2kb, 2kb+1) gives every lane 8
// consecutive rows 32kb + 8g .. 32kb + 8g + 7 (tile 2kb + g % 2 holds the
// lower four): a B operand whose contraction index runs in natural order,
// matching one 16-byte read of a k or q row.  The transposing reads of tile t
// then take the lower 8-byte half of a piece in two of their four segments
// and the upper half in the other two, which keeps them free of bank conflicts.
__device__ __forceinline__ int state_row(int t, int g, int j) {
  return 32 * (t >> 1) + 8 * g + 4 * ((t ^ g) & 1) + j;
}
// Rows 32kb + 8g .. + 7 of the state in natural order, from the tile pair
// (2kb, 2kb + 1) of lane group g.
__device__ __forceinline__ bf16x8 state_operand(const f32x4 &t0, const f32x4 &t1, int g) {
  const bf16x4 a = pack4(t0), b = pack4(t1);
  return (g & 1) ? cat8(b, a) : cat8(a, b);
}

// Operand of row r, 32-block kb of d_k: columns 32kb + 8g .. 32kb + 8g + 7.
__device__ __forceinline__ bf16x8 row_op(const bf16 *X, int r, int kb, int g) {
  return *reinterpret_cast<const bf16x8 *>(X + kq_off(r, 32 * kb + 8 * g));
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i%4 of the 8-byte pieces addressed by lanes
// 4j + i/4, j = 0..3.  If lane (m, g) addresses the 4 columns c0 + 4(m%4)..
// of row r0 + 4g + m/4, it receives column c0 + m of rows r0 + 4g + j: a
// 4-row slice of the transpose.
__device__ __forceinline__ bf16x4 tr_read(const bf16 *addr) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(addr));
  return __builtin_bit_cast(bf16x4, v);
}

// Copy 16 bytes per lane from global memory straight into LDS: lane l's
// bytes land at lds + 16 l.  `lds` must be the same for the whole wave.
__device__ __forceinline__ void dma16(const bf16 *src, bf16 *lds) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src),
                                   (__attribute__((address_space(3))) void *)(lds), 16, 0, 0);
}

// Map the launch index to a work unit so that the gs units of one (sequence,
// key head) group land on the same XCD (blocks are dealt round-robin to the 8
// XCDs), sharing that XCD's L2 for their common k and q rows, while the groups
// still start in unit order (the i-th block of every XCD belongs to the
// groups 8 (i / gs) .. 8 (i / gs) + 7).
__device__ __forceinline__ int unit_of_block(int b, int nb, int gs) {
  if (nb % (8 * gs) != 0) return b;
  const int slot = b >> 3;
  return ((slot / gs) * 8 + (b & 7)) * gs + slot % gs;
}

// Sequence that runs in launch rank `rank` of a packed batch: sequences are
// ranked by length, longest first (ties by index), so that the longest
// chains start first and the short ones fill in behind them.  Every lane
// ranks one sequence (num_seqs <= 64); the result is uniform.
__device__ __forceinline__ int seq_by_length_rank(const int32_t *cu, int num_seqs, int rank,
                                                  int lane) {
  int r = num_seqs;  // lanes without a sequence never match
  if (lane < num_seqs) {
    const int len = cu[lane + 1] - cu[lane];
    r = 0;
    for (int j = 0; j < num_seqs; ++j) {
      const int lj = cu[j + 1] - cu[j];
      r += (lj > len) || (lj == len && j < lane);
    }
  }
  const uint64_t hit = __ballot(r == rank);
  return hit ? (int)__builtin_ctzll(hit) : rank;
}

// Request the 32 rows of a k or q tile (8 loads of 1 KB; rows past the end
// re-read the last valid row, whose norm and gates are zeroed later).
// Load i, lane l: row 4i + l/16, stored piece l%16, i.e. piece (l%16) ^ swz(row).
__device__ __forceinline__ void dma_rows(const bf16 *x, int H, int hk, int64_t row0, int cl,
                                         bf16 *tile, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int piece = (lane & 15) ^ swz(r & 15);
    const int rr = min(r, cl - 1);
    dma16(x + ((row0 + rr) * H + hk) * DK + 8 * piece, tile + 512 * i);
  }
}
// Byte offsets of the 8 loads of dma_rows for a full chunk, relative to the
// chunk's first row: the same for every chunk of a workgroup, so a full
// chunk costs one scalar base per tile.
struct RowOffsets {
  uint32_t off[8];
};
__device__ __forceinline__ RowOffsets row_offsets(int H, int lane) {
  RowOffsets o;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    const int piece = (lane & 15) ^ swz(r & 15);
    o.off[i] = (uint32_t)((r * H * DK + 8 * piece) * (int)sizeof(bf16));
  }
  return o;
}
// dma_rows for a full chunk: `x` points at element (row0, hk, 0).
__device__ __forceinline__ void dma_rows_full(const bf16 *x, const RowOffsets &o, bf16 *tile) {
  const char *base = reinterpret_cast<const char *>(x);
#pragma unroll
  for (int i = 0; i < 8; ++i) dma16(reinterpret_cast<const bf16 *>(base + o.off[i]), tile + 512 * i);
}
// v tile: [32 rows][BV = 32 columns] bf16, row pitch 64 bytes; the 16-byte
// piece p of row r is stored at piece position p ^ (2 ((r / 4) % 2)), so that
// the transposing reads of 8 rows x 4 segments fill all 32 8-byte slots of a
// 256-byte bank cycle once.  Element offset of (row r, column c), c % 4 == 0:
static_assert(BV == 32, "the v tile swizzle assumes 4 pieces per row");
__device__ __forceinline__ int v_off(int r, int c) {
  return r * BV + ((((c >> 3) ^ (2 * ((r >> 2) & 1))) << 3) | (c & 7));
}
// Source piece of the 16 bytes lane l stores in a v half tile (row
// 16 h + l / 4, piece position l % 4).
__device__ __forceinline__ int v_src_piece(int lane) { return (lane & 3) ^ (2 * ((lane >> 4) & 1)); }
// Half (rows 16 h .. 16 h + 15) of the v tile: lane l takes row 16h + l/4.
__device__ __forceinline__ void dma_v_half(const bf16 *v, int H_v, int hv, int col0, int64_t row0,
                                           int cl, bf16 *tile, int half, int lane, int DV) {
  const int r = 16 * half + (lane >> 2);
  const int rr = min(r, cl - 1);
  dma16(v + ((row0 + rr) * H_v + hv) * DV + col0 + 8 * v_src_piece(lane), tile + 512 * half);
}

// a and b of the 32 rows in one load: lane l < 32 takes a of row l, lane
// 32 + l b of row l; each 2-byte value lands zero-extended in word l of `ab`.
__device__ __forceinline__ void dma_ab(const bf16 *a, const bf16 *b, int H_v, int hv, int64_t row0,
                                       int cl, uint32_t *ab, int lane) {
  const int rr = min(lane & 31, cl - 1);
  const bf16 *src = (lane < 32 ? a : b) + (row0 + rr) * H_v + hv;
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src),
                                   (__attribute__((address_space(3))) void *)(ab), 2, 0, 0);
}

// One 32-bit LDS read, complete when the statement ends.  The staging wave
// reads the raw gates with it while its own later loads into LDS are still
// in flight; a plain read would make the compiler wait for all of them.
__device__ __forceinline__ uint32_t lds_read_u32_now(const uint32_t *p) {
  uint32_t v;
  const uint32_t addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint32_t *)p;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

// The 128 bytes at p (8 16-byte LDS reads), piece i read by the i-th read from
// piece (i + rot) % 8, complete when the statement ends (see lds_read_u32_now).
// The outputs are early-clobber: a read that returns while later reads of the
// block are still to issue must not land on their address registers.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void lds_read_128B_now(const bf16 *p, int rot, u32x4 (&x)[8]) {
  const uint32_t base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const bf16 *)p;
  uint32_t a[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] = base + 16u * (uint32_t)((i + rot) & 7);
  asm volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
        "=&v"(x[6]), "=&v"(x[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
// Sum of squares of the bf16 values in 32-bit words w (bf16 pair dot products).
__device__ __forceinline__ float sumsq_words(const uint32_t *w, int n, float s) {
  for (int i = 0; i < n; ++i) {
    const bf16x2 x = __builtin_bit_cast(bf16x2, w[i]);
    s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
  }
  return s;
}

// 1/|k_r| of one chunk (staging wave 0, once its k rows have landed): lane l
// sums the squares of half a row (row l / 2) -- the swizzle keeps the 8 pieces
// of a 128-byte half together -- and its neighbour the other half.  Starting
// each lane at piece r % 8 spreads the lanes of every read over all banks.
__device__ __forceinline__ void stage_k_norms(Stage &S, int lane, int cl, float eps) {
  const int r = lane >> 1, half = lane & 1;
  const int pos = half ^ (swz(r & 15) >> 3);  // where the 8 pieces of this half are stored
  u32x4 x[8];
  lds_read_128B_now(S.K + r * DK + 64 * pos, r & 7, x);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // independent chains
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {x[i][0], x[i][1], x[i][2], x[i][3]};
    acc[i & 3] = sumsq_words(w, 4, acc[i & 3]);
  }
  float ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  ss += dpp<0xB1>(ss);  // quad_perm [1,0,3,2]: add the other half of the row
  if (half == 0) S.ik[r] = r < cl ? rsqrtf(ss + eps) : 0.f;
}

// Gates of one chunk (staging wave 1, once its raw a and b have landed):
// row r = lane % 32.
// SSD (the Mamba-2 SSD recurrence on the same scan): a is delta, neg_exp_A is
// A itself, g = A delta and beta = delta.
template <bool SSD>
__device__ __forceinline__ void stage_gates(Stage &S, int lane, int cl, float neg_exp_A,
                                            float dtb) {
  const int r = lane & 31;
  const bool valid = r < cl;
  float g, bt;
  if constexpr (SSD) {
    const float dl = __uint_as_float(lds_read_u32_now(&S.ab[r]) << 16);
    g = valid ? neg_exp_A * dl : 0.f;
    bt = valid ? dl : 0.f;
  } else {
    const float a_r = __uint_as_float(lds_read_u32_now(&S.ab[r]) << 16) + dtb;
    const float b_r = __uint_as_float(lds_read_u32_now(&S.ab[CH + r]) << 16);
    const float sp = fmaxf(a_r, 0.f) + fast_log(1.f + fast_exp(-fabsf(a_r)));
    g = valid ? neg_exp_A * sp : 0.f;
    bt = valid ? __builtin_amdgcn_rcpf(1.f + fast_exp(-b_r)) : 0.f;
  }
  const float cum = scan32(g);
  const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 31));
  if (lane < 32) {
    S.gam[r] = cum;
    S.beta[r] = bt;
    S.Gam[r] = fast_exp(cum);
    S.tail[r] = fast_exp(last - cum);
  }
  if (lane == 0) {
    S.Gc = fast_exp(last);
    S.cl = cl;
  }
}

// The two substitution sweeps of P0, interleaved, 15 steps:
//  * backward, X = T11^T, lane (r, g) holding X[r][4j + g] in x[j]: in step s
//    row i = 15 - s is final and every row r adds cB[i] X[i] (cB[i] holds
//    -A11[i][r], zero unless r < i).  X[i][4j + g] = T11[4j + g][i] is zero
//    when 4j + g < i, so registers j < (i - 3) / 4 are skipped;
//  * forward, Y = T22, lane (m, g) holding Y[m][4g + j] in y[j]: in step s
//    row i = s is final and every row m adds cF[i] Y[i] (cF[i] holds
//    -A22[m][i], zero unless i < m).  Y[i][4g + j] is zero when 4g + j > i,
//    so registers j > i are skipped.
// One update is one v_fmac_f32 whose first source is row i's register,
// broadcast to its 16-lane DPP row by row_newbcast.  Each step is one asm
// statement that starts with s_nop 1: a DPP source must be written at least
// two wait states before it is read, and within a step every register is
// read and written once.
#define GDR_FX(j, i) "v_fmac_f32_dpp %" #j ", %" #j ", %8 row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define GDR_FY(j, i) "v_fmac_f32_dpp %" #j ", %" #j ", %9 row_newbcast:" #i " row_mask:0xf bank_mask:0xf\n\t"
#define GDR_X1(i) GDR_FX(3, i)
#define GDR_X2(i) GDR_FX(3, i) GDR_FX(2, i)
#define GDR_X3(i) GDR_FX(3, i) GDR_FX(2, i) GDR_FX(1, i)
#define GDR_X4(i) GDR_FX(3, i) GDR_FX(2, i) GDR_FX(1, i) GDR_FX(0, i)
#define GDR_Y1(i) GDR_FY(4, i)
#define GDR_Y2(i) GDR_FY(4, i) GDR_FY(5, i)
#define GDR_Y3(i) GDR_FY(4, i) GDR_FY(5, i) GDR_FY(6, i)
#define GDR_Y4(i) GDR_FY(4, i) GDR_FY(5, i) GDR_FY(6, i) GDR_FY(7, i)
#define GDR_STEP(XS, YS, ib, jf)                                                          \
  asm volatile("s_nop 1\n\t" XS YS                                                        \
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(y[0]), "+v"(y[1]), \
                 "+v"(y[2]), "+v"(y[3])                                                   \
               : "v"(cB[ib]), "v"(cF[jf]))
__device__ __forceinline__ void sweeps(float (&x)[4], float (&y)[4], const float (&cB)[16],
                                       const float (&cF)[16]) {
  GDR_STEP(GDR_X1(15), GDR_Y1(0), 15, 0);
  GDR_STEP(GDR_X1(14), GDR_Y2(1), 14, 1);
  GDR_STEP(GDR_X1(13), GDR_Y3(2), 13, 2);
  GDR_STEP(GDR_X1(12), GDR_Y4(3), 12, 3);
  GDR_STEP(GDR_X2(11), GDR_Y4(4), 11, 4);
  GDR_STEP(GDR_X2(10), GDR_Y4(5), 10, 5);
  GDR_STEP(GDR_X2(9), GDR_Y4(6), 9, 6);
  GDR_STEP(GDR_X2(8), GDR_Y4(7), 8, 7);
  GDR_STEP(GDR_X3(7), GDR_Y4(8), 7, 8);
  GDR_STEP(GDR_X3(6), GDR_Y4(9), 6, 9);
  GDR_STEP(GDR_X3(5), GDR_Y4(10), 5, 10);
  GDR_STEP(GDR_X3(4), GDR_Y4(11), 4, 11);
  GDR_STEP(GDR_X4(3), GDR_Y4(12), 3, 12);
  GDR_STEP(GDR_X4(2), GDR_Y4(13), 2, 13);
  GDR_STEP(GDR_X4(1), GDR_Y4(14), 1, 14);
  // the sweeps' last writes before the matrix-core reads of x and y
  asm volatile("s_nop 7" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(y[0]),
               "+v"(y[1]), "+v"(y[2]), "+v"(y[3]));
}
#undef GDR_STEP
#undef GDR_Y4
#undef GDR_Y3
#undef GDR_Y2
#undef GDR_Y1
#undef GDR_X4
#undef GDR_X3
#undef GDR_X2
#undef GDR_X1
#undef GDR_FY
#undef GDR_FX

__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Row operands of one chunk for the prepare waves: rows m and 16 + m of k
// (and q), every 32-block of d_k.
struct RowOps {
  bf16x8 k0[4], k1[4], q0[4], q1[4];
};
template <bool WITH_Q>
__device__ __forceinline__ void read_row_ops(const Stage &S, RowOps &o, int m, int g) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    o.k0[kb] = row_op(S.K, m, kb, g);
    o.k1[kb] = row_op(S.K, 16 + m, kb, g);
    if (WITH_Q) {
      o.q0[kb] = row_op(S.Q, m, kb, g);
      o.q1[kb] = row_op(S.Q, 16 + m, kb, g);
    }
  }
}

// P0: the Gram blocks of k and T = (I + A)^-1 of one chunk, in fp32, written
// as bf16 A operands for the state waves (1/|k| from staging).  Lane (m, g)
// holds the Gram entries (k_i . k_m), i = 4g + j, of each block, which give
// column m of A11, row m of A22 (the Gram matrix is symmetric) and row m of
// A21; a round trip through P0's own LDS rows hands every lane the whole
// column (row) its sweep needs.  Every decay factor is exp(gam_r - gam_i)
// with i <= r, at most 1.
__device__ __forceinline__ void prepare_p0(const MfmaParams &p, Stage &S,
                                           float (&xs)[3][16][20], const RowOps &o, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const f32x4 bt_lo = ld4(&S.beta[4 * g]);
  const f32x4 ik_lo = ld4(&S.ik[4 * g]), ik_hi = ld4(&S.ik[16 + 4 * g]);
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  const float ik_m0 = S.ik[m], bik_m1 = S.beta[16 + m] * S.ik[16 + m];
  f32x4 t00 = z, t11 = z, t01 = z;  // (k_i . k_m) of blocks 00, 11; (k_i . k_{16+m}) of 10
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    t00 = mma32(o.k0[kb], o.k0[kb], t00);
    t11 = mma32(o.k1[kb], o.k1[kb], t11);
    t01 = mma32(o.k0[kb], o.k1[kb], t01);
  }
  f32x4 cA, rA;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * g + j;
    // -A11[i][m] = -beta_i exp(gam_i - gam_m) ik_i ik_m (k_i . k_m), i > m
    const float c0 = bt_lo[j] * ik_lo[j] * ik_m0 * fast_exp(fminf(gm_lo[j] - gm_m0, 0.f)) * t00[j];
    cA[j] = (i > m) ? -c0 : 0.f;
    // -A22[m][i] = -beta_{16+m} exp(gam_{16+m} - gam_{16+i}) ik_{16+m} ik_{16+i} (k . k), i < m
    const float c1 = bik_m1 * ik_hi[j] * fast_exp(fminf(gm_m1 - gm_hi[j], 0.f)) * t11[j];
    rA[j] = (i < m) ? -c1 : 0.f;
    // A21[m][i] = beta_{16+m} exp(gam_{16+m} - gam_i) ik_{16+m} ik_i (k_i . k_{16+m})
    xs[2][m][4 * j + g] = bik_m1 * ik_lo[j] * fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * t01[j];
  }
  *reinterpret_cast<f32x4 *>(&xs[0][m][4 * g]) = cA;
  *reinterpret_cast<f32x4 *>(&xs[1][m][4 * g]) = rA;
  wave_lds_sync();
  float cB[16], cF[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 u = ld4(&xs[0][m][4 * q]), w = ld4(&xs[1][m][4 * q]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cB[4 * q + j] = u[j];
      cF[4 * q + j] = w[j];
    }
  }
  const f32x4 a21 = ld4(&xs[2][m][4 * g]);  // A21[m][4kk + g] in register kk
  float x[4], y[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = (m == 4 * j + g) ? 1.f : 0.f;
    y[j] = (m == 4 * g + j) ? 1.f : 0.f;
  }
  sweeps(x, y, cB, cF);
  // M = A21 T11: contraction index 4kk + g in step kk (x[kk] = T11[4kk + g][n])
  f32x4 mm = z;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) mm = mma_f32(a21[kk], x[kk], mm);
  // T22 M: contraction index 4g + kk in step kk (y[kk] = T22[m][4g + kk],
  // mm[kk] = M[4g + kk][n]); lane (n, g) gets (T22 M)[4g + j][n] = -T21[4g + j][n]
  f32x4 t21 = z;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) t21 = mma_f32(y[kk], mm[kk], t21);
  // bf16 operands: T22 row m stays in this lane; T11 and T21 columns scatter
  // to the lanes that own their rows
  bf16 *T0 = reinterpret_cast<bf16 *>(S.T0);
  bf16 *T1 = reinterpret_cast<bf16 *>(S.T1);
  *reinterpret_cast<bf16x4 *>(T1 + 8 * lane + 4) = pack4(f32x4{y[0], y[1], y[2], y[3]});
  const int dst = 16 * (m >> 2), e = m & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    T0[4 * (dst + 4 * j + g) + e] = (bf16)x[j];
    T1[8 * (dst + 4 * g + j) + e] = (bf16)(-t21[j]);
  }
}

// P1: scale/|q_r| from the Gram diagonal of q, and the output mask without the
// row norms, P[r][i] = exp(gam_r - gam_i) (q_r . k_i) for i <= r, of one chunk
// (scale/|q_r| and 1/|k_i| are applied by the output waves).
__device__ __forceinline__ void prepare_p1(const MfmaParams &p, Stage &S, const RowOps &o,
                                           int lane) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  f32x4 p00 = z, p10 = z, p11 = z;  // (K Q^T) blocks: (q_r . k_i), r = 16 rb + m, i = 16 ib + 4g + j
  f32x4 qq0 = z, qq1 = z;           // Gram diagonal blocks of q
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    p00 = mma32(o.k0[kb], o.q0[kb], p00);
    p10 = mma32(o.k0[kb], o.q1[kb], p10);
    p11 = mma32(o.k1[kb], o.q1[kb], p11);
    qq0 = mma32(o.q0[kb], o.q0[kb], qq0);
    qq1 = mma32(o.q1[kb], o.q1[kb], qq1);
  }
  // scale/|q_r| from the diagonal: lane (m, g = m/4) holds |q_m|^2 in register m%4
  if (g == (m >> 2)) {
    const int cl = S.cl;
    const int j = m & 3;
    S.iq[m] = (m < cl) ? rsqrtf(qq0[j] + p.eps) * p.scale : 0.f;
    S.iq[16 + m] = (16 + m < cl) ? rsqrtf(qq1[j] + p.eps) * p.scale : 0.f;
  }
  f32x4 v00, v10, v11;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = 4 * g + j;  // column inside its 16-block
    v00[j] = (i <= m) ? fast_exp(fminf(gm_m0 - gm_lo[j], 0.f)) * p00[j] : 0.f;
    v10[j] = fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * p10[j];
    v11[j] = (i <= m) ? fast_exp(fminf(gm_m1 - gm_hi[j], 0.f)) * p11[j] : 0.f;
  }
  // row r of P at slots 8g..8g+3 (columns 4g..4g+3) and 8g+4.. (columns 16+4g..)
  S.P[0][lane] = pack8(v00, z);
  S.P[1][lane] = pack8(v10, v11);
}

// SSD mode: the output mask of one chunk split over both prepare waves (P0
// has no erase work to do there): PART 0 takes rows 0..15 (one diagonal
// block), PART 1 rows 16..31 (the block below it and the second diagonal
// block), each writing its own P slot.  Otherwise as prepare_p1 with q
// unnormalised.
template <int PART>
__device__ __forceinline__ void prepare_p_ssd(Stage &S, const RowOps &o, int lane) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  if constexpr (PART == 0) {
    f32x4 p00 = z;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) p00 = mma32(o.k0[kb], o.q0[kb], p00);
    f32x4 v00;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * g + j;
      v00[j] = (i <= m) ? fast_exp(fminf(gm_m0 - gm_lo[j], 0.f)) * p00[j] : 0.f;
    }
    S.P[0][lane] = pack8(v00, z);
    if (g == 0) {
      const int cl = S.cl;
      S.iq[m] = (m < cl) ? 1.0f : 0.f;
      S.iq[16 + m] = (16 + m < cl) ? 1.0f : 0.f;
    }
  } else {
    f32x4 p10 = z, p11 = z;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      p10 = mma32(o.k0[kb], o.q1[kb], p10);
      p11 = mma32(o.k1[kb], o.q1[kb], p11);
    }
    f32x4 v10, v11;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * g + j;
      v10[j] = fast_exp(fminf(gm_m1 - gm_lo[j], 0.f)) * p10[j];
      v11[j] = (i <= m) ? fast_exp(fminf(gm_m1 - gm_hi[j], 0.f)) * p11[j] : 0.f;
    }
    S.P[1][lane] = pack8(v10, v11);
  }
}

// DVT: d_v (64 or 128; d_k is 128).  SSD: the Mamba-2 SSD recurrence on the
// same scan -- no norms, no erase (T = I, Delta = diag(beta) V with no K S),
// g = A delta, beta = delta; the prepare wave P0 is idle.
template <int DVT, bool SSD>
__global__ __launch_bounds__(64 * NWAVES) void chunked_mfma_kernel(MfmaParams p) {
  constexpr int DV = DVT;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  constexpr int NVB = DV / BV;

  const int unit = unit_of_block(blockIdx.x, gridDim.x, (p.H_v / p.H_k) * NVB);
  const int vb = unit % NVB;
  const int h = (unit / NVB) % p.H_v;
  const int n = (p.cu && p.num_seqs <= 64)
                    ? seq_by_length_rank(p.cu, p.num_seqs, unit / (NVB * p.H_v), threadIdx.x & 63)
                    : unit / (NVB * p.H_v);
  const int hk = h / (p.H_v / p.H_k);
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;

  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const int64_t L = t1 - t0;
  const int nch = (int)((L + CH - 1) / CH);
  const size_t state_off = ((size_t)n * p.H_v + h) * DK * DV;
  const int col0 = vb * BV;
  // step `it` updates the state with chunk it-2, writes the outputs of chunk
  // it-3, prepares chunk it-1 and derives the gates of chunk it+1; every wave
  // passes nsteps + 1 barriers
  const int nsteps = nch + 3;

  if (wave >= W_C0 && wave < W_C0 + NC) {
    // ------------------------------------------------------------ state waves
    // chunk c in step c + 2: K S, R, Delta = T R, S <- Gam_last S + K^T D Delta;
    // they hand the state at chunk entry (before step c + 2) and the scaled
    // Delta (during step c + 2) to the output waves.
    const int cw = wave - W_C0;
    const int col = col0 + 16 * cw + m;
    f32x4 S[8];  // S[state_row(t, g, j)][col]
    if (p.s0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[t][j] = p.s0[state_off + (size_t)state_row(t, g, j) * DV + col];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 Sb[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[kb] = state_operand(S[2 * kb], S[2 * kb + 1], g);
    // LDS operands: the k^T tiles of this chunk (A operands of the state
    // update) are read once the K S products are issued; the k rows (A
    // operands of K S) and v of the next chunk are read after the state
    // update, so that they are in registers when the next step starts.  The
    // rows of chunk c+1 are in LDS from step c+1 on.
    bf16x8 Kr[2][4], Kt[8], vv;
    auto read_rows = [&](const Stage &sn) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) Kr[mt][kb] = row_op(sn.K, 16 * mt + m, kb, g);
    };
    auto read_kt = [&](const Stage &sn) {
      // A operand of tile t: row m is state row state_row(t, m / 4, m % 4),
      // contraction over chunk positions in slot order, i.e. lane (m, g) gets
      // k[4g + j][state_row(t, m / 4, m % 4)] and k[16 + 4g + j][...], j = 0..3
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int r = 4 * g + (m >> 2), d = state_row(t, m & 3, 0);
        Kt[t] = cat8(tr_read(sn.K + kq_off(r, d)), tr_read(sn.K + kq_off(16 + r, d)));
      }
    };
    auto read_v = [&](const Stage &sn) {
      // v[4g + j][col] and v[16 + 4g + j][col]
      const int vr = 4 * g + (m >> 2), vc = 16 * cw + 4 * (m & 3);
      vv = cat8(tr_read(sn.V + v_off(vr, vc)), tr_read(sn.V + v_off(16 + vr, vc)));
    };
    auto hand_state = [&](int c) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sm.sb[c & 1][cw][kb][lane] = Sb[kb];
    };
    block_sync();
    for (int it = 0; it < nsteps; ++it) {
      const int c = it - 2;
      if (c >= 0 && c < nch) {
        const Stage &st = sm.st[c % NSTAGE];
        const bool more = c + 1 < nch;
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        // this chunk's prepared tile and row factors
        const bf16x4 tt0 = st.T0[lane];
        const bf16x8 tt1 = st.T1[lane];
        const f32x4 bt0 = ld4(&st.beta[4 * g]), bt1 = ld4(&st.beta[16 + 4 * g]);
        const f32x4 gm0 = ld4(&st.Gam[4 * g]), gm1 = ld4(&st.Gam[16 + 4 * g]);
        const f32x4 ik0 = ld4(&st.ik[4 * g]), ik1 = ld4(&st.ik[16 + 4 * g]);
        const f32x4 tl0 = ld4(&st.tail[4 * g]), tl1 = ld4(&st.tail[16 + 4 * g]);
        const float gc = st.Gc;
        // ks[mt]: (K S)[16mt + 4g + j][m]
        f32x4 ks[2] = {z, z};
        if constexpr (!SSD) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) ks[mt] = mma32(Kr[mt][kb], Sb[kb], ks[mt]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        read_kt(st);
        __builtin_amdgcn_sched_barrier(0);
        // R = beta (V - Gam ik K S), rows 4g..4g+3 and 16+4g..16+4g+3
        f32x4 R0, R1;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          R0[j] = bt0[j] * ((float)vv[j] - gm0[j] * ik0[j] * ks[0][j]);
          R1[j] = bt1[j] * ((float)vv[4 + j] - gm1[j] * ik1[j] * ks[1][j]);
        }
        // Delta = T R, both 16-row blocks from the one bf16 operand of R in
        // slot order; SSD: no erase, Delta = R
        f32x4 d1 = R0, d2 = R1;
        if constexpr (!SSD) {
          const bf16x8 Rb = pack8(R0, R1);
          d1 = mma32(cat8(tt0, bf16x4{0, 0, 0, 0}), Rb, z);
          d2 = mma32(tt1, Rb, z);
        }
        // diag(ik) Delta for the outputs of this chunk
        sm.db[c & 1][cw][lane] = pack8(ik0 * d1, ik1 * d2);
        // S <- Gam_last S + K^T diag(tail ik) Delta
        const bf16x8 Dp = pack8(tl0 * ik0 * d1, tl1 * ik1 * d2);
#pragma unroll
        for (int t = 0; t < 8; ++t) S[t] = mma32(Kt[t], Dp, S[t] * gc);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = state_operand(S[2 * kb], S[2 * kb + 1], g);
        if (more) hand_state(c + 1);
      } else if (c == -1 && nch > 0) {
        hand_state(0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the handed-over writes are done
      {
        // operands of the next step's chunk c + 1, read unconditionally (the
        // index clamped into the sequence) so that the loads write the loop's
        // registers directly and stay in flight across the barrier
        const Stage &sr = sm.st[max(min(c + 1, nch - 1), 0) % NSTAGE];
        if constexpr (!SSD) read_rows(sr);
        read_v(sr);
      }
      // no wait for the reads in flight: their buffers are refilled only
      // steps later, and their registers are waited for where they are used
      block_sync<63, false>();
    }
    if (p.sT) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.sT[state_off + (size_t)state_row(t, g, j) * DV + col] = S[t][j];
    }
  } else if (wave >= W_O0 && wave < W_O0 + NC) {
    // ----------------------------------------------------------- output waves
    // step it: O of chunk it - 3 = (diag(ik) Delta)^T P^T + (Gam iq Q S)^T,
    // then (Q S)^T of chunk it - 2 from the state handed over at its entry.
    const int cw = wave - W_O0;
    f32x4 qsT[2];
    block_sync();
    for (int it = 0; it < nsteps; ++it) {
      const int co = it - 3;
      if (co >= 0 && co < nch) {
        const Stage &st = sm.st[co % NSTAGE];
        const bf16x8 Db = sm.db[co & 1][cw][lane];
        const bf16x8 pr0 = st.P[0][lane];
        const bf16x8 pr1 = st.P[1][lane];
        const float gm0 = st.Gam[m], gm1 = st.Gam[16 + m];
        const float iq0 = st.iq[m], iq1 = st.iq[16 + m];
        // lane (m, g) gets O[16mt + m][4g..4g+3] = iq (Gam (Q S) + P diag(ik) Delta)
        const f32x4 oc0 = mma32(Db, pr0, qsT[0] * gm0) * iq0;
        const f32x4 oc1 = mma32(Db, pr1, qsT[1] * gm1) * iq1;
        const int64_t row = t0 + (int64_t)co * CH + m;
        bf16 *orow = p.o + (row * p.H_v + h) * DV + col0 + 16 * cw + 4 * g;
        if (row < t1) *reinterpret_cast<bf16x4 *>(orow) = pack4(oc0);
        if (row + 16 < t1) *reinterpret_cast<bf16x4 *>(orow + (int64_t)16 * p.H_v * DV) = pack4(oc1);
      }
      const int c = it - 2;
      if (c >= 0 && c < nch) {
        const Stage &st = sm.st[c % NSTAGE];
        const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 Sb[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[kb] = sm.sb[c & 1][cw][kb][lane];
        // qsT[mt]: (Q S)[16mt + m][4g + j]
        qsT[0] = z;
        qsT[1] = z;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            qsT[mt] = mma32(Sb[kb], row_op(st.Q, 16 * mt + m, kb, g), qsT[mt]);
        }
      }
      block_sync<63, false>();
    }
  } else if (wave == W_P0 || wave == W_P1) {
    // ---------------------------------------------------------------- prepare
    // Each step also reads the row operands of the next chunk (published
    // one step earlier), after its own LDS writes have completed, so that
    // the reads overlap the barrier and the next step's wait.
    RowOps ops;
    block_sync();
    for (int it = 0; it < nsteps; ++it) {
      const int c = it - 1;
      // (SSD: no erase, so P0 has nothing to prepare and only keeps the barriers)
      if (c >= 0 && c < nch) {
        if constexpr (SSD) {
          if (wave == W_P0)
            prepare_p_ssd<0>(sm.st[c % NSTAGE], ops, lane);
          else
            prepare_p_ssd<1>(sm.st[c % NSTAGE], ops, lane);
        } else if (wave == W_P0) {
          prepare_p0(p, sm.st[c % NSTAGE], sm.p0x, ops, lane);
        } else {
          prepare_p1(p, sm.st[c % NSTAGE], ops, lane);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's LDS writes are done
      if (it < nch) {
        if (wave == W_P0 && !SSD)
          read_row_ops<false>(sm.st[it % NSTAGE], ops, m, g);
        else
          read_row_ops<true>(sm.st[it % NSTAGE], ops, m, g);
      }
      block_sync<63, false>();
    }
  } else {
    // ---------------------------------------------------------------- staging
    // (loads into LDS of chunks past the end are still in flight after the
    // last barrier: they are drained before the wave ends, so that no LDS
    // write lands after the workgroup has released its LDS)
    if (nch == 0) {  // nothing to load; keep the barrier count
      for (int it = 0; it <= nsteps; ++it) block_sync();
      return;
    }
    // per-lane byte offsets of full-chunk loads: k or q rows, and this wave's
    // half of the v tile (rows 16 half + lane / 4, columns col0 + 8 (lane % 4))
    const RowOffsets ko = row_offsets(p.H_k, lane);
    const int vhalf = wave - W_ST0;
    const uint32_t voff =
        (uint32_t)(((16 * vhalf + (lane >> 2)) * p.H_v * DV + col0 + 8 * v_src_piece(lane)) * (int)sizeof(bf16));
    // chunk c (clamped to the last one: requests past the end re-read it into
    // a buffer no one reads again) -> first row and valid rows
    auto rows_of = [&](int c, int64_t &row0, int &cl) {
      c = min(c, nch - 1);
      row0 = t0 + (int64_t)c * CH;
      const int64_t rem = t1 - row0;
      cl = rem < CH ? (int)rem : CH;
    };
    // Step it requests chunk it + AHEAD and waits for chunk it + 1 (read by
    // P1 in step it + 1); an extra first barrier publishes chunk 0.
    if (wave == W_ST0) {
      // k rows and the first half of v
      auto request = [&](int c) {
        int64_t row0;
        int cl;
        rows_of(c, row0, cl);
        Stage &S = sm.st[c % NSTAGE];
        if (cl == CH) {
          dma_rows_full(p.k + (row0 * p.H_k + hk) * DK, ko, S.K);
          dma16(reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(p.v + (row0 * p.H_v + h) * DV) + voff), S.V);
        } else {
          dma_rows(p.k, p.H_k, hk, row0, cl, S.K, lane);
          dma_v_half(p.v, p.H_v, h, col0, row0, cl, S.V, 0, lane, DV);
        }
      };
      // 1/|k| of chunk c once its rows have landed (c < nch)
      auto norms = [&](int c) {
        const int64_t rem = L - (int64_t)c * CH;
        const int cl = rem < CH ? (int)rem : CH;
        if constexpr (SSD) {  // keys are not normalised
          if (lane < CH) sm.st[c % NSTAGE].ik[lane] = lane < cl ? 1.0f : 0.0f;
        } else {
          stage_k_norms(sm.st[c % NSTAGE], lane, cl, p.eps);
        }
      };
      for (int c = 0; c < AHEAD; ++c) request(c);
      vm_wait<ST0_OPS * (AHEAD - 1)>();  // chunk 0 has landed
      norms(0);
      block_sync<ST0_OPS * (AHEAD - 1)>();
      for (int it = 0; it < nsteps; ++it) {
        request(it + AHEAD);
        vm_wait<ST0_OPS * (AHEAD - 1)>();  // chunk it + 1 has landed
        if (it + 1 < nch) norms(it + 1);
        block_sync<ST0_OPS * (AHEAD - 1)>();
      }
    } else {
      // q rows, the second half of v, a and b
      auto request = [&](int c) {
        int64_t row0;
        int cl;
        rows_of(c, row0, cl);
        Stage &S = sm.st[c % NSTAGE];
        if (cl == CH) {
          dma_rows_full(p.q + (row0 * p.H_k + hk) * DK, ko, S.Q);
          dma16(reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(p.v + (row0 * p.H_v + h) * DV) + voff), S.V + 512);
        } else {
          dma_rows(p.q, p.H_k, hk, row0, cl, S.Q, lane);
          dma_v_half(p.v, p.H_v, h, col0, row0, cl, S.V, 1, lane, DV);
        }
        dma_ab(p.a, SSD ? p.a : p.b, p.H_v, h, row0, cl, S.ab, lane);  // SSD: no b
      };
      const float neg_exp_A = SSD ? p.A_log[h] : -expf(p.A_log[h]);  // SSD: A itself
      const float dtb = SSD ? 0.0f : p.dt_bias[h];
      // gates of chunk c once its raw a, b have landed (c < nch)
      auto gates = [&](int c) {
        const int64_t rem = L - (int64_t)c * CH;
        stage_gates<SSD>(sm.st[c % NSTAGE], lane, rem < CH ? (int)rem : CH, neg_exp_A, dtb);
      };
      for (int c = 0; c < AHEAD; ++c) request(c);
      vm_wait<ST1_OPS * (AHEAD - 1)>();  // chunk 0 has landed
      gates(0);
      block_sync<ST1_OPS * (AHEAD - 1)>();
      for (int it = 0; it < nsteps; ++it) {
        request(it + AHEAD);
        vm_wait<ST1_OPS * (AHEAD - 1)>();  // chunk it + 1 has landed
        if (it + 1 < nch) gates(it + 1);
        block_sync<ST1_OPS * (AHEAD - 1)>();
      }
    }
    vm_wait<0>();
  }
}

template <int DVT, bool SSD>
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
  const int64_t grid = (int64_t)pr.num_seqs * pr.H_v * (DVT / BV);
  if (grid == 0) return hipSuccess;
  const size_t smem = sizeof(Smem);
  auto kern = chunked_mfma_kernel<DVT, SSD>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * NWAVES), smem, s, p);
  return hipGetLastError();
}

}  // namespace

bool chunked_mfma_supports(const Problem &p) {
  return p.mode != kModeKDA && p.dtype == GDR_BF16 && p.d_k == DK && (p.d_v == 64 || p.d_v == 128) &&
         p.chunk == CH;
}

hipError_t launch_chunked_mfma(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  if (pr.mode == 1)
    return pr.d_v == 64 ? launch_kernel<64, true>(pr, x, s) : launch_kernel<128, true>(pr, x, s);
  return pr.d_v == 64 ? launch_kernel<64, false>(pr, x, s) : launch_kernel<128, false>(pr, x, s);
}

}  // namespace gdr
