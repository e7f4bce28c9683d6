// Chunked (UT-transform) form on the gfx950 matrix cores: bf16 operands, fp32
// accumulation, fp32 state.  Instantiated for d_k = 128, d_v = 64 or 128 and
// 32-token chunks (the shape the GatedDeltaRule.ixx File Reference,
// "Detailed Description", gives: one triangular solve per 32 steps).
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
// Everything a chunk needs besides its k, q and v rows and the state -- T, P
// and the row factors -- is one 5 KB record (Rec).  Two kernels use it:
//
// Fused kernel (chunked_mfma_kernel).  A workgroup owns (sequence, value
// head, 32 columns of d_v); the columns of S evolve independently.  Eight
// waves, one workgroup barrier per chunk; chunk c lives in LDS buffer
// c % NSTAGE from the step its rows are requested until the step its outputs
// are written:
//   * 2 state waves each keep a [128 x 16] slice of S in MFMA accumulators for
//     the whole sequence and run chunk c: K S, R, Delta = T R and
//     S <- Gam_last S + K^T D Delta; they hand the state at chunk entry
//     and diag(1/|k|) Delta (bf16) to
//   * 2 output waves, which form Q S of chunk c in the same step and the
//     outputs O = P Delta + Gam Q S of chunk c one step later;
//   * 2 "prepare" waves form chunk c+1's record: P0 the Gram blocks of K
//     and the whole T = (I + A)^-1; P1 the norms of q and the output mask P;
//   * 2 staging waves request the rows of chunk c+2+AHEAD: the k, q, v rows
//     and the raw gates go straight from global memory into LDS
//     (global_load_lds), never through registers; as soon as chunk c+3 has
//     landed, staging wave 0 derives the norms of its k rows and staging
//     wave 1 its gates.
// The four workgroups of a value head each form the same records.
//
// Cooperative kernel (chunked_coop_kernel), one launch of one workgroup per
// compute unit, all resident together.  Workgroups find their role by the
// accelerator complex die (XCD) they run on: per (sequence, key head) group,
// four producer workgroups and the chain workgroups of its value heads sit on
// one XCD and share its L2.  Producer p forms the records of chunks
// c = p mod 4 for all value heads of the group, once, and writes them to a
// ring of RING slots per value head in the workspace.  A chain workgroup has
// two state, two output, two staging and two K S waves (one of each kind per
// 16-column tile, staging shared): its staging wave copies each record into
// LDS with the chunk's rows once the producer's flag for that chunk is set,
// and publishes how far it has copied, which is when the producer may reuse
// the slot; the K S waves form the part of each chunk's R that does not wait
// for the chunk before (see state_wave, LOOK).  Flags, progress words and
// records are read at device scope, past the L1 and scalar caches, in the
// shared L2.  Every wait is bounded: a wait that runs out marks the
// workspace's error word instead of hanging.
//
// The k and q tiles are stored unpadded with their 16-byte pieces XOR-swizzled
// per row, so that the operand reads (16 rows at one column) and the
// transposing reads (8 rows at 2 columns) each touch every bank once.
//
// Operand lane orders (v_mfma_f32_16x16x32_bf16: lane l = 16 g + m holds A row
// m / B column m at k = 8g..8g+7, and accumulator rows 4g..4g+3 of column m;
// v_mfma_f32_16x16x4_f32: A row m / B column m at k = g).  An accumulator
// pair covering rows 0..15 and 16..31 gives lane l the rows 4g..4g+3 and
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
// d_v is a template parameter of the kernels (64 or 128)
constexpr int CH = 32;      // tokens per chunk
constexpr int NC = 2;       // state (and output) waves, 16 columns each
constexpr int BV = 16 * NC;
constexpr int NWAVES = 8;   // fused kernel
constexpr int NSTAGE = 5;   // chunk buffers in LDS
constexpr int AHEAD = 2;    // chunks whose rows are in flight beyond the one being published
// Chunk c's buffer is refilled with chunk c + NSTAGE (rows, and the record in
// the cooperative kernel) from step c + NSTAGE - AHEAD on; its last reads are
// in step c + 2 (the state and output waves run chunk it - 2 in step it).
static_assert(AHEAD + 2 < NSTAGE, "a buffer is refilled only after its chunk was consumed");
static_assert(AHEAD == 2, "the cooperative staging wave fetches flags two steps ahead of AHEAD");

// fused kernel: wave roles (wave w runs on SIMD w % 4): the state waves share
// a SIMD with the light staging waves, the output waves one with P0 and P1
constexpr int W_C0 = 0, W_P0 = 2, W_P1 = 3, W_ST0 = 4, W_O0 = 6;

// vector-memory operations one staging wave issues per chunk (fused kernel)
constexpr int ST0_OPS = 8 + 1;       // k rows, half of v
constexpr int ST1_OPS = 8 + 1 + 1;   // q rows, half of v, a and b

// cooperative kernel: eight waves; chain workgroups use waves 0, 1 (state,
// SIMD 0, 1), 2, 3 (output, SIMD 2, 3), 4, 5 (staging, SIMD 0, 1) and 6, 7
// (K S, SIMD 2, 3)
constexpr int NWAVES_C = 8;
constexpr int CW_O0 = 2, CW_ST0 = 4, CW_KS0 = 6;
constexpr int REC_BYTES = 7168;           // one record; 7 loads of 1 KB per wave
constexpr int REC_DMAS = REC_BYTES / 1024;
constexpr int CST0_OPS = 8 + 1 + REC_DMAS;  // k rows, half of v, the record (+ 1 flag a step)
constexpr int CST1_OPS = 8 + 1;             // q rows, half of v
constexpr int PRODUCERS = 4;              // producer workgroups per group
constexpr int RING = 16;                  // record slots per value head
constexpr int TOUCH_AHEAD = PRODUCERS;  // chunks a producer touches k and q ahead of its copy
constexpr int V_TOUCH_BEHIND = 8;       // chunks behind its copy that a producer touches v
constexpr int MAX_GV = 3;                 // value heads per key head on this path
constexpr int XCD_CUS = 32;               // compute units per XCD on gfx950
constexpr int MAX_XCD = 16;
constexpr int SPIN_LIMIT = 1 << 20;       // polls before a wait gives up (well under a second)

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

// Everything one chunk needs besides its rows and the state, for one value
// head: written by P0, P1 and the staging waves (fused kernel) or by a
// producer workgroup (cooperative kernel), read by the state and output
// waves.  Lane-ordered tiles are written and read by lanes of the same index.
struct alignas(16) Rec {
  // T = (I + A)^-1 as A operands of Delta = T R in slot order:
  bf16x4 T0[64];       // rows 0..15: T11[m][4g..4g+3] (slots 8g+4.. are T12 = 0)
  bf16x8 T1[64];       // rows 16..31: T21[m][4g..4g+3], T22[m][4g..4g+3]
  bf16x8 P[2][64];     // P without 1/|k_i|: rows m, 16 + m at chunk slots 8g..
  // cooperative kernel: -diag(bgk) K_c K_{c-1}^T, the cross Gram of this
  // chunk's raw k rows against the previous chunk's scaled by minus this
  // chunk's bgk, as the A operand of its share of R: with K_c S_c =
  // Gam_last(c-1) K_c S_{c-1} + (K_c K_{c-1}^T) D_{c-1} Delta_{c-1}, R gains
  // GX D_{c-1} Delta_{c-1} (rows 16 mt + m, the previous chunk's positions
  // in slot order)
  bf16x8 GX[2][64];
  float bt[CH];        // beta_r (0 past the end)
  float bgk[CH];       // beta_r Gam_r / |k_r|: the factor of (K S) in R
  float tk[CH];        // exp(gam_last - gam_r) / |k_r|: the factor of Delta in the update
  float ik[CH];        // 1 / |k_r| (0 past the end)
  float Gm[CH];        // Gam_r = exp(gam_r)
  float iq[CH];        // scale / |q_r| (0 past the end)
  float Gc;            // exp(gam_last)
  int cl;              // valid rows of the chunk
  unsigned char pad[REC_BYTES - 5632 - 6 * 4 * CH - 8];
};
static_assert(sizeof(Rec) == REC_BYTES, "record size");

// A record under construction with the chunk's decays.
struct Prep {
  Rec r;
  alignas(16) float gam[CH];   // cumulative log decay
  alignas(16) float tail[CH];  // exp(gam_last - gam)
};

struct Stage {
  alignas(16) bf16 K[CH * DK];   // k rows, swizzled                     (loaded by staging wave 0)
  alignas(16) bf16 Q[CH * DK];   // q rows, swizzled                     (staging wave 1)
  alignas(16) bf16 V[CH * BV];   // v rows, this workgroup's columns     (both)
  Prep pp;                       // the chunk's record (+ decays: fused kernel only)
  alignas(16) uint32_t ab[2 * CH]; // raw a_r (low half of word r), b_r (word 32 + r) (fused kernel)
};

struct Smem {
  Stage st[NSTAGE];
  // handed from the state waves to the output waves, per state wave and lane:
  alignas(16) bf16x8 sb[2][NC][4][64];  // state at chunk entry, bf16 B operands (ring by chunk)
  alignas(16) bf16x8 db[2][NC][64];     // diag(1/|k|) Delta of the chunk, bf16 (ring by chunk)
  union {
    // fused kernel, P0's own exchange inside one chunk: column m of -A11,
    // row m of -A22 and row m of A21 (columns in the order 4j + g), 80-byte
    // rows so that 16 rows read at one column fill distinct 16-byte bank slots
    float p0x[3][16][20];
    // cooperative kernel: the K S waves' part of R of a chunk, for the state
    // waves, per state wave, 16-row block and lane (ring by chunk)
    f32x4 rp[2][NC][2][64];
  };
  // cooperative kernel: flag words of chunks c, fetched ahead into word block c % 4
  alignas(16) uint32_t fl[4][64];
};

// A producer workgroup's LDS (cooperative kernel): its chunk's rows and raw
// gates (two buffers: the next chunk lands while this one is worked on), the
// records under construction (two buffers: a record is copied out in the
// iteration after the one that formed it), the T waves' exchange rows, the P
// waves' decays and the progress words.
struct ProdSmem {
  alignas(16) bf16 K[2][CH * DK];
  alignas(16) bf16 Q[2][CH * DK];
  alignas(16) bf16 Kp[2][CH * DK];  // k rows of the chunk before (for the cross Gram)
  alignas(16) uint32_t ab[2][MAX_GV][2 * CH];
  Prep pp[2][MAX_GV];
  alignas(16) float xs[MAX_GV][3][16][20];
  alignas(16) float gp[MAX_GV][CH];      // P wave j: the chunk's cumulative log decay,
  alignas(16) float bgm[MAX_GV][CH];     //   beta Gam
  alignas(16) float ikp[MAX_GV][CH];     //   and 1/|k|
  alignas(16) uint32_t prg[MAX_GV][64];  // progress words, fetched by T wave j
  alignas(16) uint32_t vtouch[64];       // scratch of the loader's v touches (never read)
};

// Workspace of the cooperative kernel: one 128-byte line per XCD (arrival
// and completion counters, error word), then one block per (sequence, key
// head) group, used only by workgroups on that group's XCD: flags[gv][RING]
// (chunk + 1 of the record in each slot), progress[gv * nvb] (chunks each
// chain workgroup has copied), then the records [gv][RING].
struct XcdLine {
  uint32_t arrive, done, err, pad[29];
};
constexpr size_t WS_HEAD = sizeof(XcdLine) * MAX_XCD;
constexpr size_t GRP_FLAGS = 0, GRP_PROGRESS = 256, GRP_RECS = 512;

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
  // cooperative kernel
  unsigned char *ws;
  size_t grp_stride;
  int nxcd, slots, gs, groups;
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
// Rows 32kb + 8g .. + 7 of the state from the tile pair (2kb, 2kb + 1) of
// lane group g, in "tile order": natural for even g, the two halves of four
// exchanged for odd g (tile 2kb holds the upper four there).  No lane choice
// is made here, on the chain of chunks; the d_k operands that meet the state
// in a product take the same order instead (row_op_t).
__device__ __forceinline__ bf16x8 state_operand(const f32x4 &t0, const f32x4 &t1) {
  return cat8(pack4(t0), pack4(t1));
}

// Operand of row r, 32-block kb of d_k: columns 32kb + 8g .. 32kb + 8g + 7.
__device__ __forceinline__ bf16x8 row_op(const bf16 *X, int r, int kb, int g) {
  return *reinterpret_cast<const bf16x8 *>(X + kq_off(r, 32 * kb + 8 * g));
}
// The same columns in tile order (see state_operand): the operand of a
// product with the state.  The two 8-byte halves are read separately, each
// from the address its lane needs, rather than exchanged in registers
// afterwards; the reads stay free of bank conflicts (in each pass of 32
// lanes, lanes of even g take the lower halves of 16 distinct pieces and
// lanes of odd g the upper halves of 16 others).
//
// The offset is hidden from the compiler, which would otherwise pair the
// reads of rows r and r + 16 (same swizzle, a constant distance apart) into
// one two-address read whose halves then have to be copied into place, a
// wait for each pair.
__device__ __forceinline__ bf16x8 row_op_t(const bf16 *X, int r, int kb, int g) {
  int off = kq_off(r, 32 * kb + 8 * g);
  asm("" : "+v"(off));
  const bf16 *p = X + off;
  const int sw = (g & 1) * 4;  // elements
  return cat8(*reinterpret_cast<const bf16x4 *>(p + sw), *reinterpret_cast<const bf16x4 *>(p + (sw ^ 4)));
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
// Cache policy of a load that must see what another compute unit of the XCD
// stored during this launch: device scope (sc1), which the per-CU L1 cannot
// serve from a line it still holds; sc0 alone is workgroup scope and may hit
// a stale L1 line.
constexpr int CPOL_DEVICE = 16;
// The same, at device scope: the cooperative kernel's records, flags and
// progress words.
__device__ __forceinline__ void dma16_l2(const void *src, void *lds) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)(lds), 16, 0,
                                   CPOL_DEVICE);
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

// One 4-byte load per lane from src into the 256-byte scratch block at lds,
// to bring src's line into the L2 ahead of a later copy (the data is never
// read).
__device__ __forceinline__ void touch4(const bf16 *src, uint32_t *lds) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(src),
                                   (__attribute__((address_space(3))) void *)(lds), 4, 0, 0);
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


// scale/|x_r| of the 32 rows of a swizzled k or q tile (one wave, once the
// rows have landed), into out[r] (0 for rows r >= cl): lane l sums the squares
// of half a row (row l / 2) -- the swizzle keeps the 8 pieces of a 128-byte
// half together -- and its neighbour the other half.  Starting each lane at
// piece r % 8 spreads the lanes of every read over all banks.
__device__ __forceinline__ void tile_norms(const bf16 *X, float *out, int lane, int cl, float eps,
                                           float scale) {
  const int r = lane >> 1, half = lane & 1;
  const int pos = half ^ (swz(r & 15) >> 3);  // where the 8 pieces of this half are stored
  u32x4 x[8];
  lds_read_128B_now(X + r * DK + 64 * pos, r & 7, x);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};  // independent chains
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t w[4] = {x[i][0], x[i][1], x[i][2], x[i][3]};
    acc[i & 3] = sumsq_words(w, 4, acc[i & 3]);
  }
  float ss = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  ss += dpp<0xB1>(ss);  // quad_perm [1,0,3,2]: add the other half of the row
  if (half == 0) out[r] = r < cl ? scale * rsqrtf(ss + eps) : 0.f;
}

// Gates of one chunk (one wave, once its raw a and b have landed in `ab`):
// row r = lane % 32.  Writes the decays of `S` and its record's bt, Gm, Gc, cl.
// SSD (the Mamba-2 SSD recurrence on the same scan): a is delta, neg_exp_A is
// A itself, g = A delta and beta = delta.
template <bool SSD>
__device__ __forceinline__ void stage_gates(Prep &S, const uint32_t *ab, int lane, int cl,
                                            float neg_exp_A, float dtb) {
  const int r = lane & 31;
  const bool valid = r < cl;
  float g, bt;
  if constexpr (SSD) {
    const float dl = __uint_as_float(lds_read_u32_now(&ab[r]) << 16);
    g = valid ? neg_exp_A * dl : 0.f;
    bt = valid ? dl : 0.f;
  } else {
    const float a_r = __uint_as_float(lds_read_u32_now(&ab[r]) << 16) + dtb;
    const float b_r = __uint_as_float(lds_read_u32_now(&ab[CH + r]) << 16);
    const float sp = fmaxf(a_r, 0.f) + fast_log(1.f + fast_exp(-fabsf(a_r)));
    g = valid ? neg_exp_A * sp : 0.f;
    bt = valid ? __builtin_amdgcn_rcpf(1.f + fast_exp(-b_r)) : 0.f;
  }
  const float cum = scan32(g);
  const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cum), 31));
  if (lane < 32) {
    S.gam[r] = cum;
    S.r.bt[r] = bt;
    S.r.Gm[r] = fast_exp(cum);
    S.tail[r] = fast_exp(last - cum);
  }
  if (lane == 0) {
    S.r.Gc = fast_exp(last);
    S.r.cl = cl;
  }
}
// The cumulative log decay of one chunk's rows and beta_r Gam_r, formed as
// stage_gates forms them (a producer's P wave): row r = lane % 32, into
// gam[r] and bgm[r].
__device__ __forceinline__ void chunk_decays(float *gam, float *bgm, const uint32_t *ab, int lane,
                                             int cl, float neg_exp_A, float dtb) {
  const int r = lane & 31;
  const bool valid = r < cl;
  const float a_r = __uint_as_float(lds_read_u32_now(&ab[r]) << 16) + dtb;
  const float b_r = __uint_as_float(lds_read_u32_now(&ab[CH + r]) << 16);
  const float sp = fmaxf(a_r, 0.f) + fast_log(1.f + fast_exp(-fabsf(a_r)));
  const float bt = valid ? __builtin_amdgcn_rcpf(1.f + fast_exp(-b_r)) : 0.f;
  const float cum = scan32(valid ? neg_exp_A * sp : 0.f);
  if (lane < 32) {
    gam[r] = cum;
    bgm[r] = bt * fast_exp(cum);
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
__device__ __forceinline__ void read_row_ops(const bf16 *K, const bf16 *Q, RowOps &o, int m, int g) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    o.k0[kb] = row_op(K, m, kb, g);
    o.k1[kb] = row_op(K, 16 + m, kb, g);
    if (WITH_Q) {
      o.q0[kb] = row_op(Q, m, kb, g);
      o.q1[kb] = row_op(Q, 16 + m, kb, g);
    }
  }
}

// T = (I + A)^-1 of one chunk (P0 of the fused kernel, a T wave of a
// producer): the Gram blocks of k and the whole inverse in fp32, written as
// bf16 A operands, and the record's row factors bgk and tk.  Needs the
// chunk's decays, beta and 1/|k|.  Lane (m, g) holds the Gram entries
// (k_i . k_m), i = 4g + j, of each block, which give column m of A11, row m
// of A22 (the Gram matrix is symmetric) and row m of A21; a round trip
// through the wave's own LDS rows `xs` hands every lane the whole column
// (row) its sweep needs.  Every decay factor is exp(gam_r - gam_i) with
// i <= r, at most 1.
__device__ __forceinline__ void prepare_T(Prep &S, float (&xs)[3][16][20], const RowOps &o,
                                          int lane) {
  Rec &R = S.r;
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 gm_lo = ld4(&S.gam[4 * g]), gm_hi = ld4(&S.gam[16 + 4 * g]);
  const f32x4 bt_lo = ld4(&R.bt[4 * g]);
  const f32x4 ik_lo = ld4(&R.ik[4 * g]), ik_hi = ld4(&R.ik[16 + 4 * g]);
  const float gm_m0 = S.gam[m], gm_m1 = S.gam[16 + m];
  const float ik_m0 = R.ik[m], bik_m1 = R.bt[16 + m] * R.ik[16 + m];
  if (lane < CH) {
    const float ik = R.ik[lane];
    R.bgk[lane] = R.bt[lane] * R.Gm[lane] * ik;
    R.tk[lane] = S.tail[lane] * ik;
  }
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
  bf16 *T0 = reinterpret_cast<bf16 *>(R.T0);
  bf16 *T1 = reinterpret_cast<bf16 *>(R.T1);
  *reinterpret_cast<bf16x4 *>(T1 + 8 * lane + 4) = pack4(f32x4{y[0], y[1], y[2], y[3]});
  const int dst = 16 * (m >> 2), e = m & 3;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    T0[4 * (dst + 4 * j + g) + e] = (bf16)x[j];
    T1[8 * (dst + 4 * g + j) + e] = (bf16)(-t21[j]);
  }
}

// The output mask without the row norms, P[r][i] = exp(gam_r - gam_i)
// (q_r . k_i) for i <= r, of one chunk (scale/|q_r| and 1/|k_i| are applied
// by the output waves), into the record; gam the chunk's cumulative log decay.  IQ_GRAM (P1 of the fused kernel):
// also scale/|q_r| from the Gram diagonal of q, into the record; otherwise
// (a P wave of a producer) the norms are already there.
template <bool IQ_GRAM>
__device__ __forceinline__ void prepare_P(Prep &S, const float *gam, const RowOps &o, int lane,
                                          float eps, float scale) {
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  const f32x4 gm_lo = ld4(&gam[4 * g]), gm_hi = ld4(&gam[16 + 4 * g]);
  const float gm_m0 = gam[m], gm_m1 = gam[16 + m];
  f32x4 p00 = z, p10 = z, p11 = z;  // (K Q^T) blocks: (q_r . k_i), r = 16 rb + m, i = 16 ib + 4g + j
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    p00 = mma32(o.k0[kb], o.q0[kb], p00);
    p10 = mma32(o.k0[kb], o.q1[kb], p10);
    p11 = mma32(o.k1[kb], o.q1[kb], p11);
  }
  if constexpr (IQ_GRAM) {
    f32x4 qq0 = z, qq1 = z;  // Gram diagonal blocks of q
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      qq0 = mma32(o.q0[kb], o.q0[kb], qq0);
      qq1 = mma32(o.q1[kb], o.q1[kb], qq1);
    }
    // lane (m, g = m/4) holds |q_m|^2 in register m%4
    if (g == (m >> 2)) {
      const int cl = S.r.cl;
      const int j = m & 3;
      S.r.iq[m] = (m < cl) ? rsqrtf(qq0[j] + eps) * scale : 0.f;
      S.r.iq[16 + m] = (16 + m < cl) ? rsqrtf(qq1[j] + eps) * scale : 0.f;
    }
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
  S.r.P[0][lane] = pack8(v00, z);
  S.r.P[1][lane] = pack8(v10, v11);
}

// SSD mode: the output mask of one chunk split over both prepare waves (P0
// has no erase work to do there): PART 0 takes rows 0..15 (one diagonal
// block) and the update factors, PART 1 rows 16..31 (the block below it and
// the second diagonal block), each writing its own P slot.  Otherwise as
// prepare_P with q unnormalised.
template <int PART>
__device__ __forceinline__ void prepare_p_ssd(Prep &S, const RowOps &o, int lane) {
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
    S.r.P[0][lane] = pack8(v00, z);
    if (lane < CH) {
      const float ik = S.r.ik[lane];
      S.r.bgk[lane] = S.r.bt[lane] * S.r.Gm[lane] * ik;
      S.r.tk[lane] = S.tail[lane] * ik;
    }
    if (g == 0) {
      const int cl = S.r.cl;
      S.r.iq[m] = (m < cl) ? 1.0f : 0.f;
      S.r.iq[16 + m] = (16 + m < cl) ? 1.0f : 0.f;
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
    S.r.P[1][lane] = pack8(v10, v11);
  }
}

// ------------------------------------------------------------------ waves
// State wave for NT tiles of 16 columns (tiles cw0 .. cw0 + NT - 1 of the
// workgroup's 32): chunk c in step c + LAG: K S, R, Delta = T R,
// S <- Gam_last S + K^T D Delta; it hands the state at chunk entry (before
// step c + LAG) and the scaled Delta (during step c + LAG) to the output
// waves.  The k operands are read once for all tiles, and the tiles'
// independent chains interleave.  Passes nsteps + 1 barriers.
//
// LOOK (cooperative kernel, LAG = 2): K S of a chunk is formed from the
// update it depends on,
//   K_{c+1} S_{c+1} = Gam_last(c) (K_{c+1} S_c) + (K_{c+1} K_c^T) (D_c Delta_c),
// so that R of chunk c+1 splits into a part a K S wave (ks_wave) forms in the
// step before, from v and from the state handed over at chunk c's entry,
//   beta V - beta Gam ik Gam_last(c) (K_{c+1} S_c),
// and one product with the record's cross Gram, scaled by -beta Gam ik on the
// producer side.  The state wave then reads neither k rows nor v and runs no
// K S products: the dependent chain of its step is the two products of the
// cross Gram, the two of T R, D Delta and the update.
template <int DV, bool SSD, int LAG, bool LOOK, int NT>
__device__ __forceinline__ void state_wave(const MfmaParams &p, Smem &sm, int cw0, int lane,
                                           int nch, int nsteps, size_t state_off, int col0,
                                           uint32_t *progress = nullptr) {
  static_assert(!LOOK || (LAG == 2 && !SSD), "look-ahead needs the rows of chunk c+1 in step c+1");
  // cooperative kernel: issue priority over the staging wave on this SIMD
  if (progress) __builtin_amdgcn_s_setprio(1);
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 S[NT][8];  // S[u][t]: state rows state_row(t, g, j), column col0 + 16 (cw0 + u) + m
  bf16x8 Sb[NT][4];  // its bf16 B operands
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int col = col0 + 16 * (cw0 + u) + m;
    if (p.s0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[u][t][j] = p.s0[state_off + (size_t)state_row(t, g, j) * DV + col];
    } else {
#pragma unroll
      for (int t = 0; t < 8; ++t) S[u][t] = z;
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) Sb[u][kb] = state_operand(S[u][2 * kb], S[u][2 * kb + 1]);
  }
  // LDS operands: the k^T tiles of this chunk (A operands of the state
  // update) are read once the first products are issued, with LOOK at the
  // end of the step before; the k rows of the next chunk (A operands of K S;
  // not with LOOK) and its v are read after the state update, so that they
  // are in registers when the next step starts.
  bf16x8 Kr[2][4], Kt[8], vv[NT];
  bf16x8 dpp[NT];       // LOOK: D_c Delta_c of the chunk before
#pragma unroll
  for (int u = 0; u < NT; ++u) dpp[u] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  auto read_rows = [&](const Stage &sn) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) Kr[mt][kb] = row_op_t(sn.K, 16 * mt + m, kb, g);
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
    const int vr = 4 * g + (m >> 2);
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int vc = 16 * (cw0 + u) + 4 * (m & 3);
      vv[u] = cat8(tr_read(sn.V + v_off(vr, vc)), tr_read(sn.V + v_off(16 + vr, vc)));
    }
  };
  auto hand_state = [&](int c) {
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) sm.sb[c & 1][cw0 + u][kb][lane] = Sb[u][kb];
  };
  // K S products of the rows in Kr with the state operand of tile u
  auto k_times_s = [&](int u, f32x4 (&acc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) acc[mt] = mma32(Kr[mt][kb], Sb[u][kb], acc[mt]);
    }
  };
  block_sync();
  for (int it = 0; it < nsteps; ++it) {
    const int c = it - LAG;
    // cooperative kernel: chunks up to `it` have landed in LDS (records
    // included), so their slots may be refilled
    if (progress && cw0 == 0 && lane == 0) *progress = (uint32_t)(min(it, nch - 1) + 1);
    if (c >= 0 && c < nch) {
      const Stage &st = sm.st[c % NSTAGE];
      const Rec &rc = st.pp.r;
      const bool more = c + 1 < nch;
      // this chunk's tiles and row factors
      const bf16x4 tt0 = rc.T0[lane];
      const bf16x8 tt1 = rc.T1[lane];
      const f32x4 ik0 = ld4(&rc.ik[4 * g]), ik1 = ld4(&rc.ik[16 + 4 * g]);
      const f32x4 tk0 = ld4(&rc.tk[4 * g]), tk1 = ld4(&rc.tk[16 + 4 * g]);
      const float gc = rc.Gc;
      f32x4 bt0, bt1, bk0, bk1;  // not with LOOK
      if constexpr (!LOOK) {
        bt0 = ld4(&rc.bt[4 * g]);
        bt1 = ld4(&rc.bt[16 + 4 * g]);
        bk0 = ld4(&rc.bgk[4 * g]);
        bk1 = ld4(&rc.bgk[16 + 4 * g]);
      }
      // Rr[u][mt]: R[16mt + 4g + j][m] of tile u,
      //   R = beta V - beta Gam ik (K S), rows 4g..4g+3 and 16+4g..16+4g+3
      f32x4 Rr[NT][2];
      if constexpr (LOOK) {
        // the K S wave's beta V - beta Gam ik Gam_last(c-1) (K_c S_{c-1}) (all
        // of R for the first chunk), plus the record's -diag(beta Gam ik) K_c
        // K_{c-1}^T times D_{c-1} Delta_{c-1}
        const bf16x8 gx0 = rc.GX[0][lane], gx1 = rc.GX[1][lane];
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          Rr[u][0] = sm.rp[c & 1][cw0 + u][0][lane];
          Rr[u][1] = sm.rp[c & 1][cw0 + u][1][lane];
          if (c > 0) {
            Rr[u][0] = mma32(gx0, dpp[u], Rr[u][0]);
            Rr[u][1] = mma32(gx1, dpp[u], Rr[u][1]);
          }
        }
      }
      // ks[u][mt]: (K S)[16mt + 4g + j][m] of tile u (not with LOOK)
      f32x4 ks[NT][2];
      if constexpr (!LOOK) {
#pragma unroll
        for (int u = 0; u < NT; ++u) {
          ks[u][0] = z;
          ks[u][1] = z;
          if constexpr (!SSD) k_times_s(u, ks[u]);
        }
      }
      // Gam_last S while the matrix cores run
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t) S[u][t] *= gc;
      // (without LOOK, the k^T reads go between two scheduling barriers; with
      // it, the compiler may interleave the scaling with the products)
      if constexpr (!LOOK) {
        __builtin_amdgcn_sched_barrier(0);
        read_kt(st);  // LOOK: read at the end of the step before
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!LOOK) {
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            Rr[u][0][j] = bt0[j] * (float)vv[u][j] - bk0[j] * ks[u][0][j];
            Rr[u][1][j] = bt1[j] * (float)vv[u][4 + j] - bk1[j] * ks[u][1][j];
          }
      }
      bf16x8 Dp[NT];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const f32x4 R0 = Rr[u][0], R1 = Rr[u][1];
        // Delta = T R, both 16-row blocks from the one bf16 operand of R in
        // slot order; SSD: no erase, Delta = R
        f32x4 d1 = R0, d2 = R1;
        if constexpr (!SSD) {
          const bf16x8 Rb = pack8(R0, R1);
          d1 = mma32(cat8(tt0, bf16x4{0, 0, 0, 0}), Rb, z);
          d2 = mma32(tt1, Rb, z);
        }
        Dp[u] = pack8(tk0 * d1, tk1 * d2);
        // diag(ik) Delta for the outputs of this chunk
        sm.db[c & 1][cw0 + u][lane] = pack8(ik0 * d1, ik1 * d2);
      }
      if constexpr (LOOK) {
#pragma unroll
        for (int u = 0; u < NT; ++u) dpp[u] = Dp[u];
      }
      // S <- Gam_last S + K^T diag(tail ik) Delta
#pragma unroll
      for (int u = 0; u < NT; ++u) {
#pragma unroll
        for (int t = 0; t < 8; ++t) S[u][t] = mma32(Kt[t], Dp[u], S[u][t]);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[u][kb] = state_operand(S[u][2 * kb], S[u][2 * kb + 1]);
      }
      if (more) hand_state(c + 1);
    } else if (c == (LOOK ? -2 : -1) && nch > 0) {
      // the initial state (LOOK: a step early, for the K S wave's K_0 S_0)
      hand_state(0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the handed-over writes are done
    {
      // operands of the next step, read unconditionally (the chunk index
      // clamped into the sequence) so that the loads write the loop's
      // registers directly and stay in flight across the barrier: of chunk
      // c + 1, the k rows and v, or with LOOK the k^T tiles
      const Stage &sr = sm.st[max(min(c + 1, nch - 1), 0) % NSTAGE];
      if constexpr (!LOOK) {
        if constexpr (!SSD) read_rows(sr);
        read_v(sr);
      } else {
        read_kt(sr);
      }
    }
    // no wait for the reads in flight: their buffers are refilled only
    // steps later, and their registers are waited for where they are used
    block_sync<63, false>();
  }
  if (p.sT) {
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int col = col0 + 16 * (cw0 + u) + m;
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) p.sT[state_off + (size_t)state_row(t, g, j) * DV + col] = S[u][t][j];
    }
  }
}

// K S wave of tile cw (cooperative kernel, alongside a LOOK state wave): in
// step it, for chunk c = it - 1, the part of R that does not wait for the
// previous chunk's Delta,
//   beta V - beta Gam ik Gam_last(c-1) (K_c S_{c-1})   (beta V - beta Gam ik K_0 S_0 for c = 0),
// from the state the state wave handed over at the entry of chunk c - 1 (0),
// for the state wave's step it + 1.  Passes nsteps + 1 barriers.
template <int LAG>
__device__ __forceinline__ void ks_wave(Smem &sm, int cw, int lane, int nch, int nsteps) {
  static_assert(LAG == 2, "the state wave runs chunk it - 2 in step it");
  // issue priority over the output wave on this SIMD: the state wave waits
  // for this wave's part of R at the start of the next step
  __builtin_amdgcn_s_setprio(3);
  const int m = lane & 15, g = lane >> 4;
  const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
  block_sync();
  for (int it = 0; it < nsteps; ++it) {
    const int cn = it - 1;  // the chunk whose R is prepared
    if (cn >= 0 && cn < nch) {
      const int cs = max(it - 2, 0);  // the state's chunk
      const Stage &st = sm.st[cn % NSTAGE];
      const Rec &rc = st.pp.r;
      f32x4 acc[2] = {z, z};
      // every operand read is issued before the first product waits on one
      bf16x8 sb[4], ko[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sb[kb] = sm.sb[cs & 1][cw][kb][lane];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) ko[kb][mt] = row_op_t(st.K, 16 * mt + m, kb, g);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) acc[mt] = mma32(ko[kb][mt], sb[kb], acc[mt]);
      }
      // v[4g + j][col] and v[16 + 4g + j][col]
      const int vr = 4 * g + (m >> 2), vc = 16 * cw + 4 * (m & 3);
      const bf16x8 vv = cat8(tr_read(st.V + v_off(vr, vc)), tr_read(st.V + v_off(16 + vr, vc)));
      const float gcp = cn > 0 ? sm.st[(cn - 1) % NSTAGE].pp.r.Gc : 1.0f;
      const f32x4 bt0 = ld4(&rc.bt[4 * g]), bt1 = ld4(&rc.bt[16 + 4 * g]);
      const f32x4 bk0 = ld4(&rc.bgk[4 * g]) * gcp, bk1 = ld4(&rc.bgk[16 + 4 * g]) * gcp;
      f32x4 r0, r1;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r0[j] = bt0[j] * (float)vv[j] - bk0[j] * acc[0][j];
        r1[j] = bt1[j] * (float)vv[4 + j] - bk1[j] * acc[1][j];
      }
      sm.rp[cn & 1][cw][0][lane] = r0;
      sm.rp[cn & 1][cw][1][lane] = r1;
    }
    block_sync<63, true>();
  }
}

// Output wave for NT tiles of 16 columns (tiles cw0 ..): in step it, O of
// chunk it - LAG - 1 = (diag(ik) Delta)^T P^T + (Gam iq Q S)^T, then (Q S)^T
// of chunk it - LAG from the state handed over at its entry (the q operands
// are read once for all tiles).  The record entries of a chunk's outputs
// (P, Gam, iq) are read in the step of its Q S and held in registers, so
// that no wave reads a chunk's buffer after step c + LAG.  Passes nsteps + 1
// barriers.
template <int DV, int LAG, int NT>
__device__ __forceinline__ void output_wave(const MfmaParams &p, Smem &sm, int cw0, int lane,
                                            int nch, int nsteps, int64_t t0, int64_t t1, int h,
                                            int col0) {
  const int m = lane & 15, g = lane >> 4;
  f32x4 qsT[NT][2];
  bf16x8 pr0, pr1;
  float gm0, gm1, iq0, iq1;
  block_sync();
  for (int it = 0; it < nsteps; ++it) {
    const int co = it - LAG - 1;
    if (co >= 0 && co < nch) {
      const int64_t row = t0 + (int64_t)co * CH + m;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const bf16x8 Db = sm.db[co & 1][cw0 + u][lane];
        // lane (m, g) gets O[16mt + m][4g..4g+3] = iq (Gam (Q S) + P diag(ik) Delta)
        const f32x4 oc0 = mma32(Db, pr0, qsT[u][0] * gm0) * iq0;
        const f32x4 oc1 = mma32(Db, pr1, qsT[u][1] * gm1) * iq1;
        bf16 *orow = p.o + (row * p.H_v + h) * DV + col0 + 16 * (cw0 + u) + 4 * g;
        if (row < t1) *reinterpret_cast<bf16x4 *>(orow) = pack4(oc0);
        if (row + 16 < t1) *reinterpret_cast<bf16x4 *>(orow + (int64_t)16 * p.H_v * DV) = pack4(oc1);
      }
    }
    const int c = it - LAG;
    if (c >= 0 && c < nch) {
      const Stage &st = sm.st[c % NSTAGE];
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 Sb[NT][4];
#pragma unroll
      for (int u = 0; u < NT; ++u) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) Sb[u][kb] = sm.sb[c & 1][cw0 + u][kb][lane];
        qsT[u][0] = z;
        qsT[u][1] = z;
      }
      // qsT[u][mt]: (Q S)[16mt + m][4g + j]
      bf16x8 qop[4][2];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) qop[kb][mt] = row_op_t(st.Q, 16 * mt + m, kb, g);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
          for (int u = 0; u < NT; ++u) qsT[u][mt] = mma32(Sb[u][kb], qop[kb][mt], qsT[u][mt]);
        }
      }
      // this chunk's output factors, for the next step
      const Rec &rc = st.pp.r;
      pr0 = rc.P[0][lane];
      pr1 = rc.P[1][lane];
      gm0 = rc.Gm[m];
      gm1 = rc.Gm[16 + m];
      iq0 = rc.iq[m];
      iq1 = rc.iq[16 + m];
    }
    block_sync<63, false>();
  }
}

// Chunk c of a sequence [t0, t1) (clamped to the last one: requests past the
// end re-read it into a buffer no one reads again) -> first row and valid rows.
__device__ __forceinline__ void rows_of(int c, int nch, int64_t t0, int64_t t1, int64_t &row0,
                                        int &cl) {
  c = min(c, nch - 1);
  row0 = t0 + (int64_t)c * CH;
  const int64_t rem = t1 - row0;
  cl = rem < CH ? (int)rem : CH;
}

// Request the k (or q) rows of chunk c and one half of its v tile (this
// workgroup's columns): 8 + 1 loads.
template <int DV>
__device__ __forceinline__ void request_rows(const bf16 *x, const bf16 *v, int H_k, int H_v,
                                             int hk, int h, int col0, int64_t row0, int cl,
                                             const RowOffsets &ko, uint32_t voff, bf16 *tile,
                                             bf16 *vtile, int half, int lane) {
  if (cl == CH) {
    dma_rows_full(x + (row0 * H_k + hk) * DK, ko, tile);
    dma16(reinterpret_cast<const bf16 *>(reinterpret_cast<const char *>(v + (row0 * H_v + h) * DV) + voff),
          vtile + 512 * half);
  } else {
    dma_rows(x, H_k, hk, row0, cl, tile, lane);
    dma_v_half(v, H_v, h, col0, row0, cl, vtile, half, lane, DV);
  }
}

// DVT: d_v (64 or 128; d_k is 128).  SSD: the Mamba-2 SSD recurrence on the
// same scan -- no norms, no erase (T = I, Delta = diag(beta) V with no K S),
// g = A delta, beta = delta; the prepare wave P0 only forms half of P.
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
    state_wave<DV, SSD, 2, false, 1>(p, sm, wave - W_C0, lane, nch, nsteps, state_off, col0);
  } else if (wave >= W_O0 && wave < W_O0 + NC) {
    output_wave<DV, 2, 1>(p, sm, wave - W_O0, lane, nch, nsteps, t0, t1, h, col0);
  } else if (wave == W_P0 || wave == W_P1) {
    // ---------------------------------------------------------------- prepare
    // Each step also reads the row operands of the next chunk (published
    // one step earlier), after its own LDS writes have completed, so that
    // the reads overlap the barrier and the next step's wait.
    RowOps ops;
    block_sync();
    for (int it = 0; it < nsteps; ++it) {
      const int c = it - 1;
      if (c >= 0 && c < nch) {
        Prep &pp = sm.st[c % NSTAGE].pp;
        if constexpr (SSD) {
          if (wave == W_P0)
            prepare_p_ssd<0>(pp, ops, lane);
          else
            prepare_p_ssd<1>(pp, ops, lane);
        } else if (wave == W_P0) {
          prepare_T(pp, sm.p0x, ops, lane);
        } else {
          prepare_P<true>(pp, pp.gam, ops, lane, p.eps, p.scale);
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this step's LDS writes are done
      if (it < nch) {
        const Stage &sn = sm.st[it % NSTAGE];
        if (wave == W_P0 && !SSD)
          read_row_ops<false>(sn.K, sn.Q, ops, m, g);
        else
          read_row_ops<true>(sn.K, sn.Q, ops, m, g);
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
    // Step it requests chunk it + AHEAD and waits for chunk it + 1 (read by
    // P1 in step it + 1); an extra first barrier publishes chunk 0.
    if (wave == W_ST0) {
      // k rows and the first half of v
      auto request = [&](int c) {
        int64_t row0;
        int cl;
        rows_of(c, nch, t0, t1, row0, cl);
        Stage &S = sm.st[c % NSTAGE];
        request_rows<DV>(p.k, p.v, p.H_k, p.H_v, hk, h, col0, row0, cl, ko, voff, S.K, S.V, 0, lane);
      };
      // 1/|k| of chunk c once its rows have landed (c < nch)
      auto norms = [&](int c) {
        const int64_t rem = L - (int64_t)c * CH;
        const int cl = rem < CH ? (int)rem : CH;
        Rec &rc = sm.st[c % NSTAGE].pp.r;
        if constexpr (SSD) {  // keys are not normalised
          if (lane < CH) rc.ik[lane] = lane < cl ? 1.0f : 0.0f;
        } else {
          tile_norms(sm.st[c % NSTAGE].K, rc.ik, lane, cl, p.eps, 1.0f);
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
        rows_of(c, nch, t0, t1, row0, cl);
        Stage &S = sm.st[c % NSTAGE];
        request_rows<DV>(p.q, p.v, p.H_k, p.H_v, hk, h, col0, row0, cl, ko, voff, S.Q, S.V, 1, lane);
        dma_ab(p.a, SSD ? p.a : p.b, p.H_v, h, row0, cl, S.ab, lane);  // SSD: no b
      };
      const float neg_exp_A = SSD ? p.A_log[h] : -expf(p.A_log[h]);  // SSD: A itself
      const float dtb = SSD ? 0.0f : p.dt_bias[h];
      // gates of chunk c once its raw a, b have landed (c < nch)
      auto gates = [&](int c) {
        const int64_t rem = L - (int64_t)c * CH;
        Stage &S = sm.st[c % NSTAGE];
        stage_gates<SSD>(S.pp, S.ab, lane, rem < CH ? (int)rem : CH, neg_exp_A, dtb);
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

// ---------------------------------------------------------- cooperative kernel
// A 32-bit word read from the L2, past the scalar cache (glc), complete when
// the statement ends.  `p` is uniform across the wave.
__device__ __forceinline__ uint32_t load_l2_u32(const uint32_t *p) {
  // the address in scalar registers, whatever the compiler could prove
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint64_t sa = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32)) << 32) |
                      (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
  uint32_t v;
  asm volatile("s_load_dword %0, %1, 0x0 glc\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(sa) : "memory");
  return v;
}
// Wait until *p >= want; false, with the XCD's error word marked, if the
// bounded number of polls runs out.  Once the error word is marked every
// later wait on that XCD gives up at once, so a broken launch ends in about
// one wait's bound instead of one per chunk.
__device__ __forceinline__ bool wait_at_least(const uint32_t *p, uint32_t want, uint32_t *err) {
  for (int i = 0; i < SPIN_LIMIT; ++i) {
    if (load_l2_u32(p) >= want) return true;
    if ((i & 63) == 63 && load_l2_u32(err) != 0u) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if ((threadIdx.x & 63) == 0) atomicOr(err, 1u);
  return false;
}

// Wait until progress[r] >= want for every r < nc (nc <= 64): lane r reads
// word r from the L2, all words in one round trip per poll.  Bounded as
// wait_at_least.
__device__ __forceinline__ bool progress_at_least(const uint32_t *progress, int nc, uint32_t want,
                                                  int lane, uint32_t *err) {
  for (int i = 0; i < SPIN_LIMIT; ++i) {
    const uint32_t v = lane < nc ? __hip_atomic_load(&progress[lane], __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : want;
    if (__ballot(v < want) == 0) return true;
    if ((i & 63) == 63 && load_l2_u32(err) != 0u) return false;
    __builtin_amdgcn_s_sleep(1);
  }
  if ((threadIdx.x & 63) == 0) atomicOr(err, 1u);
  return false;
}

__device__ __forceinline__ unsigned char *group_base(const MfmaParams &p, int grp) {
  return p.ws + WS_HEAD + (size_t)grp * p.grp_stride;
}

// Producer workgroup phi of group (n, hk): the records of chunks
// c = phi, phi + PRODUCERS, ... for the gv value heads hk gv .. hk gv + gv - 1.
// Every wave works on its own from the chunk's rows: T wave j (wave j < gv)
// takes value head j's gates, the norms of k and T, P wave j (wave 3 + j)
// that head's decays, the norms of q, the cross Gram and P; the last wave
// also loads the next chunk.  One workgroup barrier per chunk, after which the
// rows of this chunk have landed and the records of the chunk before are
// whole: T wave j then copies that record into its slot (16 bytes per lane,
// not waited for) and forms this chunk's into the other record buffer.  A
// record's flag is set one iteration after its copy, once its stores have long
// reached the L2, so no wave waits on its own stores; before storing a record
// into the slot of chunk c - RING, its T wave checks (from progress words it
// fetched an iteration earlier, or by polling) that every chain workgroup of
// the group has copied that chunk.
__device__ __forceinline__ void producer(const MfmaParams &p, unsigned char *smem, int grp, int phi,
                                         int gv, int nvb, uint32_t *err) {
  ProdSmem &ps = *reinterpret_cast<ProdSmem *>(smem);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int m = lane & 15, g = lane >> 4;
  const int n = grp / p.H_k, hk = grp % p.H_k;
  const int nc = gv * nvb;  // chain workgroups of the group
  int64_t t0, t1;
  seq_bounds(p.cu, p.seq_len, n, t0, t1);
  const int nch = (int)((t1 - t0 + CH - 1) / CH);
  unsigned char *base = group_base(p, grp);
  uint32_t *flags = reinterpret_cast<uint32_t *>(base + GRP_FLAGS);
  const uint32_t *progress = reinterpret_cast<const uint32_t *>(base + GRP_PROGRESS);
  unsigned char *recs = base + GRP_RECS;
  const RowOffsets ko = row_offsets(p.H_k, lane);
  constexpr int LOADER = NWAVES_C - 1;
  auto load = [&](int c, int buf) {  // 8 + 8 + 8 + MAX_GV loads: k, q, previous k rows, a and b
    int64_t row0;
    int cl;
    rows_of(c, nch, t0, t1, row0, cl);
    if (cl == CH) {
      dma_rows_full(p.k + (row0 * p.H_k + hk) * DK, ko, ps.K[buf]);
      dma_rows_full(p.q + (row0 * p.H_k + hk) * DK, ko, ps.Q[buf]);
    } else {
      dma_rows(p.k, p.H_k, hk, row0, cl, ps.K[buf], lane);
      dma_rows(p.q, p.H_k, hk, row0, cl, ps.Q[buf], lane);
    }
    // the chunk before (always full); chunk 0 re-reads itself, its cross
    // Gram is not used
    dma_rows_full(p.k + ((row0 - (c > 0 ? CH : 0)) * p.H_k + hk) * DK, ko, ps.Kp[buf]);
#pragma unroll
    for (int j = 0; j < MAX_GV; ++j)
      dma_ab(p.a, p.b, p.H_v, hk * gv + min(j, gv - 1), row0, cl, ps.ab[buf][j], lane);
    // touch the group's v rows of chunk c - V_TOUCH_BEHIND (gv d_v bf16
    // each: lpr 128-byte lines), one 4-byte load per line into a scratch
    // block, so that the chain workgroups' copies of v find them in the L2.
    // The producers run up to RING chunks ahead of the chains; a chunk that
    // far behind their front is still a few steps ahead of the chains, close
    // enough that its lines are rarely evicted again before the copies.
    const int lpr = gv * nvb * BV / 64;
    int64_t vrow0;
    int vcl;
    rows_of(max(c - V_TOUCH_BEHIND, 0), nch, t0, t1, vrow0, vcl);
#pragma unroll
    for (int t = 0; t < (CH * 2 * MAX_GV + 63) / 64; ++t) {
      if (c >= V_TOUCH_BEHIND && 64 * t < CH * lpr) {
        const int li = min(64 * t + lane, CH * lpr - 1);
        const int r = min(li / lpr, vcl - 1);
        touch4(p.v + ((vrow0 + r) * p.H_v + hk * gv) * (nvb * BV) + 64 * (li % lpr), ps.vtouch);
      }
    }
    // and the k and q rows of this producer's next chunk after c, which the
    // next call of load copies (two 128-byte lines a row)
    if (c + TOUCH_AHEAD < nch) {
      int64_t nrow0;
      int ncl;
      rows_of(c + TOUCH_AHEAD, nch, t0, t1, nrow0, ncl);
      const int64_t rr = nrow0 + min(lane >> 1, ncl - 1);
      touch4(p.k + (rr * p.H_k + hk) * DK + 64 * (lane & 1), ps.vtouch);
      touch4(p.q + (rr * p.H_k + hk) * DK + 64 * (lane & 1), ps.vtouch);
    }
  };
  const bool t_wave = wave < gv;
  const int pj = wave - 3;
  const bool p_wave = pj >= 0 && pj < gv;
  const int j = t_wave ? wave : pj;  // value head of this wave's record part
  const int h = hk * gv + j;
  const float neg_exp_A = (t_wave || p_wave) ? -expf(p.A_log[h]) : 0.f;
  const float dtb = (t_wave || p_wave) ? p.dt_bias[h] : 0.f;
  // T waves: copy the record of chunk `prev` (formed in the last iteration)
  // into its slot, after the slot check
  auto copy_out = [&](int prev, int pbuf) {
    if (prev >= RING) {
      // the slot held chunk prev - RING: every chain workgroup must have copied it
      const uint32_t need = (uint32_t)(prev - RING + 1);
      const uint32_t seen = lds_read_u32_now(&ps.prg[j][lane]);
      if (__ballot(seen < need) != 0) progress_at_least(progress, nc, need, lane, err);
    }
    const uint4 *src = reinterpret_cast<const uint4 *>(&ps.pp[pbuf][j].r);
    uint4 *dst = reinterpret_cast<uint4 *>(recs + ((size_t)j * RING + prev % RING) * REC_BYTES);
#pragma unroll
    for (int i = 0; i < REC_DMAS; ++i) dst[64 * i + lane] = src[64 * i + lane];
  };
  if (wave == LOADER && phi < nch) load(phi, 0);
  int prev = -1;    // T waves: the chunk formed in the last iteration
  int stored = -1;  // T waves: the chunk whose record stores are in flight
  for (int c = phi, k = 0; c < nch; c += PRODUCERS, ++k) {
    const int buf = k & 1;
    const int64_t rem = t1 - (t0 + (int64_t)c * CH);
    const int cl = rem < CH ? (int)rem : CH;
    if (wave == LOADER || t_wave) {
      // loader: chunk c has landed; T waves: the stores of `stored` and the
      // progress words are done
      vm_wait<0>();
      if (t_wave && stored >= 0 && lane == 0) flags[j * RING + stored % RING] = (uint32_t)(stored + 1);
    }
    __syncthreads();
    if (wave == LOADER && c + PRODUCERS < nch) load(c + PRODUCERS, buf ^ 1);
    if (t_wave) {
      if (prev >= 0) {
        copy_out(prev, buf ^ 1);
        stored = prev;
        if (prev == phi) {
          // the first record is flagged as soon as its stores have landed
          // (the chains wait for it to start), not an iteration later
          vm_wait<0>();
          if (lane == 0) flags[j * RING + prev % RING] = (uint32_t)(prev + 1);
          stored = -1;
        }
      } else {
        stored = -1;
      }
      // progress words for the next iteration's slot check (past the L1)
      if (c >= RING)
        __builtin_amdgcn_global_load_lds(
            reinterpret_cast<const void *>(&progress[min(lane, nc - 1)]),
            (__attribute__((address_space(3))) void *)(&ps.prg[j][0]), 4, 0, CPOL_DEVICE);
      Prep &pp = ps.pp[buf][j];
      stage_gates<false>(pp, ps.ab[buf][j], lane, cl, neg_exp_A, dtb);
      tile_norms(ps.K[buf], pp.r.ik, lane, cl, p.eps, 1.0f);
      wave_lds_sync();
      RowOps ops;
      read_row_ops<false>(ps.K[buf], ps.Q[buf], ops, m, g);
      prepare_T(pp, ps.xs[j], ops, lane);
      prev = c;
    } else if (p_wave) {
      Prep &pp = ps.pp[buf][j];
      chunk_decays(ps.gp[j], ps.bgm[j], ps.ab[buf][j], lane, cl, neg_exp_A, dtb);
      tile_norms(ps.K[buf], ps.ikp[j], lane, cl, p.eps, 1.0f);
      tile_norms(ps.Q[buf], pp.r.iq, lane, cl, p.eps, p.scale);
      RowOps ops;
      read_row_ops<true>(ps.K[buf], ps.Q[buf], ops, m, g);
      // GX = K_c K_{c-1}^T: lane (n, g) of output tile (rb, cb) gets
      // (k_{c-1}[16 cb + 4g + j] . k_c[16 rb + n]) = GX[16 rb + n][16 cb + 4g + j],
      // which is its own A operand piece: tile rb, slots 8g + 4 cb + j
      const f32x4 z = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 gx[2][2] = {{z, z}, {z, z}};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const bf16x8 a0 = row_op(ps.Kp[buf], m, kb, g), a1 = row_op(ps.Kp[buf], 16 + m, kb, g);
        gx[0][0] = mma32(a0, ops.k0[kb], gx[0][0]);
        gx[0][1] = mma32(a1, ops.k0[kb], gx[0][1]);
        gx[1][0] = mma32(a0, ops.k1[kb], gx[1][0]);
        gx[1][1] = mma32(a1, ops.k1[kb], gx[1][1]);
      }
      wave_lds_sync();  // bgm and ikp
      // rows scaled by -bgk = -(beta Gam) / |k|, as the T wave forms bgk
      const float s0 = -(ps.bgm[j][m] * ps.ikp[j][m]);
      const float s1 = -(ps.bgm[j][16 + m] * ps.ikp[j][16 + m]);
      pp.r.GX[0][lane] = pack8(gx[0][0] * s0, gx[0][1] * s0);
      pp.r.GX[1][lane] = pack8(gx[1][0] * s1, gx[1][1] * s1);
      wave_lds_sync();
      prepare_P<false>(pp, ps.gp[j], ops, lane, p.eps, p.scale);
    }
  }
  // the last record: whole after the barrier, stored, flagged once stored
  __syncthreads();
  if (t_wave) {
    vm_wait<0>();
    if (stored >= 0 && lane == 0) flags[j * RING + stored % RING] = (uint32_t)(stored + 1);
    if (prev >= 0) {
      const int nk = (nch - 1 - phi) / PRODUCERS + 1;  // iterations run
      copy_out(prev, (nk - 1) & 1);
      vm_wait<0>();
      if (lane == 0) flags[j * RING + prev % RING] = (uint32_t)(prev + 1);
    }
  }
}

// Staging wave of a chain workgroup (cooperative kernel): k rows, the first
// half of v and the record (wave 0), or q rows and the second half of v
// (wave 1).  Step it requests chunk it + AHEAD and waits for chunk it + 1; an
// extra first barrier publishes chunk 0.  Wave 0 fetches the producer's flag
// of chunk c two steps before it requests the chunk (into LDS, past the L1)
// and only polls the flag itself if it was not yet set then.  Passes
// nsteps + 1 barriers.
template <int DV>
__device__ __forceinline__ void coop_staging(const MfmaParams &p, Smem &sm, int which, int lane,
                                             int nch, int nsteps, int64_t t0, int64_t t1, int hk,
                                             int h, int col0, const uint32_t *flag,
                                             const unsigned char *recs, uint32_t *err) {
  if (nch == 0) {  // nothing to load; keep the barrier count
    for (int it = 0; it <= nsteps; ++it) block_sync();
    return;
  }
  const RowOffsets ko = row_offsets(p.H_k, lane);
  const uint32_t voff =
      (uint32_t)(((16 * which + (lane >> 2)) * p.H_v * DV + col0 + 8 * v_src_piece(lane)) * (int)sizeof(bf16));
  auto rows = [&](int c) {  // 9 loads
    int64_t row0;
    int cl;
    rows_of(c, nch, t0, t1, row0, cl);
    Stage &S = sm.st[c % NSTAGE];
    if (which == 0)
      request_rows<DV>(p.k, p.v, p.H_k, p.H_v, hk, h, col0, row0, cl, ko, voff, S.K, S.V, 0, lane);
    else
      request_rows<DV>(p.q, p.v, p.H_k, p.H_v, hk, h, col0, row0, cl, ko, voff, S.Q, S.V, 1, lane);
  };
  auto fetch_flag = [&](int c) {  // 1 load
    const int cc = min(c, nch - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void *>(&flag[cc % RING]),
                                     (__attribute__((address_space(3))) void *)(&sm.fl[c & 3][0]),
                                     4, 0, CPOL_DEVICE);
  };
  auto record = [&](int c, bool fetched) {  // REC_DMAS loads
    const int cc = min(c, nch - 1);
    if (!fetched || lds_read_u32_now(&sm.fl[c & 3][0]) < (uint32_t)(cc + 1))
      wait_at_least(&flag[cc % RING], (uint32_t)(cc + 1), err);
    const unsigned char *rec = recs + (size_t)(cc % RING) * REC_BYTES;
    Stage &S = sm.st[c % NSTAGE];
#pragma unroll
    for (int i = 0; i < REC_DMAS; ++i)
      dma16_l2(rec + 1024 * i + 16 * lane, reinterpret_cast<unsigned char *>(&S.pp.r) + 1024 * i);
  };
  if (which == 0) {
    // the rows of the first chunks are requested before the wait for their
    // records' flags, so that they land while the producers form the records
    fetch_flag(2);
    fetch_flag(3);
    for (int c = 0; c < AHEAD; ++c) rows(c);
    for (int c = 0; c < AHEAD; ++c) record(c, false);
    static_assert(AHEAD == 2, "the wait below leaves only chunk 1's record in flight");
    vm_wait<REC_DMAS>();  // chunks 0 and 1 have landed but chunk 1's record, flags 2 and 3 too
    block_sync<REC_DMAS>();
    for (int it = 0; it < nsteps; ++it) {
      fetch_flag(it + AHEAD + 2);
      record(it + AHEAD, true);
      rows(it + AHEAD);
      vm_wait<CST0_OPS + 1>();  // chunk it + 1 has landed, and the flag of it + 3
      block_sync<CST0_OPS + 1>();
    }
  } else {
    for (int c = 0; c < AHEAD; ++c) rows(c);
    vm_wait<CST1_OPS * (AHEAD - 1)>();  // chunk 0 has landed
    block_sync<CST1_OPS * (AHEAD - 1)>();
    for (int it = 0; it < nsteps; ++it) {
      rows(it + AHEAD);
      vm_wait<CST1_OPS * (AHEAD - 1)>();  // chunk it + 1 has landed
      block_sync<CST1_OPS * (AHEAD - 1)>();
    }
  }
  vm_wait<0>();
}

// One workgroup per compute unit (its LDS admits no second one), all
// resident together.  Role by arrival order on this workgroup's XCD: slot s
// of XCD x holds group s * nxcd + x, whose first PRODUCERS arrivals are its
// producers and the next gv * nvb its chain workgroups (value head j = r /
// nvb, 32 columns vb = r % nvb), so a chain workgroup never waits on a
// producer that has not started.  The last workgroup of an XCD to finish
// clears that XCD's counters, flags and progress words for the next call.
template <int DVT>
__global__ __launch_bounds__(64 * NWAVES_C) void chunked_coop_kernel(MfmaParams p) {
  constexpr int DV = DVT;
  constexpr int NVB = DV / BV;
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem &sm = *reinterpret_cast<Smem *>(smem_raw);
  __shared__ int role_index, last_of_xcd;
  XcdLine *xl = reinterpret_cast<XcdLine *>(p.ws);
  const int x = (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15) % p.nxcd;  // XCC_ID
  if (threadIdx.x == 0) role_index = (int)atomicAdd(&xl[x].arrive, 1u);
  __syncthreads();
  const int idx = role_index;
  const int slot = idx / p.gs, r = idx % p.gs;
  const int grp = slot * p.nxcd + x;
  const int gv = p.H_v / p.H_k;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (slot < p.slots && grp < p.groups) {
    unsigned char *base = group_base(p, grp);
    if (r >= PRODUCERS) {
      const int rc = r - PRODUCERS;  // chain workgroup index in the group
      const int j = rc / NVB, vb = rc % NVB;
      const int n = grp / p.H_k, hk = grp % p.H_k, h = hk * gv + j;
      int64_t t0, t1;
      seq_bounds(p.cu, p.seq_len, n, t0, t1);
      const int nch = (int)((t1 - t0 + CH - 1) / CH);
      const int nsteps = nch + 3;  // state: chunk it-2, outputs: chunk it-3
      const size_t state_off = ((size_t)n * p.H_v + h) * DK * DV;
      const int col0 = vb * BV;
      if (wave < CW_O0) {
        state_wave<DV, false, 2, true, 1>(p, sm, wave, lane, nch, nsteps, state_off, col0,
                                          reinterpret_cast<uint32_t *>(base + GRP_PROGRESS) + rc);
      } else if (wave < CW_ST0) {
        output_wave<DV, 2, 1>(p, sm, wave - CW_O0, lane, nch, nsteps, t0, t1, h, col0);
      } else if (wave >= CW_KS0) {
        ks_wave<2>(sm, wave - CW_KS0, lane, nch, nsteps);
      } else {
        coop_staging<DV>(p, sm, wave - CW_ST0, lane, nch, nsteps, t0, t1, hk, h, col0,
                         reinterpret_cast<const uint32_t *>(base + GRP_FLAGS) + j * RING,
                         base + GRP_RECS + (size_t)j * RING * REC_BYTES, &xl[x].err);
      }
    } else {
      producer(p, smem_raw, grp, r, gv, NVB, &xl[x].err);
    }
  }
  vm_wait<0>();
  __syncthreads();
  if (threadIdx.x == 0) last_of_xcd = atomicAdd(&xl[x].done, 1u) == (uint32_t)(XCD_CUS - 1);
  __syncthreads();
  if (last_of_xcd) {
    // every workgroup of this XCD has finished: clear its groups' flags and
    // progress words, then its counters
    for (int s = 0; s < p.slots; ++s) {
      const int gg = s * p.nxcd + x;
      if (gg >= p.groups) break;
      uint32_t *w = reinterpret_cast<uint32_t *>(group_base(p, gg));
      for (int i = threadIdx.x; i < (int)(GRP_RECS / 4); i += blockDim.x) w[i] = 0u;
    }
    vm_wait<0>();
    __syncthreads();
    if (threadIdx.x == 0) {
      xl[x].arrive = 0u;
      xl[x].done = 0u;
    }
  }
}

template <int DVT, bool SSD>
hipError_t launch_kernel(const Problem &pr, const FwdArgs &x, hipStream_t s) {
  MfmaParams p{};
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

// The cooperative kernel's layout for a problem, or ok = false when the
// problem does not take it: the rule (not SSD) in bf16 with d_k = 128,
// d_v = 64 or 128, chunk 32, at most MAX_GV value heads per key head, and
// every (sequence, key head) group's chain and producer workgroups fitting
// one XCD of the current device at once.
struct CoopPlan {
  bool ok = false;
  int nxcd = 0, slots = 0, gs = 0, groups = 0;
  size_t grp_stride = 0, bytes = 0;
};
// The cooperative kernel keeps one workgroup per compute unit only if two of
// its LDS footprints do not fit one.
static_assert(2 * sizeof(Smem) > 160 * 1024, "one workgroup per compute unit");
static_assert(GRP_PROGRESS + 4 * MAX_GV * (DK / BV) <= GRP_RECS && 4 * MAX_GV * RING <= GRP_PROGRESS,
              "group header layout");
static_assert(sizeof(ProdSmem) <= sizeof(Smem), "a producer's LDS fits the launch's");

CoopPlan coop_plan(const Problem &pr) {
  CoopPlan c;
  if (pr.mode != kModeRule || pr.dtype != GDR_BF16 || pr.d_k != DK || pr.chunk != CH) return c;
  if (pr.d_v != 64 && pr.d_v != 128) return c;
  const int gv = pr.H_v / pr.H_k;
  if (gv > MAX_GV) return c;
  const int64_t groups = (int64_t)pr.num_seqs * pr.H_k;
  if (groups <= 0) return c;
  // the current device's compute units; with no device to ask (a host-only
  // size query), the full gfx950: 8 XCDs of 32
  int dev = 0, ncu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    ncu = 8 * XCD_CUS;
  }
  if (ncu <= 0 || ncu % XCD_CUS != 0 || ncu / XCD_CUS > MAX_XCD) return c;
  c.nxcd = ncu / XCD_CUS;
  c.gs = gv * (pr.d_v / BV) + PRODUCERS;
  c.slots = XCD_CUS / c.gs;
  if ((groups + c.nxcd - 1) / c.nxcd > c.slots) return c;
  c.groups = (int)groups;
  c.grp_stride = GRP_RECS + (size_t)gv * RING * REC_BYTES;
  c.bytes = WS_HEAD + (size_t)c.groups * c.grp_stride;
  c.ok = true;
  return c;
}

template <int DVT>
hipError_t launch_coop(const Problem &pr, const FwdArgs &x, const CoopPlan &c, void *ws,
                       hipStream_t s) {
  MfmaParams p{};
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
  p.ws = static_cast<unsigned char *>(ws);
  p.grp_stride = c.grp_stride;
  p.nxcd = c.nxcd;
  p.slots = c.slots;
  p.gs = c.gs;
  p.groups = c.groups;
  const size_t smem = sizeof(Smem);
  auto kern = chunked_coop_kernel<DVT>;
  hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  // An ordinary launch of one workgroup per compute unit: on a device that
  // runs nothing else they all start at once.  (A cooperative launch, which
  // guarantees that, costs about 20 us more per call on this runtime.)  A
  // kernel of another stream that holds compute units only delays the
  // workgroups it displaces; the bounded waits mark the error word if that
  // lasts beyond their limit.
  hipLaunchKernelGGL(kern, dim3((unsigned)(XCD_CUS * c.nxcd)), dim3(64 * NWAVES_C),
                     (unsigned)smem, s, p);
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

int chunked_coop_seqs_per_launch(const Problem &pr) {
  if (pr.num_seqs <= 0) return 0;
  Problem one = pr;
  one.num_seqs = 1;
  const CoopPlan c = coop_plan(one);
  if (!c.ok) return 0;
  const int fit = c.slots * c.nxcd / pr.H_k;  // sequences whose groups fit at once
  return fit < pr.num_seqs ? fit : pr.num_seqs;
}

size_t chunked_coop_workspace_bytes(const Problem &pr) {
  const int per = chunked_coop_seqs_per_launch(pr);
  if (per <= 0) return 0;
  Problem sub = pr;
  sub.num_seqs = per;
  const CoopPlan c = coop_plan(sub);
  return c.ok ? c.bytes : 0;
}

// Block g < groups clears group g's flags and progress words, block `groups`
// the per-XCD lines.
__global__ __launch_bounds__(128) void clear_coop_kernel(unsigned char *ws, int groups,
                                                         size_t grp_stride) {
  static_assert(GRP_RECS == 128 * 4 && WS_HEAD == 128 * 16, "one store per thread");
  const int b = blockIdx.x;
  if (b < groups) {
    reinterpret_cast<uint32_t *>(ws + WS_HEAD + (size_t)b * grp_stride)[threadIdx.x] = 0u;
  } else {
    reinterpret_cast<uint4 *>(ws)[threadIdx.x] = uint4{0u, 0u, 0u, 0u};
  }
}

hipError_t clear_chunked_coop(const Problem &pr, void *ws, hipStream_t s) {
  const CoopPlan c = coop_plan(pr);
  if (!c.ok) return hipErrorInvalidValue;
  hipLaunchKernelGGL(clear_coop_kernel, dim3((unsigned)(c.groups + 1)), dim3(128), 0, s,
                     static_cast<unsigned char *>(ws), c.groups, c.grp_stride);
  return hipGetLastError();
}

hipError_t launch_chunked_coop(const Problem &pr, const FwdArgs &x, void *ws, hipStream_t s) {
  const CoopPlan c = coop_plan(pr);
  if (!c.ok) return hipErrorInvalidValue;
  return pr.d_v == 64 ? launch_coop<64>(pr, x, c, ws, s) : launch_coop<128>(pr, x, c, ws, s);
}

}  // namespace gdr
