// Internal interface between the C-ABI layer (api.hip) and the kernel files.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

#include "gdr.h"

namespace gdr {

// A validated copy of gdr_shape with the defaults resolved.
struct Problem {
  int num_seqs;
  int seq_len;             // dense batches only
  int64_t total;           // tokens in the batch
  const int32_t *cu;       // device prefix sums, or nullptr for a dense batch
  int H_k, H_v, d_k, d_v;
  gdr_dtype dtype;
  int chunk;
  float scale;             // resolved: never <= 0
  float eps;
  // kModeRule: the gated delta rule.  kModeSSD: the Mamba-2 SSD recurrence
  // on the same kernels: no L2 norm (scale 1), no erase, g = A delta and
  // beta = delta, with `a` carrying delta, `A_log` carrying A itself and b,
  // dt_bias unused.  kModeKDA: the rule with one decay per key channel,
  // g[i] = -exp(A_log) softplus(a[i] + dt_bias[i]) with a [total, H_v, d_k]
  // and dt_bias [H_v, d_k].
  int mode = 0;
};

constexpr int kModeRule = 0;
constexpr int kModeSSD = 1;
constexpr int kModeKDA = 2;

// Pointers of one forward call (types erased; dtype in Problem).
struct FwdArgs {
  const void *q, *k, *v, *a, *b;
  const float *A_log, *dt_bias;
  const float *s0;  // may be nullptr (zeros)
  void *o;
  float *sT;        // may be nullptr (dropped); may equal s0
};

struct GatesArgs {
  const void *q, *k, *a, *b;
  const float *A_log, *dt_bias;
  void *q_hat, *k_hat;
  float *g, *beta;
};

// Short convolution + SiLU producing q, k, v (channels q | k | v of x).
struct ConvArgs {
  int width;
  const void *x;
  const float *weight, *bias;  // bias may be nullptr
  const void *s_in;            // may be nullptr (zero history)
  void *s_out;                 // may be nullptr (dropped); may equal s_in
  void *q, *k, *v;
};

// Gated RMSNorm of the rule's output rows.
struct NormArgs {
  const void *o, *z;
  const float *weight;
  float eps;
  void *out;  // may equal o or z
};

// Workspace of the segmented chunked form (byte offsets, 256-byte aligned).
struct SplitLayout {
  int P;   // segments per sequence of a dense batch (0 for a packed one)
  int NP;  // segment slots of the batch (packed: an upper bound, the rest empty)
  size_t zero_v, ident, M, Sloc, Sin;
  size_t o_m;             // the M pass's d_k-wide outputs (when d_k != d_v)
  size_t coop;            // the cooperative form's workspace for the passes (else == seg_cu)
  size_t seg_cu, seg_off; // packed batches: the segments' prefix sums and offsets
  size_t prep;  // KDA on the two-launch form: the prep records (else == bytes)
  size_t bytes;
};
// Segment slots of the segmented form: N * (T / segment_len) for a dense
// batch, total / segment_len + N for a packed one (every sequence of L tokens
// has max(1, ceil(L / segment_len)) segments).
int64_t split_slots(const Problem &p, int segment_len);
SplitLayout split_layout(const Problem &p, int segment_len);
hipError_t launch_chunked_split(const Problem &p, const FwdArgs &x, int segment_len,
                                void *workspace, hipStream_t s);

hipError_t launch_gates(const Problem &p, const GatesArgs &x, hipStream_t s);
hipError_t launch_conv_silu(const Problem &p, const ConvArgs &x, hipStream_t s);
hipError_t launch_gated_rmsnorm(const Problem &p, const NormArgs &x, hipStream_t s);
// y <- y * SiLU(z) over [total, H_v, d_v] (the SSD's optional gate).
hipError_t launch_silu_gate(const Problem &p, void *y, const void *z, hipStream_t s);
hipError_t launch_recurrent(const Problem &p, const FwdArgs &x, hipStream_t s);
hipError_t launch_chunked_vec(const Problem &p, const FwdArgs &x, hipStream_t s);
// fp32 inputs of the rule on the matrix cores in fp32 (d_k = 64 or 128,
// d_v = 16, 32, 64 or 128, chunk 32); launch_chunked_vec runs it where it
// applies.
bool chunked_f32mma_supports(const Problem &p);
hipError_t launch_chunked_f32mma(const Problem &p, const FwdArgs &x, hipStream_t s);
hipError_t launch_chunked_mfma(const Problem &p, const FwdArgs &x, hipStream_t s);

// Shapes each kernel family is instantiated for.
bool recurrent_supports(const Problem &p);
bool chunked_vec_supports(const Problem &p);
// KDA chunked form on the matrix cores (bf16, d_k = 128, d_v = 64 or 128, chunk 32).
bool chunked_kda_supports(const Problem &p);
hipError_t launch_chunked_kda(const Problem &p, const FwdArgs &x, hipStream_t s);
bool chunked_mfma_supports(const Problem &p);
// The matrix-core chunked form as one launch of one workgroup per compute
// unit (producer workgroups form every chunk's record once per value head, the
// chain workgroups read them through the workspace): 0 bytes when the problem
// or the current device does not take it.  launch_chunked_coop needs a
// zero-filled workspace of that size and leaves it zero-filled; a failed
// launch returns its error before anything runs.
size_t chunked_coop_workspace_bytes(const Problem &p);
// Sequences whose (sequence, key head) groups fit one cooperative launch at
// once (at most p.num_seqs), or 0 when the problem has no cooperative form.
// A batch of more sequences runs as consecutive launches of that many
// sequences each on one workspace of chunked_coop_workspace_bytes(p) bytes,
// which is sized for one such launch.
int chunked_coop_seqs_per_launch(const Problem &p);
hipError_t launch_chunked_coop(const Problem &p, const FwdArgs &x, void *workspace,
                               hipStream_t s);
// Whether gdr_chunked_fwd takes the cooperative form for a batch of which
// `per` sequences fit one launch (per = chunked_coop_seqs_per_launch(p)).
bool coop_runs(const Problem &p, int per);
// The cooperative form over consecutive launches of `per` sequences on one
// workspace of chunked_coop_workspace_bytes(p) bytes that is zero where
// clear_chunked_coop zeroes it (each launch leaves it so); a launch that
// fails runs the one-launch form for its sequences.
hipError_t run_coop_batches(const Problem &p, const FwdArgs &x, int per, void *workspace,
                            hipStream_t s);
// Zero, on stream s, what launch_chunked_coop needs zero in a workspace of
// chunked_coop_workspace_bytes(p) bytes (its counters, error words, flags and
// progress words; not the records), with a fill kernel.
hipError_t clear_chunked_coop(const Problem &p, void *workspace, hipStream_t s);
// KDA chunked form in two launches (per-chunk operands for every chunk of the
// batch into a workspace, then the chains): bf16, d_k = 128, d_v a multiple
// of 16, chunk 32.  kda_two_pass_bytes is 0 for other shapes.
bool kda_two_pass_supports(const Problem &p);
size_t kda_two_pass_bytes(const Problem &p);
hipError_t launch_kda_two_pass(const Problem &p, const FwdArgs &x, void *workspace,
                               hipStream_t s);
// The two launches on their own: the prep reads q, k, a, b, A_log, dt_bias
// and writes the workspace; the chains read it with v and the states.  One
// prep serves any number of chain launches on the same q, k, a, b.
hipError_t launch_kda_prep(const Problem &p, const FwdArgs &x, void *workspace, hipStream_t s);
hipError_t launch_kda_chain(const Problem &p, const FwdArgs &x, const void *workspace,
                            hipStream_t s);

}  // namespace gdr
