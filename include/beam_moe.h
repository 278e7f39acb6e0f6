/*
 * beam_moe.h -- C ABI of the Beam MoE block forward pass on one MI355X (gfx950).
 *
 * The operation (Reflection Beam 1.0 overview page, agentlenshq.com, section
 * "Mixture of Experts: 256 experts, 8 routed per token"; the same statement on
 * the aixai.ru page, section "256 experts per layer", and the dothoosh.com
 * page, section "Architecture and memory efficiency"):
 *
 *   s[t,e]   = sigmoid( x[t,:] . W_router[:,e] + b[e] )          all E experts, FP32
 *   groups   = E/G contiguous experts; group score = sum of its top-2 s
 *   kept     = the Gk best groups; chosen = the K best experts inside them
 *   w[t,k]   = alpha * s[t,e_k] / sum_k' s[t,e_k']                normalised, x alpha (2.5)
 *   y_e(x)   = W_down[e] ( SiLU(W_gate[e] x) * (W_up[e] x) )       SwiGLU expert, product in FP32
 *   out[t,:] = sum_k w[t,k] * y_{e_k}(x[t,:])                      no shared expert
 *
 * The overview page's "Residual stream" section lists the router and the
 * SwiGLU product among the places computed in FP32.  Linear outputs (h after
 * the SwiGLU product, each expert's y, the combined out) are rounded to bf16.
 *
 * Conventions for every entry point:
 *   - Pointers marked [device] are HIP device pointers; all others are host.
 *     The caller owns every buffer; the library allocates nothing and keeps no
 *     state between calls.  Device pointers must be 16-byte aligned.
 *   - Matrices are row-major.  Expert weights are stored [E, out, in]: the
 *     reduction dimension is contiguous, in row order or, when the config asks
 *     for it, in fragment order (beam_moe_wlayout below).  bf16 tensors are passed as raw
 *     16-bit patterns, e4m3 tensors as raw bytes (OCP e4m3fn: bias 7, max 448,
 *     S.1111.111 = NaN).
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     null stream) and returns without synchronising.  No call reads results
 *     back to the host, so calls can be captured into a HIP graph.
 *   - Arguments are checked before anything is enqueued: a call that returns
 *     an error has enqueued nothing (BEAM_MOE_ERR_HIP excepted: it reports a
 *     failed launch).  T == 0 returns BEAM_MOE_OK with no work.
 *   - Inputs are read-only and must not overlap outputs or the workspace.
 *     Concurrent calls on different streams need separate workspaces.
 *   - NaN or Inf in inputs give unspecified results.
 */
#ifndef BEAM_MOE_H
#define BEAM_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BEAM_MOE_OK = 0,
  BEAM_MOE_ERR_INVALID = -1,      /* null pointer, bad size, bad config */
  BEAM_MOE_ERR_UNSUPPORTED = -2,  /* a valid configuration this build does not handle */
  BEAM_MOE_ERR_WORKSPACE = -3,    /* workspace missing or too small */
  BEAM_MOE_ERR_HIP = -4           /* a HIP launch failed */
} beam_moe_status;

/* Expert weight formats.  MXFP4 (OCP Microscaling: the MI355X analogue of the
 * pages' NVFP4 checkpoint, overview page, section "Mixture of Experts"): each
 * block of 32 consecutive inputs of an output row shares an E8M0 scale byte e
 * (value 2^(e-127); codes 1..254), and each weight is an FP4 E2M1 code (values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives), two per byte with the
 * lower-indexed weight in the low nibble.  MXFP4 needs H and I to be multiples
 * of 256.  It never takes the LDS-tiled GEMMs: it runs on the one-workgroup-
 * per-CU GEMMs at 32 to 64 rows per expert on average and on the weight-
 * streaming GEMMs otherwise. */
typedef enum { BEAM_MOE_W_BF16 = 0, BEAM_MOE_W_FP8_E4M3 = 1, BEAM_MOE_W_MXFP4 = 2 } beam_moe_wtype;

/* Byte order of the expert weight matrices and, for MXFP4, of their scale matrices (FP8 scales
 * always stay in row order).  The pages fix no storage order; these are two orders of the same
 * bytes, and a forward gives bit-identical results with either.
 *   ROWS       [E, out, in] as described with each entry point: every row's bytes contiguous.
 *   FRAGMENTS  each expert matrix, taken as R rows of B bytes (B = 2*in for bf16, in for e4m3,
 *              in/2 for MXFP4 codes), is cut into blocks of 16 consecutive rows, and each block
 *              into 64-byte column slices.  Slice f of block b is stored as 1024 contiguous bytes
 *              at byte 16*B*b + 1024*f of the matrix, whose byte 16*(r + 16*c) + j holds byte
 *              64*f + 16*c + j of the block's row r (r < 16, c < 4, j < 16).  That is the order
 *              in which the 64 lanes of a wavefront take a 16 x 16 x 32 matrix-core operand, so
 *              one 16-byte load per lane reads 1 KB of consecutive addresses.  The matrix keeps
 *              its size; beam_moe_pack_weights writes this order from row order.
 *              MXFP4 scale matrices (R rows of S = in/32 bytes) take the same order with 16-byte
 *              column slices: slice g of block b is 256 bytes at byte 16*S*b + 256*g, whose byte
 *              16*r + j holds byte 16*g + j of the block's row r (the scales of four 128-deep
 *              windows of 16 rows, read as two whole cache lines); beam_moe_pack_scales writes
 *              it.  MXFP4 in this order needs H and I to be multiples of 512. */
typedef enum { BEAM_MOE_LAYOUT_ROWS = 0, BEAM_MOE_LAYOUT_FRAGMENTS = 1 } beam_moe_wlayout;

typedef enum {
  BEAM_MOE_OP_ROUTE = 0,
  BEAM_MOE_OP_PERMUTE = 1,
  BEAM_MOE_OP_FORWARD = 2,
  BEAM_MOE_OP_BLOCK = 3
} beam_moe_op;

/* Layer configuration (host struct, read at call time).
 * Beam's real shape: hidden 5120, inter 2560, 256 experts in 8 groups of 32,
 * 4 kept groups, top-8, alpha 2.5 (overview page, "Mixture of Experts"). */
typedef struct {
  int32_t hidden;       /* H: multiple of 128 (256 for MXFP4) */
  int32_t inter;        /* I: multiple of 128 (256 for MXFP4) */
  int32_t n_experts;    /* E: 1..256 */
  int32_t n_groups;     /* G: 1..64, E % G == 0, E/G >= 2 (a group's score sums its two best) */
  int32_t topk_groups;  /* Gk: 1..G */
  int32_t top_k;        /* K: 1..8, K <= Gk * E / G */
  float routed_scale;   /* alpha: finite */
  int32_t weight_type;  /* beam_moe_wtype */
  int32_t weight_layout;  /* beam_moe_wlayout of w_gate, w_up and w_down (and of MXFP4 s_gate, s_up, s_down) */
} beam_moe_config;

/* Largest T accepted by every entry point. */
#define BEAM_MOE_MAX_TOKENS 262144

/* Largest hidden size of the norm entry points (a row of fp32 squares is staged in 32 KB of LDS). */
#define BEAM_MOE_MAX_NORM_HIDDEN 8192

/* Static, NUL-terminated description of a status code (host only). */
const char* beam_moe_status_string(int status);

/* Workspace bytes that `op` needs for T tokens (host only, pure).
 * Writes *bytes and returns BEAM_MOE_OK, or an error for an invalid cfg/T/op.
 * The forward workspace holds the router partial logits, the routing table
 * (unless the caller supplies it), the permutation, the per-row SwiGLU
 * activations h [T*K, I] bf16 and the per-row expert outputs y [T*K, H] bf16. */
int beam_moe_workspace_bytes(const beam_moe_config* cfg, int32_t T, int32_t op, size_t* bytes);

/* Router and group-limited selection.
 *   x          [device] [T, H] bf16 (the MoE block's input, i.e. the pre-normed hidden state)
 *   w_router   [device] [H, E] fp32 (row h holds the E expert weights of input channel h)
 *   b_router   [device] [E] fp32, or NULL for no bias column
 *   topk_ids   [device] [T, K] int32 out: the K chosen experts, ascending expert id
 *   topk_w     [device] [T, K] fp32 out: alpha * s / sum(s) over the K chosen, same order
 *   workspace  [device] beam_moe_workspace_bytes(ROUTE) bytes (may be NULL if that is 0)
 * Ties at a selection boundary go to the lower group index / lower expert id. */
int beam_moe_route(const beam_moe_config* cfg, int32_t T,
                   const void* x, const float* w_router, const float* b_router,
                   int32_t* topk_ids, float* topk_w,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Token -> expert permutation of the T*K (token, slot) pairs p = t*K + k.
 * On one GPU the dispatch to experts and the merge back (breadlab.ai Beam
 * inference post, section "Reading 23B active and 501B resident separately")
 * become this grouping and its inverse.
 *   topk_ids        [device] [T, K] int32 in: distinct ids in [0, E) per token
 *                   (as beam_moe_route writes them); other values give
 *                   unspecified output but no out-of-bounds access
 *   expert_offsets  [device] [E+1] int32 out: rows of expert e are [off[e], off[e+1]); off[E] = T*K
 *   sorted_pairs    [device] [T*K] int32 out: pair index of each row; pairs grouped by
 *                   expert, ascending p (so ascending token) within an expert
 *   pair_to_row     [device] [T*K] int32 out: inverse of sorted_pairs
 *   workspace       [device] beam_moe_workspace_bytes(PERMUTE) bytes
 * Deterministic: the result does not depend on scheduling. */
int beam_moe_permute(const beam_moe_config* cfg, int32_t T, const int32_t* topk_ids,
                     int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pair_to_row,
                     void* workspace, size_t workspace_bytes, void* stream);

/* The whole block: route, permute, grouped SwiGLU experts, weighted combine.
 *   x, w_router, b_router   as in beam_moe_route
 *   w_gate, w_up   [device] [E, I, H] bf16; e4m3 bytes (FP8); [E, I, H/2] packed E2M1 bytes (MXFP4)
 *   w_down         [device] [E, H, I] bf16; e4m3 (FP8); [E, H, I/2] packed E2M1 (MXFP4)
 *   s_gate, s_up   [device] FP8: [E, I] fp32 per-output-channel scales; MXFP4: [E, I, H/32]
 *                  E8M0 bytes; BF16: NULL.  FP8 scales 4-byte aligned, MXFP4 scales 16-byte.
 *   s_down         [device] FP8: [E, H] fp32; MXFP4: [E, H, I/32] E8M0 bytes; BF16: NULL
 *                  an FP8 weight's value is decode(q) * scale[e, out]; an MXFP4
 *                  weight's is e2m1(q) * 2^(scale[e, out, in/32] - 127)
 *   out            [device] [T, H] bf16 out
 *   topk_ids_out, topk_w_out  [device] optional [T, K] copies of the routing (may be NULL)
 *   workspace      [device] beam_moe_workspace_bytes(FORWARD) bytes
 * Combine sums the K weighted expert rows in fp32 in ascending expert id. */
int beam_moe_forward(const beam_moe_config* cfg, int32_t T,
                     const void* x, const float* w_router, const float* b_router,
                     const void* w_gate, const void* w_up, const void* w_down,
                     const void* s_gate, const void* s_up, const void* s_down,
                     void* out, int32_t* topk_ids_out, float* topk_w_out,
                     void* workspace, size_t workspace_bytes, void* stream);

/* beam_moe_forward with stage timestamps, for measuring each kernel on the
 * stream it runs on.  stage_events is NULL (then this is beam_moe_forward) or
 * an array of 7 hipEvent_t created by the caller; event i is recorded on
 * `stream` before stage i and event 6 after the last:
 *   0 router logits | 1 router selection | 2 permutation (3 kernels) |
 *   3 gate/up GEMM + SwiGLU | 4 down GEMM | 5 combine | 6 end. */
int beam_moe_forward_timed(const beam_moe_config* cfg, int32_t T,
                           const void* x, const float* w_router, const float* b_router,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down,
                           void* out, int32_t* topk_ids_out, float* topk_w_out,
                           void* workspace, size_t workspace_bytes, void* stream,
                           void* const* stage_events);

/* Allocation-free forward, for callers that cannot allocate: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation and kernels as beam_moe_forward (bit-identical results), with
 * its workspace in a fixed device array inside this library instead of a caller
 * buffer: BEAM_MOE_NOALLOC_SCRATCH_BYTES (64 MiB) on every GPU the library runs
 * on, held until the process ends (the real-shape layer fits up to about 400
 * tokens).  The caller still passes inputs and outputs, as for beam_moe_forward.
 *   Returns BEAM_MOE_ERR_WORKSPACE, before enqueuing anything, when
 *   beam_moe_workspace_bytes(cfg, T, BEAM_MOE_OP_FORWARD) exceeds the array;
 *   BEAM_MOE_ERR_HIP if the array's address on the current device cannot be
 *   found (looked up once per device, with that device current, at the first
 *   call there).  The kernels run on the device current at the call.
 *   Every call on a device uses that device's one array: calls that overlap on
 *   one device (other streams, other threads) race on it, so issue them in
 *   order on one stream.  Nothing in the array needs to start at zero; it
 *   keeps the last call's intermediates.
 * Calls no hipMalloc, hipFree or allocating routine. */
#define BEAM_MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
int beam_moe_forward_noalloc(const beam_moe_config* cfg, int32_t T,
                             const void* x, const float* w_router, const float* b_router,
                             const void* w_gate, const void* w_up, const void* w_down,
                             const void* s_gate, const void* s_up, const void* s_down,
                             void* out, int32_t* topk_ids_out, float* topk_w_out, void* stream);

/* RMSNorm of bf16 rows (the norm before and after every sublayer: Reflection
 * Beam 1.0 overview, section "Residual stream", which fixes the norms to FP32;
 * RMSNorm with a per-channel gain is the reading, the only norm the pages name):
 *   out[t,h] = bf16( (x[t,h] * r_t) * gamma[h] ),  r_t = 1 / sqrt( ss_t / H + eps )
 * where ss_t is the FP32 sum of x[t,h]^2 in a fixed order (the channels form 64
 * contiguous blocks of whole 8-channel chunks, block l holding chunks
 * [l*n/64, (l+1)*n/64), n = H/8; each block summed in channel order, then the
 * block sums in block order) and every step is one correctly rounded FP32
 * operation, so the result is reproducible bit for bit.
 *   hidden     H: multiple of 8, at most BEAM_MOE_MAX_NORM_HIDDEN
 *   x          [device] [T, H] bf16
 *   gamma      [device] [H] fp32 (4-byte aligned)
 *   eps        finite, > 0
 *   out        [device] [T, H] bf16 out; may be the same buffer as x
 * Latency per token: an (H/64)-term chain per lane plus a 64-term chain (tokens run in parallel). */
int beam_moe_rms_norm(int32_t T, int32_t hidden, const void* x, const float* gamma, float eps, void* out,
                      void* stream);

/* One MoE sublayer with its norms and Beam's constant-scale residual mix
 * (overview page, section "Residual stream": the embedding is step 1; at step k
 * a sublayer's output joins with weight 1/sqrt(k) and the stream keeps weight
 * sqrt((k-1)/k)):
 *   x          = RMSNorm(stream_in; gamma_pre, eps)                 (beam_moe_rms_norm)
 *   moe        = the MoE block on x                                 (beam_moe_forward)
 *   post       = RMSNorm(moe; gamma_post, eps)
 *   stream_out = bf16( fp32(a * stream_in) + fp32(b * post) ),  a = fp32(sqrt((k-1)/k)), b = fp32(1/sqrt(k))
 * The post-norm and the mix run inside the combine kernel.
 *   cfg, w_router ... s_down   as in beam_moe_forward; hidden <= BEAM_MOE_MAX_NORM_HIDDEN
 *   step       k >= 2: this sublayer's position in the stream (layer L's MoE sublayer, 0-based L, is 2L+3)
 *   eps        finite, > 0 (both norms)
 *   stream_in  [device] [T, H] bf16
 *   gamma_pre, gamma_post  [device] [H] fp32
 *   stream_out [device] [T, H] bf16 out; may be the same buffer as stream_in
 *   moe_out    [device] optional [T, H] bf16 copy of the MoE output before the post-norm (may be NULL)
 *   topk_ids_out, topk_w_out  [device] optional, as in beam_moe_forward
 *   workspace  [device] beam_moe_workspace_bytes(BLOCK) bytes (the forward workspace plus x) */
int beam_moe_block_forward(const beam_moe_config* cfg, int32_t T, int32_t step, float eps,
                           const void* stream_in, const float* gamma_pre, const float* gamma_post,
                           const float* w_router, const float* b_router,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down,
                           void* stream_out, void* moe_out, int32_t* topk_ids_out, float* topk_w_out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* beam_moe_block_forward with stage timestamps: stage_events is NULL or 8
 * hipEvent_t recorded on `stream`:
 *   0 pre-norm | 1 router logits | 2 router selection | 3 permutation |
 *   4 gate/up GEMM + SwiGLU | 5 down GEMM | 6 combine + post-norm + mix | 7 end. */
int beam_moe_block_forward_timed(const beam_moe_config* cfg, int32_t T, int32_t step, float eps,
                                 const void* stream_in, const float* gamma_pre, const float* gamma_post,
                                 const float* w_router, const float* b_router,
                                 const void* w_gate, const void* w_up, const void* w_down,
                                 const void* s_gate, const void* s_up, const void* s_down,
                                 void* stream_out, void* moe_out, int32_t* topk_ids_out, float* topk_w_out,
                                 void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events);

/* Dense SwiGLU MLP: the first 3 of Beam's 52 layers use a dense SwiGLU MLP in
 * place of the MoE block (overview page, section "Architecture").  The pages do
 * not give its intermediate size, so it is a parameter.  Same arithmetic as one
 * expert of the MoE block, for every token, with no router and no combine:
 *   out[t,:] = bf16( W_down ( bf16( SiLU(W_gate x) * (W_up x) ) ) )
 * computed by the same grouped-GEMM kernels with one expert. */
typedef struct {
  int32_t hidden;       /* H: multiple of 128 (256 for MXFP4) */
  int32_t inter;        /* I: multiple of 128 (256 for MXFP4) */
  int32_t weight_type;  /* beam_moe_wtype */
  int32_t weight_layout;  /* beam_moe_wlayout of w_gate, w_up and w_down (and of MXFP4 s_gate, s_up, s_down) */
} beam_dense_config;

/* Workspace bytes of beam_dense_mlp_forward for T tokens (host only, pure): the
 * row-tile list, h [T, I] bf16 and, when the GEMMs are split over the
 * reduction to fill the GPU (small T), their fp32 partial sums. */
int beam_dense_workspace_bytes(const beam_dense_config* cfg, int32_t T, size_t* bytes);

/*   x              [device] [T, H] bf16
 *   w_gate, w_up   [device] [I, H] bf16; e4m3 bytes with s_gate, s_up [I] fp32; or MXFP4
 *                  [I, H/2] with s_gate, s_up [I, H/32] E8M0 bytes (16-byte aligned)
 *   w_down         [device] [H, I] bf16; e4m3 with s_down [H] fp32; or MXFP4 [H, I/2] with [H, I/32]
 *   out            [device] [T, H] bf16 out
 *   workspace      [device] beam_dense_workspace_bytes bytes
 * Deterministic: a split reduction adds its parts in a fixed order (for gate/up,
 * before the SwiGLU). */
int beam_dense_mlp_forward(const beam_dense_config* cfg, int32_t T, const void* x,
                           const void* w_gate, const void* w_up, const void* w_down,
                           const void* s_gate, const void* s_up, const void* s_down,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);

/* beam_dense_mlp_forward with stage timestamps: stage_events is NULL or 4
 * hipEvent_t recorded on `stream`: 0 setup | 1 gate/up GEMM + SwiGLU | 2 down GEMM | 3 end. */
int beam_dense_mlp_forward_timed(const beam_dense_config* cfg, int32_t T, const void* x,
                                 const void* w_gate, const void* w_up, const void* w_down,
                                 const void* s_gate, const void* s_up, const void* s_down,
                                 void* out, void* workspace, size_t workspace_bytes, void* stream,
                                 void* const* stage_events);

/* MXFP4 quantisation of bf16 rows (the OCP MX conversion rule): for each block
 * of 32 consecutive values of a row, shared exponent = floor(log2(max |v|)) - 2
 * (2 = E2M1's largest exponent), clamped to [-127, 127], scale byte = shared +
 * 127 (0 for an all-zero block); each v / 2^shared is rounded to the nearest
 * E2M1 value, ties to even mantissa, magnitudes past 6 saturating to 6; the
 * sign bit is set for every v < 0 (so a small negative value becomes -0).
 *   rows, cols  rows >= 0, cols >= 0 a multiple of 32; rows == 0 or cols == 0 is a no-op
 *   w           [device] [rows, cols] bf16 (finite), 16-byte aligned
 *   codes       [device] [rows, cols/2] packed E2M1 out (lower-indexed value in the low nibble), 16-byte aligned
 *   scales      [device] [rows, cols/32] E8M0 bytes out
 * Returns BEAM_MOE_ERR_INVALID for a bad size, a NULL or misaligned pointer.
 * Integer and compare operations only: the result is exact and reproducible. */
int beam_mxfp4_quantize(int32_t rows, int32_t cols, const void* w, void* codes, void* scales, void* stream);

/* Row order -> fragment order (BEAM_MOE_LAYOUT_FRAGMENTS above) of a weight matrix, or of all
 * E expert matrices of one kind at once (they are consecutive blocks of rows).
 *   rows       R: a multiple of 16 (E*I for w_gate/w_up, E*H for w_down)
 *   row_bytes  B: a multiple of 64 (2*in for bf16, in for e4m3, in/2 for MXFP4 codes)
 *   src        [device] R*B bytes in row order, 16-byte aligned
 *   dst        [device] R*B bytes out in fragment order, 16-byte aligned; must not overlap src
 * rows == 0 is a no-op.  Returns BEAM_MOE_ERR_INVALID for a bad size, a NULL or misaligned
 * pointer, or overlapping buffers.  A byte permutation: exact. */
int beam_moe_pack_weights(int64_t rows, int32_t row_bytes, const void* src, void* dst, void* stream);

/* Row order -> fragment order of MXFP4 scale matrices (E8M0 bytes, 16-byte column slices; see
 * BEAM_MOE_LAYOUT_FRAGMENTS), all E expert matrices of one kind at once.
 *   rows       R: a multiple of 16 (E*I for s_gate/s_up, E*H for s_down)
 *   row_bytes  S = in/32: a multiple of 16
 *   src, dst   as in beam_moe_pack_weights (R*S bytes each, 16-byte aligned, not overlapping)
 * rows == 0 is a no-op.  Errors as for beam_moe_pack_weights. */
int beam_moe_pack_scales(int64_t rows, int32_t row_bytes, const void* src, void* dst, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* BEAM_MOE_H */
