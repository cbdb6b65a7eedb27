/*
 * moe_fp4.h -- C ABI of the MI355X (gfx950) routed-expert MoE layer on
 * block-scaled FP4 weights.
 *
 * The layer is the one the MiMo-V2.6-Flash model cards describe:
 *   route   group-limited sigmoid top-k routing ("MiMo-V2.6-Flash -- REAP-50"
 *           card, "Pruning Method": 256 experts in n_group = 8 groups,
 *           topk_group = 4, 8 experts per token, routed_scaling_factor 2.827;
 *           "Evaluation Status Note": e_score_correction_bias)
 *   permute group the (token, k) slots by expert for one grouped kernel
 *           ("MiMo-V2.6-Flash-MOPD on one RTX PRO 6000", "What makes it fast",
 *           the exact grouped kernel of speed v4)
 *   GEMMs   SwiGLU experts, out = W_down(SiLU(W_gate h) * (W_up h)) (REAP-50
 *           card, saliency equation), weights MXFP4 (E2M1 codes + E8M0 per 32,
 *           REAP-50 card "Highlights") or their exact NVFP4 transcode (two
 *           E4M3 per 32 + a power-of-two global, "MiMo-V2.6-Flash-RL: exact
 *           NVFP4 weight conversion", "What changed"); FP32 accumulation with
 *           bfloat16 (W4A16) or NVFP4 (W4A4, unit global scale) activations
 *           ("AxionML / MiMo-V2.6-Flash-MOPD-NVFP4", header, "Usage" and
 *           "Quantization Details")
 *   combine weighted sum of the 8 expert outputs per token
 *   transcode the MXFP4 -> NVFP4 scale transcode and its audit counters
 *           (MOPD-NVFP4 card, "Reproduce the checkpoint")
 *
 * Conventions shared by every call:
 *   - Every pointer is caller-owned DEVICE memory unless stated otherwise.
 *     The library allocates nothing and keeps no state between calls.
 *   - Every call is asynchronous on `stream`; results are deterministic
 *     (no floating-point atomics; integer atomics only where the sum is exact).
 *   - Arguments are checked on the host before anything is launched; on an
 *     error nothing is written and the call returns a non-zero moe_status.
 *     moe_last_error() gives a message for the calling thread's last failure.
 *     Faults inside a kernel surface at the caller's next synchronisation.
 *   - Layouts are row-major with the reduction (K) dimension contiguous.
 *     FP4 codes: element 2i of a row is the low nibble of byte i (OCP MX);
 *     E2M1 nibble = sign | 2-bit exponent | 1-bit mantissa.
 *   - bfloat16 data are passed as `void*` (2 bytes per element).
 */
#ifndef MOE_FP4_H
#define MOE_FP4_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;
#define MOE_OK 0
#define MOE_ERR_INVALID 1      /* a null pointer, a bad size or a bad parameter */
#define MOE_ERR_UNSUPPORTED 2  /* valid in principle, not built (e.g. a shape limit) */
#define MOE_ERR_WORKSPACE 3    /* workspace too small */
#define MOE_ERR_HIP 4          /* a HIP launch failed */

const char* moe_status_string(moe_status s);
/* Message of the calling thread's last non-OK return (empty if none). Host memory, library-owned. */
const char* moe_last_error(void);
/* Library version string (host memory, library-owned). */
const char* moe_version(void);

/* ------------------------------------------------------------------ route
 * For each token t: s_e = sigmoid(logits[t,e]) in float64; c_e = s_e + bias_e
 * (bias may be NULL); group score = sum of the two largest c_e of each of the
 * n_group groups of E/n_group consecutive experts; keep the topk_group groups
 * with the largest score; from the experts of kept groups take the top_k
 * largest c_e.  Ties go to the lower group / expert index.  ids are written in
 * order of c_e descending.  weights: w_j = s_{e_j} / sum_j s_{e_j} * scale when
 * norm_topk_prob != 0, else s_{e_j} * scale (float64 math, stored as float).
 * Limits: E <= 256, E % n_group == 0, E/n_group >= 2, n_group <= 64,
 * 1 <= topk_group <= n_group, 1 <= top_k <= min(16, topk_group * E/n_group).
 *   logits  float [T, E];  correction_bias float [E] or NULL
 *   topk_ids int32 [T, top_k];  topk_weights float [T, top_k]
 * T == 0 is a no-op.  Non-finite logits give unspecified (but in-bounds) ids.
 */
typedef struct {
  int32_t num_experts;
  int32_t n_group;
  int32_t topk_group;
  int32_t top_k;
  float routed_scaling_factor;
  int32_t norm_topk_prob;
} moe_route_params;

moe_status moe_route(const float* logits, const float* correction_bias, int64_t T,
                     const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                     hipStream_t stream);

/* ---------------------------------------------------------------- permute
 * Stable counting sort of the R = T*top_k slots s = t*top_k + j by expert id.
 *   expert_offsets int32 [E+1]: exclusive prefix sum of per-expert counts
 *   sorted_slots   int32 [R]:   slot at permuted row r (ascending slot within an expert)
 *   slot_rows      int32 [R]:   inverse: permuted row of slot s
 * ids outside [0, E) are dropped: they get slot_rows = -1 and no row.
 * workspace: device memory of at least moe_permute_workspace_bytes(T, top_k, E) bytes.
 * Limits: E <= 1024, R < 2^31.
 */
size_t moe_permute_workspace_bytes(int64_t T, int32_t top_k, int32_t num_experts);
moe_status moe_permute(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t num_experts,
                       int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* --------------------------------------------------------- route + permute
 * moe_route followed by moe_permute of the ids it wrote: the same outputs, bit
 * for bit, as the two calls.  When T*top_k <= 2048 (every decode batch) both
 * run in one launch: each router workgroup counts itself in *counter after
 * writing its tokens' ids, and the last one to arrive runs the permutation,
 * then sets *counter back to zero (up to 4 tokens a single workgroup routes
 * and permutes, and the counter is not touched).  Larger batches make the two
 * separate launches (workspace as for moe_permute; counter unused).
 *   counter: one uint32 of device memory, 4-byte aligned, owned by the caller;
 *            zero before the first call, and every call leaves it zero.  Calls
 *            that share a counter must not run concurrently (same stream, or
 *            ordered by events).
 * Limits and errors as moe_route and moe_permute (E <= 256); NULL pointers and
 * a misaligned counter give MOE_ERR_INVALID.
 */
moe_status moe_route_permute(const float* logits, const float* correction_bias, int64_t T,
                             const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                             int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows,
                             uint32_t* counter, void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* ------------------------------------------------ router matmul + route
 * The router's matmul, then the group top-k of moe_route on its float64
 * logits, as two launches on `stream` ("MiMo-V2.6-Flash-MOPD on one RTX PRO
 * 6000", "What makes it fast": one matmul and a fused top-k per layer;
 * "MiMo-V2.6-Flash-RL Mixed-Quant GGUF", "Quantization targets": the router
 * weight stays F32).
 *   logits[t, e] = sum_k x[t, k] * gate_weight[e, k], each product of a bf16
 *   and an FP32 value exact in float64, summed in float64 (fixed order); the
 *   selection and weights then follow moe_route on these float64 logits.
 *   x bf16 [T, hidden]; gate_weight float [E, hidden]; correction_bias float
 *   [E] or NULL; topk_ids int32 [T, top_k]; topk_weights float [T, top_k].
 *   hidden % 512 == 0; T <= 1048560;
 *   x, gate_weight and workspace 16-byte aligned.
 * workspace: at least moe_route_gemv_workspace_bytes(T, E) bytes of device
 * memory (any contents); after the call its first T*E*8 bytes hold the
 * float64 logits [T, E].  Calls sharing a workspace must not run
 * concurrently.  Other limits and errors as moe_route.
 */
size_t moe_route_gemv_workspace_bytes(int64_t T, int32_t num_experts);
moe_status moe_route_gemv(const void* x, const float* gate_weight, const float* correction_bias, int64_t T,
                          int32_t hidden, const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------- route + permute, no allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * outputs, bit for bit, as moe_route_permute, with the hand-off counter and
 * the permutation's count table in a static device array of the library
 * (256 B + 256 KiB per GPU, held until the process ends) instead of caller
 * memory.  The call allocates nothing.  Limit: T * top_k <= 2048 always fits;
 * larger batches need T * top_k * num_experts <= 2^27 (e.g. 524,288 slots at
 * 256 experts), else MOE_ERR_UNSUPPORTED and nothing is launched.  All calls
 * on one GPU share its array: calls that overlap on one GPU (unordered
 * streams) race.  Other limits and errors as moe_route_permute.
 */
moe_status moe_route_permute_noalloc(const float* logits, const float* correction_bias, int64_t T,
                                     const moe_route_params* p, int32_t* topk_ids, float* topk_weights,
                                     int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_rows,
                                     hipStream_t stream);

/* ----------------------------------------------------------- grouped GEMM
 * Per expert e and permuted row r in [expert_offsets[e], expert_offsets[e+1]):
 *   MOE_EPI_NONE:   out[r, n]  = sum_k A[r, k] * W0[e, n, k]
 *   MOE_EPI_SWIGLU: out[r, n]  = SiLU(sum_k A[r,k] W0[e,n,k]) * (sum_k A[r,k] W1[e,n,k])
 * with exact dequantised operands and FP32 accumulation.  The result is
 * rounded to bfloat16 (out.data) and/or quantised from that bfloat16 value
 * (out.codes/out.scales in out.format: NVFP4, MXFP8 or NVFP4 planes).
 * Rows r >= expert_offsets[E] (and < rows) are not written.
 *
 * Kernels: bf16 and NVFP4-code activations run on bf16 MFMA after exact
 * in-register dequantisation (FP4 x scale has <= 6 significant bits); MXFP8
 * and NVFP4-plane activations run on gfx950's block-scaled MFMA
 * (V_MFMA_SCALE_F32_16X16X128_F8F6F4) with the FP4 weights as the native
 * E2M1 operand under their E8M0 scales.  W4A8 with MXFP8 activations is the
 * prompt path of "MiMo-V2.6-Flash-MOPD on one RTX PRO 6000" ("Quantization,
 * context and quality", Activations: E4M3 with a power-of-two scale per 32
 * values; "What makes it fast", speed v5.2: FP8 x FP4 block-scaled GEMMs).
 */
/* MOE_FP4_MXC: compact MXFP4 storage at 4.125 bits per weight (moe_fp4_compact_mx
 * writes it): the E2M1 codes unchanged, one 4-bit exponent code c per 32-value
 * block (block 2i in the low nibble of scale byte i, so scale is u8 [E, n, k/64])
 * and one power-of-two base 2^b per expert matrix in global_scale; the block's
 * scale is 2^(b + c).  Runs the weight-streaming kernel only (MOE_ALGO_DECODE or
 * AUTO) with BF16 or NVFP4 activations; needs k % 512 == 0. */
typedef enum { MOE_FP4_MX = 0, MOE_FP4_NV = 1, MOE_FP4_MXC = 2 } moe_fp4_format;

/* moe_fp4_weights.flags */
#define MOE_FP4_SCALES_POW2 1 /* NV: every E4M3 scale byte is zero or a power of two (true of
                                 fp4_transcode_mx_to_nv output); codes then convert with the
                                 scale applied by the convert instruction itself.  Setting it
                                 for other scales gives wrong results; leaving it clear is
                                 always correct (conversion through float). */
#define MOE_FP4_TILED 2       /* codes and scales are in the tiled layout that
                                 moe_fp4_tile_weights writes (needs n % 16 == 0 and
                                 k % 512 == 0); same values, bit-identical results, and
                                 every weight load of the kernels reads one contiguous
                                 block */
#define MOE_FP4_MX_EXACT 4    /* NV: the weights are an exact MXFP4 transcode (what
                                 fp4_transcode_mx_to_nv writes): both E4M3 scales of each
                                 32-block are the same power of two (zero only over
                                 all-zero codes) and the global scale is a power of two,
                                 so every 32-block has an E8M0 scale.  Required for NV
                                 weights with MXFP8 / NVFP4-plane activations (the
                                 block-scaled MFMA takes E8M0 per 32); implies
                                 MOE_FP4_SCALES_POW2. */

typedef struct {
  moe_fp4_format format;
  int32_t num_experts;
  int32_t n;                  /* output features (rows of each expert matrix) */
  int32_t k;                  /* input features; k % 128 == 0 */
  const uint8_t* packed;      /* codes [E, n, k/2] ("weight_packed")                    */
  const uint8_t* scale;       /* MX: E8M0 [E, n, k/32] | NV: E4M3 [E, n, k/16] | MXC: exponent
                                 codes u8 [E, n, k/64]                                   */
  const float* global_scale;  /* NV: float [E] (per expert matrix) | MXC: base 2^b [E] | MX: NULL */
  int32_t flags;              /* MOE_FP4_SCALES_POW2 | MOE_FP4_MX_EXACT (NV only) | MOE_FP4_TILED */
} moe_fp4_weights;

/* Rearrange expert weights into the tiled layout (flag MOE_FP4_TILED): the
 * values stay those of the model's MXFP4 / NVFP4 tensors, only their order in
 * memory changes, so that a wavefront of the GEMM kernels reads each operand
 * block as one contiguous run instead of 16 strided row pieces.  Per expert
 * matrix [n, k] (tile t = rows 16t .. 16t+15):
 *   codes:  column step s (k 128s .. 128s+127) of tile t is a 1024-byte block
 *           at (t * (k/128) + s) * 1024; its byte 16*(16*c + r) + b is byte
 *           64*s + 16*c + b of row 16t + r   (c < 4, r < 16, b < 16)
 *   scales: column window w (k 512w .. 512w+511) of tile t is a block of
 *           16*G bytes at (t * (k/512) + w) * 16*G; row 16t + r's G scale
 *           bytes of the window sit at G*r   (MX: G = 16 E8M0; NV: G = 32 E4M3;
 *           MXC: G = 8 bytes of exponent codes)
 * Global scales are unchanged.  Needs n % 16 == 0 and k % 512 == 0; the
 * outputs have the sizes of the inputs, must not overlap them and must be
 * 16-byte aligned.  num_experts == 0 is a no-op.
 */
moe_status moe_fp4_tile_weights(moe_fp4_format format, int32_t num_experts, int32_t n, int32_t k,
                                const uint8_t* packed, const uint8_t* scale, uint8_t* packed_tiled,
                                uint8_t* scale_tiled, hipStream_t stream);

/* Activation modes.  MXFP8 and NVFP4 planes run on the block-scaled MFMA and
 * need: MX weights or NV weights flagged MOE_FP4_MX_EXACT; n a multiple of 512
 * (one matrix) or 256 (SwiGLU, per matrix); k % 256 == 0; num_experts <= 1000.
 * Other shapes return MOE_ERR_UNSUPPORTED.
 *   MOE_ACT_MXFP8:        data = E4M3 codes u8 [rows_src, k], scales = E8M0
 *                         u8 [rows_src, k/32] (moe_quantize_mxfp8)
 *   MOE_ACT_NVFP4_PLANES: data = E4M3 planes u8 [rows_src, 2k], scales = E8M0
 *                         u8 [rows_src, k/16]: NVFP4 values, the global scale
 *                         folded in (moe_quantize_nvfp4_planes)               */
typedef enum {
  MOE_ACT_BF16 = 0 /* W4A16 */, MOE_ACT_NVFP4 = 1 /* W4A4, codes */, MOE_ACT_MXFP8 = 2 /* W4A8 */,
  MOE_ACT_NVFP4_PLANES = 3 /* W4A4 on the block-scaled MFMA */
} moe_act_mode;

typedef struct {
  moe_act_mode mode;
  const void* data;           /* BF16: bf16 [rows_src, k] | NVFP4: codes u8 [rows_src, k/2] | see above */
  const uint8_t* scales;      /* NVFP4: E4M3 [rows_src, k/16] | BF16: NULL | see above   */
  float input_scale;          /* NVFP4 global scale (a power of two; 1.0 = unit scale); 1.0 otherwise */
  const int32_t* gather;      /* NULL: row r reads source row r; else gather[r] / gather_div */
  int32_t gather_div;
  int64_t rows_src;
} moe_act;

typedef enum { MOE_EPI_NONE = 0, MOE_EPI_SWIGLU = 1 } moe_epilogue;

/* moe_out.format: what out.codes / out.scales hold */
#define MOE_OUT_NVFP4 0        /* codes [rows, n/2] E2M1, scales [rows, n/16] E4M3, global output_scale */
#define MOE_OUT_MXFP8 1        /* codes [rows, n] E4M3, scales [rows, n/32] E8M0 (needs n % 32 == 0) */
#define MOE_OUT_NVFP4_PLANES 2 /* codes [rows, 2n] E4M3 planes, scales [rows, n/16] E8M0: the NVFP4
                                  quantisation with global output_scale, as moe_quantize_nvfp4_planes */

typedef struct {
  void* data;                 /* bf16 [rows, n] or NULL                                   */
  uint8_t* codes;             /* quantised output (see format) or NULL (needs n % 16 == 0) */
  uint8_t* scales;            /* its scales (with codes)                                  */
  float output_scale;         /* global scale of an NVFP4 output (a power of two)         */
  void* dequant;              /* bf16 [rows, n] or NULL (NVFP4 format only): the NVFP4
                                 values themselves, codes x scale x output_scale (exact in
                                 bfloat16), so a following bf16-input GEMM computes on
                                 exactly the NVFP4 operand (W4A4 down projection)       */
  int32_t format;             /* MOE_OUT_*: MXFP8 and planes only from the MXFP8 /
                                 NVFP4-plane activation modes                             */
  float* row_sumsq;           /* float [rows, n/64] or NULL (MOE_EPI_NONE, MFMA-tiled kernels
                                 only: n % 256 == 0, k % 256 == 0, algo AUTO or PREFILL):
                                 element [r, c] is the sum of squares of row r's FP32
                                 outputs in columns 64c .. 64c+63, before any rounding --
                                 the parts of the REAP saliency's output norm
                                 (moe_reap_saliency_accumulate)                          */
} moe_out;

#define MOE_ALGO_AUTO 0       /* PREFILL when rows >= 4 * num_experts (or row_sumsq), else DECODE */
#define MOE_ALGO_DECODE 1     /* weight-streaming kernel (few rows per expert): one
                                 workgroup per (expert, block of output features)         */
#define MOE_ALGO_PREFILL 2    /* LDS-tiled MFMA kernel (many rows per expert)             */

moe_status moe_fp4_grouped_gemm(const moe_act* a, const moe_fp4_weights* w0, const moe_fp4_weights* w1,
                                moe_epilogue epi, const int32_t* expert_offsets, int64_t rows,
                                const moe_out* out, int32_t algo, hipStream_t stream);

/* ---------------------------------------------------------------- combine
 * The layer output of each token is the sum of its routed experts' outputs,
 * each weighted by the router's gate value g_{t,j} for that expert (the REAP
 * saliency equation on the "MiMo-V2.6-Flash -- REAP-50" card, "Pruning
 * Method", weighs every expert output of token t by g_{t,j}); the residual
 * stream is added in the same pass:
 * y[t, :] = bf16( residual[t, :] + sum_{j=0..top_k-1} w[t, j] * expert_out[slot_rows[t*top_k+j], :] )
 * summed in FP32 in j order (residual may be NULL; slot_rows = -1 contributes 0).
 *   expert_out bf16 [R, h]; slot_rows int32 [T*top_k] (moe_permute's inverse map);
 *   topk_weights float [T, top_k]; residual bf16 [T, h] or NULL; y bf16 [T, h].
 *   h % 8 == 0, 1 <= top_k <= 32; bf16 buffers 16-byte aligned.  T == 0 is a no-op.
 * Errors: MOE_ERR_INVALID for a NULL pointer, bad sizes or misalignment (nothing
 * is written); a slot_rows entry outside [-1, R) is the caller's error (unchecked).
 */
moe_status moe_combine(const void* expert_out, const int32_t* slot_rows, const float* topk_weights,
                       const void* residual, int64_t T, int32_t top_k, int32_t h, void* y,
                       hipStream_t stream);

/* -------------------------------------------------------------- transcode
 * Exact MXFP4 -> NVFP4 scale transcode of num_mats matrices [n, k].  Codes are
 * unchanged (the NVFP4 weights reuse `packed`).  Per matrix: G = (largest
 * finite block exponent) - 8 (0 if none); global_scale = 2^G; each E8M0 2^e
 * becomes two equal E4M3 bytes of 2^(e-G).  Exponents e-G < -9 are written as
 * 0x00 and counted in counters[1] when all 32 codes are +-0, else written as
 * 2^-9 and counted in counters[2] (re-rounded); E8M0 NaN (0xFF) becomes 0x7F
 * and is counted in counters[3]; counters[0] = number of blocks.  The counters
 * are zeroed by the call.
 *   mx_scale u8 [M, n, k/32]; packed u8 [M, n, k/2] (read only, for the
 *   all-zero test); nv_scale u8 [M, n, k/16]; global_scale float [M];
 *   counters int64 [4].  k % 32 == 0, n % 16 == 0.
 */
moe_status fp4_transcode_mx_to_nv(const uint8_t* mx_scale, const uint8_t* packed, int64_t num_mats,
                                  int32_t n, int32_t k, uint8_t* nv_scale, float* global_scale,
                                  int64_t* counters, hipStream_t stream);

/* --------------------------------------------------------- compact storage
 * MXFP4 -> compact storage (format MOE_FP4_MXC), 4.125 bits per weight.
 * "MiMo-V2.6-Flash-MOPD on one RTX PRO 6000" ("What makes it fast", speed v4)
 * stores the experts in a lossless compact encoding of 4.125 bits per weight;
 * the page gives the size, not the layout -- this one is the library's: per
 * matrix, b = (largest finite block exponent) - 15 (b = 0 if there is none),
 * global_base = 2^b, and each E8M0 2^e becomes the 4-bit code e - b.  Codes
 * below 0 are written as 0: counted in counters[1] when all 32 codes of the
 * block are +-0 (exact), else in counters[2] (re-rounded, not exact); E8M0 NaN
 * (0xFF) becomes 15, counted in counters[3]; counters[0] = number of blocks.
 * The encoding is exact when counters[2] and counters[3] are zero, and a GEMM
 * on it then gives bit-for-bit the MXFP4 result.  The counters are zeroed by
 * the call.  Codes unchanged: the compact weights reuse `packed`.
 *   mx_scale u8 [M, n, k/32]; packed u8 [M, n, k/2] (read only, for the
 *   all-zero test); exp_codes u8 [M, n, k/64]; global_base float [M];
 *   counters int64 [4].  k % 512 == 0, n % 16 == 0, buffers 16-byte aligned.
 */
moe_status moe_fp4_compact_mx(const uint8_t* mx_scale, const uint8_t* packed, int64_t num_mats, int32_t n,
                              int32_t k, uint8_t* exp_codes, float* global_base, int64_t* counters,
                              hipStream_t stream);

/* --------------------------------------------------- NVFP4 quantisation
 * Per row and 16-element block of bf16 x: s = E4M3_rne(max|x| / (6 g)) saturated
 * at 448, codes = E2M1_rne(x / (s g)) saturated at +-6 with the sign of x
 * (+0 codes when s == 0).  g = input_scale must be a power of two.
 * (MOPD-NVFP4 card, "About NVFP4 quantization" and "Quantization Details".)
 *   x bf16 [rows, k]; codes u8 [rows, k/2]; scales u8 [rows, k/16]; k % 32 == 0.
 *   dequant: bf16 [rows, k] or NULL; receives the NVFP4 values codes x s x g
 *   (exact in bfloat16), the operand a bf16-input GEMM multiplies for W4A4.
 */
moe_status moe_quantize_nvfp4(const void* x, int64_t rows, int32_t k, float input_scale,
                              uint8_t* codes, uint8_t* scales, void* dequant, hipStream_t stream);

/* ----------------------------------------------------- REAP saliency
 * REAP expert saliency ("MiMo-V2.6-Flash -- REAP-50" card, "Pruning Method":
 * S_j = mean over the tokens t routed to expert j of g_{t,j} times the L2 norm
 * of expert j's output for t), accumulated over batches:
 *   saliency_sum[e] += sum over e's permuted rows r of
 *                      topk_weights[sorted_slots[r]] * sqrt(sum_c row_sumsq[r, c])
 *   counts[e]       += number of e's rows
 * in float64, rows in order and parts in order (deterministic); S_e =
 * saliency_sum[e] / counts[e].  g is the weight the combine applies (the
 * normalised top-k weight x routed_scaling_factor); row_sumsq comes from the
 * down projection's moe_out.row_sumsq (parts = n / 64).
 *   row_sumsq float [rows, parts]; expert_offsets int32 [E+1]; sorted_slots
 *   int32 [rows]; topk_weights float [T * top_k] (slot order); saliency_sum
 *   double [E]; counts int64 [E].  rows == 0 or E == 0 is a no-op.
 */
moe_status moe_reap_saliency_accumulate(const float* row_sumsq, int64_t rows, int32_t parts,
                                        const int32_t* expert_offsets, int32_t num_experts,
                                        const int32_t* sorted_slots, const float* topk_weights, double* saliency_sum,
                                        int64_t* counts, hipStream_t stream);

/* ---------------------------------------------------- MXFP8 quantisation
 * W4A8 activations ("MiMo-V2.6-Flash-MOPD on one RTX PRO 6000", "Quantization,
 * context and quality", Activations: E4M3 with a power-of-two scale per 32
 * values).  Per row and 32-element block of bf16 x: X = 2^(floor(log2
 * max|x|) - 8) (the OCP Microscaling rule; 2^-127 for a zero block), codes =
 * E4M3_rne(x / X) saturated at +-448 with the sign of x; scales = E8M0 of X.
 *   x bf16 [rows, k]; codes u8 [rows, k]; scales u8 [rows, k/32]; k % 32 == 0;
 *   x and codes 16-byte aligned.  rows == 0 is a no-op.
 */
moe_status moe_quantize_mxfp8(const void* x, int64_t rows, int32_t k, uint8_t* codes, uint8_t* scales,
                              hipStream_t stream);

/* ----------------------------------------- NVFP4 as block-scaled planes
 * The NVFP4 quantisation of moe_quantize_nvfp4, in the form the block-scaled
 * MFMA takes (an NVFP4 scale is an arbitrary E4M3 per 16 values; the MFMA
 * takes E8M0 per 32).  Each 16-value block with E2M1 codes c_i and E4M3 scale
 * s = 2^e (lead + f1/2 + (2 f2 + f3)/8) (e = max(exponent field, 1) - 7)
 * becomes 32 E4M3 bytes, hi_i = c_i (2 lead + f1) then lo_i = c_i (2 f2 + f3) / 4,
 * and one E8M0 scale 2^(e-1) * input_scale: (hi_i + lo_i) * scale equals the
 * NVFP4 value c_i * s * input_scale exactly.
 *   x bf16 [rows, k]; planes u8 [rows, 2k]; plane_scales u8 [rows, k/16];
 *   k % 32 == 0; input_scale a power of two in [2^-100, 2^100]; x and planes
 *   16-byte aligned.  rows == 0 is a no-op.
 */
moe_status moe_quantize_nvfp4_planes(const void* x, int64_t rows, int32_t k, float input_scale, uint8_t* planes,
                                     uint8_t* plane_scales, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_FP4_H */
