/*
 * lora_mlp.h - C ABI of the MI355X (gfx950) fused LoRA SwiGLU MLP library.
 *
 * The operation is the fused LoRA MLP of "Unsloth 深度分析报告"
 * (nightvoyager.top), section "核心价值提炼 / 创新之处": a SwiGLU MLP whose
 * gate, up and down projections each add a LoRA adapter to a frozen weight,
 * with the forward and a hand-derived backward that keeps no per-activation
 * intermediates beyond the gate/up pre-activations. With T tokens, hidden H,
 * intermediate I, rank r and scale s:
 *
 *   proj(v; W, A, B) = v W^T + s (v A^T) B^T        W [out,in], A [r,in], B [out,r]
 *   G = proj(X; Wg, Ag, Bg)   U = proj(X; Wu, Au, Bu)   Z = SiLU(G) * U
 *   Y = proj(Z; Wd, Ad, Bd)   SiLU(g) = g / (1 + exp(-g))
 *
 * Backward returns dX and the gradients of all six adapter factors for an
 * upstream gradient dY. Base weights are frozen: no dW is produced.
 *
 * Conventions for every entry point
 *   - Tensors are dense, row-major, contiguous, and in device memory of the
 *     current HIP device; every pointer must be 16-byte aligned.
 *   - Activations, adapters, outputs and gradients share one dtype
 *     (lmlp_dims.dtype). Accumulation is always fp32.
 *   - The caller owns and allocates every buffer (inputs, outputs, the
 *     `saved` buffer and the workspace). The library never allocates device
 *     memory and never synchronises: all work is enqueued on `stream` (a
 *     hipStream_t; NULL = the null stream) in stream order.
 *   - Arguments are validated before anything is enqueued; a call that
 *     returns an error has enqueued no work.
 *   - Results are deterministic: no atomics, fixed reduction order.
 *   - Calls on distinct buffers may run concurrently from several threads.
 */
#ifndef LORA_MLP_H
#define LORA_MLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LMLP_OK = 0,
  LMLP_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad dimension, non-finite scale */
  LMLP_ERR_UNSUPPORTED = 2, /* valid request outside what the kernels implement, or not gfx950 */
  LMLP_ERR_WORKSPACE = 3,   /* saved/workspace buffer smaller than the size query */
  LMLP_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} lmlp_status;

typedef enum { LMLP_F32 = 0, LMLP_BF16 = 1 } lmlp_dtype;

/* Frozen base-weight storage. INT4_B64: each weight [out, in] is stored as
 * bytes [out, in/2] (element k of a row in byte k/2: even k in the low
 * nibble, odd k in the high nibble, two's complement in [-8, 7]) plus fp16
 * scales [out, in/64] (one per 64 consecutive elements of a row). The weight
 * value is bf16_round_nearest_even(q * scale) with the product taken in fp32.
 * This is the "native 4-bit QLoRA" weight path of "Unsloth 还是 AirLLM？一个炼丹，
 * 一个硬跑" (section 核心原理 / "Why it is fast"); requires dtype BF16 and
 * hidden % 64 == 0 and inter % 64 == 0. */
typedef enum { LMLP_W_DENSE = 0, LMLP_W_INT4_B64 = 1 } lmlp_wfmt;

/* flags */
#define LMLP_CONSUME_SAVED 0x1u /* backward may overwrite `saved` (saves 2*T*I elements of workspace) */
/* 4-bit weights: every product (forward gate/up and down, backward dZ and
 * dX) decodes the 4-bit codes inside its operand staging, so the workspace
 * holds no bf16 weights (only the block scales as fp32). This is the
 * default; the flag is accepted and changes nothing. */
#define LMLP_INT4_INKERNEL 0x2u
/* 4-bit weights: decode the three weights once per call into bf16 copies in
 * the workspace and run the dense bf16 products instead (faster products;
 * each workspace grows by 2*(2*I*H + H*I) bytes, and the decode passes read
 * the codes and write the copies). Not together with LMLP_INT4_INKERNEL.
 * Both modes decode by the same rule and give the same weights; the results
 * agree bit for bit except that at some shapes the backward splits its dZ
 * product differently, which changes the summation order of the rank
 * products. */
#define LMLP_INT4_BF16_COPIES 0x10u
/* Full recompute (the gradient-checkpointing variant of the fused MLP): the
 * forward keeps only the rank-r projections and the packed adapter factors
 * in `saved` (no G, U: `saved` shrinks by 2*T*I elements of dtype and the
 * forward writes 2*T*I elements less), and the backward recomputes G and U
 * with the forward's gate/up product (4*T*H*I more FLOPs) into its workspace,
 * where dG and dU then overwrite them. Outputs are bitwise equal to the
 * default mode. LMLP_CONSUME_SAVED has no effect with it. */
#define LMLP_RECOMPUTE_GU 0x4u
/* RMSNorm in front of the MLP: set for lora_mlp_norm_forward / _backward and
 * for their size queries (saved grows by 4*T bytes for the per-row
 * statistics, each workspace by T*H elements of dtype for the normalised
 * rows); lora_mlp_forward / _backward and the linear reject it. */
#define LMLP_RMSNORM 0x8u

typedef struct {
  int64_t tokens;  /* 0 <= T <= 2^24 - 64 (T == 0: forward is a no-op, backward writes zero adapter
                      gradients) */
  int64_t hidden;  /* 1 <= H <= 2^22; multiple of 8 (bf16) or 4 (fp32) */
  int64_t inter;   /* 1 <= I <= 2^22; multiple of 8 (bf16) or 4 (fp32) */
  int64_t rank;    /* r in [1, 256] */
  float scale;     /* s = alpha / r, finite */
  int32_t dtype;   /* lmlp_dtype */
  int32_t wfmt;    /* lmlp_wfmt */
  uint32_t flags;  /* bitwise OR of LMLP_CONSUME_SAVED, LMLP_INT4_INKERNEL or LMLP_INT4_BF16_COPIES,
                      LMLP_RECOMPUTE_GU, LMLP_RMSNORM, or 0 */
} lmlp_dims;

/* Bytes of the forward->backward `saved` buffer: the gate and up
 * pre-activations G, U (2*T*I elements of dtype; none with
 * LMLP_RECOMPUTE_GU), the three rank-r
 * projections X A_gate^T, X A_up^T and Z A_down^T in fp32, and the adapter
 * factors in the padded operand layouts both passes use (about
 * 16*(3H + 3I) elements of dtype at rank <= 16), padded.
 * Returns 0 if dims is invalid. */
size_t lora_mlp_saved_bytes(const lmlp_dims* dims);

/* Bytes of scratch workspace one forward (is_backward == 0) or one backward
 * (is_backward != 0) call needs. Contents need not be initialised and are
 * undefined afterwards. Returns 0 if dims is invalid. */
size_t lora_mlp_workspace_bytes(const lmlp_dims* dims, int is_backward);

/* Forward. Inputs: x [T,H]; w_gate, w_up [I,H], w_down [H,I] (dense: dtype;
 * INT4_B64: packed bytes with *_scales as described above, else the scale
 * pointers must be NULL); a_gate, a_up [r,H]; b_gate, b_up [I,r];
 * a_down [r,I]; b_down [H,r]. Output: y [T,H]. `saved` (saved_bytes long)
 * receives what backward needs. */
int lora_mlp_forward(const lmlp_dims* dims, const void* x,
                     const void* w_gate, const void* w_gate_scales,
                     const void* w_up, const void* w_up_scales,
                     const void* w_down, const void* w_down_scales,
                     const void* a_gate, const void* b_gate,
                     const void* a_up, const void* b_up,
                     const void* a_down, const void* b_down,
                     void* y, void* saved, size_t saved_bytes,
                     void* workspace, size_t workspace_bytes, void* stream);

/* Backward for upstream gradient dy [T,H], with the same x and weights as the
 * forward that filled `saved`. Outputs (overwritten, not accumulated):
 * dx [T,H]; da_gate, da_up [r,H]; db_gate, db_up [I,r]; da_down [r,I];
 * db_down [H,r]. Recomputes sigmoid(G), SiLU(G) and Z from the saved G, U.
 * `saved` is left unchanged unless flags has LMLP_CONSUME_SAVED, in which
 * case it is overwritten and a second backward needs a new forward. */
int lora_mlp_backward(const lmlp_dims* dims, const void* dy, const void* x,
                      const void* w_gate, const void* w_gate_scales,
                      const void* w_up, const void* w_up_scales,
                      const void* w_down, const void* w_down_scales,
                      const void* a_gate, const void* b_gate,
                      const void* a_up, const void* b_up,
                      const void* a_down, const void* b_down,
                      void* saved, size_t saved_bytes,
                      void* dx, void* da_gate, void* db_gate,
                      void* da_up, void* db_up, void* da_down, void* db_down,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- RMSNorm then the MLP ------------------------------------------------
 * y = MLP(RMSNorm(x)) with the MLP above and, per token row t of width H,
 *   rstd_t = (mean_h x_th^2 + eps)^(-1/2),   xn_th = x_th * rstd_t * gamma_h
 * (gamma [H] in dtype, frozen: no gradient; xn rounded once to dtype). The
 * norm is one of the forward+backward kernels of the training path in
 * "Unsloth 深度分析报告" (section 关键设计决策); as in "Unsloth支持哪些模型？
 * 主流LLM兼容性一览" (section 4.2) the backward reuses the forward's rstd
 * (kept in `saved`) instead of recomputing the row statistics. dims.flags
 * must include LMLP_RMSNORM; every other argument, flag and rule is the
 * MLP's. Backward returns dx = d/dx of <dy, y> through the norm:
 *   dx = rstd * (gamma g - xhat * mean_h(gamma g xhat)),  xhat = x rstd,
 * g the MLP's gradient at xn; the adapter gradients are the MLP's at xn.
 * x (the un-normalised rows) must be the same in both calls. */
int lora_mlp_norm_forward(const lmlp_dims* dims, float eps, const void* x, const void* gamma,
                          const void* w_gate, const void* w_gate_scales,
                          const void* w_up, const void* w_up_scales,
                          const void* w_down, const void* w_down_scales,
                          const void* a_gate, const void* b_gate,
                          const void* a_up, const void* b_up,
                          const void* a_down, const void* b_down,
                          void* y, void* saved, size_t saved_bytes,
                          void* workspace, size_t workspace_bytes, void* stream);
int lora_mlp_norm_backward(const lmlp_dims* dims, const void* dy, const void* x, const void* gamma,
                           const void* w_gate, const void* w_gate_scales,
                           const void* w_up, const void* w_up_scales,
                           const void* w_down, const void* w_down_scales,
                           const void* a_gate, const void* b_gate,
                           const void* a_up, const void* b_up,
                           const void* a_down, const void* b_down,
                           void* saved, size_t saved_bytes,
                           void* dx, void* da_gate, void* db_gate,
                           void* da_up, void* db_up, void* da_down, void* db_down,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---- Grouped (mixture-of-experts) LoRA MLP --------------------------------
 * E experts, each the MLP above with its own frozen weights and adapters,
 * applied to the token rows routed to it: the MoE form of the fused MLP that
 * "Unsloth 深度分析报告" (section 创新之处, the grouped GEMM over experts)
 * accelerates. Routing, the top-k choice and the weighted combine of expert
 * outputs stay with the caller: rows arrive grouped by expert, rows
 * offsets[e] .. offsets[e+1]-1 of x (and of y, dy, dx) belonging to expert e.
 * `offsets` is a HOST array of n_experts + 1 int64 values, rising from 0 to
 * dims.tokens (the number of routed rows); 1 <= n_experts <= 65536.
 * Per-expert tensors are stacked along a leading axis: w_gate, w_up
 * [E,I,H] and w_down [E,H,I] (INT4_B64: [E,I,H/2] and [E,H,I/2] bytes with
 * scales [E,I,H/64] and [E,H,I/64]), a_gate, a_up [E,r,H], b_gate, b_up
 * [E,I,r], a_down [E,r,I], b_down [E,H,r], and the adapter gradients in the
 * same shapes. dims.flags as for the MLP except LMLP_RMSNORM. An expert
 * with no rows gets zero adapter gradients. Ownership, determinism and
 * errors as for the MLP: every argument is checked for every expert before
 * anything is enqueued. Each GEMM of the pass runs as one grouped launch
 * over every expert's tiles, and each of its small side kernels as launches
 * merged across experts; all on `stream`. `saved` and the workspace hold one
 * region per expert (none in the workspace for an expert without rows). The
 * workspace also holds, beyond 8 experts (or when a K split is planned), a
 * region for the pass's parameter and job tables, which workgroups on
 * `stream` read into it from a pinned host buffer of the library's own (16 MB
 * plus 512 KB of completion marks, allocated on first use per device, kept
 * until exit). Where the read from the region of that buffer a call would
 * reuse has not run yet, and under graph capture, small copy kernels on
 * `stream` write the tables instead: the host never waits for the device.
 * With at most 8 experts of dense bf16 weights whose dX (or down) product's
 * 256 x 256 tiles would leave the device's last wave at most half full and
 * whose K is at least 16384, that product runs as two K splits, and the
 * workspace holds their fp32 partials, 2 * tokens * H * 4 bytes, summed in
 * split order (results stay deterministic). The sizes depend on the device's
 * compute-unit count: query them on the device that runs the call. */
size_t lora_moe_saved_bytes(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets);
size_t lora_moe_workspace_bytes(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets,
                                int is_backward);
int lora_moe_forward(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets, const void* x,
                     const void* w_gate, const void* w_gate_scales,
                     const void* w_up, const void* w_up_scales,
                     const void* w_down, const void* w_down_scales,
                     const void* a_gate, const void* b_gate,
                     const void* a_up, const void* b_up,
                     const void* a_down, const void* b_down,
                     void* y, void* saved, size_t saved_bytes,
                     void* workspace, size_t workspace_bytes, void* stream);
int lora_moe_backward(const lmlp_dims* dims, int64_t n_experts, const int64_t* offsets,
                      const void* dy, const void* x,
                      const void* w_gate, const void* w_gate_scales,
                      const void* w_up, const void* w_up_scales,
                      const void* w_down, const void* w_down_scales,
                      const void* a_gate, const void* b_gate,
                      const void* a_up, const void* b_up,
                      const void* a_down, const void* b_down,
                      void* saved, size_t saved_bytes,
                      void* dx, void* da_gate, void* db_gate,
                      void* da_up, void* db_up, void* da_down, void* db_down,
                      void* workspace, size_t workspace_bytes, void* stream);

/* ---- Fused LoRA linear (one projection: q, k, v, o, ...) ----------------
 * y = x W^T + s (x A^T) B^T and its backward, the matmul-with-LoRA fusion of
 * "Unsloth 深度分析报告" (section 创新之处): the rank-r adapter rides as r
 * extra K-steps of the base product, the projections through A and B are one
 * pass over x (forward) and over dy (backward), and the adapter gradients
 * come from two column projections. The same kernels as the MLP.
 *
 * dims: `hidden` is the input width (in), `inter` the output width (out);
 * tokens, rank, scale, dtype and wfmt as for the MLP; flags 0 or
 * LMLP_INT4_INKERNEL and LMLP_INT4_BF16_COPIES. Shapes: x [T,in]; w [out,in] (dense: dtype; INT4_B64:
 * packed bytes [out,in/2] with w_scales [out,in/64] fp16, else w_scales
 * NULL); a [r,in]; b [out,r]; y, dy [T,out]; dx [T,in]; da [r,in]; db
 * [out,r]. Ownership, streams and errors as for the MLP. */
size_t lora_linear_saved_bytes(const lmlp_dims* dims);
size_t lora_linear_workspace_bytes(const lmlp_dims* dims, int is_backward);

/* y = x W^T + s (x A^T) B^T. `saved` receives x A^T (fp32) and the adapter
 * factors in the layouts the backward reads. A bf16 product with dense
 * weights whose 256 x 256 output tiles would not fill the GPU once (few
 * tokens or a narrow output, e.g. a k/v projection) is split along K: the
 * splits' fp32 partials (in the workspace, at most 64 MiB) are summed in a
 * fixed order, so results stay bitwise reproducible. */
int lora_linear_forward(const lmlp_dims* dims, const void* x, const void* w, const void* w_scales,
                        const void* a, const void* b, void* y, void* saved, size_t saved_bytes,
                        void* workspace, size_t workspace_bytes, void* stream);

/* Allocation-free variant of lora_linear_forward, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Arguments, results, ownership and errors
 * are those of lora_linear_forward, except that there is no workspace
 * argument: the forward's workspace is a device array of the library's own,
 * LMLP_NOALLOC_SCRATCH_BYTES bytes on each GPU the library runs on (set up
 * on the first call on that GPU, held until the process ends). The call
 * allocates nothing. Dims whose lora_linear_workspace_bytes(dims, 0) exceeds
 * the array return LMLP_ERR_UNSUPPORTED before anything is enqueued. Every
 * call on one GPU uses the same array, which keeps the last call's contents
 * (nothing in it needs to start at zero): calls that overlap in time on one
 * GPU (on different streams, or from several threads) race with each other
 * and must be ordered by the caller. */
#define LMLP_NOALLOC_SCRATCH_BYTES (96u << 20)
int lora_linear_forward_noalloc(const lmlp_dims* dims, const void* x, const void* w, const void* w_scales,
                                const void* a, const void* b, void* y, void* saved, size_t saved_bytes,
                                void* stream);

/* dx = dy W + s (dy B) A; da = s (dy B)^T x; db = s dy^T (x A^T), for the
 * same x, w, a, b as the forward that filled `saved` (left unchanged).
 * Outputs are overwritten, in dtype, accumulated in fp32. */
int lora_linear_backward(const lmlp_dims* dims, const void* dy, const void* x, const void* w,
                         const void* w_scales, const void* a, const void* b, const void* saved,
                         size_t saved_bytes, void* dx, void* da, void* db, void* workspace,
                         size_t workspace_bytes, void* stream);

/* Dequantise one INT4_B64 weight (packed [out, in/2] bytes, fp16 scales
 * [out, in/64]) to bf16 [out, in] with the same device code the GEMM loaders
 * use. in % 64 == 0. Exposed so the 4-bit decode can be checked bit for bit. */
int lora_mlp_dequant_int4(const void* packed, const void* scales, int64_t out,
                          int64_t in, void* w_bf16, void* stream);

/* Per-kernel timing (measurement support). After lora_mlp_profile_begin(),
 * every kernel that forward, backward or dequant calls on this thread enqueue
 * is bracketed by a pair of hipEvents recorded on the call's stream (events
 * are created by the library on first use and reused; no device memory is
 * allocated). lora_mlp_profile_end() waits for the last recorded event,
 * writes up to `capacity` records in launch order (kernel name, duration in
 * milliseconds), stores the number of records in *count, and stops
 * recording. At most 65536 launches are recorded per session; later ones are
 * not timed. Timing adds event records between kernels, so time the plain
 * path separately. Returns LMLP_OK or LMLP_ERR_HIP. */
typedef struct {
  char name[40];
  float ms;
} lmlp_kernel_time;
int lora_mlp_profile_begin(void);
int lora_mlp_profile_end(lmlp_kernel_time* out, int capacity, int* count);

/* The bf16 matrix-core ceiling the GEMMs are measured against (measurement
 * support): one launch of `blocks` workgroups of eight waves, each wave
 * running `iters` rounds of 32 independent 16x16x32 bf16 MFMAs (fp32
 * accumulation) on operands read once from `operands`, device memory of at
 * least blocks * 8 * 768 * 16 bytes holding the bits to multiply (random
 * data keeps the arithmetic as busy as a real product's), with no other
 * memory traffic. It performs blocks * 8 * iters * 32 * 16384 FLOPs and
 * writes one float per thread to `sink` (blocks * 512 floats) so that
 * nothing is optimised away. Time it with events on `stream`. Returns
 * LMLP_OK, LMLP_ERR_INVALID_ARG (null pointer, blocks or iters < 1,
 * operand_bytes too small) or LMLP_ERR_HIP. */
int lora_mlp_mfma_probe(const void* operands, size_t operand_bytes, float* sink, int blocks, int iters,
                        void* stream);

/* Static name of a status code. */
const char* lora_mlp_status_string(int status);

/* Detail of the most recent failure on the calling thread ("" if none). */
const char* lora_mlp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MLP_H */
