/*
 * nvfp4moe.h - C ABI of the NVFP4 routed-expert MoE projection for AMD MI355X (gfx950).
 *
 * The operation (sources are the pages this library is written from, cited by title
 * and section):
 *   - NVFP4 weights: 4-bit E2M1 codes, two per byte, one FP8 E4M3 scale byte per 16
 *     consecutive inputs, and one FP32 global scale per expert tensor that multiplies
 *     the projection's output ("Strata NVFP4" README, "How it differs from upstream
 *     Strata": 4.5-bit experts with calibrated scales, per-expert FP32 scales kept and
 *     applied to each projection's output; TensorFold pull 906: plain E4M3 scale bytes,
 *     input cuts preserve groups of 16, the FP32 tensor scale).
 *   - Routed experts: for token t and slot j with expert e = topk_ids[t][j],
 *       g = gamma_gate[e] * (x_t . Wgate_e^T),  u = gamma_up[e] * (x_t . Wup_e^T)
 *       h = SiLU(g) * u,  SiLU(z) = z / (1 + exp(-z))
 *       y = gamma_down[e] * (h . Wdown_e^T)
 *       out[t] = sum_j topk_weights[t][j] * y        (FP32 accumulation, one final rounding)
 *     ("Strata NVFP4" README: routed experts kept in RAM and computed per token; the
 *     shared expert's fused SwiGLU quantizer names the SwiGLU activation.)
 *   - W4A8 prompt path: activations quantized per row to int8 with an FP32 scale
 *     absmax / 127 before each expert GEMM ("Strata NVFP4" README, "How it differs from
 *     upstream Strata": an int8 (W4A8) prompt path that keeps 8-bit activations).
 *   - W4A4 prompt path: activations quantized per row to NVFP4 before each expert GEMM
 *     ("Strata NVFP4" README, "How it differs from upstream Strata": llama.cpp's NVFP4
 *     prompt GEMM multiplies FP4 activations by FP4 weights, the path W4A8 is measured
 *     against; its quantization rule is not on the pages, see nvfp4_quant_rows_nvfp4).
 *   - Mixed packs: the down projection of a layer may be Q8_0 instead of NVFP4 ("Strata
 *     NVFP4" README, the re-quantized experts pack: Q8_0 down projections in 27 of the 48
 *     layers). The pages name the format only; its element rule here is GGML's: blocks
 *     of 32 int8 weights along the inputs with one fp16 scale each, weight = d * q.
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA tensor's
 *     data_ptr()) owned by the caller, except in the *_host entry points, which take
 *     host pointers. The library never allocates, frees or retains them, and keeps no
 *     state between calls (the host entry points keep worker threads): it is safe to
 *     call from several host threads on different streams, provided their workspaces
 *     and outputs differ.
 *   - `stream` is a hipStream_t passed as void*; NULL means the default stream. All
 *     device work is enqueued on it asynchronously; no device call synchronizes the host.
 *   - Arguments are validated completely before anything is enqueued: a call that
 *     returns an error has enqueued nothing and written nothing. A failed kernel
 *     launch returns NVFP4_EHIP.
 *   - Outputs are overwritten, never accumulated into.
 *   - Weight layout (one projection of E experts; rows are outputs):
 *       codes  uint8 [E][N][K/2]   element 2j of a row in the LOW nibble of byte j,
 *                                  element 2j+1 in the high nibble;
 *       scales uint8 [E][N][K/16]  scale byte g covers inputs 16g .. 16g+15;
 *       global float [E]           one FP32 scale per expert tensor.
 *     Q8_0 projections (format NVFP4_FMT_Q8_0, down projection only):
 *       codes  int8   [E][N][K]    one weight per byte;
 *       scales fp16   [E][N][K/32] scale b covers inputs 32b .. 32b+31 (raw fp16 bits);
 *       global float [E] or NULL   NULL means 1.
 *     K must be a multiple of 32. Code and scale planes must be 16-byte aligned.
 *   - topk_ids int32 [T][topk], topk_weights float [T][topk]. Ids outside [0, E) are
 *     dropped (they contribute nothing); the number dropped is written as an int32 to
 *     the first 4 bytes of the workspace. Duplicate ids within a token are legal and
 *     are summed. Router weights are used as given (no renormalization).
 *   - NaN/Inf in activations or weights propagate to the outputs they touch.
 */
#ifndef NVFP4MOE_H
#define NVFP4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  NVFP4_OK = 0,
  NVFP4_EINVAL = -1,       /* a null or misaligned pointer, a size out of range */
  NVFP4_EUNSUPPORTED = -2, /* a valid request this build does not implement */
  NVFP4_EWORKSPACE = -3,   /* ws_bytes smaller than the matching *_workspace_size() */
  NVFP4_EHIP = -4,         /* a HIP runtime error while enqueueing */
  NVFP4_ENOMEM = -5        /* a host allocation or worker thread could not be created (host entry points) */
} nvfp4_status;

typedef enum { NVFP4_F32 = 0, NVFP4_BF16 = 1, NVFP4_F16 = 2 } nvfp4_dtype;

/* Activation handling of the prefill path.
 *   NVFP4_ACT_BF16      bf16 activations; both expert GEMMs run on fp16 matrix cores
 *                       (x is staged in fp16 with a power-of-two exponent per row, h is
 *                       kept in fp16 with one per block; see nvfp4_moe_prefill).
 *   NVFP4_ACT_W4A8      x and h quantized per row to int8 (scale absmax/127); the GEMMs
 *                       run on int8 matrix cores (weights as exact int8 2*e2m1) with an
 *                       FP32 rescale by e4m3/2 per 16-input group (per 32 for a Q8_0
 *                       down projection): bound by that VALU rescale, slower than
 *                       NVFP4_ACT_W4A8_F16, which gives the same result to FP32 rounding.
 *   NVFP4_ACT_W4A8_F16  the same int8 activations and the same result, computed on fp16
 *                       matrix cores (int8 values are exact in fp16; x and h are stored
 *                       as 1-byte codes and widened while staged).
 *   NVFP4_ACT_W4A4      x and h quantized per row to NVFP4 by the rule of
 *                       nvfp4_quant_rows_nvfp4 (E2M1 codes, an E4M3 scale per 16 inputs, an
 *                       fp32 scale per row); both GEMMs run on fp16 matrix cores, where
 *                       code * block scale is exact for activations and weights alike, and
 *                       the row scale multiplies at the FP32 accumulator. ("Strata NVFP4"
 *                       README: the prompt path that multiplies FP4 activations by FP4
 *                       weights.) */
typedef enum { NVFP4_ACT_BF16 = 0, NVFP4_ACT_W4A8 = 1, NVFP4_ACT_W4A8_F16 = 2, NVFP4_ACT_W4A4 = 3 } nvfp4_act;

/* Weight format of a projection: NVFP4 (every projection) or Q8_0 (down only). */
typedef enum { NVFP4_FMT_NVFP4 = 0, NVFP4_FMT_Q8_0 = 1 } nvfp4_format;

/* One projection (gate, up or down) of all E experts of a layer. Device pointers. */
typedef struct {
  const uint8_t* codes;  /* NVFP4: [E][N][K/2]; Q8_0: int8 [E][N][K] */
  const uint8_t* scales; /* NVFP4: [E][N][K/16] E4M3; Q8_0: fp16 [E][N][K/32] */
  const float* global;   /* [E]; may be NULL for Q8_0 */
  int32_t N;             /* outputs per expert (rows) */
  int32_t K;             /* inputs per expert, multiple of 32 */
  int32_t format;        /* nvfp4_format; a zero-initialized struct is NVFP4 */
} nvfp4_weight;

/* Dequantize `rows` NVFP4 rows of K inputs: out[r][k] = e2m1 * e4m3 [* global[0]].
 * codes [rows][K/2], scales [rows][K/16]; global is a device pointer to ONE float, or
 * NULL for no global scale. out_dtype F32: the exact product rounded once to fp32.
 * BF16: that fp32 value rounded to bf16 (round to nearest even). F16: the same to fp16.
 * Without a global scale every product is exact in all three types. (Source: the NVFP4
 * element formats above; #2727 "tools: add opt-in FP4-Local CSF checkpoint conversion"
 * streams an NVFP4 table to BF16 in bounded row chunks, which is this call over row
 * ranges.) Errors: EINVAL for null pointers, rows < 0, K <= 0 or K % 32 != 0. */
int nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* global, int64_t rows,
                  int32_t K, int32_t out_dtype, void* out, void* stream);

/* Single-expert NVFP4 linear: out[t][n] = w->global[expert] * sum_k x[t][k] * W_e[n][k].
 * x [T][w->K] in x_dtype (F32 or BF16), out float [T][w->N]. (Same sources as above.)
 * Errors: EINVAL for null pointers, T < 0, expert outside [0, E) (E is not known here:
 * the caller guarantees the arrays hold expert+1 experts), bad K, unknown format;
 * EUNSUPPORTED for a Q8_0 weight. */
int nvfp4_linear(const void* x, int32_t x_dtype, int32_t T, const nvfp4_weight* w, int32_t expert,
                 float* out, void* stream);

/* Routing sort. Pairs p = t*topk + j are counting-sorted by expert id:
 * expert_offsets int32 [E+1] is the exclusive prefix sum of per-expert pair counts
 * (expert_offsets[E] = number of valid pairs); sorted_pairs int32 [T*topk] lists the
 * valid pairs ordered by (expert, p) ascending, followed by -1 for each dropped pair.
 * The order is deterministic and equals a stable sort. ws must hold
 * nvfp4_route_workspace_size() bytes; its first 4 bytes receive the dropped count.
 * ("Strata NVFP4" README: an MMQ group's experts gathered in one launch after one wait,
 * instead of one wait per streamed expert.) Errors: EINVAL for null pointers, T < 0,
 * topk < 1, E < 1 or E > 8192; EWORKSPACE. */
size_t nvfp4_route_workspace_size(int32_t T, int32_t topk, int32_t E);
int nvfp4_moe_route(const int32_t* topk_ids, int32_t T, int32_t topk, int32_t E,
                    int32_t* expert_offsets, int32_t* sorted_pairs, void* ws, size_t ws_bytes,
                    void* stream);

/* Per-row int8 quantization (the W4A8 activation rule): s[r] = fp32(absmax_r / 127) by
 * an fp32 division, q[r][c] = clamp(round_half_even(fp32(x[r][c] / s[r])), -127, 127);
 * an all-zero row gives s = 0 and q = 0. A row holding a NaN gets s = NaN, else a row
 * holding an infinity s = +inf, and either gets q = 0 (so q * s is NaN and the non-finite
 * value propagates). x [rows][cols] in x_dtype (F32 or BF16).
 * ("Strata NVFP4" README: the W4A8 prompt path keeps 8-bit activations.)
 * Errors: EINVAL for null pointers, rows < 0, cols < 1. */
int nvfp4_quant_rows_i8(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, int8_t* q,
                        float* scale, void* stream);

/* Per-row NVFP4 quantization (the W4A4 activation rule; "Strata NVFP4" README: FP4
 * activations on the prompt path; the NVFP4 element formats above. The pages fix the
 * formats, not this rule: the reading here is the plainest one that fills every code range):
 *   g[r] = fp32(absmax_r / 2688) by an fp32 division (2688 = 6 * 448, the largest
 *     E2M1 * E4M3 product), so the row's largest 16-group scale lands on 448;
 *   scale byte of group b = the E4M3 value nearest to fp32(blockmax / fp32(6 * g[r])),
 *     ties to the even code, saturating at 448 (0x7E);
 *   code of x[r][c] = the E2M1 magnitude nearest to |fp32(x / fp32(s * g[r]))|, ties to the
 *     even code, saturating at 6, with the sign bit of x (so -0.0, and a negative value whose
 *     magnitude rounds to zero, give the negative-zero code 8);
 * so x ~ code * scale * g. A zero row, or a block whose scale rounds to zero, gives zero
 * codes (and g = 0 for a zero row); a row holding a NaN gets g = NaN, else one holding an
 * infinity g = +inf, with zero codes and scales (so code * scale * g is NaN there).
 * x [rows][cols] in x_dtype (F32 or BF16), 16-byte aligned; codes uint8 [rows][cols/2] (two
 * per byte, the even input in the low nibble), 8-byte aligned; scales uint8
 * [rows][cols/16]; g fp32 [rows]. Device pointers, the caller's memory.
 * Errors: EINVAL for null or misaligned pointers, rows < 0, cols not a positive multiple
 * of 16, an x_dtype other than F32 and BF16. */
int nvfp4_quant_rows_nvfp4(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, uint8_t* codes,
                           uint8_t* scales, float* g, void* stream);

/* Decode (small token batches): the full routed-expert projection above for
 * 1 <= T <= 8 tokens, with FP32 arithmetic throughout and h kept in fp32 ("#1858
 * strata-safetensors": the quality profile keeps canonical FP32 expert decode).
 * x [T][H] bf16; gate/up: N = I, K = H, NVFP4; down: N = H, K = I, NVFP4 or Q8_0
 * (Q8_0 dot products in FP32, each 32-input block scaled once); out [T][H] in out_dtype
 * (F32 or BF16). ws needs nvfp4_moe_decode_workspace_size() bytes and must be
 * zero-filled before its first use (it holds a grid-barrier counter, epoch and per-block
 * release flags that every call leaves ready for the next, whatever the shapes). Bytes
 * 4..7 of ws hold an error word: bit 0 is set if a call's grid barrier timed out (the
 * output rows of the blocks that gave up are then NaN; the bit stays set until the
 * caller clears it, and the barrier state stays consistent for the next call).
 * A timeout can only happen if other work keeps some of the grid's blocks from starting
 * while the rest wait; the caller must check the word after calls whose result it uses.
 * Bytes 8..11 (int32), when positive, replace the barrier's spin limit (default 2^22
 * polls); when negative, waiting blocks do not poll at all and give up at once (for
 * testing the error path). The result does not depend on scheduling: every
 * output element is summed in a fixed order. Calls sharing one workspace must not
 * overlap. The whole call is one persistent launch when its grid (H/8 blocks) fits on the
 * device at once, else two launches with identical results.
 * Errors: EINVAL (null pointers, shapes that disagree, H or I not a multiple of 32,
 * topk < 1, E < 1, unknown format); EUNSUPPORTED for x not bf16, T > 8, topk * T > 64,
 * H or I above 8192, T * H above 40960, a Q8_0 gate or up projection; EWORKSPACE.
 * T == 0 is a no-op and may pass null tensors. */
size_t nvfp4_moe_decode_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk);
int nvfp4_moe_decode(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                     const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                     const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                     int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Decode that allocates nothing, for callers that cannot allocate or pass device memory
 * between calls: code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation. The same computation, kernels and results as nvfp4_moe_decode, with the
 * workspace taken from a static device array of 1 MiB (one copy per GPU, held until the
 * process ends) instead of the caller's ws. The caller still passes x, the weights, the
 * routing and out. The first call on a device looks up that device's array and clears
 * its barrier state with a fill kernel on `stream`, ahead of the call; the call itself
 * makes no allocation. Every call on one GPU shares its array: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialized by the caller.
 * A grid-barrier timeout (see nvfp4_moe_decode) leaves NaN in the affected output rows.
 * Errors: those of nvfp4_moe_decode, and EUNSUPPORTED when the call would need more than
 * the 1 MiB (nvfp4_moe_decode_workspace_size() above 1048576 bytes: 131,328 bytes of
 * header and flag lines plus T * topk * I * 4 bytes of h). */
int nvfp4_moe_decode_noalloc(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                             const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                             const int32_t* topk_ids, const float* topk_weights, int32_t topk, void* out,
                             int32_t out_dtype, void* stream);

/* Prefill (any T >= 0): the same projection as grouped GEMMs on matrix cores, one
 * launch per stage for all experts. x [T][H] bf16; out [T][H] bf16 or f32 (accumulated
 * in fp32, rounded once). `act` selects the activation handling (nvfp4_act).
 * ws needs nvfp4_moe_prefill_workspace_size() bytes. ("Strata NVFP4" README: prompt
 * chunks up to 32K tokens, where every chunk streams every layer's experts once.)
 * Each pair's down output is kept in fp32 and the slots of a token are summed in slot
 * order, so the result is deterministic. T == 0 is a no-op and may pass null tensors.
 * Range (act BF16): the fp16 matrix-core operands carry a power-of-two exponent per row:
 * each token row of x is scaled so that its largest magnitude lies in [2^14, 2^15) before
 * it is narrowed to fp16, and h is stored in fp16 the same way per (routed pair, block of
 * 256 intermediate indices), brought to the pair's common exponent when the down GEMM
 * stages it; every exponent is undone exactly (ldexp) at the FP32 accumulator. So any
 * finite bf16 activations are accepted, none overflows fp16, and an operand loses bits
 * only where it is below 2^-31 of its row's (block's) largest magnitude ("Strata NVFP4"
 * README, "How it differs from upstream Strata": the scale fold that left hidden
 * activations in FP16 subnormals). NaN and infinite activations or scale bytes give NaN
 * or infinite outputs where the float64 definition does.
 * The down projection may be Q8_0: its weights enter the fp16 matrix cores as
 * fp16(d * q), one rounding per weight (relative error at most 2^-11), the only
 * operand of the path that is not exact.
 * Errors: EINVAL (null pointers, shapes that disagree, unknown act or format,
 * out_dtype F16); EUNSUPPORTED for H not a multiple of 256, I not a multiple of 128 or
 * above 8192, E > 8192, x_dtype other than BF16, a Q8_0 gate or up projection;
 * EWORKSPACE. */
size_t nvfp4_moe_prefill_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                                        int32_t act);
int nvfp4_moe_prefill(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                      const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                      const int32_t* topk_ids, const float* topk_weights, int32_t topk, int32_t act,
                      void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* The layer's shared expert ("Strata NVFP4" README, 0.1.39-nvfp4.2 entry: the shared
 * expert, with its fused SwiGLU quantizer keeping the fp16 scale finite). The pages give the
 * shared expert no shape, format or weight; the reading taken here: an NVFP4 SwiGLU expert
 * of the routed experts' shape (its own gate, up and down projections, each one expert:
 * codes [1][N][K/2], scales [1][N][K/16], global [1]; the down projection in the routed
 * down projection's format) applied to every token with weight 1 and added to the routed
 * sum before the one final rounding:
 *   out[t] = sum_j topk_weights[t][j] * y_{topk_ids[t][j]}(x_t) + y_shared(x_t).
 * It runs in the same launches as the routed experts, as one more expert (index E) that
 * every token routes to as slot topk; its h goes through the same fused SwiGLU epilogue,
 * whose per-block power-of-two scale (act BF16) or per-row fp32 scale (W4A8) is finite for
 * every finite h. All arguments are those of nvfp4_moe_decode / nvfp4_moe_prefill plus the
 * three shared projections. ws needs the *_shared_workspace_size() bytes; the dropped count
 * is in its first 4 bytes as for the plain calls (ids equal to E count as dropped: only the
 * library's own slot reaches the shared expert). The prefill workspace regions are those of
 * nvfp4_moe_prefill_workspace_region(T, H, I, E + 1, topk + 1, act), followed by the routing
 * with the shared slot appended. Decode forms that slot inside its kernel (no extra launch),
 * keeps its grid-barrier state in ws like nvfp4_moe_decode and needs T * (topk + 1) <= 64.
 * Errors: those of the plain calls, and EINVAL for a shared projection that is null,
 * misaligned or of another shape, EUNSUPPORTED for a shared gate or up that is not NVFP4 or
 * a shared down whose format differs from the routed down's. */
size_t nvfp4_moe_prefill_shared_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk,
                                               int32_t act);
int nvfp4_moe_prefill_shared(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                             const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                             const nvfp4_weight* shared_gate, const nvfp4_weight* shared_up,
                             const nvfp4_weight* shared_down, const int32_t* topk_ids, const float* topk_weights,
                             int32_t topk, int32_t act, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                             void* stream);
size_t nvfp4_moe_decode_shared_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk);
int nvfp4_moe_decode_shared(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                            const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                            const nvfp4_weight* shared_gate, const nvfp4_weight* shared_up,
                            const nvfp4_weight* shared_down, const int32_t* topk_ids, const float* topk_weights,
                            int32_t topk, void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* Where a prefill call keeps its intermediate results in its workspace, for callers
 * that inspect them (tests, debugging) after running the stages: *offset receives the
 * region's byte offset from the start of ws and *bytes its size (0 when the region does
 * not exist for `act`). The contents are valid after the stage that writes them.
 *   EXPERT_OFFSETS  int32 [E+1]            stage 0 (the routing of nvfp4_moe_route)
 *   SORTED_PAIRS    int32 [T*topk]         stage 0
 *   PAIR_POSITION   int32 [T*topk]         stage 0: sorted position of pair p, -1 if dropped
 *   X_STAGED        BF16: fp16 [T][H] (x * 2^xexp[t]); W4A8*: int8 codes [T][H];
 *                   W4A4: NVFP4 codes [T][H/2]                                     stage 0
 *   X_ROWSCALE      BF16: int32 xexp [T];  W4A8*, W4A4: fp32 row scales [T]       stage 0
 *   X_BLOCKSCALE    W4A4: E4M3 [T][H/16]; others: none                            stage 0
 *   H               BF16: fp16 [P][I] in sorted order, h * 2^hexp[pos][I-block]; W4A8*,
 *                   W4A4: fp32 [P][I]                                             stage 1
 *   H_EXP           BF16: int32 [P][I/256] (I/128 when I % 256 != 0); others: none stage 1
 *   H_Q             W4A8*: int8 codes of h [P][I] (the per-row rule of
 *                   nvfp4_quant_rows_i8 applied to the fp32 H); W4A4: NVFP4 codes
 *                   [P][I/2] (nvfp4_quant_rows_nvfp4 on H); BF16: none             stage 1
 *   H_SCALE         W4A8*, W4A4: fp32 [P]; BF16: none                              stage 1
 *   H_BLOCKSCALE    W4A4: E4M3 [P][I/16]; others: none                            stage 1
 *   Y               fp32 [P][H], each pair's down row times gamma_down and its weight stage 2
 * Errors: EINVAL for null outputs, bad sizes, unknown act or region. */
typedef enum {
  NVFP4_WS_EXPERT_OFFSETS = 0,
  NVFP4_WS_SORTED_PAIRS = 1,
  NVFP4_WS_PAIR_POSITION = 2,
  NVFP4_WS_X_STAGED = 3,
  NVFP4_WS_X_ROWSCALE = 4,
  NVFP4_WS_H = 5,
  NVFP4_WS_H_EXP = 6,
  NVFP4_WS_H_Q = 7,
  NVFP4_WS_H_SCALE = 8,
  NVFP4_WS_Y = 9,
  NVFP4_WS_X_BLOCKSCALE = 10,
  NVFP4_WS_H_BLOCKSCALE = 11
} nvfp4_ws_region;
int nvfp4_moe_prefill_workspace_region(int32_t T, int32_t H, int32_t I, int32_t E, int32_t topk, int32_t act,
                                       int32_t region, size_t* offset, size_t* bytes);

/* One stage of the same sequence, for callers that interleave or time the stages.
 * Arguments, validation and workspace are those of the full call; running the stages
 * in order on one stream with the same arguments and workspace is the full call.
 * Decode stages: 0 gate/up + SwiGLU (h into the workspace), 1 down + combine.
 * Prefill stages: 0 zero the accumulator, route, stage the activations (fp16, int8 codes
 * and row scales for W4A8, NVFP4 codes and scales for W4A4); 1 gate/up + SwiGLU (W4A8,
 * W4A4: then requantize h);
 * 2 down, scaled per pair; 3 top-k combine in slot order and the final rounding.
 * Errors: those of the full call, and EINVAL for a stage outside that range. */
int nvfp4_moe_decode_stage(int32_t stage, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                           const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down,
                           int32_t E, const int32_t* topk_ids, const float* topk_weights, int32_t topk,
                           void* out, int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);
int nvfp4_moe_prefill_stage(int32_t stage, const void* x, int32_t x_dtype, int32_t T, int32_t H,
                            const nvfp4_weight* gate, const nvfp4_weight* up, const nvfp4_weight* down,
                            int32_t E, const int32_t* topk_ids, const float* topk_weights, int32_t topk,
                            int32_t act, void* out, int32_t out_dtype, void* ws, size_t ws_bytes,
                            void* stream);

/* Router (the step before the routed experts): logits[t][e] = sum_h x[t][h] * Wr[e][h] with a
 * bf16 router matrix Wr [E][H] (raw bf16 bits) and x [T][H] in F32 or BF16. The inputs are
 * used exactly ("Strata NVFP4" README: FP32-exact inputs to the prompt path's BF16
 * projections, the router among them): an fp32 x is split into three bf16 parts whose
 * products with the weights are exact, summed in fp32 on matrix cores. Then, per token,
 * topk_ids[t][0..topk) = the topk largest logits in descending order (equal logits in
 * expert-id order; NaN logits rank below every number) and topk_weights[t][j] = softmax of
 * those topk logits (the rule is this library's reading; the pages do not give it). The
 * outputs feed nvfp4_moe_decode / nvfp4_moe_prefill directly. ws needs
 * nvfp4_router_workspace_size() bytes: a 256-byte header, then the fp32 logits [T][E]. The
 * header holds a completion counter (up to 4 tokens run as one launch whose last block to
 * finish ranks the logits): zero-fill the workspace once before first use; every call
 * leaves the counter at zero, and calls sharing a workspace must not overlap. T == 0 is
 * a no-op.
 * Errors: EINVAL for null or misaligned pointers (x, w_router and ws 16-byte aligned), T < 0,
 * x_dtype other than F32/BF16, topk < 1 or topk > E; EUNSUPPORTED for H not a multiple of
 * 64, E not a multiple of 32 or above 2048, topk > 64; EWORKSPACE. */
size_t nvfp4_router_workspace_size(int32_t T, int32_t E);
int nvfp4_router_topk(const void* x, int32_t x_dtype, int32_t T, int32_t H, const uint16_t* w_router, int32_t E,
                      int32_t topk, int32_t* topk_ids, float* topk_weights, void* ws, size_t ws_bytes,
                      void* stream);

/* Host-CPU share of the experts ("Strata NVFP4" README: AVX-512 NVFP4 kernels compute the
 * CPU's share of the experts from host DRAM; a CPU without AVX-512 takes an AVX2 path).
 * The decode projection above on HOST memory, run on this process's CPU threads: every
 * pointer (x, the weight planes and scales, topk_ids, topk_weights, out) is a host pointer
 * owned by the caller, with the device layout and no alignment requirement. Each weight is
 * decoded exactly to fp32, dot products and SwiGLU run in FP32, h stays in FP32, and the
 * routed pairs of an output row are added in a fixed order, so the result does not depend
 * on n_threads. x [T][H] F32 or BF16, any T >= 0; out float [T][H]. To split a layer's
 * experts between the GPU and the CPU, give each call the same topk_ids with the other
 * side's experts replaced by -1 (dropped) and add the two outputs.
 * n_threads: 0 = one per CPU this process may run on (more than that is clamped to it).
 * Worker threads are started on first use and kept; they take the calling thread's
 * floating-point modes (MXCSR) for each call. isa: NVFP4_ISA_AUTO (the widest the
 * CPU has) or a narrower one to force (results differ only in FP32 summation order).
 * dropped (may be NULL) receives the number of pairs whose id is outside [0, E).
 * The call returns when out is written; it makes no HIP call. Concurrent calls run one
 * after the other on the library's worker threads.
 * Errors: EINVAL (null pointers, shapes that disagree, K not a multiple of 32, unknown
 * dtype, format or isa, n_threads < 0); EUNSUPPORTED for a Q8_0 gate or up projection,
 * an isa the CPU lacks, T * topk above 2^31 - 1; ENOMEM. T == 0 writes nothing. */
typedef enum { NVFP4_ISA_AUTO = 0, NVFP4_ISA_PORTABLE = 1, NVFP4_ISA_AVX2 = 2, NVFP4_ISA_AVX512 = 3 } nvfp4_isa;
int32_t nvfp4_host_isa(void); /* the widest nvfp4_isa this CPU supports */
int nvfp4_moe_decode_host(const void* x, int32_t x_dtype, int32_t T, int32_t H, const nvfp4_weight* gate,
                          const nvfp4_weight* up, const nvfp4_weight* down, int32_t E,
                          const int32_t* topk_ids, const float* topk_weights, int32_t topk, float* out,
                          int32_t n_threads, int32_t isa, int64_t* dropped);

/* A static, human-readable name for a status code. */
const char* nvfp4_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4MOE_H */
