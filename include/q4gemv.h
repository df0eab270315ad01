/*
 * q4gemv -- 4-bit weight-only dequantize-and-multiply for AMD MI355X (gfx950).
 *
 * C ABI of libq4gemv.so.  Every entry point computes
 *
 *     y[m, n] = sum_k x[m, k] * w[n, k]        (y = x . W^T, no bias)
 *
 * for a decode batch x of M rows against one weight matrix W of N rows
 * (output features) and K columns (input features), without ever writing the
 * dequantized W to memory.  Activations x and outputs y are BF16; the sum is
 * accumulated in fp32 and rounded to BF16 (round to nearest even) once.
 *
 * Types.  BF16 and fp16 values travel as uint16_t bit patterns and
 * float8_e4m3fn values as uint8_t, so C callers need no GPU half-precision
 * headers.  `stream` is a hipStream_t (NULL = the default stream).
 *
 * Memory and ownership.  All array arguments are DEVICE pointers to
 * contiguous, row-major arrays owned by the caller.  The library allocates
 * nothing, keeps no pointer after returning, and never synchronizes the host:
 * a call only enqueues kernels on `stream`, so it may be recorded into a HIP
 * graph.  Calls are thread-safe.  `y` is fully overwritten.
 *
 * Errors.  Arguments are checked on the host before anything is enqueued; a
 * rejected call returns a negative Q4_E* code and writes nothing.  A kernel
 * launch failure returns Q4_ELAUNCH.  Faults inside a kernel surface at the
 * caller's next synchronization, as with any HIP kernel.
 *
 * Common limits: 1 <= M <= 64, 1 <= N <= 2^24, 1 <= K <= 32768; x and the packed weights
 * 16-byte aligned; scale arrays 2-byte aligned (fp16) or 1-byte (e4m3); y
 * 2-byte aligned and not overlapping any input.
 */
#ifndef Q4GEMV_H
#define Q4GEMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define Q4_OK 0
#define Q4_EINVAL_PTR (-1)   /* a required pointer is NULL */
#define Q4_EINVAL_SHAPE (-2) /* M, N or K out of range for the format */
#define Q4_EALIGN (-3)       /* a pointer is not aligned as documented */
#define Q4_EALIAS (-4)       /* the output overlaps an input */
#define Q4_ELAUNCH (-5)      /* the HIP runtime refused a kernel launch */
#define Q4_EVARIANT (-6)     /* unknown variant, or the variant cannot run this shape */
#define Q4_ESCRATCH (-7)     /* the call needs more split-K scratch than the built-in array holds */

/* kernel variants (the *_gemv_variant entry points) */
#define Q4_VARIANT_AUTO 0 /* pick by (M, N, K) */
#define Q4_VARIANT_DOT2 1 /* wave-per-row packed-BF16 dot products; batch tiles of <= 8 rows */
#define Q4_VARIANT_MFMA 2 /* 16x16x32 BF16 matrix-core tiles, batch padded to 16 */
#define Q4_VARIANT_TILED 4  /* K % 128 == 0: 64-row workgroups, matrix cores, activations staged in LDS
                               per 128-column group; split over K when given a workspace
                               (the *_grouped_ws calls); the default for M >= 5 */
#define Q4_VARIANT_STREAM 3 /* M <= 4, rows of exactly 1, 2 or 4 KB (int4/NVFP4 K = 2048, 4096, 8192;
                               BF16 K = 512, 1024, 2048): every weight load issued at once, activations
                               and group parameters shared through LDS */
#define Q4_VARIANT_SKINNY 6 /* 5 <= M <= 48, K % 128 == 0: workgroups of up to 80 rows over a slice of at
                               most 16 groups of 128 columns (BF16: 8), each wave loading its own weights and
                               activation fragments straight into registers (no per-group barriers); split
                               over K when given a workspace, else int4/NVFP4 K <= 2048, BF16 K <= 1024; the
                               default for int4 at 5 <= M <= 48 and for mixed groups there */
#define Q4_VARIANT_GEMM 5   /* int4 prefill only (q4g128_gemm_variant): workgroup tiles of 128 batch
                               rows x 128 or 256 weight rows over all of K, codes unpacked from LDS
                               per wave, scale and min folded per 128-column group */

/* weight formats (q4gemv_variant_name) */
#define Q4_FMT_Q4G128 0
#define Q4_FMT_NVFP4G16 1
#define Q4_FMT_BF16 2

/*
 * int4 "g128 min/max" weights.
 * Format: rumik-oss-1-int4 model card, section "Format":
 *   qweight  uint8 [N, K/2]   two 4-bit codes per byte, LOW nibble = EVEN column
 *   scale    fp16  [N, K/128]
 *   min      fp16  [N, K/128]
 *   w[n, k] = code[n, k] * scale[n, k/128] + min[n, k/128]
 * x: bf16 [M, K]; y: bf16 [M, N].  Requires K % 128 == 0.
 */
int q4g128_gemv(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N,
                uint16_t* y, void* stream);

/* Same as q4g128_gemv with an explicit Q4_VARIANT_* choice. */
int q4g128_gemv_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv,
                        int N, uint16_t* y, int variant, void* stream);

/*
 * Several independent int4 g128 GEMVs with one batch size M, launched
 * together (as few kernel launches as the shapes allow).  This is how
 * projections that read the same activations (q, k, v, gate, up of a layer)
 * or that are independent of each other (o and down of a parallel block) go
 * out as one unit, as the Rumik TTS Fast Inference post ("What Made It
 * Faster") does by packing projections that share an input -- here without
 * re-laying out any weights.  1 <= count <= 8; every task obeys the
 * q4g128_gemv rules; no task's y may overlap any task's inputs or another y.
 */
typedef struct q4g128_task {
    const uint16_t* x;       /* bf16 [M, K] */
    const uint8_t* qweight;  /* uint8 [N, K/2] */
    const uint16_t* scale;   /* fp16 [N, K/128] */
    const uint16_t* minv;    /* fp16 [N, K/128] */
    uint16_t* y;             /* bf16 [M, N] */
    int N;
    int K;
} q4g128_task;

int q4g128_gemv_grouped(const q4g128_task* tasks, int count, int M, int variant, void* stream);

/*
 * Same as q4g128_gemv_grouped, with a caller-owned device workspace that lets
 * the Q4_VARIANT_TILED kernel split K over several workgroups when the row
 * blocks of the launch alone cannot fill the GPU (the o/down stage of a decode
 * layer at M = 48).  The partial tiles are summed in a fixed order by
 * whichever workgroup finishes a row block last, so results do not depend on
 * timing and equal those of the unsplit kernel within fp32 rounding.
 *   workspace        device memory, 256-byte aligned, ZERO-FILLED before its
 *                    first use; its first 64 KiB hold arrival counters, which
 *                    every call leaves at zero, the rest partial tiles, which
 *                    are scratch: the workspace can be reused, also by calls
 *                    with other tasks, without being cleared again
 *   workspace_bytes  at least what q4g128_workspace_bytes reports for the same
 *                    tasks and M (a workspace sized for the largest of several
 *                    calls serves them all); with less (or NULL) the call runs
 *                    unsplit
 * Calls that use one workspace must not overlap in time (same stream, or
 * ordered by events).
 */
int q4g128_gemv_grouped_ws(const q4g128_task* tasks, int count, int M, int variant, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Workspace bytes q4g128_gemv_grouped_ws needs for these tasks (0 if no
 * split is planned).  Validates like the GEMV call; *bytes is set on Q4_OK. */
int q4g128_workspace_bytes(const q4g128_task* tasks, int count, int M, size_t* bytes);

/*
 * q4g128_gemv_grouped_ws without a workspace argument and without any
 * allocation, for callers that cannot allocate device memory: code recorded
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The split-K scratch is a built-in device array of 8 MiB per
 * GPU (Q4GEMV_NOALLOC_SCRATCH_BYTES), set up on the first call on a device
 * and held until the process ends; calls whose plan needs more than that
 * (q4g128_workspace_bytes > 8 MiB; no decode-layer shape at M <= 64 does)
 * return Q4_ESCRATCH before anything is enqueued.  Same kernels, plan and
 * results as q4g128_gemv_grouped_ws with a workspace of at least that size.
 * Every call on one GPU shares that GPU's array: calls on one GPU must not
 * overlap in time (same stream, or ordered by events), or they race.
 */
#define Q4GEMV_NOALLOC_SCRATCH_BYTES (8u << 20)
int q4g128_gemv_grouped_noalloc(const q4g128_task* tasks, int count, int M, int variant, void* stream);

/*
 * NVFP4 weight-only weights.
 * Format: VoxCPM2-NVFP4 model card, section "What was quantized": 4-bit float
 * (E2M1) codes, symmetric, group size 16, float8_e4m3fn group scales and one
 * fp32 global scale per matrix; activations stay BF16.
 *   qweight      uint8 [N, K/2]   E2M1 codes, LOW nibble = EVEN column
 *   scale_e4m3   uint8 [N, K/16]  OCP float8_e4m3fn bit patterns
 *   global_scale fp32            multiplier G
 *   w[n, k] = e2m1(code[n, k]) * e4m3(scale[n, k/16]) * G
 * x: bf16 [M, K]; y: bf16 [M, N].  Requires K % 32 == 0.
 */
int nvfp4g16_gemv(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale, int N,
                  uint16_t* y, void* stream);
int nvfp4g16_gemv_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale,
                          int N, uint16_t* y, int variant, void* stream);

/*
 * Up to 8 independent NVFP4 GEMVs of one batch size M in one launch (the
 * NVFP4 q, k, gate, up projections of a decode layer read the same input;
 * Rumik TTS Fast Inference post, section "What Made It Faster": packing
 * projections that share an input).  Each task is validated as
 * nvfp4g16_gemv; outputs must not overlap any task's inputs or each other.
 * workspace / workspace_bytes: as for q4g128_gemv_grouped_ws (NULL / 0: no K
 * split); nvfp4g16_workspace_bytes gives the size (0 if no split is planned).
 */
typedef struct nvfp4g16_task {
    const uint16_t* x;          /* bf16 [M, K] */
    const uint8_t* qweight;     /* uint8 [N, K/2] E2M1 */
    const uint8_t* scale_e4m3;  /* uint8 [N, K/16] */
    float global_scale;         /* multiplier G */
    uint16_t* y;                /* bf16 [M, N] */
    int N;
    int K;
} nvfp4g16_task;

int nvfp4g16_gemv_grouped_ws(const nvfp4g16_task* tasks, int count, int M, int variant, void* workspace,
                             size_t workspace_bytes, void* stream);
int nvfp4g16_workspace_bytes(const nvfp4g16_task* tasks, int count, int M, size_t* bytes);

/*
 * Dense BF16 weights (the audio head head.audio_weight [16385, 2048] of the
 * rumik-oss-1-int4 card, section "Format"; its 2049-row codebook slice from
 * the Rumik TTS Fast Inference post, section "What Made It Faster"; and the
 * v/down projections the VoxCPM2-NVFP4 card keeps in BF16).
 *   w bf16 [N, K]; x bf16 [M, K]; y bf16 [M, N].  Requires K % 8 == 0.
 */
int bf16_gemv(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* y, void* stream);
int bf16_gemv_variant(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* y, int variant, void* stream);

/*
 * Up to 8 independent BF16 GEMVs of one batch size M in one launch, validated
 * as bf16_gemv; workspace as for q4g128_gemv_grouped_ws, sized by
 * bf16_workspace_bytes (0 if no split is planned).
 */
typedef struct bf16_task {
    const uint16_t* x;  /* bf16 [M, K] */
    const uint16_t* w;  /* bf16 [N, K] */
    uint16_t* y;        /* bf16 [M, N] */
    int N;
    int K;
} bf16_task;

int bf16_gemv_grouped_ws(const bf16_task* tasks, int count, int M, int variant, void* workspace, size_t workspace_bytes,
                         void* stream);
int bf16_workspace_bytes(const bf16_task* tasks, int count, int M, size_t* bytes);

/*
 * Grouped GEMVs of mixed weight formats: up to 8 independent GEMVs, each
 * int4, NVFP4 or BF16, with one batch size M.  When M <= 4 and every task is
 * a streaming shape (rows of 1, 2 or 4 KB: int4/NVFP4 K = 2048, 4096, 8192;
 * BF16 K = 512, 1024, 2048) they run as ONE launch -- the NVFP4 decode step's
 * BF16 v projection beside its NVFP4 q, k, gate, up (one launch per format
 * would otherwise be needed).  At 5 <= M <= 48 with K % 128 == 0 for every
 * task they run as one launch of the skinny matrix-core kernel (given a
 * workspace of at least q4gemv_mixed_workspace_bytes where a task's K needs
 * more than one slice: int4/NVFP4 K > 2048, BF16 K > 1024).  Above that, with
 * such a workspace, NVFP4 and BF16 tasks that all take the tiled matrix-core
 * kernel also run as one launch.  Otherwise the tasks run as one grouped
 * launch per format, in task order of first appearance, on the same stream
 * (sharing the workspace).
 * Streaming and per-format results equal those of the single-format calls bit
 * for bit; the one-launch matrix-core forms follow the group's plan (its K
 * slices), within the GEMV tolerance of the single calls.  Each task obeys its
 * format's single-call rules; no task's y may overlap any task's inputs or
 * another y.
 */
typedef struct q4gemv_mixed_task {
    int format;              /* Q4_FMT_Q4G128, Q4_FMT_NVFP4G16 or Q4_FMT_BF16 */
    const uint16_t* x;       /* bf16 [M, K], 16-byte aligned */
    const void* weight;      /* int4/NVFP4: uint8 codes [N, K/2]; BF16: bf16 [N, K]; 16-byte aligned */
    const void* scale;       /* int4: fp16 [N, K/128]; NVFP4: e4m3 bytes [N, K/16]; BF16: unused */
    const uint16_t* minv;    /* int4: fp16 [N, K/128]; otherwise unused */
    float global_scale;      /* NVFP4: per-matrix multiplier; otherwise unused */
    uint16_t* y;             /* bf16 [M, N] */
    int N;
    int K;
} q4gemv_mixed_task;

int q4gemv_grouped_mixed(const q4gemv_mixed_task* tasks, int count, int M, void* workspace, size_t workspace_bytes,
                         void* stream);
int q4gemv_mixed_workspace_bytes(const q4gemv_mixed_task* tasks, int count, int M, size_t* bytes);

/*
 * Fused int4 GEMVs for the decode step's elementwise neighbours.  The Rumik
 * TTS Fast Inference post ("What Made It Faster") fuses the residual and
 * normalization operations around its weight-only projections so that their
 * data movement disappears; here the two around the MLP and the residual
 * stream of a decoder layer:
 *
 *   up != NULL:        the activations of the product are
 *                          h[m, k] = RN_bf16(silu(x[m, k]) * up[m, k]),
 *                      silu(g) = g / (1 + e^-g) -- the gated MLP's
 *                      activation, formed while the activations are staged
 *                      (x holds the gate projection's output): down(h) with
 *                      no separate elementwise kernel and no h in memory;
 *   residual != NULL:  y[m, n] = RN_bf16(sum_k h[m, k] w[n, k] + residual[m, n]),
 *                      one rounding of the exact sum plus the residual (the
 *                      o and down projections adding into the residual
 *                      stream); residual may be y itself (in place).
 *
 * silu is evaluated in fp32 with the hardware exp2 and reciprocal (a few fp32
 * ulps), so h can differ from the exactly rounded value by one BF16 step when
 * the exact product lies within that error of a rounding boundary.  Kernels:
 * the streaming kernel when every task allows it (M <= 4, K = 2048, 4096 or
 * 8192), else the skinny or the tiled kernel (K % 128 == 0; see below);
 * shapes the tiled kernel cannot run return Q4_EVARIANT.  Tasks obey the q4g128_gemv rules; up is bf16 [M, K], 16-byte
 * aligned; residual is bf16 [M, N], 2-byte aligned; no y may overlap any
 * input of any task or another y, except that a task's y may be exactly its
 * own residual.  workspace / workspace_bytes as for q4g128_gemv_grouped_ws
 * (q4g128_fused_workspace_bytes sizes it; NULL runs unsplit).  Beyond the
 * streaming kernel, a workspace of that size also holds h: it is then formed
 * once by a separate pass (one extra launch), and for 5 <= M <= 48 the
 * skinny kernel (Q4_VARIANT_SKINNY) runs the GEMV with the residual in its
 * epilogue; without a workspace, or for M > 48, the tiled kernel runs, its
 * loader waves forming h for every 64-row block when no pass did (same h bit
 * for bit).
 */
typedef struct q4g128_fused_task {
    const uint16_t* x;         /* bf16 [M, K] (the gate activations when up is set) */
    const uint16_t* up;        /* NULL, or bf16 [M, K] */
    const uint8_t* qweight;    /* uint8 [N, K/2] */
    const uint16_t* scale;     /* fp16 [N, K/128] */
    const uint16_t* minv;      /* fp16 [N, K/128] */
    const uint16_t* residual;  /* NULL, or bf16 [M, N] (may equal y) */
    uint16_t* y;               /* bf16 [M, N] */
    int N;
    int K;
} q4g128_fused_task;

int q4g128_gemv_fused(const q4g128_fused_task* tasks, int count, int M, void* workspace, size_t workspace_bytes,
                      void* stream);
int q4g128_fused_workspace_bytes(const q4g128_fused_task* tasks, int count, int M, size_t* bytes);

/*
 * Prefill GEMM: y[M, N] = x[M, K] . W^T for int4 g128 weights and any M >= 1
 * (the prompt's tokens before the decode loop; the rumik-oss-1-int4 card's
 * engine lists a 4-bit prefill matrix multiply beside its decode kernels,
 * "Running it").  M <= 64 takes the q4g128_gemv choice.  Larger M runs one
 * of two kernels in one launch:
 *   - Q4_VARIANT_GEMM: workgroup tiles of 128 batch rows x 128 or 256 weight
 *     rows over all of K; the default once the 128 x 128 tiles number at
 *     least 256 (one per CU), and for K > 16384;
 *   - Q4_VARIANT_TILED: the tiled decode kernel over batch chunks of up to 64
 *     rows, every chunk an unsplit product over the same weights (chunks of
 *     64 rows up to K = 4096, 32 rows up to 12288, 16 rows up to 16384; above
 *     that Q4_EVARIANT); the default for fewer tiles.
 * Both compute sum over groups of scale * sum(code * x) + min * sum(x) in
 * fp32 with every product exact, then round to BF16 once.  Same layouts and
 * rules as q4g128_gemv, with 1 <= M <= 524288 and K % 128 == 0.
 */
int q4g128_gemm(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N,
                uint16_t* y, void* stream);
/* q4g128_gemm with an explicit variant: Q4_VARIANT_AUTO, Q4_VARIANT_TILED or
 * Q4_VARIANT_GEMM (any M >= 1 for these two; else Q4_EVARIANT). */
int q4g128_gemm_variant(const uint16_t* x, int M, int K, const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv,
                        int N, uint16_t* y, int variant, void* stream);

/*
 * Sampling from the head: the step after the path.  The Rumik TTS Fast
 * Inference post samples each audio token at temperature 0.8 with top-k 30
 * ("The Result") from the head restricted to the current codebook, 2049 rows
 * ("What Made It Faster").  Per batch row m of BF16 logits [M, V]:
 *   1. the top_k largest logits, equal logits ordered by lower index (-0 and
 *      +0 are equal), in order of (logit descending, index ascending);
 *   2. p_i = softmax(logit_i / temperature) over those top_k, in fp32;
 *   3. token[m] = the first of that order whose running sum of p exceeds
 *      u[m] (the caller's uniform draw in [0, 1); the library draws no
 *      random numbers).
 * Outputs: token [M] int32; optionally topk_index [M, top_k] int32 and
 * topk_prob [M, top_k] fp32 (NULL to skip).  1 <= top_k <= 64 and
 * top_k <= V <= 30720; temperature finite and > 0; logits must hold no NaN.
 * The selection is exact; the probabilities and the draw are fp32 (a draw
 * can differ from exact arithmetic only when u lies within fp32 rounding of a
 * cumulative boundary).  Alignment: logits 2 bytes, u and the outputs 4 bytes;
 * outputs must not overlap each other or the inputs.
 *
 * q4_sample_topk samples from logits already in memory (one launch);
 * bf16_head_sample runs the BF16 head GEMV logits = x W^T (the bf16_gemv
 * rules, N = V; logits is the caller's [M, N] buffer) and then samples (two
 * launches).  Both return Q4_EINVAL_PTR / Q4_EINVAL_SHAPE / Q4_EALIGN /
 * Q4_EALIAS before enqueueing anything, Q4_ELAUNCH on a launch failure.
 */
int q4_sample_topk(const uint16_t* logits, int M, int V, float temperature, int top_k, const float* u, int32_t* token,
                   int32_t* topk_index, float* topk_prob, void* stream);
int bf16_head_sample(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* logits, float temperature, int top_k,
                     const float* u, int32_t* token, int32_t* topk_index, float* topk_prob, void* stream);

/*
 * bf16_head_sample with a caller workspace.  Same arguments, rules, results
 * and status codes, plus a workspace of ws_bytes bytes, 4-byte aligned and
 * zero-filled before its first use: it holds arrival counters (every call
 * leaves them at zero) and per-block top-k candidates (scratch).  It must not
 * overlap any other argument (Q4_EALIAS, as are Q4_EALIGN and the sampling
 * checks, returned before anything is enqueued).  The logits and the
 * selection are bitwise those of bf16_head_sample.
 *
 * M = 1 (the single-stream decode of the pages, which replay the step,
 * sampling included, as one graph; "Rumik TTS Fast Inference", "What Made It
 * Faster"): the GEMV and the sampling run as ONE launch.  The streaming GEMV
 * workgroups store their logits; the last to finish in each block of
 * workgroups selects that block's top_k entries, and the last block selects
 * among the candidates, sorts and draws -- no workgroup waits for another.
 * Needs K in {512, 1024, 2048, 4096, 8192}.
 * 2 <= M <= 64 and N > 1024: the GEMV, then the sampler split over blocks of
 * 1024 logits per row (one workgroup each; the last of a row to finish
 * selects among the blocks' candidates and draws) -- two launches, the second
 * with M * ceil(N / 1024) workgroups instead of M.
 * Applies when bf16_head_sample_workspace_bytes(M, N, K, top_k) is nonzero
 * (top_k <= 64, heads up to 30720 rows, and the cases above) and ws_bytes is
 * at least that; otherwise the call runs bf16_head_sample.  Calls that share
 * a workspace must not overlap in time.
 */
size_t bf16_head_sample_workspace_bytes(int M, int N, int K, int top_k);
int bf16_head_sample_ws(const uint16_t* x, int M, int K, const uint16_t* w, int N, uint16_t* logits, float temperature, int top_k,
                        const float* u, int32_t* token, int32_t* topk_index, float* topk_prob, void* workspace, size_t ws_bytes,
                        void* stream);

/*
 * Diagnostic dequantization of a whole matrix to fp32 w [N, K] (16-byte
 * aligned).  Bitwise equal to the format definitions above: int4 rounds
 * code*scale+min once; NVFP4 rounds e2m1*e4m3*G once (the first product is
 * exact).  Uses the device conversion helpers of the GEMV kernels.
 */
int q4g128_dequant_f32(const uint8_t* qweight, const uint16_t* scale, const uint16_t* minv, int N, int K, float* w, void* stream);
int nvfp4g16_dequant_f32(const uint8_t* qweight, const uint8_t* scale_e4m3, float global_scale, int N, int K, float* w,
                         void* stream);

/*
 * Diagnostic plain streaming read: the reference a GEMV launch of the same
 * bytes is compared with.  Reads `count` (1..32) device buffers bufs[i] of
 * bytes[i] bytes (each 4-byte aligned, 16 <= bytes[i] < 4 GiB) in one launch
 * with 16-byte loads and writes one XOR word per wave to the device buffer
 * `sink` of sink_words 32-bit words, which must be at least
 * q4gemv_stream_read_sink_words() and must not overlap the buffers.
 * Returns Q4_EINVAL_PTR, Q4_EINVAL_SHAPE, Q4_EALIGN or Q4_EALIAS before
 * enqueueing anything; Q4_ELAUNCH if the launch fails.
 */
int q4gemv_stream_read(const void* const* bufs, const size_t* bytes, int count, uint32_t* sink, size_t sink_words,
                       void* stream);
/* Sink words q4gemv_stream_read needs for these sizes (0 on invalid input). */
size_t q4gemv_stream_read_sink_words(const size_t* bytes, int count);

/*
 * Kernel timing without host gaps: the next kernel launched by the calling
 * thread through this library records start_event when it begins executing
 * and stop_event when it ends (hipExtLaunchKernel).  Both are caller-owned
 * hipEvent_t handles (either may be NULL); they apply to one launch only, so
 * time calls that launch one kernel.  Host only, always returns Q4_OK.
 */
int q4gemv_time_next_launch(void* start_event, void* stop_event);

/* Name of the kernel a call would run ("dot2", "mfma"); host only, never fails. */
const char* q4gemv_variant_name(int fmt, int variant, int M, int N, int K);

/* Static text for a status code; host only. */
const char* q4gemv_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int q4gemv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q4GEMV_H */
