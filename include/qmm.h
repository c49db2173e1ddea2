/*
 * qmm.h -- C ABI of libqmm: fused-dequant matmul of Q4_K / Q5_K / Q6_K weights with
 * Q8_1-quantized activations on AMD Instinct MI355X (gfx950).
 *
 * Pages cited (title, then section):
 *   [8e]  minfer ch. 06, "06 · 8e/8e② — decode MMVQ: dp4a integer dot
 *         products + the llama.cpp launch table"
 *   [MMQ] ZINC, "ZINC MMQ v2 — Fused Q4_K×Q8_1 Tensor-Core GEMM (beat
 *         llama.cpp)"
 *   [GAP] ZINC, "Prefill Gap Closure Plan — ZINC CUDA vs llama.cpp"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers.  Every buffer argument is a DEVICE pointer owned by the caller
 *   (e.g. torch tensor storage) and must be 16-byte aligned; the library never
 *   allocates, frees or keeps a pointer past the call.  Outputs must not alias
 *   inputs.
 * Stream.  `stream` is a hipStream_t (NULL = the default stream).  Every call
 *   only enqueues work on that stream and returns; none synchronises.
 * Status.  Every entry point returns QMM_OK (0) or a negative qmm_status.
 *   Argument errors are detected on the host before anything is enqueued, so
 *   a failing call has no effect.  QMM_ERR_HIP reports a launch error from the
 *   HIP runtime.  Device-side data (e.g. expert ids) cannot be checked without
 *   a synchronisation; their ranges are documented preconditions.
 *
 * Layouts
 * -------
 * Q4_K weights: rows of K/256 super-blocks of 144 bytes (f16 d at 0, f16
 *   dmin at 2, 12 bytes of packed 6-bit sub-block scales/mins at 4, 128 bytes
 *   of 4-bit values at 16); weight = d*sc*q - dmin*m per 32-weight sub-block
 *   ([8e] §2 and §3.2).  Row-major [M][K/256][144].
 * Q6_K weights: rows of K/256 super-blocks of 210 bytes (ql[128] at 0,
 *   qh[64] at 128, int8 sc[16] at 192, f16 d at 208); weight = d*sc*(q6-32)
 *   per 16-weight sub-block ([8e] §3.1 and §3.3).  Row-major [M][K/256][210].
 * Q8_1 activations ("pad40"): rows of K/32 blocks of 40 bytes (f16 d at 0,
 *   two zero pad bytes, int8 q[32] at 4, int32 sum of q at 36) ([8e] §2;
 *   [MMQ] "What they do right").  Row-major [rows][K/32][40].
 * Outputs: fp32, token-major y[t*M + i] ([8e] §3.2).
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qmm_status {
    QMM_OK = 0,
    QMM_ERR_NULL = -1,        /* a required pointer is NULL                      */
    QMM_ERR_SHAPE = -2,       /* a size is out of range or not a block multiple  */
    QMM_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned                */
    QMM_ERR_WORKSPACE = -4,   /* workspace smaller than qmm_workspace_bytes()    */
    QMM_ERR_HIP = -5,         /* the HIP runtime reported an error               */
    QMM_ERR_UNSUPPORTED = -6, /* unknown format / operation code                 */
    QMM_ERR_SCRATCH = -7      /* needs more than QMM_STATIC_SCRATCH_BYTES        */
} qmm_status;

/* Weight formats for moe_grouped_mmq, moe_slot_mmvq and qmm_debug_subdots. */
#define QMM_Q4_K 12
#define QMM_Q5_K 13
#define QMM_Q6_K 14

/* Operation codes for qmm_workspace_bytes. */
#define QMM_OP_MMQ 1        /* mmq_* and mmq_*_f32                               */
#define QMM_OP_MOE 2        /* moe_grouped_mmq, weighted (expert_weights != NULL) */
#define QMM_OP_MOE_SLOTS 3  /* moe_grouped_mmq, per-slot output (no weights)      */
#define QMM_OP_MOE_FFN 4    /* moe_ffn, with M = H and K = F                      */

/* Largest token count accepted by the matvec entry points. */
#define QMM_MMVQ_MAX_T 8

/*
 * q8_1_quantize -- fp32 activations x[T][K] (row-major) -> Q8_1 xq[T][K/32].
 * Per 32-block: am = max|x|, d = am/127, di = 1/d (0 if d == 0),
 * q = clamp(rint(x*di), -128, 127) rounding half to even, stored with
 * f16(d) (round to nearest even), zero pad and the int32 sum of q
 * ([8e] §2 and the quantizer of §3.2).  IEEE fp32 division, no contraction:
 * the bytes are bit-identical to the IEEE emulation of these steps.
 * Tiny blocks: when d is below 2^-126 (max|x| < 127 * 2^-126, an fp32
 * subnormal scale) 1/d would overflow, so di = 0 as for d == 0 and the block
 * is stored as all zeros (its f16 scale rounds to 0 anyway, so the
 * dequantized block is 0 either way).  Input must be finite with
 * max|x| <= 127 * 65504 (f16 range of d).
 * Requires T >= 0, K > 0, K % 32 == 0.  T == 0 is a no-op.
 */
int q8_1_quantize(const float* x, void* xq, int64_t T, int64_t K, void* stream);

/*
 * mmvq_q4k / mmvq_q6k -- decode matvec y[T][M] = xq[T][K] . W[M][K]^T for
 * 1 <= T <= QMM_MMVQ_MAX_T ([8e] §2-§3.2: integer 4-way dot products of
 * unpacked 4-bit (6-bit) weights with int8 activations; the Q4_K min term
 * uses the activation sums: a dot product against ones, or at T = 1 the
 * integer sum stored in each Q8_1 block).  One wave64 per weight row streams
 * the row's blocks.  Requires M >= 1, K % 256 == 0.
 * Output fp32, y[t*M + i].  Deterministic: identical inputs give identical
 * bits.
 */
int mmvq_q4k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
             void* stream);
/* Q5_K weights ([M][K/256] blocks of 176 bytes; the pages name the format but
 * not its layout, which is read as GGUF's: f16 d, f16 dmin, the 12 packed
 * scale/min bytes of Q4_K, qh[32] fifth bits, qs[128] 4-bit values).  Same
 * arguments, limits and errors as mmvq_q4k; w must be 16-byte aligned. */
int mmvq_q5k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T, void* stream);
int mmvq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
             void* stream);

/*
 * mmvq_pair -- two one-token matvecs on the same activation row, in one
 * launch: ya[Ma] = xq . Wa^T and yb[Mb] = xq . Wb^T, Wa and Wb each in any
 * of QMM_Q4_K, QMM_Q5_K, QMM_Q6_K (the decode matvec of [8e] §2-§3.2; one
 * launch for products that share their input, as [GAP] lever T4 shares one
 * activation preparation across same-input products).  xq holds one Q8_1
 * row of K values; wa, wb are [Ma][K/256] and [Mb][K/256] blocks.  Each
 * output has the bits the single matvec (mmvq_q4k / mmvq_q5k / mmvq_q6k at
 * T = 1) gives for it: the workgroups of the two matrices run the same code
 * in one grid, so the launch has one tail instead of two.  Where the Q6_K
 * one-token kernel does not take a shape (rows of more than 46 super-blocks,
 * or Mb * K/256 not a multiple of 8), the two matvecs run as two launches.
 * Requires Ma, Mb >= 1, K % 256 == 0, 16-byte aligned pointers; ya and yb
 * must not overlap.  Errors as mmvq_q4k; QMM_ERR_UNSUPPORTED for any other
 * format.
 */
int mmvq_pair(int fmt_a, const void* wa, int64_t Ma, float* ya, int fmt_b, const void* wb, int64_t Mb,
              float* yb, const void* xq, int64_t K, void* stream);

/*
 * mmq_q4k / mmq_q6k -- prefill GEMM y[T][M] = xq[T][K] . W[M][K]^T for any
 * T >= 1 ([MMQ] "Kernel architecture": fused dequant inside the matrix
 * inner loop, Q8_1 activations; "Persistent kernel + atomic work queue").
 * Weights are unpacked to int8 and multiplied on int8 MFMA with int32
 * accumulation per sub-block, then scaled in fp32.  A first kernel repacks
 * the Q8_1 activations into `ws` (MFMA operand order plus per-block fp32
 * factors); output tiles are then claimed from per-XCD atomic counters in
 * `ws`.  When the call has enough 128 x 32/64 output tiles to fill the chip,
 * each tile runs its whole K loop in one workgroup (its two K halves summed
 * in a fixed order, no fixup).  A call with fewer than 256 tiles (few tokens
 * and rows) uses split-K with a deterministic in-kernel fixup instead: each
 * tile's K range is split over up to 16 workgroups, which write fp32
 * partial tiles to `ws`; the last to finish adds them in split order.
 * Either way the result of a call depends only on its shapes and data (the
 * split factor is a function of M, K and T), so results are deterministic.
 * `ws` must hold qmm_workspace_bytes(QMM_OP_MMQ, M, K, T, 0, 0) bytes (M
 * counts: it sizes the partial tiles); its contents are
 * scratch (the call initialises what it uses, no zero-fill is needed).
 * Calls sharing one workspace must be ordered on one stream.
 * Requires M >= 1, 1 <= T <= 2^24, K % 256 == 0, K/256 <= 65536 and at most
 * 2^30 output tiles (ceil(M/128) * ceil(T/64) * splits).
 */
int mmq_q4k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
            void* ws, size_t ws_bytes, void* stream);
/* Q5_K weights (layout as for mmvq_q5k); same arguments, workspace, limits and
 * errors as mmq_q4k.  The fifth bit of each weight joins its 4-bit value in
 * the int8 MFMA operand (values 0..31). */
int mmq_q5k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
            void* ws, size_t ws_bytes, void* stream);
int mmq_q6k(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
            void* ws, size_t ws_bytes, void* stream);

/*
 * mmq_q4k_noalloc -- mmq_q4k for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and result, bit for bit, but the workspace is
 * a static device array of QMM_STATIC_SCRATCH_BYTES inside the library, so
 * the caller passes only inputs and outputs.  The call allocates nothing.
 * A call whose qmm_workspace_bytes(QMM_OP_MMQ, M, K, T, 0, 0) exceeds
 * QMM_STATIC_SCRATCH_BYTES returns QMM_ERR_SCRATCH before anything is
 * enqueued (e.g. T = 1024 needs K <= 23552).  Each GPU holds one copy of the
 * array for the life of the process, shared by every call on that GPU:
 * calls that overlap on one GPU (different streams, or host threads without
 * ordering) race and give wrong results; calls ordered on one stream are
 * safe.  The call clears what must start at zero (its queue counters) in
 * its first kernel.  Same arguments, limits and other errors as mmq_q4k.
 */
#define QMM_STATIC_SCRATCH_BYTES (32u << 20)
int mmq_q4k_noalloc(const void* w, const void* xq, float* y, int64_t M, int64_t K, int64_t T,
                    void* stream);

/*
 * mmq_q4k_f32 / mmq_q6k_f32 -- the same GEMM with fp32 activations x[T][K]
 * (row-major, 16-byte aligned), quantized to Q8_1 inside the call: the
 * activation repack quantizes each 32-block with the steps of q8_1_quantize
 * ([8e] §3.2) and writes the GEMM's operand chunks directly, so the Q8_1
 * rows never go to memory ([MMQ] "What they do right": activations
 * quantized on the way into the GEMM).  The output is bit-identical to
 * q8_1_quantize followed by mmq_q4k / mmq_q6k on the same stream.  Same
 * workspace (qmm_workspace_bytes(QMM_OP_MMQ, M, K, T, 0, 0)), limits and
 * errors as mmq_q4k; x must not alias y or ws.
 */
int mmq_q4k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                void* ws, size_t ws_bytes, void* stream);
int mmq_q5k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                void* ws, size_t ws_bytes, void* stream);
int mmq_q6k_f32(const void* w, const float* x, float* y, int64_t M, int64_t K, int64_t T,
                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_mmq -- routed-expert grouped GEMM ([GAP] lever T2 and its
 * de-risk paragraph: histogram of expert ids, prefix-sum offsets, per-expert
 * slot buckets, one product per expert, scatter back; [MMQ] "MoE routing
 * (fused gather)": work entries (expert, m_tile, n_tile)).
 *   fmt                  QMM_Q4_K, QMM_Q5_K or QMM_Q6_K
 *   w                    E experts, each M rows of K weights, expert e at
 *                        (const char*)w + e*expert_stride_bytes
 *   xq                   Q8_1 activations, rows of K/32 blocks: T rows when
 *                        x_rows_per_token == 1 (row t), else T*top_k rows
 *                        (row t*top_k + k), x_rows_per_token == top_k
 *   ids                  int32 [T][top_k], every id in [0, E) (precondition)
 *   expert_weights       NULL: y is per-slot, y[(t*top_k + k)*M + i] =
 *                        W[ids[t][k]] . x_row; otherwise fp32 [T][top_k] and
 *                        y[t*M + i] = sum_k p[t][k] * (W[ids[t][k]] . x_row)
 *                        summed in increasing k (deterministic, no atomics)
 *   ws                   qmm_workspace_bytes(QMM_OP_MOE, ...) bytes for a
 *                        weighted call, QMM_OP_MOE_SLOTS for a per-slot one
 *                        (same sizes); scratch, no initialisation needed;
 *                        holds the buckets, the queue counters, the routed
 *                        rows repacked per expert and, in weighted mode, the
 *                        per-slot fp32 results
 * Work is tiled as 256 (Q4_K, Q5_K) or 128 (Q6_K) weight rows x 32 routed
 * slots of one expert, so an expert's weights are read once per 32 tokens
 * routed to it.  The route tables (counts, offsets, column tiles, buckets)
 * sit at the front of ws and depend only on ids, T, top_k and E.  Requires
 * 1 <= E <= 512, M >= 1, K % 256 == 0, K/256 <= 65536, 1 <= top_k <= min(E, 64),
 * T >= 1, T*top_k <= 2^30, at most 2^30 work entries (ceil(M/128) times the
 * column-tile bound (T*top_k + 31*min(E, T*top_k))/32),
 * x_rows_per_token in {1, top_k}, expert_stride_bytes >= M*K/256*block bytes
 * and a multiple of 16 (Q4_K) or 2 (Q6_K).
 */
int moe_grouped_mmq(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                    int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                    const int32_t* ids, const float* expert_weights, int64_t T, int64_t top_k,
                    float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_mmq_routed -- moe_grouped_mmq without the route preparation:
 * the route tables already in ws are used.  For the second grouped call of a
 * routed FFN (the down projection after gate||up), whose tokens are routed
 * exactly as for the first ([GAP] lever T2: route once per layer).
 * Precondition (not checked): the last grouped call on this ws, completed or
 * earlier on the same stream, had the same ids contents, T, top_k and E;
 * ws_bytes must cover this call's own qmm_workspace_bytes.  Same arguments,
 * results, limits and errors as moe_grouped_mmq.
 */
int moe_grouped_mmq_routed(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                           int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                           const int32_t* ids, const float* expert_weights, int64_t T, int64_t top_k,
                           float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_mmq_swiglu -- the grouped gate||up product of a routed FFN with
 * the SwiGLU glue fused into its epilogue: per routed slot, h = silu(gate) *
 * up quantized to Q8_1 ([GAP] lever T2's grouped expert GEMM; lever T4: the
 * producer emits the next product's input format directly, no fp32 round
 * trip).  Each expert's M = 2F rows hold gate in rows [0, F) and up in
 * [F, 2F), as moe_grouped_mmq's gate||up call takes them; hq receives
 * [T*top_k][F/32] Q8_1 blocks (40 bytes each), the same bytes as
 * moe_grouped_mmq (no expert_weights) followed by swiglu_q8_1.  Routing,
 * workspace (qmm_workspace_bytes(QMM_OP_MOE_SLOTS, M, K, T, E, top_k)) and
 * the route tables it leaves in ws for moe_grouped_mmq_routed are those of
 * moe_grouped_mmq.  Requires fmt QMM_Q4_K or QMM_Q5_K
 * (QMM_ERR_UNSUPPORTED otherwise) and M a multiple of 256; hq 16-byte
 * aligned.  Other arguments, limits and errors as moe_grouped_mmq.
 */
int moe_grouped_mmq_swiglu(int fmt, const void* w, int64_t E, int64_t M, int64_t K,
                           int64_t expert_stride_bytes, const void* xq, int64_t x_rows_per_token,
                           const int32_t* ids, int64_t T, int64_t top_k, void* hq, void* ws, size_t ws_bytes,
                           void* stream);

/*
 * moe_ffn -- a routed FFN layer in one call ([GAP] lever T2: route once, the
 * grouped expert GEMM for both products; lever T4: each producer emits its
 * consumer's input directly): y[T][H] = sum_k p[t][k] * down_e . SwiGLU(
 * gate_up_e . x_t) with e = ids[t][k].  w_gu holds E experts of 2F x H
 * (gate rows [0, F), up rows [F, 2F); fmt_gu QMM_Q4_K or QMM_Q5_K), w_dn E
 * experts of H x F (fmt_dn any of the three), expert strides in bytes as in
 * moe_grouped_mmq; xq the Q8_1 rows of x [T][H/32]; expert_weights p
 * [T][top_k] fp32.  The gate||up epilogue forms SwiGLU -> Q8_1 and writes the
 * down product's repacked activation chunks into ws itself, so there are no
 * SwiGLU rows and no second repack; the output is bit-identical to
 * moe_grouped_mmq_swiglu followed by moe_grouped_mmq_routed (weighted).
 * ws: qmm_workspace_bytes(QMM_OP_MOE_FFN, H, F, T, E, top_k) bytes.
 * Requires H % 256 == 0, F % 256 == 0, the limits of moe_grouped_mmq;
 * QMM_ERR_UNSUPPORTED for other formats.
 */
int moe_ffn(int fmt_gu, const void* w_gu, int64_t stride_gu, int fmt_dn, const void* w_dn, int64_t stride_dn,
            int64_t E, int64_t H, int64_t F, const void* xq, const int32_t* ids, const float* expert_weights,
            int64_t T, int64_t top_k, float* y, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_slot_mmvq -- the per-(token, slot) expert matvec that the grouped GEMM
 * replaces ([GAP] lever T2: the batched expert matvec re-reads an expert's
 * weights once per routed token; its de-risk step compares the two at
 * expert shapes).  Same arguments and per-slot output as moe_grouped_mmq
 * with expert_weights == NULL: y[(t*top_k + k)*M + i] = W[ids[t][k]] . x_row,
 * one matvec (the mmvq_q4k / mmvq_q5k / mmvq_q6k kernel at T = 1) per routed
 * slot, no workspace; fmt may also be QMM_Q5_K.  ids outside [0, E) are clamped (precondition; no fault).
 * Requires 1 <= top_k <= E, T*top_k <= 65535, K % 256 == 0, an expert
 * stride of at least M rows and a multiple of 16 bytes (Q4_K, Q5_K) or 2
 * (Q6_K), 16-byte aligned pointers.
 */
int moe_slot_mmvq(int fmt, const void* w, int64_t E, int64_t M, int64_t K, int64_t expert_stride_bytes,
                  const void* xq, int64_t x_rows_per_token, const int32_t* ids, int64_t T, int64_t top_k,
                  float* y, void* stream);

/*
 * swiglu_q8_1 -- glue between the grouped gate/up and down calls: reads the
 * per-slot gate||up rows g_u[R][2*F] (fp32; gate in columns 0..F-1, up in
 * F..2F-1), computes h = silu(gate) * up in fp32 and writes Q8_1 hq[R][F/32]
 * with the quantizer of q8_1_quantize.  The pages name fused SwiGLU producers
 * of the quantized activation ([8e] §3.2) but give no formula; silu(g)*u is
 * the reading taken.  Requires R >= 0, F % 32 == 0.
 */
int swiglu_q8_1(const float* g_u, void* hq, int64_t R, int64_t F, void* stream);

/* Bytes of workspace needed by `op` (QMM_OP_MMQ, QMM_OP_MOE or
 * QMM_OP_MOE_SLOTS) for the given sizes; unused sizes may be 0.  Returns 0
 * for an unknown op.  The workspace is the scratch the caller allocates
 * once, outside any graph-capture window, and passes in: no entry point
 * allocates ([8e] §3.1, the rule that the q8 activation scratch is never
 * allocated inside a capture window). */
size_t qmm_workspace_bytes(int op, int64_t M, int64_t K, int64_t T, int64_t E, int64_t top_k);

/* Zero-fills a workspace on `stream` with a fill kernel (no memset node).
 * Not required by any entry point (each initialises the workspace state it
 * uses); kept for callers that want deterministic workspace contents. */
int qmm_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Static text for a qmm_status value. */
const char* qmm_status_str(int status);

/*
 * qmm_debug_subdots -- test hook: the integer stage of the MMVQ
 * (path == 0) or MMQ (path == 1) kernel of format `fmt`, built from the same
 * source as the product kernels, writing the exact integer sub-block sums
 * instead of the scaled result.  Its signature extends the proposed
 * (fmt, w, xq, D, S, M, K, T, stream) by `path` (which kernel's integer stage)
 * and (ws, ws_bytes) (the GEMM path's workspace).  Q4_K: D[T][M][K/32] = sum nib*q and
 * S[T][K/32] = sum q (the ones-dot on path 0, the stored sum on path 1);
 * Q5_K the same with the 5-bit values.  Q6_K: D[T][M][K/16] = sum (q6-32)*q and S is not written.  T <= 8 for
 * path 0.  Path 1 needs an MMQ workspace (ws, ws_bytes) like mmq_q4k; path 0
 * ignores it.  D and S are zero-filled by the call.  For tests on small
 * shapes only.
 */
int qmm_debug_subdots(int fmt, int path, const void* w, const void* xq, int32_t* D, int32_t* S,
                      int64_t M, int64_t K, int64_t T, void* ws, size_t ws_bytes, void* stream);

/*
 * qmm_probe_read -- measurement hook, not part of the method: a read-only
 * streaming kernel over `bytes` bytes of `buf` (a multiple of 16) that
 * reduces them to one word written to sink[0].  Gives the HBM read ceiling
 * at a given byte count ([8e] §3.3 and §6: measure a read-only ceiling before
 * calling a bandwidth figure a limit).
 */
int qmm_probe_read(const void* buf, size_t bytes, uint32_t* sink, void* stream);

/*
 * qmm_probe_mfma -- measurement hook, not part of the method: int8 MFMA
 * (v_mfma_i32_32x32x32_i8, 65536 int8 ops each) back to back from
 * registers, four independent accumulators per wave, `iters` rounds of four
 * per wave; one workgroup of eight waves per CU per two waves per SIMD
 * (waves_per_simd 2, 4 or 8).  Ops per launch = CUs * waves_per_simd * 4 *
 * iters * 4 * 65536.  The matrix-core rate the int8 peak assumes ([MMQ]
 * "Revised priorities (post-M3 findings)": measure before tuning).
 * 1 <= iters <= 2^24.  Writes sink[0] only for an improbable value.
 */
int qmm_probe_mfma(int64_t iters, int waves_per_simd, uint32_t* sink, void* stream);

/*
 * qmm_probe_mfma_epilogue -- measurement hook: the GEMM's per-sub-block
 * inner loop without global memory ([GAP] root cause 1, the per-sub-block
 * rescale epilogue).  Per iteration and wave: two int8 MFMAs (two 32-column
 * blocks) started from the bits of 1.5*2^23 and, per output element, the two
 * fp32 FMAs of the epilogue.  mode 1: operands in registers; mode 2: row
 * scales, column factors and B operands read from LDS as the GEMM reads
 * them; mode 3: mode 2 plus the Q4_K min-term fp32 MFMA every second
 * iteration into the FMA accumulator; mode 4: that MFMA into an accumulator
 * of its own; mode 5: the min term as three bf16 MFMAs per eight
 * iterations into its own accumulator; mode 6: the same into the FMA
 * accumulator; mode 7: mode 6 with a workgroup barrier every eight
 * iterations; mode 8: mode 7 with the A operand unpacked from 4-bit values
 * each iteration; mode 9: the one-column-block loop of the grouped GEMM
 * (no software pipelining, row scales read four at a time, two workgroups
 * per CU whatever waves_per_simd says; its ops per launch are half those of
 * modes 1-8 at four waves per SIMD).  int8 ops per launch = CUs * waves_per_simd * 4 * iters * 2 *
 * 65536.  waves_per_simd 2 or 4; 1 <= iters <= 2^24.
 */
int qmm_probe_mfma_epilogue(int mode, int64_t iters, int waves_per_simd, uint32_t* sink, void* stream);

/*
 * qmm_probe_read_geom -- measurement hook: qmm_probe_read with its geometry
 * as arguments, for sweeping the HBM read ceiling ([8e] §6: concurrency
 * first).  Each thread of 256-thread workgroups issues loads_per_thread
 * (1, 2, 4, 8 or 16) lane-contiguous 16-byte loads before using any;
 * grid = 0 launches one pass over `bytes` (a multiple of 16), a smaller
 * grid strides over the buffer persistently.
 */
int qmm_probe_read_geom(const void* buf, size_t bytes, int loads_per_thread, int64_t grid, uint32_t* sink,
                        void* stream);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
