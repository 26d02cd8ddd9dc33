/*
 * mi355gemm -- half-precision GEMM with fp32 accumulation and an optional fused
 * bias + erf-GELU epilogue, written for AMD Instinct MI355X (gfx950, CDNA4).
 *
 * C ABI (C99).  No torch or HIP types appear in the signatures: device buffers are
 * plain pointers, the stream is an opaque pointer (a hipStream_t, NULL for the
 * default stream).
 *
 * The operation follows "Designing High-Performance GPU Kernels with TileLang:
 * Tensor-Core GEMM, Fused Softmax, FlashAttention, and Autotuning":
 *   - thecryptopost.io page, section 2 "Memory hierarchy - tiled tensor-core GEMM",
 *     make_matmul: A is (M, K), B is (K, N), C is (M, N), all float16 and row-major,
 *     the accumulator is "float" (fp32);
 *   - ainovat.com page, the fused-epilogue paragraph: bias addition and GELU are
 *     applied to the register-resident accumulator before the single write of C.
 *
 *   epilogue NONE       C[i][j] = fp16( sum_k A[i][k] B[k][j] )
 *   epilogue BIAS       C[i][j] = fp16( sum_k A[i][k] B[k][j] + bias[j] )
 *   epilogue BIAS_GELU  C[i][j] = fp16( GELU( sum_k A[i][k] B[k][j] + bias[j] ) )
 *   with GELU(x) = x * Phi(x) = 0.5 x (1 + erf(x / sqrt 2)) (the exact, erf form),
 *   the sum and the epilogue in fp32, and one round-to-nearest-even to fp16 at the
 *   store.  The order of the fp32 additions over k is unspecified.
 */
#ifndef MI355GEMM_H
#define MI355GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MI355GEMM_EPI_NONE = 0,
    MI355GEMM_EPI_BIAS = 1,
    MI355GEMM_EPI_BIAS_GELU = 2
} mi355gemm_epilogue;

typedef enum {
    MI355GEMM_OK = 0,
    MI355GEMM_EINVAL = 1,       /* bad argument: negative size, null pointer, bad enum */
    MI355GEMM_EUNSUPPORTED = 2, /* legal request this build cannot serve */
    MI355GEMM_EHIP = 3          /* the HIP runtime reported an error (see last_error) */
} mi355gemm_status;

/*
 * C = epilogue(A . B [+ bias]), enqueued on `stream`.
 *
 * M, N, K  problem sizes (>= 0).  M == 0 or N == 0: nothing to do, returns OK without
 *          a launch.  K == 0: C = epilogue(bias or 0) (an empty sum).
 * A        device pointer, M x K fp16, row-major, leading dimension K.
 * B        device pointer, K x N fp16, row-major, leading dimension N.
 * C        device pointer, M x N fp16, row-major, leading dimension N; written, never
 *          read.  Memory outside the M x N window is not touched.
 * bias     device pointer to N fp16 values (one per output column), required for the
 *          BIAS and BIAS_GELU epilogues, ignored (may be NULL) for NONE.
 * epi      a mi355gemm_epilogue value.
 * stream   hipStream_t to enqueue on; NULL is the default stream.
 *
 * Ownership: the caller owns every buffer; the library allocates nothing, keeps no
 * per-call state and needs no workspace.  The call is asynchronous (it returns after
 * the enqueue) and thread-safe.  C must not overlap A, B or bias (not checked).
 * Every pointer must be at least 2-byte aligned; shapes or pointers that are not
 * 16-byte friendly are served, never rejected.  Where the chosen configuration is a
 * direct one but the rows of B and C are not 16-byte friendly (N % 8 != 0, B or C not
 * 16-byte aligned, or the bias not 8-byte aligned), the call makes two launches on
 * `stream`: the direct kernel computes columns [0, N & ~7) with unaligned 16-byte
 * accesses, and a narrow kernel (fp32 vector multiply-adds, any alignment) the last
 * N % 8 columns.  Problems with at most 8 columns that the direct kernel does not take
 * run on the narrow kernel alone; other small problems take the register-staged
 * kernels, whose 2-byte load variants accept any alignment.
 *
 * Errors: EINVAL for negative sizes, null pointers with work to do, an unknown
 * epilogue, a bias epilogue with bias == NULL, or a misaligned pointer; EUNSUPPORTED
 * if K or N is 2^22 or more (the per-tile buffer descriptors use 32-bit byte offsets)
 * or M is 2^31 or more; EHIP if the launch fails.  A non-OK return leaves C untouched
 * and sets mi355gemm_last_error().
 */
mi355gemm_status mi355gemm_gemm(int64_t M, int64_t N, int64_t K,
                                const void *A, const void *B, void *C, const void *bias,
                                int epi, void *stream);

/*
 * As mi355gemm_gemm, but with the kernel configuration forced to `config_id`
 * (0 <= id < mi355gemm_num_configs()).  For sweeps and tests: a configuration that
 * cannot serve this shape or these pointers (for instance a 16-byte-load configuration
 * with K % 8 != 0) returns EUNSUPPORTED, like the tutorial's schedule sweep skipping
 * candidates over the shared-memory budget (thecryptopost.io page, section 3 "Knobs -
 * sweeping the schedule by hand").
 */
mi355gemm_status mi355gemm_gemm_config(int64_t M, int64_t N, int64_t K,
                                       const void *A, const void *B, void *C,
                                       const void *bias, int epi, void *stream,
                                       int config_id);

/*
 * As mi355gemm_gemm_config (config_id = -1: the selector's choice, as mi355gemm_gemm),
 * and in addition records two caller-created HIP events (hipEvent_t with timing enabled)
 * from the kernel dispatch itself: start_event as the call's first kernel starts,
 * stop_event as its last kernel ends (hipExtLaunchKernel).  hipEventElapsedTime(start,
 * stop) is then the kernels' own duration, the figure a kernel trace reports, without
 * the dispatch latency that events recorded before and after the call on the stream
 * also count.  For benchmarks: the tutorial times its kernels with device events
 * (thecryptopost.io page, section 2, bench()).  Either event may be NULL.  A call with
 * nothing to launch (M == 0 or N == 0) records neither; errors as mi355gemm_gemm_config.
 */
mi355gemm_status mi355gemm_gemm_timed(int64_t M, int64_t N, int64_t K,
                                      const void *A, const void *B, void *C,
                                      const void *bias, int epi, void *stream,
                                      int config_id, void *start_event, void *stop_event);

/*
 * The configuration mi355gemm_gemm would launch for these arguments, or -1 (with
 * last_error set) if the arguments are invalid.  Host-only: makes no HIP call.
 * The choice is keyed on the shape and on pointer/leading-dimension alignment; the
 * tutorial notes the best schedule depends on the architecture and the shape
 * (thecryptopost.io page, section 3).  A direct configuration returned for rows of B
 * and C that are not 16-byte friendly is the one that computes columns [0, N & ~7);
 * mi355gemm_gemm then adds the narrow kernel for the last N % 8 columns.
 */
int mi355gemm_select(int64_t M, int64_t N, int64_t K, int epi,
                     const void *A, const void *B, const void *C, const void *bias);

/*
 * Install a choice for this process: requests with exactly these sizes and epilogue, whose
 * A rows are (a_vector = 1) or are not (0) 16-byte friendly and whose B, C and bias rows
 * are (bc_vector = 1) or are not (0), take config_id in mi355gemm_gemm,
 * mi355gemm_gemm_timed with config_id -1 and mi355gemm_select, ahead of the measured
 * table and the rules.  "16-byte friendly" is as for the configurations' alignment needs:
 * K % 8 == 0 and A 16-byte aligned; N % 8 == 0, B and C 16-byte aligned and the bias
 * 8-byte aligned.  The tutorial's point that the best schedule depends on the machine
 * and the shape (thecryptopost.io page, section 3) holds from one MI355X machine to the next
 * too, so a caller may time the candidates on its device and install the winner.  An entry
 * with the same key is replaced.  Host memory only, no HIP call; safe to call while other
 * threads launch.  Returns MI355GEMM_EINVAL for negative sizes, an unknown epilogue or
 * config id, or a class other than 0 or 1; MI355GEMM_EUNSUPPORTED when the configuration
 * needs 16-byte rows the class does not promise, computes fewer than N columns (narrow),
 * or when the table already holds 64 entries.
 */
mi355gemm_status mi355gemm_set_choice(int64_t M, int64_t N, int64_t K, int epi,
                                      int a_vector, int bc_vector, int config_id);

/* Remove every choice installed with mi355gemm_set_choice. */
void mi355gemm_clear_choices(void);

/*
 * c[i] = a[i] + b[i] for 0 <= i < n, all fp16, one round-to-nearest-even per element (the
 * correctly rounded sum), enqueued on `stream`.  The tutorial's first kernel: "Designing
 * High-Performance GPU Kernels with TileLang: ...", ainovat.com page, first paragraph (a
 * vector-add kernel whose bandwidth is compared with PyTorch's).  HBM-bound: 6 bytes move
 * per element; the benchmark reports its GB/s as the measured memory roofline.
 *
 * n        number of elements (>= 0; 0 does nothing and returns OK).
 * a, b     device pointers to n fp16 values each (read).
 * c        device pointer to n fp16 values (written; may be a or b, element-wise).
 * stream   hipStream_t to enqueue on; NULL is the default stream.
 *
 * Every pointer must be at least 2-byte aligned; any such alignment is served.  The
 * caller owns the buffers; the call allocates nothing and returns after the enqueue.
 * Errors: EINVAL for n < 0, a NULL pointer with n > 0 or a misaligned pointer; EHIP if
 * the launch fails.
 */
mi355gemm_status mi355gemm_vector_add(int64_t n, const void *a, const void *b, void *c,
                                      void *stream);

/*
 * Row-wise softmax: y[i][j] = exp(x[i][j] - m_i) / sum_j exp(x[i][j] - m_i) with
 * m_i = max_j x[i][j], for an M x N fp16 row-major x; fp32 arithmetic, one rounding to
 * fp16 per output.  The tutorial's fused softmax: "Designing High-Performance GPU Kernels
 * with TileLang: ...", ainovat.com page, third paragraph (maximum and sum reductions over
 * each row, the normalisation kept in registers).  HBM-bound: 4 bytes per element.
 *
 * M, N     rows and row length (>= 0; M == 0 or N == 0 does nothing and returns OK).
 * x        device pointer to M x N fp16 (read), leading dimension N.
 * y        device pointer to M x N fp16 (written), leading dimension N; may equal x.
 * stream   hipStream_t to enqueue on; NULL is the default stream.
 *
 * Rows of up to 65536 elements are held in registers (by one wavefront up to 2048
 * elements, by 4 up to 16384, by 16 beyond); longer rows take two passes over the row by
 * one workgroup.  IEEE rules give the edge cases: a row with
 * a NaN or +inf entry, or with every entry -inf, comes out NaN.  Pointers must be 2-byte
 * aligned (any such alignment and any N are served).  The caller owns the buffers; the
 * call allocates nothing and returns after the enqueue.  Errors: EINVAL for negative
 * sizes, NULL pointers with work to do or misaligned pointers; EUNSUPPORTED for M or N
 * of 2^31 or more; EHIP if the launch fails.
 */
mi355gemm_status mi355gemm_softmax(int64_t M, int64_t N, const void *x, void *y, void *stream);

/*
 * Attention forward (the tutorial's FlashAttention: "Designing High-Performance GPU
 * Kernels with TileLang: ...", ainovat.com page, the FlashAttention paragraph -- query,
 * key and value tiles, an online softmax with running maxima, sums and rescaling, tiled
 * tensor-core products, the score matrix never written to memory; causal and non-causal).
 * For every (batch, head) pair and query row i:
 *   s_j = scale * sum_d q[i][d] k[j][d]   for the allowed keys j: all 0 <= j < seq_k, or,
 *         when causal, j <= i (the upper-left aligned mask of PyTorch's is_causal);
 *   o[i][d] = sum_j exp(s_j - m) v[j][d] / sum_j exp(s_j - m),  m = max_j s_j;
 *   lse[i] = m + log sum_j exp(s_j - m)  (natural log).
 * fp32 arithmetic; the softmax weights are rounded to fp16 for the product with v, and o
 * is rounded to fp16 once.
 *
 * batch, heads      >= 0; the pairs (b, h) are laid out one after another.
 * seq_q, seq_k      query and key/value lengths (>= 0; seq_k >= 1 when there is work).
 * head_dim          64 or 128.
 * q                 device pointer, batch x heads x seq_q x head_dim fp16 (read).
 * k, v              device pointers, batch x heads x seq_k x head_dim fp16 (read).
 * o                 device pointer, batch x heads x seq_q x head_dim fp16 (written); must
 *                   not overlap q, k or v.
 * lse               device pointer to batch x heads x seq_q fp32 (written), or NULL.
 * scale             the score scale (finite, > 0; 1/sqrt(head_dim) is the usual one).
 * causal            0 or 1.
 * stream            hipStream_t to enqueue on; NULL is the default stream.
 *
 * The caller owns every buffer; the call allocates nothing and returns after the
 * enqueue.  batch * heads == 0 or seq_q == 0 does nothing and returns OK.  Errors:
 * EINVAL for negative sizes, seq_k == 0 with work to do (the softmax over no keys is
 * undefined), a scale that is not finite and positive, NULL or misaligned pointers (q, k,
 * v, o need 16-byte alignment, lse 4-byte); EUNSUPPORTED for another head_dim, sizes
 * past the 32-bit offsets the kernel uses ((seq + 1024) * head_dim * 2 bytes must stay
 * below 2^31 per pair) or batch * heads * ceil(seq_q / 256) of 2^31 or more; EHIP if the
 * launch fails.
 */
mi355gemm_status mi355gemm_attention(int64_t batch, int64_t heads, int64_t seq_q, int64_t seq_k,
                                     int64_t head_dim, const void *q, const void *k,
                                     const void *v, void *o, float *lse, float scale,
                                     int causal, void *stream);

/* Description of one compiled kernel configuration. */
typedef struct {
    int block_m, block_n, block_k;  /* macro-tile of C per workgroup and K step */
    int stages;                     /* LDS buffers in the K pipeline */
    int waves_m, waves_n;           /* wavefront grid over the macro-tile */
    int k_groups;                   /* wave grids splitting each K step (summed at the end) */
    int threads;                    /* threads per workgroup:
                                       64 * (waves_m * waves_n * k_groups + loader_waves) */
    int lds_bytes;                  /* LDS the configuration occupies per workgroup */
    int a_vector;                   /* 1: A loaded in 16-byte vectors (needs K % 8 == 0) */
    int bc_vector;                  /* 1: B loaded and C stored in vectors (N % 8 == 0) */
    int group_m;                    /* tile-rows per group in the tile order */
    int direct;                     /* 1: HBM -> LDS copies without register staging */
    int narrow;                     /* 1: vector-ALU kernel for at most block_n (8) columns:
                                       block_m rows per workgroup, k_groups waves on
                                       interleaved block_k-wide k-blocks, no LDS tiles */
    int k_mult8;                    /* 1: needs K % 8 == 0 (A at any 2-byte alignment) */
    int pingpong;                   /* 1: two groups of four waves take turns, one
                                       multiplying while the other loads its next operands
                                       (k_groups 2: the groups take alternate K stages and
                                       sum at the end; 1: each group owns half the rows) */
    int loader_waves;               /* direct kernel: extra waves that issue every HBM -> LDS
                                       copy while the waves_m x waves_n grid only reads LDS
                                       and multiplies (0: the multiplying waves copy too) */
    int mfma_block;                 /* MFMA block edge of the wave tiles: 32
                                       (v_mfma_f32_32x32x16_f16) or 16
                                       (v_mfma_f32_16x16x32_f16); 0 for the narrow kernel */
} mi355gemm_config_desc;

/* Number of compiled configurations (ids 0 .. n-1). Host-only. */
int mi355gemm_num_configs(void);

/* Static name of a configuration, or NULL for an unknown id.  Host-only.  Names read
 * <d|p|s|n><BM>x<BN>x<BK>_w<waves_m>x<waves_n>[k<k_groups>]_...: d = direct HBM -> LDS kernel
 * (suffix [l<loader_waves>_]s<stages>[_mf16], the last for 16x16 MFMA blocks), p = the same loader and tiles with two wave groups taking turns
 * (ping-pong; suffix s<stages>), s = register-staged kernel (suffix av/an: A in 16-byte /
 * 2-byte loads, bv/bn: B and C likewise), n = narrow vector-ALU kernel for N <= 8 (any
 * alignment), e.g. "d128x128x64_w2x2_s4", "d128x128x64_w2x2_l4_s4", "p256x256x32_w2x4_s4",
 * "s64x64x64_w2x1_av_bv", "n8x8x512_w1x1k4".  The tag mirrors the candidate tag of the tutorial's schedule sweep
 * (thecryptopost.io page, section 3: block_M x block_N x block_K with stages and threads). */
const char *mi355gemm_config_name(int config_id);

/* Fill *out for config_id; EINVAL for an unknown id or NULL out. Host-only. */
mi355gemm_status mi355gemm_config_info(int config_id, mi355gemm_config_desc *out);

/* LDS bytes one workgroup may use on gfx950 (the budget every configuration is checked
 * against; 160 KiB). Host-only.  The counterpart of the tutorial's shared-memory budget
 * check, which skips schedules whose (block_M*block_K + block_K*block_N) * 2 * stages bytes
 * exceed the device's capacity (thecryptopost.io page, sections 2 and 3, smem_bytes and
 * SMEM_CAP). */
int mi355gemm_lds_budget(void);

/* Message for the last non-OK status returned on this thread ("" if none). The string
 * stays valid until the next call on the same thread. */
const char *mi355gemm_last_error(void);

/* Library version string. */
const char *mi355gemm_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MI355GEMM_H */
