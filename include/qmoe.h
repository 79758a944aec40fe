/*
 * qmoe.h -- C ABI of the block-quantized MoE expert matmul for MI355X (gfx950).
 *
 * One shared library, libqmoe.so.  Every compute entry point enqueues HIP
 * kernels on the caller's stream and returns; nothing synchronises, nothing
 * allocates, nothing prints, and no C++ exception crosses this boundary.
 * All buffers are owned by the caller.  Pointers documented as DEVICE must
 * point to device memory on the current HIP device; pointers documented as
 * HOST are ordinary host memory.  `stream` is a hipStream_t (NULL = the
 * default stream).
 *
 * Sources (web pages the method is described on):
 *   [GGUF]  "feat(gguf,dsv4): GGUF block-dequant + DSv4 kernel surface (WIP)":
 *           PR body, "Design -- CPU-side decomposition", "Kernels" 1-3, "Next"
 *           item 2, the commit fixing IQ2_XXS sign reconstruction, the
 *           MXFP4 dequant commit ("Format") and the FP8 block dequant
 *           commit (E4M3 bytes, fp32 scale per 128 x 128 block; the fused
 *           FP8 block GEMV named there as the follow-up).
 *   [DSV4]  "metal: DSV4 M1 Ultra prefill/decode campaign": PR body (map0
 *           work queue, 64-slot iq2_xxs tile, q2_K SoA down twin, sum-folded
 *           q2_K down, load-time q2_K SoA repack) and the review-fix commit
 *           (host-checked launcher contracts: <= 1024 experts, topk <= 8; the
 *           AoS q2_K codes start at byte 16 of each 84-byte block).
 *   [BAGEL] "Everything Bagel 2": expert-indexed int4 GEMV (ids read on the
 *           device, [nExperts, outDim, inDim/8] u32 weights + scales + biases),
 *           scalar-FMA top-K accumulate, fused swiglu, caller-owned scratch.
 *   [SHIM]  "WIP: metaltile shim -- Qwen3.6 mt_qmm_mma / mt_moe_gather dispatch
 *           from VLLMBridge": dense qmm and gathered MoE qmm, commit+wait per
 *           dispatch capping the win (so nothing here synchronises).
 *
 * Status codes: every entry point returns one of the QMOE_* codes below.  All
 * argument checks run on the host before any launch.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QMOE_OK              0
#define QMOE_ERR_ARG        -1  /* NULL pointer, negative size, bad enum      */
#define QMOE_ERR_UNSUPPORTED -2 /* format / dtype / epilogue combination      */
#define QMOE_ERR_BLOCK      -3  /* K (or a count) not a multiple of the block */
#define QMOE_ERR_LIMIT      -4  /* topk > 8, experts > 1024, size too large   */
#define QMOE_ERR_WORKSPACE  -5  /* plan / workspace buffer too small          */
#define QMOE_ERR_ALIGN      -6  /* pointer not aligned as documented          */
#define QMOE_ERR_ARCH       -7  /* current device is not gfx950               */
#define QMOE_ERR_LAUNCH     -8  /* HIP reported an error at launch            */

#define QMOE_MAX_EXPERTS 1024
#define QMOE_MAX_TOPK    8
#define QMOE_MAX_GEMV_BATCH 64   /* decode tokens per qmoe_moe_gemv call      */

typedef enum { QMOE_F32 = 0, QMOE_F16 = 1, QMOE_BF16 = 2 } qmoe_dtype;

typedef enum {
  QMOE_Q8_0 = 0,     /* 32-value blocks, one fp16 scale                 [GGUF Kernels 1] */
  QMOE_Q2_K = 1,     /* 256-value super-blocks, 2-bit codes, 4-bit
                        scale/min per 16, fp16 d/dmin                    [GGUF Kernels 2] */
  QMOE_IQ2_XXS = 2,  /* 256-value super-blocks, grid index + 7-bit sign
                        groups with an even-parity 8th sign, 4-bit scale [GGUF Kernels 3] */
  QMOE_INT4 = 3,     /* MLX-style affine int4: s*q + b per group         [BAGEL]          */
  QMOE_MXFP4 = 4,    /* OCP MX FP4: E2M1 codes, E8M0 scale per 32 values [GGUF MXFP4]     */
  QMOE_FP8 = 5,      /* FP8 E4M3 bytes, fp32 scale per 128 x 128 block   [GGUF FP8 block] */
  QMOE_Q4_K = 6,     /* 256-value super-blocks, 4-bit codes, 6-bit scale/min per 32,
                        fp16 d/dmin  (named by [DSV4]; layout read as the GGUF k-quant) */
  QMOE_Q6_K = 7      /* 256-value super-blocks, 6-bit codes, int8 scale per 16, fp16 d
                        (named by [DSV4]; layout read as the GGUF k-quant) */
} qmoe_format;

/* Epilogues of the matmul entry points. */
enum {
  QMOE_EPI_STORE = 0,            /* out[row, n] = y                                  */
  QMOE_EPI_SWIGLU = 1,           /* out[row, j] = silu(y[row, j]) * y[row, N/2 + j]  */
  QMOE_EPI_WEIGHTED_COMBINE = 2, /* out[t, n] += w[t, j] * y[pair (t, j), n]         */
  QMOE_EPI_ACCUMULATE = 3        /* out[row, n] += y  (fp32 out only, dense only)    */
};

/* Router scorings of qmoe_router_topk. */
enum {
  QMOE_ROUTER_SOFTMAX = 0,      /* top-k logits, softmax over the selected; with
                                   a bias: top-k of softmax + bias (LFM2-MoE)     [BAGEL] */
  QMOE_ROUTER_SQRTSOFTPLUS = 1  /* top-k of sqrt(softplus(l)) + bias, weight
                                   sqrt(softplus(l)) * scale (DeepSeek V4)        [GGUF]  */
};

/* Where the activation rows of a gathered MoE matmul come from. */
enum {
  QMOE_A_GATHER_TOKENS = 0,  /* row for pair p is a[p / topk, :]   (a is [t, K])     */
  QMOE_A_SORTED_ROWS = 1     /* row for sorted position i is a[i, :] (a is [P, K])  */
};

/* Which caller-owned buffer qmoe_workspace_bytes sizes. */
enum {
  QMOE_WS_PLAN = 0,        /* the plan buffer of qmoe_moe_plan                   */
  QMOE_WS_COMBINE_ACC = 1  /* the fp32 accumulator [t, n] of a WEIGHTED_COMBINE  */
};

/*
 * A stacked expert weight tensor W[n_experts, n, k] in its GPU-resident split
 * form, as produced from the on-disk blocks by the qmoe_split_* functions
 * ([GGUF] "Design -- CPU-side decomposition"; [DSV4] load-time q2_K SoA
 * repack).  Blocks run along k (the reduction dimension), so y = x . W^T.
 * All pointers are DEVICE pointers, 16-byte aligned; fields a format does not
 * use must be NULL.  Every tiled array covers the stacked rows E*n rounded
 * up to a multiple of 16 (qmoe_split_rows), as the splitters write them.
 *
 *   Q8_0     tiled by qmoe_split_q8_0 (k a multiple of 64);
 *            R, rb, r as below, 64-wide k tile kt:
 *            qs     int8  [R/16][k/64][4][16][16]  chunk c (16 values at
 *                                                64kt + 16c) of row 16rb + r
 *            scales fp16  [R/16][k/32][16]       block scale d of row 16rb + r
 *   Q2_K and IQ2_XXS are tiled by qmoe_split_q2_k / qmoe_split_iq2_xxs
 *   (k a multiple of 256).  Global row
 *   R = e*n + row, block rb = R/16, r = R%16, super-block sb (256 values
 *   along k), SB = k/256, t = rb*SB + sb:
 *   Q2_K     qs     u8    [t][2][16][32]         half h of row r's 64 code bytes
 *                                                (bytes 32h .. 32h+31)
 *            scales u8    [t][16][16]            row r's 16 bytes s: low nibble
 *                                                scale, high nibble min
 *            d,dmin fp16  [t][16]
 *   IQ2_XXS  qs     u32   [t][8][16][2]          group g (32 values) of row r:
 *                                                (4 grid-index bytes, aux word =
 *                                                4 x 7 sign bits (0..27) | scale (28..31))
 *            aux    NULL
 *            d      fp16  [t][16]
 *            grid   u8    [256, 8]               magnitude rows
 *            signs  u8    [128]                  sign masks (qmoe_iq2_signs_table)
 *   Q4_K     value = (d*sc_j)*q - dmin*m_j over 32-value sub-blocks j, tiled by
 *            qmoe_split_q4_k (k a multiple of 256); t, r as for Q2_K:
 *            qs     u8    [t][4][16][32]         quarter h of row r's 128 code bytes
 *                                                (byte i: element 64h+i in the low
 *                                                nibble, 64h+32+i in the high)
 *            scales u8    [t][16][16]            row r's 8 six-bit scales, then its
 *                                                8 six-bit mins, one byte each
 *            d,dmin fp16  [t][16]
 *   Q6_K     value = (d*sc_s)*(q - 32) over 16-value sub-blocks s (q = 6-bit
 *            code), tiled by qmoe_split_q6_k (k a multiple of 256):
 *            qs     u8    [t][4][16][32]         low 4 bits of the codes in the Q4_K
 *                                                code arrangement
 *            aux    u8    [t][2][16][32]         top 2 bits: half h of row r's 64
 *                                                bytes, element 128h + 32p + i at
 *                                                byte i, bits 2p, 2p+1
 *            scales int8  [t][16][16]
 *            d      fp16  [t][16]
 *   INT4     value = s*q + b per group of `group` values along k, tiled by
 *            qmoe_split_int4 (k a multiple of 64 and of group).  Global row R = e*n + row, block rb = R/16,
 *            r = R%16, 64-wide k tile kt:
 *            qs     u32 [R/16][k/64][64 lanes][2]   lane l = 16*g + r holds the 16
 *                   codes of row 16*rb + r at k = 64*kt + 16*g .. +15 as two words;
 *                   word w of those holds element 8w+2i in nibble i and 8w+2i+1
 *                   in nibble 4+i (i = 0..3)
 *            scales u32 [R/16][k/group][16]         (fp16 s) | (fp16 b) << 16 of
 *                   row 16*rb + r and each group
 *            biases NULL
 *            group  32, 64, 128 or 256 (bf16 activations in the prefill matmul:
 *                   64, 128 or 256)
 *   MXFP4    value = e2m1(code) * 2^(e - 127) over 32-value blocks (e = 0xFF:
 *            NaN), tiled by qmoe_split_mxfp4 (k a multiple of 64).  R, rb, r as above, 64-wide k tile kt:
 *            qs     u32 [R/16][k/64][2][16][4]      word w of block j (32 values
 *                   at 64kt + 32j) of row 16rb + r holds the codes of elements
 *                   8w .. 8w+7 of the block: element 8w+i in nibble i (bits
 *                   4i .. 4i+3; the block's code bytes 4w .. 4w+3 as on disk)
 *            scales u8  [R/16][k/32][16]        E8M0 exponent e of each block
 *            group  ignored (32)
 *   FP8      value = e4m3(code) * scale of its 128 x 128 block (E4M3: sign,
 *            4 exponent bits with bias 7, 3 mantissa bits, 0x7F / 0xFF NaN,
 *            largest magnitude 448), the product rounded once in fp32.  n
 *            and k multiples of 128; codes tiled by qmoe_split_fp8:
 *            qs     u8  [R/16][k/64][4][16][16]     chunk c (16 values at
 *                   64kt + 16c) of row 16rb + r (the Q8_0 code tiling)
 *            scales f32 [R/128][k/128]          block scales, the on-disk
 *                   [E][n/128][k/128] array unchanged
 *            group  ignored (128)
 */
typedef struct qmoe_weights {
  int32_t fmt;          /* qmoe_format                                    */
  int32_t n_experts;    /* 1 for a dense weight                           */
  int64_t n;            /* output rows per expert                         */
  int64_t k;            /* reduction length                               */
  int32_t group;        /* INT4 group size along k; ignored otherwise     */
  int32_t reserved;
  const void* qs;
  const void* aux;
  const void* scales;
  const void* biases;
  const void* d;
  const void* dmin;
  const uint8_t* grid;
  const uint8_t* signs;
} qmoe_weights;

/* ------------------------------------------------------------------------
 * Host-side loader split ([GGUF] "Design -- CPU-side decomposition": each
 * on-disk block is decomposed once at load into separate GPU-resident
 * arrays; [DSV4] load-time q2_K SoA repack).  HOST pointers; the caller
 * uploads the outputs.  `aos` holds the on-disk blocks of a rows x k
 * matrix, row after row (rows * k/32 blocks for Q8_0, rows * k/256 for Q2_K
 * and IQ2_XXS).  For a stack of experts, rows = n_experts * n.  Any row count
 * is accepted; the rows of the tiled outputs past `rows` (up to
 * qmoe_split_rows(rows)) are written as zeros and never used:
 *   Q8_0     34 B: fp16 d, 32 int8 codes
 *   Q2_K     84 B: 16 scale|min bytes, 64 code bytes, fp16 d, fp16 dmin
 *   IQ2_XXS  66 B: fp16 d, then 8 x (4 grid-index bytes, u32 aux)
 *   MXFP4    17 B: E8M0 exponent, 16 code bytes (element 2i in the low
 *            nibble of byte i, 2i+1 in its high nibble)  [GGUF MXFP4 "Format"]
 *   Q4_K    144 B: fp16 d, fp16 dmin, 12 bytes of packed six-bit scales and
 *            mins (sub-blocks 0-3: low 6 bits of bytes j and j+4; 4-7: the
 *            nibbles of byte j+8 plus the top 2 bits of bytes j-4 and j), 128
 *            code bytes (element e in byte 32*(e/64) + e%32, low nibble when
 *            e%64 < 32)
 *   Q6_K    210 B: 128 bytes of low nibbles, 64 bytes of top bit pairs, 16
 *            int8 scales, fp16 d (element 128n + 32p + l: low bits in byte
 *            64n + 32(p%2) + l, high nibble when p >= 2; top bits in byte
 *            32n + l at bits 2p, 2p+1)
 *   (the pages only name Q4_K and Q6_K; these are the GGUF k-quant blocks)
 * They come out in the tiled forms above (so that each wave-wide load of
 * the matmul kernels reads contiguous bytes), with R = qmoe_split_rows(rows):
 * Q8_0 qs R*k bytes, scales R*k/32; Q2_K qs R*k/4 bytes, scales R*k/16
 * bytes, d and dmin R*k/256; IQ2_XXS qs R*k/16 u32, d R*k/256; MXFP4 qs
 * R*k/8 u32, e R*k/32 bytes; Q4_K qs R*k/2 bytes, scales R*k/16 bytes, d and
 * dmin R*k/256; Q6_K qs R*k/2 bytes, qh R*k/4 bytes, scales R*k/16, d R*k/256.  Returns QMOE_ERR_ARG on NULL / negative sizes,
 * QMOE_ERR_BLOCK unless k is a multiple of 64 (Q8_0, MXFP4) or 256 (Q2_K,
 * IQ2_XXS, Q4_K, Q6_K).
 * ------------------------------------------------------------------------ */
/* rows rounded up to a multiple of 16: the row count every tiled array of
 * the splitters is sized for (-1 for a negative count). */
int64_t qmoe_split_rows(int64_t rows);
int qmoe_split_q8_0(const void* aos, int64_t rows, int64_t k, int8_t* qs, uint16_t* d);
int qmoe_split_q2_k(const void* aos, int64_t rows, int64_t k, uint32_t* qs, uint8_t* scales,
                    uint16_t* d, uint16_t* dmin);
int qmoe_split_iq2_xxs(const void* aos, int64_t rows, int64_t k, uint32_t* qs, uint16_t* d);
int qmoe_split_mxfp4(const void* aos, int64_t rows, int64_t k, uint32_t* qs, uint8_t* e);
int qmoe_split_q4_k(const void* aos, int64_t rows, int64_t k, uint8_t* qs, uint8_t* scales,
                    uint16_t* d, uint16_t* dmin);
int qmoe_split_q6_k(const void* aos, int64_t rows, int64_t k, uint8_t* qs, uint8_t* qh,
                    int8_t* scales, uint16_t* d);
/* FP8 block weights ([GGUF] FP8 block dequant commit: one E4M3 byte per
 * weight, row-major [rows][k], and one fp32 scale per 128 x 128 block) ->
 * the tiled code array above (rows*k bytes); the scales need no split.
 * QMOE_ERR_BLOCK unless rows and k are multiples of 128. */
int qmoe_split_fp8(const uint8_t* w, int64_t rows, int64_t k, uint8_t* qs);
/* int4 slabs from the on-disk (MLX) form -- words [rows][k/8] with element
 * 8w+i in nibble i of word w, fp16 scales and biases [rows][k/group] -- to the
 * tiled GPU form above: every wave-wide weight load is one contiguous 512-byte
 * block, and one mask-and-or yields two consecutive elements in the two halves
 * of a 32-bit register.  qs_out holds R*k/8 words, sb_out R*k/group (R =
 * qmoe_split_rows(rows), zero rows past `rows`).  QMOE_ERR_BLOCK unless
 * k % 64 == 0 and k % group == 0. */
int qmoe_split_int4(const uint32_t* words, const uint16_t* scales, const uint16_t* biases,
                    int64_t rows, int64_t k, int32_t group, uint32_t* qs_out, uint32_t* sb_out);
/* The 128-entry IQ2_XXS sign-mask table ([GGUF] sign-fix commit): entry i is
 * the 7 stored sign bits plus an 8th bit making the count of negated values
 * even.  HOST pointer to 128 bytes. */
void qmoe_iq2_signs_table(uint8_t out[128]);

/* ------------------------------------------------------------------------
 * Standalone dequantisation ([GGUF] "Kernels" 1-3 and the MXFP4 dequant
 * commit; [BAGEL] int4 slabs).
 * Decodes every value in fp32 exactly as the format defines it and rounds
 * once (to nearest even) to out_dtype; results are bit-exact.  DEVICE
 * pointers, 16-byte aligned; the inputs are the splitters' tiled arrays for
 * `rows` rows (any count), out holds the rows x k matrix, row-major.
 * QMOE_ERR_BLOCK unless k is a multiple of 64 (Q8_0, MXFP4), 256 (Q2_K,
 * IQ2_XXS) or 64 and group (int4).  MXFP4 values past the fp32 range
 * (e = 254, |code value| >= 2) come out as +-inf, e = 0xFF as NaN.
 * ------------------------------------------------------------------------ */
int qmoe_dequant_q8_0(const int8_t* qs, const uint16_t* d, int64_t rows, int64_t k,
                      void* out, int32_t out_dtype, void* stream);
int qmoe_dequant_q2_k(const uint32_t* qs, const uint8_t* scales, const uint16_t* d,
                      const uint16_t* dmin, int64_t rows, int64_t k,
                      void* out, int32_t out_dtype, void* stream);
int qmoe_dequant_iq2_xxs(const uint32_t* qs, const uint16_t* d, const uint8_t* grid,
                         const uint8_t* signs, int64_t rows, int64_t k,
                         void* out, int32_t out_dtype, void* stream);
/* Q4_K / Q6_K (k a multiple of 256): the tiled arrays of qmoe_split_q4_k /
 * qmoe_split_q6_k.  Q4_K values round once (the subtraction), Q6_K once (the
 * product of d*scale with q - 32). */
int qmoe_dequant_q4_k(const uint8_t* qs, const uint8_t* scales, const uint16_t* d,
                      const uint16_t* dmin, int64_t rows, int64_t k,
                      void* out, int32_t out_dtype, void* stream);
int qmoe_dequant_q6_k(const uint8_t* qs, const uint8_t* qh, const int8_t* scales,
                      const uint16_t* d, int64_t rows, int64_t k,
                      void* out, int32_t out_dtype, void* stream);
int qmoe_dequant_int4(const uint32_t* qs, const uint32_t* sb, int64_t rows, int64_t k,
                      int32_t group, void* out, int32_t out_dtype, void* stream);
int qmoe_dequant_mxfp4(const uint32_t* qs, const uint8_t* e, int64_t rows, int64_t k,
                       void* out, int32_t out_dtype, void* stream);
/* FP8 block weights ([GGUF] FP8 block dequant commit): qs tiled as in
 * qmoe_weights, scales fp32 [rows/128][k/128]; rows and k multiples of 128
 * (else QMOE_ERR_BLOCK).  0x7F / 0xFF decode to NaN. */
int qmoe_dequant_fp8(const uint8_t* qs, const float* scales, int64_t rows, int64_t k,
                     void* out, int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Dense quantised matmul ([SHIM] mt_qmm_mma; [DSV4] wide-tile q8_0 qgemm):
 * y[m, n] = sum_k x[m, k] * W[0, n, k], fp32 accumulation.
 *   x      DEVICE [m, k] act_dtype (QMOE_F16 or QMOE_BF16), rows contiguous
 *   out    DEVICE; STORE: [m, n] out_dtype; SWIGLU: [m, n/2] out_dtype;
 *          ACCUMULATE: fp32 [m, n], y is added to it
 * Any n >= 1 is accepted (the split arrays are padded to whole 16-row
 * blocks; tail columns are masked in the kernel), except FP8, whose n is a
 * multiple of its 128-row scale block (else QMOE_ERR_BLOCK), and SWIGLU,
 * which needs an even n (QMOE_ERR_ARG).  k is a multiple of 64 and of the
 * format's block (QMOE_ERR_BLOCK).  w->n_experts must be 1.  m = 0 returns
 * QMOE_OK without launching.
 * ------------------------------------------------------------------------ */
int qmoe_qmm_dense(const qmoe_weights* w, const void* x, int32_t act_dtype, int64_t m,
                   int32_t epilogue, void* out, int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Routing plan: the expert-sorted token gather with per-expert tiles ([DSV4]
 * map0 work queue feeding tiles of routed tokens to the MoE GEMM; [BAGEL]
 * ids stay on the device).
 *
 * ids DEVICE int32 [t, topk]; pair p = row * topk + j.  Pairs with an id
 * outside [0, n_experts) are dropped and counted.  Within an expert, pairs
 * keep ascending pair order; each expert's run is cut into tiles of at most
 * `bm` rows (bm a multiple of 16 from 16 to 128, else QMOE_ERR_ARG; above
 * the matmul's 80-row register tile QMOE_ERR_UNSUPPORTED).  The plan is
 * unique.  The buffer is the call's only scratch: qmoe_plan_bytes (or
 * qmoe_workspace_bytes(QMOE_WS_PLAN, ...)) gives its size.
 *
 * Layout of the DEVICE int32 plan buffer (size from qmoe_plan_bytes):
 *   [0] dropped  [1] n_tiles  [2] n_valid  [3] bm  [4] t  [5] topk  [6] n_experts
 *   [7] 512 when the buffer carries a work-balancing area, else 0
 *   counts [n_experts] | offsets [n_experts + 1] | sorted pair ids [t * topk]
 *   | tiles [max_tiles][4] = (expert, row0, nrows, 0), the full tiles (bm
 *   rows) in expert order, then the experts' partial last tiles in expert
 *   order | sorted position of each pair, -1 if dropped [t * topk] |
 *   scratch | (plans of t * topk >= 2048 pairs, from the next multiple of
 *   64 words) the work-balancing area of the ring gathered matmul: 512
 *   int32 tickets (zeroed by the plan build, left at zero by every matmul
 *   call) and 512 fp32 partial tiles of 80 x 256 values (about 40 MiB).
 *   max_tiles is
 *   min(t*topk, n_experts) + t*topk/16 (the tile array fits any bm); the
 *   sorted list starts at word 8 + 2*n_experts + 1 and the tile array at the
 *   next multiple of 4 words after it.
 * ------------------------------------------------------------------------ */
size_t qmoe_plan_bytes(int64_t t, int32_t topk, int32_t n_experts, int32_t bm);
int qmoe_moe_plan(const int32_t* ids, int64_t t, int32_t topk, int32_t n_experts, int32_t bm,
                  int32_t* plan, size_t plan_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Gathered MoE matmul over a plan ([SHIM] mt_moe_gather_qmm; [DSV4] tiled
 * MoE prefill GEMM with the iq2_xxs gate/up tile and the q2_K down twin).
 * For sorted position i holding pair p = plan.sorted[i] with expert e:
 *   y[i, n] = sum_k A_i[k] * W[e, n, k]
 * where A_i = a[p / topk] (GATHER_TOKENS, a is [t, K]) or a[i] (SORTED_ROWS,
 * a is [n_valid, K]).  Epilogues:
 *   STORE             out [n_valid, N] out_dtype, sorted order
 *   SWIGLU            out [n_valid, N/2] out_dtype, sorted order; gate = rows
 *                     0..N/2-1 of W, up = rows N/2..N-1
 *   WEIGHTED_COMBINE  out fp32 [t, N]: out[p / topk, n] += topk_w[p] * y[i, n]
 *                     by float atomics (order-dependent rounding); topk_w is
 *                     DEVICE fp32 [t, topk].  Finish with qmoe_combine_cast.
 * a, out DEVICE; the plan must come from qmoe_moe_plan with the same t, topk,
 * bm and n_experts == w->n_experts: the kernels read its header (words 3..6)
 * and a plan that names another call gives no tiles (out is left as it
 * was).  Matmul entry points need k to be a multiple of 64 and of the
 * format's block; any n (as qmoe_qmm_dense).  Determinism is chosen by entry
 * point rather than a flag: STORE + qmoe_moe_combine is bit-reproducible,
 * WEIGHTED_COMBINE (atomics) is not.
 * int4 weights, and weights of every other format with fp16 activations (N
 * a multiple of 16, of 32 with SwiGLU), on a plan with a work-balancing area:
 * when an XCD's (tile, column block) units fill its resident workgroups'
 * rounds plus a short last
 * round, those last units are split into 4 parts along K that meet through
 * the plan's area (fp32 partial sums added in part order, so the result is
 * the same on every run on the same device; it can differ in the last bits
 * from an unsplit evaluation).  The call writes the plan's area: two such
 * gathered matmuls that share one plan must not run at the same time.
 * ------------------------------------------------------------------------ */
int qmoe_moe_gather_qmm(const qmoe_weights* w, const int32_t* plan, int64_t t, int32_t topk,
                        int32_t bm, const void* a, int32_t act_dtype, int32_t a_mode,
                        const float* topk_w, int32_t epilogue,
                        void* out, int32_t out_dtype, void* stream);

/* Deterministic combine ([BAGEL] scalar-FMA top-K accumulate):
 * out[t, n] = (base ? base[t, n] : 0) + sum_j topk_w[t, j] * y[pos(t, j), n],
 * j ascending, fp32, one rounding to out_dtype.  y DEVICE [n_valid, N] in
 * y_dtype (sorted order, e.g. a STORE result); base DEVICE fp32 [t, N] or
 * NULL; dropped pairs contribute nothing.  A plan whose header names other
 * (t, topk, n_experts) makes the kernel write nothing. */
int qmoe_moe_combine(const void* y, int32_t y_dtype, const int32_t* plan, int64_t t,
                     int32_t topk, int32_t n_experts, const float* topk_w, int64_t n, const float* base,
                     void* out, int32_t out_dtype, void* stream);

/* Combine with a gated shared expert and the residual add ([BAGEL] the
 * sigmoid-gated scalar FMA with the post-MoE residual add folded in, used to
 * accumulate the top-K expert outputs):
 *   out[t, n] = residual[t, n] + g_t * shared[t, n]
 *               + sum_j topk_w[t, j] * y[pos(t, j), n],
 *   g_t = 1 / (1 + exp(-shared_gate[t]))  (g_t = 1 when shared_gate is NULL).
 * fp32: the shared term first, then the pairs in ascending j, then the
 * residual; one rounding to out_dtype.  shared DEVICE fp32 [t, N] or NULL (no
 * shared term; shared_gate must then be NULL); shared_gate DEVICE fp32 [t]
 * logits or NULL; residual DEVICE [t, N] in residual_dtype or NULL, 16-byte
 * aligned.  out may be the residual buffer itself when the dtypes agree (the
 * update is then in place); any other overlap of out and residual is
 * QMOE_ERR_ARG.  Other arguments and errors as qmoe_moe_combine. */
int qmoe_moe_combine_shared(const void* y, int32_t y_dtype, const int32_t* plan, int64_t t,
                            int32_t topk, int32_t n_experts, const float* topk_w, int64_t n,
                            const float* shared, const float* shared_gate, const void* residual,
                            int32_t residual_dtype, void* out, int32_t out_dtype, void* stream);

/* out = RNE(acc) for n_elems values, then acc = 0 (so the fp32 accumulator
 * of a WEIGHTED_COMBINE is ready for the next call).  DEVICE pointers. */
int qmoe_combine_cast(float* acc, int64_t n_elems, void* out, int32_t out_dtype, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: the
 * WEIGHTED_COMBINE gathered matmul followed by the cast, as
 *   qmoe_moe_gather_qmm(..., QMOE_EPI_WEIGHTED_COMBINE, acc, QMOE_F32) then
 *   qmoe_combine_cast(acc, t * w->n, out, out_dtype),
 * but with the fp32 accumulator acc in a fixed array inside the library
 * (qmoe_static_acc_bytes() bytes, 32 MiB, held on each GPU the library runs
 * on until the process ends) instead of a caller buffer.  Arguments as
 * qmoe_moe_gather_qmm; out DEVICE [t, w->n] in out_dtype (F32 / F16 / BF16),
 * 16-byte aligned.  The call clears the accumulator first (a kernel, no
 * memset), so no earlier call's contents matter; it allocates nothing.
 * QMOE_ERR_WORKSPACE when t * w->n * 4 exceeds qmoe_static_acc_bytes().  All
 * calls on one GPU share its array: calls that overlap on one GPU (other
 * streams, other threads) race and give wrong results. */
int qmoe_moe_gather_qmm_combine_static(const qmoe_weights* w, const int32_t* plan, int64_t t, int32_t topk,
                                       int32_t bm, const void* a, int32_t act_dtype, int32_t a_mode,
                                       const float* topk_w, void* out, int32_t out_dtype, void* stream);
/* Size in bytes of the fixed accumulator of qmoe_moe_gather_qmm_combine_static. */
size_t qmoe_static_acc_bytes(void);

/* ------------------------------------------------------------------------
 * Decode GEMV ([BAGEL] expert-indexed int4 GEMV reading expert ids on the
 * device; [DSV4] small-batch qgemv and the sum-folded q2_K down projection).
 * ids DEVICE int32 [b, topk] (entries outside [0, E) contribute nothing);
 * b <= QMOE_MAX_GEMV_BATCH.  Each expert's weights are read once per call.
 *   STORE             a = x [b, K];           out [b, topk, N]    = x_b . W[e]^T
 *   SWIGLU            a = x [b, K];           out [b, topk, N/2]  = silu(g) * u
 *   WEIGHTED_COMBINE  a = h [b, topk, K];     out [b, N] = sum_j topk_w[b, j] *
 *                     (h[b, j] . W[ids[b, j]]^T), j ascending, deterministic
 * a, out, topk_w DEVICE.  K a multiple of 32 (QMOE_ERR_BLOCK) and at most
 * 8192 (QMOE_ERR_LIMIT); any N.  On int4 with group >= 64, K <= 4096 with
 * K/32 a power of two, N a multiple of 16 (32 for SWIGLU) and, for
 * WEIGHTED_COMBINE, topk * ceil(K / 512) <= 16, the tiled matrix-core
 * kernels run; every other call takes the generic kernels.
 * ------------------------------------------------------------------------ */
int qmoe_moe_gemv(const qmoe_weights* w, const void* a, int32_t act_dtype, int64_t b,
                  const int32_t* ids, const float* topk_w, int32_t topk, int32_t epilogue,
                  void* out, int32_t out_dtype, void* stream);

/* ------------------------------------------------------------------------
 * Router top-k: expert ids and gather weights from router logits, on the
 * device, so the ids feed qmoe_moe_plan / qmoe_moe_gemv with no host
 * round trip ([BAGEL] the commit moving the MoE router top-K to the GPU;
 * [GGUF] the DeepSeek V4 sqrtsoftplus routing scoring commit).
 *   logits DEVICE [t, n_experts] row-major, logits_dtype F32 / F16 / BF16
 *          (aligned to its element size).
 *   SOFTMAX        bias NULL: selects the topk largest logits; weights[t, j]
 *                  = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected
 *                  (they sum to 1).  With a bias (DEVICE f32 [n_experts],
 *                  the LFM2-MoE softmax-then-bias routing): p = softmax of
 *                  the row over all experts in fp32, selects the topk largest
 *                  p_e + bias[e], weights = the selected p / their sum.  scale
 *                  must be 1.
 *   SQRTSOFTPLUS   s_e = sqrt(max(l, 0) + log1p(exp(-|l|))) in fp32; selects
 *                  the topk largest s_e + bias[e] (bias DEVICE f32
 *                  [n_experts], or NULL for zero); weights = s_e * scale
 *                  (no renormalisation).
 *   ids DEVICE int32 [t, topk], weights DEVICE f32 [t, topk], written in
 *   selection order (best first).  Equal selection scores go to the lower
 *   expert index; NaN scores rank below every number, -0 equals +0.
 * A NaN logit in a row makes that row's softmax weights NaN when it is
 * selected (no bias) or always (bias).
 * Errors: QMOE_ERR_ARG (NULL pointer, t < 0, topk < 1 or > n_experts, bad
 * dtype / scoring, SOFTMAX with scale != 1), QMOE_ERR_LIMIT
 * (topk > QMOE_MAX_TOPK, n_experts > QMOE_MAX_EXPERTS, t > 2^31),
 * QMOE_ERR_ALIGN; nothing is launched on error.  t == 0 launches nothing.
 * ------------------------------------------------------------------------ */
int qmoe_router_topk(const void* logits, int32_t logits_dtype, int64_t t, int32_t n_experts,
                     int32_t topk, int32_t scoring, const float* bias, float scale,
                     int32_t* ids, float* weights, void* stream);

/* Bytes of the caller-owned buffer `what` names (QMOE_WS_*), or 0 on a bad
 * argument:
 *   QMOE_WS_PLAN         the plan buffer of qmoe_moe_plan for t tokens, topk
 *                        and w->n_experts experts (= qmoe_plan_bytes);
 *   QMOE_WS_COMBINE_ACC  the fp32 [t, w->n] accumulator a WEIGHTED_COMBINE
 *                        gathered matmul adds into.
 * No other entry point needs scratch: dense qmm, STORE / SWIGLU matmuls,
 * the combines, the GEMV and the router use only their inputs and outputs. */
size_t qmoe_workspace_bytes(int32_t what, const qmoe_weights* w, int64_t t, int32_t topk, int32_t bm);

/* QMOE_OK if the current HIP device is gfx950, else QMOE_ERR_ARCH. */
int qmoe_check_device(void);
/* Static description of a status code. */
const char* qmoe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* QMOE_H */
