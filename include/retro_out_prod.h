/*
 * retro_out_prod.h - C ABI of the MI355X (gfx950) OUT_PROD library.
 *
 * OUT_PROD through a resident block-quantized weight:
 *
 *     dst[t][k] = sum_{n=0}^{N-1} W[n][k] * G[t][n]
 *
 * It gives the gradient of mul_mat(W, x) with respect to its input x: an
 * OUT_PROD of W with the transposed output gradient (llama.cpp PR #3 "cuda:
 * out_prod accepts a quantized src0", commit message). The PR admits a contiguous
 * quantized, F16 or BF16 src0 with F32 src1 and dst (section "What"); the
 * Retrograd CUDA status page lists OUT_PROD for F32, F16, BF16 and quantized
 * types (section "What works on the GPU"). W[n][k] is the value the stored
 * block decodes to.
 *
 * Layouts (all row-major and contiguous; the caller owns every buffer):
 *   W    N rows; row n starts at byte n * retro_row_bytes(type, K) and holds
 *        K elements along k as consecutive blocks of the given type.
 *   G    T x N float32 (the gradient in its natural layout; the transposition
 *        of grad^T is implied by the indexing).
 *   dst  T x K float32, overwritten (never read, never accumulated into).
 * Block formats (GGUF; fp16 fields little-endian):
 *   RETRO_F32   4 bytes per element
 *   RETRO_F16   2 bytes per element (IEEE binary16)
 *   RETRO_BF16  2 bytes per element (upper half of a binary32)
 *   RETRO_Q8_0  34 bytes / 32 elements: fp16 d, 32 int8 q; value d*q
 *   RETRO_Q4_0  18 bytes / 32 elements: fp16 d, 16 bytes of nibbles; element
 *               j<16 = low nibble of byte j, j+16 = its high nibble;
 *               value d*(q-8)
 *   RETRO_Q4_1  20 bytes / 32 elements: fp16 d, fp16 m, nibbles as Q4_0;
 *               value d*q + m
 *   RETRO_Q5_0  22 bytes / 32 elements: fp16 d, 32-bit qh (little-endian),
 *               nibbles as Q4_0; bit j of qh is element j's fifth bit;
 *               value d*(q-16)
 *   RETRO_Q5_1  24 bytes / 32 elements: fp16 d, fp16 m, qh, nibbles as
 *               Q5_0; value d*q + m
 *   RETRO_MXFP4 17 bytes / 32 elements: E8M0 scale byte e, 16 bytes of
 *               E2M1 codes in the Q4_0 nibble order (OCP Microscaling:
 *               sign, 2-bit exponent, 1-bit mantissa); value
 *               e2m1(q) * 2^(e-127), e = 255 NaN; blocks only byte-aligned
 *   RETRO_NVFP4 36 bytes / 64 elements: four FP8 E4M3 scale bytes (one per
 *               16-element sub-block: sign, 4-bit exponent with bias 7,
 *               3-bit mantissa; subnormals m * 2^-9, 0x7F/0xFF NaN), then 32
 *               bytes of E2M1 codes, 8 per sub-block: element 16s + i (i < 8)
 *               = low nibble of code byte 8s + i, 16s + 8 + i its high
 *               nibble; value e2m1(q) * scale_s. NVIDIA's NVFP4 element and
 *               scale encodings; the block layout is this library's reading
 *               (the format's per-tensor F32 scale lies outside the blocks:
 *               a caller applies it to G or dst)
 *   RETRO_Q4_K  144 bytes / 256 elements: fp16 d, fp16 dmin, 12 bytes of
 *               eight 6-bit sub-scales sc_j and sub-mins m_j (GGUF packing),
 *               128 bytes of nibbles (each 64-element chunk c uses 32 bytes:
 *               low nibbles are sub-block 2c, high nibbles sub-block 2c+1);
 *               value (d*sc_j)*q - dmin*m_j
 *   RETRO_Q5_K  176 bytes / 256 elements: fp16 d, fp16 dmin, the Q4_K 12-byte
 *               field, 32 bytes qh, 128 bytes of nibbles as Q4_K; element
 *               r of chunk c (r < 32: low nibble, else high) takes bit 2c
 *               (2c+1) of qh[r % 32] as its fifth bit; value as Q4_K
 *   RETRO_Q6_K  210 bytes / 256 elements: 128 bytes of low nibbles, 64 bytes
 *               of 2-bit high parts, 16 int8 sub-scales, fp16 d; element
 *               128h + 32p + l: nibble of byte 64h + 32(p%2) + l (high
 *               nibble for p >= 2), bits 2p..2p+1 of byte 128 + 32h + l,
 *               sub-scale 8h + 2p + l/16; value (d*sc)*(q-32)
 *   RETRO_Q2_K  84 bytes / 256 elements: 16 pair bytes (4-bit sub-scale | 4-bit
 *               sub-min << 4), 64 bytes of 2-bit codes, fp16 d, fp16 dmin;
 *               element 128h + 32p + l: bits 2p..2p+1 of byte 16 + 32h + l,
 *               pair 8h + 2p + l/16; value (d*sc)*q - dmin*m
 *   RETRO_Q3_K  110 bytes / 256 elements: 32 bytes hmask, 64 bytes of 2-bit
 *               codes, 12 bytes of sixteen 6-bit sub-scales, fp16 d; element
 *               128h + 32p + l: bits 2p..2p+1 of byte 32 + 32h + l, minus 4
 *               unless bit 4h+p of hmask[l] is set, sub-scale 8h + 2p + l/16
 *               (stored with +32); value (d*(sc-32))*q
 * The Q4_1, Q5_0, Q5_1, MXFP4, Q2_K, Q3_K, Q5_K and Q6_K layouts are the GGUF ones:
 * the pages that define this operation name them only as members of the
 * quantized types it admits (and the K-quant family through the Q4_K_M files
 * it runs on).
 *
 * Pointers: W, G and dst are device pointers (hipMalloc'd or equivalent) and
 * must be 16-byte aligned. dst must not overlap W or G. stream is a
 * hipStream_t passed as void* (NULL = the null stream).
 *
 * Execution: every compute call is asynchronous on the stream, allocates no
 * memory (no dequantized copy of W exists at any size, so the scratch
 * budget of the prior sliced design - Retrograd CUDA status, sections
 * "Building" and "Limitations" - is zero) and never falls back to the CPU:
 * an unsupported call returns an error. The library's only mutable state is
 * a small per-thread (thread-local) cache of recent launch plans; calls are
 * thread-safe.
 *
 * Errors: functions returning int return RETRO_OK (0) or a negative code;
 * nothing throws across the ABI; retro_strerror names a code.
 */
#ifndef RETRO_OUT_PROD_H
#define RETRO_OUT_PROD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Weight types: the GGUF tensor-type ids. */
enum {
    RETRO_F32 = 0,
    RETRO_F16 = 1,
    RETRO_Q4_0 = 2,
    RETRO_Q4_1 = 3,
    RETRO_Q5_0 = 6,
    RETRO_Q5_1 = 7,
    RETRO_Q8_0 = 8,
    RETRO_Q2_K = 10,
    RETRO_Q3_K = 11,
    RETRO_Q4_K = 12,
    RETRO_Q5_K = 13,
    RETRO_Q6_K = 14,
    RETRO_BF16 = 30,
    RETRO_MXFP4 = 39,
    RETRO_NVFP4 = 40
};

/* Error codes. */
enum {
    RETRO_OK = 0,
    RETRO_E_TYPE = -1,  /* unknown or unsupported weight type */
    RETRO_E_SHAPE = -2, /* negative size, K not a whole number of blocks, or a
                           size whose byte count overflows the limits below */
    RETRO_E_NULL = -3,  /* NULL buffer where the call would touch memory */
    RETRO_E_ALIGN = -4, /* W, G or dst not 16-byte aligned */
    RETRO_E_ALIAS = -5, /* dst overlaps W or G */
    RETRO_E_HIP = -6,   /* the HIP runtime reported an error at launch */
    RETRO_E_VARIANT = -7, /* retro_out_prod_variant: variant unknown or not
                             applicable to this type/shape */
    RETRO_E_WORKSPACE = -8 /* retro_out_prod_ws: a forced variant needs a
                              workspace that is missing, too small, not
                              16-byte aligned or overlapping W, G or dst */
};

/* Size limits: K, N and T are each below 2^31, T*K and T*N below 2^60, and
 * N*retro_row_bytes(type, K) below 2^62 (retro_dequantize: N*K below 2^60). */

/*
 * dst[t][k] = sum_n W[n][k] * G[t][n] for t < T, k < K.
 *   type    one of RETRO_F32/F16/BF16/Q8_0/Q4_0/Q4_1/Q5_0/Q5_1/MXFP4/NVFP4/Q2_K/Q3_K/Q4_K/Q5_K/Q6_K
 *   W       device, N * retro_row_bytes(type, K) bytes
 *   G       device, T * N floats
 *   dst     device, T * K floats, overwritten
 *   K       elements per W row (a multiple of the block: 32 for Q8_0, Q4_0,
 *           Q4_1, Q5_0, Q5_1 and MXFP4, 64 for NVFP4, 256 for the K-quants
 *           Q2_K..Q6_K, 1 otherwise)
 *   N       rows of W = the reduction length
 *   T       rows of G and dst
 * T == 0 or K == 0: returns RETRO_OK without touching memory (pointers may
 * be NULL). N == 0: dst is filled with zeros (the empty sum).
 * Returns RETRO_OK once the kernel is enqueued; a launch failure reported by
 * HIP returns RETRO_E_HIP.
 */
int retro_out_prod(int type, const void *W, const float *G, float *dst, int64_t K, int64_t N,
                   int64_t T, void *stream);

/*
 * Decode W to float32: out[n][k] = W[n][k], out is N x K floats (device,
 * 16-byte aligned, must not overlap W). The conversion the PR's converters
 * perform (section "What": dequantize through the converters mul_mat
 * already uses), exposed so that decoded values can be checked bit for bit.
 * Every value is the format's formula above evaluated in IEEE float32 in the
 * order written there, bit for bit: the sign of a zero, subnormal scales and
 * results, infinities (a scale of +-inf gives +-inf, or NaN where the formula
 * meets inf*0 or inf-inf) and NaN included; NaN payloads are unspecified.
 * The fused kernels of retro_out_prod decode with the same device functions.
 * K == 0 or N == 0: RETRO_OK, nothing touched.
 */
int retro_dequantize(int type, const void *W, float *out, int64_t K, int64_t N, void *stream);

/*
 * 1 if retro_out_prod(type, ..., K, N, T) with valid, aligned, non-aliasing
 * buffers would run, 0 otherwise (the analogue of the PR's supports_op rule,
 * section "What": any contiguous src0 with an F32 converter, src1 and dst
 * F32). Touches no device.
 */
int retro_out_prod_supported(int type, int64_t K, int64_t N, int64_t T);

/* Bytes per W row, from the block formats above (the PR's OUT_PROD reads
 * src0 as whole rows of blocks, section "What"): K/32*34 (Q8_0), K/32*18
 * (Q4_0), K/32*20 (Q4_1), K/32*22 (Q5_0), K/32*24 (Q5_1), K/32*17 (MXFP4),
 * K/64*36 (NVFP4), K/256*84 (Q2_K), K/256*110 (Q3_K), K/256*144 (Q4_K), K/256*176 (Q5_K),
 * K/256*210 (Q6_K), 4K (F32), 2K (F16, BF16). -1 for an unknown type, a
 * negative K or a K that is not a whole number of blocks. Touches no
 * device. */
int64_t retro_row_bytes(int type, int64_t K);

/* A static, NUL-terminated description of an error code (never NULL): an
 * unsupported call is reported, never run elsewhere (where the Retrograd
 * CUDA status page's runtime falls back to the CPU, section "What works on
 * the GPU"). */
const char *retro_strerror(int code);

/*
 * Kernel variants (for tests and benchmarks; retro_out_prod chooses one):
 *   RETRO_VARIANT_AUTO      what retro_out_prod runs (one variant, or two over
 *                           column ranges of dst: retro_out_prod_plan)
 *   RETRO_VARIANT_SKINNY    one pass over W per 64 rows of G, all of n per
 *                           workgroup, each decoded weight feeding one MFMA
 *                           per block of 16 rows of G (8 or 16 waves per
 *                           workgroup up to T = 16, chosen by type and T,
 *                           and 8 above; the two are summed in different
 *                           orders). retro_out_prod runs it for T <= 16, and
 *                           above where its estimate beats the tiles' (with
 *                           few tiles per CU; by 10% past one pass)
 *   RETRO_VARIANT_SKINNY_8, RETRO_VARIANT_SKINNY_16  the skinny kernel with
 *                           that many waves per workgroup (16: T <= 16)
 *   RETRO_VARIANT_SKINNY_SPLIT  retro_out_prod_ws only: the skinny kernel's
 *                           groups of 16 W rows, all slabs of 64 dst columns
 *                           in turn, cut into one equal share per CU, the
 *                           parts of a slab added through a workspace (see
 *                           retro_out_prod_ws), one pass over W per 48
 *                           rows of G. N % 16 == 0, K % 4 == 0, G rows in
 *                           16-byte units, one matrix
 *   RETRO_VARIANT_TILE_*    tiled F32-MFMA kernel, tile = rows of T x columns
 *                           of K per workgroup (256-column tiles need K tiles
 *                           that are whole K-quant super-blocks; the K-quants
 *                           take only
 *                           those)
 *   RETRO_VARIANT_WS_*      the same tiles computed by a workgroup whose
 *                           waves are split into MFMA (consumer) and load/
 *                           decode (producer) roles over double-buffered LDS;
 *                           needs G rows (or, stored t-fastest, columns) in
 *                           16-byte units (ldg % 4 == 0; ldg = N when
 *                           contiguous) and K % 4 == 0 for F32, F16, BF16;
 *                           the TILE_* kernel takes the others
 *   RETRO_VARIANT_SIMPLE    retro_mul_mat only: one thread per output, for
 *                           the shapes the tiled kernel refuses
 *   RETRO_VARIANT_WS_256x256  the 256 x 256 tile: eight MFMA waves (each
 *                           the 64 x 128 block of WS_128x256's) share one set
 *                           of four producer waves, so every decoded weight
 *                           feeds twice as many products; 144 KB of LDS, one
 *                           workgroup of 12 waves per CU
 *   RETRO_VARIANT_WS_256x128  retro_mul_mat only: 256 rows of x by 128 rows
 *                           of W per workgroup, eight MFMA waves (64 x 64
 *                           each) over one set of four producer waves
 *   RETRO_VARIANT_WS2_64x128  WS_64x128 with two pipelines in one
 *                           workgroup (even and odd 32-row chunks of W,
 *                           partial sums added in LDS in that order): two
 *                           MFMA waves per SIMD for shapes with about one
 *                           tile per CU
 *   RETRO_VARIANT_SPLIT_128x256  the K-quants (Q2_K .. Q6_K) only, never
 *                           chosen automatically: the 128 x 256 producer/
 *                           consumer tile on bf16 MFMA with exact operands.
 *                           Per super-block the sum is taken as
 *                           sum_n fl(G*d) * v minus (Q2_K, Q4_K, Q5_K)
 *                           sum_n fl(G*dmin) * m, v the integer product of
 *                           sub-block scale and code (sc*q, sc*(q - 32) for
 *                           Q6_K, (sc - 32)*q for Q3_K), every
 *                           factor cut into bf16 parts that add up to it
 *                           exactly, so every product is exact and every sum
 *                           is F32; the result differs from the F32-input
 *                           kernels by the roundings of G*d (and G*dmin) and
 *                           by the matrix core's F32 addition (it truncates).
 *                           Within the same error bars (tests), 1.7x to 2.7x
 *                           the rate. G by rows with ldg % 4 == 0.
 *   RETRO_VARIANT_SPLIT_128x128  the same form on a 128 x 128 tile for Q4_0,
 *                           Q5_0, MXFP4, BF16 and F16, never chosen
 *                           automatically: the decoded weight v (d (q - 8),
 *                           d (q - 16), the E2M1 value times its scale, or
 *                           the weight itself) is exact in F32 with at most
 *                           16 significant bits, so it is cut into one bf16
 *                           part (BF16, MXFP4) or two, and G itself into
 *                           three. G by rows with ldg % 4 == 0; BF16 and F16
 *                           rows 16-byte aligned (row pitch % 16 == 0).
 *   Both SPLIT variants take finite weights and gradients: an infinite weight
 *   meets the zero parts of the other operand (inf * 0) and gives NaN where
 *   the F32-input kernels give +-inf. Subnormal values are exact.
 */
enum {
    RETRO_VARIANT_AUTO = 0,
    RETRO_VARIANT_SKINNY = 1,
    RETRO_VARIANT_TILE_128x128 = 2,
    RETRO_VARIANT_TILE_128x256 = 3,
    RETRO_VARIANT_TILE_64x128 = 4,
    RETRO_VARIANT_TILE_64x64 = 5,
    RETRO_VARIANT_TILE_64x256 = 6,
    RETRO_VARIANT_WS_128x256 = 7,
    RETRO_VARIANT_WS_64x256 = 8,
    RETRO_VARIANT_WS_128x128 = 9,
    RETRO_VARIANT_WS_64x128 = 10,
    RETRO_VARIANT_WS_32x256 = 11,
    RETRO_VARIANT_WS_32x128 = 12,
    RETRO_VARIANT_WS2_64x128 = 13,
    RETRO_VARIANT_SIMPLE = 15,
    RETRO_VARIANT_SPLIT_128x256 = 16,
    RETRO_VARIANT_SPLIT_128x128 = 17,
    RETRO_VARIANT_WS_256x256 = 18,
    RETRO_VARIANT_WS_256x128 = 19,
    RETRO_VARIANT_SKINNY_8 = 20,
    RETRO_VARIANT_SKINNY_16 = 21,
    RETRO_VARIANT_SKINNY_SPLIT = 22
};

/* retro_out_prod with a forced kernel variant; RETRO_E_VARIANT when the
 * variant does not apply to the type or shape. Same contract otherwise. */
int retro_out_prod_variant(int variant, int type, const void *W, const float *G, float *dst,
                           int64_t K, int64_t N, int64_t T, void *stream);

/*
 * retro_out_prod on row-strided operands: W row n starts at byte n * ldw, G
 * row t at float t * ldg, dst row t at float t * ldd (elements within a row
 * stay contiguous). This takes views of larger tensors: a slice of G's
 * columns or rows, a block of dst's columns, W rows with padding between them.
 * With ldw = retro_row_bytes(type, K), ldg = N and ldd = K it is
 * retro_out_prod. This generalises the contiguous src1 and dst that the
 * llama.cpp PR #3 ("cuda: out_prod accepts a quantized src0") admits
 * (section "What") to strided ones.
 *   ldw  >= retro_row_bytes(type, K)   bytes
 *   ldg  >= N                          floats
 *   ldd  >= K                          floats
 * ldw must also be a multiple of the largest power of two (at most 16) that
 * divides the type's block bytes (F32: 4; F16, BF16, Q8_0, Q4_0, Q5_0, Q3_K,
 * Q6_K: 2; Q4_1, Q2_K: 4; Q5_1: 8; Q4_K, Q5_K: 16; MXFP4: 1), so that each row is as
 * aligned as the blocks of a contiguous row; otherwise RETRO_E_ALIGN.
 * Errors as retro_out_prod, plus RETRO_E_SHAPE for a stride shorter than its
 * row or a span beyond the size limits. Only the elements of dst's T x K
 * block are written; the bytes between its rows are left as they are.
 * RETRO_E_ALIAS compares the address ranges the operands span (first to last
 * element), so interleaved views of one tensor count as overlapping.
 */
int retro_out_prod_strided(int type, const void *W, int64_t ldw, const float *G, int64_t ldg, float *dst,
                           int64_t ldd, int64_t K, int64_t N, int64_t T, void *stream);

/* retro_out_prod_strided with a forced kernel variant (RETRO_E_VARIANT when
 * it does not apply). */
int retro_out_prod_strided_variant(int variant, int type, const void *W, int64_t ldw, const float *G,
                                   int64_t ldg, float *dst, int64_t ldd, int64_t K, int64_t N, int64_t T,
                                   void *stream);

/*
 * Batched retro_out_prod_strided over two outer dimensions, with the weight
 * broadcast over batches: for i3 < ne3, i2 < ne2
 *
 *     dst[i3][i2] = out_prod(W[i3 / (ne3 / ne03)][i2 / (ne2 / ne02)], G[i3][i2])
 *
 * This is ggml's OUT_PROD over dimensions 2 and 3, whose source operand may
 * have fewer matrices than the gradient (the broadcast ratios that the
 * llama.cpp PR #3 "cuda: out_prod accepts a quantized src0" carries through
 * its cuBLAS paths; the test table of its section "Measured" names the
 * broadcast cases). Each matrix is laid out as in retro_out_prod_strided;
 * matrix (i2, i3) of W starts i2 * sw2 + i3 * sw3 bytes after W, of G and
 * dst i2 * sg2 + i3 * sg3 and i2 * sd2 + i3 * sd3 floats after G and dst.
 *   ne02, ne03 >= 1 divide ne2, ne3 >= 0; ne2, ne3 and ne2 * ne3 <= 65535
 *   strides >= 0; sw2, sw3 multiples of 16 bytes, sg*, sd* multiples of 4
 *     floats (RETRO_E_ALIGN otherwise), so every matrix is 16-byte aligned
 *   the dst matrices must not overlap: sd2 spans at least one dst matrix and
 *     sd3 at least ne2 of them (RETRO_E_ALIAS otherwise); W and G may
 *     overlap themselves freely
 * ne2 * ne3 = 0 is a no-op. Errors as retro_out_prod_strided; RETRO_E_ALIAS
 * compares the whole spans of all batches.
 */
int retro_out_prod_batched(int type, const void *W, int64_t ldw, int64_t sw2, int64_t sw3, const float *G,
                           int64_t ldg, int64_t sg2, int64_t sg3, float *dst, int64_t ldd, int64_t sd2, int64_t sd3,
                           int64_t K, int64_t N, int64_t T, int64_t ne02, int64_t ne03, int64_t ne2, int64_t ne3,
                           void *stream);

/* retro_out_prod_batched with a forced kernel variant (RETRO_E_VARIANT when
 * it does not apply to one matrix). */
int retro_out_prod_batched_variant(int variant, int type, const void *W, int64_t ldw, int64_t sw2, int64_t sw3,
                                   const float *G, int64_t ldg, int64_t sg2, int64_t sg3, float *dst, int64_t ldd,
                                   int64_t sd2, int64_t sd3, int64_t K, int64_t N, int64_t T, int64_t ne02,
                                   int64_t ne03, int64_t ne2, int64_t ne3, void *stream);

/*
 * The most general form: retro_out_prod_batched with G in either
 * orientation. Element G[t][n] of matrix (i2, i3) is the float at
 *
 *     G + i2 * sg2 + i3 * sg3 + t * sgt + n * sgn
 *
 * with one of the two element strides equal to 1:
 *   sgn == 1           G rows contiguous (the gradient as ggml's mul_mat
 *                      writes it, which out_prod reads through grad^T, a
 *                      transposed view - llama.cpp PR #3 "cuda: out_prod
 *                      accepts a quantized src0", commit message); sgt >= N.
 *                      This is retro_out_prod_batched with ldg = sgt.
 *   sgt == 1, sgn > 1  G stored t-fastest (a contiguous src1 of ggml's
 *                      OUT_PROD: each of the N columns of G holds its T
 *                      values side by side); sgn >= T.
 * Anything else is RETRO_E_SHAPE. A stride of a dimension of size 1 is never
 * used: pass a value that satisfies the rule (for T = 1 with contiguous rows,
 * sgt = N). The producer/consumer kernels (RETRO_VARIANT_WS*) need sgt (rows)
 * or sgn (t-fastest) to be a multiple of 4; the single-role tile kernels and
 * the skinny kernel take any stride. All other arguments, limits and errors
 * as retro_out_prod_batched; RETRO_E_ALIAS compares the span from G's first
 * to its last element ((N - 1) * sgn + T floats per matrix when t-fastest).
 */
int retro_out_prod_views(int type, const void *W, int64_t ldw, int64_t sw2, int64_t sw3, const float *G, int64_t sgt,
                         int64_t sgn, int64_t sg2, int64_t sg3, float *dst, int64_t ldd, int64_t sd2, int64_t sd3,
                         int64_t K, int64_t N, int64_t T, int64_t ne02, int64_t ne03, int64_t ne2, int64_t ne3,
                         void *stream);

/* retro_out_prod_views with a forced kernel variant (RETRO_E_VARIANT when it
 * does not apply to one matrix). */
int retro_out_prod_views_variant(int variant, int type, const void *W, int64_t ldw, int64_t sw2, int64_t sw3,
                                 const float *G, int64_t sgt, int64_t sgn, int64_t sg2, int64_t sg3, float *dst,
                                 int64_t ldd, int64_t sd2, int64_t sd3, int64_t K, int64_t N, int64_t T, int64_t ne02,
                                 int64_t ne03, int64_t ne2, int64_t ne3, void *stream);

/* 1 if retro_out_prod_views_variant(variant, ...) with these strides and valid
 * buffers would run, 0 otherwise. Touches no device. */
int retro_out_prod_views_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T, int64_t ldw,
                                         int64_t sgt, int64_t sgn, int64_t ldd);

/* The variant retro_out_prod_views would run for ne2 x ne3 matrices of this
 * type, shape and strides, or a negative error code. Touches no device. */
int retro_out_prod_views_choice(int type, int64_t K, int64_t N, int64_t T, int64_t ldw, int64_t sgt, int64_t sgn,
                                int64_t ldd, int64_t ne2, int64_t ne3);

/* The variant retro_out_prod would run for this type and shape, or a
 * negative error code (as retro_out_prod_supported would refuse). When its
 * plan has two launches (retro_out_prod_plan) this is the first one's. Touches
 * no device. The views form above does the same for retro_out_prod_views. */
int retro_out_prod_choice(int type, int64_t K, int64_t N, int64_t T);

/* The launches retro_out_prod makes for this type and shape (contiguous
 * operands): returns 1 (one launch of *variant0 over all of dst; *k_split = K,
 * *variant1 = 0) or 2 (*variant0 over dst columns [0, *k_split), then
 * *variant1 over [*k_split, K)), or a negative error code (the three
 * pointers NULL: RETRO_E_NULL). RETRO_VARIANT_SKINNY counts as one launch
 * here; it makes one per 64 rows of G. Touches no device.
 * Two launches are planned when the tiles of one variant would leave the
 * last round over the 256 CUs partly empty and a larger tile fills whole
 * rounds on a leading column range (e.g. Q4_0, K = 5120, T = 2048: 128 x 256
 * tiles over 4096 columns, two-pipeline 64 x 128 over the other 1024). The
 * same rule applies to the strided, batched and views entry points. Each
 * launch computes its columns of the OUT_PROD of llama.cpp PR #3 ("cuda:
 * out_prod accepts a quantized src0", section "What") completely, so the
 * result is that of its variants on their columns. */
int retro_out_prod_plan(int type, int64_t K, int64_t N, int64_t T, int32_t *variant0, int64_t *k_split,
                        int32_t *variant1);

/* The launches retro_out_prod_views makes for ne2 x ne3 matrices of this
 * type, shape and strides (the W batch counts do not enter), as
 * retro_out_prod_plan. Touches no device. */
int retro_out_prod_views_plan(int type, int64_t K, int64_t N, int64_t T, int64_t ldw, int64_t sgt, int64_t sgn,
                              int64_t ldd, int64_t ne2, int64_t ne3, int32_t *variant0, int64_t *k_split,
                              int32_t *variant1);

/* retro_out_prod as two launches on `stream`: variant0 over dst columns
 * [0, k_split) (W's bytes before column k_split), then variant1 over
 * [k_split, K), for contiguous operands. Either variant may be
 * RETRO_VARIANT_AUTO (the choice for its part alone). 0 < k_split < K and a
 * whole number of blocks (RETRO_E_SHAPE otherwise); the W bytes before it a
 * multiple of 16 and k_split % 4 == 0 (RETRO_E_ALIGN otherwise), so that the
 * second part keeps the alignment of the whole; RETRO_E_VARIANT when a
 * variant does not apply to its part. Every check is made before either
 * launch. Pointers, aliasing, errors and execution as retro_out_prod. For
 * tests and benchmarks of the plans above. */
int retro_out_prod_column_split(int variant0, int64_t k_split, int variant1, int type, const void *W,
                                const float *G, float *dst, int64_t K, int64_t N, int64_t T, void *stream);

/*
 * retro_out_prod with a caller-owned workspace: the same contraction (the
 * OUT_PROD of llama.cpp PR #3 "cuda: out_prod accepts a quantized src0",
 * section "What") and contract, for contiguous operands. The skinny kernel
 * gives each 64-column slab of dst to one workgroup, so with fewer slabs than
 * CUs (K below 16384) part of the GPU idles; RETRO_VARIANT_SKINNY_SPLIT
 * spreads the rows of W evenly over all CUs and adds the parts of
 * each slab through the workspace (measured on MI355X, Q4_K, T = 16:
 * K = 4096, N = 14336 in 27 us against 79 us; K = 4096, N = 4096 in 11.5
 * against 25 us; at T = 32, K = 4096, N = 14336: 44 against 131 us).
 *   variant     RETRO_VARIANT_AUTO: the split when the estimated time gain is
 *               at least 10% (fewer than 193 slabs and enough rows), else
 *               what retro_out_prod runs; any other variant as
 *               retro_out_prod_variant, RETRO_VARIANT_SKINNY_SPLIT included
 *   workspace   device memory of workspace_bytes bytes, 16-byte aligned,
 *               overlapping none of W, G and dst; the split uses 1 KiB +
 *               2 MiB per block of 16 rows of G in a pass, at most
 *               6 MiB + 1 KiB (retro_out_prod_workspace_size). Its first
 *               1 KiB holds counters that must be zero before the first call
 *               that uses it (zero the whole workspace once); every call
 *               leaves them at zero, so later calls need no clearing. Calls
 *               that share a workspace must not overlap in time (one stream,
 *               or synchronised): they would race on it.
 * With RETRO_VARIANT_AUTO, a NULL workspace or one smaller than
 * retro_out_prod_workspace_size reports runs what retro_out_prod runs; a
 * forced RETRO_VARIANT_SKINNY_SPLIT returns RETRO_E_WORKSPACE instead. The
 * split adds each slab's parts in a fixed order, so its result does not
 * depend on which workgroup finishes first, but it sums in another order than
 * the skinny kernel (both within the same error bars). No waiting between
 * workgroups: every workgroup runs to its end whatever the others do.
 */
int retro_out_prod_ws(int variant, int type, const void *W, const float *G, float *dst, int64_t K, int64_t N,
                      int64_t T, void *workspace, int64_t workspace_bytes, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * retro_out_prod_ws with the library's own workspace, a static device array
 * of 6 MiB + 1 KiB on each GPU it runs on, held until the process ends. The
 * call allocates nothing and calls no allocating routine; the caller passes
 * inputs and outputs only. Same variants, results and errors as
 * retro_out_prod_ws with a workspace of that size (RETRO_E_WORKSPACE if a
 * call ever needed more; RETRO_E_HIP if the runtime cannot give the array's
 * address on the current device, which must be the stream's). Every call on
 * a GPU shares that GPU's array: calls that overlap in time on one GPU (two
 * streams, two threads) race on it and may return wrong sums, so they must
 * be ordered (one stream, or synchronised). The array's counters are zero
 * at load and every call leaves them at zero. */
int retro_out_prod_noalloc(int variant, int type, const void *W, const float *G, float *dst, int64_t K, int64_t N,
                           int64_t T, void *stream);

/* Bytes of workspace retro_out_prod_ws(variant, type, ..., K, N, T, ...) uses:
 * 0 when the call runs a kernel that needs none, else the split's fixed
 * size. A negative code for an invalid type or shape, or a variant that does
 * not apply. Touches no device. */
int64_t retro_out_prod_workspace_size(int variant, int type, int64_t K, int64_t N, int64_t T);

/* 1 if retro_out_prod_variant(variant, type, ..., K, N, T) with valid buffers
 * would run, 0 otherwise. Touches no device. */
int retro_out_prod_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T);

/* The same for retro_out_prod_strided_variant with strides ldw, ldg, ldd. */
int retro_out_prod_strided_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T, int64_t ldw,
                                           int64_t ldg, int64_t ldd);

/*
 * mul_mat, the forward of the layer whose input gradient retro_out_prod
 * computes (the llama.cpp PR #3 "cuda: out_prod accepts a quantized src0",
 * commit message, takes that input gradient as an OUT_PROD of W with the
 * transposed output gradient), through the same packed W:
 *
 *     Y[t][n] = sum_{k=0}^{K-1} W[n][k] * X[t][k]        t < T, n < N
 *
 *   W  N rows of retro_row_bytes(type, K) bytes, as for retro_out_prod
 *   X  T x K float32, row-major contiguous
 *   Y  T x N float32, row-major contiguous, overwritten (K = 0 writes zeros)
 * Pointers, alignment, aliasing, errors and execution as retro_out_prod.
 * Variants: RETRO_VARIANT_WS_256x128 / _128x128 / _64x128 / _32x128 (tiles of
 * T x N; need K % 4 == 0 for F32/F16/BF16), RETRO_VARIANT_SKINNY (T <= 16: one
 * workgroup per 16 rows of W over all of k; the same condition on K) and
 * RETRO_VARIANT_SIMPLE (any shape).
 */
int retro_mul_mat(int type, const void *W, const float *X, float *Y, int64_t K, int64_t N, int64_t T,
                  void *stream);

/* retro_mul_mat with a forced kernel variant (RETRO_E_VARIANT when it does
 * not apply). */
int retro_mul_mat_variant(int variant, int type, const void *W, const float *X, float *Y, int64_t K, int64_t N,
                          int64_t T, void *stream);

/* The variant retro_mul_mat would run (the first launch's when its plan has
 * two), or a negative error code. Touches no device. */
int retro_mul_mat_choice(int type, int64_t K, int64_t N, int64_t T);

/* The launches retro_mul_mat makes: returns 1 (*variant0 over all rows of W;
 * *n_split = N, *variant1 = 0) or 2 (*variant0 over W rows, i.e. Y columns,
 * [0, *n_split), then *variant1 over [*n_split, N)), or a negative error code
 * (the three pointers NULL: RETRO_E_NULL). Every Y[t][n] is complete in one
 * tile, so the rows of W can be split between two launches with no
 * reduction: taken where one tile size would leave the last round over the
 * 256 CUs partly empty and a larger tile fills whole rounds on the leading
 * rows. Touches no device. */
int retro_mul_mat_plan(int type, int64_t K, int64_t N, int64_t T, int32_t *variant0, int64_t *n_split,
                       int32_t *variant1);

/* retro_mul_mat as two launches on `stream`: variant0 over W rows (Y
 * columns) [0, n_split), then variant1 over [n_split, N); either may be
 * RETRO_VARIANT_AUTO (the choice for its part alone). 0 < n_split < N
 * (RETRO_E_SHAPE otherwise); n_split % 4 == 0 and the W bytes before row
 * n_split a multiple of 16 (RETRO_E_ALIGN otherwise); RETRO_E_VARIANT when a
 * variant does not apply to its part. Every check is made before either
 * launch. Pointers, aliasing, errors and execution as retro_mul_mat. For
 * tests and benchmarks of the plans above. */
int retro_mul_mat_row_split(int variant0, int64_t n_split, int variant1, int type, const void *W, const float *X,
                            float *Y, int64_t K, int64_t N, int64_t T, void *stream);

/* 1 if retro_mul_mat_variant(variant, type, ..., K, N, T) with valid buffers
 * would run, 0 otherwise. Touches no device. */
int retro_mul_mat_variant_applies(int variant, int type, int64_t K, int64_t N, int64_t T);

#ifdef __cplusplus
}
#endif

#endif /* RETRO_OUT_PROD_H */
