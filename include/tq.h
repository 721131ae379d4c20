/*
 * tq.h - C ABI of the TurboQuant KV-cache quantizer and quantized-KV decode
 * attention for AMD MI355X (gfx950).
 *
 * Sources for what each call computes (cited as [NIK] / [NAH]):
 *   [NIK] S. Nikolenko, "Eternal mathematics of TurboQuant: how to compress the
 *         KV cache down to the Shannon limit" (blog.sergeynikolenko.ru), a
 *         walkthrough of Zandieh et al. 2025, "TurboQuant: Online Vector
 *         Quantization with Near-optimal Distortion Rate".
 *   [NAH] "What exactly TurboQuant showed" (nahornyi.ai): the full prod
 *         variant needs a custom attention kernel.
 *
 * Conventions
 *   - Every call returns a tq_status. Nothing aborts and no C++ exception
 *     crosses this boundary. On failure a thread-local message is available
 *     from tq_last_error_message().
 *   - Arguments are validated synchronously, before any launch. Kernel faults
 *     are asynchronous and surface at the caller's stream synchronization.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller. The library owns
 *     only quantizer handles and the device tables inside them.
 *   - `stream` is a hipStream_t passed as void* (NULL = default stream). All
 *     device work of a call is enqueued on that stream; no call synchronizes.
 *   - Supported on the GPU: head dimension d in {64, 128, 256}, bit width
 *     b in [1, 4]. tq_codebook_build accepts 3 <= d <= 4096, 0 <= b <= 8.
 *
 * Bit layouts (the pages fix only that Q maps R^d to {0,1}^(b d); these are
 * this library's contract):
 *   VECTOR layout, per vector: `planes` bit planes of d bits. Plane p holds bit
 *     p of every centroid index; coordinate j of plane p is bit (j % 8) of
 *     byte p*d/8 + j/8. A record is planes*d/8 bytes; records are contiguous.
 *     QJL signs use the same layout with one plane (bit = 1 <=> S r >= 0).
 *   BLOCK32 layout (used for the value cache read by decode attention):
 *     vectors are grouped in blocks of 32; a block is 4*planes*d bytes. For
 *     plane p, group g in 0..3 and word w in 0..d/4-1, the little-endian
 *     32-bit word at byte ((p*4 + g)*(d/4) + w)*4 of the block holds, at bit
 *     4r+k (r, k in 0..3), plane-p bit of coordinate 4w+r of block vector
 *     4g+k, and at bit 16+4r+k the same for block vector 16+4g+k.
 *   Centroid indices ascend with centroid value; the codebook is symmetric,
 *   so the top plane is the sign of the rotated coordinate.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TQ_OK = 0,
  TQ_ERR_INVALID_ARG = 1, /* null pointer, negative size, inconsistent shapes   */
  TQ_ERR_UNSUPPORTED = 2, /* valid request this library does not implement       */
  TQ_ERR_NO_MEMORY = 3,   /* host or device allocation failed                    */
  TQ_ERR_DEVICE = 4,      /* a HIP call or kernel launch failed                  */
  TQ_ERR_WORKSPACE = 5    /* workspace pointer null or smaller than required     */
} tq_status;

typedef enum { TQ_MSE = 0, TQ_PROD = 1 } tq_variant;
typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;
typedef enum { TQ_LAYOUT_VECTOR = 0, TQ_LAYOUT_BLOCK32 = 1 } tq_layout;

/* Opaque quantizer: (d, b, variant, Pi, S) plus device tables. Immutable after
 * creation, so one handle may be used from many streams and threads at once. */
typedef struct tq_quantizer tq_quantizer;

const char* tq_status_string(tq_status s);
/* Detail of the last failure on the calling thread ("" if none). */
const char* tq_last_error_message(void);
/* Library ABI version (major*10000 + minor*100 + patch). */
int tq_version(void);

/*
 * Lloyd-Max codebook for one rotated coordinate.
 * [NIK] "Step 1: random rotation", Lemma on the coordinate density
 *   f_X(x) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - x^2)^((d-3)/2);
 * [NIK] "Step 2: optimal scalar quantization (Lloyd-Max)": 2^b centroids
 *   minimizing C(f_X, b); the codebook depends only on (d, b), no data.
 * Host only, deterministic. Outputs (host, caller-owned):
 *   centroids  [2^bits] float32, ascending (the fp64 solution rounded to nearest)
 *   thresholds [2^bits - 1] float32 (nullable): t_i = the largest float32 not
 *              above the exact midpoint of centroids i and i+1, so that for any
 *              float32 y, (y > t_i) <=> y is strictly nearer centroid i+1, and
 *              a tie goes to the lower index.
 *   cost_per_coord (nullable): C(f_X, b) in fp64; d * C is D_mse (Theorem 1).
 * bits == 0 gives the single centroid {0} (the MSE stage of prod with b = 1).
 */
tq_status tq_codebook_build(int d, int bits, float* centroids, float* thresholds,
                            double* cost_per_coord);

/*
 * Create a quantizer.
 * [NIK] "Step 0: normalization", "Step 1: random rotation", "Step 2";
 * for TQ_PROD also [NIK] "QJL: a one-bit method" and "TurboQuant proper":
 * b-1 bit MSE stage, then sign(S r) and |r| of the residual.
 *   d, bits   : head dimension and total bits per coordinate (prod: b-1 for the
 *               MSE stage plus 1 QJL bit). d in {64, 128, 256} for every call;
 *               any other multiple of 32 up to 4096 (vector search, [NIK]
 *               "Experiments": d = 1536, 3072; the parts of an outlier
 *               split, e.g. 32 and 96) for tq_quantize in the VECTOR layout,
 *               tq_inner_products, the split calls and tq_search_scores (d a
 *               multiple of 128 there) only (others return
 *               TQ_ERR_UNSUPPORTED). Orthogonality is checked exactly for
 *               d <= 256 and on four fixed pseudo-random vectors above.
 *   pi        : host, float64 [d][d] row-major, orthogonal (y = Pi u).
 *   s         : host, float64 [d][d] row-major Gaussian QJL matrix; required
 *               iff variant == TQ_PROD, ignored otherwise. It must be drawn
 *               independently of pi ([NIK] "What the community did", item 3).
 *   out       : receives the handle. The matrices are copied; the caller may
 *               free them after the call.
 * Allocates device memory on the current HIP device; the handle may be used
 * only on that device.
 */
tq_status tq_quantizer_create(int d, int bits, tq_variant variant, const double* pi,
                              const double* s, tq_quantizer** out);
/*
 * Same as tq_quantizer_create with a randomized Walsh-Hadamard rotation,
 * Pi = H diag(signs) / sqrt(d), H the Sylvester-Hadamard matrix of order d
 * (H[i][j] = (-1)^popcount(i & j)): the structured rotation the page's
 * community section ([NIK] "What the community did", item 3) reports as the
 * best MSE-stage transform, with the QJL matrix s drawn independently.
 *   signs : host, float64 [d], every entry exactly +1 or -1 (the random
 *           diagonal); copied.
 *   s     : as for tq_quantizer_create (required iff variant == TQ_PROD).
 * Errors: TQ_ERR_INVALID_ARG for a NULL pointer or a sign that is not +-1;
 * the other checks and the device tables are those of tq_quantizer_create
 * (the rotation is applied as a dense matrix by the same kernels).
 */
tq_status tq_quantizer_create_wht(int d, int bits, tq_variant variant, const double* signs,
                                  const double* s, tq_quantizer** out);
/* Frees the handle. The caller must first synchronize work that uses it. */
tq_status tq_quantizer_destroy(tq_quantizer* q);
/* Shape queries (any pointer may be NULL). code_planes = b for mse, b-1 for
 * prod; a VECTOR record has code_planes*d/8 code bytes and, for prod, d/8
 * sign bytes. */
tq_status tq_quantizer_info(const tq_quantizer* q, int* d, int* bits, tq_variant* variant,
                            int* code_planes);
/* Record sizes of one vector in the VECTOR layout ([NIK] "Step 2": b bits per
 * coordinate; "TurboQuant proper": b-1 code bits plus one sign bit for prod):
 * code_bytes = code_planes*d/8, sign_bytes = d/8 for TQ_PROD, 0 for TQ_MSE.
 * Either pointer may be NULL. Errors: TQ_ERR_INVALID_ARG for a NULL handle. */
tq_status tq_quantizer_sizes(const tq_quantizer* q, size_t* code_bytes, size_t* sign_bytes);

/*
 * Q (quantize), grouped: vector i of group g (i < n_per_group) is
 * x[g*n_per_group + i] and uses quantizer qz[g]. All handles must share
 * (d, bits, variant). One launch covers all groups.
 *   qz          : host array [n_groups] of handles.
 *   x           : device [n_groups*n_per_group][d], float32 or bfloat16.
 *   layout      : TQ_LAYOUT_VECTOR, or TQ_LAYOUT_BLOCK32 (TQ_MSE only, and
 *                 n_per_group % 32 == 0; blocks never straddle groups).
 *   codes       : device, code_planes*d/8 bytes per vector (may be NULL when
 *                 code_planes == 0).
 *   signs       : device [n][d/8] (TQ_PROD only; NULL for TQ_MSE).
 *   norms       : device float32 [n]: |x|_2 rounded to float32.
 *   rnorms      : device float32 [n]: |r|_2 of the unit-vector residual (prod).
 *   rot_dbg     : device float32 [n][d] or NULL: the rotated unit vector
 *                 y = Pi x / |x| exactly as the kernel compared it.
 *   proj_dbg    : device float32 [n][d] or NULL (prod): the projection S r
 *                 whose signs were stored.
 * A zero vector gets norm 0, rnorm 0 and all code and sign bits 0.
 * x, rot_dbg and proj_dbg must be 16-byte aligned, codes and signs 4-byte
 * aligned (TQ_ERR_INVALID_ARG otherwise). For TQ_PROD at d a multiple of 128 above 256 the
 * call takes stream-ordered scratch for the residuals (hipMallocAsync /
 * hipFreeAsync on the caller's stream, at most 1 GiB, vectors processed in
 * chunks that fit); every other configuration allocates nothing.
 * Errors: TQ_ERR_NO_MEMORY or TQ_ERR_DEVICE if that scratch cannot be had.
 */
tq_status tq_quantize(const tq_quantizer* const* qz, int n_groups, int64_t n_per_group,
                      const void* x, tq_dtype x_dtype, tq_layout layout, uint8_t* codes,
                      uint8_t* signs, float* norms, float* rnorms, float* rot_dbg,
                      float* proj_dbg, void* stream);

/*
 * One layer's new keys and values in one call: the online quantization of
 * [NIK] "Step 0" to "Step 2" applied to both tensors of a layer, keys with
 * kqz[g] (TurboQuant_mse or TurboQuant_prod) into the VECTOR layout, values
 * with vqz[g] (TurboQuant_mse) into the BLOCK32 layout, as the decode cache
 * keeps them.
 *   kqz, vqz    : host arrays [n_groups] of handles (each array one (d, bits,
 *                 variant), as for tq_quantize).
 *   xk, xv      : device [n_groups*n_per_group][d] each, x_dtype for both.
 *   kcodes, ksigns, knorms, krnorms : key records as tq_quantize writes them
 *                 (ksigns / krnorms NULL for mse keys).
 *   vcodes, vnorms : value records, BLOCK32 codes; n_per_group % 32 == 0.
 * When keys and values are both TurboQuant_mse with the same (d <= 256, bits),
 * the two tensors run in one launch; otherwise the call makes the two
 * launches that tq_quantize would. Records are identical to those of two
 * tq_quantize calls. Errors as for tq_quantize, checked for both tensors
 * before anything is launched.
 */
tq_status tq_quantize_kv(const tq_quantizer* const* kqz, const tq_quantizer* const* vqz, int n_groups,
                         int64_t n_per_group, const void* xk, const void* xv, tq_dtype x_dtype,
                         uint8_t* kcodes, uint8_t* ksigns, float* knorms, float* krnorms,
                         uint8_t* vcodes, float* vnorms, void* stream);

/* Q_mse for n vectors with one quantizer, VECTOR layout ([NIK] Theorem 1's map
 * Q_mse : R^d -> {0,1}^(b d)). Same argument meanings as tq_quantize, except:
 *   x_stride : elements from one input vector to the next (>= d; x_stride
 *              times the element size a multiple of 16 bytes), so one head's
 *              slice of a [n][heads*d] projection is read in place. */
tq_status tq_quantize_mse(const tq_quantizer* q, const void* x, tq_dtype x_dtype, int64_t n,
                          int64_t x_stride, uint8_t* codes, float* norms, float* rot_dbg, void* stream);

/* Q_prod for n vectors, VECTOR layout ([NIK] Theorem 2's map
 * Q_prod : S^(d-1) -> [2^(b-1)]^d x {-1,1}^d x R, applied to x/|x| with |x| kept).
 * x_stride as for tq_quantize_mse. */
tq_status tq_quantize_prod(const tq_quantizer* q, const void* x, tq_dtype x_dtype, int64_t n,
                           int64_t x_stride,
                           uint8_t* codes, uint8_t* signs, float* norms, float* rnorms,
                           float* rot_dbg, float* proj_dbg, void* stream);

/*
 * Q^-1 (dequantize) of n vectors:
 *   mse : x~ = |x| * Pi^T c[idx]                          ([NIK] "Step 2")
 *   prod: x~ = |x| * (Pi^T c[idx] + |r| sqrt(pi/2)/d S^T z) ([NIK] "QJL",
 *         "TurboQuant proper")
 * layout BLOCK32 requires n % 32 == 0 (mse only). x_out: device float32 [n][d].
 * signs / rnorms are ignored (may be NULL) for TQ_MSE.
 */
tq_status tq_dequantize(const tq_quantizer* q, tq_layout layout, const uint8_t* codes,
                        const uint8_t* signs, const float* norms, const float* rnorms,
                        int64_t n, float* x_out, void* stream);

/*
 * Inner products <y_i, x~_j> of m float32 queries with n packed vectors
 * (VECTOR layout), computed from the codes without materializing x~
 * ([NIK] problem statement, D_prod; used for D_prod and vector search).
 *   y   : device float32 [m][d];  out : device float32 [m][n].
 */
tq_status tq_inner_products(const tq_quantizer* q, const float* y, int64_t m,
                            const uint8_t* codes, const uint8_t* signs, const float* norms,
                            const float* rnorms, int64_t n, float* out, void* stream);

/*
 * Outlier-channel mixed precision ([NIK] "Experiments", KV cache: outlier
 * channels get more bits than the others, e.g. 32 channels at 3 bits and 96
 * at 2 bits of a 128-channel head): the channels of each input row are split
 * into parts and part p is quantized by its own quantizer (its own rotation,
 * norm, codebook and, for prod, QJL matrix) in the VECTOR layout. The rule
 * that picks the outlier channels is not given by the pages; the caller
 * passes the channel lists. Grouped as tq_quantize: row i of group g
 * (i < n_per_group) is x[g*n_per_group + i] and uses group g's handles and
 * channel lists (e.g. one group per KV head, each head with its own outlier
 * channels).
 *   qz       : host array [n_parts][n_groups] of handles (part p, group g at
 *              qz[p*n_groups + g]), 1 <= n_parts <= 8; the handles of one
 *              part share d, bits and variant (d_p = that d, at most 4
 *              MSE-stage planes); parts may differ in all three.
 *   n_groups : >= 1.
 *   channels : host int32 [n_parts][n_groups][d_p]: group g's part p takes the
 *              input channels channels[off_p + g*d_p .. + d_p), off_p =
 *              n_groups*(d_0 + .. + d_{p-1}), in that order (coordinate j of
 *              the part is that list's entry j). Every entry in [0, dim), none
 *              repeated within a group; channels left out are dropped. Copied.
 *   dim      : channels per input row, at most 512.
 *   x        : device [n_groups*n_per_group][dim], float32 or bfloat16.
 *   layout   : TQ_LAYOUT_VECTOR, or TQ_LAYOUT_BLOCK32 (every part mse,
 *              n_per_group % 32 == 0): each part's codes in blocks of 32 rows,
 *              the value-cache layout tq_decode_attention_split reads.
 *   out      : host array [n_parts] of device record buffers for all
 *              n_groups*n_per_group rows, as for tq_quantize with d = d_p
 *              (rot_dbg / proj_dbg may be NULL; codes and signs 4-byte aligned).
 * On the caller's stream. dim = 128 with d_p a multiple of 32 (mse, or prod of
 * at most 4 bits): matrix-core launches of 16 groups with the parts' matrices
 * laid over the head's channels, both parts in one pass when two parts of one
 * variant cover all 128 channels, else one launch per part. Otherwise the
 * generic fp32 kernels, one launch per part and group, where BLOCK32 adds one
 * in-place repack launch per part. Allocates nothing.
 * Errors: TQ_ERR_INVALID_ARG (NULL pointers, n_groups < 1, handles of a part
 * that differ, a channel out of range or repeated within a group, more
 * channels than dim, BLOCK32 with n_per_group % 32 != 0), TQ_ERR_UNSUPPORTED
 * (dim > 512, n_groups*n_per_group > 2^31, BLOCK32 with a prod part).
 */
typedef struct {
  uint8_t* codes;   /* code_planes*d/8 bytes per vector (NULL when code_planes == 0) */
  uint8_t* signs;   /* prod: [n][d/8] */
  float* norms;     /* [n] */
  float* rnorms;    /* prod: [n] */
  float* rot_dbg;   /* optional [n][d] */
  float* proj_dbg;  /* optional [n][d] (prod) */
} tq_records;
tq_status tq_quantize_split(const tq_quantizer* const* qz, int n_parts, int n_groups, const int32_t* channels,
                            int dim, const void* x, tq_dtype x_dtype, int64_t n_per_group, tq_layout layout,
                            const tq_records* out, void* stream);
/*
 * Inner products of m float32 queries y [m][dim] with n split records:
 *   out[i][j] = sum_p <y_i restricted to part p's channels, x~_p,j>
 * the estimate of <y_i, x_j> over the kept channels (each part as in
 * tq_inner_products). qz and channels as for tq_quantize_split with
 * n_groups = 1. recs is read only; out: device float32 [m][n].
 * Errors as for tq_quantize_split, plus m > 65535.
 */
tq_status tq_inner_products_split(const tq_quantizer* const* qz, int n_parts, const int32_t* channels,
                                  int dim, const float* y, int64_t m, const tq_records* recs, int64_t n,
                                  float* out, void* stream);

/*
 * Vector-search scoring on the matrix cores: the same inner products
 * <y_i, x~_j> as tq_inner_products ([NIK] "Experiments": nearest-neighbour
 * search over quantized embeddings), from a VECTOR-layout database, computed
 * as MFMA contractions of the queries' rotated (and, for prod, S-projected)
 * vectors with the records' bit planes, through the odd Walsh expansion of the
 * symmetric codebook. Supports d a multiple of 128 in [128, 4096] and up to 4
 * MSE-stage planes; other quantizers return TQ_ERR_UNSUPPORTED.
 *   y, m, codes, signs, norms, rnorms, n, out : as for tq_inner_products
 *               (out: device float32 [m][n], overwritten); y 16-byte aligned,
 *               codes and signs 4-byte aligned.
 *   workspace : device scratch of at least tq_search_workspace_size(q, m)
 *               bytes (per-query operands); concurrent calls need separate
 *               workspaces.
 * Errors: TQ_ERR_INVALID_ARG (NULL handle or buffer, negative size, a
 * misaligned buffer), TQ_ERR_WORKSPACE (workspace missing or too small), TQ_ERR_UNSUPPORTED
 * (d, planes, m > 65535 or n > 2^31). m == 0 or n == 0 is a no-op.
 */
tq_status tq_search_workspace_size(const tq_quantizer* q, int64_t m, size_t* bytes);
tq_status tq_search_scores(const tq_quantizer* q, const float* y, int64_t m, const uint8_t* codes,
                           const uint8_t* signs, const float* norms, const float* rnorms, int64_t n,
                           float* out, void* workspace, size_t ws_bytes, void* stream);

/*
 * Decode attention over a packed KV cache ([NIK] problem statement: the new
 * token's query is scored against every cached key and the values are
 * averaged with the softmax weights; [NAH]: prod keys need a dedicated
 * attention kernel). For each batch b and query head h with KV head
 * g = floor(h * n_kv_heads / n_q_heads):
 *   s_t = scale * <q[b,h], k~_t>,  t < ctx_lens[b]
 *   out[b,h] = sum_t softmax(s)_t v~_t
 * where k~, v~ are the dequantized key and value of token t. The kernel never
 * materializes them: keys are scored in rotated space (Pi_K q and S_K q) and
 * values are accumulated in rotated space and rotated back once.
 *
 * Cache layout (caller-owned device memory), with G = batch*n_kv_heads groups
 * indexed b*n_kv_heads + g and T = max_ctx (a multiple of 32):
 *   keys  : codes [G][T][code_planes*d/8] VECTOR layout (may be NULL if
 *           code_planes == 0); signs [G][T][d/8] (prod keys, else NULL);
 *           norms [G][T]; rnorms [G][T] (prod keys, else NULL).
 *   values: TQ_MSE quantizers only; codes [G][T/32][4*bits*d] BLOCK32 layout;
 *           norms [G][T]; signs and rnorms NULL.
 *   qz    : host array [n_kv_heads] of handles per tensor; all key handles
 *           share (d, bits, variant), all value handles share (d, bits).
 *   q     : device bfloat16 [batch][n_q_heads][d].
 *   ctx_lens : device int32 [batch]; values are clamped to [0, max_ctx]; a
 *           sequence with no tokens gets an all-zero output.
 *   out   : device float32 [batch][n_q_heads][d].
 *   scores_dbg : device float32 [batch][n_q_heads][max_ctx] or NULL: s_t for
 *           t < ctx_len (other entries untouched).
 *   workspace : device scratch of at least tq_decode_workspace_size() bytes,
 *           used only during the call's stream work. Concurrent calls need
 *           separate workspaces.
 * n_q_heads must be a multiple of n_kv_heads, with a group size of at most 8
 * or a multiple of 8. Results are deterministic for a fixed shape (fixed
 * split schedule, no floating-point atomics).
 */
typedef struct {
  int batch;
  int n_q_heads;
  int n_kv_heads;
  int head_dim;
  int64_t max_ctx;
} tq_attn_shape;

typedef struct {
  const tq_quantizer* const* qz;
  const uint8_t* codes;
  const uint8_t* signs;
  const float* norms;
  const float* rnorms;
} tq_packed_kv;

tq_status tq_decode_workspace_size(const tq_attn_shape* shape, const tq_packed_kv* k,
                                   const tq_packed_kv* v, size_t* bytes);

tq_status tq_decode_attention(const tq_attn_shape* shape, const void* q, const tq_packed_kv* k,
                              const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                              float* out, float* scores_dbg, void* workspace, size_t ws_bytes,
                              void* stream);

/*
 * Decode attention that allocates nothing: tq_decode_attention with the
 * workspace taken from a static device array of the library (32 MiB per GPU,
 * held by each GPU the library runs on until the process ends). For callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc. It calls no allocating
 * routine. Arguments, layouts and results are those of tq_decode_attention
 * (same kernels, same split schedule, so the same output bits).
 * Every call on one GPU shares that GPU's array (it keeps the last call's
 * partials; nothing in it needs to start at zero): calls that overlap on one
 * GPU, on any streams, race and must be serialized by the caller.
 * Errors: as tq_decode_attention, and TQ_ERR_WORKSPACE when the shape needs
 * more than 32 MiB of scratch (tq_decode_workspace_size() tells how much).
 */
tq_status tq_decode_attention_noalloc(const tq_attn_shape* shape, const void* q, const tq_packed_kv* k,
                                      const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                                      float* out, float* scores_dbg, void* stream);

/*
 * Decode step with append: the online use of the quantizer ([NIK] "Step 0" to
 * "Step 2": vector in, code out, nothing to train; for prod keys also "TurboQuant
 * proper") followed by the attention step that reads the cache ([NAH]: the prod
 * variant needs its own attention kernel). For every (b, h) the new key k_new[b][h]
 * is quantized with k->qz[h] and the new value v_new[b][h] with v->qz[h]; both are
 * written into the packed caches at token ctx_lens[b] (keys: vector layout record;
 * values: slot ctx_lens[b] % 32 of its BLOCK32 block, the other 31 slots kept),
 * and the query then attends ctx_lens[b] + 1 tokens, as tq_decode_attention.
 *   q             : device bf16 [B][Hq][d].
 *   k_new, v_new  : device [B][Hkv][d], float32 or bfloat16 (kv_dtype).
 *   k, v          : the caches as for tq_decode_attention; their code, sign and
 *                   norm buffers are WRITTEN at token ctx_lens[b] (device memory
 *                   owned by the caller; the const in tq_packed_kv is cast away).
 *   ctx_lens      : device int32 [B], tokens already cached; read, not advanced
 *                   (the caller adds 1 after the call). A sequence with
 *                   ctx_lens[b] >= max_ctx is not appended and attends max_ctx
 *                   tokens.
 *   dbg           : NULL, or device buffers (each may be NULL) that receive what
 *                   the new records were decided on: rot [B][Hkv][2][d] float32,
 *                   the rotated unit vectors Pi x/|x| of the key (index 0) and
 *                   the value (index 1) exactly as compared with the
 *                   thresholds; proj [B][Hkv][d] float32, S r of the key (prod)
 *                   whose signs were stored. Entries of sequences that are not
 *                   appended are left untouched.
 *   workspace     : device, at least tq_decode_append_workspace_size() bytes
 *                   (the same size as tq_decode_workspace_size()).
 * Same validation and errors as tq_decode_attention, plus TQ_ERR_INVALID_ARG
 * for NULL k_new / v_new or an unknown kv_dtype. The new tokens are quantized by
 * the launch that prepares the queries (one block per (b, h) and tensor, fp32
 * rotation, fp64 norm), before the attention reads the cache; no host
 * synchronization. Records equal those of tq_quantize except where a rotated
 * coordinate lies within rounding of a decision threshold (tq_quantize rotates
 * with split-bf16 matrix cores).
 */
typedef struct {
  float* rot;
  float* proj;
} tq_append_debug;
tq_status tq_decode_append_workspace_size(const tq_attn_shape* shape, const tq_packed_kv* k,
                                          const tq_packed_kv* v, size_t* bytes);
tq_status tq_decode_append_attention(const tq_attn_shape* shape, const void* q, const void* k_new,
                                     const void* v_new, tq_dtype kv_dtype, const tq_packed_kv* k,
                                     const tq_packed_kv* v, const int32_t* ctx_lens, float scale,
                                     float* out, const tq_append_debug* dbg, void* workspace,
                                     size_t ws_bytes, void* stream);

/*
 * Decode attention over KV caches quantized with an outlier-channel split
 * ([NIK] "Experiments", KV cache: outlier channels at more bits; the same
 * attention as tq_decode_attention, scores and outputs over the channels the
 * parts keep). Each side (keys, values) is a split of the head's channels into
 * parts, part p quantized per KV head (records [B][n_kv_heads][max_ctx], as
 * tq_quantize_split writes them with the KV heads as groups): key parts in the
 * VECTOR layout, value parts in the BLOCK32 layout (codes
 * [B][n_kv_heads][max_ctx/32][4*planes*d_p]; max_ctx % 32 == 0):
 *   s_t = scale * sum_p <q restricted to key part p's channels, k~_{p,t}>
 *   out[b,h] = sum_{t < ctx_lens[b]} softmax(s)_t v~_t, each value part written
 *   to its channels (channels no value part keeps are 0; ctx_lens[b] <= 0 gives
 *   0, lengths above max_ctx attend max_ctx tokens).
 *   qz       : host [n_parts * n_kv_heads]; part p of KV head g is
 *              qz[p * n_kv_heads + g]; the handles of one part share (d, bits,
 *              variant); d a multiple of 32; keys mse or prod, values mse;
 *              codes and signs 4-byte aligned.
 *   channels : host int32 [n_parts][n_kv_heads][d_p]: part p of KV head g
 *              keeps the channels channels[n_kv_heads * off_p + g * d_p + j],
 *              j < d_p, off_p = d_0 + .. + d_{p-1} (coordinate j of that
 *              part; the order tq_quantize_split was given for that head).
 *              Heads may pick different channels; within a head every entry
 *              lies in [0, head_dim) and none repeats. Copied.
 *   rec      : host [n_parts]; rec[p] holds part p's device arrays.
 * head_dim = the full channel count (at most 256), at most 8 KV heads and 8
 * query heads per KV head. q: device bf16 [B][n_q_heads][head_dim];
 * out: device float32 [B][n_q_heads][head_dim]; workspace: at least
 * tq_decode_split_workspace_size() bytes (per-split softmax partials and the
 * rotated query operands; the size depends on the device, which sets the number
 * of context splits). Scores and value sums run on the matrix cores as exact
 * fp16 hi/lo products, split context with a log-sum-exp combine
 * (deterministic). Errors: TQ_ERR_INVALID_ARG (also max_ctx % 32 != 0),
 * TQ_ERR_UNSUPPORTED (limits above), TQ_ERR_WORKSPACE.
 */
typedef struct {
  int n_parts;
  const tq_quantizer* const* qz;
  const int32_t* channels;
  const tq_records* rec;
} tq_split_cache;
tq_status tq_decode_split_workspace_size(const tq_attn_shape* shape, const tq_split_cache* k,
                                         const tq_split_cache* v, size_t* bytes);
tq_status tq_decode_attention_split(const tq_attn_shape* shape, const void* q, const tq_split_cache* k,
                                    const tq_split_cache* v, const int32_t* ctx_lens, float scale,
                                    float* out, void* workspace, size_t ws_bytes, void* stream);


#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
