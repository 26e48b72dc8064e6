/*
 * rbq.h - C ABI of the rotated, asymmetric K4/V3 quantized KV cache and the
 * fused decode/verify attention over it, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the page "mlx_streaming/core/cache/quant_kv.py"
 * (sparkle): the SO(4) block rotation (build_block_so4, rotate_last), the
 * asymmetric quantized cache (AsymmetricQuantizedKVCache: update_and_fetch,
 * trim) and the quantized SDPA (asym_quantized_sdpa), plus the trimmable
 * branch of commit_verified_prefix on the page "mlx_streaming/mtp/kv_cache.py".
 *
 * Conventions shared by every entry point:
 *   - Return value: RBQ_OK (0) or a negative RBQ_E* status; functions that
 *     return a count return it when >= 0 and a negative status otherwise.
 *     Nothing throws across the ABI.  rbq_status_string() names a status.
 *   - Memory: the library allocates no device memory and owns no buffer,
 *     except the fixed scratch array of rbq_quant_attn_decode_noalloc
 *     (RBQ_SCRATCH_BYTES per device, part of the loaded code object).
 *     Every pointer is owned by the caller.  "device" pointers are HIP device
 *     allocations on the current device; "host" pointers are ordinary memory.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the legacy
 *     default stream).  Device work is enqueued on it and the call returns
 *     without synchronising; buffers must outlive that work.  Launch failures
 *     return RBQ_EHIP and rbq_last_hip_error() gives the hipError_t (thread
 *     local).
 *   - Thread safety: calls on distinct caches may run concurrently.
 *   - Supported shapes in this library (gfx950): head_dim 64, 128 or 256;
 *     group_size 32, 64 or 128, dividing head_dim (the cache constructor's
 *     group_size); k_bits and v_bits each one of 2, 3, 4, 5, 6, 8 (the width
 *     list of _packed_words); dtype fp16 or bf16.  Anything else returns
 *     RBQ_EUNSUPPORTED, as do descriptors beyond these size limits (far
 *     beyond any device memory; they keep every size computation inside 64
 *     bits): capacity <= 2^40 rows, B * H_kv < 2^31 slabs, and
 *     B * H_kv * capacity <= 2^44 rows.  The default configuration (head_dim 256, group 64,
 *     K 4-bit, V 3-bit) has dedicated append and attention kernels; the
 *     others run general kernels with the same results definition.
 */
#ifndef RBQ_H
#define RBQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define RBQ_OK             0
#define RBQ_EINVAL        -1  /* bad argument: null pointer, negative size, shape mismatch  */
#define RBQ_EUNSUPPORTED  -2  /* valid but not built here (head_dim, bits, group, dtype)    */
#define RBQ_ECAPACITY     -3  /* offset + n exceeds the cache capacity; nothing was written */
#define RBQ_ERANGE        -4  /* L < 1 or L > offset (no visible key for some query row)    */
#define RBQ_EWORKSPACE    -5  /* workspace missing or smaller than required                 */
#define RBQ_EHIP          -6  /* a HIP call or kernel launch failed                         */
#define RBQ_ESCRATCH      -7  /* the call needs more than the fixed scratch array holds     */

/* Bytes of the fixed device scratch array of rbq_quant_attn_decode_noalloc
 * (one per device the library runs on, held until the process ends). */
#define RBQ_SCRATCH_BYTES (8u << 20)

/* ---- element types of the key/value/query inputs and of scales/biases ---- */
#define RBQ_F16   1
#define RBQ_BF16  2

/* ---- cache flags ----
 * RBQ_FLAG_ROUND_ROTATED: the page's own rotation precision (rotate_last on
 * the quant_kv.py page multiplies by R.astype(x.dtype), so its result is in
 * the input dtype): every rotated row - K and V before they are quantized,
 * q before the attention - is rounded to the cache dtype (round half to
 * even).  The caller passes rotation blocks already rounded to the dtype
 * (rbq_rotation_round).
 * Without the flag rotated rows stay fp32. */
#define RBQ_FLAG_ROUND_ROTATED 1

/* ---- rotation block forms (rbq_rotation_build_mode) ---- */
#define RBQ_ROT_PRINTED    0  /* L(qL) times the matrix printed for _quat_right_conj */
#define RBQ_ROT_TWO_SIDED  1  /* L(qL) times the right multiplication by conj(qR)   */

/*
 * Cache descriptor (host struct, owned by the caller).  It mirrors the six
 * arrays of AsymmetricQuantizedKVCache (_init_quant on the quant_kv.py page):
 *   k_words  uint32 [B][H_kv][capacity][head_dim*k_bits/32]   (32 words at D=256)
 *   k_scales dtype  [B][H_kv][capacity][head_dim/group_size]
 *   k_biases dtype  [B][H_kv][capacity][head_dim/group_size]
 *   v_words  uint32 [B][H_kv][capacity][head_dim*v_bits/32]   (24 words at D=256)
 *   v_scales, v_biases as for K.
 * All six are contiguous device buffers (row stride = capacity rows); the
 * word arrays start 16-byte aligned, the scale and bias arrays 4-byte
 * aligned (RBQ_EINVAL otherwise; every device allocation is).  Each
 * packed row is a little-endian bit stream: bit t of code j is bit
 * ((bits*j + t) mod 32) of word (bits*j + t) / 32.  Rows [0, offset) are
 * valid; rows at or beyond offset are never read.
 */
typedef struct rbq_kv_cache {
    int32_t B, H_kv, head_dim, group_size, k_bits, v_bits;
    int32_t dtype;          /* RBQ_F16 or RBQ_BF16: type of scales/biases and of the inputs */
    int32_t flags;          /* 0 or RBQ_FLAG_ROUND_ROTATED */
    int64_t capacity;       /* rows allocated per (b, kv head) */
    int64_t offset;         /* rows written per (b, kv head) */
    uint32_t* k_words;
    void* k_scales;
    void* k_biases;
    uint32_t* v_words;
    void* v_scales;
    void* v_biases;
} rbq_kv_cache;

/*
 * rbq_rotation_build - the blocks of the block-diagonal SO(4) rotation
 * (quant_kv.py, "SO(4) block rotation": _quat_left, _quat_right_conj,
 * build_block_so4).  Host only.
 *   draws   host float [head_dim/4][2][4]: per block the raw left and right
 *           quaternion draws (four standard normals each, cast to float32, in
 *           the page's draw order from numpy's default_rng(seed)).
 *   blocks  host float [head_dim/4][4][4], written: block b =
 *           L(qL) * Rc(qR) with qL, qR the normalised draws and L, Rc the
 *           printed 4x4 matrices; computed in double, rounded once to float.
 *           The dense rotation M is blockdiag(blocks); rows rotate as x @ M.
 * Errors: RBQ_EINVAL for null pointers, head_dim <= 0 or head_dim % 4 != 0,
 * or a zero-norm draw (nothing defined is written in that case).
 */
int rbq_rotation_build(const float* draws, int32_t head_dim, float* blocks);

/*
 * rbq_rotation_build_mode - as rbq_rotation_build with a choice of the right
 * factor (quant_kv.py, "SO(4) block rotation").  RBQ_ROT_PRINTED gives
 * exactly rbq_rotation_build.  RBQ_ROT_TWO_SIDED uses the matrix of
 * v -> v * conj(qR) (quaternions as column vectors (w, x, y, z)), the map the
 * _quat_right_conj docstring describes; each block is then
 * v -> qL * v * conj(qR), a general SO(4) element, while the printed matrix
 * is the transpose of L(qR) and gives left-isoclinic blocks only.
 * Errors: as rbq_rotation_build, and RBQ_EINVAL for an unknown mode.
 */
int rbq_rotation_build_mode(const float* draws, int32_t head_dim, int32_t mode, float* blocks);

/*
 * rbq_rotation_round - the rotation blocks rounded to the cache dtype, in
 * place: the page's own rotation precision (rotate_last on the quant_kv.py
 * page multiplies by R.astype(x.dtype)), to be used with a cache whose flags
 * hold RBQ_FLAG_ROUND_ROTATED.  Host only.
 *   blocks  host float [head_dim/4][4][4] (from rbq_rotation_build or
 *           rbq_rotation_build_mode); each entry is replaced by its
 *           round-half-to-even value in `dtype`, which a float holds exactly.
 *   dtype   RBQ_F16 or RBQ_BF16.
 * Errors: RBQ_EINVAL for null blocks, head_dim <= 0, head_dim % 4 != 0 or a
 * non-finite entry (then nothing is changed); RBQ_EUNSUPPORTED for another
 * dtype.
 */
int rbq_rotation_round(float* blocks, int32_t head_dim, int32_t dtype);

/*
 * rbq_kv_required_capacity - capacity (rows) the cache needs before n more
 * rows are appended (AsymmetricQuantizedKVCache.update_and_fetch, step 256):
 * unchanged while offset + n <= capacity (and capacity > 0); otherwise
 * ceil(n/256)*256 rows are added to the buffer, which is first cut back to
 * `offset` rows when offset % 256 != 0.  capacity == 0 means no buffer yet.
 * Returns the capacity, or RBQ_EINVAL when n < 0, offset < 0 or
 * offset > capacity, RBQ_EUNSUPPORTED when capacity, n or the result exceed
 * 2^40 rows.  Host only.
 */
int64_t rbq_kv_required_capacity(int64_t capacity, int64_t offset, int64_t n);

/*
 * rbq_kv_grow - copy a cache into larger buffers (the growth step of
 * update_and_fetch).  `dst` must describe the new buffers (same B, H_kv,
 * head_dim, group, bits, dtype; dst->capacity >= the rows kept) and
 * `src` the old ones.  Rows [0, keep) are copied, where keep = src->offset
 * when src->offset % 256 != 0 and src->capacity otherwise (the page keeps
 * the whole old buffer in that case), and rows [keep, dst->capacity) are
 * zero-filled.  dst->offset is set to src->offset.  Device work on `stream`.
 * Errors: RBQ_EINVAL (mismatched descriptors, dst too small, aliasing
 * buffers), RBQ_EUNSUPPORTED, RBQ_EHIP.
 */
int rbq_kv_grow(const rbq_kv_cache* src, rbq_kv_cache* dst, void* stream);

/*
 * rbq_kv_quant_append - rotate, quantize, bit-pack and append n rows
 * (update_and_fetch with mx.quantize; quantizer scale = (max-min)/(2^bits-1),
 * bias = min, code = clip(round-half-even((x - bias)/scale), 0, 2^bits-1) per
 * group of group_size values, scale and bias stored in `dtype` and the codes
 * computed against the stored values; a zero scale divides by 1).
 *   k, v        device dtype [B][H_kv][n][head_dim], contiguous, unrotated.
 *   rot_blocks  device float [head_dim/4][4][4] from rbq_rotation_build, or
 *               NULL for no rotation (the page's cache, whose inputs arrive
 *               already rotated).  Each 4-block of a row is rotated as an
 *               fp64 sum of exact products and rounded once to fp32.
 * Writes rows [offset, offset+n) of all six arrays and, on success, sets
 * c->offset += n (host side, immediately; the device writes are async).
 * Errors: RBQ_EINVAL (null pointers, n < 0), RBQ_ECAPACITY when
 * offset + n > capacity (nothing is written), RBQ_EUNSUPPORTED, RBQ_EHIP.
 * n == 0 is a no-op returning RBQ_OK.
 */
int rbq_kv_quant_append(rbq_kv_cache* c, const void* k, const void* v, int64_t n,
                        const float* rot_blocks, void* stream);

/*
 * rbq_kv_trim - AsymmetricQuantizedKVCache.trim: n' = min(offset, n),
 * offset -= n', returns n'.  Data is not cleared.  Host only, synchronous.
 * Errors: RBQ_EINVAL for a null cache or n < 0.
 */
int64_t rbq_kv_trim(rbq_kv_cache* c, int64_t n);

/*
 * rbq_kv_commit_verified - trimmable branch of commit_verified_prefix
 * (mtp/kv_cache.py): after verifying `verified_len` draft tokens of which
 * `accepted_len` were accepted, trim the rejected suffix.  Returns the rows
 * trimmed, or RBQ_EINVAL when accepted_len > verified_len or either is < 0.
 */
int64_t rbq_kv_commit_verified(rbq_kv_cache* c, int64_t verified_len, int64_t accepted_len);

/*
 * rbq_kv_copy_prefix - copy rows [0, src->offset) of all six arrays of `src`
 * into the same rows of `dst` and set dst->offset = src->offset; rows of dst
 * at or past that offset are not touched.  This is the device copy behind
 * cache snapshots (quant_kv.py, the snapshot interface: `state` getter and
 * setter; mtp/kv_cache.py `_snapshot`, `_restore`,
 * `commit_verified_snapshot`): a snapshot is a copy of the offset-prefix
 * into buffers of its own, a restore copies a snapshot back.  `dst` must
 * describe buffers of the same B, H_kv, head_dim, group, bits and dtype with
 * dst->capacity >= src->offset; the two caches' arrays must not overlap.
 * One kernel launch on `stream`.  Errors: RBQ_EINVAL (bad or mismatched
 * descriptors, overlapping arrays), RBQ_ECAPACITY (dst too small, nothing is
 * written), RBQ_EUNSUPPORTED, RBQ_EHIP.  src->offset == 0 only sets
 * dst->offset = 0.
 */
int rbq_kv_copy_prefix(const rbq_kv_cache* src, rbq_kv_cache* dst, void* stream);

/*
 * rbq_kv_copy_batch - the prefix copy between caches of different batch
 * sizes: destination batch entry b receives rows [0, src->offset) of source
 * entry src_b0 + b * src_b_step (every kv head); dst->offset = src->offset.
 * src_b_step = 0 with a batch-1 source repeats it P times (`tile_caches` on
 * the mtp/kv_cache.py page: a batch-1 cache spread over the P draft paths of
 * a batched verification); a batch-1 destination with src_b0 = row keeps
 * one path (`commit_tree_row`, after the trim of the rejected suffix).
 * Requirements and errors as rbq_kv_copy_prefix, except that the batch sizes
 * may differ; RBQ_EINVAL when a source entry falls outside [0, src->B).
 */
int rbq_kv_copy_batch(const rbq_kv_cache* src, int32_t src_b0, int32_t src_b_step,
                      rbq_kv_cache* dst, void* stream);

/*
 * rbq_quant_attn_splits - the split count rbq_quant_attn_decode uses when
 * called with splits == 0 for this cache state and query shape (>= 1), or a
 * negative status for invalid arguments.
 */
int32_t rbq_quant_attn_splits(const rbq_kv_cache* c, int32_t H_q, int32_t L);

/*
 * rbq_quant_attn_workspace_bytes - bytes of device workspace
 * rbq_quant_attn_decode needs for this cache state, query shape and split
 * count (splits == 0: the automatic count).  0 means no workspace is needed.
 * Returns (size_t)0 also for invalid arguments; the decode call reports those.
 * The workspace holds the split partials between the attention kernel and
 * the merge kernel that follows it on the same stream; its contents before a
 * call do not matter, and calls that overlap in time must not share one.
 */
size_t rbq_quant_attn_workspace_bytes(const rbq_kv_cache* c, int32_t H_q, int32_t L,
                                      int32_t splits);

/*
 * rbq_quant_attn_decode - fused decode/verify attention over the packed
 * cache (asym_quantized_sdpa) followed by the inverse rotation.
 *   q           device dtype [B][H_q][L][head_dim], contiguous, unrotated.
 *               Query head h reads kv head h / (H_q / H_kv).
 *   scale       multiplies q before the scores (conventionally head_dim^-1/2).
 *   causal      1: row i of the L-block sees keys t <= offset - L + i (the
 *               page's causal mask at the cache offset); 0: all offset keys.
 *   rot_blocks  device float [head_dim/4][4][4] or NULL.  With blocks, q is
 *               rotated on entry (fp64 sum of exact products -> fp32) and the
 *               output is rotated back (out = o @ M^T); with NULL neither
 *               happens and the output stays in the cache's value space, as
 *               the page's SDPA returns it.
 *   out         device float [B][H_q][L][head_dim], written (fp32).
 *   splits      number of key-range partials per (b, kv head) merged by a
 *               log-sum-exp combine (0 = automatic; the result does not
 *               depend on it beyond fp32 rounding).
 *   ws          device workspace of ws_bytes >= rbq_quant_attn_workspace_bytes
 *               (may be NULL when that is 0).
 *   Alignment: q 8-byte, out, rot_blocks and ws 16-byte aligned (RBQ_EINVAL
 *               otherwise).
 * Scores, softmax and the P.V accumulation run in fp32.  Keys [0, offset)
 * are read.  Any L from 1 (decode) to offset (prefill-length blocks) is
 * taken; L is the number of trailing cache rows the query block stands for.
 * Kernels: from 96 query rows per kv head (H_q / H_kv x L) over a bf16 or
 * fp16 cache with 4-bit K codes in groups of 64 or 128 (head_dim 64, 128 or 256, 2- to 4-bit
 * V codes) a prefill kernel (blocks of 128 query rows sharing each decoded
 * 32-key tile, key splits merged as for the dedicated kernel); otherwise
 * the default configuration (head_dim 256, group 64, K4/V3) runs a dedicated
 * kernel (blocks of 8 query rows per kv head) and every other configuration
 * the general tile kernel (one wave per workgroup up to 8 query rows per kv
 * head, and up to 16 at head_dim 64 or 128 or in groups of 32 at head_dim
 * 256; else blocks of 64 query rows against 32-key tiles decoded once per
 * workgroup).  The choice depends only on the cache descriptor, H_q, L and
 * splits, so rbq_quant_attn_splits and rbq_quant_attn_workspace_bytes
 * describe the call.  With RBQ_FLAG_ROUND_ROTATED in the cache flags the rotated q
 * is rounded to the dtype.  Errors: RBQ_EINVAL (null pointers, H_q % H_kv !=
 * 0, splits < 0), RBQ_ERANGE (L < 1 or L > offset), RBQ_EWORKSPACE,
 * RBQ_EUNSUPPORTED, RBQ_EHIP.
 */
int rbq_quant_attn_decode(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L,
                          float scale, int32_t causal, const float* rot_blocks, float* out,
                          int32_t splits, void* ws, size_t ws_bytes, void* stream);

/*
 * rbq_kv_append_attn_decode - one decode (or verify) step: rbq_kv_quant_append
 * of n rows followed by rbq_quant_attn_decode over the cache that results,
 * with the same rot_blocks (the cache update of update_and_fetch and
 * asym_quantized_sdpa on the quant_kv.py page, as one decoding step runs
 * them).  The cache rows written, c->offset and out are what those two calls
 * give, bit for bit.
 *   k, v, n     as rbq_kv_quant_append (k, v may be NULL when n == 0).
 *   q ... ws    as rbq_quant_attn_decode, for the cache after the append:
 *               L <= offset + n, and ws_bytes >= rbq_quant_attn_workspace_bytes
 *               of a descriptor whose offset is offset + n.
 * In the default configuration with 1 <= n <= 8 (k and v 8-byte aligned)
 * the attention kernel quantizes and writes the n rows itself: the
 * workgroups whose key range holds a row (one per block of 8 query rows of
 * the kv head) each write it, the same bytes, before reading it; one launch
 * fewer than the two calls.  Otherwise the two calls run as they are.  Every argument is
 * checked before anything is launched; on error nothing is written and
 * c->offset is unchanged.  Errors: those of both calls.
 */
int rbq_kv_append_attn_decode(rbq_kv_cache* c, const void* k, const void* v, int64_t n,
                              const void* q, int32_t H_q, int32_t L, float scale, int32_t causal,
                              const float* rot_blocks, float* out, int32_t splits, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * rbq_quant_attn_decode_noalloc - rbq_quant_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * split records live in a fixed device array of RBQ_SCRATCH_BYTES, one per
 * device, whose address the library takes (hipGetSymbolAddress) on the first
 * call on each device; the call itself allocates nothing.  Arguments,
 * kernels and results are those of rbq_quant_attn_decode with the same
 * splits (out is bit for bit the same).  The array keeps the last call's
 * contents and nothing in it needs clearing, but every call on one device
 * shares it: calls whose device work overlaps in time on one device (other
 * streams, other threads) race and must be serialised by the caller.
 * Errors: as rbq_quant_attn_decode, and RBQ_ESCRATCH when the call needs
 * more than RBQ_SCRATCH_BYTES of split records
 * (rbq_quant_attn_workspace_bytes tells; nothing is launched then).
 */
int rbq_quant_attn_decode_noalloc(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L,
                                  float scale, int32_t causal, const float* rot_blocks,
                                  float* out, int32_t splits, void* stream);

/* ---- attention mask element types (rbq_quant_attn_decode_mask) ---- */
#define RBQ_MASK_NONE      0
#define RBQ_MASK_BOOL      1  /* uint8: nonzero = the key is attended, 0 = skipped          */
#define RBQ_MASK_ADD_F32   2  /* float32 added to the scaled scores before the softmax      */
#define RBQ_MASK_ADD_DTYPE 3  /* the same in the cache dtype (fp16 / bf16)                 */

/*
 * rbq_quant_attn_decode_mask - rbq_quant_attn_decode with an array mask over
 * (query row, key), as asym_quantized_sdpa on the quant_kv.py page takes one
 * (a boolean mask keeps a score where true; an additive one is added to the
 * scaled scores), for batched verification of several draft paths.
 *   mask         device array or NULL (then mask_type must be RBQ_MASK_NONE
 *                and the call equals rbq_quant_attn_decode).  Element
 *                (b, q head h, query row i, key t) is at mask + b*mask_stride_b
 *                + h*mask_stride_h + i*mask_stride_l + t, in elements of the
 *                mask type; keys t in [0, offset) are read; a stride of 0
 *                broadcasts.  Strides are >= 0 and the elements read must lie
 *                in the first 2^31 - 256 bytes (else RBQ_EUNSUPPORTED).
 *   causal       applies as well when nonzero (both must keep a key).
 * A query row whose every key the boolean mask skips gives, as the page's
 * fill of skipped scores with the dtype's minimum does, the mean of the
 * dequantized values of its keys (those the causal rule leaves it, else all
 * offset keys), with equal weights, rotated back; a skipped key next to a
 * kept one has weight 0.  Errors: as rbq_quant_attn_decode, and RBQ_EINVAL
 * for a bad mask type or negative stride.
 */
int rbq_quant_attn_decode_mask(const rbq_kv_cache* c, const void* q, int32_t H_q, int32_t L,
                               float scale, int32_t causal, const void* mask, int32_t mask_type,
                               int64_t mask_stride_b, int64_t mask_stride_h,
                               int64_t mask_stride_l, const float* rot_blocks, float* out,
                               int32_t splits, void* ws, size_t ws_bytes, void* stream);

/* Static, human-readable name of a status code. */
const char* rbq_status_string(int status);

/* hipError_t of the last failed HIP call on this thread (0 if none). */
int rbq_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RBQ_H */
