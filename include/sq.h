/*
 * sq.h -- C ABI of libsq: the fused quantized gated delta-rule decode step
 * over a per-request pool of low-bit recurrent states, for AMD MI355X (gfx950).
 *
 * Sources (cited by title and section):
 *   [P1] "K1 論文詳解" (k1-news, paper of 2026-10-09), STEPQuant article,
 *        sections 背景 (background), 方法 (method), 實驗結果 (results).
 *   [P5] "线性注意力状态量化难题:Qwen状态池70并发就超模型权重" (aitest123),
 *        sections 直接量化为什么会翻车, 时间维度, 空间维度, 工程落地.
 *
 * What one decode step computes, per request n (owning slot p = slot_ids[n])
 * and head h, on that head's d_k x d_v state S (rows = key dims, columns =
 * value dims, [P5] 空间维度):
 *     S^ = decode(tile(p, h))                   stored codes -> real state
 *     u  = S^T k
 *     S' = alpha S^ + beta k (v - alpha u)^T    = alpha (I - beta k k^T) S^ + beta k v^T
 *     o  = S'^T q                                readout, before requantization
 *     tile(p, h) = encode(S')                    requantize + repack, in place
 * The update is the gated delta rule ([P5] opening and 时间维度: decay by the
 * gate, correction along the current key); every step reads, updates,
 * requantizes and stores the state ([P5] 直接量化为什么会翻车).
 *
 * STATE FORMAT (public; the CPU reference implements it independently)
 *   head_bits[h] selects the storage of head h:
 *     4, 6, 8  integer codes q in [-Q, Q], Q = 2^(b-1) - 1 ([P5]
 *              直接量化为什么会翻车: 4/6/8-bit integers), stored as the
 *              unsigned field q + 2^(b-1);
 *     16       FP16 "pivot" head, IEEE binary16, unquantized ([P1] 方法;
 *              [P5] 时间维度: the riskiest heads stay FP16);
 *     32       FP32 state, unquantized (the full-precision baseline path);
 *     144      (SQ_BITS_BF16) bfloat16 state, unquantized, 16-bit fields: a
 *              16-bit baseline beside the FP32 state, not a format of the
 *              pages; S' is rounded to bfloat16 (half to even).
 *   Dequantization uses a per-key-row factor times a per-value-column factor
 *   ([P5] 空间维度; [P1] 方法): S^_ij = q_ij * s_ij, s_ij = fl32(r_i * c_j).
 *   Requantization: q = clamp(rne(S'_ij / s_ij), -Q, Q) (round half to even).
 *   FP16 pivots round S' to binary16 (half to even).
 *   Tile layout: element (i, j) is field number
 *       n = 16 * ((i/4) * (d_v/4) + j/4) + 4 * (j%4) + (i%4)
 *   (4x4 blocks in block-row order; inside a block the four rows of a column
 *   are consecutive), and field n occupies bits [n*w, n*w + w) of the tile
 *   read as a little-endian bit stream, w = head_bits[h] (16 for
 *   SQ_BITS_BF16).  So 4-bit codes sit
 *   two per byte and 6-bit codes four per three bytes; a tile is
 *   d_k*d_v*w/8 bytes.  A slot's slab holds heads 0..H-1 in order, each tile
 *   starting on a 256-byte boundary; slot p's slab starts at p * slab_bytes.
 *
 * CONVENTIONS
 *   - Every function returns an sq_status (int); nothing throws across the ABI.
 *   - Host-checkable argument errors are reported before any HIP call is made.
 *   - Device pointers are borrowed: the caller allocates and frees them (for
 *     example as torch tensors).  The library owns only the sq_pool object and
 *     the small device tables it allocates in sq_pool_alloc.
 *   - All device work is enqueued on the caller's stream (a hipStream_t passed
 *     as void*, NULL = the null stream); no call synchronizes.  Results are
 *     visible after the caller synchronizes that stream.  Calls that touch the
 *     same pool must be ordered on one stream.
 *   - A pool lives on the device that was current at sq_pool_alloc.  Calls
 *     that enqueue work on it must be made with that device current (else
 *     SQ_ERR_INVALID, nothing enqueued); sq_pool_free switches to it itself.
 *   - A slot must not appear twice in one slot_ids batch: two workgroups would
 *     update the same tile (undefined result).  The step does not check slot
 *     ids on the device; sq_check_slots does, as a separate call, and the
 *     SQ_CHECK switch below makes every call check them on the host.
 *   - Non-finite inputs (alpha, beta, q, k, v, scales) are a caller error.  The
 *     result is defined on the updated value as the kernel evaluates it: a
 *     NaN quotient S'/s becomes code 0, +-Inf the nearest bound +-Q; FP16,
 *     BF16 and FP32 heads store the non-finite value.  The pages say nothing
 *     of non-finite values; this rule is a reading.  A NaN or infinite gate,
 *     write strength, key or value element gives the same stored result
 *     in any evaluation order; an infinite gate does not (its codes are
 *     then unspecified within [-Q, Q]).  A non-finite query only reaches the
 *     readout o.  Whenever a stored value comes from a non-finite one, the
 *     pool's sticky flag is set (sq_pool_last_device_error).  The d = 128
 *     code-tile kernel takes that decision on the update's factors (the
 *     gate, beta k_i / r_i, (v_j - alpha u_j) / c_j), the others on each
 *     value; the two agree unless finite factors overflow fp32 in their
 *     product, which takes step sizes near the bottom of the fp32 range.
 *   - d_k and d_v must be multiples of 4 and at most 256; d_k = d_v = 128 takes
 *     the tuned kernels, other shapes a plain one.
 *
 * SWITCHES (environment variables, read once per pool by sq_pool_alloc; a
 * pool keeps what it read)
 *   SQ_CHECK   set and not "0": every call that takes slot ids (store, load,
 *              step, per-channel step, readout) first copies the ids to the
 *              host, synchronizing the caller's stream, and returns
 *              SQ_ERR_INVALID before any kernel is enqueued if an id is
 *              outside [0, n_slots) or, for the calls that write the pool
 *              (store and both steps), appears twice.  A debugging aid: it
 *              costs a synchronization per call and cannot be used under
 *              graph capture.
 *   SQ_KERNEL  unset, empty or "tuned": d_k = d_v = 128 takes the tuned
 *              kernels.  "generic": every shape takes the plain per-width
 *              kernels, so that the tuned ones can be checked against a second
 *              implementation on the same data.  Any other value makes
 *              sq_pool_alloc return SQ_ERR_INVALID (before any HIP call).
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct sq_pool sq_pool; /* opaque handle */

#define SQ_BITS_BF16 144 /* head_bits value of a bfloat16 state */

typedef enum {
    SQ_OK = 0,
    SQ_ERR_INVALID = -1,     /* null pointer, bad size, misaligned pointer, buffer too small */
    SQ_ERR_UNSUPPORTED = -2, /* head_bits not in {4,6,8,16,32,144}, or d_k/d_v not supported */
    SQ_ERR_HIP = -3,         /* a HIP runtime call or kernel launch failed */
    SQ_ERR_NOMEM = -4,       /* host or device allocation of the pool's tables failed */
    SQ_ERR_DEVICE = -5       /* sq_pool_last_device_error: a kernel met a non-finite value */
} sq_status;

typedef enum {
    SQ_F32 = 0, /* IEEE binary32 */
    SQ_BF16 = 1 /* bfloat16, upcast exactly to fp32 on load */
} sq_dtype;

typedef struct {
    int32_t n_slots;          /* number of resident request states (slots), >= 1 */
    int32_t n_heads;          /* recurrent heads per request, >= 1 */
    int32_t d_k, d_v;         /* state rows (key dims) and columns (value dims) */
    const uint8_t *head_bits; /* HOST [n_heads], each in {4, 6, 8, 16, 32, 144}; copied */
    const float *row_scale;   /* DEVICE fp32, r_i > 0: [n_heads][d_k], or with a slot stride
                                 S the factors of slot p, head h at row_scale + (p*S + h)*d_k;
                                 borrowed, read by every call; entries of unquantized heads
                                 are ignored */
    const float *col_scale;   /* DEVICE fp32, c_j > 0: [n_heads][d_v], or at
                                 col_scale + (p*S + h)*d_v; as row_scale */
    int64_t scale_slot_stride;/* S: 0 = one set of factors per head, shared by every slot;
                                 else S >= n_heads and every slot has its own factors
                                 ([P5] 空间维度: each row and each column of a state matrix
                                 has its own factor); the arrays then hold n_slots*S vectors */
    void *state;              /* DEVICE, 256-byte aligned, >= sq_pool_bytes(...) bytes,
                                 laid out as described above; borrowed */
    uint64_t state_bytes;     /* size of the state buffer in bytes */
} sq_pool_desc;

/* Bytes the state buffer needs for this shape: n_slots * slab_bytes.  One
 * resident state per request slot ([P1] 背景; [P5] opening: the pool grows
 * with concurrency), each head stored at its own width ([P5] 时间维度).
 * Returns 0 if any argument is invalid or unsupported.  Host only. */
uint64_t sq_pool_bytes(int32_t n_slots, int32_t n_heads, int32_t d_k, int32_t d_v,
                       const uint8_t *head_bits);

/* Validate desc, compute the tile offsets and upload them (and the per-width
 * head lists) to a small device table: the per-request state pool ([P1] 背景;
 * [P5] opening) with per-head widths and FP16 pivots ([P5] 时间维度) and
 * row x column factors ([P5] 空间维度).  On success *out receives a handle to
 * release with sq_pool_free.  Errors: SQ_ERR_INVALID (null desc/out/pointers,
 * n_slots or n_heads < 1, state not 256-byte aligned, scales not 16-byte
 * aligned, state_bytes too small, 0 < scale_slot_stride < n_heads, an
 * SQ_KERNEL value that names no kernel family), SQ_ERR_UNSUPPORTED (bits, d_k,
 * d_v), SQ_ERR_NOMEM, SQ_ERR_HIP.
 * Synchronous (uploads with a blocking copy). */
int sq_pool_alloc(const sq_pool_desc *desc, sq_pool **out);

/* Release the handle and its device table (not the borrowed buffers).
 * NULL is a no-op.  The caller must ensure no enqueued work still uses it. */
void sq_pool_free(sq_pool *pool);

/* Byte offset and size of tile (slot, head) inside the state buffer.
 * Host only; SQ_ERR_INVALID for a null pool/out pointer or out-of-range ids. */
int sq_pool_tile_offset(const sq_pool *pool, int32_t slot, int32_t head, uint64_t *offset,
                        uint64_t *bytes);

/* Quantize-and-store: encode fp32 states S (DEVICE, [n_req][n_heads][d_k][d_v],
 * row-major) into the tiles of slots slot_ids[0..n_req) (DEVICE int32), with
 * the quantizer and layout above (the hand-off of a state computed elsewhere,
 * e.g. at prefill).  n_req == 0 is a no-op.  Asynchronous on `stream`.
 * Errors as for sq_decode_step (S must be 16-byte aligned). */
int sq_pool_store(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const float *S,
                  void *stream);

/* Load-and-dequantize, the inverse of sq_pool_store: write the states of slots
 * slot_ids[0..n_req) (DEVICE int32) as fp32 S[n_req][n_heads][d_k][d_v]
 * (DEVICE, row-major, 16-byte aligned).  Each element is the stored value
 * rounded once to fp32: fl32(q * fl32(r_i c_j)) for codes, the binary16 value
 * for pivots, the stored value for FP32 heads.  The pool is not modified.
 * n_req == 0 is a no-op.  Asynchronous on `stream`.  (Calibration,
 * checkpoint export, inspection.)  Errors as for sq_pool_store. */
int sq_pool_load(const sq_pool *pool, const int32_t *slot_ids, int32_t n_req, float *S,
                 void *stream);

/* One fused decode step for a batch of n_req requests (see the top of this
 * file).  All pointers DEVICE, row-major:
 *   slot_ids int32 [n_req], each in [0, n_slots), no duplicates;
 *   q, k     [n_req][n_heads][d_k] of qkv_dtype (sq_dtype);
 *   v        [n_req][n_heads][d_v] of qkv_dtype;
 *   alpha, beta fp32 [n_req][n_heads] (gate in (0, 1], write strength in [0, 1]);
 *   o        fp32 [n_req][n_heads][d_v], written with S'^T q; may be NULL.
 * q/k/v/o must be 16-byte aligned.  The pool's tiles are updated in place.
 * n_req == 0 is a no-op.  Asynchronous on `stream`.
 * Errors: SQ_ERR_INVALID (null pool or required pointer, n_req < 0 or
 * > n_slots, qkv_dtype not an sq_dtype, misaligned pointer, another device
 * current), SQ_ERR_UNSUPPORTED (n_req * n_heads tiles exceed one launch
 * grid), SQ_ERR_HIP (a launch failed).  Device data (slot values, alpha,
 * beta, q/k/v) is not validated; see sq_check_slots for slot ids, and the
 * SQ_CHECK switch, under which an id out of range or repeated is
 * SQ_ERR_INVALID (the load and the readout accept repeated ids). */
int sq_decode_step(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
                   const void *k, const void *v, int32_t qkv_dtype, const float *alpha,
                   const float *beta, float *o, void *stream);

/* The same step with a per-key-channel gate, for the second model family
 * ([P5] 直接量化为什么会翻车 names its gate KDA; the pages give no formula).
 * Reading taken: the gate is a vector alpha in (0, 1]^{d_k} that decays each
 * key row of the state before the delta correction,
 *     T  = diag(alpha) S^,   u = T^T k
 *     S' = T + beta k (v - u)^T  = (I - beta k k^T) diag(alpha) S^ + beta k v^T
 *     o  = S'^T q,           tile = encode(S')
 * which is sq_decode_step when all d_k entries of alpha are equal.  Arguments
 * as for sq_decode_step except
 *   alpha    fp32 [n_req][n_heads][d_k], DEVICE, 16-byte aligned.
 * Same errors; n_req == 0 is a no-op.  Asynchronous on `stream`. */
int sq_decode_step_kda(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
                       const void *k, const void *v, int32_t qkv_dtype, const float *alpha,
                       const float *beta, float *o, void *stream);

/* Readout without update ([P5] 空间维度: the head's output is the query read
 * out of the state): o = S^T q from the stored state (dequantized), for
 * slots slot_ids[0..n_req).  q: DEVICE [n_req][n_heads][d_k] of q_dtype;
 * o: DEVICE fp32 [n_req][n_heads][d_v].  Does not modify the pool.  n_req == 0
 * is a no-op.  Asynchronous on `stream`.  Errors as for sq_decode_step (q and
 * o required, 16-byte aligned). */
int sq_readout(const sq_pool *pool, const int32_t *slot_ids, int32_t n_req, const void *q,
               int32_t q_dtype, float *o, void *stream);

/* Device-side check of a batch's slot ids, for callers that cannot vouch for
 * them (the step does not check them; a repeated id makes two workgroups
 * update one tile).  Each request owns one resident state ([P1] 背景, [P5]
 * opening), so a valid batch names distinct slots in [0, n_slots).
 * Writes to *result (DEVICE int32, 4-byte aligned) 0 if the batch is valid,
 * otherwise a bit set: 1 = some id outside [0, n_slots), 2 = some id repeated.
 * slot_ids: DEVICE int32 [n_req]; n_req == 0 writes 0.  Uses per-slot stamps
 * and a generation counter in the pool's device table (no host state), so the
 * call can be captured in a HIP graph and replayed; calls on one pool must be
 * stream-ordered.
 * Errors: SQ_ERR_INVALID (null pool/result, negative n_req, misaligned
 * result), SQ_ERR_HIP.  Asynchronous on `stream`: read *result after
 * synchronizing it. */
int sq_check_slots(sq_pool *pool, const int32_t *slot_ids, int32_t n_req, int32_t *result,
                   void *stream);

/* The slot check of sq_check_slots for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation): it needs no pool, and keeps its per-slot stamps and
 * generation counter in a fixed array inside the library (one per GPU, about
 * 256 KB, held until the process ends) instead of a pool's table.  Nothing is
 * allocated, by this call or by anything it calls.
 * slot_ids: DEVICE int32 [n_req], checked against [0, n_slots); *result
 * (DEVICE int32, 4-byte aligned) receives 0, or 1 (an id out of range) | 2
 * (an id repeated), as for sq_check_slots.  n_slots must be at most
 * SQ_CHECK_NOALLOC_MAX_SLOTS.  n_req == 0 writes 0.
 * All calls on one GPU share that GPU's array: calls made on one GPU must not
 * overlap in time (order them on one stream), or their results race.
 * Errors: SQ_ERR_INVALID (null result, negative n_req, n_slots < 1, null
 * slot_ids with n_req > 0, misaligned result), SQ_ERR_UNSUPPORTED (n_slots
 * above the limit), SQ_ERR_HIP.  Asynchronous on `stream`. */
#define SQ_CHECK_NOALLOC_MAX_SLOTS 65536
int sq_check_slots_noalloc(const int32_t *slot_ids, int32_t n_req, int32_t n_slots, int32_t *result,
                           void *stream);

/* Read and clear the pool's sticky device flag.  The step, the per-channel-
 * gate step and the store set it when an updated value (the quotient S'/s for
 * codes, S' for unquantized heads) is not finite, which only non-finite or
 * huge inputs cause; the stored result then follows the rule above (NaN ->
 * code 0, +-Inf -> +-Q).  Synchronizes `stream` first (host-blocking).
 * Returns SQ_OK if no such value was met since the pool was made or the flag
 * last read, SQ_ERR_DEVICE if one was; SQ_ERR_INVALID (null pool, another
 * device current), SQ_ERR_HIP. */
int sq_pool_last_device_error(sq_pool *pool, void *stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *sq_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
