/*
 * moda.h -- C ABI of libmoda: the Mixture-of-Depths Attention (MoDA) forward
 * on AMD Instinct MI355X (gfx950).
 *
 * The operation (hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths
 * Attention (MoDA)"; chatpaper.ai abstract): every query row (b, h, t) takes
 * one softmax, scaled by 1/sqrt(d), over
 *   - the causal sequence keys K[b, g, j, :] for j = 0..t of the current layer,
 *   - the token's own L depth keys Kd[b, g, t, i, :], i = 0..L-1, written by
 *     the preceding layers (same page, section "Depth stream mechanism"),
 * where g = h / G and G = Hq / Hkv query heads share one KV head (section
 * "Hardware-efficient implementation" names G the GQA group count).  The
 * output row is the weight-averaged matching values V and Vd.  Sequence and
 * depth logits feed one online-softmax state and are normalised once
 * (section "Hardware-efficient implementation").
 *
 * Tensors (all contiguous, row-major, device memory unless stated):
 *   Q   [B, Hq,  T, d]          element type = shape.dtype
 *   K,V [B, Hkv, T, d]          element type = shape.dtype
 *   Kd,Vd [B, Hkv, T, L, d]     element type = shape.dtype
 *   O   [B, Hq,  T, d]          element type = shape.dtype (bf16: round to
 *                               nearest even from the fp32 result)
 *   LSE [B, Hq,  T]   float32   natural-log normaliser of each row (optional)
 *
 * Conventions shared by every entry point:
 *   - Ownership: the caller allocates every buffer and keeps it alive until
 *     the stream has finished the enqueued work.  The library allocates no
 *     device memory and keeps no pointer after returning.
 *   - Asynchrony: work is enqueued on `hip_stream` (a hipStream_t; NULL is
 *     the null stream) and the call returns without synchronising.
 *   - Validation happens on the host before anything is enqueued; on any
 *     error nothing is enqueued.  Errors are returned as moda_status, never
 *     by abort or exception; moda_last_error() gives the detail (per thread).
 *   - Device pointers must be 16-byte aligned.
 *   - Thread safety: every call is thread-safe.
 *   - Logging: with MODA_LOG set (to anything but "0") in the environment when
 *     the library is first used, every call that enqueues work prints one line
 *     to stderr as it returns: the entry point, the shape, the kernel variant
 *     the shape selects (moda_fwd_variant) and "ok" or the error text.
 */
#ifndef MODA_H_
#define MODA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MODA_OK = 0,
  MODA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, ... */
  MODA_ERR_UNSUPPORTED = 2, /* valid but not implemented (e.g. head dim) */
  MODA_ERR_HIP = 3          /* the HIP runtime reported an error */
} moda_status;

typedef enum { MODA_F32 = 0, MODA_BF16 = 1 } moda_dtype;

/* Problem shape.  Requirements: B, Hq, Hkv, T >= 1; L >= 0; Hq % Hkv == 0;
 * d in {32, 64, 128}; every tensor has fewer than 2^62 elements. */
typedef struct {
  int64_t B, Hq, Hkv, T, L, d;
  int32_t dtype; /* a moda_dtype */
} moda_shape;

/* Host-only shape check (no device work).  MODA_OK if every entry point
 * accepts `s`, otherwise the reason.  Safe to call without a GPU. */
moda_status moda_check_shape(const moda_shape *s);

/* Bytes the packed depth cache of shape `s` occupies; 0 if `s` is invalid or
 * has L == 0.  Host only. */
size_t moda_depth_cache_bytes(const moda_shape *s);

/* Repack the depth stream into the layout moda_fwd streams.
 *
 * Passage: hyper.ai page on arXiv 2603.15619, section "Hardware-efficient
 * implementation": the depth cache is reorganised so that the queries of one
 * chunk (and all G heads of a KV group) read one contiguous depth span.
 *
 *   k_depth, v_depth : Kd, Vd [B, Hkv, T, L, d] (read only)
 *   packed           : output, packed_bytes >= moda_depth_cache_bytes(s)
 * The packed format is opaque: a pure function of (shape, library version),
 * bit-exact copies of the inputs plus zero padding.  (In this version, for bf16
 * with d = 128: per (b, kv head), blocks of 8 consecutive tokens x 4
 * consecutive entries in MFMA operand order, so a query tile's tokens read one
 * contiguous run of blocks and a single entry of every token can be written in
 * whole 16-byte chunks.)  Pass the identical shape to moda_fwd.  Requires
 * L >= 1.
 */
moda_status moda_pack_depth_cache(const moda_shape *s, const void *k_depth,
                                  const void *v_depth, void *packed,
                                  size_t packed_bytes, void *hip_stream);

/* Depth-stream write: store n new depth entries of every token, entries
 * [first, first + n) of each token's L, into a packed depth cache in place.
 *
 * Passage: hyper.ai page on arXiv 2603.15619, section "Depth stream
 * mechanism": after a layer runs, the keys and values it produced join every
 * token's depth stream for the layers above; FFN layers add a light KV
 * projection of their own, so one layer may write two entries.
 *
 *   first, n     : the entries written, 0 <= first, n >= 1, first + n <= L
 *   k_new, v_new : [B, Hkv, T, n, d] (read only): entry first + i of token t
 *                  of (b, kv head) g is k_new[b, g, t, i, :]
 *   packed       : a cache of shape `s` (L = the stream's capacity per
 *                  token), packed_bytes >= moda_depth_cache_bytes(s).  Only
 *                  the bytes of the written entries change.
 * A cache that moda_pack_depth_cache wrote, or a zero-filled buffer, is a
 * valid start: a zero-filled cache after writes of all L entries equals
 * moda_pack_depth_cache of the same entries, byte for byte.  Entries not yet
 * written hold whatever the start held (zeros, for a zero-filled one) and
 * take part in moda_fwd like any other.  Requires L >= 1.  Same validation,
 * ownership and asynchrony rules as moda_pack_depth_cache. */
moda_status moda_append_depth(const moda_shape *s, int64_t first, int64_t n,
                              const void *k_new, const void *v_new, void *packed,
                              size_t packed_bytes, void *hip_stream);

/* MoDA forward: O (and optionally LSE) from Q, the sequence K/V and the
 * packed depth cache.
 *
 * Passage: hyper.ai page on arXiv 2603.15619, sections "Mixture-of-Depths
 * Attention (MoDA)" and "Hardware-efficient implementation".
 *
 *   q, k, v : Q, K, V as above (read only)
 *   packed  : from moda_pack_depth_cache with the same shape; must be NULL
 *             (and packed_bytes 0) when L == 0
 *   out     : O, written in full (no row is left unwritten)
 *   lse     : NULL, or LSE [B, Hq, T] float32 written in full
 * With L == 0 the result is causal grouped-query attention.
 */
moda_status moda_fwd(const moda_shape *s, const void *q, const void *k,
                     const void *v, const void *packed, size_t packed_bytes,
                     void *out, float *lse, void *hip_stream);

/* Causal-only attention: moda_fwd without the depth part (L is ignored).
 * The in-house FlashAttention-style reference that MoDA is compared with
 * (the hyper.ai page, section "Main contributions", and the chatpaper.ai
 * abstract compare MoDA's kernel with FlashAttention-2 at 64K tokens).
 * Arguments as in moda_fwd. */
moda_status moda_causal_fwd(const moda_shape *s, const void *q, const void *k,
                            const void *v, void *out, float *lse,
                            void *hip_stream);

/* MoDA forward reading the depth keys and values in their natural layout
 * [B, Hkv, T, L, d] instead of the packed cache: the same result as
 * moda_fwd up to the rounding order of the depth terms (it visits a row's
 * depth entries in other blocks), without a repack.  It measures whether the packed
 * layout earns its repack (the hyper.ai page on arXiv 2603.15619, section
 * "Hardware-efficient implementation", motivates its chunk- and group-aware
 * depth layouts by the cost of non-contiguous depth reads).
 *
 *   q, k, v          : as for moda_fwd (read only)
 *   k_depth, v_depth : depth K, V [B, Hkv, T, L, d] (read only; NULL if L == 0)
 *   out, lse         : as for moda_fwd
 * Supports bf16 with d = 128 and T * L below 2^23 (MODA_ERR_UNSUPPORTED
 * otherwise).  Same validation, ownership and asynchrony rules as moda_fwd. */
moda_status moda_fwd_natural(const moda_shape *s, const void *q, const void *k,
                             const void *v, const void *k_depth, const void *v_depth,
                             void *out, float *lse, void *hip_stream);

/* MoDA forward reading the depth stream in layer-major order: entry i of
 * every token is one contiguous tensor [B, Hkv, T, d], the keys (values)
 * that layer i of the stack produced.  The depth stream then needs no write
 * step of its own: a layer's K/V projection writes straight into its slice,
 * and the forward of layer l passes the first l slices with L = l (hyper.ai
 * page on arXiv 2603.15619, section "Depth stream mechanism": the stream
 * grows by what each layer writes, and later layers read all of it).
 * Results are the same as moda_fwd_natural's on the same entries, bit for bit.
 *
 *   q, k, v            : as for moda_fwd (read only)
 *   k_layers, v_layers : depth K, V [L, B, Hkv, T, d] (read only; NULL if L == 0);
 *                        slices past L may exist and are not read
 *   out, lse           : as for moda_fwd
 * Supports bf16 with d = 128 and T * L below 2^23 (MODA_ERR_UNSUPPORTED
 * otherwise).  Same validation, ownership and asynchrony rules as moda_fwd. */
moda_status moda_fwd_layers(const moda_shape *s, const void *q, const void *k,
                            const void *v, const void *k_layers, const void *v_layers,
                            void *out, float *lse, void *hip_stream);

/* Layout ablation: the MoDA forward with the depth stream handled the way a
 * FlashAttention-style kernel would see it without a depth-aware layout: the
 * flattened (token, entry) axis is one causal key range that every query
 * tile scans from entry 0 up to its last token's entries, with a mask that
 * keeps each row's own token's L entries only (hyper.ai page on arXiv
 * 2603.15619, section "Hardware-efficient implementation", names this
 * Flash-compatible layout and the waste of its masked, out-of-range entries).
 * The result equals moda_fwd_natural's bit for bit; only the work differs
 * (about T / (2 * 256 / G) times the depth traffic).  For measurement.
 *
 * Arguments, validation and limits as for moda_fwd_natural; requires L >= 1. */
moda_status moda_fwd_masked_scan(const moda_shape *s, const void *q, const void *k,
                                 const void *v, const void *k_depth, const void *v_depth,
                                 void *out, float *lse, void *hip_stream);

/* MoDA forward reading depth K and V rows at caller-given strides: row
 * (b, g, t, i) of each (the i-th depth entry of token t of KV head g of
 * sequence b) starts at element ((b * Hkv + g) * stride_bh + t * stride_t +
 * i * stride_i) * d of k_depth (v_depth), for i < L.  moda_fwd_layers is the
 * case (T, 1, B * Hkv * T); a natural-layout stream with room for Lcap
 * entries per token, [B, Hkv, T, Lcap, d] of which the first L are written,
 * is (T * Lcap, Lcap, 1).  Either lets each layer write its entry in place
 * and the next layer read the stream as it stands (hyper.ai page on arXiv
 * 2603.15619, section "Depth stream mechanism").  Results are the same as
 * moda_fwd_natural's on the same entries, bit for bit; rows outside the L entries are
 * never read.
 *
 * Strides are in rows of d elements, each >= 0; every addressed row must lie
 * inside the caller's buffers.  Supports bf16 with d = 128 and T * L below
 * 2^23.  Same validation, ownership and asynchrony rules as moda_fwd. */
moda_status moda_fwd_strided(const moda_shape *s, const void *q, const void *k,
                             const void *v, const void *k_depth, const void *v_depth,
                             int64_t stride_bh, int64_t stride_t, int64_t stride_i,
                             void *out, float *lse, void *hip_stream);

/* Depth attention alone: each query row (b, h, t) attends over its own
 * token's L depth entries only, under one softmax scaled by 1/sqrt(d), and
 * gets their weighted values.  No sequence key takes part.
 *
 * Passage: hyper.ai page on arXiv 2603.15619, section "Depth stream
 * mechanism" (the read step of the depth stream: attention over the keys and
 * values that the preceding layers left at the same token position).
 *
 *   q      : Q [B, Hq, T, d] (read only)
 *   packed : from moda_pack_depth_cache with the same shape (read only)
 *   out    : O [B, Hq, T, d], written in full
 *   lse    : NULL, or LSE [B, Hq, T] float32 over the depth logits alone
 * Requires L >= 1 (an empty softmax has no value): MODA_ERR_INVALID_ARG
 * otherwise.  Same validation, ownership and asynchrony as moda_fwd. */
moda_status moda_depth_fwd(const moda_shape *s, const void *q, const void *packed,
                           size_t packed_bytes, void *out, float *lse,
                           void *hip_stream);

/* MoDA backward: gradients of a loss with respect to Q, K, V and the depth
 * keys and values, given dO (the loss gradient with respect to O) and the
 * forward's O and LSE.  The chain rule through the forward's one softmax over
 * sequence and depth entries (hyper.ai page on arXiv 2603.15619, section
 * "Mixture-of-Depths Attention (MoDA)"); the depth entries' gradients follow
 * the same rule with their own token's rows only.
 *
 *   q, k, v          : as for moda_fwd (read only)
 *   k_depth, v_depth : depth K, V [B, Hkv, T, L, d] (read only; NULL if L == 0)
 *   packed           : the packed depth cache of the same shape (NULL if L == 0);
 *                      validated, not read: the gradients read k_depth and
 *                      v_depth
 *   out, lse         : O and LSE written by moda_fwd for these inputs (read only)
 *   dout             : dO [B, Hq, T, d] (read only)
 *   dq               : dQ [B, Hq, T, d], written in full
 *   dk, dv           : dK, dV [B, Hkv, T, d], written in full (summed over the
 *                      G query heads of each KV head)
 *   dk_depth, dv_depth: dKd, dVd [B, Hkv, T, L, d], written in full (NULL if L == 0)
 *   delta            : scratch [B, Hq, T] float32 that the call overwrites
 * Gradients are bf16 (fp32 accumulation).  Supports bf16 with d = 128,
 * G = Hq / Hkv up to 64 (up to 32 when L > 0), G * T below 2^23 and T * L
 * below 2^23 (MODA_ERR_UNSUPPORTED otherwise).  Same validation, ownership
 * and asynchrony rules as moda_fwd. */
moda_status moda_bwd(const moda_shape *s, const void *q, const void *k, const void *v,
                     const void *k_depth, const void *v_depth, const void *packed,
                     size_t packed_bytes, const void *out, const float *lse,
                     const void *dout, void *dq, void *dk, void *dv, void *dk_depth,
                     void *dv_depth, float *delta, void *hip_stream);

/* Bytes of device workspace moda_bwd_ws uses for shape `s`: nonzero when the
 * shape's dK/dV work would not fill the GPU (few KV heads times keys), in which
 * case moda_bwd_ws splits each key range's query rows over several workgroups
 * and adds their fp32 partial sums; 0 when no split pays, or when moda_bwd
 * does not accept `s`.  Host only. */
size_t moda_bwd_workspace_bytes(const moda_shape *s);

/* The MoDA backward of moda_bwd (same passage, arguments, results, limits and
 * rules), with a device workspace for its dK/dV split:
 *   workspace : device scratch of workspace_bytes >= moda_bwd_workspace_bytes(s)
 *               bytes (16-byte aligned; may be NULL when that is 0),
 *               overwritten; its contents need no initialisation and mean
 *               nothing after the call.  Two calls that overlap in time must
 *               not share one workspace.
 * A smaller workspace is MODA_ERR_INVALID_ARG.  The gradients equal moda_bwd's
 * up to the order in which dK and dV sum their fp32 terms. */
moda_status moda_bwd_ws(const moda_shape *s, const void *q, const void *k, const void *v,
                        const void *k_depth, const void *v_depth, const void *packed,
                        size_t packed_bytes, const void *out, const float *lse,
                        const void *dout, void *dq, void *dk, void *dv, void *dk_depth,
                        void *dv_depth, float *delta, void *workspace, size_t workspace_bytes,
                        void *hip_stream);

/* Bytes of device workspace moda_decode needs for shape `s`; 0 if moda_decode
 * does not accept `s`.  Host only. */
size_t moda_decode_workspace_bytes(const moda_shape *s);

/* MoDA decode step: the one new token of each sequence attends over the KV
 * cache and over its own depth entries.  Row (b, h) takes one softmax, scaled
 * by 1/sqrt(d), over the cache keys K[b, g, j, :] for j = 0..T-1 (the new
 * token's own key is the last of them, so every cached key is causal) and the
 * token's L depth keys Kd[b, g, i, :], with g = h / G; its output is the
 * weight-averaged matching values.  This is the forward's row t = T-1
 * (hyper.ai page on arXiv 2603.15619, section "Mixture-of-Depths Attention
 * (MoDA)"), evaluated without the other rows.
 *
 * Shape: `s->T` is the cache length including the new token, `s->L` the
 * number of the token's depth entries.
 *   q                : Q [B, Hq, d] of the new token (read only)
 *   k_cache, v_cache : K, V [B, Hkv, T, d] (read only)
 *   k_depth, v_depth : the new token's depth K, V [B, Hkv, L, d] (read only;
 *                      NULL if L == 0)
 *   out              : O [B, Hq, d], written in full
 *   lse              : NULL, or LSE [B, Hq] float32 (natural log)
 *   workspace        : device scratch of workspace_bytes >=
 *                      moda_decode_workspace_bytes(s) bytes, overwritten; its
 *                      contents need no initialisation and mean nothing after
 *                      the call.  Two calls that overlap in time must not share
 *                      one workspace.
 * Supports bf16 with d = 128, G = Hq / Hkv up to 32 and L below 2^23
 * (MODA_ERR_UNSUPPORTED otherwise).  Same validation, ownership and
 * asynchrony rules as moda_fwd. */
moda_status moda_decode(const moda_shape *s, const void *q, const void *k_cache,
                        const void *v_cache, const void *k_depth, const void *v_depth,
                        void *out, float *lse, void *workspace, size_t workspace_bytes,
                        void *hip_stream);

/* Decode step over caches of different lengths: as moda_decode, but sequence
 * b's cache holds cache_lens[b] entries, the first slots of its T (T is the
 * capacity; the new token's K/V is entry cache_lens[b] - 1).  Row (b, h) is
 * the forward's row t = cache_lens[b] - 1 of a sequence of that length.
 *
 *   cache_lens : device int32 [B] (read only), 4-byte aligned; values are
 *                clamped to [0, T].  A sequence of length 0 attends over its
 *                depth entries alone; with L == 0 as well its rows get O = 0
 *                and LSE = -inf.
 * The slots past a sequence's length are never read, whatever they hold.
 * Other arguments, the workspace size (moda_decode_workspace_bytes(s)) and
 * the limits are those of moda_decode. */
moda_status moda_decode_varlen(const moda_shape *s, const int32_t *cache_lens, const void *q,
                               const void *k_cache, const void *v_cache, const void *k_depth,
                               const void *v_depth, void *out, float *lse, void *workspace,
                               size_t workspace_bytes, void *hip_stream);

/* The decode step of moda_decode (cache_lens NULL: every sequence's cache
 * holds all T entries) or moda_decode_varlen (cache_lens given), with no
 * workspace argument and no allocation: for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The partial states that moda_decode keeps in the
 * caller's workspace live in a fixed device array of the library instead,
 * 8 MiB (8388608 bytes) per GPU, held from the first call on a GPU until the
 * process ends.  The call allocates nothing, neither device nor pinned host
 * memory; its first call on a GPU looks up the array's device address.
 *
 *   cache_lens : NULL, or device int32 [B] as for moda_decode_varlen
 *   q, k_cache, v_cache, k_depth, v_depth, out, lse : as for moda_decode
 * Results are those of moda_decode (moda_decode_varlen) on the same inputs,
 * bit for bit.  A shape whose partial states need more than the array holds
 * (moda_decode_workspace_bytes(s) > 8388608) is MODA_ERR_UNSUPPORTED, before
 * any launch; use moda_decode with a workspace for it.  All calls on one GPU
 * share the array: calls that overlap in time on the same GPU (other streams,
 * other threads) race and may return wrong results.  The array needs no
 * clearing: each call writes every partial state before reading it.
 * Other validation, limits, ownership and asynchrony as for moda_decode. */
moda_status moda_decode_noalloc(const moda_shape *s, const int32_t *cache_lens, const void *q,
                                const void *k_cache, const void *v_cache, const void *k_depth,
                                const void *v_depth, void *out, float *lse, void *hip_stream);

/* Static text of a status code (never NULL). */
const char *moda_status_string(moda_status st);

/* Detail of the last error returned on the calling thread ("" if none). */
const char *moda_last_error(void);

/* Kernel variant moda_fwd would launch for `s` (static text, for logging and
 * tests), or "" if `s` is invalid.  Host only.
 *   "mfma_bf16_d128_w8", "mfma_bf16_d128_w4": bf16 with d = 128, 8-wave
 *       (256-row) or 4-wave (128-row) workgroups;
 *   "mfma_bf16_d32", "mfma_bf16_d64", "mfma_f32_d32", "mfma_f32_d64",
 *   "mfma_f32_d128": the other dtypes and head dims, G up to 128, on the
 *       matrix cores;
 *   "generic": those dtypes and head dims with G above 128, one wave per
 *       query row on the vector ALUs. */
const char *moda_fwd_variant(const moda_shape *s);

#ifdef __cplusplus
}
#endif

#endif /* MODA_H_ */
