/*
 * sepattn.h — C ABI of the SepLLM separator-mask attention and SepCache
 * library for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (the pages about SepLLM, arXiv 2412.12094):
 *   [ANTH] anthology-of-the-sota record LIT-748, "Key takeaways": the mask
 *          bullet (each query sees the first a tokens, every separator so
 *          far and its n nearest tokens; the same mask in every head; the
 *          nine separator characters) and the streaming bullet (a bounded
 *          cache, 324 entries).
 *   [PITH] pith.science verdict for 2412.12094, pith_extraction.key_machinery:
 *          the binary mask M; the streaming cache of initial, separator and
 *          window blocks, in which leaving separators move to the separator
 *          cache and other leaving tokens are dropped.
 *   [HUB]  paperhub.cn author responses, second reviewer, answer A1: RoPE at
 *          positions counted inside the cache (position shifting), plain RoPE
 *          for training-length inputs.
 *
 * Conventions for every call:
 *   - Data pointers are device pointers owned by the caller (for example
 *     PyTorch tensors).  The library never allocates or frees device memory.
 *     Pointers documented as "host" are read before the call returns.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it and returns; none waits for the device.
 *   - The return value is a status code (SEPATTN_OK = 0 or a negative error).
 *     Arguments are validated before any launch; on error nothing is
 *     enqueued and sepattn_last_error() gives a description (per thread).
 *   - Floating-point tensors are bf16 (SEPATTN_BF16) or fp32 (SEPATTN_F32)
 *     where a call takes a dtype (sepattn_fwd: both; sepattn_bwd: bf16 only,
 *     SEPATTN_F32 gives SEPATTN_ENOTSUP); the SepCache is bf16.
 *     Accumulation is fp32.  Head dimension d is 64 or 128.
 *   - Indices are 0-based.  a = number of sinks (initial tokens), n = window
 *     size, which counts the query itself: row i keeps j in (i-n, i].
 */
#ifndef SEPATTN_H
#define SEPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifndef SEPATTN_API
#define SEPATTN_API __attribute__((visibility("default")))
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SEPATTN_OK = 0,
  SEPATTN_EINVAL = -1,  /* bad argument (shape, size, null pointer, range) */
  SEPATTN_ENOTSUP = -2, /* valid but unsupported (head dim, dtype, device)  */
  SEPATTN_EHIP = -3,    /* a HIP runtime call failed                        */
  SEPATTN_ESPACE = -4   /* caller-provided buffer or workspace too small    */
};

enum { SEPATTN_F32 = 0, SEPATTN_BF16 = 1 };

#define SEPATTN_MAX_SEP_IDS 64

/* Text of the last error returned on this thread ("" if none). */
SEPATTN_API const char* sepattn_last_error(void);
/* Library version, major * 10000 + minor * 100 + patch. */
SEPATTN_API int sepattn_version(void);

/* ------------------------------------------------------------------------
 * Mask metadata ([ANTH] mask bullet; [PITH] key_machinery (i)-(iii)).
 *
 * M[b,i,j] = (j <= i) and (j < a  or  i - j < n  or  f[b,j] = 1), where
 * f[b,j] = 1 iff token j of sequence b is a separator.  Nothing dense is
 * stored: the kernels work from the compacted lists below.
 *
 * "Anchors" are the keys every later row sees: sinks j < a and separators.
 * A sink whose token is a separator is a sink only (never in sep_idx).
 * ------------------------------------------------------------------------ */
typedef struct {
  int B, L;            /* sequences, tokens per sequence                        */
  int a, n;            /* sinks (a >= 0), window (n >= 1, counts the query)      */
  uint8_t* is_sep;     /* [B, L]   f[b, j]                                      */
  int32_t* sep_idx;    /* [B, L]   ascending separator positions j >= a; the
                                   tail after sep_cnt[b] entries is set to L     */
  int32_t* sep_before; /* [B, L+1] number of separators (j >= a) before position */
  int32_t* sep_cnt;    /* [B]      separators at positions >= a                 */
  int32_t* plain_idx;  /* [B, L]   ascending positions j >= a with f = 0; tail L */
  int32_t* plain_cnt;  /* [B]                                                   */
  int64_t* kept;       /* [B]      number of (i, j) with M = 1                   */
} sepattn_mask;

/* Bytes of one device buffer that sepattn_mask_carve() splits into the
 * arrays of a mask for B sequences of L tokens (256-byte aligned pieces). */
SEPATTN_API size_t sepattn_mask_bytes(int B, int L);
/* Fill m's pointers from one caller-owned device buffer of at least
 * sepattn_mask_bytes(B, L) bytes and set B, L, a, n.  No device work. */
SEPATTN_API int sepattn_mask_carve(sepattn_mask* m, int B, int L, int a, int n, void* buffer, size_t bytes);

/* Build the mask metadata from token ids.
 *   tok     device int32 [B, L], contiguous.
 *   sep_ids host int32 [n_sep], 1 <= n_sep <= SEPATTN_MAX_SEP_IDS: the token ids
 *           of the separators (the pages' nine characters, as token ids).
 *   m       metadata with B, L, a, n and all pointers set.
 * One launch; fills every array of m. */
SEPATTN_API int sepattn_build_mask(const int32_t* tok, const int32_t* sep_ids, int n_sep,
                       const sepattn_mask* m, void* stream);

/* The same metadata with fixed-interval anchors in place of separators
 * (FixLLM, [HUB] third reviewer A2: every delta-th token is kept outside the
 * window): f[b, j] = 1 iff (j + 1) mod delta == 0, for every sequence; n and
 * a as for sepattn_build_mask.  A subset of the separators is the other
 * anchor-set variant ([HUB] first reviewer A6): sepattn_build_mask with
 * those ids.  delta >= 1.  One launch. */
SEPATTN_API int sepattn_build_mask_fixed(int delta, const sepattn_mask* m, void* stream);

/* Expand the metadata into the dense mask, bit-packed: bits[b][i][w] holds
 * M[b,i,32w+t] in bit t, for w < ceil(L/32); bits past L are 0.  The kernel
 * walks each row the way the forward kernel does (gathered anchors, then the
 * band with its element test), so this checks the forward's traversal.
 * bits: device uint32 [B, L, ceil(L/32)].  For testing; L <= 65536. */
SEPATTN_API int sepattn_mask_bits(const sepattn_mask* m, uint32_t* bits, void* stream);

/* Rows per query tile of sepattn_fwd (and of the dQ pass of sepattn_bwd)
 * for window n: 64 for n <= 256, else 256.  -1 for n < 1. */
SEPATTN_API int sepattn_fwd_tile_rows(int n);

/* Per-query-tile descriptors: for the tile of rows [q0, q0 + tile_rows),
 * q0 = t * tile_rows, the keys its rows see, in the order the forward and
 * dQ kernels walk them ([ANTH] mask bullet):
 *   desc[b][t][0] sink_vis = min(a, band_lo): sinks left of the band;
 *   desc[b][t][1] sep_vis  = separators (j >= a) left of the band
 *                            (sep_before[b][band_lo]);
 *   desc[b][t][2] band_lo  = max(0, q0 - n + 1);
 *   desc[b][t][3] band_hi  = min(L, q0 + tile_rows).
 * Every key j < band_lo that some row of the tile keeps is one of those
 * sink_vis + sep_vis anchors, kept by every row of the tile; keys in
 * [band_lo, band_hi) take the element test.  The kernels derive these values
 * on the fly from sep_before with the same device code; this call writes
 * them out for checks.  desc: device int32 [B, ceil(L / tile_rows), 4];
 * tile_rows >= 1.  One launch. */
SEPATTN_API int sepattn_tile_desc(const sepattn_mask* m, int tile_rows, int32_t* desc, void* stream);

/* ------------------------------------------------------------------------
 * Attention under M (prefill / training; [ANTH] mask bullet: the mask is
 * trained through, forward and backward).
 *
 * Q, O, dO, dQ: [B, Hq, L, d]; K, V, dK, dV: [B, Hkv, L, d], addressed with
 * element strides (batch, head, token) and a contiguous last dimension.
 * Strides are multiples of 16 bytes, and the rows of one (sequence, head)
 * slice span less than 2 GiB ((L - 1) * token stride + d elements), else
 * SEPATTN_ENOTSUP: the kernels address a slice with 32-bit offsets.
 * q head h reads KV head h / (Hq / Hkv).  Inputs already carry their
 * positional encoding (plain RoPE for training-length inputs, [HUB] A1).
 * ------------------------------------------------------------------------ */
typedef struct {
  int B, Hq, Hkv, L, d;
  int64_t q_stride[3]; /* also used for dQ */
  int64_t k_stride[3]; /* also used for dK */
  int64_t v_stride[3]; /* also used for dV */
  int64_t o_stride[3]; /* also used for dO */
} sepattn_shape;

/* O = softmax(scale * Q K^T restricted to M) V; lse[b,h,i] = natural
 * log-sum-exp of row i's kept scaled scores.  dtype applies to q, k, v, o.
 * o_stride must keep the output rows apart (no two (b, h, l) rows may share
 * an element, e.g. no zero stride on a dimension of extent > 1), else
 * SEPATTN_EINVAL.
 * lse: device fp32 [B, Hq, L] contiguous, or NULL.  m must come from
 * sepattn_build_mask for the same B, L.  Every row keeps key j = i, so no row
 * is empty. */
SEPATTN_API int sepattn_fwd(const sepattn_shape* s, int dtype, const sepattn_mask* m,
                const void* q, const void* k, const void* v, float scale,
                void* o, float* lse, void* stream);

/* Workspace bytes for sepattn_bwd: fp32 D = rowsum(dO * O), [B, Hq, L], then
 * 1 KiB of counters that assign the dK/dV kernel's key tiles to workgroups. */
SEPATTN_API size_t sepattn_bwd_workspace_size(const sepattn_shape* s);

/* Gradients for upstream dO: with P the masked softmax,
 *   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,
 * dK/dV summed over the q heads of each KV head.  o and lse are the forward's
 * outputs; dout uses o's strides; dq, dk, dv are written (not accumulated)
 * with the strides of q, k and v, which must therefore keep rows apart (as
 * o_stride for sepattn_fwd), else SEPATTN_EINVAL.  dtype must be
 * SEPATTN_BF16 (SEPATTN_F32: SEPATTN_ENOTSUP).
 * Deterministic: every output row is written by one workgroup; the only
 * atomics choose which workgroup computes which key tile. */
SEPATTN_API int sepattn_bwd(const sepattn_shape* s, int dtype, const sepattn_mask* m,
                const void* q, const void* k, const void* v, const void* o,
                const float* lse, const void* dout, float scale,
                void* dq, void* dk, void* dv,
                void* workspace, size_t workspace_bytes, void* stream);

/* sepattn_bwd for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the workspace in a static array that the
 * library's code holds on each device (SEPATTN_BWD_NOALLOC_MAX_ROWS fp32
 * values of D, 16 MiB, and 1 KiB of counters, from the library's load until
 * the process ends).  The call
 * itself allocates nothing; the first call on a device looks up the array's
 * address there.  B * Hq * L must not exceed SEPATTN_BWD_NOALLOC_MAX_ROWS,
 * else SEPATTN_ESPACE.  Every call on a device shares its one array: calls
 * that overlap on one device (different streams, or host threads without
 * ordering) race and give wrong gradients.  Other arguments and errors as
 * sepattn_bwd. */
#define SEPATTN_BWD_NOALLOC_MAX_ROWS (1 << 22)
SEPATTN_API int sepattn_bwd_noalloc(const sepattn_shape* s, int dtype, const sepattn_mask* m,
                        const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, float scale,
                        void* dq, void* dk, void* dv, void* stream);

/* ------------------------------------------------------------------------
 * SepCache: the streaming cache ([PITH] key_machinery; [ANTH] streaming
 * bullet) with a sink block of a entries, a separator block of s entries kept
 * first-in first-out, a window of n entries (the newest token included) and,
 * with a capacity c > a + s + n, a past window of P = c - a - s - n entries.
 * A token leaving the window (or, with a past window, the past window) moves
 * to the separator block if it is a separator, dropping that block's oldest
 * entry when full, and is dropped otherwise.
 *   c = 0 or a + s + n (no past window).  Per step: append the new token,
 *   evict (the oldest of n + 1 window entries leaves), then decode: the
 *   cache holds at most a + s + n entries.
 *   c > a + s + n.  The window and past window form one queue of at most
 *   n + P tokens.  An append to a full queue first makes its oldest P + 1
 *   leave (a flush), so the queue then holds n; evict does nothing.  The
 *   cache holds at most c entries, and once the separator block is full its
 *   size cycles a + s + n, ..., c, with mean (n + c + a + s) / 2.
 * The cache's logical order is sinks, separators (oldest first), past
 * window, window (oldest first), which is ascending original position.
 *
 * All streams of a batch share the step: stream b appends its own token and
 * flag.  Physical slots per stream and KV head: [0, a) sinks, [a, a+s)
 * separator ring, [a+s, slots) window ring of n + P + 1 slots (one spare for
 * the appended token), slots = a + s + n + P + 1.  Every KV head keeps its own
 * copy of the slot metadata and counters (all copies hold the same values),
 * so the work of one (stream, KV head) never waits on another workgroup.
 * ------------------------------------------------------------------------ */
typedef struct {
  int B, Hkv, d;       /* streams, KV heads, head dim (64 or 128)              */
  int a, s, n;         /* sinks, separator capacity (>= 0), window (>= 1)       */
  void* k;             /* bf16 keys before RoPE: B * Hkv slices of
                          sepcache_k_rows(slots) * d elements, each in 16-row
                          tiles, chunk-major (see below)                       */
  void* v;             /* bf16 [B, Hkv, slots, d]                               */
  int32_t* slot_pos;   /* [B, Hkv, slots] original position held, -1 if empty  */
  uint8_t* slot_sep;   /* [B, Hkv, slots] separator flag of the token held     */
  int32_t* state;      /* [B, Hkv, 8] counters: tokens seen, sinks, sep head,
                          sep count, window head, window count, flags (bit 0:
                          an append found the window full and was dropped),
                          separator flag of the window's oldest entry          */
  float theta;         /* RoPE base: pair (i, i + d/2) turns by p * theta^(-2i/d)
                          at position p                                        */
  int c;               /* capacity: 0 or a + s + n (no past window), or more
                          (a past window of c - a - s - n entries)             */
} sepcache;

/* Physical slots per stream and KV head: max(c, a + s + n) + 1; -1 for
 * invalid sizes (a < 0, s < 0, n < 1, or 0 < c < a + s + n). */
SEPATTN_API int sepcache_slots(int a, int s, int n, int c);
/* Rows of one (stream, KV head) slice of k: slots rounded up to a multiple of
 * 16.  Within the slice, the 16-byte chunk ch (dims 8 ch .. 8 ch + 7) of the
 * key in slot r sits at chunk index ((r / 16) * (d / 8) + ch) * 16 + r % 16,
 * so a 16-row tile is contiguous and, inside it, chunk-major: the decode
 * reads each chunk of 16 keys with one contiguous load.  The padding rows
 * are neither read nor written by any call (sepcache_reset zeroes them).
 * -1 for slots < 1 or slots > 65536. */
SEPATTN_API int sepcache_k_rows(int slots);
/* Empty every stream (slot_pos = -1, counters 0, K and V zero) of every KV
 * head. */
SEPATTN_API int sepcache_reset(const sepcache* c, void* stream);
/* Append token t of every stream: k_new, v_new bf16 [B, Hkv, d] contiguous,
 * is_sep device uint8 [B].  Token t < a becomes a sink, later tokens enter the
 * window (with a past window, after the flush of a full queue: two kernels).
 * Call sepcache_evict before the next append. */
SEPATTN_API int sepcache_append(const sepcache* c, const void* k_new, const void* v_new,
                    const uint8_t* is_sep, void* stream);
/* If a stream's window holds more than n entries, its oldest entry leaves:
 * to the separator block (separator) or dropped (other).  With a past window
 * the append has made room already and this does nothing. */
SEPATTN_API int sepcache_evict(const sepcache* c, void* stream);
/* append + evict in one launch. */
SEPATTN_API int sepcache_push(const sepcache* c, const void* k_new, const void* v_new,
                  const uint8_t* is_sep, void* stream);
/* Attention of the newest token over the cache: for q head h (KV head
 * h / (Hq / Hkv)), keys rotated by RoPE at their positions, the query at its
 * own, softmax(scale * q.k) over every entry, times V.  shift != 0: positions
 * are ranks in the logical order (the query is the last rank, [HUB] A1);
 * shift == 0: original token positions.
 *   q bf16 [B, Hq, d] (before RoPE), o bf16 [B, Hq, d], contiguous;
 *   Hq / Hkv in {1, 2, 4, 8}.
 * RoPE angles are computed on the device: position times frequency is
 * reduced modulo one turn in double precision for original positions and in
 * fp32 for ranks.  The cache is only read.
 * Caches with at most 1024 rows (slots, plus the appended token's row for
 * sepcache_step) run as one kernel: the rows are shared by
 * ceil(rows / 512) workgroups per (stream, KV head), and with more than one
 * the last to finish merges the others' partial results from the workspace.
 * There the rotated keys and query enter the score product as bf16 and the
 * probabilities enter P V as bf16, both with fp32 sums.  Larger caches split
 * the rows over workgroups of at most 64 (d = 128) or 128 (d = 64) rows and
 * merge in a second kernel.  K and V of slots that hold no entry must be
 * finite (sepcache_reset zeroes them; later they only receive tokens' K and
 * V).  workspace: sepcache_decode_workspace_size() bytes of device memory (0
 * when one workgroup per (stream, KV head) suffices, where NULL is accepted),
 * zero-filled before its first use; the calls leave it ready for the next.
 * Calls that share a workspace must not overlap.
 * Decode before any append writes zeros. */
SEPATTN_API size_t sepcache_decode_workspace_size(const sepcache* c, int Hq);
SEPATTN_API int sepcache_decode(const sepcache* c, int Hq, const void* q, float scale, int shift,
                    void* o, void* workspace, size_t workspace_bytes, void* stream);
/* One decode step: append the new token (k_new, v_new, is_sep as for
 * sepcache_append), evict, and attend (q, o, workspace as for
 * sepcache_decode); the same result as sepcache_push then sepcache_decode,
 * reading the cache once (with a past window, the flush of a full queue runs
 * as a kernel of its own first). */
SEPATTN_API int sepcache_step(const sepcache* c, const void* k_new, const void* v_new,
                  const uint8_t* is_sep, int Hq, const void* q, float scale, int shift,
                  void* o, void* workspace, size_t workspace_bytes, void* stream);
/* Prompt hand-off from prefill: seeds every stream's cache with a prompt of
 * m->L tokens, leaving the state that sepcache_reset followed by m->L calls
 * of sepcache_push would leave (the sinks, the separators that left the
 * window, the window; with a past window, its queue), bit for bit.
 *   k, v      bf16 [B, Hkv, L, d], keys before RoPE, addressed with element
 *             strides k_stride / v_stride (host int64 [3]: batch, head,
 *             token; multiples of 8) and a contiguous last dimension;
 *   m         the prompt's mask metadata from sepattn_build_mask, with
 *             m->B == c->B and m->a == c->a (its is_sep, sep_idx and
 *             sep_before name the separators the cache keeps; m->n plays no
 *             part).
 * Every slot is written, and the counters: an empty window-ring slot gets
 * the K/V of the token that last left it, as pushing leaves it, and other
 * empty slots zeros, as after a reset.  One launch. */
SEPATTN_API int sepcache_prefill(const sepcache* c, const void* k, const void* v, const int64_t* k_stride,
                     const int64_t* v_stride, const sepattn_mask* m, void* stream);
/* Original positions in logical order: pos [B, slots - 1] (unused tail -1),
 * len [B] entries held.  For bit-exact checks against a reference. */
SEPATTN_API int sepcache_export_order(const sepcache* c, int32_t* pos, int32_t* len, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SEPATTN_H */
