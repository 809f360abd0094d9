/*
 * arcs.h -- on-device batched token sampling for AMD Instinct MI355X (gfx950).
 *
 * The library turns a [B, V] logits tensor that already lives in GPU memory
 * into one token id per row, without copying the logits to the host.  The
 * pages it follows (the Arc engine's pull requests) price the host path it
 * replaces: Arc PR #222 ("ARC_SAMPLE_ON_DEVICE", section 2) copies the whole
 * [B, 1, vocab] logits tensor to the host every step and samples every row
 * there; Arc PR #217 ("device decode loop", "What this does") keeps the
 * greedy token in an i32[batch] device buffer instead.
 *
 * Conventions shared by every call:
 *  - All array arguments are DEVICE pointers owned by the caller.  The
 *    library allocates nothing, keeps no state between calls, never
 *    synchronises and never reads device memory from the host.  Work is
 *    enqueued on `stream` (a hipStream_t; NULL means the default stream) and
 *    the call returns.
 *  - Logits are row-major: row b starts `b * row_stride` elements after
 *    `logits`, `row_stride >= V`.  dtype ARCS_DTYPE_BF16 (raw bfloat16) or
 *    ARCS_DTYPE_F32.  `logits` must be aligned to its element size; rows
 *    whose start is 16-byte aligned take the vector-load path.
 *  - Host-checkable argument errors are returned as a negative arcs_status
 *    before anything is launched; nothing is written in that case.
 *  - Launch failures are reported as ARCS_ERR_LAUNCH (from hipGetLastError,
 *    without synchronising).
 *  - Calls are reentrant; concurrent calls on different streams are safe.
 */
#ifndef ARCS_H
#define ARCS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum arcs_dtype {
  ARCS_DTYPE_BF16 = 0,
  ARCS_DTYPE_F32 = 1
} arcs_dtype;

typedef enum arcs_status {
  ARCS_OK = 0,
  ARCS_ERR_NULL_POINTER = -1,        /* a required pointer is NULL              */
  ARCS_ERR_BAD_BATCH = -2,           /* B <= 0 or B > 2^31 - 1                  */
  ARCS_ERR_BAD_VOCAB = -3,           /* V <= 0 or V > 2^31 - 1                  */
  ARCS_ERR_BAD_STRIDE = -4,          /* row_stride < V                          */
  ARCS_ERR_BAD_DTYPE = -5,           /* dtype is not an arcs_dtype              */
  ARCS_ERR_WORKSPACE_TOO_SMALL = -6, /* workspace_bytes < arcs_sample_workspace_bytes() */
  ARCS_ERR_LAUNCH = -7,              /* the HIP runtime rejected a launch       */
  ARCS_ERR_MISALIGNED = -8,          /* logits not aligned to the element size  */
  ARCS_ERR_BAD_HISTORY = -9,         /* exactly one of hist_ids/hist_offsets is NULL */
  ARCS_ERR_BAD_TOP_N = -10,          /* arcs_top_logprobs: n outside [1, ARCS_MAX_TOP_LOGPROBS] */
  ARCS_ERR_BAD_CAPACITY = -11,       /* arcs_commit_tokens: capacity 0, or capacity * B too large */
  ARCS_ERR_SCRATCH_TOO_SMALL = -12,  /* arcs_sample_noalloc: the shape needs more than its scratch */
  ARCS_ERR_BAD_BUDGET = -13,         /* arcs_sample_hybrid_nucleus: budget outside [0, 4096] */
  ARCS_ERR_BAD_DRY = -14             /* arcs_sample_dry: breakers NULL or n_breakers outside [0, 64] */
} arcs_status;

/* Per-row status codes written to out_status[b] (out_ids[b] = -1 when != 0). */
enum {
  ARCS_ROW_OK = 0,
  ARCS_ROW_BAD_TEMPERATURE = 1,      /* temperature NaN or < 0                  */
  ARCS_ROW_BAD_TOP_P = 2,            /* top_p NaN or <= 0                       */
  ARCS_ROW_BAD_MIN_P = 3,            /* min_p NaN, < 0 or > 1                   */
  ARCS_ROW_BAD_PENALTY = 4,          /* non-finite penalty, or repetition < 0   */
  ARCS_ROW_BAD_FLAGS = 5,            /* flags has a bit other than ARCS_ROW_TIES_WIDE */
  ARCS_ROW_HISTORY_TOO_LONG = 6,     /* penalties active, > ARCS_MAX_HISTORY distinct ids,
                                        and no long-history workspace */
  ARCS_ROW_VOCAB_TOO_LARGE = 7       /* penalties active, V > ARCS_MAX_PENALTY_VOCAB,
                                        and no long-history workspace */
};

/* Limits of the penalty tables kept in LDS (per row): distinct history ids
 * in [0, V) (the number of history entries itself is not limited) and V.
 * Beyond them a penalised call needs a long-history workspace (see
 * arcs_long_history_workspace_bytes); without one such rows get the status
 * codes above. */
#define ARCS_MAX_HISTORY 4096
#define ARCS_MAX_PENALTY_VOCAB 262144

/* Codes arcs_commit_tokens latches into its fault word (the first one stays). */
enum {
  ARCS_FAULT_NONE = 0,
  ARCS_FAULT_TOKEN_RANGE = 1,        /* a token outside [0, V) other than -1            */
  ARCS_FAULT_RING_OVERRUN = 2        /* the ring slot still holds a step not drained yet */
};

/* Limits of arcs_top_logprobs: entries per row, and V. */
#define ARCS_MAX_TOP_LOGPROBS 64
#define ARCS_TOP_LOGPROBS_MAX_VOCAB 262144

/*
 * Per-row sampling parameters, 32 bytes, device array of B records.
 * Filters follow Arc PR #222 section 3(b): the host sampler's sorted list
 * feeds zero-the-rest (top-k), the top-p walk and the min-p scan, all three
 * inert under top_k = -1, top_p = 1, min_p = 0, in which case no cutoff is
 * computed at all.
 *   temperature  0 => greedy (argmax); > 0 => q ~ exp(z'/T)
 *   top_k        <= 0 or >= V => off; 1 => greedy; else keep the k first ids
 *                of the order (value desc, id asc)
 *   top_p        >= 1 => off; else keep the shortest prefix of that order
 *                whose mass reaches top_p of the FULL mass
 *   min_p        0 => off; keep ids with q_v >= min_p * q_max
 *   presence     0 => off; z -= presence for ids in the history
 *   frequency    0 => off; z -= frequency * count for ids in the history
 *   repetition   1 (or 0) => off; z = z > 0 ? z / r : z * r for history ids
 *                (applied first, then frequency, then presence; each an
 *                IEEE binary32 operation without fused multiply-add)
 *   flags        0, or ARCS_ROW_TIES_WIDE: the kept prefix grows to every id
 *                whose value equals that of its last id (the wider tie rule
 *                the pages report for their fallback device selector, Arc PR
 *                #194, squashed commit #130); other bits are a row error
 * The kept set is the shortest of the three prefixes (no renormalisation
 * between filters).
 */
#define ARCS_ROW_TIES_WIDE 1
typedef struct arcs_row_params {
  float temperature;
  int32_t top_k;
  float top_p;
  float min_p;
  float presence;
  float frequency;
  float repetition;
  int32_t flags;
} arcs_row_params;

/*
 * Per-row DRY ("don't repeat yourself") penalty, 16 bytes, device array of B
 * records (arcs_sample_dry).  The pages name the penalty and fix one fact:
 * at its disabled default, multiplier 0.0, it touches no logit (Arc PR #222,
 * section 3(a)), so such rows keep the fast path.  Otherwise, over the last
 * min(range, ARCS_DRY_MAX_WINDOW) history ids (range 0: all, up to the
 * window), a token t gets n = the length of the longest tail of that window
 * which also ends right before an earlier occurrence of t (no sequence
 * breaker, and no id outside [0, V), inside the match or as t), and when
 * n >= allowed_length its logit loses multiplier * base^(n - allowed_length),
 * after the presence / frequency / repetition penalties (binary32: the power
 * by repeated multiplication, the product, the subtraction).
 *   multiplier      >= 0, finite (0: off)
 *   base            > 0, finite
 *   allowed_length  >= 1
 *   range           >= 0 (0: the whole window)
 * Invalid records give the row ARCS_ROW_BAD_PENALTY.  DRY needs the row's
 * history: rows without history arrays ignore the record.
 */
typedef struct arcs_dry_params {
  float multiplier;
  float base;
  int32_t allowed_length;
  int32_t range;
} arcs_dry_params;
#define ARCS_DRY_MAX_WINDOW 2048
#define ARCS_DRY_MAX_BREAKERS 64

/* Per-row diagnostics written by arcs_sample_debug only. */
typedef struct arcs_row_stats {
  int32_t id;          /* the sampled token (or -1)                         */
  int32_t argmax;      /* argmax of the penalised logits, lowest index      */
  int32_t kept;        /* size L of the kept set (0 for greedy rows)        */
  int32_t cut_index;   /* last kept id in (value desc, id asc) order        */
  float cut_value;     /* its penalised logit                               */
  float max_logit;     /* max of the penalised logits                       */
  int32_t status;      /* per-row status code                               */
  uint32_t path;       /* ARCS_PATH_* bits: which stages ran                */
  double mass_total;   /* S   = sum of weights exp((z' - max)/T), as used   */
  double mass_kept;    /* S_K = sum over the kept set, as used              */
  double uniform;      /* the uniform u that drove the draw                 */
  uint64_t reserved;
} arcs_row_stats;

enum {
  ARCS_PATH_GREEDY = 1u,      /* argmax only                                   */
  ARCS_PATH_SORT_SKIP = 2u,   /* no filter active: no cutoff computed          */
  ARCS_PATH_CUTOFF = 4u,      /* radix-select cutoff ran                       */
  ARCS_PATH_MINP_FLOOR = 8u,  /* the min-p threshold bounded the kept set      */
  ARCS_PATH_TIE_SPLIT = 16u,  /* the boundary value's ties were split by id    */
  ARCS_PATH_PENALTY = 32u,    /* penalties applied                             */
  ARCS_PATH_SPECIAL = 64u,    /* special values (all -inf, +inf or NaN) seen   */
  ARCS_PATH_RESIDENT = 128u,  /* the row was kept in registers (single HBM read) */
  ARCS_PATH_REREAD = 256u     /* fp32 row: one HBM read, then one re-read from cache */
};

/*
 * arcs_argmax: out_ids[b] = argmax_v logits[b, v], lowest index among equal
 * values (bit-exact with a host argmax; Arc PR #217, "What this does", step 2).
 * NaN counts as -inf and -0 equals +0; a row of all -inf/NaN gives 0.
 *   logits     device, [B, row_stride] of dtype
 *   out_ids    device, int32[B]
 * Returns ARCS_OK or a negative arcs_status.
 */
int arcs_argmax(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                int32_t* out_ids, void* stream);

/*
 * arcs_sample: one token per row (Arc PR #222, sections 2 and 3; penalties
 * per the parameter record above).  Per row b:
 *   z'   = logits widened to float32 (NaN -> -inf), penalties applied to the
 *          ids in hist_ids[hist_offsets[b] .. hist_offsets[b+1]) (ids outside
 *          [0, V) are skipped; duplicates count);
 *   greedy rows (T == 0 or top_k == 1): argmax of z';
 *   else K = the kept prefix, and the token is the first id of K, in id
 *   order, whose running weight exceeds u * S_K, with u the SplitMix64
 *   uniform of counter step * 2^32 + b under `seed` (Arc PR #217, "Default
 *   OFF", names SplitMix64 for the device sampler).
 *   params         device, arcs_row_params[B]
 *   hist_ids       device int32 ids, or NULL (no penalties anywhere)
 *   hist_offsets   device int64[B + 1] CSR offsets into hist_ids, or NULL
 *   seed, step     RNG key, by value
 *   out_ids        device int32[B]; -1 for rows with invalid parameters
 *   out_status     device int32[B] per-row codes, or NULL
 *   workspace      device scratch of workspace_bytes, 16-byte aligned, owned by
 *                  the caller and not read before it is written; may be NULL
 *                  when arcs_sample_workspace_bytes() returns 0.  Batches of
 *                  at most 64 bf16 rows with 8192 <= V <= 131072, V % 8 == 0
 *                  use it: their greedy rows and rows without filters are read
 *                  by P = clamp(512 / B, 8, 128) workgroups per row, which
 *                  leave per-slice partials (16 bytes each) there for the
 *                  row's own workgroup.  Calls that share a workspace must be
 *                  ordered on one stream.
 * Returns ARCS_OK or a negative arcs_status (ARCS_ERR_WORKSPACE_TOO_SMALL
 * when workspace_bytes is below arcs_sample_workspace_bytes(),
 * ARCS_ERR_NULL_POINTER for a NULL workspace the shape needs,
 * ARCS_ERR_MISALIGNED for a workspace not 16-byte aligned).
 */
int arcs_sample(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                const arcs_row_params* params, const int32_t* hist_ids,
                const int64_t* hist_offsets, uint64_t seed, uint64_t step, int32_t* out_ids,
                int32_t* out_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * arcs_sample_keyed: arcs_sample with the RNG key in device memory, for
 * decode loops captured in a HIP graph.  Arc PR #217 ("device decode loop",
 * "What this does", step 3) keeps the per-step state on the device and moves
 * it on with a device kernel, so that a captured step needs no host work
 * between launches; a key passed by value would instead be frozen into the
 * graph at capture time.
 *   key       device uint64[2] = {seed, step}, 8-byte aligned, read when the
 *             kernels run (the uniform of row b uses counter step * 2^32 + b
 *             under seed, exactly as arcs_sample)
 *   advance   nonzero: a one-thread kernel enqueued after the sampling kernel
 *             on the same stream adds 1 to key[1] (each graph replay then
 *             samples the next step); 0: key is only read
 * Other arguments, errors and outputs as arcs_sample; a NULL or misaligned
 * key is rejected before any launch.  Calls that share one key must be
 * ordered on one stream.
 */
int arcs_sample_keyed(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const arcs_row_params* params, const int32_t* hist_ids,
                      const int64_t* hist_offsets, uint64_t* key, int advance, int32_t* out_ids,
                      int32_t* out_status, void* workspace, size_t workspace_bytes, void* stream);

/*
 * arcs_sample_noalloc: arcs_sample for callers that cannot allocate device
 * memory (code under HIP graph capture, serving loops that forbid
 * allocation).  It takes no workspace: shapes that need one use a device
 * array inside the library, ARCS_NOALLOC_SCRATCH_BYTES per GPU, allocated
 * with the library's code object and held until the process ends.  The call
 * allocates nothing (no hipMalloc, no library routine that allocates); the
 * first call on a device looks up that device's copy of the array.
 * Every call on one GPU shares that GPU's array: calls on one GPU that may
 * overlap (other streams, other host threads) race and must be ordered by
 * the caller.  Shapes needing more than the array (none today: the largest
 * split workspace is 567 * 16 = 9,072 bytes) get ARCS_ERR_SCRATCH_TOO_SMALL before
 * any launch.  Arguments, outputs and other errors as arcs_sample.
 */
#define ARCS_NOALLOC_SCRATCH_BYTES 16384
int arcs_sample_noalloc(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                        const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                        uint64_t seed, uint64_t step, int32_t* out_ids, int32_t* out_status, void* stream);

/*
 * arcs_sample_dry: arcs_sample with a DRY penalty record per row (see
 * arcs_dry_params) and the call's sequence breakers.
 *   dry          device arcs_dry_params[B], or NULL (= arcs_sample)
 *   breakers     device int32 ids that break repeats, n_breakers of them
 *                (0 .. ARCS_DRY_MAX_BREAKERS; NULL when 0)
 * Rows whose DRY record is active (multiplier != 0, with history) run on the
 * general pipeline.  Other arguments, outputs and errors as arcs_sample, plus
 * ARCS_ERR_BAD_DRY.
 */
int arcs_sample_dry(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                    const arcs_row_params* params, const int32_t* hist_ids, const int64_t* hist_offsets,
                    const arcs_dry_params* dry, const int32_t* breakers, int n_breakers, uint64_t seed,
                    uint64_t step, int32_t* out_ids, int32_t* out_status, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * arcs_sample_hybrid_nucleus: a baseline nucleus (top-p) sampler, for A/B
 * timing against arcs_sample.  It is the selector the pages report for their
 * device sampler (Arc PR #194, squashed commit #130, "hybrid nucleus
 * selector"): per row, the ids of the order (value desc, id asc) are
 * enumerated one at a time, for at most `budget` ids, until their mass
 * reaches top_p of the row's mass, and the kept set is that prefix; past the
 * budget, 32 halvings of the value key find the largest threshold whose mass
 * reaches top_p, and every id at or above it is kept (ties at the boundary
 * value all kept: the wider rule).  top_p >= 1 keeps every id.  No penalties,
 * top-k or min-p.  The draw is arcs_sample's: the first kept id in id order
 * whose running weight exceeds u * S_K, u the SplitMix64 uniform of counter
 * step * 2^32 + b under seed.  fp32 weights, fp64 sums.
 *   logits       device bf16 [B, row_stride], rows 16-byte aligned,
 *                V % 8 == 0, V <= 131072
 *   temperature  device float[B], > 0 and finite (else row status 1)
 *   top_p        device float[B], > 0 (else row status 2)
 *   budget       ids enumerated before bisection takes over, 0 .. 4096
 *   out_ids      device int32[B]; out_kept device int32[B] (kept set size) or
 *                NULL; out_status device int32[B] or NULL
 * Returns ARCS_OK, ARCS_ERR_BAD_DTYPE (not bf16), ARCS_ERR_BAD_VOCAB,
 * ARCS_ERR_MISALIGNED, ARCS_ERR_BAD_BUDGET or another negative arcs_status.
 */
int arcs_sample_hybrid_nucleus(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                               const float* temperature, const float* top_p, int budget, uint64_t seed,
                               uint64_t step, int32_t* out_ids, int32_t* out_kept, int32_t* out_status,
                               void* stream);

/* Bytes of device workspace arcs_sample, arcs_sample_keyed and
 * arcs_sample_debug need for this shape: B * P * 16 for the split batches
 * described under arcs_sample, else 0. */
size_t arcs_sample_workspace_bytes(int64_t B, int64_t V, int dtype);

/*
 * arcs_long_history_workspace_bytes: B * V * 4 (saturating).  A call with
 * history arrays (arcs_sample, arcs_sample_keyed, arcs_sample_debug,
 * arcs_sample_dry) whose workspace is at least this large and 16-byte aligned
 * samples rows whose active penalties the LDS tables cannot hold (more than
 * ARCS_MAX_HISTORY distinct history ids, or V > ARCS_MAX_PENALTY_VOCAB)
 * instead of failing them: such a row's penalised logits (repetition,
 * frequency and presence, Arc PR #222 page, section 3(a); and the
 * DRY record if active) are written in binary32 to the row's slice of the
 * workspace (offset row * V * 4) and the general pipeline samples that copy,
 * in two more launches on the same stream that other rows leave at once.
 * The results equal the table path's.  The workspace is owned by the caller,
 * not read before it is written, and shared only by calls ordered on one
 * stream; smaller workspaces (or none) keep the status codes
 * ARCS_ROW_HISTORY_TOO_LONG / ARCS_ROW_VOCAB_TOO_LARGE.
 */
size_t arcs_long_history_workspace_bytes(int64_t B, int64_t V);

/* Human-readable text for an arcs_status or ARCS_ROW_* code. */
const char* arcs_status_string(int code);

/*
 * arcs_sample_debug: arcs_sample plus test hooks, kept off the hot path.
 *   uniforms    device double[B] in [0, 1) replacing the SplitMix64 draw, or NULL
 *   out_probs   device float[B, V]: the filtered distribution q (0 outside
 *               the kept set; greedy rows get a one-hot), or NULL
 *   out_stats   device arcs_row_stats[B], or NULL
 */
int arcs_sample_debug(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const arcs_row_params* params, const int32_t* hist_ids,
                      const int64_t* hist_offsets, uint64_t seed, uint64_t step,
                      int32_t* out_ids, int32_t* out_status, void* workspace,
                      size_t workspace_bytes, const double* uniforms, float* out_probs,
                      arcs_row_stats* out_stats, void* stream);

/*
 * arcs_top_logprobs: the n most probable tokens of each row with their
 * log-probabilities, next to the draw (Arc PR #222, section 3(c): the host
 * sampler finds them by a partial sort of the probabilities).  Per row b, at
 * temperature T = temperature[b] (1 when `temperature` is NULL):
 *   z = logits widened to float32 (NaN -> -inf, -0 -> +0), m = max z,
 *   w_v = exp((z_v - m) / T), w_v = 1 where z_v == m (so +inf logits share
 *   the mass and a row of -inf is uniform), S = sum of w,
 *   out_ids[b, r], r < n: the r-th id of the order (z desc, id asc);
 *   out_logprobs[b, r] = ln(w / S) of that id, computed in binary64 and
 *   rounded to binary32.
 * No penalties or filters are applied: this is the distribution of the
 * logits at temperature T.  Rows with V < n end with id -1 and -inf.
 *   logits        device, [B, row_stride] of dtype
 *   temperature   device, float[B], or NULL; a row whose T is NaN, <= 0 or
 *                 +inf gets ids -1, logprobs NaN, status ARCS_ROW_BAD_TEMPERATURE
 *   n             1 .. ARCS_MAX_TOP_LOGPROBS (else ARCS_ERR_BAD_TOP_N)
 *   out_ids       device, int32[B * n] (row-major)
 *   out_logprobs  device, float[B * n] (row-major)
 *   out_status    device, int32[B], or NULL
 * V must not exceed ARCS_TOP_LOGPROBS_MAX_VOCAB (else ARCS_ERR_BAD_VOCAB).
 * Returns ARCS_OK or a negative arcs_status (nothing launched then).
 */
int arcs_top_logprobs(const void* logits, int dtype, int64_t B, int64_t V, int64_t row_stride,
                      const float* temperature, int n, int32_t* out_ids, float* out_logprobs,
                      int32_t* out_status, void* stream);

/*
 * arcs_commit_tokens: publish the tokens of one decode step to the host
 * without a synchronisation (Arc PR #217, "What this does", step 3: the
 * token goes into the next step's input buffer, the device position moves on
 * and the token is published into a pinned, mapped host ring; the fault
 * handling there: the commit range-checks token and position before writing
 * anything and latches a code into a pinned fault word).  One launch:
 *   p = *position;
 *   refused, with *fault set to the code if it was ARCS_FAULT_NONE, when a
 *   token is outside [0, V) and is not -1 (ARCS_FAULT_TOKEN_RANGE; -1 is the
 *   sampler's mark for a row it refused, published as it is so that one
 *   request's invalid parameters do not stop the batch), or the slot p % capacity
 *   still holds a step the host has not drained, p - *drained >= capacity
 *   (ARCS_FAULT_RING_OVERRUN); also refused, silently, while *fault is set
 *   (a latched fault stops publication until the host clears it); nothing
 *   else is written then;
 *   otherwise next_input[b] = ids[b] (if next_input is not NULL),
 *   ring[(p % capacity) * B + b] = ids[b], then, after a system-scope fence,
 *   *published = p + 1 and *position = p + 1.
 *   ids          device, int32[B] (e.g. out_ids of arcs_sample)
 *   next_input   device, int32[B], or NULL
 *   position     device, uint64: the step counter
 *   ring         pinned host memory (hipHostMalloc), int32[capacity * B]
 *   published    pinned host memory, uint64: steps whose tokens are in the ring
 *   drained      pinned host memory, uint64, written by the host: steps consumed
 *   fault        pinned host memory, uint32, sticky; the host clears it
 * The host polls *published and *fault with plain volatile loads.  Calls on
 * one stream run in order; the ring and words belong to that stream.
 * Returns ARCS_OK or a negative arcs_status (nothing launched then).
 */
int arcs_commit_tokens(const int32_t* ids, int64_t B, int64_t V, int32_t* next_input, uint64_t* position,
                       int32_t* ring, uint64_t capacity, uint64_t* published, const uint64_t* drained,
                       uint32_t* fault, void* stream);

/* Library version, major * 10000 + minor * 100 + patch. */
int arcs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ARCS_H */
