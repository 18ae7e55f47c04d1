/*
 * attn.h -- C ABI of libattn.so: causal GQA prefill and varlen SDPA on
 * MI355X (gfx950).
 *
 * Every tensor argument is a DEVICE pointer to caller-owned memory; the
 * library allocates no device memory and keeps no per-call state.  Strides
 * are in ELEMENTS.  Calls are asynchronous on the given HIP stream (NULL:
 * the default stream) and return once the kernels are enqueued; a fault in
 * a kernel surfaces at the caller's next synchronisation.  All entry points
 * are thread-safe.  Device properties are read lazily on the first call that
 * passes validation, never at load time.
 *
 * Tensors are bf16 (bfloat16 bits), accumulation is fp32, outputs are
 * rounded to bf16 with round-to-nearest-even.
 *
 * Return value: an attn_status.  On anything but ATTN_OK nothing was
 * enqueued and attn_last_error() describes the reason.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* null pointer, bad size, inconsistent arguments   */
    ATTN_ERR_UNSUPPORTED = 2, /* valid, but not a layout this library computes   */
    ATTN_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
    ATTN_ERR_HIP = 4          /* the HIP runtime refused a query or a launch     */
} attn_status;

/* Bits of the varlen error word (attn_varlen_read_error).  A flagged
 * segment is not attended; its packed rows are zeroed like uncovered rows. */
#define ATTN_SEG_QRANGE 1   /* q_start < 0, q_len < 0 or q_start + q_len > T      */
#define ATTN_SEG_COL 2      /* col outside [0, cols-1): the last column is scratch */
#define ATTN_SEG_KVEND 4    /* kv_end < 0, or kv_end > rows on flat storage        */
#define ATTN_SEG_ATTR 8     /* seg_attr ring_rows > rows                           */
#define ATTN_SEG_OVERLAP 16 /* a packed row claimed by two valid segments; the
                               whole output of the call is then unspecified        */
#define ATTN_SEG_SPAN 32    /* ring storage: a query would see a key older than
                               kv_end - R, whose ring row a later position has
                               overwritten (the window is wider than
                               R - q_len + 1, or absent with kv_end > R)          */

/* Bits of the slot-write error word (attn_kv_write_read_error).  A flagged
 * token is not written. */
#define ATTN_KV_COL 1  /* seq_cols[i] outside [0, cols)            */
#define ATTN_KV_POS 2  /* positions[i] < 0                         */
#define ATTN_KV_ROWS 4 /* slot_rows[i] > rows                      */

/* Bits of the device-bound prefill's error word (attn_prefill_read_error). */
#define ATTN_BOUND_KV 1   /* kv_len outside [0, Lkv]: clamped into it          */
#define ATTN_BOUND_QPOS 2 /* |q_pos0| above 2^62: clamped                       */

/* Version of this ABI; bumped on any incompatible change. */
int attn_abi_version(void);

/* Thread-local, human-readable reason for the last non-OK return on this
 * thread ("" if none).  The string stays valid until the next call. */
const char *attn_last_error(void);

/*
 * Causal grouped-query attention prefill.
 *
 * Defines ("[CUDA] Use Triton TMA for long-context causal prefill",
 * Summary and operator-level performance table): global causal GQA softmax
 * attention of Lq prefill query rows against an Lkv-long key/value prefix,
 * head dimensions 64 and 128, output written through its real strides, and
 * a finite result for query rows that see no key.
 *
 *   q   [B, Hq,  Lq,  D]  bf16, strides q_str[4]
 *   k,v [B, Hkv, Lkv, D]  bf16, strides k_str[4], v_str[4]
 *   out [B, Hq,  Lq,  D]  bf16, strides o_str[4] (written, any B/H/L strides)
 *
 * Query head h reads key/value head h / (Hq / Hkv).  Query row i sits at
 * absolute position q_pos0 + i (pass Lkv - Lq for end-aligned prefill) and
 * sees key j iff 0 <= j < Lkv, j <= q_pos0 + i and, when window > 0,
 * j > q_pos0 + i - window (window keys including its own position).
 * o = sum_j softmax_j(scale * q.k_j) v_j over the visible keys; a row with
 * no visible key is written as exact zeros.  Keys past a workgroup's range
 * are never loaded; a NaN in a V row inside it that some of its rows do not
 * see still reaches those rows (0 * NaN), see the limitation under
 * attn_sdpa_varlen.
 *
 * Layout rules (else ATTN_ERR_UNSUPPORTED): D in {64, 128, 256} (256: the
 * head dimension the page left on its portable path, here a kernel of its
 * own); innermost stride 1 on all four tensors; base pointers 16-byte
 * aligned; every other stride a multiple of 8 elements; k/v row strides
 * (k_str[2], v_str[2]) below 2^24 elements.
 * Sizes (else ATTN_ERR_INVALID): B, Hq, Hkv >= 1; Lq, Lkv >= 0; Hq % Hkv == 0;
 * all element offsets below 2^62; q/out non-null when Lq > 0 and k/v
 * non-null when Lkv > 0.  Lq == 0 enqueues nothing; Lkv == 0 writes zeros.
 *
 * workspace: device memory of at least attn_causal_prefill_workspace(...)
 * bytes (may be NULL when that is 0), 256-byte aligned; it holds split
 * partial results and must not be shared by calls in flight.
 */
size_t attn_causal_prefill_workspace(int B, int Hq, int Hkv, int Lq, int Lkv, int D);

int attn_causal_prefill(const void *q, const void *k, const void *v, void *out,
                        int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                        const int64_t q_str[4], const int64_t k_str[4],
                        const int64_t v_str[4], const int64_t o_str[4],
                        int64_t q_pos0, int window,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * attn_causal_prefill for callers that cannot allocate device memory: code
 * under HIP graph capture that may not call hipMalloc, tight serving loops,
 * harnesses that forbid allocation.  It takes no workspace: the split
 * partials go to a static device buffer of ATTN_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends.  The
 * caller still passes inputs and outputs; the computation, the validation
 * and the launch plan are those of attn_causal_prefill, so the outputs are
 * the same bits.  The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); its first call on a device reads the
 * buffer's device address once.
 *
 * Returns ATTN_ERR_WORKSPACE when the call's split partials would exceed
 * the buffer (attn_causal_prefill_workspace(...) > ATTN_NOALLOC_SCRATCH_BYTES;
 * e.g. B=1, Hq=16, Hkv=2, Lq=1024, Lkv=131072, D=128 needs about 34 MB).
 * Every call on a device shares that device's buffer: calls that overlap in
 * time on one device (other streams, other threads) race and must be
 * serialised by the caller.  No part of the buffer needs to start at zero,
 * and each call fully writes what it later reads.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (64u << 20)

int attn_causal_prefill_noalloc(const void *q, const void *k, const void *v, void *out,
                                int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                                const int64_t q_str[4], const int64_t k_str[4],
                                const int64_t v_str[4], const int64_t o_str[4],
                                int64_t q_pos0, int window, void *stream);

/*
 * The same prefill with a device-resident KV bound.
 *
 * Defines ("[CUDA] Use Triton TMA for long-context causal prefill",
 * Summary: the long-context path is chosen for global causal attention with
 * a KV bound that lives on the device): bounds is a device int64[2] =
 * (q_pos0, kv_len), read by the kernels, so one captured graph serves every
 * chunk of a chunked prefill whose start position and key count change
 * between replays.  Lkv is then the capacity of the K/V tensors: keys
 * [0, kv_len) exist, a kv_len outside [0, Lkv] is clamped into it and
 * flagged (ATTN_BOUND_KV), a |q_pos0| above 2^62 is clamped and flagged
 * (ATTN_BOUND_QPOS).  Everything else is as attn_causal_prefill with
 * q_pos0 = bounds[0] and Lkv = kv_len; the key splits follow the capacity.
 *
 * workspace: attn_causal_prefill_dev_workspace(...) bytes (at least 256),
 * 256-byte aligned: the error word, then the split partials.
 * attn_prefill_read_error synchronises `stream` and reads the error word of
 * the last call that used this workspace.  bounds must be 8-byte aligned
 * (else ATTN_ERR_UNSUPPORTED) and non-null (else ATTN_ERR_INVALID).
 */
size_t attn_causal_prefill_dev_workspace(int B, int Hq, int Hkv, int Lq, int Lkv, int D);

int attn_causal_prefill_dev(const void *q, const void *k, const void *v, void *out,
                            int B, int Hq, int Hkv, int Lq, int Lkv, int D, float scale,
                            const int64_t q_str[4], const int64_t k_str[4],
                            const int64_t v_str[4], const int64_t o_str[4],
                            const int64_t *bounds, int window,
                            void *workspace, size_t ws_bytes, void *stream);

int attn_prefill_read_error(const void *workspace, void *stream, int32_t *err_out);

/*
 * Length-aware varlen SDPA over per-sequence KV columns.
 *
 * Defines ("[executorch][cuda] Add a length-aware Triton SDPA over
 * per-sequence KV columns", description; the stacked commits on the
 * batched-sequence manifest layout and the batched sequence cache give the
 * store layout, the slot rule and the ring size).  The K/V store is a grid
 * of rows x cols slots per KV head; a sequence keeps its keys in one column,
 * and the last column is reserved for padding writes, so it is never read.
 * A segment s of the table is one run of packed query rows
 * [q_start, q_start + q_len) that attends column col, where kv_end is the
 * sequence's key count after this step's own tokens were written.  Its
 * query j therefore has position kv_end - q_len + j, and key position k is
 * found in row k mod R of the column (R = the segment's ring rows on ring
 * storage, else rows).
 *
 *   q        [T, Hq, D]           bf16 packed query rows, strides q_str[3]
 *   k_store,
 *   v_store  [rows, cols, Hkv, D] bf16, strides k_str[4], v_str[4]
 *   out      [T, Hq, D]           bf16, strides o_str[3] (every row written)
 *   seq_info [S, 4] int32, device, contiguous: (q_start, q_len, col, kv_end)
 *   seg_attr [S, 3] int32, device, contiguous, nullable: per-segment
 *            (causal, window, ring_rows); when NULL every segment takes the
 *            call's causal / window / ring_rows.
 *
 * A query at position p sees key k iff k < kv_end, k <= p when causal, and
 * k > p - window when window > 0 (on a non-causal segment the window is this
 * lower bound only).  ring_rows <= 0 means flat storage.  Packed rows of
 * [0, T) that belong to no valid segment come back as zeros from the same
 * call.  The host never reads seq_info / seg_attr: the launch geometry is a
 * function of (S, T, Hq, Hkv, D, rows, cols) only, so one captured graph
 * serves every table later written into the same buffers.  A segment that
 * breaks a rule is not attended: its rows are zeroed and its ATTN_SEG_* bit
 * is set in the error word.
 *
 * Limitation (NaN): keys outside every workgroup's key range are never
 * loaded, so NaN or Inf there (later positions, other columns, the scratch
 * column, overwritten ring rows) cannot reach the output.  A V row inside a
 * workgroup's key range that is masked for some of its rows enters their PV
 * product with weight 0, and 0 * NaN = NaN: a NaN in such a V row spreads to
 * the rows of that workgroup.  The same holds for attn_causal_prefill.
 *
 * Layout rules as for prefill (else ATTN_ERR_UNSUPPORTED); D in {64, 128}.
 * Sizes (else ATTN_ERR_INVALID): non-null stores, q/out non-null when T > 0,
 * S >= 0, T >= 0, rows >= 1, cols >= 2,
 * S <= 2 * (cols - 1), Hq % Hkv == 0, ring_rows <= rows, and no window on a
 * non-causal call when seg_attr is NULL.
 *
 * workspace: at least attn_sdpa_varlen_workspace(...) bytes, 256-byte
 * aligned; it holds the error words and split partials.  Its size query
 * takes cols too (beyond the sizes of the call that determine the layout),
 * so that one signature validates every argument the call checks.
 */
size_t attn_sdpa_varlen_workspace(int S, int T, int Hq, int Hkv, int D, int rows, int cols);

int attn_sdpa_varlen(const void *q, const void *k_store, const void *v_store, void *out,
                     const int32_t *seq_info, int S, const int32_t *seg_attr,
                     int T, int Hq, int Hkv, int D, int rows, int cols, float scale,
                     int causal, int window, int ring_rows,
                     const int64_t q_str[3], const int64_t k_str[4],
                     const int64_t v_str[4], const int64_t o_str[3],
                     void *workspace, size_t ws_bytes, void *stream);

/*
 * Reads the error word of the last attn_sdpa_varlen call that used this
 * workspace (an OR of ATTN_SEG_* bits, 0 when every segment was valid).
 * Synchronises `stream` first.  The arguments (S, T) must be those of that
 * call: the flags are kept as several words (each written by one workgroup
 * with a plain store, so no call needs a clearing pass), and (S, T) say how
 * many to OR.
 */
int attn_varlen_read_error(const void *workspace, int S, int T, void *stream,
                           int32_t *err_out);

/*
 * The step's K/V slot write, the operation before attn_sdpa_varlen.
 *
 * Defines ("[executorch][cuda] Add a length-aware Triton SDPA over
 * per-sequence KV columns", the stacked commits on the batched-sequence
 * manifest layout and the batched sequence cache): each step token i is
 * written to slot (position mod rows) x columns + seq_cols[i] of the
 * [rows, cols, Hkv, D] stores, i.e. store row positions[i] mod R_i of column
 * seq_cols[i], where R_i is the token's ring rows (ring storage) or the store
 * rows (flat storage); the last column is scratch for padded writes.
 *
 *   k_new, v_new     [T, Hkv, D] bf16 (read), strides kn_str[3], vn_str[3]
 *   k_store, v_store [rows, cols, Hkv, D] bf16 (written), strides ks_str[4],
 *                    vs_str[4]; must not overlap k_new / v_new
 *   positions        [T] int64, device: absolute position of each token
 *   seq_cols         [T] int32, device: column of each token's sequence
 *   slot_rows        [T] int32, device, nullable: R_i (<= 0 or NULL: rows)
 *
 * Tokens whose column lies outside [0, cols), whose position is negative or
 * whose R_i exceeds rows are skipped and flagged in the error word
 * (ATTN_KV_*).  When two tokens of one call share a slot the slot receives
 * one of them, unspecified which (only padded writes to the scratch column
 * are expected to share).  The host never reads the per-token arrays, so
 * one captured graph serves any positions and columns written into them.
 *
 * Layout rules (else ATTN_ERR_UNSUPPORTED): D a multiple of 8 up to 1024;
 * innermost stride 1; other strides multiples of 8 elements; base pointers
 * 16-byte aligned, positions 8-byte and seq_cols / slot_rows 4-byte
 * aligned.  Sizes (else ATTN_ERR_INVALID): T >= 0, Hkv, D, rows, cols >= 1,
 * element offsets below 2^62, non-null pointers (per-token arrays and new
 * rows only when T > 0).  T == 0 enqueues nothing.
 *
 * workspace: at least attn_kv_write_workspace(T) bytes, 256-byte aligned;
 * it holds the error word, read by attn_kv_write_read_error (which
 * synchronises `stream`; T must be that of the call).
 */
size_t attn_kv_write_workspace(int T);

int attn_kv_write(const void *k_new, const void *v_new, void *k_store, void *v_store,
                  const int64_t *positions, const int32_t *seq_cols, const int32_t *slot_rows,
                  int T, int Hkv, int D, int rows, int cols, const int64_t kn_str[3],
                  const int64_t vn_str[3], const int64_t ks_str[4], const int64_t vs_str[4],
                  void *workspace, size_t ws_bytes, void *stream);

int attn_kv_write_read_error(const void *workspace, int T, void *stream, int32_t *err_out);

/*
 * Profiling aid (not part of the computation).  After attn_timing_begin(),
 * every attn_causal_prefill / attn_sdpa_varlen call made on the same host
 * thread records a pair of HIP events on its stream around its attention
 * kernel (the split-merge and finish kernels are not included), and the
 * attention kernels launched on the device that was current at
 * attn_timing_begin() add their workgroups' lifetimes, in shader cycles and
 * in the 100 MHz reference clock, to per-XCD sums held in a 144-byte static
 * device array (no allocation).  attn_timing_begin() clears those sums and
 * synchronises the device; call it outside graph capture.
 *
 * attn_timing_end() waits for the events, writes the summed kernel time in
 * milliseconds and the number of timed launches, and stops recording.
 * Returns ATTN_ERR_INVALID for null outputs, ATTN_ERR_HIP if an event could
 * not be read (the others are still summed).
 *
 * attn_timing_clock(), after attn_timing_end(), writes the average shader
 * clock in MHz over the timed workgroups (cycles / reference ticks x 100)
 * and, when xcd_mhz is not NULL, the same per XCD (0 for an XCD that ran
 * none).  Returns ATTN_ERR_INVALID while timing is on or for a null mhz,
 * ATTN_ERR_HIP when no sums were recorded or they could not be read.
 */
int attn_timing_begin(void);
int attn_timing_end(double *kernel_ms, int *launches);
int attn_timing_clock(double *mhz, double xcd_mhz[8]);

/*
 * attn_timing_reruns(), after attn_timing_end(), writes how many attention
 * workgroups of the timed launches finished (*workgroups; workgroups of a
 * varlen launch that found no work are not counted) and how many of them
 * found a row sum outside [2^-64, 2^64] after the pass with fixed softmax
 * references and redid their key range with the exact running maximum
 * (*redone).  The counts come from the same static device array as the
 * clock sums.  Returns ATTN_ERR_INVALID while timing is on or for null
 * outputs, ATTN_ERR_HIP when nothing was recorded or the counts could not
 * be read.
 */
int attn_timing_reruns(long long *workgroups, long long *redone);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
