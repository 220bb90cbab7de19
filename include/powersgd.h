/*
 * powersgd.h -- C ABI of the MI355X (gfx950) PowerSGD bucket-compression library.
 *
 * The library compresses one data-parallel rank's flat gradient bucket in place
 * with PowerSGD, as described on "DDP Communication Hooks -- PyTorch 1.11.0",
 * section "PowerSGD Hooks" (powerSGD_hook, steps 1 to 3.7, and
 * batched_powerSGD_hook), with the state and hyperparameters of section "PowerSGD
 * State" and the same-shape batching switch of the translated page's "Состояние
 * PowerSGD" item 5. A float16 variant fuses the loss-scale division and inf/NaN check
 * of "torch.cuda.amp -- PyTorch 1.5.0", section "Gradient Scaling"
 * (GradScaler.unscale_ and step); the fp16_compress_wrapper / bf16_compress_wrapper
 * of section "Default Communication Hooks" run either hook with a 16-bit state. The
 * state can be exported and imported as a byte string (checkpoint / resume).
 *
 * One rank: the allreduces of P, of Q and of the uncompressed tensors are the
 * identity, so no collective is issued.
 *
 * All device work is enqueued on the caller's HIP stream and runs asynchronously;
 * completion of that stream work plays the role of the hook's Future. Every
 * function returns before the device work completes unless stated otherwise.
 * A state is not thread-safe; distinct states are independent.
 *
 * Stream capture: the first compressing call of a bucket layout (and the first
 * fp16 or wrapped call before start_powerSGD_iter) allocates, clears and uploads the
 * layout's buffers and waits for its stream, so it cannot be captured. Every later
 * call on that layout enqueues kernel launches only and may be captured into a HIP
 * graph (kernel timing off). A replay repeats the captured launches with their
 * arguments: the same bucket and found_inf pointers, loss scale and, without warm
 * start, the same Q draw; the host-side iteration and statistics counters advance
 * only on real calls. With warm start each replay is one hook step.
 */
#ifndef POWERSGD_H
#define POWERSGD_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define POWERSGD_API __attribute__((visibility("default")))
#else
#define POWERSGD_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef struct powersgd_state powersgd_state; /* opaque, owned by the library */

typedef enum {
  POWERSGD_OK = 0,
  POWERSGD_ERR_INVALID_ARG = -1,     /* bad pointer, size, view or hyperparameter   */
  POWERSGD_ERR_LAYOUT_CHANGED = -2,  /* memorized bucket called with new views      */
  POWERSGD_ERR_OOM = -3,             /* device allocation failed                     */
  POWERSGD_ERR_HIP = -4,             /* a HIP runtime call failed (detail: last_error) */
  POWERSGD_ERR_UNSUPPORTED = -5,     /* e.g. a rank above POWERSGD_MAX_RANK          */
  POWERSGD_ERR_NOT_FOUND = -6        /* introspection of a bucket/view never compressed */
} powersgd_status;

typedef enum { POWERSGD_F32 = 0, POWERSGD_F16 = 1, POWERSGD_BF16 = 2 } powersgd_dtype;

#define POWERSGD_MAX_NDIM 8
#define POWERSGD_MAX_RANK 32

/*
 * Hyperparameters, named as PowerSGDState names them ("PowerSGD State" section;
 * batch_tensors_with_same_shape from the translated page). process_group is
 * absent: one rank. powersgd_hparams_init() fills the pages' defaults.
 */
typedef struct {
  int32_t matrix_approximation_rank;            /* r; default 1; 1..POWERSGD_MAX_RANK  */
  int64_t start_powerSGD_iter;                  /* default 1000; >= 0                  */
  double min_compression_rate;                  /* default 2; any finite value         */
  int32_t use_error_feedback;                   /* default 1                           */
  int32_t warm_start;                           /* default 1                           */
  double orthogonalization_epsilon;             /* default 0; >= 0, finite             */
  uint64_t random_seed;                         /* default 0                           */
  int64_t compression_stats_logging_frequency;  /* default 10000; <= 0 disables logs   */
  int32_t batch_tensors_with_same_shape;        /* default 0                           */
} powersgd_hparams;

/*
 * One per-parameter view of the flat bucket ("PowerSGD Hooks", powerSGD_hook step 1:
 * the flat bucket seen as a list of per-parameter tensors). offset and shape are in
 * elements; the view covers numel = prod(shape) contiguous elements from offset.
 * ndim 0 or 1 views are never compressed; ndim >= 2 views are compressed as the
 * row-major matrix shape[0] x prod(shape[1..ndim-1]) when they pass the rate test.
 */
typedef struct {
  int64_t offset;
  int32_t ndim;                        /* 0..POWERSGD_MAX_NDIM */
  int64_t shape[POWERSGD_MAX_NDIM];    /* entries past ndim are ignored */
} powersgd_view;

/* Fills hp with the defaults printed in the PowerSGDState signature. Never fails
 * (a NULL hp is ignored). */
POWERSGD_API void powersgd_hparams_init(powersgd_hparams* hp);

/*
 * Creates a state for device `device` ("PowerSGD State": the hyperparameters and the
 * internal state "for all the gradients during the training"). hp is copied.
 * Errors: INVALID_ARG for NULL pointers, r < 1, epsilon < 0 or not finite, a
 * non-finite rate, start_powerSGD_iter < 0; UNSUPPORTED for r > POWERSGD_MAX_RANK;
 * HIP if the device cannot be selected. Device memory is allocated lazily, per
 * bucket_index, on the first compressing call.
 */
POWERSGD_API powersgd_status powersgd_state_create(const powersgd_hparams* hp, int32_t device,
                                      powersgd_state** out);

/* Waits for the state's outstanding device work, frees everything it owns. NULL is
 * ignored. */
POWERSGD_API void powersgd_state_destroy(powersgd_state* st);

/*
 * Compresses one bucket in place: powerSGD_hook steps 1 to 3.7 on one rank.
 *
 *   bucket        device pointer, numel elements of `dtype`, caller-owned; updated in
 *                 place with P Q^T for compressed views (uncompressed views: F32 left
 *                 untouched, F16 unscaled). Must stay valid until the stream work ends.
 *   views         host array of nviews views, read during the call only; views must
 *                 lie inside [0, numel) and must not overlap. Elements outside every
 *                 view are neither read nor written.
 *   bucket_index  key of the per-bucket memory (error feedback, warm-start Q);
 *                 calling a memorized bucket_index with other views (or another
 *                 numel) returns LAYOUT_CHANGED when error feedback or warm start is
 *                 on, mirroring the "PowerSGD State" warning on rebuilt buckets;
 *                 otherwise the new layout replaces the old.
 *   is_last       non-zero on the last bucket of an iteration: advances the iteration
 *                 counter (GradBucket.is_last) after this call.
 *   dtype         F32: fp32 gradients. F16: fp16 loss-scaled gradients; the call is
 *                 GradScaler.unscale_ for this bucket (values are multiplied by
 *                 inv_loss_scale) fused with the inf/NaN check; output is unscaled
 *                 fp16, rounded to nearest even.
 *   inv_loss_scale  F16 only (ignored for F32): 1/scale; exact when a power of two.
 *   found_inf_dev   F16 only (required, device int32, caller-owned): the call ORs 1
 *                 into it when any view element is inf or NaN, and skips everything
 *                 (bucket, error memory and Q left bit-identical) when the flag is
 *                 non-zero after the check; the caller zeroes it before the first
 *                 bucket of an iteration. Never read back on the host here. With
 *                 error feedback a bucket first called with F16 keeps its error
 *                 memory in two alternating fp32 places (8 bytes per compressed
 *                 element) so that the check runs inside the first pass; a bucket
 *                 restored by powersgd_state_import keeps one and checks first.
 *   stream        hipStream_t (NULL = the legacy default stream).
 *
 * While iteration < start_powerSGD_iter the call is the vanilla allreduce: F32 is a
 * no-op, F16 does the unscale (and inf check) only; no state is created.
 * Errors are returned before anything is enqueued: INVALID_ARG (NULL state/bucket
 * or views with nviews > 0, numel < 0, view out of bounds, overlapping views,
 * ndim out of range, negative dimension, F16 without found_inf_dev, unknown dtype),
 * UNSUPPORTED (a compressed view with more than 2^31 - 65537 rows or columns),
 * LAYOUT_CHANGED, OOM, HIP (launch failure; asynchronous faults surface at the
 * caller's next synchronization).
 */
POWERSGD_API powersgd_status powersgd_compress_bucket(powersgd_state* st, int64_t bucket_index,
                                         int32_t is_last, void* bucket,
                                         powersgd_dtype dtype, int64_t numel,
                                         const powersgd_view* views, int32_t nviews,
                                         float inv_loss_scale, int32_t* found_inf_dev,
                                         void* stream);

/*
 * powerSGD_hook wrapped by fp16_compress_wrapper or bf16_compress_wrapper ("DDP
 * Communication Hooks -- PyTorch 1.11.0", section "Default Communication Hooks"): the
 * fp32 bucket is cast to 16 bits, the hook runs on the 16-bit tensor and the result is
 * cast back to fp32, in place. Every tensor the hook forms is a 16-bit value rounded to
 * nearest even where it is formed: the cast gradient, M' = G + E, P = M'Q, P after
 * Gram-Schmidt, Q = M'^T P, M_hat = P Q^T and E = M' - M_hat (also the initial draw of
 * Q, cast from its binary32 value); sums and products accumulate in fp32 (the
 * Gram-Schmidt recurrence in fp64). The bucket's error memory is a 16-bit array; with
 * error feedback it keeps M' of the latest call, from which the next call rebuilds E =
 * M' - M_hat with the same roundings (without, M' has a 16-bit array of its own); the
 * warm-start Q holds 16-bit values.
 *
 *   bucket         device pointer to numel fp32 gradients, caller-owned; compressed
 *                  views receive M_hat, uncompressed views their 16-bit cast (both as
 *                  fp32). Elements outside every view are neither read nor written.
 *   compute_dtype  POWERSGD_F16 (fp16_compress_wrapper) or POWERSGD_BF16
 *                  (bf16_compress_wrapper).
 *   bucket_index, is_last, views, nviews, stream: as for powersgd_compress_bucket; a
 *                  bucket_index memorized by another variant (or precision) is a
 *                  layout change. No loss scaling: values beyond the 16-bit range
 *                  become inf and propagate.
 *
 * Before start_powerSGD_iter the call is the cast to 16 bits and back.
 * Errors: INVALID_ARG (as for powersgd_compress_bucket; compute_dtype not F16/BF16),
 * LAYOUT_CHANGED, OOM, HIP; returned before anything is enqueued.
 */
POWERSGD_API powersgd_status powersgd_compress_bucket_wrapped(powersgd_state* st,
                                                 int64_t bucket_index, int32_t is_last,
                                                 float* bucket, powersgd_dtype compute_dtype,
                                                 int64_t numel, const powersgd_view* views,
                                                 int32_t nviews, void* stream);

/*
 * Side of the square matrix the batched variant views a bucket of `numel` elements
 * as: the smallest s with s * s >= numel (0 for numel <= 0). Pure host function.
 */
POWERSGD_API int64_t powersgd_batched_side(int64_t numel);

/*
 * batched_powerSGD_hook on one rank ("DDP Communication Hooks -- PyTorch 1.11.0",
 * section "PowerSGD Hooks", batched_powerSGD_hook steps 1 to 9): the whole bucket,
 * zero-padded, is viewed as one s x s row-major matrix M (s = powersgd_batched_side);
 * P = M Q, Gram-Schmidt with epsilon on P, Q = M^T P, M_hat = P Q^T, and the first
 * numel elements of M_hat are the new bucket. Error feedback and warm start follow
 * the state's hyperparameters as in powersgd_compress_bucket, with the error memory
 * covering all s * s entries (the padding of the gradient is zero at every call).
 * There is no rate test; the rank used is min(matrix_approximation_rank, s).
 *
 *   bucket        device pointer to `capacity` elements of `dtype`, caller-owned; the
 *                 first numel are the gradients. The call writes zeros to elements
 *                 [numel, s * s) before use (also when an fp16 call is skipped) and
 *                 leaves M_hat's padding there, so the
 *                 buffer doubles as the padded matrix (no copy); callers keep only the
 *                 first numel elements (step 9, truncation).
 *   capacity      elements available at `bucket`; must be >= s * s.
 *   bucket_index, is_last, dtype, inv_loss_scale, found_inf_dev, stream: as for
 *                 powersgd_compress_bucket. A bucket_index memorized by the per-layer
 *                 call (or with another numel) is a layout change.
 *
 * Statistics count numel elements in and 2 * s * rank communicated per call.
 * Errors: INVALID_ARG (NULL state, NULL bucket with numel > 0, numel < 0, capacity
 * below s * s, F16 without found_inf_dev, unknown dtype), UNSUPPORTED (s above
 * 2^31 - 65537), LAYOUT_CHANGED, OOM, HIP; all returned before anything is enqueued.
 */
POWERSGD_API powersgd_status powersgd_compress_bucket_batched(powersgd_state* st,
                                                 int64_t bucket_index, int32_t is_last,
                                                 void* bucket, powersgd_dtype dtype,
                                                 int64_t numel, int64_t capacity,
                                                 float inv_loss_scale, int32_t* found_inf_dev,
                                                 void* stream);

/*
 * batched_powerSGD_hook wrapped by fp16_compress_wrapper or bf16_compress_wrapper ("DDP
 * Communication Hooks -- PyTorch 1.11.0", sections "Default Communication Hooks" and
 * "PowerSGD Hooks"): the fp32 bucket is cast to 16 bits and viewed, zero-padded, as
 * the s x s matrix of powersgd_compress_bucket_batched; every tensor the hook forms is
 * a 16-bit value as in powersgd_compress_bucket_wrapped, and the first numel entries
 * of M_hat are cast back to fp32 in place.
 *
 *   bucket, numel, capacity  as for powersgd_compress_bucket_batched (fp32 only:
 *                  capacity >= s * s elements; the call zero-fills the padding).
 *   compute_dtype  POWERSGD_F16 or POWERSGD_BF16.
 *   bucket_index, is_last, stream: as for powersgd_compress_bucket.
 *
 * Errors: INVALID_ARG (NULL state, NULL bucket with numel > 0, numel < 0, capacity
 * below s * s, compute_dtype not F16/BF16), UNSUPPORTED (s above 2^31 - 65537),
 * LAYOUT_CHANGED, OOM, HIP; all returned before anything is enqueued.
 */
POWERSGD_API powersgd_status powersgd_compress_bucket_batched_wrapped(powersgd_state* st,
                                                 int64_t bucket_index, int32_t is_last,
                                                 float* bucket, powersgd_dtype compute_dtype,
                                                 int64_t numel, int64_t capacity,
                                                 void* stream);

/* Static text for a status code. */
POWERSGD_API const char* powersgd_status_string(powersgd_status s);

/* Detail of the calling thread's last failed call ("" if none). */
POWERSGD_API const char* powersgd_last_error(void);

/*
 * Host-only classification of one view under hp, without a state or a device:
 * *compress = 1 when the view would be compressed ("PowerSGD State",
 * min_compression_rate: (n + m) * rank * rate < n * m, strict, evaluated exactly on the
 * binary64 rate), *n and *m = the matrix shape (shape[0] x prod(rest); 0 for ndim < 2)
 * and *rank = min(r, n, m) (0 when not compressed). Any output pointer may be NULL.
 * INVALID_ARG for a NULL hp/view, ndim out of range or a negative dimension.
 */
POWERSGD_API powersgd_status powersgd_classify_view(const powersgd_hparams* hp, const powersgd_view* view,
                                       int32_t* compress, int64_t* n, int64_t* m,
                                       int32_t* rank);

/* --- introspection (for parity checks and statistics) ------------------------ */

/*
 * Compression decisions of a memorized bucket ("PowerSGD State", min_compression_rate):
 * out[v] = 1 when view v is compressed, else 0. nviews must equal the bucket's view
 * count. Host memory; synchronous, no device work. NOT_FOUND if the bucket was never
 * compressed.
 */
POWERSGD_API powersgd_status powersgd_get_decisions(powersgd_state* st, int64_t bucket_index,
                                       uint8_t* out, int32_t nviews);

/* Matrix shape and rank used for view v (rank = min(r, n, m)); rank 0 when the view
 * is not compressed. Synchronous, host only. */
POWERSGD_API powersgd_status powersgd_get_view_info(powersgd_state* st, int64_t bucket_index,
                                       int32_t view, int64_t* n, int64_t* m,
                                       int32_t* rank);

/*
 * Copies the latest orthogonalized P (n x rank, row-major) and Q = M'^T P (m x rank,
 * row-major; the warm-start memory) of compressed view v into caller device buffers
 * (either may be NULL), enqueued on `stream`.
 */
POWERSGD_API powersgd_status powersgd_copy_factors(powersgd_state* st, int64_t bucket_index,
                                      int32_t view, float* p_dev, float* q_dev,
                                      void* stream);

/* Copies the error-feedback memory E (n x m, row-major, fp32; a 16-bit state's values
 * widened exactly) of compressed view v into a caller device buffer, enqueued on
 * `stream`. NOT_FOUND without error feedback. */
POWERSGD_API powersgd_status powersgd_copy_error(powersgd_state* st, int64_t bucket_index,
                                    int32_t view, float* e_dev, void* stream);

/*
 * The factors of compressed view v after the bucket's latest call ("PowerSGD Hooks",
 * powerSGD_hook steps 3.4 and 3.5: P after Gram-Schmidt and Q = M'^T P, which the
 * state memorizes as the next warm-start Q). On return *P_dev points to n x r fp32
 * values (row-major, row stride r) and *Q_dev to m x r (row stride r), r = min(rank,
 * n, m); *n, *m, *r receive the shape. Any output pointer may be NULL.
 *
 * The pointers are state-owned device memory holding a copy taken for this call: the
 * copies are enqueued on the stream of the bucket's latest compressing call, behind
 * that call's work, so the values may be read once that stream has reached this
 * point. The memory stays valid until the bucket's state is released (state
 * destroyed, snapshot imported, or the bucket_index given a new layout); its contents
 * change only at the next get_factors call for the same view. The first call for a
 * view allocates (not graph-capturable); later calls enqueue copies only.
 * Errors: INVALID_ARG (NULL state, view out of range), NOT_FOUND (bucket never
 * compressed, or view not compressed), OOM, HIP.
 */
POWERSGD_API powersgd_status powersgd_get_factors(powersgd_state* st, int64_t bucket_index,
                                                  int32_t view, const float** P_dev,
                                                  const float** Q_dev, int64_t* n, int64_t* m,
                                                  int32_t* r);

/*
 * The error-feedback memory of a bucket ("PowerSGD Hooks", first warning: memory of
 * the size of the gradients, E = M' - M_hat after each call) laid out like the bucket:
 * *E_dev points to one fp32 value per bucket element (numel elements; the batched
 * variant: its s x s padded matrix), E of each compressed view at that view's
 * offset, zero elsewhere (uncompressed views carry no error on one rank). A 16-bit
 * state's values are widened exactly.
 *
 * The pointer is state-owned device memory filled for this call on the stream of the
 * bucket's latest compressing call, behind that call's work; it stays valid until the
 * bucket's state is released and its contents change only at the next get_error call
 * on the bucket. The first call allocates (not graph-capturable).
 * Errors: INVALID_ARG (NULL state or E_dev), NOT_FOUND (bucket never compressed, or
 * error feedback off), OOM, HIP.
 */
POWERSGD_API powersgd_status powersgd_get_error(powersgd_state* st, int64_t bucket_index,
                                                const float** E_dev);

/*
 * The raw initial draw of Q ("PowerSGD Hooks", powerSGD_hook step 3.1: Q initialized
 * from a standard normal distribution, before its orthogonalization) for view `view`
 * of bucket `bucket_index`, exactly as a compressing call draws it: entry e of the
 * row-major m x rank matrix is output word e mod 4 of Philox4x64-10 (Salmon et al.,
 * SC 2011) with counter (e div 4, view, epoch, 0) and key (random_seed, bucket_index);
 * words (w0, w1) and (w2, w3) give Box-Muller pairs with u = ((w_even >> 11) + 1) *
 * 2^-53 and v = (w_odd >> 11) * 2^-53 in binary64, rounded to binary32. A compressing
 * call uses epoch 0 under warm start and the iteration counter otherwise.
 *
 *   out_dev    device, m * rank floats (row-major, row stride rank), caller-owned.
 *   words_dev  device, 4 * ceil(m * rank / 4) uint64 Philox output words in counter
 *              order, caller-owned; may be NULL.
 *   stream     hipStream_t (NULL = the legacy default stream).
 * Runs on the calling thread's current HIP device. Stateless; allocates nothing. Errors: INVALID_ARG (m < 0, rank < 1, view < 0,
 * NULL out_dev with m > 0), UNSUPPORTED (rank above POWERSGD_MAX_RANK or m above
 * 2^31 - 65537), HIP.
 */
POWERSGD_API powersgd_status powersgd_draw_q0(uint64_t random_seed, int64_t bucket_index,
                                              int32_t view, uint64_t epoch, int64_t m,
                                              int32_t rank, float* out_dev,
                                              uint64_t* words_dev, void* stream);

/*
 * Iteration counter and compression statistics ("PowerSGD State",
 * compression_stats_logging_frequency): numel_in = elements seen by compressing
 * calls, numel_comm = elements an allreduce would carry ((n + m) * rank per compressed
 * view, numel per other view). Host values; synchronous.
 */
POWERSGD_API powersgd_status powersgd_get_stats(powersgd_state* st, int64_t* iteration,
                                   int64_t* numel_in, int64_t* numel_comm);

/* --- without allocation ------------------------------------------------------- */

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): one compression step of a single
 * n x m fp32 matrix, with the state held by the caller. It computes what
 * powersgd_compress_bucket computes for a bucket holding only this matrix (the same
 * kernels, work items and order of every sum, so the results are bitwise equal),
 * except that there is no min_compression_rate test and no iteration counter or
 * statistics: every call compresses, at rank r = min(matrix_approximation_rank, n, m).
 *
 *   hp            hyperparameters (host, read during the call): rank, epsilon and
 *                 random_seed are used; error feedback follows E, warm start q_valid.
 *   bucket_index, view, epoch  the key of the initial Q draw when q_valid is 0
 *                 (see powersgd_draw_q0; a compressing call uses view = the view's
 *                 index in its bucket and epoch = 0 under warm start).
 *   M             device, n * m fp32, row-major, caller-owned: the gradient in, M_hat
 *                 = P Q^T out (in place).
 *   E             device, n * m fp32, caller-owned error memory (zero before the
 *                 first step): M' = G + E in, E = M' - M_hat out. NULL: no error
 *                 feedback (M' = G).
 *   Q             device, m * r fp32, row-major, caller-owned: in, the warm-start Q
 *                 when q_valid != 0 (otherwise not read); out, Q = M'^T P, the next
 *                 warm-start Q.
 *   P             device, n * r fp32, row-major, caller-owned output: the
 *                 orthogonalized P; may be NULL.
 *   stream        hipStream_t (NULL = the legacy default stream); the current HIP
 *                 device's copy of the working array is used.
 *
 * Every pointer must be 4-byte aligned. No device memory is allocated or freed: the
 * work items, padded factors, Gram partials and partial sums live in a fixed array
 * of 64 MiB per device (allocated when the library is loaded, held until the process
 * ends), which fits every matrix of up to 16384 x 16384 at any rank. All calls on one
 * device share that array: calls that overlap on a device (several streams or
 * threads) race and must be serialized by the caller. Only kernel launches are
 * enqueued (no memset, no copy from host memory), so a call can be captured in a HIP
 * graph; a replay repeats the captured pointers and q_valid.
 * Errors, before anything is enqueued: INVALID_ARG (NULL hp or M or Q, n or m < 1,
 * misaligned pointer, hyperparameters as for powersgd_state_create), UNSUPPORTED
 * (rank above POWERSGD_MAX_RANK, a matrix whose working memory exceeds the array),
 * HIP (no device, launch failure).
 */
POWERSGD_API powersgd_status powersgd_compress_matrix_noalloc(
    const powersgd_hparams* hp, int64_t bucket_index, int32_t view, uint64_t epoch, float* M,
    int64_t n, int64_t m, float* E, float* Q, int32_t q_valid, float* P, void* stream);

/* --- state snapshot (checkpoint / resume) ------------------------------------- */

/*
 * The state PowerSGDState keeps between calls ("PowerSGD State": error memory and
 * warm-start Q per bucket, the iteration counter and the compression statistics) as
 * one host byte string, so a job can checkpoint it and resume with the same
 * trajectory. The pages give no format (GradScaler's state_dict in the AMP page,
 * "Gradient Scaling", is the analogue); this one is defined here.
 *
 * Format, version 1. Little-endian, no padding; i64/u64/u32/i32 integers, f64 and f32
 * IEEE binary64/binary32.
 *   header, 80 bytes:
 *     char[8] "PSGDSNAP"; u32 version = 1; u32 flags (bit 0 use_error_feedback,
 *     bit 1 warm_start); i32 matrix_approximation_rank; u32 reserved = 0;
 *     f64 min_compression_rate; u64 random_seed; i64 iteration; i64 numel_in;
 *     i64 numel_comm; i64 next_log_iteration (first iteration at which the next
 *     statistics line is logged); i64 B = number of bucket records.
 *   B bucket records, in ascending bucket_index:
 *     i64 bucket_index; i64 numel (the batched variant: the length before padding);
 *     u32 variant (bit 0: the batched variant; bits 8-9: the precision of a bucket
 *     compressed through a wrapped entry point, 1 binary16, 2 bfloat16, 0 otherwise;
 *     other bits zero); u32 has_q (1: a warm-start Q follows for every
 *     compressed view); i64 V = number of views;
 *     V view records: i64 offset; i64 ndim; ndim x i64 shape (the batched variant: one
 *     view, offset 0, shape (s, s), s = powersgd_batched_side(numel));
 *     then for each compressed view in view order, n x m its matrix and k = min(r, n,
 *     m) its rank: n*m f32, E row-major (only when flags bit 0 is set), then m*k f32,
 *     Q row-major (only when has_q).
 * E and Q are written as binary32 also for a 16-bit state (exactly); import rounds
 * them to the bucket's precision. A bucket is recorded once it has been called past
 * start_powerSGD_iter (fp16 pass-through tables hold no state and are not recorded).
 */

/*
 * Writes the snapshot of `st` into `host_buf` (host memory, `capacity` bytes) and
 * stores its length in *size. With host_buf NULL only *size is set (a size query).
 * The device-to-host copies are enqueued on `stream` after the work already there and
 * waited for, so the snapshot reflects every call enqueued on that stream before it;
 * calls on other streams must have completed.
 * Errors: INVALID_ARG (NULL state or size, capacity below the length), HIP.
 */
POWERSGD_API powersgd_status powersgd_state_export(powersgd_state* st, void* host_buf,
                                                   int64_t capacity, int64_t* size,
                                                   void* stream);

/*
 * Replaces the state of `st` with a snapshot from powersgd_state_export (host memory,
 * `size` bytes). The snapshot's flags, matrix_approximation_rank, min_compression_rate
 * and random_seed must equal the state's hyperparameters (they decide which memory
 * exists and which random numbers a later call draws); the other hyperparameters are
 * the state's own. Uploads are enqueued on `stream` and waited for; no call on the
 * state may be in flight. The whole snapshot is checked and the new device memory
 * filled before anything of the old state is released: on any error the state is
 * unchanged.
 * Errors: INVALID_ARG (NULL pointers, bad magic or version, mismatched
 * hyperparameters, a record that is inconsistent or runs past `size`, trailing bytes),
 * UNSUPPORTED (a view the library cannot hold), OOM, HIP.
 */
POWERSGD_API powersgd_status powersgd_state_import(powersgd_state* st, const void* host_buf,
                                                   int64_t size, void* stream);

/* --- kernel timing (HIP events on the caller's stream) ------------------------ */

#define POWERSGD_NUM_KERNELS 8
/* kernel kinds: 0 q_init, 1 pass1 (P = M'Q, plus the Gram partials of P for ranks
 * <= 8), 2 orthogonalize (Gram-Schmidt from the Gram partials, P <- P T),
 * 3 pass2 (Q = M'^T P, per row block), 4 pass3 (decompress + error), 5 unscale-only
 * (F16 pass-through), 6 pass2_reduce (sum of pass-2 row-block partials), 7 gram
 * (Gram partials read from P or Q, ranks > 8 and the initial Q) */

/* Turns per-kernel event timing on (non-zero) or off; clears accumulated times. */
POWERSGD_API powersgd_status powersgd_set_timing(powersgd_state* st, int32_t enable);

/*
 * Waits for the recorded events and returns, per kernel kind, the summed duration in
 * milliseconds, the number of launches and the algorithmic bytes those launches
 * moved (minimum HBM traffic of each pass). Arrays of POWERSGD_NUM_KERNELS entries,
 * any may be NULL.
 */
POWERSGD_API powersgd_status powersgd_get_kernel_times(powersgd_state* st, double* ms,
                                          int64_t* launches, double* bytes);

/* Name of a kernel kind ("" if out of range). */
POWERSGD_API const char* powersgd_kernel_name(int32_t kind);

#ifdef __cplusplus
}
#endif

#endif /* POWERSGD_H */
