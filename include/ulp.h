/*
 * ulp.h -- C ABI of libulp: smooth-K low-precision Ulysses pack/unpack for SageAttention
 * inputs, hand-written HIP kernels for gfx950 (MI355X).
 *
 * The method (FlashInfer pages flashinfer.comm._ulysses_lowp.k_grouped_amax,
 * .derive_k_boundary_amax and .unpack_for_sage): in Ulysses sequence parallelism each of
 * P = world_size ranks holds L = local_sequence consecutive rows of Q/K/V laid out
 * [B, L, H, D]; an all-to-all regroups them so destination p holds the full sequence
 * S = P*L for heads [p*h, (p+1)*h), h = H/P.  Instead of BF16/FP16 the exchange carries
 * INT8 Q, INT8 mean-centered ("smooth") K, FP8 E4M3 V, and FP32 scales, one scale per
 * 64-row group of the GLOBAL sequence.  A global group can straddle two shards; its amax
 * is derived from raw-K min/max of every rank touching it, so one stats all-gather is
 * enough.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers, contiguous, row-major, 16-byte aligned.
 *  - dtype is ULP_BF16 or ULP_FP16 and applies to every Q/K/V/k_mean operand of a call.
 *  - head_dim D is 64 or 128; world_size P is 2, 4, 6 or 8 (6 accepted as on the pages);
 *    B, L, H >= 1 and H % P == 0; 0 <= rank < P.
 *  - used_sequence / scale_sequence: ULP_NONE (= None on the pages) or a value in [1, S].
 *  - stream is a hipStream_t passed as void* (NULL = the default stream).  Calls are
 *    asynchronous on that stream and never synchronize the host.
 *  - The library allocates no device memory and keeps no state between calls except a
 *    thread-local error message and, for ulp_k_mean_noalloc, its per-GPU scratch array
 *    (device memory that is part of the library, not allocated).  The caller owns every
 *    buffer.
 *  - Outputs must not alias inputs (except the amax that the derive calls update in
 *    place: ulp_derive_k_boundary_amax, ulp_group_derive, ulp_derive_pack,
 *    ulp_group_derive_pack).
 *  - Every output byte is written by every call, including unused slots and padding (the
 *    chunks of the one-read pair ulp_stats_pack + ulp_derive_pack: by the two together).
 *  - Return value: ULP_OK or an error code; ulp_last_error() then describes the problem.
 *    Argument errors (ULP_EINVAL, ULP_EUNSUPPORTED, ULP_EALIGN) are found on the host
 *    before anything is launched: NOTHING is launched and nothing is written.
 *    ULP_ELAUNCH reports a HIP launch error.  Every entry point makes a single launch,
 *    except ulp_k_mean and ulp_k_mean_noalloc (two) and ulp_group_stats_with_mean (four);
 *    when one of their later
 *    launches fails, the launches queued before it still run, so their workspace and, for
 *    ulp_group_stats_with_mean, the Q statistics (q_amax, q_minmax) may be written.
 *  - Zero-filling of rows >= used_sequence in Q, K and V is a caller contract
 *    (k_grouped_amax, used_sequence parameter); it is not checked.
 *  - Q and K hold finite values.  The statistics order raw 16-bit patterns, so a NaN in
 *    a group gives that group an unspecified amax and min/max (not an error).
 *
 * Layouts (G = 64-row group size):
 *  slots(L)      = L/64 if 64 divides L, else ceil(L/64) + 1: the most global groups an
 *                  L-row shard can touch.  Slot j of rank r is global group
 *                  g0(r) + j, g0(r) = floor(r*L/64); slots the rank does not touch hold
 *                  the 1e-7 floor.
 *  grouped amax  = float [B, H, slots(L)].
 *  minmax        = float [B, H, 2, 2, D]: [.., e, s, d] with e = 0 the rank's first
 *                  touched group, e = 1 its last; s = 0 min, s = 1 max.  Raw values over
 *                  live rows (< used) only, -0 taken as +0; no live row gives
 *                  (+inf, -inf).  The gathered form is [P, B, H, 2, 2, D] in rank order.
 *  chunk         = the bytes source r sends destination p: sections q8 [B,L,h,D] int8,
 *                  k8 [B,L,h,D] int8, v8 [B,L,h,D] E4M3 for heads p*h .. p*h+h-1, then
 *                  q_scale [B,h,slots(L)] and k_scale [B,h,slots(L)] float; every section
 *                  starts on a 256-byte boundary and gaps are zero.  Its size is
 *                  ulp_chunk_bytes().
 *  unpack output = q8, k8 int8 [B, S, h, D]; v8 E4M3 bytes [B, D, h, Spad] with
 *                  Spad = ceil(S/64)*64 and columns [S, Spad) zero; q_scale, k_scale float
 *                  [B, h, W] with W = ceil(n/64), n = scale_sequence or S.
 */
#ifndef ULP_H
#define ULP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ULP_BF16 = 0, ULP_FP16 = 1 } ulp_dtype_t;

enum {
    ULP_OK = 0,
    ULP_EINVAL = 1,        /* an argument is out of its domain, or a pointer is NULL */
    ULP_EUNSUPPORTED = 2,  /* head_dim or world_size outside the supported set */
    ULP_EALIGN = 3,        /* a pointer or stride is not suitably aligned */
    ULP_ELAUNCH = 4        /* the HIP runtime rejected a kernel launch */
};

#define ULP_NONE (-1)      /* None for used_sequence, scale_sequence and aligned */
#define ULP_GROUP_ROWS 64  /* rows per scale group of the global sequence */

/* slots(L, 64) as defined above; 0 when L < 1. */
int64_t ulp_slots(int64_t local_sequence);

/* Consumer scale widths for a live prefix of n rows (unpack_for_sage description: the
 * consumer's scale tensors are as wide as the number of 64-row groups in the rows handed
 * to it).  Writes ceil(n/64) to both outputs.  Returns ULP_EINVAL when n < 1 or a pointer
 * is NULL. */
int ulp_scale_widths(int64_t n, int64_t* q_width, int64_t* k_width);

/* Bytes of one chunk (source -> destination) for batch B, local_sequence L, local_heads h,
 * head_dim D; a multiple of 256.  0 when an argument is < 1. */
int64_t ulp_chunk_bytes(int64_t B, int64_t L, int64_t h, int64_t D);

/* Message for the last nonzero status returned on the calling thread ("" if none). */
const char* ulp_last_error(void);

/* k_grouped_amax (flashinfer.comm._ulysses_lowp.k_grouped_amax: description, Returns).
 * Per touched global group, the partial amax over this rank's rows of the group and all D
 * of |RN(fp32(x) - fp32(k_mean))|, an order-independent max, floored at 1e-7.  When
 * used_sequence < S the one group mixing live rows and zero padding, (used-1)/64, is taken
 * over its live rows only; with used_sequence ULP_NONE or S the result is bit-identical to
 * the unfixed one.  Fully padded groups hold the (deterministic) value over their zero rows.
 *   x       [B, L, H, D] dtype: this rank's shard (K, or Q with k_mean NULL).
 *   k_mean  [B, H, D] dtype, the global K mean already rounded to dtype; NULL = raw values
 *           (mean +0), which is how the Q amax is formed.
 *   out     [B, H, slots(L)] float. */
int ulp_k_grouped_amax(const void* x, const void* k_mean, int dtype, int64_t B, int64_t L,
                       int64_t H, int64_t D, int rank, int world_size, int64_t used_sequence,
                       float* out, void* stream);

/* Raw boundary min/max of one rank's shard: the payload of the single stats all-gather
 * that derive_k_boundary_amax consumes (its description and gathered_minmax parameter).
 *   x    [B, L, H, D] dtype.
 *   out  [B, H, 2, 2, D] float, layout above. */
int ulp_boundary_minmax(const void* x, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
                        int rank, int world_size, int64_t used_sequence, float* out,
                        void* stream);

/* derive_k_boundary_amax (flashinfer.comm._ulysses_lowp.derive_k_boundary_amax:
 * description).  For this rank's first and last touched groups g, overwrites slot
 * g - g0(rank) with the max over every rank r touching g of
 *   max(1e-7, max_d max(RN(maxK[r,g,d] - m[d]), RN(m[d] - minK[r,g,d]))),
 * which equals the direct amax over all live rows of g, bit for bit.
 *   grouped_amax     [B, H, slots(local_sequence)] float, updated in place.
 *   gathered_minmax  [P, B, H, 2, 2, D] float in rank order.
 *   k_mean           [B, H, D] dtype; NULL = mean +0 (the Q boundary merge). */
int ulp_derive_k_boundary_amax(float* grouped_amax, const float* gathered_minmax,
                               const void* k_mean, int dtype, int64_t B, int64_t H, int64_t D,
                               int rank, int64_t local_sequence, int world_size, void* stream);

/* Pack one rank's shard into P chunks (the pack kernel that k_grouped_amax's description
 * says consumes the per-group scales; the chunks are the rows of the all-to-all buffer
 * of unpack_for_sage's recv_u8 parameter).
 * Per slot: scale = RN(amax / 127).  Per element of row l (slot of global row r*L + l):
 *   q8 = clamp(rint(RN(fp32(q) / q_scale)), -127, 127)
 *   k8 = clamp(rint(RN(RN(fp32(k) - fp32(k_mean)) / k_scale)), -127, 127)
 *   v8 = E4M3FN(fp32(v)), round to nearest even, saturating to +-448; with a V scale,
 *        E4M3FN(RN(fp32(v) / v_scale[b, head, d])) (one IEEE binary32 division).
 *   q, k, v         [B, L, H, D] dtype.
 *   k_mean          [B, H, D] dtype.
 *   q_amax, k_amax  [B, H, slots(L)] float (after derive).
 *   v_scale         NULL (V unscaled), or [B, H, D] float indexed by global head: the V
 *                   scale that unpack_for_sage's Returns leave with the caller, which passes
 *                   it on to the consumer itself.  Values should be positive and finite;
 *                   others give whatever the IEEE quotient gives (0 -> +-448, NaN -> NaN).
 *   send            chunk for destination p at send + p * dest_stride_bytes; each chunk is
 *                   ulp_chunk_bytes(B, L, H/P, D) bytes.  dest_stride_bytes must be a
 *                   multiple of 256 and >= the chunk size. */
int ulp_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
             const float* q_amax, const float* k_amax, const float* v_scale, int64_t B,
             int64_t L, int64_t H, int64_t D, int rank, int world_size, uint8_t* send,
             int64_t dest_stride_bytes, void* stream);

/* unpack_for_sage (flashinfer.comm._ulysses_lowp.unpack_for_sage: description, Returns).
 * Turns the P received chunks into contiguous logical Q/K, transposed V with a zero global
 * tail, and global-grid scales at the consumer width.  The scale of global group g comes
 * from the source holding its first row, floor(64*g/L).  Outputs are identical for every
 * value of aligned; aligned == 1 only asserts L % 128 == 0.
 *   recv     [P, chunk_bytes] uint8, source-major.
 *   aligned  ULP_NONE, 0 or 1.
 *   q8, k8   [B, S, h, D] int8;  v8 [B, D, h, Spad] uint8;  q_scale, k_scale [B, h, W]. */
int ulp_unpack_for_sage(const uint8_t* recv, int64_t B, int64_t L, int64_t h, int64_t D,
                        int world_size, int aligned, int64_t scale_sequence, int8_t* q8,
                        int8_t* k8, uint8_t* v8, float* q_scale, float* k_scale,
                        void* stream);

/* ---------------------------------------------------------------------------------
 * Whole-group entry points.  On one GPU that holds the entire Ulysses group these run
 * every rank (or every destination) of a step in a single launch each; results are
 * bit-identical to calling the per-rank entry points above for every rank.
 * Stacked shards are [P, B, L, H, D] (shard r = rows [r*L, (r+1)*L)).
 * The all-to-all buffer is [P_dst, P_src, chunk_bytes]: what rank r sends destination p
 * sits at group + (p*P + r) * chunk_bytes, and destination p's receive buffer is the
 * contiguous [P, chunk_bytes] block at group + p*P*chunk_bytes.
 * --------------------------------------------------------------------------------- */

/* Both statistics of every rank in one pass over Q and K:
 *   q_amax, k_amax    [P, B, H, slots(L)] float  (as ulp_k_grouped_amax per rank; Q raw)
 *   q_minmax, k_minmax [P, B, H, 2, 2, D] float (as ulp_boundary_minmax per rank). */
int ulp_group_stats(const void* q, const void* k, const void* k_mean, int dtype, int64_t B,
                    int64_t L, int64_t H, int64_t D, int world_size, int64_t used_sequence,
                    float* q_amax, float* k_amax, float* q_minmax, float* k_minmax,
                    void* stream);

/* ulp_derive_k_boundary_amax for every rank, for both Q (mean +0) and K. */
int ulp_group_derive(float* q_amax, float* k_amax, const float* q_minmax,
                     const float* k_minmax, const void* k_mean, int dtype, int64_t B,
                     int64_t H, int64_t D, int64_t local_sequence, int world_size,
                     void* stream);

/* ulp_pack for every rank into the all-to-all buffer `group` (layout above); v_scale
 * [B, H, D] (or NULL) is shared by every rank. */
int ulp_group_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
                   const float* q_amax, const float* k_amax, const float* v_scale, int64_t B,
                   int64_t L, int64_t H, int64_t D, int world_size, uint8_t* group,
                   void* stream);

/* ulp_unpack_for_sage for every destination; outputs are stacked over destinations:
 * q8, k8 [P, B, S, h, D]; v8 [P, B, D, h, Spad]; q_scale, k_scale [P, B, h, W]. */
int ulp_group_unpack(const uint8_t* group, int64_t B, int64_t L, int64_t h, int64_t D,
                     int world_size, int aligned, int64_t scale_sequence, int8_t* q8,
                     int8_t* k8, uint8_t* v8, float* q_scale, float* k_scale, void* stream);

/* ---------------------------------------------------------------------------------
 * Statistics and pack from one read of Q, K and V.  The step of the k_grouped_amax and
 * derive_k_boundary_amax pages (description) reads Q and K once for the statistics and
 * once more for the pack that consumes the per-group scales.  derive can change only a
 * rank's first and last slot, and of those only a slot whose group another rank also
 * touches or whose rows all lie in the zero tail (the slot "waits for derive"); every other
 * slot's amax is final as soon as the rank has seen the group's rows.  So:
 *   1. ulp_stats_pack: the grouped amax (Q raw, K centered) and the boundary min/max, as
 *      ulp_k_grouped_amax and ulp_boundary_minmax give them, and the pack of V and of every
 *      Q/K row outside the waiting slots, as ulp_pack gives it, reading each input once;
 *   2. the all-gather of the min/max (on one GPU holding the group: nothing to do);
 *   3. ulp_derive_pack: ulp_derive_k_boundary_amax on both amax (Q with mean +0, K with
 *      k_mean), in place, and the pack of the waiting slots' Q/K rows with the derived
 *      amax (it re-reads at most two groups of rows per (b, head)).
 * After step 3 the amax, min/max and chunks are bit-identical to those of
 * ulp_k_grouped_amax + ulp_boundary_minmax + derive + ulp_pack.  Arguments mean what they
 * mean there; both calls of a step take the same q, k, k_mean, used_sequence and
 * send/group.  The chunks are complete only after step 3.
 * --------------------------------------------------------------------------------- */

/*   q, k, v           [B, L, H, D] dtype (rank `rank`'s shard); k_mean [B, H, D] dtype.
 *   v_scale           NULL or [B, H, D] float, as in ulp_pack.
 *   q_amax, k_amax    [B, H, slots(L)] float (written);  q_minmax, k_minmax [B, H, 2, 2, D].
 *   send, dest_stride_bytes  as in ulp_pack. */
int ulp_stats_pack(const void* q, const void* k, const void* v, const void* k_mean, int dtype,
                   const float* v_scale, int64_t B, int64_t L, int64_t H, int64_t D, int rank,
                   int world_size, int64_t used_sequence, float* q_amax, float* k_amax,
                   float* q_minmax, float* k_minmax, uint8_t* send, int64_t dest_stride_bytes,
                   void* stream);

/*   q_amax, k_amax        [B, H, slots(L)] float from ulp_stats_pack, derived in place.
 *   q_minmax, k_minmax    gathered [P, B, H, 2, 2, D] float (every rank's min/max). */
int ulp_derive_pack(const void* q, const void* k, const void* k_mean, int dtype, float* q_amax,
                    float* k_amax, const float* q_minmax, const float* k_minmax, int64_t B,
                    int64_t L, int64_t H, int64_t D, int rank, int world_size,
                    int64_t used_sequence, uint8_t* send, int64_t dest_stride_bytes,
                    void* stream);

/* The same for every rank of a group held by one GPU: stacked shards [P, B, L, H, D],
 * q_amax, k_amax [P, B, H, slots(L)], q_minmax, k_minmax [P, B, H, 2, 2, D] (written by
 * the first call, read by the second), and the all-to-all buffer `group` laid out as for
 * ulp_group_pack.  Two launches per step instead of the statistics, derive and pack. */
int ulp_group_stats_pack(const void* q, const void* k, const void* v, const void* k_mean,
                         int dtype, const float* v_scale, int64_t B, int64_t L, int64_t H,
                         int64_t D, int world_size, int64_t used_sequence, float* q_amax,
                         float* k_amax, float* q_minmax, float* k_minmax, uint8_t* group,
                         void* stream);
int ulp_group_derive_pack(const void* q, const void* k, const void* k_mean, int dtype,
                          float* q_amax, float* k_amax, const float* q_minmax,
                          const float* k_minmax, int64_t B, int64_t L, int64_t H, int64_t D,
                          int world_size, int64_t used_sequence, uint8_t* group, void* stream);

/* ---------------------------------------------------------------------------------
 * The global K mean (the input k_mean_global of the k_grouped_amax and
 * derive_k_boundary_amax pages, Parameters: a contiguous [B, H, D] mean of K, rounded to the
 * input dtype).  Formed over the live rows [0, used) of the whole sequence from the stacked
 * shards [P, B, L, H, D]: a binary64 sum, divided by used in binary64, rounded to binary32
 * (mean_f32) and from binary32 to the dtype by round-to-nearest-even (mean_dtype).  The
 * reduction order is fixed, so results are reproducible run to run; the binary32 mean is
 * within a relative 1e-6 of the exact mean (in practice equal to the correctly rounded
 * binary64 result).  On several GPUs each rank would sum its own rows and one all-reduce of
 * the [B, H, D] binary64 sums would precede the division.
 * --------------------------------------------------------------------------------- */

/* Bytes of workspace ulp_k_mean needs: 8 * B * H * D * ceil(used / R), used = S when
 * used_sequence is ULP_NONE, with R in {32, 64, ..., 512} chosen from the shape (at most
 * 8 * B * H * D * ceil(used / 32)).  0 when an argument is out of range. */
int64_t ulp_k_mean_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t D, int world_size,
                                   int64_t used_sequence);

/*   k           [P, B, L, H, D] dtype, stacked shards.
 *   workspace   device memory of at least ulp_k_mean_workspace_bytes() bytes, owned by the
 *               caller; its contents on entry do not matter.
 *   mean_f32    [B, H, D] float.
 *   mean_dtype  [B, H, D] dtype, or NULL when only the binary32 mean is wanted. */
int ulp_k_mean(const void* k, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
               int world_size, int64_t used_sequence, void* workspace, int64_t workspace_bytes,
               float* mean_f32, void* mean_dtype, void* stream);

/* ulp_k_mean for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation and
 * bits, with the workspace taken from a device array inside the library instead of an
 * argument.  The library holds 16 MiB of it per GPU it runs on until the process ends
 * (enough for K of up to 2 GiB at any shape); a shape whose ulp_k_mean_workspace_bytes()
 * exceeds that returns ULP_EINVAL with nothing launched.  Every call on one GPU uses that
 * GPU's single array, so calls that overlap on one GPU (on two streams, or from two
 * threads) race; calls in stream order do not.  The array's contents on entry do not
 * matter.  Allocates nothing and calls no allocating routine; the first call on a device
 * looks up the array's device address.  Arguments as ulp_k_mean. */
int ulp_k_mean_noalloc(const void* k, int dtype, int64_t B, int64_t L, int64_t H, int64_t D,
                       int world_size, int64_t used_sequence, float* mean_f32,
                       void* mean_dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * Statistics of every rank together with the global K mean, reading Q and K once each.
 * The centered amax of k_grouped_amax (description) needs k_mean_global (Parameters), and
 * forming that mean is itself a pass over K; here one pass over K records, per (rank, b,
 * head, slot, channel), the raw min / max over the rows the amax runs on and the binary64
 * sum over live rows.  The mean follows from the sums (same definition as ulp_k_mean) and
 * every slot's amax from max_d max(RN(max - m), RN(m - min)) with m the dtype mean, the
 * identity derive_k_boundary_amax (description) rests on: outputs are bit-identical to
 * ulp_group_stats run with this mean.
 *   q, k        stacked [P, B, L, H, D] dtype.
 *   workspace   device memory of ulp_group_stats_with_mean_workspace_bytes() bytes, 8-byte
 *               aligned at least, owned by the caller; contents on entry do not matter.
 *   q_amax, k_amax      [P, B, H, slots(L)] float;  q_minmax, k_minmax [P, B, H, 2, 2, D].
 *   k_mean_f32  [B, H, D] float;  k_mean_dtype [B, H, D] dtype (the k_mean_global to pass
 *               on to derive and pack).
 * Four launches: the Q statistics first, then the K pass, the mean and the K amax.  A
 * ULP_ELAUNCH from one of the K launches leaves q_amax and q_minmax written.
 * --------------------------------------------------------------------------------- */
int64_t ulp_group_stats_with_mean_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t D,
                                                  int world_size);
int ulp_group_stats_with_mean(const void* q, const void* k, int dtype, int64_t B, int64_t L,
                              int64_t H, int64_t D, int world_size, int64_t used_sequence,
                              void* workspace, int64_t workspace_bytes, float* q_amax,
                              float* k_amax, float* q_minmax, float* k_minmax,
                              float* k_mean_f32, void* k_mean_dtype, void* stream);

/* ---------------------------------------------------------------------------------
 * Consumer check (not a step of the pack/unpack path).  Attention over one destination's
 * unpacked tensors, read the way the Sage consumer named by unpack_for_sage (description,
 * Returns) reads them: for rows i, t < used,
 *   score(i, t) = (q8[b,i,j,:] . k8[b,t,j,:]) * q_scale[b,j,i/64] * k_scale[b,j,t/64] / sqrt(D)
 *   out[b,i,j,d] = sum_t softmax_t(score(i, .)) * e4m3(v8[b,d,j,t]) * (v_scale ? v_scale[b,j,d] : 1)
 * INT8 Q.K on MFMA (exact integer dot products); P quantized to E4M3 after scaling by 448
 * and P.V on FP8 MFMA with FP32 accumulation, so each probability carries a relative
 * rounding error of at most 2^-4 (absolute 2^-18 in the subnormal range); each row is
 * normalized by the sum of its rounded probabilities.  Softmax without a causal mask.
 *   q8, k8     [B, S, h, D] int8;  v8 [B, D, h, Spad] E4M3 bytes, Spad = ceil(S/64)*64.
 *   q_scale, k_scale [B, h, W] float with W >= ceil(used/64); these two need only 4-byte
 *              alignment (a destination's slice of stacked scale tensors need not be
 *              16-byte aligned).
 *   v_scale    [B, h, D] float (this destination's heads) or NULL.
 *   out        [B, used, h, D] float.
 * D is 64 or 128; 1 <= used <= S; one batch entry of k8 (S*h*D bytes) and of v8
 * (D*h*Spad bytes) must each be below 2 GiB (the kernel addresses a batch entry with 32-bit
 * offsets), else ULP_EINVAL. */
int ulp_consumer_attention(const int8_t* q8, const int8_t* k8, const uint8_t* v8,
                           const float* q_scale, const float* k_scale, const float* v_scale,
                           int64_t B, int64_t S, int64_t h, int64_t D, int64_t W,
                           int64_t used, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ULP_H */
