/*
 * cpthd.h - C ABI of libcpthd, the MI355X (gfx950) library for the THD
 * context-parallel token layout and the owner gradient return.
 *
 * Tensors are packed THD: all documents concatenated along tokens, shape
 * [T, H, D], row-major, so one token ("row") is H*D elements.  Document
 * boundaries are int32 cu_seqlens[B+1] (cu[0] = 0, cu[B] = T).  W is the CP
 * size (number of ranks).  On one GPU the W ranks are emulated by W buffers
 * (slots) in the same HBM.
 *
 * Sources (web pages, by title and section):
 *  [PC]  "[PyTorch] Add experimental packed-contiguous THD all-gather CP"
 *        (TransformerEngine PR 3221): sections "Conversation" (commit
 *        messages), "Why", "Scope and constraints".
 *  [GR]  "Add stream-ordered CP gradient return primitive"
 *        (TransformerEngine PR 3235): sections "Description", "Changes",
 *        "Sequence Diagram", "Validation", and the author's reply on CP size.
 *  [LL]  "Low Latency Communication Kernels with NVSHMEM" (GPU MODE lecture
 *        87 notes): exercise list (1 KB - 16 MB sum sweep; one-shot against
 *        ring all-reduce) and the all-reduce algorithms chosen by message size.
 *  [MM]  "Kernel-level compute-communication overlapping for CP linear
 *        attention kernels via nvshmem" (cuLA issue 15): replies on buffer
 *        ownership (buffers allocated outside the module, lifetime owned by
 *        the caller).
 *
 * Conventions common to every entry point
 *  - Every data pointer is a device pointer of the CURRENT HIP device,
 *    allocated by the caller ([MM]; [GR] "Description": peer tensor views are
 *    supplied by the caller).  The library allocates no device memory.  The
 *    only host state kept between calls is the timing record of cp_profile_*
 *    and, per metadata buffer built by cp_build_meta, its policy and sizes,
 *    used to choose kernel tile shapes and the shape the permutation kernels
 *    start their row lookups (or closed-form row maps) from (every kernel
 *    checks the metadata itself and follows it, so a buffer rewritten by other
 *    means still gives exact results).
 *  - Host pointer tables (const void* const*) are read only during the call.
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream) and never synchronizes, except cp_meta_status and
 *    cp_profile_read, which say so.  ([GR] "Description": stream-ordered.)
 *  - Host-side validation runs first.  On any error nothing is launched and
 *    the status is returned: fail-closed ([GR] reply on CP size: a
 *    fail-closed validation boundary; [PC] "Scope and constraints": FP8 and
 *    unvalidated combinations are rejected).
 *  - Checks that depend on device data (the cu_seqlens values) are made on
 *    the device by cp_build_meta, which records them in the meta header.
 *    Every later kernel reads the header first and does nothing (writes no
 *    output byte) when the metadata is invalid or does not match the call;
 *    the mismatch is recorded as a sticky CP_CALL_* flag, and
 *    cp_meta_status reports both.
 *  - The metadata buffer (`meta`) is passed as a non-const pointer to every
 *    call whose kernels may write it: they OR the sticky CP_CALL_* flags into
 *    its header, and the gradient return's epoch wait records its timeout mask
 *    there (both atomically, so calls on several streams may share one
 *    metadata buffer).  Nothing else in the buffer is written after
 *    cp_build_meta.  `meta` must be 16-byte aligned (CP_ERR_ARG otherwise):
 *    kernels read its 64-byte header with 16-byte loads.
 *  - Outputs must not overlap inputs or each other (CP_ERR_ALIAS); [GR]
 *    "Description" (self-alias assertions on the rank-self slots).  The
 *    metadata header counts as an output of every call that takes `meta`, its
 *    tables (cu_seqlens and the per-rank tables after the header) as an input:
 *    over the whole cp_meta_bytes(B, W) extent when the call names B and W or
 *    the host built the metadata at that address for the call's token count
 *    (and CP size), else over the header alone.
 *  - Every buffer must be device memory of the current device (else
 *    CP_ERR_DEVICE) and, as far as the runtime reports allocation extents,
 *    lie inside one allocation for the byte count the call's sizes imply
 *    (else CP_ERR_SHAPE: the buffer is smaller than the sizes say).  Sizes
 *    whose byte counts would exceed 2^62 give CP_ERR_ARG.
 */
#ifndef CPTHD_H
#define CPTHD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t; spelled out so this header needs no HIP header. */
typedef struct ihipStream_t* cp_stream_t;

/* ------------------------------------------------------------ status codes */
enum cp_status {
  CP_OK = 0,
  CP_ERR_ARG = 1,         /* bad scalar argument or NULL pointer             */
  CP_ERR_UNSUPPORTED = 2, /* dtype / mode not supported (FP8, a gradient
                             dtype pair other than the four listed)          */
  CP_ERR_SHAPE = 3,       /* sizes inconsistent (T % W under PC, buffer too
                             small, ...)                                     */
  CP_ERR_DEVICE = 4,      /* a pointer is not device memory of the current
                             device                                          */
  CP_ERR_ALIAS = 5,       /* an output overlaps an input or another output   */
  CP_ERR_HIP = 6,         /* a HIP runtime call failed                       */
  CP_ERR_TIMEOUT = 7,     /* device-reported: an epoch wait hit its limit    */
  CP_ERR_META = 8,        /* device-reported: invalid cu_seqlens, or a call
                             that did not match its metadata                 */
  CP_ERR_TOO_LARGE = 9    /* the call needs more workspace than the static
                             one of cp_grad_return_noalloc holds             */
};

/* ownership policies ([PC] "Why" and commit messages) */
enum cp_policy {
  CP_POLICY_DUAL_CHUNK_SWAP = 0,   /* per-document 2W chunks, rank r owns r and 2W-1-r */
  CP_POLICY_PACKED_CONTIGUOUS = 1  /* rank r owns tokens [rT/W, (r+1)T/W)              */
};

/* element types; FP8 is recognised and rejected ([PC] "Scope and constraints") */
enum cp_dtype {
  CP_F32 = 0,
  CP_BF16 = 1,
  CP_F16 = 2,
  CP_FP8_E4M3 = 3,
  CP_FP8_E5M2 = 4
};

#define CP_ALL_RANKS (-1)
#define CP_MAX_CP_SIZE 64

/* phases of cp_grad_return ([GR] "Sequence Diagram": scatter, epoch publish,
 * epoch wait, accumulate); CP_PHASE_ALL runs the four in that order */
#define CP_PHASE_SCATTER 0x1
#define CP_PHASE_PUBLISH 0x2
#define CP_PHASE_WAIT    0x4
#define CP_PHASE_SUM     0x8
#define CP_PHASE_ALL     0xF

/* Accumulate mode of the owner-side sum, accepted in `phases` of cp_grad_return
 * and in `flags` of cp_grad_return_fused and cp_slot_sum.  [GR] "Sequence
 * Diagram" accumulates the writer slots 0..cp_size-1 "to dk"; read literally,
 * one slot at a time into the owner's gradient:
 *     out = (((out + s_0) + s_1) + ...) + s_{W-1}
 * in fp32 (out widened first), rounded once to out_dtype.  Without the flag
 * out is overwritten with ((s_0 + s_1) + ...) + s_{W-1}. */
#define CP_SUM_ACCUMULATE 0x10

/* ------------------------------------------------------------ metadata */
/*
 * Device metadata built by cp_build_meta in a caller-allocated buffer of
 * cp_meta_bytes(B, W) bytes:
 *   offset 0                         cp_meta_header (64 bytes)
 *   offset 64                        int32 cu_seqlens[B+1]   (copy of the input)
 *   offset 64 + 4(B+1)               int32 local_cu[W][B+1]  (per-rank cu_seqlens)
 *   offset 64 + 4(B+1)(W+1)          int32 n_local[W]        (documents per rank)
 *
 * local_cu (the per-rank sequence metadata of [PC] "Conversation"):
 *   dual-chunk-swap:    local_cu[r][b] = cu[b] / W for every r; n_local[r] = B.
 *                        (A rank's rows are document-major; inside a document,
 *                        chunk r precedes chunk 2W-1-r.)
 *   packed-contiguous:  the ascending set {0} + {cu[b] - r*T/W : r*T/W < cu[b] <
 *                        (r+1)*T/W} + {T/W}, i.e. the documents clipped at the
 *                        rank's slice, without empty segments; n_local[r] = its
 *                        length - 1; the entries after it are T/W.
 *
 * Optional row maps (dual-chunk-swap), written when the buffer holds at least
 * cp_meta_bytes_row_maps(B, W, T) bytes; cp_meta_header.row_maps is then 1:
 *   offset cp_meta_bytes(B, W)       int32 row_of_local[T]: global row of the
 *                                    flat local row p = r*(T/W) + i
 *   offset cp_meta_bytes(B, W) + 4T  int32 local_of_row[T]: the inverse
 * The permutation kernels then find any row's source and destination with one
 * load instead of searching the document table (the tables alone give the same
 * results; the maps are a lookup aid, 8 bytes per token).
 */
#define CP_META_MAGIC 0x48545043u /* "CPTH" */

/* cp_meta_header.flags: set by cp_build_meta (device-side validation) */
#define CP_META_FIRST_NOT_ZERO    0x0001 /* cu[0] != 0                                   */
#define CP_META_DECREASING        0x0002 /* cu[b+1] < cu[b] for some b                   */
#define CP_META_LAST_NOT_TOTAL    0x0004 /* cu[B] != total_tokens                        */
#define CP_META_DOC_NOT_DIVISIBLE 0x0008 /* dual-chunk-swap: some L_b % (2W) != 0        */
#define CP_META_BUILD_MASK        0x00FF
/* cp_meta_header.flags: sticky errors OR-ed in by later calls' kernels */
#define CP_CALL_BAD_MAGIC         0x0100 /* meta was never built                         */
#define CP_CALL_TOKENS_MISMATCH   0x0200 /* total_tokens differs from the meta's          */
#define CP_CALL_CP_SIZE_MISMATCH  0x0400 /* cp_size differs from the meta's               */
#define CP_CALL_POLICY_MISMATCH   0x0800 /* reserved: a call bound to the other policy     */
#define CP_CALL_USED_INVALID_META 0x1000 /* a kernel met invalid metadata and did nothing */
#define CP_CALL_DOCS_MISMATCH     0x2000 /* num_docs differs from the meta's              */

typedef struct cp_meta_header {
  uint32_t magic;             /* CP_META_MAGIC once built                        */
  int32_t flags;              /* CP_META_* | CP_CALL_*                           */
  int32_t policy;             /* enum cp_policy                                  */
  int32_t cp_size;            /* W                                               */
  int32_t num_docs;           /* B                                               */
  int32_t reserved0;
  int64_t total_tokens;       /* T                                               */
  int64_t local_tokens;       /* T / W                                           */
  uint64_t wait_timeout_ranks;/* bit o set: owner o's last epoch wait timed out  */
  int32_t row_maps;           /* 1: the row maps follow the tables, else 0       */
  int32_t reserved[3];
} cp_meta_header;

/* Bytes the caller must allocate for the metadata of B documents and W ranks
 * (a multiple of 256).  Returns 0 for B outside [0, 2^31 - 2] or W outside
 * [1, CP_MAX_CP_SIZE]. */
size_t cp_meta_bytes(int32_t num_docs, int32_t cp_size);

/* Bytes for the metadata plus the optional row maps of T tokens:
 * cp_meta_bytes(B, W) + 8T rounded up to a multiple of 256.  Returns 0 for B
 * or W out of range (as cp_meta_bytes) or T outside [0, 2^31). */
size_t cp_meta_bytes_row_maps(int32_t num_docs, int32_t cp_size, int64_t total_tokens);

/*
 * cp_build_meta - validate cu_seqlens and build the per-rank metadata.
 * Source: [PC] "Why" (dual-chunk-swap divides every sequence into 2*cp_size
 * chunks; packed-contiguous uses the whole buffer as the sharding unit, cp_size
 * equal chunks) and "Conversation" (document boundaries kept through sequence
 * metadata; packed metadata is one chunk per rank); [GR] author's reply (owner
 * o receives chunks o and 2N-1-o, sized from cp_size).
 *
 *   cu_seqlens    device int32[num_docs+1]
 *   num_docs      B in [0, 2^31 - 2] (B + 1 entries must fit an int32 count)
 *   total_tokens  T, 0 <= T < 2^31
 *   cp_size       W in [1, 64]
 *   policy        enum cp_policy
 *   meta          device buffer of at least meta_bytes >= cp_meta_bytes(B, W),
 *                 16-byte aligned; under dual-chunk-swap with meta_bytes >=
 *                 cp_meta_bytes_row_maps(B, W, T) the row maps are written too
 * Host errors: CP_ERR_ARG (range, NULL), CP_ERR_SHAPE (packed-contiguous with
 * T % W != 0; meta_bytes too small), CP_ERR_DEVICE, CP_ERR_ALIAS (meta overlaps
 * cu_seqlens), CP_ERR_HIP.  Data errors (cu[0] != 0, decreasing cu, cu[B] != T,
 * dual-chunk-swap document not divisible by 2W) are written to the header
 * flags on the device; read them with cp_meta_status.
 */
int cp_build_meta(const int32_t* cu_seqlens, int32_t num_docs, int64_t total_tokens,
                  int32_t cp_size, int32_t policy, void* meta, size_t meta_bytes,
                  cp_stream_t stream);

/*
 * cp_meta_status - synchronize `stream`, then read the header flags.
 * Returns CP_OK when no flag is set and no epoch wait timed out; CP_ERR_META
 * when a CP_META_* or CP_CALL_* flag is set; CP_ERR_TIMEOUT when only
 * wait_timeout_ranks is non-zero; CP_ERR_ARG/CP_ERR_DEVICE/CP_ERR_HIP on a bad
 * call.  *flags_out (may be NULL) receives the flags word, *timeouts_out (may be
 * NULL) the wait_timeout_ranks mask.
 */
int cp_meta_status(const void* meta, cp_stream_t stream, int32_t* flags_out,
                   uint64_t* timeouts_out);

/* ------------------------------------------------------------ attention steps */
/*
 * Per-rank attention-step metadata for all-gather CP: which local query rows
 * attend to which rows of the all-gathered key/value buffer (global token
 * order: the output of cp_gather_thd).  Source: [PC] "Why" (the per-document
 * partition performs two attention steps per rank, packed-contiguous one) and
 * "Scope and constraints" (THD self-attention, all-gather CP, full causal mask,
 * no inter-sequence padding); commit messages (document boundaries retained
 * through sequence metadata; packed metadata simplified to one chunk and one
 * attention step per rank).  Attention is causal inside each document: token t
 * sees token s when they share a document and s <= t.
 *
 *   dual-chunk-swap, rank r: step 0 = chunk r of every document, step 1 =
 *     chunk 2W-1-r; chunk k of document b (chunk length c_b = L_b / 2W) sees
 *     the document's first (k+1) c_b tokens.  B segments per step (empty
 *     documents give empty segments).
 *   packed-contiguous, rank r: one step (the second record is empty); every
 *     local segment (a document clipped to the rank's slice, as in local_cu)
 *     sees its document from the first token up to the segment's last token.
 * In every segment the queries are the LAST q_len tokens of its key range (the
 * causal mask aligned at the bottom right of the q_len x kv_len block).
 *
 * Layout (cp_attn_meta_bytes(B, W) bytes, caller-allocated, device memory):
 *   offset 0    cp_attn_header (64 bytes)
 *   offset 64   2W step records, rank-major (rank r step s at index 2r + s),
 *               each 32 + 16(B+1) bytes:
 *     int32 num_segments   m (B under dual-chunk-swap; n_local[r] or 0 under
 *                          packed-contiguous)
 *     int32 max_seqlen_q, max_seqlen_kv   longest segment (0 if m = 0)
 *     int32 total_q, total_kv             sums of the segment lengths
 *     int32 reserved[3]
 *     int32 cu_seqlens_q[B+1]   0, q_len_0, q_len_0 + q_len_1, ...; entries
 *                               after m repeat total_q
 *     int32 cu_seqlens_kv[B+1]  the same for kv_len (entries after m: total_kv)
 *     int32 q_offsets[B+1]      q_start of segment j in the rank's [T/W] local
 *                               buffer; entries from m on hold T/W
 *     int32 kv_offsets[B+1]     kv_start of segment j in the gathered [T]
 *                               buffer; entries from m on hold T
 */
#define CP_ATTN_MAGIC 0x54414350u /* "PCAT" */

typedef struct cp_attn_header {
  uint32_t magic;             /* CP_ATTN_MAGIC when built from valid metadata, else 0 */
  int32_t policy;
  int32_t cp_size;            /* W                                                    */
  int32_t num_docs;           /* B                                                    */
  int32_t num_steps;          /* 2 (dual-chunk-swap) or 1 (packed-contiguous)         */
  int32_t reserved0;
  int64_t total_tokens;       /* T                                                    */
  int64_t local_tokens;       /* T / W                                                */
  int32_t reserved[6];
} cp_attn_header;

/* Bytes of the attention-step metadata of B documents and W ranks (a multiple
 * of 256); 0 for B outside [0, 2^31 - 2] or W outside [1, CP_MAX_CP_SIZE]. */
size_t cp_attn_meta_bytes(int32_t num_docs, int32_t cp_size);

/*
 * cp_build_attn_meta - fill the attention-step metadata of every rank from
 * metadata built by cp_build_meta (either policy).
 *   meta        device metadata of num_docs documents and cp_size ranks
 *   attn        device buffer of attn_bytes >= cp_attn_meta_bytes(B, W) bytes;
 *               must not overlap meta
 * Host errors: CP_ERR_ARG (NULL, ranges), CP_ERR_SHAPE (attn_bytes too small),
 * CP_ERR_DEVICE, CP_ERR_ALIAS, CP_ERR_HIP.  On the device, invalid metadata or
 * a num_docs / cp_size that differs from the meta's sets the meta's sticky
 * CP_CALL_* flag (read with cp_meta_status), and the attention header's magic
 * is written as 0 with no step record written (fail-closed).
 */
int cp_build_attn_meta(void* meta, int32_t num_docs, int32_t cp_size, void* attn,
                       size_t attn_bytes, cp_stream_t stream);

/* ------------------------------------------------------------ token layout */
/*
 * cp_partition_thd - split a global THD tensor into the W per-rank layouts.
 * Source: [PC] "Why" and commit messages (per-document dual-chunk-swap; one
 * contiguous chunk per rank for packed-contiguous); [GR] author's reply
 * (ownership rule).  parts[r][i] = x[g_r(i)], where g_r lists rank r's global
 * tokens in local order (documented at the metadata above).  A bit copy.
 *
 *   x            device [T, H, D] of `dtype`            (input)
 *   parts        device [W, T/W, H, D] of `dtype`       (output)
 *   total_tokens T (must equal the meta's), heads H >= 1, head_dim D >= 1
 *   dtype        CP_F32 / CP_BF16 / CP_F16 (FP8 -> CP_ERR_UNSUPPORTED)
 *   meta         built by cp_build_meta (either policy)
 * total_tokens == 0 is a no-op after the scalar checks (x, parts may be NULL).
 * Errors: CP_ERR_ARG, CP_ERR_UNSUPPORTED, CP_ERR_DEVICE, CP_ERR_ALIAS
 * (parts overlaps x or meta), CP_ERR_HIP; metadata mismatch is recorded in the
 * meta flags and the kernel writes nothing.
 */
int cp_partition_thd(const void* x, void* parts, int64_t total_tokens, int32_t heads,
                     int32_t head_dim, int32_t dtype, void* meta, cp_stream_t stream);

/*
 * cp_gather_thd - inverse of cp_partition_thd: x[g_r(i)] = parts[r][i]
 * (the key/value reorder after an all-gather, [PC] commit messages: the
 * rank-major packed-contiguous layout needs no reorder, dual-chunk-swap does).
 * Same arguments, roles of x and parts swapped (parts input, x output).
 */
int cp_gather_thd(const void* parts, void* x, int64_t total_tokens, int32_t heads,
                  int32_t head_dim, int32_t dtype, void* meta, cp_stream_t stream);

/*
 * cp_partition_thd_multi / cp_gather_thd_multi - the same operations on
 * n_tensors tensors of one shape in one launch (the pages partition Q, K and
 * V together: [PC] "Why").  xs[t] and parts[t] (host tables of n_tensors
 * device pointers) are tensor t's x [T, H, D] and parts [W, T/W, H, D];
 * 1 <= n_tensors <= 8.  Every output must be disjoint from every input and
 * from every other output.  Errors as cp_partition_thd.  (The library runs
 * small tensors in one launch and tensors of >= 1 GiB of traffic each in one
 * launch per tensor, whichever streams faster.)
 */
int cp_partition_thd_multi(int32_t n_tensors, const void* const* xs, void* const* parts,
                           int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                           void* meta, cp_stream_t stream);
int cp_gather_thd_multi(int32_t n_tensors, const void* const* parts, void* const* xs,
                        int64_t total_tokens, int32_t heads, int32_t head_dim, int32_t dtype,
                        void* meta, cp_stream_t stream);

/* ------------------------------------------------------------ gradient return */
/*
 * cp_grad_return - owner gradient return: scatter, epoch publish, epoch wait,
 * fixed-order slot sum.
 * Source: [GR] "Description" (scatter global dK/dV into owner buffers in the
 * native two-chunk CP layout; publish writer epochs; wait for all writers;
 * accumulate the writer slots into the owner's dK/dV; the caller supplies the
 * peer views) and "Sequence Diagram" (slot index [owner][writer rank]; wait
 * until every epoch slot >= epoch; accumulate slots 0..cp_size-1).
 *
 *   rank         CP_ALL_RANKS: emulate all W ranks in stream order on `stream`.
 *                0..W-1: the part of rank `rank` only (scatter its own
 *                gradient to every owner, publish its epoch to every owner,
 *                wait for its own W epochs, sum its own slots).  With
 *                CP_PHASE_ALL the W ranks' calls MUST run concurrently, on W
 *                streams that map to distinct hardware queues: a wait that
 *                precedes another writer's publish in the same queue ends in
 *                CP_ERR_TIMEOUT (see `phases` for the split that avoids it).
 *   cp_size      W, must equal the meta's.  Either policy: owner o's rows
 *                are those the partition gives rank o (the two-chunk layout
 *                under dual-chunk-swap, tokens [o T/W, (o+1) T/W) under
 *                packed-contiguous).
 *   n_tensors    number of gradient tensors per rank (2 for dK, dV), >= 1
 *   grads        host table [n_tensors][W] of device [T, H, D] `in_dtype`:
 *                writer w's global gradient of tensor t
 *   slots        host table [n_tensors][W owner][W writer] of device
 *                [T/W, H, D] `in_dtype`: the owner's receive slots
 *   out          host table [n_tensors][W owner] of device [T/W, H, D]
 *                `out_dtype`: overwritten with the sum, or accumulated into
 *                with CP_SUM_ACCUMULATE
 *   in_dtype/out_dtype  (CP_F32, CP_F32), (CP_F32, CP_BF16), (CP_BF16, CP_BF16),
 *                (CP_BF16, CP_F32)
 *   phases       CP_PHASE_* mask (at least one phase), optionally with
 *                CP_SUM_ACCUMULATE; phases run in the order scatter, publish,
 *                wait, sum.  CP_PHASE_ALL is the whole protocol.  A caller that
 *                drives several emulated ranks from one process may enqueue
 *                every rank's SCATTER|PUBLISH half before any rank's WAIT|SUM
 *                half, so that ranks sharing a hardware queue cannot block
 *                each other.
 *   epochs       device uint32 [W owner][W writer].  Required when rank >= 0.
 *                In CP_ALL_RANKS mode it may be NULL: the publish and wait
 *                phases are then skipped and ordering is stream order alone.  Writers store `epoch` with release semantics;
 *                owners wait until every entry of their row is >= epoch.
 *   epoch        must exceed every value already in `epochs` (the caller owns
 *                the counter; there is no hidden per-buffer epoch state).
 *   wait_timeout_us  bound on the device-side wait (<= 0: 2 seconds).  On
 *                timeout the owner's bit in meta wait_timeout_ranks is set and
 *                the owner's sum writes nothing (fail-closed).
 * Sum: out = ((s_0 + s_1) + s_2) + ... + s_{W-1} in fp32, s_w = widened slot w,
 * accumulator seeded with s_0 (with CP_SUM_ACCUMULATE: seeded with the widened
 * out, then s_0 ... s_{W-1} added), then rounded once to out_dtype (bf16:
 * round-to-nearest-even).
 * In per-rank mode the call reads grads[t][rank], writes slots[t][o][rank] for
 * every o, reads slots[t][rank][*] and writes out[t][rank]; only those table
 * entries must be valid.
 * total_tokens == 0 is a no-op after the scalar checks (pointers may be NULL).
 * Errors: CP_ERR_ARG, CP_ERR_UNSUPPORTED (dtype pair), CP_ERR_SHAPE (T not a
 * multiple of W), CP_ERR_DEVICE, CP_ERR_ALIAS, CP_ERR_HIP; device-side
 * mismatch or timeout as above.
 */
int cp_grad_return(int32_t rank, int32_t cp_size, int32_t n_tensors,
                   const void* const* grads, void* const* slots, void* const* out,
                   int64_t total_tokens, int32_t heads, int32_t head_dim,
                   int32_t in_dtype, int32_t out_dtype, void* meta,
                   uint32_t* epochs, uint32_t epoch, int64_t wait_timeout_us,
                   int32_t phases, cp_stream_t stream);

/*
 * cp_grad_return_fused - the same result as cp_grad_return with no slots:
 * out[t][o][i] = sum over w = 0..W-1 (in that order, fp32, seeded with w = 0)
 * of grads[t][w][g_o(i)], rounded once to out_dtype.  Bitwise identical to the
 * unfused path.  Source: [GR] "Description" (scatter and accumulate, composed
 * into one pass; each owner pulls its two chunks from every writer's view).
 *
 *   rank         CP_ALL_RANKS: every owner; 0..W-1: owner `rank` only (it reads
 *                all W writers' views, which must be complete in stream order)
 *   flags        0 or CP_SUM_ACCUMULATE (seed the sum with the current out)
 *   other arguments as cp_grad_return; only grads[t][*] and out[t][o] used.
 */
int cp_grad_return_fused(int32_t rank, int32_t cp_size, int32_t n_tensors,
                         const void* const* grads, void* const* out, int64_t total_tokens,
                         int32_t heads, int32_t head_dim, int32_t in_dtype,
                         int32_t out_dtype, void* meta, int32_t flags,
                         cp_stream_t stream);

/*
 * cp_slot_sum - out[k] = ((s_0[k] + s_1[k]) + ...) + s_{W-1}[k] in fp32, for
 * flat buffers: the owner-side reduction of [GR] "Sequence Diagram" on its own,
 * as used by the small-message sweep of [LL] exercise list (1 KB - 16 MB).
 *   num_slots    W in [1, 64]
 *   slots        host table [W] of device buffers of n_elems `in_dtype`
 *   out          device buffer of n_elems `out_dtype`
 *   dtype pairs  as cp_grad_return
 *   flags        0 or CP_SUM_ACCUMULATE (out = ((out + s_0) + ...) + s_{W-1})
 * n_elems == 0 is a no-op (pointers may then be NULL).
 */
int cp_slot_sum(int32_t num_slots, const void* const* slots, void* out, int64_t n_elems,
                int32_t in_dtype, int32_t out_dtype, int32_t flags, cp_stream_t stream);

/*
 * cp_grad_return_noalloc - cp_grad_return for every rank in stream order
 * (rank = CP_ALL_RANKS, no epochs), with the owner slots kept in the library's
 * own static device workspace instead of caller buffers.  For callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The call allocates nothing; the
 * workspace is one fixed array of CP_NOALLOC_SCRATCH_BYTES bytes on each GPU,
 * reserved when the library's device code is loaded on that GPU and held until
 * the process ends.
 *
 *   cp_size, n_tensors, grads, out, total_tokens, heads, head_dim, in_dtype,
 *   out_dtype, meta   as cp_grad_return (grads [n_tensors][W] inputs, out
 *                     [n_tensors][W] outputs, every entry used)
 *   flags             0 or CP_SUM_ACCUMULATE
 * Slot [t][o][w] (T/W rows of writer w's tensor t for owner o) takes
 * (T/W) * H * D * size(in_dtype) bytes rounded up to a multiple of 256;
 * n_tensors * W * W slots must fit in CP_NOALLOC_SCRATCH_BYTES, else
 * CP_ERR_TOO_LARGE and nothing is launched.  The results are the bits
 * cp_grad_return gives with CP_ALL_RANKS, no epochs and the same flags.
 * Every call on one GPU shares that GPU's workspace, which keeps the last
 * call's slots: calls that overlap in time on one GPU (unordered streams, or
 * several host threads) race and give undefined results.  Other errors as
 * cp_grad_return.
 */
#define CP_NOALLOC_SCRATCH_BYTES 67108864 /* 64 MiB */
int cp_grad_return_noalloc(int32_t cp_size, int32_t n_tensors, const void* const* grads,
                           void* const* out, int64_t total_tokens, int32_t heads,
                           int32_t head_dim, int32_t in_dtype, int32_t out_dtype, void* meta,
                           int32_t flags, cp_stream_t stream);

/* ------------------------------------------------------------ all-reduce */
#define CP_ALLREDUCE_ONE_SHOT 0
#define CP_ALLREDUCE_RING     1
#define CP_ALLREDUCE_TWO_SHOT 2

/*
 * cp_allreduce - all W ranks, emulated by W buffers on this device, end with
 * the sum of all W inputs: out[r][k] = in[0][k] + ... + in[W-1][k] for every
 * rank r.  The algorithms of [LL] (the all-reduce menu by message size;
 * exercises 2-3, one-shot against ring over 1 KB - 16 MB), and a two-shot:
 *   CP_ALLREDUCE_ONE_SHOT  one launch: every rank reads all W inputs and sums
 *       them in rank order 0..W-1 in fp32 (seeded with in[0]), rounding once
 *       to dtype.  Every rank's out holds the same bits as cp_slot_sum.
 *   CP_ALLREDUCE_RING      the buffer is cut into W chunks of q elements,
 *       q = ceil(n_elems / W) (chunk c = [c q, (c+1) q) clipped to n_elems;
 *       the last non-empty chunk may be shorter, trailing chunks empty).  Reduce-scatter: W-1 steps;
 *       in step s rank r takes chunk (r-1-s) mod W from rank r-1 (rank r-1's
 *       input at s = 0, its out after) and writes that plus its own input
 *       chunk, added in fp32 and rounded to dtype, into out[r].  Chunk c is
 *       thus summed in rank order c, c+1, ..., c-1 (mod W), rounded after
 *       every add.  All-gather: W-1 steps; in step s rank r copies chunk
 *       (r-s) mod W from out[r-1].  2(W-1) launches, stream-ordered; W = 1 is
 *       one copy.  out[r] is the rank's working buffer throughout.
 *   CP_ALLREDUCE_TWO_SHOT  not named by [LL]: the direct two-step algorithm
 *       between the two (on an all-to-all fabric every byte crosses a link
 *       twice, in two dependent steps).  Same chunks as the ring; one launch in
 *       which rank r sums chunk r of all W inputs in rank order (fp32, one
 *       rounding) into out[r], then one launch in which every rank copies each
 *       other rank's reduced chunk.  Same bits as the one-shot.
 *   algo         a CP_ALLREDUCE_* value (else CP_ERR_ARG)
 *   cp_size      W in [1, 64]
 *   in, out      host tables [W] of device buffers of n_elems `dtype` each;
 *                outputs must not overlap any input or each other
 *                (CP_ERR_ALIAS); inputs may share memory and are not written
 *   dtype        CP_F32 or CP_BF16 (CP_F16 and FP8: CP_ERR_UNSUPPORTED)
 * n_elems == 0 is a no-op (pointers may then be NULL).
 */
int cp_allreduce(int32_t algo, int32_t cp_size, const void* const* in, void* const* out,
                 int64_t n_elems, int32_t dtype, cp_stream_t stream);

/*
 * The ring of cp_allreduce in ONE launch: the persistent, in-kernel-signalling
 * form that [LL] sets against one launch per communication step (launch
 * overhead removed; the steps of a collective run inside one kernel).  Rank r
 * of tile t waits, before each of its 2(W-1) steps but the first, until rank
 * r-1 of the same tile has published the previous step through a device flag.
 * Same chunks, same order, same rounding as CP_ALLREDUCE_RING: the results are
 * the same bits.  Each rank gets about sqrt(q / 2048) workgroups (q = chunk
 * length in elements), at most 16, and all ranks together at most half of
 * what the device holds at once, so every workgroup a wait depends on is
 * running (an unmet wait ends in a reported timeout, never a hang).  On one
 * MI355X each hop costs about as much as a kernel boundary replayed from a
 * HIP graph (agent-scope release and acquire act on whole L2 caches): this
 * form pays off against eager per-step launches for small messages only.
 *
 * cp_allreduce_signal_bytes - bytes of the signal buffer for W ranks (0 for W
 * outside [1, 64]).  Layout (uint64 words): [0] the largest epoch in which a
 * wait timed out, [1] the largest epoch found stale, then the flags
 * [W][256] = (epoch << 8) + steps finished.
 *
 * cp_allreduce_signal
 *   cp_size, in, out, n_elems, dtype   as cp_allreduce
 *   signals        device buffer of at least cp_allreduce_signal_bytes(W)
 *                  bytes (signals_bytes), caller-owned, zero-filled once before
 *                  its first use; it must not overlap any input or output
 *   epoch          in [1, 2^55), larger than the epoch of every earlier call on
 *                  this buffer (so no clearing is needed between calls); a call
 *                  whose epoch is not larger finds flags at or above its own
 *                  base, records its epoch in word [1] and stops, leaving
 *                  `out` undefined (later calls need a still larger epoch)
 *   wait_timeout_us  limit of each wait (<= 0: 2 s); a wait that runs out
 *                  records the epoch in word [0] and every workgroup stops,
 *                  leaving `out` undefined - the kernel never hangs
 * Returns CP_ERR_UNSUPPORTED when W workgroups exceed half the resident capacity.
 * W = 1 is one copy (no signalling).  Calls that share a signal buffer must
 * not overlap in time.
 *
 * cp_allreduce_signal_status - synchronize `stream`, then report the call of
 * `epoch` (or a later call on the same buffer): CP_ERR_ARG if an epoch was
 * stale, CP_ERR_TIMEOUT if a wait ran out, else CP_OK.  Not for HIP graphs:
 * a replayed call would reuse its recorded epoch, which is then stale.
 */
size_t cp_allreduce_signal_bytes(int32_t cp_size);
int cp_allreduce_signal(int32_t cp_size, const void* const* in, void* const* out, int64_t n_elems,
                        int32_t dtype, void* signals, size_t signals_bytes, uint64_t epoch,
                        int64_t wait_timeout_us, cp_stream_t stream);
int cp_allreduce_signal_status(const void* signals, int32_t cp_size, uint64_t epoch, cp_stream_t stream);

/* ------------------------------------------------------------ utilities */
/* Static text for a status code (never NULL). */
const char* cp_status_string(int status);

/* Library version, as 10000*major + 100*minor + patch. */
int cp_version(void);

/*
 * Per-kernel timing with HIP events on the launch stream, for benchmarks.
 * cp_profile_enable(1) starts recording an event pair around every kernel the
 * library launches (capacity 65536 launches; later ones are not recorded);
 * cp_profile_enable(0) stops.  cp_profile_read synchronizes the recorded
 * events, and for up to `capacity` distinct kernels writes its name (NUL-
 * terminated, at most 127 chars) into names[k*128], its launch count into
 * counts[k] and the summed milliseconds into total_ms[k]; it returns the
 * number of distinct kernels (or a negative cp_status) and clears the record.
 * Meant for one calling thread: launches issued from several threads at once
 * while recording is on may be attributed to the wrong kernel name.
 * cp_profile_select(name) limits the recording to the kernels reported under
 * exactly that name (NULL or "": every kernel again); each recorded launch
 * adds two event records to its stream, a few microseconds of GPU time, so a
 * benchmark that times whole passes records only the kernel it reports.
 * Returns CP_OK, or CP_ERR_ARG for a name longer than 127 characters.
 */
int cp_profile_enable(int enable);
int cp_profile_select(const char* name);
int cp_profile_read(char* names, int64_t* counts, double* total_ms, int capacity);

#ifdef __cplusplus
}
#endif

#endif /* CPTHD_H */
