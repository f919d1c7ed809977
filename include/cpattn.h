/*
 * cpattn.h -- C ABI of libcpattn.so: the per-rank hot path of causal
 * context-parallel ("zigzag ring") attention on AMD Instinct MI355X (gfx950).
 *
 * What the calls compute
 *   Context parallelism shards Q, K and V along the sequence dimension; a rank
 *   keeps its Q shard, attends it to every K/V shard in turn and combines the
 *   partial results (Accelerate concept guide "Context Parallel in accelerate",
 *   sections "Technical details" and "So how does it work?").  The sequence is
 *   cut into 2*cp chunks, so its length must be a multiple of 2*cp (NeMo
 *   Megatron-Bridge "Hierarchical Context Parallel Skill", "Required
 *   constraints"); rank r holds chunk r followed by chunk 2*cp-1-r, which gives
 *   every rank the same number of causal (query, key) pairs.  Each step yields a
 *   partial output O and its log-sum-exp (LSE, natural log); partials over
 *   disjoint key sets are combined by LSE weighting.
 *
 * Conventions shared by every call
 *   - Return value: CP_OK (0) or a CP_E* code; cp_last_error() then holds a
 *     message (thread-local, valid until the next call on that thread).
 *   - All argument checks run before any launch: a failed call has no side
 *     effects and launches nothing.
 *   - Ownership: the caller owns every buffer.  The library never allocates
 *     device memory; scratch space is a caller-provided workspace whose size a
 *     *_workspace query returns (cp_attn_ring_fwd_noalloc alone uses a static
 *     device array of its own instead).  Pointers marked (device) must be
 *     device memory on the current HIP device; (host) ones are ordinary host
 *     memory.
 *   - Streams: device work is enqueued asynchronously on the caller's stream,
 *     with no implicit synchronisation; a device fault surfaces at the caller's
 *     next synchronisation.  Calls are re-entrant and keep no state (apart
 *     from that array's per-device address).
 *   - Layout: tensors are [B, H, rows, D] with the D dimension contiguous
 *     ("[batch, num_heads, seq_len // context_parallel_size, head_dim]" in the
 *     guide's pseudocode); element strides for B, H and rows are passed, so row
 *     range views are legal.  Base pointers and every stride in bytes must be
 *     multiples of 16.
 *   - Positions: q_pos / k_pos give the global sequence position of every query
 *     / key row and q_lo the first position of the query row's document (NULL
 *     means 0 for every row: plain causal attention).  Key j is allowed for
 *     query i iff q_lo[i] <= k_pos[j] <= q_pos[i].  Position values are only
 *     compared, never used as addresses, so any int32 values are memory-safe.
 *   - Query head h reads key/value head h / (hq / hkv) (grouped-query heads).
 *   - cp == 1 is valid and means one rank holding the whole sequence: plain
 *     causal attention (the Accelerate plugin treats a CP size of 1 as off).
 *   - Size limits (CP_EINVAL beyond them): sq, sk < 2^30; cp <= 255; a rank's
 *     shard of at most 65535 key tiles (64 keys for bf16, 32 for fp32);
 *     b x heads x rows x d below 2^62 for q and for k/v, and every tensor's
 *     largest element offset under its strides below 2^62.  The
 *     kernels address device memory through 32-bit buffer offsets, so for bf16
 *     inputs the forward needs one (batch, kv head) of K (rows x row stride x
 *     2 bytes) and its transposed V copy (d x padded keys x 2 bytes) under
 *     4 GiB.  The backward needs 64 rows of q, dO and k, and 256 rows of v,
 *     each under 2 GiB.  Its per-row and per-key tables must also stay under
 *     2 GiB, with at most 65535 query tiles of 64 rows and 32767 query heads per
 *     kv head.
 */
#ifndef CPATTN_H
#define CPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

enum cp_status {
  CP_OK = 0,
  CP_EINVAL = 1,     /* null pointer, cp < 1, rank out of range, hq % hkv != 0, d not 64/128, bad stride, bad enum */
  CP_ESHAPE = 2,     /* sequence length not a multiple of 2*cp; cu_seqlens not monotone or not ending at S */
  CP_EDTYPE = 3,     /* unsupported dtype code */
  CP_EWORKSPACE = 4, /* workspace missing, too small or misaligned */
  CP_EHIP = 5        /* HIP launch / runtime error */
};

enum cp_dtype { CP_F32 = 0, CP_BF16 = 1 };

enum cp_shard_mode {
  CP_STREAM = 0,  /* zigzag of the packed stream: rank r holds stream chunks r and 2cp-1-r */
  CP_PER_DOC = 1, /* every document cut into 2cp chunks; rank r holds chunks r and 2cp-1-r of each */
  CP_WHOLE_DOC = 2 /* whole documents placed greedily (own design, see cp_varlen_index) */
};

/* Shape and layout descriptor of an attention call. */
typedef struct cp_shape {
  int32_t b;          /* batch */
  int32_t hq;         /* query heads */
  int32_t hkv;        /* key/value heads; hq % hkv == 0 */
  int32_t d;          /* head dimension: 64 or 128 */
  int64_t sq;         /* query rows per (batch, head) */
  int64_t sk;         /* key/value rows per (batch, kv head) */
  float scale;        /* softmax scale, finite and > 0 (usually 1/sqrt(d)) */
  int32_t in_dtype;   /* dtype of q, k, v (and dO): CP_BF16 or CP_F32 */
  int32_t out_dtype;  /* dtype of the final O of ring calls; partial outputs are always fp32 */
  int64_t q_str[3];   /* element strides of q for batch, head, row */
  int64_t k_str[3];   /* same for k */
  int64_t v_str[3];   /* same for v */
  int64_t o_str[3];   /* same for o (in elements of o's dtype) */
} cp_shape;

/* ---------------------------------------------------------------- host index builder */

/* Global positions of rank `rank`'s rows: chunk rank, then chunk 2cp-1-rank,
 * of a sequence of S tokens cut into 2cp chunks.  pos_out (host) receives S/cp
 * int32 values.  CP_ESHAPE if S % (2cp) != 0 ("Required constraints" of the
 * hierarchical-CP skill page); CP_EINVAL for cp < 1, rank outside [0, cp),
 * S < 0 or S > INT32_MAX. */
int cp_shard_zigzag(int64_t S, int32_t cp, int32_t rank, int32_t* pos_out);

/* The rank-major concatenation of every rank's positions (what gathering all
 * shards yields; the guide's "all-gather" section).  perm_out (host) receives S
 * int32 values forming a permutation of [0, S); its inverse un-shards. */
int cp_unshard_zigzag(int64_t S, int32_t cp, int32_t* perm_out);

/* Index map of packed documents.  cu_seqlens (host) holds n_docs+1 document
 * boundaries, starting at 0, non-decreasing, ending at S.  Writes S/cp
 * positions to pos_out and the start of each row's document to lo_out (host).
 * mode CP_STREAM deals the whole packed stream zigzag (needs S % 2cp == 0);
 * CP_PER_DOC deals every document zigzag on its own (needs every document
 * length % 2cp == 0), keeping documents in order, so a rank's local document
 * boundaries are cu_seqlens / cp.  CP_WHOLE_DOC keeps documents whole where it
 * can (needs S % 2cp == 0).  The whole-document and per-document sharding of
 * packed sequences is named in the FlashCP abstract, without an algorithm for
 * the former; this one is an own greedy design under the ring's constraint of
 * S/cp positions per rank: documents longest first (ties: lower index); one
 * that fits whole in some rank's remaining room goes whole to the fitting rank
 * with the least causal work so far (ties: lower rank); one that fits nowhere
 * is cut into consecutive pieces from its start, each filling the rank with the
 * most room left (ties: lower rank).  The rows [a, b) of a document that
 * starts at s count sum over p in [a, b) of (p - s + 1) causal pairs.  At most
 * cp - 1 documents are cut.  A rank's positions come out in ascending order. */
int cp_varlen_index(const int32_t* cu_seqlens, int32_t n_docs, int32_t cp, int32_t rank,
                    int32_t mode, int32_t* pos_out, int32_t* lo_out);

/* Rank whose K/V shard rank `rank` attends at ring step `step`: (rank - step)
 * mod cp; step 0 is the local shard (guide, "all-to-all vs all-gather": every
 * shard is visited once over cp steps).  Returns that rank, or -1 (with
 * cp_last_error set) for cp < 1 or rank/step outside [0, cp). */
int cp_ring_source(int32_t cp, int32_t rank, int32_t step);

/* Exact number of allowed (query, key) pairs, q_lo[i] <= k_pos[j] <= q_pos[i],
 * over host arrays (q_lo may be NULL).  It measures the work balance that the
 * 2*cp chunking exists for: the "Required constraints" of the NeMo
 * Megatron-Bridge "Hierarchical Context Parallel Skill" page ask for a sequence
 * length that is a multiple of 2*cp, and with the zigzag deal every rank of a
 * dense causal sequence then gets S(S+1)/(2cp) pairs; the FlashCP abstract
 * names the imbalance that uneven pair counts cause.  Used for FLOP accounting
 * and that balance check.  Returns the count, or -1 on a null array with n > 0
 * or a negative length. */
int64_t cp_pairs(const int32_t* q_pos, const int32_t* q_lo, int64_t nq,
                 const int32_t* k_pos, int64_t nk);

/* ---------------------------------------------------------------- device calls */

/* Workspace bytes needed by cp_attn_partial_fwd (cp = 1) and cp_attn_ring_fwd
 * (cp = ring size).  Returns 0 for an invalid descriptor.  It holds per key
 * tile its position bounds and padded key positions; for bf16 inputs, per
 * 128-row query tile its dispatch rank, and for rings of at most 1024 key
 * tiles (65536 keys) also the key tiles a document-masked query tile lists,
 * 4 bytes per query tile and key tile, computed once for every head; for dense
 * bf16 rings of 65536 keys or more, a transposed copy of V. */
size_t cp_attn_ring_fwd_workspace(const cp_shape* s, int32_t cp);

/* One ring step, the guide's attn(Q_i, K_j, V_j): every query row attends to
 * the allowed keys among the sk key rows.  q (device, in_dtype) [b,hq,sq,d];
 * k, v (device, in_dtype) [b,hkv,sk,d]; q_pos, q_lo (device int32 [sq], q_lo
 * may be NULL); k_pos (device int32 [sk]).  Writes the partial O (device fp32,
 * strides o_str) normalised over this step's allowed keys and LSE (device fp32,
 * contiguous [b,hq,sq]).  A row with no allowed key gets O = 0, LSE = -inf (the
 * identity of cp_attn_merge).  ws (device) of at least
 * cp_attn_ring_fwd_workspace(s, 1) bytes, 256-byte aligned. */
int cp_attn_partial_fwd(const cp_shape* s, const void* q, const void* k, const void* v,
                        const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos,
                        float* o, float* lse, void* ws, size_t ws_bytes, hipStream_t stream);

/* combine(): in place (o_acc, lse_acc) <- (o_acc, lse_acc) (+) (o_p, lse_p) with
 * L = max(l1,l2) + ln(e^(l1-max) + e^(l2-max)) and O = e^(l1-L) o1 + e^(l2-L) o2.
 * (0, -inf) is the identity; two empty rows stay (0, -inf).  The operation is
 * symmetric in its operands bit for bit.  Contiguous device fp32 arrays:
 * o_* [rows, d], lse_* [rows], 0 <= rows <= 2^31; d is 64 or 128.  The pages name combine() but
 * print no formula; this is the exact recombination of softmax over disjoint
 * key sets. */
int cp_attn_merge(int64_t rows, int32_t d, float* o_acc, float* lse_acc,
                  const float* o_p, const float* lse_p, hipStream_t stream);

/* A whole virtual rank's ring with every K/V shard resident: for step t =
 * 0..cp-1 the local queries attend the shard of rank (rank - t) mod cp, and the
 * partials are merged on the fly in registers.  q_loc (device, in_dtype)
 * [b,hq,sq,d]; k_all, v_all (device, in_dtype) [b,hkv,sk,d] hold every rank's
 * shard in rank-major order (rows [r*sk/cp, (r+1)*sk/cp) are rank r's), as an
 * all-gather of the shards lays them out; k_pos_all (device int32 [sk]) their
 * global positions.  Writes the final O (device, out_dtype, strides o_str) and
 * LSE (device fp32, contiguous [b,hq,sq]).  CP_ESHAPE unless sk % (2cp) == 0.
 * ws (device) of at least cp_attn_ring_fwd_workspace(s, cp) bytes, 256-byte
 * aligned. */
int cp_attn_ring_fwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                     const void* k_all, const void* v_all, const int32_t* q_pos,
                     const int32_t* q_lo, const int32_t* k_pos_all, void* o, float* lse,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* The whole ring of cp_attn_ring_fwd for callers that cannot allocate device
 * memory or hand a workspace in: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments as for cp_attn_ring_fwd,
 * without the workspace.  The tables the kernels need (key position bounds and
 * padded key positions, 272 bytes per 64-key tile for bf16, 16 per 32-key
 * tile for fp32; for bf16 also the dispatch order of the query tiles, 8 bytes
 * per 128 query rows) live in one static device array of 4 MiB per device,
 * held until the process ends; its address is resolved on the first call on
 * each device.  Rings whose tables exceed it (about 15000 bf16 key tiles,
 * 985 000 keys) are rejected with CP_EINVAL.  The per-query-tile key lists of
 * document-masked rings (see cp_attn_ring_fwd_workspace) are kept there too
 * when they fit beside the tables; otherwise each workgroup lists its key
 * tiles itself, with the same result bits.  V is always read in place (no
 * transposed copy), so a long dense ring runs somewhat slower than through
 * cp_attn_ring_fwd; the results are the same bits.  Nothing is allocated and
 * every table entry is rewritten by each call.  Calls on one device share the
 * array: calls that overlap on one device (different streams, or host threads
 * without ordering) race and give wrong results. */
int cp_attn_ring_fwd_noalloc(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                             const void* k_all, const void* v_all, const int32_t* q_pos,
                             const int32_t* q_lo, const int32_t* k_pos_all, void* o, float* lse,
                             hipStream_t stream);

/* ---------------------------------------------------------------- stepwise ring
 * The ring forward computed the way a ring of separate steps computes it
 * (Accelerate concept guide, "So how does it work?": attend the local queries
 * to one K/V shard, then combine, once per shard; the rotation of the shards
 * is the "all-to-all" method of "How to choose the right rotation method?").
 * Step t = 0..cp-1 attends q_loc to the shard of rank (rank - t) mod cp with
 * the kernel of cp_attn_partial_fwd.  Step 0 writes (o, lse); every later
 * step combines its partial with them by the rule of cp_attn_merge, in the
 * kernel's epilogue (each row is read, merged and written by the wave that
 * owns it), so no partial is stored.
 *
 * stage == NULL: every step reads its shard where it lies in k_all / v_all.
 * stage != NULL: the shards of steps 1..cp-1 are first copied into stage, two
 * slots used in turn, on copy_stream, the way a rotation ring receives them
 * from its neighbour.  The copy of a later step's shard overlaps the current
 * step's attention; a step waits only for its own shard, and a slot is
 * refilled only after the step that read it has finished.  copy_stream may be
 * stream itself (copies then run in line with the steps).  Everything the call
 * enqueues on copy_stream is joined back into stream before it returns, so
 * work queued later on stream sees o and lse complete.  k_all and v_all must
 * have contiguous rows (row stride d) when staging.
 *
 * Arguments as for cp_attn_ring_fwd, except: o (device fp32, contiguous
 * [b,hq,sq,d], o_str = {hq*sq*d, sq*d, d}) and s->out_dtype must be CP_F32
 * (the merge works on fp32; CP_EDTYPE otherwise).  ws (device) of at least
 * cp_attn_ring_fwd_stepwise_workspace(s, cp) bytes holds the step kernel's
 * tables; stage (device) of at least
 * cp_attn_ring_stage_bytes(s, cp) bytes.  Both 256-byte aligned.  Both are
 * owned by the caller and must stay untouched until stream has passed the call.
 * CP_ESHAPE unless sk % (2cp) == 0. */
size_t cp_attn_ring_fwd_stepwise_workspace(const cp_shape* s, int32_t cp);
size_t cp_attn_ring_stage_bytes(const cp_shape* s, int32_t cp);
int cp_attn_ring_fwd_stepwise(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                              const void* k_all, const void* v_all, const int32_t* q_pos,
                              const int32_t* q_lo, const int32_t* k_pos_all, float* o, float* lse,
                              void* ws, size_t ws_bytes, void* stage, size_t stage_bytes,
                              hipStream_t stream, hipStream_t copy_stream);

/* ---------------------------------------------------------------- head exchange
 * The all-to-all level of hierarchical context parallelism (NeMo
 * Megatron-Bridge "Hierarchical Context Parallel Skill": with cp_comm_type
 * "a2a+p2p" the first level is a group of g ranks that communicate
 * all-to-all; the page gives no data layout).  Reading: the exchange trades
 * heads for rows.  Before it a rank holds every head of its rows, after it
 * every row of the group for H/g of the heads.  These calls are the rank-local
 * halves of that exchange; the exchange itself (block j of rank i's send
 * buffer becomes block i of rank j's receive buffer) is the collective's.
 *
 * cp_a2a_pack: x (device) [rows, heads, d], row stride x_row_stride elements
 *   (>= heads*d, a multiple of 16 bytes), heads contiguous within a row ->
 *   send (device) [g][heads/g][rows][d] contiguous: block j holds heads
 *   j*heads/g .. of every row, head-major, the part rank j receives.
 *   inverse != 0 copies send back into x.
 * cp_a2a_unpack: recv (device) [g][heads/g][rows][d] contiguous, block i from
 *   rank i -> y (device) [heads/g][g*rows][d] contiguous: this rank's heads
 *   over the group's rows in source-rank order, the [heads, rows, d] layout
 *   (one batch) the attention calls read.  inverse != 0 copies y back into recv.
 * heads is the total head count H.  g >= 1 divides heads; heads <= 65535;
 * 0 <= rows <= 2^31, with rows x x_row_stride x element size below 2^62
 * bytes; d is 64 or 128; dtype CP_BF16 or CP_F32; pointers 16-byte aligned;
 * source and destination must not overlap.  Every value is copied exactly.
 * rows == 0 is a no-op. */
int cp_a2a_pack(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, void* x,
                int64_t x_row_stride, void* send, int32_t inverse, hipStream_t stream);
int cp_a2a_unpack(int32_t g, int32_t heads, int64_t rows, int32_t d, int32_t dtype, void* recv,
                  void* y, int32_t inverse, hipStream_t stream);

/* ---------------------------------------------------------------- backward
 * Gradients of the ring forward above with respect to q, k and v.  The pages
 * train through context-parallel attention (the Accelerate guide wraps the
 * training step, loss.backward() included, in the context-parallel context;
 * the Megatron-Bridge skill warns that ranks attending only their local chunk
 * give broken gradients) but print no backward formula; these calls compute
 * the exact gradient of softmax attention over the allowed keys, recomputing
 * the probabilities from the final LSE of the forward:
 *   P_ij = exp(scale q_i.k_j - LSE_i)     delta_i = dO_i . O_i
 *   dS_ij = P_ij (dO_i.v_j - delta_i)
 *   dq_i += scale sum_j dS_ij k_j   dk_j += scale sum_i dS_ij q_i   dv_j += sum_i P_ij dO_i
 * with key/value heads summing over the query heads that read them.  The
 * backward takes bf16 q, k, v and dO (in_dtype CP_BF16, else CP_EDTYPE);
 * gradients accumulate in fp32. */

/* Workspace bytes needed by cp_attn_partial_bwd (cp = 1) and cp_attn_ring_bwd
 * (cp = ring size).  Returns 0 for an invalid descriptor. */
size_t cp_attn_bwd_workspace(const cp_shape* s, int32_t cp);

/* delta_i = sum_d dO[i,d] O[i,d] for the sq rows of every (batch, query head).
 * dout (device bf16, strides q_str) [b,hq,sq,d]; o (device, out_dtype, strides
 * o_str) the final merged output of the forward; writes delta (device fp32,
 * contiguous [b,hq,sq]).  b x hq x sq must stay below 2^31 rows (CP_EINVAL). */
int cp_attn_bwd_delta(const cp_shape* s, const void* dout, const void* o, float* delta,
                      hipStream_t stream);

/* Backward of one ring step (the partial of cp_attn_partial_fwd): adds this
 * step's contributions to dq (device fp32, contiguous [b,hq,sq,d]) and to dk,
 * dv (device fp32, contiguous [b,hkv,sk,d]).  q, dout (device bf16, strides
 * q_str); k, v (device bf16) [b,hkv,sk,d]; lse, delta (device fp32, contiguous
 * [b,hq,sq]) are the final LSE of the whole ring and cp_attn_bwd_delta's
 * output, so that the step's probabilities are the final ones restricted to its
 * keys.  Positions as in the forward.  ws (device) of at least
 * cp_attn_bwd_workspace(s, 1) bytes, 256-byte aligned.  dq, dk, dv must not
 * overlap each other or the inputs. */
int cp_attn_partial_bwd(const cp_shape* s, const void* q, const void* k, const void* v,
                        const void* dout, const float* lse, const float* delta,
                        const int32_t* q_pos, const int32_t* q_lo, const int32_t* k_pos,
                        float* dq, float* dk, float* dv, void* ws, size_t ws_bytes,
                        hipStream_t stream);

/* A virtual rank's whole ring backward with every K/V shard resident: the
 * contributions of all cp steps (shards in the order of cp_attn_ring_fwd) are
 * added to dq (device fp32, contiguous [b,hq,sq,d]) and to dk_all, dv_all
 * (device fp32, contiguous [b,hkv,sk,d], rank-major like k_all).  On a cluster
 * the rows of shard r would travel back to rank r; summing every rank's call
 * gives the full key/value gradients.  Other arguments as in
 * cp_attn_partial_bwd and cp_attn_ring_fwd.  CP_ESHAPE unless sk % (2cp) == 0.
 * ws (device) of at least cp_attn_bwd_workspace(s, cp) bytes. */
int cp_attn_ring_bwd(const cp_shape* s, int32_t cp, int32_t rank, const void* q_loc,
                     const void* k_all, const void* v_all, const void* dout, const float* lse,
                     const float* delta, const int32_t* q_pos, const int32_t* q_lo,
                     const int32_t* k_pos_all, float* dq, float* dk_all, float* dv_all,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* Message of the last failed call on this thread ("" if none). */
const char* cp_last_error(void);

/* Library version: major*10000 + minor*100 + patch. */
int cp_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CPATTN_H */
