/*
 * ra.h -- C ABI of the ring-attention library for MI355X (gfx950).
 *
 * One context-parallel (CP) rank's share of Ring-Attention-style exact
 * attention, computed on one GPU: the rank's local Q chunk is attended against
 * the CP key/value chunks in ring order, each step as a FlashAttention-style
 * block (Q K^T, causal/document mask from global positions, online softmax,
 * P V), and the steps' partial results are combined through their log-sum-exp.
 * Beside it sit two local permutation kernels: the Ulysses sequence<->head
 * transpose and the zigzag/striped/contiguous CP reorder.
 *
 * Sources, cited by page title and section:
 *   [SP-concept] "序列並行（Sequence Parallelism）" concept page: "Ring Attention
 *                的不同思路" (ring procedure), "二、Ring Attention 的塊級線上
 *                Softmax" (online softmax, S = Q K^T / sqrt(d_k)), "三、Ulysses
 *                的 AllToAll 轉置" (N=4 worked layout).
 *   [CP-TE]      "Context Parallelism" page (Transformer Engine / Megatron):
 *                2.2 ring step order, 2.3 Ulysses, 3.1 qkv_format thd and
 *                cp_group, 3.3 / 5.2 mask offsets follow the CP split.
 *   [How-to]     DeepSpeed-Ulysses vs Ring-Attention how-to page: 3 (the
 *                ring_flash_attn_func(q, k, v, group, dropout_p=0, causal,
 *                window_size=(-1,-1)) interface, q/k/v [batch, seq_len_local,
 *                heads, head_dim], sp_group / sp_size / sp_rank), 5 (the
 *                head-divisibility assertion; GQA limit).
 *   [XTuner-09]  XTuner chapter 09, 9.5: cu_seqlens keeps packed documents
 *                from attending to each other.
 *   [LongCtx]    long-context sequence-parallel deep-dive page: timeline
 *                (Striped Attention; zigzag/stripe reorders), "线索三"
 *                (online softmax aggregates exactly across blocks).
 *
 * Conventions
 *   - The CP group (sp_group, sp_size, sp_rank) of [How-to] 3 becomes
 *     (cp_size, rank): the ring is simulated on one GPU, so every rank's K/V
 *     chunk is passed in and visited in ring order: at step t the rank holds
 *     the chunk of rank (rank - t) mod cp_size ([CP-TE] 2.2: send to the
 *     next rank, receive from the previous one).
 *   - Layout is thd with batch 1 ([CP-TE] 3.1): a tensor of T tokens, H heads
 *     and head_dim d is [T][H][d], row-major, d contiguous.
 *   - "Partition-local order" is the order in which a rank holds its global
 *     positions under the partition (RA_PART_* below). Masks use global
 *     positions ([CP-TE] 3.3).
 *   - Visibility of key position pk from query position pq:
 *       (causal == 0 || pk <= pq) && doc(pq) == doc(pk)
 *     where doc() comes from cu_seqlens ([XTuner-09] 9.5).
 *   - Scores s = softmax_scale * q.k, softmax_scale defaults to 1/sqrt(d)
 *     ([SP-concept] 二). LSE is the natural log of sum(exp(s)) over visible
 *     keys; a row with no visible key has O = 0, LSE = -inf.
 *   - GQA: query head h reads KV head h / (hq / hkv).
 *   - All device pointers are caller-owned (e.g. PyTorch tensors). The library
 *     never allocates or frees device memory; the caller supplies scratch space
 *     as `workspace` (size from ra_workspace_size). The one exception is
 *     ra_forward_noalloc, whose plan lives in a fixed array of device memory
 *     that the library holds on each GPU (its only global state). All calls are asynchronous on `stream` (a
 *     hipStream_t; NULL = the default stream). Host arrays (cu_seqlens) are
 *     read before the call returns and may be freed right after.
 *   - Errors are return codes. Arguments are validated on the host before
 *     anything is launched; a call that fails validation leaves every output
 *     untouched. RA_ERR_HIP reports a launch failure (outputs undefined).
 */
#ifndef RA_H
#define RA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RA_OK = 0,
  RA_ERR_NULL = 1,          /* a required pointer is NULL                                  */
  RA_ERR_SHAPE = 2,         /* a size is zero/negative or out of range                     */
  RA_ERR_DIVISIBILITY = 3,  /* S % cp (contiguous, striped) or S % (2 cp) (zigzag) != 0    */
  RA_ERR_HEADS = 4,         /* head count not divisible (Ulysses n, or hq % hkv)           */
  RA_ERR_CU_SEQLENS = 5,    /* cu_seqlens not 0 = c0 < c1 < ... < c_n = S                  */
  RA_ERR_RANK = 6,          /* rank outside [0, cp_size)                                   */
  RA_ERR_UNSUPPORTED = 7,   /* head_dim / dtype / element size combination not provided    */
  RA_ERR_WORKSPACE = 8,     /* workspace NULL or smaller than ra_workspace_size()          */
  RA_ERR_HIP = 9,           /* a HIP launch or copy failed                                 */
  RA_ERR_SCRATCH = 10       /* ra_forward_noalloc: the plan exceeds RA_NOALLOC_SCRATCH_BYTES */
} ra_status;

/* How the global sequence is split over CP ranks (rank r, S_l = S / cp):
 *   RA_PART_CONTIGUOUS  rank r holds positions [r S_l, (r+1) S_l)   ([How-to] 3)
 *   RA_PART_ZIGZAG      S is cut into 2 cp equal chunks; rank r holds chunk r
 *                       then chunk 2 cp - 1 - r  ([LongCtx] timeline, zigzag)
 *   RA_PART_STRIPED     rank r holds positions r, r + cp, r + 2 cp, ...
 *                       ([LongCtx] timeline, Striped Attention)
 *   RA_PART_DOC_ZIGZAG  per-document zigzag for packed documents ([How-to] 2:
 *                       variable lengths magnify Ring's imbalance; [LongCtx]
 *                       timeline, dynamic CP): every document j (cu_seqlens;
 *                       NULL = one document, length L) is cut into 2 cp pieces
 *                       at the bounds k L / 2cp rounded to the nearest multiple
 *                       of 256 tokens (halves up, capped at L; the last bound
 *                       is L). Rank r holds, document after document, piece
 *                       p = (r + j) mod cp then piece 2 cp - 1 - p, each
 *                       non-empty piece padded at its end to whole multiples
 *                       of 256 slots, then padding up to S_l, the largest
 *                       rank's slot count. Padding slots see nothing and are
 *                       seen by nothing (their O = 0, LSE = -inf, gradients
 *                       0). S_l = ra_local_length() (a multiple of 256); S need
 *                       not divide by cp. Accepted by ra_forward,
 *                       ra_forward_steps, ra_backward and ra_classify (tiles
 *                       16, 32, 64 or 128); cp_reorder_docs moves data in and
 *                       out of this layout.                                   */
typedef enum {
  RA_PART_CONTIGUOUS = 0,
  RA_PART_ZIGZAG = 1,
  RA_PART_STRIPED = 2,
  RA_PART_DOC_ZIGZAG = 3
} ra_partition;

typedef enum { RA_BF16 = 0, RA_F32 = 1 } ra_dtype;

/* Shape and numerics of one attention call. */
typedef struct {
  int64_t s_total;      /* S: global sequence length (all ranks)                        */
  int32_t hq;           /* query heads                                                  */
  int32_t hkv;          /* key/value heads; hq % hkv == 0                               */
  int32_t d;            /* head_dim: 64 or 128                                          */
  int32_t causal;       /* 1: causal mask on global positions; 0: document mask only    */
  float softmax_scale;  /* 0 selects 1/sqrt(d)                                          */
  int32_t in_dtype;     /* ra_dtype of q, k, v (RA_BF16 or RA_F32)                      */
  int32_t out_dtype;    /* ra_dtype of out: RA_BF16 or RA_F32 (RA_F32 inputs: RA_F32)  */
} ra_shape;

/* Bytes of device workspace that ra_forward / ra_forward_steps / ra_plan need for
 * this shape, CP size and document count (n_docs = 0 or 1: a single document),
 * for every partition. Returns 0 for an invalid shape. */
size_t ra_workspace_size(const ra_shape* shape, int32_t cp_size, int32_t n_docs);

/* Tokens (slots) one rank holds: S / cp, or for RA_PART_DOC_ZIGZAG the largest
 * rank's padded pieces. cu_seqlens is a HOST array (NULL: one document). Returns
 * -1 for invalid arguments (including S not divisible as the partition needs). */
int64_t ra_local_length(int64_t s_total, int32_t cp_size, int32_t partition, const int32_t* cu_seqlens,
                        int32_t n_docs);

/* Bytes of device workspace that cp_reorder_docs, and ra_classify with
 * RA_PART_DOC_ZIGZAG, need (the document tables). 0 for invalid arguments. */
size_t ra_doc_workspace_size(int64_t s_total, int32_t cp_size, const int32_t* cu_seqlens, int32_t n_docs);

/* One rank's ring attention, steps merged ([SP-concept] "Ring Attention 的不同
 * 思路" and 二; [CP-TE] 2.2 and 3.3).
 *   q          device, [S_l][hq][d] in_dtype: this rank's queries, partition-local order
 *   k, v       device, [cp][S_l][hkv][d] in_dtype: every rank's chunk, rank-major,
 *              each chunk in its owner's partition-local order
 *   cu_seqlens HOST int32 [n_docs + 1] global document offsets, or NULL (one document)
 *   out        device, [S_l][hq][d] out_dtype: normalised attention output
 *   lse        device, fp32 [hq][S_l]: natural-log LSE of each row
 *   workspace  device scratch of at least ra_workspace_size() bytes
 * Steps are combined in fp32: the accumulator and row statistics carry across
 * ring steps, which is the LSE merge done in unnormalised form. */
ra_status ra_forward(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                     int32_t n_docs, int32_t cp_size, int32_t rank, int32_t partition,
                     const ra_shape* shape, void* out, float* lse, void* workspace, size_t ws_bytes,
                     void* stream);

/* Bytes of fixed device scratch that ra_forward_noalloc can use (16 MiB). The plan
 * of a share takes about cp * S_l^2 / 4096 bytes (S_l = tokens per rank), e.g.
 * 4 MiB for 131072 tokens on one rank, 0.5 MiB for 8 ranks of 16384. */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* ra_forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same arguments,
 * results and errors as ra_forward, without the workspace: the plan lives in a
 * fixed array of RA_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * has run this call on, until the process ends. The call allocates and frees
 * nothing. Arguments whose plan needs more than RA_NOALLOC_SCRATCH_BYTES (at most
 * ra_workspace_size() bytes) give RA_ERR_SCRATCH before anything is launched.
 * `stream` must belong to the current device. Every call on one GPU uses that
 * GPU's array and leaves its plan there: calls that overlap in time on one GPU
 * (other streams, other host threads) race, so the caller orders them. */
ra_status ra_forward_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t n_docs, int32_t cp_size, int32_t rank, int32_t partition,
                             const ra_shape* shape, void* out, float* lse, void* stream);

/* Planning half of ra_forward: uploads cu_seqlens (for RA_PART_DOC_ZIGZAG, also
 * builds the block descriptors of the layout) and builds, in `workspace`, the
 * per-query-tile work list of non-SKIP (ring step, key tile) pairs with their
 * FULL / PARTIAL class ([CP-TE] 3.3) and the heaviest-first tile order.
 * A plan depends only on (shape, cu_seqlens, cp_size, rank, partition), so
 * one plan serves every layer that shares them. A RA_PART_DOC_ZIGZAG plan is
 * executed by ra_forward_planned_docs, the others by ra_forward_planned. */
ra_status ra_plan(const ra_shape* shape, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size,
                  int32_t rank, int32_t partition, void* workspace, size_t ws_bytes, void* stream);

/* Execution half of ra_forward: the attention kernel alone, reading the plan
 * that ra_plan left in `workspace` (same shape, n_docs, cp_size, rank and
 * partition; a plan made for other arguments gives undefined values but no
 * out-of-bounds access: the kernel bounds-checks every work-list entry).
 * Arguments as in ra_forward; cu_seqlens is not passed again. */
ra_status ra_forward_planned(const void* q, const void* k, const void* v, int32_t n_docs, int32_t cp_size,
                             int32_t rank, int32_t partition, const ra_shape* shape, void* out, float* lse,
                             void* workspace, size_t ws_bytes, void* stream);

/* Execution half of ra_forward for RA_PART_DOC_ZIGZAG ([How-to] 2: packed
 * documents of variable length): the attention kernel alone on the plan that
 * ra_plan left in `workspace` for the same arguments. cu_seqlens is the HOST
 * array the plan was made from; it sizes the local length S_l on the host and
 * is not uploaded again. Arguments, layouts and errors as in ra_forward with
 * partition RA_PART_DOC_ZIGZAG; a plan made for other arguments gives
 * undefined values but no out-of-bounds access. */
ra_status ra_forward_planned_docs(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                  int32_t n_docs, int32_t cp_size, int32_t rank, const ra_shape* shape, void* out,
                                  float* lse, void* workspace, size_t ws_bytes, void* stream);

/* Same inputs as ra_forward; writes each ring step's normalised partial instead
 * of the merged result:
 *   o_steps    device fp32 [cp][S_l][hq][d]: step t = attention against chunk (rank - t) mod cp
 *   lse_steps  device fp32 [cp][hq][S_l]; rows with no visible key in a step: O = 0, LSE = -inf
 * Merging the steps with ra_lse_merge gives ra_forward's result. */
ra_status ra_forward_steps(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                           int32_t n_docs, int32_t cp_size, int32_t rank, int32_t partition,
                           const ra_shape* shape, float* o_steps, float* lse_steps, void* workspace,
                           size_t ws_bytes, void* stream);

/* Bytes of device workspace that ra_backward needs for this shape, CP size and
 * document count (both kernels' work lists and the per-row sums dO . O).
 * Returns 0 for an invalid shape. */
size_t ra_backward_workspace_size(const ra_shape* shape, int32_t cp_size, int32_t n_docs);

/* Gradients of one rank's ring attention. The pages train with these layers
 * ([How-to] 4: a forward and a backward per step; [CP-TE] 4: training
 * throughput) but give no backward equations; this is the chain rule of the
 * forward's definition, with P = exp(s - LSE) the probabilities over all ring
 * steps and dO the gradient of the loss with respect to out:
 *   dV_k = sum_i P_ik dO_i;  dP_ik = dO_i . v_k;  dS_ik = P_ik (dP_ik - dO_i . O_i)
 *   dQ_i = scale sum_k dS_ik k_k;  dK_k = scale sum_i dS_ik q_i
 * (GQA: dK / dV of a KV head sum over the query heads that read it.)
 *   q, k, v, cu_seqlens, n_docs, cp_size, rank, partition, shape: as in ra_forward
 *   out        device [S_l][hq][d] out_dtype: the forward output
 *   lse        device fp32 [hq][S_l]: the forward LSE (natural log, all steps merged)
 *   dout       device [S_l][hq][d] in_dtype: gradient with respect to out
 *   dq         device fp32 [S_l][hq][d]: gradient with respect to this rank's q
 *   dk, dv     device fp32 [cp][S_l][hkv][d]: this rank's contribution to the
 *              gradient of every chunk's k and v, chunk s at index s in its owner's
 *              partition-local order (the partial of ring step (rank - s) mod cp;
 *              a real ring adds the ranks' partials as the chunk travels, so the
 *              sum over ranks is the gradient of the whole sequence). Chunks and
 *              keys that no row of the rank sees are written as 0.
 *   workspace  device scratch of at least ra_backward_workspace_size() bytes
 * Rows whose LSE is -inf contribute nothing. Deterministic: no atomics. */
ra_status ra_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size,
                      int32_t rank, int32_t partition, const ra_shape* shape, float* dq, float* dk, float* dv,
                      void* workspace, size_t ws_bytes, void* stream);

/* fp32 LSE merge of two normalised partials (derived from the online-softmax
 * update of [SP-concept] 二 at chunk granularity):
 *   LSE = ln(e^lse_a + e^lse_b);  O = e^(lse_a - LSE) o_a + e^(lse_b - LSE) o_b
 * -inf marks an empty partial (weight 0); two empty partials give (0, -inf).
 *   o_a, o_b, o_out      device fp32 [rows][h][d]
 *   lse_a, lse_b, lse_out device fp32 [h][rows]
 * o_out may alias o_a or o_b and lse_out may alias lse_a or lse_b (in place).
 * rows * h * d above 2^37 gives RA_ERR_SHAPE. */
ra_status ra_lse_merge(int64_t rows, int32_t h, int32_t d, const float* o_a, const float* lse_a,
                       const float* o_b, const float* lse_b, float* o_out, float* lse_out, void* stream);

/* Tile classification from global offsets ([CP-TE] 3.3 / 5.2; [XTuner-09] 9.5):
 * for each ring step t, query tile I (local rows [I bm, (I+1) bm)) and key tile J
 * (local keys [J bn, (J+1) bn) of chunk (rank - t) mod cp), over in-range pairs:
 *   0 SKIP (no visible pair), 1 PARTIAL, 2 FULL (every pair visible).
 *   cls        device int8 [cp][ceil(S_l / bm)][ceil(S_l / bn)]
 * shape supplies s_total and causal (heads and dtypes are not used).
 * bm, bn in [1, 65536]; RA_PART_DOC_ZIGZAG: bm, bn in {16, 32, 64, 128}, the
 * grid is over S_l = ra_local_length(), a tile holding padding is never FULL,
 * and the workspace must hold ra_doc_workspace_size() bytes. More than 2^36
 * classes (cp x tiles) gives RA_ERR_SHAPE. */
ra_status ra_classify(const ra_shape* shape, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size,
                      int32_t rank, int32_t partition, int32_t bm, int32_t bn, int8_t* cls, void* workspace,
                      size_t ws_bytes, void* stream);

/* Ulysses sequence<->head layout change for n simulated ranks ([SP-concept] 三,
 * worked N=4 example; [CP-TE] 2.3):
 *   forward  in  [n][s_local][h][d]  ->  out [n][n s_local][h/n][d]
 *            out[p][j s_local + i][h'] = in[j][i][p h/n + h']
 *   inverse  in  [n][n s_local][h/n][d]  ->  out [n][s_local][h][d]
 * h is the full head count; h % n != 0 gives RA_ERR_HEADS ([How-to] 5:
 * sequence_parallel_size must divide the head count). elem_bytes in {1,2,4,8}.
 * Bit-exact copy; in and out must not overlap. */
ra_status ulysses_permute(const void* in, void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                          int32_t elem_bytes, int32_t inverse, void* stream);

/* ulysses_permute with the n blocks of the head-split side ([n s_local][h/n][d]
 * each) placed block_stride bytes apart instead of back to back: the output of a
 * forward permute, the input of an inverse one. This lets a Ulysses x Ring grid
 * place device (u, r)'s head slice at [u][r], so that the ring chunks of one head
 * slice are contiguous (see usp_forward). block_stride is a multiple of
 * (h/n) d elem_bytes and at least n s_local (h/n) d elem_bytes; the packed side and
 * the span of the strided side must not overlap. */
ra_status ulysses_permute_strided(const void* in, void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                                  int32_t elem_bytes, int32_t inverse, int64_t block_stride, void* stream);

/* Bytes of device workspace for usp_forward (head-split Q, K, V, O of the grid and
 * one ring rank's plan). Returns 0 for an invalid shape. */
size_t usp_workspace_size(const ra_shape* shape, int32_t ulysses, int32_t ring, int32_t n_docs);

/* Hybrid Ulysses x Ring ("USP") for a grid of ulysses x ring simulated devices
 * ([CP-TE] 2.4 and 6: Ulysses head rearrangement inside a group, Ring passing the
 * sequence across groups; [How-to] 6; [LongCtx] timeline, USP):
 *   the ring partition (RA_PART_*, cp = ring) splits the sequence over `ring`
 *   groups; group r's tokens, in partition-local order, are cut into `ulysses`
 *   equal pieces, one per device (u, r). Inside each group the Ulysses permute
 *   gives device (u, r) the group's tokens for heads [u hq/U, (u+1) hq/U) (K, V:
 *   [u hkv/U, (u+1) hkv/U)); device (u, r) runs ring attention (rank r of `ring`)
 *   over the chunks of its head slice; the inverse permute returns every device
 *   its own tokens for all heads.
 *   q          device [ring][ulysses][S/(ring ulysses)][hq][d] in_dtype: every device's input
 *   k, v       device [ring][ulysses][S/(ring ulysses)][hkv][d] in_dtype
 *   out        device [ring][ulysses][S/(ring ulysses)][hq][d] out_dtype
 *   lse        device fp32 [ulysses][ring][hq/ulysses][S/ring]: device (u, r)'s ring LSE,
 *              in group r's partition-local token order
 * hq % ulysses or hkv % ulysses != 0 gives RA_ERR_HEADS (the Ulysses degree is
 * bounded by the head count, [How-to] 5); (S / ring) % ulysses != 0 gives
 * RA_ERR_DIVISIBILITY. The whole grid runs on the caller's stream. */
ra_status usp_forward(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_docs,
                      int32_t ulysses, int32_t ring, int32_t partition, const ra_shape* shape, void* out,
                      float* lse, void* workspace, size_t ws_bytes, void* stream);

/* CP reorder for RA_PART_DOC_ZIGZAG:
 *   forward  in [s][h][d] (global order) -> out [cp][S_l][h][d], padding slots zero
 *   inverse  in [cp][S_l][h][d] -> out [s][h][d] (padding slots dropped)
 * S_l = ra_local_length(s, cp, RA_PART_DOC_ZIGZAG, cu_seqlens, n_docs); cu_seqlens
 * is a HOST array (NULL: one document); workspace of ra_doc_workspace_size()
 * bytes. Bit-exact copy; in and out must not overlap. */
ra_status cp_reorder_docs(const void* in, void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                          int32_t cp_size, const int32_t* cu_seqlens, int32_t n_docs, int32_t inverse,
                          void* workspace, size_t ws_bytes, void* stream);

/* CP reorder between the global sequence and the rank-major partitioned layout
 * (contiguous, zigzag, striped; RA_PART_DOC_ZIGZAG uses cp_reorder_docs):
 *   forward  in [s][h][d] (global order) -> out [cp][s/cp][h][d], out[r][i] = in[pos_r(i)]
 *   inverse  in [cp][s/cp][h][d] -> out [s][h][d]
 * pos_r from `partition` (RA_PART_*). Bit-exact copy; in and out must not overlap. */
ra_status cp_reorder(const void* in, void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                     int32_t cp_size, int32_t partition, int32_t inverse, void* stream);

/* Static description of a status code. */
const char* ra_status_string(ra_status status);

/* ABI version of this header (incremented on any signature change). */
int32_t ra_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RA_H */
