// Host-side argument validation and workspace layout (pure C++, no HIP calls),
// so that every error path can be exercised on a machine without a GPU.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/ra.h"

namespace ra {

struct Layout {
  int s_local;
  int bm, bn;      // attention kernel tile (query rows x keys)
  int nqt, nkt;    // tiles along the local query / key index
  int wl_stride;   // work-list entries reserved per query tile (cp * nkt)
  int n_docs_dev;  // documents the kernels see (1 = no document mask)
  int doczig;      // RA_PART_DOC_ZIGZAG: cu is always uploaded, plus the block prefix and descriptors
  int nblk;        // doc-zigzag: 64-slot blocks per rank (s_local / 64)
  size_t cu_off, prefix_off, blk_off, count_off, order_off, wl_off, total;
};

// Tokens (slots) each rank holds: s_total / cp, or for RA_PART_DOC_ZIGZAG the
// largest rank's padded pieces (cu NULL: one document). Returns -1 on overflow.
int64_t local_len(const ra_shape* shape, int32_t cp_size, int32_t partition, const int32_t* cu, int32_t n_docs);

// Upper bound of local_len over every cu_seqlens with n_docs documents.
int64_t local_len_bound(const ra_shape* shape, int32_t cp_size, int32_t n_docs);

// Workspace of ra_backward: the forward's plan (dQ kernel), the key-side plan
// of the dK/dV kernel, and the per-row sums D = dO . O.
struct BwdLayout {
  Layout fwd;
  int bk, bq;          // dK/dV kernel tile: keys per workgroup x query rows per tile
  int nkt_kv, nqt_kv;  // key tiles per chunk, query tiles
  int kwl_stride;      // entries reserved per key tile (nqt_kv)
  size_t kcount_off, korder_off, kwl_off, dsum_off, total;
};

// Shape checks shared by the attention entry points (no pointer checks).
ra_status check_shape(const ra_shape* shape, int32_t cp_size, int32_t rank, int32_t partition);

// cu_seqlens checks: NULL is one document; otherwise 0 = c0 < c1 < ... < c_n = s_total.
ra_status check_cu(const int32_t* cu, int32_t n_docs, int64_t s_total);

// Workspace layout of the attention entry points for a validated shape, given the
// local length (local_len) and the partition. The work list is built for query
// tiles of bm rows; bm = 0 takes the forward kernel's tile height for the shape.
Layout attn_layout(const ra_shape* shape, int32_t cp_size, int32_t n_docs_dev, int32_t partition, int64_t s_local,
                   int bm = 0);

// Workspace layout of ra_backward for a validated shape.
BwdLayout bwd_layout(const ra_shape* shape, int32_t cp_size, int32_t n_docs_dev, int32_t partition,
                     int64_t s_local);

// Full validation of ra_backward arguments.
ra_status check_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                         const void* dout, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                         int32_t partition, const ra_shape* shape, const float* dq, const float* dk, const float* dv,
                         const void* workspace, size_t ws_bytes);

// Number of documents the kernels see for a validated cu_seqlens argument.
int32_t effective_docs(const int32_t* cu, int32_t n_docs);

// Full validation of ra_forward / ra_forward_steps arguments.
ra_status check_forward(const void* q, const void* k, const void* v, const int32_t* cu, int32_t n_docs,
                        int32_t cp_size, int32_t rank, int32_t partition, const ra_shape* shape, const void* out0,
                        const void* out1, const void* workspace, size_t ws_bytes);

// ra_plan: shape, documents and workspace (no tensor pointers).
ra_status check_plan(const ra_shape* shape, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                     int32_t partition, const void* workspace, size_t ws_bytes);

// ra_forward_planned: tensors, shape and workspace; n_docs as given to ra_plan.
ra_status check_forward_planned(const void* q, const void* k, const void* v, int32_t n_docs, int32_t cp_size,
                                int32_t rank, int32_t partition, const ra_shape* shape, const void* out,
                                const void* lse, const void* workspace, size_t ws_bytes);

ra_status check_classify(const ra_shape* shape, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                         int32_t partition, int32_t bm, int32_t bn, const int8_t* cls, const void* workspace,
                         size_t ws_bytes);

ra_status check_lse_merge(int64_t rows, int32_t h, int32_t d, const float* o_a, const float* lse_a, const float* o_b,
                          const float* lse_b, const float* o_out, const float* lse_out);

ra_status check_ulysses(const void* in, const void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                        int32_t elem_bytes, int32_t inverse);

// Ulysses permute with the head-split side's n blocks block_stride bytes apart.
ra_status check_ulysses_strided(const void* in, const void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                                int32_t elem_bytes, int32_t inverse, int64_t block_stride);

// Workspace of usp_forward: head-split Q, K, V and O of the whole grid, then one
// ring rank's attention plan (rebuilt for every ring rank).
struct UspLayout {
  ra_shape slice;       // attention shape of one device's head slice
  size_t q_off, k_off, v_off, o_off, plan_off, total;
  size_t plan_bytes;
};
UspLayout usp_layout(const ra_shape* shape, int32_t ulysses, int32_t ring, int32_t n_docs_dev);

ra_status check_usp(const void* q, const void* k, const void* v, const int32_t* cu, int32_t n_docs, int32_t ulysses,
                    int32_t ring, int32_t partition, const ra_shape* shape, const void* out, const float* lse,
                    const void* workspace, size_t ws_bytes);

// cp_reorder_docs: tensors, shape and documents (the reorder of RA_PART_DOC_ZIGZAG).
ra_status check_cp_reorder_docs(const void* in, const void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                                int32_t cp_size, const int32_t* cu, int32_t n_docs, int32_t inverse,
                                const void* workspace, size_t ws_bytes);

ra_status check_cp_reorder(const void* in, const void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                           int32_t cp_size, int32_t partition, int32_t inverse);

}  // namespace ra
