// C-ABI entry points of the ring-attention library (declared in include/ra.h).
// Each call validates on the host (ra_host.cpp) before anything is launched,
// then enqueues its kernels on the caller's stream.
#include <math.h>

#include <mutex>
#include <vector>

#include "../../include/ra.h"
#include "ra_common.h"
#include "ra_host.h"
#include "ra_internal.h"

using namespace ra;

namespace {

constexpr float kLog2e = 1.4426950408889634f;

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// Compact doc-zigzag tables (ra_classify, cp_reorder_docs): cu, per-rank block prefix, descriptors.
struct DocRegions {
  size_t cu_off, prefix_off, blk_off, total;
  int nblk;
};

DocRegions doc_regions(int32_t nd, int32_t cp, int64_t s_local) {
  DocRegions R{};
  R.cu_off = 0;
  R.prefix_off = round256((size_t)(nd + 1) * 4);
  R.blk_off = R.prefix_off + round256((size_t)cp * (nd + 1) * 4);
  R.nblk = (int)(s_local / 64);
  R.total = R.blk_off + (size_t)cp * R.nblk * 8;
  return R;
}

ra_status upload_doc_tables(char* ws, const DocRegions& R, const ra_shape* shape, const int32_t* cu, int32_t nd,
                            int32_t cp, hipStream_t st) {
  const int32_t one[2] = {0, (int32_t)shape->s_total};
  int* dcu = (int*)(ws + R.cu_off);
  if (launch_upload_i32(cu ? cu : one, nd + 1, dcu, st) != hipSuccess ||
      launch_doc_blocks(dcu, (int*)(ws + R.prefix_off), nd, cp, R.nblk, (int2*)(ws + R.blk_off), st) != hipSuccess)
    return RA_ERR_HIP;
  return RA_OK;
}

// Layout of the attention workspace for validated arguments (host cu_seqlens, or NULL).
Layout layout_for(const ra_shape* shape, int32_t cp, int32_t partition, const int32_t* cu, int32_t nd) {
  return attn_layout(shape, cp, nd, partition, local_len(shape, cp, partition, cu, nd));
}

// Uploads cu_seqlens (and, for doc-zigzag, builds the per-rank block prefix and the
// block descriptors); the device pointers land in the layout's regions of `workspace`.
ra_status upload_docs(const Layout& L, const int32_t* cu, int32_t nd, int32_t cp, int32_t partition,
                      const ra_shape* shape, char* ws, hipStream_t st) {
  int* dcu = (int*)(ws + L.cu_off);
  if (L.doczig) {
    const int32_t one[2] = {0, (int32_t)shape->s_total};
    if (launch_upload_i32(cu ? cu : one, nd + 1, dcu, st) != hipSuccess ||
        launch_doc_blocks(dcu, (int*)(ws + L.prefix_off), nd, cp, L.nblk, (int2*)(ws + L.blk_off), st) != hipSuccess)
      return RA_ERR_HIP;
  } else if (nd > 1 && launch_upload_i32(cu, nd + 1, dcu, st) != hipSuccess) {
    return RA_ERR_HIP;
  }
  return RA_OK;
}

// Uploads the document tables and builds the work list and tile order for the
// query tiles of layout L.
ra_status run_plan(const Layout& L, const int32_t* cu, int32_t nd, int32_t cp, int32_t rank, int32_t partition,
                   const ra_shape* shape, void* workspace, hipStream_t st) {
  char* ws = (char*)workspace;
  const ra_status u = upload_docs(L, cu, nd, cp, partition, shape, ws, st);
  if (u != RA_OK) return u;
  const int* dcu = nd > 1 ? (const int*)(ws + L.cu_off) : nullptr;
  const int2* blk = L.doczig ? (const int2*)(ws + L.blk_off) : nullptr;
  if (launch_worklist(dcu, blk, nd, (int)shape->s_total, L.s_local, cp, rank, partition, shape->causal, L.bm, L.bn,
                      L.nqt, L.nkt, L.wl_stride, (int*)(ws + L.wl_off), (int*)(ws + L.count_off),
                      (int*)(ws + L.order_off), st) != hipSuccess)
    return RA_ERR_HIP;
  return RA_OK;
}

// The same for the forward kernel's tile height.
ra_status run_plan(const int32_t* cu, int32_t nd, int32_t cp, int32_t rank, int32_t partition, const ra_shape* shape,
                   void* workspace, hipStream_t st) {
  return run_plan(layout_for(shape, cp, partition, cu, nd), cu, nd, cp, rank, partition, shape, workspace, st);
}

ra_status run_attention(const void* q, const void* k, const void* v, const Layout& L, int32_t nd, int32_t cp,
                        int32_t rank, int32_t partition, const ra_shape* shape, void* out, float* lse, float* o_steps,
                        float* lse_steps, void* workspace, hipStream_t st, bool steps) {
  char* ws = (char*)workspace;
  const float scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.f / sqrtf((float)shape->d);
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.o_steps = o_steps;
  a.lse_steps = lse_steps;
  a.cu = nd > 1 ? (const int*)(ws + L.cu_off) : nullptr;
  a.blk = L.doczig ? (const int2*)(ws + L.blk_off) : nullptr;
  a.wl = (const int*)(ws + L.wl_off);
  a.wl_count = (const int*)(ws + L.count_off);
  a.order = (const int*)(ws + L.order_off);
  a.n_docs = nd;
  a.s_total = (int)shape->s_total;
  a.s_local = L.s_local;
  a.cp = cp;
  a.rank = rank;
  a.part = partition;
  a.causal = shape->causal;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.nqt = L.nqt;
  a.nkt = L.nkt;
  a.wl_stride = L.wl_stride;
  a.scale_log2 = scale * kLog2e;
  const hipError_t e = launch_ring_attn(a, shape->d, shape->in_dtype == RA_BF16, shape->out_dtype == RA_BF16,
                                        steps ? 1 : 0, st);
  return e == hipSuccess ? RA_OK : RA_ERR_HIP;
}

ra_status run_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                       const void* dout, const int32_t* cu, int32_t nd, int32_t cp, int32_t rank, int32_t partition,
                       const ra_shape* shape, float* dq, float* dk, float* dv, void* workspace, hipStream_t st) {
  const BwdLayout B = bwd_layout(shape, cp, nd, partition, local_len(shape, cp, partition, cu, nd));
  const Layout& L = B.fwd;
  char* ws = (char*)workspace;
  const ra_status p = run_plan(L, cu, nd, cp, rank, partition, shape, workspace, st);
  if (p != RA_OK) return p;
  const int* dcu = nd > 1 ? (const int*)(ws + L.cu_off) : nullptr;
  const int2* blk = L.doczig ? (const int2*)(ws + L.blk_off) : nullptr;
  if (launch_kv_worklist(dcu, blk, nd, (int)shape->s_total, L.s_local, cp, rank, partition, shape->causal, B.bq, B.bk,
                         B.nqt_kv, B.nkt_kv, B.kwl_stride, (int*)(ws + B.kwl_off), (int*)(ws + B.kcount_off),
                         (int*)(ws + B.korder_off), st) != hipSuccess)
    return RA_ERR_HIP;
  float* dsum = (float*)(ws + B.dsum_off);
  if (launch_bwd_dsum(out, dout, dsum, L.s_local, shape->hq, shape->d, shape->out_dtype == RA_BF16,
                      shape->in_dtype == RA_BF16, st) != hipSuccess)
    return RA_ERR_HIP;
  const float scale = shape->softmax_scale > 0.f ? shape->softmax_scale : 1.f / sqrtf((float)shape->d);
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dsum = dsum;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu = dcu;
  a.blk = blk;
  a.wl = (const int*)(ws + L.wl_off);
  a.wl_count = (const int*)(ws + L.count_off);
  a.order = (const int*)(ws + L.order_off);
  a.kwl = (const int*)(ws + B.kwl_off);
  a.kwl_count = (const int*)(ws + B.kcount_off);
  a.korder = (const int*)(ws + B.korder_off);
  a.n_docs = nd;
  a.s_total = (int)shape->s_total;
  a.s_local = L.s_local;
  a.cp = cp;
  a.rank = rank;
  a.part = partition;
  a.causal = shape->causal;
  a.hq = shape->hq;
  a.hkv = shape->hkv;
  a.nqt = L.nqt;
  a.nkt = L.nkt;
  a.wl_stride = L.wl_stride;
  a.nkt_kv = B.nkt_kv;
  a.nqt_kv = B.nqt_kv;
  a.kwl_stride = B.kwl_stride;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  return launch_ring_bwd(a, shape->d, shape->in_dtype == RA_BF16, st) == hipSuccess ? RA_OK : RA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Fixed scratch of ra_forward_noalloc. Every GPU the library runs on holds its own
// copy of this array until the process ends. In host code `scratch` names a
// host-side stand-in, not device memory: the array's address on a device comes
// from hipGetSymbolAddress with that device current, taken once per device and
// kept in scratch_ptr[]; only that address is ever passed to kernels.
// ---------------------------------------------------------------------------
static __device__ __align__(256) char scratch[RA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];

// The current device's scratch address (looked up on the first call on that
// device), or nullptr if the runtime reports an error.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

int32_t ra_abi_version(void) { return 3; }

const char* ra_status_string(ra_status s) {
  switch (s) {
    case RA_OK: return "ok";
    case RA_ERR_NULL: return "a required pointer is NULL";
    case RA_ERR_SHAPE: return "invalid size or argument value";
    case RA_ERR_DIVISIBILITY: return "sequence length not divisible by the CP partition";
    case RA_ERR_HEADS: return "head count not divisible (Ulysses degree or query/KV head ratio)";
    case RA_ERR_CU_SEQLENS: return "cu_seqlens must be 0 = c0 < c1 < ... < c_n = S";
    case RA_ERR_RANK: return "rank outside [0, cp_size)";
    case RA_ERR_UNSUPPORTED: return "unsupported head_dim, dtype, element size or partition";
    case RA_ERR_WORKSPACE: return "workspace missing or smaller than ra_workspace_size()";
    case RA_ERR_HIP: return "HIP launch failed";
    case RA_ERR_SCRATCH: return "the plan needs more than RA_NOALLOC_SCRATCH_BYTES of fixed scratch";
  }
  return "unknown status";
}

size_t ra_workspace_size(const ra_shape* shape, int32_t cp_size, int32_t n_docs) {
  if (!shape || shape->s_total < 1 || shape->s_total > ((int64_t)1 << 30)) return 0;
  if (cp_size < 1 || cp_size > 64) return 0;
  if (shape->in_dtype != RA_BF16 && shape->in_dtype != RA_F32) return 0;
  // enough for every partition: the doc-zigzag bound on the local length, with its regions
  const int32_t nd = n_docs > 1 ? n_docs : 1;
  const size_t plain = attn_layout(shape, cp_size, nd, RA_PART_CONTIGUOUS, shape->s_total / cp_size).total;
  const size_t docs = attn_layout(shape, cp_size, nd, RA_PART_DOC_ZIGZAG, local_len_bound(shape, cp_size, nd)).total;
  return plain > docs ? plain : docs;
}

ra_status ra_forward(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_docs,
                     int32_t cp_size, int32_t rank, int32_t partition, const ra_shape* shape, void* out, float* lse,
                     void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s = check_forward(q, k, v, cu_seqlens, n_docs, cp_size, rank, partition, shape, out, lse, workspace,
                                    ws_bytes);
  if (s != RA_OK) return s;
  const hipStream_t st = as_stream(stream);
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  const ra_status p = run_plan(cu_seqlens, nd, cp_size, rank, partition, shape, workspace, st);
  if (p != RA_OK) return p;
  return run_attention(q, k, v, layout_for(shape, cp_size, partition, cu_seqlens, nd), nd, cp_size, rank, partition,
                       shape, out, lse, nullptr, nullptr, workspace, st, false);
}

ra_status ra_forward_noalloc(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                             int32_t n_docs, int32_t cp_size, int32_t rank, int32_t partition,
                             const ra_shape* shape, void* out, float* lse, void* stream) {
  // every check of ra_forward except the workspace's, which the fixed scratch replaces
  const ra_status s = check_forward(q, k, v, cu_seqlens, n_docs, cp_size, rank, partition, shape, out, lse,
                                    (const void*)out, SIZE_MAX);
  if (s != RA_OK) return s;
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  const Layout L = layout_for(shape, cp_size, partition, cu_seqlens, nd);
  if (L.total > RA_NOALLOC_SCRATCH_BYTES) return RA_ERR_SCRATCH;
  void* ws = device_scratch();
  if (!ws) return RA_ERR_HIP;
  const hipStream_t st = as_stream(stream);
  // the plan writes every scratch entry that the attention kernel reads (counts,
  // order and the first count entries of each list): nothing needs clearing
  const ra_status p = run_plan(L, cu_seqlens, nd, cp_size, rank, partition, shape, ws, st);
  if (p != RA_OK) return p;
  return run_attention(q, k, v, L, nd, cp_size, rank, partition, shape, out, lse, nullptr, nullptr, ws, st, false);
}

ra_status ra_plan(const ra_shape* shape, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size, int32_t rank,
                  int32_t partition, void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s = check_plan(shape, cu_seqlens, n_docs, cp_size, rank, partition, workspace, ws_bytes);
  if (s != RA_OK) return s;
  return run_plan(cu_seqlens, effective_docs(cu_seqlens, n_docs), cp_size, rank, partition, shape, workspace,
                  as_stream(stream));
}

ra_status ra_forward_planned(const void* q, const void* k, const void* v, int32_t n_docs, int32_t cp_size,
                             int32_t rank, int32_t partition, const ra_shape* shape, void* out, float* lse,
                             void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s = check_forward_planned(q, k, v, n_docs, cp_size, rank, partition, shape, out, lse, workspace,
                                            ws_bytes);
  if (s != RA_OK) return s;
  const int32_t nd = n_docs > 1 ? n_docs : 1;
  return run_attention(q, k, v, attn_layout(shape, cp_size, nd, partition, shape->s_total / cp_size), nd, cp_size,
                       rank, partition, shape, out, lse, nullptr, nullptr, workspace, as_stream(stream), false);
}

ra_status ra_forward_planned_docs(const void* q, const void* k, const void* v, const int32_t* cu_seqlens,
                                  int32_t n_docs, int32_t cp_size, int32_t rank, const ra_shape* shape, void* out,
                                  float* lse, void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s = check_forward(q, k, v, cu_seqlens, n_docs, cp_size, rank, RA_PART_DOC_ZIGZAG, shape, out, lse,
                                    workspace, ws_bytes);
  if (s != RA_OK) return s;
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  return run_attention(q, k, v, layout_for(shape, cp_size, RA_PART_DOC_ZIGZAG, cu_seqlens, nd), nd, cp_size, rank,
                       RA_PART_DOC_ZIGZAG, shape, out, lse, nullptr, nullptr, workspace, as_stream(stream), false);
}

ra_status ra_forward_steps(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_docs,
                           int32_t cp_size, int32_t rank, int32_t partition, const ra_shape* shape, float* o_steps,
                           float* lse_steps, void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s = check_forward(q, k, v, cu_seqlens, n_docs, cp_size, rank, partition, shape, o_steps, lse_steps,
                                    workspace, ws_bytes);
  if (s != RA_OK) return s;
  const hipStream_t st = as_stream(stream);
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  const ra_status p = run_plan(cu_seqlens, nd, cp_size, rank, partition, shape, workspace, st);
  if (p != RA_OK) return p;
  return run_attention(q, k, v, layout_for(shape, cp_size, partition, cu_seqlens, nd), nd, cp_size, rank, partition,
                       shape, nullptr, nullptr, o_steps, lse_steps, workspace, st, true);
}

size_t ra_backward_workspace_size(const ra_shape* shape, int32_t cp_size, int32_t n_docs) {
  if (!shape || shape->s_total < 1 || shape->s_total > ((int64_t)1 << 30)) return 0;
  if (cp_size < 1 || cp_size > 64) return 0;
  if (shape->in_dtype != RA_BF16 && shape->in_dtype != RA_F32) return 0;
  if (shape->hq < 1 || shape->hq > 4096) return 0;
  // enough for every partition (the doc-zigzag bound on the local length)
  const int32_t nd = n_docs > 1 ? n_docs : 1;
  const size_t plain = bwd_layout(shape, cp_size, nd, RA_PART_CONTIGUOUS, shape->s_total / cp_size).total;
  const size_t docs = bwd_layout(shape, cp_size, nd, RA_PART_DOC_ZIGZAG, local_len_bound(shape, cp_size, nd)).total;
  return plain > docs ? plain : docs;
}

ra_status ra_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                      const void* dout, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size, int32_t rank,
                      int32_t partition, const ra_shape* shape, float* dq, float* dk, float* dv, void* workspace,
                      size_t ws_bytes, void* stream) {
  const ra_status s = check_backward(q, k, v, out, lse, dout, cu_seqlens, n_docs, cp_size, rank, partition, shape, dq,
                                     dk, dv, workspace, ws_bytes);
  if (s != RA_OK) return s;
  return run_backward(q, k, v, out, lse, dout, cu_seqlens, effective_docs(cu_seqlens, n_docs), cp_size, rank,
                      partition, shape, dq, dk, dv, workspace, as_stream(stream));
}

ra_status ra_lse_merge(int64_t rows, int32_t h, int32_t d, const float* o_a, const float* lse_a, const float* o_b,
                       const float* lse_b, float* o_out, float* lse_out, void* stream) {
  const ra_status s = check_lse_merge(rows, h, d, o_a, lse_a, o_b, lse_b, o_out, lse_out);
  if (s != RA_OK) return s;
  if (rows == 0) return RA_OK;
  return launch_lse_merge(rows, h, d, o_a, lse_a, o_b, lse_b, o_out, lse_out, as_stream(stream)) == hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

ra_status ra_classify(const ra_shape* shape, const int32_t* cu_seqlens, int32_t n_docs, int32_t cp_size, int32_t rank,
                      int32_t partition, int32_t bm, int32_t bn, int8_t* cls, void* workspace, size_t ws_bytes,
                      void* stream) {
  const ra_status s =
      check_classify(shape, cu_seqlens, n_docs, cp_size, rank, partition, bm, bn, cls, workspace, ws_bytes);
  if (s != RA_OK) return s;
  const hipStream_t st = as_stream(stream);
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  const int s_local = (int)local_len(shape, cp_size, partition, cu_seqlens, nd);
  int* dcu = nd > 1 ? (int*)workspace : nullptr;
  const int2* blk = nullptr;
  if (partition == RA_PART_DOC_ZIGZAG) {
    const DocRegions R = doc_regions(nd, cp_size, s_local);
    const ra_status u = upload_doc_tables((char*)workspace, R, shape, cu_seqlens, nd, cp_size, st);
    if (u != RA_OK) return u;
    dcu = nd > 1 ? (int*)((char*)workspace + R.cu_off) : nullptr;
    blk = (const int2*)((char*)workspace + R.blk_off);
  } else if (nd > 1 && launch_upload_i32(cu_seqlens, nd + 1, dcu, st) != hipSuccess) {
    return RA_ERR_HIP;
  }
  const int nqt = (s_local + bm - 1) / bm, nkt = (s_local + bn - 1) / bn;
  return launch_classify(dcu, blk, nd, (int)shape->s_total, s_local, cp_size, rank, partition, shape->causal, bm, bn,
                         nqt, nkt, cls, st) == hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

ra_status ulysses_permute(const void* in, void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                          int32_t elem_bytes, int32_t inverse, void* stream) {
  const ra_status s = check_ulysses(in, out, n, s_local, h, d, elem_bytes, inverse);
  if (s != RA_OK) return s;
  const int64_t run_bytes = (int64_t)(h / n) * d * elem_bytes;
  return launch_ulysses(in, out, n, s_local, run_bytes, inverse, (int64_t)n * s_local, as_stream(stream)) ==
                 hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

ra_status ulysses_permute_strided(const void* in, void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                                  int32_t elem_bytes, int32_t inverse, int64_t block_stride, void* stream) {
  const ra_status s = check_ulysses_strided(in, out, n, s_local, h, d, elem_bytes, inverse, block_stride);
  if (s != RA_OK) return s;
  const int64_t run_bytes = (int64_t)(h / n) * d * elem_bytes;
  return launch_ulysses(in, out, n, s_local, run_bytes, inverse, block_stride / run_bytes, as_stream(stream)) ==
                 hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

size_t usp_workspace_size(const ra_shape* shape, int32_t ulysses, int32_t ring, int32_t n_docs) {
  if (!shape || shape->s_total < 1 || shape->s_total > ((int64_t)1 << 30)) return 0;
  if (ring < 1 || ring > 64 || ulysses < 1 || shape->s_total % ring) return 0;
  if (shape->hq < 1 || shape->hkv < 1 || shape->hq % ulysses || shape->hkv % ulysses) return 0;
  if (shape->in_dtype != RA_BF16 && shape->in_dtype != RA_F32) return 0;
  if (shape->d < 1) return 0;
  return usp_layout(shape, ulysses, ring, n_docs > 1 ? n_docs : 1).total;
}

ra_status usp_forward(const void* q, const void* k, const void* v, const int32_t* cu_seqlens, int32_t n_docs,
                      int32_t ulysses, int32_t ring, int32_t partition, const ra_shape* shape, void* out, float* lse,
                      void* workspace, size_t ws_bytes, void* stream) {
  const ra_status s =
      check_usp(q, k, v, cu_seqlens, n_docs, ulysses, ring, partition, shape, out, lse, workspace, ws_bytes);
  if (s != RA_OK) return s;
  const hipStream_t st = as_stream(stream);
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  const UspLayout U = usp_layout(shape, ulysses, ring, nd);
  const int64_t S = shape->s_total, sl = S / ring, shard = sl / ulysses, d = shape->d;
  const int64_t ei = shape->in_dtype == RA_BF16 ? 2 : 4, eo = shape->out_dtype == RA_BF16 ? 2 : 4;
  const int64_t hq = shape->hq, hkv = shape->hkv, hqs = hq / ulysses, hkvs = hkv / ulysses;
  char* ws = (char*)workspace;
  char *QU = ws + U.q_off, *KU = ws + U.k_off, *VU = ws + U.v_off, *OU = ws + U.o_off;
  void* plan = ws + U.plan_off;
  const Layout plan_layout = attn_layout(&U.slice, ring, nd, partition, sl);
  // 1. Ulysses all-to-all inside every ring group r: device (u, r)'s head slice lands at [u][r]
  for (int32_t r = 0; r < ring; ++r) {
    const int64_t gq = r * ulysses * shard * hq * d * ei, gk = r * ulysses * shard * hkv * d * ei;
    if (launch_ulysses((const char*)q + gq, QU + r * sl * hqs * d * ei, ulysses, shard, hqs * d * ei, 0,
                       (int64_t)ring * sl, st) != hipSuccess ||
        launch_ulysses((const char*)k + gk, KU + r * sl * hkvs * d * ei, ulysses, shard, hkvs * d * ei, 0,
                       (int64_t)ring * sl, st) != hipSuccess ||
        launch_ulysses((const char*)v + gk, VU + r * sl * hkvs * d * ei, ulysses, shard, hkvs * d * ei, 0,
                       (int64_t)ring * sl, st) != hipSuccess)
      return RA_ERR_HIP;
  }
  // 2. ring attention of device (u, r) over the R chunks of head slice u
  for (int32_t r = 0; r < ring; ++r) {
    const ra_status p = run_plan(cu_seqlens, nd, ring, r, partition, &U.slice, plan, st);
    if (p != RA_OK) return p;
    for (int32_t u = 0; u < ulysses; ++u) {
      const int64_t dev = (int64_t)u * ring + r;
      const ra_status a = run_attention(QU + dev * sl * hqs * d * ei, KU + (int64_t)u * ring * sl * hkvs * d * ei,
                                        VU + (int64_t)u * ring * sl * hkvs * d * ei, plan_layout, nd, ring, r,
                                        partition, &U.slice,
                                        OU + dev * sl * hqs * d * eo, lse + dev * hqs * sl, nullptr, nullptr, plan, st,
                                        false);
      if (a != RA_OK) return a;
    }
  }
  // 3. inverse all-to-all inside every ring group
  for (int32_t r = 0; r < ring; ++r) {
    if (launch_ulysses(OU + r * sl * hqs * d * eo, (char*)out + r * ulysses * shard * hq * d * eo, ulysses, shard,
                       hqs * d * eo, 1, (int64_t)ring * sl, st) != hipSuccess)
      return RA_ERR_HIP;
  }
  return RA_OK;
}

int64_t ra_local_length(int64_t s_total, int32_t cp_size, int32_t partition, const int32_t* cu_seqlens,
                        int32_t n_docs) {
  if (s_total < 1 || s_total > ((int64_t)1 << 30) || cp_size < 1 || cp_size > 64) return -1;
  if (partition < RA_PART_CONTIGUOUS || partition > RA_PART_DOC_ZIGZAG) return -1;
  if (check_cu(cu_seqlens, n_docs, s_total) != RA_OK) return -1;
  ra_shape shp{};
  shp.s_total = s_total;
  if (partition != RA_PART_DOC_ZIGZAG) {
    const int64_t div = partition == RA_PART_ZIGZAG ? 2 * (int64_t)cp_size : cp_size;
    return s_total % div == 0 ? s_total / cp_size : -1;
  }
  return local_len(&shp, cp_size, partition, cu_seqlens, effective_docs(cu_seqlens, n_docs));
}

size_t ra_doc_workspace_size(int64_t s_total, int32_t cp_size, const int32_t* cu_seqlens, int32_t n_docs) {
  const int64_t sl = ra_local_length(s_total, cp_size, RA_PART_DOC_ZIGZAG, cu_seqlens, n_docs);
  if (sl < 1) return 0;
  return doc_regions(effective_docs(cu_seqlens, n_docs), cp_size, sl).total;
}

ra_status cp_reorder_docs(const void* in, void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                          int32_t cp_size, const int32_t* cu_seqlens, int32_t n_docs, int32_t inverse,
                          void* workspace, size_t ws_bytes, void* stream) {
  const ra_status c =
      check_cp_reorder_docs(in, out, s, h, d, elem_bytes, cp_size, cu_seqlens, n_docs, inverse, workspace, ws_bytes);
  if (c != RA_OK) return c;
  const hipStream_t st = as_stream(stream);
  const int32_t nd = effective_docs(cu_seqlens, n_docs);
  ra_shape shp{};
  shp.s_total = s;
  const int64_t sl = local_len(&shp, cp_size, RA_PART_DOC_ZIGZAG, cu_seqlens, nd);
  const DocRegions R = doc_regions(nd, cp_size, sl);
  char* ws = (char*)workspace;
  const ra_status u = upload_doc_tables(ws, R, &shp, cu_seqlens, nd, cp_size, st);
  if (u != RA_OK) return u;
  return launch_cp_reorder_docs(in, out, (int64_t)h * d * elem_bytes, cp_size, (int)sl,
                                (const int2*)(ws + R.blk_off), inverse, st) == hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

ra_status cp_reorder(const void* in, void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes, int32_t cp_size,
                     int32_t partition, int32_t inverse, void* stream) {
  const ra_status st = check_cp_reorder(in, out, s, h, d, elem_bytes, cp_size, partition, inverse);
  if (st != RA_OK) return st;
  const int64_t row_bytes = (int64_t)h * d * elem_bytes;
  return launch_cp_reorder(in, out, s, row_bytes, cp_size, partition, inverse, as_stream(stream)) == hipSuccess
             ? RA_OK
             : RA_ERR_HIP;
}

}  // extern "C"
