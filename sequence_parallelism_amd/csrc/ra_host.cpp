// Host-side validation and workspace layout. Pure C++: no HIP calls, so the
// error paths run (and are tested) on machines without a GPU.
#include "ra_host.h"

#include <math.h>

namespace ra {

namespace {

constexpr int64_t kMaxTokens = (int64_t)1 << 30;  // positions and tile indices stay in int32
constexpr int32_t kMaxCp = 64;                    // ring step fits the work-list entry (6 bits)
constexpr int32_t kMaxHeads = 4096;

// Tile shapes of the attention kernels (must match the device code).
constexpr int kBf16BM = 128, kBf16BN = 64;
constexpr int kBf16D128BM = 256;  // forward, bf16, head_dim 128
constexpr int kF32BM = 64, kF32BN = 32;
constexpr int kBwdBf16BK = 128, kBwdBf16BQ = 64;
constexpr int kBwdF32BK = 64, kBwdF32BQ = 32;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool valid_partition(int32_t p) {
  return p == RA_PART_CONTIGUOUS || p == RA_PART_ZIGZAG || p == RA_PART_STRIPED || p == RA_PART_DOC_ZIGZAG;
}

ra_status check_divisible(int64_t s, int32_t cp, int32_t partition) {
  if (partition == RA_PART_DOC_ZIGZAG) return RA_OK;  // pieces are padded
  if (partition == RA_PART_ZIGZAG) return s % (2 * (int64_t)cp) == 0 ? RA_OK : RA_ERR_DIVISIBILITY;
  return s % cp == 0 ? RA_OK : RA_ERR_DIVISIBILITY;
}

constexpr int64_t kDocBlock = 64;     // doc-zigzag block (must match the device code)
constexpr int64_t kDocGranule = 256;  // doc-zigzag piece bound granule (must match the device code)

// Document-relative bound k (0..2cp) of the doc-zigzag pieces of a document of
// length L: k L / 2cp rounded to the nearest multiple of the granule (halves
// up), capped at L; bound 2cp is L.
int64_t doc_bound(int64_t L, int32_t cp, int64_t k) {
  const int64_t n = 2 * (int64_t)cp;
  if (k >= n) return L;
  const int64_t b = kDocGranule * ((2 * k * L + n * kDocGranule) / (2 * n * kDocGranule));
  return b < L ? b : L;
}

// 64-slot blocks that rank r holds of document j (length L): piece pair
// p = (r + j) mod cp, i.e. pieces p and 2cp-1-p, each padded to whole granules.
int64_t doc_rank_blocks(int64_t L, int32_t cp, int32_t r, int32_t j) {
  const int64_t p = (r + (int64_t)j) % cp, q = 2 * (int64_t)cp - 1 - p;
  const int64_t a = doc_bound(L, cp, p + 1) - doc_bound(L, cp, p);
  const int64_t b = doc_bound(L, cp, q + 1) - doc_bound(L, cp, q);
  const int64_t g = kDocGranule / kDocBlock;
  return g * ((a + kDocGranule - 1) / kDocGranule + (b + kDocGranule - 1) / kDocGranule);
}

bool overlaps(const void* a, const void* b, uint64_t bytes) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + bytes && y < x + bytes;
}

}  // namespace

ra_status check_shape(const ra_shape* shape, int32_t cp_size, int32_t rank, int32_t partition) {
  if (!shape) return RA_ERR_NULL;
  if (shape->s_total < 1 || shape->s_total > kMaxTokens) return RA_ERR_SHAPE;
  if (shape->hq < 1 || shape->hkv < 1 || shape->hq > kMaxHeads || shape->hkv > kMaxHeads) return RA_ERR_SHAPE;
  if (shape->causal != 0 && shape->causal != 1) return RA_ERR_SHAPE;
  if (!(shape->softmax_scale >= 0.f) || isinf(shape->softmax_scale)) return RA_ERR_SHAPE;
  if (cp_size < 1 || cp_size > kMaxCp) return RA_ERR_SHAPE;
  if (!valid_partition(partition)) return RA_ERR_UNSUPPORTED;
  if (rank < 0 || rank >= cp_size) return RA_ERR_RANK;
  if (shape->hq % shape->hkv != 0) return RA_ERR_HEADS;
  if (shape->d != 64 && shape->d != 128) return RA_ERR_UNSUPPORTED;
  if (shape->in_dtype != RA_BF16 && shape->in_dtype != RA_F32) return RA_ERR_UNSUPPORTED;
  if (shape->out_dtype != RA_BF16 && shape->out_dtype != RA_F32) return RA_ERR_UNSUPPORTED;
  if (shape->in_dtype == RA_F32 && shape->out_dtype != RA_F32) return RA_ERR_UNSUPPORTED;
  const ra_status st = check_divisible(shape->s_total, cp_size, partition);
  if (st != RA_OK) return st;
  // the kernels address one rank's Q and one K/V chunk with 32-bit byte offsets
  const int64_t heads = shape->hq > shape->hkv ? shape->hq : shape->hkv;
  const int64_t elem = shape->in_dtype == RA_BF16 ? 2 : 4;
  if ((shape->s_total / cp_size) * heads * shape->d * elem > 0x7fffffffLL) return RA_ERR_SHAPE;
  return RA_OK;
}

ra_status check_cu(const int32_t* cu, int32_t n_docs, int64_t s_total) {
  if (!cu) return RA_OK;
  if (n_docs < 1 || n_docs > s_total) return RA_ERR_CU_SEQLENS;
  if (cu[0] != 0 || cu[n_docs] != s_total) return RA_ERR_CU_SEQLENS;
  for (int32_t i = 0; i < n_docs; ++i)
    if (cu[i + 1] <= cu[i]) return RA_ERR_CU_SEQLENS;
  return RA_OK;
}

int32_t effective_docs(const int32_t* cu, int32_t n_docs) { return cu ? n_docs : 1; }

int64_t local_len(const ra_shape* shape, int32_t cp_size, int32_t partition, const int32_t* cu, int32_t n_docs) {
  if (partition != RA_PART_DOC_ZIGZAG) return shape->s_total / cp_size;
  const int32_t nd = cu ? n_docs : 1;
  int64_t widest = 0;
  for (int32_t r = 0; r < cp_size; ++r) {
    int64_t blocks = 0;
    for (int32_t j = 0; j < nd; ++j) {
      const int64_t L = cu ? (int64_t)cu[j + 1] - cu[j] : shape->s_total;
      blocks += doc_rank_blocks(L, cp_size, r, j);
      if (blocks * kDocBlock > ((int64_t)1 << 31) - 1) return -1;
    }
    widest = blocks > widest ? blocks : widest;
  }
  return widest * kDocBlock;
}

int64_t local_len_bound(const ra_shape* shape, int32_t cp_size, int32_t n_docs) {
  // a piece exceeds L / 2cp by at most one granule (each bound moves by at most
  // half a granule), and only a document's last piece is padded (by less than a
  // granule): a rank holds at most L / cp + 3 granules of slots per document
  const int64_t nd = n_docs > 1 ? n_docs : 1;
  const int64_t base = (shape->s_total + cp_size - 1) / cp_size;
  return ((base + 3 * kDocGranule * nd + kDocGranule - 1) / kDocGranule) * kDocGranule;
}

Layout attn_layout(const ra_shape* shape, int32_t cp_size, int32_t n_docs_dev, int32_t partition, int64_t s_local,
                   int bm) {
  Layout L{};
  L.s_local = (int)s_local;
  const bool bf16 = shape->in_dtype == RA_BF16;
  L.bm = bm > 0 ? bm : bf16 ? (shape->d == 128 ? kBf16D128BM : kBf16BM) : kF32BM;
  L.bn = bf16 ? kBf16BN : kF32BN;
  L.nqt = (L.s_local + L.bm - 1) / L.bm;
  L.nkt = (L.s_local + L.bn - 1) / L.bn;
  L.wl_stride = cp_size * L.nkt;
  L.n_docs_dev = n_docs_dev < 1 ? 1 : n_docs_dev;
  L.doczig = partition == RA_PART_DOC_ZIGZAG;
  L.nblk = L.doczig ? (int)(s_local / kDocBlock) : 0;
  const size_t cu_bytes = (L.n_docs_dev > 1 || L.doczig) ? (size_t)(L.n_docs_dev + 1) * 4 : 0;
  L.cu_off = 0;
  L.prefix_off = align256(L.cu_off + cu_bytes);
  L.blk_off = align256(L.prefix_off + (L.doczig ? (size_t)cp_size * (L.n_docs_dev + 1) * 4 : 0));
  L.count_off = align256(L.blk_off + (L.doczig ? (size_t)cp_size * L.nblk * 8 : 0));
  L.order_off = align256(L.count_off + (size_t)L.nqt * 4);
  L.wl_off = align256(L.order_off + (size_t)L.nqt * 4);
  L.total = align256(L.wl_off + (size_t)L.nqt * L.wl_stride * 4);
  return L;
}

BwdLayout bwd_layout(const ra_shape* shape, int32_t cp_size, int32_t n_docs_dev, int32_t partition,
                     int64_t s_local) {
  BwdLayout B{};
  const bool bf16 = shape->in_dtype == RA_BF16;
  // the dQ kernel walks the query-side work list in its own tile height
  B.fwd = attn_layout(shape, cp_size, n_docs_dev, partition, s_local, bf16 ? kBf16BM : kF32BM);
  B.bk = bf16 ? kBwdBf16BK : kBwdF32BK;
  B.bq = bf16 ? kBwdBf16BQ : kBwdF32BQ;
  const int sl = B.fwd.s_local;
  B.nkt_kv = (sl + B.bk - 1) / B.bk;
  B.nqt_kv = (sl + B.bq - 1) / B.bq;
  B.kwl_stride = B.nqt_kv;
  const size_t n_kt = (size_t)cp_size * B.nkt_kv;
  B.kcount_off = B.fwd.total;
  B.korder_off = align256(B.kcount_off + n_kt * 4);
  B.kwl_off = align256(B.korder_off + n_kt * 4);
  B.dsum_off = align256(B.kwl_off + n_kt * B.kwl_stride * 4);
  B.total = align256(B.dsum_off + (size_t)shape->hq * sl * 4);
  return B;
}

// Local length for the arguments, and the 32-bit byte bound of one rank's rows
// and one chunk at `elem` bytes per element (doc-zigzag lengths exceed S / cp).
ra_status checked_local_len(const ra_shape* shape, int32_t cp_size, int32_t partition, const int32_t* cu,
                            int32_t n_docs, int64_t elem, int64_t& s_local) {
  s_local = local_len(shape, cp_size, partition, cu, n_docs);
  if (s_local < 1) return RA_ERR_SHAPE;
  const int64_t heads = shape->hq > shape->hkv ? shape->hq : shape->hkv;
  if (s_local * heads * shape->d * elem > 0x7fffffffLL) return RA_ERR_SHAPE;
  return RA_OK;
}

ra_status check_backward(const void* q, const void* k, const void* v, const void* out, const float* lse,
                         const void* dout, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                         int32_t partition, const ra_shape* shape, const float* dq, const float* dk, const float* dv,
                         const void* workspace, size_t ws_bytes) {
  if (!q || !k || !v || !out || !lse || !dout || !shape || !dq || !dk || !dv) return RA_ERR_NULL;
  ra_status s = check_shape(shape, cp_size, rank, partition);
  if (s != RA_OK) return s;
  s = check_cu(cu, n_docs, shape->s_total);
  if (s != RA_OK) return s;
  // the fp32 gradients of one rank's rows and of one chunk stay within 2^31 bytes
  int64_t sl;
  s = checked_local_len(shape, cp_size, partition, cu, n_docs, 4, sl);
  if (s != RA_OK) return s;
  const BwdLayout B = bwd_layout(shape, cp_size, effective_docs(cu, n_docs), partition, sl);
  if ((int64_t)B.fwd.nqt * shape->hq > 0x7fffffffLL) return RA_ERR_SHAPE;
  if ((int64_t)cp_size * B.nkt_kv * shape->hkv > 0x7fffffffLL) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < B.total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

ra_status check_forward(const void* q, const void* k, const void* v, const int32_t* cu, int32_t n_docs,
                        int32_t cp_size, int32_t rank, int32_t partition, const ra_shape* shape, const void* out0,
                        const void* out1, const void* workspace, size_t ws_bytes) {
  if (!q || !k || !v || !shape || !out0 || !out1) return RA_ERR_NULL;
  ra_status s = check_shape(shape, cp_size, rank, partition);
  if (s != RA_OK) return s;
  s = check_cu(cu, n_docs, shape->s_total);
  if (s != RA_OK) return s;
  int64_t sl;
  s = checked_local_len(shape, cp_size, partition, cu, n_docs, shape->in_dtype == RA_BF16 ? 2 : 4, sl);
  if (s != RA_OK) return s;
  const Layout L = attn_layout(shape, cp_size, effective_docs(cu, n_docs), partition, sl);
  if ((int64_t)L.nqt * shape->hq > 0x7fffffffLL) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < L.total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

ra_status check_plan(const ra_shape* shape, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                     int32_t partition, const void* workspace, size_t ws_bytes) {
  if (!shape) return RA_ERR_NULL;
  ra_status s = check_shape(shape, cp_size, rank, partition);
  if (s != RA_OK) return s;
  s = check_cu(cu, n_docs, shape->s_total);
  if (s != RA_OK) return s;
  int64_t sl;
  s = checked_local_len(shape, cp_size, partition, cu, n_docs, shape->in_dtype == RA_BF16 ? 2 : 4, sl);
  if (s != RA_OK) return s;
  const Layout L = attn_layout(shape, cp_size, effective_docs(cu, n_docs), partition, sl);
  if ((int64_t)L.nqt * shape->hq > 0x7fffffffLL) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < L.total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

ra_status check_forward_planned(const void* q, const void* k, const void* v, int32_t n_docs, int32_t cp_size,
                                int32_t rank, int32_t partition, const ra_shape* shape, const void* out,
                                const void* lse, const void* workspace, size_t ws_bytes) {
  if (!q || !k || !v || !shape || !out || !lse) return RA_ERR_NULL;
  ra_status s = check_shape(shape, cp_size, rank, partition);
  if (s != RA_OK) return s;
  if (n_docs < 0 || n_docs > shape->s_total) return RA_ERR_CU_SEQLENS;
  if (partition == RA_PART_DOC_ZIGZAG) return RA_ERR_UNSUPPORTED;  // its local length needs cu_seqlens
  const Layout L = attn_layout(shape, cp_size, n_docs > 1 ? n_docs : 1, partition, shape->s_total / cp_size);
  if ((int64_t)L.nqt * shape->hq > 0x7fffffffLL) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < L.total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

// Compact doc-zigzag tables of ra_classify / cp_reorder_docs: cu, the per-rank
// block prefix (each 256-byte aligned), then the block descriptors.
size_t classify_doc_ws(int32_t nd, int32_t cp_size, int64_t s_local) {
  return align256((size_t)(nd + 1) * 4) + align256((size_t)cp_size * (nd + 1) * 4) +
         (size_t)cp_size * (size_t)(s_local / kDocBlock) * 8;
}

ra_status check_classify(const ra_shape* shape, const int32_t* cu, int32_t n_docs, int32_t cp_size, int32_t rank,
                         int32_t partition, int32_t bm, int32_t bn, const int8_t* cls, const void* workspace,
                         size_t ws_bytes) {
  if (!shape || !cls) return RA_ERR_NULL;
  if (shape->s_total < 1 || shape->s_total > kMaxTokens) return RA_ERR_SHAPE;
  if (shape->causal != 0 && shape->causal != 1) return RA_ERR_SHAPE;
  if (cp_size < 1 || cp_size > kMaxCp) return RA_ERR_SHAPE;
  if (!valid_partition(partition)) return RA_ERR_UNSUPPORTED;
  if (rank < 0 || rank >= cp_size) return RA_ERR_RANK;
  if (bm < 1 || bn < 1 || bm > 65536 || bn > 65536) return RA_ERR_SHAPE;
  ra_status s = check_divisible(shape->s_total, cp_size, partition);
  if (s != RA_OK) return s;
  s = check_cu(cu, n_docs, shape->s_total);
  if (s != RA_OK) return s;
  const int32_t nd = effective_docs(cu, n_docs);
  {
    // one launch thread per (step, query tile, key tile): at most 2^36 classes
    const int64_t sl = local_len(shape, cp_size, partition, cu, n_docs);
    if (sl < 1) return RA_ERR_SHAPE;
    const int64_t nqt = (sl + bm - 1) / bm, nkt = (sl + bn - 1) / bn;
    if (nqt > ((int64_t)1 << 36) / nkt / cp_size) return RA_ERR_SHAPE;
  }
  size_t need = nd > 1 ? (size_t)(nd + 1) * 4 : 0;
  if (partition == RA_PART_DOC_ZIGZAG) {
    // tiles must not span more than two 64-slot blocks
    const auto pow2_le128 = [](int32_t x) { return x == 16 || x == 32 || x == 64 || x == 128; };
    if (!pow2_le128(bm) || !pow2_le128(bn)) return RA_ERR_UNSUPPORTED;
    const int64_t sl = local_len(shape, cp_size, partition, cu, n_docs);
    if (sl < 1) return RA_ERR_SHAPE;
    need = classify_doc_ws(nd, cp_size, sl);
  }
  if (need > 0 && (!workspace || ws_bytes < need)) return RA_ERR_WORKSPACE;
  return RA_OK;
}

ra_status check_lse_merge(int64_t rows, int32_t h, int32_t d, const float* o_a, const float* lse_a, const float* o_b,
                          const float* lse_b, const float* o_out, const float* lse_out) {
  if (rows < 0 || h < 1 || d < 1) return RA_ERR_SHAPE;
  // at most 2^37 elements per tensor (512 GiB of fp32, beyond any one GPU): the
  // launch grids (one thread per (row, head) pair, or per 4 x 16 bytes) stay in range
  if (rows > ((int64_t)1 << 37) / ((int64_t)h * d)) return RA_ERR_SHAPE;
  if (rows == 0) return RA_OK;
  if (!o_a || !lse_a || !o_b || !lse_b || !o_out || !lse_out) return RA_ERR_NULL;
  return RA_OK;
}

ra_status check_ulysses(const void* in, const void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                        int32_t elem_bytes, int32_t inverse) {
  if (!in || !out) return RA_ERR_NULL;
  if (n < 1 || s_local < 1 || h < 1 || d < 1) return RA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return RA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return RA_ERR_UNSUPPORTED;
  if (h % n != 0) return RA_ERR_HEADS;
  if ((int64_t)n * s_local > kMaxTokens) return RA_ERR_SHAPE;
  const uint64_t bytes = (uint64_t)n * (uint64_t)s_local * (uint64_t)h * (uint64_t)d * (uint64_t)elem_bytes;
  if (bytes > ((uint64_t)1 << 42)) return RA_ERR_SHAPE;
  if (overlaps(in, out, bytes)) return RA_ERR_SHAPE;
  return RA_OK;
}

ra_status check_ulysses_strided(const void* in, const void* out, int32_t n, int64_t s_local, int32_t h, int32_t d,
                                int32_t elem_bytes, int32_t inverse, int64_t block_stride) {
  if (!in || !out) return RA_ERR_NULL;
  if (n < 1 || s_local < 1 || h < 1 || d < 1) return RA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return RA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return RA_ERR_UNSUPPORTED;
  if (h % n != 0) return RA_ERR_HEADS;
  if ((int64_t)n * s_local > kMaxTokens) return RA_ERR_SHAPE;
  const uint64_t bytes = (uint64_t)n * (uint64_t)s_local * (uint64_t)h * (uint64_t)d * (uint64_t)elem_bytes;
  if (bytes > ((uint64_t)1 << 42)) return RA_ERR_SHAPE;
  const uint64_t run = (uint64_t)(h / n) * (uint64_t)d * (uint64_t)elem_bytes;
  const uint64_t block = bytes / (uint64_t)n;
  if (block_stride < 0 || (uint64_t)block_stride < block || (uint64_t)block_stride % run != 0) return RA_ERR_SHAPE;
  const uint64_t span = (uint64_t)(n - 1) * (uint64_t)block_stride + block;
  if (span > ((uint64_t)1 << 44)) return RA_ERR_SHAPE;
  // the packed side and the strided side must not overlap
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out;
  const uint64_t ea = inverse ? span : bytes, eb = inverse ? bytes : span;
  if (a < b + eb && b < a + ea) return RA_ERR_SHAPE;
  return RA_OK;
}

UspLayout usp_layout(const ra_shape* shape, int32_t ulysses, int32_t ring, int32_t n_docs_dev) {
  UspLayout U{};
  U.slice = *shape;
  U.slice.hq = shape->hq / ulysses;
  U.slice.hkv = shape->hkv / ulysses;
  const size_t ei = shape->in_dtype == RA_BF16 ? 2 : 4, eo = shape->out_dtype == RA_BF16 ? 2 : 4;
  const size_t S = (size_t)shape->s_total, d = (size_t)shape->d;
  U.q_off = 0;
  U.k_off = align256(U.q_off + S * shape->hq * d * ei);
  U.v_off = align256(U.k_off + S * shape->hkv * d * ei);
  U.o_off = align256(U.v_off + S * shape->hkv * d * ei);
  U.plan_off = align256(U.o_off + S * shape->hq * d * eo);
  U.plan_bytes = attn_layout(&U.slice, ring, n_docs_dev, RA_PART_CONTIGUOUS, shape->s_total / ring).total;
  U.total = align256(U.plan_off + U.plan_bytes);
  return U;
}

ra_status check_usp(const void* q, const void* k, const void* v, const int32_t* cu, int32_t n_docs, int32_t ulysses,
                    int32_t ring, int32_t partition, const ra_shape* shape, const void* out, const float* lse,
                    const void* workspace, size_t ws_bytes) {
  if (!q || !k || !v || !shape || !out || !lse) return RA_ERR_NULL;
  if (ulysses < 1 || ulysses > kMaxHeads) return RA_ERR_SHAPE;
  if (partition == RA_PART_DOC_ZIGZAG) return RA_ERR_UNSUPPORTED;
  ra_status s = check_shape(shape, ring, 0, partition);
  if (s != RA_OK) return s;
  if (shape->hq % ulysses != 0 || shape->hkv % ulysses != 0) return RA_ERR_HEADS;
  if ((shape->s_total / ring) % ulysses != 0) return RA_ERR_DIVISIBILITY;
  s = check_cu(cu, n_docs, shape->s_total);
  if (s != RA_OK) return s;
  const UspLayout U = usp_layout(shape, ulysses, ring, effective_docs(cu, n_docs));
  const Layout L = attn_layout(&U.slice, ring, effective_docs(cu, n_docs), partition, shape->s_total / ring);
  if ((int64_t)L.nqt * U.slice.hq > 0x7fffffffLL) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < U.total) return RA_ERR_WORKSPACE;
  return RA_OK;
}

ra_status check_cp_reorder(const void* in, const void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                           int32_t cp_size, int32_t partition, int32_t inverse) {
  if (!in || !out) return RA_ERR_NULL;
  if (s < 1 || s > kMaxTokens || h < 1 || d < 1) return RA_ERR_SHAPE;
  if (cp_size < 1 || cp_size > 65536) return RA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return RA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return RA_ERR_UNSUPPORTED;
  if (!valid_partition(partition) || partition == RA_PART_DOC_ZIGZAG) return RA_ERR_UNSUPPORTED;
  const ra_status st = check_divisible(s, cp_size, partition);
  if (st != RA_OK) return st;
  const uint64_t bytes = (uint64_t)s * (uint64_t)h * (uint64_t)d * (uint64_t)elem_bytes;
  if (bytes > ((uint64_t)1 << 42)) return RA_ERR_SHAPE;
  if (overlaps(in, out, bytes)) return RA_ERR_SHAPE;
  return RA_OK;
}

ra_status check_cp_reorder_docs(const void* in, const void* out, int64_t s, int32_t h, int32_t d, int32_t elem_bytes,
                                int32_t cp_size, const int32_t* cu, int32_t n_docs, int32_t inverse,
                                const void* workspace, size_t ws_bytes) {
  if (!in || !out) return RA_ERR_NULL;
  if (s < 1 || s > kMaxTokens || h < 1 || d < 1) return RA_ERR_SHAPE;
  if (cp_size < 1 || cp_size > kMaxCp) return RA_ERR_SHAPE;
  if (inverse != 0 && inverse != 1) return RA_ERR_SHAPE;
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return RA_ERR_UNSUPPORTED;
  ra_status st = check_cu(cu, n_docs, s);
  if (st != RA_OK) return st;
  ra_shape shp{};
  shp.s_total = s;
  const int64_t sl = local_len(&shp, cp_size, RA_PART_DOC_ZIGZAG, cu, n_docs);
  if (sl < 1) return RA_ERR_SHAPE;
  const uint64_t row = (uint64_t)h * (uint64_t)d * (uint64_t)elem_bytes;
  const uint64_t in_bytes = inverse ? (uint64_t)cp_size * sl * row : (uint64_t)s * row;
  const uint64_t out_bytes = inverse ? (uint64_t)s * row : (uint64_t)cp_size * sl * row;
  if (in_bytes > ((uint64_t)1 << 42) || out_bytes > ((uint64_t)1 << 42)) return RA_ERR_SHAPE;
  const uintptr_t a = (uintptr_t)in, b = (uintptr_t)out;
  if (a < b + out_bytes && b < a + in_bytes) return RA_ERR_SHAPE;
  if (!workspace || ws_bytes < classify_doc_ws(effective_docs(cu, n_docs), cp_size, sl)) return RA_ERR_WORKSPACE;
  return RA_OK;
}

}  // namespace ra
