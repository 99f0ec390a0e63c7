// Device-side helpers shared by the ring-attention kernels (gfx950).
//
// Position runs: a range of a rank's local indices maps to global positions
// that form at most two arithmetic progressions ("runs"):
//   contiguous: pos = owner*S_l + i                    (one run, stride 1)
//   striped:    pos = owner + cp*i                     (one run, stride cp)
//   zigzag:     i <  S_l/2: pos = owner*half + i       (run 1, stride 1)
//               i >= S_l/2: pos = (2cp-1-owner)*half + (i - half)   (run 2)
//   doc-zigzag: every packed document is cut into 2cp pieces padded to
//               multiples of 64 slots; local index i lies in 64-slot block
//               i / 64, whose first `cnt` slots hold positions start, start+1,
//               ... (a per-block descriptor) and whose other slots are padding
//               (position -1). An aligned range of at most 128 indices spans at
//               most two blocks, so it is at most two runs as well.
// (partition definitions: ra.h, RA_PART_*; zigzag and striped are the
// load-balancing reorders named on the long-context deep-dive page's timeline.)
//
// Visibility of key position pk from query position pq is the interval test
//   lo(pq) <= pk <= hi(pq),  lo = start of pq's document,
//   hi = pq (causal) or end of pq's document - 1 (non-causal),
// which is the causal mask on global positions of the Context Parallelism
// page (3.3, 5.2) restricted to pq's packed document (XTuner chapter 9.5).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ra {

enum { PART_CONTIGUOUS = 0, PART_ZIGZAG = 1, PART_STRIPED = 2, PART_DOC_ZIGZAG = 3 };

// Slots per doc-zigzag block (each block holds one run of positions, then padding).
constexpr int kDocBlock = 64;
constexpr int kDocGranule = 256;  // doc-zigzag piece bounds fall on multiples of this many tokens
enum { CLS_SKIP = 0, CLS_PARTIAL = 1, CLS_FULL = 2 };

// Work-list entry: bits 0-1 class, bits 2-7 ring step, bits 8-31 key tile.
__host__ __device__ inline int wl_pack(int t, int J, int cls) { return (J << 8) | (t << 2) | cls; }
__host__ __device__ inline int wl_cls(int e) { return e & 3; }
__host__ __device__ inline int wl_step(int e) { return (e >> 2) & 63; }
__host__ __device__ inline int wl_tile(int e) { return (int)((unsigned)e >> 8); }

struct Run {
  int start;   // global position of element 0
  int stride;  // 1 or cp
  int cnt;     // number of elements (0 = empty)
  int off;     // index of element 0 within the tile
};

struct PartInfo {
  int part;  // PART_*
  int s_local;
  int cp;
  const int2* blk;  // doc-zigzag: [cp][s_local / 64] block descriptors {start, cnt}
};

// Doc-zigzag block descriptor i, read through the constant address space: at a
// wave-uniform index this is a scalar load, waited for on the scalar/LDS
// counter, so the wait does not also drain the vector-memory loads in flight
// (the tile prefetch of the attention kernels). The table is never written
// while a kernel reads it.
__device__ __forceinline__ int2 blk_at(const int2* blk, int i) {
  const __attribute__((address_space(4))) int* c = (const __attribute__((address_space(4))) int*)blk;
  return make_int2(c[2 * i], c[2 * i + 1]);
}

// Global position of local index i of `owner` (-1: doc-zigzag padding).
__device__ __forceinline__ int pos_of(const PartInfo& p, int owner, int i) {
  if (p.part == PART_DOC_ZIGZAG) {
    const int2 b = blk_at(p.blk, owner * (p.s_local / kDocBlock) + i / kDocBlock);
    const int o = i % kDocBlock;
    return o < b.y ? b.x + o : -1;
  }
  if (p.part == PART_CONTIGUOUS) return owner * p.s_local + i;
  if (p.part == PART_STRIPED) return owner + p.cp * i;
  const int half = p.s_local >> 1;
  return i < half ? owner * half + i : (2 * p.cp - 1 - owner) * half + (i - half);
}

// Runs covering local indices [a, b) of `owner`, in two fixed slots (a slot
// with cnt == 0 is empty): slot 0 holds the contiguous / striped run or the
// part in the first zigzag half, slot 1 the part in the second zigzag half.
// Fixed slots keep both runs in registers (no dynamically indexed array).
__device__ __forceinline__ void runs_of(const PartInfo& p, int owner, int a, int b, Run& r0, Run& r1) {
  r0 = Run{0, 1, 0, 0};
  r1 = Run{0, 1, 0, 0};
  if (b <= a) return;
  if (p.part == PART_DOC_ZIGZAG) {  // [a, b) spans at most two blocks (aligned tiles of <= 128)
    const int nb = p.s_local / kDocBlock;
    const int A = a / kDocBlock, oa = a % kDocBlock, ea = (A + 1) * kDocBlock;
    const int2 ba = blk_at(p.blk, owner * nb + A);
    const int e0 = (b < ea ? b : ea) - A * kDocBlock;
    const int c0 = (e0 < ba.y ? e0 : ba.y) - oa;
    r0 = Run{ba.x + oa, 1, c0 > 0 ? c0 : 0, 0};
    if (b > ea) {
      const int2 bb = blk_at(p.blk, owner * nb + A + 1);
      const int c1 = b - ea < bb.y ? b - ea : bb.y;
      r1 = Run{bb.x, 1, c1 > 0 ? c1 : 0, ea - a};
    }
    return;
  }
  if (p.part == PART_CONTIGUOUS) {
    r0 = Run{owner * p.s_local + a, 1, b - a, 0};
    return;
  }
  if (p.part == PART_STRIPED) {
    r0 = Run{owner + p.cp * a, p.cp, b - a, 0};
    return;
  }
  const int half = p.s_local >> 1;
  if (a < half) {
    const int e = b < half ? b : half;
    r0 = Run{owner * half + a, 1, e - a, 0};
  }
  if (b > half) {
    const int s0 = a > half ? a : half;
    r1 = Run{(2 * p.cp - 1 - owner) * half + (s0 - half), 1, b - s0, s0 - a};
  }
}

// Document containing position p: largest j with cu[j] <= p (cu has n_docs+1 entries).
__device__ __forceinline__ int doc_of(const int* cu, int n_docs, int p) {
  int lo = 0, hi = n_docs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Visible key-position interval [lo, hi] of query position pq (empty for padding, pq < 0).
__device__ __forceinline__ void row_interval(const int* cu, int n_docs, int s_total, int causal, int pq,
                                             int& lo, int& hi) {
  if (pq < 0) {
    lo = 1;
    hi = 0;
    return;
  }
  if (n_docs <= 1) {
    lo = 0;
    hi = causal ? pq : s_total - 1;
    return;
  }
  const int d = doc_of(cu, n_docs, pq);
  lo = cu[d];
  hi = causal ? pq : cu[d + 1] - 1;
}

// Visible query-position interval [lo, hi] of key position pk: the queries of
// pk's document at or after pk (causal), or the whole document (non-causal).
// The same relation as row_interval, solved for the query.
__device__ __forceinline__ void key_interval(const int* cu, int n_docs, int s_total, int causal, int pk,
                                             int& lo, int& hi) {
  if (pk < 0) {
    lo = 1;
    hi = 0;
    return;
  }
  if (n_docs <= 1) {
    lo = causal ? pk : 0;
    hi = s_total - 1;
    return;
  }
  const int d = doc_of(cu, n_docs, pk);
  lo = causal ? pk : cu[d];
  hi = cu[d + 1] - 1;
}

// Indices n in [0, cnt) with A <= start + stride*n <= B, as [n0, n1] (empty if n0 > n1).
// Positions stay below 2^30, so 32-bit differences cannot overflow.
__device__ __forceinline__ void run_range(const Run& r, int A, int B, int& n0, int& n1) {
  if (r.cnt <= 0 || B < A || B < r.start) { n0 = 1; n1 = 0; return; }
  const int da = A - r.start;
  const int db = B - r.start;
  if (r.stride == 1) {
    n0 = da <= 0 ? 0 : da;
    n1 = db < r.cnt - 1 ? db : r.cnt - 1;
  } else {
    const unsigned st = (unsigned)r.stride;
    n0 = da <= 0 ? 0 : (int)(((unsigned)da + st - 1u) / st);
    const int nb = (int)((unsigned)db / st);
    n1 = nb < r.cnt - 1 ? nb : r.cnt - 1;
  }
}

__device__ __forceinline__ int doc_start_of(const int* cu, int n_docs, int p) {
  return n_docs <= 1 ? 0 : cu[doc_of(cu, n_docs, p)];
}
__device__ __forceinline__ int doc_end_of(const int* cu, int n_docs, int s_total, int p) {
  return n_docs <= 1 ? s_total : cu[doc_of(cu, n_docs, p) + 1];
}

// Exact class of the pairs (q in Q, k in K) for two runs.
__device__ inline int classify_runs(const Run& Q, const Run& K, const int* cu, int n_docs, int s_total,
                                    int causal) {
  if (Q.cnt <= 0 || K.cnt <= 0) return CLS_SKIP;
  const int qmin = Q.start, qmax = Q.start + Q.stride * (Q.cnt - 1);
  const int kmin = K.start, kmax = K.start + K.stride * (K.cnt - 1);
  // FULL: every k within [max_q lo(q), min_q hi(q)] = [docstart(qmax), hi(qmin)]
  const int lo_max = doc_start_of(cu, n_docs, qmax);
  const int hi_min = causal ? qmin : doc_end_of(cu, n_docs, s_total, qmin) - 1;
  if (kmin >= lo_max && kmax <= hi_min) return CLS_FULL;
  if (n_docs <= 1) return (!causal || kmin <= qmax) ? CLS_PARTIAL : CLS_SKIP;
  // Any visible pair: some document D holds q in Q and k in K (with k <= q if causal).
  const int dq0 = doc_of(cu, n_docs, qmin), dq1 = doc_of(cu, n_docs, qmax);
  const int dk0 = doc_of(cu, n_docs, kmin), dk1 = doc_of(cu, n_docs, kmax);
  const int d0 = dq0 > dk0 ? dq0 : dk0, d1 = dq1 < dk1 ? dq1 : dk1;
  for (int D = d0; D <= d1; ++D) {
    const int A = cu[D], B = cu[D + 1] - 1;
    int qn0, qn1, kn0, kn1;
    run_range(Q, A, B, qn0, qn1);
    if (qn0 > qn1) continue;
    run_range(K, A, B, kn0, kn1);
    if (kn0 > kn1) continue;
    if (!causal) return CLS_PARTIAL;
    if (K.start + K.stride * kn0 <= Q.start + Q.stride * qn1) return CLS_PARTIAL;
  }
  return CLS_SKIP;
}

// Class of the tile (query rows [qa, qb) of `rank`) x (keys [ka, kb) of `owner`).
__device__ inline int classify_tile(const PartInfo& p, int rank, int qa, int qb, int owner, int ka, int kb,
                                    const int* cu, int n_docs, int s_total, int causal) {
  Run q0, q1, k0, k1;
  runs_of(p, rank, qa, qb, q0, q1);
  runs_of(p, owner, ka, kb, k0, k1);
  bool any = false, all = true;
  auto pair = [&](const Run& q, const Run& k) {
    if (q.cnt <= 0 || k.cnt <= 0) return;
    const int c = classify_runs(q, k, cu, n_docs, s_total, causal);
    any |= c != CLS_SKIP;
    all &= c == CLS_FULL;
  };
  pair(q0, k0);
  pair(q0, k1);
  pair(q1, k0);
  pair(q1, k1);
  if (!any) return CLS_SKIP;
  // a tile whose runs miss some of its indices (doc-zigzag padding) is never FULL
  const bool covered = q0.cnt + q1.cnt == qb - qa && k0.cnt + k1.cnt == kb - ka;
  return all && covered ? CLS_FULL : CLS_PARTIAL;
}

// Arguments of the attention kernels (one rank, all ring steps).
struct AttnArgs {
  const void* q;      // [S_l][hq][d]
  const void* k;      // [cp][S_l][hkv][d]
  const void* v;      // [cp][S_l][hkv][d]
  void* out;          // [S_l][hq][d] (fused mode)
  float* lse;         // [hq][S_l]    (fused mode)
  float* o_steps;     // [cp][S_l][hq][d] (steps mode)
  float* lse_steps;   // [cp][hq][S_l]    (steps mode)
  const int* cu;      // device cu_seqlens [n_docs+1] (unused when n_docs <= 1)
  const int2* blk;    // doc-zigzag block descriptors (else unused)
  const int* wl;      // work list [nqt][wl_stride]
  const int* wl_count;  // [nqt]
  const int* order;   // [nqt] query tiles, heaviest first
  int n_docs;
  int s_total;
  int s_local;
  int cp;
  int rank;
  int part;
  int causal;
  int hq;
  int hkv;
  int nqt;
  int nkt;
  int wl_stride;
  float scale_log2;   // softmax_scale * log2(e)
};

// Arguments of the backward kernels (one rank, all ring steps).
struct BwdArgs {
  const void* q;       // [S_l][hq][d]
  const void* k;       // [cp][S_l][hkv][d]
  const void* v;       // [cp][S_l][hkv][d]
  const void* dout;    // [S_l][hq][d], same dtype as q
  const float* lse;    // [hq][S_l] natural log, softmax over all ring steps
  const float* dsum;   // [hq][S_l] sum_c dout * out per row
  float* dq;           // [S_l][hq][d]
  float* dk;           // [cp][S_l][hkv][d]
  float* dv;           // [cp][S_l][hkv][d]
  const int* cu;       // device cu_seqlens [n_docs+1] (unused when n_docs <= 1)
  const int2* blk;     // doc-zigzag block descriptors (else unused)
  const int* wl;       // dQ kernel: the forward's work list [nqt][wl_stride]
  const int* wl_count;
  const int* order;
  const int* kwl;      // dK/dV kernel: per key tile, the non-SKIP query tiles [cp*nkt_kv][kwl_stride]
  const int* kwl_count;
  const int* korder;   // key tiles, heaviest first
  int n_docs;
  int s_total;
  int s_local;
  int cp;
  int rank;
  int part;
  int causal;
  int hq;
  int hkv;
  int nqt;
  int nkt;
  int wl_stride;
  int nkt_kv;          // key tiles per chunk (dK/dV kernel)
  int nqt_kv;          // query tiles (dK/dV kernel)
  int kwl_stride;
  float scale;         // softmax_scale
  float scale_log2;    // softmax_scale * log2(e)
};

}  // namespace ra
