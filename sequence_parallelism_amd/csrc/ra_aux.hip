// Auxiliary kernels: cu_seqlens upload, work-list construction and ordering,
// tile classification, the standalone fp32 LSE merge, and the two local
// permutation copies (CP reorder and Ulysses sequence<->head transpose).
#include "ra_common.h"
#include "ra_internal.h"

namespace ra {

// ---------------------------------------------------------------------------
// cu_seqlens upload through kernel arguments (no host staging buffer, so the
// host array may be freed as soon as the call returns).
// ---------------------------------------------------------------------------
struct CuChunk {
  int n;
  int v[kCuChunk];
};

__global__ void __launch_bounds__(256) upload_i32_kernel(const CuChunk c, int32_t* dst) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < c.n) dst[i] = c.v[i];
}

hipError_t launch_upload_i32(const int32_t* host, int n, int32_t* dst, hipStream_t st) {
  for (int off = 0; off < n; off += kCuChunk) {
    CuChunk c;
    c.n = n - off < kCuChunk ? n - off : kCuChunk;
    for (int i = 0; i < c.n; ++i) c.v[i] = host[off + i];
    hipLaunchKernelGGL(upload_i32_kernel, dim3((c.n + 255) / 256), dim3(256), 0, st, c, dst + off);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Work list: for query tile I, every (ring step t, key tile J) whose class is
// not SKIP, in step-major order, packed with its class. One block per tile.
// A tile is FULL when all its 128-row parts are, SKIP when all are.
// ---------------------------------------------------------------------------
struct WlArgs {
  const int* cu;
  const int2* blk;
  int n_docs, s_total, s_local, cp, rank, part, causal, bm, bn, nqt, nkt, wl_stride;
  int* wl;
  int* wl_count;
};

// 1024 threads per tile: each classification is a chain of dependent loads
// (block descriptors, document bounds), so the more of them in flight the better.
constexpr int kWlThreads = 1024, kWlWaves = kWlThreads / 64;
__global__ void __launch_bounds__(kWlThreads) worklist_kernel(const WlArgs w) {
  __shared__ int wave_tot[kWlWaves];
  const int I = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PartInfo p{w.part, w.s_local, w.cp, w.blk};
  const int qa = I * w.bm;
  const int qb = qa + w.bm < w.s_local ? qa + w.bm : w.s_local;
  const int nent = w.cp * w.nkt;
  int* out = w.wl + (size_t)I * w.wl_stride;
  int base = 0;
  for (int e0 = 0; e0 < nent; e0 += kWlThreads) {
    const int e = e0 + tid;
    int c = CLS_SKIP, t = 0, J = 0;
    if (e < nent) {
      t = e / w.nkt;
      J = e - t * w.nkt;
      const int owner = (w.rank - t + w.cp) % w.cp;
      const int ka = J * w.bn;
      const int kb = ka + w.bn < w.s_local ? ka + w.bn : w.s_local;
      // tiles taller than 128 rows: merge the classes of their 128-row parts (a
      // part's rows form at most two runs under every partition)
      bool any = false, all = true;
      for (int pa = qa; pa < qb; pa += 128) {
        const int pb = pa + 128 < qb ? pa + 128 : qb;
        const int cp = classify_tile(p, w.rank, pa, pb, owner, ka, kb, w.cu, w.n_docs, w.s_total, w.causal);
        any |= cp != CLS_SKIP;
        all &= cp == CLS_FULL;
      }
      c = !any ? CLS_SKIP : all ? CLS_FULL : CLS_PARTIAL;
    }
    const unsigned long long bal = __ballot(c != CLS_SKIP);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    // prefix over the waves' counts: lane i of every wave holds the sum of waves 0..i
    int inc = lane < kWlWaves ? wave_tot[lane] : 0;
#pragma unroll
    for (int o = 1; o < kWlWaves; o <<= 1) {
      const int up = __shfl_up(inc, o, 64);
      inc += lane >= o ? up : 0;
    }
    const int total = __shfl(inc, kWlWaves - 1, 64);
    const int before = wave > 0 ? __shfl(inc, wave - 1, 64) : 0;
    if (c != CLS_SKIP) out[base + before + below] = wl_pack(t, J, c);
    base += total;
    __syncthreads();
  }
  if (tid == 0) w.wl_count[I] = base;
}

// Orders query tiles by descending work (entry count), ties by index, so that
// the longest workgroups start first.
__global__ void __launch_bounds__(1024) order_kernel(const int* count, int nqt, int* order) {
  __shared__ int sc[8192];
  const bool staged = nqt <= 8192;
  if (staged)
    for (int i = threadIdx.x; i < nqt; i += 1024) sc[i] = count[i];
  __syncthreads();
  for (int i = threadIdx.x; i < nqt; i += 1024) {
    const int wi = staged ? sc[i] : count[i];
    int r = 0;
    for (int j = 0; j < nqt; ++j) {
      const int wj = staged ? sc[j] : count[j];
      r += (wj > wi) || (wj == wi && j < i);
    }
    order[r] = i;
  }
}

hipError_t launch_worklist(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                           int part, int causal, int bm, int bn, int nqt, int nkt, int wl_stride, int* wl,
                           int* wl_count, int* order, hipStream_t st) {
  if (nqt == 0) return hipSuccess;
  WlArgs w{cu, blk, n_docs, s_total, s_local, cp, rank, part, causal, bm, bn, nqt, nkt, wl_stride, wl, wl_count};
  hipLaunchKernelGGL(worklist_kernel, dim3(nqt), dim3(kWlThreads), 0, st, w);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_order(wl_count, nqt, order, st);
}

hipError_t launch_order(const int* count, int n, int* order, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, st, count, n, order);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Doc-zigzag block descriptors. Document j (length L) is cut into 2cp pieces at
// the bounds k L / 2cp rounded to the nearest multiple of kDocGranule (halves
// up, capped at L); rank r holds, document after document, piece p = (r + j)
// mod cp and then piece 2cp-1-p, each padded to whole granules, real tokens
// first. prefix[r][j] counts the 64-slot blocks rank r holds before document j.
// ---------------------------------------------------------------------------
__device__ __forceinline__ long long doc_bound(long long L, int cp, int k) {
  const long long n = 2 * cp;
  if (k >= n) return L;
  const long long b = kDocGranule * ((2 * k * L + n * kDocGranule) / (2 * n * kDocGranule));
  return b < L ? b : L;
}

__device__ __forceinline__ int granule_blocks(long long len) {
  return (int)((len + kDocGranule - 1) / kDocGranule) * (kDocGranule / kDocBlock);
}

// One workgroup per rank: blocks of every document, scanned in chunks of 256.
__global__ void __launch_bounds__(256) doc_prefix_kernel(const int* cu, int n_docs, int cp, int* prefix) {
  __shared__ int part[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  int* pr = prefix + (size_t)r * (n_docs + 1);
  if (tid == 0) pr[0] = 0;
  int carry = 0;
  for (int j0 = 0; j0 < n_docs; j0 += 256) {
    const int j = j0 + tid;
    int nb = 0;
    if (j < n_docs) {
      const long long L = cu[j + 1] - cu[j];
      const int p = (int)((r + (long long)j) % cp), q = 2 * cp - 1 - p;
      nb = granule_blocks(doc_bound(L, cp, p + 1) - doc_bound(L, cp, p)) +
           granule_blocks(doc_bound(L, cp, q + 1) - doc_bound(L, cp, q));
    }
    part[tid] = nb;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan (Hillis-Steele)
      const int add = tid >= o ? part[tid - o] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (j < n_docs) pr[j + 1] = carry + part[tid];
    carry += part[255];
    __syncthreads();
  }
}

// One thread per (rank, block): the document by binary search in the rank's
// prefix, then the piece and the block's offset in it.
__global__ void __launch_bounds__(256) doc_blocks_kernel(const int* cu, const int* prefix, int n_docs, int cp,
                                                         int nblk, int2* blk) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= cp * nblk) return;
  const int r = idx / nblk, b = idx - r * nblk;
  const int* pr = prefix + (size_t)r * (n_docs + 1);
  if (b >= pr[n_docs]) {  // the rank's end padding
    blk[idx] = make_int2(0, 0);
    return;
  }
  int lo = 0, hi = n_docs - 1;  // document: smallest j with pr[j + 1] > b
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pr[mid + 1] > b) hi = mid; else lo = mid + 1;
  }
  const int j = lo;
  const long long L = cu[j + 1] - cu[j];
  const int p = (int)((r + (long long)j) % cp), q = 2 * cp - 1 - p;
  const long long p0 = doc_bound(L, cp, p), p1 = doc_bound(L, cp, p + 1);
  const int first_blocks = granule_blocks(p1 - p0);
  int lb = b - pr[j];
  long long start = p0, len = p1 - p0;
  if (lb >= first_blocks) {
    lb -= first_blocks;
    start = doc_bound(L, cp, q);
    len = doc_bound(L, cp, q + 1) - start;
  }
  long long cnt = len - (long long)lb * kDocBlock;
  cnt = cnt < 0 ? 0 : (cnt > kDocBlock ? kDocBlock : cnt);
  blk[idx] = make_int2(cu[j] + (int)start + lb * kDocBlock, (int)cnt);
}

hipError_t launch_doc_blocks(const int* cu, int* prefix, int n_docs, int cp, int nblk, int2* blk, hipStream_t st) {
  hipLaunchKernelGGL(doc_prefix_kernel, dim3(cp), dim3(256), 0, st, cu, n_docs, cp, prefix);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long n = (long long)cp * nblk;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(doc_blocks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, cu, prefix, n_docs, cp,
                     nblk, blk);
  return hipGetLastError();
}

// Doc-zigzag reorder, one wave per row of the rank-major layout R = (rank, slot),
// whose global row comes from the block descriptors. Forward: row R takes that
// global row, or zeros for padding. Inverse: the global row takes row R (every
// real token is held by exactly one slot, so every output row is written once).
struct DocCopyArgs {
  const void* in;
  void* out;
  long long nrows;   // rank-major rows: cp * s_local
  long long cpr;     // chunks per row
  int s_local;
  const int2* blk;
};

__device__ __forceinline__ long long doc_global_row(const DocCopyArgs& c, long long R) {
  const int r = (int)(R / c.s_local), i = (int)(R - (long long)r * c.s_local);
  const int2 b = c.blk[r * (c.s_local / kDocBlock) + i / kDocBlock];
  const int o = i % kDocBlock;
  return o < b.y ? (long long)(b.x + o) : -1;
}

template <typename T, bool INVERSE>
__global__ void __launch_bounds__(256) copy_doc_rows_kernel(const DocCopyArgs c) {
  const int lane = threadIdx.x & 63;
  const long long nw = (long long)gridDim.x * 4;
  for (long long R = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); R < c.nrows; R += nw) {
    const long long G = doc_global_row(c, R);
    if (INVERSE && G < 0) continue;  // padding slot: nothing to put back
    T* dst = (T*)c.out + (INVERSE ? G : R) * c.cpr;
    if (G < 0) {
      for (long long i = lane; i < c.cpr; i += 64) dst[i] = T{};
      continue;
    }
    const T* src = (const T*)c.in + (INVERSE ? R : G) * c.cpr;
    long long i = lane;
    for (; i + 192 < c.cpr; i += 256) {
      const T a0 = src[i], a1 = src[i + 64], a2 = src[i + 128], a3 = src[i + 192];
      dst[i] = a0;
      dst[i + 64] = a1;
      dst[i + 128] = a2;
      dst[i + 192] = a3;
    }
    for (; i < c.cpr; i += 64) dst[i] = src[i];
  }
}

// 16-byte-aligned rows of a power-of-two number of chunks: the rank-major side is
// walked as one flat array of 16-byte chunks (the destination of the forward, the
// source of the inverse), each thread keeping kDocUnroll nontemporal loads in
// flight, as the other permutations do; a chunk's row maps through its block
// descriptor, and padding slots read as zeros (forward) or are skipped (inverse).
constexpr int kDocUnroll = 4;

template <bool INVERSE>
__global__ void __launch_bounds__(256) copy_doc_pow2_kernel(const DocCopyArgs c, int log2_cpr) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  const u4* src = (const u4*)c.in;
  u4* dst = (u4*)c.out;
  const long long total = c.nrows << log2_cpr;
  const long long cmask = (1ll << log2_cpr) - 1;
  const long long step = (long long)gridDim.x * 256 * kDocUnroll;
  for (long long base = (long long)blockIdx.x * 256 * kDocUnroll + threadIdx.x; base < total; base += step) {
    u4 v[kDocUnroll];
    long long g[kDocUnroll];
#pragma unroll
    for (int u = 0; u < kDocUnroll; ++u) {
      const long long idx = base + u * 256;
      g[u] = -1;
      v[u] = u4{0u, 0u, 0u, 0u};
      if (idx < total) {
        g[u] = doc_global_row(c, idx >> log2_cpr);
        if (INVERSE) {
          v[u] = __builtin_nontemporal_load(src + idx);
        } else if (g[u] >= 0) {
          v[u] = __builtin_nontemporal_load(src + ((g[u] << log2_cpr) | (idx & cmask)));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDocUnroll; ++u) {
      const long long idx = base + u * 256;
      if (idx < total) {
        if (!INVERSE) {
          dst[idx] = v[u];
        } else if (g[u] >= 0) {
          dst[(g[u] << log2_cpr) | (idx & cmask)] = v[u];
        }
      }
    }
  }
}

template <bool INVERSE>
static hipError_t launch_doc_copy(DocCopyArgs c, long long row_bytes, hipStream_t st) {
  if (c.nrows == 0 || row_bytes == 0) return hipSuccess;
  {
    const uintptr_t al = (uintptr_t)c.in | (uintptr_t)c.out | (uintptr_t)row_bytes;
    const long long cpr16 = row_bytes / 16;
    if (al % 16 == 0 && cpr16 <= 1024 && (cpr16 & (cpr16 - 1)) == 0) {
      int lg = 0;
      while ((1ll << lg) < cpr16) ++lg;
      long long blocks = ((c.nrows << lg) + 256 * kDocUnroll - 1) / (256 * kDocUnroll);
      if (blocks > 65536) blocks = 65536;
      c.cpr = cpr16;
      hipLaunchKernelGGL((copy_doc_pow2_kernel<INVERSE>), dim3((unsigned)blocks), dim3(256), 0, st, c, lg);
      return hipGetLastError();
    }
  }
  long long blocks = (c.nrows + 3) / 4;
  if (blocks > 65536) blocks = 65536;
  const uintptr_t al = (uintptr_t)c.in | (uintptr_t)c.out | (uintptr_t)row_bytes;
  const dim3 grid((unsigned)blocks), block(256);
  if (al % 16 == 0) {
    c.cpr = row_bytes / 16;
    hipLaunchKernelGGL((copy_doc_rows_kernel<uint4, INVERSE>), grid, block, 0, st, c);
  } else if (al % 4 == 0) {
    c.cpr = row_bytes / 4;
    hipLaunchKernelGGL((copy_doc_rows_kernel<uint32_t, INVERSE>), grid, block, 0, st, c);
  } else {
    c.cpr = row_bytes;
    hipLaunchKernelGGL((copy_doc_rows_kernel<uint8_t, INVERSE>), grid, block, 0, st, c);
  }
  return hipGetLastError();
}

hipError_t launch_cp_reorder_docs(const void* in, void* out, int64_t row_bytes, int cp, int s_local, const int2* blk,
                                  int inverse, hipStream_t st) {
  DocCopyArgs c{in, out, (long long)cp * s_local, 0, s_local, blk};
  return inverse ? launch_doc_copy<true>(c, row_bytes, st) : launch_doc_copy<false>(c, row_bytes, st);
}

// ---------------------------------------------------------------------------
// Public tile classification: one thread per (step, query tile, key tile).
// ---------------------------------------------------------------------------
struct ClsArgs {
  const int* cu;
  const int2* blk;
  int n_docs, s_total, s_local, cp, rank, part, causal, bm, bn, nqt, nkt;
  int8_t* cls;
};

__global__ void __launch_bounds__(256) classify_kernel(const ClsArgs c) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per_step = (long long)c.nqt * c.nkt;
  if (idx >= per_step * c.cp) return;
  const int t = (int)(idx / per_step);
  const long long rem = idx - t * per_step;
  const int I = (int)(rem / c.nkt), J = (int)(rem - (long long)I * c.nkt);
  const PartInfo p{c.part, c.s_local, c.cp, c.blk};
  const int owner = (c.rank - t + c.cp) % c.cp;
  const int qa = I * c.bm, qb = qa + c.bm < c.s_local ? qa + c.bm : c.s_local;
  const int ka = J * c.bn, kb = ka + c.bn < c.s_local ? ka + c.bn : c.s_local;
  c.cls[idx] = (int8_t)classify_tile(p, c.rank, qa, qb, owner, ka, kb, c.cu, c.n_docs, c.s_total, c.causal);
}

hipError_t launch_classify(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                           int part, int causal, int bm, int bn, int nqt, int nkt, int8_t* cls, hipStream_t st) {
  const long long total = (long long)cp * nqt * nkt;
  if (total == 0) return hipSuccess;
  ClsArgs c{cu, blk, n_docs, s_total, s_local, cp, rank, part, causal, bm, bn, nqt, nkt, cls};
  hipLaunchKernelGGL(classify_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, c);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// fp32 LSE merge: LSE = ln(e^a + e^b), O = e^(a-LSE) O_a + e^(b-LSE) O_b.
// A group of d/4 lanes (inside one wave) serves one (row, head): every lane of
// the group reads both LSE values before any lane writes, so in-place calls
// (o_out == o_a, lse_out == lse_a) are safe.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void merge_weights(float la, float lb, float& wa, float& wb, float& lse) {
  const float mx = fmaxf(la, lb);
  if (mx == -INFINITY) {
    wa = 0.f;
    wb = 0.f;
    lse = -INFINITY;
    return;
  }
  lse = mx + logf(expf(la - mx) + expf(lb - mx));
  wa = expf(la - lse);
  wb = expf(lb - lse);
}

// Four 16-byte chunks per thread: a block covers 4 consecutive spans of 256
// chunks, and every load is issued (nontemporal) before the first store, so
// that 8 loads per thread are in flight. A (row, head) pair's d/4 lanes sit in
// one wave for each span, so in-place merges stay safe.
typedef float mf32x4 __attribute__((ext_vector_type(4)));
constexpr int kMergeChunks = 4;
__global__ void __launch_bounds__(256) lse_merge_vec4_kernel(long long rows, int h, int d, const float* o_a,
                                                             const float* lse_a, const float* o_b, const float* lse_b,
                                                             float* o_out, float* lse_out, long long chunks) {
  const int per = d >> 2;  // lanes per (row, head): a power of two <= 64
  const long long c0 = (long long)blockIdx.x * (256 * kMergeChunks) + threadIdx.x;
  mf32x4 a[kMergeChunks], b[kMergeChunks];
  float la[kMergeChunks], lb[kMergeChunks];
  size_t li[kMergeChunks];
#pragma unroll
  for (int k = 0; k < kMergeChunks; ++k) {
    const long long c = c0 + 256 * k;
    const long long cc = c < chunks ? c : chunks - 1;  // past the end: a valid chunk, never stored
    const long long pair = cc / per;
    const long long row = pair / h;
    li[k] = (size_t)(pair - row * h) * rows + row;
    la[k] = lse_a[li[k]];
    lb[k] = lse_b[li[k]];
    a[k] = __builtin_nontemporal_load((const mf32x4*)o_a + cc);
    b[k] = __builtin_nontemporal_load((const mf32x4*)o_b + cc);
  }
#pragma unroll
  for (int k = 0; k < kMergeChunks; ++k) {
    const long long c = c0 + 256 * k;
    if (c >= chunks) continue;
    float wa, wb, lse;
    merge_weights(la[k], lb[k], wa, wb, lse);
    __builtin_nontemporal_store(wa * a[k] + wb * b[k], (mf32x4*)o_out + c);
    if ((c & (per - 1)) == 0) lse_out[li[k]] = lse;
  }
}


__global__ void __launch_bounds__(256) lse_merge_scalar_kernel(long long rows, int h, int d, const float* o_a,
                                                               const float* lse_a, const float* o_b,
                                                               const float* lse_b, float* o_out, float* lse_out) {
  const long long pair = (long long)blockIdx.x * 256 + threadIdx.x;
  if (pair >= rows * h) return;
  const long long row = pair / h;
  const int hh = (int)(pair - row * h);
  const size_t li = (size_t)hh * rows + row;
  float wa, wb, lse;
  merge_weights(lse_a[li], lse_b[li], wa, wb, lse);
  for (int c = 0; c < d; ++c) {
    const size_t oi = (size_t)pair * d + c;
    o_out[oi] = wa * o_a[oi] + wb * o_b[oi];
  }
  lse_out[li] = lse;
}

hipError_t launch_lse_merge(int64_t rows, int h, int d, const float* o_a, const float* lse_a, const float* o_b,
                            const float* lse_b, float* o_out, float* lse_out, hipStream_t st) {
  const long long pairs = (long long)rows * h;
  if (pairs == 0) return hipSuccess;
  const int per = d / 4;
  const bool vec = d % 4 == 0 && per <= 64 && (per & (per - 1)) == 0 &&
                   ((uintptr_t)o_a | (uintptr_t)o_b | (uintptr_t)o_out) % 16 == 0;
  if (vec) {
    const long long chunks = pairs * per;
    const long long blocks = (chunks + 256 * kMergeChunks - 1) / (256 * kMergeChunks);
    hipLaunchKernelGGL(lse_merge_vec4_kernel, dim3((unsigned)blocks), dim3(256), 0, st, rows, h, d, o_a, lse_a, o_b,
                       lse_b, o_out, lse_out, chunks);
  } else {
    hipLaunchKernelGGL(lse_merge_scalar_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, st, rows, h, d,
                       o_a, lse_a, o_b, lse_b, o_out, lse_out);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-gather copies. Destination row R (cpr chunks of sizeof(T) bytes) is
// copied from source row src_row(R). One wave per row; lanes stride the row.
// ---------------------------------------------------------------------------
enum { MAP_REORDER_FWD = 0, MAP_REORDER_INV = 1, MAP_ULY_FWD = 2, MAP_ULY_INV = 3 };

struct CopyArgs {
  const void* in;
  void* out;
  long long nrows;
  long long cpr;  // chunks per row
  int s_local;    // CP reorder: tokens per rank; Ulysses: tokens per simulated rank
  int cp;         // CP reorder: cp size; Ulysses: n
  int part;
  long long bstride;  // Ulysses: runs between the n blocks of the head-split side (n s_local if packed)
};

template <int KIND>
__device__ __forceinline__ long long src_row(const CopyArgs& c, long long R) {
  if constexpr (KIND == MAP_REORDER_FWD) {
    const int r = (int)(R / c.s_local), i = (int)(R - (long long)r * c.s_local);
    return pos_of(PartInfo{c.part, c.s_local, c.cp, nullptr}, r, i);
  } else if constexpr (KIND == MAP_REORDER_INV) {
    const int p = (int)R;
    int r, i;
    if (c.part == PART_CONTIGUOUS) {
      r = p / c.s_local;
      i = p - r * c.s_local;
    } else if (c.part == PART_STRIPED) {
      r = p % c.cp;
      i = p / c.cp;
    } else {
      const int half = c.s_local >> 1;
      const int ch = p / half, off = p - ch * half;
      if (ch < c.cp) {
        r = ch;
        i = off;
      } else {
        r = 2 * c.cp - 1 - ch;
        i = half + off;
      }
    }
    return (long long)r * c.s_local + i;
  } else if constexpr (KIND == MAP_ULY_FWD) {
    // dst run (rho, j*s_local + i) <- src run ((j*s_local + i), rho); R counts packed dst runs
    const long long T = (long long)c.cp * c.s_local;
    const long long rho = R / T, tok = R - rho * T;
    return tok * c.cp + rho;
  } else {
    // dst run ((j*s_local + i), rho) <- src run (rho, j*s_local + i), head-split blocks bstride apart
    const long long tok = R / c.cp, rho = R - tok * c.cp;
    return rho * c.bstride + tok;
  }
}

// Destination run of packed destination index R (the Ulysses forward writes its
// head-split blocks bstride runs apart; every other map is packed).
template <int KIND>
__device__ __forceinline__ long long dst_row(const CopyArgs& c, long long R) {
  if constexpr (KIND == MAP_ULY_FWD) {
    const long long T = (long long)c.cp * c.s_local;
    const long long rho = R / T;
    return rho * c.bstride + (R - rho * T);
  } else {
    return R;
  }
}

template <typename T, int KIND>
__global__ void __launch_bounds__(256) copy_rows_kernel(const CopyArgs c) {
  const int lane = threadIdx.x & 63;
  const long long nw = (long long)gridDim.x * 4;
  for (long long R = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); R < c.nrows; R += nw) {
    const long long S = src_row<KIND>(c, R);
    const T* src = (const T*)c.in + S * c.cpr;
    T* dst = (T*)c.out + dst_row<KIND>(c, R) * c.cpr;
    long long i = lane;
    for (; i + 192 < c.cpr; i += 256) {
      const T a0 = src[i], a1 = src[i + 64], a2 = src[i + 128], a3 = src[i + 192];
      dst[i] = a0;
      dst[i + 64] = a1;
      dst[i + 128] = a2;
      dst[i + 192] = a3;
    }
    for (; i < c.cpr; i += 64) dst[i] = src[i];
  }
}

// 16-byte chunks, rows of a power-of-two number of chunks (at most 1024): the
// destination is walked as one flat array of chunks, each thread keeping
// kCopyUnroll loads in flight; row and column come from shifts.
// Loads are nontemporal, stores ordinary: on MI355X, with the cache flushed
// before each launch, ordinary stores copy 3-5 % faster than nontemporal ones
// (Ulysses forward 6.46 against 6.18 TB/s, same process); the LSE merge, which
// reads two inputs per output, keeps nontemporal stores (5.87 against 6.01).
constexpr int kCopyUnroll = 4;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// SCATTER: walk the source in order and send row R to destination row map(R)
// (map is then the inverse permutation); otherwise walk the destination and
// gather destination row R from source row map(R).
template <int KIND, bool SCATTER>
__global__ void __launch_bounds__(256) copy_rows_pow2_kernel(const CopyArgs c, int log2_cpr) {
  const u32x4* src = (const u32x4*)c.in;
  u32x4* dst = (u32x4*)c.out;
  const long long total = c.nrows << log2_cpr;
  const long long cmask = (1ll << log2_cpr) - 1;
  const long long step = (long long)gridDim.x * 256 * kCopyUnroll;
  for (long long base = (long long)blockIdx.x * 256 * kCopyUnroll + threadIdx.x; base < total; base += step) {
    u32x4 v[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const long long idx = base + u * 256;
      if (idx < total) {
        if constexpr (SCATTER) {
          v[u] = __builtin_nontemporal_load(src + idx);
        } else {
          const long long R = idx >> log2_cpr;
          v[u] = __builtin_nontemporal_load(src + ((src_row<KIND>(c, R) << log2_cpr) | (idx & cmask)));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const long long idx = base + u * 256;
      if (idx < total) {
        if constexpr (SCATTER) {
          const long long R = idx >> log2_cpr;
          dst[(src_row<KIND>(c, R) << log2_cpr) | (idx & cmask)] = v[u];
        } else {
          const long long R = idx >> log2_cpr;
          dst[(dst_row<KIND>(c, R) << log2_cpr) | (idx & cmask)] = v[u];
        }
      }
    }
  }
}

// Strided transpose of runs, dst run (rho * bstride + tok) <- src run (tok * n + rho)
// for tok < nrows / n and rho < n: the Ulysses forward (runs of hq / n heads, tokens
// of all n source ranks) and the striped CP reorder (runs are rows, rho the rank).
// For runs of at most 8 KiB: one block per (group of G consecutive tokens, rho),
// rho varying fastest across blocks. A block reads the G runs (tok, rho) of the
// source -- n runs apart -- and writes them as one contiguous 8 KiB piece, so the
// blocks in flight write n sequential streams and read one. Two 16-byte chunks
// per thread; loads nontemporal, stores ordinary (as in copy_rows_pow2_kernel).
constexpr int kUlyChunks = 512;
__global__ void __launch_bounds__(256) ulysses_fwd_kernel(const CopyArgs c, int log2_cpr) {
  constexpr int U = kUlyChunks / 256;
  const u32x4* src = (const u32x4*)c.in;
  u32x4* dst = (u32x4*)c.out;
  const int n = c.cp;
  const long long ntok = c.nrows / n;
  const int G = kUlyChunks >> log2_cpr;
  const long long cmask = (1ll << log2_cpr) - 1;
  const long long rho = blockIdx.x % n;
  const long long tok0 = (long long)(blockIdx.x / n) * G;
  u32x4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = threadIdx.x + 256 * u;
    const long long tok = tok0 + (q >> log2_cpr);
    if (tok < ntok) v[u] = __builtin_nontemporal_load(src + (((tok * n + rho) << log2_cpr) | (q & cmask)));
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int q = threadIdx.x + 256 * u;
    const long long tok = tok0 + (q >> log2_cpr);
    if (tok < ntok) dst[((rho * c.bstride + tok) << log2_cpr) | (q & cmask)] = v[u];
  }
}

template <int KIND, bool SCATTER = false>
static hipError_t launch_copy(const void* in, void* out, long long nrows, long long row_bytes, int s_local, int cp,
                              int part, hipStream_t st, long long bstride = 0) {
  if (nrows == 0 || row_bytes == 0) return hipSuccess;
  const uintptr_t al = (uintptr_t)in | (uintptr_t)out | (uintptr_t)row_bytes;
  const long long cpr16 = row_bytes / 16;
  if (al % 16 == 0 && cpr16 <= 1024 && (cpr16 & (cpr16 - 1)) == 0) {
    int lg = 0;
    while ((1ll << lg) < cpr16) ++lg;
    const long long chunks = nrows * cpr16;
    long long blocks = (chunks + 256 * kCopyUnroll - 1) / (256 * kCopyUnroll);
    if (blocks > 65536) blocks = 65536;
    CopyArgs c{in, out, nrows, cpr16, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_pow2_kernel<KIND, SCATTER>), dim3((unsigned)blocks), dim3(256), 0, st, c, lg);
    return hipGetLastError();
  }
  if constexpr (SCATTER) return hipErrorInvalidValue;  // scatter walks exist only for the 16-byte path
  long long blocks = (nrows + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid((unsigned)blocks), block(256);
  if (al % 16 == 0) {
    CopyArgs c{in, out, nrows, row_bytes / 16, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_kernel<uint4, KIND>), grid, block, 0, st, c);
  } else if (al % 8 == 0) {
    CopyArgs c{in, out, nrows, row_bytes / 8, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_kernel<uint2, KIND>), grid, block, 0, st, c);
  } else if (al % 4 == 0) {
    CopyArgs c{in, out, nrows, row_bytes / 4, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_kernel<uint32_t, KIND>), grid, block, 0, st, c);
  } else if (al % 2 == 0) {
    CopyArgs c{in, out, nrows, row_bytes / 2, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_kernel<uint16_t, KIND>), grid, block, 0, st, c);
  } else {
    CopyArgs c{in, out, nrows, row_bytes, s_local, cp, part, bstride};
    hipLaunchKernelGGL((copy_rows_kernel<uint8_t, KIND>), grid, block, 0, st, c);
  }
  return hipGetLastError();
}

// The strided transpose above for 16-byte-aligned power-of-two runs of at most 8 KiB
// (nruns = n * tokens); false when the runs do not fit it.
static bool launch_strided_transpose(const void* in, void* out, long long nruns, long long run_bytes, int n,
                                     long long bstride, hipStream_t st, hipError_t& err) {
  const uintptr_t al = (uintptr_t)in | (uintptr_t)out | (uintptr_t)run_bytes;
  const long long cpr16 = run_bytes / 16;
  if (al % 16 != 0 || cpr16 < 1 || cpr16 > kUlyChunks || (cpr16 & (cpr16 - 1)) != 0 || nruns <= 0) return false;
  int lg = 0;
  while ((1ll << lg) < cpr16) ++lg;
  const long long G = kUlyChunks / cpr16, ntok = nruns / n;
  const long long blocks = ((ntok + G - 1) / G) * n;
  if (blocks > 0x7fffffffLL) {
    err = hipErrorInvalidValue;
    return true;
  }
  CopyArgs c{in, out, nruns, cpr16, 0, n, 0, bstride};
  hipLaunchKernelGGL(ulysses_fwd_kernel, dim3((unsigned)blocks), dim3(256), 0, st, c, lg);
  err = hipGetLastError();
  return true;
}

hipError_t launch_cp_reorder(const void* in, void* out, int64_t s, int64_t row_bytes, int cp, int part, int inverse,
                             hipStream_t st) {
  const int s_local = (int)(s / cp);
  if (inverse) return launch_copy<MAP_REORDER_INV>(in, out, s, row_bytes, s_local, cp, part, st);
  // striped: rank r's row i is global row i cp + r, the strided transpose with n = cp
  hipError_t e;
  if (part == PART_STRIPED && launch_strided_transpose(in, out, s, row_bytes, cp, s_local, st, e)) return e;
  return launch_copy<MAP_REORDER_FWD>(in, out, s, row_bytes, s_local, cp, part, st);
}

hipError_t launch_ulysses(const void* in, void* out, int n, int64_t s_local, int64_t run_bytes, int inverse,
                          int64_t block_runs, hipStream_t st) {
  const long long runs = (long long)n * n * s_local;
  if (inverse) return launch_copy<MAP_ULY_INV>(in, out, runs, run_bytes, (int)s_local, n, 0, st, block_runs);
  // forward: 16-byte-aligned power-of-two runs of at most 8 KiB take the blocked walk
  // (contiguous 8 KiB writes per block, head block fastest across blocks); runs of up
  // to 16 KiB walk the source in order and scatter; anything else gathers row by row
  hipError_t e;
  if (launch_strided_transpose(in, out, runs, run_bytes, n, block_runs, st, e)) return e;
  const uintptr_t al = (uintptr_t)in | (uintptr_t)out | (uintptr_t)run_bytes;
  const long long cpr16 = run_bytes / 16;
  const bool pow2 = al % 16 == 0 && cpr16 >= 1 && (cpr16 & (cpr16 - 1)) == 0;
  if (pow2 && cpr16 <= 1024)
    return launch_copy<MAP_ULY_INV, true>(in, out, runs, run_bytes, (int)s_local, n, 0, st, block_runs);
  return launch_copy<MAP_ULY_FWD>(in, out, runs, run_bytes, (int)s_local, n, 0, st, block_runs);
}

}  // namespace ra
