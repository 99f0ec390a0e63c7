// Internal declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ra {

// Tile shapes of the attention kernels (query rows x keys per work-list entry).
constexpr int kAttnBf16BM = 128;
constexpr int kAttnBf16BN = 64;
constexpr int kAttnBf16D128BM = 256;  // forward, bf16, head_dim 128 (two-group schedule)
constexpr int kAttnF32BM = 64;
constexpr int kAttnF32BN = 32;

// Tile shapes of the dK/dV kernels (keys per workgroup x query rows per tile).
constexpr int kBwdBf16BK = 128;
constexpr int kBwdBf16BQ = 64;
constexpr int kBwdF32BK = 64;
constexpr int kBwdF32BQ = 32;

// Largest batch of cu_seqlens entries passed by value to the upload kernel.
constexpr int kCuChunk = 960;

struct AttnArgs;
struct BwdArgs;

hipError_t launch_ring_attn(const AttnArgs& a, int d, int in_bf16, int out_bf16, int steps, hipStream_t st);
hipError_t launch_ring_attn_pp(const AttnArgs& a, int out_bf16, int steps, hipStream_t st);

// Copies host cu_seqlens[0..n) into device memory dst (kernel arguments, no host staging buffer).
hipError_t launch_upload_i32(const int32_t* host, int n, int32_t* dst, hipStream_t st);

// Work list of non-SKIP (step, key tile) entries per query tile, and the tile order by work.
hipError_t launch_worklist(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                           int part, int causal, int bm, int bn, int nqt, int nkt, int wl_stride, int* wl,
                           int* wl_count, int* order, hipStream_t st);

// Doc-zigzag block descriptors [cp][nblk] from device cu_seqlens [n_docs+1]; the
// per-rank block prefix [cp][n_docs+1] (blocks rank r holds before document j) is
// written to `prefix` on the way.
hipError_t launch_doc_blocks(const int* cu, int* prefix, int n_docs, int cp, int nblk, int2* blk, hipStream_t st);

// Doc-zigzag CP reorder through the block descriptors: forward [s][row] ->
// [cp][s_local][row] (padding rows zero); inverse [cp][s_local][row] -> [s][row].
hipError_t launch_cp_reorder_docs(const void* in, void* out, int64_t row_bytes, int cp, int s_local, const int2* blk,
                                  int inverse, hipStream_t st);

// Orders n tiles by descending count (ties by index) into order[0..n).
hipError_t launch_order(const int* count, int n, int* order, hipStream_t st);

// Key-side work list of the dK/dV kernels: for key tile kt = s * nkt + J (keys
// [J bk, (J+1) bk) of chunk s), the non-SKIP query tiles of `rank`; then the
// heaviest-first key-tile order.
hipError_t launch_kv_worklist(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                              int part, int causal, int bq, int bk, int nqt, int nkt, int stride, int* wl, int* count,
                              int* order, hipStream_t st);

// dsum[h][i] = sum_c dout[i][h][c] * out[i][h][c] (fp32).
hipError_t launch_bwd_dsum(const void* out, const void* dout, float* dsum, int rows, int hq, int d, int out_bf16,
                           int in_bf16, hipStream_t st);

// dQ kernel then dK/dV kernel.
hipError_t launch_ring_bwd(const BwdArgs& a, int d, int in_bf16, hipStream_t st);

hipError_t launch_classify(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                           int part, int causal, int bm, int bn, int nqt, int nkt, int8_t* cls, hipStream_t st);

hipError_t launch_lse_merge(int64_t rows, int h, int d, const float* o_a, const float* lse_a, const float* o_b,
                            const float* lse_b, float* o_out, float* lse_out, hipStream_t st);

hipError_t launch_cp_reorder(const void* in, void* out, int64_t s, int64_t row_bytes, int cp, int part, int inverse,
                             hipStream_t st);

// Ulysses permute; block_runs = runs (of run_bytes) between the n head-split blocks
// (n * s_local when they are packed).
hipError_t launch_ulysses(const void* in, void* out, int n, int64_t s_local, int64_t run_bytes, int inverse,
                          int64_t block_runs, hipStream_t st);

}  // namespace ra
