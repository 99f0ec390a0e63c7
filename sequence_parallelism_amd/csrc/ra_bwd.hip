// Backward of the ring-step attention for gfx950 (CDNA4).
//
// The pages train with these layers (forward and backward of every step) but
// print no backward equations; the kernels compute the chain rule of the
// forward's definition. With P_ik = exp(s_ik - LSE_i) the probabilities of the
// whole ring (LSE from the forward, so nothing is renormalised per step) and
// dO the gradient of the rank's output rows:
//     D_i   = sum_c dO_ic O_ic                 (= sum_k P_ik dP_ik)
//     dP_ik = dO_i . v_k,   dS_ik = P_ik (dP_ik - D_i)
//     dQ_i  = scale sum_k dS_ik k_k
//     dK_k  = scale sum_i dS_ik q_i,   dV_k = sum_i P_ik dO_i
// P is recomputed from Q, K and the stored LSE instead of being kept from the
// forward (the recompute-for-memory trade that the Sequence Parallelism
// concept page names for activations).
//
// Two kernels, no atomics (results are bit-reproducible):
//  * dQ, query-tile parallel, over the forward's work list (same tiles): the
//    transposed forward, S^T = K Q^T and dP^T = V dO^T (K and V rows from
//    LDS, Q and dO of the lane's row in registers), then dQ^T += K^T dS^T with
//    K^T from the transposing LDS read.
//  * dK and dV, key-tile parallel: a workgroup owns 128 keys of one chunk and
//    one KV head and walks the query tiles (64 rows) that see them, for every
//    query head of the GQA group: X = Q K^T and dP = dO V^T (Q and dO rows
//    from LDS), then dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T from
//    the transposing read. At head_dim 128 (ring_bwd_dkv_pp_kernel) 8 waves
//    share the 128 keys two ways: waves w and w + 4 own the same 32 keys, take
//    the two 32-row halves of each tile and sit on one SIMD; K and V live in
//    LDS, and the two halves' partial dK, dV are added at the end. At head_dim
//    64 (ring_bwd_dkv_bf16_kernel) 4 waves of 32 keys hold K and V in
//    registers and take both halves. One ring step's contribution to a chunk
//    is exactly that chunk's key tiles, so dK / dV of chunk s are this rank's
//    step-(rank - s) partials.
// Both MFMA kernels keep the lane <-> (query row or key) ownership of the
// forward: every softmax-side quantity is a per-lane scalar or a 16-wide
// per-lane vector, and P / dS become the next MFMA's B operand in place.
#include "ra_common.h"
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

// ---------------------------------------------------------------------------
// D_i = sum_c dO_ic O_ic per (row, head): d/8 lanes per pair, 8 elements each.
// ---------------------------------------------------------------------------
template <bool OUT_BF16, bool IN_BF16>
__global__ void __launch_bounds__(256) bwd_dsum_kernel(const void* out, const void* dout, float* dsum, int rows,
                                                       int hq, int d) {
  const int per = d >> 3;  // 8 or 16 lanes, a power of two dividing 64
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long pair = gid / per;
  const int sub = (int)(gid - pair * per);
  float acc = 0.f;
  const bool ok = pair < (long long)rows * hq;
  if (ok) {
    const size_t off = (size_t)pair * d + 8 * sub;
    float o[8], g[8];
    if constexpr (OUT_BF16) {
      const bf16x8 x = *(const bf16x8*)((const __bf16*)out + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) o[i] = (float)x[i];
    } else {
      const f32x4 x0 = *(const f32x4*)((const float*)out + off), x1 = *(const f32x4*)((const float*)out + off + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = x0[i], o[4 + i] = x1[i];
    }
    if constexpr (IN_BF16) {
      const bf16x8 x = *(const bf16x8*)((const __bf16*)dout + off);
#pragma unroll
      for (int i = 0; i < 8; ++i) g[i] = (float)x[i];
    } else {
      const f32x4 x0 = *(const f32x4*)((const float*)dout + off), x1 = *(const f32x4*)((const float*)dout + off + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) g[i] = x0[i], g[4 + i] = x1[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(o[i], g[i], acc);
  }
  for (int m = per >> 1; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (ok && sub == 0) {
    const long long row = pair / hq;
    const int h = (int)(pair - row * hq);
    dsum[(size_t)h * rows + row] = acc;
  }
}

// ---------------------------------------------------------------------------
// dQ, bf16 inputs, MFMA path. Tiles, grid and work list of the forward kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256, 2) ring_bwd_dq_bf16_kernel(const BwdArgs a) {
  constexpr int BM = kAttnBf16BM, BN = kAttnBf16BN;
  static_assert(BM == 128 && BN == 64, "tile shape is baked into the lane mapping");
  // head_dim 128: direct global->LDS tile loads into 256-byte rows, chunks
  // placed by swz_rt (K is read row-wise and transposed, V row-wise);
  // head_dim 64: register-staged tiles with 16-byte padded rows.
  constexpr bool DMA = D == 128;
  constexpr int ROW = DMA ? D : D + 8;
  constexpr int TILE = BN * ROW, STAGE = 2 * TILE;
  constexpr int CHUNKS = BN * D / 8, PER = CHUNKS / 256, CPR = D / 8;
  constexpr int NCT = D / 32, NKD = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi32 = lane >> 5, l32 = lane & 31;
  const int qt = a.order[blockIdx.x / a.hq];
  if (qt < 0 || qt >= a.nqt) return;
  const int h = head_of_slot(blockIdx.x % a.hq, a.hq);
  const int g = h / (a.hq / a.hkv);
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int row = qt * BM + wave * 32 + l32;
  const bool row_ok = row < a.s_local;
  const float C = a.scale_log2;

  // B operands of S^T = K Q^T and dP^T = V dO^T: lane holds 8 elements of its row.
  bf16x8 qreg[NKD], oreg[NKD];
  {
    const uint32_t bytes = (uint32_t)a.s_local * a.hq * D * 2u;
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(a.q, bytes);
    const __amdgpu_buffer_rsrc_t orr = buffer_rsrc(a.dout, bytes);
    const uint32_t off = ((uint32_t)row * a.hq + h) * D * 2u + 16u * hi32;
#pragma unroll
    for (int j = 0; j < NKD; ++j) {
      qreg[j] = __builtin_bit_cast(bf16x8, buffer_load16(qr, off + 32u * j));
      oreg[j] = __builtin_bit_cast(bf16x8, buffer_load16(orr, off + 32u * j));
    }
  }
  // Rows past the end, or with no visible key (LSE = -inf), get P = 0: exp2(x - inf).
  float lse2 = INFINITY, dsum = 0.f;
  int lo = 1, hi = 0;
  if (row_ok) {
    const float l = a.lse[(size_t)h * a.s_local + row];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dsum = a.dsum[(size_t)h * a.s_local + row];
    row_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, a.rank, row), lo, hi);
  }

  f32x16 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x16{};

  const uint32_t kv_row_bytes = (uint32_t)a.hkv * D * 2u;
  const uint32_t chunk_bytes = (uint32_t)a.s_local * kv_row_bytes;
  const int n_ent = clamp_count(a.wl_count[qt], a.wl_stride);
  const int* list = a.wl + (size_t)qt * a.wl_stride;

  // Direct loads: wave w fills rows 16 w .. 16 w + 15 of a tile, 4 rows per
  // instruction; lane L lands in slot L % 16 of row L / 16 and fetches the
  // logical chunk that swz_rt places there.
  uint32_t d_off[4];
  uint32_t goff[PER];
  int slot[PER];
  if constexpr (DMA) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4), pc = lane & 15;
      d_off[i] = (uint32_t)r * kv_row_bytes + ((uint32_t)g * D + 8 * (pc ^ swz_rt(r))) * 2u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * 256;
      const int r = c / CPR, c8 = c % CPR;
      goff[i] = (uint32_t)r * kv_row_bytes + ((uint32_t)g * D + c8 * 8) * 2u;
      slot[i] = r * ROW + c8 * 8;
    }
  }
  uint4 rk[DMA ? 1 : PER], rv[DMA ? 1 : PER];
  auto load_tile = [&](int ent, int buf) {
    const int t = wl_step(ent), J = wl_tile(ent);
    const size_t cbase = (size_t)ring_owner(a.rank, t, a.cp) * chunk_bytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc((const char*)a.k + cbase, chunk_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc((const char*)a.v + cbase, chunk_bytes);
    const uint32_t toff = (uint32_t)J * BN * kv_row_bytes;
    if constexpr (DMA) {
      __attribute__((address_space(3))) char* kl =
          (__attribute__((address_space(3))) char*)(smem + buf * STAGE) + 4096 * wave;
      __attribute__((address_space(3))) char* vl = kl + TILE * 2;
      const uint32_t kb = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)kl);
      const uint32_t vb = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)vl);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16_lds(kr, toff + d_off[i], kb + 1024u * i);
        dma16_lds(vr, toff + d_off[i], vb + 1024u * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        rk[i] = buffer_load16(kr, toff + goff[i]);
        rv[i] = buffer_load16(vr, toff + goff[i]);
      }
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (DMA) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      __bf16* ks = smem + buf * STAGE;
      __bf16* vs = ks + TILE;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        *(uint4*)(ks + slot[i]) = rk[i];
        *(uint4*)(vs + slot[i]) = rv[i];
      }
    }
  };

  // Per-lane LDS element offsets at key rows 0..31 (swz_rt is unchanged by a shift of 16
  // rows, so the second 32-key half and the 16-row steps only add constants):
  //   rd_off[j]      row-wise read of row l32, logical chunk 2 j + hi32 (A operand of S^T, dP^T)
  //   tr0/1_off[c]   transposing reads of rows 4 hi32 + (lane % 16) / 4 and 8 more, columns
  //                  32 c + 16 ((lane / 16) % 2) + 4 (lane % 4) (A operand of dQ^T)
  int rd_off[NKD], tr0_off[NCT], tr1_off[NCT];
#pragma unroll
  for (int j = 0; j < NKD; ++j) {
    const int kc = 2 * j + hi32;
    rd_off[j] = l32 * ROW + 8 * (DMA ? (kc ^ swz_rt(l32)) : kc);
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int r0 = 4 * hi32 + ((lane & 15) >> 2);
    const int c0 = c * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    tr0_off[c] = r0 * ROW + (DMA ? ((((c0 >> 3) ^ swz_rt(r0)) << 3) | (c0 & 7)) : c0);
    tr1_off[c] = (r0 + 8) * ROW + (DMA ? ((((c0 >> 3) ^ swz_rt(r0 + 8)) << 3) | (c0 & 7)) : c0);
  }

  // The work list is read entry by entry here: a register window (as in the
  // other kernels) costs this kernel spills at its 256-register limit.
  if (n_ent > 0) {
    load_tile(list[0], 0);
    store_tile(0);
  }
  __syncthreads();

  for (int e = 0; e < n_ent; ++e) {
    const int ent = list[e];
    const int t = wl_step(ent), J = wl_tile(ent), cls = wl_cls(ent);
    const bool ent_ok = t < a.cp && J < a.nkt && cls != CLS_SKIP;
    if (e + 1 < n_ent) load_tile(list[e + 1], (e + 1) & 1);

    const int ka = J * BN;
    const int kb = ka + BN < a.s_local ? ka + BN : a.s_local;
    bool need_mask = kb - ka < BN || cls == CLS_PARTIAL;
    bool do_tile = ent_ok;
    TileMask tm{0, BN, 0, 0};
    if (do_tile && need_mask) {
      tm = tile_mask(pinfo, ring_owner(a.rank, t, a.cp), ka, kb, cls, row_ok, lo, hi);
      do_tile = __any(tm.la > 0 || tm.lb > 0);
      need_mask = !__all(tile_all_visible(tm, BN) || !row_ok);
    }

    if (do_tile) {
      const __bf16* ks = smem + (e & 1) * STAGE;
      const __bf16* vs = ks + TILE;
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int j = 0; j < NKD; ++j)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int o = kt * 32 * ROW + rd_off[j];
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(ks + o), qreg[j], s[kt], 0, 0, 0);
          dp[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(vs + o), oreg[j], dp[kt], 0, 0, 0);
        }
      // issue order: the LDS reads run 4 ahead of the MFMAs that use them
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 28; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_s_setprio(0);
      // lane holds keys n = 32 kt + 8 (i/4) + 4 hi32 + (i%4) of its row; dS^T in place of S^T
      if (!need_mask) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], C, -lse2));
            s[kt][i] = p * (dp[kt][i] - dsum);
          }
      } else {
        const int ba = 4 * hi32 - tm.i0a, bb = 4 * hi32 - tm.i0b;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int n = kt * 32 + 8 * (i >> 2) + (i & 3);
            const bool vis = ((unsigned)(n + ba) < (unsigned)tm.la) | ((unsigned)(n + bb) < (unsigned)tm.lb);
            const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], C, -lse2)) : 0.f;
            s[kt][i] = vis ? p * (dp[kt][i] - dsum) : 0.f;
          }
      }
      // dQ^T += K^T dS^T
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 sb0 = __builtin_convertvector(s[kt].lo, bf16x8);
        const bf16x8 sb1 = __builtin_convertvector(s[kt].hi, bf16x8);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int ro = (kt * 32 + jj * 16) * ROW;
            const bf16x8 kk = __builtin_shufflevector(lds_read_tr(ks + ro + tr0_off[c]),
                                                      lds_read_tr(ks + ro + tr1_off[c]), 0, 1, 2, 3, 4, 5, 6, 7);
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kk, jj ? sb1 : sb0, acc[c], 0, 0, 0);
          }
      }
      // issue order: the transposing reads run 2 MFMAs ahead of their use
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 14; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_s_setprio(0);
    }

    if (e + 1 < n_ent) store_tile((e + 1) & 1);
    __syncthreads();
  }

  if (row_ok) {
    float* dq = a.dq + ((size_t)row * a.hq + h) * D;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = c * 32 + 8 * i4 + 4 * hi32;
        *(f32x4*)(dq + col) = f32x4{acc[c][4 * i4], acc[c][4 * i4 + 1], acc[c][4 * i4 + 2], acc[c][4 * i4 + 3]} *
                              a.scale;
      }
  }
}

// ---------------------------------------------------------------------------
// dK and dV, bf16 inputs, MFMA path. Workgroup = (key tile of 128 keys of one
// chunk, KV head); wave = 32 keys; query tiles of 64 rows.
// ---------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256, 1) ring_bwd_dkv_bf16_kernel(const BwdArgs a) {
  constexpr int BK = kBwdBf16BK, BQ = kBwdBf16BQ;
  static_assert(BK == 128 && BQ == 64, "tile shape is baked into the lane mapping");
  constexpr bool DMA = D == 128;
  constexpr int ROW = DMA ? D : D + 8;
  constexpr int TILE = BQ * ROW, STAGE = 2 * TILE;
  constexpr int CHUNKS = BQ * D / 8, PER = CHUNKS / 256, CPR = D / 8;
  constexpr int NCT = D / 32, NKD = D / 16;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][BQ];  // [buf][LSE * log2 e | D][row]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi32 = lane >> 5, l32 = lane & 31;
  const int n_kt = a.cp * a.nkt_kv;
  const int kt = a.korder[blockIdx.x / a.hkv];
  if (kt < 0 || kt >= n_kt) return;
  const int g = head_of_slot(blockIdx.x % a.hkv, a.hkv);
  const int G = a.hq / a.hkv;
  const int owner = kt / a.nkt_kv, J = kt - owner * a.nkt_kv;
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int key = J * BK + wave * 32 + l32;
  const bool key_ok = key < a.s_local;
  const float C = a.scale_log2;

  // B operands of X = Q K^T and dP = dO V^T: lane holds 8 elements of its key.
  const uint32_t kv_row_bytes = (uint32_t)a.hkv * D * 2u;
  const uint32_t chunk_bytes = (uint32_t)a.s_local * kv_row_bytes;
  bf16x8 kreg[NKD], vreg[NKD];
  {
    const size_t cbase = (size_t)owner * chunk_bytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc((const char*)a.k + cbase, chunk_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc((const char*)a.v + cbase, chunk_bytes);
    const uint32_t off = (uint32_t)key * kv_row_bytes + (uint32_t)g * D * 2u + 16u * hi32;
#pragma unroll
    for (int j = 0; j < NKD; ++j) {
      kreg[j] = __builtin_bit_cast(bf16x8, buffer_load16(kr, off + 32u * j));
      vreg[j] = __builtin_bit_cast(bf16x8, buffer_load16(vr, off + 32u * j));
    }
  }
  int plo = 1, phi = 0;  // visible query positions of this key
  if (key_ok) key_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, owner, key), plo, phi);

  f32x16 dk[NCT], dv[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) dk[c] = dv[c] = f32x16{};

  const int n_ent = clamp_count(a.kwl_count[kt], a.kwl_stride);
  const int* list = a.kwl + (size_t)kt * a.kwl_stride;
  const int total = n_ent * G;
  const uint32_t q_row_bytes = (uint32_t)a.hq * D * 2u;
  const uint32_t q_bytes = (uint32_t)a.s_local * q_row_bytes;
  const __amdgpu_buffer_rsrc_t qrs = buffer_rsrc(a.q, q_bytes);
  const __amdgpu_buffer_rsrc_t ors = buffer_rsrc(a.dout, q_bytes);

  uint32_t d_off[4];
  uint32_t goff[PER];
  int slot[PER];
  if constexpr (DMA) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * wave + 4 * i + (lane >> 4), pc = lane & 15;
      d_off[i] = (uint32_t)r * q_row_bytes + 8u * (pc ^ swz_rt(r)) * 2u;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + i * 256;
      const int r = c / CPR, c8 = c % CPR;
      goff[i] = (uint32_t)r * q_row_bytes + c8 * 16u;
      slot[i] = r * ROW + c8 * 8;
    }
  }
  uint4 rq[DMA ? 1 : PER], ro[DMA ? 1 : PER];
  // wave 0: LSE and D of row `lane` of the next tile, as loaded; they are converted
  // only when stored, so that no wait for these loads (which would also wait for
  // the tile's direct loads issued before them) lands right after the issue
  float rl = 0.f, rd = 0.f;
  bool rok = false;
  auto load_tile = [&](int hh, int ent, int buf) {
    const int h = g * G + hh, I = wl_tile(ent);
    const uint32_t toff = (uint32_t)I * BQ * q_row_bytes + (uint32_t)h * D * 2u;
    if constexpr (DMA) {
      __attribute__((address_space(3))) char* ql =
          (__attribute__((address_space(3))) char*)(smem + buf * STAGE) + 4096 * wave;
      __attribute__((address_space(3))) char* ol = ql + TILE * 2;
      const uint32_t qb = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)ql);
      const uint32_t ob = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)ol);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dma16_lds(qrs, toff + d_off[i], qb + 1024u * i);
        dma16_lds(ors, toff + d_off[i], ob + 1024u * i);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        rq[i] = buffer_load16(qrs, toff + goff[i]);
        ro[i] = buffer_load16(ors, toff + goff[i]);
      }
    }
    if (wave == 0) {
      const int r = I * BQ + lane;
      rok = r < a.s_local && I < a.nqt_kv;
      const size_t idx = rok ? (size_t)h * a.s_local + r : 0;
      rl = a.lse[idx];
      rd = a.dsum[idx];
    }
  };
  auto store_tile = [&](int buf) {
    if constexpr (DMA) {
      __builtin_amdgcn_s_waitcnt(0);
    } else {
      __bf16* qs = smem + buf * STAGE;
      __bf16* os = qs + TILE;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        *(uint4*)(qs + slot[i]) = rq[i];
        *(uint4*)(os + slot[i]) = ro[i];
      }
    }
    if (wave == 0) {
      rowv[buf][0][lane] = rok && rl != -INFINITY ? rl * kLog2e : INFINITY;  // LSE * log2 e; +inf: no row
      rowv[buf][1][lane] = rok ? rd : 0.f;
    }
  };

  // Per-lane LDS element offsets at qh = 0, jj = 0. swz_rt is unchanged by a shift of
  // 16 rows, so the 32-row halves and 16-row steps only add constants:
  //   rd_off[j]      row-wise read of row l32, logical chunk 2 j + hi32 (A operand of X, dP)
  //   tr0/1_off[c]   transposing reads of rows 4 hi32 + (lane % 16) / 4 and 8 more, columns
  //                  32 c + 16 ((lane / 16) % 2) + 4 (lane % 4) (A operand of dV^T, dK^T)
  int rd_off[NKD], tr0_off[NCT], tr1_off[NCT];
#pragma unroll
  for (int j = 0; j < NKD; ++j) {
    const int kc = 2 * j + hi32;
    rd_off[j] = l32 * ROW + 8 * (DMA ? (kc ^ swz_rt(l32)) : kc);
  }
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int r0 = 4 * hi32 + ((lane & 15) >> 2);
    const int c0 = c * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    tr0_off[c] = r0 * ROW + (DMA ? ((((c0 >> 3) ^ swz_rt(r0)) << 3) | (c0 & 7)) : c0);
    tr1_off[c] = (r0 + 8) * ROW + (DMA ? ((((c0 >> 3) ^ swz_rt(r0 + 8)) << 3) | (c0 & 7)) : c0);
  }

  ListWindow<true> wl;
  wl.init(list, n_ent, lane);
  if (total > 0) {
    load_tile(0, wl.get(0), 0);
    store_tile(0);
  }
  __syncthreads();

  // iteration it = hh * n_ent + idx: query head g G + hh, list entry idx
  int hh = 0, idx = 0;
  for (int it = 0; it < total; ++it) {
    const int ent = wl.get(idx);
    const int I = wl_tile(ent), cls = wl_cls(ent);
    const bool ent_ok = I < a.nqt_kv && cls != CLS_SKIP;
    const bool wrap = idx + 1 == n_ent;
    if (it + 1 < total) load_tile(wrap ? hh + 1 : hh, wl.get(wrap ? 0 : idx + 1), (it + 1) & 1);

    const int qa = I * BQ;
    const int qb = qa + BQ < a.s_local ? qa + BQ : a.s_local;
    bool need_mask = qb - qa < BQ || cls == CLS_PARTIAL;
    bool do_tile = ent_ok;
    TileMask tm{0, BQ, 0, 0};
    if (do_tile && need_mask) {
      tm = tile_mask(pinfo, a.rank, qa, qb, cls, key_ok, plo, phi);
      do_tile = __any(tm.la > 0 || tm.lb > 0);
      need_mask = !__all(tile_all_visible(tm, BQ) || !key_ok);
    }

    if (do_tile) {
      const int buf = it & 1;
      const __bf16* qs = smem + buf * STAGE;
      const __bf16* os = qs + TILE;
      const float* l2s = rowv[buf][0];
      const float* dss = rowv[buf][1];
#pragma unroll 1
      for (int qh = 0; qh < 2; ++qh) {
        const __bf16* qh_q = qs + qh * 32 * ROW;
        const __bf16* qh_o = os + qh * 32 * ROW;
        f32x16 x = f32x16{}, dp = f32x16{};
        // this half's LSE and D (lane rows 8 i4 + 4 hi32 + 0..3), read under the products
        f32x4 Lr[4], Dr[4];
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int j = 0; j < NKD; ++j) {
          x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qh_q + rd_off[j]), kreg[j], x, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qh_o + rd_off[j]), vreg[j], dp, 0, 0, 0);
        }
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          Lr[i4] = *(const f32x4*)(l2s + qh * 32 + 8 * i4 + 4 * hi32);
          Dr[i4] = *(const f32x4*)(dss + qh * 32 + 8 * i4 + 4 * hi32);
        }
        // issue order: the LDS reads run 8 ahead of the MFMAs that use them; the
        // 8 row-vector reads go under the last products
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_s_setprio(0);
        // lane holds query rows n = 32 qh + 8 (i/4) + 4 hi32 + (i%4) of its key: P into x, dS into dp
        if (!need_mask) {
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 L = Lr[i4], Dd = Dr[i4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int i = 4 * i4 + u;
              const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], C, -L[u]));
              x[i] = p;
              dp[i] = p * (dp[i] - Dd[u]);
            }
          }
        } else {
          const int ba = 4 * hi32 - tm.i0a, bb = 4 * hi32 - tm.i0b;
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const f32x4 L = Lr[i4], Dd = Dr[i4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int i = 4 * i4 + u, n = qh * 32 + 8 * i4 + u;
              const bool vis = ((unsigned)(n + ba) < (unsigned)tm.la) | ((unsigned)(n + bb) < (unsigned)tm.lb);
              const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], C, -L[u])) : 0.f;
              x[i] = p;
              dp[i] = vis ? p * (dp[i] - Dd[u]) : 0.f;
            }
          }
        }
        const bf16x8 pb0 = __builtin_convertvector(x.lo, bf16x8), pb1 = __builtin_convertvector(x.hi, bf16x8);
        const bf16x8 sb0 = __builtin_convertvector(dp.lo, bf16x8), sb1 = __builtin_convertvector(dp.hi, bf16x8);
        // dV^T += dO^T P,  dK^T += Q^T dS
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int ro = jj * 16 * ROW;
            const bf16x8 ot = __builtin_shufflevector(lds_read_tr(qh_o + ro + tr0_off[c]),
                                                      lds_read_tr(qh_o + ro + tr1_off[c]), 0, 1, 2, 3, 4, 5, 6, 7);
            const bf16x8 qt8 = __builtin_shufflevector(lds_read_tr(qh_q + ro + tr0_off[c]),
                                                       lds_read_tr(qh_q + ro + tr1_off[c]), 0, 1, 2, 3, 4, 5, 6, 7);
            dv[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, jj ? pb1 : pb0, dv[c], 0, 0, 0);
            dk[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt8, jj ? sb1 : sb0, dk[c], 0, 0, 0);
          }
        // issue order: the transposing reads run 4 MFMAs ahead of their use (left
        // to itself the compiler waits for each group of 8 before its 4 MFMAs)
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int i = 0; i < 12; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        __builtin_amdgcn_s_setprio(0);
      }
    }

    if (it + 1 < total) store_tile((it + 1) & 1);
    __syncthreads();
    if (wrap) {
      wl.restart(lane);
      idx = 0;
      ++hh;
    } else {
      wl.advance(idx, lane);
      ++idx;
    }
  }

  if (key_ok) {
    const size_t base = (((size_t)owner * a.s_local + key) * a.hkv + g) * D;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = c * 32 + 8 * i4 + 4 * hi32;
        *(f32x4*)(a.dk + base + col) =
            f32x4{dk[c][4 * i4], dk[c][4 * i4 + 1], dk[c][4 * i4 + 2], dk[c][4 * i4 + 3]} * a.scale;
        *(f32x4*)(a.dv + base + col) = f32x4{dv[c][4 * i4], dv[c][4 * i4 + 1], dv[c][4 * i4 + 2], dv[c][4 * i4 + 3]};
      }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU path. dQ: one wave, one query row per lane, the forward's
// fp32 work list (key tiles of 32 staged in LDS). A workgroup accumulates
// kBwdF32Cols of the D output columns (blockIdx.x % (D / kBwdF32Cols) picks
// which), so that the per-lane accumulator stays in registers at head_dim 128;
// the scores and dP still take the full dot products over D.
// ---------------------------------------------------------------------------
constexpr int kBwdF32Cols = 64;

template <int D>
__global__ void __launch_bounds__(64) ring_bwd_dq_f32_kernel(const BwdArgs a) {
  constexpr int BM = kAttnF32BM, BN = kAttnF32BN;
  constexpr int DC = D < kBwdF32Cols ? D : kBwdF32Cols, NH = D / DC;
  static_assert(BM == 64, "one query row per lane");
  __shared__ float qs[BM][D + 1];
  __shared__ float gs[BM][D + 1];
  __shared__ __attribute__((aligned(16))) float ks[BN][D];
  __shared__ __attribute__((aligned(16))) float vs[BN][D];

  const int lane = threadIdx.x;
  const int c0 = (int)(blockIdx.x % NH) * DC, bid = (int)(blockIdx.x / NH);
  const int qt = a.order[bid / a.hq];
  if (qt < 0 || qt >= a.nqt) return;
  const int h = bid % a.hq;
  const int g = h / (a.hq / a.hkv);
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int row = qt * BM + lane;
  const bool row_ok = row < a.s_local;
  const float C = a.scale_log2;
  {
    const float* qp = (const float*)a.q + ((size_t)row * a.hq + h) * D;
    const float* gp = (const float*)a.dout + ((size_t)row * a.hq + h) * D;
    for (int c = 0; c < D; ++c) {
      qs[lane][c] = row_ok ? qp[c] : 0.f;
      gs[lane][c] = row_ok ? gp[c] : 0.f;
    }
  }
  float lse2 = INFINITY, dsum = 0.f;
  int lo = 1, hi = 0;
  if (row_ok) {
    const float l = a.lse[(size_t)h * a.s_local + row];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    dsum = a.dsum[(size_t)h * a.s_local + row];
    row_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, a.rank, row), lo, hi);
  }
  float acc[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) acc[c] = 0.f;
  const size_t kv_row = (size_t)a.hkv * D;
  const size_t kv_chunk = (size_t)a.s_local * kv_row;
  const int n_ent = clamp_count(a.wl_count[qt], a.wl_stride);
  const int* list = a.wl + (size_t)qt * a.wl_stride;

  for (int e = 0; e < n_ent; ++e) {
    const int ent = list[e];
    const int t = wl_step(ent), J = wl_tile(ent), cls = wl_cls(ent);
    if (t >= a.cp || J >= a.nkt || cls == CLS_SKIP) continue;  // uniform across the block
    const int owner = ring_owner(a.rank, t, a.cp);
    __syncthreads();
    {
      const float* kb = (const float*)a.k + owner * kv_chunk + (size_t)g * D;
      const float* vb = (const float*)a.v + owner * kv_chunk + (size_t)g * D;
      for (int idx = lane; idx < BN * D / 4; idx += 64) {
        const int r = idx / (D / 4), c4 = idx % (D / 4);
        const int j = J * BN + r;
        f32x4 kv = {0.f, 0.f, 0.f, 0.f}, vv = {0.f, 0.f, 0.f, 0.f};
        if (j < a.s_local) {
          kv = *(const f32x4*)(kb + (size_t)j * kv_row + 4 * c4);
          vv = *(const f32x4*)(vb + (size_t)j * kv_row + 4 * c4);
        }
        *(f32x4*)&ks[r][4 * c4] = kv;
        *(f32x4*)&vs[r][4 * c4] = vv;
      }
    }
    __syncthreads();
    const int ka = J * BN;
    const int kb = ka + BN < a.s_local ? ka + BN : a.s_local;
    const TileMask tm = tile_mask(pinfo, owner, ka, kb, cls, row_ok, lo, hi);
    for (int j = 0; j < BN; ++j) {
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) {
        s = __builtin_fmaf(qs[lane][c], ks[j][c], s);
        dp = __builtin_fmaf(gs[lane][c], vs[j][c], dp);
      }
      const bool vis = ((unsigned)(j - tm.i0a) < (unsigned)tm.la) | ((unsigned)(j - tm.i0b) < (unsigned)tm.lb);
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, C, -lse2)) : 0.f;
      const float ds = p * (dp - dsum);
      const int jj = opaque(j);  // read again: see the dK/dV kernel
#pragma unroll
      for (int c = 0; c < DC; ++c) acc[c] = __builtin_fmaf(ds, ks[jj][c0 + c], acc[c]);
    }
  }
  if (row_ok) {
    float* dq = a.dq + ((size_t)row * a.hq + h) * D + c0;
    for (int c = 0; c < DC; ++c) dq[c] = acc[c] * a.scale;
  }
}

// dK and dV, fp32 VALU path: one wave, one key per lane (64 keys of one chunk
// and one KV head), query tiles of 32 rows staged in LDS; kBwdF32Cols of the D
// output columns per workgroup, as in the dQ kernel.
template <int D>
__global__ void __launch_bounds__(64) ring_bwd_dkv_f32_kernel(const BwdArgs a) {
  constexpr int BK = kBwdF32BK, BQ = kBwdF32BQ;
  constexpr int DC = D < kBwdF32Cols ? D : kBwdF32Cols, NH = D / DC;
  static_assert(BK == 64, "one key per lane");
  __shared__ float ks[BK][D + 1];
  __shared__ float vs[BK][D + 1];
  __shared__ __attribute__((aligned(16))) float qs[BQ][D];
  __shared__ __attribute__((aligned(16))) float gs[BQ][D];
  __shared__ float l2s[BQ], dss[BQ];

  const int lane = threadIdx.x;
  const int n_kt = a.cp * a.nkt_kv;
  const int c0 = (int)(blockIdx.x % NH) * DC, bid = (int)(blockIdx.x / NH);
  const int kt = a.korder[bid / a.hkv];
  if (kt < 0 || kt >= n_kt) return;
  const int g = bid % a.hkv;
  const int G = a.hq / a.hkv;
  const int owner = kt / a.nkt_kv, J = kt - owner * a.nkt_kv;
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int key = J * BK + lane;
  const bool key_ok = key < a.s_local;
  const float C = a.scale_log2;
  const size_t kv_row = (size_t)a.hkv * D;
  {
    const float* kp = (const float*)a.k + ((size_t)owner * a.s_local + key) * kv_row + (size_t)g * D;
    const float* vp = (const float*)a.v + ((size_t)owner * a.s_local + key) * kv_row + (size_t)g * D;
    for (int c = 0; c < D; ++c) {
      ks[lane][c] = key_ok ? kp[c] : 0.f;
      vs[lane][c] = key_ok ? vp[c] : 0.f;
    }
  }
  int plo = 1, phi = 0;
  if (key_ok) key_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, owner, key), plo, phi);
  float dk[DC], dv[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) dk[c] = dv[c] = 0.f;
  const int n_ent = clamp_count(a.kwl_count[kt], a.kwl_stride);
  const int* list = a.kwl + (size_t)kt * a.kwl_stride;
  const size_t q_row = (size_t)a.hq * D;

  for (int it = 0; it < n_ent * G; ++it) {
    const int hh = it / n_ent;
    const int ent = list[it - hh * n_ent];
    const int I = wl_tile(ent), cls = wl_cls(ent);
    if (I >= a.nqt_kv || cls == CLS_SKIP) continue;  // uniform across the block
    const int h = g * G + hh;
    __syncthreads();
    for (int idx = lane; idx < BQ * D / 4; idx += 64) {
      const int r = idx / (D / 4), c4 = idx % (D / 4);
      const int i = I * BQ + r;
      f32x4 qv = {0.f, 0.f, 0.f, 0.f}, gv = {0.f, 0.f, 0.f, 0.f};
      if (i < a.s_local) {
        qv = *(const f32x4*)((const float*)a.q + (size_t)i * q_row + (size_t)h * D + 4 * c4);
        gv = *(const f32x4*)((const float*)a.dout + (size_t)i * q_row + (size_t)h * D + 4 * c4);
      }
      *(f32x4*)&qs[r][4 * c4] = qv;
      *(f32x4*)&gs[r][4 * c4] = gv;
    }
    if (lane < BQ) {
      const int i = I * BQ + lane;
      float l2 = INFINITY, ds = 0.f;
      if (i < a.s_local) {
        const float l = a.lse[(size_t)h * a.s_local + i];
        l2 = l == -INFINITY ? INFINITY : l * kLog2e;
        ds = a.dsum[(size_t)h * a.s_local + i];
      }
      l2s[lane] = l2;
      dss[lane] = ds;
    }
    __syncthreads();
    const int qa = I * BQ;
    const int qb = qa + BQ < a.s_local ? qa + BQ : a.s_local;
    const TileMask tm = tile_mask(pinfo, a.rank, qa, qb, cls, key_ok, plo, phi);
    for (int r = 0; r < BQ; ++r) {
      float s = 0.f, dp = 0.f;
      // the lane's key row is read from LDS for every query row: kept opaque, the
      // optimiser would hold all 2 D values in registers beside dK and dV and spill
      const int kl = opaque(lane);
#pragma unroll 16
      for (int c = 0; c < D; ++c) {
        s = __builtin_fmaf(qs[r][c], ks[kl][c], s);
        dp = __builtin_fmaf(gs[r][c], vs[kl][c], dp);
      }
      const bool vis = ((unsigned)(r - tm.i0a) < (unsigned)tm.la) | ((unsigned)(r - tm.i0b) < (unsigned)tm.lb);
      const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s, C, -l2s[r])) : 0.f;
      const float ds = p * (dp - dss[r]);
      // the row is read again rather than kept from the dot products above (up to
      // 2 D more live registers)
      const int rr = opaque(r);
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        dk[c] = __builtin_fmaf(ds, qs[rr][c0 + c], dk[c]);
        dv[c] = __builtin_fmaf(p, gs[rr][c0 + c], dv[c]);
      }
    }
  }
  if (key_ok) {
    const size_t base = ((size_t)owner * a.s_local + key) * kv_row + (size_t)g * D + c0;
    for (int c = 0; c < DC; ++c) {
      a.dk[base + c] = dk[c] * a.scale;
      a.dv[base + c] = dv[c];
    }
  }
}

// ---------------------------------------------------------------------------
// Key-side work list: for key tile kt = (chunk s, tile J), every query tile of
// the rank whose class against it is not SKIP, packed with its class.
// ---------------------------------------------------------------------------
struct KvWlArgs {
  const int* cu;
  const int2* blk;
  int n_docs, s_total, s_local, cp, rank, part, causal, bq, bk, nqt, nkt, stride;
  int* wl;
  int* count;
};

__global__ void __launch_bounds__(256) kv_worklist_kernel(const KvWlArgs w) {
  __shared__ int wave_tot[4];
  const int kt = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const PartInfo p{w.part, w.s_local, w.cp, w.blk};
  const int owner = kt / w.nkt, J = kt - owner * w.nkt;
  const int ka = J * w.bk;
  const int kb = ka + w.bk < w.s_local ? ka + w.bk : w.s_local;
  int* out = w.wl + (size_t)kt * w.stride;
  int base = 0;
  for (int i0 = 0; i0 < w.nqt; i0 += 256) {
    const int I = i0 + tid;
    int c = CLS_SKIP;
    if (I < w.nqt) {
      const int qa = I * w.bq;
      const int qb = qa + w.bq < w.s_local ? qa + w.bq : w.s_local;
      c = classify_tile(p, w.rank, qa, qb, owner, ka, kb, w.cu, w.n_docs, w.s_total, w.causal);
    }
    const unsigned long long bal = __ballot(c != CLS_SKIP);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) wave_tot[wave] = __popcll(bal);
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      before += i < wave ? wave_tot[i] : 0;
      tot += wave_tot[i];
    }
    if (c != CLS_SKIP) out[base + before + below] = wl_pack(0, I, c);
    base += tot;
    __syncthreads();
  }
  if (tid == 0) w.count[kt] = base;
}

hipError_t launch_kv_worklist(const int* cu, const int2* blk, int n_docs, int s_total, int s_local, int cp, int rank,
                              int part, int causal, int bq, int bk, int nqt, int nkt, int stride, int* wl, int* count,
                              int* order, hipStream_t st) {
  const int n = cp * nkt;
  if (n == 0) return hipSuccess;
  KvWlArgs w{cu, blk, n_docs, s_total, s_local, cp, rank, part, causal, bq, bk, nqt, nkt, stride, wl, count};
  hipLaunchKernelGGL(kv_worklist_kernel, dim3(n), dim3(256), 0, st, w);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_order(count, n, order, st);
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_bwd_dsum(const void* out, const void* dout, float* dsum, int rows, int hq, int d, int out_bf16,
                           int in_bf16, hipStream_t st) {
  const long long threads = (long long)rows * hq * (d / 8);
  if (threads == 0) return hipSuccess;
  const dim3 grid((unsigned)((threads + 255) / 256));
  if (out_bf16 && in_bf16) {
    hipLaunchKernelGGL((bwd_dsum_kernel<true, true>), grid, dim3(256), 0, st, out, dout, dsum, rows, hq, d);
  } else if (!out_bf16 && in_bf16) {
    hipLaunchKernelGGL((bwd_dsum_kernel<false, true>), grid, dim3(256), 0, st, out, dout, dsum, rows, hq, d);
  } else if (!out_bf16 && !in_bf16) {
    hipLaunchKernelGGL((bwd_dsum_kernel<false, false>), grid, dim3(256), 0, st, out, dout, dsum, rows, hq, d);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dK and dV, bf16 inputs, head_dim 128, two waves per SIMD. Workgroup = (key tile
// of 128 keys of one chunk, KV head), 8 waves. Wave w owns keys 32 (w % 4) .. +31;
// waves w and w + 4 share those keys and a SIMD, and take the two 32-row halves of
// every 64-row query tile (group w / 4 takes rows 32 (w / 4) .. +31). K and V of the
// workgroup's keys sit in LDS (read per product, as Q and dO are), so a wave needs
// the dK, dV accumulators and one half's X, dP but no K, V registers. At the end,
// the second group's partial dK, dV pass through LDS and the first group adds them
// (a fixed order: the result is bit-reproducible).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(512, 1) ring_bwd_dkv_pp_kernel(const BwdArgs a) {
  constexpr int D = 128;
  constexpr int BK = kBwdBf16BK, BQ = kBwdBf16BQ;
  static_assert(BK == 128 && BQ == 64, "tile shape is baked into the lane mapping");
  constexpr int ROW = D;
  constexpr int TILE = BQ * ROW, STAGE = 2 * TILE;
  constexpr int KVT = BK * ROW;  // elements of the K (or V) tile of the workgroup's keys
  constexpr int NCT = D / 32, NKD = D / 16;
  // [K tile | V tile | stage 0 (Q, dO) | stage 1 (Q, dO)]; reused for the final reduction
  __shared__ __attribute__((aligned(1024))) __bf16 smem[2 * KVT + 2 * STAGE];
  __shared__ __attribute__((aligned(16))) float rowv[2][2][BQ];  // [buf][LSE * log2 e | D][row]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3;
  const int hi32 = lane >> 5, l32 = lane & 31;
  const int n_kt = a.cp * a.nkt_kv;
  const int kt = a.korder[blockIdx.x / a.hkv];
  if (kt < 0 || kt >= n_kt) return;
  const int g = head_of_slot(blockIdx.x % a.hkv, a.hkv);
  const int G = a.hq / a.hkv;
  const int owner = kt / a.nkt_kv, J = kt - owner * a.nkt_kv;
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int key = J * BK + wq * 32 + l32;
  const bool key_ok = key < a.s_local;
  const float C = a.scale_log2;

  __bf16* const ks = smem;
  __bf16* const vs = smem + KVT;
  __bf16* const stages = smem + 2 * KVT;

  // K and V of the workgroup's 128 keys into LDS, row r chunk c at chunk slot
  // c ^ swz_rt(r) (keys past the end read as zeros through the buffer bound)
  const uint32_t kv_row_bytes = (uint32_t)a.hkv * D * 2u;
  const uint32_t chunk_bytes = (uint32_t)a.s_local * kv_row_bytes;
  {
    const size_t cbase = (size_t)owner * chunk_bytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc((const char*)a.k + cbase, chunk_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc((const char*)a.v + cbase, chunk_bytes);
#pragma unroll
    for (int i = 0; i < (BK * D / 8) / 512; ++i) {
      const int c = tid + 512 * i;  // 16-byte chunk of the tile
      const int r = c >> 4, c8 = c & 15;
      const uint32_t off = (uint32_t)(J * BK + r) * kv_row_bytes + (uint32_t)g * D * 2u + 16u * c8;
      const uint4 kv = buffer_load16(kr, off), vv = buffer_load16(vr, off);
      const int slot = r * ROW + 8 * (c8 ^ swz_rt(r));
      *(uint4*)(ks + slot) = kv;
      *(uint4*)(vs + slot) = vv;
    }
  }
  int plo = 1, phi = 0;  // visible query positions of this key
  if (key_ok) key_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, owner, key), plo, phi);

  f32x16 dk[NCT], dv[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) dk[c] = dv[c] = f32x16{};

  const int n_ent = clamp_count(a.kwl_count[kt], a.kwl_stride);
  const int* list = a.kwl + (size_t)kt * a.kwl_stride;
  const int total = n_ent * G;
  const uint32_t q_row_bytes = (uint32_t)a.hq * D * 2u;
  const uint32_t q_bytes = (uint32_t)a.s_local * q_row_bytes;
  // this wave's tile source: Q for the first group, dO for the second
  const __amdgpu_buffer_rsrc_t mrs = buffer_rsrc(grp ? a.dout : a.q, q_bytes);

  // direct loads: waves 0-3 fill the Q tile, waves 4-7 the dO tile, 16 rows each
  uint32_t d_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wq + 4 * i + (lane >> 4), pc = lane & 15;
    d_off[i] = (uint32_t)r * q_row_bytes + 8u * (pc ^ swz_rt(r)) * 2u;
  }
  float rl = 0.f, rd = 0.f;
  bool rok = false;
  auto load_tile = [&](int hh, int ent, int buf) {
    const int h = g * G + hh, I = wl_tile(ent);
    const uint32_t toff = (uint32_t)I * BQ * q_row_bytes + (uint32_t)h * D * 2u;
    __attribute__((address_space(3))) char* dl =
        (__attribute__((address_space(3))) char*)(stages + buf * STAGE + grp * TILE) + 4096 * wq;
    const uint32_t db = __builtin_amdgcn_readfirstlane((uint32_t)(size_t)dl);
#pragma unroll
    for (int i = 0; i < 4; ++i) dma16_lds(mrs, toff + d_off[i], db + 1024u * i);
    if (wave == 0) {
      const int r = I * BQ + opaque(lane);
      rok = r < a.s_local && I < a.nqt_kv;
      const size_t idx = rok ? (size_t)h * a.s_local + r : 0;
      rl = a.lse[idx];
      rd = a.dsum[idx];
    }
  };
  auto store_tile = [&](int buf) {
    __builtin_amdgcn_s_waitcnt(0);
    if (wave == 0) {
      const int ln = opaque(lane);
      rowv[buf][0][ln] = rok && rl != -INFINITY ? rl * kLog2e : INFINITY;
      rowv[buf][1][ln] = rok ? rd : 0.f;
    }
  };

  // per-lane LDS element offsets (see the one-wave kernel): row-wise reads of row
  // l32 at logical chunk 2 j + hi32, transposing reads of rows 4 hi32 + (lane%16)/4
  // and 8 more at columns 32 c + 16 ((lane/16)%2) + 4 (lane%4)
  int rd_off[NKD], tr0_off[NCT], tr1_off[NCT];
#pragma unroll
  for (int j = 0; j < NKD; ++j) rd_off[j] = l32 * ROW + 8 * ((2 * j + hi32) ^ swz_rt(l32));
#pragma unroll
  for (int c = 0; c < NCT; ++c) {
    const int r0 = 4 * hi32 + ((lane & 15) >> 2);
    const int c0 = c * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    tr0_off[c] = r0 * ROW + ((((c0 >> 3) ^ swz_rt(r0)) << 3) | (c0 & 7));
    tr1_off[c] = (r0 + 8) * ROW + ((((c0 >> 3) ^ swz_rt(r0 + 8)) << 3) | (c0 & 7));
  }

  ListWindow<true> wl;
  wl.init(list, n_ent, lane);
  if (total > 0) {
    load_tile(0, wl.get(0), 0);
    store_tile(0);
  }
  __syncthreads();

  int hh = 0, idx = 0;
  for (int it = 0; it < total; ++it) {
    const int ent = wl.get(idx);
    const int I = wl_tile(ent), cls = wl_cls(ent);
    const bool ent_ok = I < a.nqt_kv && cls != CLS_SKIP;
    const bool wrap = idx + 1 == n_ent;
    if (it + 1 < total) load_tile(wrap ? hh + 1 : hh, wl.get(wrap ? 0 : idx + 1), (it + 1) & 1);

    // this group's 32-row half of the tile
    const int qa = I * BQ;
    const int qb = qa + BQ < a.s_local ? qa + BQ : a.s_local;
    bool need_mask = qb - qa < BQ || cls == CLS_PARTIAL;
    bool do_tile = ent_ok;
    TileMask tm{0, BQ, 0, 0};
    if (do_tile && need_mask) {
      tm = tile_mask(pinfo, a.rank, qa, qb, cls, key_ok, plo, phi);
      do_tile = __any(tm.la > 0 || tm.lb > 0);
      need_mask = !__all(tile_all_visible(tm, BQ) || !key_ok);
    }

    if (do_tile) {
      const int buf = it & 1;
      const __bf16* qs = stages + buf * STAGE;
      const __bf16* os = qs + TILE;
      const int qh = grp;
      const __bf16* qh_q = qs + qh * 32 * ROW;
      const __bf16* qh_o = os + qh * 32 * ROW;
      const float* l2s = rowv[buf][0];
      const float* dss = rowv[buf][1];
      f32x16 x = f32x16{}, dp = f32x16{};
      f32x4 Lr[4], Dr[4];
      __builtin_amdgcn_s_setprio(1);
      // the key-side base kept opaque: the per-read addresses are then formed at each
      // use (one add) instead of being hoisted out of the loop into registers
      const int kvo = opaque(wq * 32 * ROW);
#pragma unroll
      for (int j = 0; j < NKD; ++j) {
        const bf16x8 kf = *(const bf16x8*)(ks + kvo + rd_off[j]);
        const bf16x8 vf = *(const bf16x8*)(vs + kvo + rd_off[j]);
        x = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qh_q + rd_off[j]), kf, x, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(qh_o + rd_off[j]), vf, dp, 0, 0, 0);
      }
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        Lr[i4] = *(const f32x4*)(l2s + qh * 32 + 8 * i4 + 4 * hi32);
        Dr[i4] = *(const f32x4*)(dss + qh * 32 + 8 * i4 + 4 * hi32);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      __builtin_amdgcn_s_setprio(0);
      if (!need_mask) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 L = Lr[i4], Dd = Dr[i4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * i4 + u;
            const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], C, -L[u]));
            x[i] = p;
            dp[i] = p * (dp[i] - Dd[u]);
          }
        }
      } else {
        const int ba = 4 * hi32 - tm.i0a, bb = 4 * hi32 - tm.i0b;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const f32x4 L = Lr[i4], Dd = Dr[i4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = 4 * i4 + u, n = qh * 32 + 8 * i4 + u;
            const bool vis = ((unsigned)(n + ba) < (unsigned)tm.la) | ((unsigned)(n + bb) < (unsigned)tm.lb);
            const float p = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], C, -L[u])) : 0.f;
            x[i] = p;
            dp[i] = vis ? p * (dp[i] - Dd[u]) : 0.f;
          }
        }
      }
      const bf16x8 pb0 = __builtin_convertvector(x.lo, bf16x8), pb1 = __builtin_convertvector(x.hi, bf16x8);
      const bf16x8 sb0 = __builtin_convertvector(dp.lo, bf16x8), sb1 = __builtin_convertvector(dp.hi, bf16x8);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int ro = jj * 16 * ROW;
          const bf16x8 ot = __builtin_shufflevector(lds_read_tr(qh_o + ro + tr0_off[c]),
                                                    lds_read_tr(qh_o + ro + tr1_off[c]), 0, 1, 2, 3, 4, 5, 6, 7);
          const bf16x8 qt8 = __builtin_shufflevector(lds_read_tr(qh_q + ro + tr0_off[c]),
                                                     lds_read_tr(qh_q + ro + tr1_off[c]), 0, 1, 2, 3, 4, 5, 6, 7);
          dv[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ot, jj ? pb1 : pb0, dv[c], 0, 0, 0);
          dk[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt8, jj ? sb1 : sb0, dk[c], 0, 0, 0);
        }
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
      __builtin_amdgcn_s_setprio(0);
    }

    if (it + 1 < total) store_tile((it + 1) & 1);
    __syncthreads();
    if (wrap) {
      wl.restart(lane);
      idx = 0;
      ++hh;
    } else {
      wl.advance(idx, lane);
      ++idx;
    }
  }

  // the second group's partials through LDS (2 x 4 x 16 floats per lane = 32 KiB per
  // wave, 128 KiB for the group: the whole of the K, V and stage space)
  __syncthreads();
  float* red = (float*)smem;
  if (grp == 1) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[((wq * 2 * NCT + c) * 16 + i) * 64 + lane] = dk[c][i];
        red[((wq * 2 * NCT + NCT + c) * 16 + i) * 64 + lane] = dv[c][i];
      }
  }
  __syncthreads();
  if (grp == 0 && key_ok) {
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dk[c][i] += red[((wq * 2 * NCT + c) * 16 + i) * 64 + lane];
        dv[c][i] += red[((wq * 2 * NCT + NCT + c) * 16 + i) * 64 + lane];
      }
    const size_t base = (((size_t)owner * a.s_local + key) * a.hkv + g) * D;
    // the output pointers are read from the argument segment here (a volatile load),
    // not kept in scalar registers through the loop
    typedef __attribute__((address_space(4))) const BwdArgs KArgs;
    KArgs* ka = (KArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    float* const dkp = *(float* const volatile __attribute__((address_space(4)))*)&ka->dk;
    float* const dvp = *(float* const volatile __attribute__((address_space(4)))*)&ka->dv;
#pragma unroll
    for (int c = 0; c < NCT; ++c)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int col = c * 32 + 8 * i4 + 4 * hi32;
        *(f32x4*)(dkp + base + col) =
            f32x4{dk[c][4 * i4], dk[c][4 * i4 + 1], dk[c][4 * i4 + 2], dk[c][4 * i4 + 3]} * a.scale;
        *(f32x4*)(dvp + base + col) = f32x4{dv[c][4 * i4], dv[c][4 * i4 + 1], dv[c][4 * i4 + 2], dv[c][4 * i4 + 3]};
      }
  }
}

template <int D>
static hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((ring_bwd_dq_bf16_kernel<D>), dim3((unsigned)a.nqt * (unsigned)a.hq), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (D == 128) {
    hipLaunchKernelGGL(ring_bwd_dkv_pp_kernel, dim3((unsigned)(a.cp * a.nkt_kv) * (unsigned)a.hkv), dim3(512), 0, st,
                       a);
  } else {
    hipLaunchKernelGGL((ring_bwd_dkv_bf16_kernel<D>), dim3((unsigned)(a.cp * a.nkt_kv) * (unsigned)a.hkv), dim3(256),
                       0, st, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_f32(const BwdArgs& a, hipStream_t st) {
  constexpr unsigned NH = D < kBwdF32Cols ? 1 : D / kBwdF32Cols;  // column groups per row or key
  hipLaunchKernelGGL((ring_bwd_dq_f32_kernel<D>), dim3((unsigned)a.nqt * (unsigned)a.hq * NH), dim3(64), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ring_bwd_dkv_f32_kernel<D>), dim3((unsigned)(a.cp * a.nkt_kv) * (unsigned)a.hkv * NH), dim3(64),
                     0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_bwd(const BwdArgs& a, int d, int in_bf16, hipStream_t st) {
  if (a.nqt == 0 || a.hq == 0) return hipSuccess;
  if (in_bf16) {
    if (d == 128) return launch_bwd_bf16<128>(a, st);
    if (d == 64) return launch_bwd_bf16<64>(a, st);
    return hipErrorInvalidValue;
  }
  if (d == 128) return launch_bwd_f32<128>(a, st);
  if (d == 64) return launch_bwd_f32<64>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
