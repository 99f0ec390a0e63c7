// Ring-step attention kernels for gfx950 (CDNA4).
//
// One workgroup owns one (query tile, query head) pair of a CP rank and walks
// the ring: for step t it visits the KV chunk of rank (rank - t) mod cp (the
// ring order of the Context Parallelism page, 2.2: send to the next rank,
// receive from the previous), one key tile at a time, in the order of a
// precomputed work list that holds only the non-SKIP tiles with their
// FULL / PARTIAL class. Each tile is a FlashAttention-style block:
//     S = Q K^T (bf16 MFMA, fp32 accumulate) -> mask on global positions
//     (PARTIAL tiles only) -> online softmax (running max m, sum l, scaled by
//     exp(m_old - m_new)) -> O += P V (bf16 MFMA)
// as in the online-softmax update of the Sequence Parallelism concept page
// (section 二; S = Q K^T / sqrt(d_k), and the rescale factor on O read as
// exp(m_old - m_new), the same as on l).
//
// Combining ring steps: the accumulator and (m, l) carry from one step to the
// next, which is the LSE merge of the steps' partials done in unnormalised
// form (LSE = logaddexp, weights exp(LSE_t - LSE)); the steps variant instead
// writes each step's normalised partial and its LSE for an explicit merge.
//
// MFMA mapping (v_mfma_f32_32x32x16_bf16, wave64): each wave owns 32 query
// rows. Scores are computed transposed, S^T = K Q^T, so a lane holds 16 keys
// of ONE query row (lane % 32): the row max needs one lane exchange (lane ^ 32,
// v_permlane32_swap) and the per-row rescale is a per-lane scalar. O is also
// accumulated transposed, O^T = V^T P^T: the P^T operand is the score
// accumulator converted to bf16 in place (v_cvt_pk_bf16_f32) with the MFMA
// reduction index permuted to match, and the V^T operand is read from the
// row-major V tile with ds_read_b64_tr_b16 (4x4 transposing LDS read), so V
// is never transposed in memory. exp is exp2 with softmax_scale*log2(e)
// folded into one FMA (e^x = 2^(x log2 e)).
#include "ra_common.h"
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

// The accumulator is rescaled whenever a row's running max grows by more than
// this (log2 units). It is 0: the running max stays exact, so the key that sets
// it gets P = 1 exactly and only the smaller P values carry bf16 rounding. A
// stale max (a lazy threshold of 2^8 was 2.4% faster) also rounds the dominant
// key's P and lets the output error reach 2^-9 of the largest |v|, about 1e-2.
constexpr float kRescaleTau = 0.0f;

// ---------------------------------------------------------------------------
// bf16 inputs, MFMA path. 4 waves x 32 query rows, key tiles of 64. Launched
// for head_dim 64 (head_dim 128 runs the two-group kernel of ra_attn_pp.hip).
// ---------------------------------------------------------------------------
template <int D, bool OUT_BF16, bool STEPS>
__global__ void __launch_bounds__(256, 2) ring_attn_bf16_kernel(const AttnArgs a) {
  constexpr int BM = kAttnBf16BM, BN = kAttnBf16BN;
  static_assert(BM == 128 && BN == 64, "tile shape is baked into the lane mapping");
  // LDS: register-staged, double-buffered tiles with padded rows against bank
  // conflicts (K pitch d + 8, V pitch d + 16 elements).
  constexpr int KROW = D + 8;
  constexpr int VROW = D + 16;
  constexpr int KTILE = BN * KROW, VTILE = BN * VROW, STAGE = KTILE + VTILE;
  constexpr int CHUNKS = BN * D / 8;         // 16-byte chunks per tile
  constexpr int PER = CHUNKS / 256;          // per thread
  constexpr int CPR = D / 8;                 // chunks per row
  constexpr int NCT = D / 32;                // 32-wide output column tiles
  constexpr int NKD = D / 16;                // 16-deep reduction steps over d
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hi32 = lane >> 5, l32 = lane & 31;
  const int qt = a.order[blockIdx.x / a.hq];
  if (qt < 0 || qt >= a.nqt) return;  // plan made for other arguments: nothing safe to do
  const int h = head_of_slot(blockIdx.x % a.hq, a.hq);
  const int g = h / (a.hq / a.hkv);
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int row = qt * BM + wave * 32 + l32;
  const bool row_ok = row < a.s_local;
  const float C = a.scale_log2;

  // Q^T operand (B of S^T = K Q^T): lane holds q[row][16 j + 8 hi32 + 0..7]; rows past
  // the end read as 0 through the buffer range check.
  bf16x8 qreg[NKD];
  {
    const __amdgpu_buffer_rsrc_t qr = buffer_rsrc(a.q, (uint32_t)a.s_local * a.hq * D * 2u);
    const uint32_t qoff = ((uint32_t)row * a.hq + h) * D * 2u + 16u * hi32;
#pragma unroll
    for (int j = 0; j < NKD; ++j) qreg[j] = __builtin_bit_cast(bf16x8, buffer_load16(qr, qoff + 32u * j));
  }
  int lo = 1, hi = 0;  // empty interval for rows past the end
  if (row_ok) row_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, a.rank, row), lo, hi);

  f32x16 acc[NCT];
#pragma unroll
  for (int c = 0; c < NCT; ++c) acc[c] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const uint32_t kv_row_bytes = (uint32_t)a.hkv * D * 2u;
  const uint32_t chunk_bytes = (uint32_t)a.s_local * kv_row_bytes;
  const int n_ent = clamp_count(a.wl_count[qt], a.wl_stride);
  const int* list = a.wl + (size_t)qt * a.wl_stride;

  // per-thread byte offsets of its 16-byte chunks inside a key tile, and LDS slots
  uint32_t goff[PER];
  int kslot[PER], vslot[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = tid + i * 256;
    const int r = c / CPR, c8 = c % CPR;
    goff[i] = (uint32_t)r * kv_row_bytes + ((uint32_t)g * D + c8 * 8) * 2u;
    kslot[i] = r * KROW + c8 * 8;
    vslot[i] = r * VROW + c8 * 8;
  }

  uint4 rk[PER], rv[PER];
  auto load_tile = [&](int ent, int buf) {
    const int t = wl_step(ent), J = wl_tile(ent);
    const size_t cbase = (size_t)ring_owner(a.rank, t, a.cp) * chunk_bytes;
    const __amdgpu_buffer_rsrc_t kr = buffer_rsrc((const char*)a.k + cbase, chunk_bytes);
    const __amdgpu_buffer_rsrc_t vr = buffer_rsrc((const char*)a.v + cbase, chunk_bytes);
    const uint32_t toff = (uint32_t)J * BN * kv_row_bytes;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      rk[i] = buffer_load16(kr, toff + goff[i]);
      rv[i] = buffer_load16(vr, toff + goff[i]);
    }
  };
  auto store_tile = [&](int buf) {
    __bf16* ks = smem + buf * STAGE;
    __bf16* vs = ks + KTILE;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      *(uint4*)(ks + kslot[i]) = rk[i];
      *(uint4*)(vs + vslot[i]) = rv[i];
    }
  };
  auto reset = [&]() {
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x16{};
    m = -INFINITY;
    l = 0.f;
  };
  // normalised partial of the current state (steps mode)
  auto flush = [&](int t) {
    const float lt = swap_half_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row_ok) {
      float* op = a.o_steps + ((size_t)t * a.s_local * a.hq + (size_t)row * a.hq + h) * D;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int col = c * 32 + 8 * i4 + 4 * hi32;
          f32x4 o4 = {acc[c][4 * i4] * inv, acc[c][4 * i4 + 1] * inv, acc[c][4 * i4 + 2] * inv,
                      acc[c][4 * i4 + 3] * inv};
          *(f32x4*)(op + col) = o4;
        }
      if (hi32 == 0)
        a.lse_steps[(size_t)t * a.hq * a.s_local + (size_t)h * a.s_local + row] =
            lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
  };

  ListWindow<> wl;
  wl.init(list, n_ent, lane);
  int cur_t = 0;
  if (n_ent > 0) {
    load_tile(wl.get(0), 0);
    store_tile(0);
  }
  __syncthreads();

  for (int e = 0; e < n_ent; ++e) {
    const int ent = wl.get(e);
    const int t = wl_step(ent), J = wl_tile(ent), cls = wl_cls(ent);
    const bool ent_ok = t < a.cp && J < a.nkt && cls != CLS_SKIP;
    if constexpr (STEPS) {
      while (ent_ok && cur_t < t) {
        flush(cur_t);
        reset();
        ++cur_t;
      }
    }
    if (e + 1 < n_ent) load_tile(wl.get(e + 1), (e + 1) & 1);

    const int ka = J * BN;
    const int kb = ka + BN < a.s_local ? ka + BN : a.s_local;
    const bool ragged = kb - ka < BN;
    bool need_mask = ragged || cls == CLS_PARTIAL;
    bool do_tile = ent_ok;
    TileMask tm{0, BN, 0, 0};
    if (do_tile && need_mask) {
      tm = tile_mask(pinfo, ring_owner(a.rank, t, a.cp), ka, kb, cls, row_ok, lo, hi);
      do_tile = __any(tm.la > 0 || tm.lb > 0);
      need_mask = !__all(tile_all_visible(tm, BN) || !row_ok);
    }

    if (do_tile) {
      const __bf16* ks = smem + (e & 1) * STAGE;
      const __bf16* vs = ks + KTILE;
      // S^T = K Q^T for 2 x 32 keys
      __builtin_amdgcn_s_setprio(1);
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int j = 0; j < NKD; ++j)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const int kr = kt * 32 + l32, kc = 2 * j + hi32;
          const bf16x8 ka8 = *(const bf16x8*)(ks + kr * KROW + 8 * kc);
          s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka8, qreg[j], s[kt], 0, 0, 0);
        }
      __builtin_amdgcn_s_setprio(0);
      // mask (branch-free): lane holds keys n = 32 kt + 8 (i/4) + 4 hi32 + (i%4)
      if (need_mask) {
        const int ba = 4 * hi32 - tm.i0a, bb = 4 * hi32 - tm.i0b;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int n = kt * 32 + 8 * (i >> 2) + (i & 3);
            const bool vis = ((unsigned)(n + ba) < (unsigned)tm.la) | ((unsigned)(n + bb) < (unsigned)tm.lb);
            s[kt][i] = vis ? s[kt][i] : -INFINITY;
          }
      }
      // online softmax in the log2 domain, rescaled when the running max grows
      float mx = s[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
      mx = swap_half_max(mx) * C;
      const bool grow = mx > m + kRescaleTau;
      if (__any(grow)) {
        // rows that do not grow keep alpha = 1 exactly (their m may still be -inf)
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
        l *= alpha;
#pragma unroll
        for (int c = 0; c < NCT; ++c) acc[c] *= alpha;
        m = grow ? mx : m;
      }
      const float m_use = m == -INFINITY ? 0.f : m;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][i], C, -m_use));
          s[kt][i] = p;
          rs += p;
        }
      l += rs;
      // O^T += V^T P^T
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 pb0 = __builtin_convertvector(s[kt].lo, bf16x8);
        const bf16x8 pb1 = __builtin_convertvector(s[kt].hi, bf16x8);
#pragma unroll
        for (int c = 0; c < NCT; ++c)
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int r0 = kt * 32 + jj * 16 + 4 * hi32 + ((lane & 15) >> 2);
            const int c0 = c * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            const bf16x4 v0 = lds_read_tr(vs + r0 * VROW + c0);
            const bf16x4 v1 = lds_read_tr(vs + (r0 + 8) * VROW + c0);
            const bf16x8 va = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, jj ? pb1 : pb0, acc[c], 0, 0, 0);
          }
      }
      __builtin_amdgcn_s_setprio(0);
    }

    if (e + 1 < n_ent) store_tile((e + 1) & 1);
    __syncthreads();
    wl.advance(e, lane);
  }

  if constexpr (STEPS) {
    while (cur_t < a.cp) {
      flush(cur_t);
      reset();
      ++cur_t;
    }
  } else {
    const float lt = swap_half_sum(l);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (row_ok) {
      const size_t base = ((size_t)row * a.hq + h) * D;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int col = c * 32 + 8 * i4 + 4 * hi32;
          f32x4 o4 = {acc[c][4 * i4] * inv, acc[c][4 * i4 + 1] * inv, acc[c][4 * i4 + 2] * inv,
                      acc[c][4 * i4 + 3] * inv};
          if constexpr (OUT_BF16) {
            *(bf16x4*)((__bf16*)a.out + base + col) = __builtin_convertvector(o4, bf16x4);
          } else {
            *(f32x4*)((float*)a.out + base + col) = o4;
          }
        }
      if (hi32 == 0)
        a.lse[(size_t)h * a.s_local + row] = lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs, VALU path (one wave, one query row per lane, key tiles of 32).
// ---------------------------------------------------------------------------
template <int D, bool STEPS>
__global__ void __launch_bounds__(64) ring_attn_f32_kernel(const AttnArgs a) {
  constexpr int BM = kAttnF32BM, BN = kAttnF32BN;
  static_assert(BM == 64, "one query row per lane");
  __shared__ float qs[BM][D + 1];
  __shared__ __attribute__((aligned(16))) float ks[BN][D];
  __shared__ __attribute__((aligned(16))) float vs[BN][D];

  const int lane = threadIdx.x;
  const int qt = a.order[blockIdx.x / a.hq];
  if (qt < 0 || qt >= a.nqt) return;
  const int h = blockIdx.x % a.hq;
  const int g = h / (a.hq / a.hkv);
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int row = qt * BM + lane;
  const bool row_ok = row < a.s_local;
  const float C = a.scale_log2;

  {
    const float* qp = (const float*)a.q + ((size_t)row * a.hq + h) * D;
    for (int c = 0; c < D; ++c) qs[lane][c] = row_ok ? qp[c] : 0.f;
  }
  int lo = 1, hi = 0;
  if (row_ok) row_interval(a.cu, a.n_docs, a.s_total, a.causal, pos_of(pinfo, a.rank, row), lo, hi);

  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const size_t kv_row = (size_t)a.hkv * D;
  const size_t kv_chunk = (size_t)a.s_local * kv_row;
  const int n_ent = clamp_count(a.wl_count[qt], a.wl_stride);
  const int* list = a.wl + (size_t)qt * a.wl_stride;

  auto flush = [&](int t) {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok) {
      float* op = a.o_steps + ((size_t)t * a.s_local * a.hq + (size_t)row * a.hq + h) * D;
      for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
      a.lse_steps[(size_t)t * a.hq * a.s_local + (size_t)h * a.s_local + row] =
          l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
  };
  int cur_t = 0;
  ListWindow<> wl;
  wl.init(list, n_ent, lane);

  for (int e = 0; e < n_ent; wl.advance(e, lane), ++e) {
    const int ent = wl.get(e);
    const int t = wl_step(ent), J = wl_tile(ent), cls = wl_cls(ent);
    if (t >= a.cp || J >= a.nkt || cls == CLS_SKIP) continue;  // uniform across the block
    const int owner = ring_owner(a.rank, t, a.cp);
    if constexpr (STEPS) {
      while (cur_t < t) {
        flush(cur_t);
        for (int c = 0; c < D; ++c) acc[c] = 0.f;
        m = -INFINITY;
        l = 0.f;
        ++cur_t;
      }
    }
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
    float s[BN];
    float mx = -INFINITY;
    for (int j = 0; j < BN; ++j) {
      float dot = 0.f;
      // the query row is read from LDS for every key: kept in registers beside the
      // D accumulators it makes the per-step variant spill at head_dim 128
      const int ql = opaque(lane);
#pragma unroll
      for (int c = 0; c < D; ++c) dot = __builtin_fmaf(qs[ql][c], ks[j][c], dot);
      const bool vis = ((unsigned)(j - tm.i0a) < (unsigned)tm.la) | ((unsigned)(j - tm.i0b) < (unsigned)tm.lb);
      s[j] = vis ? dot : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m, mx * C);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) acc[c] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], C, -m_use));
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) acc[c] = __builtin_fmaf(p, vs[j][c], acc[c]);
    }
    m = m_new;
  }

  if constexpr (STEPS) {
    while (cur_t < a.cp) {
      flush(cur_t);
      for (int c = 0; c < D; ++c) acc[c] = 0.f;
      m = -INFINITY;
      l = 0.f;
      ++cur_t;
    }
  } else {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok) {
      float* op = (float*)a.out + ((size_t)row * a.hq + h) * D;
      for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
      a.lse[(size_t)h * a.s_local + row] = l > 0.f ? (m + __builtin_amdgcn_logf(l)) * kLn2 : -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, bool OUT_BF16, bool STEPS>
static hipError_t launch_bf16(const AttnArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.nqt * (unsigned)a.hq;
  hipLaunchKernelGGL((ring_attn_bf16_kernel<D, OUT_BF16, STEPS>), dim3(grid), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <int D, bool STEPS>
static hipError_t launch_f32(const AttnArgs& a, hipStream_t st) {
  const unsigned grid = (unsigned)a.nqt * (unsigned)a.hq;
  hipLaunchKernelGGL((ring_attn_f32_kernel<D, STEPS>), dim3(grid), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_ring_attn(const AttnArgs& a, int d, int in_bf16, int out_bf16, int steps, hipStream_t st) {
  if (a.nqt == 0 || a.hq == 0) return hipSuccess;
  if (in_bf16) {
    if (d == 128) return launch_ring_attn_pp(a, out_bf16, steps, st);
    if (d == 64) {
      if (steps) return launch_bf16<64, false, true>(a, st);
      return out_bf16 ? launch_bf16<64, true, false>(a, st) : launch_bf16<64, false, false>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (d == 128) return steps ? launch_f32<128, true>(a, st) : launch_f32<128, false>(a, st);
  if (d == 64) return steps ? launch_f32<64, true>(a, st) : launch_f32<64, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace ra
