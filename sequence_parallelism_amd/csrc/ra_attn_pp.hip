// Ring-step attention for bf16 inputs with head_dim 128: a two-group
// ("ping-pong") schedule for gfx950.
//
// It computes what the generic bf16 kernel computes (the FlashAttention-style
// block of the Sequence Parallelism concept page, section 二, per key tile of
// the work list: S = Q K^T, mask on global positions, online softmax with the
// exact running max, O += P V, and the LSE of each row), with the same
// transposed MFMA mapping (S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_bf16, P^T from the score accumulator converted in place,
// V^T through ds_read_b64_tr_b16). What differs is how the work is scheduled.
//
// One workgroup of 8 waves owns 256 query rows of one head; wave w owns rows
// 32 w .. 32 w + 31, so waves 0-3 (group 0) hold rows [0, 128) and waves 4-7
// (group 1) rows [128, 256), and waves w and w + 4 share a SIMD. For key tile
// e a wave runs two phases:
//   M(e)  matrix products: S(e) = K(e) Q^T and O += V(e-1)^T P(e-1)
//   V(e)  online softmax of S(e) into P(e) (vector ALU and exp)
// in the order M(0) V(0) M(1) ... V(n-1) M(n). A workgroup barrier ends every
// phase, and group 1 runs one phase behind group 0, so while one wave of a
// SIMD issues MFMAs the other runs its softmax, and they swap at each barrier.
// One workgroup per CU (96 KiB of LDS) keeps two waves per SIMD.
//
// Key and value tiles arrive by direct global->LDS loads, three LDS stages of
// each. In V(e), group 0 loads K(e+2) and group 1 loads V(e+2); each wave waits
// for its own loads two phases later, just before the barrier that publishes
// them (K(e) is read in slots 2e and 2e+1, V(e) in slots 2e+2 and 2e+3; slot s
// is phase s of group 0 and phase s-1 of group 1). The loads are written in
// inline assembly: the compiler would otherwise order every transposing LDS
// read after all outstanding direct loads, and the barrier here is a bare
// s_barrier after an LDS-only wait for the same reason (a __syncthreads fence
// also waits for every outstanding load); both waits are counted by hand.
#include "ra_common.h"
#include "ra_device.h"
#include "ra_internal.h"

namespace ra {

namespace {

constexpr int kPpD = 128;
constexpr int kPpBM = kAttnBf16D128BM;  // 256 query rows per workgroup
constexpr int kPpBN = kAttnBf16BN;      // 64 keys per tile
constexpr int kPpStages = 3;
constexpr int kPpTile = kPpBN * kPpD;  // elements of one K or V tile (16 KiB)

// List entries as this kernel reads them: an entry that fails the range checks
// becomes 0 (class SKIP: a fully masked tile), and the ragged last key tile, if
// any, is PARTIAL. After this, the class alone decides how a tile is masked.
struct PpCook {
  int cp, nkt, ragged;  // ragged: the key tile shorter than 64 keys, or -1
  __device__ __forceinline__ int operator()(int v) const {
    const int t = wl_step(v), J = wl_tile(v), c = wl_cls(v);
    const bool ok = t < cp && J < nkt && c != CLS_SKIP;
    return ok ? wl_pack(t, J, J == ragged ? CLS_PARTIAL : c) : 0;
  }
};

}  // namespace

template <bool OUT_BF16, bool STEPS>
__global__ void __launch_bounds__(512, 1) ring_attn_pp_kernel(const AttnArgs a) {
  constexpr int D = kPpD, BM = kPpBM, BN = kPpBN;
  constexpr int NCT = D / 32;  // 32-wide output column tiles
  constexpr int NKD = D / 16;  // 16-deep reduction steps over d
  // LDS: K tile row r, 16-byte chunk c at chunk slot c ^ (r & 15) (16-byte reads
  // down 16 rows); V tile chunk c of row r at c ^ 4 (r & 3) (transposing reads of
  // 4 rows x 4 chunks). Neither read has bank conflicts.
  __shared__ __attribute__((aligned(1024))) __bf16 kbuf[kPpStages][kPpTile];
  __shared__ __attribute__((aligned(1024))) __bf16 vbuf[kPpStages][kPpTile];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in scalar registers
  const int grp = wave >> 2, wq = wave & 3;
  const int hi32 = lane >> 5, l32 = lane & 31;
  const int qt = a.order[blockIdx.x / a.hq];
  if (qt < 0 || qt >= a.nqt) return;  // plan made for other arguments: nothing safe to do
  const int h = head_of_slot(blockIdx.x % a.hq, a.hq);
  const int g = h / (a.hq / a.hkv);
  const PartInfo pinfo{a.part, a.s_local, a.cp, a.blk};
  const int row = qt * BM + wave * 32 + l32;
  const bool row_ok = row < a.s_local;
  const float C = a.scale_log2;

  // Q^T operand: lane holds q[row][16 j + 8 hi32 + 0..7]; rows past the end read 0.
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
  float m = -INFINITY, l = 0.f;  // running max (log2 units) and sum of P
  bf16x8 pb[4];  // P^T(e) in bf16: from V(e) to M(e+1)

  const uint32_t kv_row_bytes = (uint32_t)a.hkv * D * 2u;
  const uint32_t chunk_bytes = (uint32_t)a.s_local * kv_row_bytes;
  const int n = clamp_count(a.wl_count[qt], a.wl_stride);
  ListWindow<false, PpCook> wl;
  wl.init(a.wl + (size_t)qt * a.wl_stride, n, lane, PpCook{a.cp, a.nkt, a.s_local % BN ? a.nkt - 1 : -1});

  // Direct loads: wave wq of a group fills rows 16 wq .. 16 wq + 15 of a tile,
  // 4 rows per instruction; lane L lands in chunk slot L % 16 of row L / 16 and
  // fetches the chunk that the swizzle maps there (group 0: K, group 1: V).
  // d_off[i] is that offset within the tile less 1024 i, the immediate offset
  // of load i (dma16x4_lds).
  uint32_t d_off[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * wq + 4 * i + (lane >> 4), pc = lane & 15;
    const int chunk = grp ? (pc ^ (4 * (r & 3))) : (pc ^ (r & 15));
    d_off[i] = (uint32_t)r * kv_row_bytes + ((uint32_t)g * D + 8 * chunk) * 2u - 1024u * i;
  }
  const uint32_t lds_k = (uint32_t)(size_t)(__attribute__((address_space(3))) __bf16*)&kbuf[0][0];
  const uint32_t lds_v = (uint32_t)(size_t)(__attribute__((address_space(3))) __bf16*)&vbuf[0][0];
  // wave-uniform; read from lane 0 so that it stays in a scalar register
  const uint32_t lds_mine = __builtin_amdgcn_readfirstlane((grp ? lds_v : lds_k) + 4096u * wq);
  const void* src_mine = grp ? a.v : a.k;

  // The work list is consumed through a pipeline: each entry is fetched and
  // decoded once, in the V phase two entries before its own, where its tiles are
  // loaded. The record keeps the list value, the owner of the key chunk and,
  // under per-document zigzag, the descriptor {first position, count} of the
  // 64-slot block that is the key tile (a scalar load; the record is pinned
  // before the barrier that ends the phase, so the wait falls where the barrier
  // waits anyway). Indices past the end read as 0: an entry that fails the range
  // checks (as do those that fail them), whose loads (tile 0 of a valid chunk)
  // land in a stage nothing reads.
  struct Ent {
    int ent, owner, dx, dy;
  };
  static_assert(kPpBN == kDocBlock, "a key tile is one doc-zigzag block");
  const int n_blk = a.s_local / kDocBlock;
  auto fetch = [&](int idx) {
    Ent x;
    x.ent = wl.get(idx);
    const int t = wl_step(x.ent);  // below cp
    x.owner = a.rank - t + (a.rank < t ? a.cp : 0);
    x.dx = 0;
    x.dy = 0;
    if (a.part == PART_DOC_ZIGZAG) {
      const int2 d = blk_at(a.blk, x.owner * n_blk + wl_tile(x.ent));
      x.dx = d.x;
      x.dy = d.y;
    }
    return x;
  };
  auto pin_ent = [](Ent& x) {
    pin_s(x.ent);
    pin_s(x.owner);
    pin_s(x.dx);
    pin_s(x.dy);
  };
  // Stages are passed as byte offsets (stage * 16 KiB), held in scalar registers.
  // This group's tile of entry x into the LDS stage at offset sb (4 direct loads per wave).
  auto issue = [&](uint32_t sb, const Ent& x) {
    const size_t cbase = (size_t)(uint32_t)x.owner * chunk_bytes;
    const __amdgpu_buffer_rsrc_t r = buffer_rsrc((const char*)src_mine + cbase, chunk_bytes);
    const uint32_t toff = (uint32_t)wl_tile(x.ent) * BN * kv_row_bytes;
    uint32_t voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = toff + d_off[i];
    dma16x4_lds(r, voff, lds_mine + sb);
  };

  // Per-lane LDS element offsets inside a tile at key half kt = 0, j = 0 / jj = 0:
  //   k_off[j]  row l32, logical chunk 2 j + hi32 (A operand of S^T); +32 rows for kt = 1
  //   v_off[c]  transposing read of rows 4 hi32 + (lane % 16) / 4 (and +8), columns
  //             32 c + 16 ((lane / 16) % 2) + 4 (lane % 4) (A operand of O^T)
  int k_off[NKD], v_off[NCT];
#pragma unroll
  for (int j = 0; j < NKD; ++j) k_off[j] = l32 * D + 8 * ((2 * j + hi32) ^ (l32 & 15));
  {
    const int r0 = 4 * hi32 + ((lane & 15) >> 2);
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      const int c0 = c * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      v_off[c] = r0 * D + (c0 ^ (32 * (r0 & 3)));
    }
  }

  // M phase parts: S^T(e) = K(e) Q^T into sc from the stage at sb, and
  // O^T += V(e-1)^T P^T(e-1) from the stage at sb.
  typedef __attribute__((address_space(3))) char lds_char;
  // The same offsets as LDS byte addresses in stage 0: a read's address is then one
  // add of the stage's scalar offset. The per-step kernel, whose flushes need more
  // registers, re-derives them from the element offsets at each use instead (kept
  // opaque to the optimiser, which otherwise hoists them into registers of their own).
  uint32_t k_adr[NKD], v_adr[NCT];
#pragma unroll
  for (int j = 0; j < NKD; ++j) k_adr[j] = lds_k + 2u * (uint32_t)k_off[j];
#pragma unroll
  for (int c = 0; c < NCT; ++c) v_adr[c] = lds_v + 2u * (uint32_t)v_off[c];
  auto qk = [&](uint32_t sb, f32x16 (&sc)[2]) {
    uint32_t ko[NKD];
#pragma unroll
    for (int j = 0; j < NKD; ++j) ko[j] = (STEPS ? lds_k + 2u * (uint32_t)opaque(k_off[j]) : k_adr[j]) + sb;
#pragma unroll
    for (int j = 0; j < NKD; ++j)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 ka8 = *(const __attribute__((address_space(3))) bf16x8*)((const lds_char*)(size_t)ko[j] + kt * 32 * D * 2);
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka8, qreg[j], j ? sc[kt] : f32x16{}, 0, 0, 0);
      }
  };
  auto pv = [&](uint32_t sb) {
    uint32_t vo[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) vo[c] = (STEPS ? lds_v + 2u * (uint32_t)opaque(v_off[c]) : v_adr[c]) + sb;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const lds_char* p = (const lds_char*)(size_t)vo[c] + (kt * 32 + jj * 16) * D * 2;
          const bf16x8 va = __builtin_shufflevector(__builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p),
                                                    __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p + 16 * D)),
                                                    0, 1, 2, 3, 4, 5, 6, 7);
          acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[2 * kt + jj], acc[c], 0, 0, 0);
        }
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
          *(f32x4*)(op + col) = f32x4{acc[c][4 * i4], acc[c][4 * i4 + 1], acc[c][4 * i4 + 2], acc[c][4 * i4 + 3]} *
                                inv;
        }
      if (hi32 == 0)
        a.lse_steps[(size_t)t * a.hq * a.s_local + (size_t)h * a.s_local + row] =
            lt > 0.f ? (m + __builtin_amdgcn_logf(lt)) * kLn2 : -INFINITY;
    }
  };
  auto reset = [&]() {
#pragma unroll
    for (int c = 0; c < NCT; ++c) acc[c] = f32x16{};
    m = -INFINITY;
    l = 0.f;
  };
  int cur_t = 0;

  // Issue order of a full M phase (16 K reads, 16 MFMAs of S, 32 transposing V
  // reads, 16 MFMAs of O): the LDS reads run about 8 ahead of the MFMAs that use
  // them, and the V reads start under the last MFMAs of S.
  auto m_order = [&]() {
    constexpr int kDsRead = 0x100, kMfma = 0x008;
    __builtin_amdgcn_sched_group_barrier(kDsRead, 6, 0);
#pragma unroll
    for (int i = 0; i < 10; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kMfma, 6, 0);
  };

  // V phase: online softmax of S^T(e) into P^T(e) for the entry record x. An
  // entry that fails the range checks is a fully masked tile (P = 0, state
  // unchanged).
  auto v_phase = [&](f32x16 (&sc)[2], const Ent& x) {
    const int ent = x.ent, owner = x.owner, dx = x.dx, dy = x.dy;
    const bool ok = wl_cls(ent) != CLS_SKIP;
    const int t = wl_step(ent), J = wl_tile(ent), cls = wl_cls(ent);
    if constexpr (STEPS) {
      while (ok && cur_t < t) {
        flush(cur_t);
        reset();
        ++cur_t;
      }
    }
    {
      // The lane's row sees every key of the tile, none of them (the row is masked
      // as a whole through the exponent's bias), or some (a per-key mask, taken
      // when any lane of the wave needs it).
      bool row_vis = ok;
      if (cls == CLS_PARTIAL) {  // the ragged key tile included
        const int ka = J * BN;
        const int kb = ka + BN < a.s_local ? ka + BN : a.s_local;
        Run k0{}, k1{};
        if (a.part == PART_DOC_ZIGZAG) {  // the tile's keys: the first dy slots of the block
          const int c = kb - ka < dy ? kb - ka : dy;
          k0 = Run{dx, 1, c > 0 ? c : 0, 0};
        } else {
          runs_of(pinfo, owner, ka, kb, k0, k1);
        }
        const TileMask tm = tile_mask_runs(k0, k1, ka, kb, cls, row_ok, lo, hi);
        const bool none = tm.la <= 0 && tm.lb <= 0;
        row_vis = !none;
        if (__any(!none && !tile_all_visible(tm, BN))) {
          row_vis = true;
          // after the shift, bit 32 kt + 8 (i/4) + (i%4) is the lane's element (kt, i)
          const uint64_t vb = mask_bits(tm) >> (4 * hi32);
          const uint32_t w[2] = {(uint32_t)vb, (uint32_t)(vb >> 32)};
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) sc[kt][i] = keep_or_ninf(sc[kt][i], w[kt], 8 * (i >> 2) + (i & 3));
        }
      }
      // online softmax in the log2 domain; the running max is exact
      // IEEE maximum (v_maximum3_f32 on gfx950): unlike fmaxf it needs no
      // canonicalising of the MFMA results; scores are finite or -inf here
      float mx = sc[0][0];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, sc[kt][i]);
      // a row that sees none of the tile: max -inf and P = exp2(-inf) = 0, through
      // an added -inf (arithmetic rather than a select, which the compiler turns
      // into a branch around the row maximum)
      const float mb = row_vis ? 0.f : -INFINITY;
      mx = __builtin_fmaf(swap_half_max(mx), C, mb);
      // rows that do not grow keep alpha = 1 exactly (their m may still be -inf)
      const bool grow = mx > m;
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mx) : 1.f;
      m = grow ? mx : m;
      const float bias = (m == -INFINITY ? 0.f : -m) + mb;
      float rs = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kt][i], C, bias));
          sc[kt][i] = p;
          rs += p;
        }
      l = __builtin_fmaf(l, alpha, rs);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        pb[2 * kt] = __builtin_convertvector(sc[kt].lo, bf16x8);
        pb[2 * kt + 1] = __builtin_convertvector(sc[kt].hi, bf16x8);
      }
      // The compiler places the rescale right after alpha, ahead of the exps;
      // holding it back until after them (an empty asm on rs) measured 4 % slower.
      if (__any(grow)) {
#pragma unroll
        for (int c = 0; c < NCT; ++c) acc[c] *= alpha;
      }
    }
  };

  if (n > 0) {
    // prologue: group 0 loads K(0), K(1) and publishes K(0); group 1 loads V(0)
    // (entry 1 is loaded even when n == 1: past the end it reads as entry 0)
    Ent x0 = fetch(0), x1 = fetch(1);
    issue(0, x0);
    if (grp == 0) {
      issue(kPpTile * 2u, x1);
      wait_vmcnt<4>();
    }
    lds_barrier();
    if (grp == 1) {  // slot 0: group 1 has no phase yet; it loads V(1)
      issue(kPpTile * 2u, x1);
      lds_barrier();
    }
    // byte offsets of the stages of entry e (s_cur), of e - 1 and e + 2 (s_prv),
    // and of e + 1 (s_nxt); they rotate by one stage per entry
    uint32_t s_cur = 0, s_nxt = kPpTile * 2u, s_prv = 2 * kPpTile * 2u;
    for (int e = 0; e < n; ++e) {
      // M(e)
      f32x16 sc[2];
      __builtin_amdgcn_s_setprio(2);
      if (e > 0) {
        qk(s_cur, sc);
        pv(s_prv);
        m_order();
      } else {
        qk(s_cur, sc);
      }
      __builtin_amdgcn_s_setprio(0);
      if (grp == 1) wait_vmcnt<4>();  // V(e) must have landed; V(e+1) may still be in flight
      lds_barrier();
      // V(e)
      // this group's tile of entry e + 2 is requested first, ahead of the softmax
      Ent x2 = fetch(e + 2);
      issue(s_prv, x2);
      v_phase(sc, x0);
      // a list refill (every 64 entries) is waited for here, which also waits for
      // this wave's tile loads in flight
      wl.advance(e, lane);
      if (grp == 0) wait_vmcnt<4>();  // K(e+1) must have landed; K(e+2) may still be in flight
      // pinned here, or the optimiser sinks the softmax below the barrier that ends
      // its phase, next to the products that consume P, and the two groups' vector
      // and matrix work no longer alternate
#pragma unroll
      for (int k = 0; k < 4; ++k) pin(pb[k]);
#pragma unroll
      for (int c = 0; c < NCT; ++c) pin(acc[c]);
      pin(l);
      pin(m);
      pin_ent(x2);
      lds_barrier();
      x0 = x1;
      x1 = x2;
      const uint32_t s_old = s_prv;
      s_prv = s_cur;
      s_cur = s_nxt;
      s_nxt = s_old;
    }
    // M(n): the last product
    __builtin_amdgcn_s_setprio(2);
    pv(s_prv);
    __builtin_amdgcn_s_setprio(0);
    wait_vmcnt<0>();  // the two loads past the end must land before the workgroup's LDS is released
    lds_barrier();
    if (grp == 0) lds_barrier();  // last slot: group 1's M(n)
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

hipError_t launch_ring_attn_pp(const AttnArgs& a, int out_bf16, int steps, hipStream_t st) {
  const unsigned grid = (unsigned)a.nqt * (unsigned)a.hq;
  if (steps)
    hipLaunchKernelGGL((ring_attn_pp_kernel<false, true>), dim3(grid), dim3(512), 0, st, a);
  else if (out_bf16)
    hipLaunchKernelGGL((ring_attn_pp_kernel<true, false>), dim3(grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((ring_attn_pp_kernel<false, false>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace ra
