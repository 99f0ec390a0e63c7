// Device helpers shared by the attention kernels (forward and backward):
// vector types, wave-half exchanges, the transposing LDS read, raw buffer
// loads, the XCD-aware head mapping, ring ownership and per-lane tile masks.
#pragma once
#include "ra_common.h"

namespace ra {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Slot of logical 16-byte chunk c of row r in an LDS tile of 256-byte rows that
// is read both row-wise (16 B per lane, one chunk down 16 consecutive rows per
// 16-lane group) and through the transposing read (4 consecutive rows x 4
// chunks per 32 lanes): slot = c ^ swz_rt(r). Over any 16 aligned rows
// swz_rt is a permutation of 0..15 (distinct slots for the row-wise read), and
// over 4 aligned rows its bits 2-3 take 4 distinct values (the 4 chunks of
// each row land in distinct 64-byte groups), so neither read has bank conflicts.
__device__ __forceinline__ int swz_rt(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

// x, hidden from the optimiser (an empty asm that reads and rewrites the
// register). Uses: per-phase LDS addresses built from it are not split into
// loop-invariant parts hoisted into registers; and a freshly loaded register
// passed through it is waited for at that point, so no load stays pending
// into later code, where the wait would also drain other loads in flight.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// A block's work list read 64 entries at a time, one entry per lane, so that
// taking entry i is a lane read of a register, never a wait on memory: `cur`
// holds entries [base, base + 64) and `nxt` the 64 after them; valid indices
// are [base, base + 128). advance(i), after entry i has been used, moves the
// window at every multiple of 64 and fetches the chunk 64 entries ahead of its
// first use. With RESTART, `first` also keeps entries [0, 64) (valid at any
// time) and restart() goes back to entry 0 for another pass over the list.
// Entries are read through a buffer resource of `count` entries, so indices
// past the end read 0 without a branch (a branch around the load would make
// the compiler wait for it at the join). Every lane of the wave calls each
// method with the same arguments. An optional `cook` maps each entry once, as
// it is loaded (one lane per entry), to the value that get() returns.
struct NoCook {
  __device__ __forceinline__ int operator()(int v) const { return v; }
};
template <bool RESTART = false, class Cook = NoCook>
struct ListWindow {
  __amdgpu_buffer_rsrc_t rsrc;
  int base, first, cur, nxt;
  Cook cook;
  __device__ __forceinline__ int fetch(int i) const {
    return cook(opaque(__builtin_amdgcn_raw_buffer_load_b32(rsrc, 4 * i, 0, 0)));
  }
  __device__ __forceinline__ void init(const int* l, int n, int lane, Cook c = Cook{}) {
    cook = c;
    rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<int*>(l), (short)0, 4 * n, 0x00020000);
    base = 0;
    cur = fetch(lane);
    if constexpr (RESTART) first = cur;
    nxt = fetch(64 + lane);
  }
  __device__ __forceinline__ int get(int i) const {
    // select values, not members: a select of member addresses becomes a memory read
    const int c = cur, n = nxt;
    int v = i - base < 64 ? c : n;
    if constexpr (RESTART) {
      const int f = first;
      v = i < 64 ? f : v;
    }
    return __builtin_amdgcn_readlane(v, i & 63);
  }
  // The refill is waited for before returning (one wait per 64 entries).
  __device__ __forceinline__ void advance(int i, int lane) {
    if (((i + 1) & 63) == 0) {
      base += 64;
      cur = nxt;
      nxt = fetch(base + 64 + lane);
    }
  }
  __device__ __forceinline__ void restart(int lane) {
    static_assert(RESTART, "restart needs the first chunk kept");
    if (base != 0) {
      base = 0;
      cur = first;
      nxt = fetch(64 + lane);
    }
  }
};

// Direct global->LDS load of 16 bytes per lane from buffer r at byte offset
// voff: lane L writes LDS bytes [lds + 16 L, lds + 16 L + 16); lds is
// wave-uniform. Written in assembly so that the compiler does not track it:
// otherwise it orders LDS reads after every direct load in flight (waiting for
// the next tile's prefetch before the current tile's reads). The caller waits
// for completion itself (s_waitcnt vmcnt) before publishing the data. A direct
// load that reads M0 needs one wait state after a scalar write of M0 (the
// compiler's hazard pass cannot see into the asm, hence the s_nop).
__device__ __forceinline__ void dma16_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
               "s"(r)
               : "memory", "m0");
}

// Four direct loads of 16 bytes per lane, as dma16_lds at (voff[i] + 1024 i,
// lds + 1024 i) for i = 0..3. The immediate offset applies to both the buffer
// and the LDS address, so one M0 serves all four (voff[i] carries the rest).
// lds is wave-uniform; the read of lane 0 keeps it in a scalar register where
// the compiler cannot prove that.
__device__ __forceinline__ void dma16x4_lds(__amdgpu_buffer_rsrc_t r, const uint32_t (&voff)[4], uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %5, 0 offen lds\n\t"
      "buffer_load_dwordx4 %2, %5, 0 offen offset:1024 lds\n\t"
      "buffer_load_dwordx4 %3, %5, 0 offen offset:2048 lds\n\t"
      "buffer_load_dwordx4 %4, %5, 0 offen offset:3072 lds" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
      "v"(voff[0]), "v"(voff[1]), "v"(voff[2]), "v"(voff[3]), "s"(r)
      : "memory", "m0");
}

// Waits until at most N of this wave's vector-memory operations are in flight
// (the count includes the direct loads above, which the compiler does not see).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's LDS reads and writes have completed. It
// does not wait for vector-memory loads (a __syncthreads fence would, draining
// the direct loads kept in flight across barriers).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Pins x in registers at this point of the program (an empty asm that reads and
// rewrites it): the code computing x runs before later volatile asm, a barrier
// included, instead of being sunk past it towards x's uses.
template <class T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

__device__ __forceinline__ float swap_half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bf16x4 lds_read_tr(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
      (lds_bf16x4*)((__attribute__((address_space(3))) char*)p));
}

// Query head served by block-slot hs: blocks hs, hs+8, ... share an XCD, so a
// contiguous run of hq/8 heads (one KV head under 4:1 GQA) lands on one XCD.
__device__ __forceinline__ int head_of_slot(int hs, int hq) {
  return (hq % 8 == 0) ? (hs % 8) * (hq / 8) + hs / 8 : hs;
}

// Chunk owner visited at ring step t (any t >= 0).
__device__ __forceinline__ int ring_owner(int rank, int t, int cp) { return ((rank - t) % cp + cp) % cp; }

// ring_owner without a division, for 0 <= rank < cp: exact for steps t < cp,
// and `rank` for any other step (the step of an entry that fails its checks).
__device__ __forceinline__ int ring_owner_valid(int rank, int t, int cp) {
  return t < cp ? (rank >= t ? rank - t : rank - t + cp) : rank;
}

// Pins a wave-uniform value in scalar registers at this point (see pin()).
__device__ __forceinline__ void pin_s(int& x) { asm volatile("" : "+s"(x)); }

// Work-list length of a tile, clamped to the reserved stride.
__device__ __forceinline__ int clamp_count(int n, int stride) { return n < 0 ? 0 : (n > stride ? stride : n); }

// Per-lane visible tile-local key indices: [i0a, i0a + la) U [i0b, i0b + lb).
struct TileMask {
  int i0a, la, i0b, lb;
};

// The mask of a lane whose row sees positions [lo, hi], for the tile's keys
// [ka, kb) given as the runs k0, k1 (runs_of).
__device__ __forceinline__ TileMask tile_mask_runs(const Run& k0, const Run& k1, int ka, int kb, int cls, bool row_ok,
                                                   int lo, int hi) {
  TileMask t{0, 0, 0, 0};
  if (!row_ok) return t;
  if (cls == CLS_FULL) {
    t.la = kb - ka;
    return t;
  }
  int n0, n1;
  run_range(k0, lo, hi, n0, n1);  // an empty slot gives an empty interval
  t.i0a = k0.off + n0;
  t.la = n1 >= n0 ? n1 - n0 + 1 : 0;
  run_range(k1, lo, hi, n0, n1);
  t.i0b = k1.off + n0;
  t.lb = n1 >= n0 ? n1 - n0 + 1 : 0;
  return t;
}

__device__ __forceinline__ TileMask tile_mask(const PartInfo& p, int owner, int ka, int kb, int cls, bool row_ok,
                                              int lo, int hi) {
  if (!row_ok || cls == CLS_FULL) return tile_mask_runs(Run{}, Run{}, ka, kb, cls, row_ok, lo, hi);
  Run k0, k1;
  runs_of(p, owner, ka, kb, k0, k1);
  return tile_mask_runs(k0, k1, ka, kb, cls, row_ok, lo, hi);
}

// The lane's interval set as a bit mask over the tile's indices: bit n set when
// index n is visible (tiles of at most 64 indices).
__device__ __forceinline__ uint64_t interval_bits(int i0, int len) {
  if (len <= 0) return 0;
  const uint64_t m = len >= 64 ? ~0ull : (1ull << len) - 1ull;
  return m << (i0 & 63);  // a non-empty interval has i0 + len <= 64
}
__device__ __forceinline__ uint64_t mask_bits(const TileMask& t) {
  return interval_bits(t.i0a, t.la) | interval_bits(t.i0b, t.lb);
}

// x when bit b of w is set, else -inf; branch-free (a sign-extending bit field
// extract and one bitwise select), for the per-element masks of score tiles.
__device__ __forceinline__ float keep_or_ninf(float x, uint32_t w, int b) {
  const int mk = (int)(w << (31 - b)) >> 31;  // all ones when the bit is set
  return __int_as_float((__float_as_int(x) & mk) | (~mk & (int)0xff800000u));
}

// True when the lane's interval set covers all n indices of the tile.
__device__ __forceinline__ bool tile_all_visible(const TileMask& t, int n) {
  return (t.i0a == 0 && t.la == n) || (t.i0b == 0 && t.lb == n);
}

// Raw buffer resource over [base, base + bytes): loads past the end return 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

}  // namespace ra
