// Device helpers shared by the gfx950 kernels of the draft-tree round.
//
// Cost model these helpers are written for (measured on MI355X): a barrier
// of a 1024-thread workgroup is ~25 cycles, an LDS round trip ~70-90 cycles,
// a 64-bit cross-lane shuffle through ds_bpermute ~190 cycles per step. Wave
// reductions therefore use DPP lane moves inside each 16-lane row and four
// v_readlane reads across rows, never ds_bpermute chains.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// LDS-qualified pointers (address space 3): accesses compile to ds_* ops.
#define LDS __attribute__((address_space(3)))

namespace dartree {

constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Order-preserving map of an fp32 value to an unsigned key: a > b as numbers
// iff key(a) > key(b). -0 is folded onto +0 so that equal numbers tie.
__device__ __forceinline__ uint32_t f32_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_f32(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}
// The same map for bf16 bit patterns: key = 0x8000 +/- magnitude, so -0 and
// +0 share 0x8000 and every bf16 value maps into [1, 0xFFFF] (0 stays free).
__device__ __forceinline__ uint32_t bf16_key(uint32_t b) {
  const uint32_t mag = b & 0x7FFFu;
  return (b & 0x8000u) ? (0x8000u - mag) : (0x8000u + mag);
}
__device__ __forceinline__ float bf16_key_to_f32(uint32_t k) {
  const uint32_t b = k >= 0x8000u ? (k - 0x8000u) : (0x8000u | (0x8000u - k));
  return bf16_to_f32(b);
}

// fp32 -> three bf16 parts by truncation: x == hi + mid + lo exactly for
// normal x (each part carries the next 8 significant bits).
__device__ __forceinline__ void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  const uint32_t u = __float_as_uint(x);
  const float r1 = x - __uint_as_float(u & 0xFFFF0000u);
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);
  hi = u >> 16;
  mid = u1 >> 16;
  lo = __float_as_uint(r2) >> 16;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- DPP lane moves (gfx9 encodings) -------------------------------------
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

// Every pattern used here is a permutation inside each 16-lane row, so all
// lanes have a source and no old value is needed.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t readlane(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}

// Exact lane exchanges x[lane ^ J] for the sorting networks. Strides 1..8
// stay inside a 16-lane row (one or two DPP moves: quad xor 3 followed by a
// half-row mirror is xor 4, a row mirror followed by a half-row mirror is
// xor 8); strides 16 and 32 use the gfx950 permlane swaps: with the same
// register as both operands, v_permlane16_swap returns the even rows copied
// over the odd ones and the odd rows copied over the even ones (and
// v_permlane32_swap the same for the two halves), so one select per lane
// picks the partner's value.
constexpr int kDppXor3 = 0x1B;        // quad_perm [3,2,1,0]
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return dpp<kDppXor1>(v);
  } else if constexpr (J == 2) {
    return dpp<kDppXor2>(v);
  } else if constexpr (J == 4) {
    return dpp<kDppHalfMirror>(dpp<kDppXor3>(v));
  } else if constexpr (J == 8) {
    return dpp<kDppHalfMirror>(dpp<kDppMirror>(v));
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "stride");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? r[0] : r[1];
  }
}

// x[63 - lane]: a row mirror (lane ^ 15) followed by the exchanges of 16-lane
// rows and 32-lane halves.
__device__ __forceinline__ uint32_t lane_rev(uint32_t v) { return lane_xor<32>(lane_xor<16>(dpp<kDppMirror>(v))); }

// One compare-exchange stage of a bitonic network over 64-bit keys (hi, lo)
// held one per lane; after the stage (K, J) every block of K lanes is
// ordered descending where lane & K == 0 and ascending elsewhere. Written
// with selects only (no branches).
template <int K, int J>
__device__ __forceinline__ void bitonic_stage(uint32_t& hi, uint32_t& lo) {
  const uint32_t lane = __lane_id();
  const uint32_t ph = lane_xor<J>(hi), pl = lane_xor<J>(lo);
  const uint64_t me = ((uint64_t)hi << 32) | lo, pa = ((uint64_t)ph << 32) | pl;
  const bool gt = pa > me;
  const bool take_max = (((lane / J) ^ (lane / K)) & 1u) == 0u;
  const bool pick = gt == take_max;   // equal keys: either value is right
  hi = pick ? ph : hi;
  lo = pick ? pl : lo;
}
// Sorts the wave's 64 32-bit keys descending (lane 0 holds the largest).
// Each merge of width K starts with a flip (lane i against lane i ^ (K-1)),
// then half-cleaners (lane i against lane i ^ J, J = K/4 .. 1). In every
// compare-exchange the lower lane of the pair keeps the larger key, so the
// direction is one lane bit: an all-ones / zero mask per bit, applied with a
// bitfield select (no lane-mask registers).
__device__ __forceinline__ void wave_sort_desc32(uint32_t& k) {
  const uint32_t lane = __lane_id();
  uint32_t m[6];
#pragma unroll
  for (int b = 0; b < 6; ++b) m[b] = 0u - ((lane >> b) & 1u);
  auto cx = [&](uint32_t pk, int b) {
    const uint32_t mx = max(k, pk), mn = min(k, pk);
    k = (mn & m[b]) | (mx & ~m[b]);
  };
  auto x16 = [&](uint32_t v) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (r[0] & m[4]) | (r[1] & ~m[4]);
  };
  auto x32 = [&](uint32_t v) {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (r[0] & m[5]) | (r[1] & ~m[5]);
  };
  auto x4 = [&](uint32_t v) { return dpp<kDppHalfMirror>(dpp<kDppXor3>(v)); };
  auto x8 = [&](uint32_t v) { return dpp<kDppHalfMirror>(dpp<kDppMirror>(v)); };
  cx(dpp<kDppXor1>(k), 0);
  cx(dpp<kDppXor3>(k), 1);
  cx(dpp<kDppXor1>(k), 0);
  cx(dpp<kDppHalfMirror>(k), 2);
  cx(dpp<kDppXor2>(k), 1);
  cx(dpp<kDppXor1>(k), 0);
  cx(dpp<kDppMirror>(k), 3);
  cx(x4(k), 2);
  cx(dpp<kDppXor2>(k), 1);
  cx(dpp<kDppXor1>(k), 0);
  cx(x16(dpp<kDppMirror>(k)), 4);
  cx(x8(k), 3);
  cx(x4(k), 2);
  cx(dpp<kDppXor2>(k), 1);
  cx(dpp<kDppXor1>(k), 0);
  cx(x32(x16(dpp<kDppMirror>(k))), 5);
  cx(x16(k), 4);
  cx(x8(k), 3);
  cx(x4(k), 2);
  cx(dpp<kDppXor2>(k), 1);
  cx(dpp<kDppXor1>(k), 0);
}

// Sorts the wave's 64 keys descending (lane 0 holds the largest).
__device__ __forceinline__ void wave_sort_desc(uint32_t& hi, uint32_t& lo) {
  bitonic_stage<2, 1>(hi, lo);
  bitonic_stage<4, 2>(hi, lo);
  bitonic_stage<4, 1>(hi, lo);
  bitonic_stage<8, 4>(hi, lo);
  bitonic_stage<8, 2>(hi, lo);
  bitonic_stage<8, 1>(hi, lo);
  bitonic_stage<16, 8>(hi, lo);
  bitonic_stage<16, 4>(hi, lo);
  bitonic_stage<16, 2>(hi, lo);
  bitonic_stage<16, 1>(hi, lo);
  bitonic_stage<32, 16>(hi, lo);
  bitonic_stage<32, 8>(hi, lo);
  bitonic_stage<32, 4>(hi, lo);
  bitonic_stage<32, 2>(hi, lo);
  bitonic_stage<32, 1>(hi, lo);
  bitonic_stage<64, 32>(hi, lo);
  bitonic_stage<64, 16>(hi, lo);
  bitonic_stage<64, 8>(hi, lo);
  bitonic_stage<64, 4>(hi, lo);
  bitonic_stage<64, 2>(hi, lo);
  bitonic_stage<64, 1>(hi, lo);
}

// Merges a descending 64-key list held one key per lane (hi, lo) with the
// descending list b (one key per lane) and keeps the 64 largest, descending:
// the elementwise maximum of one list and the other reversed holds the 64
// best of both as a bitonic sequence, which six half-cleaner stages sort.
__device__ __forceinline__ void wave_merge_desc(uint32_t& ah, uint32_t& al, uint64_t b) {
  const uint32_t bh = lane_rev((uint32_t)(b >> 32)), bl = lane_rev((uint32_t)b);
  const bool tb = (((uint64_t)bh << 32) | bl) > (((uint64_t)ah << 32) | al);
  ah = tb ? bh : ah;
  al = tb ? bl : al;
  bitonic_stage<64, 32>(ah, al);
  bitonic_stage<64, 16>(ah, al);
  bitonic_stage<64, 8>(ah, al);
  bitonic_stage<64, 4>(ah, al);
  bitonic_stage<64, 2>(ah, al);
  bitonic_stage<64, 1>(ah, al);
}

// Wave reductions; the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  v = min(v, dpp<kDppXor1>(v));
  v = min(v, dpp<kDppXor2>(v));
  v = min(v, dpp<kDppHalfMirror>(v));
  v = min(v, dpp<kDppMirror>(v));
  return min(min(readlane(v, 0), readlane(v, 16)), min(readlane(v, 32), readlane(v, 48)));
}
// Wave-wide max / sum: four butterfly steps inside each 16-lane row, then two
// row broadcasts (row_bcast:15 into rows 1 and 3, row_bcast:31 into rows 2
// and 3) leave the total in lane 63, each step one VALU instruction with its
// DPP operand fused (the s_nop 1 covers the two wait states a DPP read needs
// after a VALU write). Fixed pattern: every call combines in the same order,
// so results are reproducible bit for bit.
__device__ __forceinline__ float wave_max_f32(float x) {
  float r;
  asm volatile(
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_readlane_b32 %0, %1, 63"
      : "=s"(r), "+v"(x));
  return r;
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  float r;
  asm volatile(
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_add_f32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_readlane_b32 %0, %1, 63"
      : "=s"(r), "+v"(x));
  return r;
}
__device__ __forceinline__ int wave_sum_i32(int x) {
  uint32_t v = (uint32_t)x;
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  v += dpp<kDppHalfMirror>(v);
  v += dpp<kDppMirror>(v);
  return (int)(readlane(v, 0) + readlane(v, 16) + readlane(v, 32) + readlane(v, 48));
}

// Largest of the 64 lanes' unsigned values, as a scalar (the DPP pattern of
// wave_max_f32).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  uint32_t r;
  asm volatile(
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 row_mirror row_mask:0xf bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_max_u32_dpp %1, %1, %1 row_bcast:31 row_mask:0xc bank_mask:0xf\n\t"
      "s_nop 1\n\t"
      "v_readlane_b32 %0, %1, 63"
      : "=s"(r), "+v"(x));
  return r;
}

// m-th largest of the lanes' values among lanes with valid set (wave-uniform;
// 0 when fewer than m lanes are valid). For m <= 8 the largest remaining
// value is taken out m times at most (all lanes holding it at once, their
// count added up); otherwise a bit-by-bit search on ballots.
__device__ __forceinline__ uint32_t wave_mth_largest(uint32_t v, bool valid, int m, int nbits) {
  const uint64_t vm = __builtin_amdgcn_ballot_w64(valid);
  uint32_t t = 0;
  if (m <= 8) {
    v = valid ? v : 0u;
    int have = 0;
    for (int it = 0; it < m; ++it) {
      t = wave_max_u32(v);
      have += __popcll(__builtin_amdgcn_ballot_w64(v == t) & vm);
      if (have >= m || t == 0u) break;
      v = v == t ? 0u : v;
    }
    return have >= m ? t : 0u;
  }
  for (int b = nbits - 1; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    const int n = __popcll(__builtin_amdgcn_ballot_w64(v >= c) & vm);
    if (n >= m) t = c;
  }
  return t;
}

// The same through the 64-lane sort network (21 DPP / permlane stages, no
// SALU round trips), for m above 8. All 64 lanes must be active.
__device__ __forceinline__ uint32_t wave_mth_largest_sorted(uint32_t v, bool valid, int m) {
  uint32_t k = valid ? v : 0u;
  wave_sort_desc32(k);
  return readlane(k, m - 1);
}

// Coalesced weight fragments. The MFMA operand layout puts 16 different rows
// on adjacent lanes (lane n + 16c: row n, 16-byte chunk c), so a direct load
// touches a cache line per lane. Loading instead with lane 4n + c reading
// chunk c of row n makes each 4-lane group read one 64-byte segment; four
// ds_bpermute then move each lane's 16 bytes to its operand lane.
__device__ __forceinline__ int coal_row(int lane) { return lane >> 2; }
// rows 8..15 take their chunks in the order 2, 3, 0, 1, so that each 32-lane
// half of a permute reads 32 different source lanes modulo 32 (no LDS bank
// conflicts); every 4-lane group still reads one 64-byte segment
__device__ __forceinline__ int coal_col(int lane) { return ((lane & 3) ^ ((lane >> 5) << 1)) * 8; }
__device__ __forceinline__ u16x8_t to_mfma_lanes(u16x8_t v, int lane) {
  const int n = lane & 15, c = lane >> 4;
  const int src = (n * 4 + (c ^ ((n >> 3) << 1))) * 4;   // byte index of the lane that loaded row n, chunk c
  const u32x4_t x = __builtin_bit_cast(u32x4_t, v);
  u32x4_t y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)x[i]);
  return __builtin_bit_cast(u16x8_t, y);
}

// Inclusive prefix sum over the 64 lanes: shifts by 1, 2, 4 and 8 inside each
// 16-lane row (lanes without a source add zero), then row 0's total into row
// 1 and row 1's into rows 2 and 3 (row_bcast:15), then row 1's running total
// into rows 2 and 3 (row_bcast:31). All 64 lanes must be active.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// tanh(x) = 1 - 2 / (2^(2 x log2 e) + 1) on the hardware exp2 and reciprocal
// (each within about 1 ulp): absolute error a few 1e-7, saturating to +-1.
__device__ __forceinline__ float tanh_fast(float x) {
  const float e = __builtin_amdgcn_exp2f(x * 2.8853900817779268f);
  return __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(e + 1.f), 1.f);
}

// two fp32 values to fp16, rounding toward zero (v_cvt_pkrtz_f16_f32)
__device__ __forceinline__ h16x2_t pkrtz(float a, float b) {
  typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(h16x2_t, (fp16x2_t)__builtin_amdgcn_cvt_pkrtz(a, b));
}

// 8 bf16 weights as fp16: exact for bf16 values of magnitude in [2^-17, 2^16)
// or zero; smaller ones are truncated by at most 2^-25; magnitudes of 2^16 or
// more are beyond fp16 and come out as +-65504 (rounding toward zero), so
// callers must keep such weights away (the block-decoding kernel's
// precondition)
__device__ __forceinline__ h16x8_t bf16x8_to_f16(u16x8_t x) {
  h16x8_t r;
#pragma unroll
  for (int i = 0; i < 8; i += 2) {
    const h16x2_t p = pkrtz(bf16_to_f32(x[i]), bf16_to_f32(x[i + 1]));
    r[i] = p.x;
    r[i + 1] = p.y;
  }
  return r;
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete when it arrives, its outstanding global loads (also those that
// write LDS directly) are not waited for. A wave that needs its direct-to-LDS
// loads published waits with vmcnt_zero() before the barrier. The wait and
// the barrier are one asm statement with a memory clobber, so no LDS access
// moves across it. (__syncthreads() would also wait for every outstanding
// global load that writes LDS.)
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void vmcnt_zero() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup-scope atomics on LDS-qualified addresses.
__device__ __forceinline__ int lds_add(LDS int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ unsigned lds_max(LDS unsigned* p, unsigned v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int lds_or(LDS int* p, int v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ uint32_t mbcnt64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ f32x4_t mfma_f16(const h16x8_t& a, const h16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_bf16(const u16x8_t& a, const u16x8_t& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Block-wide exact top-K of unique 64-bit keys (0 = empty) with an int
// payload carried along. All threads of the block must call these.
//
//   block_select = bound + select_compact (+ select_exact) + select_rank
//
// (1) Bound: each wave whose 64 lanes all hold a key takes the m-th largest of
//     its lane maxima (high 32 bits), m = ceil(K / such waves); at least K keys
//     reach the minimum tau of those values.
// (2) select_compact: keys with high word >= tau are compacted into LDS.
// (3) select_rank: survivors are ranked by counting, rank(i) = #{j : key_j >
//     key_i}, split over the whole block, and scattered to their ranks.
// (4) select_exact: if more than `cap` survive (massive ties, or no bound),
//     the K-th largest key is found by a bitwise search over the 64 bits and
//     exactly the keys at or above it are compacted.
//
// misc[0..7] must be zero on entry to a selection; select_rank leaves it zero.
// ---------------------------------------------------------------------------
struct SelSmem {
  LDS uint64_t* key;      // [cap]
  LDS int* pay;           // [cap]
  LDS uint64_t* out_key;  // [>= K]
  LDS int* out_pay;       // [>= K]
  LDS int* misc;          // [8]
  int cap;
};

// Compacts keys whose high word is >= thr_hi; returns the survivor count
// (which may exceed cap; then only the first cap are stored).
template <int EPT>
__device__ __forceinline__ int select_compact(const uint64_t (&k)[EPT], const int (&p)[EPT], uint32_t thr_hi, const SelSmem& sm) {
  const int lane = lane_id();
  uint64_t bal[EPT];
  int wtot = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bal[e] = __ballot(k[e] != 0ull && (uint32_t)(k[e] >> 32) >= thr_hi);
    wtot += __popcll(bal[e]);
  }
  int base = 0;
  if (lane == 0 && wtot) base = lds_add(&sm.misc[3], wtot);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (bal[e]) {
      if ((bal[e] >> lane) & 1ull) {
        const int pos = base + (int)mbcnt64(bal[e]);
        if (pos < sm.cap) {
          sm.key[pos] = k[e];
          sm.pay[pos] = p[e];
        }
      }
      base += __popcll(bal[e]);
    }
  }
  __syncthreads();
  return sm.misc[3];
}

// Exact fallback: compacts exactly the min(K, #keys) largest keys.
template <int EPT>
__device__ __forceinline__ int select_exact(const uint64_t (&k)[EPT], const int (&p)[EPT], int K, const SelSmem& sm) {
  const int tid = threadIdx.x, lane = lane_id();
  LDS int* misc = sm.misc;
  int ntot = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) ntot += __popcll(__ballot(k[e] != 0ull));
  if (tid == 0) { misc[1] = 0; misc[5] = 0; }
  __syncthreads();
  if (lane == 0 && ntot) lds_add(&misc[1], ntot);
  __syncthreads();
  const int need = min(K, misc[1]);
  uint64_t T = 0;
  for (int b = 63; b >= 0; --b) {
    const uint64_t c = T | (1ull << b);
    int n = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) n += __popcll(__ballot(k[e] != 0ull && k[e] >= c));
    if (lane == 0 && n) lds_add(&misc[5], n);
    __syncthreads();
    const int tot = misc[5];
    __syncthreads();
    if (tid == 0) misc[5] = 0;
    __syncthreads();
    if (tot >= need) T = c;
  }
  if (tid == 0) misc[3] = 0;
  __syncthreads();
  uint64_t bal[EPT];
  int wtot = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    bal[e] = __ballot(k[e] != 0ull && k[e] >= T);
    wtot += __popcll(bal[e]);
  }
  int base = 0;
  if (lane == 0 && wtot) base = lds_add(&misc[3], wtot);
  base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (bal[e]) {
      if ((bal[e] >> lane) & 1ull) {
        const int pos = base + (int)mbcnt64(bal[e]);
        sm.key[pos] = k[e];
        sm.pay[pos] = p[e];
      }
      base += __popcll(bal[e]);
    }
  }
  __syncthreads();
  return misc[3];
}

// Ranks ns (<= cap) compacted keys and scatters the K largest, descending, to
// out_key/out_pay; zero-fills out_key[n..K). Keys are distinct. A key's rank
// is the number of larger keys, counted by a group of G = 2^lg threads (up to
// 16, as many as the block holds) over segments of the keys and summed across
// the group's lanes by DPP; the group's first thread writes the key at its
// rank. Leaves misc zeroed for the next selection.
__device__ __forceinline__ int select_rank(int ns, int K, const SelSmem& sm) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  if (ns > 0) {
    int lg = 4;
    while (lg > 0 && (ns << lg) > nthr) --lg;
    const int G = 1 << lg;
    const int per = (ns + G - 1) >> lg;
    // passes of nthr threads (more than one only when ns > nthr, G = 1); the
    // trip count is the block's, so every lane reaches the group sum
    for (int t0 = 0; t0 < (ns << lg); t0 += nthr) {
      const int t = t0 + tid;
      const int x = t >> lg, seg = t & (G - 1);
      uint64_t kx = 0ull;
      uint32_t c = 0u;
      if (x < ns) {
        kx = sm.key[x];
        const int y0 = seg * per, y1 = min(ns, y0 + per);
        int y = y0;
        for (; y + 4 <= y1; y += 4) {
          const uint64_t k0 = sm.key[y], k1 = sm.key[y + 1], k2 = sm.key[y + 2], k3 = sm.key[y + 3];
          c += (k0 > kx ? 1u : 0u) + (k1 > kx ? 1u : 0u) + (k2 > kx ? 1u : 0u) + (k3 > kx ? 1u : 0u);
        }
        for (; y < y1; ++y) c += sm.key[y] > kx ? 1u : 0u;
      }
      if (G >= 2) c += lane_xor<1>(c);
      if (G >= 4) c += lane_xor<2>(c);
      if (G >= 8) c += lane_xor<4>(c);
      if (G >= 16) c += lane_xor<8>(c);
      if (x < ns && seg == 0 && (int)c < K) {
        sm.out_key[c] = kx;
        sm.out_pay[c] = sm.pay[x];
      }
    }
  }
  const int n_out = min(ns, K);
  for (int i = n_out + tid; i < K; i += nthr) sm.out_key[i] = 0ull;
  if (tid < 8) sm.misc[tid] = 0;
  __syncthreads();
  return n_out;
}

template <int EPT>
__device__ __forceinline__ int block_select(const uint64_t (&k)[EPT], const int (&p)[EPT], int K, int hi_bits, const SelSmem& sm) {
  const int lane = lane_id();
  LDS int* misc = sm.misc;
  uint32_t lmax = 0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) lmax = max(lmax, (uint32_t)(k[e] >> 32));
  const bool full = __ballot(lmax != 0u) == ~0ull;
  if (lane == 0 && full) lds_add(&misc[0], 1);
  __syncthreads();
  const int nwf = misc[0];
  if (nwf > 0) {
    const int m = (K + nwf - 1) / nwf;
    if (m <= kWave && full) {
      const uint32_t t = wave_mth_largest(lmax, true, m, hi_bits);
      if (lane == 0) {
        lds_max((LDS unsigned*)&misc[2], ~t);   // min of t, complemented
        misc[4] = 1;
      }
    }
  }
  __syncthreads();
  const uint32_t thr = misc[4] ? ~(uint32_t)misc[2] : 0u;
  int ns = select_compact<EPT>(k, p, thr, sm);
  if (ns > sm.cap) ns = select_exact<EPT>(k, p, K, sm);
  return select_rank(ns, K, sm);
}

// ---------------------------------------------------------------------------
// Sorted top-K by a value histogram, for K in the hundreds.
//
// Keys are unique and nonzero, 64-bit, with the value key in the high word.
// Only keys whose value key is >= lo_v take part; hi_v is >= every such value
// key. Each key falls in bin (value key - lo_v) >> shift, shift chosen so
// that hi_v lands in bin 255 or lower. The binning is monotone in the key, so
// counting down from the top bin finds the boundary bin b*: fewer than K keys
// lie above it and at least K at or above it (all keys when fewer than K take
// part). The keys of bin b* and above are scattered into buckets (one per
// bin, at its offset among the keys above), and each key is placed at its
// bucket's offset plus its rank within the bucket, counted against the
// bucket's other keys. Buckets hold one value each when the values span fewer
// than 256 keys, so the counting is short; the positions below K are the K
// largest keys in descending order. Out of the K slots, those past the number
// of keys taking part are zero.
//
// Its barriers wait for LDS traffic only (outstanding global loads, e.g. a
// prefetch into registers, stay in flight). hist and cursor must be zero on
// entry. Returns false, with only hist,
// cursor, base and misc written, when the keys of bin b* and above exceed cap
// (massive ties); the caller then selects by another route.
// ---------------------------------------------------------------------------
struct HistSmem {
  LDS int* hist;         // [256]
  LDS int* cursor;       // [256]
  LDS int* base;         // [256]
  LDS int* misc;         // [2]
  LDS uint64_t* bucket;  // [cap]
  LDS uint64_t* out;     // [>= K]
  int cap;
};

// Bin shift for value keys in [lo_v, hi_v]: the span lands in bin 255 or lower.
__device__ __forceinline__ int hist_shift(uint32_t lo_v, uint32_t hi_v) {
  const uint32_t span = hi_v > lo_v ? hi_v - lo_v : 0u;
  const int nb = span ? 32 - __builtin_clz(span) : 0;
  return nb > 8 ? nb - 8 : 0;
}
__device__ __forceinline__ int hist_bin(uint32_t hv, uint32_t lo_v, int shift) {
  return (int)min(255u, (hv - lo_v) >> shift);
}

// With hist complete: wave 0 writes each bin's offset among the keys above
// it (base) and the boundary bin b* and the count of keys in b* and above
// (misc[0..1]). The caller syncs afterwards.
__device__ __forceinline__ void hist_boundary(int K, const HistSmem& sm) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    // lane l holds bins 255 - 4l .. 252 - 4l, so lanes run from the top bin down
    const int b0 = 255 - 4 * tid;
    const int h0 = sm.hist[b0], h1 = sm.hist[b0 - 1], h2 = sm.hist[b0 - 2], h3 = sm.hist[b0 - 3];
    const int s = h0 + h1 + h2 + h3;
    const int inc = wave_incl_scan_i32(s);
    const int a0 = inc - s, a1 = a0 + h0, a2 = a1 + h1, a3 = a2 + h2;
    const int total = (int)readlane((uint32_t)inc, kWave - 1);
    const int kk = min(K, total);
    sm.base[b0] = a0;
    sm.base[b0 - 1] = a1;
    sm.base[b0 - 2] = a2;
    sm.base[b0 - 3] = a3;
    if (kk == 0) {
      if (tid == 0) { sm.misc[0] = 256; sm.misc[1] = 0; }
    } else {
      // exactly one bin has above < kk <= above + count
      if (a0 < kk && kk <= a1) { sm.misc[0] = b0; sm.misc[1] = a1; }
      if (a1 < kk && kk <= a2) { sm.misc[0] = b0 - 1; sm.misc[1] = a2; }
      if (a2 < kk && kk <= a3) { sm.misc[0] = b0 - 2; sm.misc[1] = a3; }
      if (a3 < kk && kk <= a3 + h3) { sm.misc[0] = b0 - 3; sm.misc[1] = a3 + h3; }
    }
  }
}

// One key into its bucket when its bin is b* or above.
__device__ __forceinline__ void hist_scatter(uint64_t x, int bin, int bstar, const HistSmem& sm) {
  if (bin >= bstar) {
    const int slot = lds_add(&sm.cursor[bin], 1);
    sm.bucket[sm.base[bin] + slot] = x;
  }
}

// With the buckets filled: each key at its bucket's offset plus its rank in
// the bucket; the positions below K are the K largest, descending; zeros
// past narea. Ends with a sync.
__device__ __forceinline__ void hist_rank_out(int K, uint32_t lo_v, int shift, int narea, const HistSmem& sm) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  for (int p = tid; p < narea; p += nthr) {
    const uint64_t x = sm.bucket[p];
    const int b = hist_bin((uint32_t)(x >> 32), lo_v, shift);
    const int lo = sm.base[b], hi = lo + sm.hist[b];
    int r = 0, q = lo;
    for (; q + 4 <= hi; q += 4) {
      const uint64_t y0 = sm.bucket[q], y1 = sm.bucket[q + 1], y2 = sm.bucket[q + 2], y3 = sm.bucket[q + 3];
      r += (y0 > x ? 1 : 0) + (y1 > x ? 1 : 0) + (y2 > x ? 1 : 0) + (y3 > x ? 1 : 0);
    }
    for (; q < hi; ++q) r += sm.bucket[q] > x ? 1 : 0;
    if (lo + r < K) sm.out[lo + r] = x;
  }
  for (int i = narea + tid; i < K; i += nthr) sm.out[i] = 0ull;
  lds_sync();
}

template <int EPT>
__device__ __forceinline__ bool hist_topk(const uint64_t (&k)[EPT], uint32_t lo_v, uint32_t hi_v, int K,
                                          const HistSmem& sm) {
  const int shift = hist_shift(lo_v, hi_v);
  int bin[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    const uint32_t hv = (uint32_t)(k[e] >> 32);
    bin[e] = (k[e] != 0ull && hv >= lo_v) ? hist_bin(hv, lo_v, shift) : -1;
    if (bin[e] >= 0) lds_add(&sm.hist[bin[e]], 1);
  }
  lds_sync();
  hist_boundary(K, sm);
  lds_sync();
  const int bstar = sm.misc[0], narea = sm.misc[1];
  if (narea > sm.cap) return false;
#pragma unroll
  for (int e = 0; e < EPT; ++e) hist_scatter(k[e], bin[e], bstar, sm);
  lds_sync();
  hist_rank_out(K, lo_v, shift, narea, sm);
  return true;
}

}  // namespace dartree
