// Device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix-core conventions (checked on gfx950 with a layout probe):
//   v_mfma_f32_32x32x16_bf16: C[m][n] += sum_k A[m][k] B[k][n].
//     A operand, lane l: row m = l % 32, k = (l / 32) * 8 + j   (8 bf16)
//     B operand, lane l: col n = l % 32, k = (l / 32) * 8 + j   (8 bf16)
//     C/D, lane l, register i: row (i / 4) * 8 + (l / 32) * 4 + (i % 4), col l % 32.
//   v_mfma_f32_16x16x32_bf16: A lane l: row l % 16, k = (l / 16) * 8 + j;
//     B lane l: col l % 16, same k; C/D lane l, register i: row (l / 16) * 4 + i, col l % 16.
//   ds_read_tr16_b64: in each group of 16 lanes, output lane i, element e is
//     element (i % 4) of the 8 bytes addressed by lane 4 * e + i / 4 of the group.
//     Four lanes that address consecutive 8-byte pieces of one row give the
//     16 lanes one column each, so a row-major [key][d] tile is read as
//     key-contiguous operand registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// 16-byte-chunk XOR swizzle inside a row of D bf16 values.
// D = 128 (16 chunks, one row spans all 64 banks): the swizzle is a bijection
// of the row's low 4 bits, so 16 lanes reading 16 distinct rows at one logical
// chunk touch 16 distinct chunks, and a transposed read of rows r..r+3 over 4
// adjacent chunks also touches 16 distinct chunks.
// D = 64 (8 chunks, two rows per bank line): rows r, r+1 share a bank line,
// so the chunk is XORed with bits 1..3 of the row.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  if constexpr (D == 128) {
    return chunk ^ (((row & 3) << 2) | ((row >> 2) & 3));
  } else {
    return chunk ^ ((row >> 1) & 7);
  }
}

// Row permutation inside a 32-row block of the score tile: swapping bits 2
// and 3 makes the score accumulator of a 32x32 MFMA hold, in registers
// 8h..8h+7 of lane l, the eight consecutive keys 16h + 8(l/32) .. +7. Those
// registers are then directly the B operand (key-contiguous) of the P.V MFMA.
__device__ __forceinline__ int kappa(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// max(x, x of lane ^ 32) with one v_permlane32_swap (no LDS round trip).
// Maximum that propagates NaN (IEEE 754-2019 maximum). Unlike fmaxf it needs
// no canonicalising of MFMA results first, and gfx950 does three operands in
// one v_maximum3_f32.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max_with_lane_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// x + x of lane ^ 32 with one v_permlane32_swap; the same value in both lanes.
__device__ __forceinline__ float sum_with_lane_xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max(x, x of lane ^ 16) with one v_permlane16_swap.
__device__ __forceinline__ float max_with_lane_xor16(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 32-bit LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(__attribute__((address_space(3))) const void*)p;
}

// Direct global -> LDS copies of 16 bytes per lane: lane l's bytes land at
// LDS byte `lds_base + 16 l` (lds_base must be wave-uniform). Issued through
// inline assembly so that the compiler does not make every later LDS read
// wait for these copies; callers wait with wait_vmcnt0() before the barrier
// that publishes the data.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

// Debug builds with FA_LDS_POISON: before a copy is issued, the 16 bytes it
// will write are set to all-ones (NaN in bf16, fp32 and E4M3). A reader that
// runs ahead of the copy's wait and barrier, or lags behind the next copy into
// the same slot, then reads NaN, which reaches O and fails every parity test,
// instead of reading finite stale data.
__device__ __forceinline__ void lds_poison16(uint32_t lds_base) {
#ifdef FA_LDS_POISON
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  lds_u32x4* p = (lds_u32x4*)(size_t)(lds_base + 16u * (threadIdx.x & 63u));
  *p = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#else
  (void)lds_base;
#endif
}

// Same copy with a wave-uniform 64-bit global base in SGPRs and a 32-bit
// per-lane byte offset (no per-lane 64-bit address arithmetic).
__device__ __forceinline__ void dma16_sbase(const void* sbase, uint32_t voff, uint32_t lds_base) {
  lds_poison16(lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for rows read exactly once (the
// query rows of a block).
__device__ __forceinline__ void dma16_sbase_nt(const void* sbase, uint32_t voff, uint32_t lds_base) {
  lds_poison16(lds_base);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Cooperative copy of a [rows x D] bf16 tile from global memory (row-major,
// row stride D) into registers, 16 bytes per thread per step, then into LDS
// (swizzled). Rows at or past `nvalid` read as zero and are never fetched.
template <int D, int ROWS, int NT>
struct TileCopy {
  static constexpr int CHUNKS = D / 8;
  static constexpr int PER_T = ROWS * CHUNKS / NT;
  static_assert(ROWS * CHUNKS % NT == 0, "tile must split evenly over threads");
  u32x4 r[PER_T];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ src, int nvalid, int tid) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + i * NT;
      const int row = id / CHUNKS, ch = id % CHUNKS;
      if (row < nvalid) {
        r[i] = *reinterpret_cast<const u32x4*>(src + (size_t)row * D + ch * 8);
      } else {
        r[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int id = tid + i * NT;
      const int row = id / CHUNKS, ch = id % CHUNKS;
      *reinterpret_cast<u32x4*>(lds + row * D + swz<D>(row, ch) * 8) = r[i];
    }
  }
};

// A operand (K rows, 8 d values) of the score MFMA S^T = K Q^T for the 32-row
// block starting at tile row `r0`, k-step `s` (d = 16 s .. 16 s + 15).
template <int D>
__device__ __forceinline__ bf16x8 load_k_operand(const uint16_t* lds, int r0, int s, int lane) {
  const int row = r0 + kappa(lane & 31);
  const int ch = s * 2 + (lane >> 5);
  return *reinterpret_cast<const bf16x8*>(lds + row * D + swz<D>(row, ch) * 8);
}

// A operand (V^T: d row, 8 consecutive keys) of the MFMA O^T += V^T P^T for
// d block `db` (d = 32 db .. 32 db + 31) and keys kb + 8 (lane / 32) + 0..7,
// read with two transposing LDS reads from the row-major [key][d] tile.
template <int D>
__device__ __forceinline__ bf16x8 load_vt_operand(const uint16_t* lds, int kb, int db, int lane) {
  const int grp = lane >> 4, w = lane & 15;
  const int e = w >> 2, j = w & 3;
  const int row0 = kb + (lane >> 5) * 8 + e;
  const int ch = db * 4 + (grp & 1) * 2 + (j >> 1);
  const int sub = (j & 1) * 4;
  const uint16_t* p0 = lds + row0 * D + swz<D>(row0, ch) * 8 + sub;
  const uint16_t* p1 = lds + (row0 + 4) * D + swz<D>(row0 + 4, ch) * 8 + sub;
  bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p0));
  bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p1));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Global key index held by lane `lane`, register i of the score accumulator of
// the 32-row block starting at tile row r0 (after the kappa permutation).
__device__ __forceinline__ int score_key(int r0, int i, int lane) {
  return r0 + (i >> 3) * 16 + (lane >> 5) * 8 + (i & 7);
}

// Two floats rounded to bf16 (nearest even), a in the low half: one
// v_cvt_pk_bf16_f32 (converting the halves separately and merging them costs
// three more instructions).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

}  // namespace fa
