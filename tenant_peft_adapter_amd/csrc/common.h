// Shared device helpers for the gfx950 kernels: element types, 8-element
// operand fragments and the 16x16 MFMA step.
//
// Fragment convention (used by every MFMA kernel here).  One
// v_mfma_f32_16x16x32 step multiplies a 16x32 operand "a" by a 32x16 operand
// "b".  Lane l holds row (l % 16) of a and column (l % 16) of b, each as 8
// consecutive k values starting at k = 8 * (l / 16).  Both operands use the
// same k order, so any fixed permutation of k inside a step is harmless.
// The 4 fp32 results of lane l are D[4 * (l / 16) + v][l % 16], v = 0..3.
//
// Kernels compute D = W_tile · X_tileᵀ (a = weight rows = output columns,
// b = input rows), so a lane ends up holding output columns of one input
// row.  With NB column blocks per wave, block b's a-row i is mapped to the
// output column 4·NB·(i / 4) + 4·b + (i % 4): lane l then holds the 4·NB
// consecutive columns [4·NB·(l / 16), 4·NB·(l / 16 + 1)) of row l % 16, so
// epilogues load and store contiguous runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpa {

typedef _Float16 f16;
typedef __bf16 bf16;
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <typename T>
struct Frag;
template <>
struct Frag<f16> {
  typedef f16x8 V;
};
template <>
struct Frag<bf16> {
  typedef bf16x8 V;
};
template <>
struct Frag<float> {
  typedef f32x8 V;
};

// Loads through a global-address-space pointer.  Pointers read from device
// memory (the slot records' fields) are generic to the compiler, which then
// emits flat loads; those count against both the vector-memory and the LDS /
// scalar counters, so every wait on them drains both.  All operands loaded
// this way live in device global memory.
#define TPA_GLOBAL __attribute__((address_space(1)))
template <typename V, typename T>
__device__ __forceinline__ V gload(const T* p) {
  return *(const TPA_GLOBAL V*)(p);
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::V load_frag(const T* p) {
  return gload<typename Frag<T>::V>(p);
}

template <typename T>
__device__ __forceinline__ typename Frag<T>::V zero_frag() {
  typename Frag<T>::V v = {};
  return v;
}

__device__ __forceinline__ f32x4 mma(f32x4 acc, f16x8 a, f16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma(f32x4 acc, f32x8 a, f32x8 b) {
#pragma unroll
  for (int t = 0; t < 8; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[t], b[t], acc, 0, 0, 0);
  return acc;
}

template <typename T>
__device__ __forceinline__ T to_t(float v);
template <>
__device__ __forceinline__ f16 to_t<f16>(float v) {
  return (f16)v;
}
template <>
__device__ __forceinline__ bf16 to_t<bf16>(float v) {
  return (bf16)v;
}
template <>
__device__ __forceinline__ float to_t<float>(float v) {
  return v;
}

template <typename T>
__device__ __forceinline__ float to_f(T v) {
  return (float)v;
}

// s_waitcnt operand that waits for vmcnt <= n and nothing else (gfx9 layout:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at
// their maxima).  The direct global-to-LDS loads count as vector loads.
constexpr unsigned waitcnt_vm(int n) { return (unsigned)((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14)); }

// Chunk permutation of the direct-load kernels' 128-byte LDS rows: chunk c
// of row r is stored at c ^ swz<SH>(r), so that the fragment reads (16 rows,
// one chunk each) hit distinct bank groups: with l = r & 3 and h = bits SH,
// SH+1 of the row (the lane's i >> 2 under perm_col), any 8 lanes differ in
// (row * 128 + 16 * chunk) mod 128 and any 16 lanes in that mod 256.
template <int SH>
__device__ __forceinline__ int swz(int r) {
  const int l = r & 3, h = (r >> SH) & 3;
  return ((l >> 1) & 1) | ((h & 1) << 1) | ((((h >> 1) ^ l) & 1) << 2);
}

// 16 consecutive elements of one row, to or from fp32 registers.
template <typename T>
__device__ __forceinline__ void load_run16(const T* src, float* v) {
  typename Frag<T>::V lo = *reinterpret_cast<const typename Frag<T>::V*>(src);
  typename Frag<T>::V hi = *reinterpret_cast<const typename Frag<T>::V*>(src + 8);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    v[j] = to_f<T>(lo[j]);
    v[8 + j] = to_f<T>(hi[j]);
  }
}
template <>
__device__ __forceinline__ void load_run16<float>(const float* src, float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x4 x = *reinterpret_cast<const f32x4*>(src + 4 * q);
    v[4 * q] = x[0];
    v[4 * q + 1] = x[1];
    v[4 * q + 2] = x[2];
    v[4 * q + 3] = x[3];
  }
}
template <typename T>
__device__ __forceinline__ void store_run16(T* dst, const float* v) {
  typename Frag<T>::V lo, hi;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    lo[j] = to_t<T>(v[j]);
    hi[j] = to_t<T>(v[8 + j]);
  }
  *reinterpret_cast<typename Frag<T>::V*>(dst) = lo;
  *reinterpret_cast<typename Frag<T>::V*>(dst + 8) = hi;
}
template <>
__device__ __forceinline__ void store_run16<float>(float* dst, const float* v) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<f32x4*>(dst + 4 * q) = f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
}

// Output column, within a wave's group of 16*NB columns, of a-row i of
// column block b (see the file comment).
template <int NB>
__device__ __forceinline__ int perm_col(int i, int b) {
  return 4 * NB * (i >> 2) + 4 * b + (i & 3);
}

// Barrier that waits for this wave's LDS operations only (the callers
// exchange data through LDS, never through global memory).
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Inclusive prefix sum across the 64 lanes of a wave in registers: four
// row shifts (within each 16-lane row), then the last lane of row 0 and 2
// added into rows 1 and 3, then lane 31 into rows 2 and 3.  Lanes whose
// source lies outside the row keep the identity (0).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Term class of a slot, as ordered by the row plan.
enum { CLS_OWNED = 0, CLS_SHARED = 1, CLS_NONE = 2 };

// Per-slot device record: what a row of this slot needs in the hot path.
// cls < 0 marks a slot that is not loaded.
struct SlotDev {
  int32_t cls;        // CLS_OWNED / CLS_SHARED / CLS_NONE, or -1
  int32_t rank;       // rank of the owned term (CLS_OWNED)
  int32_t has_R;      // OFT rotation present
  int32_t oft_block;  // block size of R
  const void* A;      // owned: c·A as [rank][d_in]
  const void* Bt;     // owned: B diag(e) as [d_out][rank]
  const float* s;     // output scale [d_out] or null
  const float* b;     // output shift [d_out] or null
  const float* d;     // VeRA inner vector c·d [r_v] or null
  const float* e;     // VeRA outer vector [d_out] or null
  const void* Rt;     // OFT blocks, each stored transposed: [d_in / bs][bs][bs]
};

// Workspace counters written by the plan kernel.
enum {
  CNT_NSEG = 0,
  CNT_NTILES = 1,
  CNT_NOFT = 2,
  CNT_INVALID = 3,
  CNT_CLASS0 = 4,  // class_ptr[0..3] at 4..7
  CNT_WORDS = 16
};

}  // namespace tpa
