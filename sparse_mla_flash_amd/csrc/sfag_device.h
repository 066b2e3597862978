// sfag_device.h -- gfx950 device helpers shared by the SparseFlashAttentionGrad kernels.
//
// MFMA shape: v_mfma_f32_16x16x32_bf16 / _f16 (one wave, 64 lanes).  Operand lane layout,
// with g = lane / 16 and c = lane % 16:
//   A (16 x 32, M x K): lane holds A[c][8g + e], e = 0..7
//   B (32 x 16, K x N): lane holds B[8g + e][c]
//   C (16 x 16):        lane holds C[4g + v][c], v = 0..3
//
// LDS tiles are row-major bf16 with a row length that is a multiple of 64 elements,
// split into 16-byte chunks; chunk index j of row r is stored at j ^ (r & 7) (XOR
// swizzle inside aligned groups of 8 chunks) so that 16 lanes reading the same
// column chunk of 16 different rows hit different banks.
//
// ds_read_b64_tr_b16 (transpose read): inside each 16-lane group, lane i receives,
// for r = 0..3, element (i % 4) of the 4-element piece addressed by lane 4r + i/4.
// Pointing lane j at X[k0 + j/4][n0 + 4 (j % 4)] therefore hands lane i the column
// X[k0 .. k0+3][n0 + i]: a row-major (K x N) tile read as MFMA B fragments, or a
// row-major (K x M) tile read as A fragments of its transpose.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sfag {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte copies kept in VGPRs
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kDn = 512;          // nope width
constexpr int kDr = 64;           // rope width
constexpr int kDk = kDn + kDr;    // gathered key row width
constexpr int kDacc = kDk + kDn;  // fp32 accumulator row: dK | dKRope | dV

// Compile-time loop: calls f(std::integral_constant<int, I>) for I = B .. E-1, so register
// arrays indexed inside the body see constant indices before scalar replacement runs.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Element type of the 16-bit tensors: bf16 (F16 = false) or fp16 (F16 = true).  Fragments are
// carried as bf16x8 bit patterns either way; the MFMA reinterprets them.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool F16>
__device__ __forceinline__ f32x4 mfma_t(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// element offset of (row, col) in a swizzled tile whose rows hold `row_chunks` 16-byte chunks
__device__ __forceinline__ int swz(int row, int col, int row_chunks) {
  const int chunk = col >> 3;
  return row * row_chunks * 8 + ((chunk ^ (row & 7)) << 3) + (col & 7);
}

__device__ __forceinline__ bf16x8 lds_read8(const uint16_t* tile, int row, int col, int row_chunks) {
  return *reinterpret_cast<const bf16x8*>(tile + swz(row, col, row_chunks));
}

__device__ __forceinline__ i16x4 lds_tr4(const uint16_t* tile, int row, int col, int row_chunks) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + swz(row, col, row_chunks)));
}

// Fragment (K = 32 rows k0 + 8g .. k0 + 8g + 7, column n0 + c) of a row-major tile, via two
// transpose reads.  Works for B fragments of X[k][n] and for A fragments of X^T.
__device__ __forceinline__ bf16x8 lds_frag_tr(const uint16_t* tile, int k0, int n0, int row_chunks,
                                              int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int r = k0 + 8 * g + (j >> 2);
  const int col = n0 + 4 * (j & 3);
  const i16x4 lo = lds_tr4(tile, r, col, row_chunks);
  const i16x4 hi = lds_tr4(tile, r + 4, col, row_chunks);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Padded (unswizzled) tiles: element (row, col) at row * pitch + col.  With a pitch of
// 584 (576 + 8) or 72 (64 + 8) elements consecutive rows start 36 or 4 banks apart, so 16
// lanes reading the same 16-byte column of 16 rows hit distinct banks, and every address is
// a per-lane base plus a compile-time offset.
__device__ __forceinline__ bf16x8 lds_read8p(const uint16_t* tile, int row, int col, int pitch) {
  return *reinterpret_cast<const bf16x8*>(tile + row * pitch + col);
}

__device__ __forceinline__ bf16x8 lds_frag_trp(const uint16_t* tile, int k0, int n0, int pitch, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = tile + (k0 + 8 * g + (j >> 2)) * pitch + n0 + 4 * (j & 3);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * pitch));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// Workgroup barrier for data exchanged through LDS by ds_write / ds_read only: waits for this
// wave's LDS instructions (lgkmcnt(0); vmcnt and expcnt left at their maximum) but, unlike
// __syncthreads(), not for global loads, stores or direct-to-LDS loads still in flight.  The
// caller guarantees that no LDS location read after it is the target of a direct-to-LDS load
// still in flight.  The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// B fragment of a 16x16x32 MFMA (lane (g, c): rows 8 g .. 8 g + 7 of column n0 + c) from a
// chunk-major tile: element (row k, column n) at ((n / 8) * 32 + k) * 8 + n % 8, i.e. 16-byte
// chunks of 8 columns stored [column chunk][32 rows]; two transposing reads.
__device__ __forceinline__ bf16x8 lds_frag_tr_cm(const uint16_t* tile, int n0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const int k = 8 * g + (j >> 2), n = n0 + 4 * (j & 3);
  const uint16_t* p = tile + ((n >> 3) * 32 + k) * 8 + (n & 7);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 4 * 8));
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// MFMA fragment from two transposing reads at P and P + HI (elements): lane i of each 16-lane
// group gets the 4 elements of the first read, then the 4 of the second (see the note on
// ds_read_b64_tr_b16 above).  The caller points every lane at its own base.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* p, int hi) {
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
  const i16x4 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + hi));
  const i16x8 v = __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ uint16_t f2bf(float f) {
  // round to nearest even; NaN stays NaN
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Two floats rounded to nearest even bf16 by the hardware conversion (v_cvt_pk_bf16_f32), lo in
// bits 0..15.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// The same for either element type: fp16 by v_cvt_f16_f32 (nearest even in the default mode;
// out-of-range values become infinities).
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
template <bool F16>
__device__ __forceinline__ uint32_t pack_x2(float lo, float hi) {
  if constexpr (F16) {
    const f16x2_t v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
  } else {
    return pack_bf16x2(lo, hi);
  }
}

template <bool F16>
__device__ __forceinline__ uint16_t f2x(float f) {
  if constexpr (F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  else return f2bf(f);
}

template <bool F16>
__device__ __forceinline__ float x2f(uint16_t b) {
  if constexpr (F16) return (float)__builtin_bit_cast(_Float16, b);
  else return bf2f(b);
}

// Geometry of one query row.  BSND: batch b = row / S1, keys of batch b start at b * S2.
// TND: `cum` (LDS, filled by cum_lengths) holds the first query row of every sequence in
// cum[0..B] and the first key row in cum[257..257+B].
struct RowGeo {
  int b, i, lq, lkv;
  int64_t kstart;
  int hi;        // largest valid key position (inclusive); -1 = none
  bool active;
};

template <typename Lens>
__device__ __forceinline__ void cum_lengths(const Lens& L, int B, int32_t* cum) {
  for (int t = threadIdx.x; t <= B; t += blockDim.x) {
    int32_t sq = 0, skv = 0;
    for (int b = 0; b < t; ++b) {
      sq += L.lq[b];
      skv += L.lkv[b];
    }
    cum[t] = sq;
    cum[257 + t] = skv;
  }
}

template <typename Lens>
__device__ __forceinline__ RowGeo row_geo(const Lens& L, const int32_t* cum, int B, int tnd,
                                          int64_t S1, int64_t S2, int64_t row, int mode3) {
  RowGeo r;
  int b;
  int64_t qstart;
  if (!tnd) {
    b = (int)(row / S1);
    qstart = (int64_t)b * S1;
    r.kstart = (int64_t)b * S2;
  } else {
    int lo = 0, hi = B - 1;  // last sequence whose first row <= row (empty ones share it)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)cum[mid] <= row) lo = mid; else hi = mid - 1;
    }
    b = lo;
    qstart = cum[b];
    r.kstart = cum[257 + b];
  }
  r.b = b;
  r.i = (int)(row - qstart);
  r.lq = L.lq[b];
  r.lkv = L.lkv[b];
  r.active = r.i < r.lq;
  int hi = r.lkv - 1;
  if (mode3) hi = min(hi, r.i + r.lkv - r.lq);
  r.hi = hi;
  return r;
}

// Key position named by slot s of a query row whose sparseIndices row is irow, with block
// selection (SparseFlashAttentionGrad README, "function description": each index selects a
// block of sparseBlockSize keys; index j covers key positions j * bs .. j * bs + bs - 1).  The
// row has topk * bs slots; slot s is key s % bs of block irow[s / bs].  Negative block indices
// give -1; positions past the key range stay out of range (the caller checks them against the
// row's valid range).
__device__ __forceinline__ int slot_key(const int32_t* irow, int s, int bs) {
  if (bs == 1) return irow[s];
  const int jb = irow[s / bs];
  if (jb < 0) return -1;
  return (int)min((int64_t)jb * bs + s % bs, (int64_t)0x7fffffff);
}

}  // namespace sfag
