// Small gfx950 (CDNA4) building blocks shared by the gradient kernels:
// vector types, a 16-byte-chunk XOR swizzle for LDS tiles that serves both
// row reads (MFMA A operand, ds_read_b128) and transposed reads
// (ds_read_b64_tr_b16), and a tile copy HBM -> LDS by buffer_load ... lds.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cdna4 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Swizzle of an LDS tile with rows of D bf16 (2D bytes, 2D/16 chunks of 16
// bytes): chunk c of row r is stored at chunk c ^ swz<D>(r).
//   * Row reads: 16 consecutive rows read the same logical chunk; the mask
//     takes 16 (d=128) or 8 (d=64, two rows per 256-byte bank line) distinct
//     values over them, so the 16 lanes hit distinct banks.
//   * Transposed reads: 4 consecutive rows (a multiple of 4 first) read 32
//     or 64 bytes each; the mask moves each row by whole 64-byte groups, so
//     the rows land in distinct bank groups.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Byte offset, within a tile of rows of D bf16, of 16-byte logical chunk c of row r.
template <int D>
__host__ __device__ constexpr int chunk_off(int r, int c) {
  return r * 2 * D + ((c ^ swz<D>(r)) << 4);
}

// Row-read operand (MFMA 32x32x16 A operand, or a B operand laid out the
// same way): lane l gets row row0 + l%32, elements 16 ks + 8 (l/32) .. +7.
template <int D>
__device__ __forceinline__ bf16x8 row_operand(const char* tile, int row0, int ks, int lane) {
  const int r = row0 + (lane & 31);
  return *reinterpret_cast<const bf16x8*>(tile + chunk_off<D>(r, 2 * ks + (lane >> 5)));
}

// Transposed operand over 16 rows of a tile, for one 32-column block:
// A[i][k] = tile[row0 + perm(k)][32 ct + i] where the row order perm matches
// the 32x32 accumulator layout (the rows lane-half h holds are
// 4h + {0..3} and 8 + 4h + {0..3}).  Lane a of each 16-lane group points at
// row a/4 of a 4-row group and columns cbase + 4(a%4); the transposed read
// hands it column cbase + a of those 4 rows.
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, int row0, int ct, int lane) {
  const int a = lane & 15, cg = (lane >> 4) & 1, h = lane >> 5;
  const int r = row0 + 4 * h + (a >> 2);
  const int col = 32 * ct + 16 * cg + 4 * (a & 3);              // first of 4 bf16
  const char* p0 = tile + chunk_off<D>(r, col >> 3) + 2 * (col & 7);
  const char* p1 = tile + chunk_off<D>(r + 8, col >> 3) + 2 * (col & 7);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1);
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy of rows [row0, row0 + ROWS) of one head's [N][D] bf16 matrix into a
// swizzled LDS tile, by THREADS threads; each issue moves 1 KiB per wave
// (16 bytes per lane).  The buffer starts at row row0 and ends at row `end`:
// rows past it read as zeros, with no branch.
template <int D, int ROWS, int THREADS>
struct TileCopy {
  static constexpr int kBytes = ROWS * 2 * D;
  static constexpr int kIssues = kBytes / (THREADS * 16);
  static_assert(kIssues * THREADS * 16 == kBytes, "tile is not a whole number of copies");
  unsigned voff;     // global byte offset (within the tile) this lane fetches for issue 0

  __device__ __forceinline__ void init(int tid) {
    constexpr int kChunks = 2 * D / 16;
    const int r = tid / kChunks, pc = tid % kChunks;
    voff = (unsigned)(r * 2 * D + ((pc ^ swz<D>(r)) << 4));
  }

  // Issue i moves the LDS bytes [i THREADS 16, (i+1) THREADS 16); the
  // swizzle depends on the row modulo 16, which a step of THREADS 16 bytes
  // (a multiple of 16 rows) does not change.
  __device__ __forceinline__ void issue(const char* head, int row0, int end, char* dst, int tid, int i) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int rows = max(end - row0, 0);
    const char* base = head + (size_t)min(row0, end) * (2 * D);
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, rows * 2 * D, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + i * THREADS * 16 + (tid & ~63) * 16), 16,
                                             voff + i * THREADS * 16, 0, 0, 0);
#endif
  }
};

// Copy of floats [row0, row0 + 64) of one head's [N] fp32 vector into LDS
// (one wave, 4 bytes per lane); entries at or past `end` read as zeros.
__device__ __forceinline__ void copy_row_stats(const float* head, int row0, int end, char* dst, int lane) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int rows = max(end - row0, 0);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)(head + min(row0, end)), 0, rows * 4, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)dst, 4, lane * 4, 0, 0, 0);
#endif
}

}  // namespace cdna4
