// fa_rows.hpp -- output rows through LDS for the training kernels.
//
// After a transposed product (O^T, dQ^T, dK^T, dV^T in the MFMA C layout) a
// lane holds one output row in 8-byte pieces; stored straight to global
// memory, every store instruction would touch 32 rows with 16 bytes each.
// Instead each lane puts its pieces into a [rows][D] LDS tile with
// put_row4(), and after a barrier write_rows() sends whole rows to global
// memory with 16-byte stores, consecutive lanes on consecutive chunks (16
// lanes per 256-byte row at D = 128 in bf16).
//
// Tile layout: with PAD, rows are D*e + 16 bytes apart (row r starts 4 banks
// after row r-1); without it, rows are unpadded and the 16-byte chunks of
// row r are XOR-swizzled by the row's index among the rows that start on
// the same bank: r itself when a row spans all 64 banks (256 bytes), r / 2
// when it spans half of them (128 bytes, so rows alternate between the two
// halves).  Both keep the 8-byte writes of a half-wave (16 rows x 2 lanes)
// and the row reads of 16 lanes on distinct banks; PAD needs 16 more bytes
// per row of LDS.
#pragma once

#include "fa_common.hpp"

namespace fa {

template <typename T, int D, bool PAD>
struct RowTile {
  static constexpr int RBo = D * (int)sizeof(T);          // bytes of one output row
  static constexpr int CPR = RBo / 16;                    // 16-byte chunks per row
  static constexpr int RS = RBo + (PAD ? 16 : 0);         // row stride in the tile
  static constexpr int RPS = RBo >= 256 ? 1 : 256 / RBo;  // rows per 256-byte bank span
  __device__ static int chunk(int row, int c) {
    return PAD ? c : c ^ ((row / RPS) & (CPR - 1));
  }
};

// Four values of row `row`, columns col .. col+3 (col a multiple of 4).
template <typename T, int D, bool PAD>
__device__ __forceinline__ void put_row4(unsigned char* tile, int row, int col, float a, float b,
                                         float c, float d) {
  using L = RowTile<T, D, PAD>;
  const int byte = col * (int)sizeof(T);
  Elem<T>::store4(reinterpret_cast<T*>(tile + row * L::RS + 16 * L::chunk(row, byte >> 4) +
                                       (byte & 15)),
                  a, b, c, d);
}

// Rows 0 .. nvalid-1 of a ROWS-row tile go to `out` (row r at out + r*D);
// NTHR threads, this one is t.
template <typename T, int D, bool PAD, int ROWS, int NTHR>
__device__ __forceinline__ void write_rows(const unsigned char* tile, T* out, int nvalid, int t) {
  using L = RowTile<T, D, PAD>;
  static_assert((ROWS * L::CPR) % NTHR == 0, "rows must split evenly over the threads");
#pragma unroll
  for (int pass = 0; pass < ROWS * L::CPR / NTHR; ++pass) {
    const int idx = pass * NTHR + t;
    const int r = idx / L::CPR, cc = idx % L::CPR;
    if (r < nvalid)
      *reinterpret_cast<uint4*>(reinterpret_cast<unsigned char*>(out) + (size_t)r * L::RBo +
                                16 * cc) =
          *reinterpret_cast<const uint4*>(tile + r * L::RS + 16 * L::chunk(r, cc));
  }
}

}  // namespace fa
