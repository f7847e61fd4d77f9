// Byte offsets of rows gathered through a caller's row index.
//
// The expert MLPs of the routed experts read their input rows from the
// token matrix through row_token ("Scaling Diffusion Transformers to 16
// Billion Parameters", MoE recap: only the selected experts evaluate a
// token).  The GEMM kernels read those rows with buffer loads whose
// descriptor spans exactly the caller's matrix, src_rows rows of row_bytes
// bytes, so a load at or past src_rows * row_bytes returns zero and touches
// no memory.  An index entry outside [0, src_rows) is mapped to row
// src_rows, just past the end: the whole row then reads zero, whatever
// column offset the kernel adds.  This header has no HIP dependency, so the
// host-side unit tests compile it as plain C++.
#pragma once

#include <stdint.h>

namespace moe {

// The largest column offset a kernel adds to a row's base offset is below
// row_bytes + 256 (a k stage may start up to one 64-element stage past the
// row's last chunk), so with (src_rows + 1) * row_bytes + 256 <= 2^32 no
// offset wraps around the 32-bit range.
__host__ __device__ inline bool gather_fits(int64_t src_rows,
                                            int64_t row_bytes) {
  return src_rows >= 0 && row_bytes > 0 &&
         (src_rows + 1) * row_bytes + 256 <= (int64_t(1) << 32);
}

// Byte offset of byte col_byte of source row `src` (an index entry, any
// value): src * row_bytes + col_byte for 0 <= src < src_rows, else
// src_rows * row_bytes + col_byte (past the descriptor's range).
__host__ __device__ inline uint32_t gather_row_offset(int32_t src,
                                                      uint32_t src_rows,
                                                      uint32_t row_bytes,
                                                      uint32_t col_byte) {
  const uint32_t r = static_cast<uint32_t>(src);
  return (r < src_rows ? r : src_rows) * row_bytes + col_byte;
}

// Whether an index entry names a row of the matrix (plain loads skip the
// others and use zeros).
__host__ __device__ inline bool gather_row_valid(int64_t src,
                                                 int64_t src_rows) {
  return src >= 0 && src < src_rows;
}

}  // namespace moe
