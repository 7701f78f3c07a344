/*
 * Reference out-of-place transpose -- TEST INFRASTRUCTURE ONLY.
 *
 * This file is the oracle that the HIP path is checked against.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it;
 * the library never links or calls it, and it shares no header, helper or
 * table with the library.
 *
 * What it computes is the plain definition of a transpose: the element in
 * row i, column j of the input lands in row j, column i of the output.
 * On the pages each thread copies an input element into the on-chip tile
 * and a second phase writes the tile's transposed element to the output
 * ("Shared memory and the bank conflict", section "Turn the tile around on
 * chip"); for a non-square matrix of width W and height H the element at
 * row r, column c lands at output offset c*H + r ("Shared-memory tiling and
 * bank conflicts", section "Reference summary").  Both collapse to the loop
 * below once the tile is taken away.  Leading
 * dimensions and batch strides are counted in elements; a batch of matrices
 * is the same definition applied to each one.
 *
 * No arithmetic is done on the values: they are moved as unsigned integers of
 * the element's width, so every bit (NaN payloads, -0, subnormals) survives.
 * Output elements outside rows [0, cols) x columns [0, rows) of each output
 * matrix -- the leading-dimension padding and the gaps between batch entries
 * -- are never written.
 *
 * Single-threaded on purpose: slow, obvious, and independent of any tiling.
 */
#include <stdint.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL (-1)

static void xpose_u8(uint8_t *out, const uint8_t *in, int64_t batch,
                     int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                     int64_t stride_in, int64_t stride_out) {
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < cols; ++j)
        out[b * stride_out + j * ld_out + i] = in[b * stride_in + i * ld_in + j];
}

static void xpose_u16(uint16_t *out, const uint16_t *in, int64_t batch,
                      int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                      int64_t stride_in, int64_t stride_out) {
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < cols; ++j)
        out[b * stride_out + j * ld_out + i] = in[b * stride_in + i * ld_in + j];
}

static void xpose_u32(uint32_t *out, const uint32_t *in, int64_t batch,
                      int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                      int64_t stride_in, int64_t stride_out) {
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < cols; ++j)
        out[b * stride_out + j * ld_out + i] = in[b * stride_in + i * ld_in + j];
}

static void xpose_u64(uint64_t *out, const uint64_t *in, int64_t batch,
                      int64_t rows, int64_t cols, int64_t ld_in, int64_t ld_out,
                      int64_t stride_in, int64_t stride_out) {
  for (int64_t b = 0; b < batch; ++b)
    for (int64_t i = 0; i < rows; ++i)
      for (int64_t j = 0; j < cols; ++j)
        out[b * stride_out + j * ld_out + i] = in[b * stride_in + i * ld_in + j];
}

/*
 * out, in      host buffers owned by the caller; they must not overlap.
 * batch        number of matrices (>= 0).
 * rows, cols   input matrix shape (>= 0); the output matrix is cols x rows.
 * ld_in        input row pitch in elements, >= cols.
 * ld_out       output row pitch in elements, >= rows.
 * stride_in    distance between input matrices in elements (ignored when
 *              batch <= 1), >= 0; input matrices may overlap.
 * stride_out   distance between output matrices in elements (ignored when
 *              batch <= 1), >= (cols - 1) * ld_out + rows.
 * elem_bytes   1, 2, 4 or 8.
 * Returns 0, or -1 for arguments outside those ranges (nothing is written).
 */
int oracle_xpose(void *out, const void *in, int64_t batch, int64_t rows,
                 int64_t cols, int64_t ld_in, int64_t ld_out,
                 int64_t stride_in, int64_t stride_out, int64_t elem_bytes) {
  if (batch < 0 || rows < 0 || cols < 0) return ORACLE_EINVAL;
  if (batch == 0 || rows == 0 || cols == 0) return ORACLE_OK;
  if (!out || !in) return ORACLE_EINVAL;
  if (ld_in < cols || ld_out < rows) return ORACLE_EINVAL;
  /* Input matrices are only read, so they may overlap (stride_in >= 0);
   * output matrices must not: each spans (cols-1)*ld_out + rows elements. */
  if (batch > 1 && (stride_in < 0 || stride_out < (cols - 1) * ld_out + rows))
    return ORACLE_EINVAL;
  switch (elem_bytes) {
    case 1: xpose_u8(out, in, batch, rows, cols, ld_in, ld_out, stride_in, stride_out); break;
    case 2: xpose_u16(out, in, batch, rows, cols, ld_in, ld_out, stride_in, stride_out); break;
    case 4: xpose_u32(out, in, batch, rows, cols, ld_in, ld_out, stride_in, stride_out); break;
    case 8: xpose_u64(out, in, batch, rows, cols, ld_in, ld_out, stride_in, stride_out); break;
    default: return ORACLE_EINVAL;
  }
  return ORACLE_OK;
}
