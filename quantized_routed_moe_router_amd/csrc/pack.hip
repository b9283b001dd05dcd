// Repacking canonical 2-bit super-blocks into the HBM unit layout, and the
// reference dequantization of that layout (for bit-exact checks).
//
// Canonical block (the 2-bit K-quant super-block of the ds4 README "Models"
// section): 84 bytes per 256 consecutive weights of the row-major flattened
// matrix: scales[16] @0 (low nibble scale, high nibble min), qs[64] @16
// (weight i at byte i/4, bits 2*(i%4)), d @80, dmin @82 (binary16).
#include "common.h"
#include "launch.h"

namespace ds4 {

// One workgroup of 64 threads builds one 1344-byte unit (16 rows x 256 cols).
__global__ __launch_bounds__(64) void k_pack(uint8_t *__restrict__ dst, const uint8_t *__restrict__ src,
                                             int64_t rows, int64_t cols, int nchunks) {
  const int64_t unit = blockIdx.x;            // (mat, row_tile, chunk), chunk fastest
  const int64_t n_rt = rows / 16;
  const int chunk = (int)(unit % nchunks);
  const int64_t rt = (unit / nchunks) % n_rt;
  const int64_t mat = unit / nchunks / n_rt;
  const uint8_t *m = src + mat * (rows * cols / 256) * 84;
  uint8_t *u = dst + unit * DS4_UNIT_BYTES;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int64_t row = rt * 16 + r;
  const int64_t kbase = (int64_t)chunk * 256;

  // codes: dword q of lane (r,g) = sub-block 4q+g of row r
  uint32_t raw[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t v = 0;
    const int j = 4 * q + g;
    for (int i = 0; i < 16; ++i) {
      const int64_t k = kbase + 16 * j + i;
      uint32_t code = 0;
      if (k < cols) {
        const int64_t f = row * cols + k;
        const uint8_t *blk = m + (f >> 8) * 84;
        const int w = (int)(f & 255);
        code = (blk[16 + (w >> 2)] >> (2 * (w & 3))) & 3u;
      }
      v |= code << (4 * (i & 7) + 2 * (i >> 3));
    }
    raw[q] = v;
  }
  *reinterpret_cast<u4 *>(u + 16 * lane) = (u4){raw[0], raw[1], raw[2], raw[3]};

  if (lane < 16) {
    // scale / min nibbles of row `lane`
    const int64_t rw = rt * 16 + lane;
    uint32_t sc[16], mn[16];
    for (int j = 0; j < 16; ++j) {
      const int64_t k = kbase + 16 * j;
      sc[j] = 0;
      mn[j] = 0;
      if (k < cols) {
        const int64_t f = rw * cols + k;
        const uint8_t b = m[(f >> 8) * 84 + ((f & 255) >> 4)];
        sc[j] = b & 15u;
        mn[j] = b >> 4;
      }
    }
    // halfword gg: byte 0 = scales of sub-blocks gg (low nibble) and 8+gg (high),
    // byte 1 = scales of 4+gg and 12+gg; w2/w3: mins of sub-blocks 0-7 / 8-15,
    // byte b holding sub-block b (low nibble) and 4+b (high)
    uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
    for (int gg = 0; gg < 4; ++gg) {
      const uint32_t hw = (sc[gg] | (sc[8 + gg] << 4)) | ((sc[4 + gg] | (sc[12 + gg] << 4)) << 8);
      if (gg == 0) w0 |= hw;
      if (gg == 1) w0 |= hw << 16;
      if (gg == 2) w1 |= hw;
      if (gg == 3) w1 |= hw << 16;
    }
    for (int b = 0; b < 4; ++b) {
      w2 |= (mn[b] | (mn[4 + b] << 4)) << (8 * b);
      w3 |= (mn[8 + b] | (mn[12 + b] << 4)) << (8 * b);
    }
    *reinterpret_cast<u4 *>(u + DS4_SCALE_OFF + 16 * lane) = (u4){w0, w1, w2, w3};
    // d and dmin of the block holding this row's chunk
    const int64_t f = rw * cols + kbase;
    const uint8_t *blk = m + (f >> 8) * 84;
    const uint32_t d = (uint32_t)blk[80] | ((uint32_t)blk[81] << 8);
    const uint32_t dm = (uint32_t)blk[82] | ((uint32_t)blk[83] << 8);
    *reinterpret_cast<uint32_t *>(u + DS4_DD_OFF + 4 * lane) = d | (dm << 16);
  }
}

// One thread per output weight.
__global__ __launch_bounds__(256) void k_dequant(float *__restrict__ dst, const uint8_t *__restrict__ src,
                                                 int64_t rows, int64_t cols, int nchunks, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int64_t k = idx % cols;
  const int64_t row = (idx / cols) % rows;
  const int64_t mat = idx / cols / rows;
  const int64_t rt = row >> 4;
  const int r = (int)(row & 15);
  const int chunk = (int)(k >> 8);
  const int kk = (int)(k & 255);
  const int j = kk >> 4, i = kk & 15;
  const int g = j & 3, q = j >> 2;
  const uint8_t *u = src + ((mat * (rows / 16) + rt) * nchunks + chunk) * DS4_UNIT_BYTES;
  const uint32_t raw = *reinterpret_cast<const uint32_t *>(u + 16 * (16 * g + r) + 4 * q);
  const uint32_t code = (raw >> (4 * (i & 7) + 2 * (i >> 3))) & 3u;
  const uint16_t schw = *reinterpret_cast<const uint16_t *>(u + DS4_SCALE_OFF + 16 * r + 2 * g);
  const uint32_t sc = (schw >> (8 * (q & 1) + 4 * (q >> 1))) & 15u;
  const int jj = j & 7;
  const uint8_t mb = u[DS4_SCALE_OFF + 16 * r + 8 + 4 * (j >> 3) + (jj & 3)];
  const uint32_t mn = (mb >> (4 * (jj >> 2))) & 15u;
  const uint32_t dd = *reinterpret_cast<const uint32_t *>(u + DS4_DD_OFF + 4 * r);
  const float d = half_bits_to_float((uint16_t)(dd & 0xFFFF));
  const float dmin = half_bits_to_float((uint16_t)(dd >> 16));
  // each product is exact in fp32 (<= 17 significant bits): one rounding
  const float a = (d * (float)sc) * (float)code;
  const float b = dmin * (float)mn;
  dst[idx] = a - b;
}

hipError_t launch_pack(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols,
                       hipStream_t s) {
  const int nchunks = (int)((cols + 255) / 256);
  const int64_t units = n_mats * (rows / 16) * nchunks;
  if (units == 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)units), dim3(64), 0, s, (uint8_t *)dst, (const uint8_t *)canonical,
                     rows, cols, nchunks);
  return hipGetLastError();
}

hipError_t launch_dequant(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols,
                          hipStream_t s) {
  const int nchunks = (int)((cols + 255) / 256);
  const int64_t total = n_mats * rows * cols;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dst,
                     (const uint8_t *)packed, rows, cols, nchunks, total);
  return hipGetLastError();
}

}  // namespace ds4
