// Repacking canonical 2-, 4-, 5- or 6-bit super-blocks into the HBM unit
// layout, and the reference dequantization of that layout (for bit-exact
// checks).
//
// Canonical block (the 2-bit K-quant super-block of the ds4 README "Models"
// section): 84 bytes per 256 consecutive weights of the row-major flattened
// matrix: scales[16] @0 (low nibble scale, high nibble min), qs[64] @16
// (weight i at byte i/4, bits 2*(i%4)), d @80, dmin @82 (binary16).  The
// 4-bit block is the same with 4-bit codes: qs[128] @16 (weight i at byte i/2,
// bits 4*(i%2)), d @144, dmin @146 (148 bytes).  The 5- and 6-bit blocks hold
// their codes as one bit stream from byte 16, lowest bits first (weight i at
// bits b*i .. b*i+b-1, the order of the 2- and 4-bit blocks), d and dmin
// after them (180 and 212 bytes).
#include "common.h"
#include "launch.h"

namespace ds4 {

// code of weight w (0..255) of a canonical block with B-bit codes (the byte
// after the last code byte is d's, inside the block)
template <int B>
__device__ __forceinline__ uint32_t canon_code(const uint8_t *blk, int w) {
  const int bit = B * w;
  const uint32_t two = blk[16 + (bit >> 3)] | ((uint32_t)blk[16 + (bit >> 3) + 1] << 8);
  return (two >> (bit & 7)) & ((1u << B) - 1u);
}

// Position of code i (0..15) of a sub-block inside its lane's code dwords:
// B = 2: one dword per sub-block, element i at bits 4*(i%8) + 2*(i/8), so a
// byte converted as two fp4 values yields two codes of one MFMA step.
// B = 4: two dwords per sub-block (elements 0-7, then 8-15); element e of a
// dword sits in nibble 2e (e < 4) or 2(e-4)+1 (e >= 4), so the low nibbles
// of its bytes hold elements 0-3 and the high nibbles 4-7 in order.
template <int B>
__device__ __forceinline__ int code_shift(int i) {
  if (B == 2) return 4 * (i & 7) + 2 * (i >> 3);
  const int e = i & 7;
  return 4 * (e < 4 ? 2 * e : 2 * (e - 4) + 1);
}

// One workgroup of 64 threads builds one unit (16 rows x 256 cols) of width
// B from canonical blocks with CBITS-bit codes (CBITS = B, or 5 for B = 6).
template <int B, int CBITS>
__global__ __launch_bounds__(64) void k_pack(uint8_t *__restrict__ dst, const uint8_t *__restrict__ src,
                                             int64_t rows, int64_t cols, int nchunks) {
  constexpr int CB = canon_block_bytes<CBITS>();
  const int64_t unit = blockIdx.x;            // (mat, row_tile, chunk), chunk fastest
  const int64_t n_rt = rows / 16;
  const int chunk = (int)(unit % nchunks);
  const int64_t rt = (unit / nchunks) % n_rt;
  const int64_t mat = unit / nchunks / n_rt;
  const uint8_t *m = src + mat * (rows * cols / 256) * CB;
  uint8_t *u = dst + unit * Unit<B>::BYTES;
  const int lane = threadIdx.x;
  const int r = lane & 15, g = lane >> 4;
  const int64_t row = rt * 16 + r;
  const int64_t kbase = (int64_t)chunk * 256;

  // codes: lane (r,g) holds sub-blocks g, 4+g, 8+g, 12+g of row r; dword
  // (B/2)*q + h holds elements 8h.. of sub-block 4q+g (h = 0 only for B = 2);
  // B = 6: dwords 0-7 the low 4 bits as for B = 4, dword 8+q the high 2 bits
  // of sub-block 4q+g as for B = 2; dword d of the lane sits in code plane
  // d/4, at 1024*(d/4) + 16*lane + 4*(d%4)
  constexpr int ND = 2 * B;  // dwords per lane
  uint32_t raw[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) raw[d] = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = 4 * q + g;
    for (int i = 0; i < 16; ++i) {
      const int64_t k = kbase + 16 * j + i;
      uint32_t code = 0;
      if (k < cols) {
        const int64_t f = row * cols + k;
        code = canon_code<CBITS>(m + (f >> 8) * CB, (int)(f & 255));
      }
      if constexpr (B == 6) {
        raw[2 * q + (i >> 3)] |= (code & 15u) << code_shift<4>(i);
        raw[8 + q] |= (code >> 4) << code_shift<2>(i);
      } else {
        const int d = B == 2 ? q : 2 * q + (i >> 3);
        raw[d] |= code << code_shift<B>(i);
      }
    }
  }
#pragma unroll
  for (int d = 0; d < ND; d += 4)
    *reinterpret_cast<u4 *>(u + 256 * d + 16 * lane) = (u4){raw[d], raw[d + 1], raw[d + 2], raw[d + 3]};

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
        const uint8_t b = m[(f >> 8) * CB + ((f & 255) >> 4)];
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
    *reinterpret_cast<u4 *>(u + Unit<B>::SCALE_OFF + 16 * lane) = (u4){w0, w1, w2, w3};
    // d and dmin of the block holding this row's chunk
    const int64_t f = rw * cols + kbase;
    const uint8_t *blk = m + (f >> 8) * CB;
    const uint32_t d = (uint32_t)blk[CB - 4] | ((uint32_t)blk[CB - 3] << 8);
    const uint32_t dm = (uint32_t)blk[CB - 2] | ((uint32_t)blk[CB - 1] << 8);
    *reinterpret_cast<uint32_t *>(u + Unit<B>::DD_OFF + 4 * lane) = d | (dm << 16);
  }
}

// One thread per output weight.
template <int B>
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
  const uint8_t *u = src + ((mat * (rows / 16) + rt) * nchunks + chunk) * Unit<B>::BYTES;
  auto lane_dword = [&](int dw) {
    return *reinterpret_cast<const uint32_t *>(u + 1024 * (dw >> 2) + 16 * (16 * g + r) + 4 * (dw & 3));
  };
  uint32_t code;
  if constexpr (B == 6) {
    code = ((lane_dword(2 * q + (i >> 3)) >> code_shift<4>(i)) & 15u) |
           (((lane_dword(8 + q) >> code_shift<2>(i)) & 3u) << 4);
  } else {
    const int dw = B == 2 ? q : 2 * q + (i >> 3);
    code = (lane_dword(dw) >> code_shift<B>(i)) & ((1u << B) - 1u);
  }
  const uint16_t schw = *reinterpret_cast<const uint16_t *>(u + Unit<B>::SCALE_OFF + 16 * r + 2 * g);
  const uint32_t sc = (schw >> (8 * (q & 1) + 4 * (q >> 1))) & 15u;
  const int jj = j & 7;
  const uint8_t mb = u[Unit<B>::SCALE_OFF + 16 * r + 8 + 4 * (j >> 3) + (jj & 3)];
  const uint32_t mn = (mb >> (4 * (jj >> 2))) & 15u;
  const uint32_t dd = *reinterpret_cast<const uint32_t *>(u + Unit<B>::DD_OFF + 4 * r);
  const float d = half_bits_to_float((uint16_t)(dd & 0xFFFF));
  const float dmin = half_bits_to_float((uint16_t)(dd >> 16));
  // each product is exact in fp32 (<= 21 significant bits): one rounding
  const float a = (d * (float)sc) * (float)code;
  const float b = dmin * (float)mn;
  dst[idx] = a - b;
}

hipError_t launch_pack(void *dst, const void *canonical, int64_t n_mats, int64_t rows, int64_t cols, int bits,
                       hipStream_t s) {
  const int nchunks = (int)((cols + 255) / 256);
  const int64_t units = n_mats * (rows / 16) * nchunks;
  if (units == 0) return hipSuccess;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(64), 0, s, (uint8_t *)dst, (const uint8_t *)canonical,
                       rows, cols, nchunks);
  };
  switch (bits) {
    case 2: go(k_pack<2, 2>); break;
    case 4: go(k_pack<4, 4>); break;
    case 5: go(k_pack<6, 5>); break;
    case 6: go(k_pack<6, 6>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_dequant(float *dst, const void *packed, int64_t n_mats, int64_t rows, int64_t cols, int bits,
                          hipStream_t s) {
  const int nchunks = (int)((cols + 255) / 256);
  const int64_t total = n_mats * rows * cols;
  if (total == 0) return hipSuccess;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, dst, (const uint8_t *)packed,
                       rows, cols, nchunks, total);
  };
  switch (unit_bits(bits)) {
    case 2: go(k_dequant<2>); break;
    case 4: go(k_dequant<4>); break;
    case 6: go(k_dequant<6>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace ds4
