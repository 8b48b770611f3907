// Per-token fp8 (OCP e4m3fn) quantization for the fp8 Lightning Indexer path.
//
// The pages fix no fp8 format; this follows the OCP 8-bit float definition (E4M3: bias 7,
// 3 mantissa bits, no infinities, largest finite 448).  Per row: scale = amax / 448 (1 for an
// all-zero row), y = x / scale in fp32 with correctly rounded division, code = y rounded to
// nearest-even on the e4m3 grid, saturating at +-448.  The rounding is done with integer
// operations on the fp32 bits so it is exact and independent of the conversion hardware.
#include "dsa_device.h"

namespace dsa {

namespace {

__device__ __forceinline__ uint8_t e4m3fn_rne_sat(float y) {
  const uint32_t b = __float_as_uint(y);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = fabsf(y);
  if (a != a) return 0x7Fu;                 // NaN
  if (a >= 448.0f) return (uint8_t)(sign | 0x7Eu);
  const uint32_t e32 = (b >> 23) & 0xFFu;
  uint32_t code;
  if (e32 >= 121u) {                        // a >= 2^-6: normal e4m3
    uint32_t E = e32 - 127u + 7u;           // biased e4m3 exponent, 1 .. 15
    const uint32_t man = b & 0x7FFFFFu;
    uint32_t m3 = man >> 20;
    const uint32_t rem = man & 0xFFFFFu;
    if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0u; ++E; }
    code = (E << 3) | m3;
  } else {                                  // subnormal grid: multiples of 2^-9
    code = (uint32_t)rintf(a * 512.0f);     // 0 .. 8; 8 encodes 2^-6 (exponent 1, mantissa 0)
  }
  return (uint8_t)(sign | code);
}

}  // namespace

__global__ __launch_bounds__(256) void k_quant_fp8_rows(QuantArgs a) {
  __shared__ float red[4];
  const long long row = blockIdx.x;
  const uint16_t* x = a.x + row * a.cols;
  uint8_t* y = a.y + row * a.cols;
  float m = 0.f;
  for (int c = threadIdx.x; c < a.cols; c += 256) m = fmaxf(m, fabsf(bf16_to_f32(x[c])));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
  for (int c = threadIdx.x; c < a.cols; c += 256) y[c] = e4m3fn_rne_sat(bf16_to_f32(x[c]) / scale);
  if (threadIdx.x == 0) a.scale[row] = scale;
}

hipError_t launch_quant_fp8_rows(const QuantArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  k_quant_fp8_rows<<<(unsigned)a.rows, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace dsa
