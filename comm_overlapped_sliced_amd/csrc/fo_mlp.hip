// The activation between the two projections of the MLP block (libflashovl, gfx950).
//
// The FlashOverlap page measures its MLP-layer latency (technical summary section 4) on the
// block that the column-parallel projection (Flash-AG) and the row-parallel projection
// (Flash-RS) make together (section 2). For the Llama-3.1 shapes of those measurements the
// activation is SwiGLU: h = silu(gate) * up, silu(g) = g / (1 + e^-g), where gate and up are the
// two halves of the gate+up projection's output. HBM-bound: each element of y is read once and
// each element of h written once, with 16-byte accesses.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fo_internal.h"

namespace fo {
namespace {

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// two fp32 -> packed bf16 (a low), round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Thread (x, row) converts 8 consecutive columns: blockIdx.y walks the rows with a stride of
// gridDim.y, threads of a row walk its 8-column chunks.
__global__ __launch_bounds__(256) void swiglu_kernel(const uint16_t* y, uint16_t* h, int64_t rows,
                                                     int64_t inter) {
  const int64_t chunks = inter / 8;
  const int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= chunks) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const uint16_t* yr = y + r * 2 * inter + c * 8;
    const uint4 g = *(const uint4*)yr;
    const uint4 u = *(const uint4*)(yr + inter);
    uint4 o;
    o.x = pack_bf16(silu_mul(bf16_lo(g.x), bf16_lo(u.x)), silu_mul(bf16_hi(g.x), bf16_hi(u.x)));
    o.y = pack_bf16(silu_mul(bf16_lo(g.y), bf16_lo(u.y)), silu_mul(bf16_hi(g.y), bf16_hi(u.y)));
    o.z = pack_bf16(silu_mul(bf16_lo(g.z), bf16_lo(u.z)), silu_mul(bf16_hi(g.z), bf16_hi(u.z)));
    o.w = pack_bf16(silu_mul(bf16_lo(g.w), bf16_lo(u.w)), silu_mul(bf16_hi(g.w), bf16_hi(u.w)));
    *(uint4*)(h + r * inter + c * 8) = o;
  }
}

}  // namespace

hipError_t launch_swiglu(const void* y, void* h, int64_t rows, int64_t inter, hipStream_t s) {
  if (rows < 0 || inter < 0 || inter % 8) return hipErrorInvalidValue;
  if (rows == 0 || inter == 0) return hipSuccess;
  const int64_t chunks = inter / 8;
  const unsigned gx = (unsigned)((chunks + 255) / 256);
  const unsigned gy = (unsigned)(rows < 65535 ? rows : 65535);
  hipLaunchKernelGGL(swiglu_kernel, dim3(gx, gy), dim3(256), 0, s, (const uint16_t*)y,
                     (uint16_t*)h, rows, inter);
  return hipGetLastError();
}

}  // namespace fo
