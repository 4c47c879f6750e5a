// Internal helpers shared by the gfx950 kernels of libqlora_nf4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qlora_nf4.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

#define QL_DEV __device__ __forceinline__

namespace ql {

// ---- bf16 <-> float --------------------------------------------------------
QL_DEV float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
QL_DEV float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
QL_DEV float bf16_to_f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }

// Round two floats to bf16 (nearest, ties to even) and pack: lo in bits 0-15.
QL_DEV uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 b = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}
QL_DEV uint16_t f_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// ---- MFMA wrappers (gfx950) -------------------------------------------------
// 32x32x16 bf16: lane l supplies A[row l%32][k 8(l/32)..+7] and
// B[k 8(l/32)..+7][col l%32]; it holds D[8(i/4) + 4(l/32) + i%4][l%32].
QL_DEV f32x16 mfma32(const uint4 &a, const uint4 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 16x16x32 bf16: lane l supplies A[row l%16][k 8(l/16)..+7] and
// B[k 8(l/16)..+7][col l%16]; it holds D[4(l/16) + i][l%16].
QL_DEV f32x4 mfma16(const uint4 &a, const uint4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---- NF4 block scale ---------------------------------------------------------
// Dequantised block scale a' = fl(fl(q * s2) + mu), or the stored absmax.
// Compiled with -ffp-contract=off, so the product and sum round separately.
struct ScaleSrc {
  const float *absmax;   // no double quant
  const int8_t *q;       // double quant
  const float *s2;
  const float *mu;
  int dq;
};
QL_DEV float block_scale(const ScaleSrc &s, int64_t blk, float mu) {
  if (!s.dq) return s.absmax[blk];
  float p = (float)s.q[blk] * s.s2[blk >> 8];
  return p + mu;
}

QL_DEV uint4 zero4() { return make_uint4(0u, 0u, 0u, 0u); }

}  // namespace ql

// ---- host-side launch helpers ------------------------------------------------
#define QL_LAUNCH_CHECK()                                   \
  do {                                                      \
    if (hipGetLastError() != hipSuccess) return QLORA_ERR_HIP; \
  } while (0)

__host__ __device__ static inline int64_t ql_cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ static inline int64_t ql_rup(int64_t a, int64_t b) { return ql_cdiv(a, b) * b; }
