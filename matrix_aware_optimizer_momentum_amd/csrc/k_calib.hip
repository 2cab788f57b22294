// MFMA ceiling probe, for benchmarks only (no part of the optimizer step).
//
// The NS GEMMs are priced against the nominal bf16 dense peak of the chip,
// which assumes every matrix pipe busy at the top shader clock.  Under a
// sustained matrix load the chip lowers its clock, so the attainable rate is
// lower; this kernel measures it with the smallest possible GEMM inner loop:
// one workgroup of four waves per CU, each wave holding a 128x128 float32
// accumulator block as 4x4 v_mfma_f32_32x32x16_bf16 tiles (the layout of
// the NS kernels), and per k16 slice sixteen MFMAs on fragments that change
// every slice.  With LDS=1 the eight fragments of a slice are read from a
// 64 KB LDS array of pseudo-random bf16 values, as a GEMM's k loop reads
// them; with LDS=0 they rotate in registers.  No global memory is touched
// inside the loop, so the rate is an upper bound for any bf16 GEMM kernel
// with this tile shape on the same chip.
#include "sm_internal.hpp"

namespace sm {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_c;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_c;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_c;

constexpr int kLdsVecs = 4096;  // 64 KB of 16-byte vectors

// bf16 pairs with random sign and mantissa and exponents in [1, 4): the
// operand bits toggle like real data, and the float32 sums stay finite.
__device__ __forceinline__ uint32_t rnd_bf16x2(uint32_t h) {
  return (h & 0x807f807fu) | 0x3f803f80u | ((h >> 7) & 0x00800080u);
}

__device__ __forceinline__ uint32_t mix32(uint32_t h) {
  h ^= h >> 16;
  h *= 0x7feb352du;
  h ^= h >> 15;
  h *= 0x846ca68bu;
  h ^= h >> 16;
  return h;
}

template <int LDS>
__global__ __launch_bounds__(256) void k_mfma_ceiling(float* out, int iters) {
  __shared__ u32x4_c lds[kLdsVecs];
  const int tid = threadIdx.x;
  for (int i = tid; i < kLdsVecs; i += 256) {
    const uint32_t h = mix32((uint32_t)i * 0x9e3779b9u + blockIdx.x);
    u32x4_c v;
    v.x = rnd_bf16x2(h);
    v.y = rnd_bf16x2(mix32(h + 1));
    v.z = rnd_bf16x2(mix32(h + 2));
    v.w = rnd_bf16x2(mix32(h + 3));
    lds[i] = v;
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  f32x16_c acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16_c){};
  bf16x8_c fa[4], fb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    fa[i] = __builtin_bit_cast(bf16x8_c, lds[(wave * 1024 + i * 64 + lane) & (kLdsVecs - 1)]);
    fb[i] = __builtin_bit_cast(bf16x8_c,
                               lds[(wave * 1024 + 512 + i * 64 + lane) & (kLdsVecs - 1)]);
  }
  for (int it = 0; it < iters; ++it) {
    if constexpr (LDS) {
      const int base = (it * 512) & (kLdsVecs - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        fa[i] = __builtin_bit_cast(bf16x8_c, lds[(base + i * 64 + lane) & (kLdsVecs - 1)]);
        fb[i] = __builtin_bit_cast(bf16x8_c, lds[(base + 256 + i * 64 + lane) & (kLdsVecs - 1)]);
      }
    } else {
      const bf16x8_c t = fa[0];
      fa[0] = fb[3];
      fb[3] = fa[2];
      fa[2] = fb[1];
      fb[1] = t;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][j][e];
  out[(int64_t)blockIdx.x * 256 + tid] = s;
}

}  // namespace

}  // namespace sm

extern "C" sm_status sm_mfma_ceiling(int lds_operands, int blocks, int iters, float* out,
                                     hipStream_t s) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u)) return SM_ERR_ARG;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 10000000) return SM_ERR_SHAPE;
  if (lds_operands)
    hipLaunchKernelGGL(sm::k_mfma_ceiling<1>, dim3(blocks), dim3(256), 0, s, out, iters);
  else
    hipLaunchKernelGGL(sm::k_mfma_ceiling<0>, dim3(blocks), dim3(256), 0, s, out, iters);
  return sm::check_launch();
}
