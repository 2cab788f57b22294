// MFMA ceiling probe, for benchmarks only (no part of the optimizer step).
//
// The NS GEMMs are priced against the nominal bf16 dense peak of the chip,
// which assumes every matrix pipe busy at the top shader clock.  Under a
// sustained matrix load the chip lowers its clock, so the attainable rate is
// lower; this kernel measures it with the smallest possible GEMM inner loop:
// one workgroup of four waves per CU, each wave holding a 128x128 float32
// accumulator block as 4x4 v_mfma_f32_32x32x16_bf16 tiles (the layout of
// the NS kernels), and per k16 slice sixteen MFMAs on fragments that change
// every slice.  Modes:
//   0  fragments rotated in registers;
//   1  the eight fragments of a slice read from a 64 KB LDS array of
//      pseudo-random bf16 values, as a GEMM's k loop reads them;
//   2  mode 1 plus the NS kernels' operand staging per k32 step (two
//      slices): eight direct-to-LDS 16-byte loads per wave, in the NS
//      kernels' issue form, from a caller buffer small enough to stay in L2,
//      into an LDS area no fragment read touches, a wait for the loads
//      issued three steps before (the lead the NS kernels' five-stage ring
//      gives a stage), and one workgroup barrier.
// Modes 0 and 1 touch no global memory inside the loop: their rate bounds
// any bf16 GEMM kernel with this tile shape on the same chip.  Mode 2 is
// the NS kernels' k loop without cache misses, tile changes or epilogues.
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

// One direct-to-LDS load in the NS kernels' issue form: each lane's 16 bytes
// at base + voff land at LDS byte address m0 + 16 lane; the asm carries the
// wait states the hazard recognizer cannot see (5 after the readfirstlane
// that writes the scalar base, 1 after writing M0).
__device__ __forceinline__ void dma16_probe(const char* base, uint32_t voff, uint32_t m0) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const uint64_t sb = ((uint64_t)hi << 32) | (uint64_t)lo;
  const uint32_t sm0 = (uint32_t)__builtin_amdgcn_readfirstlane(m0);
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(sm0)
               : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters untouched (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vm_probe() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

template <int MODE>
__global__ __launch_bounds__(256) void k_mfma_ceiling(float* out, int iters, const char* src,
                                                      uint32_t src_mask) {
  __shared__ u32x4_c lds[kLdsVecs];
  __shared__ u32x4_c stage[MODE == 2 ? 2048 : 1];   // 32 KB: 8 KB per wave
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
  // mode 2: this wave's 8 KB of the staging area and of the source stream
  const uint32_t st_lds =
      (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)stage + wave * 8192u;
  const uint32_t src0 = (blockIdx.x * 4u + (uint32_t)wave) * 8192u;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE >= 1) {
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
    for (int q = 0; q < 16; ++q) {
      acc[q >> 2][q & 3] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[q >> 2], fb[q & 3], acc[q >> 2][q & 3], 0, 0, 0);
      if constexpr (MODE == 2) {
        // the second slice of a k32 step: one 1 KB load after each of its
        // last eight MFMAs (offsets 1 KB aligned, inside src_mask + 1 bytes)
        if ((it & 1) && q >= 8) {
          const uint32_t off =
              (src0 + (uint32_t)it * 37u * 1024u + (uint32_t)(q - 8) * 1024u) & src_mask;
          dma16_probe(src, off + (uint32_t)lane * 16u, st_lds + (uint32_t)(q - 8) * 1024u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == 2) {
      if ((it & 1) == 0) {   // between a step's slices: the stage wait and the barrier
        wait_vm_probe<24>();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
  }
  if constexpr (MODE == 2) wait_vm_probe<0>();
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

extern "C" sm_status sm_mfma_ceiling(int mode, int blocks, int iters, const void* src,
                                     size_t src_bytes, float* out, hipStream_t s) {
  if (!out || (reinterpret_cast<uintptr_t>(out) & 3u)) return SM_ERR_ARG;
  if (mode < 0 || mode > 2) return SM_ERR_ARG;
  if (blocks < 1 || blocks > 65536 || iters < 1 || iters > 10000000) return SM_ERR_SHAPE;
  uint32_t mask = 0;
  if (mode == 2) {
    // a power of two from 64 KB to 64 MB, 16-byte aligned
    if (!src || (reinterpret_cast<uintptr_t>(src) & 15u)) return SM_ERR_ARG;
    if (src_bytes < (size_t(1) << 16) || src_bytes > (size_t(1) << 26) ||
        (src_bytes & (src_bytes - 1)))
      return SM_ERR_SHAPE;
    mask = (uint32_t)(src_bytes - 1024);
  }
  const char* sp = static_cast<const char*>(src);
  if (mode == 0)
    hipLaunchKernelGGL(sm::k_mfma_ceiling<0>, dim3(blocks), dim3(256), 0, s, out, iters, sp, mask);
  else if (mode == 1)
    hipLaunchKernelGGL(sm::k_mfma_ceiling<1>, dim3(blocks), dim3(256), 0, s, out, iters, sp, mask);
  else
    hipLaunchKernelGGL(sm::k_mfma_ceiling<2>, dim3(blocks), dim3(256), 0, s, out, iters, sp, mask);
  return sm::check_launch();
}
