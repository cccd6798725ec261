// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bfloat16 is carried as its 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bfloat16, round to nearest, ties to even (gfx950's v_cvt_pk_bf16_f32).
MOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Element-type traits: load/store one element as float.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  MOE_DEV static float load(const float* p) { return *p; }
  MOE_DEV static void store(float* p, float v) { *p = v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
  MOE_DEV static float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
  MOE_DEV static void store(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }
};

// 16 bytes of T unpacked to float (4 floats or 8 bf16 -> 8 floats).
MOE_DEV void unpack16(const uint4& v, float* out, float) {
  out[0] = __uint_as_float(v.x);
  out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z);
  out[3] = __uint_as_float(v.w);
}
MOE_DEV void unpack16(const uint4& v, float* out, bf16_t) {
  out[0] = __uint_as_float(v.x << 16);
  out[1] = __uint_as_float(v.x & 0xffff0000u);
  out[2] = __uint_as_float(v.y << 16);
  out[3] = __uint_as_float(v.y & 0xffff0000u);
  out[4] = __uint_as_float(v.z << 16);
  out[5] = __uint_as_float(v.z & 0xffff0000u);
  out[6] = __uint_as_float(v.w << 16);
  out[7] = __uint_as_float(v.w & 0xffff0000u);
}
MOE_DEV uint4 pack16(const float* in, float) {
  return make_uint4(__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                    __float_as_uint(in[3]));
}
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
MOE_DEV uint4 pack16(const float* in, bf16_t) {
  auto p2 = [](float lo, float hi) { return pack_bf16x2(lo, hi); };
  return make_uint4(p2(in[0], in[1]), p2(in[2], in[3]), p2(in[4], in[5]), p2(in[6], in[7]));
}

MOE_DEV float gelu_erf(float u) { return 0.5f * u * (1.0f + erff(u * 0.70710678118654752440f)); }
MOE_DEV float sigmoid_f(float u) { return 1.0f / (1.0f + expf(-u)); }
// silu(u) = u sigmoid(u) with the hardware exponential and reciprocal (about 1 ulp each; the
// result is rounded to bfloat16 at once): 5 vector instructions instead of about 20 for a
// correctly rounded exp and division, in the up projection's epilogue. A large negative u
// gives -0, as the exact form does. Same-box A/B, 3 rounds: Mixtral-shaped up projection
// 3.09 -> 2.94 ms (layer 4.64 -> 4.50 ms), fine-grained layer 1.72 -> 1.66 ms.
MOE_DEV float silu_f(float u) { return u * __builtin_amdgcn_rcpf(1.0f + __expf(-u)); }

MOE_DEV int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Wave-wide sums / maxima through cross-lane shuffles (fixed butterfly order, so every lane
// gets the same bitwise result).
MOE_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
MOE_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}


// ---- streaming operands into LDS (the grouped GEMMs)

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS at lds_base + 16 * lane
// (global_load_lds_dwordx4; M0 holds the wave-uniform LDS base). Written as asm so the
// compiler's wait insertion, which cannot tell the four stage buffers apart once more than a
// few copies are in flight, does not stall every LDS read on every copy: the kernel waits
// for each stage explicitly. The instruction has no register outputs.
MOE_DEV void lds_dma16(const void* src, uint16_t* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds_base;
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m0) : "memory", "m0");
}
// The same copy with the address as a 64-bit scalar base plus a 32-bit per-lane offset
// (global_load_lds_dwordx4's saddr form), so a copy whose per-lane part is fixed for a tile
// needs no vector address arithmetic.
MOE_DEV void lds_dma16_s(const void* sbase, uint32_t voff, uint16_t* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds_base;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// Grouped copies: four copies whose LDS destinations are consecutive 1 KiB blocks share one
// M0 write. The instruction's immediate offset is added to both the global and the LDS
// address (checked on gfx950), so copy c (0..3) of a group carries offset 1024 c, and its
// global address is passed 1024 c lower to cancel it. Each M0 write costs the wave about as
// much as a copy's own issue (probe: 64 MFMAs and 8 copies per slab, 1275 -> 1220 cycles).
// lds_m0 sets M0 to the group's first destination; nothing between it and the group's last
// copy may write M0 (the kernels' loops use no other M0-based instruction).
MOE_DEV void lds_m0(uint16_t* lds_base) {
  const uint32_t m0 = (uint32_t)(uintptr_t)(lds_void*)lds_base;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" ::"s"(m0) : "memory", "m0");
}
// copy C of a group, saddr form: reads sbase + voff + 1024 C, writes M0 + 1024 C + 16 lane.
template <int C>
MOE_DEV void lds_dma16_sg(const void* sbase, uint32_t voff) {
  static_assert(C >= 0 && C < 4, "four copies per M0");
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" ::"v"(voff), "s"(sbase), "i"(C * 1024) : "memory");
}
// copy C of a group, 64-bit per-lane address: reads src + 1024 C, writes M0 + 1024 C + 16 lane.
template <int C>
MOE_DEV void lds_dma16_g(const void* src) {
  static_assert(C >= 0 && C < 4, "four copies per M0");
  asm volatile("global_load_lds_dwordx4 %0, off offset:%1" ::"v"(src), "i"(C * 1024) : "memory");
}
// s_waitcnt vmcnt(N) lgkmcnt(0): this wave's loads older than its last N have landed in LDS
// and its own LDS accesses are done.
template <int N> MOE_DEV void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
}
// Workgroup barrier without a memory fence: __syncthreads() would also wait for every load
// in flight (the stages still being prefetched). The waits each phase needs are explicit;
// the clobber keeps the compiler from moving memory accesses across it.
MOE_DEV void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace moe
