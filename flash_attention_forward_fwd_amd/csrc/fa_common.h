// Device helpers shared by the gfx950 attention kernels: vector types, the
// bf16/fp16 MFMA and pack selection, LDS transposing reads, lane exchange.
//
// gfx950 facts these helpers rely on (checked on the device by a layout test):
//  * v_mfma_f32_32x32x16_{bf16,f16}: A operand lane l holds A[m = l%32][k = 8*(l/32) + e],
//    B operand lane l holds B[k = 8*(l/32) + e][n = l%32] (e = 0..7), and the
//    accumulator register r of lane l is C[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lanes 4e..4e+3 each
//    name 4 consecutive 16-bit elements of "row e" (lane 4e+q the columns
//    4q..4q+3) and lane i of the group receives column i of rows 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

enum : int { kBF16 = 0, kFP16 = 1 };

template <int DT>
struct Elt;

template <>
struct Elt<kBF16> {
  // C += A * B on the 32x32x16 bf16 matrix core, fp32 accumulate.
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> packed pair, round to nearest even (v_cvt_pk_bf16_f32)
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    bf16x2 r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ __forceinline__ float widen(unsigned short bits) {
    return __uint_as_float(((unsigned)bits) << 16);
  }
  // acc + lo + hi of a packed pair, fp32 accumulate (v_dot2_f32_bf16 with ones)
  static __device__ __forceinline__ float sum2(unsigned pair, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                           __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
  }
};

template <>
struct Elt<kFP16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ unsigned pack2(float lo, float hi) {
    f16x2 r;
    r[0] = (_Float16)lo;
    r[1] = (_Float16)hi;
    return __builtin_bit_cast(unsigned, r);
  }
  static __device__ __forceinline__ float widen(unsigned short bits) {
    return (float)__builtin_bit_cast(_Float16, bits);
  }
  static __device__ __forceinline__ float sum2(unsigned pair, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pair),
                                  __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
  }
};

// 16-byte global load / store (global_load_dwordx4 / global_store_dwordx4).
__device__ __forceinline__ u32x4 gload16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Transposing 64-bit LDS read (see the lane mapping above).
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* lds) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds));
  return __builtin_bit_cast(u32x2, t);
}

// gfx9 buffer resource word 3: 32-bit data format, raw (unswizzled) access
constexpr int kBufferFlags = 0x00020000;
// a byte offset past the end of any buffer range the kernels describe (their
// sizes are < 2^31): buffer loads from it read zeros
constexpr unsigned kPastEnd = 0x7FFFFFF0u;

// s_waitcnt vmcnt(0): every vector-memory operation of this wave has finished
// (for a buffer load to LDS: its data is in LDS)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt vmcnt(N): at most N vector-memory operations of this wave are
// still outstanding (they complete in order, so all older ones are done)
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// 16-byte buffer load straight to LDS: lane j of the wave writes bytes
// [16 j, 16 j + 16) after `dst` (a wave-uniform LDS address) with the 16
// bytes at byte offset voff + soff of the buffer (zeros past its end).  A
// function of its own: used directly inside a kernel's lambdas, the builtin
// kept the host-side launch stub of the kernel from being emitted.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, uint16_t* dst, unsigned voff,
                                          int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const uint16_t* lds) {
  return *reinterpret_cast<const u32x4*>(lds);
}

__device__ __forceinline__ void lds_write16(uint16_t* lds, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds) = v;
}

// Accesses that other workgroups, on any XCD, read or write in the same
// launch.  The XCDs' L2 caches are not coherent with each other; loads and
// stores with the sc1 cache policy (what an agent-scope relaxed atomic access
// compiles to) are, so records and counters cross workgroups without an L2
// writeback or invalidate.  Order comes from waiting for the stores to
// complete (wait_vmem) before a counter or flag says they are there.
constexpr int kCoherent = 16;  // buffer cache policy sc1
__device__ __forceinline__ f32x4 ld4_coherent(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCoherent));
}
__device__ __forceinline__ f32x2 ld2_coherent(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kCoherent));
}
__device__ __forceinline__ void st4_coherent(__amdgpu_buffer_rsrc_t rs, int off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCoherent);
}
__device__ __forceinline__ void st2_coherent(__amdgpu_buffer_rsrc_t rs, int off, f32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), rs, off, 0, kCoherent);
}
__device__ __forceinline__ unsigned ld_flag(const unsigned* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_flag(unsigned* p, unsigned v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// returns the value before the add
__device__ __forceinline__ unsigned add_flag(unsigned* p, unsigned v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// max / sum of a value with the same value in lane l ^ 32 (v_permlane32_swap).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

constexpr float kLn2 = 0.693147180559945309417232121458f;

// A run of N MFMAs as an explicit software pipeline: the LDS operand of
// MFMA j is read LA MFMAs before it, and a scheduling fence after
// every (MFMA j, read j + LA) pair keeps that distance from being collapsed
// by the compiler's own scheduling.  load(j) returns MFMA j's operand (or
// operands: any value type), mfma(j, a) issues MFMA j.
template <int J, int N, int LA, class Load, class Mfma, class T>
__device__ __forceinline__ void m_pipe(Load& load, Mfma& mfma, T (&buf)[LA]) {
  if constexpr (J < N) {
    mfma(std::integral_constant<int, J>{}, buf[J % LA]);
    if constexpr (J + LA < N) buf[J % LA] = load(std::integral_constant<int, J + LA>{});
    __builtin_amdgcn_sched_barrier(0);
    m_pipe<J + 1, N, LA>(load, mfma, buf);
  }
}
template <int J, int N, int LA, class Load, class T>
__device__ __forceinline__ void m_prime(Load& load, T (&buf)[LA]) {
  if constexpr (J < N && J < LA) {
    buf[J] = load(std::integral_constant<int, J>{});
    m_prime<J + 1, N, LA>(load, buf);
  }
}
template <int N, int LA, class Load, class Mfma>
__device__ __forceinline__ void m_pipeline(Load& load, Mfma& mfma) {
  using T = decltype(load(std::integral_constant<int, 0>{}));
  T buf[LA];
  m_prime<0, N, LA>(load, buf);
  __builtin_amdgcn_sched_barrier(0);
  m_pipe<0, N, LA>(load, mfma, buf);
}

}  // namespace fa
