// Device helpers shared by the GEMM kernels (gfx950).
//
// Citations: [TDI] = Tencent engineer article on deterministic LLM inference
// ("AI インフラの深化：大規模モデルに確定的な出力を実現する方法").
#pragma once

#include <type_traits>
#include <utility>

#include "imm_internal.h"

namespace imm {
namespace dev {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define IMM_LDS(p) ((__attribute__((address_space(3))) void*)(p))

template <int IN>
struct InT {
  static constexpr bool I8 = IN == GEMM_I8;  // int8 (Ozaki slices), int32 accumulators
  // fp8 data widened to fp16 for the 16x16x32 step (kInE4M3W, kInE5M2W)
  static constexpr bool W16 = (IN & kInWiden) != 0;
  static constexpr int F8 = IN & ~kInWiden;   // the fp8 format of the data
  static constexpr int EB = (F8 == GEMM_F8_E4M3 || F8 == GEMM_F8_E5M2 || I8) ? 1 : 2;
  // The 32x32-block step (mfma_v): bytes of K per instruction per row, and
  // 16-byte pieces per lane per operand.
  static constexpr int KSTEP_B = (EB == 2 || I8) ? 32 : 64;
  static constexpr int FRAG = KSTEP_B / 32;
};

// The matrix-core steps.  The bits of a product depend on the instruction
// that accumulates it ([TDI] "Batch Invariance の由来", BLOCK_K paragraph),
// so every GEMM kernel uses one step per input dtype:
//   fp16 / bf16: mfma16_v, a 16x16 output block, K = 32.  Lane l supplies
//     row (l % 16) of A and column (l % 16) of B, with the K elements
//     [8 (l / 16), 8 (l / 16) + 8) of the step in increasing k; it holds
//     rows 4 (l / 16) .. 4 (l / 16) + 3 of column (l % 16) of the block.
//     (Measured on MI355X: the same bits as the 32x32x16 instruction, and
//     about 15 % less energy per flop on random data, which is what sets the
//     clock of a large product.)
//   fp8: mfma16_f8, a 16x16 block, K = 128 (about 8 % less energy per flop
//     than the 32x32x64 step on random data, measured).
//   int8 (Ozaki slices): mfma_v, a 32x32 block, K = 32, int32 accumulators
//     carried in the fp32 registers' bits.  Lane l supplies row (l % 32) of A
//     and column (l % 32) of B, with the K elements [h*half, (h+1)*half) of
//     the step, h = l / 32, in increasing k.
// The Ozaki slice products accumulate exact chains, where the instruction
// cannot change a bit; there 16-bit and fp8 slices use mfma_v (32x32x16,
// 32x32x64), whose fragments leave room for the fp64 accumulators.

// The 32x32 step on whole-operand registers: 4 dwords (16-bit inputs and
// int8) or 8 dwords (fp8) per lane, allocated as one register tuple.
template <int IN>
struct FragOf {
  using type = typename std::conditional<
      InT<IN>::W16, i32x2, typename std::conditional<InT<IN>::FRAG == 1, i32x4, i32x8>::type>::type;
};

template <int IN>
__device__ __forceinline__ f32x16 mfma_v(const typename FragOf<IN>::type& a,
                                         const typename FragOf<IN>::type& b, f32x16 c) {
  if constexpr (IN == GEMM_F16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else if constexpr (IN == GEMM_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else if constexpr (IN == GEMM_I8) {
    return __builtin_bit_cast(
        f32x16, __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, __builtin_bit_cast(i32x16, c), 0, 0, 0));
  } else {
    // cbsz / blgp select the operand formats: 0 = fp8 e4m3, 1 = bf8 e5m2.
    constexpr int fmt = IN == GEMM_F8_E4M3 ? 0 : 1;
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, fmt, fmt, 0, 0, 0, 0);
  }
}

// The 16x16x128 step of fp8 inputs: 8 dwords (32 fp8 values) per lane and
// operand.  Lane l supplies row (l % 16) of A and column (l % 16) of B with
// the K elements [32 (l / 16), 32 (l / 16) + 32) of the step in increasing k;
// it holds rows 4 (l / 16) .. 4 (l / 16) + 3 of column (l % 16) of the block
// (the layout of the 16-bit 16x16 blocks).  cbsz / blgp select the operand
// formats: 0 = fp8 e4m3, 1 = bf8 e5m2; the scales are unit.
template <int IN>
__device__ __forceinline__ f32x4 mfma16_f8(const i32x8& a, const i32x8& b, f32x4 c) {
  static_assert(IN == GEMM_F8_E4M3 || IN == GEMM_F8_E5M2, "fp8 inputs only");
  constexpr int fmt = IN == GEMM_F8_E4M3 ? 0 : 1;
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, fmt, fmt, 0, 0, 0, 0);
}

// The 16x16x32 step of 16-bit inputs: 4 dwords per lane and operand.
template <int IN>
__device__ __forceinline__ f32x4 mfma16_v(const i32x4& a, const i32x4& b, f32x4 c) {
  static_assert(IN == GEMM_F16 || IN == GEMM_BF16, "16-bit inputs only");
  if constexpr (IN == GEMM_F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Eight fp8 values (K-consecutive, one per byte) widened to the eight fp16
// values of a 16x16x32 operand, in the same order.  Every e4m3 and e5m2 value
// (NaN and, for e5m2, infinity included) is an fp16 value, and the unit scale
// makes the conversion exact.
template <int F8>
__device__ __forceinline__ i32x4 widen_f8(const i32x2& v) {
  static_assert(F8 == GEMM_F8_E4M3 || F8 == GEMM_F8_E5M2, "fp8 formats");
  typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
  i32x4 r;
#pragma unroll
  for (int d = 0; d < 2; ++d) {
    const unsigned u = (unsigned)v[d];
    f16x2 lo, hi;
    if constexpr (F8 == GEMM_F8_E4M3) {
      lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, false);
      hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(u, 1.0f, true);
    } else {
      lo = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(u, 1.0f, false);
      hi = __builtin_amdgcn_cvt_scalef32_pk_f16_bf8(u, 1.0f, true);
    }
    r[2 * d] = __builtin_bit_cast(int, lo);
    r[2 * d + 1] = __builtin_bit_cast(int, hi);
  }
  return r;
}

// fp32 -> bf16, round to nearest, ties to even; a NaN keeps its sign and
// the top of its payload, with the quiet bit set (upper half-word | 0x0040).
// gfx950's v_cvt_pk_bf16_f32 does exactly this (measured on MI355X against
// the integer form u + 0x7fff + ((u >> 16) & 1) on every upper half-word with
// eight lower halves each, ties and NaN payloads included: no difference).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  return __builtin_bit_cast(unsigned short, static_cast<__bf16>(f));
}

template <int OUT>
__device__ __forceinline__ void store_out(void* C, int64_t idx, float v) {
  if constexpr (OUT == GEMM_F32) {
    static_cast<float*>(C)[idx] = v;
  } else if constexpr (OUT == GEMM_F16) {
    // v_cvt_f16_f32: round to nearest even, fp16 subnormals kept, overflow to inf
    static_cast<_Float16*>(C)[idx] = static_cast<_Float16>(v);
  } else {
    static_cast<unsigned short*>(C)[idx] = f32_to_bf16(v);
  }
}

// One output element at a byte address.
template <int OUT>
__device__ __forceinline__ void store_at(char* p, float v) {
  if constexpr (OUT == GEMM_F32) {
    *reinterpret_cast<float*>(p) = v;
  } else if constexpr (OUT == GEMM_F16) {
    *reinterpret_cast<_Float16*>(p) = static_cast<_Float16>(v);
  } else {
    *reinterpret_cast<unsigned short*>(p) = f32_to_bf16(v);
  }
}

// The epilogue of one output element: the fp32 sum times the fp32 product
// of the scales, plus the fp32 bias of its column when there is one (one
// fp32 add), converted to the output format.  The multiply and the add
// round separately (never fused); a scale of 1 leaves the sum as it is
// (also a NaN's payload bits).
template <int OUT>
__device__ __forceinline__ void store_final(void* C, int64_t idx, float sum, float scale,
                                            const float* bias, int64_t col) {
#pragma clang fp contract(off)
  float v = scale == 1.0f ? sum : sum * scale;
  if (bias) v = v + bias[col];
  store_out<OUT>(C, idx, v);
}

// Transposing LDS reads (gfx950), and plain 16-byte LDS reads, at an LDS
// byte address plus a compile-time offset (the instruction's offset field).
// Issued as inline assembly: the compiler's own transposing-read builtin makes
// it wait for every outstanding buffer->LDS transfer before each read (it
// cannot tell which LDS bytes a transfer writes), which would drain the
// prefetch pipeline every stage.  The caller must wait for lgkmcnt before
// using a result, and must keep every result live until such a wait (the
// compiler takes an assembly output as written at issue, so a result it
// proves unused could share its registers with live values that the arriving
// data then overwrites).  In each group of 16 lanes of a transposing read,
// lanes 4t..4t+3 (16-bit) or 2t..2t+1 (8-bit) supply row t from their own
// addresses and lane j receives column j of those rows.
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr16_b64(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  i32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ i32x2 ds_read_tr8_b64(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  i32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
template <int OFF>
__device__ __forceinline__ i32x4 ds_read_b128_at(unsigned addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds_read offset field");
  i32x4 v;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "n"(OFF));
  return v;
}
// Keeps the N dwords of v live (in their registers) up to this point.
template <int N, class V>
__device__ __forceinline__ void keep_live(const V& v) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int x = v[e];
    asm volatile("" : : "v"(x));
  }
}

// Calls f(std::integral_constant<int, I>) for I = LO .. HI-1 in order, so that
// the body can use I in constant expressions (immediate offsets, wait counts).
template <int LO, class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, LO + I>{}), ...);
}
template <int LO, int HI, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (HI > LO) static_for_impl<LO>(f, std::make_integer_sequence<int, HI - LO>{});
}

// s_waitcnt immediate that waits until at most `n` vector-memory operations
// of this wave are outstanding (LDS/scalar and export counters unconstrained).
__host__ __device__ constexpr int vmcnt_imm(int n) {
  return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
}
// ... and until at most `n` LDS operations are outstanding.
__host__ __device__ constexpr int lgkmcnt_imm(int n) { return 15 | (3 << 14) | (7 << 4) | (n << 8); }

}  // namespace dev
}  // namespace imm
