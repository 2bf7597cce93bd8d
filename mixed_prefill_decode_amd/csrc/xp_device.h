// Device-side helpers shared by the gfx950 kernels: storage types, conversions,
// wave-level reductions and the MFMA operand abstraction.
//
// MFMA operand layout used everywhere (wave64):
//   32x32 tiles: lane l supplies row (or column) l % 32 and the k-slots
//                [8*(l/32), 8*(l/32) + 8) of a 16-deep k step;
//   16x16 tiles: lane l supplies row (or column) l % 16 and the k-slots
//                [8*(l/16), 8*(l/16) + 8) of a 32-deep k step, or
//                [4*(l/16), 4*(l/16) + 4) of a 16-deep k step.
// For bf16 one gfx950 MFMA consumes the whole step.  For fp32 the step is
// issued as several fp32 MFMAs whose single k-slot per lane group walks the
// same k-slots in order, so both types share one operand layout and the
// accumulator layouts below:
//   32x32 accumulator (16 floats): element r of lane l is row
//         8*(r/4) + 4*(l/32) + (r%4), column l%32;
//   16x16 accumulator (4 floats):  element r of lane l is row 4*(l/16) + r,
//         column l%16.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xp {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

// bf16 is carried as its 16-bit pattern.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest even (NaN stays NaN): gfx950's v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// ---- storage-type traits ---------------------------------------------------
template <typename T> struct St;
template <> struct St<bf16_t> {
  static constexpr int bytes = 2;
  __device__ static __forceinline__ float load(const void* p, long i) {
    return bf2f(reinterpret_cast<const uint16_t*>(p)[i]);
  }
  __device__ static __forceinline__ void store(void* p, long i, float v) {
    reinterpret_cast<uint16_t*>(p)[i] = f2bf(v);
  }
};
template <> struct St<float> {
  static constexpr int bytes = 4;
  __device__ static __forceinline__ float load(const void* p, long i) {
    return reinterpret_cast<const float*>(p)[i];
  }
  __device__ static __forceinline__ void store(void* p, long i, float v) {
    reinterpret_cast<float*>(p)[i] = v;
  }
};

// 4 consecutive elements at index i (i a multiple of 4, 4-element aligned storage)
template <typename T> struct St4;
template <> struct St4<bf16_t> {
  __device__ static __forceinline__ float4 load(const void* p, long i) {
    const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(p) + i);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u), __uint_as_float(w.y << 16),
                       __uint_as_float(w.y & 0xffff0000u));
  }
  __device__ static __forceinline__ void store(void* p, long i, float4 v) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(p) + i) =
        make_uint2(pack_bf16x2_(v.x, v.y), pack_bf16x2_(v.z, v.w));
  }
  __device__ static __forceinline__ uint32_t pack_bf16x2_(float a, float b) {
    return uint32_t(f2bf(a)) | (uint32_t(f2bf(b)) << 16);
  }
};
template <> struct St4<float> {
  __device__ static __forceinline__ float4 load(const void* p, long i) {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + i);
  }
  __device__ static __forceinline__ void store(void* p, long i, float4 v) {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(p) + i) = v;
  }
};

// Element offset of slot s, dim j inside a page's K plane.  The plane is stored
// 16-byte-chunk-major: chunk c holds dims [c E, (c + 1) E) of one slot (E = 16 bytes
// of T), and the chunks of one dim range are consecutive over the page's S slots
// ([d / E][S][E]).  An MFMA operand fragment of 16 keys then reads one contiguous run.
template <typename T>
__device__ __forceinline__ long k_elem(int s, int j, int S) {
  constexpr int E = 16 / St<T>::bytes;
  return (long(j / E) * S + s) * E + (j % E);
}

// value after a round trip through the storage type
template <typename T> __device__ __forceinline__ float round_st(float v);
template <> __device__ __forceinline__ float round_st<bf16_t>(float v) { return bf2f(f2bf(v)); }
template <> __device__ __forceinline__ float round_st<float>(float v) { return v; }

// ---- 8-element operand fragments --------------------------------------------
template <typename T> struct Frag8;
template <> struct Frag8<bf16_t> { uint4 v; };             // 8 x bf16 = 16 bytes
template <> struct Frag8<float> { float4 lo, hi; };        // 8 x fp32 = 32 bytes
template <typename T> struct Frag4;
template <> struct Frag4<bf16_t> { uint2 v; };             // 4 x bf16
template <> struct Frag4<float> { float4 v; };             // 4 x fp32

__device__ __forceinline__ void load_frag8(Frag8<bf16_t>& f, const void* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void load_frag8(Frag8<float>& f, const void* p) {
  f.lo = reinterpret_cast<const float4*>(p)[0];
  f.hi = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void zero_frag(Frag8<bf16_t>& f) { f.v = make_uint4(0, 0, 0, 0); }
__device__ __forceinline__ void zero_frag(Frag8<float>& f) {
  f.lo = make_float4(0.f, 0.f, 0.f, 0.f);
  f.hi = f.lo;
}
__device__ __forceinline__ void load_frag4(Frag4<bf16_t>& f, const void* p) {
  f.v = *reinterpret_cast<const uint2*>(p);
}
__device__ __forceinline__ void load_frag4(Frag4<float>& f, const void* p) {
  f.v = *reinterpret_cast<const float4*>(p);
}

// element e of a fragment as float / set from float
__device__ __forceinline__ float frag_get(const Frag8<bf16_t>& f, int e) {
  uint32_t w = (e < 2) ? f.v.x : (e < 4) ? f.v.y : (e < 6) ? f.v.z : f.v.w;
  return bf2f(uint16_t((e & 1) ? (w >> 16) : (w & 0xffffu)));
}
__device__ __forceinline__ float frag_get(const Frag8<float>& f, int e) {
  const float4& h = (e < 4) ? f.lo : f.hi;
  int k = e & 3;
  return k == 0 ? h.x : k == 1 ? h.y : k == 2 ? h.z : h.w;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
__device__ __forceinline__ void set_frag4(Frag4<bf16_t>& f, float a, float b, float c, float d) {
  f.v = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}
__device__ __forceinline__ void set_frag4(Frag4<float>& f, float a, float b, float c, float d) {
  f.v = make_float4(a, b, c, d);
}
__device__ __forceinline__ void set_frag8(Frag8<bf16_t>& f, const float* x) {
  f.v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7]));
}
__device__ __forceinline__ void set_frag8(Frag8<float>& f, const float* x) {
  f.lo = make_float4(x[0], x[1], x[2], x[3]);
  f.hi = make_float4(x[4], x[5], x[6], x[7]);
}

// ---- MFMA: 32x32 output, 16-deep k step --------------------------------------
__device__ __forceinline__ void mma32x32_k16(f32x16& acc, const Frag8<bf16_t>& a, const Frag8<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma32x32_k16(f32x16& acc, const Frag8<float>& a, const Frag8<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// ---- MFMA: 16x16 output, 32-deep k step ---------------------------------------
__device__ __forceinline__ void mma16x16_k32(f32x4& acc, const Frag8<bf16_t>& a, const Frag8<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a.v),
                                                __builtin_bit_cast(bf16x8, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16x16_k32(f32x4& acc, const Frag8<float>& a, const Frag8<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// ---- MFMA: 16x16 output, 16-deep k step (4 k-slots per lane group) ------------
__device__ __forceinline__ void mma16x16_k16(f32x4& acc, const Frag4<bf16_t>& a, const Frag4<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a.v),
                                                  __builtin_bit_cast(i16x4, b.v), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16x16_k16(f32x4& acc, const Frag4<float>& a, const Frag4<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.x, b.v.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.y, b.v.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.z, b.v.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v.w, b.v.w, acc, 0, 0, 0);
}

// ---- wave-level helpers ------------------------------------------------------
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }

// v of this lane and of lane l ^ 32, through gfx950's register lane swap between the two
// halves of the wave.  Unlike a bpermute it does not go through the LDS queue, so it does
// not wait behind the LDS reads in flight.  Each lane gets its own value in one of the
// two results and its partner's in the other.
__device__ __forceinline__ void halves_xor32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// the same for lanes l and l ^ 16 (the swap between neighbouring 16-lane rows)
__device__ __forceinline__ void halves_xor16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace xp
