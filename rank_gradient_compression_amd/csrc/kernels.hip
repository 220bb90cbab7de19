// gfx950 kernels of the PowerSGD bucket-compression step.
//
// The step follows "DDP Communication Hooks -- PyTorch 1.11.0", section "PowerSGD
// Hooks", powerSGD_hook steps 3.2 to 3.7 on one rank (both allreduces are the
// identity), with error feedback (first warning of that section) and the fp16
// unscale / inf-check of "torch.cuda.amp -- PyTorch 1.5.0", section "Gradient
// Scaling". Every kernel covers all tensors of a bucket in one launch, driven by
// a device table of work items, so a launch has thousands of workgroups.
//
//   Streaming passes share one tiling: (row block x 256-column block) work items;
//   a lane owns 4 consecutive columns (16-byte accesses) and keeps several rows of
//   loads in flight; narrow matrices pack several rows into one wavefront.
//   error memory  with error feedback, E's place keeps M' of the previous step
//           instead of E = M' - M_hat (binary32 for an fp32 state, 16 bits for the
//           wrappers' 16-bit states): with the step's P and Q (which the state keeps
//           anyway) the error is rebuilt exactly, as E = M'_prev - P Q^T with the very
//           arithmetic and rounding pass 3 uses for M_hat. Pass 3 then only writes
//           M_hat. A device flag says when E's place still holds the error itself.
//           An fp16 step skipped for inf must leave M'_prev intact: its plan keeps
//           M' in two alternating places (a device index names the current one; pass
//           1 writes the other, pass 3 of a step that ran switches them), or, with
//           one place, the whole bucket is checked before pass 1.
//   pass 1  M' = G (+ E), the error rebuilt from M'_prev and M' written over it (or
//           into the other place);
//           P = M' Q. Vector ranks: a workgroup owns whole rows, so each dot product is
//           finished inside it (shuffles, then LDS across wavefronts); matrix-core
//           ranks: 32 rows x 4096 columns per workgroup, a partial P per column group,
//           summed by the Gram kernel. fp16: x * inv_scale (and an OR of "not finite"
//           into found_inf when no check ran before).
//   orth    Gram-Schmidt with epsilon on P (and on the initial Q draw), run on the
//           columns of the Cholesky factor of P^T P (see the orthogonalization
//           section); ranks <= 8 do this in the prologue of every pass-2 workgroup
//           for its own rows from pass 1's Gram partials, larger ranks in kernels of
//           their own.
//   pass 2  Q = M'^T P. A workgroup owns a 256-column block of a row block; its row
//           slots and wavefronts are combined in a fixed order; tensors with several
//           row blocks write one partial per block, summed in a fixed order by the
//           pass-3 workgroups of that column block (vector ranks) or by a small
//           kernel of its own (matrix-core ranks): deterministic, no atomics, no
//           inter-workgroup fences (the kernel boundary publishes the partials).
//   pass 3  M_hat = P Q^T written into the bucket (fp16: round to nearest even).
//   q_init  Philox4x64-10 + Box-Muller draw of the initial Q (counter layout in
//           the public header's companion documentation).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "internal.h"

namespace psgd {
// Kernels and their device helpers live in a named namespace so that profiler
// output shows readable names (psgd::kern::k_pass1<...>).
namespace kern {

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n >> 1); }

__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ bool half_bits_not_finite(uint16_t h) {
  return (h & 0x7C00u) == 0x7C00u;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  return __half2float(__ushort_as_half(h));
}

// Loads 4 gradient values starting at bucket element idx (valid = elements left in
// the row); fp16 values are unscaled and checked.
template <bool F16>
__device__ __forceinline__ void load_grad4(const void* bucket, int64_t idx, bool vec,
                                           int valid, float inv_scale, float (&x)[4],
                                           int& bad) {
  if constexpr (F16) {
    const uint16_t* h = static_cast<const uint16_t*>(bucket) + idx;
    uint16_t raw[4] = {0, 0, 0, 0};
    if (vec) {
      const uint2 w = *reinterpret_cast<const uint2*>(h);
      raw[0] = w.x & 0xFFFFu;
      raw[1] = w.x >> 16;
      raw[2] = w.y & 0xFFFFu;
      raw[3] = w.y >> 16;
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a < valid) raw[a] = h[a];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      bad |= half_bits_not_finite(raw[a]) ? 1 : 0;
      x[a] = half_bits_to_float(raw[a]) * inv_scale;
    }
  } else {
    const float* f = static_cast<const float*>(bucket) + idx;
    if (vec) {
      const float4 w = *reinterpret_cast<const float4*>(f);
      x[0] = w.x;
      x[1] = w.y;
      x[2] = w.z;
      x[3] = w.w;
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a) x[a] = (a < valid) ? f[a] : 0.f;
    }
  }
}

__device__ __forceinline__ void load_f32x4(const float* p, bool vec, int valid,
                                           float (&x)[4]) {
  if (vec) {
    const float4 w = *reinterpret_cast<const float4*>(p);
    x[0] = w.x;
    x[1] = w.y;
    x[2] = w.z;
    x[3] = w.w;
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) x[a] = (a < valid) ? p[a] : 0.f;
  }
}

__device__ __forceinline__ void store_f32x4(float* p, bool vec, int valid,
                                            const float (&x)[4]) {
  if (vec) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (a < valid) p[a] = x[a];
  }
}

__device__ __forceinline__ void store_f16x4(uint16_t* h, bool vec, int valid,
                                            const float (&x)[4]) {
  uint16_t o[4];
#pragma unroll
  for (int a = 0; a < 4; ++a) o[a] = __half_as_ushort(__float2half_rn(x[a]));
  if (vec) {
    uint2 w;
    w.x = static_cast<uint32_t>(o[0]) | (static_cast<uint32_t>(o[1]) << 16);
    w.y = static_cast<uint32_t>(o[2]) | (static_cast<uint32_t>(o[3]) << 16);
    *reinterpret_cast<uint2*>(h) = w;
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (a < valid) h[a] = o[a];
  }
}

// q[a][k] = Q[(c + a) * R + k] for rows c..c+3 of a row-major (m x R) block; rows at
// or beyond m read as zero.
template <int R>
__device__ __forceinline__ void load_q_rows(const float* __restrict__ Q, int c, int m,
                                            float (&q)[4][R]) {
  if (c + 3 < m) {
    const float4* p = reinterpret_cast<const float4*>(Q + static_cast<int64_t>(c) * R);
    if constexpr (R == 1) {
      const float4 w = p[0];
      q[0][0] = w.x;
      q[1][0] = w.y;
      q[2][0] = w.z;
      q[3][0] = w.w;
    } else if constexpr (R == 2) {
      const float4 w0 = p[0], w1 = p[1];
      q[0][0] = w0.x;
      q[0][1] = w0.y;
      q[1][0] = w0.z;
      q[1][1] = w0.w;
      q[2][0] = w1.x;
      q[2][1] = w1.y;
      q[3][0] = w1.z;
      q[3][1] = w1.w;
    } else {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int k4 = 0; k4 < R / 4; ++k4) {
          const float4 w = p[a * (R / 4) + k4];
          q[a][4 * k4 + 0] = w.x;
          q[a][4 * k4 + 1] = w.y;
          q[a][4 * k4 + 2] = w.z;
          q[a][4 * k4 + 3] = w.w;
        }
      }
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int k = 0; k < R; ++k)
        q[a][k] = (c + a < m) ? Q[static_cast<int64_t>(c + a) * R + k] : 0.f;
    }
  }
}

// Loads 4 gradient values of a 16-byte aligned group without a branch (address
// already clamped into the matrix); fp16 values are unscaled, `raw_bad` tells whether
// any of them is inf or NaN.
template <bool F16>
__device__ __forceinline__ void load_grad4_vec(const void* bucket, int64_t idx, float inv_scale,
                                               float (&x)[4], bool& raw_bad) {
  if constexpr (F16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(bucket) + idx);
    const uint16_t raw[4] = {static_cast<uint16_t>(w.x & 0xFFFFu), static_cast<uint16_t>(w.x >> 16),
                             static_cast<uint16_t>(w.y & 0xFFFFu), static_cast<uint16_t>(w.y >> 16)};
    raw_bad = false;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      raw_bad |= half_bits_not_finite(raw[a]);
      x[a] = half_bits_to_float(raw[a]) * inv_scale;
    }
  } else {
    const float4 w = *reinterpret_cast<const float4*>(static_cast<const float*>(bucket) + idx);
    x[0] = w.x;
    x[1] = w.y;
    x[2] = w.z;
    x[3] = w.w;
    raw_bad = false;
  }
}

__device__ __forceinline__ void load_f4(const float* p, float (&x)[4]) {
  const float4 w = *reinterpret_cast<const float4*>(p);
  x[0] = w.x;
  x[1] = w.y;
  x[2] = w.z;
  x[3] = w.w;
}

// How the vector-rank passes access a matrix's rows (chosen per matrix):
//   kLdAligned    rows 16-byte aligned (m % 4 == 0): one aligned 16-byte load per lane.
//   kLdUnaligned  rows only 4-byte aligned (2-byte for fp16), m >= 4: one unaligned
//                 16-byte (fp16: 8-byte) load per lane, which gfx950 performs in one
//                 instruction; a row's last, partial group is loaded ending at column
//                 m - 1 and moved into place with selects, so no load needs a branch.
//   kLdScalar     m < 4: four scalar loads at offsets clamped into the row.
constexpr int kLdScalar = 0;
constexpr int kLdUnaligned = 1;
constexpr int kLdAligned = 2;

typedef float f32x4u __attribute__((ext_vector_type(4), aligned(4)));
typedef unsigned int u32x2u __attribute__((ext_vector_type(2), aligned(2)));

// w[shift + a] for a = 0..3, zero past w[3]: the group loaded `shift` (0..3) elements
// early. Two conditional shifts (by 1, then by 2) of plain two-way selects.
__device__ __forceinline__ void shift_down4(const float (&w)[4], int shift, float (&x)[4]) {
  const bool s1 = (shift & 1) != 0;
  const bool s2 = (shift & 2) != 0;
  const float a0 = s1 ? w[1] : w[0];
  const float a1 = s1 ? w[2] : w[1];
  const float a2 = s1 ? w[3] : w[2];
  const float a3 = s1 ? 0.f : w[3];
  x[0] = s2 ? a2 : a0;
  x[1] = s2 ? a3 : a1;
  x[2] = s2 ? 0.f : a2;
  x[3] = s2 ? 0.f : a3;
}

// Branch-free loads of 4 consecutive values starting at element `p` of a row that has
// `valid` >= 1 elements left from there (the row index is clamped by the caller); the
// values past the row's end read as zero.
template <int LD>
__device__ __forceinline__ void ld_f32x4(const float* p, int valid, float (&x)[4]) {
  if constexpr (LD == kLdAligned) {
    load_f4(p, x);
  } else if constexpr (LD == kLdUnaligned) {
    const int shift = valid >= 4 ? 0 : 4 - valid;
    const f32x4u v = *reinterpret_cast<const f32x4u*>(p - shift);
    const float w[4] = {v[0], v[1], v[2], v[3]};
    shift_down4(w, shift, x);
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const float v = p[min(a, valid - 1)];
      x[a] = a < valid ? v : 0.f;
    }
  }
}

// Gradient values (fp16: unscaled; `raw_bad` = one of the values in the row is inf/NaN).
template <bool F16, int LD>
__device__ __forceinline__ void ld_grad4(const void* bucket, int64_t idx, int valid,
                                         float inv_scale, float (&x)[4], bool& raw_bad) {
  if constexpr (LD == kLdAligned) {
    load_grad4_vec<F16>(bucket, idx, inv_scale, x, raw_bad);
  } else if constexpr (F16 && LD == kLdUnaligned) {
    const int shift = valid >= 4 ? 0 : 4 - valid;
    const u32x2u v =
        *reinterpret_cast<const u32x2u*>(static_cast<const uint16_t*>(bucket) + idx - shift);
    const uint16_t raw[4] = {static_cast<uint16_t>(v[0] & 0xFFFFu), static_cast<uint16_t>(v[0] >> 16),
                             static_cast<uint16_t>(v[1] & 0xFFFFu), static_cast<uint16_t>(v[1] >> 16)};
    float w[4];
    raw_bad = false;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      raw_bad |= (a >= shift) && half_bits_not_finite(raw[a]);  // the row's own values
      w[a] = half_bits_to_float(raw[a]) * inv_scale;
    }
    shift_down4(w, shift, x);
  } else if constexpr (F16) {
    const uint16_t* h = static_cast<const uint16_t*>(bucket) + idx;
    raw_bad = false;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint16_t v = h[min(a, valid - 1)];
      const bool in = a < valid;
      raw_bad |= in && half_bits_not_finite(v);
      x[a] = in ? half_bits_to_float(v) * inv_scale : 0.f;
    }
  } else {
    ld_f32x4<LD>(static_cast<const float*>(bucket) + idx, valid, x);
    raw_bad = false;
  }
}

template <int LD>
__device__ __forceinline__ void st_f32x4(float* p, int valid, const float (&x)[4]) {
  if constexpr (LD == kLdAligned) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
  } else if constexpr (LD == kLdUnaligned) {
    if (valid >= 4) {
      *reinterpret_cast<f32x4u*>(p) = f32x4u{x[0], x[1], x[2], x[3]};
    } else {
#pragma unroll
      for (int a = 0; a < 3; ++a)
        if (a < valid) p[a] = x[a];
    }
  } else {
    store_f32x4(p, false, valid, x);
  }
}

template <int LD>
__device__ __forceinline__ void st_f16x4(uint16_t* h, int valid, const float (&x)[4]) {
  if constexpr (LD == kLdUnaligned) {
    if (valid >= 4) {
      uint16_t o[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) o[a] = __half_as_ushort(__float2half_rn(x[a]));
      *reinterpret_cast<u32x2u*>(h) =
          u32x2u{static_cast<uint32_t>(o[0]) | (static_cast<uint32_t>(o[1]) << 16),
                 static_cast<uint32_t>(o[2]) | (static_cast<uint32_t>(o[3]) << 16)};
      return;
    }
  }
  store_f16x4(h, LD == kLdAligned, valid, x);
}

// Q rows c..c+3 (R values each) of a row-major block; rows at or past m read as zero.
template <int R, int LD>
__device__ __forceinline__ void ld_q4(const float* __restrict__ Q, int c, int valid,
                                      float (&q)[4][R]) {
  if constexpr (LD != kLdScalar) {
    // kLdUnaligned: the four rows ending at row m - 1 when fewer than four are left
    const int shift = (LD == kLdAligned || valid >= 4) ? 0 : 4 - valid;
    const float* src = Q + static_cast<int64_t>(c - shift) * R;
    float f[4 * R];
#pragma unroll
    for (int i = 0; i < R; ++i) {
      float w[4];
      if constexpr (LD == kLdAligned || R % 4 == 0) {
        load_f4(src + 4 * i, w);
      } else {
        const f32x4u v = *reinterpret_cast<const f32x4u*>(src + 4 * i);
        w[0] = v[0];
        w[1] = v[1];
        w[2] = v[2];
        w[3] = v[3];
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) f[4 * i + a] = w[a];
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const float w[4] = {f[k], f[R + k], f[2 * R + k], f[3 * R + k]};
      float x[4];
      shift_down4(w, shift, x);
#pragma unroll
      for (int a = 0; a < 4; ++a) q[a][k] = x[a];
    }
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int k = 0; k < R; ++k) {
        const float v = Q[static_cast<int64_t>(c + min(a, valid - 1)) * R + k];
        q[a][k] = a < valid ? v : 0.f;
      }
  }
}

// Lane geometry of a tile (see TensorDesc): row slot, column group and first column.
// ------------------------------------------------------- 16-bit state values
//
// The wrapped hook keeps M' and E as 16-bit values (binary16 or bfloat16), rounded to
// nearest even wherever a value is formed; arithmetic stays in fp32.

// bfloat16 bits of x rounded to nearest even (ties to the even significand), +-inf past
// the largest finite value, a NaN kept a quiet NaN with its sign and upper payload bits:
// the compiler's __bf16 conversion, one v_cvt_pk_bf16_f32 on gfx950 (which equals
// adding 0x7FFF plus the kept part's lowest bit to the binary32 pattern and keeping its
// upper half, for every non-NaN input).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

template <int ST>
__device__ __forceinline__ uint16_t to_h16(float x) {
  if constexpr (ST == kStBF16)
    return f32_to_bf16_bits(x);
  else
    return __half_as_ushort(__float2half_rn(x));
}

template <int ST>
__device__ __forceinline__ float from_h16(uint32_t h) {
  if constexpr (ST == kStBF16)
    return __uint_as_float((h & 0xFFFFu) << 16);
  else
    return half_bits_to_float(static_cast<uint16_t>(h & 0xFFFFu));
}

// x rounded to the state's precision (the identity for an fp32 state).
template <int ST>
__device__ __forceinline__ float rnd16(float x) {
  if constexpr (ST == kStF32)
    return x;
  else
    return from_h16<ST>(to_h16<ST>(x));
}

// 4 consecutive 16-bit state values of a row (the same access modes as ld_f32x4).
template <int ST, int LD>
__device__ __forceinline__ void ld_h4(const uint16_t* p, int valid, float (&x)[4]) {
  if constexpr (LD == kLdAligned) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    x[0] = from_h16<ST>(v.x);
    x[1] = from_h16<ST>(v.x >> 16);
    x[2] = from_h16<ST>(v.y);
    x[3] = from_h16<ST>(v.y >> 16);
  } else if constexpr (LD == kLdUnaligned) {
    const int shift = valid >= 4 ? 0 : 4 - valid;
    const u32x2u v = *reinterpret_cast<const u32x2u*>(p - shift);
    const float w[4] = {from_h16<ST>(v[0]), from_h16<ST>(v[0] >> 16), from_h16<ST>(v[1]),
                        from_h16<ST>(v[1] >> 16)};
    shift_down4(w, shift, x);
  } else {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint16_t v = p[min(a, valid - 1)];
      x[a] = a < valid ? from_h16<ST>(v) : 0.f;
    }
  }
}

// Two values rounded to the state's precision, packed (a in the low half): bfloat16
// pairs take one conversion instruction.
template <int ST>
__device__ __forceinline__ uint32_t pack_h16x2(float a, float b) {
  if constexpr (ST == kStBF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
  else
    return static_cast<uint32_t>(to_h16<ST>(a)) | (static_cast<uint32_t>(to_h16<ST>(b)) << 16);
}

// Rounds 4 values to the state's precision and stores the first `valid` of them.
template <int ST, int LD>
__device__ __forceinline__ void st_h4(uint16_t* p, int valid, const float (&x)[4]) {
  if constexpr (LD == kLdAligned) {
    *reinterpret_cast<uint2*>(p) =
        make_uint2(pack_h16x2<ST>(x[0], x[1]), pack_h16x2<ST>(x[2], x[3]));
  } else {
    if (LD == kLdUnaligned && valid >= 4) {
      *reinterpret_cast<u32x2u*>(p) =
          u32x2u{pack_h16x2<ST>(x[0], x[1]), pack_h16x2<ST>(x[2], x[3])};
      return;
    }
    uint32_t o[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) o[a] = to_h16<ST>(x[a]);
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (a < valid) p[a] = static_cast<uint16_t>(o[a]);
  }
}

struct LaneGeom {
  int lpr;      // lanes per row slot
  int rpw;      // row slots per wavefront
  int slot;     // this lane's row slot
  int g;        // this lane's column group inside the slot
  int c;        // first of this lane's 4 columns
  bool col_ok;  // the lane owns at least one column of the matrix
  int valid;    // columns left in the row from c
};

__device__ __forceinline__ LaneGeom lane_geom(const TensorDesc& d, int cb, int lane) {
  LaneGeom L;
  L.lpr = d.lpr;
  L.rpw = 64 / d.lpr;
  L.slot = lane / d.lpr;
  L.g = lane - L.slot * d.lpr;
  L.c = cb * kColBlock + L.g * 4;
  L.col_ok = L.c < d.m;
  L.valid = d.m - L.c;
  return L;
}

// Geometry of a tile of a matrix at least 256 columns wide: a row slot is a whole
// wavefront, so the row a wavefront works on is uniform and P rows are scalar loads.
template <bool WIDE>
__device__ __forceinline__ LaneGeom tile_geom(const TensorDesc& d, int cb, int lane) {
  if constexpr (WIDE) {
    LaneGeom L;
    L.lpr = 64;
    L.rpw = 1;
    L.slot = 0;
    L.g = lane;
    L.c = cb * kColBlock + lane * 4;
    L.col_ok = L.c < d.m;
    L.valid = d.m - L.c;
    return L;
  } else {
    return lane_geom(d, cb, lane);
  }
}

// P row `row` (R floats, 16-byte aligned when R >= 4).
template <int R>
__device__ __forceinline__ void load_p_row(const float* __restrict__ Pt, int row,
                                           float (&p)[R]) {
  const float* src = Pt + static_cast<int64_t>(row) * R;
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int k4 = 0; k4 < R / 4; ++k4) {
      const float4 w = reinterpret_cast<const float4*>(src)[k4];
      p[4 * k4 + 0] = w.x;
      p[4 * k4 + 1] = w.y;
      p[4 * k4 + 2] = w.z;
      p[4 * k4 + 3] = w.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < R; ++k) p[k] = src[k];
  }
}

// The same row when `row` is uniform across the wavefront: read through the constant
// address space, so the compiler issues scalar loads (read-only; P was written by an
// earlier kernel of the stream).
template <int R>
__device__ __forceinline__ void load_p_row_uniform(const float* __restrict__ Pt, int row,
                                                   float (&p)[R]) {
  typedef const __attribute__((address_space(4))) float cfloat;
  cfloat* src = (cfloat*)(Pt + static_cast<int64_t>(row) * R);
#pragma unroll
  for (int k = 0; k < R; ++k) p[k] = src[k];
}

template <int R>
__device__ __forceinline__ void store_p_row(float* __restrict__ Pt, int row,
                                            const float (&p)[R]) {
  float* dst = Pt + static_cast<int64_t>(row) * R;
  if constexpr (R % 4 == 0) {
#pragma unroll
    for (int k4 = 0; k4 < R / 4; ++k4)
      reinterpret_cast<float4*>(dst)[k4] =
          make_float4(p[4 * k4], p[4 * k4 + 1], p[4 * k4 + 2], p[4 * k4 + 3]);
  } else {
#pragma unroll
    for (int k = 0; k < R; ++k) dst[k] = p[k];
  }
}

// M_hat = P Q^T for 4 consecutive columns of one row (vector ranks): one fused
// multiply-add chain in rank order per value. Pass 3 writes these values and the error
// memory is rebuilt from them (E = M' - M_hat), so every user computes them here.
template <int R>
__device__ __forceinline__ void mhat4(const float (&p)[R], const float (&q)[4][R],
                                      float (&mh)[4]) {
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    float s = p[0] * q[a][0];
#pragma unroll
    for (int k = 1; k < R; ++k) s = __builtin_fmaf(p[k], q[a][k], s);
    mh[a] = s;
  }
}

// With error feedback, E's place keeps M' of the previous step and the error is rebuilt
// from it and the step's factors: in binary32 for an fp32 state (fp32 or fp16 buckets),
// in the state's 16 bits for the wrappers' 16-bit states.
template <bool F16, bool EF, int ST>
constexpr bool stored_mprime() { return EF; }

// The previous error rebuilt from M'_prev (w) and M_hat_prev = P Q^T (mh, as the
// matrix product left it) with pass 3's rounding: w - mh for an fp32 state; a 16-bit
// state's pass 3 rounded M_hat to 16 bits and the error M' - M_hat again.
template <int ST>
__device__ __forceinline__ float rebuilt_error(float w, float mh) {
  if constexpr (ST == kStF32)
    return w - mh;
  else
    return rnd16<ST>(w - rnd16<ST>(mh));
}

// Whether pass 1 rebuilds the previous error from M'_prev in E's place: a state keeping
// M', given the previous factors, unless E's place still holds the error itself.
__device__ __forceinline__ bool rebuild_error(const Pass1Args& a) {
  return a.Pe != nullptr && !(a.wflag != nullptr && *a.wflag != 0);
}

// Whether E's place holds the error itself at a materialization.
__device__ __forceinline__ bool holds_error(const Pass3Args& a) {
  return a.wflag != nullptr && *a.wflag != 0;
}

// Offset (floats) of E's current place, holding M'_prev (or the error): 0 for one
// buffer; with two (wstride apart, an fp16 bucket's double-buffered M') the one *widx
// names. A step's pass 1 writes M' into the other place, wstride - w_cur.
__device__ __forceinline__ int64_t w_cur(const int32_t* widx, int64_t wstride) {
  return (wstride != 0 && *widx != 0) ? wstride : 0;
}

// Pass 3 of a step that ran (after its inf check) marks E's place as holding M': one
// lane of workgroup 0 (a vector store).
template <bool F16, bool EF, int ST, bool MAT>
__device__ __forceinline__ void mark_mprime(const Pass3Args& a) {
  if constexpr (stored_mprime<F16, EF, ST>() && !MAT) {
    if (a.wflag != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
      *a.wflag = 0;
      // double-buffered M': the place pass 1 wrote becomes the current one
      if (a.wstride != 0) *a.widx = 1 - *a.widx;
    }
  }
}

// A materialized error (4 values from element off of E's layout): binary32 into Eout,
// or, called without Eout, back into E's current place (wc: its offset), in 16 bits for
// a 16-bit state.
template <int ST, int LD>
__device__ __forceinline__ void store_materialized(const Pass3Args& a, int64_t wc, int64_t off,
                                                   int valid, const float (&e)[4]) {
  if (a.Eout == nullptr) {
    if constexpr (ST != kStF32)
      st_h4<ST, LD>(a.Eh + off, valid, e);
    else
      st_f32x4<LD>(a.E + wc + off, valid, e);
    return;
  }
  st_f32x4<LD>(a.Eout + off, valid, e);
}

// ----------------------------------------------------------------------- pass 1

// inf/NaN check of an fp16 range: the values before the first 16-byte boundary one
// by one, then eight per 16-byte load, then the tail.
__device__ __forceinline__ int f16_pair_not_finite(uint32_t w) {
  return ((w & 0x7C00u) == 0x7C00u || (w & 0x7C000000u) == 0x7C000000u) ? 1 : 0;
}

__device__ void f16_check_range(const FlatTile ft, const void* bucket,
                                int32_t* found_inf) {
  const uint16_t* h = static_cast<const uint16_t*>(bucket) + ft.start;
  const int64_t mis = static_cast<int64_t>((reinterpret_cast<uintptr_t>(h) >> 1) & 7);
  const int64_t head = min(ft.len, (8 - mis) & 7);
  const int64_t nv = (ft.len - head) / 8;
  int bad = 0;
  for (int64_t i = threadIdx.x; i < head; i += blockDim.x)
    bad |= half_bits_not_finite(h[i]) ? 1 : 0;
  const uint4* v = reinterpret_cast<const uint4*>(h + head);
  auto check8 = [](const uint4 w) {
    return f16_pair_not_finite(w.x) | f16_pair_not_finite(w.y) | f16_pair_not_finite(w.z) |
           f16_pair_not_finite(w.w);
  };
  const int64_t bd = blockDim.x;
  int64_t i = threadIdx.x;
  for (; i + 3 * bd < nv; i += 4 * bd) {  // four loads in flight
    const uint4 w0 = v[i], w1 = v[i + bd], w2 = v[i + 2 * bd], w3 = v[i + 3 * bd];
    bad |= check8(w0) | check8(w1) | check8(w2) | check8(w3);
  }
  for (; i < nv; i += bd) bad |= check8(v[i]);
  for (int64_t i = head + 8 * nv + threadIdx.x; i < ft.len; i += blockDim.x)
    bad |= half_bits_not_finite(h[i]) ? 1 : 0;
  if (__any(bad) && (threadIdx.x & 63) == 0) atomicOr(found_inf, 1);
}

// Adds the outer product of one P row (masked to the rank in use) to packed fp64
// Gram accumulators.
template <int R>
__device__ __forceinline__ void gram_add(double (&gacc)[gram_size<R>()], const float (&p)[R]) {
#pragma unroll
  for (int i = 0; i < R; ++i)
#pragma unroll
    for (int j = i; j < R; ++j)
      gacc[tri_index(i, j, R)] += static_cast<double>(p[i]) * static_cast<double>(p[j]);
}

// Sums NG doubles over the workgroup in a fixed order (wavefront shuffles, then the
// four wavefronts in order) and writes them to dst (threads < NG).
template <int NG>
__device__ __forceinline__ void block_sum_to(double (&v)[NG], double* dst, double (*red)[NG]) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
#pragma unroll
  for (int e = 0; e < NG; ++e) {
    double x = v[e];
#pragma unroll
    for (int mask = 32; mask >= 1; mask >>= 1) x += __shfl_xor(x, mask);
    v[e] = x;
  }
  if (lane == 0) {
#pragma unroll
    for (int e = 0; e < NG; ++e) red[wave][e] = v[e];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < NG; e += kThreads)
    dst[e] = ((red[0][e] + red[1][e]) + red[2][e]) + red[3][e];
}

template <int R>
constexpr int pass1_ng() { return R <= kMaxFusedGramRank ? gram_size<R>() : 1; }

// P = M' Q over one row block. Threads of a row slot sweep the row's columns,
// U rows per thread are loaded before any is used, and the slot's partial dot
// products are summed with shuffles (and through LDS when a slot spans wavefronts).
// LD: how the matrix's rows are loaded (kLdAligned, kLdUnaligned, kLdScalar). The rows
// of a slot are clamped into the row block, so every load of an iteration is issued
// before any is used; the results of clamped duplicate rows are discarded.
template <int R, int U, bool F16, bool EF, int LD, int ST>
__device__ __forceinline__ void pass1_body(const Pass1Args& args, const TensorDesc& d,
                                           const Tile& t, float* red,
                                           double (*gred)[pass1_ng<R>()]) {
  constexpr bool GRAM = R <= kMaxFusedGramRank;
  constexpr int NG = pass1_ng<R>();
  double gacc[NG];
#pragma unroll
  for (int e = 0; e < NG; ++e) gacc[e] = 0.0;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_index();
  const int m = d.m;
  const int lprw = d.lprw;
  const int slots = kThreads / lprw;
  const int slot = tid / lprw;
  const int g = tid - slot * lprw;
  const int sweep = 4 * lprw;
  const int r0 = t.a * d.rpb1;
  const int r1 = min(d.n, r0 + d.rpb1);
  const float* __restrict__ Qt = args.Q + d.qoff;
  // E's current place holds M'_prev (or the error); M' goes to the other place (the
  // same one with a single buffer)
  const int64_t wc = w_cur(args.widx, args.wstride);
  float* __restrict__ Ebase = args.E + d.eoff;  // both places derive from it (they may be one)
  const float* Ein = Ebase + wc;
  float* Eout = Ebase + (args.wstride - wc);
  constexpr bool SM = stored_mprime<F16, EF, ST>();
  // E's place holds M'_prev: rebuild E = M'_prev - Pe Q^T (Q is the warm-start Q)
  const bool rebuild = SM && rebuild_error(args);
  int bad = 0;
  for (int rw = r0; rw < r1; rw += slots * U) {
    int64_t rbase[U];
    bool rok[U];
    float pe[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = rw + u * slots + slot;
      rok[u] = row < r1;
      rbase[u] = static_cast<int64_t>(min(row, r1 - 1)) * m;
      if constexpr (SM) {
        if (rebuild) load_p_row<R>(args.Pe + d.poff, min(row, r1 - 1), pe[u]);
      }
    }
    float acc[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < R; ++k) acc[u][k] = 0.f;
    for (int c = g * 4; c < m; c += sweep) {
      const int valid = m - c;
      float q[4][R];
      ld_q4<R, LD>(Qt, c, valid, q);
      float x[U][4];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        bool rb;
        ld_grad4<F16, LD>(args.bucket, d.boff + rbase[u] + c, valid, args.inv_scale, x[u], rb);
        if constexpr (F16) bad |= (rok[u] && rb) ? 1 : 0;
      }
      if constexpr (ST != kStF32) {
        // the wrapper's cast, then M' = G + E formed in 16 bits and kept for passes 2, 3
        // (with error feedback Mh is E's place itself: M' replaces M'_prev there)
        if constexpr (EF) {
          float e[U][4];
#pragma unroll
          for (int u = 0; u < U; ++u) ld_h4<ST, LD>(args.Eh + d.eoff + rbase[u] + c, valid, e[u]);
          if (rebuild) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
              float mh[4];
              mhat4<R>(pe[u], q, mh);
#pragma unroll
              for (int a = 0; a < 4; ++a) e[u][a] = rebuilt_error<ST>(e[u][a], mh[a]);
            }
          }
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < 4; ++a) x[u][a] = rnd16<ST>(rnd16<ST>(x[u][a]) + e[u][a]);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < 4; ++a) x[u][a] = rnd16<ST>(x[u][a]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (rok[u]) st_h4<ST, LD>(args.Mh + d.eoff + rbase[u] + c, valid, x[u]);
      } else if constexpr (EF) {
        float e[U][4];
#pragma unroll
        for (int u = 0; u < U; ++u) ld_f32x4<LD>(Ein + rbase[u] + c, valid, e[u]);
        if (rebuild) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float mh[4];
            mhat4<R>(pe[u], q, mh);
#pragma unroll
            for (int a = 0; a < 4; ++a) e[u][a] = rebuilt_error<ST>(e[u][a], mh[a]);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
          for (int a = 0; a < 4; ++a) x[u][a] += e[u][a];
          if (rok[u]) st_f32x4<LD>(Eout + rbase[u] + c, valid, x[u]);  // M' in E's place
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int k = 0; k < R; ++k)
          acc[u][k] += x[u][0] * q[0][k] + x[u][1] * q[1][k] + x[u][2] * q[2][k] +
                       x[u][3] * q[3][k];
    }
    if (lprw >= 64) {
      // sums over the whole wavefront: each of the first log2(U) exchanges halves the
      // rows a lane holds (lanes with bit 32 >> s set keep the upper half and send the
      // lower), then the one row left is summed over the remaining lane bits. Lane l
      // ends with the sums of row uu(l); the lanes with the low bits clear write them.
      constexpr int H = (U >= 2) + (U >= 4) + (U >= 8) + (U >= 16);
      static_assert((1 << H) == U, "rows per lane must be a power of two");
#pragma unroll
      for (int s = 0; s < H; ++s) {
        const int mask = 32 >> s;
        const int half = (U >> s) / 2;
        const bool up = (lane & mask) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i)
#pragma unroll
          for (int k = 0; k < R; ++k) {
            const float lo = acc[i][k];
            const float hi = acc[i + half][k];
            acc[i][k] = (up ? hi : lo) + __shfl_xor(up ? lo : hi, mask);
          }
      }
      for (int mask = 32 >> H; mask > 0; mask >>= 1) {
#pragma unroll
        for (int k = 0; k < R; ++k) acc[0][k] += __shfl_xor(acc[0][k], mask);
      }
      int uu = 0;
#pragma unroll
      for (int s = 0; s < H; ++s) uu += (lane & (32 >> s)) ? (U >> (s + 1)) : 0;
      const int row = rw + uu * slots + slot;
      if ((lane & ((64 >> H) - 1)) == 0 && row < r1) {
        if (lprw == 64) {
          float pr[R];
#pragma unroll
          for (int k = 0; k < R; ++k) pr[k] = (k < d.rank) ? rnd16<ST>(acc[0][k]) : 0.f;
          store_p_row<R>(args.P + d.poff, row, pr);
          if constexpr (GRAM) gram_add<R>(gacc, pr);
        } else {
          // a slot spans wps wavefronts: park this wavefront's sums until the tile ends
          const int wps = lprw >> 6;
          float* dst = red + ((row - r0) * wps + (wave & (wps - 1))) * R;
#pragma unroll
          for (int k = 0; k < R; ++k) dst[k] = acc[0][k];
        }
      }
    } else {
      // a slot inside a wavefront: sum over its lprw lanes, its first lane writes
      for (int mask = lprw >> 1; mask > 0; mask >>= 1) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int k = 0; k < R; ++k) acc[u][k] += __shfl_xor(acc[u][k], mask);
      }
      if (g == 0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int row = rw + u * slots + slot;
          if (rok[u]) {
            float pr[R];
#pragma unroll
            for (int k = 0; k < R; ++k) pr[k] = (k < d.rank) ? rnd16<ST>(acc[u][k]) : 0.f;
            store_p_row<R>(args.P + d.poff, row, pr);
            if constexpr (GRAM) gram_add<R>(gacc, pr);
          }
        }
      }
    }
  }
  if (lprw > 64) {
    // add the wavefront sums of every row in wavefront order
    __syncthreads();
    const int wps = lprw >> 6;
    for (int i = tid; i < r1 - r0; i += kThreads) {
      float pr[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        float v = 0.f;
        for (int w = 0; w < wps; ++w) v += red[(i * wps + w) * R + k];
        pr[k] = (k < d.rank) ? rnd16<ST>(v) : 0.f;
      }
      store_p_row<R>(args.P + d.poff, r0 + i, pr);
      if constexpr (GRAM) gram_add<R>(gacc, pr);
    }
  }
  if constexpr (F16) {
    if (__any(bad) && lane == 0) atomicOr(args.found_inf, 1);
  }
  if constexpr (GRAM)
    block_sum_to<NG>(gacc, args.gram + d.goff + static_cast<int64_t>(t.a) * NG, gred);
}

template <int R, int U, bool F16, bool EF, int ST>
__global__ void __launch_bounds__(kThreads) k_pass1(Pass1Args args) {
  __shared__ float red[kPass1SlotSums * R];
  __shared__ double gred[kThreads / 64][pass1_ng<R>()];
  if constexpr (F16 && stored_mprime<F16, EF, ST>()) {
    // a step already known to be skipped (the bucket's check ran before this pass, or,
    // with two E places, another workgroup of it found inf) needs none of its results
    if (*args.found_inf) return;
  }
  if (static_cast<int>(blockIdx.x) >= args.ntiles) {
    if constexpr (F16)
      f16_check_range(args.ftiles[blockIdx.x - args.ntiles], args.bucket, args.found_inf);
    return;
  }
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if (d.vec)
    pass1_body<R, U, F16, EF, kLdAligned, ST>(args, d, t, red, gred);
  else if (d.m >= 4)
    pass1_body<R, U, F16, EF, kLdUnaligned, ST>(args, d, t, red, gred);
  else
    pass1_body<R, U, F16, EF, kLdScalar, ST>(args, d, t, red, gred);
}

// ------------------------------------------------------------ orthogonalization
//
// Gram-Schmidt with epsilon (step 3.4) needs only the inner products of the columns
// of P, so it can run on any vectors that have the same inner products. The columns
// of the upper-triangular Cholesky factor C of the Gram matrix G = P^T P = C^T C are
// such vectors: r of them, r entries long. The recurrence runs on them in fp64 while
// the same linear steps are applied to coefficient vectors, which gives the r x r
// transform T with orthogonalized P = P T (applied once, in fp64). Modified
// Gram-Schmidt loses orthogonality in proportion to cond(C) = cond(P), not to its
// square, and C is factored in double-double arithmetic.
//
// G arrives as partial sums over row blocks. Products of binary32 values are exact
// in binary64, so only the sums round: pass 1 accumulates fp64 partials for ranks <= 8;
// the Gram kernel (matrix-core ranks, and the initial Q at every rank) accumulates
// double-double ones. An fp64 sum rounds by about sqrt(n) 2^-53 of the diagonal, so a
// Cholesky pivot below kCholTau of its diagonal entry is not resolved by it: the Gram
// matrix of that P is then recomputed in double-double from P's rows. This happens for
// (numerically) rank-deficient P, e.g. M' of rank below r.

constexpr double kCholTau = 0x1p-36;

// Double-double arithmetic (Dekker 1971; Knuth, TAOCP vol. 2, 4.2.2): a value is the
// unevaluated sum hi + lo with |lo| <= ulp(hi) / 2.
struct DD {
  double hi, lo;
};

// s + e = a + b exactly.
__device__ __forceinline__ DD dd_two_sum(double a, double b) {
  const double s = a + b;
  const double bv = s - a;
  const double e = (a - (s - bv)) + (b - bv);
  return DD{s, e};
}

// s + e = a + b exactly, for |a| >= |b|.
__device__ __forceinline__ DD dd_fast_two_sum(double a, double b) {
  const double s = a + b;
  return DD{s, b - (s - a)};
}

__device__ __forceinline__ DD dd_add(DD a, DD b) {
  DD s = dd_two_sum(a.hi, b.hi);
  const DD t = dd_two_sum(a.lo, b.lo);
  s.lo += t.hi;
  s = dd_fast_two_sum(s.hi, s.lo);
  s.lo += t.lo;
  return dd_fast_two_sum(s.hi, s.lo);
}

__device__ __forceinline__ DD dd_add_d(DD a, double b) {
  DD s = dd_two_sum(a.hi, b);
  s.lo += a.lo;
  return dd_fast_two_sum(s.hi, s.lo);
}

// The exact product of two doubles is p + fma(a, b, -p); the cross terms of the low
// parts are added to that error term.
__device__ __forceinline__ DD dd_mul(DD a, DD b) {
  const double p = a.hi * b.hi;
  double e = fma(a.hi, b.hi, -p);
  e = fma(a.hi, b.lo, e);
  e = fma(a.lo, b.hi, e);
  return dd_fast_two_sum(p, e);
}

__device__ __forceinline__ DD dd_neg(DD a) { return DD{-a.hi, -a.lo}; }

// a / b, b != 0: the fp64 quotient and two corrections from the remainder.
__device__ __forceinline__ DD dd_div(DD a, DD b) {
  const double q1 = a.hi / b.hi;
  DD r = dd_add(a, dd_neg(dd_mul(DD{q1, 0.0}, b)));
  const double q2 = r.hi / b.hi;
  r = dd_add(r, dd_neg(dd_mul(DD{q2, 0.0}, b)));
  const double q3 = r.hi / b.hi;
  return dd_add_d(dd_fast_two_sum(q1, q2), q3);
}

// sqrt(a), a.hi > 0: one Newton step from the fp64 root.
__device__ __forceinline__ DD dd_sqrt(DD a) {
  const double x = sqrt(a.hi);
  const DD r = dd_add(a, dd_neg(dd_mul(DD{x, 0.0}, DD{x, 0.0})));
  return dd_fast_two_sum(x, r.hi / (2.0 * x));
}

// 1 / sqrt(a), a.hi > 0: one Newton step for the reciprocal root from the fp64 value
// x, y = x + x (1 - a x^2) / 2 (the relative error squares: about 2^-104).
__device__ __forceinline__ DD dd_rsqrt(DD a) {
  const double x = 1.0 / sqrt(a.hi);
  const DD e = dd_add(DD{1.0, 0.0}, dd_neg(dd_mul(a, dd_mul(DD{x, 0.0}, DD{x, 0.0}))));
  return dd_add_d(DD{x, 0.0}, 0.5 * x * e.hi);
}

// Lanes that share one Gram entry when the orthogonalization sums the partials: the
// largest power of two with NG * GS <= 256 threads, at most a wavefront (1 = a thread
// per entry).
template <int R>
constexpr int orth_group_size() {
  int gs = 64;
  while (gs > 1 && gs * gram_size<R>() > kThreads) gs /= 2;
  return gs;
}

// Working set of the orthogonalization of one matrix (LDS).
template <int R>
struct OrthShared {
  double Gh[R][R + 1];  // Gram matrix, then its Cholesky factor (upper); high parts
  double Gl[R][R + 1];  // low parts (rows padded: lane j reads row j without conflicts)
  double D[R];          // diagonal of the Gram matrix before factoring
  double T[R][R];       // P <- P T
  double Y[R];          // the normalized column being removed
  double Cc[R];         // its coefficient vector
  double Sh[kThreads];  // row-sum partials of a Gram matrix recomputed from P (high)
  double Sl[kThreads];  // (low)
  int redo;             // the fp64 Gram matrix did not resolve a pivot
};

__device__ __forceinline__ void tri_entry(int e, int R, int& a, int& b) {
  int rem = e;
  a = 0;
  while (rem >= R - a) {
    rem -= R - a;
    ++a;
  }
  b = a + rem;
}

// Sums the job's fp64 Gram partials into sh.Gh (sh.Gl = 0); every thread of the
// workgroup takes part and it ends with a barrier. `issued` runs once the first loads
// of partials are in flight and before any is used, so a caller can queue loads of its
// own behind them. Small ranks: a group of GS lanes of one wavefront per Gram entry,
// lane i adding partials i, i + GS, ... (8 loads in flight), then a butterfly over the
// group. Larger ranks: a thread per entry, the partials in order.
template <int R, typename Issued>
__device__ __forceinline__ void orth_gram_sum(const OrthJob& j, const double* __restrict__ gram,
                                              OrthShared<R>& sh, Issued issued) {
  constexpr int NG = gram_size<R>();
  constexpr int GS = orth_group_size<R>();
  const int tid = threadIdx.x;
  auto store_entry = [&](int e, double v) {
    int a, b;
    tri_entry(e, R, a, b);
    sh.Gh[a][b] = v;
    sh.Gh[b][a] = v;
    sh.Gl[a][b] = 0.0;
    sh.Gl[b][a] = 0.0;
  };
  if constexpr (GS > 1) {
    const int e = min(tid / GS, NG - 1);  // threads past the last entry mirror it
    const int gi = tid - (tid / GS) * GS;
    auto load = [&](int p0, double (&v)[8]) {
#pragma unroll
      for (int b = 0; b < 8; ++b)
        v[b] = gram[j.goff + static_cast<int64_t>(min(p0 + b * GS, j.nparts - 1)) * NG + e];
    };
    auto add = [&](int p0, const double (&v)[8], double& s) {
#pragma unroll
      for (int b = 0; b < 8; ++b) s += (p0 + b * GS < j.nparts) ? v[b] : 0.0;
    };
    double v[8];
    load(gi, v);
    // keep the issue order: the caller's loads go behind these
    __builtin_amdgcn_sched_barrier(0);
    issued();
    __builtin_amdgcn_sched_barrier(0);
    double s = 0.0;
    add(gi, v, s);
    for (int p0 = gi + 8 * GS; p0 < j.nparts; p0 += 8 * GS) {
      load(p0, v);
      add(p0, v, s);
    }
#pragma unroll
    for (int mask = GS / 2; mask >= 1; mask >>= 1) s += __shfl_xor(s, mask);
    if (gi == 0 && tid / GS < NG) store_entry(e, s);
  } else {
    constexpr int PER = (NG + kThreads - 1) / kThreads;
    double s[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) s[i] = 0.0;
    issued();
    for (int p0 = 0; p0 < j.nparts; p0 += 8) {
      double v[PER][8];
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int e = min(tid + i * kThreads, NG - 1);
#pragma unroll
        for (int b = 0; b < 8; ++b)
          v[i][b] = gram[j.goff + static_cast<int64_t>(min(p0 + b, j.nparts - 1)) * NG + e];
      }
#pragma unroll
      for (int i = 0; i < PER; ++i)
#pragma unroll
        for (int b = 0; b < 8; ++b) s[i] += (p0 + b < j.nparts) ? v[i][b] : 0.0;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = tid + i * kThreads;
      if (e < NG) store_entry(e, s[i]);
    }
  }
  __syncthreads();
}

// Sums the job's double-double Gram partials (partial p: NG high parts, then NG low
// parts, at goff + 2 NG p) into sh.Gh / sh.Gl, a thread per entry, partials in order
// (several at a time for all the thread's entries at once; NTH threads).
// Every thread takes part; ends with a barrier.
template <int R, int NTH>
__device__ __forceinline__ void orth_gram_sum_dd(const OrthJob& j, const double* __restrict__ gram,
                                                 OrthShared<R>& sh) {
  constexpr int NG = gram_size<R>();
  constexpr int PER = (NG + NTH - 1) / NTH;  // entries per thread
  constexpr int B = PER == 1 ? 16 : 8;       // partials per entry in flight
  const int tid = threadIdx.x;
  DD s[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) s[i] = DD{0.0, 0.0};
  for (int p0 = 0; p0 < j.nparts; p0 += B) {
    // B partials of every entry the thread owns in flight, then added in order
    double vh[PER][B], vl[PER][B];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const double* src = gram + j.goff + min(tid + i * NTH, NG - 1);
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int64_t p = min(p0 + q, j.nparts - 1);
        vh[i][q] = src[p * 2 * NG];
        vl[i][q] = src[p * 2 * NG + NG];
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i)
#pragma unroll
      for (int q = 0; q < B; ++q)
        if (p0 + q < j.nparts) s[i] = dd_add(s[i], DD{vh[i][q], vl[i][q]});
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = tid + i * NTH;
    if (e < NG) {
      int a, b;
      tri_entry(e, R, a, b);
      sh.Gh[a][b] = s[i].hi;
      sh.Gh[b][a] = s[i].hi;
      sh.Gl[a][b] = s[i].lo;
      sh.Gl[b][a] = s[i].lo;
    }
  }
  __syncthreads();
}

// The Gram matrix of the `rows` x R block X (row stride R, binary32) in double-double,
// read directly: thread t sums entry t / S over the rows t % S, t % S + S, ... (S =
// threads per entry), then the S sums of an entry are added in order. Every thread of
// the workgroup takes part; ends with a barrier.
template <int R>
__device__ __forceinline__ void orth_gram_rows_dd(const float* __restrict__ X, int rows,
                                                  OrthShared<R>& sh) {
  constexpr int NG = gram_size<R>();
  constexpr int S = kThreads / NG;
  static_assert(S >= 1, "one thread per Gram entry at least");
  const int tid = threadIdx.x;
  const int e = tid / S;
  const int ph = tid - e * S;
  if (e < NG) {
    int a, b;
    tri_entry(e, R, a, b);
    DD s{0.0, 0.0};
    for (int row = ph; row < rows; row += S) {
      const float* x = X + static_cast<int64_t>(row) * R;
      s = dd_add_d(s, static_cast<double>(x[a]) * static_cast<double>(x[b]));  // exact
    }
    sh.Sh[tid] = s.hi;
    sh.Sl[tid] = s.lo;
  }
  __syncthreads();
  if (tid < NG) {
    DD s{0.0, 0.0};
    for (int i = 0; i < S; ++i) s = dd_add(s, DD{sh.Sh[tid * S + i], sh.Sl[tid * S + i]});
    int a, b;
    tri_entry(tid, R, a, b);
    sh.Gh[a][b] = s.hi;
    sh.Gh[b][a] = s.hi;
    sh.Gl[a][b] = s.lo;
    sh.Gl[b][a] = s.lo;
  }
  __syncthreads();
}

// Cholesky factor of the leading rank x rank block of G (sh.Gh + sh.Gl) in
// double-double, in place in the upper triangle, by wavefront 0 alone (its LDS
// accesses take effect in program order; wave barriers only keep the compiler from
// reordering). Lane j owns column j. A pivot that is not positive gives a zero row
// (the column adds no new direction: it is exactly dependent, or zero). With tau > 0,
// sh.redo is set when a pivot falls below tau times its diagonal entry (only for a
// column that is not zero). No workgroup barrier: callers synchronize.
template <int R>
__device__ __forceinline__ void orth_cholesky(int rank, double tau, OrthShared<R>& sh) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  if (lane < R) sh.D[lane] = sh.Gh[lane][lane];
  int redo = 0;
  __builtin_amdgcn_wave_barrier();
  for (int k = 0; k < rank; ++k) {
    const DD d{sh.Gh[k][k], sh.Gl[k][k]};
    const bool pos = d.hi > 0.0;
    if (tau > 0.0 && sh.D[k] > 0.0 && !(d.hi >= tau * sh.D[k])) redo = 1;
    const DD piv = pos ? dd_sqrt(d) : DD{0.0, 0.0};
    __builtin_amdgcn_wave_barrier();
    // row k of the factor: C_kj = G_kj / C_kk (lane j), C_kk (lane k)
    if (lane >= k && lane < rank) {
      DD c{0.0, 0.0};
      if (pos) c = lane == k ? piv : dd_div(DD{sh.Gh[k][lane], sh.Gl[k][lane]}, piv);
      sh.Gh[k][lane] = c.hi;
      sh.Gl[k][lane] = c.lo;
    }
    __builtin_amdgcn_wave_barrier();
    // trailing block: G_ij -= C_ki C_kj for k < i <= j (lane j updates column j)
    if (lane > k && lane < rank) {
      const DD ckj{sh.Gh[k][lane], sh.Gl[k][lane]};
      for (int i = k + 1; i <= lane; ++i) {
        const DD cki{sh.Gh[k][i], sh.Gl[k][i]};
        const DD g = dd_add(DD{sh.Gh[i][lane], sh.Gl[i][lane]}, dd_neg(dd_mul(cki, ckj)));
        sh.Gh[i][lane] = g.hi;
        sh.Gl[i][lane] = g.lo;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0 && tau > 0.0) sh.redo = redo;
}

// The factor of orth_cholesky without the pivot check (tau = 0), each column step
// spread over the whole workgroup: the lanes of wavefront 0 form row k (the row times
// the reciprocal root of the pivot, in double-double), then every thread updates
// entries of the trailing block (the same operations as orth_cholesky). Every thread
// takes part; ends with a barrier.
template <int R>
__device__ __forceinline__ void orth_cholesky_wg(int rank, OrthShared<R>& sh) {
  const int tid = threadIdx.x;
  for (int k = 0; k < rank; ++k) {
    if (tid >= k && tid < rank) {
      // C_kj = G_kj / sqrt(G_kk) as G_kj times the reciprocal root (C_kk = G_kk times it)
      const DD d{sh.Gh[k][k], sh.Gl[k][k]};
      DD c{0.0, 0.0};
      if (d.hi > 0.0) c = dd_mul(DD{sh.Gh[k][tid], sh.Gl[k][tid]}, dd_rsqrt(d));
      sh.Gh[k][tid] = c.hi;
      sh.Gl[k][tid] = c.lo;
    }
    __syncthreads();
    // G_ij -= C_ki C_kj for k < i <= j < rank
    const int w = rank - k - 1;
    for (int e = tid; e < w * w; e += blockDim.x) {
      const int i = k + 1 + e / w;
      const int jj = k + 1 + e % w;
      if (i <= jj) {
        const DD cki{sh.Gh[k][i], sh.Gl[k][i]};
        const DD ckj{sh.Gh[k][jj], sh.Gl[k][jj]};
        const DD g = dd_add(DD{sh.Gh[i][jj], sh.Gl[i][jj]}, dd_neg(dd_mul(cki, ckj)));
        sh.Gh[i][jj] = g.hi;
        sh.Gl[i][jj] = g.lo;
      }
    }
    __syncthreads();
  }
}

// Gram-Schmidt with epsilon on the columns of the factor (sh.Gh, upper triangle; the
// high parts, rounded to fp64), carrying coefficient vectors: column i is divided by
// (|column| + eps), then removed from every later column with the dot product, exactly
// the steps of the pages' recurrence. Writes the coefficients to sh.T (columns past
// the rank: the unit vector, so those P columns, kept at zero, stay zero). Run by
// wavefront 0, lane j owning column j; ends with a workgroup barrier.
template <int R>
__device__ __forceinline__ void orth_from_factor(int rank, double eps, OrthShared<R>& sh) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 64) {
    double y[R], c[R];
#pragma unroll
    for (int l = 0; l < R; ++l) {
      c[l] = (l == lane) ? 1.0 : 0.0;
      y[l] = (lane < rank && l <= lane) ? sh.Gh[l][min(lane, R - 1)] : 0.0;
    }
    for (int i = 0; i < rank; ++i) {
      if (lane == i) {
        double nn = 0.0;
#pragma unroll
        for (int l = 0; l < R; ++l) nn += y[l] * y[l];
        const double inv = 1.0 / (sqrt(nn) + eps);
#pragma unroll
        for (int l = 0; l < R; ++l) {
          y[l] *= inv;
          c[l] *= inv;
          sh.Y[l] = y[l];
          sh.Cc[l] = c[l];
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (lane > i && lane < rank) {
        double coef = 0.0;
#pragma unroll
        for (int l = 0; l < R; ++l) coef += y[l] * sh.Y[l];
#pragma unroll
        for (int l = 0; l < R; ++l) {
          y[l] -= coef * sh.Y[l];
          c[l] -= coef * sh.Cc[l];
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (lane < R) {
#pragma unroll
      for (int l = 0; l < R; ++l) sh.T[l][lane] = c[l];
    }
  }
  __syncthreads();
}

// The recurrence of orth_from_factor with a thread per element: thread t takes element
// l = t % R of column j = t / R (R * R threads at least). A column's norm and its dot
// products are shuffle-tree sums over its R lanes (one aligned group of a wavefront);
// the normalized column and its coefficients go through LDS, alternating between two
// buffers, so a step needs one barrier. Writes sh.T; ends with a barrier.
template <int R>
__device__ __forceinline__ void orth_from_factor_wg(int rank, double eps, OrthShared<R>& sh,
                                                    double (*ybuf)[2][R]) {
  const int tid = threadIdx.x;
  const int j = tid / R;
  const int l = tid - j * R;
  const bool mine = j < R;
  double y = 0.0, c = 0.0;
  if (mine) {
    c = (l == j) ? 1.0 : 0.0;
    y = (j < rank && l <= j) ? sh.Gh[l][j] : 0.0;
  }
  auto group_sum = [](double v) {
#pragma unroll
    for (int mask = R / 2; mask >= 1; mask >>= 1) v += __shfl_xor(v, mask);
    return v;
  };
  for (int i = 0; i < rank; ++i) {
    double(*buf)[R] = ybuf[i & 1];
    if (j == i) {
      const double inv = 1.0 / (sqrt(group_sum(y * y)) + eps);
      y *= inv;
      c *= inv;
      buf[0][l] = y;
      buf[1][l] = c;
    }
    __syncthreads();
    if (mine && j > i && j < rank) {
      const double yi = buf[0][l];
      const double coef = group_sum(y * yi);
      y -= coef * yi;
      c -= coef * buf[1][l];
    }
  }
  if (mine) sh.T[l][j] = c;
  __syncthreads();
}

// ----------------------------------------------------------------------- pass 2

// M' at element `off` of a matrix (fp32 state with error feedback: pass 1 wrote M' into
// E's place; without: the (unscaled) gradient; 16-bit state: M' from Mt, which is E's
// place with error feedback).
template <bool F16, bool EF, int LD, int ST = kStF32>
__device__ __forceinline__ void ld_mprime4(const void* bucket, const float* Et, int64_t boff,
                                           int64_t off, int valid, float inv_scale,
                                           float (&x)[4], const uint16_t* Mt = nullptr) {
  if constexpr (ST != kStF32) {
    ld_h4<ST, LD>(Mt + off, valid, x);  // a 16-bit state keeps M' of pass 1
    return;
  }
  if constexpr (stored_mprime<F16, EF, ST>()) {
    ld_f32x4<LD>(Et + off, valid, x);  // pass 1 left M' in E's place
    return;
  }
  bool rb;
  ld_grad4<F16, LD>(bucket, boff + off, valid, inv_scale, x, rb);
}

// Gram-Schmidt of P (step 3.4) for the rows of one pass-2 tile: the workgroup sums the
// Gram partials pass 1 left, runs the recurrence and applies P <- P T (fp64, rounded
// once) to its rows, which stay in LDS (sP, rows relative to r0). Tiles of column
// block 0 also store them as the orthogonalized P. Every workgroup of a matrix takes
// the same steps in the same order, so they all hold identical rows.
template <int R, int ST, typename Issued>
__device__ __forceinline__ void pass2_orth_rows(const Pass2Args& args, const TensorDesc& d,
                                                const Tile& t, int r0, int r1,
                                                OrthShared<R>& sh, float* sP, Issued issued) {
  constexpr int PT = kPass2StageFloats / R / kThreads;  // rows per thread
  static_assert(PT >= 1, "pass-2 row staging too small for this rank");
  const int tid = threadIdx.x;
  const float* __restrict__ Pt = args.P + d.poff;
  float praw[PT][R];  // loaded before the Gram partials are summed
#pragma unroll
  for (int i = 0; i < PT; ++i) load_p_row<R>(Pt, min(r0 + tid + i * kThreads, r1 - 1), praw[i]);
  __builtin_amdgcn_sched_barrier(0);
  const OrthJob j{d.poff, d.goff, -1, d.n, d.rank, (d.n + d.rpb1 - 1) / d.rpb1, d.rpb1, 0, 0};
  orth_gram_sum<R>(j, args.gram, sh, issued);
  orth_cholesky<R>(d.rank, kCholTau, sh);
  __syncthreads();
  if (sh.redo) {
    // an fp64 pivot was not resolved: the Gram matrix again, in double-double from P
    orth_gram_rows_dd<R>(Pt, d.n, sh);
    orth_cholesky<R>(d.rank, 0.0, sh);
    __syncthreads();
  }
  orth_from_factor<R>(d.rank, args.eps, sh);
#pragma unroll
  for (int i = 0; i < PT; ++i) {
    const int row = r0 + tid + i * kThreads;
    if (row < r1) {
      float pr[R];
#pragma unroll
      for (int k = 0; k < R; ++k) {
        double acc = 0.0;
#pragma unroll
        for (int l = 0; l < R; ++l) acc += static_cast<double>(praw[i][l]) * sh.T[l][k];
        pr[k] = rnd16<ST>(static_cast<float>(acc));
        sP[(row - r0) * R + k] = pr[k];
      }
      if (t.b == 0) store_p_row<R>(args.Pout + d.poff, row, pr);
    }
  }
  __syncthreads();
}

// Q = M'^T P over one tile (P rows from LDS); row slots and wavefronts are combined in
// a fixed order; with several row blocks each writes a partial slot (summed at the
// start of pass 3). Rows are clamped into the tile so all loads of an iteration are
// issued together; clamped duplicate rows are zeroed before they are accumulated. The
// first rows of M' are requested during the orthogonalization prologue, after its own
// loads (waits count loads in issue order) and before its barriers, which wait on
// LDS only, so their latency overlaps it.
template <int R, int U, bool F16, bool EF, int LD, bool WIDE, int ST>
__device__ __forceinline__ void pass2_body(const Pass2Args& args, const TensorDesc& d,
                                           const Tile& t, float* red, OrthShared<R>& sh,
                                           float* sP) {
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const LaneGeom L = tile_geom<WIDE>(d, t.b, lane);
  const int r0 = t.a * d.rpb;
  const int r1 = min(d.n, r0 + d.rpb);
  const int stride = 4 * L.rpw;
  const int rw0 = r0 + wave * L.rpw;
  // the step's M' (pass 1 wrote it to the place other than E's current one, which is
  // the same place with a single buffer)
  const float* __restrict__ Et =
      args.E + d.eoff + (args.wstride - w_cur(args.widx, args.wstride));
  // lanes past the last column load (and then ignore) an in-range group, so the first
  // loads need no branch and the wait counts stay exact: the row's last 4 elements
  // (m >= 4; valid = 4 keeps the unaligned access from shifting further back) or its
  // last element (m < 4)
  const int cc = L.col_ok ? L.c : (LD == kLdScalar ? d.m - 1 : d.m - 4);
  const int vv = L.col_ok ? L.valid : (LD == kLdScalar ? 1 : 4);
  float x[U][4];
  auto load_rows = [&](int rw) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rowc = min(rw + u * stride + L.slot, r1 - 1);
      ld_mprime4<F16, EF, LD, ST>(args.bucket, Et, d.boff,
                                   static_cast<int64_t>(rowc) * d.m + cc, vv, args.inv_scale,
                                   x[u], ST != kStF32 ? args.Mh + d.eoff : nullptr);
    }
  };
  // the first rows of M' queue behind the loads of P rows and Gram partials
  pass2_orth_rows<R, ST>(args, d, t, r0, r1, sh, sP, [&] { load_rows(rw0); });
  float acc[4][R];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int k = 0; k < R; ++k) acc[a][k] = 0.f;
  if (L.col_ok) {
    for (int rw = rw0; rw < r1; rw += stride * U) {
      if (rw != rw0) load_rows(rw);
      float p[U][R];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = rw + u * stride + L.slot;
        const bool ok = row < r1;
        const int rowc = min(row, r1 - 1);
#pragma unroll
        for (int k = 0; k < R; ++k) p[u][k] = ok ? sP[(rowc - r0) * R + k] : 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) x[u][a] = ok ? x[u][a] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
          for (int k = 0; k < R; ++k) acc[a][k] += x[u][a] * p[u][k];
    }
  }
  // sum over the row slots of the wavefront (lanes with the same column group)
  for (int mask = L.lpr; mask < 64; mask <<= 1) {
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int k = 0; k < R; ++k) acc[a][k] += __shfl_xor(acc[a][k], mask);
  }
  // combine the wavefronts in a fixed order: w0 + (w1 + (w2 + w3))
  const bool writer = L.slot == 0;
  float* mine = red + L.g * 4 * R;
  for (int w = 3; w >= 1; --w) {
    if (wave == w && writer) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int k = 0; k < R; ++k)
          mine[a * R + k] = (w == 3) ? acc[a][k] : acc[a][k] + mine[a * R + k];
    }
    __syncthreads();
  }
  float* Qt = args.Q + d.qoff;
  if (d.nrb == 1) {
    if (wave == 0 && writer && L.col_ok) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
        if (a < L.valid) {
#pragma unroll
          for (int k = 0; k < R; ++k)
            Qt[static_cast<int64_t>(L.c + a) * R + k] =
                (k < d.rank) ? rnd16<ST>(acc[a][k] + mine[a * R + k]) : 0.f;
        }
    }
    return;
  }
  if (wave == 0 && writer) {
    float* dst = args.partial +
                 static_cast<int64_t>(d.pslot + t.b * d.nrb + t.a) * (kColBlock * R) +
                 L.g * 4 * R;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int k = 0; k < R; ++k) dst[a * R + k] = acc[a][k] + mine[a * R + k];
  }
}

// WO: compiled with the wide aligned body only (the host launches it when every
// tensor of the table takes that body; a tile of any other tensor is left alone).
template <int R, int U, bool F16, bool EF, int ST, bool WO = false>
__global__ void __launch_bounds__(kThreads) k_pass2(Pass2Args args) {
  if (F16 && *args.found_inf) return;
  __shared__ float red[64 * 4 * R];
  __shared__ OrthShared<R> sh;
  __shared__ float sP[kPass2StageFloats];
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if constexpr (WO) {
    if (d.vec && d.lpr == 64)
      pass2_body<R, U, F16, EF, kLdAligned, true, ST>(args, d, t, red, sh, sP);
  } else if (d.vec && d.lpr == 64)
    pass2_body<R, U, F16, EF, kLdAligned, true, ST>(args, d, t, red, sh, sP);
  else if (d.vec)
    pass2_body<R, U, F16, EF, kLdAligned, false, ST>(args, d, t, red, sh, sP);
  else if (d.m >= 4)
    pass2_body<R, U, F16, EF, kLdUnaligned, false, ST>(args, d, t, red, sh, sP);
  else
    pass2_body<R, U, F16, EF, kLdScalar, false, ST>(args, d, t, red, sh, sP);
}

// Q of the tensors with several row blocks: the partial slots of a column block summed
// in a fixed order. A slot is 64R float4; the workgroup's threads split the float4 of
// a slot and, when there are more threads than float4, the row blocks (subset s takes
// row blocks s, s + NS, ...), so one round of loads covers many row blocks. The
// subsets are then added in subset order through LDS.
template <int R, int ST>
__global__ void __launch_bounds__(kReduceThreads) k_pass2_reduce(Pass2ReduceArgs args) {
  if (args.found_inf != nullptr && *args.found_inf) return;
  constexpr int F4 = kColBlock * R / 4;
  constexpr int W = F4 < kReduceThreads ? F4 : kReduceThreads;  // threads per subset
  constexpr int PER = F4 / W;                                     // float4 per thread
  constexpr int NS = kReduceThreads / W;                          // row-block subsets
  constexpr int B = NS >= 8 ? 4 : 8;                              // loads in flight
  __shared__ float4 part[NS > 1 ? NS - 1 : 1][NS > 1 ? W : 1];
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  const int tid = threadIdx.x;
  const int sub = tid / W;
  const int j0 = tid - sub * W;
  const float4* src = reinterpret_cast<const float4*>(
      args.partial + static_cast<int64_t>(d.pslot + t.b * d.nrb) * (kColBlock * R));
  float4 s[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) s[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int rb0 = sub; rb0 < d.nrb; rb0 += NS * B) {
    float4 v[B][PER];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int rb = min(rb0 + b * NS, d.nrb - 1);
#pragma unroll
      for (int i = 0; i < PER; ++i) v[b][i] = src[static_cast<int64_t>(rb) * F4 + j0 + i * W];
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const bool ok = rb0 + b * NS < d.nrb;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        s[i].x += ok ? v[b][i].x : 0.f;
        s[i].y += ok ? v[b][i].y : 0.f;
        s[i].z += ok ? v[b][i].z : 0.f;
        s[i].w += ok ? v[b][i].w : 0.f;
      }
    }
  }
  if constexpr (NS > 1) {
    if (sub > 0) part[sub - 1][j0] = s[0];
    __syncthreads();
    if (sub != 0) return;
#pragma unroll 1
    for (int q = 0; q < NS - 1; ++q) {
      const float4 w = part[q][j0];
      s[0].x += w.x;
      s[0].y += w.y;
      s[0].z += w.z;
      s[0].w += w.w;
    }
  }
  float* Qt = args.Q + d.qoff;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const float vals[4] = {s[i].x, s[i].y, s[i].z, s[i].w};
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int f = 4 * (j0 + i * W) + a;  // float index inside the slot: column * R + k
      const int col = t.b * kColBlock + f / R;
      const int k = f % R;
      if (col < d.m) {
        const float q = (k < d.rank) ? rnd16<ST>(vals[a]) : 0.f;
        Qt[static_cast<int64_t>(col) * R + k] = q;
        if (args.QT != nullptr) args.QT[d.qtoff + static_cast<int64_t>(k) * d.mstride + col] = q;
      }
    }
  }
}

// ----------------------------------------------------------------------- pass 3

__device__ void f16_unscale_range(const FlatTile ft, void* bucket, float inv_scale) {
  uint16_t* h = static_cast<uint16_t*>(bucket) + ft.start;
  for (int64_t i = threadIdx.x; i < ft.len; i += blockDim.x)
    h[i] = __half_as_ushort(__float2half_rn(half_bits_to_float(h[i]) * inv_scale));
}

// The wrapper's cast to 16 bits and back, in place over an fp32 range.
template <int ST>
__device__ void round_range(const FlatTile ft, void* bucket) {
  float* x = static_cast<float*>(bucket) + ft.start;
  for (int64_t i = threadIdx.x; i < ft.len; i += blockDim.x) x[i] = rnd16<ST>(x[i]);
}

// Q for the lane's 4 columns when pass 2 split the matrix into several row blocks
// (vector ranks): the partial slots of the column block are summed here instead of in
// a kernel of their own. Wavefront w adds slots w, w + 4, ... in order; the four
// sums are added in wavefront order through LDS (qred: 4 x 4R x 64 floats), so
// every workgroup of the column block gets the same Q. Row block 0 stores it as the
// warm-start Q.
template <int R, int ST>
__device__ __forceinline__ void pass3_q_from_partials(const Pass3Args& args, const TensorDesc& d,
                                                      const Tile& t, const LaneGeom& L,
                                                      int lane, int wave, float* qred,
                                                      float (&q)[4][R]) {
  constexpr int F = 4 * R;  // floats per lane: 4 columns x R
  constexpr int NB = 4;     // slots in flight per lane
  const float* base = args.partial + static_cast<int64_t>(d.pslot + t.b * d.nrb) * (kColBlock * R) +
                      L.g * F;
  float s[F];
#pragma unroll
  for (int f = 0; f < F; ++f) s[f] = 0.f;
  for (int rb0 = wave; rb0 < d.nrb; rb0 += 4 * NB) {
    float v[NB][F];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const float4* src = reinterpret_cast<const float4*>(
          base + static_cast<int64_t>(min(rb0 + 4 * b, d.nrb - 1)) * (kColBlock * R));
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const float4 w = src[i];
        v[b][4 * i + 0] = w.x;
        v[b][4 * i + 1] = w.y;
        v[b][4 * i + 2] = w.z;
        v[b][4 * i + 3] = w.w;
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const bool ok = rb0 + 4 * b < d.nrb;
#pragma unroll
      for (int f = 0; f < F; ++f) s[f] += ok ? v[b][f] : 0.f;
    }
  }
#pragma unroll
  for (int f = 0; f < F; ++f) qred[(wave * F + f) * 64 + lane] = s[f];
  __syncthreads();
#pragma unroll
  for (int f = 0; f < F; ++f) {
    float v = qred[f * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v += qred[(w * F + f) * 64 + lane];
    q[f / R][f % R] = rnd16<ST>(v);
  }
  if (t.a == 0 && wave == 0 && L.slot == 0 && L.col_ok) {
    float* Qt = args.Q + d.qoff;
#pragma unroll
    for (int a = 0; a < 4; ++a)
      if (a < L.valid) {
#pragma unroll
        for (int k = 0; k < R; ++k)
          Qt[static_cast<int64_t>(L.c + a) * R + k] = (k < d.rank) ? q[a][k] : 0.f;
      }
  }
}

// M_hat = P Q^T into the bucket over one tile. All loads of an iteration come from rows
// clamped into the tile; stores are kept to real rows. With error feedback the error is
// not written (the next pass 1 rebuilds it from M' and the factors); MAT (the error
// materialization) writes E = M' - M_hat to Eout (or E's place) instead of M_hat to the
// bucket, with the same M_hat.
template <int R, int U, bool F16, bool EF, int LD, bool WIDE, int ST, bool MAT = false>
__device__ __forceinline__ void pass3_body(const Pass3Args& args, const TensorDesc& d,
                                           const Tile& t, float* qred) {
  // M' is read only to materialize the error (E's place holds it with error feedback)
  constexpr bool LOADX = EF && MAT;
  const bool we = MAT && holds_error(args);  // materialization: E's place holds E
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const LaneGeom L = tile_geom<WIDE>(d, t.b, lane);
  float q[4][R];
  if (d.nrb > 1 && !MAT) {
    pass3_q_from_partials<R, ST>(args, d, t, L, lane, wave, qred, q);
  } else {
    load_q_rows<R>(args.Q + d.qoff, L.c, d.m, q);
  }
  if (!L.col_ok) return;
  const int r0 = t.a * d.rpb3;
  const int r1 = min(d.n, r0 + d.rpb3);
  const int stride = 4 * L.rpw;
  const float* __restrict__ Pt = args.P + d.poff;
  const int64_t wc = MAT ? w_cur(args.widx, args.wstride) : 0;
  const float* __restrict__ Et = args.E + d.eoff + wc;  // M' (materialization)
  for (int rw = r0 + wave * L.rpw; rw < r1; rw += stride * U) {
    float x[U][4];
    float p[U][R];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int rowc = min(rw + u * stride + L.slot, r1 - 1);
      if constexpr (LOADX)
        ld_mprime4<F16, EF, LD, ST>(args.bucket, Et, d.boff,
                                     static_cast<int64_t>(rowc) * d.m + L.c, L.valid,
                                     args.inv_scale, x[u],
                                     ST != kStF32 ? args.Mh + d.eoff : nullptr);
      if constexpr (WIDE)
        load_p_row_uniform<R>(Pt, __builtin_amdgcn_readfirstlane(rowc), p[u]);
      else
        load_p_row<R>(Pt, rowc, p[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = rw + u * stride + L.slot;
      if (row >= r1) continue;
      const int64_t off = static_cast<int64_t>(row) * d.m + L.c;
      float mh[4];
      mhat4<R>(p[u], q, mh);
#pragma unroll
      for (int a = 0; a < 4; ++a) mh[a] = rnd16<ST>(mh[a]);
      if constexpr (MAT) {
        float e[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) e[a] = we ? x[u][a] : rebuilt_error<ST>(x[u][a], mh[a]);
        store_materialized<ST, LD>(args, wc, d.eoff + off, L.valid, e);
        continue;
      }
      if constexpr (F16)
        st_f16x4<LD>(static_cast<uint16_t*>(args.bucket) + d.boff + off, L.valid, mh);
      else
        st_f32x4<LD>(static_cast<float*>(args.bucket) + d.boff + off, L.valid, mh);
    }
  }
}

template <int R, int U, bool F16, bool EF, int ST, bool MAT = false>
__global__ void __launch_bounds__(kThreads) k_pass3(Pass3Args args) {
  if (F16 && *args.found_inf) return;
  mark_mprime<F16, EF, ST, MAT>(args);
  __shared__ float qred[4 * 4 * R * 64];
  if constexpr (MAT) {
    if (static_cast<int>(blockIdx.x) >= args.ntiles) return;
    const Tile t = args.tiles[blockIdx.x];
    const TensorDesc d = args.td[t.tensor];
    if (d.vec && d.lpr == 64)
      pass3_body<R, U, F16, EF, kLdAligned, true, ST, true>(args, d, t, qred);
    else if (d.vec)
      pass3_body<R, U, F16, EF, kLdAligned, false, ST, true>(args, d, t, qred);
    else if (d.m >= 4)
      pass3_body<R, U, F16, EF, kLdUnaligned, false, ST, true>(args, d, t, qred);
    else
      pass3_body<R, U, F16, EF, kLdScalar, false, ST, true>(args, d, t, qred);
    return;
  }
  if (static_cast<int>(blockIdx.x) >= args.ntiles) {
    if constexpr (F16)
      f16_unscale_range(args.ftiles[blockIdx.x - args.ntiles], args.bucket, args.inv_scale);
    else if constexpr (ST != kStF32)
      round_range<ST>(args.ftiles[blockIdx.x - args.ntiles], args.bucket);
    return;
  }
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if (d.vec && d.lpr == 64)
    pass3_body<R, U, F16, EF, kLdAligned, true, ST>(args, d, t, qred);
  else if (d.vec)
    pass3_body<R, U, F16, EF, kLdAligned, false, ST>(args, d, t, qred);
  else if (d.m >= 4)
    pass3_body<R, U, F16, EF, kLdUnaligned, false, ST>(args, d, t, qred);
  else
    pass3_body<R, U, F16, EF, kLdScalar, false, ST>(args, d, t, qred);
}

// ------------------------------------------------- matrix-core passes (R = 16, 32)
//
// For ranks 16 and 32 each element of M' meets R multiply-adds in every pass, so the
// three passes run on v_mfma_f32_16x16x4f32 (lane l supplies A[l%16][l/16] and
// B[l/16][l%16]; D register v of lane l is D[4*(l/16)+v][l%16]). A lane's 16-byte
// load of 4 consecutive columns feeds 4 MFMA K-steps (or 4 output rows) directly.

typedef float mfma_f4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ mfma_f4 mfma16(float a, float b, mfma_f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// The 16-bit matrix cores (v_mfma_f32_16x16x16 f16, or bf16_1k) for values that are
// exact in the state's 16 bits: lane l supplies A[l%16][4(l/16)..4(l/16)+3] and
// B[4(l/16)..4(l/16)+3][l%16], four 16-bit values in two registers (the first in the
// low half); D as above. The products are exact, so the result differs from four
// v_mfma_f32_16x16x4f32 steps over the same values only in the fp32 accumulation.
typedef short mfma_s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 mfma_h16x4 __attribute__((ext_vector_type(4)));

template <int ST>
__device__ __forceinline__ mfma_f4 mfma16x16x16(uint2 a, uint2 b, mfma_f4 c) {
  if constexpr (ST == kStBF16)
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(mfma_s16x4, a),
                                                     __builtin_bit_cast(mfma_s16x4, b), c, 0, 0,
                                                     0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mfma_h16x4, a),
                                                 __builtin_bit_cast(mfma_h16x4, b), c, 0, 0, 0);
}

// A 16 x 16 block of M_hat^T = Q P^T from the KQ ranks each lane holds of a Q row (qa)
// and a P row (pb), lane group h holding ranks h KQ .. h KQ + KQ - 1. An fp32 state
// takes KQ fp32 MFMA steps (written out where it is used); a 16-bit state (P and Q
// exact in 16 bits) the KQ / 4 16-bit steps over the groups of four of those ranks
// here. Pass 3 and the error rebuild of pass 1 take the same steps, so their values
// agree bit for bit.
template <int ST, int KQ>
__device__ __forceinline__ mfma_f4 mhat_block16(const float (&qa)[KQ], const float (&pb)[KQ]) {
  static_assert(ST != kStF32 && KQ % 4 == 0, "a 16-bit state, whole groups of four ranks");
  mfma_f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KQ / 4; ++j) {
    const uint2 a = make_uint2(pack_h16x2<ST>(qa[4 * j], qa[4 * j + 1]),
                               pack_h16x2<ST>(qa[4 * j + 2], qa[4 * j + 3]));
    const uint2 b = make_uint2(pack_h16x2<ST>(pb[4 * j], pb[4 * j + 1]),
                               pack_h16x2<ST>(pb[4 * j + 2], pb[4 * j + 3]));
    acc = mfma16x16x16<ST>(a, b, acc);
  }
  return acc;
}

// Pass 1, P = M' Q, for rows that are not 16-byte aligned (or a bucket that is not): the
// 16-row group grp of the work item's rows, over its column group. Wavefront w takes
// the 64-column chunks w, w + 4, w + 8, ... of the group (U = 4 K-steps of 16 columns
// each), so in every round the workgroup reads a contiguous 1 KB of each of its rows; lane group h loads columns
// 4h..4h+3 of a K-step (one 16-byte load per four MFMA K-steps) and the matching 16
// bytes of Q^T rows 16nt + cl. The wavefronts' partial P are added in wavefront
// order through LDS at the end (red: 4 x NT x 4 x 64 floats). VEC: rows are 16-byte
// aligned, so all loads of a chunk are issued from clamped addresses before any is
// used, and invalid lanes are masked after.
template <int R, bool F16, bool EF, bool VEC, int ST>
__device__ __forceinline__ void pass1_mfma_body(const Pass1Args& args, const TensorDesc& d,
                                                const Tile& t, int grp, int lane, int wave,
                                                float* red) {
  constexpr int NT = R / 16;
  constexpr int U = 4;
  const int m = d.m;
  const int r0 = t.a * d.rpb1 + 16 * grp;  // the work item's row group grp
  const int r1 = min(min(d.n, t.a * d.rpb1 + d.rpb1), r0 + 16);
  const int h = lane >> 4;
  const int cl = lane & 15;
  // the work item's column group: columns c0 .. c1 - 1 (its P is a partial sum)
  const int c0 = t.b * kPass1Cols;
  const int c1 = min(m, c0 + kPass1Cols);
  const int row = r0 + cl;
  const bool row_ok = row < r1;
  const int rowc = min(row, r1 - 1);
  // M'_prev (or the error) from E's current place, M' to the other one
  const int64_t wc = w_cur(args.widx, args.wstride);
  float* __restrict__ Ebase = args.E + d.eoff;  // both places derive from it (they may be one)
  const float* Ein = Ebase + wc;
  float* Eout = Ebase + (args.wstride - wc);
  const float* __restrict__ QTt = args.QT + d.qtoff;
  constexpr bool SM = stored_mprime<F16, EF, ST>();
  constexpr int KQ = R / 4;
  // E's place holds M'_prev: E = M'_prev - Pe Q^T, with pass 3's matrix-core steps (lane
  // (h, cl) holds columns 4h..4h+3 of a 16-column group of row cl, which is this body's
  // element layout)
  const bool rebuild = SM && rebuild_error(args);
  float pe[KQ];
  if constexpr (SM) {
    if (rebuild) {
#pragma unroll
      for (int k4 = 0; k4 < KQ / 4; ++k4) {
        float w[4];
        load_f4(args.Pe + d.poff + static_cast<int64_t>(rowc) * R + h * KQ + 4 * k4, w);
#pragma unroll
        for (int a = 0; a < 4; ++a) pe[4 * k4 + a] = w[a];
      }
    }
  }
  mfma_f4 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  int bad = 0;
  for (int k0 = c0 + 64 * wave; k0 < c1; k0 += 256) {
    float x[U][4];
    float e[U][4];
    float b[U][NT][4];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = k0 + 16 * u + 4 * h;
      ok[u] = row_ok && col < m;
      if constexpr (VEC) {
        const int colc = min(col, m - 4);
        const int64_t off = static_cast<int64_t>(rowc) * m + colc;
        bool rb;
        load_grad4_vec<F16>(args.bucket, d.boff + off, args.inv_scale, x[u], rb);
        if (ok[u] && rb) bad = 1;
        if constexpr (EF && ST != kStF32)
          ld_h4<ST, kLdAligned>(args.Eh + d.eoff + off, 4, e[u]);
        else if constexpr (EF)
          load_f4(Ein + off, e[u]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          load_f4(QTt + static_cast<int64_t>(16 * nt + cl) * d.mstride + colc, b[u][nt]);
      } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          x[u][a] = 0.f;
          e[u][a] = 0.f;
        }
        if (ok[u]) {
          const int64_t off = static_cast<int64_t>(row) * m + col;
          load_grad4<F16>(args.bucket, d.boff + off, false, m - col, args.inv_scale, x[u], bad);
          if constexpr (EF && ST != kStF32)
            ld_h4<ST, kLdScalar>(args.Eh + d.eoff + off, m - col, e[u]);
          else if constexpr (EF)
            load_f32x4(Ein + off, false, m - col, e[u]);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int a = 0; a < 4; ++a)
            b[u][nt][a] = (col + a < m) ? QTt[static_cast<int64_t>(16 * nt + cl) * d.mstride + col + a]
                                        : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int col = k0 + 16 * u + 4 * h;
      if constexpr (VEC) {
        if (col >= m) {  // clamped duplicate columns: contribute nothing
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int a = 0; a < 4; ++a) b[u][nt][a] = 0.f;
        }
      }
      if constexpr (SM) {
        if (rebuild) {
          const int qcol = min(k0 + 16 * u + cl, m - 1);
          float qa[KQ];
#pragma unroll
          for (int k4 = 0; k4 < KQ / 4; ++k4) {
            float w[4];
            load_f4(args.Q + d.qoff + static_cast<int64_t>(qcol) * R + h * KQ + 4 * k4, w);
#pragma unroll
            for (int a = 0; a < 4; ++a) qa[4 * k4 + a] = w[a];
          }
          mfma_f4 mh = {0.f, 0.f, 0.f, 0.f};
          if constexpr (ST != kStF32) {
            mh = mhat_block16<ST, KQ>(qa, pe);
          } else {
#pragma unroll
            for (int kq = 0; kq < KQ; ++kq) mh = mfma16(qa[kq], pe[kq], mh);
          }
#pragma unroll
          for (int a = 0; a < 4; ++a) e[u][a] = rebuilt_error<ST>(e[u][a], mh[a]);
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float v = x[u][a];
        if constexpr (ST != kStF32) {
          v = rnd16<ST>(v);  // the wrapper's cast; M' = G + E formed in 16 bits
          if constexpr (EF) v = rnd16<ST>(v + e[u][a]);
        } else if constexpr (EF) {
          v += e[u][a];
        }
        x[u][a] = ok[u] ? v : 0.f;
      }
      if constexpr (ST != kStF32) {
        if (ok[u]) {
          if constexpr (VEC)
            st_h4<ST, kLdAligned>(args.Mh + d.eoff + static_cast<int64_t>(row) * m + col, 4, x[u]);
          else
            st_h4<ST, kLdScalar>(args.Mh + d.eoff + static_cast<int64_t>(row) * m + col, m - col,
                                 x[u]);
        }
      } else if constexpr (SM) {
        if (ok[u]) store_f32x4(Eout + static_cast<int64_t>(row) * m + col, VEC, m - col, x[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ST != kStF32) {
        // a 16-bit state's M' and Q are exact in 16 bits: one K = 16 step
        const uint2 a = make_uint2(pack_h16x2<ST>(x[u][0], x[u][1]), pack_h16x2<ST>(x[u][2], x[u][3]));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const uint2 bb = make_uint2(pack_h16x2<ST>(b[u][nt][0], b[u][nt][1]),
                                      pack_h16x2<ST>(b[u][nt][2], b[u][nt][3]));
          acc[nt] = mfma16x16x16<ST>(a, bb, acc[nt]);
        }
      } else {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma16(x[u][s4], b[u][nt][s4], acc[nt]);
      }
    }
  }
  if constexpr (F16) {
    if (__any(bad) && lane == 0) atomicOr(args.found_inf, 1);
  }
  // partial P of every wavefront to LDS; wavefront 0 adds them in order
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int v = 0; v < 4; ++v) red[((wave * NT + nt) * 4 + v) * 64 + lane] = acc[nt][v];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float sum = red[(nt * 4 + v) * 64 + lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) sum += red[((w * NT + nt) * 4 + v) * 64 + lane];
        const int prow = r0 + 4 * h + v;
        const int k = 16 * nt + cl;
        if (prow < r1)
          args.Ppart[d.p1off + (static_cast<int64_t>(t.b) * d.n + prow) * R + k] = (k < d.rank) ? sum : 0.f;
      }
    }
  }
}

// Pass 1 on matrix cores with row-contiguous memory traffic (rows 16-byte aligned): the
// workgroup's MT groups of 16 rows are processed in 256-column chunks. Row phase:
// wavefront w loads rows 4MT w .. 4MT w + 4MT - 1 of the chunk (lane l: columns
// 4l..4l+3, 1 KB of a row per load), forms M' (with error feedback: stored back the
// same way) and writes it to an LDS tile. MFMA phase: wavefront w takes the chunk's
// columns 64w..64w+63 (four K-steps of 16) of every row group, with the matching 16
// bytes of Q^T rows 16nt + cl per K-step, loaded once for all MT groups; a 16-bit
// state's K-step of 16 is one 16-bit MFMA (its M' and Q are exact in 16 bits) instead
// of four fp32 ones. The next chunk's rows are requested before the MFMA phase of this
// one.
constexpr int kPass1TileStride = kColBlock + 4;  // LDS row stride (floats), padded
constexpr int kPass1Groups = kMfmaPass1Rows / 16;

template <int R, bool F16, bool EF, int ST>
__device__ __forceinline__ void pass1_mfma_rows(const Pass1Args& args, const TensorDesc& d,
                                                const Tile& t, int lane, int wave, float* red,
                                                float* tile, float* mh_tile, float* qx_tile) {
  constexpr int NT = R / 16;
  constexpr int MT = kPass1Groups;
  constexpr int RW = 4 * MT;  // rows per wavefront in the row phase
  constexpr int LS = kPass1TileStride;
  const int m = d.m;
  const int r0 = t.a * d.rpb1;
  const int r1 = min(d.n, r0 + d.rpb1);
  const int h = lane >> 4;
  const int cl = lane & 15;
  // the work item's column group: columns c0 .. c1 - 1 (its P is a partial sum)
  const int c0 = t.b * kPass1Cols;
  const int c1 = min(m, c0 + kPass1Cols);
  // M'_prev (or the error) from E's current place, M' to the other one
  const int64_t wc = w_cur(args.widx, args.wstride);
  float* __restrict__ Ebase = args.E + d.eoff;  // both places derive from it (they may be one)
  const float* Ein = Ebase + wc;
  float* Eout = Ebase + (args.wstride - wc);
  const float* __restrict__ QTt = args.QT + d.qtoff;
  constexpr bool SM = stored_mprime<F16, EF, ST>();
  constexpr int KQ = R / 4;
  // Q^T fragments of a chunk: lane (h, cl) holds rows 16nt + cl, columns 16u + 4h..4h+3
  // of wavefront w's 64 columns; loaded one chunk ahead
  auto load_b = [&](int k0, float (&bq)[4][NT][4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int colc = min(k0 + 64 * wave + 16 * u + 4 * h, m - 4);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        load_f4(QTt + static_cast<int64_t>(16 * nt + cl) * d.mstride + colc, bq[u][nt]);
    }
  };
  // E's place holds M'_prev: E = M'_prev - Pe Q^T. A chunk's M_hat_prev is formed with
  // pass 3's matrix-core steps (wavefront w: the chunk's columns 64w..64w+63, lane (h,
  // cl) columns 4h..4h+3 of each 16-column group of row cl of a row group) into the LDS
  // tile mh_tile, one chunk ahead, between the barriers that already separate the
  // phases; the row phase reads its rows back from there. The Q operand (lane (h, cl):
  // column cl of the group, ranks h R/4 .. h R/4 + R/4 - 1) is the chunk's Q^T
  // fragments transposed through the wavefront's own LDS region qx (16 columns x QS
  // floats), the same values pass 3 read as Q.
  constexpr int QS = R + 4;
  float* qx = qx_tile + wave * 16 * QS;
  const bool rebuild = SM && rebuild_error(args);
  float pe[MT][KQ];
  auto rebuild_chunk = [&](const float (&bq)[4][NT][4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) qx[(4 * h + s4) * QS + 16 * nt + cl] = bq[g][nt][s4];
      // the wavefront's LDS accesses take effect in program order; the fences keep
      // the compiler from moving them across
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float qa[KQ];
#pragma unroll
      for (int k4 = 0; k4 < KQ / 4; ++k4) {
        const float4 w = *reinterpret_cast<const float4*>(qx + cl * QS + h * KQ + 4 * k4);
        qa[4 * k4 + 0] = w.x;
        qa[4 * k4 + 1] = w.y;
        qa[4 * k4 + 2] = w.z;
        qa[4 * k4 + 3] = w.w;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        mfma_f4 mh = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ST != kStF32) {
          mh = mhat_block16<ST, KQ>(qa, pe[mt]);
        } else {
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) mh = mfma16(qa[kq], pe[mt][kq], mh);
        }
        *reinterpret_cast<float4*>(mh_tile + (16 * mt + cl) * LS + 64 * wave + 16 * g + 4 * h) =
            make_float4(mh[0], mh[1], mh[2], mh[3]);
      }
    }
  };
  float b[4][NT][4];
  load_b(c0, b);
  if constexpr (SM) {
    if (rebuild) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int prow = min(r0 + 16 * mt + cl, r1 - 1);
#pragma unroll
        for (int k4 = 0; k4 < KQ / 4; ++k4) {
          float w[4];
          load_f4(args.Pe + d.poff + static_cast<int64_t>(prow) * R + h * KQ + 4 * k4, w);
#pragma unroll
          for (int a = 0; a < 4; ++a) pe[mt][4 * k4 + a] = w[a];
        }
      }
      rebuild_chunk(b);
      __syncthreads();
    }
  }
  mfma_f4 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  int bad = 0;
  // row phase geometry: rows RW w .. RW w + RW - 1 of the work item, columns 4l..4l+3
  // of the chunk
  int64_t rbase[RW];
  bool rok[RW];
#pragma unroll
  for (int i = 0; i < RW; ++i) {
    const int row = r0 + RW * wave + i;
    rok[i] = row < r1;
    rbase[i] = static_cast<int64_t>(min(row, r1 - 1)) * m;
  }
  float xg[RW][4], xe[RW][4];
  auto load_rows = [&](int k0) {
    const int colc = min(k0 + 4 * lane, m - 4);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      bool rb;
      load_grad4_vec<F16>(args.bucket, d.boff + rbase[i] + colc, args.inv_scale, xg[i], rb);
      if (rok[i] && k0 + 4 * lane < m && rb) bad = 1;
      if constexpr (EF && ST != kStF32)
        ld_h4<ST, kLdAligned>(args.Eh + d.eoff + rbase[i] + colc, 4, xe[i]);
      else if constexpr (EF)
        load_f4(Ein + rbase[i] + colc, xe[i]);
    }
  };
  load_rows(c0);
  for (int k0 = c0; k0 < c1; k0 += kColBlock) {
    const int col = k0 + 4 * lane;
    const bool cok = col < m;
    if constexpr (SM) {
      if (rebuild) {
        // the wavefront's rows of M_hat_prev, all requested before the first is used
        float4 mh[RW];
#pragma unroll
        for (int i = 0; i < RW; ++i)
          mh[i] = *reinterpret_cast<const float4*>(mh_tile + (RW * wave + i) * LS + 4 * lane);
#pragma unroll
        for (int i = 0; i < RW; ++i) {
          xe[i][0] = rebuilt_error<ST>(xe[i][0], mh[i].x);
          xe[i][1] = rebuilt_error<ST>(xe[i][1], mh[i].y);
          xe[i][2] = rebuilt_error<ST>(xe[i][2], mh[i].z);
          xe[i][3] = rebuilt_error<ST>(xe[i][3], mh[i].w);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      float v[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float x = xg[i][a];
        if constexpr (ST != kStF32) {
          x = rnd16<ST>(x);
          if constexpr (EF) x = rnd16<ST>(x + xe[i][a]);
        } else if constexpr (EF) {
          x += xe[i][a];
        }
        v[a] = (rok[i] && cok) ? x : 0.f;
      }
      if constexpr (ST != kStF32) {
        if (rok[i] && cok) st_h4<ST, kLdAligned>(args.Mh + d.eoff + rbase[i] + col, 4, v);
      } else if constexpr (SM) {
        if (rok[i] && cok) store_f32x4(Eout + rbase[i] + col, true, 4, v);  // M' in E's place
      }
      *reinterpret_cast<float4*>(tile + (RW * wave + i) * LS + 4 * lane) =
          make_float4(v[0], v[1], v[2], v[3]);
    }
    if (k0 + kColBlock < c1) load_rows(k0 + kColBlock);
    // the next chunk's Q^T fragments (clamped in bounds after the last chunk)
    float bn[4][NT][4];
    load_b(k0 + kColBlock, bn);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kc = 64 * wave + 16 * u + 4 * h;  // column inside the chunk
      if (k0 + kc >= m) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int a = 0; a < 4; ++a) b[u][nt][a] = 0.f;
      }
      if constexpr (ST != kStF32) {
        // a 16-bit state's M' and Q are exact in 16 bits: one K = 16 step per block
        uint2 bb[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bb[nt] = make_uint2(pack_h16x2<ST>(b[u][nt][0], b[u][nt][1]),
                              pack_h16x2<ST>(b[u][nt][2], b[u][nt][3]));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float4 av = *reinterpret_cast<const float4*>(tile + (16 * mt + cl) * LS + kc);
          const uint2 a = make_uint2(pack_h16x2<ST>(av.x, av.y), pack_h16x2<ST>(av.z, av.w));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = mfma16x16x16<ST>(a, bb[nt], acc[mt][nt]);
        }
      } else {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const float4 av = *reinterpret_cast<const float4*>(tile + (16 * mt + cl) * LS + kc);
          const float a4[4] = {av.x, av.y, av.z, av.w};
#pragma unroll
          for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              acc[mt][nt] = mfma16(a4[s4], b[u][nt][s4], acc[mt][nt]);
        }
      }
    }
    if constexpr (SM) {
      // the next chunk's M_hat_prev: this chunk's row phase read mh_tile before the
      // barrier above
      if (rebuild && k0 + kColBlock < c1) rebuild_chunk(bn);
    }
    __syncthreads();  // the tiles are rewritten by the next chunk
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int a = 0; a < 4; ++a) b[u][nt][a] = bn[u][nt][a];
  }
  if constexpr (F16) {
    if (__any(bad) && lane == 0) atomicOr(args.found_inf, 1);
  }
  // partial P of every wavefront to LDS; the (row group, column group) pairs are split
  // over the wavefronts, each adding the four partials in wavefront order
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[(((wave * MT + mt) * NT + nt) * 4 + v) * 64 + lane] = acc[mt][nt][v];
  __syncthreads();
  for (int pr = wave; pr < MT * NT; pr += 4) {
    const int mt = pr / NT;
    const int nt = pr - mt * NT;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float sum = red[((mt * NT + nt) * 4 + v) * 64 + lane];
#pragma unroll
      for (int w = 1; w < 4; ++w) sum += red[(((w * MT + mt) * NT + nt) * 4 + v) * 64 + lane];
      const int prow = r0 + 16 * mt + 4 * h + v;
      const int k = 16 * nt + cl;
      if (prow < r1)
        args.Ppart[d.p1off + (static_cast<int64_t>(t.b) * d.n + prow) * R + k] = (k < d.rank) ? sum : 0.f;
    }
  }
}

template <int R, bool F16, bool EF, int ST>
__global__ void __launch_bounds__(kThreads) k_pass1_mfma(Pass1Args args) {
  static_assert(kMfmaPass1Rows % 16 == 0, "a workgroup owns whole 16-row MFMA groups");
  // the wavefronts' partial P (4 x MT x NT x 4 x 64 floats) go through the M' tile once
  // the last chunk's barrier has freed it
  static_assert(4 * kPass1Groups * (R / 16) * 4 * 64 <= kMfmaPass1Rows * kPass1TileStride,
                "partial P fits the tile");
  __shared__ float tile[kMfmaPass1Rows * kPass1TileStride];
  __shared__ float mh_tile[stored_mprime<F16, EF, ST>() ? kMfmaPass1Rows * kPass1TileStride : 1];
  __shared__ float qx_tile[stored_mprime<F16, EF, ST>() ? 4 * 16 * (R + 4) : 1];
  float* red = tile;
  const int lane = threadIdx.x & 63;
  if constexpr (F16 && stored_mprime<F16, EF, ST>()) {
    // a step already known to be skipped (the bucket's check ran before this pass, or,
    // with two E places, another workgroup of it found inf) needs none of its results
    if (*args.found_inf) return;
  }
  if (static_cast<int>(blockIdx.x) >= args.ntiles) {
    if constexpr (F16)
      f16_check_range(args.ftiles[blockIdx.x - args.ntiles], args.bucket, args.found_inf);
    return;
  }
  const int wave = wave_index();
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if (d.vec) {
    pass1_mfma_rows<R, F16, EF, ST>(args, d, t, lane, wave, red, tile, mh_tile, qx_tile);
  } else {
    // one row group after the other (the partial-P area is reused)
    for (int grp = 0; grp < kPass1Groups && t.a * d.rpb1 + 16 * grp < d.n; ++grp) {
      if (grp) __syncthreads();
      pass1_mfma_body<R, F16, EF, false, ST>(args, d, t, grp, lane, wave, red);
    }
  }
}

// Pass 2, Q = M'^T P: a wavefront owns 64 columns of the tile; lane group h takes row
// 4 * step + h, lane cl the columns 4cl..4cl+3, so accumulator s holds the output
// columns c0 + 4i + s (i = MFMA output row).
template <int R, bool F16, bool EF, bool VEC, int ST>
__device__ __forceinline__ void pass2_mfma_body(const Pass2Args& args, const TensorDesc& d,
                                                const Tile& t, int lane, int wave) {
  constexpr int NT = R / 16;
  constexpr int U = 4;
  const int m = d.m;
  const int r0 = t.a * d.rpb;
  const int r1 = min(d.n, r0 + d.rpb);
  const int h = lane >> 4;
  const int cl = lane & 15;
  const int c0 = t.b * kColBlock + 64 * wave;
  if (c0 >= m) return;
  const int col = c0 + 4 * cl;
  const bool col_ok = col < m;
  const int colc = VEC ? min(col, m - 4) : col;
  const float* __restrict__ Pt = args.P + d.poff;
  // the step's M' (the place pass 1 wrote)
  const float* __restrict__ Et =
      args.E + d.eoff + (args.wstride - w_cur(args.widx, args.wstride));
  mfma_f4 acc[4][NT];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[s4][nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  // the operands of the 4U-row step at rr (the next step's are requested before this
  // step's MFMAs)
  auto load_step = [&](int rr, float (&x)[U][4], float (&p)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = rr + 4 * u + h;
      const int rowc = min(row, r1 - 1);
      if constexpr (VEC && ST != kStF32) {
        ld_h4<ST, kLdAligned>(args.Mh + d.eoff + static_cast<int64_t>(rowc) * m + colc, 4, x[u]);
      } else if constexpr (VEC) {
        const int64_t off = static_cast<int64_t>(rowc) * m + colc;
        if constexpr (stored_mprime<F16, EF, ST>()) {
          load_f4(Et + off, x[u]);  // pass 1 left M' in E's place
        } else {
          bool rb;
          load_grad4_vec<F16>(args.bucket, d.boff + off, args.inv_scale, x[u], rb);
        }
      } else {
        if (row < r1 && col_ok) {
          ld_mprime4<F16, EF, kLdScalar, ST>(args.bucket, Et, d.boff,
                                             static_cast<int64_t>(row) * m + col, m - col,
                                             args.inv_scale, x[u],
                                             ST != kStF32 ? args.Mh + d.eoff : nullptr);
        } else {
#pragma unroll
          for (int a = 0; a < 4; ++a) x[u][a] = 0.f;
        }
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p[u][nt] = Pt[static_cast<int64_t>(rowc) * R + 16 * nt + cl];
    }
  };
  auto compute_step = [&](int rr, float (&x)[U][4], float (&p)[U][NT]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool rok = rr + 4 * u + h < r1;
#pragma unroll
      for (int a = 0; a < 4; ++a) x[u][a] = (rok && col_ok) ? x[u][a] : 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) p[u][nt] = rok ? p[u][nt] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[s4][nt] = mfma16(x[u][s4], p[u][nt], acc[s4][nt]);
  };
  if constexpr (ST == kStF32) {
    // two register sets in turn: a step's MFMAs run while the next step's loads are in
    // flight. On the 16-byte path the loads need no branch (clamped rows) and the
    // scheduling barriers keep the compiler from moving them next to their use.
    // Steps go in pairs; a pair's second step past the last row is masked to zero (its
    // loads are clamped), so the loop has no exit between the two halves.
    float xa[U][4], xb[U][4];
    float pa[U][NT], pb[U][NT];
    load_step(r0, xa, pa);
    for (int rr = r0; rr < r1; rr += 8 * U) {
      if (VEC || rr + 4 * U < r1) load_step(rr + 4 * U, xb, pb);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(rr, xa, pa);
      if (VEC || rr + 8 * U < r1) load_step(rr + 8 * U, xa, pa);
      __builtin_amdgcn_sched_barrier(0);
      compute_step(rr + 4 * U, xb, pb);
    }
  } else {
    // a 16-bit state's rows without 16-byte alignment: one register set, so the kernel
    // that also holds the 16-bit body keeps its occupancy
    for (int rr = r0; rr < r1; rr += 4 * U) {
      float x[U][4];
      float p[U][NT];
      load_step(rr, x, p);
      compute_step(rr, x, p);
    }
  }
  float* Qt = args.Q + d.qoff;
  float* part = args.partial + static_cast<int64_t>(d.pslot + t.b * d.nrb + t.a) * (kColBlock * R);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int qcol = c0 + 16 * h + 4 * v + s4;  // output row i = 4h + v -> column c0 + 4i + s
        const int k = 16 * nt + cl;
        if (qcol < m) {
          const float val = acc[s4][nt][v];
          if (d.nrb == 1) {
            const float q = (k < d.rank) ? rnd16<ST>(val) : 0.f;
            Qt[static_cast<int64_t>(qcol) * R + k] = q;
            args.QT[d.qtoff + static_cast<int64_t>(k) * d.mstride + qcol] = q;
          } else {
            part[(qcol - t.b * kColBlock) * R + k] = val;
          }
        }
      }
    }
  }
}

// Pass 2 for a 16-bit state on the 16-bit matrix cores (mfma16x16x16): M' and P hold
// 16-bit values, so their products are exact and the result differs from the fp32
// matrix cores only in the fp32 accumulation order, at a quarter of the instructions.
// Lane (h, cl) loads rows 4h..4h+3 of each 16-row step at columns c0 + 4cl..4cl+3 (four
// 8-byte loads): column s of that 4 x 4 block is the A operand of MFMA s (output
// columns c0 + 4i + s, as in pass2_mfma_body), and B holds the same four rows of P's
// column 16nt + cl.

template <int R, int ST>
__device__ __forceinline__ void pass2_mfma16_rows(const Pass2Args& args, const TensorDesc& d,
                                                  const Tile& t, int lane, int wave) {
  constexpr int NT = R / 16;
  constexpr int U2 = 2;  // 16-row steps loaded before use
  const int m = d.m;
  const int r0 = t.a * d.rpb;
  const int r1 = min(d.n, r0 + d.rpb);
  const int h = lane >> 4;
  const int cl = lane & 15;
  const int c0 = t.b * kColBlock + 64 * wave;
  if (c0 >= m) return;
  const int col = c0 + 4 * cl;
  const bool col_ok = col < m;
  const int colc = min(col, m - 4);
  const float* __restrict__ Pt = args.P + d.poff;
  const uint16_t* __restrict__ Mt = args.Mh + d.eoff;
  mfma_f4 acc[4][NT];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[s4][nt] = mfma_f4{0.f, 0.f, 0.f, 0.f};
  for (int rr = r0; rr < r1; rr += 16 * U2) {
    uint2 xm[U2][4];
    float pv[U2][4][NT];
#pragma unroll
    for (int u = 0; u < U2; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rowc = min(rr + 16 * u + 4 * h + j, r1 - 1);
        xm[u][j] = *reinterpret_cast<const uint2*>(Mt + static_cast<int64_t>(rowc) * m + colc);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          pv[u][j][nt] = Pt[static_cast<int64_t>(rowc) * R + 16 * nt + cl];
      }
#pragma unroll
    for (int u = 0; u < U2; ++u) {
      float pz[4][NT];  // P values (16-bit exact: P is rounded where it is formed)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool rok = rr + 16 * u + 4 * h + j < r1;
        if (!(rok && col_ok)) xm[u][j] = make_uint2(0u, 0u);  // +0 in both formats
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) pz[j][nt] = rok ? pv[u][j][nt] : 0.f;
      }
      uint2 b[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        b[nt] = make_uint2(pack_h16x2<ST>(pz[0][nt], pz[1][nt]), pack_h16x2<ST>(pz[2][nt], pz[3][nt]));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        // column s4 of the 4 x 4 block: element s4 of each row's four 16-bit values
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = (s4 < 2) ? xm[u][j].x : xm[u][j].y;
          e[j] = (s4 & 1) ? (w >> 16) : (w & 0xFFFFu);
        }
        const uint2 a = make_uint2(e[0] | (e[1] << 16), e[2] | (e[3] << 16));
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[s4][nt] = mfma16x16x16<ST>(a, b[nt], acc[s4][nt]);
      }
    }
  }
  float* Qt = args.Q + d.qoff;
  float* part = args.partial + static_cast<int64_t>(d.pslot + t.b * d.nrb + t.a) * (kColBlock * R);
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int qcol = c0 + 16 * h + 4 * v + s4;
        const int k = 16 * nt + cl;
        if (qcol < m) {
          const float val = acc[s4][nt][v];
          if (d.nrb == 1) {
            const float q = (k < d.rank) ? rnd16<ST>(val) : 0.f;
            Qt[static_cast<int64_t>(qcol) * R + k] = q;
            args.QT[d.qtoff + static_cast<int64_t>(k) * d.mstride + qcol] = q;
          } else {
            part[(qcol - t.b * kColBlock) * R + k] = val;
          }
        }
      }
    }
  }
}

template <int R, bool F16, bool EF, int ST>
__global__ void __launch_bounds__(kThreads) k_pass2_mfma(Pass2Args args) {
  if (F16 && *args.found_inf) return;
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if constexpr (ST != kStF32) {
    if (d.vec) {
      pass2_mfma16_rows<R, ST>(args, d, t, lane, wave);
      return;
    }
  } else {
    if (d.vec) {
      pass2_mfma_body<R, F16, EF, true, ST>(args, d, t, lane, wave);
      return;
    }
  }
  pass2_mfma_body<R, F16, EF, false, ST>(args, d, t, lane, wave);
}

// Pass 3, M_hat = P Q^T (or, materializing, E = M' - M_hat), computed as (Q P^T)^T so
// that lane l holds 4 consecutive columns (4h..4h+3) of row cl of each 16 x 16 output
// block.
// MFMA K-step kq of lane group h uses rank index h * KQ + kq, so A and B fragments are
// KQ consecutive floats of a Q row and of a P row.
template <int R, bool F16, bool EF, bool VEC, int ST, bool MAT = false>
__device__ __forceinline__ void pass3_mfma_body(const Pass3Args& args, const TensorDesc& d,
                                                const Tile& t, int lane, int wave) {
  // M' is read only to materialize the error (E's place holds it with error feedback)
  constexpr bool LOADX = EF && MAT;
  const bool we = MAT && holds_error(args);  // materialization: E's place holds E
  constexpr int KQ = R / 4;
  constexpr int UR = 2;  // 16-row steps loaded before use
  const int m = d.m;
  const int r0 = t.a * d.rpb3;
  const int r1 = min(d.n, r0 + d.rpb3);
  const int h = lane >> 4;
  const int cl = lane & 15;
  const int c0 = t.b * kColBlock + 64 * wave;
  if (c0 >= m) return;
  const float* __restrict__ Pt = args.P + d.poff;
  const float* __restrict__ Qt = args.Q + d.qoff;
  const int64_t wc = MAT ? w_cur(args.widx, args.wstride) : 0;
  const float* __restrict__ Et = args.E + d.eoff + wc;  // M' (materialization)
  float qa[4][KQ];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int qcol = min(c0 + 16 * g + cl, m - 1);
#pragma unroll
    for (int k4 = 0; k4 < KQ / 4; ++k4) {
      float w[4];
      load_f4(Qt + static_cast<int64_t>(qcol) * R + h * KQ + 4 * k4, w);
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[g][4 * k4 + a] = w[a];
    }
  }
  for (int rr = r0; rr < r1; rr += 16 * UR) {
    float pb[UR][KQ];
    float x[UR][4][4];
#pragma unroll
    for (int ur = 0; ur < UR; ++ur) {
      const int row = rr + 16 * ur + cl;
      const int rowc = min(row, r1 - 1);
#pragma unroll
      for (int k4 = 0; k4 < KQ / 4; ++k4) {
        float w[4];
        load_f4(Pt + static_cast<int64_t>(rowc) * R + h * KQ + 4 * k4, w);
#pragma unroll
        for (int a = 0; a < 4; ++a) pb[ur][4 * k4 + a] = w[a];
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = c0 + 16 * g + 4 * h;
        if constexpr (!LOADX) {
          // M' is not needed
        } else if constexpr (VEC && ST != kStF32) {
          ld_h4<ST, kLdAligned>(args.Mh + d.eoff + static_cast<int64_t>(rowc) * m +
                                    min(col, m - 4), 4, x[ur][g]);
        } else if constexpr (VEC) {
          load_f4(Et + static_cast<int64_t>(rowc) * m + min(col, m - 4), x[ur][g]);
        } else {
          if (row < r1 && col < m)
            ld_mprime4<F16, EF, kLdScalar, ST>(args.bucket, Et, d.boff,
                                               static_cast<int64_t>(row) * m + col, m - col,
                                               args.inv_scale, x[ur][g],
                                               ST != kStF32 ? args.Mh + d.eoff : nullptr);
        }
      }
    }
#pragma unroll
    for (int ur = 0; ur < UR; ++ur) {
      const int row = rr + 16 * ur + cl;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        mfma_f4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ST != kStF32) {
          acc = mhat_block16<ST, KQ>(qa[g], pb[ur]);
        } else {
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) acc = mfma16(qa[g][kq], pb[ur][kq], acc);
        }
        const int col = c0 + 16 * g + 4 * h;
        if (row < r1 && col < m) {
          const int64_t off = static_cast<int64_t>(row) * m + col;
          float mh[4] = {rnd16<ST>(acc[0]), rnd16<ST>(acc[1]), rnd16<ST>(acc[2]),
                         rnd16<ST>(acc[3])};
          if constexpr (MAT) {
            float e[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
              e[a] = we ? x[ur][g][a] : rebuilt_error<ST>(x[ur][g][a], mh[a]);
            store_materialized<ST, VEC ? kLdAligned : kLdScalar>(args, wc, d.eoff + off, m - col,
                                                                 e);
            continue;
          }
          if constexpr (F16)
            store_f16x4(static_cast<uint16_t*>(args.bucket) + d.boff + off, VEC, m - col, mh);
          else
            store_f32x4(static_cast<float*>(args.bucket) + d.boff + off, VEC, m - col, mh);
        }
      }
    }
  }
}

// Pass 3 on matrix cores with row-contiguous memory traffic (rows 16-byte aligned):
// each 32-row step the wavefronts compute their 16 x 16 blocks of M_hat = (Q P^T)^T as
// above (wavefront w: columns 64w..64w+63 of the 256-column block) into an LDS tile of
// 32 rows x 256 columns; after a barrier wavefront w takes rows 8w..8w+7 of the tile,
// lane l columns 4l..4l+3, so the M_hat stores (and, materializing the error, the M'
// loads and E stores) cover 1 KB of one row per instruction instead of 64 bytes of 16
// rows. The step's M' rows are requested before its MFMAs.
constexpr int kPass3TileStride = kColBlock + 4;  // LDS row stride (floats), padded

template <int R, bool F16, bool EF, int ST, bool MAT = false>
__device__ __forceinline__ void pass3_mfma_rows(const Pass3Args& args, const TensorDesc& d,
                                                const Tile& t, int lane, int wave,
                                                float* tile) {
  // M' is read only to materialize the error (E's place holds it with error feedback)
  constexpr bool LOADX = EF && MAT;
  const bool we = MAT && holds_error(args);  // materialization: E's place holds E
  constexpr int KQ = R / 4;
  constexpr int UR = 2;         // 16-row MFMA groups per step
  constexpr int SR = 16 * UR;   // rows per step
  constexpr int RW = SR / 4;    // rows per wavefront in the row phase
  constexpr int LS = kPass3TileStride;
  const int m = d.m;
  const int r0 = t.a * d.rpb3;
  const int r1 = min(d.n, r0 + d.rpb3);
  const int h = lane >> 4;
  const int cl = lane & 15;
  const int cw = t.b * kColBlock + 64 * wave;  // MFMA phase: this wavefront's columns
  const int cr = t.b * kColBlock + 4 * lane;   // row phase: this lane's 4 columns
  const bool cr_ok = cr < m;
  const int crc = min(cr, m - 4);
  const float* __restrict__ Pt = args.P + d.poff;
  const float* __restrict__ Qt = args.Q + d.qoff;
  const int64_t wc = MAT ? w_cur(args.widx, args.wstride) : 0;
  const float* __restrict__ Et = args.E + d.eoff + wc;  // M' (materialization)
  float qa[4][KQ];
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int qcol = min(cw + 16 * g + cl, m - 1);
#pragma unroll
    for (int k4 = 0; k4 < KQ / 4; ++k4) {
      float w[4];
      load_f4(Qt + static_cast<int64_t>(qcol) * R + h * KQ + 4 * k4, w);
#pragma unroll
      for (int a = 0; a < 4; ++a) qa[g][4 * k4 + a] = w[a];
    }
  }
  // P rows of the step at rr (the next step's are requested before this step's MFMAs)
  auto load_pb = [&](int rr, float (&pb)[UR][KQ]) {
#pragma unroll
    for (int ur = 0; ur < UR; ++ur) {
      const int rowc = min(rr + 16 * ur + cl, r1 - 1);
#pragma unroll
      for (int k4 = 0; k4 < KQ / 4; ++k4) {
        float w[4];
        load_f4(Pt + static_cast<int64_t>(rowc) * R + h * KQ + 4 * k4, w);
#pragma unroll
        for (int a = 0; a < 4; ++a) pb[ur][4 * k4 + a] = w[a];
      }
    }
  };
  float pb[UR][KQ];
  load_pb(r0, pb);
  for (int rr = r0; rr < r1; rr += SR) {
    float x[RW][4];
    if constexpr (LOADX) {
#pragma unroll
      for (int i = 0; i < RW; ++i) {
        const int row = min(rr + RW * wave + i, r1 - 1);
        ld_mprime4<F16, EF, kLdAligned, ST>(args.bucket, Et, d.boff,
                                            static_cast<int64_t>(row) * m + crc, 4,
                                            args.inv_scale, x[i],
                                            ST != kStF32 ? args.Mh + d.eoff : nullptr);
      }
    }
    float pbn[UR][KQ];
    if (rr + SR < r1) load_pb(rr + SR, pbn);
#pragma unroll
    for (int ur = 0; ur < UR; ++ur) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        mfma_f4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ST != kStF32) {
          acc = mhat_block16<ST, KQ>(qa[g], pb[ur]);
        } else {
#pragma unroll
          for (int kq = 0; kq < KQ; ++kq) acc = mfma16(qa[g][kq], pb[ur][kq], acc);
        }
        *reinterpret_cast<float4*>(tile + (16 * ur + cl) * LS + 64 * wave + 16 * g + 4 * h) =
            make_float4(acc[0], acc[1], acc[2], acc[3]);
      }
    }
    __syncthreads();
    // the wavefront's rows of the tile, all requested before the first is stored
    float4 tv[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i)
      tv[i] = *reinterpret_cast<const float4*>(tile + (RW * wave + i) * LS + 4 * lane);
#pragma unroll
    for (int i = 0; i < RW; ++i) {
      const int row = rr + RW * wave + i;
      if (row < r1 && cr_ok) {
        const float4 v = tv[i];
        const float mh[4] = {rnd16<ST>(v.x), rnd16<ST>(v.y), rnd16<ST>(v.z), rnd16<ST>(v.w)};
        const int64_t off = static_cast<int64_t>(row) * m + cr;
        if constexpr (MAT) {
          float e[4];
#pragma unroll
          for (int a = 0; a < 4; ++a) e[a] = we ? x[i][a] : rebuilt_error<ST>(x[i][a], mh[a]);
          store_materialized<ST, kLdAligned>(args, wc, d.eoff + off, 4, e);
          continue;
        }
        if constexpr (F16)
          store_f16x4(static_cast<uint16_t*>(args.bucket) + d.boff + off, true, 4, mh);
        else
          store_f32x4(static_cast<float*>(args.bucket) + d.boff + off, true, 4, mh);
      }
    }
    __syncthreads();  // the tile is rewritten by the next step
#pragma unroll
    for (int ur = 0; ur < UR; ++ur)
#pragma unroll
      for (int kq = 0; kq < KQ; ++kq) pb[ur][kq] = pbn[ur][kq];
  }
}

template <int R, bool F16, bool EF, int ST, bool MAT = false>
__global__ void __launch_bounds__(kThreads) k_pass3_mfma(Pass3Args args) {
  if (F16 && *args.found_inf) return;
  mark_mprime<F16, EF, ST, MAT>(args);
  if (static_cast<int>(blockIdx.x) >= args.ntiles) {
    if constexpr (MAT)
      return;
    else if constexpr (F16)
      f16_unscale_range(args.ftiles[blockIdx.x - args.ntiles], args.bucket, args.inv_scale);
    else if constexpr (ST != kStF32)
      round_range<ST>(args.ftiles[blockIdx.x - args.ntiles], args.bucket);
    return;
  }
  __shared__ float tile[32 * kPass3TileStride];
  const int lane = threadIdx.x & 63;
  const int wave = wave_index();
  const Tile t = args.tiles[blockIdx.x];
  const TensorDesc d = args.td[t.tensor];
  if (d.vec)
    pass3_mfma_rows<R, F16, EF, ST, MAT>(args, d, t, lane, wave, tile);
  else
    pass3_mfma_body<R, F16, EF, false, ST, MAT>(args, d, t, lane, wave);
}

// ------------------------------------------------------------ orthogonalization

// Gram partials of one row chunk of a job, staged through LDS, as double-double sums
// of the exact products: partial p holds NG high parts, then NG low parts. A job whose
// rows are pass 1's column-group partials sums them first (in group order, rounded to
// the state's precision) and writes the result as its rows.
// Matrix-core ranks: a thread owns a 4 x 4 block of entries (column groups ga <= gb)
// and one of S row phases (rows ph, ph + S, ...), adding each exact product to a
// binary64 sum with TwoSum and the rounding errors to a second sum (Ogita, Rump and
// Oishi, "Accurate sum and dot product", algorithm Sum2); the S sums of an entry are
// then added in phase order through LDS, eight entries of every block at a time.
// Vector ranks: a thread per entry, rows in order.
template <int R>
constexpr int gram_blocks() {
  return (R / 4) * (R / 4 + 1) / 2;
}
template <int R>
constexpr int gram_lds_floats() {
  if constexpr (R >= kMfmaMinRank) {
    constexpr int comb = gram_blocks<R>() * (kThreads / gram_blocks<R>()) * 8 * 2 * 2;
    return comb > kGramRows * R ? comb : kGramRows * R;
  } else {
    return kGramRows * R;
  }
}

__device__ __forceinline__ void gram_block_of(int blk, int nb, int& ga, int& gb) {
  int rem = blk;
  ga = 0;
  while (rem >= nb - ga) {
    rem -= nb - ga;
    ++ga;
  }
  gb = ga + rem;
}

template <int R, int ST>
__global__ void __launch_bounds__(kThreads)
    k_gram(const Tile* __restrict__ tiles, const OrthJob* __restrict__ jobs,
           float* __restrict__ base, const float* __restrict__ part,
           double* __restrict__ gram, const int32_t* __restrict__ found_inf) {
  if (found_inf != nullptr && *found_inf) return;
  constexpr int NG = gram_size<R>();
  __shared__ __align__(16) float xs[gram_lds_floats<R>()];
  const Tile t = tiles[blockIdx.x];
  const OrthJob j = jobs[t.tensor];
  const int r0 = t.a * j.rpp;
  const int nr = min(j.rpp, j.rows - r0);
  float* X = base + j.off + static_cast<int64_t>(r0) * R;
  double* out = gram + j.goff + static_cast<int64_t>(t.a) * 2 * NG;
  const int tid = threadIdx.x;
  if constexpr (R >= kMfmaMinRank) {
    constexpr int NB = R / 4;
    constexpr int NBLK = gram_blocks<R>();
    constexpr int S = kThreads / NBLK;
    static_assert(S >= 1, "a row phase per block at least");
    // rows are 16-byte aligned (R and the job offsets are multiples of 4)
    if (j.ncg > 0) {
      // P = the sum of the pass-1 partials, group after group, rounded once
      const float* src = part + j.part + static_cast<int64_t>(r0) * R;
      const int64_t gstride = static_cast<int64_t>(j.rows) * R;
      for (int f = tid; f < nr * R / 4; f += kThreads) {
        float4 v = *reinterpret_cast<const float4*>(src + 4 * f);
        for (int g0 = 1; g0 < j.ncg; g0 += 8) {
          float4 w[8];  // eight groups' partials in flight, then added in group order
#pragma unroll
          for (int i = 0; i < 8; ++i)
            w[i] = *reinterpret_cast<const float4*>(src + min(g0 + i, j.ncg - 1) * gstride + 4 * f);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            if (g0 + i < j.ncg) {
              v.x += w[i].x;
              v.y += w[i].y;
              v.z += w[i].z;
              v.w += w[i].w;
            }
          }
        }
        v = make_float4(rnd16<ST>(v.x), rnd16<ST>(v.y), rnd16<ST>(v.z), rnd16<ST>(v.w));
        *reinterpret_cast<float4*>(X + 4 * f) = v;
        *reinterpret_cast<float4*>(xs + 4 * f) = v;
      }
    } else {
      for (int f = tid; f < nr * R / 4; f += kThreads)
        *reinterpret_cast<float4*>(xs + 4 * f) = *reinterpret_cast<const float4*>(X + 4 * f);
    }
    __syncthreads();
    const int blk = tid / S;
    const int ph = tid - blk * S;
    int ga = 0, gb = 0;
    if (blk < NBLK) gram_block_of(blk, NB, ga, gb);
    double sh[16], sc[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) sh[q] = sc[q] = 0.0;
    if (blk < NBLK) {
      for (int r = ph; r < nr; r += S) {
        const float4 va = *reinterpret_cast<const float4*>(xs + r * R + 4 * ga);
        const float4 vb = *reinterpret_cast<const float4*>(xs + r * R + 4 * gb);
        const double a[4] = {va.x, va.y, va.z, va.w};
        const double b[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const DD u = dd_two_sum(sh[4 * i + q], a[i] * b[q]);  // the product is exact
            sh[4 * i + q] = u.hi;
            sc[4 * i + q] += u.lo;
          }
      }
    }
    __syncthreads();  // the staged rows are no longer needed: their LDS takes the sums
    double* red = reinterpret_cast<double*>(xs);
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {
      if (blk < NBLK) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const DD v = dd_two_sum(sh[8 * half + q], sc[8 * half + q]);
          red[((blk * 8 + q) * S + ph) * 2] = v.hi;
          red[((blk * 8 + q) * S + ph) * 2 + 1] = v.lo;
        }
      }
      __syncthreads();
      for (int idx = tid; idx < NBLK * 8; idx += kThreads) {
        const int b2 = idx / 8;
        const int k = 8 * half + (idx - b2 * 8);
        int ga2, gb2;
        gram_block_of(b2, NB, ga2, gb2);
        const int a = 4 * ga2 + k / 4;
        const int b = 4 * gb2 + k % 4;
        if (a <= b) {
          DD sum{red[idx * S * 2], red[idx * S * 2 + 1]};
          for (int p = 1; p < S; ++p)
            sum = dd_add(sum, DD{red[(idx * S + p) * 2], red[(idx * S + p) * 2 + 1]});
          const int e = a * R - a * (a - 1) / 2 + (b - a);  // upper-triangle index
          out[e] = sum.hi;
          out[NG + e] = sum.lo;
        }
      }
      __syncthreads();
    }
  } else {
    for (int f = tid; f < nr * R; f += kThreads) xs[f] = X[f];
    __syncthreads();
    for (int e = tid; e < NG; e += kThreads) {
      int a, b;
      tri_entry(e, R, a, b);
      DD s{0.0, 0.0};
      for (int r = 0; r < nr; ++r)
        s = dd_add_d(s, static_cast<double>(xs[r * R + a]) * static_cast<double>(xs[r * R + b]));
      out[e] = s.hi;
      out[NG + e] = s.lo;
    }
  }
}

// The transform T of one job (one workgroup of kOrthThreads per job): its
// double-double Gram partials summed, factored, and the recurrence run on the factor.
// T goes to tmat (R x R fp64 per job, job after job).
template <int R>
__global__ void __launch_bounds__(kOrthThreads)
    k_orth_t(const OrthJob* __restrict__ jobs, const double* __restrict__ gram,
             double* __restrict__ tmat, double eps, const int32_t* __restrict__ found_inf) {
  static_assert(kOrthThreads >= R * R, "a thread per element of the factor");
  if (found_inf != nullptr && *found_inf) return;
  __shared__ OrthShared<R> sh;
  __shared__ double ybuf[2][2][R];
  const OrthJob j = jobs[blockIdx.x];
  orth_gram_sum_dd<R, kOrthThreads>(j, gram, sh);
  orth_cholesky_wg<R>(j.rank, sh);
  orth_from_factor_wg<R>(j.rank, eps, sh, ybuf);
  double* dst = tmat + static_cast<int64_t>(blockIdx.x) * R * R;
  for (int f = threadIdx.x; f < R * R; f += kOrthThreads) dst[f] = sh.T[f / R][f % R];
}

// X <- X T in fp64, rounded to fp32 (and to the state's 16 bits), for orth_rows(R) rows
// of a job per workgroup; with toff >= 0 the result is also written transposed. Each
// output is one fp64 chain over l = 0..R-1; matrix-core ranks: a row per thread, four
// outputs at a time; vector ranks: four rows per thread loaded before any is
// transformed.
template <int R, int ST>
__global__ void __launch_bounds__(kThreads)
    k_orth(const OrthJob* __restrict__ jobs, float* __restrict__ base, float* __restrict__ tbase,
           const double* __restrict__ tmat, const int32_t* __restrict__ found_inf) {
  if (found_inf != nullptr && *found_inf) return;
  __shared__ double T[R][R];
  const OrthJob j = jobs[blockIdx.y];
  const int tid = threadIdx.x;
  const int row_begin = blockIdx.x * orth_rows(R);
  if (row_begin >= j.rows) return;
  const double* src = tmat + static_cast<int64_t>(blockIdx.y) * R * R;
  for (int f = tid; f < R * R; f += kThreads) T[f / R][f % R] = src[f];
  __syncthreads();
  float* X = base + j.off;
  const int row_end = min(j.rows, row_begin + orth_rows(R));
  if constexpr (R >= kMfmaMinRank) {
    const int row = row_begin + tid;
    if (row >= row_end) return;
    float x[R];
    load_p_row<R>(X, row, x);
    float* dst = X + static_cast<int64_t>(row) * R;
#pragma unroll 1
    for (int k0 = 0; k0 < R; k0 += 4) {
      double s[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
      for (int l = 0; l < R; ++l) {
        const double xl = static_cast<double>(x[l]);
#pragma unroll
        for (int q = 0; q < 4; ++q) s[q] += xl * T[l][k0 + q];
      }
      float v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = rnd16<ST>(static_cast<float>(s[q]));
      *reinterpret_cast<float4*>(dst + k0) = make_float4(v[0], v[1], v[2], v[3]);
      if (j.toff >= 0) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          tbase[j.toff + static_cast<int64_t>(k0 + q) * j.tstride + row] = v[q];
      }
    }
    return;
  } else {
    constexpr int B = 4;
    for (int row0 = row_begin + tid; row0 < row_end; row0 += kThreads * B) {
      float x[B][R];
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int row = row0 + b * kThreads;
        if (row < row_end) {
          load_p_row<R>(X, row, x[b]);
        } else {
#pragma unroll
          for (int l = 0; l < R; ++l) x[b][l] = 0.f;
        }
      }
#pragma unroll
      for (int b = 0; b < B; ++b) {
        const int row = row0 + b * kThreads;
        if (row >= row_end) continue;
        float* dst = X + static_cast<int64_t>(row) * R;
#pragma unroll 1
        for (int k = 0; k < R; ++k) {
          double s = 0.0;
#pragma unroll
          for (int l = 0; l < R; ++l) s += static_cast<double>(x[b][l]) * T[l][k];
          const float v = rnd16<ST>(static_cast<float>(s));
          dst[k] = v;
          if (j.toff >= 0) tbase[j.toff + static_cast<int64_t>(k) * j.tstride + row] = v;
        }
      }
    }
  }
}

// -------------------------------------------------------------------- q draw

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// Philox4x64 with 10 rounds (Salmon et al., SC 2011).
__device__ __forceinline__ void philox4x64_10(uint64_t (&x)[4], uint64_t k0, uint64_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t hi0 = __umul64hi(kPhiloxM0, x[0]);
    const uint64_t lo0 = kPhiloxM0 * x[0];
    const uint64_t hi1 = __umul64hi(kPhiloxM1, x[2]);
    const uint64_t lo1 = kPhiloxM1 * x[2];
    const uint64_t y0 = hi1 ^ x[1] ^ k0;
    const uint64_t y2 = hi0 ^ x[3] ^ k1;
    x[0] = y0;
    x[1] = lo1;
    x[2] = y2;
    x[3] = lo0;
  }
}

// Box-Muller in fp64: u in (0, 1] from the even word, v in [0, 1) from the odd word.
__device__ __forceinline__ void box_muller(uint64_t we, uint64_t wo, double& z0,
                                           double& z1) {
  const double u = (static_cast<double>(we >> 11) + 1.0) * 0x1p-53;
  const double v = static_cast<double>(wo >> 11) * 0x1p-53;
  const double radius = sqrt(-2.0 * log(u));
  const double angle = (2.0 * 3.141592653589793) * v;
  z0 = radius * cos(angle);
  z1 = radius * sin(angle);
}

// Draw of one job: block b of the m x rank matrix is Philox counter (b, view, epoch, 0)
// under key (seed, bucket_key); entry e = 4b + a is word a, via Box-Muller on the word
// pairs, stored at Q[qoff + (e / rank) * R + e % rank]. words (optional) receives the
// raw Philox output words in counter order.
template <int ST>
__device__ __forceinline__ void qinit_job(const QInitJob& j, float* __restrict__ Q, int R,
                                          uint64_t seed, uint64_t bucket_key, uint64_t epoch,
                                          int64_t first, int64_t stride,
                                          uint64_t* __restrict__ words) {
  const int64_t count = static_cast<int64_t>(j.m) * j.rank;
  const int64_t nblocks = (count + 3) / 4;
  for (int64_t b = first; b < nblocks; b += stride) {
    uint64_t w[4] = {static_cast<uint64_t>(b), static_cast<uint64_t>(j.view), epoch, 0};
    philox4x64_10(w, seed, bucket_key);
    if (words) {
#pragma unroll
      for (int a = 0; a < 4; ++a) words[4 * b + a] = w[a];
    }
    double z[4];
    box_muller(w[0], w[1], z[0], z[1]);
    box_muller(w[2], w[3], z[2], z[3]);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int64_t e = 4 * b + a;
      if (e < count) {
        const int64_t row = e / j.rank;
        const int k = static_cast<int>(e % j.rank);
        Q[j.qoff + row * R + k] = rnd16<ST>(static_cast<float>(z[a]));  // binary32 draw
      }
    }
  }
}

template <int ST>
__global__ void __launch_bounds__(256)
    k_qinit(const QInitJob* __restrict__ jobs, float* __restrict__ Q, int R, uint64_t seed,
            uint64_t bucket_key, uint64_t epoch) {
  qinit_job<ST>(jobs[blockIdx.y], Q, R, seed, bucket_key, epoch,
                static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                static_cast<int64_t>(gridDim.x) * blockDim.x, nullptr);
}

// One view's draw with the job passed by value (introspection; row stride = rank).
__global__ void __launch_bounds__(256)
    k_qdraw(QInitJob j, float* __restrict__ Q, uint64_t seed, uint64_t bucket_key,
            uint64_t epoch, uint64_t* __restrict__ words) {
  qinit_job<kStF32>(j, Q, j.rank, seed, bucket_key, epoch,
                    static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x,
                    static_cast<int64_t>(gridDim.x) * blockDim.x, words);
}

// ------------------------------------------------------- fp16 pass-through only

__global__ void __launch_bounds__(64) k_set_flag(int32_t* flag, int32_t value) {
  if (threadIdx.x == 0) *flag = value;
}

__global__ void __launch_bounds__(256)
    k_f16_check(const FlatTile* __restrict__ ft, const void* bucket, int32_t* found_inf) {
  f16_check_range(ft[blockIdx.x], bucket, found_inf);
}

__global__ void __launch_bounds__(256)
    k_f16_unscale(const FlatTile* __restrict__ ft, void* bucket, float inv_scale,
                  const int32_t* __restrict__ found_inf) {
  if (*found_inf) return;
  f16_unscale_range(ft[blockIdx.x], bucket, inv_scale);
}

__global__ void __launch_bounds__(256)
    k_fill_zero(void* base, int elem_bytes, int64_t start, int64_t count) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < count; i += gridDim.x * 256ll) {
    if (elem_bytes == 2)
      static_cast<uint16_t*>(base)[start + i] = 0;
    else
      static_cast<float*>(base)[start + i] = 0.f;
  }
}

template <int ST>
__global__ void __launch_bounds__(256) k_round16(const FlatTile* __restrict__ ft, void* bucket) {
  round_range<ST>(ft[blockIdx.x], bucket);
}

template <int ST>
__global__ void __launch_bounds__(256)
    k_widen16(const uint16_t* __restrict__ src, float* __restrict__ dst, int64_t count) {
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < count; i += gridDim.x * 256ll)
    dst[i] = from_h16<ST>(src[i]);
}

// ------------------------------------------------------------------ dispatch

// Rows loaded per lane before use, by rank (register budget).
template <int R, int ST = kStF32>
constexpr int unroll1() {
  return ST == kStF32 ? pass1_unroll(R) : (R <= 4 ? PSGD_PASS1_ROWS_H : 1);
}
template <int R, int ST = kStF32>
constexpr int unroll2() {
  return R <= 4 ? (ST == kStF32 ? PSGD_PASS2_ROWS : PSGD_PASS2_ROWS_H) : (R <= 8 ? 4 : 1);
}
template <int R, int ST = kStF32>
constexpr int unroll3() {
  return R <= 8 ? (ST == kStF32 ? PSGD_PASS3_ROWS : PSGD_PASS3_ROWS_H) : 1;
}

// Kernel K<..., F16, EF, ST> for the run-time (f16, ef, st); a 16-bit state has an fp32
// bucket. Returns false for a combination that does not exist.
#define PSGD_VARIANTS(LAUNCH)                                   \
  if (st == kStF16) {                                           \
    if (f16) return false;                                      \
    if (ef) LAUNCH(false, true, kStF16);                        \
    else LAUNCH(false, false, kStF16);                          \
  } else if (st == kStBF16) {                                   \
    if (f16) return false;                                      \
    if (ef) LAUNCH(false, true, kStBF16);                       \
    else LAUNCH(false, false, kStBF16);                         \
  } else {                                                      \
    if (f16 && ef) LAUNCH(true, true, kStF32);                  \
    else if (f16) LAUNCH(true, false, kStF32);                  \
    else if (ef) LAUNCH(false, true, kStF32);                   \
    else LAUNCH(false, false, kStF32);                          \
  }                                                             \
  return true;

template <int R>
bool pass1_vec(bool f16, bool ef, int st, const Pass1Args& a, dim3 grid, hipStream_t s) {
#define PSGD_L1(F, E, S) k_pass1<R, unroll1<R, S>(), F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_L1)
#undef PSGD_L1
}

template <int R>
bool pass2_vec(bool f16, bool ef, int st, const Pass2Args& a, dim3 grid, hipStream_t s) {
#define PSGD_L2(F, E, S) k_pass2<R, unroll2<R, S>(), F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_L2)
#undef PSGD_L2
}

template <int R>
bool pass3_vec(bool f16, bool ef, int st, const Pass3Args& a, dim3 grid, hipStream_t s) {
#define PSGD_L3(F, E, S) k_pass3<R, unroll3<R, S>(), F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_L3)
#undef PSGD_L3
}

template <int R>
bool pass1_mma(bool f16, bool ef, int st, const Pass1Args& a, dim3 grid, hipStream_t s) {
#define PSGD_M1(F, E, S) k_pass1_mfma<R, F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_M1)
#undef PSGD_M1
}

template <int R>
bool pass2_mma(bool f16, bool ef, int st, const Pass2Args& a, dim3 grid, hipStream_t s) {
#define PSGD_M2(F, E, S) k_pass2_mfma<R, F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_M2)
#undef PSGD_M2
}

template <int R>
bool pass3_mma(bool f16, bool ef, int st, const Pass3Args& a, dim3 grid, hipStream_t s) {
#define PSGD_M3(F, E, S) k_pass3_mfma<R, F, E, S><<<grid, kThreads, 0, s>>>(a)
  PSGD_VARIANTS(PSGD_M3)
#undef PSGD_M3
}

template <int R>
hipError_t pass1_r(bool f16, bool ef, int st, const Pass1Args& a, hipStream_t s) {
  const dim3 grid(a.ntiles + (f16 ? a.nftiles : 0));
  if (grid.x == 0) return hipSuccess;
  if constexpr (R >= kMfmaMinRank) {
    if (!pass1_mma<R>(f16, ef, st, a, grid, s)) return hipErrorInvalidValue;
  } else {
    if (!pass1_vec<R>(f16, ef, st, a, grid, s)) return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The 16-bit state's pass 2 with the wide aligned body alone.
template <int R>
bool pass2_wide16(bool ef, int st, const Pass2Args& a, dim3 grid, hipStream_t s) {
  if (st == kStF16) {
    if (ef) k_pass2<R, unroll2<R, kStF16>(), false, true, kStF16, true><<<grid, kThreads, 0, s>>>(a);
    else k_pass2<R, unroll2<R, kStF16>(), false, false, kStF16, true><<<grid, kThreads, 0, s>>>(a);
  } else if (st == kStBF16) {
    if (ef) k_pass2<R, unroll2<R, kStBF16>(), false, true, kStBF16, true><<<grid, kThreads, 0, s>>>(a);
    else k_pass2<R, unroll2<R, kStBF16>(), false, false, kStBF16, true><<<grid, kThreads, 0, s>>>(a);
  } else {
    return false;
  }
  return true;
}

template <int R>
hipError_t pass2_r(bool f16, bool ef, int st, bool wide_only, const Pass2Args& a,
                   hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  const dim3 grid(a.ntiles);
  if constexpr (R >= kMfmaMinRank) {
    if (!pass2_mma<R>(f16, ef, st, a, grid, s)) return hipErrorInvalidValue;
  } else {
    if (wide_only && !f16 && st != kStF32) {
      if (!pass2_wide16<R>(ef, st, a, grid, s)) return hipErrorInvalidValue;
    } else if (!pass2_vec<R>(f16, ef, st, a, grid, s)) {
      return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <int R>
hipError_t pass3_r(bool f16, bool ef, int st, const Pass3Args& a, hipStream_t s) {
  // extra workgroups: fp16 unscale, or the 16-bit state's cast, of uncompressed views
  const dim3 grid(a.ntiles + ((f16 || st != kStF32) ? a.nftiles : 0));
  if (grid.x == 0) return hipSuccess;
  if constexpr (R >= kMfmaMinRank) {
    if (!pass3_mma<R>(f16, ef, st, a, grid, s)) return hipErrorInvalidValue;
  } else {
    if (!pass3_vec<R>(f16, ef, st, a, grid, s)) return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kern

using namespace kern;

#define PSGD_RANK_SWITCH(R, ...)                    \
  switch (R) {                                      \
    case 1: { constexpr int RR = 1; __VA_ARGS__; }   \
    case 2: { constexpr int RR = 2; __VA_ARGS__; }   \
    case 4: { constexpr int RR = 4; __VA_ARGS__; }   \
    case 8: { constexpr int RR = 8; __VA_ARGS__; }   \
    case 16: { constexpr int RR = 16; __VA_ARGS__; } \
    case 32: { constexpr int RR = 32; __VA_ARGS__; } \
    default: return hipErrorInvalidValue;           \
  }

hipError_t launch_pass1(int R, bool f16, bool ef, int st, const Pass1Args& a, hipStream_t s) {
  PSGD_RANK_SWITCH(R, return pass1_r<RR>(f16, ef, st, a, s))
}

hipError_t launch_pass2(int R, bool f16, bool ef, int st, bool wide_only, const Pass2Args& a,
                        hipStream_t s) {
  PSGD_RANK_SWITCH(R, return pass2_r<RR>(f16, ef, st, wide_only, a, s))
}

hipError_t launch_pass2_reduce(int R, int st, const Pass2ReduceArgs& a, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  PSGD_RANK_SWITCH(R, {
    if (st == kStF16)
      k_pass2_reduce<RR, kStF16><<<dim3(a.ntiles), kReduceThreads, 0, s>>>(a);
    else if (st == kStBF16)
      k_pass2_reduce<RR, kStBF16><<<dim3(a.ntiles), kReduceThreads, 0, s>>>(a);
    else
      k_pass2_reduce<RR, kStF32><<<dim3(a.ntiles), kReduceThreads, 0, s>>>(a);
    return hipGetLastError();
  })
}

hipError_t launch_pass3(int R, bool f16, bool ef, int st, const Pass3Args& a, hipStream_t s) {
  PSGD_RANK_SWITCH(R, return pass3_r<RR>(f16, ef, st, a, s))
}

template <int R, int ST>
void materialize_r(const Pass3Args& a, dim3 grid, hipStream_t s) {
  if constexpr (R >= kMfmaMinRank)
    k_pass3_mfma<R, false, true, ST, true><<<grid, kThreads, 0, s>>>(a);
  else
    k_pass3<R, unroll3<R, ST>(), false, true, ST, true><<<grid, kThreads, 0, s>>>(a);
}

hipError_t launch_error_materialize(int R, int st, const Pass3Args& a, hipStream_t s) {
  if (a.ntiles == 0) return hipSuccess;
  const dim3 grid(a.ntiles);
  PSGD_RANK_SWITCH(R, {
    if (st == kStF16)
      materialize_r<RR, kStF16>(a, grid, s);
    else if (st == kStBF16)
      materialize_r<RR, kStBF16>(a, grid, s);
    else
      materialize_r<RR, kStF32>(a, grid, s);
    return hipGetLastError();
  })
}

hipError_t launch_gram(int R, const Tile* tiles, int ntiles, const OrthJob* jobs,
                       float* base, const float* part, double* gram,
                       const int32_t* found_inf, int st, hipStream_t s) {
  if (ntiles == 0) return hipSuccess;
  PSGD_RANK_SWITCH(R, {
    if (st == kStF16)
      k_gram<RR, kStF16><<<dim3(ntiles), kThreads, 0, s>>>(tiles, jobs, base, part, gram, found_inf);
    else if (st == kStBF16)
      k_gram<RR, kStBF16><<<dim3(ntiles), kThreads, 0, s>>>(tiles, jobs, base, part, gram, found_inf);
    else
      k_gram<RR, kStF32><<<dim3(ntiles), kThreads, 0, s>>>(tiles, jobs, base, part, gram, found_inf);
    return hipGetLastError();
  })
}

hipError_t launch_orth(int R, const OrthJob* jobs, int njobs, int max_rows, float* base,
                       float* tbase, const double* gram, double* tmat, double eps,
                       const int32_t* found_inf, int st, hipStream_t s) {
  if (njobs == 0) return hipSuccess;
  const dim3 grid((max_rows + orth_rows(R) - 1) / orth_rows(R), njobs);
  PSGD_RANK_SWITCH(R, {
    k_orth_t<RR><<<dim3(njobs), kOrthThreads, 0, s>>>(jobs, gram, tmat, eps, found_inf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (st == kStF16)
      k_orth<RR, kStF16><<<grid, kThreads, 0, s>>>(jobs, base, tbase, tmat, found_inf);
    else if (st == kStBF16)
      k_orth<RR, kStBF16><<<grid, kThreads, 0, s>>>(jobs, base, tbase, tmat, found_inf);
    else
      k_orth<RR, kStF32><<<grid, kThreads, 0, s>>>(jobs, base, tbase, tmat, found_inf);
    return hipGetLastError();
  })
}

hipError_t launch_qinit(int R, const QInitJob* jobs, int njobs, int64_t max_count,
                        float* Q, uint64_t seed, uint64_t bucket_key, uint64_t epoch, int st,
                        hipStream_t s) {
  if (njobs == 0) return hipSuccess;
  const int64_t blocks = ((max_count + 3) / 4 + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks)),
                  static_cast<unsigned>(njobs));
  if (st == kStF16)
    k_qinit<kStF16><<<grid, 256, 0, s>>>(jobs, Q, R, seed, bucket_key, epoch);
  else if (st == kStBF16)
    k_qinit<kStBF16><<<grid, 256, 0, s>>>(jobs, Q, R, seed, bucket_key, epoch);
  else
    k_qinit<kStF32><<<grid, 256, 0, s>>>(jobs, Q, R, seed, bucket_key, epoch);
  return hipGetLastError();
}

hipError_t launch_qdraw(int64_t m, int rank, int view, float* out, uint64_t* words,
                       uint64_t seed, uint64_t bucket_key, uint64_t epoch, hipStream_t s) {
  const int64_t count = m * rank;
  if (count <= 0) return hipSuccess;
  const int64_t blocks = ((count + 3) / 4 + 255) / 256;
  const QInitJob j{0, static_cast<int32_t>(m), rank, view, 0};
  k_qdraw<<<dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), 256, 0, s>>>(
      j, out, seed, bucket_key, epoch, words);
  return hipGetLastError();
}

hipError_t launch_widen16(const uint16_t* src, float* dst, int64_t count, int st, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  const dim3 grid(static_cast<unsigned>(blocks < 1024 ? blocks : 1024));
  if (st == kStF16)
    k_widen16<kStF16><<<grid, 256, 0, s>>>(src, dst, count);
  else if (st == kStBF16)
    k_widen16<kStBF16><<<grid, 256, 0, s>>>(src, dst, count);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_round_only(const FlatTile* ftiles, int nftiles, void* bucket, int st,
                             hipStream_t s) {
  if (nftiles == 0) return hipSuccess;
  if (st == kStF16)
    k_round16<kStF16><<<dim3(nftiles), 256, 0, s>>>(ftiles, bucket);
  else if (st == kStBF16)
    k_round16<kStBF16><<<dim3(nftiles), 256, 0, s>>>(ftiles, bucket);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* base, bool f16, int64_t start, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  k_fill_zero<<<dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), 256, 0, s>>>(
      base, f16 ? 2 : 4, start, count);
  return hipGetLastError();
}

hipError_t launch_set_flag(int32_t* flag, int32_t value, hipStream_t s) {
  k_set_flag<<<dim3(1), 64, 0, s>>>(flag, value);
  return hipGetLastError();
}

hipError_t launch_unscale_only(const FlatTile* ftiles, int nftiles, void* bucket,
                               float inv_scale, int32_t* found_inf, bool check,
                               hipStream_t s) {
  if (nftiles == 0) return hipSuccess;
  if (check)
    k_f16_check<<<dim3(nftiles), 256, 0, s>>>(ftiles, bucket, found_inf);
  else
    k_f16_unscale<<<dim3(nftiles), 256, 0, s>>>(ftiles, bucket, inv_scale, found_inf);
  return hipGetLastError();
}

}  // namespace psgd
