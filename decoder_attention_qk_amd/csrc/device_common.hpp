// Device helpers shared by the libmuseattn kernels (gfx950, wave64).
//
// The per-element arithmetic of the Q/K norm + RoPE step and of the output
// norm + gate step lives here once, so the standalone kernels and the fused
// attention kernel apply the same operations in the same order and produce
// identical bits.  Sums of squares use one fixed reduction tree (a per-chunk
// fma chain, then pairwise sums over chunk indices); every kernel that
// normalises a row reproduces that tree whatever its lane layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace muse {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bfloat16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 bits, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ float round_bf16(float x) {
  __bf16 a = (__bf16)x;
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, a) << 16);
}

// 8 bf16 in a uint4 <-> 8 floats.
__device__ __forceinline__ void unpack8(const uint4 &v, float (&x)[8]) {
  x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x);
  x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
  x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z);
  x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
}
__device__ __forceinline__ uint4 pack8(const float (&y)[8]) {
  uint4 r;
  r.x = pack_bf16x2(y[0], y[1]);
  r.y = pack_bf16x2(y[2], y[3]);
  r.z = pack_bf16x2(y[4], y[5]);
  r.w = pack_bf16x2(y[6], y[7]);
  return r;
}

// ---------------------------------------------------------------------------
// Sums of squares.  A row of D values is cut into chunks of CH consecutive
// elements; each chunk's partial is an fma chain from element 0 upwards; the
// chunk partials are combined by pairwise sums over chunk indices
// (c, c^1), then pairs (c>>1, (c>>1)^1), and so on -- the order a butterfly
// over lanes produces.
// ---------------------------------------------------------------------------
template <int CH>
__device__ __forceinline__ float chunk_sumsq(const float *x) {
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < CH; ++e) acc = __builtin_fmaf(x[e], x[e], acc);
  return acc;
}

// In-register pairwise tree over N chunk partials (N a power of two).
template <int N>
__device__ __forceinline__ float tree_sum(float (&p)[N]) {
#pragma unroll
  for (int w = 1; w < N; w <<= 1) {
#pragma unroll
    for (int c = 0; c < N; c += 2 * w) p[c] = p[c] + p[c + w];
  }
  return p[0];
}

// DPP row permutations (within 16-lane rows).
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within each 8 lanes
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within each 16 lanes

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the LPR lanes (8 or 16, aligned) holding one row, in the shared
// tree order: pairs of chunks (c, c^1), then pairs of pairs, ...  Each step
// adds the partner group's partial, so every lane ends with the same bits.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
  v = v + dpp<kDppXor1>(v);
  v = v + dpp<kDppXor2>(v);
  if constexpr (LPR >= 8) v = v + dpp<kDppHalfMirror>(v);
  if constexpr (LPR >= 16) v = v + dpp<kDppMirror>(v);
  return v;
}

// 1 / sqrt(mean + eps) with correctly rounded sqrt and division.
__device__ __forceinline__ float rms_rstd(float sumsq, float inv_d, float eps) {
  return 1.0f / __builtin_sqrtf(__builtin_fmaf(sumsq, inv_d, 0.0f) + eps);
}

// ---------------------------------------------------------------------------
// Q/K norm + query scale + RoPE on one chunk of 8 consecutive elements
// (4 adjacent pairs), in two stages so a caller may split them:
//   norm_chunk:       bf16((x * r) * w) for each pair (one packed conversion)
//   scale_rope_chunk: optional bf16(. * qscale), then the FP32 rotation of each
//                     pair by (c, s), rounded to bf16.
// x: inputs; w: effective gains; c, s: cos/sin of the 4 pairs (ignored when
// !rope).  Each rounded pair is one packed conversion; the rounded values feed
// the next step.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint4 norm_chunk(const float (&x)[8], const float (&w)[8], float r) {
  uint32_t out[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2((x[2 * i] * r) * w[2 * i], (x[2 * i + 1] * r) * w[2 * i + 1]);
  return make_uint4(out[0], out[1], out[2], out[3]);
}
// The Q/K-dtype rotation of one packed pair (apply_rotary_embedding with
// upcast=False): C and S cast to bf16, each product rounded to bf16, then the
// difference / sum rounded to bf16 -- each a bf16 operation evaluated in FP32
// and rounded once.  (Products of two bf16 values are exact in FP32.)
__device__ __forceinline__ uint32_t rope_pair_v2(uint32_t p, float c, float s) {
  const float a = bf16_lo(p), b = bf16_hi(p);
  const float cb = round_bf16(c), sb = round_bf16(s);
  const float y0 = round_bf16(round_bf16(a * cb) - round_bf16(b * sb));
  const float y1 = round_bf16(round_bf16(a * sb) + round_bf16(b * cb));
  return pack_bf16x2(y0, y1);   // exact: both already bf16 values
}
// rope_v2 selects the Q/K-dtype rotation above instead of the FP32 one.
__device__ __forceinline__ uint4 scale_rope_chunk(const uint4 &v, bool apply_qscale, float qscale, bool rope,
                                                  const float (&c)[4], const float (&s)[4], bool rope_v2 = false) {
  uint32_t out[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t p = out[i];
    if (apply_qscale) p = pack_bf16x2(bf16_lo(p) * qscale, bf16_hi(p) * qscale);
    if (rope) {
      if (rope_v2) {
        p = rope_pair_v2(p, c[i], s[i]);
      } else {
        const float a = bf16_lo(p), b = bf16_hi(p);
        p = pack_bf16x2(__builtin_fmaf(a, c[i], -(b * s[i])), __builtin_fmaf(a, s[i], b * c[i]));
      }
    }
    out[i] = p;
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}
__device__ __forceinline__ uint4 qk_chunk(const float (&x)[8], const float (&w)[8], float r,
                                          bool apply_qscale, float qscale, bool rope,
                                          const float (&c)[4], const float (&s)[4], bool rope_v2 = false) {
  return scale_rope_chunk(norm_chunk(x, w, r), apply_qscale, qscale, rope, c, s, rope_v2);
}

// ---------------------------------------------------------------------------
// Output norm + gate on one element: bf16((o * r) * sigmoid(g)), sigmoid in
// FP32 as 1 / (1 + 2^(-g log2 e)).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigmoidf(float g) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -kLog2e));
}
__device__ __forceinline__ float gate_elem(float o, float r, float g) {
  return (o * r) * sigmoidf(g);
}

}  // namespace muse
