// Q/K RMSNorm + zero-centred gain + bf16 cast + query_scale + adjacent-pair
// RoPE (layers page, _qk_norm_rope_core, _rms_norm_core,
// apply_rotary_embedding with upcast=True).
//
// HBM-bound.  Each (token, head) row of D bf16 values is spread over D/8
// lanes holding 8 consecutive elements (one 16-byte load); the row's sum of
// squares is a per-lane fma chain followed by an xor butterfly over those
// lanes.  Every thread keeps ROWS_IN_FLIGHT rows' loads outstanding before it
// computes.  Q rows come first (row r = token * Hq + head), then K rows.
#include "device_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsInFlight = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(QkNormArgs a) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RPP = kThreads / LPR;      // rows per pass of the block
  const int c = threadIdx.x % LPR;         // chunk: elements [8c, 8c+8)
  const int rsub = threadIdx.x / LPR;
  const int base = blockIdx.x * RPP * kRowsInFlight;

  // effective gains of this lane's 8 columns (fixed for every row it touches)
  float wq[8], wk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    wq[e] = a.q_gain ? a.gain_center + a.q_gain[c * 8 + e] : 1.0f;
    wk[e] = a.k_gain ? a.gain_center + a.k_gain[c * 8 + e] : 1.0f;
  }

  uint4 xin[kRowsInFlight];
#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int r = base + j * RPP + rsub;
    xin[j] = make_uint4(0, 0, 0, 0);
    if (r < a.total_rows) {
      const uint16_t *src = r < a.q_rows ? a.q + (int64_t)r * D : a.k + (int64_t)(r - a.q_rows) * D;
      xin[j] = *reinterpret_cast<const uint4 *>(src + c * 8);
    }
  }

#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int r = base + j * RPP + rsub;
    const bool valid = r < a.total_rows;
    const bool is_q = r < a.q_rows;
    float x[8];
    unpack8(xin[j], x);
    float ss = chunk_sumsq<8>(x);
#pragma unroll
    for (int w = 1; w < LPR; w <<= 1) ss = ss + __shfl_xor(ss, w);
    if (!valid) continue;
    const float rstd = rms_rstd(ss, 1.0f / (float)D, a.eps);
    const int rr = is_q ? r : r - a.q_rows;            // row inside its own tensor
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
    if (a.use_rope) {
      const int tok = (int)(is_q ? a.hq_div.div((uint32_t)rr) : a.hkv_div.div((uint32_t)rr));
      const int p = rope_position(a.lay, tok, a.n_pos);
      const float4 cv = *reinterpret_cast<const float4 *>(a.cos_tab + p * (D / 2) + c * 4);
      const float4 sv = *reinterpret_cast<const float4 *>(a.sin_tab + p * (D / 2) + c * 4);
      cs[0] = cv.x; cs[1] = cv.y; cs[2] = cv.z; cs[3] = cv.w;
      sn[0] = sv.x; sn[1] = sv.y; sn[2] = sv.z; sn[3] = sv.w;
    }
    const uint4 y = qk_chunk(x, is_q ? wq : wk, rstd, is_q && a.query_scale != 1.0f, a.query_scale,
                             a.use_rope != 0, cs, sn);
    uint16_t *dst = is_q ? a.q_out : a.k_out;
    *reinterpret_cast<uint4 *>(dst + (int64_t)rr * D + c * 8) = y;
    if (c == 0) {
      float *rs = is_q ? a.q_rstd : a.k_rstd;
      if (rs) rs[rr] = rstd;
    }
  }
}

}  // namespace

hipError_t launch_qk_norm_rope(int head_dim, const QkNormArgs &a, hipStream_t stream) {
  if (a.total_rows == 0) return hipSuccess;
  const int lpr = head_dim / 8;
  const int64_t rows_per_block = (int64_t)(kThreads / lpr) * kRowsInFlight;
  const int64_t blocks = (a.total_rows + rows_per_block - 1) / rows_per_block;
  if (head_dim == 128)
    hipLaunchKernelGGL(qk_norm_rope_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(qk_norm_rope_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muse
