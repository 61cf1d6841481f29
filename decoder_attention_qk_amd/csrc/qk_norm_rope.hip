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
  const int64_t base = (int64_t)blockIdx.x * RPP * kRowsInFlight;

  uint4 xin[kRowsInFlight];
  int64_t rows[kRowsInFlight];
#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int64_t r = base + (int64_t)j * RPP + rsub;
    rows[j] = r;
    xin[j] = make_uint4(0, 0, 0, 0);
    if (r < a.total_rows) {
      const uint16_t *src = r < a.q_rows ? a.q + r * D : a.k + (r - a.q_rows) * D;
      xin[j] = *reinterpret_cast<const uint4 *>(src + c * 8);
    }
  }

#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int64_t r = rows[j];
    const bool valid = r < a.total_rows;
    const bool is_q = r < a.q_rows;
    float x[8];
    unpack8(xin[j], x);
    float ss = chunk_sumsq<8>(x);
#pragma unroll
    for (int w = 1; w < LPR; w <<= 1) ss = ss + __shfl_xor(ss, w);
    if (!valid) continue;
    const float rstd = rms_rstd(ss, 1.0f / (float)D, a.eps);

    const float *gain = is_q ? a.q_gain : a.k_gain;
    float w[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = gain ? a.gain_center + gain[c * 8 + e] : 1.0f;

    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t tok;
    int heads;
    if (is_q) { tok = r / a.hq; heads = a.hq; } else { tok = (r - a.q_rows) / a.hkv; heads = a.hkv; }
    (void)heads;
    if (a.use_rope) {
      const int p = rope_position(a.lay, (int)tok, a.n_pos);
      const float4 cv = *reinterpret_cast<const float4 *>(a.cos_tab + (int64_t)p * (D / 2) + c * 4);
      const float4 sv = *reinterpret_cast<const float4 *>(a.sin_tab + (int64_t)p * (D / 2) + c * 4);
      cs[0] = cv.x; cs[1] = cv.y; cs[2] = cv.z; cs[3] = cv.w;
      sn[0] = sv.x; sn[1] = sv.y; sn[2] = sv.z; sn[3] = sv.w;
    }
    float y[8];
    qk_chunk(x, w, rstd, is_q && a.query_scale != 1.0f, a.query_scale, a.use_rope != 0, cs, sn, y);
    uint16_t *dst = is_q ? a.q_out + r * D : a.k_out + (r - a.q_rows) * D;
    *reinterpret_cast<uint4 *>(dst + c * 8) = pack8(y);
    if (c == 0) {
      if (is_q) { if (a.q_rstd) a.q_rstd[r] = rstd; }
      else if (a.k_rstd) a.k_rstd[r - a.q_rows] = rstd;
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
