// Parameter-free output RMSNorm times the sigmoid output gate (layers page,
// _output_norm_gate_core): out = bf16(o * rstd * sigmoid(gate)), in FP32.
//
// HBM-bound: reads O and the gate once, writes out once.  Each row of D
// values spreads over D/8 lanes of 8 consecutive elements.  The sum of
// squares treats each lane's 8 elements as two 4-element groups (an fma
// chain each), adds the pair, then reduces over the row's lanes with DPP
// (row_sum) -- the same tree the fused attention epilogue uses on its own
// layout.
#include "device_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsInFlight = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void out_norm_gate_kernel(OutGateArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  const int c = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  const int64_t base = (int64_t)blockIdx.x * RPP * kRowsInFlight;

  uint4 oin[kRowsInFlight], gin[kRowsInFlight];
#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int64_t r = base + (int64_t)j * RPP + rsub;
    oin[j] = make_uint4(0, 0, 0, 0);
    gin[j] = make_uint4(0, 0, 0, 0);
    if (r < a.rows) {
      oin[j] = *reinterpret_cast<const uint4 *>(a.o + r * D + c * 8);
      gin[j] = *reinterpret_cast<const uint4 *>(a.gate + r * D + c * 8);
    }
  }
#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int64_t r = base + (int64_t)j * RPP + rsub;
    float x[8], g[8];
    unpack8(oin[j], x);
    unpack8(gin[j], g);
    const float ss = row_sum<LPR>(chunk_sumsq<4>(x) + chunk_sumsq<4>(x + 4));
    if (r >= a.rows) continue;
    const float rstd = rms_rstd(ss, 1.0f / (float)D, a.eps);
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = gate_elem(x[e], rstd, g[e]);
    *reinterpret_cast<uint4 *>(a.out + r * D + c * 8) = pack8(y);
    if (c == 0 && a.o_rstd) a.o_rstd[r] = rstd;
  }
}

}  // namespace

hipError_t launch_out_norm_gate(int head_dim, const OutGateArgs &a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int lpr = head_dim / 8;
  const int64_t rows_per_block = (int64_t)(kThreads / lpr) * kRowsInFlight;
  const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
  if (head_dim == 128)
    hipLaunchKernelGGL(out_norm_gate_kernel<128>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(out_norm_gate_kernel<64>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muse
