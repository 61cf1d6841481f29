// Backward of the elementwise stages of the core (the chain rule through
// layers page, _output_norm_gate_core and _qk_norm_rope_core, as autograd
// differentiates them: a gradient takes its primal's dtype).
//
// out_norm_gate_bwd: with y = o r, r = (mean(o^2) + eps)^-1/2, s = sigmoid(g):
//   dgate = dout y s (1 - s);  dy = dout s;  do = r dy - r^3 o mean(dy o)
//   (both rounded to bf16), and delta = rowsum(do * o) in FP32, the softmax
//   correction the attention backward needs.
// qk_norm_rope_bwd: the FP32 rotation's transpose (dy0 C + dy1 S, -dy0 S + dy1 C)
//   rounded to bf16, times query_scale (Q, rounded again), then the RMSNorm
//   backward with u = dx~ w: dx = r u - r^3 x mean(u x) (bf16), and the gain
//   gradient sum over rows of dx~ x r (FP32).
//
// Both are HBM-bound and use the forward kernels' row layout: a row of D
// values over D/8 lanes of 8 consecutive elements, row sums by DPP.  r is
// recomputed with the forward's reduction tree, so it equals the forward's
// bits.  Gain gradients are reduced deterministically: every block walks a
// fixed set of rows, sums its lanes' partials through LDS in a fixed order,
// and a second kernel adds the block partials of each column in block order.
#include <mutex>

#include "device_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int kThreads = 256;
constexpr int kOgRows = 4;          // rows in flight per thread (out_norm_gate_bwd)
constexpr int kQkRows = 2;          // rows in flight per thread per step (qk_norm_rope_bwd)
constexpr int kMaxQkBlocks = 2048;  // blocks per tensor (partial-sum rows)

// ---------------------------------------------------------------------------
template <int D, bool GATE>
__global__ __launch_bounds__(kThreads) void out_norm_gate_bwd_kernel(OutGateBwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  const int c = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;
  const int64_t base = (int64_t)blockIdx.x * RPP * kOgRows;

  uint4 oin[kOgRows], gin[kOgRows], din[kOgRows];
#pragma unroll
  for (int j = 0; j < kOgRows; ++j) {
    const int64_t r = base + (int64_t)j * RPP + rsub;
    oin[j] = gin[j] = din[j] = make_uint4(0, 0, 0, 0);
    if (r < a.rows) {
      oin[j] = *reinterpret_cast<const uint4 *>(a.o + r * D + c * 8);
      if (GATE) gin[j] = *reinterpret_cast<const uint4 *>(a.gate + r * D + c * 8);
      din[j] = *reinterpret_cast<const uint4 *>(a.dout + r * D + c * 8);
    }
  }
  constexpr float inv_d = 1.0f / (float)D;
#pragma unroll
  for (int j = 0; j < kOgRows; ++j) {
    const int64_t r = base + (int64_t)j * RPP + rsub;
    float x[8], dd[8];
    unpack8(oin[j], x);
    unpack8(din[j], dd);
    if constexpr (GATE) {
      float g[8];
      unpack8(gin[j], g);
      const float rstd = rms_rstd(row_sum<LPR>(chunk_sumsq<4>(x) + chunk_sumsq<4>(x + 4)), inv_d, a.eps);
      float dy[8], dg[8], t = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float s = sigmoidf(g[e]);
        const float y = x[e] * rstd;
        dg[e] = ((dd[e] * y) * s) * (1.0f - s);
        dy[e] = dd[e] * s;
        t = __builtin_fmaf(dy[e], x[e], t);
      }
      const float mean = row_sum<LPR>(t) * inv_d;
      const float r3m = rstd * rstd * rstd * mean;
      float dox[8], dl = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        dox[e] = round_bf16(rstd * dy[e] - r3m * x[e]);
        dl = __builtin_fmaf(dox[e], x[e], dl);
      }
      const float delta = row_sum<LPR>(dl);
      if (r >= a.rows) continue;
      *reinterpret_cast<uint4 *>(a.d_o + r * D + c * 8) = pack8(dox);
      *reinterpret_cast<uint4 *>(a.dgate + r * D + c * 8) = pack8(dg);
      if (c == 0) a.delta[r] = delta;
    } else {
      float dl = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) dl = __builtin_fmaf(dd[e], x[e], dl);
      const float delta = row_sum<LPR>(dl);
      if (r < a.rows && c == 0) a.delta[r] = delta;
    }
  }
}

// ---------------------------------------------------------------------------
// ROPE: rotate the gradient back (the transpose of the forward's rotation:
// FP32 cos/sin, or their bf16 casts after the Q/K-dtype rotation); QS:
// query_scale != 1; NORM: false for the norm-free (vision) rotation.
template <int D, bool ROPE, bool QS, bool NORM>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_bwd_kernel(QkNormBwdArgs a) {
  constexpr int LPR = D / 8;
  constexpr int RPP = kThreads / LPR;
  static_assert(LPR == 8 || LPR == 16, "row_sum covers 8 or 16 lanes");
  __shared__ float red[RPP][D];
  const int c = threadIdx.x % LPR;
  const int rsub = threadIdx.x / LPR;

  const bool is_q = (int)blockIdx.x < a.q_blocks;
  const int blk = is_q ? (int)blockIdx.x : (int)blockIdx.x - a.q_blocks;
  const int nblk = is_q ? a.q_blocks : a.k_blocks;
  const int nrows = is_q ? a.q_rows : a.k_rows;
  const uint16_t *xsrc = is_q ? a.q : a.k;
  const uint16_t *gsrc = is_q ? a.dq_hat : a.dk_hat;
  uint16_t *dst = is_q ? a.dq : a.dk;
  const float *gain = is_q ? a.q_gain : a.k_gain;
  float *part = is_q ? a.q_part : a.k_part;
  const FastDiv hdiv = is_q ? a.hq_div : a.hkv_div;
  const float qs = is_q ? a.query_scale : 1.0f;

  float w[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if (NORM && gain) {
    const float4 g0 = *reinterpret_cast<const float4 *>(gain + c * 8);
    const float4 g1 = *reinterpret_cast<const float4 *>(gain + c * 8 + 4);
    w[0] = a.gain_center + g0.x; w[1] = a.gain_center + g0.y;
    w[2] = a.gain_center + g0.z; w[3] = a.gain_center + g0.w;
    w[4] = a.gain_center + g1.x; w[5] = a.gain_center + g1.y;
    w[6] = a.gain_center + g1.z; w[7] = a.gain_center + g1.w;
  }
  float gacc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr float inv_d = 1.0f / (float)D;

  // row groups blk, blk + nblk, ...; kQkRows of them per step
  for (int grp = blk * kQkRows; grp * RPP < nrows; grp += nblk * kQkRows) {
    uint4 xin[kQkRows], gin[kQkRows];
#pragma unroll
    for (int j = 0; j < kQkRows; ++j) {
      const int r = (grp + j) * RPP + rsub;
      xin[j] = gin[j] = make_uint4(0, 0, 0, 0);
      if (r < nrows) {
        if (NORM) xin[j] = *reinterpret_cast<const uint4 *>(xsrc + (int64_t)r * D + c * 8);
        gin[j] = *reinterpret_cast<const uint4 *>(gsrc + (int64_t)r * D + c * 8);
      }
    }
    // the group's rows are consecutive: one segment search per group
    PosCursor pc{0, 0, 0};
    if constexpr (ROPE) pc = pos_cursor(a.lay, (int)hdiv.div((uint32_t)(grp * RPP)));
#pragma unroll
    for (int j = 0; j < kQkRows; ++j) {
      const int r = (grp + j) * RPP + rsub;
      float dx[8];
      unpack8(gin[j], dx);
      if constexpr (ROPE) {
        const int t = (int)hdiv.div((uint32_t)min(r, nrows - 1));
        const int p = rope_position(a.lay, pc, t, a.n_pos);
        const float4 cv = *reinterpret_cast<const float4 *>(a.cos_tab + (int64_t)p * (D / 2) + c * 4);
        const float4 sv = *reinterpret_cast<const float4 *>(a.sin_tab + (int64_t)p * (D / 2) + c * 4);
        float cs[4] = {cv.x, cv.y, cv.z, cv.w}, sn[4] = {sv.x, sv.y, sv.z, sv.w};
        if (a.rope_v2) {
          // the Q/K-dtype rotation multiplied by bf16 cos/sin; its bf16 product
          // and sum roundings are differentiated as the identity
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            cs[i] = round_bf16(cs[i]);
            sn[i] = round_bf16(sn[i]);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float d0 = dx[2 * i], d1 = dx[2 * i + 1];
          dx[2 * i] = round_bf16(__builtin_fmaf(d0, cs[i], d1 * sn[i]));
          dx[2 * i + 1] = round_bf16(__builtin_fmaf(d1, cs[i], -(d0 * sn[i])));
        }
      }
      if constexpr (QS) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dx[e] = round_bf16(dx[e] * qs);
      }
      if constexpr (NORM) {
        float x[8];
        unpack8(xin[j], x);
        const float rstd = rms_rstd(row_sum<LPR>(chunk_sumsq<8>(x)), inv_d, a.eps);
        float u[8], t = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          gacc[e] = __builtin_fmaf(dx[e], x[e] * rstd, gacc[e]);   // zero for rows past the end
          u[e] = dx[e] * w[e];
          t = __builtin_fmaf(u[e], x[e], t);
        }
        const float r3m = rstd * rstd * rstd * (row_sum<LPR>(t) * inv_d);
#pragma unroll
        for (int e = 0; e < 8; ++e) dx[e] = rstd * u[e] - r3m * x[e];
      }
      if (r < nrows) *reinterpret_cast<uint4 *>(dst + (int64_t)r * D + c * 8) = pack8(dx);
    }
  }

  if (!NORM || !part) return;   // uniform per block
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rsub][c * 8 + e] = gacc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < RPP; ++i) s += red[i][threadIdx.x];
    part[(int64_t)blk * D + threadIdx.x] = s;
  }
}

// Column sums of the block partials in a fixed order: a block of 1024
// threads takes 32 columns; each of the 32 slices of a column sums the
// partial rows slice, slice + 32, ... with 8 loads in flight (8 independent
// accumulators added pairwise), and the 32 slice sums are added pairwise
// through LDS.  Deterministic, and wide enough that a few thousand partial
// rows cost a few microseconds.
constexpr int kRedThreads = 1024;
__global__ __launch_bounds__(kRedThreads) void gain_reduce_kernel(const float *part, float *out, int blocks,
                                                                   int d) {
  __shared__ float red[32][33];
  const int cl = threadIdx.x & 31;
  const int sl = threadIdx.x >> 5;          // slice 0..31
  const int c = blockIdx.x * 32 + cl;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (c < d) {
    int b = sl;
    for (; b + 7 * 32 < blocks; b += 8 * 32) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] += part[(int64_t)(b + u * 32) * d + c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (b + u * 32 < blocks) acc[u] += part[(int64_t)(b + u * 32) * d + c];
  }
  red[sl][cl] = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  __syncthreads();
#pragma unroll
  for (int w = 16; w >= 1; w >>= 1) {
    if (sl < w) red[sl][cl] = red[sl][cl] + red[sl + w][cl];
    __syncthreads();
  }
  if (sl == 0 && c < d) out[c] = red[0][cl];
}

template <int D, bool ROPE, bool NORM>
void launch_qs(const QkNormBwdArgs &a, dim3 grid, hipStream_t stream) {
  if (a.q_rows > 0 && a.query_scale != 1.0f)
    hipLaunchKernelGGL((qk_norm_rope_bwd_kernel<D, ROPE, true, NORM>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((qk_norm_rope_bwd_kernel<D, ROPE, false, NORM>), grid, dim3(kThreads), 0, stream, a);
}

template <int D>
void launch_qk_bwd_d(const QkNormBwdArgs &a, dim3 grid, hipStream_t stream) {
  if (a.skip_norm) {
    if (a.use_rope) launch_qs<D, true, false>(a, grid, stream);
    else launch_qs<D, false, false>(a, grid, stream);
  } else {
    if (a.use_rope) launch_qs<D, true, true>(a, grid, stream);
    else launch_qs<D, false, true>(a, grid, stream);
  }
}

}  // namespace

hipError_t launch_out_norm_gate_bwd(int head_dim, const OutGateBwdArgs &a, hipStream_t stream) {
  if (a.rows == 0) return hipSuccess;
  const int64_t per_block = (int64_t)(kThreads / (head_dim / 8)) * kOgRows;
  const dim3 grid((unsigned)((a.rows + per_block - 1) / per_block));
  const bool gate = a.gate != nullptr;
  if (head_dim == 128) {
    if (gate) hipLaunchKernelGGL((out_norm_gate_bwd_kernel<128, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((out_norm_gate_bwd_kernel<128, false>), grid, dim3(kThreads), 0, stream, a);
  } else {
    if (gate) hipLaunchKernelGGL((out_norm_gate_bwd_kernel<64, true>), grid, dim3(kThreads), 0, stream, a);
    else hipLaunchKernelGGL((out_norm_gate_bwd_kernel<64, false>), grid, dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

void qk_norm_bwd_blocks(int head_dim, int64_t q_rows, int64_t k_rows, int32_t *q_blocks, int32_t *k_blocks) {
  const int64_t rpp = kThreads / (head_dim / 8);
  auto nb = [&](int64_t rows) -> int32_t {
    const int64_t groups = (rows + rpp - 1) / rpp;
    const int64_t b = (groups + kQkRows - 1) / kQkRows;
    return (int32_t)(b < kMaxQkBlocks ? b : kMaxQkBlocks);
  };
  *q_blocks = nb(q_rows);
  *k_blocks = nb(k_rows);
}

// Scratch of muse_qk_norm_rope_bwd_static: the gain partial sums of both
// tensors at the largest block count ([2][kMaxQkBlocks][128] floats, 2 MiB),
// one copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is a stand-in, not a device
// address): the launch takes the address hipGetSymbolAddress reports for the
// current device.
constexpr size_t kStaticScratchFloats = 2 * (size_t)kMaxQkBlocks * 128;
static __device__ __align__(256) float scratch[kStaticScratchFloats];

hipError_t qk_norm_bwd_static_scratch(float **ptr, size_t *bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float *>(p);
  }
  *ptr = addr[dev];
  *bytes = kStaticScratchFloats * sizeof(float);
  return hipSuccess;
}

hipError_t launch_qk_norm_rope_bwd(int head_dim, const QkNormBwdArgs &args, hipStream_t stream) {
  QkNormBwdArgs a = args;
  qk_norm_bwd_blocks(head_dim, a.q_rows, a.k_rows, &a.q_blocks, &a.k_blocks);
  const int blocks = a.q_blocks + a.k_blocks;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) launch_qk_bwd_d<128>(a, dim3(blocks), stream);
  else launch_qk_bwd_d<64>(a, dim3(blocks), stream);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.skip_norm) return e;
  if (a.q_part && a.q_blocks > 0) {
    hipLaunchKernelGGL(gain_reduce_kernel, dim3((head_dim + 31) / 32), dim3(kRedThreads), 0, stream, a.q_part,
                       a.dq_gain, a.q_blocks, head_dim);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (a.k_part && a.k_blocks > 0) {
    hipLaunchKernelGGL(gain_reduce_kernel, dim3((head_dim + 31) / 32), dim3(kRedThreads), 0, stream, a.k_part,
                       a.dk_gain, a.k_blocks, head_dim);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace muse
