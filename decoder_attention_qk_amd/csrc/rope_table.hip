// FP32 RoPE cos/sin tables.
//
// 1-D (layers page, MuseSparkRotaryEmbedding: FP32 adjacent-pair frequencies;
// cosine/sine of width head_dim / 2): pair i of position p has the angle
// p * theta^(-2i/D).
//
// 2-D (vision page, _rope_frequencies: adjacent-pair 2-D frequencies of one
// row-major patch grid): the first D/4 pairs of patch (y, x) take the 1-D
// angles of a D/2-wide head at coordinate y, the last D/4 pairs those at x.
//
// One thread per (position, pair); each entry is rope_entry's (inverse
// frequency and cosine/sine in double, rounded once to binary32; the angle
// the binary32 product of the coordinate and that frequency).
#include "kernels.hpp"

namespace muse {

__global__ __launch_bounds__(256) void rope_table_kernel(RopeTableArgs a) {
  const int half = a.head_dim / 2;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)a.n_pos * half) return;
  const int p = (int)(idx / half);
  const int i = (int)(idx % half);
  int coord = p, j = i, width = a.head_dim;
  if (a.grid_w > 0) {
    const int quarter = half / 2;
    width = half;
    coord = i < quarter ? p / a.grid_w : p % a.grid_w;
    j = i < quarter ? i : i - quarter;
  }
  float c, s;
  rope_entry(a.theta, j, width, coord, c, s);
  a.cos_out[idx] = c;
  a.sin_out[idx] = s;
}

hipError_t launch_rope_table(const RopeTableArgs &a, hipStream_t stream) {
  const int64_t n = (int64_t)a.n_pos * (a.head_dim / 2);
  if (n == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace muse
