// Q/K RMSNorm + zero-centred gain + bf16 cast + query_scale + adjacent-pair
// RoPE (layers page, _qk_norm_rope_core, _rms_norm_core,
// apply_rotary_embedding); without the norm, the rotation of the vision
// attention (vision page, _apply_vision_rope).
//
// HBM-bound.  Each (token, head) row of D bf16 values is spread over D/8
// lanes holding 8 consecutive elements (one 16-byte load); the row's sum of
// squares is a per-lane fma chain followed by a DPP reduction over those
// lanes (no LDS traffic).  Every thread keeps kRowsInFlight rows' loads
// outstanding before it computes.  The first q_blocks blocks take Q rows
// (row r = token * Hq + head), the others K rows, so the tensor, its gain and
// the query scale are uniform per block.
//
// Table mode (TAB): a block's rows are consecutive, so they touch a short
// run of tokens; the block first evaluates the cos/sin rows of those tokens'
// positions (one entry per thread and pass, rope_entry's arithmetic as in the
// table kernel, with the inverse frequencies computed once per block),
// keeps them in LDS for its own rotations and writes them to the table, so
// the table costs no launch of its own.  Tokens that share a position write
// identical bits.
#include "device_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsInFlight = 2;

// ROPE: 0 no rotation, 1 FP32 rotation (upcast_rope), 2 rotation in the Q/K
// dtype; QS: query_scale != 1 (K rows then take the exact identity scale 1,
// which leaves their bf16 values unchanged); NORM: false skips the RMSNorm
// and gain (the vision attention rotates un-normalised Q/K); TAB: table mode
// (ROPE != 0).
template <int D, int ROPE, bool QS, bool NORM, bool TAB>
__global__ __launch_bounds__(kThreads) void qk_norm_rope_kernel(QkNormArgs a) {
  constexpr int LPR = D / 8;               // lanes per row
  constexpr int RPP = kThreads / LPR;      // rows per pass of the block
  constexpr int RPB = RPP * kRowsInFlight; // rows of a block (consecutive)
  constexpr int HALF = D / 2;
  static_assert(LPR == 8 || LPR == 16, "row_sum covers 8 or 16 lanes");
  static_assert(!TAB || ROPE != 0, "table mode rotates");
  // cos then sin rows of the block's tokens (at most RPB tokens), and the
  // inverse frequencies they share
  __shared__ __attribute__((aligned(16))) float tab[TAB ? 2 * RPB * HALF : 1];
  __shared__ float inv_freq[TAB ? HALF : 1];
  const int c = threadIdx.x % LPR;         // chunk: elements [8c, 8c+8)
  const int rsub = threadIdx.x / LPR;

  const bool is_q = (int)blockIdx.x < a.q_blocks;
  const int blk = is_q ? (int)blockIdx.x : (int)blockIdx.x - a.q_blocks;
  const int nrows = is_q ? a.q_rows : a.k_rows;
  const uint16_t *src = is_q ? a.q : a.k;
  uint16_t *dst = is_q ? a.q_out : a.k_out;
  float *rs = is_q ? a.q_rstd : a.k_rstd;
  const float *gain = is_q ? a.q_gain : a.k_gain;
  const FastDiv hdiv = is_q ? a.hq_div : a.hkv_div;
  const float qs = is_q ? a.query_scale : 1.0f;
  const int base = blk * RPP * kRowsInFlight + rsub;

  uint4 xin[kRowsInFlight];
#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int r = base + j * RPP;
    xin[j] = r < nrows ? *reinterpret_cast<const uint4 *>(src + (int64_t)r * D + c * 8) : make_uint4(0, 0, 0, 0);
  }

  // effective gains of this lane's 8 columns
  float w[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
  if (NORM && gain) {
    const float4 g0 = *reinterpret_cast<const float4 *>(gain + c * 8);
    const float4 g1 = *reinterpret_cast<const float4 *>(gain + c * 8 + 4);
    w[0] = a.gain_center + g0.x; w[1] = a.gain_center + g0.y;
    w[2] = a.gain_center + g0.z; w[3] = a.gain_center + g0.w;
    w[4] = a.gain_center + g1.x; w[5] = a.gain_center + g1.y;
    w[6] = a.gain_center + g1.z; w[7] = a.gain_center + g1.w;
  }

  // table mode: the cos/sin rows of tokens t_first .. t_last (every row of
  // this block has r < nrows; blocks are sized to start below nrows)
  int t_first = 0;
  if constexpr (TAB) {
    const int r0 = blk * RPB;
    const int r1 = min(r0 + RPB, nrows) - 1;
    t_first = (int)hdiv.div((uint32_t)r0);
    const int n = ((int)hdiv.div((uint32_t)r1) - t_first + 1) * HALF;
    for (int i = threadIdx.x; i < HALF; i += kThreads) inv_freq[i] = rope_inv_freq(a.theta, i, D);
    const PosCursor pc = pos_cursor(a.lay, t_first);
    __syncthreads();
    for (int idx = threadIdx.x; idx < n; idx += kThreads) {
      const int t = t_first + idx / HALF;
      const int i = idx % HALF;
      const int p = rope_position(a.lay, pc, t, a.n_pos);
      float cv, sv;
      rope_cos_sin(p, inv_freq[i], cv, sv);   // = rope_entry(a.theta, i, D, p, ...)
      tab[idx] = cv;
      tab[RPB * HALF + idx] = sv;
      a.cos_out[(int64_t)p * HALF + i] = cv;
      a.sin_out[(int64_t)p * HALF + i] = sv;
    }
    __syncthreads();
  }

  // RoPE positions of this thread's rows; in table mode the row's token
  // instead (its LDS row).  The block's rows are consecutive, so a packed
  // layout's segment search runs once per block (pos_cursor).
  int pos[kRowsInFlight];
  if constexpr (TAB) {
#pragma unroll
    for (int j = 0; j < kRowsInFlight; ++j)
      pos[j] = (int)hdiv.div((uint32_t)min(base + j * RPP, nrows - 1)) - t_first;
  } else if constexpr (ROPE != 0) {
    const PosCursor pc = pos_cursor(a.lay, (int)hdiv.div((uint32_t)(blk * RPB)));
#pragma unroll
    for (int j = 0; j < kRowsInFlight; ++j)
      pos[j] = rope_position(a.lay, pc, (int)hdiv.div((uint32_t)min(base + j * RPP, nrows - 1)), a.n_pos);
  }

#pragma unroll
  for (int j = 0; j < kRowsInFlight; ++j) {
    const int r = base + j * RPP;
    float rstd = 1.0f;
    if constexpr (NORM) {
      float x[8];
      unpack8(xin[j], x);
      const float ss = row_sum<LPR>(chunk_sumsq<8>(x));   // every lane takes part
      rstd = rms_rstd(ss, 1.0f / (float)D, a.eps);
    }
    if (r >= nrows) continue;
    float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (ROPE != 0) {
      const float *ct = TAB ? tab + pos[j] * HALF : a.cos_tab + (int64_t)pos[j] * HALF;
      const float *st = TAB ? tab + RPB * HALF + pos[j] * HALF : a.sin_tab + (int64_t)pos[j] * HALF;
      const float4 cv = *reinterpret_cast<const float4 *>(ct + c * 4);
      const float4 sv = *reinterpret_cast<const float4 *>(st + c * 4);
      cs[0] = cv.x; cs[1] = cv.y; cs[2] = cv.z; cs[3] = cv.w;
      sn[0] = sv.x; sn[1] = sv.y; sn[2] = sv.z; sn[3] = sv.w;
    }
    uint4 y;
    if constexpr (NORM) {
      float x[8];
      unpack8(xin[j], x);
      y = qk_chunk(x, w, rstd, QS, qs, ROPE != 0, cs, sn, ROPE == 2);
    } else {
      y = scale_rope_chunk(xin[j], QS, qs, ROPE != 0, cs, sn, ROPE == 2);
    }
    *reinterpret_cast<uint4 *>(dst + (int64_t)r * D + c * 8) = y;
    if (NORM && rs && c == 0) rs[r] = rstd;
  }
}

template <int D, int ROPE, bool NORM, bool TAB>
void launch_t(const QkNormArgs &a, dim3 grid, hipStream_t stream) {
  if (a.q_rows > 0 && a.query_scale != 1.0f)
    hipLaunchKernelGGL((qk_norm_rope_kernel<D, ROPE, true, NORM, TAB>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((qk_norm_rope_kernel<D, ROPE, false, NORM, TAB>), grid, dim3(kThreads), 0, stream, a);
}

template <int D, int ROPE, bool NORM>
void launch_r(const QkNormArgs &a, dim3 grid, hipStream_t stream) {
  if constexpr (ROPE != 0) {
    if (a.cos_out) {
      launch_t<D, ROPE, NORM, true>(a, grid, stream);
      return;
    }
  }
  launch_t<D, ROPE, NORM, false>(a, grid, stream);
}

template <int D, bool NORM>
void launch_n(const QkNormArgs &a, dim3 grid, hipStream_t stream) {
  if (!a.use_rope) launch_r<D, 0, NORM>(a, grid, stream);
  else if (a.rope_v2) launch_r<D, 2, NORM>(a, grid, stream);
  else launch_r<D, 1, NORM>(a, grid, stream);
}

template <int D>
void launch_d(const QkNormArgs &a, dim3 grid, hipStream_t stream) {
  if (a.skip_norm) launch_n<D, false>(a, grid, stream);
  else launch_n<D, true>(a, grid, stream);
}

}  // namespace

hipError_t launch_qk_norm_rope(int head_dim, const QkNormArgs &args, hipStream_t stream) {
  const int lpr = head_dim / 8;
  const int64_t rows_per_block = (int64_t)(kThreads / lpr) * kRowsInFlight;
  QkNormArgs a = args;
  a.q_blocks = (int)((a.q_rows + rows_per_block - 1) / rows_per_block);
  const int64_t blocks = a.q_blocks + (a.k_rows + rows_per_block - 1) / rows_per_block;
  if (blocks == 0) return hipSuccess;
  if (head_dim == 128) launch_d<128>(a, dim3((unsigned)blocks), stream);
  else launch_d<64>(a, dim3((unsigned)blocks), stream);
  return hipGetLastError();
}

}  // namespace muse
