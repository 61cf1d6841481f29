// Causal GQA flash attention forward on bf16 MFMA (gfx950), optionally fused
// with the Q norm/RoPE prologue and the output norm/gate epilogue.
//
// Semantics: layers page, MuseSparkAttention (scaling = head_dim^-0.5, KV
// heads repeated to the query-head count, per-layer sliding window), model
// page _causal_mask (window = number of visible causal keys including the
// query), packed documents attend only inside themselves; _qk_norm_rope_core
// and _output_norm_gate_core for the fused prologue/epilogue.
//
// Work item: (row/segment, kv head, head chunk, block of 32*TB query tokens).
// The workgroup holds HPW query heads of one KV group x TB sub-blocks of 32
// tokens: one wave per (head, sub-block).  K and V tiles of BN = 64 keys are
// staged once in LDS and read by every wave of the group.
//
// Layout in registers (v_mfma_f32_32x32x16_bf16, 64 lanes): each wave computes
// S^T = K Q^T, so lane l owns query column n = l % 32 and key rows
// 8*(i/4) + 4*(l/32) + i%4 of each 32-key tile.  The row max therefore needs
// one cross-lane exchange (lanes l, l^32), the row sum none until the end, and
// the probabilities P^T land directly in the B-operand layout of
// O^T += V^T P^T.  V is written to LDS transposed ([d][key]) with keys
// permuted so each lane's 8 keys of a k-step are one 16-byte read.
//
// Tiles are visited from the diagonal downwards; tiles no query of the
// workgroup can see are never loaded, tiles every query of a wave sees skip
// the element mask.
#include <cmath>

#include "device_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int BN = 64;         // keys per tile
constexpr int kMaxWaves = 8;

// Position of key `key` (0..BN-1) inside a transposed V row: within each
// 16-key step, swap bits 2 and 3 so lane group g's keys {4g..4g+3, 8+4g..8+4g+3}
// sit contiguously at [8g, 8g+8).
__device__ __forceinline__ int vt_pos(int key) {
  const int kl = key & 15;
  return (key & ~15) | (((kl >> 2) & 1) << 3) | ((kl >> 3) << 2) | (kl & 3);
}

__device__ __forceinline__ uint32_t word_of(const uint4 &v, int w) {
  return w == 0 ? v.x : (w == 1 ? v.y : (w == 2 ? v.z : v.w));
}

template <int D, bool FUSED>
__global__ __launch_bounds__(64 * kMaxWaves) void attn_fwd_kernel(AttnArgs a) {
  constexpr int KS = D / 16;   // QK^T k-steps
  constexpr int DT = D / 32;   // O^T row tiles
  constexpr int MT = BN / 32;  // S^T row tiles
  constexpr int KK = BN / 16;  // PV k-steps
  constexpr int KSTR = D + 8;  // LDS row stride of the K tile (elements)
  constexpr int VSTR = BN + 8; // LDS row stride of the V^T tile
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VSTR];

  const int tid = threadIdx.x;
  const int nthreads = blockDim.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // ---- work item (q blocks in descending order: longest first)
  const int per_qb = a.lay.num_segments * a.hkv * a.head_chunks;
  const int b = blockIdx.x;
  const int qb = a.q_blocks - 1 - b / per_qb;
  int rest = b % per_qb;
  const int hc = rest % a.head_chunks;
  rest /= a.head_chunks;
  const int kvh = rest % a.hkv;
  const int seg = rest / a.hkv;

  int s0, L;
  if (a.lay.cu_seqlens) {
    const int T = a.lay.n_tokens;
    int c0 = a.lay.cu_seqlens[seg];
    int c1 = a.lay.cu_seqlens[seg + 1];
    c0 = min(max(c0, 0), T);
    c1 = min(max(c1, c0), T);
    s0 = c0;
    L = c1 - c0;
  } else {
    s0 = seg * a.lay.seqlen;
    L = a.lay.seqlen;
  }
  const int BM = 32 * a.tok_blocks;
  const int q0 = qb * BM;
  if (q0 >= L) return;
  const int q1 = min(q0 + BM, L);

  const int hl = wave / a.tok_blocks;
  const int tb = wave % a.tok_blocks;
  const int head = kvh * a.group + hc * a.heads_per_wg + hl;
  const int q0w = q0 + tb * 32;
  const int q1w = min(q0w + 32, L);
  const bool wave_active = q0w < L;
  const int qpos = q0w + n;
  const bool qvalid = qpos < L;
  const int64_t qrow = ((int64_t)(s0 + (qvalid ? qpos : 0)) * a.hq + head) * D;

  // ---- Q fragment: B operand of S^T = K Q^T; lane holds d = 16 ks + 8 g + [0, 8)
  bf16x8 qf[KS];
  {
    uint4 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      raw[ks] = qvalid ? *reinterpret_cast<const uint4 *>(a.q + qrow + ks * 16 + g * 8)
                       : make_uint4(0, 0, 0, 0);
    if constexpr (FUSED) {
      float x[KS][8];
      float all[2 * KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        unpack8(raw[ks], x[ks]);
        const float own = chunk_sumsq<8>(x[ks]);
        const float other = __shfl_xor(own, 32);
        all[2 * ks] = g ? other : own;       // chunk index 2 ks + g holds d = 16 ks + 8 g
        all[2 * ks + 1] = g ? own : other;
      }
      const float rstd = rms_rstd(tree_sum(all), 1.0f / (float)D, a.eps);
      int p = 0;
      if (a.use_rope) {
        p = a.lay.position_ids ? a.lay.position_ids[s0 + (qvalid ? qpos : 0)] : (qvalid ? qpos : 0);
        p = p < 0 ? 0 : (p >= a.n_pos ? a.n_pos - 1 : p);
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 16 + g * 8;
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = a.q_gain ? a.gain_center + a.q_gain[d0 + e] : 1.0f;
        float cs[4] = {1.f, 1.f, 1.f, 1.f}, sn[4] = {0.f, 0.f, 0.f, 0.f};
        if (a.use_rope) {
          const float4 cv = *reinterpret_cast<const float4 *>(a.cos_tab + (int64_t)p * (D / 2) + d0 / 2);
          const float4 sv = *reinterpret_cast<const float4 *>(a.sin_tab + (int64_t)p * (D / 2) + d0 / 2);
          cs[0] = cv.x; cs[1] = cv.y; cs[2] = cv.z; cs[3] = cv.w;
          sn[0] = sv.x; sn[1] = sv.y; sn[2] = sv.z; sn[3] = sv.w;
        }
        float y[8];
        qk_chunk(x[ks], w, rstd, a.query_scale != 1.0f, a.query_scale, a.use_rope != 0, cs, sn, y);
        qf[ks] = __builtin_bit_cast(bf16x8, pack8(y));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
    }
  }

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;
  float l_run = 0.0f;

  const int W = a.window;
  const int lo = W > 0 ? max(0, q0 - W + 1) : 0;
  const int kt_lo = lo / BN;
  const int kt_hi = (q1 - 1) / BN;
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const uint16_t *kbase = a.k + ((int64_t)s0 * a.hkv + kvh) * D;
  const uint16_t *vbase = a.v + ((int64_t)s0 * a.hkv + kvh) * D;

  for (int kt = kt_hi; kt >= kt_lo; --kt) {
    const int k0 = kt * BN;
    __syncthreads();  // every wave is done with the previous tile
    for (int u = tid; u < BN * (D / 8); u += nthreads) {
      const int row = u / (D / 8);
      const int ch = u % (D / 8);
      uint4 val = make_uint4(0, 0, 0, 0);
      if (k0 + row < L) val = *reinterpret_cast<const uint4 *>(kbase + (int64_t)(k0 + row) * kv_stride + ch * 8);
      *reinterpret_cast<uint4 *>(&Ks[row * KSTR + ch * 8]) = val;
    }
    for (int u = tid; u < (BN / 4) * (D / 8); u += nthreads) {
      const int qd = u % (BN / 4);
      const int ch = u / (BN / 4);
      uint4 r4[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = qd * 4 + rr;
        r4[rr] = (k0 + key < L) ? *reinterpret_cast<const uint4 *>(vbase + (int64_t)(k0 + key) * kv_stride + ch * 8)
                                : make_uint4(0, 0, 0, 0);
      }
      const int pos = vt_pos(qd * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t w4[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t wd = word_of(r4[rr], e >> 1);
          w4[rr] = (e & 1) ? (wd >> 16) : (wd & 0xffffu);
        }
        uint2 out;
        out.x = w4[0] | (w4[1] << 16);
        out.y = w4[2] | (w4[3] << 16);
        *reinterpret_cast<uint2 *>(&Vt[(ch * 8 + e) * VSTR + pos]) = out;
      }
    }
    __syncthreads();
    if (!wave_active) continue;
    const bool none_visible = (k0 > q1w - 1) || (W > 0 && k0 + BN - 1 <= q0w - W);
    if (none_visible) continue;
    const bool all_visible = (k0 + BN - 1 <= q0w) && (W <= 0 || k0 > q1w - 1 - W);

    f32x16 sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&Ks[(mt * 32 + n) * KSTR + ks * 16 + g * 8]);
        sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sacc[mt], 0, 0, 0);
      }
    }
    if (!all_visible) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kpos = k0 + mt * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          const bool vis = kpos <= qpos && (W <= 0 || kpos > qpos - W);
          if (!vis) sacc[mt][i] = -INFINITY;
        }
      }
    }

    float tmax = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, sacc[mt][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_use) * a.scale_log2);
    const float mc = m_use * a.scale_log2;
    float psum = 0.0f;
    bf16x8 pb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      float pf[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kk >> 1][(kk & 1) * 8 + j], a.scale_log2, -mc));
        psum += pv;
        pf[j] = pv;
      }
      pb[kk] = __builtin_bit_cast(bf16x8, pack8(pf));
    }
    l_run = __builtin_fmaf(l_run, alpha, psum);
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8 *>(&Vt[(dt * 32 + n) * VSTR + kk * 16 + g * 8]);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[kk], oacc[dt], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv_l = 1.0f / l_tot;

  // O^T element i of tile dt: d = 32 dt + 8 (i/4) + 4 g + i%4, rounded to bf16
  // (the attention output's dtype boundary).
  float o[DT][16];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = round_bf16(oacc[dt][i] * inv_l);

  if constexpr (!FUSED) {
    if (qvalid) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          uint2 w;
          w.x = pack_bf16x2(o[dt][i4 * 4 + 0], o[dt][i4 * 4 + 1]);
          w.y = pack_bf16x2(o[dt][i4 * 4 + 2], o[dt][i4 * 4 + 3]);
          *reinterpret_cast<uint2 *>(a.o + qrow + dt * 32 + i4 * 8 + g * 4) = w;
        }
    }
  } else {
    // Output RMSNorm: group partials of 4 elements, pairs of groups form the
    // 8-element chunk c = 4 dt + i4 (lanes g = 0, 1 hold its halves), then the
    // pairwise tree over chunks.
    float s1[DT * 4];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float own = chunk_sumsq<4>(&o[dt][i4 * 4]);
        const float other = __shfl_xor(own, 32);
        s1[dt * 4 + i4] = g ? other + own : own + other;
      }
    const float rstd = rms_rstd(tree_sum(s1), 1.0f / (float)D, a.out_eps);
    if (qvalid) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int64_t off = qrow + dt * 32 + i4 * 8 + g * 4;
          const uint2 gw = *reinterpret_cast<const uint2 *>(a.gate + off);
          uint2 w;
          w.x = pack_bf16x2(gate_elem(o[dt][i4 * 4 + 0], rstd, bf16_lo(gw.x)),
                            gate_elem(o[dt][i4 * 4 + 1], rstd, bf16_hi(gw.x)));
          w.y = pack_bf16x2(gate_elem(o[dt][i4 * 4 + 2], rstd, bf16_lo(gw.y)),
                            gate_elem(o[dt][i4 * 4 + 3], rstd, bf16_hi(gw.y)));
          *reinterpret_cast<uint2 *>(a.o + off) = w;
        }
    }
  }
  if (a.lse && qvalid && g == 0) {
    const float m_fin = (m_run == -INFINITY) ? 0.0f : m_run;
    a.lse[(int64_t)(s0 + qpos) * a.hq + head] =
        __builtin_fmaf(m_fin, a.scaling, __builtin_amdgcn_logf(l_tot) * kLn2);
  }
}

}  // namespace

hipError_t launch_attn_fwd(int head_dim, bool fused, const AttnArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.q_blocks * a.lay.num_segments * a.hkv * a.head_chunks;
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks);
  const dim3 block(64 * a.heads_per_wg * a.tok_blocks);
  if (head_dim == 128) {
    if (fused) hipLaunchKernelGGL((attn_fwd_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (fused) hipLaunchKernelGGL((attn_fwd_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((attn_fwd_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace muse
