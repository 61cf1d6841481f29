// Backward of the causal/windowed/bidirectional GQA attention on bf16 MFMA
// (gfx950): the chain rule through layers page, MuseSparkAttention's softmax
// attention (scaling = head_dim^-0.5, KV heads repeated to the query-head
// count, model page _causal_mask), given the forward's LSE and
// delta = rowsum(dO * O):
//   P = exp(scaling q k^T - lse),  dP = dO v^T,  dS = P (dP - delta),
//   dq = scaling dS k,  dk = scaling dS^T q,  dv = P^T dO
// with dk and dv summed over the query heads of each KV head.
//
// Two kernels, no atomics, so every result is deterministic:
//
// dQ kernel -- the forward's work shape: a workgroup of 4 waves owns 128
//   (token, head) query columns of one KV group; K and V tiles of 64 keys
//   stream through LDS by DMA (double-buffered).  Per 32-key half a wave
//   forms S^T = K Q^T and dP^T = V dO^T (lane l owns query column l % 32, so
//   its LSE and delta are one register each), P^T and dS^T in registers, and
//   dQ^T += K^T dS^T with dS^T in the B-operand layout and K^T read by
//   ds_read_b64_tr_b16 -- the forward's O^T += V^T P^T step.
//
// dK/dV kernel -- keys stationary: a workgroup owns 128 keys of one KV head,
//   32 per wave, held as B fragments (K and V) in registers; Q and dO tiles
//   of 64 tokens of one query head stream through LDS together with their
//   LSE and delta rows, the group's heads of one token tile in turn, the
//   token tiles in an order shared by neighbouring key blocks (so blocks
//   resident together on an XCD read each tile from one L2 fill).  Per 32-query half a
//   wave forms S = Q K^T and dP = dO V^T (lane l owns key column l % 32),
//   then dV^T += dO^T P and dK^T += Q^T dS with P and dS in the B-operand
//   layout and dO^T, Q^T read transposed from LDS.
//
// At D = 128 dK/dV runs as attn_bwd_dkdv_rs_kernel below: the
// same steps split between two waves per SIMD, one forming S, P and dV (and
// issuing the tile DMA), the other dP, dS and dK, with P handed over through
// LDS.
//
// Tiles are read both row-wise and transposed, so their 16-byte chunks use
// the swizzle that keeps both patterns free of bank conflicts (Tile::swz_kv).
// Masked scores get P = 0 explicitly (a query whose every key is padding has
// lse = -inf).  Tiles no wave of the workgroup can see are never loaded.
#include <cmath>
#include <type_traits>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int BN = 64;        // keys (dQ) or queries (dK/dV) per LDS tile
constexpr int NW = 4;         // waves per workgroup
constexpr int COLS = 32 * NW; // dQ: query columns per workgroup; dK/dV: keys per workgroup
static_assert(BN == 64, "Tile<D> holds 64-row tiles");

// Row-fragment read addresses (A operand: lane row n, chunk 2 ks + g) and the
// two transposed-read address sets (rows 4 g + (r >> 2) and 8 more) of a
// swz_kv tile.
template <int D>
struct TileAddr {
  int row[D / 16];
  int tr_lo[D / 32], tr_hi[D / 32];
  __device__ __forceinline__ void init(int lane) {
    using T = Tile<D>;
    constexpr int RB = T::ROW_BYTES;
    const int n = lane & 31, g = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) row[ks] = n * RB + (((2 * ks + g) ^ T::swz_kv(n)) << 4);
    const int r = lane & 15, q = (lane >> 4) & 1;
    const int r0 = 4 * g + (r >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int ch = dt * 4 + 2 * q + ((r & 3) >> 1);
      tr_lo[dt] = r0 * RB + ((ch ^ T::swz_kv(r0)) << 4) + (r & 1) * 8;
      tr_hi[dt] = (r0 + 8) * RB + ((ch ^ T::swz_kv(r0 + 8)) << 4) + (r & 1) * 8;
    }
  }
};

// A fragments of 32 rows x D from a tile (rows base .. base + 31), then
// acc += A B over the D/16 k-steps.
template <int D>
__device__ __forceinline__ f32x16 rows_times(const lds_char *tile, const TileAddr<D> &ad, int base_bytes,
                                             const bf16x8 (&b)[D / 16]) {
  constexpr int KS = D / 16;
  bf16x8 af[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    af[ks] = *(const __attribute__((address_space(3))) bf16x8 *)(tile + ad.row[ks] + base_bytes);
  __builtin_amdgcn_sched_barrier(0);
  f32x16 acc = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], b[ks], acc, 0, 0, 0);
  return acc;
}

// acc[dt] += (tile rows base .. base + 31)^T (D x 32) times the B fragments
// b0 (rows base .. base + 15) and b1 (base + 16 .. base + 31).
template <int D>
__device__ __forceinline__ void tr_times(const lds_char *tile, const TileAddr<D> &ad, int base_row,
                                         const bf16x8 &b0, const bf16x8 &b1, f32x16 (&acc)[D / 32]) {
  constexpr int RB = Tile<D>::ROW_BYTES;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      const int r0 = (base_row + 16 * kk) * RB;
      const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4 *)(tile + ad.tr_lo[dt] + r0));
      const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (__attribute__((address_space(3))) bf16x4 *)(tile + ad.tr_hi[dt] + r0));
      const bf16x8 af = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, kk ? b1 : b0, acc[dt], 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void pack16(const float (&x)[16], bf16x8 &b0, bf16x8 &b1) {
  uint4 lo, hi;
  lo.x = pack_bf16x2(x[0], x[1]);   lo.y = pack_bf16x2(x[2], x[3]);
  lo.z = pack_bf16x2(x[4], x[5]);   lo.w = pack_bf16x2(x[6], x[7]);
  hi.x = pack_bf16x2(x[8], x[9]);   hi.y = pack_bf16x2(x[10], x[11]);
  hi.z = pack_bf16x2(x[12], x[13]); hi.w = pack_bf16x2(x[14], x[15]);
  b0 = __builtin_bit_cast(bf16x8, lo);
  b1 = __builtin_bit_cast(bf16x8, hi);
}

// Store a D x 32 accumulator (element i of tile dt: d = 32 dt + 8 (i/4) +
// 4 g + i%4, column = this lane's) scaled by s, as bf16, to row ptr.
template <int D>
__device__ __forceinline__ void store_cols(uint16_t *ptr, const f32x16 (&acc)[D / 32], float s, int g,
                                           bool zero) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      uint2 w;
      w.x = zero ? 0u : pack_bf16x2(acc[dt][i4 * 4 + 0] * s, acc[dt][i4 * 4 + 1] * s);
      w.y = zero ? 0u : pack_bf16x2(acc[dt][i4 * 4 + 2] * s, acc[dt][i4 * 4 + 3] * s);
      *reinterpret_cast<uint2 *>(ptr + dt * 32 + i4 * 8 + g * 4) = w;
    }
}

// Segment bounds of segment `seg` (BSHD row or packed document).
__device__ __forceinline__ void segment_bounds(const TokenLayout &l, int seg, int &s0, int &L) {
  if (l.cu_seqlens) {
    const int T_ = l.n_tokens;
    int c0 = l.cu_seqlens[seg];
    int c1 = l.cu_seqlens[seg + 1];
    c0 = min(max(c0, 0), T_);
    c1 = min(max(c1, c0), T_);
    s0 = c0;
    L = c1 - c0;
  } else {
    s0 = seg * l.seqlen;
    L = l.seqlen;
  }
}

// ===========================================================================
template <int D, bool PAD>
__global__ __launch_bounds__(64 * NW, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  using T = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DMA_PER_WAVE = T::TILE_BYTES / 1024 / NW;
  __shared__ __attribute__((aligned(16))) char lds_k0[T::TILE_BYTES], lds_v0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_k1[T::TILE_BYTES], lds_v1[T::TILE_BYTES];
  auto kbuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_k1 : lds_k0); };
  auto vbuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_v1 : lds_v0); };

  const int tid = threadIdx.x;
  // wave-uniform, so the per-wave work tests below are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // work item: as the forward (segment-major, longest query blocks first,
  // part, kv head)
  const int heads_items = a.hkv * a.head_chunks;
  const int per_seg = a.q_blocks * a.dq_parts * heads_items;
  const int b = blockIdx.x;
  const int seg = b / per_seg;
  int rest = b % per_seg;
  const int qb = a.q_blocks - 1 - rest / (a.dq_parts * heads_items);
  rest %= a.dq_parts * heads_items;
  const int part = rest / heads_items;
  rest %= a.hkv * a.head_chunks;
  const int hc = rest % a.head_chunks;
  const int kvh = rest / a.head_chunks;
  int s0, L;
  segment_bounds(a.lay, seg, s0, L);
  const int HPW = a.heads_per_wg;
  const int BMT = a.tok_per_wg;
  const int q0 = qb * BMT;
  if (q0 >= L) return;
  const int q1 = min(q0 + BMT, L);

  const int col = wave * 32 + n;
  const int ct = col / HPW;
  const int head = kvh * a.group + hc * HPW + (col - ct * HPW);
  const int qpos = q0 + ct;
  const bool qvalid = ct < BMT && qpos < L;
  const int wcol0 = wave * 32;
  const int wcol1 = min(wcol0 + 31, BMT * HPW - 1);
  const bool wave_active = wcol0 < BMT * HPW && q0 + wcol0 / HPW < L;
  const int q0w = q0 + wcol0 / HPW;
  const int q1w = min(q0 + wcol1 / HPW + 1, q1);
  const int64_t lrow = (int64_t)(s0 + (qvalid ? qpos : 0)) * a.hq + (qvalid ? head : 0);
  const int64_t qrow = lrow * D;

  // stationary B fragments: q_hat and dO of this lane's column (d = 16 ks + 8 g + [0, 8))
  bf16x8 qf[KS], dof[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // qrow always addresses a real row (row 0 of the segment for an idle
    // column): load, then select against a constant (a select between two
    // addresses would put the zero in scratch and make both loads flat)
    const uint4 rq = *reinterpret_cast<const uint4 *>(a.q + qrow + ks * 16 + g * 8);
    const uint4 ro = *reinterpret_cast<const uint4 *>(a.d_o + qrow + ks * 16 + g * 8);
    qf[ks] = __builtin_bit_cast(bf16x8, qvalid ? rq : make_uint4(0, 0, 0, 0));
    dof[ks] = __builtin_bit_cast(bf16x8, qvalid ? ro : make_uint4(0, 0, 0, 0));
  }
  const float lse2 = qvalid ? a.lse[lrow] * kLog2e : 0.0f;
  const float dlt = qvalid ? a.delta[lrow] : 0.0f;

  const int64_t kv_stride = (int64_t)a.hkv * D;
  const uint16_t *kbase = a.k + ((int64_t)s0 * a.hkv + kvh) * D;
  const uint16_t *vbase = a.v + ((int64_t)s0 * a.hkv + kvh) * D;
  int off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int slot = (wave * DMA_PER_WAVE + i) * 64 + lane;
    const int row = slot / T::CHUNKS;
    const int pch = slot % T::CHUNKS;
    off[i] = (row * (int)kv_stride + (pch ^ T::swz_kv(row)) * 8) * 2;
  }
  TileAddr<D> ad;
  ad.init(lane);

  const uint8_t *kvalid = a.key_valid + s0;   // read only when PAD
  int vbyte = 1;
  uint64_t kmask = ~0ull;
  auto take_mask = [&]() __attribute__((always_inline)) {
    if constexpr (PAD) kmask = __ballot(vbyte != 0);
  };

  auto issue_dma = [&](int kt, int buf) {
    const int k0 = kt * BN;
    if constexpr (PAD) vbyte = k0 + lane < L ? (int)kvalid[k0 + lane] : 0;
    lds_char *kdst = kbuf(buf) + wave * DMA_PER_WAVE * 1024;
    lds_char *vdst = vbuf(buf) + wave * DMA_PER_WAVE * 1024;
    const int valid_bytes = ((min(L - k0, BN) - 1) * (int)kv_stride + D) * 2;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)k0 * kv_stride, valid_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)k0 * kv_stride, valid_bytes);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      dma16(kr, off[i], kdst + i * 1024);
      dma16(vr, off[i], vdst + i * 1024);
    }
  };

  f32x16 dqv[1][DT];
  f32x16 (&dqacc)[DT] = dqv[0];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dqacc[dt] = f32x16{};

  const int W = a.window;
  const bool bidir = a.bidirectional != 0;
  const float c2 = a.scale_log2;
  constexpr int RB = T::ROW_BYTES;
  // causal: qpos - kp in [0, W) (or [0, inf) without a window); bidirectional:
  // L - 1 - kp in [0, L), i.e. kp inside the segment
  const int mask_base = bidir ? L - 1 : qpos;
  const uint32_t mask_lim = bidir ? (uint32_t)L : (W > 0 ? (uint32_t)W : 0x7FFFFFFFu);

  auto compute = [&](int kt, int BUF) __attribute__((always_inline)) {
    const int k0 = kt * BN;
    const bool none_visible = !wave_active || (!bidir && ((k0 > q1w - 1) || (W > 0 && k0 + BN - 1 <= q0w - W)));
    if (none_visible) return;
    const bool all_visible = bidir ? k0 + BN <= L : (k0 + BN - 1 <= q0w) && (W <= 0 || k0 > q1w - 1 - W);
    const bool padded = PAD && kmask != ~0ull;
    const lds_char *Kt = kbuf(BUF);
    const lds_char *Vt = vbuf(BUF);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const f32x16 s = rows_times<D>(Kt, ad, half * 32 * RB, qf);
      const f32x16 dp = rows_times<D>(Vt, ad, half * 32 * RB, dof);
      float p[16], ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse2));
      if (!all_visible || padded) {
        // key kp is visible iff (unsigned)(mask_base - kp) < mask_lim (one compare, no branches)
        const uint32_t kbits = padded ? (uint32_t)(kmask >> (half * 32 + g * 4)) : ~0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kp = k0 + half * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
          const bool vis = ((uint32_t)(mask_base - kp) < mask_lim) & ((kbits >> ((i >> 2) * 8 + (i & 3))) & 1u);
          p[i] = vis ? p[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp[i] - dlt);
      bf16x8 d0, d1;
      pack16(ds, d0, d1);
      tr_times<D>(Kt, ad, half * 32, d0, d1, dqacc);
    }
  };

  const int lo = W > 0 && !bidir ? max(0, q0 - W + 1) : 0;
  const int kt_lo = lo / BN;
  const int kt_hi = ((bidir ? L : q1) - 1) / BN;
  const int ntiles = kt_hi - kt_lo + 1;
  // split: this part takes tiles kt_hi - it for it in [it0, it1) (the last
  // launched part takes any remainder)
  const int span = a.dq_parts > 1 ? a.dq_span : ntiles;
  const int nparts = min((ntiles + span - 1) / span, a.dq_parts);
  if (part >= nparts) return;
  const int it0 = part * span;
  const int it1 = part == nparts - 1 ? ntiles : it0 + span;

  issue_dma(kt_hi - it0, 0);
  vmem_wait_all();
  __syncthreads();
  for (int it = it0;;) {
    take_mask();
    if (it + 1 < it1) issue_dma(kt_hi - it - 1, 1);
    compute(kt_hi - it, 0);
    vmem_wait_all();
    __syncthreads();
    if (++it >= it1) break;
    take_mask();
    if (it + 1 < it1) issue_dma(kt_hi - it - 1, 0);
    compute(kt_hi - it, 1);
    vmem_wait_all();
    __syncthreads();
    if (++it >= it1) break;
  }
  if (!wave_active) return;
  if (nparts > 1) {
    const int64_t item = (((int64_t)seg * a.q_blocks + qb) * a.hkv + kvh) * a.head_chunks + hc;
    constexpr int SLOT = DT * 16 * 64;
    if (!split_sum(dqv, a.part_acc + (item * a.dq_parts * NW + wave) * SLOT, (int64_t)NW * SLOT, part, nparts,
                   a.part_cnt + item * NW + wave))
      return;
  }
  if (!qvalid) return;
  store_cols<D>(a.dq + qrow, dqacc, a.scaling, g, false);
}

// ===========================================================================
// One wave holds both accumulators and both fragment sets: at D = 64 two
// waves fit a SIMD; D = 128 (2 x 64 accumulator and 2 x 32 fragment registers)
// runs as the role-split kernel below instead.
template <int D, bool PAD>
__global__ __launch_bounds__(64 * NW, D == 128 ? 1 : 2) void attn_bwd_dkdv_kernel(AttnBwdArgs a) {
  using T = Tile<D>;
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int DMA_PER_WAVE = T::TILE_BYTES / 1024 / NW;
  constexpr int RB = T::ROW_BYTES;
  __shared__ __attribute__((aligned(16))) char lds_q0[T::TILE_BYTES], lds_o0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_q1[T::TILE_BYTES], lds_o1[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_l0[BN], lds_d0[BN], lds_l1[BN], lds_d1[BN];
  auto qbuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_q1 : lds_q0); };
  auto obuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_o1 : lds_o0); };
  auto lbuf = [&](int buf) __attribute__((always_inline)) {
    return (__attribute__((address_space(3))) float *)(buf ? lds_l1 : lds_l0);
  };
  auto dbuf = [&](int buf) __attribute__((always_inline)) {
    return (__attribute__((address_space(3))) float *)(buf ? lds_d1 : lds_d0);
  };

  const int tid = threadIdx.x;
  // wave-uniform, so the per-wave work tests below are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // work item: segment-major, key blocks ascending (the most queries first),
  // then kv head -- consecutive workgroups take consecutive kv heads, so each
  // XCD keeps one head group's Q/dO rows in its L2.
  const int per_seg = a.k_blocks * a.dkv_parts * a.hkv;
  const int b = blockIdx.x;
  const int seg = b / per_seg;
  int rest = b % per_seg;
  const int kb = rest / (a.dkv_parts * a.hkv);
  rest %= a.dkv_parts * a.hkv;
  const int part = rest / a.hkv;
  const int kvh = rest % a.hkv;
  int s0, L;
  segment_bounds(a.lay, seg, s0, L);
  const int kb0 = kb * COLS;
  if (kb0 >= L) return;
  const int kw0 = kb0 + wave * 32;
  const int kw1 = min(kw0 + 31, L - 1);
  const bool wave_active = kw0 < L;
  const int key = kw0 + n;
  const bool kin = key < L;
  const int64_t krow = ((int64_t)(s0 + (kin ? key : 0)) * a.hkv + kvh) * D;

  bf16x8 kf[KS], vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    // krow always addresses a real row (row 0 of the segment past its end)
    const uint4 rk = *reinterpret_cast<const uint4 *>(a.k + krow + ks * 16 + g * 8);
    const uint4 rv = *reinterpret_cast<const uint4 *>(a.v + krow + ks * 16 + g * 8);
    kf[ks] = __builtin_bit_cast(bf16x8, kin ? rk : make_uint4(0, 0, 0, 0));
    vf[ks] = __builtin_bit_cast(bf16x8, kin ? rv : make_uint4(0, 0, 0, 0));
  }
  bool kpad = false;
  if constexpr (PAD) kpad = kin && a.key_valid[s0 + key] == 0;

  const int W = a.window;
  const bool bidir = a.bidirectional != 0;
  const float c2 = a.scale_log2;
  // causal: qp - key in [0, min(W, L - key)) -- the query is at or after the
  // key, inside the window and inside the segment; bidirectional: qp in [0, L)
  const int mask_base = bidir ? 0 : key;
  const int lim_c = W > 0 ? min(W, L - key) : L - key;
  const uint32_t mask_lim = bidir ? (uint32_t)L : (uint32_t)max(lim_c, 0);
  // queries that can see a key of this block
  const int qlo = bidir ? 0 : kb0;
  const int qhi = bidir || W <= 0 ? L - 1 : min(L - 1, min(kb0 + COLS - 1, L - 1) + W - 1);
  const int qt_lo = qlo / BN;
  const int qt_hi = qhi / BN;
  const int nqt = qt_hi - qt_lo + 1;
  const int ntiles = nqt * a.group;
  // Visiting order of the query tiles.  Workgroups of neighbouring key blocks
  // run side by side on one XCD; walking their tiles in a common order makes
  // them read the same tile at about the same time, so one L2 fill serves
  // them all.  Without a window every block's tiles end at the segment's
  // last tile: walk down from there.  With a window every block's tiles form
  // a run of the same length R (fewer at the segment's end), which holds one
  // multiple of R: start the walk there, go up and wrap round.  The G heads
  // of a tile are consecutive steps (their rows are adjacent in memory).
  const bool windowed = !bidir && W > 0 && W < L;
  int rot = 0;
  if (windowed) {
    const int R = (COLS - 2 + W) / BN + 1;
    const int s = (qt_lo + R - 1) / R * R;
    rot = s <= qt_hi ? s - qt_lo : 0;
  }
  auto step_tile = [&](int it, int &h) __attribute__((always_inline)) {
    const int ti = it / a.group;
    h = kvh * a.group + (it - ti * a.group);
    if (!windowed) return qt_hi - ti;
    const int x = rot + ti;
    return qt_lo + (x >= nqt ? x - nqt : x);
  };
  // split: this part takes steps [it0, it1) (the last launched part takes any remainder)
  const int span = a.dkv_parts > 1 ? a.dkv_span : ntiles;
  const int nparts = min((ntiles + span - 1) / span, a.dkv_parts);
  if (part >= nparts) return;
  const int it0 = part * span;
  const int it1 = part == nparts - 1 ? ntiles : it0 + span;

  const int64_t q_stride = (int64_t)a.hq * D;
  int off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int slot = (wave * DMA_PER_WAVE + i) * 64 + lane;
    const int row = slot / T::CHUNKS;
    const int pch = slot % T::CHUNKS;
    off[i] = (row * (int)q_stride + (pch ^ T::swz_kv(row)) * 8) * 2;
  }
  TileAddr<D> ad;
  ad.init(lane);

  auto issue_dma = [&](int it, int buf) {
    int h;
    const int t0 = step_tile(it, h) * BN;
    const int rows = min(L - t0, BN);
    const int64_t r0 = (int64_t)(s0 + t0) * a.hq + h;
    const int valid_bytes = ((rows - 1) * (int)q_stride + D) * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + r0 * D, valid_bytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.d_o + r0 * D, valid_bytes);
    lds_char *qdst = qbuf(buf) + wave * DMA_PER_WAVE * 1024;
    lds_char *odst = obuf(buf) + wave * DMA_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      dma16(qr, off[i], qdst + i * 1024);
      dma16(orr, off[i], odst + i * 1024);
    }
    // the tile's LSE and delta rows (rows past the segment read as 0)
    if (wave < 2) {
      const int fbytes = ((rows - 1) * a.hq + 1) * 4;
      const __amdgpu_buffer_rsrc_t fr = make_rsrc((wave ? a.delta : a.lse) + r0, fbytes);
      dma4(fr, lane * a.hq * 4, (lds_char *)(wave ? dbuf(buf) : lbuf(buf)));
    }
  };

  f32x16 dkv[2][DT];
  f32x16 (&dkacc)[DT] = dkv[0];
  f32x16 (&dvacc)[DT] = dkv[1];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkacc[dt] = dvacc[dt] = f32x16{};

  auto compute = [&](int it, int BUF) __attribute__((always_inline)) {
    int h;
    const int t0 = step_tile(it, h) * BN;
    const bool none_visible = !wave_active || (!bidir && (t0 + BN - 1 < kw0 || (W > 0 && t0 > kw1 + W - 1)));
    if (none_visible) return;
    const bool all_visible = t0 + BN <= L && (bidir || (t0 >= kw1 && (W <= 0 || t0 + BN - 1 <= kw0 + W - 1)));
    const lds_char *Qt = qbuf(BUF);
    const lds_char *Ot = obuf(BUF);
    const __attribute__((address_space(3))) float *Lt = lbuf(BUF);
    const __attribute__((address_space(3))) float *Dl = dbuf(BUF);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const f32x16 s = rows_times<D>(Qt, ad, half * 32 * RB, kf);
      const f32x16 dp = rows_times<D>(Ot, ad, half * 32 * RB, vf);
      float p[16], ds[16], dl[16];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)(Lt + half * 32 + 8 * j + 4 * g);
        const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)(Dl + half * 32 + 8 * j + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          p[4 * j + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * j + e], c2, -(l4[e] * kLog2e)));
          dl[4 * j + e] = d4[e];
        }
      }
      if (!all_visible) {
        // query qp sees this lane's key iff (unsigned)(qp - mask_base) < mask_lim
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qp = t0 + half * 32 + (i >> 2) * 8 + 4 * g + (i & 3);
          p[i] = (uint32_t)(qp - mask_base) < mask_lim ? p[i] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) ds[i] = p[i] * (dp[i] - dl[i]);
      bf16x8 p0, p1, d0, d1;
      pack16(p, p0, p1);
      pack16(ds, d0, d1);
      tr_times<D>(Ot, ad, half * 32, p0, p1, dvacc);
      tr_times<D>(Qt, ad, half * 32, d0, d1, dkacc);
    }
  };

  issue_dma(it0, 0);
  vmem_wait_all();
  __syncthreads();
  for (int it = it0;;) {
    if (it + 1 < it1) issue_dma(it + 1, 1);
    compute(it, 0);
    vmem_wait_all();
    __syncthreads();
    if (++it >= it1) break;
    if (it + 1 < it1) issue_dma(it + 1, 0);
    compute(it, 1);
    vmem_wait_all();
    __syncthreads();
    if (++it >= it1) break;
  }
  if (!wave_active) return;
  if (nparts > 1) {
    const int64_t item = ((int64_t)seg * a.k_blocks + kb) * a.hkv + kvh;
    constexpr int SLOT = 2 * DT * 16 * 64;
    if (!split_sum(dkv, a.part_acc + (item * a.dkv_parts * NW + wave) * SLOT, (int64_t)NW * SLOT, part, nparts,
                   a.part_cnt + item * NW + wave))
      return;
  }
  if (!kin) return;
  // a padded key is seen by no query: its gradients are zero
  store_cols<D>(a.dk + krow, dkacc, a.scaling, g, kpad);
  store_cols<D>(a.dv + krow, dvacc, 1.0f, g, kpad);
}

// ===========================================================================
// dK/dV at D = 128 with each SIMD's work split by role.  The one-wave-per-SIMD
// kernel above leaves a SIMD's MFMA pipe idle whenever its only wave runs
// VALU work or waits; here a workgroup of eight waves owns the same 128 keys
// and waves c and c + 4 (the same SIMD) share key group c: wave c (A) forms
// S = Q K^T, P = exp(S - LSE) and dV^T += dO^T P, wave c + 4 (B) forms
// dP = dO V^T, dS = P (dP - delta) and dK^T += Q^T dS.  Each holds only its own
// operand (K or V) and accumulator (dV or dK), so two waves fit a SIMD.  P
// travels from A to B through LDS as fp16 (P <= 1, so the rounding is 2^-11
// relative, below dS's own bf16 rounding).  Phases: one per (query tile,
// head) step; in phase u wave A works on step u and wave B on step u - 1,
// and a workgroup barrier ends the phase.  Q/dO tiles with their LSE and
// delta rows sit in three LDS stages: in phase u, A reads step u's stage, B
// step u - 1's, and the B waves' DMA fills step u + 1's.  Steps visit the
// tiles in the order of the kernel above, parts of a split item included.
namespace rs {
constexpr int D = 128;
constexpr int NC = 4;                  // key groups (A/B wave pairs) per workgroup
constexpr int NWAVES = 2 * NC;
constexpr int KS = D / 16;
constexpr int DT = D / 32;
constexpr int NSTAGE = 3;
using T = Tile<D>;
constexpr int RB = T::ROW_BYTES;
constexpr int DMA_PER_WAVE = T::TILE_BYTES / 1024 / NC;   // KiB of one tile per B wave
constexpr int PHALF = 2 * 64 * 16;     // fp16 P of one 32-query half: [chunk 0/1][lane] of 16 bytes
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int J>
using ic = std::integral_constant<int, J>;

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, f16x2{(_Float16)a, (_Float16)b});
}
// Workgroup barrier over LDS traffic only (the DMA of a stage is waited for
// explicitly by the waves that issue it, before the barrier that precedes
// its first reader).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
}  // namespace rs

// SPLIT: the launch cuts key blocks into parts (a separate instantiation, so
// the unsplit kernel carries none of the part bookkeeping)
template <bool PAD, bool SPLIT>
__global__ __launch_bounds__(64 * rs::NWAVES, 1) void attn_bwd_dkdv_rs_kernel(AttnBwdArgs a) {
  using namespace rs;
  // one array per stage, addressed with compile-time stage numbers, so the
  // DMA into one stage never aliases (and never delays) reads of another
  __shared__ __attribute__((aligned(16))) char lds_q0[T::TILE_BYTES], lds_q1[T::TILE_BYTES], lds_q2[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_o0[T::TILE_BYTES], lds_o1[T::TILE_BYTES], lds_o2[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float lds_l0[BN], lds_l1[BN], lds_l2[BN];
  __shared__ __attribute__((aligned(16))) float lds_d0[BN], lds_d1[BN], lds_d2[BN];
  __shared__ __attribute__((aligned(16))) char lds_p[NC][2][2 * PHALF];
  auto qst = [&](auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value % NSTAGE;
    return (lds_char *)(st == 0 ? lds_q0 : st == 1 ? lds_q1 : lds_q2);
  };
  auto ost = [&](auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value % NSTAGE;
    return (lds_char *)(st == 0 ? lds_o0 : st == 1 ? lds_o1 : lds_o2);
  };
  auto lst = [&](auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value % NSTAGE;
    return (__attribute__((address_space(3))) float *)(st == 0 ? lds_l0 : st == 1 ? lds_l1 : lds_l2);
  };
  auto dst_ = [&](auto S) __attribute__((always_inline)) {
    constexpr int st = decltype(S)::value % NSTAGE;
    return (__attribute__((address_space(3))) float *)(st == 0 ? lds_d0 : st == 1 ? lds_d1 : lds_d2);
  };

  const int tid = threadIdx.x;
  // wave-uniform, so the role and per-step tests below are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = wave & (NC - 1);
  const bool role_a = wave < NC;
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // work item: as the one-wave kernel (segment-major, key blocks ascending,
  // then part, then kv head)
  const int dkv_parts = SPLIT ? a.dkv_parts : 1;
  const int per_seg = a.k_blocks * dkv_parts * a.hkv;
  const int b = blockIdx.x;
  const int seg = b / per_seg;
  int rest = b % per_seg;
  const int kb = rest / (dkv_parts * a.hkv);
  rest %= dkv_parts * a.hkv;
  const int part = rest / a.hkv;
  const int kvh = rest % a.hkv;
  int s0, L;
  segment_bounds(a.lay, seg, s0, L);
  const int kb0 = kb * (32 * NC);
  if (kb0 >= L) return;
  const int kw0 = kb0 + c * 32;
  const int kw1 = min(kw0 + 31, L - 1);
  const bool wave_active = kw0 < L;
  const int key = kw0 + n;
  const bool kin = key < L;
  const int64_t krow = ((int64_t)(s0 + (kin ? key : 0)) * a.hkv + kvh) * D;

  const int W = a.window;
  const bool bidir = a.bidirectional != 0;
  const float c2 = a.scale_log2;
  const int mask_base = bidir ? 0 : key;
  const int lim_c = W > 0 ? min(W, L - key) : L - key;
  const uint32_t mask_lim = bidir ? (uint32_t)L : (uint32_t)max(lim_c, 0);
  const int qlo = bidir ? 0 : kb0;
  const int qhi = bidir || W <= 0 ? L - 1 : min(L - 1, min(kb0 + 32 * NC - 1, L - 1) + W - 1);
  const int qt_lo = qlo / BN;
  const int qt_hi = qhi / BN;
  const int nqt = qt_hi - qt_lo + 1;
  const int ntiles = nqt * a.group;
  // split: this part takes steps [it0, it0 + nsteps) (the last launched part
  // takes any remainder); uniform per workgroup
  const int span = SPLIT ? a.dkv_span : ntiles;
  const int nparts = SPLIT ? min((ntiles + span - 1) / span, dkv_parts) : 1;
  if (part >= nparts) return;
  const int it0 = part * span;
  const int nsteps = (part == nparts - 1 ? ntiles : it0 + span) - it0;
  // the step order of the one-wave kernel (shared by neighbouring key blocks)
  const bool windowed = !bidir && W > 0 && W < L;
  int rot = 0;
  if (windowed) {
    const int R = (32 * NC - 2 + W) / BN + 1;
    const int s_ = (qt_lo + R - 1) / R * R;
    rot = s_ <= qt_hi ? s_ - qt_lo : 0;
  }
  // the query tile of this part's step u (and its head h)
  auto step_tile = [&](int u, int &h) __attribute__((always_inline)) {
    const int it = it0 + u;
    const int ti = it / a.group;
    h = kvh * a.group + (it - ti * a.group);
    if (!windowed) return qt_hi - ti;
    const int x = rot + ti;
    return qt_lo + (x >= nqt ? x - nqt : x);
  };
  // the part's accumulator slots and arrival counters: per (item, key group)
  // the one-wave kernel's slot of [dK | dV], B summing the dK half and A the
  // dV half, each with its own counter (B's, then A's after all of B's)
  constexpr int HALF_SLOT = DT * 16 * 64;
  const int64_t item = ((int64_t)seg * a.k_blocks + kb) * a.hkv + kvh;
  const int64_t n_items = (int64_t)a.lay.num_segments * a.k_blocks * a.hkv;
  float *slot0 = a.part_acc + (item * dkv_parts * NC + c) * (2 * HALF_SLOT);
  // this key group's view of the query tile starting at t0
  auto visibility = [&](int t0, bool &all_visible) __attribute__((always_inline)) {
    const bool none = !wave_active || (!bidir && (t0 + BN - 1 < kw0 || (W > 0 && t0 > kw1 + W - 1)));
    all_visible = !none && t0 + BN <= L && (bidir || (t0 >= kw1 && (W <= 0 || t0 + BN - 1 <= kw0 + W - 1)));
    return !none;
  };

  TileAddr<D> ad;
  ad.init(lane);
  lds_char *pbase = (lds_char *)lds_p[c][0];

  const int64_t q_stride = (int64_t)a.hq * D;
  int off[DMA_PER_WAVE];
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int slot = (c * DMA_PER_WAVE + i) * 64 + lane;
    const int row = slot / T::CHUNKS;
    const int pch = slot % T::CHUNKS;
    off[i] = (row * (int)q_stride + (pch ^ T::swz_kv(row)) * 8) * 2;
  }
  // the step's Q and dO tiles, and (waves 0, 1) its LSE and delta rows; rows
  // past the segment read as 0
  auto issue_dma = [&](int it, auto S) __attribute__((always_inline)) {
    int h;
    const int t0 = step_tile(it, h) * BN;
    const int rows = min(L - t0, BN);
    const int64_t r0 = (int64_t)(s0 + t0) * a.hq + h;
    const int valid_bytes = ((rows - 1) * (int)q_stride + D) * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.q + r0 * D, valid_bytes);
    const __amdgpu_buffer_rsrc_t orr = make_rsrc(a.d_o + r0 * D, valid_bytes);
    lds_char *qdst = qst(S) + c * DMA_PER_WAVE * 1024;
    lds_char *odst = ost(S) + c * DMA_PER_WAVE * 1024;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      dma16(qr, off[i], qdst + i * 1024);
      dma16(orr, off[i], odst + i * 1024);
    }
    if (c < 2) {
      const int fbytes = ((rows - 1) * a.hq + 1) * 4;
      const __amdgpu_buffer_rsrc_t fr = make_rsrc((c ? a.delta : a.lse) + r0, fbytes);
      dma4(fr, lane * a.hq * 4, (lds_char *)(c ? dst_(S) : lst(S)));
    }
  };
  if (role_a) {
    // ============ wave A: DMA; S, P, dV ============
    bf16x8 kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 rk = *reinterpret_cast<const uint4 *>(a.k + krow + ks * 16 + g * 8);
      kf[ks] = __builtin_bit_cast(bf16x8, kin ? rk : make_uint4(0, 0, 0, 0));
    }
    f32x16 dvv[1][DT];
    f32x16 (&dvacc)[DT] = dvv[0];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dvacc[dt] = f32x16{};
    if (nsteps > 0) issue_dma(0, ic<0>{});
    vmem_wait_all();
    lds_barrier();   // the first step's stage has landed
    auto phase = [&](int u, auto J) __attribute__((always_inline)) {
      constexpr int js = decltype(J)::value;   // u % NSTAGE
      // step u + 1 into the stage step u - 2 left (A read it in phase u - 2,
      // B in phase u - 1).  A issues the DMA: B's phase is the longer one
      if (u + 1 < nsteps) issue_dma(u + 1, ic<js + 1>{});
      if (u < nsteps) {
        int h;
        const int t0 = step_tile(u, h) * BN;
        bool all_visible;
        if (visibility(t0, all_visible)) {
          const lds_char *Qt = qst(J);
          const lds_char *Ot = ost(J);
          const __attribute__((address_space(3))) float *Lt = lst(J);
          lds_char *slot = pbase + (u & 1) * (2 * PHALF);
          // P of one half from its scores (exp, then the mask after it: a
          // query with no visible key has LSE = -inf)
          auto probs = [&](const f32x16 &sv, int half, float (&p)[16]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const f32x4 l4 = *(const __attribute__((address_space(3))) f32x4 *)(Lt + half * 32 + 8 * j + 4 * g);
#pragma unroll
              for (int e = 0; e < 4; ++e)
                p[4 * j + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[4 * j + e], c2, -(l4[e] * kLog2e)));
            }
          };
          auto mask_p = [&](float (&p)[16], int half) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int qp = t0 + half * 32 + (i >> 2) * 8 + 4 * g + (i & 3);
              p[i] = (uint32_t)(qp - mask_base) < mask_lim ? p[i] : 0.0f;
            }
          };
          auto hand_over = [&](const float (&p)[16], int half, bf16x8 &b0, bf16x8 &b1) __attribute__((always_inline)) {
            u32x4 h0, h1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              h0[i] = pack_f16x2(p[2 * i], p[2 * i + 1]);
              h1[i] = pack_f16x2(p[8 + 2 * i], p[8 + 2 * i + 1]);
            }
            *(__attribute__((address_space(3))) u32x4 *)(slot + half * PHALF + lane * 16) = h0;
            *(__attribute__((address_space(3))) u32x4 *)(slot + half * PHALF + 1024 + lane * 16) = h1;
            pack16(p, b0, b1);
          };
          // the second half's S chain beside the first half's exp, the first
          // half's dV MFMAs beside the second half's exp
          const f32x16 s0 = rows_times<D>(Qt, ad, 0, kf);
          const f32x16 s1 = rows_times<D>(Qt, ad, 32 * RB, kf);
          float pa[16], pb[16];
          probs(s0, 0, pa);
          if (!all_visible) mask_p(pa, 0);
          bf16x8 a0, a1, b0, b1;
          hand_over(pa, 0, a0, a1);
          tr_times<D>(Ot, ad, 0, a0, a1, dvacc);
          probs(s1, 1, pb);
          if (!all_visible) mask_p(pb, 1);
          hand_over(pb, 1, b0, b1);
          tr_times<D>(Ot, ad, 32, b0, b1, dvacc);
        }
      }
      vmem_wait_all();   // step u + 1 has landed before the phase that reads it
      lds_barrier();
    };
    for (int r = 0;; r += 3) {
      phase(r, ic<0>{}); if (r == nsteps) break;
      phase(r + 1, ic<1>{}); if (r + 1 == nsteps) break;
      phase(r + 2, ic<2>{}); if (r + 2 == nsteps) break;
    }
    if (!wave_active) return;
    if constexpr (SPLIT) {
      if (!split_sum(dvv, slot0 + HALF_SLOT, (int64_t)NC * 2 * HALF_SLOT, part, nparts,
                     a.part_cnt + n_items * NC + item * NC + c))
        return;
    }
    if (!kin) return;
    bool kpad = false;
    if constexpr (PAD) kpad = a.key_valid[s0 + key] == 0;
    // a padded key is seen by no query: its gradients are zero
    store_cols<D>(a.dv + krow, dvacc, 1.0f, g, kpad);
    return;
  }

  // ============ wave B: dP, dS, dK ============
  bf16x8 vf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint4 rv = *reinterpret_cast<const uint4 *>(a.v + krow + ks * 16 + g * 8);
    vf[ks] = __builtin_bit_cast(bf16x8, kin ? rv : make_uint4(0, 0, 0, 0));
  }
  f32x16 dkv1[1][DT];
  f32x16 (&dkacc)[DT] = dkv1[0];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) dkacc[dt] = f32x16{};

  vmem_wait_all();
  lds_barrier();
  auto bphase = [&](int u, auto J) __attribute__((always_inline)) {
    constexpr int j = decltype(J)::value;   // u % NSTAGE
    if (u >= 1) {
      int h;
      const int t0 = step_tile(u - 1, h) * BN;
      bool all_visible;
      if (visibility(t0, all_visible)) {
        const lds_char *Qt = qst(ic<j + 2>{});   // stage of step u - 1
        const lds_char *Ot = ost(ic<j + 2>{});
        const __attribute__((address_space(3))) float *Dl = dst_(ic<j + 2>{});
        const lds_char *slot = pbase + ((u - 1) & 1) * (2 * PHALF);
        auto dscores = [&](const f32x16 &dp, int half, bf16x8 &d0, bf16x8 &d1) __attribute__((always_inline)) {
          const u32x4 h0 = *(const __attribute__((address_space(3))) u32x4 *)(slot + half * PHALF + lane * 16);
          const u32x4 h1 = *(const __attribute__((address_space(3))) u32x4 *)(slot + half * PHALF + 1024 + lane * 16);
          // dS = P (dP - delta) as fma(P, dP - delta, +0), so the fp16 P
          // enters a mixed-precision fma as it is (v_fma_mix_f32: no
          // conversion); the result equals the product except that an exact
          // -0 becomes +0
          _Float16 ph[16];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const f16x2 lo = __builtin_bit_cast(f16x2, (uint32_t)h0[i]);
            const f16x2 hi = __builtin_bit_cast(f16x2, (uint32_t)h1[i]);
            ph[2 * i] = lo[0];
            ph[2 * i + 1] = lo[1];
            ph[8 + 2 * i] = hi[0];
            ph[8 + 2 * i + 1] = hi[1];
          }
          float ds[16];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const f32x4 d4 = *(const __attribute__((address_space(3))) f32x4 *)(Dl + half * 32 + 8 * jj + 4 * g);
#pragma unroll
            for (int e = 0; e < 4; ++e)
              ds[4 * jj + e] = __builtin_fmaf((float)ph[4 * jj + e], dp[4 * jj + e] - d4[e], 0.0f);
          }
          pack16(ds, d0, d1);
        };
        const f32x16 dp0 = rows_times<D>(Ot, ad, 0, vf);
        const f32x16 dp1 = rows_times<D>(Ot, ad, 32 * RB, vf);
        bf16x8 a0, a1, b0, b1;
        dscores(dp0, 0, a0, a1);
        tr_times<D>(Qt, ad, 0, a0, a1, dkacc);
        dscores(dp1, 1, b0, b1);
        tr_times<D>(Qt, ad, 32, b0, b1, dkacc);
      }
    }
    lds_barrier();
  };
  for (int r = 0;; r += 3) {
    bphase(r, ic<0>{}); if (r == nsteps) break;
    bphase(r + 1, ic<1>{}); if (r + 1 == nsteps) break;
    bphase(r + 2, ic<2>{}); if (r + 2 == nsteps) break;
  }
  if (!wave_active) return;
  if constexpr (SPLIT) {
    if (!split_sum(dkv1, slot0, (int64_t)NC * 2 * HALF_SLOT, part, nparts, a.part_cnt + item * NC + c)) return;
  }
  if (!kin) return;
  bool kpad = false;
  if constexpr (PAD) kpad = a.key_valid[s0 + key] == 0;
  store_cols<D>(a.dk + krow, dkacc, a.scaling, g, kpad);
}

template <int D, bool PAD>
hipError_t launch_d(const AttnBwdArgs &a, hipStream_t stream) {
  const int64_t nseg = a.lay.num_segments;
  const int64_t dq_blocks = (int64_t)a.q_blocks * nseg * a.hkv * a.head_chunks * a.dq_parts;
  const int64_t kv_blocks = (int64_t)a.k_blocks * nseg * a.hkv * a.dkv_parts;
  if (dq_blocks > 0)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<D, PAD>), dim3((unsigned)dq_blocks), dim3(64 * NW), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (kv_blocks > 0) {
    if constexpr (D == 128) {
      if (a.dkv_parts > 1)
        hipLaunchKernelGGL((attn_bwd_dkdv_rs_kernel<PAD, true>), dim3((unsigned)kv_blocks), dim3(64 * rs::NWAVES), 0,
                           stream, a);
      else
        hipLaunchKernelGGL((attn_bwd_dkdv_rs_kernel<PAD, false>), dim3((unsigned)kv_blocks), dim3(64 * rs::NWAVES), 0,
                           stream, a);
    } else
      hipLaunchKernelGGL((attn_bwd_dkdv_kernel<D, PAD>), dim3((unsigned)kv_blocks), dim3(64 * NW), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

int attn_bwd_keys_per_workgroup() { return COLS; }

hipError_t launch_attn_bwd(int head_dim, const AttnBwdArgs &a, hipStream_t stream) {
  if (a.heads_per_wg < 1 || a.heads_per_wg > COLS || a.tok_per_wg < 1 || a.tok_per_wg * a.heads_per_wg > COLS)
    return hipErrorInvalidConfiguration;
  for (const int parts : {a.dq_parts, a.dkv_parts})
    if (parts < 1 || parts > kMaxKvParts) return hipErrorInvalidConfiguration;
  if ((a.dq_parts > 1 && a.dq_span < 1) || (a.dkv_parts > 1 && a.dkv_span < 1) ||
      ((a.dq_parts > 1 || a.dkv_parts > 1) && (!a.part_acc || !a.part_cnt)))
    return hipErrorInvalidConfiguration;
  const bool pad = a.key_valid != nullptr;
  if (head_dim == 128) return pad ? launch_d<128, true>(a, stream) : launch_d<128, false>(a, stream);
  return pad ? launch_d<64, true>(a, stream) : launch_d<64, false>(a, stream);
}

}  // namespace muse
