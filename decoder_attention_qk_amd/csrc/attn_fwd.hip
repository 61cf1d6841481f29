// Causal GQA flash attention forward on bf16 MFMA (gfx950), optionally fused
// with the Q norm/RoPE prologue and the output norm/gate epilogue.
//
// Semantics: layers page, MuseSparkAttention (scaling = head_dim^-0.5, KV
// heads repeated to the query-head count, per-layer sliding window), model
// page _causal_mask (window = number of visible causal keys including the
// query); packed documents attend only inside themselves; _qk_norm_rope_core
// and _output_norm_gate_core for the fused prologue/epilogue.
//
// Work item: (row/segment, kv head, head chunk, block of query tokens).  A
// workgroup of NW = 4 waves owns 32*NW query columns; a column is a (token,
// head) pair of the KV group, token-major, so any group size fills the
// columns (G = 5 uses 25 tokens x 5 heads + 3 idle columns).  K and V tiles
// of BN = 64 keys are shared by all columns through LDS.  A grid too small to
// fill the device may cut each item's key tiles into parts (KV split): each
// part runs its tiles and publishes per wave its unnormalised O, reference and
// sums; the last part of a wave to arrive combines them in part order.
//
// Registers (v_mfma_f32_32x32x16_bf16, 64 lanes): each wave computes
// S^T = K Q^T, so lane l owns query column n = l % 32 and key rows
// 8*(i/4) + 4*(l/32) + i%4 of each 32-key tile.  The row max needs one
// exchange between lanes l and l^32, the row sum none until the end, and P^T
// lands directly in the B-operand layout of O^T += V^T P^T.
//
// LDS: K and V tiles arrive by direct global->LDS DMA (buffer_load ... lds, 16
// bytes per lane, one contiguous KiB per wave instruction; the buffer
// resource ends at the segment's last row, so rows past it read as zeros),
// double-buffered:
// the DMA of tile j+1 runs while tile j is computed, so no registers stage
// tiles and one barrier per tile suffices.  V stays row-major; the PV A
// operand is read with ds_read_b64_tr_b16 (within each 16-lane group, lane r
// receives element r%4 of the 4-vectors addressed by lanes r/4 + 4j), which
// hands lane (d, g) keys {4g..4g+3, 8+4g..8+4g+3} of a 16-key step -- the same
// key order P^T has in the S^T accumulator.  16-byte chunks are XOR-swizzled
// per row on the DMA source side so both read patterns avoid bank conflicts.
//
// A workgroup first issues the DMA of its first tile, then loads and
// normalises its Q fragments (and, at D = 128, fetches its gate fragments)
// while that DMA is in flight.  Tiles are visited from the diagonal downwards; tiles no column of the
// workgroup sees are never loaded, tiles every column of a wave sees skip the
// element mask.  Softmax keeps a per-column reference (a score already seen)
// instead of a running max: each 32-key half forms its probabilities against
// it and is kept when no lane's partial sum exceeds kSumLimit, so no
// probability is near overflow; only a half that fails (or a column without a
// reference yet) takes the exact column max, rescales O and the sum, and forms
// its probabilities again.  The final division by the sum removes the
// reference.  Bidirectional mode
// (vision page, MuseSparkVisionAttention) sees every key of the segment;
// padded keys of a BSHD batch (model page, MuseSparkTextModel.forward
// attention_mask) are masked per tile, and a query left with no key gives
// the zero row.
#include <algorithm>
#include <cmath>

#include "attn_common.hpp"
#include "kernels.hpp"

namespace muse {

namespace {

constexpr int BN = 64;        // keys per tile
constexpr int NW = 4;         // waves per workgroup
constexpr int COLS = 32 * NW; // query columns per workgroup
// largest per-lane probability sum of a 32-key half kept without moving the reference
constexpr float kSumLimit = 1048576.0f;

static_assert(BN == 64, "Tile<D> holds 64-row tiles");

// PAD: keys may be padding (a.key_valid given); a separate instantiation so
// the unpadded kernel carries none of its registers.
template <int D, bool FUSED, bool PAD>
__global__ __launch_bounds__(64 * NW, 2) void attn_fwd_kernel(AttnArgs a) {
  using T = Tile<D>;
  constexpr int DMA_PER_WAVE = T::TILE_BYTES / 1024 / NW;   // KiB of one tile per wave
  constexpr int KS = D / 16;   // QK^T k-steps
  constexpr int DT = D / 32;   // O^T row tiles
  constexpr int RB = T::ROW_BYTES;
  // One array per buffer: distinct objects let the compiler see that the DMA
  // into one stage never aliases reads of the other, so LDS reads of the
  // current tile do not wait for the next tile's DMA.
  __shared__ __attribute__((aligned(16))) char lds_k0[T::TILE_BYTES], lds_v0[T::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_k1[T::TILE_BYTES], lds_v1[T::TILE_BYTES];
  auto kbuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_k1 : lds_k0); };
  auto vbuf = [&](int buf) __attribute__((always_inline)) { return (lds_char *)(buf ? lds_v1 : lds_v0); };

  const int tid = threadIdx.x;
  // wave-uniform, so the per-wave tile tests below are scalar branches
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int n = lane & 31;
  const int g = lane >> 5;

  // ---- work item: segment-major, then query blocks in descending order
  // (longest first), then KV part, then (kv head, head chunk).  Consecutive
  // workgroups take consecutive kv heads, so with the round-robin dispatch
  // over the XCDs each XCD works on one (segment, kv head) pair at a time and
  // its K/V stays in that XCD's L2.
  const int heads_items = a.hkv * a.head_chunks;
  const int per_seg = a.q_blocks * a.kv_parts * heads_items;
  const int b = blockIdx.x;
  const int seg = b / per_seg;
  int rest = b % per_seg;
  const int qb = a.q_blocks - 1 - rest / (a.kv_parts * heads_items);
  rest %= a.kv_parts * heads_items;
  const int part = rest / heads_items;
  rest %= heads_items;
  const int hc = rest % a.head_chunks;
  const int kvh = rest / a.head_chunks;

  int s0, L;
  if (a.lay.cu_seqlens) {
    const int T_ = a.lay.n_tokens;
    int c0 = a.lay.cu_seqlens[seg];
    int c1 = a.lay.cu_seqlens[seg + 1];
    c0 = min(max(c0, 0), T_);
    c1 = min(max(c1, c0), T_);
    s0 = c0;
    L = c1 - c0;
  } else {
    s0 = seg * a.lay.seqlen;
    L = a.lay.seqlen;
  }
  const int HPW = a.heads_per_wg;
  const int BMT = a.tok_per_wg;              // tokens per workgroup
  const int q0 = qb * BMT;
  if (q0 >= L) return;
  const int q1 = min(q0 + BMT, L);

  // ---- this lane's column and this wave's token range
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
  const int64_t qrow = ((int64_t)(s0 + (qvalid ? qpos : 0)) * a.hq + (qvalid ? head : 0)) * D;

  // ---- Q fragment: B operand of S^T = K Q^T; lane holds d = 16 ks + 8 g + [0, 8)
  bf16x8 qf[KS];
  // (run after the first K/V tile's DMA is issued, so its latency hides the loads)
  auto load_q = [&]() __attribute__((always_inline)) {
    uint4 raw[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      raw[ks] = qvalid ? *reinterpret_cast<const uint4 *>(a.q + qrow + ks * 16 + g * 8)
                       : make_uint4(0, 0, 0, 0);
    if constexpr (FUSED) {
      // Two phases, each with all of its loads issued before any result is
      // used: (1) Q and the gains -> normalised bf16 chunks; (2) the cos/sin
      // rows -> query scale and rotation.  Splitting them keeps the gains and
      // the table rows from being live at the same time.
      const bool has_gain = a.q_gain != nullptr, rope = a.use_rope != 0;
      uint4 nq[KS];
      {
        float4 gv[KS][2];
        if (has_gain) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            gv[ks][0] = *reinterpret_cast<const float4 *>(a.q_gain + ks * 16 + g * 8);
            gv[ks][1] = *reinterpret_cast<const float4 *>(a.q_gain + ks * 16 + g * 8 + 4);
          }
        }
        float all[2 * KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float x[8];
          unpack8(raw[ks], x);
          const float own = chunk_sumsq<8>(x);
          float lo, hi;
          swap32(own, lo, hi);
          all[2 * ks] = lo;          // chunk 2 ks + g holds d = 16 ks + 8 g
          all[2 * ks + 1] = hi;
        }
        const float rstd = rms_rstd(tree_sum(all), 1.0f / (float)D, a.eps);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          float w[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
          if (has_gain) {
            w[0] = a.gain_center + gv[ks][0].x; w[1] = a.gain_center + gv[ks][0].y;
            w[2] = a.gain_center + gv[ks][0].z; w[3] = a.gain_center + gv[ks][0].w;
            w[4] = a.gain_center + gv[ks][1].x; w[5] = a.gain_center + gv[ks][1].y;
            w[6] = a.gain_center + gv[ks][1].z; w[7] = a.gain_center + gv[ks][1].w;
          }
          float x[8];
          unpack8(raw[ks], x);
          nq[ks] = norm_chunk(x, w, rstd);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (rope) {
        int p = a.lay.position_ids ? a.lay.position_ids[s0 + (qvalid ? qpos : 0)] : (qvalid ? qpos : 0);
        p = p < 0 ? 0 : (p >= a.n_pos ? a.n_pos - 1 : p);
        float4 cv[KS], sv[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          cv[ks] = *reinterpret_cast<const float4 *>(a.cos_tab + (int64_t)p * (D / 2) + ks * 8 + g * 4);
          sv[ks] = *reinterpret_cast<const float4 *>(a.sin_tab + (int64_t)p * (D / 2) + ks * 8 + g * 4);
        }
        const bool qscale = a.query_scale != 1.0f, v2 = a.rope_v2 != 0;
        auto rot = [&](int ks, bool qs, bool rv2) __attribute__((always_inline)) {
          const float cs[4] = {cv[ks].x, cv[ks].y, cv[ks].z, cv[ks].w};
          const float sn[4] = {sv[ks].x, sv[ks].y, sv[ks].z, sv[ks].w};
          qf[ks] = __builtin_bit_cast(bf16x8, scale_rope_chunk(nq[ks], qs, a.query_scale, true, cs, sn, rv2));
        };
        if (!qscale && !v2) {
          // the common case with its flags known at compile time (no branches)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) rot(ks, false, false);
        } else {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) rot(ks, qscale, v2);
        }
      } else {
        const float one[4] = {1.f, 1.f, 1.f, 1.f}, zero[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qf[ks] = __builtin_bit_cast(
              bf16x8, scale_rope_chunk(nq[ks], a.query_scale != 1.0f, a.query_scale, false, one, zero));
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, raw[ks]);
    }
  };

  // ---- per-lane DMA source offsets (elements) and LDS read addresses (bytes)
  const int64_t kv_stride = (int64_t)a.hkv * D;
  const uint16_t *kbase = a.k + ((int64_t)s0 * a.hkv + kvh) * D;
  const uint16_t *vbase = a.v + ((int64_t)s0 * a.hkv + kvh) * D;
  int off_k[DMA_PER_WAVE], off_v[DMA_PER_WAVE];   // byte offsets inside a tile's rows
#pragma unroll
  for (int i = 0; i < DMA_PER_WAVE; ++i) {
    const int slot = (wave * DMA_PER_WAVE + i) * 64 + lane;
    const int row = slot / T::CHUNKS;
    const int pch = slot % T::CHUNKS;
    off_k[i] = (row * (int)kv_stride + (pch ^ T::swz_k(row)) * 8) * 2;
    off_v[i] = (row * (int)kv_stride + (pch ^ T::swz_v(row)) * 8) * 2;
  }
  int ka[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) ka[ks] = n * RB + (((2 * ks + g) ^ T::swz_k(n)) << 4);
  int va[DT];
  {
    const int r = lane & 15, q = (lane >> 4) & 1;
    const int row = 4 * g + (r >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int ch = dt * 4 + 2 * q + ((r & 3) >> 1);
      va[dt] = row * RB + ((ch ^ T::swz_v(row)) << 4) + (r & 1) * 8;
    }
  }

  // Padded keys (BSHD attention_mask): each lane fetches the validity byte of
  // one key of the tile together with the tile's DMA, so it has arrived by
  // the barrier before the tile is computed; after that barrier a ballot
  // turns the 64 bytes into a wave-uniform key mask (scalar registers), and
  // the byte register is free for the next tile's fetch.
  const uint8_t *kvalid = a.key_valid + s0;   // read only when PAD
  int vbyte = 1;
  uint64_t kmask = ~0ull;   // bit j: key k0 + j of the current tile is not padding
  auto take_mask = [&]() __attribute__((always_inline)) {
    if constexpr (PAD) kmask = __ballot(vbyte != 0);
  };

  auto issue_dma = [&](int kt, int buf) {
    const int k0 = kt * BN;
    if constexpr (PAD) vbyte = k0 + lane < L ? (int)kvalid[k0 + lane] : 0;
    lds_char *kdst = kbuf(buf) + wave * DMA_PER_WAVE * 1024;
    lds_char *vdst = vbuf(buf) + wave * DMA_PER_WAVE * 1024;
    // the tile's rows k0 .. L-1 of this kv head; rows past the segment read as zeros
    // (zero keys are masked out of every score, zero values add nothing)
    const int valid_bytes = ((min(L - k0, BN) - 1) * (int)kv_stride + D) * 2;
    const __amdgpu_buffer_rsrc_t kr = make_rsrc(kbase + (int64_t)k0 * kv_stride, valid_bytes);
    const __amdgpu_buffer_rsrc_t vr = make_rsrc(vbase + (int64_t)k0 * kv_stride, valid_bytes);
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      dma16(kr, off_k[i], kdst + i * 1024);
      dma16(vr, off_v[i], vdst + i * 1024);
    }
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
  float m_run = -INFINITY;   // reference max (raw score units) of this lane's column
  float mc = 0.0f;           // m_run * scale_log2 (0 without a reference)
  float sum_lim = -1.0f;     // kSumLimit once the column has a reference
  float l_run = 0.0f;

  const int W = a.window;
  const bool bidir = a.bidirectional != 0;
  const float c2 = a.scale_log2;
  // key kp is visible iff (unsigned)(mask_base - kp) < mask_lim: causal,
  // qpos - kp in [0, W) (or [0, inf) without a window); bidirectional,
  // L - 1 - kp in [0, L)
  const int mask_base = bidir ? L - 1 : qpos;
  const uint32_t mask_lim = bidir ? (uint32_t)L : (W > 0 ? (uint32_t)W : 0x7FFFFFFFu);

  // called with literal buffer indices so LDS offsets fold into immediates
  auto compute = [&](int kt, int BUF) __attribute__((always_inline)) {
    const int k0 = kt * BN;
    // bidirectional: every key of the segment (the last tile may end past it)
    const bool none_visible = !wave_active || (!bidir && ((k0 > q1w - 1) || (W > 0 && k0 + BN - 1 <= q0w - W)));
    if (none_visible) return;
    const bool all_visible = bidir ? k0 + BN <= L : (k0 + BN - 1 <= q0w) && (W <= 0 || k0 > q1w - 1 - W);
    const bool padded = PAD && kmask != ~0ull;
    const lds_char *Kt = kbuf(BUF);
    const lds_char *Vt = vbuf(BUF);

    // The tile is processed as two 32-key halves; the per-column reference
    // makes a per-half softmax exact (order below).
    auto mask = [&](f32x16 &sv, int half) __attribute__((always_inline)) {
      // this lane's keys of the half as bits at compile-time positions
      // (8 (i/4) + i%4) of one 32-bit word; visibility is one unsigned range
      // compare per key (no branches)
      const uint32_t kbits = padded ? (uint32_t)(kmask >> (half * 32 + g * 4)) : ~0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kp = k0 + half * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
        const bool vis = ((uint32_t)(mask_base - kp) < mask_lim) & ((kbits >> ((i >> 2) * 8 + (i & 3))) & 1u);
        sv[i] = vis ? sv[i] : -INFINITY;
      }
    };
    auto softmax = [&](const f32x16 &sv, bf16x8 &p0, bf16x8 &p1) __attribute__((always_inline)) -> float {
      float pf[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) pf[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[i], c2, -mc));
      float t[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) t[j] = (pf[4 * j] + pf[4 * j + 1]) + (pf[4 * j + 2] + pf[4 * j + 3]);
      const float tsum = (t[0] + t[1]) + (t[2] + t[3]);
      uint4 lo, hi;
      lo.x = pack_bf16x2(pf[0], pf[1]);   lo.y = pack_bf16x2(pf[2], pf[3]);
      lo.z = pack_bf16x2(pf[4], pf[5]);   lo.w = pack_bf16x2(pf[6], pf[7]);
      hi.x = pack_bf16x2(pf[8], pf[9]);   hi.y = pack_bf16x2(pf[10], pf[11]);
      hi.z = pack_bf16x2(pf[12], pf[13]); hi.w = pack_bf16x2(pf[14], pf[15]);
      p0 = __builtin_bit_cast(bf16x8, lo);
      p1 = __builtin_bit_cast(bf16x8, hi);
      return tsum;
    };

    // One half: probabilities against the current reference; the half is
    // kept when every lane's partial sum is at most kSumLimit (so no
    // probability is near overflow) and its column has a reference.  Else the
    // column's exact max over the half becomes the reference (if larger), O and
    // l are rescaled, and the probabilities are formed again.
    auto half_step = [&](const f32x16 &sv, bf16x8 &p0, bf16x8 &p1) __attribute__((always_inline)) {
      float t = softmax(sv, p0, p1);
      if (__any(!(t <= sum_lim))) {
        float m4[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) m4[j] = fmaxf(fmaxf(sv[4 * j], sv[4 * j + 1]), fmaxf(sv[4 * j + 2], sv[4 * j + 3]));
        float cm = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
        float lo, hi;
        swap32(cm, lo, hi);
        const float m_new = fmaxf(m_run, fmaxf(lo, hi));
        // a column without a reference has l = 0 and O = 0 (no half was kept)
        const float alpha = m_run == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f((m_run - m_new) * c2);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_run = m_new;
        mc = m_run == -INFINITY ? 0.0f : m_run * c2;
        sum_lim = m_run == -INFINITY ? -1.0f : kSumLimit;
        t = softmax(sv, p0, p1);
      }
      l_run += t;
    };

    // Order: QK(h0), [mask h0], QK(h1) beside softmax(h0), [mask h1], PV(h0)
    // beside softmax(h1), PV(h1).  The masks sit in wave-uniform branches of
    // their own, so on unmasked tiles each MFMA run and the softmax it overlaps
    // share one basic block and the wave interleaves them.
    const bool masked = __builtin_amdgcn_readfirstlane((int)(!all_visible || padded)) != 0;
    bf16x8 pa0, pa1, pb0, pb1;
    // QK^T of the first half: its K fragments are all read before the chain
    // (the LDS latency is paid once), and the second half's fragments are
    // read one per MFMA of it, so they have landed when the second chain
    // starts.
    bf16x8 k0f[KS], k1f[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      k0f[ks] = *(const __attribute__((address_space(3))) bf16x8 *)(Kt + ka[ks]);
    __builtin_amdgcn_sched_barrier(0);
    f32x16 s0v = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0f[ks], qf[ks], s0v, 0, 0, 0);
      k1f[ks] = *(const __attribute__((address_space(3))) bf16x8 *)(Kt + ka[ks] + 32 * RB);
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
    }
    if (masked) mask(s0v, 0);
    // the first 16 keys' V fragments of the first half are read beside the
    // second QK^T chain
    bf16x8 v0f[DT];
    f32x16 s1v = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s1v = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1f[ks], qf[ks], s1v, 0, 0, 0);
      if (ks < DT) {
        const bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(Vt + va[ks]));
        const bf16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(Vt + va[ks] + 8 * RB));
        v0f[ks] = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
    half_step(s0v, pa0, pa1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);   // one MFMA of the second chain
      if (ks < DT) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);   // two transposed V reads
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 1);   // five VALU ops of the softmax
    }
    if (masked) mask(s1v, 1);
    // PV of the first half, with the second half's V fragments read beside
    // it (two transposed reads per MFMA), so the last chain starts at once
    bf16x8 v1f[2][DT];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x8 vf;
        if (kk == 0) {
          vf = v0f[dt];
        } else {
          const int r0 = (16 * kk) * RB;
          const bf16x4 vlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4 *)(Vt + va[dt] + r0));
          const bf16x4 vhi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4 *)(Vt + va[dt] + r0 + 8 * RB));
          vf = __builtin_shufflevector(vlo, vhi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, kk ? pa1 : pa0, oacc[dt], 0, 0, 0);
        const int r1 = (32 + 16 * kk) * RB;
        const bf16x4 wlo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(Vt + va[dt] + r1));
        const bf16x4 whi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4 *)(Vt + va[dt] + r1 + 8 * RB));
        v1f[kk][dt] = __builtin_shufflevector(wlo, whi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    }
    half_step(s1v, pb0, pb1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1f[kk][dt], kk ? pb1 : pb0, oacc[dt], 0, 0, 0);
  };

  const int lo = W > 0 && !bidir ? max(0, q0 - W + 1) : 0;
  const int kt_lo = lo / BN;
  const int kt_hi = ((bidir ? L : q1) - 1) / BN;
  const int ntiles = kt_hi - kt_lo + 1;
  // KV split: this part takes tiles kt_hi - it for it in [it0, it1); parts
  // past the item's last tile have nothing to do (uniform per workgroup).
  // The last launched part takes any remainder, so every item's parts are
  // all launched whatever its length.
  const int span = a.kv_parts > 1 ? a.kv_span : ntiles;
  const int nparts = min((ntiles + span - 1) / span, a.kv_parts);
  if (part >= nparts) return;
  const int it0 = part * span;
  const int it1 = part == nparts - 1 ? ntiles : it0 + span;

  issue_dma(kt_hi - it0, 0);
  load_q();
  // The gate fragments of the epilogue (qrow always addresses a real row).
  // At D = 128 they are fetched now, so their latency is long hidden when
  // they are needed; at D = 64 holding them through the loop costs more than
  // fetching them after it (measured), so the epilogue fetches them.
  constexpr bool kGateEarly = D == 128;
  uint2 gw[DT][4];
  auto load_gate = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        gw[dt][i4] = *reinterpret_cast<const uint2 *>(a.gate + qrow + dt * 32 + i4 * 8 + g * 4);
  };
  if constexpr (FUSED && kGateEarly) load_gate();
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
    // Each part publishes its wave's unnormalised O fragment and per-lane
    // (reference, partial sum); the wave of the last part to arrive combines
    // all parts in part order, so the result does not depend on which
    // arrives last.  No wave waits for another.  Slot layout (floats):
    // [O element e][lane], then [reference, sum][lane].
    const int64_t item = (((int64_t)seg * a.q_blocks + qb) * a.hkv + kvh) * a.head_chunks + hc;
    constexpr int SLOT = (DT * 16 + 2) * 64;
    auto slot = [&](int p) __attribute__((always_inline)) {
      return a.part_o + ((item * a.kv_parts + p) * NW + wave) * SLOT + lane;
    };
    // The slots are written and read with device-coherent (device-scope
    // atomic) stores and loads, and a store completes only once it is visible
    // device-wide, so waiting for this wave's stores before arriving orders
    // them before the arrival.  Release/acquire fences would instead write
    // back and invalidate the whole L2 of the XCD, which its other workgroups
    // pay for in K/V refetches.
    auto st = [&](float *p, float v) __attribute__((always_inline)) {
      __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    {
      float *dst = slot(part);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) st(dst + (dt * 16 + i) * 64, oacc[dt][i]);
      st(dst + DT * 16 * 64, m_run);
      st(dst + (DT * 16 + 1) * 64, l_run);
    }
    // compiler-only fences: the relaxed atomics to other addresses stay on
    // their side of the wait
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    uint32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(a.part_cnt + item * NW + wave, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    prev = __builtin_amdgcn_readfirstlane(prev);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (prev != (uint32_t)(nparts - 1)) return;
    if (lane == 0) a.part_cnt[item * NW + wave] = 0u;   // zero again for the next launch
    auto ld = [&](const float *p) __attribute__((always_inline)) {
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };
    float m_all = -INFINITY;
    for (int p = 0; p < nparts; ++p) m_all = fmaxf(m_all, ld(slot(p) + DT * 16 * 64));
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = f32x16{};
    float l_all = 0.0f;
    for (int p = 0; p < nparts; ++p) {
      const float *src = slot(p);
      const float mp = ld(src + DT * 16 * 64);
      // a part without a reference saw no key: l = 0, O = 0
      const float sc = mp == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f((mp - m_all) * c2);
      l_all = __builtin_fmaf(sc, ld(src + (DT * 16 + 1) * 64), l_all);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = __builtin_fmaf(sc, ld(src + (dt * 16 + i) * 64), oacc[dt][i]);
    }
    m_run = m_all;
    l_run = l_all;
  }
  if constexpr (FUSED && !kGateEarly) load_gate();
  float l_lo, l_hi;
  swap32(l_run, l_lo, l_hi);
  const float l_tot = l_lo + l_hi;
  // a query whose every key is padding has l = 0: the zero row (lse = -inf)
  const float inv_l = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;

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
        float lo, hi;
        swap32(own, lo, hi);
        s1[dt * 4 + i4] = lo + hi;
      }
    const float rstd = rms_rstd(tree_sum(s1), 1.0f / (float)D, a.out_eps);
    if (qvalid) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int64_t off = qrow + dt * 32 + i4 * 8 + g * 4;
          const uint2 gv = gw[dt][i4];
          uint2 w;
          w.x = pack_bf16x2(gate_elem(o[dt][i4 * 4 + 0], rstd, bf16_lo(gv.x)),
                            gate_elem(o[dt][i4 * 4 + 1], rstd, bf16_hi(gv.x)));
          w.y = pack_bf16x2(gate_elem(o[dt][i4 * 4 + 2], rstd, bf16_lo(gv.y)),
                            gate_elem(o[dt][i4 * 4 + 3], rstd, bf16_hi(gv.y)));
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

template <int D, bool FUSED>
hipError_t launch_one(const AttnArgs &a, dim3 grid, hipStream_t stream) {
  // all LDS is static (Tile<D>::LDS_BYTES), so no dynamic allocation
  if (a.key_valid)
    hipLaunchKernelGGL((attn_fwd_kernel<D, FUSED, true>), grid, dim3(64 * NW), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<D, FUSED, false>), grid, dim3(64 * NW), 0, stream, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t *p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

}  // namespace

hipError_t launch_zero_u32(uint32_t *p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

int attn_columns_per_workgroup() { return COLS; }
int attn_waves_per_workgroup() { return NW; }
int attn_keys_per_tile() { return BN; }

hipError_t launch_attn_fwd(int head_dim, bool fused, const AttnArgs &a, hipStream_t stream) {
  const int64_t blocks = (int64_t)a.q_blocks * a.lay.num_segments * a.hkv * a.head_chunks * a.kv_parts;
  if (blocks == 0) return hipSuccess;
  if (a.kv_parts < 1 || a.kv_parts > kMaxKvParts || (a.kv_parts > 1 && (a.kv_span < 1 || !a.part_o || !a.part_cnt)))
    return hipErrorInvalidConfiguration;
  if (a.heads_per_wg < 1 || a.heads_per_wg > COLS || a.tok_per_wg < 1 || a.tok_per_wg * a.heads_per_wg > COLS)
    return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)blocks);
  if (head_dim == 128)
    return fused ? launch_one<128, true>(a, grid, stream) : launch_one<128, false>(a, grid, stream);
  return fused ? launch_one<64, true>(a, grid, stream) : launch_one<64, false>(a, grid, stream);
}

}  // namespace muse
