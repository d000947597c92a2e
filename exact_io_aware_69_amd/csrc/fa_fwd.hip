// Forward attention kernel for gfx950.
//
// Method (FlashAttention-2 review, "Proposed method"; Stanford FlashAttention
// summary, tiling and incremental softmax): the query rows are cut into
// tiles, one workgroup per (batch, head, query tile) so a single head is
// also spread over sequence length; key/value tiles stream through LDS and
// an online softmax keeps a running row max m and row sum l, rescaling the
// unnormalised output accumulator by exp(m_old - m_new). The division by l
// happens once, in the epilogue, and only the logsumexp is saved.
//
// gfx950 mapping:
//   * 4 waves per workgroup, each owns 32 query rows of a 128-row tile
//     (rows are split between waves, keys are not, so no cross-wave
//     reduction is needed).
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: lane l then holds query l % 32 and 16 keys
//     per 32-key block, so the row max / row sum are an in-lane reduction
//     plus one permlane32 swap, and the per-query rescale factor is a
//     per-lane scalar.
//   * The fp32 probabilities are rounded to bf16 in registers and used
//     directly as the B operand of O^T += V^T P^T; V^T comes out of the
//     row-major LDS tile with ds_read_tr16_b64.
//   * K/V tiles are copied HBM -> LDS with global_load_lds_dwordx4 (no
//     register staging), two LDS stages each, one barrier per tile: the next
//     tile's copy is in flight while the current one is consumed.
//   * Vector-ALU work per score is one FMA, one exp2 and one add, plus a
//     share of max3 and bf16 packing; the other waves of a SIMD (three
//     workgroups per CU at d = 128 with 32-key tiles, up to four at d = 64)
//     run their MFMAs while one wave takes its exponentials.
//   * The reference max used in the exponent is only moved when a row max
//     grows by more than 2^8 (in the exp2 domain); until then the
//     accumulator is not rescaled. The result is unchanged because O and l
//     share the reference; fp32 holds the at most 256x larger terms. The
//     default d = 64 tiles do not even take the row max of every tile: they
//     test each k-step's sum of probabilities against 2^8 instead, and take
//     the row max only when that test fails or on a row's first tile.
#include <type_traits>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {

template <int D, int BN, int WAVES, bool CAUSAL, bool SPARSE, bool DEBUG, bool DROP = false>
// Two 4-wave workgroups per CU unless the two K/V stages of one exceed half
// the LDS; three at d = 128 with 32-key tiles (not with dropout, whose
// generator needs more registers).
__global__ __launch_bounds__(64 * WAVES, (WAVES == 4 && D == 128 && BN == 32 && !DROP) ? 3
                                         : (WAVES == 4 && BN * D <= 64 * 128)          ? 2
                                                                                       : 1) void fa_fwd_kernel(const FwdParams p) {
  constexpr int BM = 32 * WAVES;  // query rows per workgroup
  static_assert(MASK_BLOCK % BN == 0 && BM <= 2 * MASK_BLOCK, "a tile spans at most one mask column, two mask rows");
  constexpr int TILEB = BN * D * 2;
  constexpr int NS = BN / 32;  // 32-key blocks per tile
  constexpr float TAU = 8.0f;  // lazy-rescale threshold (log2 domain)
  // The default d = 64 configuration moves the reference max lazily, without
  // a row max per tile (see softmax_pv); at d = 128 that measured no faster.
  constexpr bool LAZY_MAX = D == 64 && BN == 64 && WAVES == 4;
  // LDS reads issued ahead of their products (below). Not in the lazy d = 64
  // configuration (they gained nothing at d = 64, and their registers would
  // cost it the fourth wave per SIMD), nor in the 8-wave d = 128, 128-key
  // configuration, which has no registers left for them, nor in the d = 128,
  // 32-key one, whose third workgroup per CU leaves 168 registers a wave:
  // there only the K reads go ahead (KAHEAD k-steps; its registers peak in
  // the P V phase, not in the score products).
  constexpr bool AHEAD = !LAZY_MAX && !(D == 128 && BN == 128 && WAVES == 8) &&
                         !(D == 128 && BN == 32 && WAVES == 4 && !DROP);
  constexpr bool AHEAD_K = AHEAD || (D == 128 && BN == 32 && WAVES == 4 && !DROP);
  constexpr int KAHEAD = AHEAD ? 2 : 3;
  constexpr float SUM_MAX = 256.0f;  // largest probability allowed against the reference (2^TAU)
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  // Two LDS stages for K and two for V, as four separate objects: the stage
  // of every access is a compile-time constant (the loop is unrolled by
  // two), so the compiler can tell the in-flight copies from the reads and
  // does not insert waits for the copies before reading the other stage.
  __shared__ __attribute__((aligned(1024))) uint8_t k0_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t k1_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v0_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v1_raw[TILEB];
  FA_LDS uint8_t* const kst[2] = {(FA_LDS uint8_t*)k0_raw, (FA_LDS uint8_t*)k1_raw};
  FA_LDS uint8_t* const vst[2] = {(FA_LDS uint8_t*)v0_raw, (FA_LDS uint8_t*)v1_raw};

  const int tid = threadIdx.x;
  const int lane = tid & 63, h2 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform (scalar)

  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  int bh, qt;
  head_rank_order(lid, p.n_qt, p.hgrp, bh, qt);
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // longest query tiles first
  const int h = bh % p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;

  const int q_lo = qt * BM;
  const int q_last = min(q_lo + BM, N) - 1;
  const int q0 = q_lo + 32 * w;     // first query of this wave
  const int qi = q0 + (lane & 31);  // query of this lane
  int kt_end = p.n_kt;
  if (CAUSAL) kt_end = min(kt_end, q_last / BN + 1);
  // Block-sparse: the query tile spans one or two 128-row mask blocks. The
  // workgroup visits a key tile when any of them keeps it; a wave computes
  // it only when the block of its own 32 queries keeps it.
  MaskScan scan_wg, scan_w;  // kept blocks of the workgroup's mask rows, of this wave's row
  if (SPARSE) {
    const uint8_t* mh = p.mask + (size_t)h * p.nb * p.nb;
    const uint8_t* mrow0 = mh + (size_t)(q_lo / MASK_BLOCK) * p.nb;
    const uint8_t* mrow1 = mh + (size_t)(q_last / MASK_BLOCK) * p.nb;
    scan_wg.init(mrow0, mrow1 != mrow0 ? mrow1 : nullptr, 1, p.nb);
    scan_w.init(mh + (size_t)(min(q0, N - 1) / MASK_BLOCK) * p.nb, nullptr, 1, p.nb);
  }
  auto next_tile = [&](int j) __attribute__((always_inline)) {
    if (SPARSE && j < kt_end) {
      const int b = (j * BN) / MASK_BLOCK;
      const int bk = scan_wg.next_kept(b);
      if (bk != b) j = bk * (MASK_BLOCK / BN);
    }
    return j;
  };
  // Whether this wave computes tile j (< kt_end): some query of the wave
  // sees some key.
  auto wave_active = [&](int j) __attribute__((always_inline)) {
    return (!CAUSAL || j * BN <= q0 + 31) && (!SPARSE || scan_w.kept((j * BN) / MASK_BLOCK));
  };

  // Q^T fragment (B operand): lane holds Q[qi][16*kk + 8*h2 .. +7].
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + head + (size_t)min(qi, N - 1) * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld_global16(qrow + 16 * kk));
  }

  // K and V of this head as buffer resources: tail rows past N read as zero.
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const TileDMA<D, BN, WAVES> cp(w, lane);
  auto dma_kv = [&](int j, FA_LDS uint8_t* kdst, FA_LDS uint8_t* vdst) __attribute__((always_inline)) {
    cp.copy(p.k + head, head_bytes, j * BN * D * 2, kdst, w);
    cp.copy(p.v + head, head_bytes, j * BN * D * 2, vdst, w);
  };

  // Per-lane LDS offsets, computed once and opaque to the compiler, so that
  // the stage bases (compile-time constants) and the 32-key block and k-step
  // offsets fold into the instructions' offset fields: the K row of k-step
  // kk, and the two transposing reads of V^T (rows +0 and +8 of a 16-key
  // k-step; the swizzle repeats every 16 rows) for 32-column block dt.
  uint32_t kofs[D / 16], vofs[2][D / 32];
  {
    const int g = (lane >> 4) & 1, jj = lane & 15;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kofs[kk] = opaque(tile_off<D>(lane & 31, 16 * kk + 8 * h2));
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        vofs[pt][dt] = opaque(tile_off<D>(4 * h2 + (jj >> 2) + 8 * pt, 32 * dt + 16 * g + 4 * (jj & 3)));
  }

  // S^T tile = K_j Q^T from an LDS stage.
  auto scores = [&](const FA_LDS uint8_t* ks, f32x16 (&s)[NS]) __attribute__((always_inline)) {
#pragma unroll
    for (int mt = 0; mt < NS; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
    // k-step outer so consecutive MFMAs go to independent accumulators
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mt = 0; mt < NS; ++mt)
        s[mt] = mfma32(ld_lds16(ks + 32 * mt * D * 2, kofs[kk]), qf[kk], s[mt]);
    // Issue order: the K reads of the first KAHEAD k-steps, then each
    // k-step's products followed by the reads KAHEAD k-steps ahead.
    if constexpr (AHEAD_K) {
      __builtin_amdgcn_sched_group_barrier(0x100, KAHEAD * NS, 0);
#pragma unroll
      for (int kk = 0; kk < D / 16 - KAHEAD; ++kk) {
        __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, NS, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KAHEAD * NS, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  float m_run = -INFINITY;  // reference max of S * c (log2 domain)
  float l_run = 0.f;        // sum of exp2(S*c - m_run) over this lane's keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
  const float c = p.c;

  // Online softmax of one score tile and O^T += V^T P^T.
  auto softmax_pv = [&](f32x16 (&s)[NS], int j, const FA_LDS uint8_t* vs, bool need_mask)
                        __attribute__((always_inline)) {
    if (need_mask) {
      // Value r of block mt is key j*BN + 32*mt + 8*(r/4) + 4*h2 + r%4; it is
      // visible iff key <= min(N - 1, qi) (causal) or key <= N - 1.
      const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - j * BN - 4 * h2;
#pragma unroll
      for (int mt = 0; mt < NS; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (32 * mt + 8 * (r >> 2) + (r & 3) > lim) s[mt][r] = -INFINITY;
    }
    // Move the reference max to the tile's row max when that grows by more
    // than TAU (slack > 0), or when it grows at all (slack = 0).
    auto rebase = [&](float slack) __attribute__((always_inline)) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < NS; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = xhalf_max(mx) * c;
      const bool grow = mx > m_run + slack;
      const float m_new = grow ? mx : m_run;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      m_run = m_new;
    };
    // d = 128: the row max of every tile. d = 64 (vector-bound): the
    // exponentials of a k-step are taken against the current reference and
    // the reference is moved only on a row's first tile and when a
    // probability would exceed 2^TAU, which the sum of the k-step's eight
    // values shows (a value above 2^TAU, an infinity or a NaN fails the test).
    if constexpr (LAZY_MAX) {
      if (__builtin_amdgcn_ballot_w64(m_run == -INFINITY) != 0) rebase(0.f);
    } else {
      rebase(TAU);
    }
    // P^T as B operand: slot i of half h2 in k-step kk is key
    // 16*kk + 8*(i/4) + 4*h2 + i%4, i.e. value r = 8*(kk%2) + i of block kk/2.
    // V^T fragments are read one k-step ahead: the reads of k-step kk + 1
    // are issued before k-step kk's exponentials and products, so their LDS
    // latency is covered by a whole k-step of work.
    auto read_vt = [&](int kk, bf16x8 (&vT)[D / 32]) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        vT[dt] = join_tr(ld_lds_tr(vs + 16 * kk * D * 2, vofs[0][dt]), ld_lds_tr(vs + 16 * kk * D * 2, vofs[1][dt]));
    };
    bf16x8 vnext[D / 32];
    if constexpr (AHEAD) {
      read_vt(0, vnext);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      bf16x8 vT[D / 32];
      if constexpr (AHEAD) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) vT[dt] = vnext[dt];
        if (kk + 1 < BN / 16) read_vt(kk + 1, vnext);
      } else {
        read_vt(kk, vT);
      }
      const f32x16& t = s[kk >> 1];
      const int r0 = 8 * (kk & 1);
      float e[8];
      auto exps = [&]() __attribute__((always_inline)) {
        const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fast_exp2(fmaf(t[r0 + i], c, -m_use));
        return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      };
      float esum = exps();
      if constexpr (LAZY_MAX) {
        if (__builtin_amdgcn_ballot_w64(!(esum <= SUM_MAX)) != 0) {
          rebase(0.f);
          esum = exps();
        }
      }
      l_run += esum;
      if (DROP) {
        // Dropout after the row sum (the softmax is of the undropped row):
        // slots 0-3 are keys kd .. kd+3 and slots 4-7 keys kd+8 .. kd+11,
        // each four consecutive keys one generator call.
        const int kd = j * BN + 16 * kk + 4 * h2;
        uint32_t w0[4], w1[4];
        philox4x32_10((uint32_t)kd >> 2, (uint32_t)qi, (uint32_t)bh, p.drop.off, p.drop.k0, p.drop.k1, w0);
        philox4x32_10((uint32_t)(kd + 8) >> 2, (uint32_t)qi, (uint32_t)bh, p.drop.off, p.drop.k0, p.drop.k1, w1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (w0[i] < p.drop.t) e[i] = 0.f;
          if (w1[i] < p.drop.t) e[4 + i] = 0.f;
        }
      }
      const bf16x8 pb = to_bf16x8(e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) oacc[dt] = mfma32(vT[dt], pb, oacc[dt]);
      // Order within the k-step: the next k-step's transposed reads, then
      // the vector work, then this k-step's products; nothing moves across
      // k-steps (hoisting every V read of the tile would exceed the
      // register budget of two waves per SIMD).
      if (!AHEAD || kk + 1 < BN / 16) __builtin_amdgcn_sched_group_barrier(0x100, 2 * (D / 32), 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 64, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, D / 32, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  int jc = next_tile(0);
  int pl = 0;  // LDS stage of the last tile (stage 1 - pl is free afterwards)
  if (jc < kt_end) {
    bool act = wave_active(jc);
    dma_kv(jc, kst[0], vst[0]);
    wait_vmem();
    __syncthreads();
    // One step (parity P = index of the current tile mod 2): tile jc is in
    // stage P; the next visited tile is copied into stage 1-P meanwhile. Its
    // skip decisions are taken before that copy is issued, so a mask read
    // never waits behind it.
    auto step = [&](auto parity) __attribute__((always_inline)) -> bool {
      constexpr int P = decltype(parity)::value;
      const int jn = next_tile(jc + 1);
      const bool act_n = jn < kt_end && wave_active(jn);
      if (jn < kt_end) dma_kv(jn, kst[1 - P], vst[1 - P]);
      if (DEBUG && tid == 0) p.visited[((size_t)bh * p.n_qt + qt) * p.n_kt + jc] = 1;
      if (act) {
        f32x16 s[NS];
        scores(kst[P], s);
        const bool need_mask = (jc * BN + BN > N) || (CAUSAL && jc * BN + BN - 1 > q0);
        softmax_pv(s, jc, vst[P], need_mask);
      }
      // After the last tile no copy is in flight and no LDS access follows.
      // Under causal masking the waves of the lower rows skip the last key
      // tiles, so each wave goes on to its epilogue without waiting for the
      // others (jn < kt_end is the same for every wave of the workgroup).
      // Dense waves finish together and keep the barrier (measured faster).
      if (!CAUSAL || jn < kt_end) {
        wait_vmem();
        __syncthreads();
      }
      jc = jn;
      act = act_n;
      pl = P;
      return jn < kt_end;
    };
    while (step(std::integral_constant<int, 0>()) && step(std::integral_constant<int, 1>())) {
    }
  }

  // Epilogue: O = acc / l (deferred normalisation), lse = ln sum exp. O goes
  // out through this wave's slice of the LDS stage that held the tile before
  // the last (no wave reads it any more, and no copy targets it).
  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.f ? (DROP ? p.drop.scale : 1.0f) / l_tot : 0.f;
  {
    constexpr int SLICE = 2 * TILEB / WAVES;
    constexpr int PER = TILEB / SLICE;  // slices per stage buffer
    FA_LDS uint8_t* const kfree = pl ? (FA_LDS uint8_t*)k0_raw : (FA_LDS uint8_t*)k1_raw;
    FA_LDS uint8_t* const vfree = pl ? (FA_LDS uint8_t*)v0_raw : (FA_LDS uint8_t*)v1_raw;
    FA_LDS uint8_t* const slice = (w < PER ? kfree : vfree) + (w % PER) * SLICE;
    uint16_t* const obase = p.o + head + (size_t)q0 * D;
    store_tile<D / 32, false, SLICE>(oacc, inv, slice, lane, N - q0,
                                     [&](int r) __attribute__((always_inline)) { return obase + (size_t)r * D; });
  }
  if (qi < N && h2 == 0) p.lse[(size_t)bh * N + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
}

template <int D, int BN, int WAVES, bool CAUSAL, bool SPARSE, bool DEBUG, bool DROP = false>
hipError_t launch_fwd_t(const FwdParams& p, int BH, hipStream_t st) {
  const auto kernel = fa_fwd_kernel<D, BN, WAVES, CAUSAL, SPARSE, DEBUG, DROP>;
  static const int wgs = wgs_per_cu((const void*)kernel, 64 * WAVES);
  FwdParams q = p;
  // Dense causal launches interleave heads (see head_group); block-sparse
  // work per tile depends on the mask, so those keep head order.
  q.hgrp = (CAUSAL && !SPARSE) ? head_group(wgs, cus_per_xcd(), BH, p.n_qt) : 1;
  hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * p.n_qt)), dim3(64 * WAVES), 0, st, q);
  return hipGetLastError();
}

template <int D, int BN, int WAVES>
hipError_t launch_fwd_c(const FwdParams& p, int BH, bool causal, bool sparse, bool debug, hipStream_t st) {
  if (debug) {
    if (causal)
      return sparse ? launch_fwd_t<D, BN, WAVES, true, true, true>(p, BH, st)
                    : launch_fwd_t<D, BN, WAVES, true, false, true>(p, BH, st);
    return sparse ? launch_fwd_t<D, BN, WAVES, false, true, true>(p, BH, st)
                  : launch_fwd_t<D, BN, WAVES, false, false, true>(p, BH, st);
  }
  if (causal)
    return sparse ? launch_fwd_t<D, BN, WAVES, true, true, false>(p, BH, st)
                  : launch_fwd_t<D, BN, WAVES, true, false, false>(p, BH, st);
  return sparse ? launch_fwd_t<D, BN, WAVES, false, true, false>(p, BH, st)
                : launch_fwd_t<D, BN, WAVES, false, false, false>(p, BH, st);
}

// Tile configurations compiled in: (query rows per workgroup, keys per
// tile). The first is the default of fa_fwd; the others exist for the
// tile-size study (fa_fwd_tiles). Debug visit maps use the default only.
bool fwd_config_supported(int bm, int bn) {
  return (bm == 128 && (bn == 32 || bn == 64 || bn == 128)) || (bm == 256 && (bn == 64 || bn == 128));
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, int BH, int bm, int bn, bool causal, bool sparse, bool debug,
                        hipStream_t st) {
  if (debug) return launch_fwd_c<D, fwd_bn<D>(), FWD_BM / 32>(p, BH, causal, sparse, true, st);
  if (bm == 128 && bn == 32) return launch_fwd_c<D, 32, 4>(p, BH, causal, sparse, false, st);
  if (bm == 128 && bn == 64) return launch_fwd_c<D, 64, 4>(p, BH, causal, sparse, false, st);
  if (bm == 128 && bn == 128) return launch_fwd_c<D, 128, 4>(p, BH, causal, sparse, false, st);
  if (bm == 256 && bn == 64) return launch_fwd_c<D, 64, 8>(p, BH, causal, sparse, false, st);
  if (bm == 256 && bn == 128) return launch_fwd_c<D, 128, 8>(p, BH, causal, sparse, false, st);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdParams& p, int BH, int d, int bm, int bn, bool causal, bool sparse, bool debug,
                      hipStream_t st) {
  return d == 64 ? launch_fwd_d<64>(p, BH, bm, bn, causal, sparse, debug, st)
                 : launch_fwd_d<128>(p, BH, bm, bn, causal, sparse, debug, st);
}

// Forward with dropout (default tiles only).
template <int D>
hipError_t launch_fwd_dropout_d(const FwdParams& p, int BH, bool causal, bool sparse, hipStream_t st) {
  constexpr int W = FWD_BM / 32;
  if (causal)
    return sparse ? launch_fwd_t<D, fwd_bn<D>(), W, true, true, false, true>(p, BH, st)
                  : launch_fwd_t<D, fwd_bn<D>(), W, true, false, false, true>(p, BH, st);
  return sparse ? launch_fwd_t<D, fwd_bn<D>(), W, false, true, false, true>(p, BH, st)
                : launch_fwd_t<D, fwd_bn<D>(), W, false, false, false, true>(p, BH, st);
}

hipError_t launch_fwd_dropout(const FwdParams& p, int BH, int d, bool causal, bool sparse, hipStream_t st) {
  return d == 64 ? launch_fwd_dropout_d<64>(p, BH, causal, sparse, st)
                 : launch_fwd_dropout_d<128>(p, BH, causal, sparse, st);
}

// Keep mask of the dropout generator, one byte per (b*H + h, i, j): one
// thread per four consecutive keys of a row. For tests of the generator
// against an independent implementation.
__global__ __launch_bounds__(256) void fa_dropout_keep_kernel(uint8_t* __restrict__ keep, int N, int ngrp,
                                                              size_t total, Dropout dr) {
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;  // (bh, i, group)
  if (gid >= total) return;
  const int grp = (int)(gid % ngrp);
  const size_t row = gid / ngrp;  // bh * N + i
  const int i = (int)(row % N);
  const uint32_t bh = (uint32_t)(row / N);
  uint32_t w[4];
  philox4x32_10((uint32_t)grp, (uint32_t)i, bh, dr.off, dr.k0, dr.k1, w);
  uint8_t* out = keep + row * N;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = 4 * grp + e;
    if (j < N) out[j] = w[e] >= dr.t ? 1 : 0;
  }
}

hipError_t launch_dropout_keep(uint8_t* keep, int BH, int N, const Dropout& dr, hipStream_t st) {
  const int ngrp = (N + 3) / 4;
  const size_t total = (size_t)BH * N * ngrp;
  hipLaunchKernelGGL(fa_dropout_keep_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, keep, N, ngrp,
                     total, dr);
  return hipGetLastError();
}

}  // namespace fa
