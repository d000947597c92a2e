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
//     v_mfma_f32_32x32x16_bf16: lane l then holds query l % 32 and 16 keys,
//     so the row max / row sum are an in-lane reduction plus one
//     permlane32 swap, and the per-query rescale factor is a per-lane
//     scalar.
//   * The fp32 probabilities are rounded to bf16 in registers and used
//     directly as the B operand of O^T += V^T P^T; V^T comes out of the
//     row-major LDS tile with ds_read_tr16_b64.
//   * K/V tiles are double-buffered in LDS (one barrier per tile); the
//     next tile's global loads are in flight while the current one is
//     consumed.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// 16-byte chunk swizzles of a [rows][D] bf16 tile in LDS.
// K is read row-wise by 32 consecutive rows at one chunk: XOR with the row.
template <int D>
__device__ __forceinline__ uint32_t k_off(int row, int chunk) {
  constexpr int CH = D / 8;
  return (uint32_t)(row * D * 2 + ((chunk ^ (row & (CH - 1))) << 4));
}
// V is read with the transposing read: 8 rows x 64 bytes per wave. XOR the
// chunk with 4*row so that neighbouring rows land in different 64-byte
// bank groups.
template <int D>
__device__ __forceinline__ uint32_t v_off(int row, int col) {
  constexpr int CH = D / 8;
  return (uint32_t)(row * D * 2 + ((((col >> 3) ^ ((row * 4) & (CH - 1)))) << 4) + ((col & 7) << 1));
}

template <int D, int BN, bool CAUSAL, bool SPARSE, bool DEBUG>
__global__ __launch_bounds__(256, 2) void fa_fwd_kernel(const FwdParams p) {
  constexpr int BM = FWD_BM;
  constexpr int CH = D / 8;
  constexpr int TILEB = BN * D * 2;
  constexpr int LOADS = BN * CH / 256;
  static_assert(LOADS * 256 == BN * CH, "tile must split evenly over 256 threads");
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * 2 * TILEB];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h2 = lane >> 5;

  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = lid / p.n_qt;
  int qt = lid % p.n_qt;
  if (CAUSAL) qt = p.n_qt - 1 - qt;  // longest query tiles first
  const int h = bh % p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;

  const int q_lo = qt * BM;
  const int q_last = min(q_lo + BM, N) - 1;
  const int q0 = q_lo + 32 * w;          // first query of this wave
  const int qi = q0 + (lane & 31);       // query of this lane
  int kt_end = p.n_kt;
  if (CAUSAL) kt_end = min(kt_end, q_last / BN + 1);
  const uint8_t* mrow = SPARSE ? p.mask + ((size_t)h * p.nb + (q_lo / MASK_BLOCK)) * p.nb : nullptr;
  auto next_tile = [&](int j) {
    if (SPARSE)
      while (j < kt_end && mrow[(j * BN) / MASK_BLOCK] == 0) ++j;
    return j;
  };

  // Q^T fragment (B operand): lane holds Q[qi][16*kk + 8*h2 .. +7].
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow = p.q + head + (size_t)qi * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 t = {0u, 0u, 0u, 0u};
      if (qi < N) t = ld_global16(qrow + 16 * kk);
      qf[kk] = __builtin_bit_cast(bf16x8, t);
    }
  }

  const uint16_t* kg = p.k + head;
  const uint16_t* vg = p.v + head;
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int idx = u * 256 + tid;
      const int row = idx / CH, c = idx % CH;
      const int key = j * BN + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < N) {
        a = ld_global16(kg + (size_t)key * D + 8 * c);
        b = ld_global16(vg + (size_t)key * D + 8 * c);
      }
      kreg[u] = a;
      vreg[u] = b;
    }
  };
  auto swrite = [&](int stage) {
    FA_LDS uint8_t* ks = smem + stage * 2 * TILEB;
    FA_LDS uint8_t* vs = ks + TILEB;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int idx = u * 256 + tid;
      const int row = idx / CH, c = idx % CH;
      st_lds16(ks, k_off<D>(row, c), kreg[u]);
      st_lds16(vs, v_off<D>(row, 8 * c), vreg[u]);
    }
  };

  float m_run = -INFINITY;  // running max of S * c (log2 domain)
  float l_run = 0.f;        // running sum of exp2(S*c - m_run), this lane's keys
  f32x16 oacc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;

  const float c = p.c;
  int j = next_tile(0);
  if (j < kt_end) {
    gload(j);
    swrite(0);
  }
  __syncthreads();
  int stage = 0;
  while (j < kt_end) {
    const int jn = next_tile(j + 1);
    if (jn < kt_end) gload(jn);
    const int kbase = j * BN;
    if (DEBUG && tid == 0) p.visited[((size_t)bh * p.n_qt + qt) * p.n_kt + j] = 1;
    // A wave whose 32 queries all precede the tile's first key skips it.
    const bool wave_active = !CAUSAL || kbase <= q0 + 31;
    if (wave_active) {
      const FA_LDS uint8_t* ks = smem + stage * 2 * TILEB;
      const FA_LDS uint8_t* vs = ks + TILEB;
      f32x16 s[BN / 32];
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[mt][r] = 0.f;
        const int row = 32 * mt + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[mt] = mfma32(ld_lds16(ks, k_off<D>(row, 2 * kk + h2)), qf[kk], s[mt]);
      }
      // Mask only tiles that straddle the diagonal or the end of the sequence.
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > q0);
      if (need_mask) {
#pragma unroll
        for (int mt = 0; mt < BN / 32; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kbase + 32 * mt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (key >= N || (CAUSAL && key > qi)) s[mt][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = xhalf_max(mx);
      const float m_new = fmaxf(m_run, mx * c);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = fast_exp2(fmaf(s[mt][r], c, -m_use));
          s[mt][r] = e;
          lsum += e;
        }
      l_run = fmaf(l_run, alpha, lsum);
      m_run = m_new;
      if (__builtin_amdgcn_ballot_w64(alpha != 1.0f) != 0) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      }
      // P^T as B operand: slot i of half h2 in k-step kk is key
      // 16*kk + 8*(i/4) + 4*h2 + i%4, i.e. value r = 8*(kk%2) + i of tile kk/2.
      bf16x8 pb[BN / 16];
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        const f32x16& t = s[kk >> 1];
        const int r0 = 8 * (kk & 1);
        pb[kk] = to_bf16x8(t[r0], t[r0 + 1], t[r0 + 2], t[r0 + 3], t[r0 + 4], t[r0 + 5], t[r0 + 6], t[r0 + 7]);
      }
      // V^T as A operand via transposing reads: the lane group of 16 picks
      // rows 16*kk + 4*h2 (+8) and columns 32*dt + 16*((lane/16)&1).
      const int g = lane >> 4, jj = lane & 15;
      const int vrow = 4 * h2 + (jj >> 2);
      const int vcol = 16 * (g & 1) + 4 * (jj & 3);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int kk = 0; kk < BN / 16; ++kk) {
          const s16x4 lo = ld_lds_tr(vs, v_off<D>(16 * kk + vrow, 32 * dt + vcol));
          const s16x4 hi = ld_lds_tr(vs, v_off<D>(16 * kk + 8 + vrow, 32 * dt + vcol));
          oacc[dt] = mfma32(join_tr(lo, hi), pb[kk], oacc[dt]);
        }
      }
    }
    if (jn < kt_end) swrite(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    j = jn;
  }

  // Epilogue: O = acc / l (deferred normalisation), lse = ln sum exp.
  const float l_tot = xhalf_sum(l_run);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (qi < N) {
    uint16_t* orow = p.o + head + (size_t)qi * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * dt + 8 * rg + 4 * h2;
        *reinterpret_cast<u32x2*>(orow + d0) =
            pack4_bf16(oacc[dt][4 * rg] * inv, oacc[dt][4 * rg + 1] * inv, oacc[dt][4 * rg + 2] * inv,
                       oacc[dt][4 * rg + 3] * inv);
      }
    if (h2 == 0) p.lse[(size_t)bh * N + qi] = l_tot > 0.f ? (m_run + log2f(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool SPARSE, bool DEBUG>
hipError_t launch_fwd_t(const FwdParams& p, int BH, hipStream_t st) {
  const dim3 grid((unsigned)(BH * p.n_qt));
  hipLaunchKernelGGL((fa_fwd_kernel<D, FWD_BN, CAUSAL, SPARSE, DEBUG>), grid, dim3(256), 0, st, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_fwd_d(const FwdParams& p, int BH, bool causal, bool sparse, bool debug, hipStream_t st) {
  if (debug) {
    if (causal) return sparse ? launch_fwd_t<D, true, true, true>(p, BH, st) : launch_fwd_t<D, true, false, true>(p, BH, st);
    return sparse ? launch_fwd_t<D, false, true, true>(p, BH, st) : launch_fwd_t<D, false, false, true>(p, BH, st);
  }
  if (causal) return sparse ? launch_fwd_t<D, true, true, false>(p, BH, st) : launch_fwd_t<D, true, false, false>(p, BH, st);
  return sparse ? launch_fwd_t<D, false, true, false>(p, BH, st) : launch_fwd_t<D, false, false, false>(p, BH, st);
}

hipError_t launch_fwd(const FwdParams& p, int BH, int d, bool causal, bool sparse, bool debug, hipStream_t st) {
  return d == 64 ? launch_fwd_d<64>(p, BH, causal, sparse, debug, st)
                 : launch_fwd_d<128>(p, BH, causal, sparse, debug, st);
}

}  // namespace fa
