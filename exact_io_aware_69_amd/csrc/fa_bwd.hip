// Backward attention kernels for gfx950.
//
// Method (Stanford FlashAttention summary: the forward keeps the softmax
// normalisation statistic so the backward recomputes attention on chip
// instead of reading a stored N x N matrix; FlashAttention-2 review,
// "Proposed method": parallel over sequence length, causal blocks skipped).
// With P = exp(S - lse) recomputed per tile, the gradient is
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_k dO_ik O_ik,
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Three kernels, enqueued in order on one stream:
//   1. fa_bwd_pre_kernel   D = rowsum(dO o O) into the workspace;
//   2. fa_bwd_dkdv_kernel  one workgroup per (batch, head, 128-key tile),
//                          streaming 64-row query tiles; dK, dV stay in
//                          registers for the whole sweep;
//   3. fa_bwd_dq_kernel    one workgroup per (batch, head, 128-query tile),
//                          streaming 64-row key tiles (recomputes S and dP).
// No atomics: every output element is written once, so results are
// deterministic.
#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// ------------------------------------------------------------------ D = rowsum(dO o O)
template <int D>
__global__ __launch_bounds__(256) void fa_bwd_pre_kernel(const uint16_t* __restrict__ o,
                                                         const uint16_t* __restrict__ dO,
                                                         float* __restrict__ Dvec, size_t rows) {
  constexpr int CH = D / 8;      // lanes per row, 8 elements each
  constexpr int RPB = 256 / CH;  // rows per workgroup
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / CH;
  const int c = threadIdx.x % CH;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = ld_global16(o + row * D + 8 * c);
    const u32x4 b = ld_global16(dO + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc = fmaf(__uint_as_float(a[i] << 16), __uint_as_float(b[i] << 16), acc);
      acc = fmaf(__uint_as_float(a[i] & 0xFFFF0000u), __uint_as_float(b[i] & 0xFFFF0000u), acc);
    }
  }
#pragma unroll
  for (int off = CH / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) Dvec[row] = acc;
}

// ------------------------------------------------------------------ dK, dV
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG>
__global__ __launch_bounds__(256, 1) void fa_bwd_dkdv_kernel(const BwdParams p) {
  constexpr int BNK = BWD_KV_BN;  // keys per workgroup (32 per wave)
  constexpr int BMQ = BWD_KV_BM;  // query rows per streamed tile
  constexpr int CH = D / 8;
  constexpr int TILEB = BMQ * D * 2;
  constexpr int LOADS = BMQ * CH / 256;
  constexpr int STAGEB = 2 * TILEB + 2 * BMQ * 4;  // Q, dO, lse*log2e, D
  static_assert(LOADS * 256 == BMQ * CH, "tile must split evenly over 256 threads");
  static_assert(BNK == MASK_BLOCK, "one key tile per mask column");
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * STAGEB];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h2 = lane >> 5;
  const int n_kt = (p.N + BNK - 1) / BNK;
  const int n_qt = (p.N + BMQ - 1) / BMQ;
  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = lid / n_kt;
  const int jt = lid % n_kt;  // ascending: for causal the first key tiles see the most queries
  const int h = bh % p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const int kb = jt * BNK;
  const int k0w = kb + 32 * w;           // first key of this wave
  const int key = k0w + (lane & 31);     // key of this lane

  // K and V rows of this lane's key as B operands (d slots 16*kk + 8*h2 + i).
  bf16x8 kf[D / 16], vf[D / 16];
  {
    const uint16_t* kr = p.k + head + (size_t)key * D + 8 * h2;
    const uint16_t* vr = p.v + head + (size_t)key * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (key < N) {
        a = ld_global16(kr + 16 * kk);
        b = ld_global16(vr + 16 * kk);
      }
      kf[kk] = __builtin_bit_cast(bf16x8, a);
      vf[kk] = __builtin_bit_cast(bf16x8, b);
    }
  }
  f32x16 dkt[D / 32], dvt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dkt[dt][r] = 0.f;
      dvt[dt][r] = 0.f;
    }

  const int it_begin = CAUSAL ? kb / BMQ : 0;
  const uint8_t* mcol = SPARSE ? p.mask + (size_t)h * p.nb * p.nb + jt : nullptr;
  auto next_tile = [&](int i) {
    if (SPARSE)
      while (i < n_qt && mcol[(size_t)((i * BMQ) / MASK_BLOCK) * p.nb] == 0) ++i;
    return i;
  };

  const uint16_t* qg = p.q + head;
  const uint16_t* dog = p.dO + head;
  const float* lseg = p.lse + (size_t)bh * N;
  const float* Dg = p.Dvec + (size_t)bh * N;
  u32x4 qreg[LOADS], doreg[LOADS];
  float lreg = 0.f, dreg = 0.f;
  auto gload = [&](int i) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int idx = u * 256 + tid;
      const int row = idx / CH, c = idx % CH;
      const int q = i * BMQ + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (q < N) {
        a = ld_global16(qg + (size_t)q * D + 8 * c);
        b = ld_global16(dog + (size_t)q * D + 8 * c);
      }
      qreg[u] = a;
      doreg[u] = b;
    }
    if (tid < BMQ) {
      const int q = i * BMQ + tid;
      // Rows past N or with no visible key get +inf so that P = exp2(. - inf) = 0.
      float l2 = INFINITY, dd = 0.f;
      if (q < N) {
        const float l = lseg[q];
        l2 = l == -INFINITY ? INFINITY : l * kLog2e;
        dd = Dg[q];
      }
      lreg = l2;
      dreg = dd;
    }
  };
  auto swrite = [&](int stage) {
    FA_LDS uint8_t* qs = smem + stage * STAGEB;
    FA_LDS uint8_t* dos = qs + TILEB;
    FA_LDS float* ls = (FA_LDS float*)(dos + TILEB);
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int idx = u * 256 + tid;
      const int row = idx / CH, c = idx % CH;
      st_lds16(qs, tile_off<D>(row, 8 * c), qreg[u]);
      st_lds16(dos, tile_off<D>(row, 8 * c), doreg[u]);
    }
    if (tid < BMQ) {
      ls[tid] = lreg;
      ls[BMQ + tid] = dreg;
    }
  };

  const float c = p.c;
  int i = next_tile(it_begin);
  if (i < n_qt) {
    gload(i);
    swrite(0);
  }
  __syncthreads();
  int stage = 0;
  const int g = lane >> 4, jj = lane & 15;
  const int trow = 4 * h2 + (jj >> 2);
  const int tcol = 16 * (g & 1) + 4 * (jj & 3);
  while (i < n_qt) {
    const int in = next_tile(i + 1);
    if (in < n_qt) gload(in);
    if (DEBUG && tid == 0) p.visited_kv[((size_t)bh * n_kt + jt) * n_qt + i] = 1;
    const FA_LDS uint8_t* qs = smem + stage * STAGEB;
    const FA_LDS uint8_t* dos = qs + TILEB;
    const FA_LDS float* ls = (const FA_LDS float*)(dos + TILEB);
#pragma unroll
    for (int qb = 0; qb < BMQ / 32; ++qb) {
      const int qbase = i * BMQ + 32 * qb;
      if (CAUSAL && qbase + 31 < k0w) continue;  // every query of the block precedes every key of the wave
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[r] = 0.f;
        dp[r] = 0.f;
      }
      const int arow = 32 * qb + (lane & 31);
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32(ld_lds16(qs, tile_off<D>(arow, 16 * kk + 8 * h2)), kf[kk], s);
        dp = mfma32(ld_lds16(dos, tile_off<D>(arow, 16 * kk + 8 * h2)), vf[kk], dp);
      }
      // value r of this lane is query qbase + 8*(r/4) + 4*h2 + r%4, key `key`
      const bool need_mask = CAUSAL && (k0w + 31 > qbase);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int ql = 32 * qb + 8 * rg + 4 * h2;
        const f32x4 l4 = *reinterpret_cast<const FA_LDS f32x4*>(ls + ql);
        const f32x4 d4 = *reinterpret_cast<const FA_LDS f32x4*>(ls + BMQ + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * rg + e;
          float pe = fast_exp2(fmaf(s[r], c, -l4[e]));
          if (need_mask && key > qbase + 8 * rg + 4 * h2 + e) pe = 0.f;
          s[r] = pe;
          dp[r] = pe * (dp[r] - d4[e]);
        }
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 8 * ks;
        pb[ks] = to_bf16x8(s[r0], s[r0 + 1], s[r0 + 2], s[r0 + 3], s[r0 + 4], s[r0 + 5], s[r0 + 6], s[r0 + 7]);
        dsb[ks] = to_bf16x8(dp[r0], dp[r0 + 1], dp[r0 + 2], dp[r0 + 3], dp[r0 + 4], dp[r0 + 5], dp[r0 + 6], dp[r0 + 7]);
      }
      // dV^T += dO^T P and dK^T += Q^T dS; query slots of k-step ks are
      // 16*ks + 8*(i/4) + 4*h2 + i%4 on both operands.
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int rr = 32 * qb + 16 * ks + trow;
          const int cc = 32 * dt + tcol;
          const bf16x8 doT = join_tr(ld_lds_tr(dos, tile_off<D>(rr, cc)), ld_lds_tr(dos, tile_off<D>(rr + 8, cc)));
          dvt[dt] = mfma32(doT, pb[ks], dvt[dt]);
          const bf16x8 qT = join_tr(ld_lds_tr(qs, tile_off<D>(rr, cc)), ld_lds_tr(qs, tile_off<D>(rr + 8, cc)));
          dkt[dt] = mfma32(qT, dsb[ks], dkt[dt]);
        }
      }
    }
    if (in < n_qt) swrite(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    i = in;
  }

  if (key < N) {
    uint16_t* dkr = p.dk + head + (size_t)key * D;
    uint16_t* dvr = p.dv + head + (size_t)key * D;
    const float sc = p.scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * dt + 8 * rg + 4 * h2;
        *reinterpret_cast<u32x2*>(dkr + d0) = pack4_bf16(dkt[dt][4 * rg] * sc, dkt[dt][4 * rg + 1] * sc,
                                                         dkt[dt][4 * rg + 2] * sc, dkt[dt][4 * rg + 3] * sc);
        *reinterpret_cast<u32x2*>(dvr + d0) =
            pack4_bf16(dvt[dt][4 * rg], dvt[dt][4 * rg + 1], dvt[dt][4 * rg + 2], dvt[dt][4 * rg + 3]);
      }
  }
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG>
__global__ __launch_bounds__(256, 1) void fa_bwd_dq_kernel(const BwdParams p) {
  constexpr int BM = BWD_Q_BM;
  constexpr int BN = BWD_Q_BN;
  constexpr int CH = D / 8;
  constexpr int TILEB = BN * D * 2;
  constexpr int LOADS = BN * CH / 256;
  static_assert(LOADS * 256 == BN * CH, "tile must split evenly over 256 threads");
  __shared__ __attribute__((aligned(16))) uint8_t smem_raw[2 * 2 * TILEB];
  FA_LDS uint8_t* smem = (FA_LDS uint8_t*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, h2 = lane >> 5;
  const int n_qt = (p.N + BM - 1) / BM;
  const int n_kt = (p.N + BN - 1) / BN;
  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  const int bh = lid / n_qt;
  int qt = lid % n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;
  const int h = bh % p.H;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const int q_lo = qt * BM;
  const int q_last = min(q_lo + BM, N) - 1;
  const int q0 = q_lo + 32 * w;
  const int qi = q0 + (lane & 31);
  int kt_end = n_kt;
  if (CAUSAL) kt_end = min(kt_end, q_last / BN + 1);
  const uint8_t* mrow = SPARSE ? p.mask + ((size_t)h * p.nb + (q_lo / MASK_BLOCK)) * p.nb : nullptr;
  auto next_tile = [&](int j) {
    if (SPARSE)
      while (j < kt_end && mrow[(j * BN) / MASK_BLOCK] == 0) ++j;
    return j;
  };

  bf16x8 qf[D / 16], dof[D / 16];
  {
    const uint16_t* qr = p.q + head + (size_t)qi * D + 8 * h2;
    const uint16_t* dr = p.dO + head + (size_t)qi * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (qi < N) {
        a = ld_global16(qr + 16 * kk);
        b = ld_global16(dr + 16 * kk);
      }
      qf[kk] = __builtin_bit_cast(bf16x8, a);
      dof[kk] = __builtin_bit_cast(bf16x8, b);
    }
  }
  float lse2 = INFINITY, Dq = 0.f;
  if (qi < N) {
    const float l = p.lse[(size_t)bh * N + qi];
    lse2 = l == -INFINITY ? INFINITY : l * kLog2e;
    Dq = p.Dvec[(size_t)bh * N + qi];
  }
  f32x16 dqt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[dt][r] = 0.f;

  const uint16_t* kg = p.k + head;
  const uint16_t* vg = p.v + head;
  u32x4 kreg[LOADS], vreg[LOADS];
  auto gload = [&](int j) {
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int idx = u * 256 + tid;
      const int row = idx / CH, c = idx % CH;
      const int kr = j * BN + row;
      u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
      if (kr < N) {
        a = ld_global16(kg + (size_t)kr * D + 8 * c);
        b = ld_global16(vg + (size_t)kr * D + 8 * c);
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
      st_lds16(ks, tile_off<D>(row, 8 * c), kreg[u]);
      st_lds16(vs, tile_off<D>(row, 8 * c), vreg[u]);
    }
  };

  const float c = p.c;
  int j = next_tile(0);
  if (j < kt_end) {
    gload(j);
    swrite(0);
  }
  __syncthreads();
  int stage = 0;
  const int g = lane >> 4, jj = lane & 15;
  const int trow = 4 * h2 + (jj >> 2);
  const int tcol = 16 * (g & 1) + 4 * (jj & 3);
  while (j < kt_end) {
    const int jn = next_tile(j + 1);
    if (jn < kt_end) gload(jn);
    const int kbase = j * BN;
    if (DEBUG && tid == 0) p.visited_q[((size_t)bh * n_qt + qt) * n_kt + j] = 1;
    const bool wave_active = !CAUSAL || kbase <= q0 + 31;
    if (wave_active) {
      const FA_LDS uint8_t* ks = smem + stage * 2 * TILEB;
      const FA_LDS uint8_t* vs = ks + TILEB;
      f32x16 s[BN / 32], dp[BN / 32];
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[mt][r] = 0.f;
          dp[mt][r] = 0.f;
        }
        const int row = 32 * mt + (lane & 31);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s[mt] = mfma32(ld_lds16(ks, tile_off<D>(row, 16 * kk + 8 * h2)), qf[kk], s[mt]);
          dp[mt] = mfma32(ld_lds16(vs, tile_off<D>(row, 16 * kk + 8 * h2)), dof[kk], dp[mt]);
        }
      }
      const bool need_mask = (kbase + BN > N) || (CAUSAL && kbase + BN - 1 > q0);
#pragma unroll
      for (int mt = 0; mt < BN / 32; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pe = fast_exp2(fmaf(s[mt][r], c, -lse2));
          if (need_mask) {
            const int kr = kbase + 32 * mt + 8 * (r >> 2) + 4 * h2 + (r & 3);
            if (kr >= N || (CAUSAL && kr > qi)) pe = 0.f;
          }
          dp[mt][r] = pe * (dp[mt][r] - Dq);
        }
      // dQ^T += K^T dS^T; key slots of k-step kk are 16*kk + 8*(i/4) + 4*h2 + i%4.
#pragma unroll
      for (int kk = 0; kk < BN / 16; ++kk) {
        const f32x16& t = dp[kk >> 1];
        const int r0 = 8 * (kk & 1);
        const bf16x8 dsb = to_bf16x8(t[r0], t[r0 + 1], t[r0 + 2], t[r0 + 3], t[r0 + 4], t[r0 + 5], t[r0 + 6], t[r0 + 7]);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const int rr = 16 * kk + trow;
          const int cc = 32 * dt + tcol;
          const bf16x8 kT = join_tr(ld_lds_tr(ks, tile_off<D>(rr, cc)), ld_lds_tr(ks, tile_off<D>(rr + 8, cc)));
          dqt[dt] = mfma32(kT, dsb, dqt[dt]);
        }
      }
    }
    if (jn < kt_end) swrite(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    j = jn;
  }

  if (qi < N) {
    uint16_t* dqr = p.dq + head + (size_t)qi * D;
    const float sc = p.scale;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * dt + 8 * rg + 4 * h2;
        *reinterpret_cast<u32x2*>(dqr + d0) = pack4_bf16(dqt[dt][4 * rg] * sc, dqt[dt][4 * rg + 1] * sc,
                                                         dqt[dt][4 * rg + 2] * sc, dqt[dt][4 * rg + 3] * sc);
      }
  }
}

// ------------------------------------------------------------------ launchers
// stages: bit 0 = D preprocess, bit 1 = dK/dV kernel, bit 2 = dQ kernel.
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG>
hipError_t launch_bwd_t(const BwdParams& p, int BH, int stages, hipStream_t st) {
  if (stages & 1) {
    const size_t rows = (size_t)BH * p.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((fa_bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, st, p.o,
                       p.dO, p.Dvec, rows);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 2) {
    const int n_kt1 = (p.N + BWD_KV_BN - 1) / BWD_KV_BN;
    hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, CAUSAL, SPARSE, DEBUG>), dim3((unsigned)(BH * n_kt1)), dim3(256), 0,
                       st, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const int n_qt2 = (p.N + BWD_Q_BM - 1) / BWD_Q_BM;
    hipLaunchKernelGGL((fa_bwd_dq_kernel<D, CAUSAL, SPARSE, DEBUG>), dim3((unsigned)(BH * n_qt2)), dim3(256), 0, st,
                       p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, int BH, bool causal, bool sparse, bool debug, int stages, hipStream_t st) {
  if (debug) {
    if (causal) return sparse ? launch_bwd_t<D, true, true, true>(p, BH, stages, st) : launch_bwd_t<D, true, false, true>(p, BH, stages, st);
    return sparse ? launch_bwd_t<D, false, true, true>(p, BH, stages, st) : launch_bwd_t<D, false, false, true>(p, BH, stages, st);
  }
  if (causal) return sparse ? launch_bwd_t<D, true, true, false>(p, BH, stages, st) : launch_bwd_t<D, true, false, false>(p, BH, stages, st);
  return sparse ? launch_bwd_t<D, false, true, false>(p, BH, stages, st) : launch_bwd_t<D, false, false, false>(p, BH, stages, st);
}

hipError_t launch_bwd(const BwdParams& p, int BH, int d, bool causal, bool sparse, bool debug, int stages,
                      hipStream_t st) {
  return d == 64 ? launch_bwd_d<64>(p, BH, causal, sparse, debug, stages, st)
                 : launch_bwd_d<128>(p, BH, causal, sparse, debug, stages, st);
}

}  // namespace fa
