// FlashAttention-1-style forward for gfx950: the work partitioning that
// FlashAttention-2 replaced, kept as a measured ablation (FlashAttention-2
// review: Abstract, items (1)-(3), and "Research questions", RQ2 on how much
// the partitioning and the non-matmul FLOPs cost; FlashAttention-1 reaches
// 25-40% of peak where FlashAttention-2 reaches 50-73% on A100).
//
// What differs from the IO-aware forward (fa_fwd.hip), by design:
//   * parallelism over (batch, head) only: one workgroup per head, which
//     walks every query tile of the head itself (no sequence parallelism).
//     With G > 1 query-tile groups the head's 32-row query tiles are dealt
//     round-robin to G workgroups (tile i to group i mod G), which adds the
//     sequence parallelism of FlashAttention-2 (its item (1)) and nothing
//     else, so the two can be measured apart;
//   * loop order: K/V tiles outside, query tiles inside. The running output,
//     max and sum of every query row live in a device workspace and are read
//     and written back once per K/V tile;
//   * the waves split the keys of a tile (32 keys each), so the row max, the
//     row sum and the partial P V products are combined across the waves
//     through LDS with barriers;
//   * eager normalisation: the stored output is divided by the running sum
//     after every K/V tile (O_new = (l_old e^(m_old - m_new) O_old + P V) /
//     l_new), as in the incremental softmax written for one tile at a time.
// Same results as fa_fwd up to rounding.
#include <stdint.h>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {

struct Fa1Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  float* ows;  // running output, fp32 [B*H][N][D]
  float* mws;  // running max (log2 domain), fp32 [B*H][4 waves][N]
  float* lws;  // running sum, fp32 [B*H][4 waves][N]
  int N;
  int G;    // query-tile groups per head (1 = one workgroup per head)
  float c;  // scale * log2(e)
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fa_fwd_fa1_kernel(const Fa1Params p) {
  constexpr int BNK = 128;  // keys per K/V tile, 32 per wave
  constexpr int TILEB = BNK * D * 2;
  constexpr int DT = D / 32;
  __shared__ __attribute__((aligned(1024))) uint8_t k_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v_raw[TILEB];
  __shared__ __attribute__((aligned(16))) float opart[4 * DT * 16 * 64];  // [wave][dt][r][lane]
  __shared__ float mred[4][32];
  __shared__ float lred[4][32];
  FA_LDS uint8_t* const ks = (FA_LDS uint8_t*)k_raw;
  FA_LDS uint8_t* const vs = (FA_LDS uint8_t*)v_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63, h2 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = p.G;
  const int bh = blockIdx.x / G, grp = blockIdx.x % G;
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  float* Ow = p.ows + head;
  float* mw = p.mws + ((size_t)bh * 4 + w) * N;
  float* lw = p.lws + ((size_t)bh * 4 + w) * N;
  const int n_q = (N + 31) / 32;
  // Query tiles grp, grp + G, ... (the host keeps G <= n_q, so there is at
  // least one); under causal masking only the K/V tiles up to the last of
  // them are visible.
  const int i_last = grp + (n_q - 1 - grp) / G * G;
  const int n_kt = CAUSAL ? min((N + BNK - 1) / BNK, (32 * i_last + 31) / BNK + 1) : (N + BNK - 1) / BNK;
  const float c = p.c;
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const TileDMA<D, BNK> cp(w, lane);
  const int g = lane >> 4, jj = lane & 15;
  const int vrow = 4 * h2 + (jj >> 2);
  const int vcol = 16 * (g & 1) + 4 * (jj & 3);

  for (int jt = 0; jt < n_kt; ++jt) {
    __syncthreads();  // every wave is done with the previous K/V tile
    cp.copy(p.k + head, head_bytes, jt * BNK * D * 2, ks, w);  // rows past N read as zero
    cp.copy(p.v + head, head_bytes, jt * BNK * D * 2, vs, w);
    wait_vmem();
    __syncthreads();
    const int kw = jt * BNK + 32 * w;  // first key of this wave
    const int i_min = CAUSAL ? (jt * BNK) / 32 : 0;  // earlier query tiles see none of these keys
    const int i_begin = i_min + ((grp - i_min) % G + G) % G;
    for (int i = i_begin; i < n_q; i += G) {
      const int qi = 32 * i + (lane & 31);
      // Q^T fragments (B operand), read again for every K/V tile.
      bf16x8 qf[D / 16];
      const uint16_t* qrow = p.q + head + (size_t)min(qi, N - 1) * D + 8 * h2;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) qf[kk] = __builtin_bit_cast(bf16x8, ld_global16(qrow + 16 * kk));
      // S^T = K_w Q^T for this wave's 32 keys; value r is key kw + 8*(r/4) + 4*h2 + r%4.
      f32x16 s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        s = mfma32(ld_lds16(ks, tile_off<D>(32 * w + (lane & 31), 16 * kk + 8 * h2)), qf[kk], s);
      const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - kw - 4 * h2;
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
        mx = fmaxf(mx, s[r]);
      }
      mx = xhalf_max(mx) * c;
      if (h2 == 0) mred[w][lane & 31] = mx;
      __syncthreads();
      const float m_tile =
          fmaxf(fmaxf(mred[0][lane & 31], mred[1][lane & 31]), fmaxf(mred[2][lane & 31], mred[3][lane & 31]));
      const bool first = jt == 0;  // every row sees key tile 0 first (under causal too)
      const float m_old = (first || qi >= N) ? -INFINITY : mw[qi];
      const float l_old = (first || qi >= N) ? 0.f : lw[qi];
      const float m_new = fmaxf(m_old, m_tile);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      float e[16], ls = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        e[r] = fast_exp2(fmaf(s[r], c, -m_use));
        ls += e[r];
      }
      ls = xhalf_sum(ls);
      if (h2 == 0) lred[w][lane & 31] = ls;
      // O^T partial = V_w^T P^T over this wave's 32 keys (two 16-key steps).
      f32x16 oacc[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] = 0.f;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const bf16x8 pb = to_bf16x8(e[8 * kk], e[8 * kk + 1], e[8 * kk + 2], e[8 * kk + 3], e[8 * kk + 4],
                                    e[8 * kk + 5], e[8 * kk + 6], e[8 * kk + 7]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const int rr = 32 * w + 16 * kk;
          const bf16x8 vT = join_tr(ld_lds_tr(vs, tile_off<D>(rr + vrow, 32 * dt + vcol)),
                                    ld_lds_tr(vs, tile_off<D>(rr + 8 + vrow, 32 * dt + vcol)));
          oacc[dt] = mfma32(vT, pb, oacc[dt]);
        }
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) opart[((w * DT + dt) * 16 + r) * 64 + lane] = oacc[dt][r];
      __syncthreads();
      const float l_tile = (lred[0][lane & 31] + lred[1][lane & 31]) + (lred[2][lane & 31] + lred[3][lane & 31]);
      const float alpha = m_old == -INFINITY ? 0.f : fast_exp2(m_old - m_use);
      const float l_new = l_old * alpha + l_tile;
      const float inv = l_new > 0.f ? 1.0f / l_new : 0.f;
      // Wave w combines and normalises the d-slice 32w .. 32w+31 of the rows.
      if (w < DT && qi < N) {
        const int dt = w;
        float* orow = Ow + (size_t)qi * D;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int d0 = 32 * dt + 8 * rg + 4 * h2;
          f32x4 old = {0.f, 0.f, 0.f, 0.f};
          if (!first) old = *reinterpret_cast<const f32x4*>(orow + d0);
          f32x4 nw;
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            const int r = 4 * rg + e2;
            float sum = 0.f;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) sum += opart[((ww * DT + dt) * 16 + r) * 64 + lane];
            nw[e2] = (old[e2] * l_old * alpha + sum) * inv;
          }
          *reinterpret_cast<f32x4*>(orow + d0) = nw;
        }
      }
      if (qi < N && h2 == 0) {
        mw[qi] = m_new;
        lw[qi] = l_new;
      }
      __syncthreads();  // mred, lred, opart are reused by the next query tile
    }
  }
  // O (already normalised) to bf16, lse = ln(sum) + max.
  for (int i = grp; i < n_q; i += G) {
    const int qi = 32 * i + (lane & 31);
    if (qi >= N) continue;
    if (w < DT) {
      const float* orow = Ow + (size_t)qi * D;
      uint16_t* out = p.o + head + (size_t)qi * D;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = 32 * w + 8 * rg + 4 * h2;
        const f32x4 x = *reinterpret_cast<const f32x4*>(orow + d0);
        *reinterpret_cast<u32x2*>(out + d0) = pack4_bf16(x[0], x[1], x[2], x[3]);
      }
    }
    if (w == 0 && h2 == 0) {
      const float l = lw[qi];
      p.lse[(size_t)bh * N + qi] = l > 0.f ? (mw[qi] + log2f(l)) * kLn2 : -INFINITY;
    }
  }
}

size_t fa1_workspace_bytes(int B, int H, int N, int d) {
  const size_t rows = (size_t)B * H * N;
  const size_t o_bytes = (rows * d * 4 + 255) & ~(size_t)255;
  const size_t ml_bytes = (rows * 4 * 4 + 255) & ~(size_t)255;
  return o_bytes + 2 * ml_bytes;
}

hipError_t launch_fa1(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int H,
                      int N, int d, bool causal, float scale, int groups, void* workspace, hipStream_t st) {
  Fa1Params p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  const size_t rows = (size_t)B * H * N;
  const size_t o_bytes = (rows * d * 4 + 255) & ~(size_t)255;
  const size_t ml_bytes = (rows * 4 * 4 + 255) & ~(size_t)255;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  p.ows = reinterpret_cast<float*>(ws);
  p.mws = reinterpret_cast<float*>(ws + o_bytes);
  p.lws = reinterpret_cast<float*>(ws + o_bytes + ml_bytes);
  p.N = N;
  p.G = min(groups, (N + 31) / 32);
  p.c = scale * kLog2e;
  const dim3 grid((unsigned)(B * H * p.G)), block(256);
  if (d == 64) {
    if (causal) hipLaunchKernelGGL((fa_fwd_fa1_kernel<64, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fa_fwd_fa1_kernel<64, false>), grid, block, 0, st, p);
  } else {
    if (causal) hipLaunchKernelGGL((fa_fwd_fa1_kernel<128, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((fa_fwd_fa1_kernel<128, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace fa
