// Backward attention kernels for gfx950.
//
// Method (Stanford FlashAttention summary: the forward keeps the softmax
// normalisation statistic so the backward recomputes attention on chip
// instead of reading a stored N x N matrix; FlashAttention-2 review,
// "Proposed method": parallel over sequence length, causal blocks skipped).
// With P = exp(S - lse) recomputed per tile, the gradient is
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = sum_k dO_ik O_ik,
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// Two kernels, enqueued in order on one stream (three with a block mask):
//   0. fa_bwd_sched_kernel block-sparse only: one workgroup per head ranks
//                          the key and query tiles by falling work;
//   1. fa_bwd_dq_kernel    one workgroup per (batch, head, 128-query tile),
//                          streaming 64-row key tiles (recomputes S and dP);
//                          it also forms each row's -D = -rowsum(dO o O) and
//                          lse * log2(e) and writes them to the workspace,
//                          whose rows are padded per head to a multiple of
//                          128 (padding: -D = 0, lse = +inf, so a padded or
//                          fully masked row has P = 0 without any test in
//                          the hot loops);
//   2. fa_bwd_dkdv_kernel  one workgroup per (batch, head, 128-key tile),
//                          streaming 64-row query tiles and reading -D and
//                          lse * log2(e) from the workspace; dK, dV stay in
//                          registers for the whole sweep.
// dQ is not accumulated with atomics: fp32 global atomics run at a fraction
// of the plain store rate on this GPU, and the separate pass keeps every
// output written once, so results are deterministic.
//
// Both attention kernels copy their streamed tiles HBM -> LDS with
// global_load_lds (no register staging) into two LDS stages whose index is
// a compile-time constant (the tile loop is unrolled by two), so the next
// tile's copy is in flight while the current one is consumed, with one
// barrier per tile. Two workgroups (eight waves) share a CU, so one wave's
// exponentials overlap another's matrix products.
#include <type_traits>

#include "fa_device.h"
#include "fa_params.h"

namespace fa {

// ------------------------------------------------------------------ block-sparse schedule
// One workgroup per head: the work of each key tile (mask blocks of its
// column that some query sees) and of each query tile (blocks of its row),
// then a stable ranking by falling work, so that the dK/dV and dQ launches
// start their longest tiles first (the tail of a launch is then made of
// short tiles). tpb = key tiles per mask block (1 or 2). Up to
// SCHED_MAX_NB blocks per row; larger masks keep the plain order.
__device__ __forceinline__ void bwd_sched_head(const uint8_t* __restrict__ mask, int* __restrict__ korder,
                                               int* __restrict__ qorder, int nb, int tpb, int causal, int h) {
  __shared__ int kw[SCHED_MAX_NB];  // work of each key block (kept blocks of its column)
  __shared__ int qw[SCHED_MAX_NB];  // work of each query block (kept blocks of its row)
  __shared__ int kr[SCHED_MAX_NB];  // rank of each key block
  __shared__ int qr[SCHED_MAX_NB];  // rank of each query block
  const int tid = (int)threadIdx.x;
  const uint8_t* m = mask + (size_t)h * nb * nb;
  int* ko = korder + (size_t)h * sparse_kslots(nb);
  int* qo = qorder + (size_t)h * nb;
  if (nb > SCHED_MAX_NB) {
    for (int i = tid; i < nb; i += 256) {
      qo[i] = i;
      for (int t = 0; t < tpb; ++t) ko[i * tpb + t] = i * tpb + t;
    }
    return;
  }
  for (int i = tid; i < nb; i += 256) {
    kw[i] = 0;
    qw[i] = 0;
    kr[i] = 0;
    qr[i] = 0;
  }
  __syncthreads();
  // Both passes walk the nb x nb elements with consecutive threads on
  // consecutive columns; (row, column) of element e advance by
  // (256 / nb, 256 % nb) per step of 256.
  const int nn = nb * nb;
  const int dr = 256 / nb, dc = 256 % nb;
  auto advance = [&](int& r, int& c) __attribute__((always_inline)) {
    r += dr;
    c += dc;
    if (c >= nb) {
      c -= nb;
      ++r;
    }
  };
  // Work: a kept (and, under causal, visible) block adds to its row's and
  // its column's count. Sixteen loads in flight per thread.
  {
    int r = tid / nb, c = tid % nb;
    for (int e0 = 0; e0 < nn; e0 += 16 * 256) {
      uint8_t v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int e = e0 + u * 256 + tid;
        v[u] = e < nn ? m[e] : (uint8_t)0;
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        if (v[u] != 0 && (!causal || c <= r)) {
          atomicAdd(&kw[c], 1);
          atomicAdd(&qw[r], 1);
        }
        advance(r, c);
      }
    }
  }
  __syncthreads();
  // Rank by falling work, ties by index: element (j, i) adds one to the rank
  // of block i when block j comes before it.
  {
    int j = tid / nb, i = tid % nb;
    for (int e = tid; e < nn; e += 256) {
      const int wi = kw[i], wj = kw[j], vi = qw[i], vj = qw[j];
      if (wj > wi || (wj == wi && j < i)) atomicAdd(&kr[i], 1);
      if (vj > vi || (vj == vi && j < i)) atomicAdd(&qr[i], 1);
      advance(j, i);
    }
  }
  __syncthreads();
  for (int i = tid; i < nb; i += 256) {
    qo[qr[i]] = i;
    for (int t = 0; t < tpb; ++t) ko[kr[i] * tpb + t] = i * tpb + t;
  }
}

struct SchedArgs {
  const uint8_t* mask;
  int* korder;
  int* qorder;
  int nb, tpb, causal;
};

__global__ __launch_bounds__(256) void fa_bwd_sched_kernel(const SchedArgs sa) {
  bwd_sched_head(sa.mask, sa.korder, sa.qorder, sa.nb, sa.tpb, sa.causal, (int)blockIdx.x);
}

// ------------------------------------------------------------------ dK, dV
// A workgroup of 8 waves owns 128 keys. Waves w and w + 4 share keys
// 32w .. 32w + 31 and split the four products of every query tile evenly:
//   P-wave  (w < 4):  holds K; S = Q K^T, P = exp2(S*c - lse*log2e), passes
//                     P (bf16) to its partner through LDS; dV^T += dO^T P.
//   dS-wave (w >= 4): holds V; dP - D = dO V^T - D (the product accumulates
//                     onto -D), reads P, dS = P o (dP - D); dK^T += Q^T dS.
// Each wave keeps one operand (32 keys x d) and one accumulator in
// registers, so a SIMD runs one wave of each role.
//
// The query tiles are software-pipelined with one barrier per tile. In step
// t the dS-wave forms dS of tile t-1 from its partner's P, runs tile t's dP
// products, then tile t-1's dK products; the P-wave runs tile t's S
// products and exponentials, then tile t-1's dV products (with dropout, the
// dV products come first: they use the registers the exponentials refill).
// Three LDS stages
// rotate: tile t-1 (read by the transposed products), tile t (row products)
// and tile t+1 (being copied); each stage also holds its tile's P.
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG, bool DROP = false>
__global__ __launch_bounds__(bwd_kv_waves<D>() * 64, bwd_kv_waves<D>() == 8 ? 1 : 2) void fa_bwd_dkdv_kernel(
    const BwdParams p) {
  constexpr int BNK = bwd_kv_bn<D>();  // keys per workgroup
  constexpr int BMQ = bwd_kv_bm<D>();  // query rows per streamed tile
  constexpr int QB = BMQ / 32;    // 32-query blocks per tile
  constexpr int KG = BNK / 32;    // key groups (one P-wave and one dS-wave each)
  constexpr int TILEB = BMQ * D * 2;
  constexpr int PXB = KG * QB * 2048;  // P of a tile: [key group][query block][half][lane] x 16 bytes
  constexpr int LROW = 64;             // lse / -D floats per stage and array (one 4-byte copy per lane)
  static_assert(2 * KG == bwd_kv_waves<D>() && KG >= 2, "one P-wave and one dS-wave per key group");
  static_assert(MASK_BLOCK % BNK == 0 && MASK_BLOCK % BMQ == 0, "tiles lie inside one mask block");
  static_assert(BMQ % 32 == 0 && BMQ <= LROW, "lse/D rows of a tile fit one wave-wide 4-byte copy");
  // P-waves accumulate dV^T by head-dimension block (block kg, all keys of
  // the workgroup) rather than by key group: a 32-column block of dO^T is a
  // quarter of the transposing LDS reads of the full d. Needs one block per
  // key group, and P in LDS as the P-wave computed it (with dropout that copy
  // carries the keep bit in its sign, so the dropout kernels keep the key
  // split).
  constexpr bool DV_BY_D = !DROP && D / 32 == KG;
  // Three stages of each kind of data, one array per kind.
  __shared__ __attribute__((aligned(1024))) uint8_t q_raw[3 * TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t o_raw[3 * TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t p_raw[3 * PXB];
  __shared__ __attribute__((aligned(256))) float l_raw[3 * 2 * LROW];  // per stage: lse*log2e rows, then -D rows
  struct Stage {
    FA_LDS uint8_t* q;   // Q tile
    FA_LDS uint8_t* o;   // dO tile
    FA_LDS float* l;     // lse*log2e rows; -D rows at l + LROW
    FA_LDS uint8_t* px;  // P of the tile
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, h2 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform (scalar)
  const bool dswave = w >= KG;         // wave-uniform role
  const int kg = dswave ? w - KG : w;  // key group shared by waves kg and kg + KG
  const int n_kt = (p.N + BNK - 1) / BNK;
  const int n_qt = (p.N + BMQ - 1) / BMQ;
  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  // Ascending key tiles: under causal the first ones see the most queries.
  // Block-sparse: the schedule's key tile of this rank (the grid has a slot
  // for two tiles per mask block; slots past the last tile have no work).
  int bh, jt;
  head_rank_order(lid, SPARSE ? p.nb * (MASK_BLOCK / BNK) : n_kt, p.hgrp, bh, jt);
  const int h = bh % p.H;
  if (SPARSE) {
    jt = p.korder[(size_t)h * sparse_kslots(p.nb) + jt];
    if (jt < 0 || jt >= n_kt) return;  // whole workgroup, before any barrier
  }
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const int kb = jt * BNK;
  const int k0w = kb + 32 * kg;       // first key of this wave
  const int key = k0w + (lane & 31);  // key of this lane

  // K (P-wave) or V (dS-wave) rows of this lane's key as B operands
  // (d slots 16*kk + 8*h2 + i). Keys past N load a copy of key N-1; their
  // gradients are never stored.
  bf16x8 kvf[D / 16];
  {
    const uint16_t* src = (dswave ? p.v : p.k) + head + (size_t)min(key, N - 1) * D + 8 * h2;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) kvf[kk] = __builtin_bit_cast(bf16x8, ld_global16(src + 16 * kk));
  }
  f32x16 acc[D / 32];  // dV^T (P-wave) or dK^T (dS-wave)
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  const int it_begin = CAUSAL ? kb / BMQ : 0;
  MaskScan scan;  // kept blocks of the mask column of this key tile
  if (SPARSE) scan.init(p.mask + (size_t)h * p.nb * p.nb + (jt * BNK) / MASK_BLOCK, nullptr, p.nb, p.nb);
  auto next_tile = [&](int i) __attribute__((always_inline)) {
    if (SPARSE && i < n_qt) {
      const int b = (i * BMQ) / MASK_BLOCK;
      const int bk = scan.next_kept(b);
      if (bk != b) i = bk * (MASK_BLOCK / BMQ);
    }
    return i;
  };

  // Q, dO of this head and its lse*log2e / -D rows as buffer resources. Rows
  // past N read as zero; their lse is +inf in the padded workspace, so they
  // contribute P = 0.
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const uint32_t row_bytes = (uint32_t)p.Npad * 4;
  const float* l2g = p.lse2 + (size_t)bh * p.Npad;
  const float* Dg = p.Dneg + (size_t)bh * p.Npad;
  // The P-waves issue every tile copy: they wait at the barrier for their
  // partners anyway, so the dS-waves never stall on the copy queue.
  const TileDMA<D, BMQ, KG> cp(kg, lane);
  auto dma_q = [&](int i, const Stage& sb) __attribute__((always_inline)) {  // P-waves only
    cp.copy(p.q + head, head_bytes, i * BMQ * D * 2, sb.q, kg);
    cp.copy(p.dO + head, head_bytes, i * BMQ * D * 2, sb.o, kg);
    if (w == 0) dma4(l2g, row_bytes, lane * 4, i * BMQ * 4, (FA_LDS void*)sb.l);
    if (w == 1) dma4(Dg, row_bytes, lane * 4, i * BMQ * 4, (FA_LDS void*)(sb.l + LROW));
  };

  const float c = p.c;
  const int hh = lane >> 5, g = lane >> 4, jj = lane & 15;
  const int trow = 4 * hh + (jj >> 2);
  const int tcol = 16 * (g & 1) + 4 * (jj & 3);
  const int arow = lane & 31;
  // Per-lane LDS offsets, computed once and opaque to the compiler, so that
  // every stage and block base (compile-time constants) folds into the
  // instructions' offset fields: the row read of k-step kk (32-row blocks and
  // 16-row k-steps differ by constants, the swizzle repeating every 16 rows),
  // the two transposing reads (rows +0 and +8) of 32-column block dt, this
  // lane's 16-byte slot in the P exchange and its f32x4 of lse / -D rows.
  uint32_t rofs[D / 16], tofs[2][D / 32];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) rofs[kk] = opaque(tile_off<D>(arow, 16 * kk + 8 * hh));
#pragma unroll
  for (int pt = 0; pt < 2; ++pt)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) tofs[pt][dt] = opaque(tile_off<D>(trow + 8 * pt, 32 * dt + tcol));
  const uint32_t pofs = opaque(lane * 16);
  const uint32_t lofs = opaque(16 * hh);

  f32x16 sd[QB];       // S (P-wave) or dP - D (dS-wave) of the current tile
  bf16x8 pend[QB][2];  // P (P-wave) or dS (dS-wave) of the previous tile, B operand of its deferred product

  // S^T = K Q^T (P-wave, from zero) or dP^T - D = V dO^T - D (dS-wave, from
  // the -D rows) of tile i. Value r of block qb is query
  // i*BMQ + 32*qb + 8*(r/4) + 4*hh + r%4, key `key`.
  auto products_a = [&](auto role, int i, const Stage& sb) __attribute__((always_inline)) {
    constexpr bool DSW = decltype(role)::value;
    __builtin_amdgcn_sched_barrier(0);
    const FA_LDS uint8_t* a1 = DSW ? sb.o : sb.q;
    if (DEBUG && tid == 0) p.visited_kv[((size_t)bh * n_kt + jt) * n_qt + i] = 1;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (DSW) {
        const FA_LDS uint8_t* dl = reinterpret_cast<const FA_LDS uint8_t*>(sb.l + LROW);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 d4 = *reinterpret_cast<const FA_LDS f32x4*>(dl + 4 * (32 * qb + 8 * rg) + lofs);
#pragma unroll
          for (int e = 0; e < 4; ++e) sd[qb][4 * rg + e] = d4[e];
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) sd[qb][r] = 0.f;
      }
    }
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        sd[qb] = mfma32(ld_lds16(a1 + 32 * qb * D * 2, rofs[kk]), kvf[kk], sd[qb]);
    // Issue order: the -D rows and the operands of the first two k-steps,
    // then each k-step's products followed by the reads two k-steps ahead.
    __builtin_amdgcn_sched_group_barrier(0x100, (DSW ? 4 * QB : 0) + 2 * QB, 0);
#pragma unroll
    for (int kk = 0; kk < D / 16 - 2; ++kk) {
      __builtin_amdgcn_sched_group_barrier(0x008, QB, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, QB, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2 * QB, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // Causal mask of tile i on the P-wave's S: masked (S = -inf, so P = 0)
  // where the query precedes the key. Only tiles that reach the diagonal
  // need it; blocks wholly before the keys end up all zero.
  auto causal_mask = [&](int i) __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int lim = key - (i * BMQ + 32 * qb) - 4 * hh;  // masked iff 8*(r/4) + r%4 < lim
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + (r & 3) < lim) sd[qb][r] = -INFINITY;
    }
  };
  // dV^T += dO^T P (P-wave) or dK^T += Q^T dS (dS-wave) for the previous
  // tile, whose rows are in stage sb; query slots of k-step ks are
  // 16*ks + 8*(e/4) + 4*hh + e%4 on both operands.
  auto products_b = [&](auto role, const Stage& sb) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!decltype(role)::value && DV_BY_D) {
      // P-wave kg: dV^T rows of head-dimension block kg for all KG key
      // groups, from the P that every P-wave stored for its partner. One
      // transposed dO^T fragment (two transposing reads) feeds KG products,
      // one per key group, whose P operand is a plain 16-byte row read.
      const FA_LDS uint8_t* a2 = sb.o;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const FA_LDS uint8_t* a2r = a2 + (32 * qb + 16 * ks) * D * 2;
          const bf16x8 aT = join_tr(ld_lds_tr(a2r, tofs[0][kg]), ld_lds_tr(a2r, tofs[1][kg]));
#pragma unroll
          for (int g2 = 0; g2 < KG; ++g2) {
            const bf16x8 pb =
                *reinterpret_cast<const FA_LDS bf16x8*>(sb.px + (g2 * QB + qb) * 2048 + ks * 1024 + pofs);
            acc[g2] = mfma32(aT, pb, acc[g2]);
          }
        }
      // Issue order: the reads of the first (query block, k-step) unit, then
      // each unit's products, each followed by reads of the next unit.
      constexpr int NU = QB * 2;
      __builtin_amdgcn_sched_group_barrier(0x100, 2 + KG, 0);
#pragma unroll
      for (int u = 0; u < NU - 1; ++u) {
        // 2 + KG reads per unit: two after each of the first two products,
        // one after each of the others.
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int g2 = 2; g2 < KG; ++g2) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      __builtin_amdgcn_sched_group_barrier(0x008, KG, 0);
      __builtin_amdgcn_sched_barrier(0);
      return;
    }
    const FA_LDS uint8_t* a2 = decltype(role)::value ? sb.q : sb.o;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const FA_LDS uint8_t* a2r = a2 + (32 * qb + 16 * ks) * D * 2;
          const bf16x8 aT = join_tr(ld_lds_tr(a2r, tofs[0][dt]), ld_lds_tr(a2r, tofs[1][dt]));
          acc[dt] = mfma32(aT, pend[qb][ks], acc[dt]);
        }
    // Issue order: the reads of the first four products, then each product
    // followed by the two reads of the product four places ahead.
    constexpr int NM = QB * 2 * (D / 32);
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int m = 0; m < NM - 4; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  // P of the current tile (P-wave): bf16 into pnew and into the stage's P.
  // With dropout, P keeps its sign where the key is kept and is negated
  // where it is dropped in the copy for the partner (so the keep bit travels
  // with it), and the dV operand is P on kept entries, 0 elsewhere.
  auto exp_p = [&](int i, const Stage& sb, bf16x8 (&pnew)[QB][2]) __attribute__((always_inline)) {
    const FA_LDS uint8_t* ls = reinterpret_cast<const FA_LDS uint8_t*>(sb.l);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float pe[16];
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const f32x4 l4 = *reinterpret_cast<const FA_LDS f32x4*>(ls + 4 * (32 * qb + 8 * rg) + lofs);
#pragma unroll
        for (int e = 0; e < 4; ++e) pe[4 * rg + e] = fast_exp2(fmaf(sd[qb][4 * rg + e], c, -l4[e]));
      }
      FA_LDS uint8_t* dst = sb.px + (kg * QB + qb) * 2048 + pofs;
      if (DROP) {
        // Values 4*rg .. 4*rg+3 are queries i0 .. i0+3 at this lane's key.
        // The quad of lanes holding keys 4m .. 4m+3 makes the four
        // generator calls of the 4 x 4 block (lane t: query i0 + t, four
        // keys) and transposes the words so each lane gets its own key.
        float px[16];
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int i0 = i * BMQ + 32 * qb + 8 * rg + 4 * hh;
          uint32_t wv[4];
          philox4x32_10((uint32_t)key >> 2, (uint32_t)(i0 + (lane & 3)), (uint32_t)bh, p.drop.off, p.drop.k0,
                        p.drop.k1, wv);
          quad_transpose4(wv, lane & 3);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bool kept = wv[e] >= p.drop.t;
            px[4 * rg + e] = kept ? pe[4 * rg + e] : -pe[4 * rg + e];
            pe[4 * rg + e] = kept ? pe[4 * rg + e] : 0.f;
          }
        }
        *reinterpret_cast<FA_LDS bf16x8*>(dst) = to_bf16x8(px[0], px[1], px[2], px[3], px[4], px[5], px[6], px[7]);
        *reinterpret_cast<FA_LDS bf16x8*>(dst + 1024) =
            to_bf16x8(px[8], px[9], px[10], px[11], px[12], px[13], px[14], px[15]);
      }
      pnew[qb][0] = to_bf16x8(pe[0], pe[1], pe[2], pe[3], pe[4], pe[5], pe[6], pe[7]);
      pnew[qb][1] = to_bf16x8(pe[8], pe[9], pe[10], pe[11], pe[12], pe[13], pe[14], pe[15]);
      if (!DROP) {
        // Two 1 KiB halves, 16 bytes per lane in each (conflict-free).
        *reinterpret_cast<FA_LDS bf16x8*>(dst) = pnew[qb][0];
        *reinterpret_cast<FA_LDS bf16x8*>(dst + 1024) = pnew[qb][1];
      }
    }
  };
  // dS of the previous tile (dS-wave) from its dP - D (sd) and the
  // partner's P stored in that tile's stage.
  auto form_ds = [&](const Stage& sb) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 pp[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const FA_LDS uint8_t* src = sb.px + (kg * QB + qb) * 2048 + pofs;
      pp[qb][0] = *reinterpret_cast<const FA_LDS bf16x8*>(src);
      pp[qb][1] = *reinterpret_cast<const FA_LDS bf16x8*>(src + 1024);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float ds[16];
      if (DROP) {
        // Kept (P >= 0): dS = P (dP - D) with dP, D both in units of
        // 1 - p; dropped (P stored negated): dS = -P D = P' * D.
        const FA_LDS uint8_t* dl = reinterpret_cast<const FA_LDS uint8_t*>(sb.l + LROW);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 d4 = *reinterpret_cast<const FA_LDS f32x4*>(dl + 4 * (32 * qb + 8 * rg) + lofs);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * rg + e;
            const float pv = (float)(r < 8 ? pp[qb][0][r] : pp[qb][1][r - 8]);
            ds[r] = pv * (pv >= 0.f ? sd[qb][r] : -d4[e]);
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) ds[r] = (float)(r < 8 ? pp[qb][0][r] : pp[qb][1][r - 8]) * sd[qb][r];
      }
      pend[qb][0] = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      pend[qb][1] = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * QB, 0);  // all P reads first
    __builtin_amdgcn_sched_barrier(0);
  };
  auto needs_mask = [&](int i) __attribute__((always_inline)) { return CAUSAL && k0w + 31 > i * BMQ; };
  auto stage = [&](int S) __attribute__((always_inline)) {
    return Stage{(FA_LDS uint8_t*)q_raw + S * TILEB, (FA_LDS uint8_t*)o_raw + S * TILEB,
                 (FA_LDS float*)l_raw + S * 2 * LROW, (FA_LDS uint8_t*)p_raw + S * PXB};
  };

  // The whole sweep, instantiated once per role so that each role's
  // loop-invariant addresses stay in its own branch. Both roles pass the
  // same number of barriers.
  auto sweep = [&](auto role) __attribute__((always_inline)) -> int {
    constexpr bool DSW = decltype(role)::value;
    int ic = next_tile(it_begin);
    if (ic >= n_qt) return 0;
    // The last tile's transposed products (its rows are in stage s).
    auto tail = [&](int s) __attribute__((always_inline)) {
      if (DSW) form_ds(stage(s));
      products_b(role, stage(s));
    };
    // One step: tile ic in stage SC; the previous tile is in stage SP, the
    // next one is copied into stage SN. Returns false after the last tile.
    auto step = [&](auto scur) __attribute__((always_inline)) -> bool {
      const int SC = scur;  // a compile-time constant in the unrolled loop
      const int SP = SC == 0 ? 2 : SC - 1, SN = SC == 2 ? 0 : SC + 1;
      const int in = next_tile(ic + 1);
      if (!DSW && in < n_qt) dma_q(in, stage(SN));
      if (DSW) {
        form_ds(stage(SP));
        products_a(role, ic, stage(SC));
        products_b(role, stage(SP));
      } else if constexpr (DV_BY_D) {
        // Row products and exponentials of this tile first, then the
        // previous tile's dV products, whose P comes from LDS. (Running the
        // dV products first, out of phase with the partner's dK products,
        // was 2-5% slower once they read only a quarter of dO^T.)
        products_a(role, ic, stage(SC));
        if (needs_mask(ic)) causal_mask(ic);
        exp_p(ic, stage(SC), pend);
        products_b(role, stage(SP));
      } else {
        // The previous tile's dV products take its P from registers (pend),
        // so they run before this tile's exponentials overwrite it.
        products_b(role, stage(SP));
        products_a(role, ic, stage(SC));
        if (needs_mask(ic)) causal_mask(ic);
        exp_p(ic, stage(SC), pend);
      }
      wait_vmem();
      __syncthreads();
      ic = in;
      return ic < n_qt;
    };
    // First tile (stage 0): its row products and P only.
    if (!DSW) dma_q(ic, stage(0));
    wait_vmem();
    __syncthreads();
    const int in = next_tile(ic + 1);
    if (!DSW && in < n_qt) dma_q(in, stage(1));
    products_a(role, ic, stage(0));
    if (!DSW) {
      if (needs_mask(ic)) causal_mask(ic);
      exp_p(ic, stage(0), pend);
    }
    wait_vmem();
    __syncthreads();
    ic = in;
    if (ic >= n_qt) {
      tail(0);
      return 0;
    }
    // Stages rotate 1, 2, 0, 1, ...; the last tile's transposed products
    // (tail) use the stage it was in. Without dropout the loop is unrolled
    // by three, so that every stage index is a compile-time constant and each
    // LDS address a per-lane register plus an immediate; the dropout kernels
    // need those registers for the generator and keep the run-time index.
    int last = 1;
    if constexpr (DROP) {
      while (step(last)) last = last == 2 ? 0 : last + 1;
    } else {
      for (;;) {
        if (!step(std::integral_constant<int, 1>())) break;
        last = 2;
        if (!step(std::integral_constant<int, 2>())) break;
        last = 0;
        if (!step(std::integral_constant<int, 0>())) break;
        last = 1;
      }
    }
    tail(last);
    return last;
  };
  // LDS stage of the last tile (0 without tiles). The other two stages are
  // free from here on: every wave passed the barrier after their last
  // reads, and no copy targets them.
  const int last = dswave ? sweep(std::true_type()) : sweep(std::false_type());

  // dK / dV go out through this wave's slice of the free stages (Q and dO
  // tile buffers of the two stages other than `last`).
  constexpr int SLICE = 32 * D * 2;
  constexpr int PER = TILEB / SLICE;  // slices per tile buffer
  static_assert(PER >= 1 && 4 * PER >= 2 * KG, "the free stages hold one slice per wave");
  const int bi = w / PER, f0 = last == 2 ? 0 : last + 1, f1 = last == 0 ? 2 : last - 1;
  FA_LDS uint8_t* const slice =
      (bi < 2 ? (FA_LDS uint8_t*)q_raw : (FA_LDS uint8_t*)o_raw) + ((bi & 1) ? f1 : f0) * TILEB + (w % PER) * SLICE;
  if (DV_BY_D && !dswave) {
    // dV of head-dimension block kg for the keys of every key group.
    uint16_t* const vbase = p.dv + head + (size_t)kb * D + 32 * kg;
    store_tile<KG, true, SLICE>(acc, 1.0f, slice, lane, N - kb,
                                [&](int r) __attribute__((always_inline)) { return vbase + (size_t)r * D; });
  } else {
    uint16_t* const base = (dswave ? p.dk : p.dv) + head + (size_t)k0w * D;
    const float sc = (dswave ? p.scale : 1.0f) * (DROP ? p.drop.scale : 1.0f);
    store_tile<D / 32, false, SLICE>(acc, sc, slice, lane, N - k0w,
                                     [&](int r) __attribute__((always_inline)) { return base + (size_t)r * D; });
  }
}

// ------------------------------------------------------------------ dQ
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG, bool DROP = false>
__global__ __launch_bounds__(256, 2) void fa_bwd_dq_kernel(const BwdParams p) {
  constexpr int BM = BWD_Q_BM;
  constexpr int BN = bwd_q_bn<D, CAUSAL, DROP>();
  static_assert(MASK_BLOCK % BN == 0 && MASK_BLOCK % BM == 0, "tiles lie inside one mask block");
  constexpr int NS = BN / 32;
  constexpr int TILEB = BN * D * 2;
  __shared__ __attribute__((aligned(1024))) uint8_t k0_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t k1_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v0_raw[TILEB];
  __shared__ __attribute__((aligned(1024))) uint8_t v1_raw[TILEB];
  FA_LDS uint8_t* const kst[2] = {(FA_LDS uint8_t*)k0_raw, (FA_LDS uint8_t*)k1_raw};
  FA_LDS uint8_t* const vst[2] = {(FA_LDS uint8_t*)v0_raw, (FA_LDS uint8_t*)v1_raw};

  const int tid = threadIdx.x;
  const int lane = tid & 63, h2 = lane >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, wave-uniform (scalar)
  const int n_qt = (p.N + BM - 1) / BM;
  const int n_kt = (p.N + BN - 1) / BN;
  const int lid = xcd_grouped_block(blockIdx.x, gridDim.x);
  int bh, qt;
  head_rank_order(lid, n_qt, p.hgrp, bh, qt);
  const int h = bh % p.H;
  if (SPARSE)
    qt = min(max(p.qorder[(size_t)h * p.nb + qt], 0), n_qt - 1);  // the schedule's tile of this rank
  else if (CAUSAL)
    qt = n_qt - 1 - qt;  // longest query tiles first
  const int N = p.N;
  const size_t head = (size_t)bh * N * D;
  const int q_lo = qt * BM;
  const int q_last = min(q_lo + BM, N) - 1;
  const int q0 = q_lo + 32 * w;
  const int qi = q0 + (lane & 31);
  int kt_end = n_kt;
  if (CAUSAL) kt_end = min(kt_end, q_last / BN + 1);
  MaskScan scan;  // kept blocks of the mask row of this query tile
  if (SPARSE) scan.init(p.mask + ((size_t)h * p.nb + (q_lo / MASK_BLOCK)) * p.nb, nullptr, 1, p.nb);
  auto next_tile = [&](int j) __attribute__((always_inline)) {
    if (SPARSE && j < kt_end) {
      const int b = (j * BN) / MASK_BLOCK;
      const int bk = scan.next_kept(b);
      if (bk != b) j = bk * (MASK_BLOCK / BN);
    }
    return j;
  };
  auto wave_active = [&](int j) __attribute__((always_inline)) { return !CAUSAL || j * BN <= q0 + 31; };

  // Q^T and dO^T fragments (B operands, lane = query). Queries past N load a
  // copy of row N-1; their lse * log2(e) is +inf, so P = 0.
  bf16x8 qf[D / 16], dof[D / 16];
  float Dq, lse2;  // -D and lse * log2(e) of this lane's query
  const size_t qr = (size_t)min(qi, N - 1) * D + 8 * h2;
  u32x4 of[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = __builtin_bit_cast(bf16x8, ld_global16(p.q + head + qr + 16 * kk));
    dof[kk] = __builtin_bit_cast(bf16x8, ld_global16(p.dO + head + qr + 16 * kk));
    of[kk] = ld_global16(p.o + head + qr + 16 * kk);
  }
  const float lrow = qi < N ? p.lse[(size_t)bh * N + qi] : -INFINITY;

  // K and V of this head as buffer resources: tail rows past N read as zero
  // (and are masked).
  const uint32_t head_bytes = (uint32_t)N * D * 2;
  const TileDMA<D, BN> cp(w, lane);
  auto dma_kv = [&](int j, FA_LDS uint8_t* kdst, FA_LDS uint8_t* vdst) __attribute__((always_inline)) {
    cp.copy(p.k + head, head_bytes, j * BN * D * 2, kdst, w);
    cp.copy(p.v + head, head_bytes, j * BN * D * 2, vdst, w);
  };

  // The first key tile's copy is issued before the row terms below wait
  // for O and dO, so both round trips to memory overlap.
  int jc = next_tile(0);
  if (jc < kt_end) dma_kv(jc, kst[0], vst[0]);
  __builtin_amdgcn_sched_barrier(0);
  {
    // D = rowsum(dO o O): this lane holds half of its row's elements, the
    // lane 32 apart the other half. With dropout dP is kept in units of
    // 1 - p, and so is D.
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      const u32x4 dw = __builtin_bit_cast(u32x4, dof[kk]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc = fmaf(__uint_as_float(of[kk][e] << 16), __uint_as_float(dw[e] << 16), acc);
        acc = fmaf(__uint_as_float(of[kk][e] & 0xFFFF0000u), __uint_as_float(dw[e] & 0xFFFF0000u), acc);
      }
    }
    acc = xhalf_sum(acc);
    Dq = qi < N ? -acc * p.dfac : 0.f;
    lse2 = lrow == -INFINITY ? INFINITY : lrow * kLog2e;
  }
  f32x16 dqt[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqt[dt][r] = 0.f;

  const float c = p.c;
  // Per-lane LDS offsets, computed once and opaque to the compiler (stage and
  // block bases are compile-time constants that fold into the instructions'
  // offset fields): the K / V row read of k-step kk (32-row blocks differ by
  // a constant) and the two transposing reads of Kᵀ (rows +0 and +8 of a
  // 16-key k-step) for 32-column block dt.
  uint32_t rofs[D / 16], tofs[2][D / 32];
  {
    const int g = lane >> 4, jj = lane & 15;
    const int trow = 4 * h2 + (jj >> 2);
    const int tcol = 16 * (g & 1) + 4 * (jj & 3);
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) rofs[kk] = opaque(tile_off<D>(lane & 31, 16 * kk + 8 * h2));
#pragma unroll
    for (int pt = 0; pt < 2; ++pt)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) tofs[pt][dt] = opaque(tile_off<D>(trow + 8 * pt, 32 * dt + tcol));
  }

  auto tile = [&](int j, const FA_LDS uint8_t* ks, const FA_LDS uint8_t* vs, bool need_mask)
                  __attribute__((always_inline)) {
    const int kbase = j * BN;
    f32x16 s[NS], dp[NS];
#pragma unroll
    for (int mt = 0; mt < NS; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        s[mt][r] = 0.f;
        dp[mt][r] = 0.f;
      }
    // S^T = K Q^T and dP^T = V dO^T; k-step outer so consecutive products
    // go to independent accumulators.
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
      for (int mt = 0; mt < NS; ++mt) {
        s[mt] = mfma32(ld_lds16(ks + 32 * mt * D * 2, rofs[kk]), qf[kk], s[mt]);
        dp[mt] = mfma32(ld_lds16(vs + 32 * mt * D * 2, rofs[kk]), dof[kk], dp[mt]);
      }
    // Value r of block mt is key kbase + 32*mt + 8*(r/4) + 4*h2 + r%4; it is
    // visible iff key <= min(N - 1, qi) (causal) or key <= N - 1.
    const int lim = (CAUSAL ? min(qi, N - 1) : N - 1) - kbase - 4 * h2;
    // dQ^T += K^T dS^T; key slots of k-step kk are 16*kk + 8*(i/4) + 4*h2 + i%4,
    // i.e. value r = 8*(kk%2) + i of block kk/2.
#pragma unroll
    for (int kk = 0; kk < BN / 16; ++kk) {
      const int mt = kk >> 1, r0 = 8 * (kk & 1);
      float pe[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pe[i] = fast_exp2(fmaf(s[mt][r0 + i], c, -lse2));
      if (need_mask) {  // diagonal or tail tiles only
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = r0 + i;
          if (32 * mt + 8 * (r >> 2) + (r & 3) > lim) pe[i] = 0.f;
        }
      }
      bf16x8 dsb;
      if (DROP) {
        // Slots 0-3 are keys kd .. kd+3, slots 4-7 keys kd+8 .. kd+11. Kept:
        // dS = P (dP - D); dropped: dS = -P D (dP and D in units of 1 - p).
        const int kd = kbase + 16 * kk + 4 * h2;
        uint32_t w0[4], w1[4];
        philox4x32_10((uint32_t)kd >> 2, (uint32_t)qi, (uint32_t)bh, p.drop.off, p.drop.k0, p.drop.k1, w0);
        philox4x32_10((uint32_t)(kd + 8) >> 2, (uint32_t)qi, (uint32_t)bh, p.drop.off, p.drop.k0, p.drop.k1, w1);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const bool kept = (i < 4 ? w0[i] : w1[i - 4]) >= p.drop.t;
          dsb[i] = (__bf16)(pe[i] * ((kept ? dp[mt][r0 + i] : 0.f) + Dq));
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) dsb[i] = (__bf16)(pe[i] * (dp[mt][r0 + i] + Dq));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const FA_LDS uint8_t* kr = ks + 16 * kk * D * 2;
        const bf16x8 kT = join_tr(ld_lds_tr(kr, tofs[0][dt]), ld_lds_tr(kr, tofs[1][dt]));
        dqt[dt] = mfma32(kT, dsb, dqt[dt]);
      }
      // No scheduling fence between k-steps: the next k-step's transposing
      // reads may start during this one's vector work (0.4-1.9% faster than
      // fencing each k-step, and no more registers).
    }
  };

  int pl = 0;  // LDS stage of the last tile (stage 1 - pl is free afterwards)
  if (jc < kt_end) {
    wait_vmem();
    __syncthreads();
    auto step = [&](auto parity) __attribute__((always_inline)) -> bool {
      constexpr int P = decltype(parity)::value;
      const int jn = next_tile(jc + 1);
      if (jn < kt_end) dma_kv(jn, kst[1 - P], vst[1 - P]);
      if (DEBUG && tid == 0) p.visited_q[((size_t)bh * n_qt + qt) * n_kt + jc] = 1;
      if (wave_active(jc)) {
        const bool need_mask = (jc * BN + BN > N) || (CAUSAL && jc * BN + BN - 1 > q0);
        tile(jc, kst[P], vst[P], need_mask);
      }
      // After the last tile no copy is in flight and no LDS access follows;
      // under causal masking each wave then goes on to its epilogue without
      // waiting for the others, as in the forward kernel.
      if (!CAUSAL || jn < kt_end) {
        wait_vmem();
        __syncthreads();
      }
      jc = jn;
      pl = P;
      return jn < kt_end;
    };
    while (step(std::integral_constant<int, 0>()) && step(std::integral_constant<int, 1>())) {
    }
  }

  // The dK/dV pass reads -D and lse * log2(e) from the workspace, padded to
  // whole query tiles per head (rows past N: -D = 0, lse * log2(e) = +inf).
  // Stored only now: the tile loop's waits for its copies count stores too,
  // so stores issued before it would hold up the first tile.
  if (h2 == 0) {
    p.Dneg[(size_t)bh * p.Npad + qi] = Dq;
    p.lse2[(size_t)bh * p.Npad + qi] = lse2;
  }
  // dQ goes out through this wave's slice of the LDS stage that held the tile
  // before the last (no wave reads it any more, and no copy targets it).
  {
    constexpr int SLICE = 2 * TILEB / 4;
    constexpr int PER = TILEB / SLICE;  // slices per stage buffer
    FA_LDS uint8_t* const kfree = pl ? (FA_LDS uint8_t*)k0_raw : (FA_LDS uint8_t*)k1_raw;
    FA_LDS uint8_t* const vfree = pl ? (FA_LDS uint8_t*)v0_raw : (FA_LDS uint8_t*)v1_raw;
    FA_LDS uint8_t* const slice = (w < PER ? kfree : vfree) + (w % PER) * SLICE;
    uint16_t* const qbase = p.dq + head + (size_t)q0 * D;
    store_tile<D / 32, false, SLICE>(dqt, p.scale * (DROP ? p.drop.scale : 1.0f), slice, lane, N - q0,
                                     [&](int r) __attribute__((always_inline)) { return qbase + (size_t)r * D; });
  }
}

// ------------------------------------------------------------------ fp32 atomic-add rate
// The accumulation a dQ-by-atomics backward would make: every wave adds the
// 16 registers of a 32 x 32 fp32 MFMA result (lanes 0-31 one row, lanes
// 32-63 the row four below, 32 consecutive floats each) into a [rows][128]
// fp32 matrix, `reps` times, with global atomic adds (no return). Workgroup
// b adds into 32 KiB block b % nblk. Measures the rate that decides between
// atomics and a separate dQ pass.
__global__ __launch_bounds__(256) void fa_atomic_probe_kernel(float* __restrict__ dst, size_t nblk, int reps) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float* base = dst + (blockIdx.x % nblk) * (64 * 128);
  for (int it = 0; it < reps; ++it) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = (16 * w + 8 * (r / 4) + 4 * (lane / 32) + (r % 4)) % 64;
      atomicAdd(base + row * 128 + 32 * (it % 4) + (lane & 31), 1.0f);
    }
  }
}

hipError_t launch_atomic_probe(float* dst, size_t nblk, int wgs, int reps, hipStream_t st) {
  hipLaunchKernelGGL(fa_atomic_probe_kernel, dim3((unsigned)wgs), dim3(256), 0, st, dst, nblk, reps);
  return hipGetLastError();
}

// ------------------------------------------------------------------ launchers
// stages: bit 0 = block-sparse schedule (nothing without a mask), bit 1 =
// dQ kernel (also writes -D and lse * log2(e) per row to the workspace),
// bit 2 = dK/dV kernel (reads them). Enqueued in that order.
template <int D, bool CAUSAL, bool SPARSE, bool DEBUG, bool DROP = false>
hipError_t launch_bwd_t(const BwdParams& p, int BH, int stages, hipStream_t st) {
  static_assert(BWD_Q_BM == BWD_PAD_ROWS, "dQ tiles cover the padded workspace rows exactly");
  if (SPARSE && (stages & 1)) {
    const SchedArgs sa{p.mask, p.korder, p.qorder, p.nb, MASK_BLOCK / bwd_kv_bn<D>(), (int)CAUSAL};
    hipLaunchKernelGGL(fa_bwd_sched_kernel, dim3((unsigned)p.H), dim3(256), 0, st, sa);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // Dense causal launches interleave heads (see head_group), as do
  // block-sparse ones, whose tiles the schedule orders by falling work.
  constexpr bool INTERLEAVE = CAUSAL || SPARSE;
  if (stages & 2) {
    const int n_qt2 = (p.N + BWD_Q_BM - 1) / BWD_Q_BM;
    const auto kernel = fa_bwd_dq_kernel<D, CAUSAL, SPARSE, DEBUG, DROP>;
    static const int wgs = wgs_per_cu((const void*)kernel, 256);
    BwdParams q = p;
    q.hgrp = INTERLEAVE ? head_group(wgs, cus_per_xcd(), BH, n_qt2) : 1;
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * n_qt2)), dim3(256), 0, st, q);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (stages & 4) {
    const int n_kt1 = (p.N + bwd_kv_bn<D>() - 1) / bwd_kv_bn<D>();
    // Block-sparse: one slot per (mask block, key tile of the block).
    const int slots = SPARSE ? p.nb * (MASK_BLOCK / bwd_kv_bn<D>()) : n_kt1;
    const auto kernel = fa_bwd_dkdv_kernel<D, CAUSAL, SPARSE, DEBUG, DROP>;
    static const int wgs = wgs_per_cu((const void*)kernel, 64 * bwd_kv_waves<D>());
    BwdParams q = p;
    // Dense causal: a wider group (see head_group); block-sparse: the default.
    q.hgrp = !INTERLEAVE ? 1 : SPARSE ? head_group(wgs, cus_per_xcd(), BH, slots)
                                      : head_group(wgs, cus_per_xcd(), BH, slots, 8, 8);
    hipLaunchKernelGGL(kernel, dim3((unsigned)(BH * slots)), dim3(64 * bwd_kv_waves<D>()), 0, st, q);
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

// Backward with dropout.
template <int D>
hipError_t launch_bwd_dropout_d(const BwdParams& p, int BH, bool causal, bool sparse, int stages, hipStream_t st) {
  if (causal) return sparse ? launch_bwd_t<D, true, true, false, true>(p, BH, stages, st) : launch_bwd_t<D, true, false, false, true>(p, BH, stages, st);
  return sparse ? launch_bwd_t<D, false, true, false, true>(p, BH, stages, st) : launch_bwd_t<D, false, false, false, true>(p, BH, stages, st);
}

hipError_t launch_bwd_dropout(const BwdParams& p, int BH, int d, bool causal, bool sparse, int stages,
                              hipStream_t st) {
  return d == 64 ? launch_bwd_dropout_d<64>(p, BH, causal, sparse, stages, st)
                 : launch_bwd_dropout_d<128>(p, BH, causal, sparse, stages, st);
}

}  // namespace fa
