// Kernel argument blocks and tile sizes shared by the host launcher and the
// gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Forward: 4 waves per workgroup, 32 query rows per wave (the waves split
// the query rows of the tile, never the keys), key/value tiles of fwd_bn<D>()
// rows. At d = 128, 32-key tiles let three workgroups share a CU (32 KiB of
// LDS and at most 168 registers each), which measured faster than two with
// 64-key tiles; d = 64 keeps 64-key tiles at four workgroups per CU. The
// dropout forward uses the same tiles (two workgroups per CU at d = 128),
// so that with p = 0 it gives the plain forward's results bit for bit.
constexpr int FWD_BM = 128;
template <int D>
constexpr int fwd_bn() { return D == 128 ? 32 : 64; }
// Backward dK/dV kernel: a workgroup owns bwd_kv_bn<D>() keys, one P-wave
// and one dS-wave per 32 keys (one computes P and dV, the other dP, dS and
// dK); query tiles of bwd_kv_bm<D>() rows stream through LDS. d = 128: 128
// keys, 8 waves, 64-row tiles, one workgroup per CU. d = 64: 64 keys,
// 4 waves, 32-row tiles, up to four workgroups per CU (measured faster at
// d = 64, slower at d = 128 where only two fit).
template <int D>
constexpr int bwd_kv_bn() { return D == 128 ? 128 : 64; }
template <int D>
constexpr int bwd_kv_bm() { return D == 128 ? 64 : 32; }
template <int D>
constexpr int bwd_kv_waves() { return 2 * bwd_kv_bn<D>() / 32; }
// Backward dQ kernel: a workgroup owns BWD_Q_BM queries (32 per wave) and
// streams key tiles of bwd_q_bn() rows. 64-key tiles halve the copies and
// barriers per product; at d = 128 they fit the 256 registers that two
// waves per SIMD allow only in the causal kernel without dropout (the others
// spill), so those use 32-key tiles.
constexpr int BWD_Q_BM = 128;
template <int D, bool CAUSAL, bool DROP>
constexpr int bwd_q_bn() { return (D == 64 || (CAUSAL && !DROP)) ? 64 : 32; }
// Workspace rows per head are padded to a multiple of this.
constexpr int BWD_PAD_ROWS = 128;
// Block-sparse masks are given at this granularity.
constexpr int MASK_BLOCK = 128;

// Attention dropout on the probabilities (counter-based keep mask, see
// philox4x32_10 in fa_device.h): element (b*H + h, i, j) is kept iff word
// j % 4 of Philox4x32-10(counter (j / 4, i, b*H + h, off), key (k0, k1)) is
// >= t; kept probabilities are scaled by `scale` = 1 / (1 - p).
struct Dropout {
  uint32_t t;       // floor(p * 2^32)
  uint32_t k0, k1;  // seed, low and high 32 bits
  uint32_t off;     // offset (counter word 3)
  float scale;      // 1 / (1 - p)
};

struct FwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const uint8_t* mask;  // [H][nb][nb] or nullptr
  uint8_t* visited;     // debug map [B*H][n_qt][n_kt] or nullptr
  int H, N;
  int n_qt, n_kt, nb;
  float c;  // scale * log2(e)
  Dropout drop;  // used by the dropout instantiations only
  int hgrp;      // heads per dispatch group (head_rank_order), set by the launcher
};

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dO;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  const float* lse;  // forward's lse, [B*H*N]
  float* Dneg;       // workspace: -rowsum(dO * O), [B*H][Npad]
  float* lse2;       // workspace: lse * log2(e) (+inf for no visible key or padding), [B*H][Npad]
  const uint8_t* mask;
  uint8_t* visited_kv;  // [B*H][n_kt1][n_qt1] or nullptr
  uint8_t* visited_q;   // [B*H][n_qt2][n_kt2] or nullptr
  int H, N;
  int Npad;  // N rounded up to a multiple of BWD_PAD_ROWS
  int nb;
  float c;      // scale * log2(e)
  float scale;  // scale, applied to dQ and dK
  float dfac;   // factor on -D in the workspace: 1, or 1 - p with dropout
  Dropout drop;  // used by the dropout instantiations only
  int hgrp;      // heads per dispatch group (head_rank_order), set per launch
  // Block-sparse schedule in the workspace (written by the schedule stage):
  // per head, the key tiles (korder, SPARSE_KSLOTS(nb) entries) and the
  // query tiles (qorder, nb entries) in order of falling work.
  int* korder;
  int* qorder;
};

// Key-tile slots per head in the block-sparse schedule: two per mask block,
// enough for 64-key tiles (128-key tiles use the first nb).
__host__ __device__ inline int sparse_kslots(int nb) { return 2 * nb; }
// Mask blocks per row up to which the schedule is sorted (larger masks keep
// the plain order).
constexpr int SCHED_MAX_NB = 2048;

// (head, tile rank) of logical workgroup `lid` in a grid of heads x
// `ntile` tiles, ordered in groups of G consecutive heads (G divides the
// number of heads): within a group, rank 0 of every head, then rank 1, and
// so on. G = 1 is plain head-by-head order. For causal attention the rank
// is ordered heaviest first; each XCD receives a contiguous range of
// logical indices (xcd_grouped_block), so with G > 1 the heaviest tiles of
// G heads start together instead of the last head's starting near the end
// of the launch (the launcher picks G, see head_group).
__host__ __device__ inline void head_rank_order(int lid, int ntile, int G, int& bh, int& rank) {
  const int per = G * ntile;
  const int r = lid % per;
  rank = r / G;
  bh = (lid / per) * G + r % G;
}

// Workgroups of `kernel` (launched with `block` threads, no dynamic LDS)
// that one CU holds at once; 1 if the runtime cannot tell (the error is
// cleared so that the launch that follows reports only its own).
inline int wgs_per_cu(const void* kernel, int block) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, block, 0) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = 1;
  }
  return n;
}
// CUs of one XCD of the current device (eight XCDs per device).
inline int cus_per_xcd() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8) {
    (void)hipGetLastError();
    return 32;
  }
  return cus / 8;
}

// Heads per dispatch group for a launch of BH heads x ntile tiles whose
// per-head work falls with the tile rank (causal), given the workgroups one
// CU holds and the CUs of one XCD. Each XCD runs BH / 8 consecutive heads.
// Ordered head by head, the last head's heavy tiles start near the end and
// the XCD idles while they finish; interleaving G heads rank by rank starts
// the heavy tiles of G heads together. Too large a G spreads the XCD's
// slots over more heads at once and lowers the L2 reuse of each head's K/V
// (or Q/dO). G is the smallest divisor of BH / 8 with G * ntile >= cover *
// slots (1 when 8 does not divide BH). With cover = 2 (forward, dQ and the
// block-sparse dK/dV) it was as fast as or faster than both G = 1 and
// G = BH / 8 on causal d = 64 and 128 shapes. The dense causal dK/dV launch
// (one long workgroup per CU) takes cover = 8 with the cap at 8: 1-3% faster
// from N = 4096 to 16384 and up to 3.6% at N = 512, not slower anywhere
// measured (d = 64 and 128, N = 512 to 16384). G is capped at the largest
// divisor of BH / 8 not above `cap` (default kMaxHeadGroup): short
// sequences have few tiles per head, and at N = 512 (ntile 4) the uncapped
// rule picked G = 64, 10-17% slower than 16 in the forward and dK/dV passes
// of causal d = 64 and 128 launches; at N = 1024 the two choices were within
// a few percent either way, and from N = 2048 the cap does not bind.
constexpr int kMaxHeadGroup = 16;
inline int head_group(int wgs_per_cu, int cus_per_xcd, int BH, int ntile, int cover = 2,
                      int cap = kMaxHeadGroup) {
  if (BH % 8 != 0 || ntile < 1) return 1;
  const int hx = BH / 8;
  const int slots = wgs_per_cu * cus_per_xcd;
  int g = 1;
  while (g < hx && g < cap && (g * ntile < cover * slots || hx % g != 0)) ++g;
  while (hx % g != 0) --g;  // largest divisor of hx not above the cap
  return g;
}

}  // namespace fa
