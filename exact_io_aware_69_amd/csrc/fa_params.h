// Kernel argument blocks and tile sizes shared by the host launcher and the
// gfx950 kernels.
#pragma once

#include <stdint.h>

namespace fa {

// Forward: 4 waves per workgroup, 32 query rows per wave (the waves split
// the query rows of the tile, never the keys), key/value tiles of FWD_BN rows.
constexpr int FWD_BM = 128;
constexpr int FWD_BN = 64;
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
// streams key tiles of bwd_q_bn<D>() rows (32 at d = 128 keeps a wave within
// the 256 registers that two waves per SIMD allow).
constexpr int BWD_Q_BM = 128;
template <int D>
constexpr int bwd_q_bn() { return D == 128 ? 32 : 64; }
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
};

}  // namespace fa
