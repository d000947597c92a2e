// Device-side building blocks for the gfx950 attention kernels.
//
// Matrix-core conventions used throughout (CDNA4 v_mfma_f32_32x32x16_bf16,
// checked on the hardware):
//   * A operand (32 x 16, M x K): lane l holds row m = l % 32 and one half of
//     K (8 bf16) selected by l / 32. B operand (16 x 32): lane l holds column
//     n = l % 32 and the same half of K. Which 8 of the 16 K indices a half
//     carries is free, as long as A and B agree, so every kernel states its
//     own "slot -> index" map.
//   * C/D (32 x 32 fp32, 16 values per lane): lane l, value r holds row
//     8*(r/4) + 4*(l/32) + (r%4), column l % 32.
//   * ds_read_tr16_b64 (16-lane groups): if source lane j of a group points
//     at element [k0 + j/4][n0 + 4*(j%4)] of a row-major bf16 matrix, lane i
//     of the group receives [k0 + r][n0 + i] for r = 0..3, i.e. four
//     consecutive rows of column n0 + i. This is how a row-major [key][d]
//     tile in LDS becomes a K-contiguous MFMA operand without a transpose
//     pass.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a per-lane value with the lane 32 apart (same MFMA column).
__device__ __forceinline__ float xhalf_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte global load / store of bf16 data.
__device__ __forceinline__ u32x4 ld_global16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st_lds16(FA_LDS uint8_t* base, uint32_t off, const u32x4& v) {
  *reinterpret_cast<FA_LDS u32x4*>(base + off) = v;
}
__device__ __forceinline__ bf16x8 ld_lds16(const FA_LDS uint8_t* base, uint32_t off) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const FA_LDS u32x4*>(base + off));
}
// Transposing 8-byte LDS read (see the header comment).
__device__ __forceinline__ s16x4 ld_lds_tr(const FA_LDS uint8_t* base, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(base + off));
}
__device__ __forceinline__ bf16x8 join_tr(const s16x4& lo, const s16x4& hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 t = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, t);
}

// Round eight fp32 values to bf16 (nearest-even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 to_bf16x8(float a0, float a1, float a2, float a3, float a4, float a5,
                                            float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// Four fp32 -> four bf16 packed in 8 bytes.
__device__ __forceinline__ u32x2 pack4_bf16(float a0, float a1, float a2, float a3) {
  bf16x4 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Stores a wave's tile of MFMA results to global memory as bf16 rows, staged
// through LDS. Written straight from the C/D layout, each store instruction
// puts 8 bytes into each of 32 different rows, one memory request per row
// segment; read back from LDS in row order, each instruction writes whole
// 16-byte chunks of a few consecutive rows (16 times fewer segments for a
// 32 x 128 tile).
//   The tile is NB result blocks acc[b] (C/D layout above; the value of lane
// l, index r sits in column x = 8*(r/4) + 4*(l/32) + r%4 of the block's
// 32 x 32 and row l % 32). BY_BLOCK = false: block b holds tile columns
// 32b + x of the 32 tile rows l % 32. BY_BLOCK = true: block b holds tile
// rows 32b + l % 32 of the 32 tile columns x. Every value is multiplied by
// `scale` (per lane) and rounded to bf16. buf is this wave's LDS slice of
// SLICE bytes, touched by no other wave meanwhile; the tile passes through it
// in as many column passes as it needs (chunk c of row r is stored at chunk
// c ^ (r mod chunks per row), so the 8-byte writes and 16-byte reads of a
// wave spread over the banks). Tile row r goes to rowp(r) (bf16 pointer of
// its first column) when r < nrows.
template <int NB, bool BY_BLOCK, int SLICE, typename RowPtr>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[NB], float scale, FA_LDS uint8_t* buf, int lane,
                                           int nrows, RowPtr rowp) {
  constexpr int PB = BY_BLOCK ? NB : (SLICE / 2048 < NB ? SLICE / 2048 : NB);  // blocks per pass
  static_assert(PB >= 1 && NB % PB == 0 && (!BY_BLOCK || SLICE >= NB * 2048), "LDS slice too small");
  constexpr int W = BY_BLOCK ? 32 : 32 * PB;  // tile columns per pass
  constexpr int R = BY_BLOCK ? 32 * NB : 32;  // tile rows
  constexpr int NCH = W / 8;                  // 16-byte chunks per row
  constexpr int ROWB = 2 * W;
  constexpr int RPI = 1024 / ROWB;  // rows per 64-lane read of 16 bytes each
  const int c = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ps = 0; ps < NB / PB; ++ps) {
#pragma unroll
    for (int bb = 0; bb < PB; ++bb)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int b = ps * PB + bb;
        const int row = BY_BLOCK ? 32 * b + c : c;
        const int ch = BY_BLOCK ? rg : 4 * bb + rg;
        *reinterpret_cast<FA_LDS u32x2*>(buf + row * ROWB + ((ch ^ (row % NCH)) * 16) + 8 * h) =
            pack4_bf16(acc[b][4 * rg] * scale, acc[b][4 * rg + 1] * scale, acc[b][4 * rg + 2] * scale,
                       acc[b][4 * rg + 3] * scale);
      }
#pragma unroll
    for (int it = 0; it < R / RPI; ++it) {
      const int row = it * RPI + lane / NCH, ch = lane % NCH;
      const u32x4 v = *reinterpret_cast<const FA_LDS u32x4*>(buf + row * ROWB + ((ch ^ (row % NCH)) * 16));
      if (row < nrows) *reinterpret_cast<u32x4*>(rowp(row) + ps * W + ch * 8) = v;
    }
  }
}

// Logical workgroup index such that consecutive logical indices land on the
// same XCD: the dispatcher hands consecutive hardware ids to XCDs round
// robin, so hardware id i runs on XCD i % 8.
__device__ __forceinline__ int xcd_grouped_block(int bid, int nwg) {
  constexpr int kXcd = 8;
  const int xcd = bid % kXcd, slot = bid / kXcd;
  const int per = nwg / kXcd, rem = nwg % kXcd;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Wait until this wave's outstanding memory loads (including copies into LDS)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// The value x, opaque to the compiler (an empty asm that claims to rewrite
// the register; no instruction is emitted). Per-lane LDS offsets computed
// once and passed through this are added to compile-time stage bases as
// plain additions, which the compiler folds into the instructions' offset
// fields instead of materialising one register per (stage, offset) pair.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Byte offset of element (row, col) of a [rows][D] bf16 tile in LDS whose
// 16-byte chunks are XOR-swizzled per row. The swizzle value runs through
// all D/8 chunk indices over D/8 consecutive rows (row-wise operand reads by
// 32 consecutive rows spread over the banks) and moves rows r..r+3 into
// different 64-byte groups (the transposing reads touch 4 rows x 64 bytes
// per 16 lanes).
template <int D>
__device__ __forceinline__ uint32_t tile_off(int row, int col) {
  constexpr int CH = D / 8, G = CH / 4;
  const int sw = ((row % G) * 4 + (row / G) % 4) & (CH - 1);
  return (uint32_t)(row * D * 2 + ((((col >> 3) ^ sw)) << 4) + ((col & 7) << 1));
}

// Buffer resource over `bytes` bytes starting at `base` (raw addressing, no
// stride). Loads at offsets >= bytes return zero, which is how tail tiles
// are padded: rows past the end of a head arrive as zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Copying a ROWS x D bf16 tile into a swizzled LDS tile (see tile_off) with
// the WAVES waves of the workgroup, straight from memory into LDS
// (buffer_load_dwordx4 ... lds): wave w issues NI 1-KiB copies; lane l of
// copy i fills 16 bytes of row `row`, physical chunk l % CH, which holds
// logical chunk (l % CH) ^ swizzle(row). The per-lane byte offsets are
// computed once; each tile only adds a uniform offset.
// Copy 4 (dma4) or 16 (dma16) bytes per lane from a buffer of `bytes`
// bytes at `base`, byte offset lane_off + tile_bytes, into LDS at
// lds + size * lane. These wrappers are plain (non-template) functions:
// target builtins reached from template instantiations break the host
// compilation pass of the kernels.
// tile_bytes is the same for every lane of the wave; readfirstlane states
// so, and keeps the compiler from wrapping the copy in a per-lane loop when
// it cannot prove the value uniform.
__device__ __forceinline__ void dma4(const void* base, uint32_t bytes, int lane_off, int tile_bytes,
                                     FA_LDS void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), lds, 4, lane_off,
                                           __builtin_amdgcn_readfirstlane(tile_bytes), 0, 0);
}
__device__ __forceinline__ void dma16(const void* base, uint32_t bytes, int lane_off, int tile_bytes,
                                      FA_LDS void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc(base, bytes), lds, 16, lane_off,
                                           __builtin_amdgcn_readfirstlane(tile_bytes), 0, 0);
}

template <int D, int ROWS, int WAVES = 4>
struct TileDMA {
  static constexpr int CH = D / 8;     // 16-byte chunks per row
  static constexpr int RPI = 64 / CH;  // rows per wave-wide copy
  static constexpr int NI = ROWS / RPI / WAVES;
  static_assert(NI * RPI * WAVES == ROWS, "tile rows must split over the waves");
  int voff[NI];  // byte offset of this lane's chunk from the tile's first row

  __device__ __forceinline__ TileDMA(int w, int lane) {
    constexpr int G = CH / 4;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int row = (w * NI + i) * RPI + lane / CH;
      const int sw = ((row % G) * 4 + (row / G) % 4) & (CH - 1);
      voff[i] = (row * D + 8 * ((lane % CH) ^ sw)) * 2;
    }
  }
  // Copy the tile whose first row starts `tile_bytes` into a buffer of
  // `bytes` bytes at `base` (rows past the end arrive as zeros).
  __device__ __forceinline__ void copy(const void* base, uint32_t bytes, int tile_bytes, FA_LDS uint8_t* lds,
                                       int w) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) dma16(base, bytes, voff[i], tile_bytes, (FA_LDS void*)(lds + (w * NI + i) * 1024));
  }
};

// Wave-wide ballot: bit l is lane l's predicate.
__device__ __forceinline__ uint64_t ballot64(bool pred) { return __builtin_amdgcn_ballot_w64(pred); }

// The kept blocks of one row of a block mask (or one column, with a stride),
// read 64 blocks at a time: lane l loads the byte of block wb + l and a
// ballot packs the window into one 64-bit word. The skip decisions of a tile
// loop are then bit operations on that word, with one memory round trip per
// 64 blocks instead of one per tile. row2, when not null, is a second row
// whose kept blocks are added (a tile that spans two mask rows). Every lane
// of the wave calls the members together, with wave-uniform arguments.
struct MaskScan {
  const uint8_t* row;
  const uint8_t* row2;
  int stride;     // bytes between consecutive blocks
  int nb;         // blocks in the row
  int wb;         // first block of the loaded window, -1 before the first load
  uint64_t bits;  // bit k: block wb + k is kept

  __device__ __forceinline__ void init(const uint8_t* r, const uint8_t* r2, int s, int n) {
    row = r;
    row2 = r2;
    stride = s;
    nb = n;
    wb = -1;
    bits = 0;
  }
  __device__ __forceinline__ void load(int b) {
    wb = b & ~63;
    const int i = wb + (int)(threadIdx.x & 63);
    bool k = false;
    if (i < nb) {
      k = row[(size_t)i * stride] != 0;
      if (row2) k = k || row2[(size_t)i * stride] != 0;
    }
    bits = ballot64(k);
  }
  // Whether block b (0 <= b < nb) is kept.
  __device__ __forceinline__ bool kept(int b) {
    if (wb < 0 || b < wb || b >= wb + 64) load(b);
    return ((bits >> (b - wb)) & 1) != 0;
  }
  // First kept block >= b, or a value >= nb when there is none.
  __device__ __forceinline__ int next_kept(int b) {
    while (b < nb) {
      if (wb < 0 || b < wb || b >= wb + 64) load(b);
      const uint64_t m = bits >> (b - wb);
      if (m != 0) return b + __builtin_ctzll(m);
      b = wb + 64;
    }
    return b;
  }
};

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC 2011): each round multiplies counter
// words 0 and 2 by the round constants into 64-bit products and forms the
// new counter (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key advances by
// the Weyl constants between rounds. The key is wave-uniform, so its
// schedule stays in scalar registers.
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3, uint32_t k0,
                                              uint32_t k1, uint32_t (&out)[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0;
  out[1] = c1;
  out[2] = c2;
  out[3] = c3;
}

// 4 x 4 transpose across the four lanes of a quad (lane t = lane % 4 holds
// a[0..3]); afterwards lane t holds a[s] = the old a[t] of lane s. Two
// exchange stages with quad-permute DPP moves: lanes t and t^1 swap the
// off-diagonal elements of their 2 x 2 blocks, then lanes t and t^2.
__device__ __forceinline__ uint32_t quad_swap1(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
}
__device__ __forceinline__ uint32_t quad_swap2(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ void quad_transpose4(uint32_t (&a)[4], int t) {
  const bool odd = (t & 1) != 0, hi = (t & 2) != 0;
  {
    const uint32_t r0 = quad_swap1(odd ? a[0] : a[1]);
    const uint32_t r1 = quad_swap1(odd ? a[2] : a[3]);
    if (odd) {
      a[0] = r0;
      a[2] = r1;
    } else {
      a[1] = r0;
      a[3] = r1;
    }
  }
  {
    const uint32_t r0 = quad_swap2(hi ? a[0] : a[2]);
    const uint32_t r1 = quad_swap2(hi ? a[1] : a[3]);
    if (hi) {
      a[0] = r0;
      a[1] = r1;
    } else {
      a[2] = r0;
      a[3] = r1;
    }
  }
}

}  // namespace fa
