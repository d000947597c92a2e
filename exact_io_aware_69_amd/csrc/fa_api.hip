// C ABI of libfa.so: argument validation, launch geometry and status codes.
// The declarations and the contract of every entry point are in include/fa.h.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/fa.h"
#include "fa_params.h"

namespace fa {
hipError_t launch_fwd(const FwdParams& p, int BH, int d, int bm, int bn, bool causal, bool sparse, bool debug,
                      hipStream_t st);
bool fwd_config_supported(int bm, int bn);
size_t std_workspace_bytes(int B, int H, int N);
int std_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int H, int N,
            int d, bool causal, float scale, const uint8_t* mask, void* workspace, hipStream_t st);
constexpr int kStdMaxN = 16384;
size_t fa1_workspace_bytes(int B, int H, int N, int d);
hipError_t launch_fa1(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o, float* lse, int B, int H,
                      int N, int d, bool causal, float scale, int groups, void* workspace, hipStream_t st);
hipError_t launch_bwd(const BwdParams& p, int BH, int d, bool causal, bool sparse, bool debug, int stages,
                      hipStream_t st);
hipError_t launch_fwd_dropout(const FwdParams& p, int BH, int d, bool causal, bool sparse, hipStream_t st);
hipError_t launch_bwd_dropout(const BwdParams& p, int BH, int d, bool causal, bool sparse, int stages,
                              hipStream_t st);
hipError_t launch_dropout_keep(uint8_t* keep, int BH, int N, const Dropout& dr, hipStream_t st);
hipError_t launch_atomic_probe(float* dst, size_t nblk, int wgs, int reps, hipStream_t st);
}  // namespace fa

namespace {

// Largest supported sizes: one head of one tensor (N*d*2 bytes) must be
// addressable by a 32-bit buffer offset, and B*H*N*d elements fit
// comfortably in 64-bit offsets.
constexpr long long kMaxN = 1LL << 22;
constexpr long long kMaxElems = 1LL << 40;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int B, int H, int N, int d, float scale) {
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  if ((long long)B * H * N * d > kMaxElems) return FA_ERR_SHAPE;
  if ((long long)B * H * ((N + 63) / 64) > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_SCALE;
  return FA_OK;
}

int padded_rows(int N) { return (N + fa::BWD_PAD_ROWS - 1) / fa::BWD_PAD_ROWS * fa::BWD_PAD_ROWS; }

// Two fp32 arrays of B*H*Npad rows: D = rowsum(dO * O) and lse * log2(e).
size_t workspace_half(int B, int H, int N) {
  const size_t rows = (size_t)B * H * padded_rows(N);
  return (rows * sizeof(float) + 255) & ~(size_t)255;
}
// Block-sparse schedule: per head, sparse_kslots(nb) key-tile and nb
// query-tile int32 entries (fa_params.h).
size_t schedule_bytes(int H, int N) {
  const size_t nb = (size_t)(N + fa::MASK_BLOCK - 1) / fa::MASK_BLOCK;
  return ((size_t)H * (fa::sparse_kslots((int)nb) + nb) * sizeof(int) + 255) & ~(size_t)255;
}
size_t workspace_bytes_for(int B, int H, int N) { return 2 * workspace_half(B, H, N) + schedule_bytes(H, N); }

// Dropout arguments -> generator parameters; p must lie in [0, 1).
int make_dropout(float p, uint64_t seed, uint32_t offset, fa::Dropout* dr) {
  if (!(p >= 0.f) || !(p < 1.f)) return FA_ERR_DROPOUT;
  dr->t = (uint32_t)std::min(floor((double)p * 4294967296.0), 4294967295.0);
  dr->k0 = (uint32_t)(seed & 0xFFFFFFFFu);
  dr->k1 = (uint32_t)(seed >> 32);
  dr->off = offset;
  dr->scale = (float)(1.0 / (1.0 - (double)p));
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
             int causal, float scale, const uint8_t* mask, bool sparse, uint8_t* visited, void* stream,
             int bm = fa::FWD_BM, int bn = 0, const fa::Dropout* drop = nullptr) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (bn == 0) bn = d == 128 ? fa::fwd_bn<128>() : fa::fwd_bn<64>();  // the default tiles
  if (sparse && !mask) return FA_ERR_MASK;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return FA_ERR_ALIGN;
  fa::FwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.mask = mask;
  p.visited = visited;
  p.H = H;
  p.N = N;
  p.n_qt = (N + bm - 1) / bm;
  p.n_kt = (N + bn - 1) / bn;
  p.nb = (N + fa::MASK_BLOCK - 1) / fa::MASK_BLOCK;
  p.c = scale * 1.4426950408889634f;
  p.drop = drop ? *drop : fa::Dropout{0, 0, 0, 0, 1.0f};
  p.hgrp = 1;  // set per launch
  hipError_t e = drop ? fa::launch_fwd_dropout(p, B * H, d, causal != 0, sparse, (hipStream_t)stream)
                      : fa::launch_fwd(p, B * H, d, bm, bn, causal != 0, sparse, visited != nullptr,
                                       (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int bwd_impl(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
             void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
             const uint8_t* mask, bool sparse, void* workspace, size_t workspace_bytes, uint8_t* visited_kv,
             uint8_t* visited_q, int stages, void* stream, const fa::Dropout* drop = nullptr, float dropout_p = 0.f) {
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (sparse && !mask) return FA_ERR_MASK;
  if (!workspace || workspace_bytes < workspace_bytes_for(B, H, N)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv) || !aligned16(workspace))
    return FA_ERR_ALIGN;
  if ((visited_kv == nullptr) != (visited_q == nullptr)) return FA_ERR_NULL;
  fa::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.lse = lse;
  p.dO = static_cast<const uint16_t*>(dO);
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.Dneg = static_cast<float*>(workspace);
  p.lse2 = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + workspace_half(B, H, N));
  p.korder = reinterpret_cast<int*>(static_cast<uint8_t*>(workspace) + 2 * workspace_half(B, H, N));
  p.qorder = p.korder + (size_t)H * fa::sparse_kslots((N + fa::MASK_BLOCK - 1) / fa::MASK_BLOCK);
  p.mask = mask;
  p.visited_kv = visited_kv;
  p.visited_q = visited_q;
  p.H = H;
  p.N = N;
  p.Npad = padded_rows(N);
  p.nb = (N + fa::MASK_BLOCK - 1) / fa::MASK_BLOCK;
  p.c = scale * 1.4426950408889634f;
  p.scale = scale;
  p.dfac = drop ? (float)(1.0 - (double)dropout_p) : 1.0f;
  p.drop = drop ? *drop : fa::Dropout{0, 0, 0, 0, 1.0f};
  p.hgrp = 1;  // set per launch
  hipError_t e = drop ? fa::launch_bwd_dropout(p, B * H, d, causal != 0, sparse, stages, (hipStream_t)stream)
                      : fa::launch_bwd(p, B * H, d, causal != 0, sparse, visited_kv != nullptr, stages,
                                       (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

// ---------------------------------------------------------------- fa_bwd_noalloc
// The backward's scratch (D and lse * log2(e) per row, the block-sparse
// schedule) for callers that cannot allocate: one file-scope device array.
// Every GPU the library runs on holds its own copy until the process ends.
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device (hipGetSymbolAddress, with the
// device current) and only that address is handed to the kernels.
constexpr size_t kNoallocScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (FA_ERR_HIP if the
// runtime cannot tell).
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return FA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d, int causal,
           float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, nullptr, false, nullptr, stream);
}

int fa_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                       int causal, float scale, const uint8_t* block_mask, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, true, nullptr, stream);
}

int fa_fwd_tiles(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                 int causal, float scale, const uint8_t* block_mask, int bm, int bn, void* stream) {
  if (!fa::fwd_config_supported(bm, bn)) return FA_ERR_SHAPE;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, block_mask != nullptr, nullptr, stream,
                  bm, bn);
}

int fa_std_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, 1.0f);
  if (st != FA_OK) return st;
  if (N > fa::kStdMaxN) return FA_ERR_SHAPE;
  *bytes = fa::std_workspace_bytes(B, H, N);
  return FA_OK;
}

int fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, const uint8_t* block_mask, void* workspace, size_t workspace_bytes,
               void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (N > fa::kStdMaxN) return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < fa::std_workspace_bytes(B, H, N)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace)) return FA_ERR_ALIGN;
  const int r = fa::std_fwd(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                            static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B, H, N, d, causal != 0,
                            scale, block_mask, workspace, (hipStream_t)stream);
  return r == 0 ? FA_OK : FA_ERR_HIP;
}

int fa_fa1_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, 1.0f);
  if (st != FA_OK) return st;
  *bytes = fa::fa1_workspace_bytes(B, H, N, d);
  return FA_OK;
}

int fa_fwd_fa1(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
               int causal, float scale, int seq_groups, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (seq_groups < 1 || (long long)B * H * std::min(seq_groups, (N + 31) / 32) > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!workspace || workspace_bytes < fa::fa1_workspace_bytes(B, H, N, d)) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(workspace)) return FA_ERR_ALIGN;
  const hipError_t e = fa::launch_fa1(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                                      static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, B, H, N, d,
                                      causal != 0, scale, seq_groups, workspace, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_workspace_size(int B, int H, int N, int d, size_t* bytes) {
  if (!bytes) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, 1.0f);
  if (st != FA_OK) return st;
  *bytes = workspace_bytes_for(B, H, N);
  return FA_OK;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO, void* dq,
           void* dk, void* dv, int B, int H, int N, int d, int causal, float scale, void* workspace,
           size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, nullptr, false, workspace,
                  workspace_bytes, nullptr, nullptr, 7, stream);
}

int fa_bwd_blocksparse(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                       void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                       const uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, true, workspace,
                  workspace_bytes, nullptr, nullptr, 7, stream);
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                   const uint8_t* block_mask, void* stream) {
  // Every argument check, the scratch limit included, comes before the
  // first HIP call.
  if (!q || !k || !v || !o || !lse || !dO || !dq || !dk || !dv) return FA_ERR_NULL;
  int st = check_common(B, H, N, d, scale);
  if (st != FA_OK) return st;
  if (workspace_bytes_for(B, H, N) > kNoallocScratchBytes) return FA_ERR_WORKSPACE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dO) || !aligned16(dq) ||
      !aligned16(dk) || !aligned16(dv))
    return FA_ERR_ALIGN;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != FA_OK) return st;
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, block_mask != nullptr, ws,
                  kNoallocScratchBytes, nullptr, nullptr, 7, stream);
}

int fa_bwd_stage(int stage, const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dO, void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                 const uint8_t* block_mask, void* workspace, size_t workspace_bytes, void* stream) {
  if (stage < 0 || stage > 2) return FA_ERR_SHAPE;
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, block_mask != nullptr,
                  workspace, workspace_bytes, nullptr, nullptr, 1 << stage, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                   int causal, float scale, const uint8_t* block_mask, float dropout_p, uint64_t seed,
                   uint32_t offset, void* stream) {
  fa::Dropout dr;
  const int st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, block_mask != nullptr, nullptr, stream,
                  fa::FWD_BM, 0, &dr);
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                   void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                   const uint8_t* block_mask, float dropout_p, uint64_t seed, uint32_t offset, void* workspace,
                   size_t workspace_bytes, void* stream) {
  fa::Dropout dr;
  const int st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, block_mask != nullptr,
                  workspace, workspace_bytes, nullptr, nullptr, 7, stream, &dr, dropout_p);
}

int fa_dropout_keep(int B, int H, int N, float dropout_p, uint64_t seed, uint32_t offset, uint8_t* keep,
                    void* stream) {
  if (!keep) return FA_ERR_NULL;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN) return FA_ERR_SHAPE;
  if ((long long)B * H * N * ((N + 3) / 4) / 256 >= 0x7fffffffLL) return FA_ERR_SHAPE;
  fa::Dropout dr;
  const int st = make_dropout(dropout_p, seed, offset, &dr);
  if (st != FA_OK) return st;
  const hipError_t e = fa::launch_dropout_keep(keep, B * H, N, dr, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_atomic_add_probe(float* dst, size_t dst_floats, int workgroups, int reps, void* stream) {
  if (!dst) return FA_ERR_NULL;
  if (!aligned16(dst)) return FA_ERR_ALIGN;
  const size_t nblk = dst_floats / (64 * 128);
  if (nblk < 1 || workgroups < 1 || reps < 1) return FA_ERR_SHAPE;
  const hipError_t e = fa::launch_atomic_probe(dst, nblk, workgroups, reps, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

#ifndef FA_BUILD_ID
#define FA_BUILD_ID "unknown"
#endif
const char* fa_build_id(void) { return FA_BUILD_ID; }

int fa_tile_config(int pass, int d, int causal, int* bm, int* bn) {
  if (!bm || !bn) return FA_ERR_NULL;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED_D;
  switch (pass) {
    case 0: *bm = fa::FWD_BM; *bn = d == 128 ? fa::fwd_bn<128>() : fa::fwd_bn<64>(); return FA_OK;
    case 1:
      *bm = d == 128 ? fa::bwd_kv_bm<128>() : fa::bwd_kv_bm<64>();
      *bn = d == 128 ? fa::bwd_kv_bn<128>() : fa::bwd_kv_bn<64>();
      return FA_OK;
    case 2:
      *bm = fa::BWD_Q_BM;
      if (d == 64)
        *bn = fa::bwd_q_bn<64, false, false>();
      else
        *bn = causal ? fa::bwd_q_bn<128, true, false>() : fa::bwd_q_bn<128, false, false>();
      return FA_OK;
    default: return FA_ERR_SHAPE;
  }
}

int fa_fwd_debug_visits(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N, int d,
                        int causal, float scale, const uint8_t* block_mask, uint8_t* visited, void* stream) {
  if (!visited) return FA_ERR_NULL;
  return fwd_impl(q, k, v, o, lse, B, H, N, d, causal, scale, block_mask, block_mask != nullptr, visited, stream);
}

int fa_bwd_debug_visits(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dO,
                        void* dq, void* dk, void* dv, int B, int H, int N, int d, int causal, float scale,
                        const uint8_t* block_mask, void* workspace, size_t workspace_bytes, uint8_t* visited_kv,
                        uint8_t* visited_q, void* stream) {
  if (!visited_kv || !visited_q) return FA_ERR_NULL;
  return bwd_impl(q, k, v, o, lse, dO, dq, dk, dv, B, H, N, d, causal, scale, block_mask, block_mask != nullptr,
                  workspace, workspace_bytes, visited_kv, visited_q, 7, stream);
}

const char* fa_status_str(int status) {
  switch (status) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: B, H, N out of range";
    case FA_ERR_UNSUPPORTED_D: return "FA_ERR_UNSUPPORTED_D: head dimension must be 64 or 128";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale must be finite and > 0";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: backward workspace missing or too small";
    case FA_ERR_MASK: return "FA_ERR_MASK: block-sparse call without a block mask";
    case FA_ERR_HIP: return "FA_ERR_HIP: a HIP launch or rocBLAS call failed";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: device pointers must be 16-byte aligned";
    case FA_ERR_DROPOUT: return "FA_ERR_DROPOUT: dropout probability must be in [0, 1)";
    default: return "unknown fa status";
  }
}

}  // extern "C"
