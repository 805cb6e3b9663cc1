// Internal launch interface between the C-ABI layer (fa2_api.cpp) and the
// kernel translation units.  Not installed, not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa2 {

// Arguments shared by every forward kernel.  All pointers are device
// pointers; shapes have been validated by the caller.
struct FwdArgs {
  const void *q;          // [B*H][Nq][d]
  const void *k, *v;      // [B*H_kv][Nk][d]
  void *o;                // [B*H][Nq][d]
  float *lse;             // [B*H][Nq] or nullptr
  int bh;                 // B*H
  int h;                  // H, query heads per batch index
  int group;              // H / H_kv, query heads per K/V head (1: none shared)
  int nq;                 // query rows per head
  int nk;                 // key rows per head
  int n_splits;           // key ranges computed separately, then merged
  float *o_part;          // [n_splits][B*H][Nq][d] fp32 (n_splits > 1)
  float *lse_part;        // [n_splits][B*H][Nq] fp32 (n_splits > 1)
  int d;                  // head dimension (64 or 128)
  float scale;            // multiplies q.k
  bool causal;
};

// Arguments of the backward pass (device pointers, validated shapes).
struct BwdArgs {
  const void *q, *o, *dout;          // [B*H][N][d] bf16
  const void *k, *v;                 // [B*H_kv][N][d] bf16
  const float *lse;                  // [B*H][N]
  float *delta;                      // [B*H][N], written
  void *dq;                          // [B*H][N][d], written
  void *dk, *dv;                     // [B*H_kv][N][d], written
  int bh;                            // B*H
  int h;                             // H, query heads per batch index
  int group;                         // H / H_kv (1: no shared K/V heads)
  int n_gsplits;                     // ranges of a group's query heads whose
                                     // dK/dV sums separate workgroups compute
  float *dkv_part;                   // [2][n_gsplits][B*H_kv][N][d] fp32
                                     // (n_gsplits > 1)
  int n;
  int d;
  float scale;
  bool causal;
};

// bf16 q/k/v on MFMA; o is bf16 (o32 == false) or fp32 (o32 == true).
hipError_t launch_fwd_bf16(const FwdArgs &a, bool o32, hipStream_t s);

// Bytes of the library's static device workspace (fa2_fwd_splitkv_noalloc:
// the fp32 partial outputs and lse of the key ranges).
constexpr size_t kFwdScratchBytes = size_t(32) << 20;
// Device address of that workspace on the current device (looked up once
// per device); no allocation.
hipError_t fwd_scratch(float **ptr);

// Gradients (bf16 MFMA); dq/dk/dv bf16 (o32 == false) or fp32 (true).
hipError_t launch_bwd_bf16(const BwdArgs &a, bool o32, hipStream_t s);

// fp32 q/k/v/o, fp32 arithmetic throughout.
hipError_t launch_fwd_fp32(const FwdArgs &a, hipStream_t s);

// FP8 block quantisation of one bf16 tensor [B*H][N][d].
struct QuantArgs {
  const void *x;       // bf16
  void *codes;         // e4m3 codes, same layout
  int *exps;           // [B*H][ceil(N / block_rows)] block exponents
  const float *signs;  // [d] +-1 (rotation) or nullptr
  int bh, n, d, block_rows;
};
hipError_t launch_quantize_fp8(const QuantArgs &a, hipStream_t s);

// FP8 attention on quantised Q (128-row blocks), K and V (64-row blocks).
struct Fp8Args {
  const void *q, *k, *v;     // e4m3 codes [B*H][N][d]
  const int *qe, *ke, *ve;   // block exponents
  void *o;                   // bf16 or fp32 [B*H][N][d]
  float *lse;                // [B*H][N] or nullptr
  int bh, n, d;
  float scale;               // already divided by d for rotated Q, K
  bool causal;
};
hipError_t launch_fwd_fp8(const Fp8Args &a, bool o32, hipStream_t s);

// FA2_DEBUG_ONE_WG_PER_CU=1 in the environment (read at every launch):
// *pad receives the dynamic LDS to request beside the kernel's static LDS so
// that one workgroup takes more than half of a compute unit's 160 KB and at
// most one runs per compute unit.  The kernels never touch that memory; the
// changed timing and co-residency test their barriers and LDS reuse, which
// must leave every output bit unchanged.  *pad = 0 when the switch is off.
hipError_t debug_lds_pad(const void *kernel, unsigned *pad);

// Query rows per workgroup of each kernel (the grid is B*H*ceil(N/rows)).
constexpr int kBf16RowsPerBlock = 128;
constexpr int kFp32RowsPerBlock = 64;
// FP8 path: Q blocks of 128 rows, K/V tiles of 64 rows (one exponent each).
constexpr int kFp8RowsPerBlock = 128;
constexpr int kFp8KvRowsPerBlock = 64;
// Rows (queries or keys) per workgroup of the backward kernels.
constexpr int kBf16BwdRowsPerBlock = 128;

}  // namespace fa2
