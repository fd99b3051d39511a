// Internal host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  void* stream;
};

// Work layouts of the bf16 prefill (the numbers are the FA_LAYOUT_* values of
// the public header).
enum FwdLayoutKind {
  kLayoutKvParity = 0,        // 128 rows, KV-parity wave groups
  kLayoutKvParityPaired = 1,  // same, causal pairs of query blocks
  kLayoutRows = 2,            // 256 rows, row groups
  kLayoutRowsPaired = 3,      // same, causal pairs
  kLayoutWideOneGroup = 4,    // d = 192/256: 4 waves, two workgroups per CU
  kLayoutWideTwoGroups = 5,   // d = 192/256: 8 waves, KV-parity groups
};

struct FwdPlan {
  int layout;  // FwdLayoutKind
  int n_qt;    // query blocks per head in the layout's block size
  long n_wg;   // workgroups
};

struct SplitArgs {
  FwdArgs f;
  int num_splits;
  float* o_part;    // [B, Hq, S, Nq, d]
  float* lse_part;  // [B, Hq, S, Nq]
  // Paged K/V when `paged` is set: f.k, f.v are [num_pages, Hkv,
  // 2^log2_page, d] caches and f.Nk is unused (per-sequence lengths instead).
  int paged = 0;
  const int* block_table = nullptr;  // [B, max_pages]
  const int* seq_lens = nullptr;     // [B]
  int num_pages = 0, log2_page = 0, max_pages = 0;
};

struct CombineArgs {
  const float* o_part;
  const float* lse_part;
  void* o;
  float* lse;
  int B, Hq, Nq, d, num_splits;
  void* stream;
};

// Backward: f carries q, k, v, the forward's lse, sizes, scale, mask, stream.
struct BwdArgs {
  FwdArgs f;
  const void* o;     // forward output [B, Hq, Nq, d] bf16
  const void* dout;  // dO [B, Hq, Nq, d] bf16
  void* dq;          // [B, Hq, Nq, d] bf16
  void* dk;          // [B, Hkv, Nk, d] bf16
  void* dv;          // [B, Hkv, Nk, d] bf16
  float* dsum;       // workspace: fp32 D [B, Hq, Nq]
};

hipError_t launch_fwd_bf16(const FwdArgs& a);       // d = 64, 128
FwdPlan plan_fwd_bf16(int B, int Hq, int Nq, int causal);
int fwd_wide_layout(int B, int Hq, int Nq);
hipError_t launch_fwd_bf16_wide(const FwdArgs& a);  // d = 192, 256
hipError_t launch_fwd_fp32(const FwdArgs& a);
// q, k, v of `a` are E4M3 bytes (d = 128); o is bf16, lse fp32.
hipError_t launch_fwd_fp8(const FwdArgs& a, float q_descale, float k_descale, float v_descale);
hipError_t launch_splitkv_partial(const SplitArgs& a);
hipError_t launch_combine(const CombineArgs& a);
hipError_t launch_bwd(const BwdArgs& a);

// Grid sizes (workgroups) the launchers would use; the ABI layer checks them
// against the hardware limit before launching.
long fwd_bf16_grid(int B, int Hq, int Nq);
long fwd_fp32_grid(int B, int Hq, int Nq);
long fwd_fp8_grid(int B, int Hq, int Nq);
long splitkv_grid(int B, int Hq, int Hkv, int Nq, int num_splits);
long combine_grid(int B, int Hq, int Nq);
long bwd_grid(int B, int Hkv, int Nk);

}  // namespace fa
