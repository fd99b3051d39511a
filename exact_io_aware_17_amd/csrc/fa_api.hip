// C ABI of the attention library: host-side argument checks, workspace sizing
// and dispatch to the kernel launchers. No device memory is allocated here and
// nothing is enqueued unless every check passes.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_internal.h"

// Scratch of fa_fwd_splitkv_noalloc: the split partials (O_s, then LSE_s)
// live here instead of in a caller workspace. Each GPU holds its own copy
// for the life of the process. Host code never uses the name `scratch` as a
// device address (on the host it is only a stand-in for the symbol); the
// device address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxSplits = 1024;
constexpr long kMaxGridX = 2147483647L;
constexpr long kMaxGridYZ = 65535L;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Element count of a [a, b, c, d] tensor, or -1 if it does not fit in int64
// with room to spare for byte offsets.
long long elems4(long long a, long long b, long long c, long long d) {
  const long long lim = (1LL << 60);
  long long r = 1;
  for (long long x : {a, b, c, d}) {
    if (x < 0) return -1;
    if (x != 0 && r > lim / x) return -1;
    r *= x;
  }
  return r;
}

fa_status check_common(const void* q, const void* k, const void* v, const void* o, const void* lse, int B,
                       int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal) {
  if (B < 0 || Nq < 0 || Nk < 0 || Hq < 1 || Hkv < 1 || d < 1) return FA_ERR_SHAPE;
  if (Hq % Hkv != 0) return FA_ERR_SHAPE;
  const long long nq = elems4(B, Hq, Nq, d), nkv = elems4(B, Hkv, Nk, d);
  if (nq < 0 || nkv < 0) return FA_ERR_SHAPE;
  if ((long long)B * Hq > 0x7fffffffLL || (long long)B * Hkv > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (d != 64 && d != 128 && d != 192 && d != 256) return FA_ERR_UNSUPPORTED;
  if (!(scale > 0.f) || !isfinite(scale)) return FA_ERR_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  // Pointers of empty tensors may be NULL (allocators hand out NULL for them).
  if (nq > 0 && (!q || !o || !lse)) return FA_ERR_NULL;
  if (nkv > 0 && (!k || !v)) return FA_ERR_NULL;
  for (const void* p : {q, k, v, o, lse})
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  return FA_OK;
}

fa_status launched(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

size_t round256(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Workspace layout of the split path: O_s then (256-aligned) LSE_s.
bool split_ws_sizes(int B, int Hq, int Nq, int d, int S, size_t* o_bytes, size_t* total) {
  if (B < 0 || Hq < 1 || Nq < 0 || S < 1 || S > kMaxSplits || (d != 64 && d != 128)) return false;
  const long long rows = elems4(B, Hq, S, Nq);
  if (rows < 0 || rows > (1LL << 50)) return false;
  *o_bytes = round256((size_t)rows * (size_t)d * 4u);
  *total = *o_bytes + round256((size_t)rows * 4u);
  return true;
}

// Workspace of the backward pass: the fp32 row sums D.
bool bwd_ws_sizes(int B, int Hq, int Nq, int d, size_t* total) {
  if (B < 0 || Hq < 1 || Nq < 0 || (d != 64 && d != 128)) return false;
  const long long rows = elems4(B, Hq, Nq, 1);
  if (rows < 0 || rows > (1LL << 50)) return false;
  *total = round256((size_t)rows * 4u);  // fp32 D per row
  return true;
}

// Device address of `scratch` on device `dev`, looked up on the first call
// for that device (with the device current) and cached.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

fa_status noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FA_ERR_LAUNCH;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_LAUNCH;
    }
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA_ERR_LAUNCH;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return FA_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

#ifndef FA_SOURCE_HASH
#define FA_SOURCE_HASH "unknown"
#endif

const char* fa_build_hash(void) { return FA_SOURCE_HASH; }

float fa_default_scale(int d) { return d >= 1 ? (float)(1.0 / sqrt((double)d)) : 0.f; }

const char* fa_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid or overflowing sizes, or Hq % Hkv != 0";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: head size or mode not implemented";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: a pointer is not 16-byte aligned (workspace: 256-byte)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: kernel launch failed";
    case FA_ERR_ARG: return "FA_ERR_ARG: scale not finite and > 0, causal not 0/1, or bad split count";
  }
  return "unknown fa_status";
}

static_assert(fa::kLayoutKvParity == FA_LAYOUT_KV_PARITY && fa::kLayoutKvParityPaired == FA_LAYOUT_KV_PARITY_PAIRED &&
                  fa::kLayoutRows == FA_LAYOUT_ROWS && fa::kLayoutRowsPaired == FA_LAYOUT_ROWS_PAIRED &&
                  fa::kLayoutWideOneGroup == FA_LAYOUT_WIDE_ONE_GROUP &&
                  fa::kLayoutWideTwoGroups == FA_LAYOUT_WIDE_TWO_GROUPS,
              "layout numbers must match the header");

int fa_fwd_layout(int B, int Hq, int Nq, int d, int causal) {
  if (d == 64 || d == 128) return fa::plan_fwd_bf16(B, Hq, Nq, causal ? 1 : 0).layout;
  if (d == 192 || d == 256) return fa::fwd_wide_layout(B, Hq, Nq);
  return -1;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (fa::fwd_bf16_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  return launched(d > 128 ? fa::launch_fwd_bf16_wide(a) : fa::launch_fwd_bf16(a));
}

fa_status fa_fwd_fp32(const float* q, const float* k, const float* v, float* o, float* lse, int B, int Hq,
                      int Hkv, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  if (fa::fwd_fp32_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  return launched(fa::launch_fwd_fp32(a));
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, float q_descale, float k_descale,
                     float v_descale, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                     float scale, int causal, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d != 128) return FA_ERR_UNSUPPORTED;
  for (float x : {q_descale, k_descale, v_descale})
    if (!(x > 0.f) || !isfinite(x)) return FA_ERR_ARG;
  // The score scale the kernel uses (scale * q_descale * k_descale * log2 e)
  // must be a finite, non-zero fp32 value.
  const double sl2 = (double)scale * q_descale * k_descale * 1.4426950408889634;
  if (!(sl2 >= 1.1754943508222875e-38) || !(sl2 <= 3.4028234663852886e38)) return FA_ERR_ARG;
  if (fa::fwd_fp8_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  return launched(fa::launch_fwd_fp8(a, q_descale, k_descale, v_descale));
}

size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq, int d) {
  size_t total = 0;
  if (!bwd_ws_sizes(B, Hq, Nq, d, &total)) return 0;
  return total;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                 void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                 int causal, void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  const long long nq = elems4(B, Hq, Nq, d), nkv = elems4(B, Hkv, Nk, d);
  if (nq > 0 && (!dout || !dq)) return FA_ERR_NULL;
  if (nkv > 0 && (!dk || !dv)) return FA_ERR_NULL;
  for (const void* p : {dout, (const void*)dq, (const void*)dk, (const void*)dv})
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  size_t total = 0;
  if (!bwd_ws_sizes(B, Hq, Nq, d, &total)) return FA_ERR_SHAPE;
  if (nq > 0) {
    if (!workspace || workspace_bytes < total) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  }
  // Grids: dK/dV kernel bwd_grid, D kernel B*Hq*Nq/4 (rounded up); the dQ
  // kernel's B*Hq*ceil(Nq/128) is never larger than the D kernel's.
  if (fa::bwd_grid(B, Hkv, Nk) > kMaxGridX || (long long)B * Hq * Nq / 4 + 1 > kMaxGridX)
    return FA_ERR_UNSUPPORTED;
  if (nq == 0 && nkv == 0) return FA_OK;
  fa::FwdArgs f{q, k, v, nullptr, const_cast<float*>(lse), B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  fa::BwdArgs a{f, o, dout, dq, dk, dv, (float*)workspace};
  return launched(fa::launch_bwd(a));
}

size_t fa_splitkv_workspace_bytes(int B, int Hq, int Nq, int d, int num_splits) {
  size_t ob = 0, total = 0;
  if (!split_ws_sizes(B, Hq, Nq, d, num_splits, &ob, &total)) return 0;
  return total;
}

fa_status fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                         int Hkv, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                         void* workspace, size_t workspace_bytes, void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  size_t ob = 0, total = 0;
  if (!split_ws_sizes(B, Hq, Nq, d, num_splits, &ob, &total)) return FA_ERR_SHAPE;
  const long long rows = (long long)B * Hq * Nq;
  if (rows > 0) {
    if (!workspace || workspace_bytes < total) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  }
  if (fa::splitkv_grid(B, Hq, Hkv, Nq, num_splits) > kMaxGridX || B > kMaxGridYZ || Hkv > kMaxGridYZ)
    return FA_ERR_UNSUPPORTED;
  if (fa::combine_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  if (rows == 0) return FA_OK;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + ob);
  fa::FwdArgs f{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  fa::SplitArgs sa{f, num_splits, o_part, lse_part};
  st = launched(fa::launch_splitkv_partial(sa));
  if (st != FA_OK) return st;
  fa::CombineArgs ca{o_part, lse_part, o, lse, B, Hq, Nq, d, num_splits, stream};
  return launched(fa::launch_combine(ca));
}

fa_status fa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                                 int Hkv, int Nq, int Nk, int d, float scale, int causal, int num_splits,
                                 void* stream) {
  fa_status st = check_common(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  size_t ob = 0, total = 0;
  if (!split_ws_sizes(B, Hq, Nq, d, num_splits, &ob, &total)) return FA_ERR_SHAPE;
  if (total > (size_t)FA_NOALLOC_SCRATCH_BYTES) return FA_ERR_WORKSPACE;
  if (fa::splitkv_grid(B, Hq, Hkv, Nq, num_splits) > kMaxGridX || B > kMaxGridYZ || Hkv > kMaxGridYZ)
    return FA_ERR_UNSUPPORTED;
  if (fa::combine_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  if ((long long)B * Hq * Nq == 0) return FA_OK;
  void* ws = nullptr;
  st = noalloc_scratch(stream, &ws);
  if (st != FA_OK) return st;
  // The partial kernel writes every element of both partial arrays (an empty
  // chunk writes O_s = 0 and LSE_s = -inf), so nothing left in the scratch by
  // an earlier call is read.
  float* o_part = (float*)ws;
  float* lse_part = (float*)((char*)ws + ob);
  fa::FwdArgs f{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream};
  fa::SplitArgs sa{f, num_splits, o_part, lse_part};
  st = launched(fa::launch_splitkv_partial(sa));
  if (st != FA_OK) return st;
  fa::CombineArgs ca{o_part, lse_part, o, lse, B, Hq, Nq, d, num_splits, stream};
  return launched(fa::launch_combine(ca));
}

fa_status fa_fwd_splitkv_paged(const void* q, const void* k_cache, const void* v_cache, const int* block_table,
                               const int* seq_lens, void* o, float* lse, int B, int Hq, int Hkv, int Nq, int d,
                               int num_pages, int page_size, int max_pages, float scale, int causal, int num_splits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (page_size < 16 || page_size > (1 << 16) || (page_size & (page_size - 1)) != 0) return FA_ERR_ARG;
  if (num_pages < 0 || max_pages < 0) return FA_ERR_SHAPE;
  if ((long long)max_pages * page_size > 0x7fffffffLL) return FA_ERR_SHAPE;
  // The caches as [num_pages, Hkv, page_size, d] for the shared checks.
  fa_status st = check_common(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, 0, d, scale, causal);
  if (st != FA_OK) return st;
  if (d > 128) return FA_ERR_UNSUPPORTED;
  if (elems4(num_pages, Hkv, page_size, d) < 0 || elems4(B, max_pages, 1, 1) < 0) return FA_ERR_SHAPE;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  size_t ob = 0, total = 0;
  if (!split_ws_sizes(B, Hq, Nq, d, num_splits, &ob, &total)) return FA_ERR_SHAPE;
  const long long rows = (long long)B * Hq * Nq;
  if (rows == 0) return FA_OK;
  if (!seq_lens) return FA_ERR_NULL;
  if (max_pages > 0) {
    // Keys may exist: the caches and the table must be there.
    if (!block_table || !k_cache || !v_cache) return FA_ERR_NULL;
    if (num_pages < 1) return FA_ERR_SHAPE;
  }
  for (const void* p : {(const void*)k_cache, (const void*)v_cache})
    if (p && !aligned16(p)) return FA_ERR_ALIGN;
  for (const void* p : {(const void*)block_table, (const void*)seq_lens})
    if (p && ((uintptr_t)p & 3u) != 0) return FA_ERR_ALIGN;
  if (!workspace || workspace_bytes < total) return FA_ERR_WORKSPACE;
  if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  if (fa::splitkv_grid(B, Hq, Hkv, Nq, num_splits) > kMaxGridX || B > kMaxGridYZ || Hkv > kMaxGridYZ)
    return FA_ERR_UNSUPPORTED;
  if (fa::combine_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  int log2_page = 0;
  while ((1 << log2_page) < page_size) ++log2_page;
  float* o_part = (float*)workspace;
  float* lse_part = (float*)((char*)workspace + ob);
  fa::FwdArgs f{q, k_cache, v_cache, o, lse, B, Hq, Hkv, Nq, 0, d, scale, causal, stream};
  fa::SplitArgs sa{f, num_splits, o_part, lse_part};
  // With max_pages == 0 every sequence is empty and no table entry is read.
  sa.paged = 1;
  sa.block_table = block_table;
  sa.seq_lens = seq_lens;
  sa.num_pages = num_pages > 0 ? num_pages : 1;
  sa.log2_page = log2_page;
  sa.max_pages = max_pages;
  st = launched(fa::launch_splitkv_partial(sa));
  if (st != FA_OK) return st;
  fa::CombineArgs ca{o_part, lse_part, o, lse, B, Hq, Nq, d, num_splits, stream};
  return launched(fa::launch_combine(ca));
}

fa_status fa_combine(const float* o_part, const float* lse_part, void* o, float* lse, int B, int Hq, int Nq,
                     int d, int num_splits, void* stream) {
  if (B < 0 || Hq < 1 || Nq < 0) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_ARG;
  size_t ob = 0, total = 0;
  if (!split_ws_sizes(B, Hq, Nq, d, num_splits, &ob, &total)) return FA_ERR_SHAPE;
  const long long rows = (long long)B * Hq * Nq;
  if (rows == 0) return FA_OK;
  if (!o_part || !lse_part || !o || !lse) return FA_ERR_NULL;
  for (const void* p : {(const void*)o_part, (const void*)lse_part, (const void*)o, (const void*)lse})
    if (!aligned16(p)) return FA_ERR_ALIGN;
  if (fa::combine_grid(B, Hq, Nq) > kMaxGridX) return FA_ERR_UNSUPPORTED;
  fa::CombineArgs ca{o_part, lse_part, o, lse, B, Hq, Nq, d, num_splits, stream};
  return launched(fa::launch_combine(ca));
}

}  // extern "C"
