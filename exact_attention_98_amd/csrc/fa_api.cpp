// C ABI of the attention library: argument checks, workspace sizing and
// dispatch to the gfx950 kernels.  Every check runs before any launch, the
// library allocates and synchronizes nothing, and no exception crosses the
// boundary.  Its only state is the per-device address of the fixed scratch
// behind fa_bwd_noalloc.
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/fa.h"
#include "kernels.hpp"

namespace {

// Share of exponentials given to the FMA polynomial by fa_fwd.
constexpr int kDefaultPolyQuarters = 0;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}

// Shape checks shared by forward and backward.
int check_shape(int B, int Hq, int Hkv, int N, int D, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || N < 1 || D < 1) return FA_ERR_INVALID;
  if (Hq % Hkv != 0) return FA_ERR_INVALID;
  if (!isfinite(scale)) return FA_ERR_INVALID;
  if (!(scale > 0.f)) return FA_ERR_UNSUPPORTED;
  if (D != 64 && D != 128) return FA_ERR_UNSUPPORTED;
  const uint64_t elems = (uint64_t)B * (uint64_t)Hq * (uint64_t)N * (uint64_t)D;
  if (elems >= (1ull << 31)) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

// Largest byte range of one head's fp32 rows that the kernels address with
// 32-bit signed offsets (the atomic dQ accumulator, the split-KV partials).
constexpr uint64_t kMaxFp32HeadBytes = 0x7FFFFFFFull;

// The dQ mode (the deterministic argument): 0 atomic, 1 stored dS, 2
// recompute.  Stored-dS blocks of one head are addressed with 32-bit offsets,
// with offsets from 2^32 - 4096 up reserved as "no block"; the atomic mode's
// fp32 accumulator rows of one head with 32-bit signed offsets.
int check_mode(int N, int D, int deterministic) {
  if (deterministic < 0 || deterministic > 2) return FA_ERR_INVALID;
  if (deterministic == 1 && fa::ds_head_bytes(N) > 0xFFFFF000ull - 4096) return FA_ERR_TOO_LARGE;
  if (deterministic == 0 && (uint64_t)N * (uint64_t)D * 4u > kMaxFp32HeadBytes) return FA_ERR_TOO_LARGE;
  return FA_OK;
}

int fwd_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int N, int D, int causal, float scale, int poly_quarters, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  int rc = check_shape(B, Hq, Hkv, N, D, scale);
  if (rc != FA_OK) return rc;
  if (poly_quarters < 0 || poly_quarters > 2) return FA_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t qbytes = (size_t)B * Hq * N * D * 2, kvbytes = (size_t)B * Hkv * N * D * 2;
  const size_t lbytes = (size_t)B * Hq * N * 4;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
      overlaps(o, qbytes, v, kvbytes) || overlaps(lse, lbytes, o, qbytes) ||
      overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kvbytes) ||
      overlaps(lse, lbytes, v, kvbytes))
    return FA_ERR_INVALID;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, D, causal ? 1 : 0, scale, poly_quarters};
  hipError_t e = fa::launch_fwd(a, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int N, int D, int causal, float scale, void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, scale, kDefaultPolyQuarters, stream);
}

int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
              int Hkv, int N, int D, int causal, float scale, int exp_poly_quarters,
              void* stream) {
  return fwd_impl(q, k, v, o, lse, B, Hq, Hkv, N, D, causal, scale, exp_poly_quarters, stream);
}

size_t fa_fwd_varlen_workspace_size(int B, int total) {
  if (B < 1 || total < 0) return 0;
  return fa::varlen_workspace_bytes(B, total);
}

int fa_varlen_max_seqlen(void) { return fa::varlen_max_seqlen_limit(); }

int fa_exp2_poly_eval(const float* x, float* y, int n, void* stream) {
  if (n < 0 || (n > 0 && (!x || !y))) return FA_ERR_INVALID;
  return fa::launch_exp2_poly_eval(x, y, n, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens, int B, int Hq, int Hkv, int total, int max_seqlen, int D,
                  int causal, float scale, void* workspace, size_t workspace_bytes,
                  void* stream) {
  if (!q || !k || !v || !o || !lse || !cu_seqlens || !workspace) return FA_ERR_INVALID;
  if (B < 1 || total < 0 || max_seqlen < 1 || max_seqlen > fa::varlen_max_seqlen_limit())
    return FA_ERR_INVALID;
  // Shape checks as for one sequence of total tokens (at least 1).
  int rc = check_shape(1, Hq, Hkv, total > 0 ? total : 1, D, scale);
  if (rc != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(cu_seqlens))
    return FA_ERR_ALIGN;
  if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  const size_t wbytes = fa::varlen_workspace_bytes(B, total);
  if (workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
  const size_t qbytes = (size_t)Hq * total * D * 2, kvbytes = (size_t)Hkv * total * D * 2;
  const size_t lbytes = (size_t)Hq * total * 4, cbytes = (size_t)(B + 1) * 4;
  const void* outs[3] = {o, lse, workspace};
  const size_t osz[3] = {qbytes, lbytes, wbytes};
  const void* ins[4] = {q, k, v, cu_seqlens};
  const size_t isz[4] = {qbytes, kvbytes, kvbytes, cbytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_INVALID;
    for (int j = 0; j < 3; ++j)
      if (j != i && overlaps(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_INVALID;
  }
  if (total == 0) return FA_OK;
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, max_seqlen, D, causal ? 1 : 0, scale, 0};
  const fa::VarlenArgs va{cu_seqlens, B, total, max_seqlen, workspace};
  return fa::launch_fwd_varlen(a, va, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // extern "C"

namespace {

// dQ mode of the variable-length backward: 0, 1 or 2.  In mode 1 one head's
// region of dS blocks (bounded by total, B and max_seqlen) is addressed with
// 32-bit offsets, as in the dense stored-dS mode; in mode 0 one head's fp32
// accumulator rows (all total of them) with 32-bit signed offsets.
int check_varlen_mode(int B, int total, int max_seqlen, int D, int deterministic) {
  if (deterministic < 0 || deterministic > 2) return FA_ERR_INVALID;
  if (deterministic == 1 && fa::varlen_ds_head_bytes(B, total, max_seqlen) > 0xFFFFF000ull - 4096)
    return FA_ERR_TOO_LARGE;
  if (deterministic == 0) return check_mode(total, D, 0);
  return FA_OK;
}

// Shape checks of the split-KV forward (q and k checked as their own
// tensors, which may differ in length).
int check_split(int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, float scale) {
  if (Nq < 1 || Nk < 1) return FA_ERR_INVALID;
  if (causal && Nq > Nk) return FA_ERR_INVALID;
  int rc = check_shape(B, Hq, Hkv, Nq, D, scale);
  if (rc != FA_OK) return rc;
  return check_shape(B, Hkv, Hkv, Nk, D, scale);
}

int resolve_splits(int B, int Hq, int Hkv, int Nq, int Nk, int num_splits) {
  if (num_splits == 0) return fa::split_auto(B, Hq, Hkv, Nq, Nk);
  if (num_splits < 0 || num_splits > fa::split_max(Nk)) return -1;
  return num_splits;
}

// With more than one key range, the fp32 partial rows of one K/V head group
// (G * Nq rows of D) are addressed with 32-bit signed offsets.
int check_split_partials(int Hq, int Hkv, int Nq, int D, int splits) {
  if (splits > 1 && (uint64_t)(Hq / Hkv) * (uint64_t)Nq * (uint64_t)D * 4u > kMaxFp32HeadBytes)
    return FA_ERR_TOO_LARGE;
  return FA_OK;
}

}  // namespace

extern "C" {

size_t fa_bwd_varlen_workspace_size(int B, int Hq, int Hkv, int total, int max_seqlen, int D,
                                    int deterministic) {
  if (B < 1 || total < 0) return 0;
  if (max_seqlen < 1 || max_seqlen > fa::varlen_max_seqlen_limit() / 2) return 0;
  if (check_shape(1, Hq, Hkv, total > 0 ? total : 1, D, 1.0f) != FA_OK) return 0;
  if (check_varlen_mode(B, total, max_seqlen, D, deterministic) != FA_OK) return 0;
  return fa::bwd_varlen_workspace_bytes(B, Hq, total, D, deterministic, max_seqlen);
}

int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens,
                  int B, int Hq, int Hkv, int total, int max_seqlen, int D, int causal,
                  float scale, void* workspace, size_t workspace_bytes, int deterministic,
                  void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !cu_seqlens || !workspace)
    return FA_ERR_INVALID;
  if (B < 1 || total < 0 || max_seqlen < 1 || max_seqlen > fa::varlen_max_seqlen_limit() / 2)
    return FA_ERR_INVALID;
  int rc = check_shape(1, Hq, Hkv, total > 0 ? total : 1, D, scale);
  if (rc != FA_OK) return rc;
  rc = check_varlen_mode(B, total, max_seqlen, D, deterministic);
  if (rc != FA_OK) return rc;
  const void* all[11] = {q, k, v, o, lse, dout, dq, dk, dv, cu_seqlens, workspace};
  for (int i = 0; i < 10; ++i)
    if (!aligned16(all[i])) return FA_ERR_ALIGN;
  if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  const size_t wbytes = fa::bwd_varlen_workspace_bytes(B, Hq, total, D, deterministic, max_seqlen);
  if (workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
  const size_t qb = (size_t)Hq * total * D * 2, kb = (size_t)Hkv * total * D * 2;
  const size_t lb = (size_t)Hq * total * 4, cb = (size_t)(B + 1) * 4;
  const void* ins[7] = {q, k, v, o, lse, dout, cu_seqlens};
  const size_t isz[7] = {qb, kb, kb, qb, lb, qb, cb};
  const void* outs[4] = {dq, dk, dv, workspace};
  const size_t osz[4] = {qb, kb, kb, wbytes};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 7; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_INVALID;
    for (int j = 0; j < 4; ++j)
      if (j != i && overlaps(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_INVALID;
  }
  if (total == 0) return FA_OK;
  const fa::BwdArgs a{q, k, v, o, lse, dout, dq, dk, dv, 1, Hq, Hkv, total, D, causal ? 1 : 0,
                      scale, deterministic, workspace};
  const fa::VarlenArgs va{cu_seqlens, B, total, max_seqlen, workspace};
  return fa::launch_bwd_varlen(a, va, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_fwd_fp8_workspace_size(int B, int Hq, int Hkv, int N, int D) {
  if (check_shape(B, Hq, Hkv, N, D, 1.0f) != FA_OK) return 0;
  size_t total = 0;
  fa::fp8_layout(B, Hq, Hkv, N, D, nullptr, &total);
  return total;
}

int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int D, int causal, float scale, const float* signs,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_INVALID;
  int rc = check_shape(B, Hq, Hkv, N, D, scale);
  if (rc != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      (signs && !aligned16(signs)))
    return FA_ERR_ALIGN;
  if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  size_t wbytes = 0;
  fa::fp8_layout(B, Hq, Hkv, N, D, nullptr, &wbytes);
  if (workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
  const size_t qb = (size_t)B * Hq * N * D * 2, kb = (size_t)B * Hkv * N * D * 2;
  const size_t lb = (size_t)B * Hq * N * 4, sbytes = (size_t)D * 4;
  const void* ins[4] = {q, k, v, signs};
  const size_t isz[4] = {qb, kb, kb, signs ? sbytes : 0};
  const void* outs[3] = {o, lse, workspace};
  const size_t osz[3] = {qb, lb, wbytes};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (isz[j] && overlaps(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_INVALID;
    for (int j = 0; j < 3; ++j)
      if (j != i && overlaps(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_INVALID;
  }
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, N, D, causal ? 1 : 0, scale, 0};
  return fa::launch_fwd_fp8(a, signs, workspace, (hipStream_t)stream) == hipSuccess ? FA_OK
                                                                                    : FA_ERR_HIP;
}

int fa_fwd_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
  if (check_split(B, Hq, Hkv, Nq, Nk, D, 0, 1.0f) != FA_OK) return 0;
  return fa::split_auto(B, Hq, Hkv, Nq, Nk);
}

size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                     int num_splits) {
  if (check_split(B, Hq, Hkv, Nq, Nk, D, 0, 1.0f) != FA_OK) return 0;
  const int sp = resolve_splits(B, Hq, Hkv, Nq, Nk, num_splits);
  if (sp < 1) return 0;
  if (check_split_partials(Hq, Hkv, Nq, D, sp) != FA_OK) return 0;
  return fa::split_workspace_bytes(B, Hq, Nq, D, sp);
}

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int D, int causal, float scale,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID;
  int rc = check_split(B, Hq, Hkv, Nq, Nk, D, causal, scale);
  if (rc != FA_OK) return rc;
  const int sp = resolve_splits(B, Hq, Hkv, Nq, Nk, num_splits);
  if (sp < 1) return FA_ERR_INVALID;
  rc = check_split_partials(Hq, Hkv, Nq, D, sp);
  if (rc != FA_OK) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  const size_t wbytes = fa::split_workspace_bytes(B, Hq, Nq, D, sp);
  if (wbytes > 0) {
    if (!workspace || workspace_bytes < wbytes) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  }
  const size_t qb = (size_t)B * Hq * Nq * D * 2, kb = (size_t)B * Hkv * Nk * D * 2;
  const size_t lb = (size_t)B * Hq * Nq * 4;
  const void* outs[3] = {o, lse, workspace};
  const size_t osz[3] = {qb, lb, wbytes};
  const void* ins[3] = {q, k, v};
  const size_t isz[3] = {qb, kb, kb};
  for (int i = 0; i < 3; ++i) {
    if (osz[i] == 0) continue;
    for (int j = 0; j < 3; ++j)
      if (overlaps(outs[i], osz[i], ins[j], isz[j])) return FA_ERR_INVALID;
    for (int j = 0; j < 3; ++j)
      if (j != i && osz[j] > 0 && overlaps(outs[i], osz[i], outs[j], osz[j])) return FA_ERR_INVALID;
  }
  fa::FwdArgs a{q, k, v, o, lse, B, Hq, Hkv, Nq, D, causal ? 1 : 0, scale, 0};
  const fa::SplitArgs sa{Nq, Nk, sp, workspace};
  return fa::launch_fwd_split(a, sa, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int D, int deterministic) {
  if (check_shape(B, Hq, Hkv, N, D, 1.0f) != FA_OK) return 0;
  if (check_mode(N, D, deterministic) != FA_OK) return 0;
  return fa::bwd_layout(B, Hq, Hkv, N, D, deterministic).total;
}

}  // extern "C"

namespace {

struct Buf {
  const void* p;
  size_t bytes;
};

// Checks shared by the backward entry points: shape, scale, workspace size
// and alignment, pointer alignment, and that no written buffer overlaps any
// other buffer of the call.
int check_bwd(int B, int Hq, int Hkv, int N, int D, float scale, const void* workspace,
              size_t workspace_bytes, int deterministic, std::initializer_list<Buf> reads,
              std::initializer_list<Buf> writes, bool allow_head_split = true,
              bool own_workspace = false) {
  for (const Buf& b : reads)
    if (!b.p) return FA_ERR_INVALID;
  for (const Buf& b : writes)
    if (!b.p) return FA_ERR_INVALID;
  int rc = check_shape(B, Hq, Hkv, N, D, scale);
  if (rc != FA_OK) return rc;
  rc = check_mode(N, D, deterministic);
  if (rc != FA_OK) return rc;
  for (const Buf& b : reads)
    if (!aligned16(b.p)) return FA_ERR_ALIGN;
  for (const Buf& b : writes)
    if (!aligned16(b.p)) return FA_ERR_ALIGN;
  const fa::BwdLayout lay = fa::bwd_layout(B, Hq, Hkv, N, D, deterministic, allow_head_split);
  if (own_workspace) {
    // The library's fixed scratch stands in for the workspace.
    if (lay.total > fa::noalloc_scratch_bytes()) return FA_ERR_SCRATCH;
  } else {
    if (!workspace || workspace_bytes < lay.total) return FA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return FA_ERR_ALIGN;
  }
  const Buf ws{workspace, own_workspace ? 0 : lay.total};
  const Buf* wb = writes.begin();
  const size_t nw = writes.size();
  for (size_t i = 0; i < nw; ++i) {
    for (const Buf& r : reads)
      if (overlaps(wb[i].p, wb[i].bytes, r.p, r.bytes)) return FA_ERR_INVALID;
    for (size_t j = 0; j < nw; ++j)
      if (j != i && overlaps(wb[i].p, wb[i].bytes, wb[j].p, wb[j].bytes)) return FA_ERR_INVALID;
    if (overlaps(wb[i].p, wb[i].bytes, ws.p, ws.bytes)) return FA_ERR_INVALID;
  }
  for (const Buf& r : reads)
    if (overlaps(r.p, r.bytes, ws.p, ws.bytes)) return FA_ERR_INVALID;
  return FA_OK;
}

fa::BwdArgs bwd_args(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                     int D, int causal, float scale, void* workspace, int deterministic) {
  return fa::BwdArgs{q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, causal ? 1 : 0, scale,
                     deterministic, workspace};
}

size_t qbytes(int B, int Hq, int N, int D) { return (size_t)B * Hq * N * D * 2; }
size_t lbytes(int B, int Hq, int N) { return (size_t)B * Hq * N * 4; }

}  // namespace

extern "C" {

int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int Hq, int Hkv,
                      int N, int D, void* workspace, size_t workspace_bytes, int deterministic,
                      void* stream) {
  const size_t qb = qbytes(B, Hq, N, D), lb = lbytes(B, Hq, N);
  int rc = check_bwd(B, Hq, Hkv, N, D, 1.0f, workspace, workspace_bytes, deterministic,
                     {{o, qb}, {dout, qb}, {lse, lb}}, {});
  if (rc != FA_OK) return rc;
  const fa::BwdArgs a = bwd_args(nullptr, nullptr, nullptr, o, lse, dout, nullptr, nullptr,
                                 nullptr, B, Hq, Hkv, N, D, 0, 1.0f, workspace, deterministic);
  return fa::launch_bwd_preprocess(a, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_main(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                int B, int Hq, int Hkv, int N, int D, int causal, float scale, void* workspace,
                size_t workspace_bytes, int deterministic, void* stream) {
  const size_t qb = qbytes(B, Hq, N, D), kb = qbytes(B, Hkv, N, D);
  int rc = check_bwd(B, Hq, Hkv, N, D, scale, workspace, workspace_bytes, deterministic,
                     {{q, qb}, {k, kb}, {v, kb}, {dout, qb}}, {{dk, kb}, {dv, kb}});
  if (rc != FA_OK) return rc;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, nullptr, dout, nullptr, dk, dv, B, Hq, Hkv, N,
                                 D, causal, scale, workspace, deterministic);
  return fa::launch_bwd_main(a, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B,
              int Hq, int Hkv, int N, int D, int causal, float scale, void* workspace,
              size_t workspace_bytes, int deterministic, void* stream) {
  const size_t qb = qbytes(B, Hq, N, D), kb = qbytes(B, Hkv, N, D);
  int rc = check_bwd(B, Hq, Hkv, N, D, scale, workspace, workspace_bytes, deterministic,
                     {{q, qb}, {k, kb}, {v, kb}, {dout, qb}}, {{dq, qb}});
  if (rc != FA_OK) return rc;
  const fa::BwdArgs a = bwd_args(q, k, v, nullptr, nullptr, dout, dq, nullptr, nullptr, B, Hq, Hkv,
                                 N, D, causal, scale, workspace, deterministic);
  return fa::launch_bwd_dq(a, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N, int D,
           int causal, float scale, void* workspace, size_t workspace_bytes, int deterministic,
           void* stream) {
  const size_t qb = qbytes(B, Hq, N, D), kb = qbytes(B, Hkv, N, D), lb = lbytes(B, Hq, N);
  int rc = check_bwd(B, Hq, Hkv, N, D, scale, workspace, workspace_bytes, deterministic,
                     {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {lse, lb}, {dout, qb}},
                     {{dq, qb}, {dk, kb}, {dv, kb}});
  if (rc != FA_OK) return rc;
  const fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, causal,
                                 scale, workspace, deterministic);
  hipStream_t s = (hipStream_t)stream;
  if (fa::launch_bwd_preprocess(a, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_main(a, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dq(a, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int N,
                   int D, int causal, float scale, void* stream) {
  constexpr int kMode = 2;  // fixed-order dQ recomputing dS: row constants only
  const size_t qb = qbytes(B, Hq, N, D), kb = qbytes(B, Hkv, N, D), lb = lbytes(B, Hq, N);
  int rc = check_bwd(B, Hq, Hkv, N, D, scale, nullptr, 0, kMode,
                     {{q, qb}, {k, kb}, {v, kb}, {o, qb}, {lse, lb}, {dout, qb}},
                     {{dq, qb}, {dk, kb}, {dv, kb}}, false, true);
  if (rc != FA_OK) return rc;
  void* ws = nullptr;
  if (fa::noalloc_scratch(&ws) != hipSuccess) return FA_ERR_HIP;
  fa::BwdArgs a = bwd_args(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, D, causal, scale, ws,
                           kMode);
  a.allow_head_split = 0;
  hipStream_t s = (hipStream_t)stream;
  if (fa::launch_bwd_preprocess(a, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_main(a, s) != hipSuccess) return FA_ERR_HIP;
  if (fa::launch_bwd_dq(a, s) != hipSuccess) return FA_ERR_HIP;
  return FA_OK;
}

const char* fa_strerror(int status) {
  switch (status) {
    case FA_OK: return "success";
    case FA_ERR_INVALID: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_ALIGN: return "pointer not aligned (16 bytes; workspace 256 bytes)";
    case FA_ERR_WORKSPACE: return "workspace missing or too small";
    case FA_ERR_HIP: return "HIP runtime error at launch";
    case FA_ERR_TOO_LARGE: return "tensor too large (2^31 elements or more)";
    case FA_ERR_SCRATCH: return "problem needs more than the fixed scratch of fa_bwd_noalloc";
    default: return "unknown status";
  }
}

}  // extern "C"
