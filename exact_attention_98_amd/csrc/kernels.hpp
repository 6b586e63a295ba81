// Internal launch interface between the C ABI (fa_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int B, Hq, Hkv, N, D;
  int causal;
  float scale;
  int poly_quarters;
};

// Kernel-side parameters of the forward (passed by value).
struct FwdParams {
  int BH;     // B * Hq
  int Hq;
  int G;      // Hq / Hkv
  int N;
  int nqb;    // query tiles per head
  float c;    // scale * log2(e)
  // Variable length only: cumulative sequence starts (B + 1), the work list
  // of (sequence, query tile) pairs and its length, and the token count.
  const int* cu;
  const int* items;
  const int* n_items;
  int total;
  // Split-KV only: query and key lengths, the key-range split, and the fp32
  // partial results [B*Hkv][splits][G*Nq][D] and [B*Hkv][splits][G*Nq].
  int Nq, Nk;
  int splits, tiles_per_split;
  float* o_part;
  float* l_part;
};

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// y[i] = exp2_poly(x[i]) on the device (the forward's FMA-only exp2).
hipError_t launch_exp2_poly_eval(const float* x, float* y, int n, hipStream_t stream);

// Variable-length forward.  Layout: q, o [Hq][total][D]; k, v [Hkv][total][D];
// lse [Hq][total]; sequence b is rows cu[b] .. cu[b+1] of every head.
struct VarlenArgs {
  const int* cu;       // device, B + 1 entries
  int B;
  int total;
  int max_seqlen;
  void* workspace;     // varlen_workspace_bytes(B, total)
};
size_t varlen_workspace_bytes(int B, int total);
// Items one work list holds (tiles of 128 rows or more): total / 128 + B.
int varlen_item_capacity(int B, int total);
// Largest max_seqlen the work-list builder supports (its histogram lives in LDS).
int varlen_max_seqlen_limit();
hipError_t launch_fwd_varlen(const FwdArgs& a, const VarlenArgs& v, hipStream_t stream);
// Work list of a variable-length batch into n_items / items (2 ints per item,
// at most varlen_item_capacity(B, total) items, enough for tiles of rows >= 128
// of sequences that do not overlap): kind 0 = (sequence, query tile of `rows`) by 64-key tiles
// walked; kind 1 = (sequence, key block of `rows`) by query steps of qstep
// walked; largest first.
hipError_t launch_varlen_schedule(const VarlenArgs& v, int causal, int kind, int qstep, int rows,
                                  int* n_items, int* items, hipStream_t stream);

// Split-KV forward for decode-shaped problems: q, o [B][Hq][Nq][D], k, v
// [B][Hkv][Nk][D], lse [B][Hq][Nq]; causal rows are aligned to the end of the
// keys (query i sees keys j <= Nk - Nq + i).
struct SplitArgs {
  int Nq, Nk;
  int splits;        // >= 1 (already resolved)
  void* workspace;   // split_workspace_bytes(...)
};
int split_auto(int B, int Hq, int Hkv, int Nq, int Nk);
int split_max(int Nk);
size_t split_workspace_bytes(int B, int Hq, int Nq, int D, int splits);
hipError_t launch_fwd_split(const FwdArgs& a, const SplitArgs& s, hipStream_t stream);

// FP8 forward: quantized copies of Q, K (rotated) and V (transposed per
// 64-key tile) and their per-tile scales, all in the caller's workspace.
struct Fp8Layout {
  int N, Np, nt;       // rows, rows padded to whole 64-row tiles, tiles per head
  int BHq, BHkv;       // B * Hq, B * Hkv
  uint8_t* q8;         // e4m3 [B*Hq][Np][D]
  uint8_t* k8;         // e4m3 [B*Hkv][Np][D]
  uint8_t* v8;         // e4m3 [B*Hkv][nt][D][64], keys in P-operand order
  float* qs;           // dequantization factors [B*Hq][nt]
  float* ks;           // [B*Hkv][nt]
  int* ve;             // V factor exponents e (2^e) [B*Hkv][nt]
};
Fp8Layout fp8_layout(int B, int Hq, int Hkv, int N, int D, void* workspace, size_t* total);
hipError_t launch_fwd_fp8(const FwdArgs& a, const float* signs, void* workspace, hipStream_t stream);

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int B, Hq, Hkv, N, D;
  int causal;
  float scale;
  int deterministic;
  void* workspace;
  // 0: the main kernel never splits a K/V head's query heads over several
  // workgroups (no fp32 partial dK, dV in the workspace).
  int allow_head_split = 1;
};

// Workspace layout of the backward (offsets in bytes, 256-byte aligned).
struct BwdLayout {
  size_t delta;     // fp32 [B][Hq][N]
  size_t lse2;      // fp32 [B][Hq][N], LSE * log2(e)
  size_t dq_acc;    // fp32 [B][Hq][N][D] (atomic mode only)
  size_t ds;        // dS^T blocks, ds_head_bytes(N) per (b, hq) (stored-dS mode only)
  size_t kv_part;   // fp32 [hsplit][2][B][Hkv][N][D] partial dK, dV (hsplit > 1 only)
  int hsplit;       // query-head groups per K/V head in the main kernel's grid
  size_t total;
};

// Number of parts the G query heads of a K/V head are cut into in the main
// backward kernel's grid (D = 128, fixed-order dQ modes): more than one when
// B * Hkv * ceil(N / 128) key tiles alone would leave the grid short of
// workgroups; the parts' dK, dV are then summed in a fixed order.
int bwd_head_split(int B, int Hq, int Hkv, int N, int D, int deterministic);

// Bytes of the stored-dS blocks of one (batch, query head).
size_t ds_head_bytes(int N);

BwdLayout bwd_layout(int B, int Hq, int Hkv, int N, int D, int deterministic,
                     bool allow_head_split = true);

// The library's own fixed scratch for fa_bwd_noalloc: its size, and its
// device address on the current device (looked up once per device).
size_t noalloc_scratch_bytes();
hipError_t noalloc_scratch(void** ptr);
// The three backward stages; each reads only the BwdArgs fields it needs.
hipError_t launch_bwd_preprocess(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_main(const BwdArgs& a, hipStream_t stream);
// By dQ mode (the deterministic argument): 0 atomic, dq = bf16(scale *
// accumulated dQ); 1 stored dS, the fixed-order dS K pass; 2 recompute, the
// fixed-order pass that recomputes S, dP and dS.
hipError_t launch_bwd_dq(const BwdArgs& a, hipStream_t stream);

// Variable-length backward, dQ modes 0 (atomic), 1 (stored dS) and 2
// (recompute): a holds the packed tensors as B = 1, N = total; v the
// sequences.  Workspace layout: the dense layout for (1, Hq, total) (mode 1:
// that of mode 2), then (mode 1) Hq regions of ds_head bytes of dS blocks,
// the two work lists and (mode 1) the B + 1 block offsets.
struct VarlenBwdLayout {
  size_t ds, ds_head;   // stored-dS regions (mode 1): offset, bytes per head
  int cap_blocks;       // 32 x 32 blocks per head region
  size_t main_list, dq_list, blk_off, total;
};
// Bytes of one head's stored-dS region for packed sequences no longer than
// max_seqlen.
size_t varlen_ds_head_bytes(int B, int total, int max_seqlen);
VarlenBwdLayout bwd_varlen_layout(int B, int Hq, int total, int D, int deterministic, int max_seqlen);
size_t bwd_varlen_workspace_bytes(int B, int Hq, int total, int D, int deterministic, int max_seqlen);
hipError_t launch_bwd_varlen(const BwdArgs& a, const VarlenArgs& v, hipStream_t stream);

}  // namespace fa
