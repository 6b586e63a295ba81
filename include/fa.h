/*
 * fa.h -- C ABI of the fused exact-attention library for AMD Instinct MI355X (gfx950).
 *
 * The library computes O = softmax(scale * Q K^T) V and its gradients.  The
 * forward never forms the N x N score matrix: Q tiles stay resident while K/V
 * tiles stream past them, with a running row max and row sum (online
 * softmax).  The backward recomputes the probabilities tile by tile; its
 * fastest dQ mode (deterministic = 1) does keep one N x N quantity, the bf16
 * dS blocks on and below the diagonal, in the caller's workspace, while modes
 * 0 and 2 need only O(N) workspace per head (see fa_bwd).
 * Passages followed:
 *   - tiling and online softmax: "FlashAttention-4 算法解析" (zeeklog), section 4,
 *     the tiled forward pseudocode;
 *   - exp2 with the scale folded into log2(e), conditional rescale with
 *     tau = log2(256) = 8 and one final correction, optional cubic-polynomial
 *     exp2 after a 2^n / fraction split: hotelren FlashAttention-4 summary,
 *     sections 3.2 and 3.3; danialwang explainer, section 04 (巧招一, 巧招二);
 *   - backward recomputing P and forming dV, dP, dS, dK, dQ, with atomic dQ
 *     accumulation or a fixed-order deterministic mode: hotelren summary,
 *     sections 4.1-4.2; danialwang explainer, sections 05-06;
 *   - query heads sharing one K/V head (multi-query / grouped): hotdry
 *     article, kernel-fusion section.
 *
 * Conventions shared by every entry point
 *   - Tensors are contiguous, layout [B][H][N][D] with D innermost.  q, o, dout
 *     and dq have Hq heads; k, v, dk and dv have Hkv heads; Hq % Hkv == 0 and
 *     query head h reads K/V head h / (Hq / Hkv).
 *   - q, k, v, o, dout, dq, dk, dv are bfloat16; lse is float32 [B][Hq][N].
 *   - LSE is the natural log of sum_j exp(scale * q_i . k_j) over the keys row
 *     i may attend to.
 *   - causal != 0 masks key j for query i when j > i (queries and keys share
 *     the same length N and start at position 0).
 *   - Every pointer is a device pointer (HIP), 16-byte aligned.
 *   - stream is a hipStream_t passed as void*; NULL means the null stream.
 *   - Ownership: the caller allocates and frees every buffer, workspace
 *     included.  The library never allocates device memory, never frees and
 *     never synchronizes: each call only enqueues kernels on `stream` and
 *     returns.  Outputs are valid once that stream's work has completed.
 *     (fa_bwd_noalloc uses a fixed buffer that is part of the library's code
 *     object instead of a workspace; see there.)
 *   - Errors: every argument check runs before any launch, so a call that
 *     returns an error has launched nothing.  No exception crosses the ABI.
 *   - Supported now: D in {64, 128}; N >= 1; B, Hq, Hkv >= 1; B*Hq*N*D below
 *     2^31 elements per tensor.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID = -1,     /* null pointer, non-positive size, Hq % Hkv != 0, non-finite scale, aliasing */
    FA_ERR_UNSUPPORTED = -2, /* valid request the library does not handle (D not in {64,128}, scale <= 0) */
    FA_ERR_ALIGN = -3,       /* a pointer is not 16-byte aligned */
    FA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than fa_bwd_workspace_size() */
    FA_ERR_HIP = -5,         /* the HIP runtime reported an error at launch */
    FA_ERR_TOO_LARGE = -6,   /* a tensor exceeds 2^31 elements */
    FA_ERR_SCRATCH = -7      /* fa_bwd_noalloc: the problem needs more than the library's fixed scratch */
} fa_status;

/* Size of the fixed device scratch behind fa_bwd_noalloc (per GPU, held until
 * the process ends). */
#define FA_BWD_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * Forward pass.
 *   q [B][Hq][N][D], k/v [B][Hkv][N][D] (bf16, read)
 *   o [B][Hq][N][D] (bf16, written), lse [B][Hq][N] (fp32, written)
 *   scale: the softmax scale (typically 1/sqrt(D)), finite and > 0
 *   (non-finite: FA_ERR_INVALID; zero or negative: FA_ERR_UNSUPPORTED).
 * o must not overlap q, k or v.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int N, int D, int causal, float scale, void* stream);

/*
 * Forward pass with the exp2 split exposed: exp_poly_quarters in {0, 1, 2}
 * is the share (in quarters) of exponentials evaluated with the FMA-only
 * cubic polynomial after the 2^n / fraction split instead of the hardware
 * v_exp_f32 (hotelren summary, section 3.2, mixed execution).  fa_fwd uses
 * the library's default share.  Same arguments and errors as fa_fwd, plus
 * FA_ERR_INVALID for a share outside {0, 1, 2}.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int Hq, int Hkv, int N, int D, int causal, float scale,
              int exp_poly_quarters, void* stream);

/*
 * Bytes of device workspace fa_bwd needs for this problem and dQ mode
 * (deterministic, see fa_bwd): per-row Delta = rowsum(dO * O) and
 * LSE * log2(e), plus the fp32 dQ accumulator (mode 0) or the bf16 dS blocks
 * (mode 1); with grouped heads (Hq > Hkv), in modes 1 and 2, when
 * B * Hkv * ceil(N / 128) is small the query heads of each group are split
 * over several workgroups and the workspace also holds their fp32 partial dK
 * and dV (at most 2 * Hq/Hkv * B * Hkv * N * D * 4 bytes more).  Returns 0 for
 * invalid sizes or modes.
 */
size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int D, int deterministic);

/*
 * Backward pass.  Recomputes P from q, k and lse (never stored by the
 * forward), then forms dV = P^T dO, dP = dO V^T, dS = P o (dP - Delta),
 * dK = scale dS^T Q and dQ = scale dS K.
 *   q, k, v, o, lse: exactly as given to / returned by fa_fwd (read)
 *   dout [B][Hq][N][D] (bf16, read)
 *   dq [B][Hq][N][D], dk/dv [B][Hkv][N][D] (bf16, written)
 *   workspace: device memory of at least fa_bwd_workspace_size() bytes,
 *     256-byte aligned, owned by the caller; its contents on entry do not
 *     matter and are scratch afterwards.  Two calls in flight at once must
 *     not share a workspace.
 *   deterministic selects how dQ is accumulated (danialwang explainer,
 *   sections 05-06, atomic and fixed-order accumulation):
 *   0: each key tile's dQ contribution is added into an fp32 accumulator
 *     with atomics (no run-to-run bitwise guarantee for dq); workspace
 *     B*Hq*N*(D+2)*4 bytes.
 *   1: the main pass stores dS in bf16 blocks of 32 x 32 and a separate pass
 *     that owns each query tile sums dS K over the key tiles in a fixed
 *     ascending order; workspace about B*Hq*N*N*2 bytes (one head's blocks
 *     must stay below 4 GiB - 8 KiB, else FA_ERR_TOO_LARGE).
 *   2: as 1, but the separate pass recomputes S, dP and dS instead of
 *     reading them; workspace B*Hq*N*8 bytes (plus the grouped-head partials
 *     above).
 *   Modes 1 and 2 give dq, dk and dv bit-identical across calls with the
 *   same inputs on the same device.  Other values: FA_ERR_INVALID.
 * With Hq != Hkv, dk and dv sum over the query heads that share a K/V head.
 * dq, dk, dv must not overlap any input.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int N, int D, int causal, float scale,
           void* workspace, size_t workspace_bytes, int deterministic, void* stream);

/*
 * The three stages fa_bwd runs, exported so that a caller can schedule or
 * time them separately.  Called in this order on one stream with the same
 * problem and workspace, they are exactly fa_bwd.  Arguments have the
 * meaning given for fa_bwd; each stage checks the arguments it uses and
 * returns the same codes.
 *   fa_bwd_preprocess: Delta_i = rowsum(dO * O) and LSE_i * log2(e) into the
 *     workspace, and (mode 0) clears the workspace's fp32 dQ accumulator.
 *   fa_bwd_main: recomputes P tile by tile from q, k and the workspace's
 *     LSE * log2(e), and forms dK, dV (written to dk, dv); in mode 0 it
 *     also accumulates the unscaled dQ sums in the workspace, in mode 1 it
 *     stores the dS blocks there.
 *   fa_bwd_dq: mode 0: dq = bf16(scale * accumulated dQ) (q, k, v, dout
 *     unused but checked); modes 1 and 2: the fixed-order dQ pass.
 */
int fa_bwd_preprocess(const void* o, const void* dout, const float* lse, int B, int Hq, int Hkv,
                      int N, int D, void* workspace, size_t workspace_bytes, int deterministic,
                      void* stream);
int fa_bwd_main(const void* q, const void* k, const void* v, const void* dout, void* dk, void* dv,
                int B, int Hq, int Hkv, int N, int D, int causal, float scale, void* workspace,
                size_t workspace_bytes, int deterministic, void* stream);
int fa_bwd_dq(const void* q, const void* k, const void* v, const void* dout, void* dq, int B,
              int Hq, int Hkv, int N, int D, int causal, float scale, void* workspace,
              size_t workspace_bytes, int deterministic, void* stream);

/*
 * Backward pass that allocates nothing and takes no workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * training or serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, layout and results as fa_bwd in dQ mode 2 (fixed-order dQ,
 * recomputing dS; dq, dk, dv bit-identical run to run), except that:
 *   - its scratch (per-row Delta and LSE * log2(e), 256-byte aligned) lives
 *     in a fixed buffer of FA_BWD_NOALLOC_SCRATCH_BYTES inside the library,
 *     one per GPU, kept for the life of the process.  A problem that needs
 *     more (B*Hq*N*8 bytes plus alignment, i.e. B*Hq*N above about 4.19
 *     million rows) returns FA_ERR_SCRATCH before anything is launched;
 *   - the query heads of a K/V head are never split over several workgroups
 *     (no fp32 partial dK, dV), so with Hq > Hkv the sum over a group's
 *     heads runs in one workgroup: dk and dv can differ from fa_bwd's in the
 *     last bits, within the same tolerances;
 *   - every call on one GPU shares that buffer: calls that may overlap in
 *     time on one GPU (other streams, other threads) race and must be
 *     serialized by the caller.  Nothing in it needs clearing between calls.
 * The first call on a device looks the buffer's device address up once
 * (hipGetSymbolAddress, with that device current); no call allocates or frees.
 * The buffer used is the current device's, so stream must be a stream of the
 * current device (or NULL).
 * Errors as fa_bwd, plus FA_ERR_SCRATCH; FA_ERR_HIP also if the lookup fails.
 */
int fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv,
                   int B, int Hq, int Hkv, int N, int D, int causal, float scale, void* stream);

/*
 * Variable-length batches (forward).  B sequences of lengths len_b are packed
 * along one token axis of total = sum_b len_b tokens:
 *   q, o [Hq][total][D], k, v [Hkv][total][D] (bf16), lse [Hq][total] (fp32);
 *   sequence b is rows cu_seqlens[b] .. cu_seqlens[b+1] - 1 of every head's
 *   [total][D] matrix, and attends only within itself (causal: key j <= query
 *   i, positions counted from the sequence start).
 *   cu_seqlens: device int32[B + 1], nondecreasing, cu_seqlens[0] = 0,
 *     cu_seqlens[B] = total (read on the device only; entries outside
 *     [0, total] are clamped, so a malformed array cannot make a kernel
 *     address outside the tensors, but its results are unspecified).
 *     Sequences of length 0 are allowed.
 *   max_seqlen: an upper bound of every len_b, 1 <= max_seqlen <=
 *     fa_varlen_max_seqlen() (sizes the scheduler; a sequence longer than it
 *     is still computed correctly, only scheduled as if it were max_seqlen).
 *   workspace: device memory of fa_fwd_varlen_workspace_size(B, total)
 *     bytes, 256-byte aligned, caller-owned scratch for the work list.
 * The work is scheduled on the device, without a host round trip: a first
 * kernel lists every (sequence, 128-query tile) and sorts the list by the
 * number of K/V tiles each item processes, largest first (danialwang
 * explainer, section 06, starting the longest work first); the attention
 * kernel takes items in that order.  total = 0 is valid and writes nothing.
 * Errors as fa_fwd, plus FA_ERR_WORKSPACE, and FA_ERR_INVALID for B < 1,
 * total < 0 or max_seqlen outside its range.
 */
size_t fa_fwd_varlen_workspace_size(int B, int total);
int fa_varlen_max_seqlen(void);
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* cu_seqlens, int B, int Hq, int Hkv, int total, int max_seqlen,
                  int D, int causal, float scale, void* workspace, size_t workspace_bytes,
                  void* stream);

/*
 * Variable-length backward: the gradients of fa_fwd_varlen, same packing:
 *   q, o, dout, dq [Hq][total][D], k, v, dk, dv [Hkv][total][D], lse
 *   [Hq][total]; cu_seqlens, B, total, max_seqlen as for fa_fwd_varlen, with
 *   max_seqlen <= fa_varlen_max_seqlen() / 2.
 *   deterministic: 0, 1 or 2 as for fa_bwd.  Mode 1 keeps, per query head,
 *     each sequence's grid of 32 x 32 dS blocks in the workspace, packed one
 *     sequence after another; its size is bounded with max_seqlen, so in
 *     mode 1 every sequence must be at most max_seqlen long for a correct dQ
 *     (a longer one stays memory-safe: blocks beyond the region are neither
 *     written nor read, and that dQ is unspecified).  Mode 1 returns
 *     FA_ERR_TOO_LARGE when one head's region would exceed 4 GiB
 *     ((ceil(total/32) + B) * ceil(max_seqlen/32) blocks of 2 KiB); mode 0
 *     when one head's fp32 accumulator, total * D * 4 bytes, reaches 2 GiB.
 *   workspace: fa_bwd_varlen_workspace_size(B, Hq, Hkv, total, max_seqlen, D,
 *     deterministic) bytes, 256-byte aligned (0 for an invalid argument).
 * Work lists are built on the device as for the forward: the dK/dV pass takes
 * (sequence, 128-key block) items by decreasing number of query steps, the
 * dQ pass (sequence, 128-query tile) items by decreasing number of key tiles.
 * total = 0 is valid and writes nothing.
 */
size_t fa_bwd_varlen_workspace_size(int B, int Hq, int Hkv, int total, int max_seqlen, int D,
                                    int deterministic);
int fa_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens,
                  int B, int Hq, int Hkv, int total, int max_seqlen, int D, int causal,
                  float scale, void* workspace, size_t workspace_bytes, int deterministic,
                  void* stream);

/*
 * Decode-shaped forward with the keys split across workgroups (split-KV).
 * For few queries over long keys, typically G = Hq / Hkv query heads
 * sharing one K/V head (multi-query / grouped attention, hotdry article,
 * kernel-fusion section):
 *   q, o [B][Hq][Nq][D], k, v [B][Hkv][Nk][D] (bf16), lse [B][Hq][Nq] (fp32),
 *   1 <= Nq, 1 <= Nk, and Nq <= Nk when causal.
 * causal != 0 aligns the queries with the end of the keys: query i sees keys
 * j <= Nk - Nq + i (the Nq queries are the newest Nq positions).
 * The G * Nq query rows of a K/V group are processed together against one
 * range of keys per workgroup; with more than one range, each range writes
 * an fp32 partial (O_s normalised, LSE_s) to the workspace and a second
 * kernel merges them: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 *   num_splits: number of key ranges, 1 .. ceil(Nk / 64); 0 picks
 *     fa_fwd_splitkv_num_splits() (enough workgroups to fill the GPU).
 *   workspace: fa_fwd_splitkv_workspace_size() bytes (0 when one range:
 *     workspace may then be NULL), 256-byte aligned, caller-owned scratch.
 * Errors as fa_fwd, plus FA_ERR_INVALID for Nq < 1, Nk < 1, causal with
 * Nq > Nk, or num_splits out of range, and FA_ERR_WORKSPACE.
 */
int fa_fwd_splitkv_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int D);
size_t fa_fwd_splitkv_workspace_size(int B, int Hq, int Hkv, int Nq, int Nk, int D,
                                     int num_splits);
int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int D, int causal, float scale,
                   int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * FP8 forward (OCP e4m3 matrix products), for the same tensors and layout as
 * fa_fwd.  Following the hotdry article's FP8 passage ("incoherent
 * processing"): Q and K are rotated by x -> (x o signs) H / sqrt(D), H the
 * Walsh-Hadamard matrix, which leaves Q K^T unchanged and spreads outlier
 * channels; Q, K and V are quantized to e4m3 with one scale per 64 rows of
 * each (batch, head) (Q, K: largest magnitude -> 448; V: a power of two);
 * both products run on the FP8 matrix cores; P is rounded to e4m3 (as 256 P,
 * kept <= 1 before scaling by rescaling whenever a row maximum grows).  O is
 * bf16 and LSE fp32 as in fa_fwd.  The rounding to e4m3 costs accuracy
 * (about 2^-4 relative per element of P and of the inputs); see the tests
 * for the bounds used.
 *   signs: device float[D] of +1 / -1 (drawn by the caller; NULL = no
 *     rotation).
 *   workspace: fa_fwd_fp8_workspace_size() bytes, 256-byte aligned: the
 *     quantized copies and their scales.
 * Errors as fa_fwd, plus FA_ERR_WORKSPACE.
 */
size_t fa_fwd_fp8_workspace_size(int B, int Hq, int Hkv, int N, int D);
int fa_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
               int Hkv, int N, int D, int causal, float scale, const float* signs,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Diagnostic: y[i] = the forward's FMA-only exp2 of x[i] (2^n times the cubic
 * in the fraction, n = floor(x); the polynomial share of fa_fwd_ex; hotelren
 * FlashAttention-4 summary, section 3.2), evaluated on the device exactly as
 * the forward kernel evaluates it, so a test can compare it bit for bit with
 * a host evaluation.  x, y: device float[n] (may alias), n >= 0; nothing is
 * launched for n = 0.  Returns FA_ERR_INVALID for n < 0 or a null pointer
 * with n > 0, FA_ERR_HIP if the launch fails.
 */
int fa_exp2_poly_eval(const float* x, float* y, int n, void* stream);

/* Static text for a status code. */
const char* fa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
